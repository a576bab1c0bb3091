"""The usage example in README.md runs as written and its streaming loop
reproduces the frame sliding-window forward (bf16 rounding for O; LSE to
the bf16 tolerance)."""
import pathlib
import re

import pytest
import torch

pytestmark = pytest.mark.gpu


def test_readme_example_runs():
    text = (pathlib.Path(__file__).resolve().parent.parent / "README.md").read_text()
    code = re.search(r"## Use\n\n```python\n(.*?)```", text, re.S).group(1)
    env: dict = {}
    exec(compile(code, "README.md", "exec"), env)
    tra, q, k, v = env["tra"], env["q"], env["k"], env["v"]
    f, s = env["f"], env["s"]
    assert env["out"].shape == q.shape and env["lse"].shape == q.shape[:3]
    assert env["qg"].grad is not None and torch.isfinite(env["qg"].grad.float()).all()
    ref, ref_lse = tra.sparse_attn_fwd(q, k, v, env["window"])
    last = slice((f - 1) * s, f * s)
    torch.cuda.synchronize()
    assert float((env["o_t"].float() - ref[:, :, last].float()).abs().max()) <= 2e-2
    assert float((env["lse_t"] - ref_lse[:, :, last]).abs().max()) <= 1e-3
    for m in ("mask", "radius", "window"):
        env[m].free()
    env["cache"].free()
