"""SALAD linear branch (ReLU-kernel linear attention) vs the oracle's
per-row form.  bf16 inputs, fp32 accumulation, the d x d summary applied as
a bf16 pair, O in bf16: max |dO| <= 2e-2 and relative RMS <= 1e-2.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tra():
    import static_sparse_spatiotemporal_amd as m
    assert torch.cuda.is_available()
    m.load_library()
    return m


def check(tra, B, H, n, D, seed, rows=None, scale=1.0):
    print(f"[linear] B={B} H={H} n={n} D={D}", flush=True)
    w = workloads.Workload("lin", "dense", "element", 1, n, B, H, D, "bf16", seed=seed, value_scale=scale)
    q, k, v = workloads.make_qkv(w, device="cuda")
    out = tra.linear_attn_fwd(q, k, v)
    torch.cuda.synchronize()
    arrs = [workloads.to_oracle_array(x) for x in (q, k, v)]
    ref = oracle.linear_attention_rows(*arrs, rows=rows, eps=1e-6)
    got = (out.float().cpu().numpy().reshape(-1, D) if rows is None
           else out[rows[:, 0], rows[:, 1], rows[:, 2]].float().cpu().numpy())
    err = float(np.abs(got - ref).max())
    rel = float(np.sqrt(((got - ref) ** 2).sum() / (ref ** 2).sum()))
    print(f"         max|dO|={err:.3e} rel-rms={rel:.2e} max|ref|={np.abs(ref).max():.3f}", flush=True)
    assert err <= 2e-2 and rel <= 1e-2


@pytest.mark.parametrize("n,D", [(1, 64), (300, 64), (300, 128), (128, 128), (2048, 64), (2100, 128),
                                 (4100, 128), (5000, 64)])
def test_linear_full_parity(tra, n, D):
    check(tra, 2, 2, n, D, seed=900 + n + D)


def test_linear_headline_shape(tra):
    """n = 131072, 24 heads, d = 128 (the headline's Q, K, V shape), sampled rows."""
    rng = np.random.default_rng(12)
    rows = np.array([(0, h, int(t)) for h in (0, 23) for t in
                     np.concatenate([[0, 1, 131071], rng.integers(0, 131072, 20)])], np.int64)
    check(tra, 1, 24, 131072, 128, seed=1005, rows=rows)


def test_linear_errors(tra):
    q = torch.zeros((1, 1, 128, 64), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError, match="holds 16 bytes"):
        tra.linear_attn_fwd(q, q, q, workspace=ws)  # workspace too small
    with pytest.raises(ValueError, match="dtype"):
        tra.linear_attn_fwd(q.float(), q.float(), q.float())
    assert tra.linear_attn_workspace_bytes(1, 1, 128, 96) == 0
    # the library refuses the same on its own (called directly)
    lib = tra.load_library()
    d = tra._desc(q)
    r = ctypes.byref
    assert lib.tra_linear_attn_fwd(r(d), r(d), r(d), r(d), 1e-6, ctypes.c_void_p(ws.data_ptr()), 16, None) == -1
    f = tra._desc(q.float())
    need = tra.linear_attn_workspace_bytes(1, 1, 128, 64)
    big = torch.empty(need + 256, dtype=torch.uint8, device="cuda")
    assert lib.tra_linear_attn_fwd(r(f), r(f), r(f), r(f), 1e-6, ctypes.c_void_p(big.data_ptr()), need,
                                   None) == -2


def test_linear_strided_views(tra):
    """[B, H, n, D] views of [B, n, H, D] storage (inputs and output) give the
    contiguous run's output bit for bit."""
    w = workloads.Workload("lin", "dense", "element", 1, 3000, 2, 3, 128, "bf16", seed=77)
    q, k, v = workloads.make_qkv(w, device="cuda")
    ref = tra.linear_attn_fwd(q, k, v)
    view = lambda x: x.transpose(1, 2).contiguous().transpose(1, 2)
    qs, ks, vs = (view(x) for x in (q, k, v))
    assert not qs.is_contiguous()
    out = torch.empty(2, 3000, 3, 128, dtype=torch.bfloat16, device="cuda").transpose(1, 2)
    tra.linear_attn_fwd(qs, ks, vs, out=out)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
