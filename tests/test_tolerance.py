"""The per-row LSE bound of the bf16 kernels' query rounding, checked with the
oracle alone: the fp64 attention over the exact bf16 queries and the one over
the rounded scaled queries (with the scale ln 2, i.e. the same scores in
natural units) differ by no more than the bound on every row, and by far
less than the rounding itself on O."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.tolerance import QUERY_ROUNDING, TOL_LSE_EXACT, lse_bound, rounded_query


@pytest.mark.parametrize("kind,f,s,D,extra", [
    ("radial", 8, 64, 64, {}),
    ("radial", 4, 128, 128, {}),
    ("swa", 6, 40, 128, dict(window=3)),
    ("dense", 2, 96, 64, {}),
])
def test_query_rounding_within_bound(kind, f, s, D, extra):
    w = workloads.Workload(f"{kind}_f{f}_s{s}", kind, "element", f, s, 1, 2, D, "bf16", seed=77 + D, **extra)
    q, k, v = workloads.make_qkv(w, device="cpu")
    spec = oracle.MaskSpec(kind, f, s, **extra)
    arr = workloads.to_oracle_array
    ref_o, ref_l = oracle.attention_rows(arr(q), arr(k), arr(v), spec)
    qr = rounded_query(q)
    got_o, got_l = oracle.attention_rows(arr(qr), arr(k), arr(v), spec, scale=math.log(2.0))
    dl = np.abs(got_l - ref_l)
    bound = lse_bound(q, k)
    assert np.all(dl <= bound - TOL_LSE_EXACT)
    # the rounding is visible (the test is not vacuous) and stays well inside
    # the bound, whose Cauchy-Schwarz step is loose for random inputs
    assert dl.max() > 1e-6 and dl.max() < 0.5 * (bound - TOL_LSE_EXACT).max()
    assert np.abs(got_o - ref_o).max() < 2e-2


def test_rounded_query_is_one_bf16_rounding():
    """Each rounded query element is within the bf16 unit roundoff 2^-8
    (relative) of q * scale * log2(e); bf16 inputs times that constant are
    not bf16 values, so the rounding is real."""
    g = torch.Generator().manual_seed(3)
    q = torch.randn(1, 1, 64, 128, generator=g).to(torch.bfloat16)
    qr = rounded_query(q).double()
    exact = q.double() * (1.0 / math.sqrt(128) * 1.4426950408889634)
    nz = exact != 0
    rel = ((qr - exact).abs()[nz] / exact.abs()[nz])
    assert rel.max().item() <= QUERY_ROUNDING and rel.max().item() > 2.0 ** -10
    assert (rel > 0).float().mean().item() > 0.9
