"""Pins of the oracle's SALAD linear branch (ReLU-kernel linear attention).

CPU only.  Reference points: the associative form phi(Q)(phi(K)^T V) evaluated
with torch matmuls in float64 (a library routine), and closed forms.
"""
import numpy as np
import torch

import oracle


def _inputs(B, H, n, d, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    xs = [torch.randn(B, H, n, d, generator=g) for _ in range(3)]
    if dtype == "bf16":
        xs = [x.to(torch.bfloat16) for x in xs]
    return xs


def _np(x):
    if x.dtype == torch.bfloat16:
        return x.contiguous().view(torch.int16).numpy().view(np.uint16)
    return x.contiguous().numpy()


def test_matches_associative_form():
    """sum_t w_t V_t / (sum_t w_t + eps) equals phi(Q)(phi(K)^T V) /
    (phi(Q) phi(K)^T 1 + eps) (matrix products in float64)."""
    for dtype in ("f32", "bf16"):
        q, k, v = _inputs(2, 2, 200, 16, dtype, seed=31)
        o = oracle.linear_attention_rows(_np(q), _np(k), _np(v), eps=1e-6, threads=4)
        fq, fk, v64 = q.double().relu(), k.double().relu(), v.double()
        kv = fk.transpose(-1, -2) @ v64
        z = fk.sum(dim=2, keepdim=True)
        ref = (fq @ kv) / (fq @ z.transpose(-1, -2) + 1e-6)
        np.testing.assert_allclose(o, ref.reshape(-1, 16).numpy(), rtol=1e-12, atol=1e-12)


def test_equal_keys_give_mean_of_v():
    """All keys equal (and positive somewhere): the weights are equal, so O is
    the mean of V (up to eps)."""
    q, _, v = _inputs(1, 1, 50, 8, "f32", seed=4)
    k = torch.ones_like(q) * 0.5
    o = oracle.linear_attention_rows(_np(q), _np(k), _np(v), eps=0.0)
    fq = q.relu().sum(-1).reshape(-1).numpy()
    want = np.repeat(v.double().mean(dim=2).numpy().reshape(1, 8), 50, axis=0)
    ok = fq > 0
    np.testing.assert_allclose(o[ok], want[ok], rtol=1e-12, atol=1e-12)
    assert not o[~ok].any()


def test_nonpositive_query_gives_zero():
    """phi(Q) = 0 for a query with no positive component: O = 0 exactly."""
    q, k, v = _inputs(1, 1, 30, 8, "f32", seed=5)
    q = -q.abs()
    o = oracle.linear_attention_rows(_np(q), _np(k), _np(v), eps=1e-6)
    assert not o.any()


def test_unit_query_picks_a_key_column():
    """Q = e_i: w_t = relu(K[t, i]), a weighted mean of V by one column of K."""
    _, k, v = _inputs(1, 1, 40, 8, "f32", seed=6)
    q = torch.zeros_like(k)
    q[0, 0, :, 3] = 1.0
    o = oracle.linear_attention_rows(_np(q), _np(k), _np(v), eps=0.0)
    w = k[0, 0, :, 3].double().relu().numpy()
    want = (w[:, None] * v[0, 0].double().numpy()).sum(0) / w.sum()
    np.testing.assert_allclose(o, np.repeat(want[None], 40, axis=0), rtol=1e-12, atol=1e-12)
