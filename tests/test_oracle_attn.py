"""Pins of the oracle's attention (Radial Attention section 2, eq. 1 and eq. 2).

CPU only.  The reference points are a library routine (torch's
scaled_dot_product_attention in float64), closed forms and invariants.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import MaskSpec, brute


def _inputs(B, H, n, d, dtype, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    xs = [torch.randn(B, H, n, d, generator=g) * scale for _ in range(3)]
    if dtype == "bf16":
        xs = [x.to(torch.bfloat16) for x in xs]
    return xs


def _np(x):
    if x.dtype == torch.bfloat16:
        return x.contiguous().view(torch.int16).numpy().view(np.uint16)
    return x.contiguous().numpy()


def _sdpa64(q, k, v, keep=None, scale=None):
    q, k, v = (x.to(torch.float64) for x in (q, k, v))
    mask = None if keep is None else torch.from_numpy(keep.astype(bool))
    return F.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=scale)


def _dilated(spec):
    keep = oracle.block_counts(spec) > 0
    b = spec.block
    return np.kron(keep.astype(np.uint8), np.ones((b, b), np.uint8))[:spec.n, :spec.n]


def _keep_matrix(spec):
    """Element view of the mask built without the oracle's mask code where
    possible (brute force for the block-index reading)."""
    if spec.granularity == "element":
        return oracle.element_matrix(spec)
    if spec.granularity == "block_eq4":
        keep = brute.radial_blocks(spec.f, spec.s, spec.block, spec.sink_frames)
        return np.kron(keep, np.ones((spec.block, spec.block), np.uint8))
    return _dilated(spec)


SPECS = [
    MaskSpec("radial", 6, 16),
    MaskSpec("radial", 24, 3),                      # reaches eq. 4 case (b)
    MaskSpec("radius3d", 4, 20, grid_h=4, grid_w=5, r_t=1, r_s=1),
    MaskSpec("swa", 8, 8, window=3),
    MaskSpec("dense", 3, 20),
    MaskSpec("radial", 16, 16, granularity="block_any"),
    MaskSpec("radial", 5, 80, granularity="block_any"),   # n = 400: ragged last block
    MaskSpec("radial", 6, 16, sink_frames=1),
    MaskSpec("swa", 6, 10, window=2, sink_frames=1),
    MaskSpec("radial", 12, 16, granularity="block_eq4", block=8),
    MaskSpec("radial", 9, 16, granularity="block_eq4", block=4, sink_frames=1),
]


@pytest.mark.parametrize("spec", SPECS, ids=lambda s: f"{s.kind}-{s.granularity}-{s.f}x{s.s}-sink{s.sink_frames}")
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_matches_sdpa_float64(spec, dtype):
    """eq. 2 with M from the family equals torch SDPA with the boolean mask."""
    B, H, d = 2, 2, 16
    q, k, v = _inputs(B, H, spec.n, d, dtype, seed=11)
    o, lse = oracle.attention_rows(_np(q), _np(k), _np(v), spec, threads=4)
    keep = _keep_matrix(spec)
    ref = _sdpa64(q, k, v, keep).reshape(-1, d).numpy()
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)
    # LSE: log of the softmax denominator of the kept scaled scores.
    s = (q.double() @ k.double().transpose(-1, -2)) / np.sqrt(d)
    s = s.masked_fill(~torch.from_numpy(keep.astype(bool)), float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=-1).reshape(-1).numpy(), rtol=0, atol=1e-12)


def test_dense_is_eq1():
    """An all-zero M reproduces standard attention (eq. 1)."""
    spec = MaskSpec("dense", 4, 24)
    q, k, v = _inputs(1, 3, spec.n, 32, "f32", seed=5)
    o, _ = oracle.attention_rows(_np(q), _np(k), _np(v), spec)
    np.testing.assert_allclose(o, _sdpa64(q, k, v).reshape(-1, 32).numpy(), rtol=0, atol=1e-12)


def test_radius_zero_is_identity():
    """r_t = r_s = 0: the only key is the token itself, so O = V exactly and
    LSE = q.q / sqrt(d)."""
    T, H, W, d = 3, 4, 4, 8
    spec = MaskSpec("radius3d", T, H * W, grid_h=H, grid_w=W, r_t=0, r_s=0)
    q, k, v = _inputs(1, 2, spec.n, d, "f32", seed=3)
    o, lse = oracle.attention_rows(_np(q), _np(k), _np(v), spec)
    np.testing.assert_array_equal(o, v.double().reshape(-1, d).numpy())
    np.testing.assert_allclose(lse, ((q.double() * k.double()).sum(-1) / np.sqrt(d)).reshape(-1).numpy(),
                               rtol=1e-14, atol=0)


def test_constant_v():
    spec = MaskSpec("radial", 9, 5)
    q, k, _ = _inputs(1, 1, spec.n, 8, "f32", seed=4)
    v = torch.full_like(q, 0.375)
    o, _ = oracle.attention_rows(_np(q), _np(k), _np(v), spec)
    np.testing.assert_allclose(o, 0.375, rtol=0, atol=1e-15)


@pytest.mark.parametrize("spec", [MaskSpec("radial", 20, 6), MaskSpec("swa", 9, 4, window=3),
                                  MaskSpec("radius3d", 3, 12, grid_h=3, grid_w=4, r_t=1, r_s=1),
                                  MaskSpec("radial", 10, 40, granularity="block_any")],
                         ids=lambda s: f"{s.kind}-{s.granularity}")
def test_zero_query_is_uniform(spec):
    """Q = 0: every kept key scores 0, so LSE = ln(#kept keys) and O is the mean
    of V over the kept keys."""
    d = 8
    _, k, v = _inputs(1, 1, spec.n, d, "f32", seed=9)
    q = torch.zeros_like(k)
    o, lse = oracle.attention_rows(_np(q), _np(k), _np(v), spec)
    keep = (oracle.element_matrix(spec) if spec.granularity == "element" else _dilated(spec)).astype(bool)
    np.testing.assert_allclose(lse, np.log(keep.sum(1)), rtol=0, atol=1e-13)
    vv = v[0, 0].double().numpy()
    want = np.stack([vv[keep[i]].mean(0) for i in range(spec.n)])
    np.testing.assert_allclose(o, want, rtol=0, atol=1e-13)


def test_swa_window_one_is_per_frame_attention():
    f, s, d = 6, 7, 16
    spec = MaskSpec("swa", f, s, window=1)
    q, k, v = _inputs(1, 2, f * s, d, "bf16", seed=21)
    o, _ = oracle.attention_rows(_np(q), _np(k), _np(v), spec)
    qf, kf, vf = (x.double().reshape(1, 2, f, s, d) for x in (q, k, v))
    ref = F.scaled_dot_product_attention(qf, kf, vf).reshape(-1, d).numpy()
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)


def test_rows_are_convex_combinations_and_normalised():
    """softmax rows sum to 1 (exp(S - LSE) over kept keys) and O lies in the
    convex hull of the kept V rows, per column."""
    spec = MaskSpec("radial", 12, 8)
    d = 16
    q, k, v = _inputs(1, 1, spec.n, d, "f32", seed=13, scale=2.0)
    o, lse = oracle.attention_rows(_np(q), _np(k), _np(v), spec)
    keep = oracle.element_matrix(spec).astype(bool)
    s = (q[0, 0].double() @ k[0, 0].double().T).numpy() / np.sqrt(d)
    for i in range(spec.n):
        w = np.exp(s[i, keep[i]] - lse[i])
        assert abs(w.sum() - 1.0) < 1e-12
        vk = v[0, 0].double().numpy()[keep[i]]
        assert (o[i] >= vk.min(0) - 1e-12).all() and (o[i] <= vk.max(0) + 1e-12).all()


def test_bf16_widening_is_exact():
    """The bf16 path widens the stored bit patterns exactly: same result as the
    float32 path on the same (bf16-representable) values."""
    spec = MaskSpec("radial", 5, 9)
    qb, kb, vb = _inputs(1, 2, spec.n, 16, "bf16", seed=2)
    o1, l1 = oracle.attention_rows(_np(qb), _np(kb), _np(vb), spec)
    o2, l2 = oracle.attention_rows(_np(qb.float()), _np(kb.float()), _np(vb.float()), spec)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_row_subset_matches_full():
    spec = MaskSpec("radial", 8, 16, granularity="block_any")
    q, k, v = _inputs(2, 3, spec.n, 16, "bf16", seed=8)
    o, lse = oracle.attention_rows(_np(q), _np(k), _np(v), spec)
    rows = np.array([[1, 2, 5], [0, 0, 127], [1, 0, 0], [0, 1, 64]], dtype=np.int64)
    o2, lse2 = oracle.attention_rows(_np(q), _np(k), _np(v), spec, rows=rows)
    flat = (rows[:, 0] * 3 + rows[:, 1]) * spec.n + rows[:, 2]
    np.testing.assert_array_equal(o2, o[flat])
    np.testing.assert_array_equal(lse2, lse[flat])
