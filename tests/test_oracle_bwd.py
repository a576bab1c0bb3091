"""Pins of the oracle's gradients of eq. 2 (the backward pass).

CPU only.  Reference points: torch autograd through scaled_dot_product_attention
in float64 (a library routine), central finite differences of
L = sum(O * dO), and identities of the softmax Jacobian.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import MaskSpec, brute


def _inputs(B, H, n, d, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    xs = [torch.randn(B, H, n, d, generator=g) for _ in range(4)]
    if dtype == "bf16":
        xs = [x.to(torch.bfloat16) for x in xs]
    return xs


def _np(x):
    if x.dtype == torch.bfloat16:
        return x.contiguous().view(torch.int16).numpy().view(np.uint16)
    return x.contiguous().numpy()


def _keep(spec):
    if spec.granularity == "element":
        return oracle.element_matrix(spec)
    if spec.granularity == "block_eq4":
        keep = brute.radial_blocks(spec.f, spec.s, spec.block, spec.sink_frames)
        return np.kron(keep, np.ones((spec.block, spec.block), np.uint8))
    bk = oracle.block_counts(spec) > 0
    return np.kron(bk.astype(np.uint8), np.ones((spec.block, spec.block), np.uint8))[:spec.n, :spec.n]


SPECS = [
    MaskSpec("radial", 6, 16),
    MaskSpec("radial", 24, 3),
    MaskSpec("radius3d", 4, 20, grid_h=4, grid_w=5, r_t=1, r_s=1),
    MaskSpec("swa", 8, 8, window=3),
    MaskSpec("dense", 3, 20),
    MaskSpec("radial", 5, 80, granularity="block_any"),
    MaskSpec("radial", 12, 16, granularity="block_eq4", block=8),
    MaskSpec("radial", 6, 16, sink_frames=1),
]


@pytest.mark.parametrize("spec", SPECS, ids=lambda s: f"{s.kind}-{s.granularity}-{s.f}x{s.s}-sink{s.sink_frames}")
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_grads_match_autograd_float64(spec, dtype):
    """dQ, dK, dV equal torch autograd of SDPA (float64, boolean mask)."""
    B, H, d = 1, 2, 8
    q, k, v, do = _inputs(B, H, spec.n, d, dtype, seed=21)
    dq, dk, dv = oracle.attention_bwd_rows(_np(q), _np(k), _np(v), _np(do), spec, threads=4)
    mask = torch.from_numpy(_keep(spec).astype(bool))
    q64, k64, v64 = (x.double().requires_grad_() for x in (q, k, v))
    out = F.scaled_dot_product_attention(q64, k64, v64, attn_mask=mask)
    out.backward(do.double())
    for got, ref in ((dq, q64.grad), (dk, k64.grad), (dv, v64.grad)):
        np.testing.assert_allclose(got, ref.reshape(-1, d).numpy(), rtol=0, atol=1e-11)


def test_grads_match_finite_differences():
    """Central differences of L = sum(O * dO) with respect to single entries
    of Q, K and V (fp64 forward of the oracle)."""
    spec = MaskSpec("radial", 6, 3)  # n = 18, eq. 4 case (b) reached
    rng = np.random.default_rng(3)
    n, d = spec.n, 4
    q, k, v, do = (rng.standard_normal((1, 1, n, d)).astype(np.float32) for _ in range(4))
    dq, dk, dv = oracle.attention_bwd_rows(q, k, v, do, spec, threads=2)

    def loss(qq, kk, vv):
        o, _ = oracle.attention_rows(qq, kk, vv, spec, threads=2)
        return float((o * do.reshape(-1, d).astype(np.float64)).sum())

    h = 1e-2  # fp32 inputs: the step must be exactly representable
    for (arr, grad) in ((q, dq), (k, dk), (v, dv)):
        for (i, x) in ((0, 0), (7, 2), (17, 3), (11, 1)):
            plus, minus = arr.copy(), arr.copy()
            plus[0, 0, i, x] += np.float32(h)
            minus[0, 0, i, x] -= np.float32(h)
            step = float(plus[0, 0, i, x]) - float(minus[0, 0, i, x])
            args_p = [plus if a is arr else a for a in (q, k, v)]
            args_m = [minus if a is arr else a for a in (q, k, v)]
            fd = (loss(*args_p) - loss(*args_m)) / step
            assert abs(fd - grad[i, x]) <= 1e-4 * max(1.0, abs(fd)), (i, x, fd, grad[i, x])


@pytest.mark.parametrize("spec", [MaskSpec("radial", 10, 12), MaskSpec("swa", 9, 7, window=2),
                                  MaskSpec("radial", 7, 100, granularity="block_any")])
def test_softmax_jacobian_identities(spec):
    """Every row's probabilities sum to 1, so sum_t dV[t] = sum_q dO[q]; the
    rows of dS sum to 0, so sum_t dK[t] = 0."""
    q, k, v, do = _inputs(1, 1, spec.n, 16, "f32", seed=8)
    dq, dk, dv = oracle.attention_bwd_rows(_np(q), _np(k), _np(v), _np(do), spec, threads=4)
    np.testing.assert_allclose(dv.sum(0), do.double().reshape(-1, 16).sum(0).numpy(), rtol=0, atol=1e-10)
    np.testing.assert_allclose(dk.sum(0), np.zeros(16), rtol=0, atol=1e-10)


def test_single_key_rows():
    """r_t = r_s = 0: each query keeps only itself, P = 1, so dV = dO and
    dQ = dK = 0 exactly."""
    spec = MaskSpec("radius3d", 2, 12, grid_h=3, grid_w=4, r_t=0, r_s=0)
    q, k, v, do = _inputs(1, 2, spec.n, 8, "f32", seed=9)
    dq, dk, dv = oracle.attention_bwd_rows(_np(q), _np(k), _np(v), _np(do), spec, threads=2)
    np.testing.assert_array_equal(dv, do.double().reshape(-1, 8).numpy())
    assert not dq.any() and not dk.any()


def test_row_subsets():
    """Selected rows equal the same rows of the full computation."""
    spec = MaskSpec("radial", 8, 16, granularity="block_any", block=16)
    q, k, v, do = _inputs(2, 2, spec.n, 8, "bf16", seed=10)
    arrs = [_np(x) for x in (q, k, v, do)]
    dq, dk, dv = oracle.attention_bwd_rows(*arrs, spec, threads=3)
    qr = np.array([[1, 0, 5], [0, 1, 127], [1, 1, 64]], np.int64)
    kr = np.array([[0, 1, 3], [1, 0, 100], [0, 1, 77]], np.int64)
    sq, sk, sv = oracle.attention_bwd_rows(*arrs, spec, q_rows=qr, k_rows=kr, threads=2)
    idx = lambda r: (r[:, 0] * 2 + r[:, 1]) * spec.n + r[:, 2]
    np.testing.assert_array_equal(sq, dq[idx(qr)])
    np.testing.assert_allclose(sk, dk[idx(kr)], rtol=0, atol=1e-13)
    np.testing.assert_allclose(sv, dv[idx(kr)], rtol=0, atol=1e-13)
