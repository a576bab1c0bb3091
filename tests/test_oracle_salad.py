"""Pins of the oracle's SALAD gate and output combination.

CPU only.  The gate (page "SALAD", section 2.2) is the mean over tokens of a
sigmoid of a linear map; the output adds the gated, projected linear branch
to the sparse branch in the merged-head channel space (section 2.1-2.2).
Pins are closed forms that a dropped term, a wrong sign, a transposed weight
or a wrong head/channel mapping would fail.
"""
import math

import numpy as np

import oracle


def _rng(seed):
    return np.random.default_rng(seed)


def _bf16(a):
    """float32 array -> uint16 bfloat16 bits (round to nearest even)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def _widen(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32)


def test_gate_zero_weight_is_sigmoid_of_bias():
    """w = 0: every token's pre-activation is the bias, so g = sigmoid(bias);
    bias = ln 3 gives exactly 3/4 (a sign slip would give 1/4, a sum instead
    of a mean 3N/4)."""
    x = _rng(1).standard_normal((3, 17, 24)).astype(np.float32)
    w = np.zeros(24, np.float32)
    g = oracle.salad_gate(x, w, bias=math.log(3.0))
    np.testing.assert_allclose(g, 0.75, rtol=0, atol=1e-15)


def test_gate_one_hot_weight_reads_one_channel_per_sample():
    """w = e_c: g[b] = mean_n sigmoid(x[b, n, c]); x constant per sample in
    that channel gives sigmoid of that constant, distinct per sample."""
    B, N, C, c = 4, 9, 16, 5
    x = _rng(2).standard_normal((B, N, C)).astype(np.float32)
    vals = np.array([-2.0, -0.5, 0.0, 1.25], np.float32)
    x[:, :, c] = vals[:, None]
    w = np.zeros(C, np.float32)
    w[c] = 1.0
    g = oracle.salad_gate(x, w, bias=0.0)
    np.testing.assert_allclose(g, 1.0 / (1.0 + np.exp(-vals.astype(np.float64))), rtol=0, atol=1e-15)
    assert g[2] == 0.5


def test_gate_negation_symmetry():
    """sigmoid(-z) = 1 - sigmoid(z): negating w and the bias gives 1 - g."""
    x = _rng(3).standard_normal((2, 50, 32)).astype(np.float32)
    w = (_rng(4).standard_normal(32) / math.sqrt(32)).astype(np.float32)
    g = oracle.salad_gate(x, w, bias=0.3)
    gn = oracle.salad_gate(x, -w, bias=-0.3)
    np.testing.assert_allclose(gn, 1.0 - g, rtol=0, atol=1e-14)
    assert np.all((g > 0) & (g < 1))


def test_gate_bf16_inputs_widen_exactly():
    """bf16 inputs give the gate of their exact float32 values."""
    x = _rng(5).standard_normal((2, 20, 16)).astype(np.float32)
    w = _rng(6).standard_normal(16).astype(np.float32)
    xb, wb = _bf16(x), _bf16(w)
    np.testing.assert_array_equal(oracle.salad_gate(xb, wb, 0.1), oracle.salad_gate(_widen(xb), _widen(wb), 0.1))


def _perm_weight(C, perm):
    """W with W[c', perm[c']] = 1: out channel c' reads input channel perm[c']."""
    W = np.zeros((C, C), np.float32)
    W[np.arange(C), perm] = 1.0
    return W


def test_output_permutation_weight_moves_channels_across_heads():
    """W a permutation matrix (not symmetric, crossing heads): the projection
    of token n's channels is the permuted channel vector, so
    out[c'] = O_s[c'] + g * O_l[perm[c']].  A transposed W (the inverse
    permutation) or a wrong head/channel split fails this."""
    B, H, N, d = 2, 3, 5, 4
    C = H * d
    rng = _rng(7)
    os_ = rng.standard_normal((B, H, N, d)).astype(np.float32)
    ol = rng.standard_normal((B, H, N, d)).astype(np.float32)
    perm = rng.permutation(C)
    assert np.any(perm[perm] != np.arange(C))
    g = np.array([0.25, 0.75])
    out = oracle.salad_output_rows(os_, ol, _perm_weight(C, perm), None, g)
    merged = lambda a: a.astype(np.float64).transpose(0, 2, 1, 3).reshape(B * N, C)
    want = merged(os_) + np.repeat(g, N)[:, None] * merged(ol)[:, perm]
    np.testing.assert_allclose(out, want, rtol=0, atol=1e-15)


def test_output_zero_gate_is_sparse_branch():
    B, H, N, d = 1, 2, 6, 8
    C = H * d
    rng = _rng(8)
    os_, ol = (rng.standard_normal((B, H, N, d)).astype(np.float32) for _ in range(2))
    W = rng.standard_normal((C, C)).astype(np.float32)
    out = oracle.salad_output_rows(os_, ol, W, rng.standard_normal(C), np.zeros(1))
    np.testing.assert_array_equal(out, os_.astype(np.float64).transpose(0, 2, 1, 3).reshape(N, C))


def test_output_bias_only():
    """O_l = 0: out = O_s + g * bias (the bias is added before the gate)."""
    B, H, N, d = 2, 2, 3, 4
    C = H * d
    rng = _rng(9)
    os_ = rng.standard_normal((B, H, N, d)).astype(np.float32)
    ol = np.zeros_like(os_)
    W = rng.standard_normal((C, C)).astype(np.float32)
    bias = rng.standard_normal(C)
    g = np.array([0.5, 2.0])
    out = oracle.salad_output_rows(os_, ol, W, bias, g)
    want = os_.astype(np.float64).transpose(0, 2, 1, 3).reshape(B * N, C) + np.repeat(g, N)[:, None] * bias
    np.testing.assert_allclose(out, want, rtol=0, atol=1e-15)


def test_output_single_channel_weight_column():
    """O_l = e_c at one token (all other channels 0): the projection is
    column c of W, i.e. out[c'] = O_s[c'] + g * (W[c', c] + bias[c'])."""
    B, H, N, d = 1, 2, 4, 4
    C = H * d
    rng = _rng(10)
    os_ = rng.standard_normal((B, H, N, d)).astype(np.float32)
    ol = np.zeros_like(os_)
    c, n = 6, 2
    ol[0, c // d, n, c % d] = 1.0
    W = rng.standard_normal((C, C)).astype(np.float32)
    bias = rng.standard_normal(C)
    out = oracle.salad_output_rows(os_, ol, W, bias, np.array([0.4]), rows=np.array([[0, n]]))
    want = os_[0, :, n, :].astype(np.float64).reshape(C) + 0.4 * (W[:, c].astype(np.float64) + bias)
    np.testing.assert_allclose(out[0], want, rtol=0, atol=1e-14)


def test_output_row_subset_matches_full():
    B, H, N, d = 2, 2, 7, 8
    C = H * d
    rng = _rng(11)
    os_, ol = (_bf16(rng.standard_normal((B, H, N, d))) for _ in range(2))
    W = _bf16(rng.standard_normal((C, C)) / math.sqrt(C))
    g = np.array([0.3, 0.6])
    full = oracle.salad_output_rows(os_, ol, W, None, g)
    rows = np.array([[1, 6], [0, 0], [1, 2]])
    sub = oracle.salad_output_rows(os_, ol, W, None, g, rows=rows)
    np.testing.assert_array_equal(sub, full[rows[:, 0] * N + rows[:, 1]])
