"""Pins of the oracle's masks against what the pages and the mathematics fix.

CPU only.  Each test names the passage it pins.
"""
import math
import os

import numpy as np
import pytest

import oracle
from oracle import MaskSpec, brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

# f > s sizes are the only ones that reach eq. 4's second case.
RADIAL_SIZES = [(1, 1), (2, 3), (5, 2), (7, 5), (8, 3), (9, 4), (16, 2), (64, 4), (33, 3),
                (3, 7), (12, 1), (40, 1), (17, 6)]


def radial(f, s, **kw):
    return MaskSpec("radial", f, s, **kw)


# ---------------------------------------------------------------- radial eq. 4

@pytest.mark.parametrize("f,s", RADIAL_SIZES)
def test_radial_matches_bruteforce(f, s):
    """Radial Attention section 3 eq. 4, evaluated literally on (i, j, k, l)."""
    np.testing.assert_array_equal(oracle.element_matrix(radial(f, s)), brute.radial(f, s))


def _pair(mat, s, i, j):
    return mat[i * s:(i + 1) * s, j * s:(j + 1) * s]


@pytest.mark.parametrize("f,s", [(12, 16), (9, 7), (6, 33)])
def test_radial_central_band_dense(f, s):
    """Section 3.1: the central band (same and adjacent frames) is 100% dense."""
    m = oracle.element_matrix(radial(f, s))
    for i in range(f):
        for j in range(max(0, i - 1), min(f, i + 2)):
            assert _pair(m, s, i, j).all()


@pytest.mark.parametrize("f,s", [(40, 16), (20, 24), (33, 5)])
def test_radial_diagonal_width(f, s):
    """Section 3.2: between frames i and j the kept entries form a diagonal band
    of width floor(s / 2^r), r = floor(log2(max(|i-j|, 1))), i.e. exactly the
    (k, l) with |k - l| < floor(s / 2^r), while that width is >= 1."""
    m = oracle.element_matrix(radial(f, s))
    k, l = np.meshgrid(np.arange(s), np.arange(s), indexing="ij")
    for i in range(f):
        for j in range(f):
            r = int(math.floor(math.log2(max(abs(i - j), 1))))
            width = s // (2 ** r)
            if width >= 1:
                np.testing.assert_array_equal(_pair(m, s, i, j), (abs(k - l) < width).astype(np.uint8))


@pytest.mark.parametrize("f,s", [(64, 4), (40, 3), (33, 1), (70, 5)])
def test_radial_sampled_diagonals(f, s):
    """Section 3.2: once the width falls below 1, only the sampled diagonal
    k = l of frame pairs with |i-j| a multiple of ceil(2^r / s) survives."""
    m = oracle.element_matrix(radial(f, s))
    eye = np.eye(s, dtype=np.uint8)
    seen_on, seen_off = 0, 0
    for i in range(f):
        for j in range(f):
            d = abs(i - j)
            r = int(math.floor(math.log2(max(d, 1))))
            if 2 ** r <= s:
                continue
            stride = -(-(2 ** r) // s)
            blk = _pair(m, s, i, j)
            if d % stride == 0:
                np.testing.assert_array_equal(blk, eye)
                seen_on += 1
            else:
                assert not blk.any()
                seen_off += 1
    assert seen_on > 0 and seen_off > 0


def _pair_count_closed_form(s, d):
    """Kept entries of an s x s frame pair at frame distance d: with width
    w = floor(s / 2^r) >= 1 the band |k-l| <= w-1 holds s + 2 * sum_{x=1}^{w-1} (s - x)
    = s(2m+1) - m(m+1) entries (m = w-1)."""
    r = int(math.floor(math.log2(max(d, 1))))
    w = s // (2 ** r)
    if w >= 1:
        mm = w - 1
        return s * (2 * mm + 1) - mm * (mm + 1)
    stride = -(-(2 ** r) // s)
    return s if d % stride == 0 else 0


@pytest.mark.parametrize("f,s", [(8, 64), (11, 13), (30, 4), (5, 100)])
def test_radial_count_closed_form(f, s):
    expect = sum(_pair_count_closed_form(s, abs(i - j)) for i in range(f) for j in range(f))
    assert oracle.kept_elements(radial(f, s)) == expect


def test_radial_f8_s64_zero_count():
    """The element-level radial workload (f=8, s=64): its mask zero count
    (kept entries) from the frame-pair closed form: 8 pairs at d=0 and 14 at
    d=1 are dense (4096 each), 22 at d in {2,3} keep 3040, 20 at d >= 4 keep 1744."""
    assert _pair_count_closed_form(64, 2) == 3040 and _pair_count_closed_form(64, 4) == 1744
    expect = 8 * 4096 + 14 * 4096 + 22 * 3040 + 20 * 1744
    assert expect == 191872
    assert oracle.kept_elements(radial(8, 64)) == expect


def test_radial_zero_count_bound():
    """Section 4, eq. 5-6: #zeros of M (kept entries) <= 4 s^2 f floor(log2 f),
    for f >= 2 (at f = 1 the right-hand side is 0 while s^2 entries are kept)."""
    for f in range(2, 41, 3):
        for s in (1, 2, 3, 5, 8, 16, 31, 64):
            kept = oracle.kept_elements(radial(f, s))
            assert kept <= 4 * s * s * f * int(math.floor(math.log2(f))), (f, s)
    # and the equality 4 s^2 f log2 f = 4 s n (log2 n - log2 s) for powers of two
    for f, s in ((8, 64), (128, 1024)):
        n = f * s
        assert 4 * s * s * f * math.log2(f) == pytest.approx(4 * s * n * (math.log2(n) - math.log2(s)))


def test_radial_s1_powers_of_two():
    """s = 1: case (a) keeps |i-j| <= 1, case (b) keeps |i-j| divisible by its
    own leading power of two, i.e. exactly the powers of two."""
    f = 200
    m = oracle.element_matrix(radial(f, 1))
    for i in range(f):
        for j in range(f):
            d = abs(i - j)
            assert m[i, j] == (1 if d == 0 or (d & (d - 1)) == 0 else 0), (i, j)


@pytest.mark.parametrize("f,s", [(1, 7), (2, 9), (2, 1)])
def test_radial_small_f_dense(f, s):
    assert oracle.element_matrix(radial(f, s)).all()


@pytest.mark.parametrize("f,s", [(9, 4), (40, 3), (13, 11)])
def test_radial_symmetric_with_diagonal(f, s):
    m = oracle.element_matrix(radial(f, s))
    np.testing.assert_array_equal(m, m.T)
    assert np.diag(m).all()


# ---------------------------------------------------------------- radius 3-D

@pytest.mark.parametrize("T,H,W,rt,rs", [(3, 4, 5, 1, 1), (4, 3, 3, 0, 1), (2, 5, 4, 1, 2),
                                         (5, 2, 6, 2, 0), (3, 3, 3, 3, 5), (1, 4, 4, 0, 0)])
def test_radius_matches_bruteforce(T, H, W, rt, rs):
    spec = MaskSpec("radius3d", T, H * W, grid_h=H, grid_w=W, r_t=rt, r_s=rs)
    np.testing.assert_array_equal(oracle.element_matrix(spec), brute.radius3d(T, H, W, rt, rs))


def test_radius_page_counts():
    """Interior-token neighbourhood sizes printed on the Token Radius page."""
    rows = [l.split() for l in open(os.path.join(GOLDEN, "radius_neighbourhood.txt"))
            if l.strip() and not l.startswith("#")]
    assert rows
    for rt, rs, count in rows:
        rt, rs, count = int(rt), int(rs), int(count)
        T, H, W = 5, 7, 7
        spec = MaskSpec("radius3d", T, H * W, grid_h=H, grid_w=W, r_t=rt, r_s=rs)
        q = (2 * H + 3) * W + 3  # t=2, h=3, w=3: interior
        seen = sum(oracle.keep(spec, q, t) for t in range(spec.n))
        assert seen == count


def test_radius_separable_count():
    """The kept count factorises over the axes: prod_axis sum_x (#x' with |x-x'| <= r).
    For the T8 x H16 x W16, r_t = 1, r_s = 4 workload it is 22 * 124 * 124."""
    def axis(N, r):
        return sum(min(x + r, N - 1) - max(x - r, 0) + 1 for x in range(N))
    assert axis(8, 1) == 22 and axis(16, 4) == 124
    spec = MaskSpec("radius3d", 8, 256, grid_h=16, grid_w=16, r_t=1, r_s=4)
    assert oracle.kept_elements(spec) == 22 * 124 * 124 == 338272
    spec = MaskSpec("radius3d", 5, 6 * 7, grid_h=6, grid_w=7, r_t=2, r_s=1)
    assert oracle.kept_elements(spec) == axis(5, 2) * axis(6, 1) * axis(7, 1)


def test_radius_corner_truncated():
    """Keys outside the grid do not exist (truncation, no padding, no wrap):
    the corner token sees (r_t+1)(r_s+1)^2 keys."""
    spec = MaskSpec("radius3d", 6, 64, grid_h=8, grid_w=8, r_t=2, r_s=3)
    assert sum(oracle.keep(spec, 0, t) for t in range(spec.n)) == 3 * 4 * 4


def test_token_grid_counts():
    """Patch arithmetic printed on the Token Radius pages; the T8xH16xW16 grid
    of the radius workload is the first line's 2048 tokens."""
    rows = [list(map(int, l.split())) for l in open(os.path.join(GOLDEN, "token_grid.txt"))
            if l.strip() and not l.startswith("#")]
    for fr, h, w, pt, ph, pw, tokens in rows:
        assert (fr // pt) * (h // ph) * (w // pw) == tokens
    import workloads
    wl = workloads.WORKLOADS["radius3d_t8_h16_w16"]
    assert (wl.f, wl.grid_h, wl.grid_w) == (16 // 2, 256 // 16, 256 // 16) and wl.n == rows[0][-1]


# ---------------------------------------------------------------- sliding window

@pytest.mark.parametrize("f,s,W", [(7, 3, 2), (10, 2, 4), (5, 4, 1), (6, 2, 9), (12, 1, 16)])
def test_swa_matches_bruteforce(f, s, W):
    spec = MaskSpec("swa", f, s, window=W)
    np.testing.assert_array_equal(oracle.element_matrix(spec), brute.swa_causal(f, s, W))


def test_swa_count_closed_form():
    """Frame i sees min(i+1, W) frames: kept = s^2 * sum_i min(i+1, W).
    The f=64, s=256, W=16 workload: 256^2 * 904."""
    assert sum(min(i + 1, 16) for i in range(64)) == 904
    assert oracle.kept_elements(MaskSpec("swa", 64, 256, window=16)) == 256 * 256 * 904
    f, s, W = 13, 5, 4
    assert oracle.kept_elements(MaskSpec("swa", f, s, window=W)) == s * s * sum(min(i + 1, W) for i in range(f))


def test_swa_special_cases():
    f, s = 9, 3
    # W = 1: every frame sees only itself (block diagonal).
    m1 = oracle.element_matrix(MaskSpec("swa", f, s, window=1))
    np.testing.assert_array_equal(m1, np.kron(np.eye(f, dtype=np.uint8), np.ones((s, s), np.uint8)))
    # W >= f: plain frame-level causal mask (block lower triangular).
    mf = oracle.element_matrix(MaskSpec("swa", f, s, window=f))
    np.testing.assert_array_equal(mf, np.kron(np.tril(np.ones((f, f), np.uint8)), np.ones((s, s), np.uint8)))
    # never a future frame (causal, section 2.1)
    m = oracle.element_matrix(MaskSpec("swa", f, s, window=4))
    fi = np.arange(f * s) // s
    assert not (m.astype(bool) & (fi[None, :] > fi[:, None])).any()


# ---------------------------------------------------------------- block granularity

@pytest.mark.parametrize("spec", [
    MaskSpec("radial", 9, 4, block=8), MaskSpec("radial", 40, 3, block=16),
    MaskSpec("radial", 7, 5, block=4), MaskSpec("radius3d", 3, 20, grid_h=4, grid_w=5, r_t=1, r_s=1, block=8),
    MaskSpec("swa", 10, 3, window=3, block=7),
])
def test_block_counts_match_bruteforce(spec):
    elem = oracle.element_matrix(spec)
    counts = oracle.block_counts(spec, threads=3)
    nb = spec.nb
    pad = np.zeros((nb * spec.block, nb * spec.block), dtype=np.int64)
    pad[:spec.n, :spec.n] = elem
    np.testing.assert_array_equal(counts, pad.reshape(nb, spec.block, nb, spec.block).sum(axis=(1, 3)))
    _, keep = brute.dilate_any(elem, spec.block)
    np.testing.assert_array_equal(counts > 0, keep.astype(bool))
    assert counts.sum() == oracle.kept_elements(spec)


def test_block_bits128():
    spec = MaskSpec("radial", 12, 40)  # n = 480: 4 blocks, the last one ragged
    elem = oracle.element_matrix(spec)
    for qb in range(spec.nb):
        for kb in range(spec.nb):
            bits = oracle.block_bits128(spec, qb, kb)
            unpacked = np.zeros((128, 128), dtype=np.uint8)
            for c in range(128):
                unpacked[:, c] = (bits[:, c // 32] >> np.uint32(c % 32)) & 1
            want = np.zeros((128, 128), dtype=np.uint8)
            tile = elem[qb * 128:(qb + 1) * 128, kb * 128:(kb + 1) * 128]
            want[:tile.shape[0], :tile.shape[1]] = tile
            np.testing.assert_array_equal(unpacked, want)


def test_block_any_contains_element_mask():
    """Block granularity only adds entries: no element kept by eq. 4 is dropped."""
    spec = MaskSpec("radial", 20, 24, block=128)
    elem = oracle.element_matrix(spec)
    keep = oracle.block_counts(spec) > 0
    dil = np.kron(keep.astype(np.uint8), np.ones((128, 128), np.uint8))[:spec.n, :spec.n]
    assert not (elem.astype(bool) & ~dil.astype(bool)).any()


def test_block_counts_rows_subset():
    spec = MaskSpec("radial", 11, 40, block=128)
    full = oracle.block_counts(spec)
    rows = np.array([3, 0, 2], dtype=np.int64)
    np.testing.assert_array_equal(oracle.block_counts_rows(spec, rows, threads=2), full[rows])


# ---------------------------------------------------------------- sink frames

@pytest.mark.parametrize("spec,base", [
    (MaskSpec("radial", 9, 4, sink_frames=1), lambda: brute.radial(9, 4)),
    (MaskSpec("radial", 33, 3, sink_frames=2), lambda: brute.radial(33, 3)),
    (MaskSpec("radius3d", 4, 12, grid_h=3, grid_w=4, r_t=1, r_s=1, sink_frames=1),
     lambda: brute.radius3d(4, 3, 4, 1, 1)),
    (MaskSpec("swa", 7, 5, window=2, sink_frames=1), lambda: brute.swa_causal(7, 5, 2)),
], ids=["radial", "radial-f33-sink2", "radius", "swa"])
def test_sink_matches_bruteforce(spec, base):
    """Sink reading of Radial Attention section 4's count: the family's mask
    plus every key of the first sink_frames frames, for every query."""
    np.testing.assert_array_equal(oracle.element_matrix(spec), brute.with_sink(base(), spec.s, spec.sink_frames))


def test_sink_degenerate():
    """sink_frames = 0 changes nothing; sink_frames >= f keeps everything."""
    np.testing.assert_array_equal(oracle.element_matrix(radial(10, 6, sink_frames=0)), brute.radial(10, 6))
    assert oracle.element_matrix(radial(10, 6, sink_frames=10)).all()
    assert oracle.element_matrix(MaskSpec("swa", 5, 4, window=1, sink_frames=7)).all()


@pytest.mark.parametrize("f,s", [(8, 16), (20, 5), (3, 9)])
def test_sink_central_band_count(f, s):
    """Section 4 counts "central band + sink" as 4 s^2 f.  With one sink frame
    the frame pairs with |i - j| <= 1 or j = 0 are all kept: the band has
    3f - 2 frame pairs, the sink adds the f - 2 pairs (i >= 2, j = 0) it does
    not already hold, so they hold exactly s^2 (4f - 4) <= 4 s^2 f entries."""
    m = oracle.element_matrix(radial(f, s, sink_frames=1)).astype(bool)
    fi = np.arange(f * s) // s
    sel = (np.abs(fi[:, None] - fi[None, :]) <= 1) | (fi[None, :] == 0)
    assert m[sel].all()
    assert int(sel.sum()) == s * s * (4 * f - 4) <= 4 * s * s * f


# ---------------------------------------------------------------- eq. 4 on block indices

@pytest.mark.parametrize("f,s,block,sink", [(9, 8, 4, 0), (33, 12, 4, 0), (17, 6, 2, 1), (64, 4, 4, 0),
                                            (5, 16, 8, 2)])
def test_block_eq4_matches_bruteforce(f, s, block, sink):
    """Second block reading of section 6: eq. 4 on (query block, key block)
    with s / block blocks per frame (brute force on the block grid)."""
    spec = MaskSpec("radial", f, s, granularity="block_eq4", block=block, sink_frames=sink)
    np.testing.assert_array_equal(oracle.block_keep(spec), brute.radial_blocks(f, s, block, sink))


def test_block_eq4_headline_count():
    """n = 131072 (f = 128, s = 1024, 128 x 128 blocks, 8 blocks per frame):
    the frame-pair closed form at s = 8 gives 111,552 kept blocks of
    1,048,576 (89.4% sparse)."""
    expect = sum(_pair_count_closed_form(8, abs(i - j)) for i in range(128) for j in range(128))
    assert expect == 111552
    spec = MaskSpec("radial", 128, 1024, granularity="block_eq4")
    assert int(oracle.block_keep(spec).sum()) == expect


def test_block_keep_matches_counts():
    """block_keep at element / block_any granularity = non-empty blocks."""
    for spec in (MaskSpec("radial", 12, 40), MaskSpec("radial", 7, 100, granularity="block_any")):
        np.testing.assert_array_equal(oracle.block_keep(spec), oracle.block_counts(spec) > 0)


def test_row_counts_match_matrices():
    """Per-row attended-key counts equal the row sums of the element matrix,
    or of the brute-force block matrix expanded to tokens."""
    for spec in (MaskSpec("radial", 9, 7), MaskSpec("swa", 6, 5, window=2, sink_frames=1)):
        rows = np.arange(spec.n)
        np.testing.assert_array_equal(oracle.row_counts(spec, rows), oracle.element_matrix(spec).sum(1))
    spec = MaskSpec("radial", 10, 8, granularity="block_eq4", block=4)
    keep = np.kron(brute.radial_blocks(10, 8, 4), np.ones((4, 4), np.uint8))
    np.testing.assert_array_equal(oracle.row_counts(spec, np.arange(spec.n)), keep.sum(1))
    spec = MaskSpec("radial", 5, 80, granularity="block_any")
    bk = oracle.block_counts(spec) > 0
    dil = np.kron(bk.astype(np.uint8), np.ones((128, 128), np.uint8))[:spec.n, :spec.n]
    np.testing.assert_array_equal(oracle.row_counts(spec, np.arange(spec.n), block_keep=bk), dil.sum(1))
