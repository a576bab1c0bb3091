"""The per-row LSE tolerance, checked with the oracle alone.

The tolerance (tests/tolerance.py) is meant to make the plain LSE comparison
fail when one 128-key block is dropped from a row or added to it.  These
tests drop one kept block from the oracle's own block mask (fp64, bf16
inputs of the workloads' distribution) and check that the LSE of the rows
that kept it moves past the tolerance, and that the tolerance takes the
values its derivation states on the workloads.
"""
import math

import numpy as np
import pytest

import oracle
import workloads
from tests import expected
from tests.tolerance import TOL_LSE, lse_tol


def _drop_block_shift(spec, w, qb, kb_pick, seed):
    q, k, v = workloads.make_qkv(w, device="cpu")
    arr = [workloads.to_oracle_array(x) for x in (q, k, v)]
    keep = expected.cached_block_counts(spec) > 0
    kept = np.nonzero(keep[qb])[0]
    kb = kept[kb_pick % len(kept)]
    rows = np.array([(0, 0, qb * 128 + r) for r in range(128)], dtype=np.int64)
    _, lse_all = oracle.attention_rows(*arr, spec, rows=rows, block_keep=keep)
    dropped = keep.copy()
    dropped[qb, kb] = False
    _, lse_drop = oracle.attention_rows(*arr, spec, rows=rows, block_keep=dropped)
    tol = lse_tol(spec, w.dtype, rows[:, 2], block_keep=keep)
    return np.abs(lse_all - lse_drop), tol


@pytest.mark.parametrize("qb,pick", [(37, 0), (37, 5), (80, 11), (119, 3)])
def test_one_dropped_block_exceeds_the_tolerance(qb, pick):
    """Radial eq. 4 at 128 x 128 blocks (any-element), f = 20 frames of 1536
    tokens, bf16 inputs scaled by 1/sqrt(2) (the f = 20 workload, one head):
    dropping one kept key block moves the LSE of most of its 128 rows by more
    than the tolerance, and of none by less than a tenth of it."""
    w = workloads.WORKLOADS["radial_f20_s1536_block"].replace(H=1)
    spec = oracle.MaskSpec(w.kind, w.f, w.s, granularity=w.granularity)
    shift, tol = _drop_block_shift(spec, w, qb, pick, seed=w.seed)
    frac = float((shift > tol).mean())
    print(f"qb={qb}: shift median {np.median(shift):.2e} min {shift.min():.2e}, tol {tol.min():.2e}..{tol.max():.2e}, "
          f"rows past tol {frac:.2f}")
    assert frac >= 0.75
    assert np.all(shift > 0.1 * tol)


def test_dropped_block_at_d64_window():
    """Frame sliding window (W = 16 frames of 256 tokens, d = 64, bf16): the
    same holds for a row block that keeps 16 x 2 key blocks."""
    w = workloads.WORKLOADS["swa_f64_s256_w16"].replace(f=20, H=1)
    spec = oracle.MaskSpec(w.kind, w.f, w.s, window=w.window)
    # element granularity: drop a block through a block_any twin of the mask
    spec_b = oracle.MaskSpec(w.kind, w.f, w.s, granularity="block_any", window=w.window)
    shift, tol = _drop_block_shift(spec_b, w, 36, 7, seed=w.seed)
    assert float((shift > tol).mean()) >= 0.75
    # the window mask is whole 128 x 128 blocks, so both readings keep the same keys
    rows = np.arange(36 * 128, 37 * 128)
    assert np.array_equal(oracle.row_counts(spec, rows), oracle.row_counts(spec_b, rows))


def test_tolerance_values_on_the_workloads():
    """tol = min(T, 0.5 ln(1 + 128 / K)): T binds at the n = 131072 radial
    workload (K = 35,584 .. 55,680 keys per row, so the block term is
    1.15e-3 .. 1.8e-3), the block term binds on the radius workload (K <= 243),
    and fp32 rows get 1e-4."""
    spec = oracle.MaskSpec("radial", 128, 1024, granularity="block_any")
    keep = expected.cached_block_counts(spec) > 0
    per_row_blocks = keep.sum(axis=1)
    assert per_row_blocks.min() == 278 and per_row_blocks.max() == 435
    rows = np.concatenate([np.arange(128), np.arange(64 * 1024, 64 * 1024 + 128)])
    t = lse_tol(spec, "bf16", rows, block_keep=keep)
    assert np.all(t == TOL_LSE["bf16"])
    term = 0.5 * np.log1p(128.0 / (128 * per_row_blocks))
    assert 1.14e-3 < term.min() < 1.16e-3 and 1.79e-3 < term.max() < 1.81e-3

    r = oracle.MaskSpec("radius3d", 8, 256, grid_h=16, grid_w=16, r_t=1, r_s=4)
    allq = np.arange(r.n)
    K = oracle.row_counts(r, allq)
    assert K.max() == 3 * 9 * 9 and K.min() == 2 * 5 * 5
    t = lse_tol(r, "bf16", allq)
    assert np.allclose(t, np.minimum(1e-3, 0.5 * np.log1p(128.0 / K)))
    assert t.max() == 1e-3 and math.isclose(t.max(), min(1e-3, 0.5 * math.log1p(128 / 50)))

    c1 = oracle.MaskSpec("radial", 8, 64)
    assert np.all(lse_tol(c1, "f32", np.arange(c1.n)) == 1e-4)
