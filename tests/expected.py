"""Expected compiled-mask arrays derived from the oracle's block counts.

Test helper (not collected).  Block classes follow the library contract
(include/tra.h): a block is kept when any element is kept; it carries an
element bitmask ("partial") when it reaches past n or, at element
granularity, when not every in-range element is kept.
"""
from __future__ import annotations

import numpy as np

import oracle

BLOCK = 128


def block_classes(spec: oracle.MaskSpec, counts: np.ndarray | None = None):
    """(counts, classes) with classes 0 = empty, 1 = full, 2 = partial."""
    assert spec.block == BLOCK
    if counts is None:
        counts = oracle.block_counts(spec)
    n, nb = spec.n, spec.nb
    rows_in = np.minimum(BLOCK, n - np.arange(nb) * BLOCK)
    cols_in = rows_in.copy()
    area = rows_in[:, None] * cols_in[None, :]
    cls = np.zeros((nb, nb), dtype=np.uint8)
    kept = counts > 0
    ragged_cols = np.broadcast_to(cols_in[None, :] < BLOCK, cls.shape)
    if spec.granularity == "block_eq4":
        kept = oracle.block_keep(spec) > 0  # whole blocks; n is a multiple of 128
    if spec.granularity == "element":
        partial = kept & (ragged_cols | (counts != area))
    else:
        partial = kept & ragged_cols
    cls[kept] = 1
    cls[partial] = 2
    return counts, cls


def csr(cls: np.ndarray):
    nb = cls.shape[0]
    row_ptr = np.zeros(nb + 1, dtype=np.int32)
    cols, eidx = [], []
    npart = 0
    for r in range(nb):
        ks = np.nonzero(cls[r])[0]
        row_ptr[r + 1] = row_ptr[r] + len(ks)
        for kb in ks:
            cols.append(kb)
            if cls[r, kb] == 2:
                eidx.append(npart)
                npart += 1
            else:
                eidx.append(-1)
    return row_ptr, np.array(cols, dtype=np.int32), np.array(eidx, dtype=np.int32)


def pair_schedule(keep: np.ndarray, s: int):
    """(items, tile loads) of the library's pair schedule over the rows of
    the boolean block matrix `keep`, by its stated rule: rows are taken in
    order; an unpaired row r takes, among the unpaired rows r + 1 and
    r + s / 128 (the latter when s is a multiple of 128 above 128), the one
    whose kept-block set has the larger Jaccard overlap with r's, the first
    on ties, if that overlap is above 0 (two empty sets count as 1).  A pair
    loads the union of its two rows' blocks."""
    nr = keep.shape[0]
    offs = [1] + ([s // BLOCK] if s % BLOCK == 0 and s // BLOCK > 1 else [])
    used = np.zeros(nr, dtype=bool)
    items, loads = 0, 0
    for r in range(nr):
        if used[r]:
            continue
        best, bj = -1, 0.0
        for off in offs:
            r2 = r + off
            if r2 >= nr or used[r2]:
                continue
            inter = int((keep[r] & keep[r2]).sum())
            uni = int((keep[r] | keep[r2]).sum())
            j = inter / uni if uni else 1.0
            if j > bj:
                bj, best = j, r2
        used[r] = True
        items += 1
        if best >= 0:
            used[best] = True
            loads += int((keep[r] | keep[best]).sum())
        else:
            loads += int(keep[r].sum())
    return items, loads


def bitmap(cls: np.ndarray):
    nb = cls.shape[0]
    words = (nb + 31) // 32
    out = np.zeros((nb, words), dtype=np.uint32)
    for r in range(nb):
        for kb in np.nonzero(cls[r])[0]:
            out[r, kb // 32] |= np.uint32(1) << np.uint32(kb % 32)
    return out


def partial_bits(spec: oracle.MaskSpec, qb: int, kb: int) -> np.ndarray:
    """128 x 4 words of a partial block: the element predicate at element
    granularity, every in-range key at block granularity."""
    if spec.granularity == "element":
        return oracle.block_bits128(spec, qb, kb)
    out = np.zeros((BLOCK, 4), dtype=np.uint32)
    rows = min(BLOCK, spec.n - qb * BLOCK)
    cols = min(BLOCK, spec.n - kb * BLOCK)
    for c in range(cols):
        out[:rows, c // 32] |= np.uint32(1) << np.uint32(c % 32)
    return out


def kept_keys_per_row(spec: oracle.MaskSpec, cls: np.ndarray, counts_elem_rows=None) -> np.ndarray:
    """Keys attended by every query row at block granularity (kept blocks,
    cut at n)."""
    assert spec.granularity in ("block_any", "block_eq4")
    nb, n = spec.nb, spec.n
    cols_in = np.minimum(BLOCK, n - np.arange(nb) * BLOCK)
    per_block_row = (cls > 0).astype(np.int64) @ cols_in
    return np.repeat(per_block_row, BLOCK)[:n]


_COUNT_CACHE: dict = {}


def cached_block_counts(spec: oracle.MaskSpec) -> np.ndarray:
    """oracle.block_counts memoised per element predicate (the largest masks
    take seconds); the counts do not depend on the granularity."""
    key = (spec.kind, spec.f, spec.s, spec.block, spec.grid_h, spec.grid_w,
           spec.r_t, spec.r_s, spec.window, spec.sink_frames)
    if key not in _COUNT_CACHE:
        _COUNT_CACHE[key] = oracle.block_counts(spec)
    return _COUNT_CACHE[key]


def sample_rows(n: int, B: int, H: int, heads_per_batch: int, blocks: int, seed: int,
                heavy_first=None) -> np.ndarray:
    """(b, h, q) triples: per sampled (b, h) the first and last query block,
    `blocks` random blocks (plus the first entries of `heavy_first`), and in
    each block rows 0, 1, 63, 64, 127 and three random rows (cut at n)."""
    rng = np.random.default_rng(seed)
    nb = (n + BLOCK - 1) // BLOCK
    out = []
    for b in range(B):
        hs = sorted(set([0, H - 1]) | set(rng.choice(H, size=min(H, heads_per_batch), replace=False).tolist()))
        for h in hs:
            qbs = {0, nb - 1} | set(rng.choice(nb, size=min(nb, blocks), replace=False).tolist())
            if heavy_first is not None:
                qbs |= set(int(x) for x in heavy_first[:2])
            for qb in sorted(qbs):
                rs = {0, 1, 63, 64, 127} | set(rng.integers(0, BLOCK, size=3).tolist())
                for r in sorted(rs):
                    q = qb * BLOCK + r
                    if q < n:
                        out.append((b, h, q))
    return np.array(out, dtype=np.int64)
