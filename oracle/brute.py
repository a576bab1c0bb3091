"""Pure-Python brute-force enumeration of the three mask families.

TEST INFRASTRUCTURE ONLY (imported by tests).  Small sizes only.

It is written independently of ``oracle.c`` and in a different style, so that
agreement pins the C oracle's integer rewrites:

  * the radial mask walks the 4-D index space (i, j, k, l) of Radial Attention
    section 3 eq. 4 and evaluates the printed conditions with real-valued
    log2, floor, ceil and the real division s / 2^r (exact for the small
    integers used here), then scatters each entry to token indices
    (i * s + k, j * s + l);
  * the radius neighbourhood enumerates grid offsets (dt, dh, dw) around each
    query on the (T, H, W) grid, like the offset loops of the Token Radius
    Attention demo, and drops offsets that leave the grid (no padding);
  * the sliding window lists, for each query frame i, the key frames
    max(0, i - W + 1) .. i of the Vera 1.1 temporal module section 2.2;
  * sink frames (the "sink" of Radial Attention section 4's count) set whole
    key-frame columns of an existing matrix;
  * the block-index reading of section 6 reuses ``radial`` on the block grid.
"""
from __future__ import annotations

import math

import numpy as np


def radial(f: int, s: int) -> np.ndarray:
    n = f * s
    out = np.zeros((n, n), dtype=np.uint8)
    for i in range(f):
        for j in range(f):
            r = math.floor(math.log2(max(abs(i - j), 1)))
            width = s / (2 ** r)
            stride = math.ceil((2 ** r) / s)
            for k in range(s):
                for l in range(s):
                    case_a = (2 ** r) <= s and abs(k - l) + 1 <= width
                    case_b = (abs(i - j) % stride) == 0 and k == l
                    if case_a or case_b:
                        out[i * s + k, j * s + l] = 1
    return out


def radius3d(T: int, H: int, W: int, r_t: int, r_s: int) -> np.ndarray:
    n = T * H * W
    out = np.zeros((n, n), dtype=np.uint8)
    for t in range(T):
        for h in range(H):
            for w in range(W):
                qi = (t * H + h) * W + w
                for dt in range(-r_t, r_t + 1):
                    for dh in range(-r_s, r_s + 1):
                        for dw in range(-r_s, r_s + 1):
                            t2, h2, w2 = t + dt, h + dh, w + dw
                            if 0 <= t2 < T and 0 <= h2 < H and 0 <= w2 < W:
                                out[qi, (t2 * H + h2) * W + w2] = 1
    return out


def swa_causal(f: int, s: int, window: int) -> np.ndarray:
    n = f * s
    out = np.zeros((n, n), dtype=np.uint8)
    for i in range(f):
        for j in range(max(0, i - window + 1), i + 1):
            out[i * s:(i + 1) * s, j * s:(j + 1) * s] = 1
    return out


def dilate_any(elem: np.ndarray, block: int) -> np.ndarray:
    """Block granularity: a block x block tile is kept iff any entry is kept
    (tail tiles are cut at n).  Returns the element-level view of the
    dilated mask together with the per-block keep matrix."""
    n = elem.shape[0]
    nb = (n + block - 1) // block
    keep = np.zeros((nb, nb), dtype=np.uint8)
    out = np.zeros_like(elem)
    for a in range(nb):
        for b in range(nb):
            tile = elem[a * block:(a + 1) * block, b * block:(b + 1) * block]
            if tile.any():
                keep[a, b] = 1
                out[a * block:(a + 1) * block, b * block:(b + 1) * block] = 1
    return out, keep


def with_sink(elem: np.ndarray, s: int, sink_frames: int) -> np.ndarray:
    """Every query also keeps every key of frames 0 .. sink_frames - 1."""
    out = elem.copy()
    out[:, :min(elem.shape[1], sink_frames * s)] = 1
    return out


def radial_blocks(f: int, s: int, block: int, sink_frames: int = 0) -> np.ndarray:
    """Kept-block matrix of eq. 4 applied to block indices: the block grid is
    a video of f frames with s / block blocks per frame."""
    assert s % block == 0
    sb = s // block
    return with_sink(radial(f, sb), sb, sink_frames)
