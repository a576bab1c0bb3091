"""fp64 CPU oracle for static sparse spatiotemporal attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` import this package.  The product
library (``static_sparse_spatiotemporal_amd``) never imports, links or calls
it, and it imports nothing from the product.

Definitions followed (pages on the method; see ``oracle.h`` for detail):
  * Radial Attention, section 2, eq. 1 and eq. 2 -- (masked) softmax attention
  * Radial Attention, section 3, eq. 4 -- the radial mask over frames/positions
  * Token Radius Attention, radius design section -- (r_t, r_s) neighbourhood
  * Vera 1.1 temporal module, sections 2.1-2.2 -- frame sliding-window causal
  * Radial Attention, section 6 -- 128 x 128 block granularity (any-element
    dilation, or eq. 4 on block indices as a second reading)
  * Radial Attention, section 4 -- the "sink" of the complexity count, as
    key frames every query keeps (sink_frames)
  * SALAD, sections 2.1-2.2 -- the ReLU-kernel linear-attention branch, the
    scalar sigmoid gate and the gated, projected sum of the two branches

The C part (``oracle.c``) does the arithmetic; this module only marshals numpy
arrays through ctypes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

DENSE, RADIAL, RADIUS3D, SWA = 0, 1, 2, 3
ELEMENT, BLOCK_ANY, BLOCK_EQ4 = 0, 1, 2
F32, BF16 = 0, 1

KIND_BY_NAME = {"dense": DENSE, "radial": RADIAL, "radius3d": RADIUS3D, "swa": SWA}
GRAN_BY_NAME = {"element": ELEMENT, "block_any": BLOCK_ANY, "block_eq4": BLOCK_EQ4}


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (plain -O2, pthreads)."""
    src = os.path.join(_HERE, "oracle.c")
    if not force and os.path.exists(_LIB_PATH) and os.path.getmtime(_LIB_PATH) >= os.path.getmtime(src):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-o", tmp, src, "-lm", "-lpthread"],
                   check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class _Mask(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("granularity", ctypes.c_int32),
                ("f", ctypes.c_int64), ("s", ctypes.c_int64), ("block", ctypes.c_int64),
                ("grid_h", ctypes.c_int64), ("grid_w", ctypes.c_int64),
                ("r_t", ctypes.c_int64), ("r_s", ctypes.c_int64), ("window", ctypes.c_int64),
                ("sink_frames", ctypes.c_int64)]


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.POINTER
        lib.orc_keep.argtypes = [P(_Mask), ctypes.c_int64, ctypes.c_int64]
        lib.orc_keep.restype = ctypes.c_int
        lib.orc_elem_matrix.argtypes = [P(_Mask), ctypes.c_void_p]
        lib.orc_keep_block_eq4.argtypes = [P(_Mask), ctypes.c_int64, ctypes.c_int64]
        lib.orc_keep_block_eq4.restype = ctypes.c_int
        lib.orc_block_keep.argtypes = [P(_Mask), ctypes.c_void_p, ctypes.c_int]
        lib.orc_block_counts.argtypes = [P(_Mask), ctypes.c_void_p, ctypes.c_int]
        lib.orc_block_counts_rows.argtypes = [P(_Mask), ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                              ctypes.c_int]
        lib.orc_kept_elements.argtypes = [P(_Mask), ctypes.c_int]
        lib.orc_kept_elements.restype = ctypes.c_int64
        lib.orc_block_bits128.argtypes = [P(_Mask), ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p]
        lib.orc_attention_bwd_rows.argtypes = [
            ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
            P(_Mask), ctypes.c_void_p, ctypes.c_double, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
        lib.orc_linear_attention_rows.argtypes = [
            ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_double,
            ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int]
        lib.orc_salad_gate.argtypes = [
            ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_double,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int]
        lib.orc_salad_output_rows.argtypes = [
            ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
            ctypes.c_void_p, ctypes.c_int]
        lib.orc_row_counts.argtypes = [P(_Mask), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                       ctypes.c_void_p]
        lib.orc_attention_rows.argtypes = [
            ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
            P(_Mask), ctypes.c_void_p, ctypes.c_double, ctypes.c_void_p, ctypes.c_int64,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
        _lib = lib
    return _lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


class MaskSpec:
    """A mask family with its parameters (kind and granularity by name)."""

    def __init__(self, kind: str, f: int, s: int, granularity: str = "element", block: int = 128,
                 grid_h: int = 0, grid_w: int = 0, r_t: int = 0, r_s: int = 0, window: int = 0,
                 sink_frames: int = 0):
        self.kind, self.granularity = kind, granularity
        self.f, self.s, self.block = int(f), int(s), int(block)
        self.grid_h, self.grid_w = int(grid_h), int(grid_w)
        self.r_t, self.r_s, self.window = int(r_t), int(r_s), int(window)
        self.sink_frames = int(sink_frames)
        if granularity == "block_eq4":
            assert kind == "radial" and self.s % self.block == 0, "block_eq4 needs radial, s % block == 0"

    @property
    def n(self) -> int:
        return self.f * self.s

    @property
    def nb(self) -> int:
        return (self.n + self.block - 1) // self.block

    def _c(self) -> _Mask:
        return _Mask(KIND_BY_NAME[self.kind], GRAN_BY_NAME[self.granularity], self.f, self.s,
                     self.block, self.grid_h, self.grid_w, self.r_t, self.r_s, self.window,
                     self.sink_frames)


def keep(spec: MaskSpec, q: int, t: int) -> bool:
    m = spec._c()
    return bool(_load().orc_keep(ctypes.byref(m), q, t))


def element_matrix(spec: MaskSpec) -> np.ndarray:
    """n x n uint8 matrix of the element predicate (1 = kept, i.e. M = 0)."""
    out = np.zeros((spec.n, spec.n), dtype=np.uint8)
    m = spec._c()
    _load().orc_elem_matrix(ctypes.byref(m), out.ctypes.data)
    return out


def keep_block_eq4(spec: MaskSpec, bq: int, bk: int) -> bool:
    m = spec._c()
    return bool(_load().orc_keep_block_eq4(ctypes.byref(m), bq, bk))


def block_keep(spec: MaskSpec, threads: int | None = None) -> np.ndarray:
    """nb x nb uint8 kept-block matrix at the spec's granularity."""
    out = np.zeros((spec.nb, spec.nb), dtype=np.uint8)
    m = spec._c()
    _load().orc_block_keep(ctypes.byref(m), out.ctypes.data, threads or default_threads())
    return out


def block_counts(spec: MaskSpec, threads: int | None = None) -> np.ndarray:
    """nb x nb int64 kept-element counts per block (edge spec.block)."""
    out = np.zeros((spec.nb, spec.nb), dtype=np.int64)
    m = spec._c()
    _load().orc_block_counts(ctypes.byref(m), out.ctypes.data, threads or default_threads())
    return out


def block_counts_rows(spec: MaskSpec, rows, threads: int | None = None) -> np.ndarray:
    """len(rows) x nb int64 kept-element counts of the listed block rows."""
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    out = np.zeros((rows.size, spec.nb), dtype=np.int64)
    m = spec._c()
    _load().orc_block_counts_rows(ctypes.byref(m), rows.ctypes.data, rows.size, out.ctypes.data,
                                  threads or default_threads())
    return out


def kept_elements(spec: MaskSpec, threads: int | None = None) -> int:
    m = spec._c()
    return int(_load().orc_kept_elements(ctypes.byref(m), threads or default_threads()))


def block_bits128(spec: MaskSpec, qb: int, kb: int) -> np.ndarray:
    """128 x 4 uint32 row bitmaps of block (qb, kb); requires spec.block == 128."""
    assert spec.block == 128
    out = np.zeros((128, 4), dtype=np.uint32)
    m = spec._c()
    _load().orc_block_bits128(ctypes.byref(m), qb, kb, out.ctypes.data)
    return out


def row_counts(spec: MaskSpec, rows, block_keep: np.ndarray | None = None) -> np.ndarray:
    """Keys attended by each listed query row (int64), by the rule
    attention_rows uses."""
    rows = np.ascontiguousarray(rows, dtype=np.int64).reshape(-1)
    out = np.zeros(rows.size, dtype=np.int64)
    bk_ptr = None
    if spec.granularity == "block_any":
        if block_keep is None:
            block_keep = block_counts(spec) > 0
        block_keep = np.ascontiguousarray(block_keep, dtype=np.uint8)
        bk_ptr = block_keep.ctypes.data
    m = spec._c()
    _load().orc_row_counts(ctypes.byref(m), bk_ptr, rows.ctypes.data, rows.size, out.ctypes.data)
    return out


def attention_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, spec: MaskSpec,
                   rows: np.ndarray | None = None, scale: float | None = None,
                   block_keep: np.ndarray | None = None, threads: int | None = None):
    """fp64 masked attention (eq. 2) for selected rows.

    q, k, v: [B, H, n, d] numpy arrays, float32 or uint16 (raw bfloat16 bits).
    rows: int64 array of (b, h, query) triples; None = every row.
    Returns (O [nrows, d] float64, LSE [nrows] float64).
    """
    B, H, n, d = q.shape
    assert k.shape == q.shape and v.shape == q.shape and n == spec.n
    if q.dtype == np.float32:
        dtype = F32
    elif q.dtype == np.uint16:
        dtype = BF16
    else:
        raise TypeError("q/k/v must be float32 or uint16 (bfloat16 bits)")
    assert k.dtype == q.dtype and v.dtype == q.dtype
    q, k, v = (np.ascontiguousarray(a) for a in (q, k, v))
    if rows is None:
        bb, hh, qq = np.meshgrid(np.arange(B), np.arange(H), np.arange(n), indexing="ij")
        rows = np.stack([bb.ravel(), hh.ravel(), qq.ravel()], axis=1)
    rows = np.ascontiguousarray(rows, dtype=np.int64).reshape(-1, 3)
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    bk_ptr = None
    if spec.granularity == "block_any":
        if block_keep is None:
            block_keep = block_counts(spec, threads) > 0
        block_keep = np.ascontiguousarray(block_keep, dtype=np.uint8)
        assert block_keep.shape == (spec.nb, spec.nb)
        bk_ptr = block_keep.ctypes.data
    o = np.zeros((rows.shape[0], d), dtype=np.float64)
    lse = np.zeros((rows.shape[0],), dtype=np.float64)
    m = spec._c()
    _load().orc_attention_rows(dtype, q.ctypes.data, k.ctypes.data, v.ctypes.data, B, H, n, d,
                               ctypes.byref(m), bk_ptr, float(scale), rows.ctypes.data,
                               rows.shape[0], o.ctypes.data, lse.ctypes.data,
                               threads or default_threads())
    return o, lse


def attention_bwd_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, dout: np.ndarray, spec: MaskSpec,
                       q_rows: np.ndarray | None = None, k_rows: np.ndarray | None = None,
                       scale: float | None = None, block_keep: np.ndarray | None = None,
                       threads: int | None = None):
    """fp64 gradients of eq. 2 (dQ for q_rows, dK and dV for k_rows).

    Arrays as attention_rows plus dout (the gradient of O).  Row lists are
    (b, h, index) triples; None = every row.  Returns (dQ [nq, d], dK [nk, d],
    dV [nk, d]) as float64.
    """
    B, H, n, d = q.shape
    assert k.shape == q.shape and v.shape == q.shape and dout.shape == q.shape and n == spec.n
    if q.dtype == np.float32:
        dtype = F32
    elif q.dtype == np.uint16:
        dtype = BF16
    else:
        raise TypeError("q/k/v/dout must be float32 or uint16 (bfloat16 bits)")
    assert k.dtype == q.dtype and v.dtype == q.dtype and dout.dtype == q.dtype
    q, k, v, dout = (np.ascontiguousarray(a) for a in (q, k, v, dout))

    def all_rows():
        bb, hh, ii = np.meshgrid(np.arange(B), np.arange(H), np.arange(n), indexing="ij")
        return np.stack([bb.ravel(), hh.ravel(), ii.ravel()], axis=1)

    q_rows = all_rows() if q_rows is None else q_rows
    k_rows = all_rows() if k_rows is None else k_rows
    q_rows = np.ascontiguousarray(q_rows, dtype=np.int64).reshape(-1, 3)
    k_rows = np.ascontiguousarray(k_rows, dtype=np.int64).reshape(-1, 3)
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    bk_ptr = None
    if spec.granularity == "block_any":
        if block_keep is None:
            block_keep = block_counts(spec, threads) > 0
        block_keep = np.ascontiguousarray(block_keep, dtype=np.uint8)
        assert block_keep.shape == (spec.nb, spec.nb)
        bk_ptr = block_keep.ctypes.data
    dq = np.zeros((q_rows.shape[0], d), dtype=np.float64)
    dk = np.zeros((k_rows.shape[0], d), dtype=np.float64)
    dv = np.zeros((k_rows.shape[0], d), dtype=np.float64)
    m = spec._c()
    _load().orc_attention_bwd_rows(dtype, q.ctypes.data, k.ctypes.data, v.ctypes.data, dout.ctypes.data,
                                   B, H, n, d, ctypes.byref(m), bk_ptr, float(scale),
                                   q_rows.ctypes.data, q_rows.shape[0], dq.ctypes.data,
                                   k_rows.ctypes.data, k_rows.shape[0], dk.ctypes.data, dv.ctypes.data,
                                   threads or default_threads())
    return dq, dk, dv


def linear_attention_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, rows: np.ndarray | None = None,
                          eps: float = 1e-6, threads: int | None = None) -> np.ndarray:
    """fp64 ReLU-kernel linear attention (SALAD linear branch) for selected rows.

    Arrays as attention_rows; every key of the (b, h) counts.  Returns O
    [nrows, d] float64.
    """
    B, H, n, d = q.shape
    assert k.shape == q.shape and v.shape == q.shape
    if q.dtype == np.float32:
        dtype = F32
    elif q.dtype == np.uint16:
        dtype = BF16
    else:
        raise TypeError("q/k/v must be float32 or uint16 (bfloat16 bits)")
    q, k, v = (np.ascontiguousarray(a) for a in (q, k, v))
    if rows is None:
        bb, hh, qq = np.meshgrid(np.arange(B), np.arange(H), np.arange(n), indexing="ij")
        rows = np.stack([bb.ravel(), hh.ravel(), qq.ravel()], axis=1)
    rows = np.ascontiguousarray(rows, dtype=np.int64).reshape(-1, 3)
    o = np.zeros((rows.shape[0], d), dtype=np.float64)
    _load().orc_linear_attention_rows(dtype, q.ctypes.data, k.ctypes.data, v.ctypes.data, B, H, n, d,
                                      float(eps), rows.ctypes.data, rows.shape[0], o.ctypes.data,
                                      threads or default_threads())
    return o


def _dtype_code(*arrs) -> int:
    if all(a.dtype == np.float32 for a in arrs):
        return F32
    if all(a.dtype == np.uint16 for a in arrs):
        return BF16
    raise TypeError("arrays must all be float32 or all uint16 (bfloat16 bits)")


def salad_gate(x: np.ndarray, w: np.ndarray, bias: float = 0.0, threads: int | None = None) -> np.ndarray:
    """fp64 SALAD gate: g[b] = mean_n sigmoid(x[b, n, :] . w + bias).

    x: [B, N, C], w: [C], both float32 or both uint16 bfloat16 bits.
    Returns g [B] float64.
    """
    B, N, C = x.shape
    assert w.shape == (C,)
    dtype = _dtype_code(x, w)
    x, w = np.ascontiguousarray(x), np.ascontiguousarray(w)
    g = np.zeros(B, dtype=np.float64)
    _load().orc_salad_gate(dtype, x.ctypes.data, w.ctypes.data, float(bias), B, N, C, g.ctypes.data,
                           threads or default_threads())
    return g


def salad_output_rows(o_sparse: np.ndarray, o_lin: np.ndarray, w: np.ndarray, bias, g: np.ndarray,
                      rows: np.ndarray | None = None, threads: int | None = None) -> np.ndarray:
    """fp64 SALAD output rows: O_s + g[b] * (O_l W^T + bias) in the merged-head
    channel space (channel h * d + e of token n is [b, h, n, e]).

    o_sparse, o_lin: [B, H, N, d]; w: [H*d, H*d] (same dtype: float32 or
    uint16 bfloat16 bits); bias: None or [H*d] float; g: [B] float.
    rows: (b, n) pairs, default all.  Returns [nrows, H*d] float64.
    """
    B, H, N, d = o_sparse.shape
    C = H * d
    assert o_lin.shape == o_sparse.shape and w.shape == (C, C)
    dtype = _dtype_code(o_sparse, o_lin, w)
    o_sparse, o_lin, w = (np.ascontiguousarray(a) for a in (o_sparse, o_lin, w))
    bias_arr = None if bias is None else np.ascontiguousarray(bias, dtype=np.float64).reshape(C)
    g = np.ascontiguousarray(g, dtype=np.float64).reshape(B)
    if rows is None:
        bb, nn = np.meshgrid(np.arange(B), np.arange(N), indexing="ij")
        rows = np.stack([bb.ravel(), nn.ravel()], axis=1)
    rows = np.ascontiguousarray(rows, dtype=np.int64).reshape(-1, 2)
    out = np.zeros((rows.shape[0], C), dtype=np.float64)
    _load().orc_salad_output_rows(dtype, o_sparse.ctypes.data, o_lin.ctypes.data, w.ctypes.data,
                                  None if bias_arr is None else bias_arr.ctypes.data, g.ctypes.data,
                                  B, H, N, d, rows.ctypes.data, rows.shape[0], out.ctypes.data,
                                  threads or default_threads())
    return out
