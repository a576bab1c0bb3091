"""Static sparse spatiotemporal attention for AMD Instinct MI355X (gfx950).

Thin Python binding of ``libtra.so`` (C ABI in ``include/tra.h``).  This
module only marshals arguments: torch supplies device memory and the HIP
stream, and every step of the computation runs in the library's HIP kernels.
There is no fallback: if the library is not built, importing the binding's
functions raises.

    mask = build_mask(f=128, s=1024, kind="radial", granularity="block_any")
    out, lse = sparse_attn_fwd(q, k, v, mask)      # q, k, v: [B, H, n, D] on cuda

Computes softmax((Q K^T + M) / sqrt(D)) V (Radial Attention section 2, eq. 2)
with M one of: the radial mask of eq. 4, a (r_t, r_s) token-radius
neighbourhood on a t-h-w grid, or a frame sliding-window causal mask.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

__all__ = ["build_mask", "sparse_attn_fwd", "sparse_attn_bwd", "sparse_attn_bwd_workspace_bytes", "linear_attn_fwd", "salad_gate", "salad_combine",
           "KVCache", "Mask", "TraError", "library_path", "load_library", "probe_mfma_peak",
           "KINDS", "GRANULARITIES"]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libtra.so")

KINDS = {"dense": 0, "radial": 1, "radius3d": 2, "swa": 3}
GRANULARITIES = {"element": 0, "block_any": 1, "block_eq4": 2}
_F32, _BF16 = 0, 1
_STATUS = {0: "TRA_OK", -1: "TRA_ERR_INVALID", -2: "TRA_ERR_UNSUPPORTED", -3: "TRA_ERR_SHAPE",
           -4: "TRA_ERR_OOM", -5: "TRA_ERR_HIP"}


class TraError(RuntimeError):
    def __init__(self, status: int, what: str, hip_error: int = 0):
        self.status = status
        self.hip_error = hip_error
        extra = f" (hipError {hip_error})" if status in (-4, -5) else ""
        super().__init__(f"{what}: {_STATUS.get(status, status)}{extra}")


class MaskParams(ctypes.Structure):
    _fields_ = [("granularity", ctypes.c_int32), ("block", ctypes.c_int32),
                ("grid_h", ctypes.c_int32), ("grid_w", ctypes.c_int32),
                ("r_t", ctypes.c_int32), ("r_s", ctypes.c_int32), ("window", ctypes.c_int32),
                ("sink_frames", ctypes.c_int32), ("reserved", ctypes.c_int32 * 8)]


class MaskInfo(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int64), ("f", ctypes.c_int64), ("s", ctypes.c_int64),
                ("nqb", ctypes.c_int64), ("nkb", ctypes.c_int64),
                ("kept_blocks", ctypes.c_int64), ("partial_blocks", ctypes.c_int64),
                ("kept_elems", ctypes.c_int64), ("pred_elems", ctypes.c_int64),
                ("min_row_blocks", ctypes.c_int64), ("max_row_blocks", ctypes.c_int64),
                ("bitmap_words", ctypes.c_int64), ("work_items", ctypes.c_int64),
                ("tile_loads", ctypes.c_int64), ("kind", ctypes.c_int32),
                ("granularity", ctypes.c_int32), ("bwd_work_items", ctypes.c_int64),
                ("bwd_tile_loads", ctypes.c_int64)]


class TensorDesc(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("B", ctypes.c_int64), ("H", ctypes.c_int64), ("N", ctypes.c_int64),
                ("D", ctypes.c_int64), ("stride", ctypes.c_int64 * 4)]


_lib = None


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libtra.so once.  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is missing; build it with "
                           "`python -m static_sparse_spatiotemporal_amd._build`")
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.POINTER
    vp = ctypes.c_void_p
    lib.tra_build_mask.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, P(MaskParams), vp, P(vp)]
    lib.tra_build_mask.restype = ctypes.c_int
    lib.tra_sparse_attn_fwd.argtypes = [P(TensorDesc), P(TensorDesc), P(TensorDesc), vp, P(TensorDesc),
                                        vp, ctypes.c_float, vp]
    lib.tra_sparse_attn_fwd.restype = ctypes.c_int
    i64 = ctypes.c_int64
    lib.tra_sparse_attn_bwd_workspace_bytes.argtypes = [i64, i64, i64, i64]
    lib.tra_sparse_attn_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.tra_sparse_attn_bwd.argtypes = [P(TensorDesc), P(TensorDesc), P(TensorDesc), P(TensorDesc),
                                        P(TensorDesc), vp, vp, P(TensorDesc), P(TensorDesc), P(TensorDesc),
                                        vp, ctypes.c_size_t, ctypes.c_float, vp]
    lib.tra_sparse_attn_bwd.restype = ctypes.c_int
    lib.tra_linear_attn_workspace_bytes.argtypes = [i64, i64, i64, i64]
    lib.tra_linear_attn_workspace_bytes.restype = ctypes.c_size_t
    lib.tra_linear_attn_fwd.argtypes = [P(TensorDesc), P(TensorDesc), P(TensorDesc), P(TensorDesc),
                                        ctypes.c_float, vp, ctypes.c_size_t, vp]
    lib.tra_linear_attn_fwd.restype = ctypes.c_int
    lib.tra_salad_gate_workspace_bytes.argtypes = [i64, i64]
    lib.tra_salad_gate_workspace_bytes.restype = ctypes.c_size_t
    lib.tra_salad_gate.argtypes = [P(TensorDesc), vp, ctypes.c_float, vp, vp, ctypes.c_size_t, vp]
    lib.tra_salad_gate.restype = ctypes.c_int
    lib.tra_salad_combine.argtypes = [P(TensorDesc), P(TensorDesc), vp, vp, vp, P(TensorDesc), vp]
    lib.tra_salad_combine.restype = ctypes.c_int
    lib.tra_kvcache_create.argtypes = [i64, i64, i64, i64, ctypes.c_int32, ctypes.c_int32, P(vp)]
    lib.tra_kvcache_create.restype = ctypes.c_int
    lib.tra_kvcache_append.argtypes = [vp, P(TensorDesc), P(TensorDesc), vp]
    lib.tra_kvcache_append.restype = ctypes.c_int
    lib.tra_kvcache_attn.argtypes = [vp, P(TensorDesc), P(TensorDesc), vp, ctypes.c_float, vp]
    lib.tra_kvcache_attn.restype = ctypes.c_int
    lib.tra_kvcache_get_frames.argtypes = [vp, P(i64), P(i64)]
    lib.tra_kvcache_get_frames.restype = ctypes.c_int
    lib.tra_kvcache_reset.argtypes = [vp]
    lib.tra_kvcache_reset.restype = ctypes.c_int
    lib.tra_kvcache_free.argtypes = [vp]
    lib.tra_kvcache_free.restype = None
    lib.tra_mask_get_info.argtypes = [vp, P(MaskInfo)]
    lib.tra_mask_get_info.restype = ctypes.c_int
    lib.tra_mask_export.argtypes = [vp, vp, vp, vp, vp, vp, vp]
    lib.tra_mask_export.restype = ctypes.c_int
    lib.tra_mask_free.argtypes = [vp]
    lib.tra_mask_free.restype = None
    lib.tra_status_string.argtypes = [ctypes.c_int]
    lib.tra_status_string.restype = ctypes.c_char_p
    lib.tra_last_hip_error.argtypes = []
    lib.tra_last_hip_error.restype = ctypes.c_int32
    lib.tra_version.argtypes = []
    lib.tra_version.restype = ctypes.c_int32
    lib.tra_probe_mfma_peak.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p,
                                        ctypes.POINTER(ctypes.c_int64), ctypes.c_void_p]
    lib.tra_probe_mfma_peak.restype = ctypes.c_int
    _lib = lib
    return lib


def _check(status: int, what: str):
    if status != 0:
        raise TraError(status, what, load_library().tra_last_hip_error())


def _stream_handle(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(int(stream.cuda_stream))


class Mask:
    """A compiled static mask (owns device memory until freed)."""

    def __init__(self, handle: ctypes.c_void_p):
        self._h = handle
        info = MaskInfo()
        _check(load_library().tra_mask_get_info(self._h, ctypes.byref(info)), "tra_mask_get_info")
        self.info = {k: getattr(info, k) for k, _ in MaskInfo._fields_}

    @property
    def handle(self) -> ctypes.c_void_p:
        if self._h is None:
            raise ValueError("mask was freed")
        return self._h

    def export(self) -> dict:
        """Host copies of the compiled mask (see tra_mask_export)."""
        i = self.info
        out = {
            "bitmap": np.zeros((i["nqb"], i["bitmap_words"]), dtype=np.uint32),
            "row_ptr": np.zeros(i["nqb"] + 1, dtype=np.int32),
            "col_idx": np.zeros(i["kept_blocks"], dtype=np.int32),
            "emask_idx": np.zeros(i["kept_blocks"], dtype=np.int32),
            "emask": np.zeros((i["partial_blocks"], 128, 4), dtype=np.uint32),
            "order": np.zeros(i["nqb"], dtype=np.int32),
        }
        _check(load_library().tra_mask_export(
            self.handle, *(a.ctypes.data if a.size else None for a in
                           (out["bitmap"], out["row_ptr"], out["col_idx"], out["emask_idx"],
                            out["emask"], out["order"]))), "tra_mask_export")
        return out

    def free(self):
        if self._h is not None:
            load_library().tra_mask_free(self._h)
            self._h = None

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass


def build_mask(f: int, s: int, kind: str, granularity: str = "element", grid_h: int = 0,
               grid_w: int = 0, r_t: int = 0, r_s: int = 0, window: int = 0, sink_frames: int = 0,
               stream=None) -> Mask:
    """Compile a static mask for n = f * s tokens (synchronous; see tra_build_mask)."""
    lib = load_library()
    p = MaskParams()
    p.granularity = GRANULARITIES[granularity]
    p.block = 128
    p.grid_h, p.grid_w, p.r_t, p.r_s, p.window = grid_h, grid_w, r_t, r_s, window
    p.sink_frames = sink_frames
    h = ctypes.c_void_p()
    _check(lib.tra_build_mask(int(f), int(s), KINDS[kind], ctypes.byref(p), _stream_handle(stream),
                              ctypes.byref(h)), "tra_build_mask")
    return Mask(h)


def _desc(t: torch.Tensor) -> TensorDesc:
    if t.dim() != 4:
        raise ValueError("expected a [B, H, N, D] tensor")
    if t.dtype == torch.bfloat16:
        dt = _BF16
    elif t.dtype == torch.float32:
        dt = _F32
    else:
        raise TypeError(f"unsupported dtype {t.dtype}")
    d = TensorDesc()
    d.data = t.data_ptr()
    d.dtype = dt
    d.B, d.H, d.N, d.D = t.shape
    for i, st in enumerate(t.stride()):
        d.stride[i] = st
    return d


def sparse_attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, mask: Mask,
                    out: torch.Tensor | None = None, lse: torch.Tensor | bool | None = True,
                    scale: float | None = None, stream=None):
    """O = softmax((Q K^T + M) * scale) V on the GPU (see tra_sparse_attn_fwd).

    q, k, v: [B, H, n, D] cuda tensors (bf16 or fp32).  `out` defaults to a new
    contiguous tensor; `lse` = True allocates a [B, H, n] fp32 tensor, a tensor
    is written in place, False/None skips it.  Returns (out, lse or None).
    """
    if not (q.is_cuda and k.is_cuda and v.is_cuda):
        raise ValueError("q, k, v must be on a HIP device")
    if out is None:
        out = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    if lse is True:
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    elif lse is False:
        lse = None
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous()
                            or tuple(lse.shape) != tuple(q.shape[:3])):
        raise ValueError("lse must be a contiguous float32 [B, H, n] tensor")
    dq, dk, dv, do = _desc(q), _desc(k), _desc(v), _desc(out)
    _check(load_library().tra_sparse_attn_fwd(
        ctypes.byref(dq), ctypes.byref(dk), ctypes.byref(dv), mask.handle, ctypes.byref(do),
        ctypes.c_void_p(lse.data_ptr()) if lse is not None else None,
        float(scale) if scale else 0.0, _stream_handle(stream)), "tra_sparse_attn_fwd")
    return out, lse


def sparse_attn_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor, lse: torch.Tensor,
                    dout: torch.Tensor, mask: Mask, scale: float | None = None, grads=None,
                    workspace: torch.Tensor | None = None, stream=None):
    """Gradients (dQ, dK, dV) of sparse_attn_fwd on the GPU (see tra_sparse_attn_bwd).

    q, k, v, out, dout: [B, H, n, D] bf16 cuda tensors; lse: the forward's
    [B, H, n] fp32 output.  `grads` = (dq, dk, dv) output tensors (default:
    new contiguous ones); `workspace` a uint8 cuda tensor of at least
    sparse_attn_bwd_workspace_bytes bytes (default: new).
    """
    lib = load_library()
    B, H, n, D = q.shape
    if grads is None:
        grads = tuple(torch.empty(q.shape, dtype=q.dtype, device=q.device) for _ in range(3))
    if workspace is None:
        workspace = torch.empty(int(lib.tra_sparse_attn_bwd_workspace_bytes(B, H, n, D)), dtype=torch.uint8,
                                device=q.device)
    if lse.dtype != torch.float32 or not lse.is_contiguous() or tuple(lse.shape) != tuple(q.shape[:3]):
        raise ValueError("lse must be a contiguous float32 [B, H, n] tensor")
    descs = [_desc(t) for t in (q, k, v, out, dout)]
    gd = [_desc(t) for t in grads]
    _check(lib.tra_sparse_attn_bwd(
        *(ctypes.byref(d) for d in descs), ctypes.c_void_p(lse.data_ptr()), mask.handle,
        *(ctypes.byref(d) for d in gd), ctypes.c_void_p(workspace.data_ptr()), workspace.numel(),
        float(scale) if scale else 0.0, _stream_handle(stream)), "tra_sparse_attn_bwd")
    return grads


def sparse_attn_bwd_workspace_bytes(B: int, H: int, n: int, D: int) -> int:
    return int(load_library().tra_sparse_attn_bwd_workspace_bytes(B, H, n, D))


class KVCache:
    """Frame-streaming K/V ring for the frame sliding-window causal mask (see
    tra_kvcache_create).  append(k, v) adds the next frame ([B, H, s, D] bf16);
    attn(q) returns (O, LSE) of that frame's queries over the cached frames."""

    def __init__(self, B: int, H: int, s: int, D: int, window: int):
        lib = load_library()
        h = ctypes.c_void_p()
        _check(lib.tra_kvcache_create(B, H, s, D, window, _BF16, ctypes.byref(h)), "tra_kvcache_create")
        self._h = h
        self.shape = (B, H, s, D)
        self.window = window

    @property
    def handle(self):
        if self._h is None:
            raise ValueError("cache was freed")
        return self._h

    def append(self, k: torch.Tensor, v: torch.Tensor, stream=None):
        dk, dv = _desc(k), _desc(v)
        _check(load_library().tra_kvcache_append(self.handle, ctypes.byref(dk), ctypes.byref(dv),
                                                 _stream_handle(stream)), "tra_kvcache_append")

    def attn(self, q: torch.Tensor, out: torch.Tensor | None = None, lse: torch.Tensor | bool | None = True,
             scale: float | None = None, stream=None):
        if out is None:
            out = torch.empty(q.shape, dtype=q.dtype, device=q.device)
        if lse is True:
            lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
        elif lse is False:
            lse = None
        dq, do = _desc(q), _desc(out)
        _check(load_library().tra_kvcache_attn(
            self.handle, ctypes.byref(dq), ctypes.byref(do),
            ctypes.c_void_p(lse.data_ptr()) if lse is not None else None,
            float(scale) if scale else 0.0, _stream_handle(stream)), "tra_kvcache_attn")
        return out, lse

    def frames(self):
        a, c = ctypes.c_int64(), ctypes.c_int64()
        _check(load_library().tra_kvcache_get_frames(self.handle, ctypes.byref(a), ctypes.byref(c)),
               "tra_kvcache_get_frames")
        return a.value, c.value

    def reset(self):
        _check(load_library().tra_kvcache_reset(self.handle), "tra_kvcache_reset")

    def free(self):
        if self._h is not None:
            load_library().tra_kvcache_free(self._h)
            self._h = None

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass


def linear_attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor | None = None,
                    eps: float = 1e-6, workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """SALAD ReLU-kernel linear attention on the GPU (see tra_linear_attn_fwd).

    q, k, v: [B, H, n, D] bf16 cuda tensors.  `workspace` (uint8 cuda tensor of
    at least linear_attn_workspace_bytes bytes) defaults to a new one.
    """
    lib = load_library()
    B, H, n, D = q.shape
    need = int(lib.tra_linear_attn_workspace_bytes(B, H, n, D))
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    descs = [_desc(t) for t in (q, k, v, out)]
    _check(lib.tra_linear_attn_fwd(*(ctypes.byref(d) for d in descs), float(eps),
                                   ctypes.c_void_p(workspace.data_ptr()), workspace.numel(),
                                   _stream_handle(stream)), "tra_linear_attn_fwd")
    return out


def linear_attn_workspace_bytes(B: int, H: int, n: int, D: int) -> int:
    return int(load_library().tra_linear_attn_workspace_bytes(B, H, n, D))


def salad_gate(x: torch.Tensor, w: torch.Tensor, bias: float = 0.0, gate: torch.Tensor | None = None,
               workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """SALAD gate on the GPU (see tra_salad_gate): gate[b] = mean over tokens
    of sigmoid(x[b, n] . w + bias).

    x: [B, N, C] bf16 cuda tensor (the block input); w: [C] bf16.  Returns
    `gate` ([B] float32, a new tensor by default).
    """
    lib = load_library()
    if x.dim() != 3:
        raise ValueError("expected x as [B, N, C]")
    B, N, C = x.shape
    need = int(lib.tra_salad_gate_workspace_bytes(B, N))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=x.device)
    if gate is None:
        gate = torch.empty(B, dtype=torch.float32, device=x.device)
    xd = _desc(x.unsqueeze(1))
    _check(lib.tra_salad_gate(ctypes.byref(xd), ctypes.c_void_p(w.data_ptr()), float(bias),
                              ctypes.c_void_p(gate.data_ptr()), ctypes.c_void_p(workspace.data_ptr()),
                              workspace.numel(), _stream_handle(stream)), "tra_salad_gate")
    return gate


def salad_gate_workspace_bytes(B: int, N: int) -> int:
    return int(load_library().tra_salad_gate_workspace_bytes(B, N))


def probe_mfma_peak(iterations: int = 200000, blocks: int | None = None, stream=None) -> tuple[float, int]:
    """Measured bf16 MFMA peak (see tra_probe_mfma_peak): runs the register-only
    MFMA loop once per compute unit and returns (milliseconds, flops)."""
    lib = load_library()
    if blocks is None:
        blocks = torch.cuda.get_device_properties(torch.cuda.current_device()).multi_processor_count
    out = torch.empty(blocks, dtype=torch.float32, device="cuda")
    flops = ctypes.c_int64(0)
    st = torch.cuda.current_stream() if stream is None else stream
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    _check(lib.tra_probe_mfma_peak(int(iterations), int(blocks), ctypes.c_void_p(out.data_ptr()), ctypes.byref(flops),
                                   _stream_handle(st)), "tra_probe_mfma_peak")
    e1.record(st)
    e1.synchronize()
    return e0.elapsed_time(e1), int(flops.value)


def salad_combine(o_sparse: torch.Tensor, o_lin: torch.Tensor, weight: torch.Tensor, gate: torch.Tensor,
                  bias: torch.Tensor | None = None, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """SALAD output on the GPU (see tra_salad_combine): out = O_sparse +
    gate[b] * (O_lin W^T + bias) over the merged-head channels h * D + e.

    o_sparse, o_lin: [B, H, N, D] bf16 cuda tensors; weight: [H*D, H*D] bf16
    (row = output channel); gate: [B] float32; bias: [H*D] float32 or None.
    `out` defaults to a new tensor; it may be o_sparse itself.
    """
    lib = load_library()
    if out is None:
        out = torch.empty(o_sparse.shape, dtype=o_sparse.dtype, device=o_sparse.device)
    descs = [_desc(t) for t in (o_sparse, o_lin, out)]
    _check(lib.tra_salad_combine(ctypes.byref(descs[0]), ctypes.byref(descs[1]),
                                 ctypes.c_void_p(weight.data_ptr()),
                                 ctypes.c_void_p(None if bias is None else bias.data_ptr()),
                                 ctypes.c_void_p(gate.data_ptr()), ctypes.byref(descs[2]),
                                 _stream_handle(stream)), "tra_salad_combine")
    return out
