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

import contextlib
import ctypes
import os

import numpy as np
import torch

__all__ = ["build_mask", "sparse_attn_fwd", "sparse_attn_bwd", "sparse_attn_bwd_workspace_bytes", "linear_attn_fwd", "salad_gate", "salad_gate_noalloc", "salad_combine",
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
    lib.tra_salad_gate_noalloc.argtypes = [P(TensorDesc), vp, ctypes.c_float, vp, vp]
    lib.tra_salad_gate_noalloc.restype = ctypes.c_int
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
    lib.tra_debug_live_allocations.argtypes = []
    lib.tra_debug_live_allocations.restype = ctypes.c_int64
    lib.tra_debug_fail_allocations.argtypes = [ctypes.c_int64]
    lib.tra_debug_fail_allocations.restype = ctypes.c_int64
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


# ---- argument checks -------------------------------------------------------
# The C ABI takes raw device pointers and cannot tell a host pointer, a tensor
# of the wrong dtype or one that is too small from a good one: every tensor is
# checked here, before anything is handed to the library.

def _fail(msg: str):
    raise ValueError(msg)


def _need_tensor(name: str, t, device: torch.device | None, dtype=None, shape=None, contiguous: bool = False):
    """`t` is a tensor on `device` (the call's device: that of its first
    tensor; None for that first tensor itself, which must be on a HIP
    device), of `dtype` (one dtype or a tuple), of `shape` when given, and
    contiguous when asked."""
    if not isinstance(t, torch.Tensor):
        _fail(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    if device is None:
        if not t.is_cuda:
            _fail(f"{name} must be on a HIP device (got {t.device})")
    elif (not t.is_cuda or t.get_device() != device.index) if device.type == "cuda" else t.device != device:
        _fail(f"{name} is on {t.device}, the call runs on {device}")
    if dtype is not None:
        td = t.dtype
        if td is not dtype and (not isinstance(dtype, tuple) or td not in dtype):
            ok = dtype if isinstance(dtype, tuple) else (dtype,)
            _fail(f"{name} must have dtype {' or '.join(str(d) for d in ok)}, got {td}")
    if shape is not None and t.shape != shape:
        _fail(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if contiguous and not t.is_contiguous():
        _fail(f"{name} must be contiguous")
    return t


def _need_bhnd(name: str, t, device: torch.device | None, dtype=None, shape=None):
    """A [B, H, N, D] view the kernels can read: unit stride in D, the other
    strides non-negative multiples of 16 bytes, data 16-byte aligned."""
    _need_tensor(name, t, device, dtype=dtype, shape=shape)
    if t.dim() != 4:
        _fail(f"{name} must be a [B, H, N, D] tensor, got {t.dim()} dims")
    if t.numel() == 0:
        return t
    vec = 16 // t.element_size()
    s0, s1, s2, s3 = t.stride()
    if s3 != 1 and t.shape[3] > 1:
        _fail(f"{name} must have unit stride in its last dimension")
    if s0 < 0 or s1 < 0 or s2 < 0 or s0 % vec or s1 % vec or s2 % vec:
        _fail(f"{name}: strides {(s0, s1, s2)} must be multiples of {vec} elements (16 bytes)")
    if t.data_ptr() % 16:
        _fail(f"{name} data must be 16-byte aligned")
    return t


def _need_workspace(name: str, t, device: torch.device, need: int):
    _need_tensor(name, t, device, dtype=torch.uint8, contiguous=True)
    if t.numel() < need:
        _fail(f"{name} holds {t.numel()} bytes, the call needs {need}")
    if t.data_ptr() % 256:
        _fail(f"{name} must be 256-byte aligned")
    return t


def _call_stream(stream, device: torch.device):
    """The torch stream the call runs on (the device's current stream by
    default); it must belong to the tensors' device."""
    if stream is None:
        return torch.cuda.current_stream(device)
    if not isinstance(stream, torch.cuda.Stream):
        _fail(f"stream must be a torch.cuda.Stream, got {type(stream).__name__}")
    if stream.device != device:
        _fail(f"stream is on {stream.device}, the tensors on {device}")
    return stream


def _new(shape, dtype, device, stream):
    """A tensor allocated for use on `stream`: the caching allocator hands its
    block out again only in that stream's order, so a default buffer that is
    dropped when the call returns cannot be reused while the call's kernels
    still read or write it."""
    with torch.cuda.stream(stream):
        return torch.empty(shape, dtype=dtype, device=device)


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


_DT = {torch.bfloat16: _BF16, torch.float32: _F32}
_STRIDES = ctypes.c_int64 * 4


_DESC_CACHE: dict = {}


def _desc(t: torch.Tensor) -> TensorDesc:
    """The C view of a [B, H, N, D] tensor.  Views are memoised on everything
    they hold (pointer, dtype, shape, strides), so a repeated call with the
    same tensors skips building the ctypes structure; the library only reads
    it during the call."""
    key = (t.data_ptr(), t.dtype, t.shape, t.stride())
    d = _DESC_CACHE.get(key)
    if d is not None:
        return d
    if t.dim() != 4:
        raise ValueError("expected a [B, H, N, D] tensor")
    dt = _DT.get(t.dtype)
    if dt is None:
        raise ValueError(f"unsupported dtype {t.dtype}")
    B, H, N, D = t.shape
    d = TensorDesc(t.data_ptr(), dt, 0, B, H, N, D, _STRIDES(*t.stride()))
    if len(_DESC_CACHE) >= 512:
        _DESC_CACHE.clear()
    _DESC_CACHE[key] = d
    return d


def _on(dev: torch.device):
    """Makes `dev` the current device for the library call (only switches when
    it is not current already)."""
    return contextlib.nullcontext() if torch.cuda.current_device() == dev.index else torch.cuda.device(dev)


def _ptr(t: torch.Tensor | None) -> ctypes.c_void_p:
    return ctypes.c_void_p(t.data_ptr() if t is not None else None)


def _lse_arg(lse, q: torch.Tensor, stream):
    """`lse` = True: a new [B, H, n] fp32 tensor; a tensor: checked and written
    in place; False/None: not computed."""
    if lse is True:
        return _new(q.shape[:3], torch.float32, q.device, stream)
    if lse is False or lse is None:
        return None
    return _need_tensor("lse", lse, q.device, dtype=torch.float32, shape=q.shape[:3], contiguous=True)


def sparse_attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, mask: Mask,
                    out: torch.Tensor | None = None, lse: torch.Tensor | bool | None = True,
                    scale: float | None = None, stream=None):
    """O = softmax((Q K^T + M) * scale) V on the GPU (see tra_sparse_attn_fwd).

    q, k, v: [B, H, n, D] cuda tensors (bf16 or fp32, one dtype) on one
    device.  `out` defaults to a new contiguous tensor; `lse` = True allocates
    a [B, H, n] fp32 tensor, a tensor is written in place, False/None skips
    it.  Returns (out, lse or None).
    """
    _need_bhnd("q", q, None, dtype=(torch.bfloat16, torch.float32))
    dev = q.device
    _need_bhnd("k", k, dev, dtype=q.dtype, shape=q.shape)
    _need_bhnd("v", v, dev, dtype=q.dtype, shape=q.shape)
    st = _call_stream(stream, dev)
    if out is None:
        out = _new(q.shape, q.dtype, dev, st)
    _need_bhnd("out", out, dev, dtype=q.dtype, shape=q.shape)
    lse = _lse_arg(lse, q, st)
    dq, dk, dv, do = _desc(q), _desc(k), _desc(v), _desc(out)
    with _on(dev):
        _check(load_library().tra_sparse_attn_fwd(
            ctypes.byref(dq), ctypes.byref(dk), ctypes.byref(dv), mask.handle, ctypes.byref(do),
            _ptr(lse), float(scale) if scale else 0.0, _stream_handle(st)), "tra_sparse_attn_fwd")
    return out, lse


def sparse_attn_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor, lse: torch.Tensor,
                    dout: torch.Tensor, mask: Mask, scale: float | None = None, grads=None,
                    workspace: torch.Tensor | None = None, stream=None):
    """Gradients (dQ, dK, dV) of sparse_attn_fwd on the GPU (see tra_sparse_attn_bwd).

    q, k, v, out, dout: [B, H, n, D] cuda tensors of one dtype (bf16 or
    fp32); lse: the forward's [B, H, n] fp32 output.  `grads` = (dq, dk, dv)
    output tensors of that dtype (default: new contiguous ones);
    `workspace` a uint8 cuda tensor of at least
    sparse_attn_bwd_workspace_bytes bytes (default: new).
    """
    lib = load_library()
    _need_bhnd("q", q, None, dtype=(torch.bfloat16, torch.float32))
    dev = q.device
    B, H, n, D = q.shape
    for name, t in (("k", k), ("v", v), ("out", out), ("dout", dout)):
        _need_bhnd(name, t, dev, dtype=q.dtype, shape=q.shape)
    _need_tensor("lse", lse, dev, dtype=torch.float32, shape=q.shape[:3], contiguous=True)
    st = _call_stream(stream, dev)
    if grads is None:
        grads = tuple(_new(q.shape, q.dtype, dev, st) for _ in range(3))
    if len(grads) != 3:
        _fail("grads must be (dq, dk, dv)")
    for name, t in zip(("dq", "dk", "dv"), grads):
        _need_bhnd(name, t, dev, dtype=q.dtype, shape=q.shape)
    need = int(lib.tra_sparse_attn_bwd_workspace_bytes(B, H, n, D))
    if workspace is None:
        workspace = _new(max(need, 1), torch.uint8, dev, st)
    _need_workspace("workspace", workspace, dev, need)
    descs = [_desc(t) for t in (q, k, v, out, dout)]
    gd = [_desc(t) for t in grads]
    with _on(dev):
        _check(lib.tra_sparse_attn_bwd(
            *(ctypes.byref(d) for d in descs), _ptr(lse), mask.handle,
            *(ctypes.byref(d) for d in gd), _ptr(workspace), workspace.numel(),
            float(scale) if scale else 0.0, _stream_handle(st)), "tra_sparse_attn_bwd")
    return grads


class _SparseAttention(torch.autograd.Function):
    """sparse_attn_fwd as an autograd node: the backward calls
    sparse_attn_bwd with the saved inputs, output and row log-sum-exp."""

    @staticmethod
    def forward(ctx, q, k, v, mask, scale):
        out, lse = sparse_attn_fwd(q, k, v, mask, scale=scale)
        ctx.save_for_backward(q, k, v, out, lse)
        ctx.mask, ctx.scale = mask, scale
        return out

    @staticmethod
    def backward(ctx, dout):
        q, k, v, out, lse = ctx.saved_tensors
        # the upstream gradient may be an expanded or strided view; the
        # kernels read [B, H, N, D] views with unit stride in D
        dq, dk, dv = sparse_attn_bwd(q, k, v, out, lse, dout.contiguous(), ctx.mask, scale=ctx.scale)
        return dq, dk, dv, None, None


def sparse_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, mask: Mask,
                     scale: float | None = None) -> torch.Tensor:
    """Differentiable O = softmax((Q K^T + M) * scale) V: the forward and, when
    autograd asks for them, the gradients of q, k and v, both through the
    library's kernels (tra_sparse_attn_fwd, tra_sparse_attn_bwd; Radial
    Attention page, section 6, trains through a block-sparse backward).
    Same arguments as sparse_attn_fwd; `mask` must stay alive (not freed)
    until the backward has run."""
    return _SparseAttention.apply(q, k, v, mask, scale)


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
        self.device = torch.device("cuda", torch.cuda.current_device())

    @property
    def handle(self):
        if self._h is None:
            raise ValueError("cache was freed")
        return self._h

    def append(self, k: torch.Tensor, v: torch.Tensor, stream=None):
        _need_bhnd("k", k, self.device, dtype=torch.bfloat16, shape=self.shape)
        _need_bhnd("v", v, self.device, dtype=torch.bfloat16, shape=self.shape)
        st = _call_stream(stream, self.device)
        dk, dv = _desc(k), _desc(v)
        with _on(self.device):
            _check(load_library().tra_kvcache_append(self.handle, ctypes.byref(dk), ctypes.byref(dv),
                                                     _stream_handle(st)), "tra_kvcache_append")

    def attn(self, q: torch.Tensor, out: torch.Tensor | None = None, lse: torch.Tensor | bool | None = True,
             scale: float | None = None, stream=None):
        _need_bhnd("q", q, self.device, dtype=torch.bfloat16, shape=self.shape)
        st = _call_stream(stream, self.device)
        if out is None:
            out = _new(q.shape, q.dtype, q.device, st)
        _need_bhnd("out", out, self.device, dtype=torch.bfloat16, shape=self.shape)
        lse = _lse_arg(lse, q, st)
        dq, do = _desc(q), _desc(out)
        with _on(self.device):
            _check(load_library().tra_kvcache_attn(
                self.handle, ctypes.byref(dq), ctypes.byref(do), _ptr(lse),
                float(scale) if scale else 0.0, _stream_handle(st)), "tra_kvcache_attn")
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
    _need_bhnd("q", q, None, dtype=torch.bfloat16)
    dev = q.device
    _need_bhnd("k", k, dev, dtype=torch.bfloat16, shape=q.shape)
    _need_bhnd("v", v, dev, dtype=torch.bfloat16, shape=q.shape)
    B, H, n, D = q.shape
    st = _call_stream(stream, dev)
    need = int(lib.tra_linear_attn_workspace_bytes(B, H, n, D))
    if workspace is None:
        workspace = _new(max(need, 1), torch.uint8, dev, st)
    _need_workspace("workspace", workspace, dev, need)
    if out is None:
        out = _new(q.shape, q.dtype, dev, st)
    _need_bhnd("out", out, dev, dtype=torch.bfloat16, shape=q.shape)
    descs = [_desc(t) for t in (q, k, v, out)]
    with _on(dev):
        _check(lib.tra_linear_attn_fwd(*(ctypes.byref(d) for d in descs), float(eps), _ptr(workspace),
                                       workspace.numel(), _stream_handle(st)), "tra_linear_attn_fwd")
    return out


def linear_attn_workspace_bytes(B: int, H: int, n: int, D: int) -> int:
    return int(load_library().tra_linear_attn_workspace_bytes(B, H, n, D))


def _need_gate_x(x, w):
    if not isinstance(x, torch.Tensor) or x.dim() != 3:
        _fail("expected x as a [B, N, C] tensor")
    _need_tensor("x", x, None, dtype=torch.bfloat16)
    dev = x.device
    B, N, C = x.shape
    _need_tensor("w", w, dev, dtype=torch.bfloat16, shape=(C,), contiguous=True)
    if w.numel() and w.data_ptr() % 16:
        _fail("w data must be 16-byte aligned")
    return dev, B, N, C


def salad_gate(x: torch.Tensor, w: torch.Tensor, bias: float = 0.0, gate: torch.Tensor | None = None,
               workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """SALAD gate on the GPU (see tra_salad_gate): gate[b] = mean over tokens
    of sigmoid(x[b, n] . w + bias).

    x: [B, N, C] bf16 cuda tensor (the block input); w: [C] bf16.  Returns
    `gate` ([B] float32, a new tensor by default).
    """
    lib = load_library()
    dev, B, N, C = _need_gate_x(x, w)
    st = _call_stream(stream, dev)
    need = int(lib.tra_salad_gate_workspace_bytes(B, N))
    if workspace is None:
        workspace = _new(max(need, 256), torch.uint8, dev, st)
    _need_workspace("workspace", workspace, dev, need)
    if gate is None:
        gate = _new((B,), torch.float32, dev, st)
    _need_tensor("gate", gate, dev, dtype=torch.float32, shape=(B,), contiguous=True)
    xd = _desc(x.unsqueeze(1))
    with _on(dev):
        _check(lib.tra_salad_gate(ctypes.byref(xd), _ptr(w), float(bias), _ptr(gate), _ptr(workspace),
                                  workspace.numel(), _stream_handle(st)), "tra_salad_gate")
    return gate


def salad_gate_noalloc(x: torch.Tensor, w: torch.Tensor, bias: float = 0.0, gate: torch.Tensor | None = None,
                       stream=None) -> torch.Tensor:
    """salad_gate without a workspace (see tra_salad_gate_noalloc): the library
    keeps the partial sums in a fixed device array, so the call allocates
    nothing when `gate` is given.  Calls that overlap in time on one device
    race on that array."""
    lib = load_library()
    dev, B, N, C = _need_gate_x(x, w)
    st = _call_stream(stream, dev)
    if gate is None:
        gate = _new((B,), torch.float32, dev, st)
    _need_tensor("gate", gate, dev, dtype=torch.float32, shape=(B,), contiguous=True)
    xd = _desc(x.unsqueeze(1))
    with _on(dev):
        _check(lib.tra_salad_gate_noalloc(ctypes.byref(xd), _ptr(w), float(bias), _ptr(gate), _stream_handle(st)),
               "tra_salad_gate_noalloc")
    return gate


def salad_gate_workspace_bytes(B: int, N: int) -> int:
    return int(load_library().tra_salad_gate_workspace_bytes(B, N))


def probe_mfma_peak(iterations: int = 200000, blocks: int | None = None, stream=None) -> tuple[float, int]:
    """Measured bf16 MFMA peak (see tra_probe_mfma_peak): runs the register-only
    MFMA loop once per compute unit and returns (milliseconds, flops)."""
    lib = load_library()
    dev = torch.device("cuda", torch.cuda.current_device())
    if blocks is None:
        blocks = torch.cuda.get_device_properties(dev).multi_processor_count
    st = _call_stream(stream, dev)
    out = _new((blocks,), torch.float32, dev, st)
    flops = ctypes.c_int64(0)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    _check(lib.tra_probe_mfma_peak(int(iterations), int(blocks), _ptr(out), ctypes.byref(flops),
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
    _need_bhnd("o_sparse", o_sparse, None, dtype=torch.bfloat16)
    dev = o_sparse.device
    B, H, N, D = o_sparse.shape
    C = H * D
    _need_bhnd("o_lin", o_lin, dev, dtype=torch.bfloat16, shape=o_sparse.shape)
    _need_tensor("weight", weight, dev, dtype=torch.bfloat16, shape=(C, C), contiguous=True)
    _need_tensor("gate", gate, dev, dtype=torch.float32, shape=(B,), contiguous=True)
    if bias is not None:
        _need_tensor("bias", bias, dev, dtype=torch.float32, shape=(C,), contiguous=True)
    for name, t in (("weight", weight), ("bias", bias)):
        if t is not None and t.numel() and t.data_ptr() % 16:
            _fail(f"{name} data must be 16-byte aligned")
    st = _call_stream(stream, dev)
    if out is None:
        out = _new(o_sparse.shape, o_sparse.dtype, dev, st)
    _need_bhnd("out", out, dev, dtype=torch.bfloat16, shape=o_sparse.shape)
    descs = [_desc(t) for t in (o_sparse, o_lin, out)]
    with _on(dev):
        _check(lib.tra_salad_combine(ctypes.byref(descs[0]), ctypes.byref(descs[1]), _ptr(weight), _ptr(bias),
                                     _ptr(gate), ctypes.byref(descs[2]), _stream_handle(st)),
               "tra_salad_combine")
    return out
