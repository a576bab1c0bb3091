"""C ABI checks that need no GPU: the library loads, exports every declared
entry point, and rejects bad arguments on the host before any HIP call."""
import ctypes
import glob
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))


@pytest.fixture(scope="module")
def lib():
    import static_sparse_spatiotemporal_amd as tra
    return tra.load_library()


def _declared_functions():
    names = set()
    for header in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(header).read(), flags=re.S)
        names.update(re.findall(r"\b(tra_[a-z_0-9]+)\s*\(", text))
    return sorted(names)


def test_exports_every_declared_symbol(lib):
    assert [os.path.basename(h) for h in HEADERS] == ["tra.h", "tra_debug.h"]
    names = _declared_functions()
    assert "tra_build_mask" in names and "tra_sparse_attn_fwd" in names
    assert "tra_debug_fail_allocations" in names
    for name in names:
        assert hasattr(lib, name), name


def test_allocation_hooks_on_host(lib):
    """The failure-injection setting round-trips (negative = off) and
    setting it allocates and releases nothing."""
    live = lib.tra_debug_live_allocations()
    assert live >= 0
    assert lib.tra_debug_fail_allocations(3) == -1
    assert lib.tra_debug_fail_allocations(-7) == 3
    assert lib.tra_debug_fail_allocations(-1) == -1
    assert lib.tra_debug_live_allocations() == live


def test_status_strings_and_version(lib):
    for code, name in [(0, b"TRA_OK"), (-1, b"TRA_ERR_INVALID"), (-2, b"TRA_ERR_UNSUPPORTED"),
                       (-3, b"TRA_ERR_SHAPE"), (-4, b"TRA_ERR_OOM"), (-5, b"TRA_ERR_HIP")]:
        assert lib.tra_status_string(code) == name
    assert lib.tra_status_string(42) == b"TRA_ERR_UNKNOWN"
    assert lib.tra_version() >= 100
    assert lib.tra_last_hip_error() == 0


def _params(**kw):
    import static_sparse_spatiotemporal_amd as tra
    p = tra.MaskParams()
    p.block = 128
    for k, v in kw.items():
        setattr(p, k, v)
    return p


@pytest.mark.parametrize("f,s,kind,kw,expect", [
    (0, 8, 1, {}, -1),                      # f < 1
    (8, 0, 1, {}, -1),                      # s < 1
    (8, 8, 9, {}, -1),                      # unknown kind
    (8, 8, 1, {"granularity": 5}, -1),      # unknown granularity
    (8, 8, 1, {"block": 64}, -2),           # only 128 x 128 blocks
    (8, 8, 1, {"window": 3}, -1),           # field the family does not use
    (8, 8, 1, {"r_s": 1}, -1),
    (8, 8, 3, {}, -1),                      # SWA needs window >= 1
    (8, 8, 3, {"window": -2}, -1),
    (8, 12, 2, {"grid_h": 3, "grid_w": 5}, -3),   # s != grid_h * grid_w
    (8, 12, 2, {"grid_h": 3, "grid_w": 4, "r_t": -1}, -1),
    (8, 12, 2, {"grid_h": 0, "grid_w": 4}, -1),
    (1 << 20, 1 << 12, 1, {}, -2),          # n >= 2^31
    (8, 8, 1, {"sink_frames": -1}, -1),     # negative sink
    (8, 256, 3, {"granularity": 2, "window": 2}, -1),  # eq. 4 on blocks is radial only
    (8, 200, 1, {"granularity": 2}, -2),    # ... and needs s % 128 == 0
    (8, 8, 1, {"granularity": 3}, -1),      # unknown granularity
])
def test_build_mask_rejects_on_host(lib, f, s, kind, kw, expect):
    out = ctypes.c_void_p(123)
    p = _params(**kw)
    st = lib.tra_build_mask(f, s, kind, ctypes.byref(p), None, ctypes.byref(out))
    assert st == expect
    assert out.value is None


def test_build_mask_null_arguments(lib):
    p = _params()
    assert lib.tra_build_mask(8, 8, 1, ctypes.byref(p), None, None) == -1
    out = ctypes.c_void_p()
    assert lib.tra_build_mask(8, 8, 1, None, None, ctypes.byref(out)) == -1
    p.reserved[3] = 1
    assert lib.tra_build_mask(8, 8, 1, ctypes.byref(p), None, ctypes.byref(out)) == -1


def test_null_handles(lib):
    import static_sparse_spatiotemporal_amd as tra
    info = tra.MaskInfo()
    assert lib.tra_mask_get_info(None, ctypes.byref(info)) == -1
    assert lib.tra_mask_export(None, None, None, None, None, None, None) == -1
    lib.tra_mask_free(None)
    t = tra.TensorDesc()
    assert lib.tra_sparse_attn_fwd(None, None, None, None, None, None, 0.0, None) == -1
    assert lib.tra_sparse_attn_fwd(ctypes.byref(t), ctypes.byref(t), ctypes.byref(t), None,
                                   ctypes.byref(t), None, 0.0, None) == -1


def test_oracle_and_product_are_independent():
    """The product package never imports or includes the oracle, and the
    oracle never imports or includes the product; only the workload
    generators are shared."""
    imp_oracle = re.compile(r"^\s*(import\s+oracle|from\s+oracle\b)|#\s*include\s*\"oracle\.h\"", re.M)
    imp_prod = re.compile(r"^\s*(import|from)\s+static_sparse_spatiotemporal_amd\b|#\s*include\s*\"tra(_internal)?\.h\"", re.M)
    pkg = os.path.join(ROOT, "static_sparse_spatiotemporal_amd")
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".cpp", ".hip", ".h")):
                assert not imp_oracle.search(open(os.path.join(dirpath, fn)).read()), fn
    for fn in os.listdir(os.path.join(ROOT, "oracle")):
        if fn.endswith((".py", ".c", ".h")):
            assert not imp_prod.search(open(os.path.join(ROOT, "oracle", fn)).read()), fn
    wl = open(os.path.join(ROOT, "workloads", "__init__.py")).read()
    assert not imp_oracle.search(wl) and not imp_prod.search(wl)


def _tdesc(B=1, H=1, N=128, D=64, dtype=1, data=0x10000):
    import static_sparse_spatiotemporal_amd as tra
    t = tra.TensorDesc()
    t.data = data
    t.dtype = dtype
    t.B, t.H, t.N, t.D = B, H, N, D
    for i, st in enumerate((H * N * D, N * D, D, 1)):
        t.stride[i] = st
    return t


def test_bwd_rejects_on_host(lib):
    t = _tdesc()
    r = ctypes.byref
    assert lib.tra_sparse_attn_bwd(None, r(t), r(t), r(t), r(t), None, None, r(t), r(t), r(t), None, 0, 0.0,
                                   None) == -1
    assert lib.tra_sparse_attn_bwd(r(t), r(t), r(t), r(t), r(t), None, None, r(t), r(t), r(t), None, 0, 0.0,
                                   None) == -1
    # workspace size: two fp32 values per row, parts 256-byte aligned
    assert lib.tra_sparse_attn_bwd_workspace_bytes(1, 2, 100, 128) == 1024 + 1024
    assert lib.tra_sparse_attn_bwd_workspace_bytes(1, 24, 131072, 128) == 24 * 131072 * 8
    assert lib.tra_sparse_attn_bwd_workspace_bytes(1, 1, 10, 96) == 0
    assert lib.tra_sparse_attn_bwd_workspace_bytes(-1, 1, 10, 64) == 0


def test_probe_rejects_on_host(lib):
    flops = ctypes.c_int64(0)
    out = ctypes.c_void_p(16)
    assert lib.tra_probe_mfma_peak(0, 1, out, ctypes.byref(flops), None) == -1
    assert lib.tra_probe_mfma_peak(10, 0, out, ctypes.byref(flops), None) == -1
    assert lib.tra_probe_mfma_peak(10, 1, None, ctypes.byref(flops), None) == -1
    assert lib.tra_probe_mfma_peak(10, 1, out, None, None) == -1


def test_kvcache_rejects_on_host(lib):
    out = ctypes.c_void_p(7)
    assert lib.tra_kvcache_create(1, 1, 128, 64, 4, 1, None) == -1
    assert lib.tra_kvcache_create(0, 1, 128, 64, 4, 1, ctypes.byref(out)) == -1 and out.value is None
    assert lib.tra_kvcache_create(1, 1, 128, 64, 0, 1, ctypes.byref(out)) == -1
    assert lib.tra_kvcache_create(1, 1, 100, 64, 4, 1, ctypes.byref(out)) == -2  # s % 128 != 0
    assert lib.tra_kvcache_create(1, 1, 128, 96, 4, 1, ctypes.byref(out)) == -2  # D
    assert lib.tra_kvcache_create(1, 1, 128, 64, 4, 0, ctypes.byref(out)) == -2  # fp32
    t = _tdesc()
    assert lib.tra_kvcache_append(None, ctypes.byref(t), ctypes.byref(t), None) == -1
    assert lib.tra_kvcache_attn(None, ctypes.byref(t), ctypes.byref(t), None, 0.0, None) == -1
    assert lib.tra_kvcache_get_frames(None, None, None) == -1
    assert lib.tra_kvcache_reset(None) == -1
    lib.tra_kvcache_free(None)


def test_linear_rejects_on_host(lib):
    r = ctypes.byref
    assert lib.tra_linear_attn_workspace_bytes(1, 1, 128, 96) == 0
    assert lib.tra_linear_attn_workspace_bytes(2, 3, 300, 64) > 0
    t = _tdesc()
    f = _tdesc(dtype=0)
    assert lib.tra_linear_attn_fwd(None, r(t), r(t), r(t), 1e-6, None, 0, None) == -1
    assert lib.tra_linear_attn_fwd(r(f), r(f), r(f), r(f), 1e-6, None, 0, None) == -2
    assert lib.tra_linear_attn_fwd(r(t), r(t), r(t), r(t), 1e-6, None, 0, None) == -1      # no workspace
    assert lib.tra_linear_attn_fwd(r(t), r(t), r(t), r(t), -1.0, None, 0, None) == -1      # eps < 0
    odd = _tdesc(N=129)
    assert lib.tra_linear_attn_fwd(r(t), r(odd), r(t), r(t), 1e-6, None, 0, None) == -3   # shapes differ
    empty = _tdesc(N=0, data=0)
    assert lib.tra_linear_attn_fwd(r(empty), r(empty), r(empty), r(empty), 1e-6, None, 0, None) == 0


def test_salad_rejects_on_host(lib):
    r = ctypes.byref
    assert lib.tra_salad_gate_workspace_bytes(-1, 10) == 0
    assert lib.tra_salad_gate_workspace_bytes(2, 300) % 256 == 0 and lib.tra_salad_gate_workspace_bytes(2, 300) > 0
    x = _tdesc(B=2, H=1, N=300, D=256)
    w = ctypes.c_void_p(0x20000)
    g = ctypes.c_void_p(0x30000)
    assert lib.tra_salad_gate(None, w, 0.0, g, None, 0, None) == -1
    assert lib.tra_salad_gate(r(_tdesc(B=2, H=2, N=300, D=256)), w, 0.0, g, None, 0, None) == -3   # H != 1
    assert lib.tra_salad_gate(r(_tdesc(B=2, H=1, N=300, D=256, dtype=0)), w, 0.0, g, None, 0, None) == -2
    assert lib.tra_salad_gate(r(_tdesc(B=2, H=1, N=300, D=12)), w, 0.0, g, None, 0, None) == -2    # C % 8
    assert lib.tra_salad_gate(r(_tdesc(B=2, H=1, N=0, D=256)), w, 0.0, g, None, 0, None) == -1     # mean of none
    assert lib.tra_salad_gate(r(_tdesc(B=0, H=1, N=5, D=256)), w, 0.0, g, None, 0, None) == 0      # nothing to do
    assert lib.tra_salad_gate(r(x), None, 0.0, g, None, 0, None) == -1
    assert lib.tra_salad_gate(r(x), w, 0.0, None, None, 0, None) == -1
    assert lib.tra_salad_gate(r(_tdesc(B=2, H=1, N=300, D=256, data=0x10002)), w, 0.0, g, None, 0, None) == -2
    assert lib.tra_salad_gate(r(x), w, 0.0, g, None, 0, None) == -1                                  # no workspace

    t = _tdesc(B=1, H=2, N=300, D=64)
    other = _tdesc(B=1, H=2, N=300, D=64, data=0x40000)
    out = _tdesc(B=1, H=2, N=300, D=64, data=0x50000)
    W = ctypes.c_void_p(0x60000)
    assert lib.tra_salad_combine(None, r(other), W, None, g, r(out), None) == -1
    assert lib.tra_salad_combine(r(_tdesc(B=1, H=2, N=300, D=64, dtype=0)), r(other), W, None, g, r(out), None) == -2
    assert lib.tra_salad_combine(r(t), r(_tdesc(B=1, H=2, N=301, D=64, data=0x40000)), W, None, g, r(out), None) == -3
    assert lib.tra_salad_combine(r(_tdesc(B=1, H=2, N=300, D=96)), r(_tdesc(B=1, H=2, N=300, D=96, data=0x40000)),
                                 W, None, g, r(_tdesc(B=1, H=2, N=300, D=96, data=0x50000)), None) == -2  # D
    assert lib.tra_salad_combine(r(t), r(other), None, None, g, r(out), None) == -1                # no W
    assert lib.tra_salad_combine(r(t), r(other), W, None, None, r(out), None) == -1                # no gate
    assert lib.tra_salad_combine(r(t), r(other), W, None, g, r(_tdesc(B=1, H=2, N=300, D=64, data=0x40000)),
                                 None) == -1                                                        # out is O_lin
    assert lib.tra_salad_combine(r(t), r(other), W, ctypes.c_void_p(0x70004), g, r(out), None) == -2  # bias align
    empty = [_tdesc(B=1, H=2, N=0, D=64, data=0) for _ in range(3)]
    assert lib.tra_salad_combine(r(empty[0]), r(empty[1]), None, None, None, r(empty[2]), None) == 0
