"""Error paths of the allocating entry points, driven by failure injection.

tra_build_mask makes about 27 device allocations and tra_kvcache_create 4;
a failure at any of them must return TRA_ERR_OOM, release everything the
call had allocated so far, and leave the library able to build the same
object afterwards.  The injection (include/tra_debug.h) makes the k-th
allocation fail for k = 0, 1, ... until the call goes through.
"""
import ctypes

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

TRA_OK, TRA_ERR_OOM = 0, -4


@pytest.fixture(scope="module")
def tra():
    import static_sparse_spatiotemporal_amd as m
    assert torch.cuda.is_available()
    m.load_library()
    return m


@pytest.fixture
def lib(tra):
    lib = tra.load_library()
    yield lib
    lib.tra_debug_fail_allocations(-1)


def _sweep(lib, call, release, max_allocs=64):
    """Run `call` with the k-th allocation failing for k = 0, 1, ...; return
    the k at which it first succeeds (its allocation count)."""
    base = lib.tra_debug_live_allocations()
    for k in range(max_allocs):
        lib.tra_debug_fail_allocations(k)
        st, obj = call()
        lib.tra_debug_fail_allocations(-1)
        torch.cuda.synchronize()
        if st == TRA_OK:
            # the object keeps its buffers (a mask frees its build temporaries)
            assert base < lib.tra_debug_live_allocations() <= base + k, k
            release(obj)
            assert lib.tra_debug_live_allocations() == base
            return k
        assert st == TRA_ERR_OOM, (k, st)
        assert lib.tra_last_hip_error() == 2, k  # hipErrorOutOfMemory
        assert lib.tra_debug_live_allocations() == base, f"leak after failure at allocation {k}"
    raise AssertionError(f"no success within {max_allocs} allocations")


@pytest.mark.parametrize("f,s,kind,kw", [
    (8, 256, "radial", dict(granularity="element")),
    (16, 384, "radial", dict(granularity="block_any", sink_frames=1)),
    (8, 256, "radius3d", dict(grid_h=16, grid_w=16, r_t=1, r_s=4)),
    (12, 256, "swa", dict(window=4)),
])
def test_build_mask_releases_everything_on_failure(tra, lib, f, s, kind, kw):
    print(f"[alloc] build_mask {kind} f={f} s={s}", flush=True)
    p = tra.MaskParams()
    p.granularity = tra.GRANULARITIES[kw.get("granularity", "element")]
    p.block = 128
    p.grid_h, p.grid_w = kw.get("grid_h", 0), kw.get("grid_w", 0)
    p.r_t, p.r_s, p.window = kw.get("r_t", 0), kw.get("r_s", 0), kw.get("window", 0)
    p.sink_frames = kw.get("sink_frames", 0)

    def call():
        h = ctypes.c_void_p()
        st = lib.tra_build_mask(f, s, tra.KINDS[kind], ctypes.byref(p), None, ctypes.byref(h))
        return st, h

    n = _sweep(lib, call, lambda h: lib.tra_mask_free(h))
    assert 20 <= n <= 30
    # the mask built after the failures is the same as a plain build
    ref = tra.build_mask(f, s, kind, **kw)
    again = tra.build_mask(f, s, kind, **kw)
    a, b = ref.export(), again.export()
    assert ref.info == again.info
    for key in a:
        assert np.array_equal(a[key], b[key]), key
    ref.free()
    again.free()


def test_kvcache_create_releases_everything_on_failure(tra, lib):
    print("[alloc] kvcache_create", flush=True)

    def call():
        h = ctypes.c_void_p()
        st = lib.tra_kvcache_create(1, 2, 256, 64, 3, 1, ctypes.byref(h))
        return st, h

    n = _sweep(lib, call, lambda h: lib.tra_kvcache_free(h))
    assert n == 4
