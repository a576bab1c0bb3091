"""Argument checks of the Python binding, on the CPU.

The C ABI takes raw pointers: a host tensor, a tensor of the wrong dtype or
one that is too small would reach a kernel as a bad address.  The binding
checks every tensor before it calls into the library.  These tests run
without a GPU: the library handle is replaced by one that fails the test on
any call, so a check that let a bad argument through would be seen.  The
checks of the tensors after the first one (same device, dtype, shape,
layout) are exercised through the helpers with the CPU as the call's device;
tests/test_gpu_args.py repeats them through the public functions on a GPU.
"""
import pytest
import torch

import static_sparse_spatiotemporal_amd as tra


class _NoCalls:
    """Stands in for libtra.so: any use of it is a test failure."""

    def __getattr__(self, name):
        raise AssertionError(f"the binding called {name} with a bad argument")


@pytest.fixture
def no_lib(monkeypatch):
    monkeypatch.setattr(tra, "_lib", _NoCalls())


class _FakeMask:
    handle = None


def _host(*shape, dtype=torch.bfloat16):
    return torch.zeros(*shape, dtype=dtype)


def test_host_tensors_are_refused_before_any_call(no_lib):
    q = _host(1, 2, 256, 64)
    m = _FakeMask()
    with pytest.raises(ValueError, match="HIP device"):
        tra.sparse_attn_fwd(q, q, q, m)
    with pytest.raises(ValueError, match="HIP device"):
        tra.sparse_attention(q, q, q, m)
    with pytest.raises(ValueError, match="HIP device"):
        tra.sparse_attn_bwd(q, q, q, q, _host(1, 2, 256, dtype=torch.float32), q, m)
    with pytest.raises(ValueError, match="HIP device"):
        tra.linear_attn_fwd(q, q, q)
    with pytest.raises(ValueError, match="HIP device"):
        tra.salad_gate(_host(2, 256, 128), _host(128))
    with pytest.raises(ValueError, match="HIP device"):
        tra.salad_combine(q, q, _host(128, 128), _host(1, dtype=torch.float32))


def test_non_tensors_are_refused(no_lib):
    with pytest.raises(ValueError, match="torch.Tensor"):
        tra.sparse_attn_fwd(None, None, None, _FakeMask())
    with pytest.raises(ValueError, match="\\[B, N, C\\]"):
        tra.salad_gate(_host(256, 128), _host(128))


CPU = torch.device("cpu")


def test_device_dtype_shape_and_contiguity():
    t = _host(1, 2, 256, 64)
    assert tra._need_tensor("t", t, CPU, dtype=torch.bfloat16, shape=(1, 2, 256, 64)) is t
    with pytest.raises(ValueError, match="is on cpu, the call runs on meta"):
        tra._need_tensor("t", t, torch.device("meta"))
    with pytest.raises(ValueError, match="dtype"):
        tra._need_tensor("lse", t, CPU, dtype=torch.float32)
    with pytest.raises(ValueError, match="dtype"):
        tra._need_tensor("q", t.float(), CPU, dtype=(torch.bfloat16, torch.float16))
    with pytest.raises(ValueError, match="shape"):
        tra._need_tensor("out", t, CPU, shape=(1, 2, 128, 64))
    with pytest.raises(ValueError, match="contiguous"):
        tra._need_tensor("lse", t.transpose(1, 2), CPU, contiguous=True)


def test_bhnd_layout_rules():
    base = _host(1, 2, 256, 72)
    ok = base[..., :64]                       # row pitch 72 elements = 144 bytes
    assert tra._need_bhnd("k", ok, CPU) is ok
    with pytest.raises(ValueError, match="\\[B, H, N, D\\]"):
        tra._need_bhnd("k", _host(2, 256, 64), CPU)
    with pytest.raises(ValueError, match="unit stride"):
        tra._need_bhnd("k", _host(1, 2, 64, 256).transpose(2, 3), CPU)
    with pytest.raises(ValueError, match="multiples of 8"):
        tra._need_bhnd("k", _host(1, 2, 256, 68)[..., :64], CPU)
    with pytest.raises(ValueError, match="multiples of 4"):
        tra._need_bhnd("k", _host(1, 2, 256, 66, dtype=torch.float32)[..., :64], CPU)
    with pytest.raises(ValueError, match="16-byte aligned"):
        tra._need_bhnd("k", _host(1, 2, 256, 72)[..., 4:68], CPU)
    empty = _host(0, 2, 256, 64)
    assert tra._need_bhnd("q", empty, CPU) is empty


def test_workspace_rules():
    raw = torch.zeros(4096 + 512, dtype=torch.uint8)
    a0 = (-raw.data_ptr()) % 256          # first 256-byte boundary
    ws = raw[a0:a0 + 4096]
    assert tra._need_workspace("workspace", ws, CPU, 4096) is ws
    with pytest.raises(ValueError, match="holds 4095 bytes, the call needs 4096"):
        tra._need_workspace("workspace", ws[:4095], CPU, 4096)
    with pytest.raises(ValueError, match="dtype"):
        tra._need_workspace("workspace", ws.view(torch.int32), CPU, 16)
    with pytest.raises(ValueError, match="256-byte aligned"):
        tra._need_workspace("workspace", ws[16:16 + 512], CPU, 512)


def test_stream_argument():
    with pytest.raises(ValueError, match="torch.cuda.Stream"):
        tra._call_stream(object(), torch.device("cuda", 0))
