"""The gate entry point that allocates nothing, through the C ABI.

tra_salad_gate_noalloc keeps the gate's partial sums in a fixed device array
of the library instead of a caller workspace.  It must give the workspace
entry point's result bit for bit (same kernels, same summation order), also
on a second call with a smaller input after a larger one (the array keeps the
previous call's contents), and refuse requests past its limit before
enqueuing anything.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tra():
    import static_sparse_spatiotemporal_amd as m
    assert torch.cuda.is_available()
    m.load_library()
    return m


def _x_desc(tra, x):
    return tra._desc(x.unsqueeze(1))  # [B, 1, N, C]


def _gate_noalloc_abi(tra, x, w, bias):
    lib = tra.load_library()
    gate = torch.full((x.shape[0],), float("nan"), dtype=torch.float32, device="cuda")
    d = _x_desc(tra, x)
    st = lib.tra_salad_gate_noalloc(ctypes.byref(d), ctypes.c_void_p(w.data_ptr()), float(bias),
                                    ctypes.c_void_p(gate.data_ptr()), None)
    assert st == 0, st
    return gate


def _gate_workspace_abi(tra, x, w, bias):
    lib = tra.load_library()
    B, N, _ = x.shape
    gate = torch.full((B,), float("nan"), dtype=torch.float32, device="cuda")
    need = int(lib.tra_salad_gate_workspace_bytes(B, N))
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
    d = _x_desc(tra, x)
    st = lib.tra_salad_gate(ctypes.byref(d), ctypes.c_void_p(w.data_ptr()), float(bias),
                            ctypes.c_void_p(gate.data_ptr()), ctypes.c_void_p(ws.data_ptr()), ws.numel(), None)
    assert st == 0, st
    return gate


def test_noalloc_gate_matches_workspace_gate(tra):
    """Two calls in a row (the second smaller: fewer samples and parts, so the
    array still holds the first call's partial sums past its range), each
    equal bit for bit to the workspace entry point and within 1e-4 of the
    fp64 oracle."""
    for B, N, C, seed in ((5, 20000, 1536, 11), (2, 300, 256, 12)):
        print(f"[noalloc gate] B={B} N={N} C={C}", flush=True)
        d = workloads.make_salad_inputs(B, 1, N, C, seed=seed, device="cuda")
        got = _gate_noalloc_abi(tra, d["x"], d["w_gate"], 0.3)
        ref = _gate_workspace_abi(tra, d["x"], d["w_gate"], 0.3)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), (got, ref)
        want = oracle.salad_gate(workloads.to_oracle_array(d["x"]), workloads.to_oracle_array(d["w_gate"]), 0.3)
        assert np.abs(got.cpu().numpy().astype(np.float64) - want).max() <= 1e-4
    # the binding's wrapper calls the same entry point
    again = tra.salad_gate_noalloc(d["x"], d["w_gate"], 0.3)
    torch.cuda.synchronize()
    assert torch.equal(again, ref)


def test_noalloc_gate_limit_is_refused_on_host(tra):
    """B * min(1024, ceil(N / 64)) above 65536 partial sums is refused before
    anything is enqueued (a stride-0 view stands for the large input)."""
    lib = tra.load_library()
    row = torch.zeros(8, dtype=torch.bfloat16, device="cuda")
    w = torch.zeros(8, dtype=torch.bfloat16, device="cuda")
    gate = torch.zeros(65, dtype=torch.float32, device="cuda")
    x = row.as_strided((65, 65536, 8), (0, 0, 1))
    d = _x_desc(tra, x)
    st = lib.tra_salad_gate_noalloc(ctypes.byref(d), ctypes.c_void_p(w.data_ptr()), 0.0,
                                    ctypes.c_void_p(gate.data_ptr()), None)
    assert st == -2
    x = row.as_strided((64, 65536, 8), (0, 0, 1))  # exactly at the limit: accepted
    d = _x_desc(tra, x)
    st = lib.tra_salad_gate_noalloc(ctypes.byref(d), ctypes.c_void_p(w.data_ptr()), 0.0,
                                    ctypes.c_void_p(gate.data_ptr()), None)
    torch.cuda.synchronize()
    assert st == 0
    # every token scores sigmoid(0) = 1/2
    assert torch.equal(gate[:64], torch.full((64,), 0.5, device="cuda"))
