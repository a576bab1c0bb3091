"""SALAD gate and output on the GPU vs the oracle.

Gate: fp32 sums of bf16 products, compared with the fp64 oracle within 1e-4
(a mean of sigmoids, so values lie in (0, 1)); bitwise reproducible.
Output: out = O_s + g (O_l W^T + bias), bf16 inputs, fp32 accumulation, bf16
output: |out - ref| <= 1e-2 + 1e-2 |ref| per element and relative RMS <= 1e-2
(bf16 output rounding is at most 2^-8 relative).
"""
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


def _arr(t):
    return workloads.to_oracle_array(t)


@pytest.mark.parametrize("B,N,C", [(2, 300, 256), (1, 1, 64), (3, 5000, 1536), (1, 70000, 8)])
def test_gate_parity(tra, B, N, C):
    print(f"[salad gate] B={B} N={N} C={C}", flush=True)
    d = workloads.make_salad_inputs(B, 1, N, C, seed=700 + N + C, device="cuda")
    g1 = tra.salad_gate(d["x"], d["w_gate"], bias=0.25)
    g2 = tra.salad_gate(d["x"], d["w_gate"], bias=0.25)
    torch.cuda.synchronize()
    assert torch.equal(g1, g2)
    ref = oracle.salad_gate(_arr(d["x"]), _arr(d["w_gate"]), 0.25)
    got = g1.cpu().numpy().astype(np.float64)
    print(f"         gate={got} max|dg|={np.abs(got - ref).max():.2e}", flush=True)
    assert np.abs(got - ref).max() <= 1e-4


def _check_out(got, ref):
    err = np.abs(got - ref)
    rel = float(np.sqrt(((got - ref) ** 2).sum() / max((ref ** 2).sum(), 1e-30)))
    print(f"         max|dout|={err.max():.3e} rel-rms={rel:.2e} max|ref|={np.abs(ref).max():.2f}", flush=True)
    assert np.all(err <= 1e-2 + 1e-2 * np.abs(ref)) and rel <= 1e-2


def _merged(t):
    """[B, H, N, D] -> [B * N, H * D] float64 on the host."""
    B, H, N, D = t.shape
    return t.float().permute(0, 2, 1, 3).reshape(B * N, H * D).cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("B,H,N,D,with_bias", [(2, 2, 300, 64, True), (1, 3, 1000, 128, False),
                                               (2, 4, 513, 64, True), (1, 1, 1, 64, True),
                                               (3, 5, 700, 128, True)])
def test_combine_parity(tra, B, H, N, D, with_bias):
    print(f"[salad combine] B={B} H={H} N={N} D={D} bias={with_bias}", flush=True)
    d = workloads.make_salad_inputs(B, H, N, D, seed=800 + N + H, device="cuda")
    bias = d["bias"] if with_bias else None
    out = tra.salad_combine(d["o_s"], d["o_l"], d["W"], d["gate"], bias=bias)
    torch.cuda.synchronize()
    ref = oracle.salad_output_rows(_arr(d["o_s"]), _arr(d["o_l"]), _arr(d["W"]),
                                   None if bias is None else bias.cpu().numpy().astype(np.float64),
                                   d["gate"].cpu().numpy().astype(np.float64))
    _check_out(_merged(out), ref)


def test_combine_in_place_and_strided(tra):
    """out = O_s in place gives the out-of-place result bit for bit; strided
    (non-contiguous head/token) views give the same values."""
    B, H, N, D = 2, 3, 400, 64
    d = workloads.make_salad_inputs(B, H, N, D, seed=901, device="cuda")
    ref = tra.salad_combine(d["o_s"], d["o_l"], d["W"], d["gate"], bias=d["bias"])
    inplace = d["o_s"].clone()
    tra.salad_combine(inplace, d["o_l"], d["W"], d["gate"], bias=d["bias"], out=inplace)
    # [B, N, H, D] storage viewed as [B, H, N, D]
    os_t = d["o_s"].permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    ol_t = d["o_l"].permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    out_t = torch.empty((B, N, H, D), dtype=torch.bfloat16, device="cuda").permute(0, 2, 1, 3)
    tra.salad_combine(os_t, ol_t, d["W"], d["gate"], bias=d["bias"], out=out_t)
    torch.cuda.synchronize()
    assert torch.equal(inplace, ref)
    assert torch.equal(out_t, ref)


def test_combine_headline_shape_sampled(tra):
    """B=1, H=24, N=131072, D=128 (C = 3072, the n = 131072 video's heads),
    sampled token rows against the oracle."""
    B, H, N, D = 1, 24, 131072, 128
    print(f"[salad combine] headline B={B} H={H} N={N} D={D}", flush=True)
    d = workloads.make_salad_inputs(B, H, N, D, seed=1005, device="cuda")
    out = tra.salad_combine(d["o_s"], d["o_l"], d["W"], d["gate"], bias=d["bias"])
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    ns = np.unique(np.concatenate([[0, 1, 255, 256, N - 1], rng.integers(0, N, 19)]))
    rows = np.stack([np.zeros_like(ns), ns], axis=1)
    ref = oracle.salad_output_rows(_arr(d["o_s"]), _arr(d["o_l"]), _arr(d["W"]),
                                   d["bias"].cpu().numpy().astype(np.float64),
                                   d["gate"].cpu().numpy().astype(np.float64), rows=rows)
    got = out[0, :, torch.as_tensor(ns, device="cuda"), :].permute(1, 0, 2).reshape(len(ns), H * D)
    _check_out(got.float().cpu().numpy().astype(np.float64), ref)


def test_salad_errors(tra):
    d = workloads.make_salad_inputs(1, 2, 64, 64, seed=5, device="cuda")
    with pytest.raises(tra.TraError) as e:
        tra.salad_combine(d["o_s"], d["o_l"], d["W"], d["gate"], out=d["o_l"])
    assert e.value.status == -1
    with pytest.raises(tra.TraError) as e:
        tra.salad_gate(d["x"][:, :0], d["w_gate"])
    assert e.value.status == -1
