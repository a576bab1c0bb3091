"""Argument checks of the binding through its public functions, on the GPU.

Every tensor a call hands to the library (outputs, LSE, gradients,
workspaces, weights, bias, gate) is checked for device, dtype, shape and
layout before the call: a bad one raises ValueError and nothing is launched.
Default buffers are allocated for the call's stream, so a call on a side
stream that drops them gives the same results as one on the current stream.
"""
import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tra():
    import static_sparse_spatiotemporal_amd as m
    assert torch.cuda.is_available()
    m.load_library()
    return m


@pytest.fixture(scope="module")
def case(tra):
    w = workloads.Workload("radial_f4_s128", "radial", "element", 4, 128, 1, 2, 64, "bf16", seed=5)
    q, k, v = workloads.make_qkv(w, device="cuda")
    mask = tra.build_mask(w.f, w.s, w.kind)
    yield w, q, k, v, mask
    mask.free()


def test_forward_outputs_checked(tra, case):
    print("[args] forward", flush=True)
    w, q, k, v, mask = case
    bad_out = [torch.empty_like(q, device="cpu"), torch.empty_like(q, dtype=torch.float32),
               torch.empty_like(q)[:, :1], torch.empty(1, 2, w.n, 72, dtype=q.dtype, device="cuda")[..., 4:68]]
    for out in bad_out:
        with pytest.raises(ValueError):
            tra.sparse_attn_fwd(q, k, v, mask, out=out)
    bad_lse = [torch.empty(q.shape[:3]), torch.empty(q.shape[:3], dtype=torch.bfloat16, device="cuda"),
               torch.empty(1, 2, w.n - 1, device="cuda"), torch.empty(1, w.n, 2, device="cuda").transpose(1, 2)]
    for lse in bad_lse:
        with pytest.raises(ValueError):
            tra.sparse_attn_fwd(q, k, v, mask, lse=lse)
    with pytest.raises(ValueError, match="k is on cpu"):
        tra.sparse_attn_fwd(q, k.cpu(), v, mask)
    with pytest.raises(ValueError, match="HIP device"):
        tra.sparse_attn_fwd(q.cpu(), k, v, mask)


def test_backward_arguments_checked(tra, case):
    print("[args] backward", flush=True)
    w, q, k, v, mask = case
    out, lse = tra.sparse_attn_fwd(q, k, v, mask)
    dout = torch.randn_like(q)
    with pytest.raises(ValueError, match="lse"):
        tra.sparse_attn_bwd(q, k, v, out, lse.cpu(), dout, mask)
    with pytest.raises(ValueError, match="dout"):
        tra.sparse_attn_bwd(q, k, v, out, lse, dout.float(), mask)
    grads = [torch.empty_like(q) for _ in range(3)]
    for i, bad in enumerate((torch.empty_like(q, device="cpu"), torch.empty_like(q)[:, :, :64],
                             torch.empty_like(q, dtype=torch.float32))):
        g = list(grads)
        g[i] = bad
        with pytest.raises(ValueError):
            tra.sparse_attn_bwd(q, k, v, out, lse, dout, mask, grads=tuple(g))
    with pytest.raises(ValueError, match="workspace"):
        tra.sparse_attn_bwd(q, k, v, out, lse, dout, mask, workspace=torch.empty(1 << 20, dtype=torch.uint8))


def test_linear_and_salad_arguments_checked(tra, case):
    print("[args] linear branch and SALAD", flush=True)
    w, q, k, v, mask = case
    with pytest.raises(ValueError, match="out"):
        tra.linear_attn_fwd(q, k, v, out=torch.empty_like(q, device="cpu"))
    need = tra.linear_attn_workspace_bytes(*q.shape)
    with pytest.raises(ValueError, match="holds"):
        tra.linear_attn_fwd(q, k, v, workspace=torch.empty(need - 1, dtype=torch.uint8, device="cuda"))
    B, H, N, D = q.shape
    C = H * D
    x = torch.randn(B, N, C, device="cuda").to(torch.bfloat16)
    wg = torch.randn(C, device="cuda").to(torch.bfloat16)
    with pytest.raises(ValueError, match="w"):
        tra.salad_gate(x, wg.float())
    with pytest.raises(ValueError, match="gate"):
        tra.salad_gate(x, wg, gate=torch.empty(B, dtype=torch.float64, device="cuda"))
    gate = tra.salad_gate(x, wg)
    W = torch.randn(C, C, device="cuda").to(torch.bfloat16)
    bias = torch.randn(C, device="cuda")
    bad = [dict(weight=W.float()), dict(weight=W[:, :C // 2]), dict(weight=W.t()),
           dict(bias=bias.to(torch.bfloat16)), dict(bias=bias[:C // 2]), dict(bias=bias.cpu()),
           dict(gate=gate.to(torch.bfloat16)), dict(gate=torch.empty(B + 1, device="cuda")),
           dict(out=torch.empty_like(q, dtype=torch.float32))]
    for kw in bad:
        args = dict(weight=W, bias=bias, gate=gate)
        args.update(kw)
        with pytest.raises(ValueError):
            tra.salad_combine(q, q, args["weight"], args["gate"], bias=args["bias"], out=args.get("out"))


def test_side_stream_defaults(tra, case):
    """Calls on a side stream with every buffer left to the binding (outputs
    and workspaces, the latter dropped at return) match the same calls on the
    current stream bit for bit."""
    print("[args] side stream", flush=True)
    w, q, k, v, mask = case
    dout = torch.randn_like(q)
    ref_o, ref_l = tra.sparse_attn_fwd(q, k, v, mask)
    ref_g = tra.sparse_attn_bwd(q, k, v, ref_o, ref_l, dout, mask)
    ref_lin = tra.linear_attn_fwd(q, k, v)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    o, l = tra.sparse_attn_fwd(q, k, v, mask, stream=side)
    g = tra.sparse_attn_bwd(q, k, v, o, l, dout, mask, stream=side)
    lin = tra.linear_attn_fwd(q, k, v, stream=side)
    # allocations on the current stream meanwhile must not take the side
    # stream's dropped workspaces
    junk = [torch.full((1 << 20,), 7, dtype=torch.uint8, device="cuda") for _ in range(8)]
    side.synchronize()
    torch.cuda.synchronize()
    del junk
    assert torch.equal(o, ref_o) and torch.equal(l, ref_l) and torch.equal(lin, ref_lin)
    assert all(torch.equal(a, b) for a, b in zip(g, ref_g))
