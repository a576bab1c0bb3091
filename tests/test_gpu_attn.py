"""GPU attention vs the fp64 oracle through the C ABI.

Tolerances (max |O_gpu - O_oracle| over compared elements): 1e-4 for fp32
inputs, 2e-2 for bf16 inputs with fp32 accumulation.  LSE: per row
min(T, 0.5 ln(1 + 128 / K)) with K the row's kept keys and T = 1e-4 (fp32),
1e-3 (bf16) (tests/tolerance.py: half the smallest LSE move of one dropped or
added 128-key block).  The Q = 0 probe pins the mask the kernel applied: with
every score 0 the softmax is uniform over the kept keys, so LSE = ln(#kept
keys) and O = mean of V over them, at any size.
"""
import ctypes
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests import expected
from tests.tolerance import TOL_O, TOL_LSE_EXACT, lse_tol

pytestmark = pytest.mark.gpu



@pytest.fixture(scope="module")
def tra():
    import static_sparse_spatiotemporal_amd as m
    assert torch.cuda.is_available()
    m.load_library()
    return m


def spec_of(w: workloads.Workload) -> oracle.MaskSpec:
    return oracle.MaskSpec(w.kind, w.f, w.s, granularity=w.granularity, grid_h=w.grid_h,
                           grid_w=w.grid_w, r_t=w.r_t, r_s=w.r_s, window=w.window,
                           sink_frames=w.sink_frames)


def build(tra, w):
    return tra.build_mask(w.f, w.s, w.kind, **w.mask_kwargs())


def run_and_compare(tra, w, q, k, v, rows=None, mask=None, block_keep=None, tag=""):
    """Runs the kernel, then the oracle on `rows` (None = all).  Returns
    (max |dO|, max |dLSE| / per-row LSE tolerance, O, LSE)."""
    print(f"[attn] {w.name}{tag} B={w.B} H={w.H} n={w.n} D={w.D} {w.dtype}", flush=True)
    own = mask is None
    if own:
        mask = build(tra, w)
    out, lse = tra.sparse_attn_fwd(q, k, v, mask)
    torch.cuda.synchronize()
    spec = spec_of(w)
    if spec.granularity == "block_any" and block_keep is None:
        block_keep = expected.cached_block_counts(spec) > 0
    if rows is None:
        ref_o, ref_l = oracle.attention_rows(*(workloads.to_oracle_array(x) for x in (q, k, v)), spec,
                                             block_keep=block_keep)
        got_o = out.float().cpu().numpy().reshape(-1, w.D)
        got_l = lse.cpu().numpy().reshape(-1)
    else:
        # only the sampled heads travel to the host
        heads = sorted(set((int(b), int(h)) for b, h, _ in rows))
        index = {bh: i for i, bh in enumerate(heads)}
        sel = lambda x: torch.stack([x[b, h] for b, h in heads])[None]
        arrs = [workloads.to_oracle_array(sel(x)) for x in (q, k, v)]
        sub_rows = np.array([(0, index[(int(b), int(h))], int(qq)) for b, h, qq in rows], dtype=np.int64)
        ref_o, ref_l = oracle.attention_rows(*arrs, spec, rows=sub_rows, block_keep=block_keep)
        bi, hi, qi = (torch.as_tensor(rows[:, i], device=out.device) for i in range(3))
        got_o = out[bi, hi, qi].float().cpu().numpy()
        got_l = lse[bi, hi, qi].cpu().numpy()
    if own:
        mask.free()
    err_o = float(np.abs(got_o - ref_o).max())
    dl = np.abs(got_l - ref_l)
    queries = np.tile(np.arange(w.n), w.B * w.H) if rows is None else rows[:, 2]
    tol = lse_tol(spec, w.dtype, queries, block_keep=block_keep)
    ratio = float((dl / tol).max())
    print(f"       max|dO|={err_o:.3e} max|dLSE|={float(dl.max()):.3e} (max/tol {ratio:.3f}) "
          f"rows={ref_o.shape[0]}", flush=True)
    return err_o, ratio, out, lse


SMALL = ["radial_f8_s64_fp32", "radius3d_t8_h16_w16"]
LARGE = ["swa_f64_s256_w16", "radial_f20_s1536_block", "radial_f128_s1024_block",
         "radial_f128_s1024_block_eq4"]


@pytest.mark.parametrize("name", SMALL)
def test_workload_full_parity(tra, name):
    w = workloads.WORKLOADS[name]
    q, k, v = workloads.make_qkv(w, device="cuda")
    eo, el, _, _ = run_and_compare(tra, w, q, k, v)
    assert eo <= TOL_O[w.dtype] and el <= 1


@pytest.mark.parametrize("name", LARGE)
def test_workload_sampled_parity(tra, name):
    """Full-size inputs in the benchmark's launch configuration; the oracle
    recomputes sampled rows one by one."""
    w = workloads.WORKLOADS[name]
    q, k, v = workloads.make_qkv(w, device="cuda")
    rows = expected.sample_rows(w.n, w.B, w.H, heads_per_batch=2, blocks=4, seed=w.seed)
    eo, el, _, _ = run_and_compare(tra, w, q, k, v, rows=rows)
    assert eo <= TOL_O[w.dtype] and el <= 1


@pytest.mark.parametrize("name", ["radius3d_t8_h16_w16", "swa_f64_s256_w16", "radial_f20_s1536_block",
                                  "radial_f128_s1024_block", "radial_f128_s1024_block_eq4"])
def test_zero_query_probe(tra, name):
    """Q = 0: LSE of every row must be ln(#kept keys of that row) (exact in
    fp32 below 2^24 keys), O the mean of V over them (sampled rows)."""
    w = workloads.WORKLOADS[name]
    _, k, v = workloads.make_qkv(w, device="cuda")
    q = torch.zeros_like(k)
    spec = spec_of(w)
    mask = build(tra, w)
    out, lse = tra.sparse_attn_fwd(q, k, v, mask)
    torch.cuda.synchronize()
    print(f"[q0] {name}", flush=True)
    if spec.granularity != "element":
        counts, cls = expected.block_classes(spec, expected.cached_block_counts(spec))
        kept = expected.kept_keys_per_row(spec, cls)
    elif spec.kind == "swa":
        i = np.arange(spec.n) // spec.s
        kept = spec.s * (i - np.maximum(0, i - spec.window + 1) + 1)
        for qq in (0, spec.n // 2 + 3, spec.n - 1):  # the closed form against the predicate
            assert kept[qq] == sum(oracle.keep(spec, qq, t) for t in range(spec.n))
    else:
        kept = oracle.element_matrix(spec).sum(1)
    want = np.log(kept.astype(np.float64))
    got = lse.cpu().numpy().astype(np.float64)
    err = float(np.abs(got - want[None, None, :]).max())
    print(f"       max|dLSE| = {err:.3e}", flush=True)
    assert err <= 1e-4
    rows = expected.sample_rows(w.n, w.B, w.H, heads_per_batch=1, blocks=2, seed=7)
    eo, _, _, _ = run_and_compare(tra, w, q, k, v, rows=rows, mask=mask, tag=" (Q=0)")
    assert eo <= TOL_O[w.dtype]
    mask.free()


RAGGED = [
    # (kind, f, s, granularity, extra, B, H, D, dtype)
    ("radial", 10, 50, "element", {}, 1, 2, 64, "bf16"),
    ("radial", 10, 50, "element", {}, 1, 2, 128, "bf16"),
    ("radial", 10, 50, "element", {}, 1, 2, 64, "f32"),
    ("radial", 300, 3, "element", {}, 1, 1, 64, "bf16"),
    ("radial", 256, 1, "element", {}, 2, 1, 128, "bf16"),
    ("radial", 7, 100, "block_any", {}, 1, 3, 128, "bf16"),
    ("radial", 7, 100, "block_any", {}, 1, 2, 64, "f32"),
    ("radial", 1, 200, "element", {}, 1, 2, 64, "bf16"),
    ("radius3d", 3, 100, "element", dict(grid_h=10, grid_w=10, r_t=1, r_s=2), 2, 2, 64, "bf16"),
    ("radius3d", 4, 128, "element", dict(grid_h=8, grid_w=16, r_t=0, r_s=0), 1, 2, 128, "bf16"),
    ("swa", 9, 37, "element", dict(window=3), 1, 2, 128, "bf16"),
    ("swa", 5, 128, "element", dict(window=1), 1, 2, 64, "f32"),
    ("dense", 3, 100, "element", {}, 1, 2, 128, "bf16"),
    ("dense", 4, 128, "block_any", {}, 1, 2, 128, "bf16"),
    ("radial", 10, 50, "element", dict(sink_frames=1), 1, 2, 128, "bf16"),
    ("radial", 7, 100, "block_any", dict(sink_frames=2), 1, 2, 64, "f32"),
    ("swa", 9, 37, "element", dict(window=3, sink_frames=2), 1, 2, 64, "bf16"),
    ("radial", 12, 256, "block_eq4", {}, 1, 2, 128, "bf16"),
    ("radial", 9, 256, "block_eq4", dict(sink_frames=1), 1, 2, 64, "bf16"),
    ("radial", 12, 256, "block_eq4", {}, 1, 2, 64, "f32"),
    ("radial", 6, 70, "element", dict(sink_frames=1), 1, 2, 128, "f32"),
    ("swa", 4, 100, "element", dict(window=2), 2, 1, 128, "f32"),
]


@pytest.mark.parametrize("case", RAGGED, ids=lambda c: f"{c[0]}-f{c[1]}-s{c[2]}-{c[3]}-D{c[7]}-{c[8]}")
def test_ragged_and_degenerate_full_parity(tra, case):
    kind, f, s, gran, extra, B, H, D, dt = case
    w = workloads.Workload(f"{kind}_f{f}_s{s}", kind, gran, f, s, B, H, D, dt, seed=4242 + f + s + D, **extra)
    q, k, v = workloads.make_qkv(w, device="cuda")
    eo, el, out, _ = run_and_compare(tra, w, q, k, v)
    assert eo <= TOL_O[dt] and el <= 1
    if kind == "radius3d" and extra["r_t"] == 0 and extra["r_s"] == 0:
        # the only key is the token itself: weight exactly 1, O == V bit for bit
        assert torch.equal(out, v)


RAMP = [
    # (kind, f, s, granularity, extra, D, dtype): head 0 ramps up, head 1 down
    ("radial", 10, 200, "element", {}, 64, "bf16"),
    ("radial", 10, 200, "element", {}, 128, "bf16"),
    ("radial", 10, 200, "element", {}, 64, "f32"),
    ("radial", 10, 200, "element", {}, 128, "f32"),
    ("radial", 12, 256, "block_eq4", {}, 128, "bf16"),
    ("radial", 12, 256, "block_eq4", {}, 64, "bf16"),
    ("radial", 7, 100, "block_any", dict(sink_frames=1), 64, "bf16"),
    ("swa", 9, 128, "element", dict(window=3, sink_frames=1), 128, "bf16"),
]


@pytest.mark.parametrize("case", RAMP, ids=lambda c: f"{c[0]}-f{c[1]}-s{c[2]}-{c[3]}-D{c[5]}-{c[6]}")
def test_growing_and_shrinking_scores(tra, case):
    """Scores that ramp by about 240 log2 units along each row: the running
    row maximum moves by far more than the rescale threshold between key
    blocks, up on one head and down on the other, and an exponent taken
    against a stale maximum would overflow fp32."""
    kind, f, s, gran, extra, D, dt = case
    w = workloads.Workload(f"ramp_{kind}_f{f}_s{s}", kind, gran, f, s, 1, 2, D, dt, seed=515 + f + D, **extra)
    q, k, v = workloads.make_ramp_qkv(w, span=240.0, device="cuda")
    eo, el, out, lse = run_and_compare(tra, w, q, k, v)
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    assert eo <= TOL_O[dt] and el <= 1


@pytest.mark.parametrize("D,dt", [(64, "bf16"), (128, "bf16"), (64, "f32"), (128, "f32")])
def test_scores_far_from_zero(tra, D, dt):
    """Every score about 150 log2 units above 0, spread over a few units:
    the LSE is about 104 and the probabilities are taken against a maximum
    of that size from the first tile on."""
    w = workloads.Workload(f"offset_radial_f10_s200_D{D}", "radial", "element", 10, 200, 1, 2, D, dt, seed=717 + D)
    q, k, v = workloads.make_ramp_qkv(w, span=0.0, device="cuda", offset=150.0)
    eo, el, out, lse = run_and_compare(tra, w, q, k, v)
    assert float(lse.min()) > 90.0
    assert eo <= TOL_O[dt] and el <= 1


def test_strided_views(tra):
    """Q, K, V as [B, H, n, D] views of [B, n, H, D] storage (the layout a fused
    QKV projection produces), output into a strided view as well."""
    w = workloads.WORKLOADS["radius3d_t8_h16_w16"].replace(H=4)
    q, k, v = workloads.make_qkv(w, device="cuda")
    qs, ks, vs = (x.transpose(1, 2).contiguous().transpose(1, 2) for x in (q, k, v))
    assert not qs.is_contiguous()
    mask = build(tra, w)
    ref, ref_lse = tra.sparse_attn_fwd(q, k, v, mask)
    out_store = torch.empty(w.B, w.n, w.H, w.D, dtype=q.dtype, device=q.device)
    out = out_store.transpose(1, 2)
    tra.sparse_attn_fwd(qs, ks, vs, mask, out=out)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    mask.free()


def test_deterministic_and_reusable(tra):
    """Every row is reduced by one workgroup in CSR order: results are bit
    identical across calls, whatever the queue order.  The mask's work
    counter resets itself, so back-to-back calls (also with other inputs) work."""
    w = workloads.WORKLOADS["radial_f20_s1536_block"].replace(H=3)
    q, k, v = workloads.make_qkv(w, device="cuda")
    mask = build(tra, w)
    o1, l1 = tra.sparse_attn_fwd(q, k, v, mask)
    o2, l2 = tra.sparse_attn_fwd(q, k, v, mask)
    q2, k2, v2 = workloads.make_qkv(w, device="cuda", seed=99)
    o3, _ = tra.sparse_attn_fwd(q2, k2, v2, mask)
    o4, l4 = tra.sparse_attn_fwd(q, k, v, mask)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2) and torch.equal(o1, o4) and torch.equal(l1, l4)
    assert not torch.equal(o1, o3)
    rows = expected.sample_rows(w.n, w.B, w.H, heads_per_batch=1, blocks=2, seed=5)
    eo, el, _, _ = run_and_compare(tra, w, q2, k2, v2, rows=rows, mask=mask, tag=" (reuse)")
    assert eo <= TOL_O["bf16"] and el <= 1
    mask.free()


def test_empty_batch_is_a_no_op(tra):
    w = workloads.WORKLOADS["radial_f8_s64_fp32"].replace(dtype="bf16")
    mask = build(tra, w)
    q = torch.zeros(0, 2, w.n, w.D, dtype=torch.bfloat16, device="cuda")
    out, lse = tra.sparse_attn_fwd(q, q, q, mask)
    assert out.shape == q.shape and lse.shape == (0, 2, w.n)
    q = torch.zeros(1, 0, w.n, w.D, dtype=torch.bfloat16, device="cuda")
    tra.sparse_attn_fwd(q, q, q, mask)
    torch.cuda.synchronize()
    mask.free()


def test_errors_are_reported(tra):
    w = workloads.WORKLOADS["radial_f8_s64_fp32"].replace(dtype="bf16")
    mask = build(tra, w)
    q, k, v = workloads.make_qkv(w, device="cuda")
    with pytest.raises(tra.TraError, match="SHAPE"):
        tra.sparse_attn_fwd(q[:, :, :256], k[:, :, :256], v[:, :, :256], mask)
    with pytest.raises(tra.TraError, match="UNSUPPORTED"):
        x = torch.zeros(1, 1, w.n, 96, dtype=torch.bfloat16, device="cuda")
        tra.sparse_attn_fwd(x, x, x, mask)
    # the binding refuses what the library would refuse too: call the C ABI
    # directly for those
    lib = tra.load_library()

    def raw(qq, kk, vv, oo):
        d = [tra._desc(t) for t in (qq, kk, vv, oo)]
        return lib.tra_sparse_attn_fwd(*(ctypes.byref(x) for x in d[:3]), mask.handle, ctypes.byref(d[3]),
                                       None, 0.0, None)
    o = torch.empty_like(q)
    assert raw(q, k[:, :, :, :32].contiguous(), v, o) == -3            # shapes disagree
    assert raw(q, k.float(), v, o) == -2                               # mixed dtypes
    big = torch.zeros(1, 1, w.n, 68, dtype=torch.bfloat16, device="cuda")[..., :64]
    assert raw(big, k, v, o) == -2                                     # row pitch 68 not a multiple of 8
    assert raw(q[:, :, 1:], k[:, :, 1:], v[:, :, 1:], o[:, :, 1:]) == -3  # N != mask n
    with pytest.raises(ValueError, match="shape"):
        tra.sparse_attn_fwd(q, k[:, :, :, :32].contiguous(), v, mask)
    with pytest.raises(ValueError, match="dtype"):
        tra.sparse_attn_fwd(q, k.float(), v, mask)
    with pytest.raises(ValueError, match="multiples of 8"):
        tra.sparse_attn_fwd(big, k, v, mask)
    with pytest.raises(tra.TraError, match="SHAPE"):
        tra.build_mask(8, 12, "radius3d", grid_h=3, grid_w=5)
    mask.free()


def test_mfma_probe_is_plausible(tra):
    """The measured-peak loop runs and lands between a third of the
    data-sheet bf16 peak and the peak itself; its flop count follows the
    documented formula."""
    ms, flops = tra.probe_mfma_peak(20000, blocks=4)
    assert flops == 4 * 8 * 4 * 20000 * 32768
    ms, flops = tra.probe_mfma_peak(100000)
    tflops = flops / (ms * 1e-3) / 1e12
    print(f"[probe] MFMA loop {tflops:.0f} TFLOP/s", flush=True)
    assert 2516.6 / 3 < tflops <= 2516.6 * 1.001


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("scale", [0.03, 0.2])
def test_custom_scale(tra, dt, scale):
    """A caller scale instead of 1/sqrt(d): the oracle with the same scale and
    the same tolerances."""
    w = workloads.Workload("radial_f6_s100", "radial", "element", 6, 100, 1, 2, 128, dt, seed=31 + int(100 * scale))
    q, k, v = workloads.make_qkv(w, device="cuda")
    mask = build(tra, w)
    out, lse = tra.sparse_attn_fwd(q, k, v, mask, scale=scale)
    torch.cuda.synchronize()
    spec = spec_of(w)
    ref_o, ref_l = oracle.attention_rows(*(workloads.to_oracle_array(x) for x in (q, k, v)), spec, scale=scale)
    eo = float(np.abs(out.float().cpu().numpy().reshape(-1, w.D) - ref_o).max())
    dl = np.abs(lse.cpu().numpy().reshape(-1) - ref_l)
    ratio = float((dl / lse_tol(spec, dt, np.tile(np.arange(w.n), w.B * w.H))).max())
    print(f"[scale] {dt} scale={scale}: max|dO|={eo:.3e} max|dLSE|={float(dl.max()):.3e} (max/tol {ratio:.3f})",
          flush=True)
    assert eo <= TOL_O[dt] and ratio <= 1
    mask.free()


def test_lse_output_is_optional(tra):
    """Skipping the LSE output leaves O bit for bit unchanged."""
    w = workloads.WORKLOADS["radial_f20_s1536_block"].replace(H=2)
    q, k, v = workloads.make_qkv(w, device="cuda")
    mask = build(tra, w)
    o1, l1 = tra.sparse_attn_fwd(q, k, v, mask)
    o2, l2 = tra.sparse_attn_fwd(q, k, v, mask, lse=False)
    torch.cuda.synchronize()
    assert l2 is None and l1 is not None
    assert torch.equal(o1, o2)
    mask.free()


def test_mask_serves_other_batch_and_head_counts(tra):
    """The mask is shared by every (b, h) and the work queue is sized per call:
    one mask serves B=1, H=3 and then B=2, H=5 (sampled rows vs the oracle,
    and the first call repeated bit for bit afterwards)."""
    base = workloads.WORKLOADS["radial_f20_s1536_block"]
    mask = build(tra, base)
    first = None
    for B, H in ((1, 3), (2, 5)):
        w = base.replace(B=B, H=H)
        q, k, v = workloads.make_qkv(w, device="cuda")
        rows = expected.sample_rows(w.n, w.B, w.H, heads_per_batch=2, blocks=2, seed=B * 10 + H)
        eo, el, out, _ = run_and_compare(tra, w, q, k, v, rows=rows, mask=mask, tag=f" (B={B} H={H})")
        assert eo <= TOL_O["bf16"] and el <= 1
        if first is None:
            first = (q, k, v, out.clone())
    q, k, v, out1 = first
    again, _ = tra.sparse_attn_fwd(q, k, v, mask)
    torch.cuda.synchronize()
    assert torch.equal(again, out1)
    mask.free()


TAIL = [
    # (kind, f, s, granularity, extra, B, H, D, dtype, ramp): few items per
    # workgroup, so the queues' last chunks run as two halves of their key
    # blocks that meet in the second half to finish
    ("swa", 24, 256, "element", dict(window=10), 1, 3, 64, "bf16", False),
    ("radial", 16, 256, "element", {}, 1, 2, 128, "bf16", False),
    ("radial", 16, 256, "element", dict(sink_frames=1), 1, 2, 64, "bf16", False),
    ("swa", 12, 256, "element", dict(window=12), 1, 2, 128, "bf16", True),
    ("swa", 12, 256, "element", dict(window=12), 1, 2, 64, "bf16", True),
]


@pytest.mark.parametrize("case", TAIL, ids=lambda c: f"{c[0]}-f{c[1]}-s{c[2]}-D{c[7]}-{'ramp' if c[9] else 'gauss'}")
def test_tail_split_halves(tra, case):
    """Items split over their key blocks: the halves' partial states are
    combined in half order, so the output matches the oracle and is the same
    bit for bit on every call, whichever half ends first.  The ramped inputs
    put the two halves' row maxima hundreds of log2 units apart (one half's
    weights vanish against the other's); the radial mask leaves rows that
    keep no key of one half."""
    kind, f, s, gran, extra, B, H, D, dt, ramp = case
    w = workloads.Workload(f"tail_{kind}_f{f}_s{s}", kind, gran, f, s, B, H, D, dt, seed=900 + f + D, **extra)
    if ramp:
        q, k, v = workloads.make_ramp_qkv(w, span=240.0, device="cuda")
    else:
        q, k, v = workloads.make_qkv(w, device="cuda")
    mask = build(tra, w)
    eo, el, out, lse = run_and_compare(tra, w, q, k, v, mask=mask)
    assert eo <= TOL_O[dt] and el <= 1
    for _ in range(3):
        o2, l2 = tra.sparse_attn_fwd(q, k, v, mask)
        torch.cuda.synchronize()
        assert torch.equal(o2, out) and torch.equal(l2, lse)
    mask.free()
