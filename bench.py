"""Throughput of the block-sparse attention forward on one MI355X.

One step = one tra_sparse_attn_fwd call (Q K^T, element masks, online softmax,
P V, epilogue) over the whole workload, with Q/K/V resident in HBM and the
static mask compiled beforehand (its build time is reported separately).

Prints one JSON line.  `value` is effective TFLOP/s on kept 128 x 128 blocks
(4 * D * 128^2 flop per kept block per (batch, head)), `ms_per_step` the
wall-clock ms per call.  The roofline object prices the attention kernel's
own launches (HIP events on the stream it runs on) against the bf16 dense
MFMA peak; `cpu_baseline` times the fp64 oracle on a bounded sample of the
same workload on the host cores.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload NAME]
"""
from __future__ import annotations

import argparse
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
HBM_PEAK_GBS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")


def kernel_source_digest() -> str:
    import hashlib
    h = hashlib.sha256()
    for fn in ("attn_fwd_bf16.hip", "attn_common.h", "tra_internal.h", "tra_sched.h", "tra_sched.cpp"):
        with open(os.path.join(ROOT, "static_sparse_spatiotemporal_amd", "csrc", fn), "rb") as f:
            h.update(f.read())
    # the forward's compiler options decide its code as much as its source
    from static_sparse_spatiotemporal_amd import _build
    h.update(" ".join(_build.FILE_FLAGS.get("attn_fwd_bf16.hip", [])).encode())
    return h.hexdigest()[:16]


def host_cpu_model() -> str:
    """The host CPU's model name, as the kernel reports it (empty if unknown)."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return ""


def measured_traffic(workload: str):
    """HBM bytes per launch of the attention kernel from the committed rocprofv3
    counter summary, if it was taken on the current kernel source."""
    path = os.path.join(PROFILES, f"attn_fwd_bf16_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        m = re.match(r"^\s*([a-z_]+)\s*:\s*(\S+)", line)
        if m:
            fields[m.group(1)] = m.group(2)
    if fields.get("kernel_source_digest") != kernel_source_digest():
        return None
    try:
        return float(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(w, q, k, v, mask_info, target_s: float):
    """fp64 oracle on sampled rows of the workload; returns the JSON object."""
    import oracle
    import workloads
    from oracle import MaskSpec

    spec = MaskSpec(w.kind, w.f, w.s, granularity=w.granularity, grid_h=w.grid_h, grid_w=w.grid_w,
                    r_t=w.r_t, r_s=w.r_s, window=w.window, sink_frames=w.sink_frames)
    threads = oracle.default_threads()
    rng = np.random.default_rng(w.seed)
    nb = spec.nb
    heads = [(0, 0), (0, w.H - 1)] if w.H > 1 else [(0, 0)]
    qblocks = sorted(set(rng.choice(nb, size=min(nb, 128), replace=False).tolist()))
    block_keep = None
    if spec.granularity == "block_any":
        counts = oracle.block_counts_rows(spec, qblocks, threads)
        block_keep = np.zeros((nb, nb), dtype=np.uint8)
        block_keep[qblocks] = counts > 0
    elif spec.granularity == "block_eq4":
        block_keep = oracle.block_keep(spec)  # for counting kept keys; the oracle tests blocks itself
    sel = lambda x: np.stack([workloads.to_oracle_array(x[b, h]) for b, h in heads])[None]
    qa, ka, va = sel(q), sel(k), sel(v)
    cand = np.array([(0, hi, qb * 128 + r) for hi in range(len(heads)) for qb in qblocks
                     for r in range(128) if qb * 128 + r < spec.n], dtype=np.int64)
    cand = cand[rng.permutation(len(cand))]

    def kept_keys(rows):
        return oracle.row_counts(spec, rows[:, 2], block_keep=block_keep)

    # calibrate on a few rows, then size the sample to about target_s seconds
    probe = cand[:threads]
    t0 = time.perf_counter()
    oracle.attention_rows(qa, ka, va, spec, rows=probe, block_keep=block_keep, threads=threads)
    dt = max(time.perf_counter() - t0, 1e-3)
    nrows = int(min(len(cand), max(threads, threads * int(target_s / dt))))
    rows = cand[:nrows]
    t0 = time.perf_counter()
    oracle.attention_rows(qa, ka, va, spec, rows=rows, block_keep=block_keep, threads=threads)
    elapsed = time.perf_counter() - t0
    flops = float(4 * w.D * kept_keys(rows).sum())
    return {
        "value": flops / elapsed / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"{nrows} query rows (fp64, all their kept keys) drawn from {len(qblocks)} query blocks "
                   f"of heads {[h for _, h in heads]}, {elapsed:.1f} s on {threads} threads"),
    }


# The other workloads of the benchmark set, timed beside the headline: the
# element-exact radial mask (fp32), the 3-D token radius, the frame sliding
# window (d = 64) and the f = 20 radial block mask.
OTHER_WORKLOADS = ["radial_f8_s64_fp32", "radius3d_t8_h16_w16", "swa_f64_s256_w16", "radial_f20_s1536_block"]


def time_forward(tra, workloads, name: str, dev, stream, calls: int = 50, warmup: int = 10) -> dict:
    """One workload's forward: per-call HIP-event time on the launch stream
    (mean and median), wall time per call over back-to-back calls, and the
    kept-block rate and share of the bf16 peak, both from the event mean."""
    import torch
    w = workloads.WORKLOADS[name]
    mask = tra.build_mask(w.f, w.s, w.kind, **w.mask_kwargs())
    info = mask.info
    q, k, v = workloads.make_qkv(w, device=dev)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    for _ in range(warmup):
        tra.sparse_attn_fwd(q, k, v, mask, out=out, lse=lse, stream=stream)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(calls)]
    for e0, e1 in ev:
        e0.record(stream)
        tra.sparse_attn_fwd(q, k, v, mask, out=out, lse=lse, stream=stream)
        e1.record(stream)
    torch.cuda.synchronize()
    ev_ms = np.array([e0.elapsed_time(e1) for e0, e1 in ev])
    t0 = time.perf_counter()
    for _ in range(calls):
        tra.sparse_attn_fwd(q, k, v, mask, out=out, lse=lse, stream=stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / calls
    flops = 4.0 * w.D * 128 * 128 * info["kept_blocks"] * w.B * w.H
    ms = float(ev_ms.mean())
    rec = {"shape": f"{w.B}x{w.H}x{w.n}x{w.D} {w.dtype}",
           "ms_event_mean": round(ms, 4), "ms_event_median": round(float(np.median(ev_ms)), 4),
           "ms_wall_per_call": round(wall_ms, 4),
           "tflops_kept_blocks": round(flops / (ms * 1e-3) / 1e12, 2)}
    if w.dtype == "bf16":
        rec["pct_bf16_peak"] = round(100 * flops / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 2)
    # backward on the same mask and inputs (gradients from the saved LSE)
    g = torch.Generator(device=dev)
    g.manual_seed(w.seed + 7)
    dout = torch.randn(q.shape, generator=g, device=dev).to(q.dtype)
    grads = tuple(torch.empty_like(q) for _ in range(3))
    ws = torch.empty(max(1, tra.sparse_attn_bwd_workspace_bytes(*q.shape)), dtype=torch.uint8, device=dev)
    tra.sparse_attn_bwd(q, k, v, out, lse, dout, mask, grads=grads, workspace=ws, stream=stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(5):
        tra.sparse_attn_bwd(q, k, v, out, lse, dout, mask, grads=grads, workspace=ws, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    rec["bwd_ms_event_mean"] = round(e0.elapsed_time(e1) / 5, 4)
    mask.free()
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-bwd", action="store_true")
    ap.add_argument("--no-probe", action="store_true",
                    help="skip the measured-MFMA-peak loop (for profiled runs)")
    ap.add_argument("--no-others", action="store_true",
                    help="skip timing the other workloads of the benchmark set")
    ap.add_argument("--cpu-seconds", type=float, default=30.0)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run only a plain 2 GiB device copy (counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "the library runs on one GPU; --gpus must be 1",
                          "gpus": args.gpus}))
        sys.exit(2)

    import torch
    import static_sparse_spatiotemporal_amd as tra
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.calibrate_copy:
        x = torch.empty(1 << 30, dtype=torch.int16, device=dev).fill_(1)
        y = torch.empty_like(x)
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "copy", "bytes_read": x.numel() * 2, "bytes_written": y.numel() * 2}))
        return

    name = args.workload or workloads.HEADLINE
    w = workloads.WORKLOADS[name]
    stream = torch.cuda.current_stream()

    # the first build of the process also pays for loading the library's
    # code object; the second one is the steady-state cost of a build
    t0 = time.perf_counter()
    mask = tra.build_mask(w.f, w.s, w.kind, **w.mask_kwargs())
    torch.cuda.synchronize()
    build_cold_ms = (time.perf_counter() - t0) * 1e3
    mask.free()
    t0 = time.perf_counter()
    mask = tra.build_mask(w.f, w.s, w.kind, **w.mask_kwargs())
    torch.cuda.synchronize()
    build_ms = (time.perf_counter() - t0) * 1e3
    info = mask.info
    q, k, v = workloads.make_qkv(w, device=dev)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)

    for _ in range(args.warmup):
        tra.sparse_attn_fwd(q, k, v, mask, out=out, lse=lse, stream=stream)
    torch.cuda.synchronize()

    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        starts[i].record(stream)
        tra.sparse_attn_fwd(q, k, v, mask, out=out, lse=lse, stream=stream)
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev_ms = np.array([s.elapsed_time(e) for s, e in zip(starts, ends)])
    ms_per_step = wall * 1e3 / args.steps
    launch_ms = float(ev_ms.mean())

    bh = w.B * w.H
    flops_blocks = 4.0 * w.D * 128 * 128 * info["kept_blocks"] * bh
    flops_elems = 4.0 * w.D * info["kept_elems"] * bh
    flops_pred = 4.0 * w.D * info["pred_elems"] * bh
    value = flops_blocks / (ms_per_step * 1e-3) / 1e12
    achieved = flops_blocks / (launch_ms * 1e-3) / 1e12
    traffic = measured_traffic(name)
    alg_bytes = (4 * bh * w.n * w.D * (2 if w.dtype == "bf16" else 4) + 4 * bh * w.n
                 + 8 * info["kept_blocks"] + 2048 * info["partial_blocks"])

    extra = {
        "seed": w.seed,
        "torch": torch.__version__,
        "host_cpu": host_cpu_model(),
        "mask_build_ms": round(build_ms, 3),
        "mask_build_first_ms": round(build_cold_ms, 3),
        "launch_ms_mean": round(launch_ms, 4),
        "launch_ms_median": round(float(np.median(ev_ms)), 4),
        "launch_ms_p10": round(float(np.percentile(ev_ms, 10)), 4),
        "launch_ms_p90": round(float(np.percentile(ev_ms, 90)), 4),
        "tflops_kept_elements": round(flops_elems / (launch_ms * 1e-3) / 1e12, 2),
        "tflops_eq4_elements": round(flops_pred / (launch_ms * 1e-3) / 1e12, 2),
        "pct_bf16_peak": round(100 * achieved / BF16_PEAK_TFLOPS, 2),
        "algorithmic_bytes": alg_bytes,
        "algorithmic_gbs": round(alg_bytes / (launch_ms * 1e-3) / 1e9, 1),
    }
    mask.free()

    if w.dtype == "bf16" and not args.no_probe:
        # measured peak: register-only MFMA loop, one workgroup of two waves
        # per SIMD on every compute unit (about 80 ms, after a short warm-up)
        tra.probe_mfma_peak(20000, stream=stream)
        loop_ms, loop_flops = tra.probe_mfma_peak(600000, stream=stream)
        loop_tflops = loop_flops / (loop_ms * 1e-3) / 1e12
        extra.update({"mfma_loop_tflops": round(loop_tflops, 1),
                      "pct_mfma_loop": round(100 * achieved / loop_tflops, 2)})

    if not args.no_dense and w.kind != "dense" and name == workloads.HEADLINE:
        dmask = tra.build_mask(w.f, w.s, "dense", granularity="block_any")
        tra.sparse_attn_fwd(q, k, v, dmask, out=out, lse=lse, stream=stream)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 3
        e0.record(stream)
        for _ in range(reps):
            tra.sparse_attn_fwd(q, k, v, dmask, out=out, lse=lse, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        dense_ms = e0.elapsed_time(e1) / reps
        dflops = 4.0 * w.D * 128 * 128 * dmask.info["kept_blocks"] * bh
        extra.update({"dense_ms": round(dense_ms, 3),
                      "dense_tflops": round(dflops / (dense_ms * 1e-3) / 1e12, 2),
                      "speedup_vs_dense": round(dense_ms / launch_ms, 3)})
        dmask.free()

    if not args.no_bwd and w.dtype == "bf16":
        # backward (gradients from the saved LSE) on the same mask and inputs
        bmask = tra.build_mask(w.f, w.s, w.kind, **w.mask_kwargs())
        g = torch.Generator(device=dev)
        g.manual_seed(w.seed + 7)
        dout = torch.randn(q.shape, generator=g, device=dev).to(torch.bfloat16)
        tra.sparse_attn_fwd(q, k, v, bmask, out=out, lse=lse, stream=stream)
        grads = tuple(torch.empty_like(q) for _ in range(3))
        ws = torch.empty(tra.sparse_attn_bwd_workspace_bytes(*q.shape), dtype=torch.uint8, device=dev)
        tra.sparse_attn_bwd(q, k, v, out, lse, dout, bmask, grads=grads, workspace=ws, stream=stream)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 5
        e0.record(stream)
        for _ in range(reps):
            tra.sparse_attn_bwd(q, k, v, out, lse, dout, bmask, grads=grads, workspace=ws, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        bwd_ms = e0.elapsed_time(e1) / reps
        extra.update({"bwd_ms": round(bwd_ms, 3),
                      # 5 products per kept block (S, dP, dV, dK, dQ) is the usual accounting
                      "bwd_tflops_5gemm": round(2.5 * flops_blocks / (bwd_ms * 1e-3) / 1e12, 2),
                      # the backward recomputes S and dP for dQ: 7 products are executed
                      "bwd_mfma_tflops_7gemm": round(3.5 * flops_blocks / (bwd_ms * 1e-3) / 1e12, 2),
                      "bwd_pct_bf16_peak_7gemm": round(100 * 3.5 * flops_blocks / (bwd_ms * 1e-3) / 1e12
                                                       / BF16_PEAK_TFLOPS, 2)})
        del grads, ws, dout
        bmask.free()

    if not args.no_bwd and w.dtype == "bf16" and name == workloads.HEADLINE:
        # SALAD linear branch on the same Q, K, V (HBM-bound: Q, K, V read once, O written once)
        lout = torch.empty_like(q)
        lws = torch.empty(tra.linear_attn_workspace_bytes(*q.shape), dtype=torch.uint8, device=dev)
        tra.linear_attn_fwd(q, k, v, out=lout, workspace=lws, stream=stream)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 10
        e0.record(stream)
        for _ in range(reps):
            tra.linear_attn_fwd(q, k, v, out=lout, workspace=lws, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        lin_ms = e0.elapsed_time(e1) / reps
        lbytes = 4 * q.numel() * q.element_size()
        extra.update({"linear_branch_ms": round(lin_ms, 4),
                      "linear_branch_gbs": round(lbytes / (lin_ms * 1e-3) / 1e9, 1),
                      "linear_branch_pct_hbm": round(100 * lbytes / (lin_ms * 1e-3) / 8e12, 2)})

        # SALAD gate (HBM-bound GEMV over the block input) and output (the
        # linear branch projected by a C x C weight, gated, added to the
        # sparse branch: an MFMA GEMM) with synthetic weights; the branch
        # outputs are this run's sparse and linear outputs
        B_, H_, N_, D_ = q.shape
        C_ = H_ * D_
        sd = workloads.make_salad_inputs(B_, H_, N_, D_, seed=w.seed + 11, device=dev)
        del sd["o_s"], sd["o_l"]
        gate = torch.empty(B_, dtype=torch.float32, device=dev)
        gws = torch.empty(max(256, tra.salad_gate_workspace_bytes(B_, N_)), dtype=torch.uint8, device=dev)
        sout = torch.empty_like(q)

        def _timed(fn, reps=10):
            fn()
            torch.cuda.synchronize()
            t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            t0.record(stream)
            for _ in range(reps):
                fn()
            t1.record(stream)
            torch.cuda.synchronize()
            return t0.elapsed_time(t1) / reps

        gate_ms = _timed(lambda: tra.salad_gate(sd["x"], sd["w_gate"], 0.0, gate=gate, workspace=gws,
                                                stream=stream))
        comb_ms = _timed(lambda: tra.salad_combine(out, lout, sd["W"], gate, bias=sd["bias"], out=sout,
                                                   stream=stream))
        gbytes = sd["x"].numel() * 2
        cflops = 2.0 * B_ * N_ * C_ * C_
        extra.update({"salad_gate_ms": round(gate_ms, 4),
                      "salad_gate_gbs": round(gbytes / (gate_ms * 1e-3) / 1e9, 1),
                      "salad_combine_ms": round(comb_ms, 4),
                      "salad_combine_tflops": round(cflops / (comb_ms * 1e-3) / 1e12, 1),
                      "salad_combine_pct_bf16_peak": round(100 * cflops / (comb_ms * 1e-3) / 1e12
                                                           / BF16_PEAK_TFLOPS, 2)})
        del lout, lws, sd, gate, gws, sout

    if w.kind == "swa" and w.dtype == "bf16" and w.s % 128 == 0:
        # frame streaming through the K/V ring: steady state (ring full), one
        # step = append the next frame's K, V + attention of its queries
        cache = tra.KVCache(w.B, w.H, w.s, w.D, w.window)
        fr = lambda x, i: x[:, :, (i % w.f) * w.s:(i % w.f + 1) * w.s]
        fo = torch.empty_like(fr(q, 0))
        flse = torch.empty(fo.shape[:3], dtype=torch.float32, device=dev)
        for i in range(w.window):
            cache.append(fr(k, i), fr(v, i), stream=stream)
            cache.attn(fr(q, i), out=fo, lse=flse, stream=stream)
        torch.cuda.synchronize()
        reps = 20
        e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
        e0.record(stream)
        for i in range(w.window, w.window + reps):
            cache.append(fr(k, i), fr(v, i), stream=stream)
            cache.attn(fr(q, i), out=fo, lse=flse, stream=stream)
        e1.record(stream)
        for i in range(reps):
            cache.attn(fr(q, i), out=fo, lse=flse, stream=stream)
        e2.record(stream)
        torch.cuda.synchronize()
        step_ms = e0.elapsed_time(e1) / reps
        attn_ms = e1.elapsed_time(e2) / reps
        sflops = 4.0 * w.D * w.s * w.window * w.s * w.B * w.H
        extra.update({"stream_window_frames": w.window,
                      "stream_step_ms": round(step_ms, 4),
                      "stream_attn_ms": round(attn_ms, 4),
                      "stream_attn_tflops": round(sflops / (attn_ms * 1e-3) / 1e12, 2),
                      "full_sequence_ms_per_frame": round(launch_ms / w.f, 4)})
        cache.free()

    if not args.no_dense and name == workloads.HEADLINE:
        # second block reading on the same inputs: eq. 4 on block indices
        w2 = workloads.WORKLOADS["radial_f128_s1024_block_eq4"]
        m2 = tra.build_mask(w2.f, w2.s, w2.kind, **w2.mask_kwargs())
        tra.sparse_attn_fwd(q, k, v, m2, out=out, lse=lse, stream=stream)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 10
        e0.record(stream)
        for _ in range(reps):
            tra.sparse_attn_fwd(q, k, v, m2, out=out, lse=lse, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        eq4_ms = e0.elapsed_time(e1) / reps
        eflops = 4.0 * w.D * 128 * 128 * m2.info["kept_blocks"] * bh
        extra.update({"block_eq4_workload": w2.name,
                      "block_eq4_kept_blocks_per_head": m2.info["kept_blocks"],
                      "block_eq4_ms": round(eq4_ms, 3),
                      "block_eq4_tflops": round(eflops / (eq4_ms * 1e-3) / 1e12, 2),
                      "block_eq4_pct_bf16_peak": round(100 * eflops / (eq4_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 2)})
        m2.free()

    if not args.no_others and name == workloads.HEADLINE:
        extra["other_workloads"] = {o: time_forward(tra, workloads, o, dev, stream) for o in OTHER_WORKLOADS}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, q, k, v, info, args.cpu_seconds)

    line = {
        "metric": "ms/call + effective TFLOP/s on kept blocks (% of bf16 MFMA peak) at n=131072",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {
            "workload": name,
            "mask": f"{w.kind} ({w.granularity}), 128x128 blocks",
            "frames": w.f, "tokens_per_frame": w.s, "n": w.n, "batch": w.B, "heads": w.H,
            "head_dim": w.D,
            "kept_blocks_per_head": info["kept_blocks"], "total_blocks_per_head": info["nqb"] * info["nkb"],
            "block_sparsity": round(1 - info["kept_blocks"] / (info["nqb"] * info["nkb"]), 4),
            "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / BF16_PEAK_TFLOPS, 4),
            "traffic": traffic,
        },
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
