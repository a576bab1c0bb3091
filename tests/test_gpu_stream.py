"""Frame-streaming K/V cache (sliding-window causal family) vs the oracle.

After appending frame i, attention for frame i's queries must equal the rows
of frame i of the TRA_MASK_SWA_CAUSAL attention over frames 0 .. i (the ring
keeps only the last `window` frames, which are exactly the frames those rows
keep).  Same tolerances as the forward (bf16: 2e-2 on O, the per-row LSE
tolerance of tests/tolerance.py).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.tolerance import lse_tol

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tra():
    import static_sparse_spatiotemporal_amd as m
    assert torch.cuda.is_available()
    m.load_library()
    return m


def frames_qkv(B, H, f, s, D, seed):
    w = workloads.Workload("stream", "swa", "element", f, s, B, H, D, "bf16", seed=seed)
    return workloads.make_qkv(w, device="cuda")  # [B, H, f * s, D]


def check_stream(tra, B, H, s, D, window, nframes, seed, check_frames=None, rows_per_frame=None, qkv=None):
    q, k, v = frames_qkv(B, H, nframes, s, D, seed) if qkv is None else qkv
    cache = tra.KVCache(B, H, s, D, window)
    errs = []
    for i in range(nframes):
        sl = slice(i * s, (i + 1) * s)
        cache.append(k[:, :, sl], v[:, :, sl])
        out, lse = cache.attn(q[:, :, sl])
        torch.cuda.synchronize()
        assert cache.frames() == (i + 1, min(i + 1, window))
        if check_frames is not None and i not in check_frames:
            continue
        print(f"[stream] B={B} H={H} s={s} D={D} W={window} frame {i}", flush=True)
        spec = oracle.MaskSpec("swa", i + 1, s, window=window)
        n = (i + 1) * s
        arrs = [workloads.to_oracle_array(x[:, :, :n]) for x in (q, k, v)]
        rr = range(s) if rows_per_frame is None else rows_per_frame
        rows = np.array([(b, h, i * s + r) for b in range(B) for h in range(H) for r in rr], np.int64)
        ref_o, ref_l = oracle.attention_rows(*arrs, spec, rows=rows)
        got_o = out[rows[:, 0], rows[:, 1], rows[:, 2] - i * s].float().cpu().numpy()
        got_l = lse[rows[:, 0], rows[:, 1], rows[:, 2] - i * s].cpu().numpy()
        dl = np.abs(got_l - ref_l)
        eo, el = float(np.abs(got_o - ref_o).max()), float((dl / lse_tol(spec, "bf16", rows[:, 2])).max())
        print(f"         max|dO|={eo:.3e} max|dLSE|={float(dl.max()):.3e} (max/bound {el:.3f})", flush=True)
        errs.append((i, eo, el))
    cache.free()
    for i, eo, el in errs:
        assert eo <= 2e-2 and el <= 1, (i, eo, el)


@pytest.mark.parametrize("D", [64, 128])
def test_stream_fill_and_wrap(tra, D):
    """Window 3: frames 0-1 fill the ring, frames 3+ evict; every frame checked."""
    check_stream(tra, B=2, H=2, s=128, D=D, window=3, nframes=7, seed=600 + D)


def test_stream_window_one(tra):
    """Window 1: each frame attends only to itself."""
    check_stream(tra, B=1, H=3, s=256, D=64, window=1, nframes=3, seed=700)


def test_stream_odd_query_blocks(tra):
    """384 tokens per frame: three query blocks, so the second pair of query
    blocks holds one block."""
    check_stream(tra, B=1, H=2, s=384, D=128, window=2, nframes=4, seed=710)


def test_stream_growing_and_shrinking_scores(tra):
    """Scores ramping by about 480 log2 units along the sequence (up on head
    0, down on head 1), about 240 within each row's three-frame window: the
    maxima of the key splits the merge combines are over 100 log2 units
    apart, so a merge that took exponents against the wrong maximum would
    overflow or flush to zero."""
    w = workloads.Workload("stream_ramp", "swa", "element", 6, 128, 1, 2, 128, "bf16", seed=909)
    qkv = workloads.make_ramp_qkv(w, span=480.0, device="cuda")
    check_stream(tra, 1, 2, 128, 128, 3, 6, 909, qkv=qkv)


def test_stream_repeat_is_bitwise(tra):
    """The splits are merged in a fixed order: calling again on the same frame
    gives the same bits."""
    B, H, s, D, W = 1, 8, 256, 64, 8
    q, k, v = frames_qkv(B, H, W + 2, s, D, 720)
    cache = tra.KVCache(B, H, s, D, W)
    for i in range(W + 2):
        sl = slice(i * s, (i + 1) * s)
        cache.append(k[:, :, sl], v[:, :, sl])
    sl = slice((W + 1) * s, (W + 2) * s)
    outs = [cache.attn(q[:, :, sl]) for _ in range(4)]
    torch.cuda.synchronize()
    for o, l in outs[1:]:
        assert torch.equal(o, outs[0][0]) and torch.equal(l, outs[0][1])
    cache.free()


def test_stream_workload_shape(tra):
    """The n = 16384 sliding-window workload's shape (16 heads, 256 tokens per
    frame, d = 64, window 16), streamed for 20 frames (the ring wraps at 16)."""
    check_stream(tra, B=1, H=16, s=256, D=64, window=16, nframes=20, seed=1003,
                 check_frames={0, 7, 15, 16, 19}, rows_per_frame=(0, 1, 63, 128, 200, 255))


def test_stream_matches_full_sequence_kernel(tra):
    """Streaming frame by frame gives the rows of the full-sequence kernel
    (same bf16 inputs; the two differ only by the order of fp32 sums)."""
    B, H, s, D, W, f = 1, 4, 128, 128, 4, 9
    q, k, v = frames_qkv(B, H, f, s, D, 811)
    mask = tra.build_mask(f, s, "swa", window=W)
    full, full_lse = tra.sparse_attn_fwd(q, k, v, mask)
    cache = tra.KVCache(B, H, s, D, W)
    for i in range(f):
        sl = slice(i * s, (i + 1) * s)
        cache.append(k[:, :, sl], v[:, :, sl])
        out, lse = cache.attn(q[:, :, sl])
        torch.cuda.synchronize()
        assert float((out.float() - full[:, :, sl].float()).abs().max()) <= 1e-2
        assert float((lse - full_lse[:, :, sl]).abs().max()) <= 1e-4
    cache.reset()
    assert cache.frames() == (0, 0)
    cache.free()
    mask.free()


def test_stream_errors(tra):
    with pytest.raises(tra.TraError) as e:
        tra.KVCache(1, 1, 100, 64, 4)
    assert e.value.status == -2  # tokens per frame must be a multiple of 128
    cache = tra.KVCache(1, 1, 128, 64, 2)
    q = torch.zeros((1, 1, 128, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(tra.TraError) as e:
        cache.attn(q)
    assert e.value.status == -1  # nothing appended yet
    with pytest.raises(ValueError, match="shape"):
        cache.append(q[:, :, :64], q[:, :, :64])  # refused by the binding
    cache.free()
