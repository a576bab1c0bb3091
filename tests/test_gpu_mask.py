"""GPU mask builder vs the oracle, bit for bit, through the C ABI."""
import numpy as np
import pytest

import oracle
import workloads
from tests import expected

pytestmark = pytest.mark.gpu


def _spec_from(kind, f, s, gran="element", **kw):
    return oracle.MaskSpec(kind, f, s, granularity=gran, **kw)


CASES = {
    # the named workloads (the headline one has its own test below)
    **{name: _spec_from(w.kind, w.f, w.s, w.granularity, grid_h=w.grid_h, grid_w=w.grid_w,
                        r_t=w.r_t, r_s=w.r_s, window=w.window, sink_frames=w.sink_frames)
       for name, w in workloads.WORKLOADS.items() if w.n < 131072},
    # eq. 4 case (b) (2^r > s) only occurs with f > s
    "radial_f256_s1": _spec_from("radial", 256, 1),
    "radial_f64_s2": _spec_from("radial", 64, 2),
    "radial_f300_s3_ragged": _spec_from("radial", 300, 3),
    "radial_f10_s50_ragged": _spec_from("radial", 10, 50),
    "radial_f7_s100_block_ragged": _spec_from("radial", 7, 100, "block_any"),
    "radial_f1_s200_single_frame": _spec_from("radial", 1, 200),
    "radial_f33_s24_block": _spec_from("radial", 33, 24, "block_any"),
    "radius_t3_h10_w10_ragged": _spec_from("radius3d", 3, 100, grid_h=10, grid_w=10, r_t=1, r_s=2),
    "radius_t4_h8_w16_r0": _spec_from("radius3d", 4, 128, grid_h=8, grid_w=16, r_t=0, r_s=0),
    "radius_t2_h5_w7_big": _spec_from("radius3d", 2, 35, grid_h=5, grid_w=7, r_t=4, r_s=9),
    "swa_f9_s37_w3_ragged": _spec_from("swa", 9, 37, window=3),
    "swa_f5_s128_w1": _spec_from("swa", 5, 128, window=1),
    "swa_f6_s40_w16_block": _spec_from("swa", 6, 40, "block_any", window=16),
    "dense_f3_s100": _spec_from("dense", 3, 100),
    "dense_f2_s128_block": _spec_from("dense", 2, 128, "block_any"),
    "tiny_f1_s1": _spec_from("radial", 1, 1),
    # sink frames (every family), and eq. 4 on block indices
    "radial_f10_s50_sink1_ragged": _spec_from("radial", 10, 50, sink_frames=1),
    "radial_f7_s100_block_sink2": _spec_from("radial", 7, 100, "block_any", sink_frames=2),
    "radius_t3_h10_w10_sink1": _spec_from("radius3d", 3, 100, grid_h=10, grid_w=10, r_t=0, r_s=1,
                                          sink_frames=1),
    "swa_f9_s37_w3_sink2": _spec_from("swa", 9, 37, window=3, sink_frames=2),
    "radial_f6_s64_sink_all": _spec_from("radial", 6, 64, sink_frames=9),
    "radial_f40_s256_block_eq4": _spec_from("radial", 40, 256, "block_eq4"),
    "radial_f33_s128_block_eq4": _spec_from("radial", 33, 128, "block_eq4"),
    "radial_f20_s384_block_eq4_sink1": _spec_from("radial", 20, 384, "block_eq4", sink_frames=1),
}


def check_mask(spec: oracle.MaskSpec, counts=None):
    import static_sparse_spatiotemporal_amd as tra
    print(f"[mask] {spec.kind} f={spec.f} s={spec.s} {spec.granularity} sink={spec.sink_frames}", flush=True)
    m = tra.build_mask(spec.f, spec.s, spec.kind, granularity=spec.granularity, grid_h=spec.grid_h,
                       grid_w=spec.grid_w, r_t=spec.r_t, r_s=spec.r_s, window=spec.window,
                       sink_frames=spec.sink_frames)
    got = m.export()
    counts, cls = expected.block_classes(spec, counts)
    row_ptr, col_idx, eidx = expected.csr(cls)
    np.testing.assert_array_equal(got["row_ptr"], row_ptr)
    np.testing.assert_array_equal(got["col_idx"], col_idx)
    np.testing.assert_array_equal(got["emask_idx"], eidx)
    np.testing.assert_array_equal(got["bitmap"], expected.bitmap(cls))
    # element bitmasks of the partial blocks, in CSR order
    k = 0
    for r in range(spec.nb):
        for e in range(row_ptr[r], row_ptr[r + 1]):
            if eidx[e] >= 0:
                np.testing.assert_array_equal(got["emask"][eidx[e]], expected.partial_bits(spec, r, col_idx[e]),
                                              err_msg=f"block ({r}, {col_idx[e]})")
                k += 1
    assert k == got["emask"].shape[0]
    # chunk-wise heaviest-first order: each chunk of 64 consecutive query
    # blocks is permuted in place, by non-increasing kept-block count, ties by index
    per_row = np.diff(row_ptr)
    order = got["order"]
    for c0 in range(0, spec.nb, 64):
        part = order[c0:c0 + 64]
        np.testing.assert_array_equal(np.sort(part), np.arange(c0, min(spec.nb, c0 + 64)))
        keyed = [(-per_row[x], x) for x in part]
        assert keyed == sorted(keyed)
    info = m.info
    assert info["n"] == spec.n and info["nqb"] == spec.nb and info["nkb"] == spec.nb
    assert info["kept_blocks"] == int((cls > 0).sum())
    assert info["partial_blocks"] == int((cls == 2).sum())
    assert info["pred_elems"] == int(counts.sum())
    if spec.granularity == "element":
        assert info["kept_elems"] == int(counts.sum())
    else:
        assert info["kept_elems"] == int(expected.kept_keys_per_row(spec, cls).sum())
    assert info["min_row_blocks"] == per_row.min() and info["max_row_blocks"] == per_row.max()
    # the kernels' pair schedules, over query blocks (forward, dQ) and over
    # key blocks (dK/dV), against their rule restated on the block classes
    keep = cls > 0
    assert (info["work_items"], info["tile_loads"]) == expected.pair_schedule(keep, spec.s)
    assert (info["bwd_work_items"], info["bwd_tile_loads"]) == expected.pair_schedule(keep.T, spec.s)
    m.free()
    return counts, cls


@pytest.mark.parametrize("name", list(CASES))
def test_mask_matches_oracle(name):
    check_mask(CASES[name])


def test_headline_mask_matches_oracle():
    """n = 131072 (f=128, s=1024) radial mask dilated to 128 x 128 blocks: every
    block class, CSR entry and bitmap bit vs the oracle's element enumeration."""
    w = workloads.WORKLOADS[workloads.HEADLINE]
    spec = _spec_from(w.kind, w.f, w.s, w.granularity)
    counts = expected.cached_block_counts(spec)
    _, cls = check_mask(spec, counts)
    # eq. 5-6 bound on the element-level kept count (f >= 2)
    assert counts.sum() <= 4 * w.s * w.s * w.f * int(np.floor(np.log2(w.f)))


def test_headline_block_eq4_mask_matches_oracle():
    """Same n = 131072 video, eq. 4 on block indices: 111,552 whole blocks."""
    w = workloads.WORKLOADS["radial_f128_s1024_block_eq4"]
    spec = _spec_from(w.kind, w.f, w.s, w.granularity)
    _, cls = check_mask(spec, expected.cached_block_counts(spec))
    assert int((cls > 0).sum()) == 111552 and not (cls == 2).any()
