"""The ramped-score parity inputs reach the bf16 forward's lazy-maximum redo.

Once every row of a wave has a finite maximum, the bf16 forward takes a
tile's exponentials against the maximum in use without looking for the
tile's own maximum, and redoes them (maximum, rescale, exponentials) only
when some lane's sum passes 2^32.  test_growing_and_shrinking_scores checks
parity on inputs whose scores ramp by about 240 log2 units along each row.
This replays the kernel's vote on inputs of the same recipe, drawn on the
CPU (the noise differs from the GPU draw; the ramp does not), and checks
that every bf16 case redoes wave-tiles, so that those GPU cases run the
branch.  Layout replayed: a wave's 32 query rows walk their kept 128-key
tiles in ascending order; a lane holds one row and the 64 keys k of a tile
with (k / 4) % 2 equal to its half.
"""
import math

import numpy as np
import pytest

import oracle
import workloads
from tests.test_gpu_attn import RAMP


def replay_redo_count(kind, f, s, gran, extra, D, span=240.0):
    w = workloads.Workload(f"ramp_{kind}_f{f}_s{s}", kind, gran, f, s, 1, 2, D, "bf16",
                           seed=515 + f + D, **extra)
    q, k, _ = workloads.make_ramp_qkv(w, span=span, device="cpu")
    q = q.double().numpy()[0]
    k = k.double().numpy()[0]
    n = w.n
    nb = (n + 127) // 128
    if gran == "element":
        keep = oracle.element_matrix(oracle.MaskSpec(kind, f, s, granularity="element", **extra)).astype(bool)
    else:
        bk = oracle.block_keep(oracle.MaskSpec(kind, f, s, granularity=gran, **extra)).astype(bool)
        keep = np.repeat(np.repeat(bk, 128, 0), 128, 1)[:n, :n]
    c2 = math.log2(math.e) / math.sqrt(D)
    tau = 8.0 / c2                      # rescale threshold: 2^8 in the probabilities
    half_of_key = (np.arange(128) // 4) % 2
    redo = 0
    for h in range(2):
        S = q[h] @ k[h].T
        for qb in range(nb):
            kbs = [kb for kb in range(nb) if keep[qb * 128:(qb + 1) * 128, kb * 128:(kb + 1) * 128].any()]
            for r0 in range(qb * 128, min(qb * 128 + 128, n), 32):
                rows = np.arange(r0, min(r0 + 32, n))
                m = np.full(len(rows), -np.inf)
                muse = np.zeros(len(rows))
                for kb in kbs:
                    cols = np.arange(kb * 128, min(kb * 128 + 128, n))
                    st = np.where(keep[np.ix_(rows, cols)], S[np.ix_(rows, cols)], -np.inf)

                    def take_max():
                        nonlocal m, muse
                        mt = st.max(axis=1)
                        if (mt > m + tau).any():
                            m = np.maximum(m, mt)
                            muse = np.where(np.isfinite(m), m, 0.0)

                    def lane_sums():
                        with np.errstate(over="ignore"):
                            p = np.exp2((st - muse[:, None]) * c2)
                        hk = half_of_key[:len(cols)]
                        return np.stack([p[:, hk == 0].sum(1), p[:, hk == 1].sum(1)])

                    lazy = bool(np.isfinite(m).all())
                    if not lazy:
                        take_max()
                    if lazy and not (lane_sums() <= 2.0 ** 32).all():
                        redo += 1
                        take_max()
                    # after the redo every lane's sum is back in range
                    assert np.isfinite(lane_sums()).all()
    return redo


@pytest.mark.parametrize("case", [c for c in RAMP if c[6] == "bf16"],
                         ids=lambda c: f"{c[0]}-f{c[1]}-s{c[2]}-{c[3]}-D{c[5]}")
def test_ramp_cases_reach_the_redo(case):
    kind, f, s, gran, extra, D, _ = case
    assert replay_redo_count(kind, f, s, gran, extra, D) > 0
