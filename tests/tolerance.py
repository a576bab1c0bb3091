"""Comparison bounds of the GPU attention outputs against the fp64 oracle.

Test helper (not collected).

O (the benchmark spec bound): max-abs 1e-4 for fp32 inputs, 2e-2 for bf16 inputs
with fp32 accumulation.

LSE, fp32 inputs: max-abs 1e-4.

LSE, bf16 inputs: a bound per row, derived from the arithmetic of the bf16
kernels.  They multiply each query by scale * log2(e) once and round the
product to bf16, a relative error of at most 2^-8 per element (the unit
roundoff of an 8-bit significand).  A score
scale * q.k therefore moves by at most 2^-8 * scale * sum_i |q_i k_i|, which
Cauchy-Schwarz bounds by 2^-8 * scale * |q| * |k|.  The log-sum-exp moves by
no more than the largest move of its terms, so the bound of a row is
2^-8 * scale * |q| * max_t |k_t| (largest key norm of the head), plus 1e-4
for the fp32 accumulation.  The Q = 0 probe (every score exactly 0) and the
rounded-query test (the oracle given the kernel's rounded queries) hold
tighter: 1e-4.
"""
from __future__ import annotations

import numpy as np
import torch

TOL_O = {"f32": 1e-4, "bf16": 2e-2}
TOL_LSE_EXACT = 1e-4
QUERY_ROUNDING = 2.0 ** -8 * (1 + 2.0 ** -7)  # bf16 rounding of q * c, c itself rounded to fp32


def lse_bound(q: torch.Tensor, k: torch.Tensor, rows: np.ndarray | None = None,
              scale: float | None = None) -> np.ndarray:
    """Per-row LSE bound for the rows compared: `rows` as (b, h, query)
    triples, or None for every row in (b, h, query) order."""
    B, H, n, D = q.shape
    count = B * H * n if rows is None else len(rows)
    if q.dtype != torch.bfloat16:
        return np.full(count, TOL_LSE_EXACT)
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    kmax = k.float().norm(dim=-1).amax(dim=-1).double().cpu().numpy()  # [B, H]
    qn = q.float().norm(dim=-1).double().cpu().numpy()                  # [B, H, n]
    if rows is None:
        per = qn * kmax[:, :, None]
        per = per.reshape(-1)
    else:
        b, h, r = rows[:, 0], rows[:, 1], rows[:, 2]
        per = qn[b, h, r] * kmax[b, h]
    return TOL_LSE_EXACT + QUERY_ROUNDING * scale * per


def rounded_query(q: torch.Tensor, scale: float | None = None) -> torch.Tensor:
    """The bf16 queries the bf16 kernels compute with, scaled by
    scale * log2(e) (an oracle given these and scale ln 2 evaluates the same
    scores)."""
    D = q.shape[-1]
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    c = np.float32(scale * 1.4426950408889634)
    return (q.float() * float(c)).to(torch.bfloat16)
