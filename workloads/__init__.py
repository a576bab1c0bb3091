"""Named synthetic workloads and their seeded input generators.

Shared by the tests, the benchmark, the HIP path and the oracle.  It holds
shapes, mask parameters and random-number generation only -- none of the
method's arithmetic.

The pages measure on real video models (HunyuanVideo, Mochi 1, Wan2.1, a
Vera 1.1 temporal module) whose activations are not available; i.i.d.
Gaussian Q/K/V of the same shapes stand in for them.  Values are drawn in
fp32 from one seeded ``torch.Generator`` per workload in the order Q, K, V,
multiplied by ``value_scale`` in fp32 and rounded to nearest-even to bf16
where the workload is bf16.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import math

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "radial" | "radius3d" | "swa" | "dense"
    granularity: str     # "element" | "block_any" | "block_eq4"
    f: int               # frames (T for the radius grid)
    s: int               # tokens per frame
    B: int
    H: int
    D: int
    dtype: str           # "f32" | "bf16"
    seed: int
    value_scale: float = 1.0
    grid_h: int = 0
    grid_w: int = 0
    r_t: int = 0
    r_s: int = 0
    window: int = 0
    sink_frames: int = 0
    note: str = field(default="", compare=False)

    @property
    def n(self) -> int:
        return self.f * self.s

    def mask_kwargs(self) -> dict:
        return dict(granularity=self.granularity, grid_h=self.grid_h, grid_w=self.grid_w,
                    r_t=self.r_t, r_s=self.r_s, window=self.window, sink_frames=self.sink_frames)

    def replace(self, **kw) -> "Workload":
        d = {k: getattr(self, k) for k in self.__dataclass_fields__}
        d.update(kw)
        return Workload(**d)


WORKLOADS = {
    # Radial mask (eq. 4) at element level, f=8 frames of s=64 tokens, fp32.
    "radial_f8_s64_fp32": Workload("radial_f8_s64_fp32", "radial", "element", 8, 64, 1, 1, 64,
                                   "f32", 1001, note="eq. 4 element mask, 1 head, d=64"),
    # 3-D token radius on a T8 x H16 x W16 grid (t-h-w flatten), r_t=1, r_s=4 (Chebyshev).
    "radius3d_t8_h16_w16": Workload("radius3d_t8_h16_w16", "radius3d", "element", 8, 256, 2, 12,
                                    64, "bf16", 1002, grid_h=16, grid_w=16, r_t=1, r_s=4),
    # Frame sliding-window causal, f=64 frames x s=256 tokens, window 16 frames.
    "swa_f64_s256_w16": Workload("swa_f64_s256_w16", "swa", "element", 64, 256, 1, 16, 64,
                                 "bf16", 1003, window=16),
    # Radial eq. 4 dilated to 128 x 128 blocks (kept if any element kept), f=20 x s=1536.
    "radial_f20_s1536_block": Workload("radial_f20_s1536_block", "radial", "block_any", 20, 1536,
                                       1, 12, 128, "bf16", 1004, value_scale=2.0 ** -0.5),
    # Radial eq. 4 dilated to 128 x 128 blocks, f=128 x s=1024 (n=131072), 24 heads, d=128.
    "radial_f128_s1024_block": Workload("radial_f128_s1024_block", "radial", "block_any", 128,
                                        1024, 1, 24, 128, "bf16", 1005),
    # Same shape and inputs, second block reading: eq. 4 on block indices
    # (8 blocks per frame), 111,552 kept blocks of 1,048,576.
    "radial_f128_s1024_block_eq4": Workload("radial_f128_s1024_block_eq4", "radial", "block_eq4",
                                            128, 1024, 1, 24, 128, "bf16", 1005),
}

# The headline throughput workload (n = 131072 tokens, one GPU).
HEADLINE = "radial_f128_s1024_block"


def make_qkv(w: Workload, device="cpu", seed: int | None = None, heads: int | None = None):
    """Seeded Q, K, V of shape [B, H, n, D] on `device`.

    fp32 N(0, 1) drawn from one generator on `device` in the order Q, K, V,
    times `value_scale` in fp32, then rounded to bf16 (nearest-even) for bf16
    workloads.  `heads` overrides H (the draws are then a different stream).
    """
    H = w.H if heads is None else heads
    g = torch.Generator(device=device)
    g.manual_seed(w.seed if seed is None else seed)
    shape = (w.B, H, w.n, w.D)
    out = []
    for _ in range(3):
        x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        if w.value_scale != 1.0:
            x = x * torch.tensor(w.value_scale, dtype=torch.float32, device=device)
        if w.dtype == "bf16":
            x = x.to(torch.bfloat16)
        out.append(x)
    return tuple(out)


def make_ramp_qkv(w: Workload, span: float, device="cpu", seed: int | None = None, offset: float = 0.0):
    """Seeded Q, K, V of shape [B, H, n, D] whose scores ramp along the key
    index, so that a query row's largest score keeps growing (even heads) or
    keeps shrinking (odd heads) from one key block to the next.

    With t_j spaced evenly over [-A, A] along the n keys (A chosen so that
    q . k / sqrt(D) * log2(e) moves by about `span` over the sequence for
    q near the all-ones vector) and c the shift that raises every score by
    about `offset` in the same units: Q = 1 + 0.1 N(0, 1), K[j] = c +/- t_j
    + 0.5 N(0, 1) (+ on even heads), V = 0.5 N(0, 1); one generator on
    `device`, drawn in the order Q, K, V, then rounded to bf16 for bf16
    workloads.  A span well above 128 makes an exponent taken against a
    stale row maximum overflow fp32; span 0 with a large offset gives rows
    of nearly equal scores that are all far from 0.
    """
    g = torch.Generator(device=device)
    g.manual_seed(w.seed if seed is None else seed)
    shape = (w.B, w.H, w.n, w.D)
    unit = math.log2(math.e) * math.sqrt(w.D)   # score change, log2 units, per unit of t
    half = span / unit / 2
    t = torch.linspace(-half, half, w.n, dtype=torch.float32, device=device)
    sign = torch.tensor([1.0 if h % 2 == 0 else -1.0 for h in range(w.H)], dtype=torch.float32,
                        device=device)
    q = 1.0 + 0.1 * torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    k = (offset / unit + sign[None, :, None, None] * t[None, None, :, None]) + \
        0.5 * torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    v = 0.5 * torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    out = (q, k, v)
    if w.dtype == "bf16":
        out = tuple(x.to(torch.bfloat16) for x in out)
    return out


def make_salad_inputs(B: int, H: int, N: int, D: int, seed: int, device="cpu"):
    """Seeded synthetic inputs of the SALAD gate and output, as a dict.

    One generator on `device`, drawn in this order, all fp32 N(0, 1) before
    scaling and rounding to bf16 (nearest-even) unless noted:
      x      [B, N, C]  the block input (C = H * D);
      w_gate [C]        times 1 / sqrt(C);
      W      [C, C]     times 1 / sqrt(C) (row = output channel);
      bias   [C]        times 0.1, kept fp32;
      o_s    [B, H, N, D] and o_l [B, H, N, D]: stand-ins for the sparse and
                        linear branch outputs;
      gate   [B]        uniform in (0, 1), fp32.
    """
    C = H * D
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    f32 = dict(generator=g, device=device, dtype=torch.float32)
    inv = torch.tensor(1.0 / math.sqrt(C), dtype=torch.float32, device=device)
    x = torch.randn((B, N, C), **f32).to(torch.bfloat16)
    w_gate = (torch.randn((C,), **f32) * inv).to(torch.bfloat16)
    W = (torch.randn((C, C), **f32) * inv).to(torch.bfloat16)
    bias = torch.randn((C,), **f32) * torch.tensor(0.1, dtype=torch.float32, device=device)
    o_s = torch.randn((B, H, N, D), **f32).to(torch.bfloat16)
    o_l = torch.randn((B, H, N, D), **f32).to(torch.bfloat16)
    gate = torch.rand((B,), **f32)
    return dict(x=x, w_gate=w_gate, W=W, bias=bias, o_s=o_s, o_l=o_l, gate=gate)


def to_oracle_array(x: torch.Tensor):
    """Host numpy view for the oracle: float32 as is, bf16 as raw uint16 bits."""
    x = x.detach().to("cpu").contiguous()
    if x.dtype == torch.bfloat16:
        return x.view(torch.int16).numpy().view("uint16")
    if x.dtype == torch.float32:
        return x.numpy()
    raise TypeError(f"unsupported dtype {x.dtype}")
