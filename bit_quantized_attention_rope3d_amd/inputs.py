"""Seeded synthetic workloads shaped like 3D-RoPE video-DiT attention.

Shared by the tests, the benchmark and the CPU oracle's callers.  This module
only draws random tensors and describes shapes; it holds none of the method's
arithmetic.

The pages measure on Wan2.2 and HunyuanVideo generations, whose activations
are not available here.  Seeded normal tensors stand in for them, with
outlier channels placed the way the RotateAttention review describes the
RoPE-induced outliers (Sec. 3 / Fig. 2): confined to RoPE segments, in one
half of each segment, and at the same channels in Q and K.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace

import numpy as np

ROT = {"none": 0, "interleaved": 1, "half": 2, "full": 3}


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    heads: int
    head_dim: int
    grid: tuple            # (F, H, W) token grid, w fastest
    seg: tuple             # (frame, height, width) head-dim split
    rot: str = "half"      # none | interleaved | half | full
    dtype: str = "bf16"    # input dtype: bf16 | f32
    theta: float = 10000.0
    seed: int = 0
    outlier_segments: tuple = (0, 1, 2)   # segments that carry outlier channels
    outliers_per_segment: tuple = (1, 1, 1)
    outlier_scale: tuple = (10.0, 30.0)   # U[lo, hi] multiplier per channel
    outlier_dist: str = "normal"          # normal | student_t3
    extra: dict = field(default_factory=dict, compare=False)

    @property
    def tokens(self) -> int:
        F, H, W = self.grid
        return F * H * W

    @property
    def rot_id(self) -> int:
        return ROT[self.rot]

    def ops(self) -> float:
        """Algorithmic work of one attention forward: 4 N^2 D H B."""
        return 4.0 * self.tokens ** 2 * self.head_dim * self.heads * self.batch

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


def tiny_segments(head_dim: int):
    """Even frame/height/width split: h = w = 2*floor(D/6), f = D - 2h
    (gives 44/42/42 at D = 128 and 24/20/20 at D = 64)."""
    hw = 2 * (head_dim // 6)
    return (head_dim - 2 * hw, hw, hw)


WORKLOADS = {
    # Tiny: 2 heads, D = 64, 2x4x4 grid, fp32, 4 outlier channels per segment x20.
    "tiny": Workload("tiny", 1, 2, 64, (2, 4, 4), tiny_segments(64), rot="interleaved",
                     dtype="f32", seed=0, outliers_per_segment=(4, 4, 4),
                     outlier_scale=(20.0, 20.0)),
    # Wan-like 480p: 40 heads, D = 128, 21x30x52 = 32,760 tokens.
    "wan480": Workload("wan480", 1, 40, 128, (21, 30, 52), (44, 42, 42), rot="interleaved",
                       seed=1),
    # Wan-like 720p: 40 heads, D = 128, 21x45x80 = 75,600 tokens.
    "wan720": Workload("wan720", 1, 40, 128, (21, 45, 80), (44, 42, 42), rot="half", seed=2),
    # HunyuanVideo-like 720p: 24 heads, D = 128, 33x45x80 = 118,800 tokens,
    # heavy-tailed outliers in the height and width segments only.
    "hy720": Workload("hy720", 1, 24, 128, (33, 45, 80), (16, 56, 56), rot="interleaved",
                      seed=3, outlier_segments=(1, 2), outliers_per_segment=(0, 1, 2),
                      outlier_dist="student_t3"),
}


def get(name: str) -> Workload:
    return WORKLOADS[name]


def with_inputs(w: Workload, recipe: str) -> Workload:
    """The workload with another outlier recipe: 'recipe' (its own), 'plain'
    (no outlier channels), 'mild' (multipliers U[3, 5] instead of
    U[10, 30]) or 'student_t3' (heavy-tailed channels in the height and width
    segments, as in the HunyuanVideo-like workload)."""
    if recipe == "recipe":
        return w
    if recipe == "plain":
        return w.with_(outliers_per_segment=(0, 0, 0))
    if recipe == "mild":
        return w.with_(outlier_scale=(3.0, 5.0))
    if recipe == "student_t3":
        return w.with_(outlier_segments=(1, 2), outliers_per_segment=(0, 1, 2), outlier_dist="student_t3")
    raise ValueError("unknown input recipe %r" % recipe)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even float32 -> bfloat16 bit patterns (uint16)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def outlier_channels(w: Workload, rng: np.random.Generator):
    """Per head: list of (channel, multiplier), in the second half of each
    outlier-carrying segment, shared by Q and K."""
    chans = []
    offs = np.cumsum((0,) + tuple(w.seg))
    for _h in range(w.heads):
        sel = []
        for s in w.outlier_segments:
            L = w.seg[s]
            n = w.outliers_per_segment[s]
            if n == 0:
                continue
            lo = offs[s] + L // 2
            picks = rng.choice(np.arange(lo, offs[s] + L), size=n, replace=False)
            mult = rng.uniform(w.outlier_scale[0], w.outlier_scale[1], size=n)
            sel.extend(zip(picks.tolist(), mult.tolist()))
        chans.append(sel)
    return chans


def generate(w: Workload, seed: int | None = None):
    """Return (q, k, v, info): arrays [B, N, H, D], float32 or bf16 bits (uint16)."""
    seed = w.seed if seed is None else seed
    rng = np.random.default_rng(seed)
    B, N, H, D = w.batch, w.tokens, w.heads, w.head_dim
    shape = (B, N, H, D)
    q = rng.standard_normal(shape, dtype=np.float32)
    k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    chans = outlier_channels(w, rng)
    for h, sel in enumerate(chans):
        for c, mult in sel:
            if w.outlier_dist == "student_t3":
                q[:, :, h, c] = rng.standard_t(3, size=(B, N)).astype(np.float32) * mult
                k[:, :, h, c] = rng.standard_t(3, size=(B, N)).astype(np.float32) * mult
            else:
                q[:, :, h, c] *= np.float32(mult)
                k[:, :, h, c] *= np.float32(mult)
    info = dict(seed=seed, outliers=chans)
    if w.dtype == "bf16":
        return f32_to_bf16_bits(q), f32_to_bf16_bits(k), f32_to_bf16_bits(v), info
    return q, k, v, info


def small(name="small", heads=3, head_dim=128, grid=(3, 5, 7), seg=None, rot="half",
          dtype="bf16", seed=11, batch=1) -> Workload:
    """A multi-tile case with a ragged tail (3*5*7 = 105 tokens by default)."""
    seg = seg or tiny_segments(head_dim)
    return Workload(name, batch, heads, head_dim, tuple(grid), tuple(seg), rot=rot,
                    dtype=dtype, seed=seed)


def schedule_seed(step: int, block: int, n_blocks: int = 40) -> int:
    """Seed of the fresh tensors of one call in the step x block sweep."""
    return 1000 + step * n_blocks + block


def generate_device(w: Workload, seed: int, device="cuda"):
    """Fresh Q, K, V [B, N, H, D] drawn on the device, for sweeps that need a
    new full-size tensor per call (drawing 75,600 x 40 x 128 normals on the
    host takes seconds).  Normals come from torch's Philox generator seeded
    with `seed`; the outlier channels and multipliers are drawn on the host
    from the same seed, as in generate().  Returns tensors of the workload's
    dtype (bf16 or float32)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    B, N, H, D = w.batch, w.tokens, w.heads, w.head_dim
    shape = (B, N, H, D)
    mult = np.ones((H, D), np.float32)
    heavy = []
    for h, sel in enumerate(outlier_channels(w, np.random.default_rng(seed))):
        for c, m in sel:
            mult[h, c] = m
            heavy.append((h, c))
    mult_d = torch.from_numpy(mult).to(device)
    out = []
    for _ in range(3):
        out.append(torch.randn(shape, generator=g, device=device, dtype=torch.float32))
    q, k, v = out
    if w.outlier_dist == "student_t3":
        # t(3) = z / sqrt(chi2_3 / 3) on the outlier channels of Q and K.
        for x in (q, k):
            for h, c in heavy:
                z = torch.randn((B, N), generator=g, device=device)
                chi = torch.randn((3, B, N), generator=g, device=device).square().sum(0)
                x[:, :, h, c] = z / torch.sqrt(chi / 3.0)
    q.mul_(mult_d)
    k.mul_(mult_d)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    return q.to(dt), k.to(dt), v.to(dt)
