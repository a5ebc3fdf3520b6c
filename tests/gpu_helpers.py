"""Shared helpers of the GPU parity tests (host-side marshalling only)."""
from __future__ import annotations

import numpy as np
import torch

import progress

# INT4 output against the oracle's binary64 float path: max-abs bound.  The
# integers (codes, scores, P codes, PV sums, running max) are exact on both
# sides; what differs is binary32 against binary64 in the rescale factor
# 2^(m_old - m), the accumulation of at most N / 64 exact per-step sums and
# the final division, a few binary32 ulps of outputs of size O(1).
OUT_TOL = 1e-5


def say(*a):
    progress.say(*a)


def dev(x: np.ndarray) -> torch.Tensor:
    """numpy float32 or bf16 bit patterns (uint16) -> CUDA tensor."""
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to("cuda").view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda")


def plan_for(w, prec="int4", out_dtype="f32", p_mode=0, v_hadamard=0):
    from bit_quantized_attention_rope3d_amd.api import Plan
    return Plan(w.batch, w.heads, w.head_dim, w.grid, w.seg, rot=w.rot, prec=prec,
                in_dtype=w.dtype, out_dtype=out_dtype, rope_theta=w.theta, p_mode=p_mode,
                v_hadamard=v_hadamard)


def cosine(a, b):
    a = np.asarray(a, np.float64).ravel()
    b = np.asarray(b, np.float64).ravel()
    return float(a @ b / np.sqrt((a @ a) * (b @ b)))


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even to bf16, returned as float32."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    u = (u + np.uint32(0x7FFF) + ((u >> 16) & 1)) & np.uint32(0xFFFF0000)
    return u.view(np.float32)
