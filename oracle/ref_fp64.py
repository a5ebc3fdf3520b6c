"""Textbook full-precision attention with 3D RoPE, in numpy float64.

TEST INFRASTRUCTURE ONLY.  Written independently of ``ra_oracle.c``: RoPE is
expressed as multiplication of each adjacent channel pair, read as a complex
number, by exp(i * pos * freq) (the RoFormer formulation), and the rotations
are built as explicit orthogonal matrices.

Page: "RotateAttention: RoPE-Aware Rotation and Range Rectification for INT4
Quantized Attention in Video Generation" (pith.science review) -- Sec. 3 /
Fig. 2 (frame/height/width RoPE segments), Sec. 4.1 / Fig. 3 (Interleaved and
Half rotations; orthogonality keeps (QR)(KR)^T = QK^T), abstract (attention
as softmax of QK^T).
"""
from __future__ import annotations

import numpy as np

ROT_NONE, ROT_INTERLEAVED, ROT_HALF = 0, 1, 2


def positions(grid, offset=(0, 0, 0)):
    """Per-token (f, h, w) coordinates, w fastest, shifted by `offset`."""
    F, Hh, W = grid
    f, h, w = np.meshgrid(np.arange(F), np.arange(Hh), np.arange(W), indexing="ij")
    return np.stack([f.ravel(), h.ravel(), w.ravel()], axis=1) + np.asarray(offset)


def rope3d(x, grid, seg, theta=10000.0, offset=(0, 0, 0)):
    """x [..., N, H, D] real -> RoPE-rotated copy (fp64), pairs (2j, 2j+1)."""
    x = np.asarray(x, dtype=np.float64)
    pos = positions(grid, offset)               # [N, 3]
    out = np.empty_like(x)
    off = 0
    for s, L in enumerate(seg):
        j = np.arange(L // 2)
        freq = theta ** (-2.0 * j / L)          # [L/2]
        phase = np.exp(1j * pos[:, s:s + 1] * freq[None, :])   # [N, L/2]
        z = x[..., off:off + L:2] + 1j * x[..., off + 1:off + L:2]   # [..., N, H, L/2]
        z = z * phase[:, None, :]
        out[..., off:off + L:2] = z.real
        out[..., off + 1:off + L:2] = z.imag
        off += L
    return out


def rotation_matrix(seg, rot):
    """The D x D block-diagonal rotation R applied after RoPE (x -> x R^T rows)."""
    D = int(sum(seg))
    R = np.eye(D)
    if rot == ROT_NONE:
        return R
    r = 1.0 / np.sqrt(2.0)
    off = 0
    for L in seg:
        R_s = np.zeros((L, L))
        if rot == ROT_INTERLEAVED:
            # R(pi/4) on each adjacent pair (a, b) -> (r(a - b), r(a + b))
            for j in range(L // 2):
                a, b = 2 * j, 2 * j + 1
                R_s[a, a], R_s[a, b] = r, -r
                R_s[b, a], R_s[b, b] = r, r
        elif rot == ROT_HALF:
            # H2 on (i, i + L/2) -> (r(u + w), r(u - w))
            hh = L // 2
            for i in range(hh):
                R_s[i, i], R_s[i, i + hh] = r, r
                R_s[i + hh, i], R_s[i + hh, i + hh] = r, -r
        R[off:off + L, off:off + L] = R_s
        off += L
    return R


def rope_rotate(x, grid, seg, theta=10000.0, rot=ROT_HALF):
    """RoPE followed by the RoPE-aware rotation, fp64."""
    y = rope3d(x, grid, seg, theta)
    R = rotation_matrix(seg, rot)
    return y @ R.T


def attention(q, k, v, scale=None):
    """softmax(q k^T * scale) v per head; q,k,v [N, H, D] or [B, N, H, D] fp64."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    squeeze = q.ndim == 3
    if squeeze:
        q, k, v = q[None], k[None], v[None]
    D = q.shape[-1]
    scale = 1.0 / np.sqrt(D) if scale is None else scale
    qh = np.transpose(q, (0, 2, 1, 3))
    kh = np.transpose(k, (0, 2, 1, 3))
    vh = np.transpose(v, (0, 2, 1, 3))
    s = qh @ np.swapaxes(kh, -1, -2) * scale
    s = s - s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    p /= p.sum(axis=-1, keepdims=True)
    o = np.transpose(p @ vh, (0, 2, 1, 3))
    return o[0] if squeeze else o


def attention_rows(q, k, v, rows, scale=None):
    """Rows `rows` of textbook attention for one head: q,k,v [N, D] fp64."""
    q = np.asarray(q, np.float64)[rows]
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    D = q.shape[-1]
    scale = 1.0 / np.sqrt(D) if scale is None else scale
    s = q @ k.T * scale
    s -= s.max(axis=1, keepdims=True)
    p = np.exp(s)
    p /= p.sum(axis=1, keepdims=True)
    return p @ v


def reference_output(q, k, v, grid, seg, theta=10000.0, scale=None):
    """Full-precision target: softmax(RoPE(q) RoPE(k)^T scale) v (no rotation,
    no quantization)."""
    qr = rope3d(q, grid, seg, theta)
    kr = rope3d(k, grid, seg, theta)
    return attention(qr, kr, v, scale)
