"""A second, independent evaluation of the INT4 attention recursion, for
pinning the C oracle (test infrastructure only).

Page: RotateAttention review -- abstract (INT4 Q, K, V inside FlashAttention;
p = exp(QK - max QK)), Sec. 4.2 and the free-parameter ledger (code =
round(15 p) - 8; the symmetric baseline round(7 p)).

Written from the definition, not from the oracle's code: numpy over all query
rows at once, every binary32 rounding the definition asks for done exactly
(the exponent d = f32(S c - m) is the exact value rounded once, obtained from
an exact binary64 sum and a correction for binary32 midpoints), the P code
taken as round-half-up(P 2^d) by binary64 exponentiation with ties checked in
40-digit decimal (no threshold table), and the output formed both by the
online recursion and by the closed sum over key steps

    o_c = sum_s 2^(m_s - m_last) num_sc s_v[c] / sum_s 2^(m_s - m_last) U_s

which the recursion must equal.
"""
from __future__ import annotations

from decimal import ROUND_FLOOR, Decimal, getcontext

import numpy as np

BLOCK = 64
HASH_MUL = 2654435761


def f32_of_exact_sum(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """binary32 round-to-nearest-even of the exact sum a + b of binary64
    arrays (each sum's error term from Knuth's two-sum; a correction is only
    needed where the binary64 sum falls exactly on a binary32 midpoint)."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    with np.errstate(invalid="ignore"):
        s = a + b
        bp = s - a
        ap = s - bp
        err = (a - ap) + (b - bp)
    err = np.where(np.isfinite(s), err, 0.0)
    f = s.astype(np.float32)
    up = f.astype(np.float64) > s
    lo = np.where(up, np.nextafter(f, np.float32(-np.inf)), f)
    hi = np.where(up, f, np.nextafter(f, np.float32(np.inf)))
    with np.errstate(invalid="ignore"):
        mid = (lo.astype(np.float64) + hi.astype(np.float64)) / 2
    tie = np.isfinite(s) & (s == mid) & (f.astype(np.float64) != s)
    out = np.where(tie & (err > 0), hi, np.where(tie & (err < 0), lo, f))
    return out.astype(np.float32)


def round_half_up_scaled_exp2(d: np.ndarray, P: int) -> np.ndarray:
    """round-half-up(P * 2^d) for binary32 d <= 0 (d may be slightly above
    0 or -inf), as int64, decided in binary64 with near-ties in decimal."""
    d64 = np.asarray(d, np.float32).astype(np.float64)
    y = P * np.exp2(d64)
    u = np.floor(y + 0.5).astype(np.int64)
    near = np.isfinite(y) & (np.abs((y + 0.5) - np.round(y + 0.5)) < 1e-9)
    if near.any():
        getcontext().prec = 40
        ln2 = Decimal(2).ln()
        for idx in zip(*np.nonzero(near)):
            yd = Decimal(P) * (Decimal(float(d64[idx])) * ln2).exp()
            u[idx] = int((yd + Decimal("0.5")).to_integral_value(rounding=ROUND_FLOOR))
    return np.minimum(u, P)


def attention(qc, sq, kc, sk, vc, sv, rows, softmax_scale=None, p_mode=0, dump=False):
    """INT4 attention of the query rows `rows` of one (b, h) slice.

    qc, kc, vc: [N, D] integer codes; sq, sk: [ceil(N/64)]; sv: [D].
    Returns dict: o (recursion, binary64), o_direct (closed sum), m (final
    running max, binary32), dig_sum / dig_hash (per-row sums of u and of
    u h(j) mod 2^32), and with dump=True per key step s: S, d, code, pv, m."""
    qc = np.asarray(qc, np.int64)
    kc = np.asarray(kc, np.int64)
    vc = np.asarray(vc, np.int64)
    sq = np.asarray(sq, np.float32)
    sk = np.asarray(sk, np.float32)
    sv = np.asarray(sv, np.float32)
    rows = np.asarray(rows, np.int64)
    N, D = qc.shape
    P, zp = (15, 8) if p_mode == 0 else (7, 0)
    scale = softmax_scale if softmax_scale else 1.0 / np.sqrt(D)
    alpha = np.float32(np.log2(np.e) * scale)
    R = rows.size
    qrows = qc[rows]                                    # [R, D]
    csq = sq[rows // BLOCK]                             # [R]
    m = np.full(R, -np.inf, np.float32)
    A = np.zeros((R, D))
    L = np.zeros(R)
    steps = []
    ds = np.zeros(R, np.uint64)
    dh = np.zeros(R, np.uint64)
    for s in range((N + BLOCK - 1) // BLOCK):
        j0, j1 = s * BLOCK, min(N, s * BLOCK + BLOCK)
        S = qrows @ kc[j0:j1].T                         # exact integers [R, nj]
        c = (csq * sk[s]).astype(np.float32) * alpha    # binary32 products
        c = c.astype(np.float32)
        prod = S.astype(np.float64) * c.astype(np.float64)[:, None]   # exact (|S| < 2^13)
        t = prod.astype(np.float32)
        m_new = np.maximum(m, t.max(axis=1))
        d = f32_of_exact_sum(prod, -m_new.astype(np.float64)[:, None])
        u = round_half_up_scaled_exp2(d, P)             # [R, nj]
        U = u.sum(axis=1)
        num = u @ vc[j0:j1]                             # exact integers [R, D]
        beta = np.exp2(m.astype(np.float64) - m_new.astype(np.float64))
        A = A * beta[:, None] + num
        L = L * beta + U
        m = m_new
        keys = np.arange(j0, j1, dtype=np.uint64)
        ds += U.astype(np.uint64)
        h = (np.uint64(HASH_MUL) * (keys + np.uint64(1))) & np.uint64(0xFFFFFFFF)
        dh = (dh + ((u.astype(np.uint64) * h[None, :]) & np.uint64(0xFFFFFFFF)).sum(axis=1)) \
            & np.uint64(0xFFFFFFFF)
        steps.append(dict(S=S, d=d, code=u - zp, pv=(u - zp) @ vc[j0:j1], m=m.copy(), U=U, num=num))
    o = A * sv.astype(np.float64)[None, :] / L[:, None]
    w = [np.exp2(st["m"].astype(np.float64) - m.astype(np.float64)) for st in steps]
    num_d = sum(wi[:, None] * st["num"] for wi, st in zip(w, steps))
    den_d = sum(wi * st["U"] for wi, st in zip(w, steps))
    o_direct = num_d * sv.astype(np.float64)[None, :] / den_d[:, None]
    out = dict(o=o, o_direct=o_direct, m=m, dig_sum=ds.astype(np.uint32), dig_hash=dh.astype(np.uint32))
    if dump:
        out["steps"] = steps
    return out
