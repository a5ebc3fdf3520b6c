"""ctypes wrapper around ``ra_oracle.c`` (test infrastructure only).

Each wrapper names the step of the method it runs; the arithmetic itself lives
in ``ra_oracle.c``, which documents the page passages it follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ra_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libra_oracle.so")
_lib = None
_lock = threading.Lock()

ROT_NONE, ROT_INTERLEAVED, ROT_HALF, ROT_FULL = 0, 1, 2, 3
ROT_NAMES = {"none": ROT_NONE, "interleaved": ROT_INTERLEAVED, "half": ROT_HALF, "full": ROT_FULL}
BLOCK = 64

__all__ = [
    "build", "lib", "ROT_NONE", "ROT_INTERLEAVED", "ROT_HALF", "ROT_FULL", "ROT_NAMES",
    "BLOCK", "bf16_bits_to_f32", "as_f32", "rope_table", "rope_rotate",
    "quant_qk", "quant_v", "fwht", "prologue", "pmap_thresholds", "pmap", "P_SCALE", "P_ZERO",
    "attention_rows", "attention_tile", "attention_full", "code_digests", "schedule_full_precision",
    "set_threads", "get_threads",
]


def build(force: bool = False) -> str:
    """Compile ra_oracle.c into libra_oracle.so next to it.  With
    ORA_LIB_PATH set, that prebuilt variant is used instead (tests that plant
    a mistake in a copy of the oracle point the suite at it)."""
    if os.environ.get("ORA_LIB_PATH"):
        return os.environ["ORA_LIB_PATH"]
    if force or not os.path.exists(_LIB_PATH) or (
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=gnu11", "-fopenmp", "-ffp-contract=off",
               "-fno-fast-math", "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    with _lock:
        if _lib is None:
            L = ctypes.CDLL(build())
            P = ctypes.c_void_p
            i32, f64 = ctypes.c_int, ctypes.c_double
            L.ora_block.restype = i32
            L.ora_set_threads.argtypes = [i32]
            L.ora_get_threads.restype = i32
            L.ora_rope_table.argtypes = [i32, i32, f64, i32, P, P]
            L.ora_rope_rotate.argtypes = [P, P, i32, i32, i32, i32, i32, i32, P, f64, i32]
            L.ora_quant_qk.argtypes = [P, i32, i32, i32, i32, P, P]
            L.ora_quant_v.argtypes = [P, i32, i32, i32, i32, P, P]
            L.ora_pmap_thresholds_p.argtypes = [i32, P]
            L.ora_pmap_p.argtypes = [P, ctypes.c_int64, i32, P]
            L.ora_fwht_rows.argtypes = [P, ctypes.c_int64, i32]
            L.ora_attention_head.argtypes = [P, P, P, P, P, P, i32, i32, f64, i32, i32,
                                             P, i32, P, P, i32, P, P, P, P, P]
            L.ora_code_digests.argtypes = [P, P, P, P, i32, i32, f64, i32, P, i32, P, P, P]
            L.ora_schedule_full_precision.argtypes = [i32] * 8
            for name in ("ora_rope_table", "ora_rope_rotate", "ora_quant_qk",
                         "ora_quant_v", "ora_pmap_thresholds_p", "ora_pmap_p", "ora_fwht_rows",
                         "ora_attention_head", "ora_code_digests",
                         "ora_schedule_full_precision"):
                getattr(L, name).restype = i32
            _lib = L
    return _lib


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def _check(rc, what):
    if rc != 0:
        raise ValueError("oracle %s rejected its arguments (rc=%d)" % (what, rc))


def set_threads(n: int) -> None:
    lib().ora_set_threads(int(n))


def get_threads() -> int:
    return lib().ora_get_threads()


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns (uint16) to float32."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


def as_f32(x: np.ndarray) -> np.ndarray:
    if x.dtype == np.uint16:
        return np.ascontiguousarray(bf16_bits_to_f32(x))
    return np.ascontiguousarray(x, dtype=np.float32)


def rope_table(npos: int, L: int, theta: float, rot: int):
    cs = np.empty((npos, L // 2), np.float32)
    sn = np.empty((npos, L // 2), np.float32)
    _check(lib().ora_rope_table(npos, L, float(theta), int(rot), _p(cs), _p(sn)), "rope_table")
    return cs, sn


def rope_rotate(x, grid, seg, theta=10000.0, rot=ROT_HALF) -> np.ndarray:
    """3D RoPE + RoPE-aware rotation of x [B, N, H, D] in binary32."""
    x = as_f32(x)
    B, N, H, D = x.shape
    F, Hh, W = grid
    assert N == F * Hh * W
    y = np.empty_like(x)
    seg_a = np.asarray(seg, dtype=np.int32)
    _check(lib().ora_rope_rotate(_p(x), _p(y), B, H, D, F, Hh, W, _p(seg_a),
                                 float(theta), int(rot)), "rope_rotate")
    return y


def quant_qk(y):
    """Per-(b, h, 64-token block) symmetric INT4 -> codes [B,H,N,D], scales [B,H,nblk]."""
    y = as_f32(y)
    B, N, H, D = y.shape
    nblk = (N + BLOCK - 1) // BLOCK
    codes = np.empty((B, H, N, D), np.int8)
    scales = np.empty((B, H, nblk), np.float32)
    _check(lib().ora_quant_qk(_p(y), B, N, H, D, _p(codes), _p(scales)), "quant_qk")
    return codes, scales


def quant_v(v):
    """Per-(b, h, channel) symmetric INT4 -> codes [B,H,N,D], scales [B,H,D]."""
    v = as_f32(v)
    B, N, H, D = v.shape
    codes = np.empty((B, H, N, D), np.int8)
    scales = np.empty((B, H, D), np.float32)
    _check(lib().ora_quant_v(_p(v), B, N, H, D, _p(codes), _p(scales)), "quant_v")
    return codes, scales


def fwht(x):
    """Orthonormal Walsh-Hadamard transform of the last axis in binary32
    (butterflies h = 1, 2, ..., then x f32(1/sqrt(D)))."""
    x = np.array(as_f32(x), dtype=np.float32, copy=True, order="C")
    D = x.shape[-1]
    _check(lib().ora_fwht_rows(_p(x), x.size // D, D), "fwht_rows")
    return x


def prologue(q, k, v, grid, seg, theta=10000.0, rot=ROT_HALF, v_hadamard=False):
    """RoPE + rotation + INT4 quantization of Q/K, and INT4 quantization of V
    (of V H when v_hadamard)."""
    qr = rope_rotate(q, grid, seg, theta, rot)
    kr = rope_rotate(k, grid, seg, theta, rot)
    qc, sq = quant_qk(qr)
    del qr
    kc, sk = quant_qk(kr)
    del kr
    vc, sv = quant_v(fwht(v) if v_hadamard else v)
    return dict(q_codes=qc, s_q=sq, k_codes=kc, s_k=sk, v_codes=vc, s_v=sv)


P_SCALE = {0: 15, 1: 7}        # p_mode 0: range-optimized; 1: symmetric
P_ZERO = {0: 8, 1: 0}          # zero-point: code = u - P_ZERO[p_mode]


def pmap_thresholds(p_mode: int = 0) -> np.ndarray:
    """T_k (binary32): the smallest d with P * 2^d >= k + 1/2, k = 0..P-1."""
    T = np.empty(P_SCALE[p_mode], np.float32)
    _check(lib().ora_pmap_thresholds_p(int(p_mode), _p(T)), "pmap_thresholds")
    return T


def pmap(d, p_mode: int = 0) -> np.ndarray:
    """u = code + zero-point = round(P * 2^d) (half up) for binary32 exponents d."""
    d = np.ascontiguousarray(d, dtype=np.float32)
    u = np.empty(d.shape, np.uint8)
    _check(lib().ora_pmap_p(_p(d), d.size, int(p_mode), _p(u)), "pmap")
    return u


def _head(pro, b, h):
    return (np.ascontiguousarray(pro["q_codes"][b, h]), np.ascontiguousarray(pro["s_q"][b, h]),
            np.ascontiguousarray(pro["k_codes"][b, h]), np.ascontiguousarray(pro["s_k"][b, h]),
            np.ascontiguousarray(pro["v_codes"][b, h]), np.ascontiguousarray(pro["s_v"][b, h]))


def attention_rows(pro, b, h, rows, softmax_scale=None, with_m=False, p_mode=0, v_hadamard=False):
    """Oracle output rows (binary64) of head (b, h) for query indices `rows`."""
    qc, sq, kc, sk, vc, sv = _head(pro, b, h)
    N, D = qc.shape
    scale = float(softmax_scale) if softmax_scale else 1.0 / np.sqrt(D)
    rows = np.ascontiguousarray(rows, dtype=np.int32)
    o = np.empty((rows.size, D), np.float64)
    m = np.empty(rows.size, np.float32)
    _check(lib().ora_attention_head(_p(qc), _p(sq), _p(kc), _p(sk), _p(vc), _p(sv), N, D,
                                    scale, int(p_mode), int(bool(v_hadamard)), _p(rows), rows.size,
                                    _p(o), _p(m), -1,
                                    None, None, None, None, None), "attention_head")
    return (o, m) if with_m else o


def attention_tile(pro, b, h, q_blk, kv_blk, softmax_scale=None, p_mode=0):
    """Tile dump after key step kv_blk for the 64 query rows of q_blk.

    Rows past N are absent; returns dict of s_int [r,64], p_code [r,64],
    d_val [r,64] (the binary32 exponent of each key, -inf past N), pv_int [r,D],
    m_after [r] for the valid rows r."""
    qc, sq, kc, sk, vc, sv = _head(pro, b, h)
    N, D = qc.shape
    scale = float(softmax_scale) if softmax_scale else 1.0 / np.sqrt(D)
    r0 = q_blk * BLOCK
    rows = np.arange(r0, min(N, r0 + BLOCK), dtype=np.int32)
    n = rows.size
    o = np.empty((n, D), np.float64)
    s_int = np.zeros((n, BLOCK), np.int32)
    p_code = np.zeros((n, BLOCK), np.int8)
    d_val = np.zeros((n, BLOCK), np.float32)
    pv = np.zeros((n, D), np.int32)
    m_after = np.zeros(n, np.float32)
    _check(lib().ora_attention_head(_p(qc), _p(sq), _p(kc), _p(sk), _p(vc), _p(sv), N, D,
                                    scale, int(p_mode), 0, _p(rows), n, _p(o), None, int(kv_blk),
                                    _p(s_int), _p(p_code), _p(d_val), _p(pv), _p(m_after)),
           "attention_tile")
    return dict(s_int=s_int, p_code=p_code, d_val=d_val, pv_int=pv, m_after=m_after)


def attention_full(pro, softmax_scale=None, p_mode=0, v_hadamard=False):
    """Oracle output [B, N, H, D] (binary64) for every row of every head."""
    B, H, N, D = pro["q_codes"].shape
    out = np.empty((B, N, H, D), np.float64)
    rows = np.arange(N, dtype=np.int32)
    for b in range(B):
        for h in range(H):
            out[b, :, h, :] = attention_rows(pro, b, h, rows, softmax_scale, p_mode=p_mode,
                                             v_hadamard=v_hadamard)
    return out


def code_digests(pro, b, h, rows, softmax_scale=None, p_mode=0):
    """Per selected row of head (b, h): (sum of u over all keys, sum of
    u * h(j) mod 2^32 with h(j) = 2654435761 (j + 1) mod 2^32, final running
    max), u = code + zero-point -- a fingerprint of every P code of the row."""
    qc, sq, kc, sk, _, _ = _head(pro, b, h)
    N, D = qc.shape
    scale = float(softmax_scale) if softmax_scale else 1.0 / np.sqrt(D)
    rows = np.ascontiguousarray(rows, dtype=np.int32)
    ds = np.empty(rows.size, np.uint32)
    dh = np.empty(rows.size, np.uint32)
    m = np.empty(rows.size, np.float32)
    _check(lib().ora_code_digests(_p(qc), _p(sq), _p(kc), _p(sk), N, D, scale, int(p_mode),
                                  _p(rows), rows.size, _p(ds), _p(dh), _p(m)), "code_digests")
    return ds, dh, m


def schedule_full_precision(sched, step, n_steps, block, n_blocks) -> bool:
    sh, st, bh, bt = sched
    return bool(lib().ora_schedule_full_precision(sh, st, bh, bt, step, n_steps, block, n_blocks))
