"""Pins of the oracle's range-optimized P map against what the pages fix.

Page: RotateAttention review, Sec. 4.2 and the free-parameter ledger: P in
[0, 1] is mapped onto the full signed INT4 range [-8, 7] with scale 15 and
zero-point -8, i.e. code = round(15 p) - 8; abstract: p = exp(QK - max QK).
The oracle takes p = 2^d for a binary32 exponent d <= 0 and decides the
rounding by counting binary32 thresholds T_k.  Here the same map is evaluated
other ways: 40-digit decimal exponentiation at and next to every threshold,
and binary64 exponentiation over every binary32 d from below the lowest
threshold up to 0.
"""
import json
import os
from concurrent.futures import ThreadPoolExecutor
from decimal import ROUND_FLOOR, Decimal, getcontext

import numpy as np
import pytest

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_facts.json")))


def p_decimal(d: float, P: int) -> Decimal:
    """P * 2^d to 40 significant digits (d is a binary32 value, held exactly)."""
    getcontext().prec = 40
    return Decimal(P) * (Decimal(float(d)) * Decimal(2).ln()).exp()


def u_decimal(d: float, P: int = 15) -> int:
    """round-half-up(P * 2^d) for d <= 0."""
    y = p_decimal(d, P)
    return int((y + Decimal("0.5")).to_integral_value(rounding=ROUND_FLOOR))


def prev32(x):
    return np.nextafter(np.float32(x), np.float32(-np.inf))


def next32(x):
    return np.nextafter(np.float32(x), np.float32(np.inf))


def test_endpoints_match_pages(ora):
    pm = GOLD["p_map"]
    zp = pm["zero_point"]
    # p = 1 is d = 0; p = 0 is d = -inf (and any very negative d).
    u = ora.pmap(np.array([0.0, -0.0, -np.inf, -1e30, -3.0e6], np.float32)).astype(int)
    codes = u + zp
    want = {e["p"]: e["code"] for e in pm["endpoints"]}
    assert codes[0] == want[1.0] and codes[1] == want[1.0]
    assert codes[2] == want[0.0] and codes[3] == want[0.0] and codes[4] == want[0.0]
    assert codes.min() >= pm["code_min"] and codes.max() <= pm["code_max"]
    assert pm["scale"] == 15


def test_half_probability_rounds_to_zero_code(ora):
    # p = 1/2 -> 15 p = 7.5, the only exact tie; half-up gives 8 -> code 0.
    assert int(ora.pmap(np.array([-1.0], np.float32))[0]) - 8 == 0
    assert int(ora.pmap(prev32(-1.0)[None])[0]) - 8 == -1


@pytest.mark.parametrize("p_mode", [0, 1])
def test_thresholds_against_high_precision(ora, p_mode):
    """T_k is the smallest binary32 d with P * 2^d >= k + 1/2: it meets the
    bound and the next binary32 value below it does not."""
    P = ora.P_SCALE[p_mode]
    T = ora.pmap_thresholds(p_mode)
    assert T.dtype == np.float32 and T.size == P
    for k, t in enumerate(T.tolist()):
        half = Decimal(k) + Decimal("0.5")
        assert p_decimal(t, P) >= half > p_decimal(float(prev32(t)), P), (k, t)
    assert np.all(np.diff(T) > 0)


def test_thresholds_near_closed_form(ora):
    """T_k sits within one binary32 step of log2((2k+1)/30), and the p = 1/2
    threshold is exactly -1."""
    T = ora.pmap_thresholds().astype(np.float64)
    k = np.arange(15)
    exact = np.log2((2 * k + 1) / 30.0)
    assert np.all(np.abs(T - exact) <= np.spacing(np.float32(np.abs(exact))).astype(np.float64))
    assert T[7] == -1.0


def _all_f32_between(lo: float, hi: float):
    """Bit patterns of every binary32 value in [lo, hi] with lo <= hi <= -0,
    in chunks (as uint32 arrays)."""
    a = int(np.array(hi, np.float32).view(np.uint32))
    b = int(np.array(lo, np.float32).view(np.uint32))
    a = a if hi != 0 else 0x80000000
    step = 1 << 24
    for s in range(a, b + 1, step):
        yield np.arange(s, min(s + step, b + 1), dtype=np.uint32)


@pytest.mark.parametrize("p_mode", [0, 1])
def test_every_f32_exponent_against_float64_evaluation(ora, p_mode):
    """Every binary32 d in [T_0 - 1, -0] (about 1.1e9 values): the oracle's
    code equals round-half-up(P * 2^d) evaluated in binary64.  binary64
    decides the rounding: apart from the exact tie at d = -1, no P * 2^d lies
    within 1e-9 of a half-integer (checked; such values would be decided in
    40-digit decimal instead)."""
    P = ora.P_SCALE[p_mode]
    T = ora.pmap_thresholds(p_mode)
    lo = float(T[0]) - 1.0

    def check(bits):
        d = bits.view(np.float32)
        y = P * np.exp2(d.astype(np.float64))
        near = np.abs((y + 0.5) - np.round(y + 0.5)) < 1e-9
        near &= d != -1.0
        want = np.floor(y + 0.5).astype(np.uint8)
        for i in np.nonzero(near)[0]:
            want[i] = u_decimal(float(d[i]), P)
        got = ora.pmap(d, p_mode=p_mode)
        bad = np.nonzero(got != want)[0]
        return d.size, (d[bad[:5]], got[bad[:5]], want[bad[:5]]) if bad.size else None

    n = 0
    with ThreadPoolExecutor(max_workers=8) as ex:
        for cnt, bad in ex.map(check, _all_f32_between(lo, -0.0)):
            assert bad is None, bad
            n += cnt
    assert n > 1_000_000_000
    # and the exact tie itself
    assert int(ora.pmap(np.array([-1.0], np.float32), p_mode=p_mode)[0]) == (8 if P == 15 else 4)


def test_spot_values_with_decimal(ora):
    rng = np.random.default_rng(5)
    ds = (-rng.exponential(1.5, size=300)).astype(np.float32).tolist()
    T = ora.pmap_thresholds()
    ds += [0.0, -1.0, float(prev32(-1.0))] + T.tolist() + [float(prev32(t)) for t in T]
    got = ora.pmap(np.array(ds, np.float32)).astype(int).tolist()
    assert got == [u_decimal(d) for d in ds]


def test_monotone_and_full_range(ora):
    T = ora.pmap_thresholds()
    d = np.linspace(float(T[0]) - 1, 0, 200001).astype(np.float32)
    u = ora.pmap(d).astype(int)
    assert np.all(np.diff(u) >= 0)
    assert set(u.tolist()) == set(range(16))


# ---- symmetric mode (p_mode = 1) -------------------------------------------
# Same page, Sec. 4.2 and the summary: the baseline the range-optimized map
# replaces quantizes P >= 0 on the symmetric INT4 grid, which reaches only the
# codes 0..7: code = round(7 p), zero-point 0.

def test_symmetric_endpoints_and_half(ora):
    u = ora.pmap(np.array([0.0, -np.inf, -1e30, -1.0, prev32(-1.0)], np.float32), p_mode=1).astype(int)
    assert u[0] == 7                       # p = 1 -> 7
    assert u[1] == 0 and u[2] == 0         # p = 0 -> 0
    assert u[3] == 4                       # p = 1/2 -> 3.5, half-up
    assert u[4] == 3
    assert ora.P_SCALE[1] == 7 and ora.P_ZERO[1] == 0


def test_symmetric_spot_values_with_decimal(ora):
    rng = np.random.default_rng(6)
    ds = (-rng.exponential(1.5, size=200)).astype(np.float32).tolist() + [0.0, -1.0]
    got = ora.pmap(np.array(ds, np.float32), p_mode=1).astype(int).tolist()
    assert got == [u_decimal(d, 7) for d in ds]


def test_symmetric_uses_half_the_codes_of_the_optimized_map(ora):
    """The point of Sec. 4.2: over the same exponents the symmetric map takes 8
    distinct values and the range-optimized one 16, and its step in p is
    1/7 against 1/15."""
    T = ora.pmap_thresholds()
    d = np.linspace(float(T[0]) - 1, 0, 100001).astype(np.float32)
    assert len(set(ora.pmap(d, p_mode=1).tolist())) == 8
    assert len(set(ora.pmap(d).tolist())) == 16
    assert np.all(np.diff(ora.pmap(d, p_mode=1).astype(int)) >= 0)
