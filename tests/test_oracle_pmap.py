"""Pins of the oracle's range-optimized P map against what the pages fix.

Page: RotateAttention review, Sec. 4.2 and the free-parameter ledger: P in
[0, 1] is mapped onto the full signed INT4 range [-8, 7] with scale 15 and
zero-point -8, i.e. code = round(15 p) - 8.
The oracle evaluates p = 2^(x/G) for an integer exponent x on a grid of G
steps per log2 unit and counts thresholds; here the same map is evaluated a
different way (direct high-precision exponentiation).
"""
import json
import os
from decimal import ROUND_FLOOR, Decimal, getcontext

import numpy as np

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_facts.json")))


def u_decimal(x: int, G: int) -> int:
    """round-half-up(15 * 2^(x/G)) clipped to [0, 15], 40 significant digits."""
    getcontext().prec = 40
    y = Decimal(15) * ((Decimal(x) / Decimal(G)) * Decimal(2).ln()).exp()
    u = int((y + Decimal("0.5")).to_integral_value(rounding=ROUND_FLOOR))
    return min(max(u, 0), 15)


def test_endpoints_match_pages(ora):
    pm = GOLD["p_map"]
    zp = pm["zero_point"]
    # p = 1 is exponent 0; p = 0 is exponent -inf (and any very negative x).
    u = ora.pmap(np.array([0.0, -np.inf, -1e30, -3.0e6], np.float32)).astype(int)
    codes = u + zp
    want = {e["p"]: e["code"] for e in pm["endpoints"]}
    assert codes[0] == want[1.0]
    assert codes[1] == want[0.0] and codes[2] == want[0.0] and codes[3] == want[0.0]
    assert codes.min() >= pm["code_min"] and codes.max() <= pm["code_max"]
    assert pm["scale"] == 15


def test_half_probability_rounds_to_zero_code(ora):
    G = ora.pgrid()
    # p = 1/2 -> 15 p = 7.5, the only exact tie; half-up gives 8 -> code 0.
    assert int(ora.pmap(np.array([-G], np.float32))[0]) - 8 == 0
    assert int(ora.pmap(np.array([-G - 1], np.float32))[0]) - 8 == -1


def test_thresholds_against_high_precision(ora):
    G = ora.pgrid()
    tau = ora.pmap_thresholds()
    getcontext().prec = 40
    ln2 = Decimal(2).ln()
    for k, t in enumerate(tau.tolist()):
        half = Decimal(k) + Decimal("0.5")
        at = Decimal(15) * ((Decimal(t) / G) * ln2).exp()
        below = Decimal(15) * ((Decimal(t - 1) / G) * ln2).exp()
        assert at >= half > below, (k, t)


def test_exhaustive_grid_against_float64_evaluation(ora):
    """Every grid exponent from below the lowest threshold to above 0."""
    G = ora.pgrid()
    tau = ora.pmap_thresholds()
    x = np.arange(int(tau[0]) - 200, 201, dtype=np.int64)
    y = 15.0 * np.exp2(x / G)
    # float64 decides the rounding unambiguously on this grid: the closest
    # approach of 15*2^(x/G) to a half-integer (other than the exact tie at
    # x = -G) is far above float64 error.
    frac = np.abs((y + 0.5) - np.round(y + 0.5))
    frac[x == -G] = 1.0
    assert frac.min() > 1e-6
    want = np.clip(np.floor(y + 0.5), 0, 15).astype(np.uint8)
    got = ora.pmap(x.astype(np.float32))
    assert np.array_equal(got, want)


def test_spot_values_with_decimal(ora):
    G = ora.pgrid()
    rng = np.random.default_rng(5)
    xs = rng.integers(-30000, 1, size=300).tolist() + [0, -1, -G, -G + 1, -2 * G]
    got = ora.pmap(np.array(xs, np.float32)).astype(int).tolist()
    assert got == [u_decimal(x, G) for x in xs]


def test_monotone_and_full_range(ora):
    tau = ora.pmap_thresholds()
    x = np.arange(int(tau[0]) - 10, 10, dtype=np.float32)
    u = ora.pmap(x).astype(int)
    assert np.all(np.diff(u) >= 0)
    assert set(u.tolist()) == set(range(16))


def test_grid_keeps_clear_of_rounding_boundaries(ora):
    """No grid point except the p = 1/2 tie lies within 2e-5 (relative) of a
    rounding boundary of 15 p; this margin is what lets a hardware exp2 with
    ~1e-7 error decide the codes exactly."""
    G = ora.pgrid()
    tau = ora.pmap_thresholds()
    getcontext().prec = 40
    ln2 = Decimal(2).ln()
    worst = Decimal(1)
    for k, t in enumerate(tau.tolist()):
        half = Decimal(k) + Decimal("0.5")
        for x in (t - 1, t):
            y = Decimal(15) * ((Decimal(x) / G) * ln2).exp()
            gap = abs(y - half) / half
            if gap != 0:
                worst = min(worst, gap)
    assert worst > Decimal("2e-5")


# ---- symmetric mode (p_mode = 1) -------------------------------------------
# Same page, Sec. 4.2 and the summary: the baseline the range-optimized map
# replaces quantizes P >= 0 on the symmetric INT4 grid, which reaches only the
# codes 0..7: code = round(7 p), zero-point 0.  Evaluated here independently
# of the oracle's threshold counting.

def u_decimal_sym(x: int, G: int) -> int:
    """round-half-up(7 * 2^(x/G)) clipped to [0, 7], 40 significant digits."""
    getcontext().prec = 40
    y = Decimal(7) * ((Decimal(x) / Decimal(G)) * Decimal(2).ln()).exp()
    u = int((y + Decimal("0.5")).to_integral_value(rounding=ROUND_FLOOR))
    return min(max(u, 0), 7)


def test_symmetric_endpoints_and_half(ora):
    G = ora.pgrid()
    u = ora.pmap(np.array([0.0, -np.inf, -1e30, -G, -G - 1], np.float32), p_mode=1).astype(int)
    assert u[0] == 7                       # p = 1 -> 7
    assert u[1] == 0 and u[2] == 0         # p = 0 -> 0
    assert u[3] == 4                       # p = 1/2 -> 3.5, half-up
    assert u[4] == 3
    assert ora.P_SCALE[1] == 7 and ora.P_ZERO[1] == 0


def test_symmetric_thresholds_against_high_precision(ora):
    G = ora.pgrid()
    tau = ora.pmap_thresholds(p_mode=1)
    assert tau.size == 7
    getcontext().prec = 40
    ln2 = Decimal(2).ln()
    for k, t in enumerate(tau.tolist()):
        half = Decimal(k) + Decimal("0.5")
        at = Decimal(7) * ((Decimal(t) / G) * ln2).exp()
        below = Decimal(7) * ((Decimal(t - 1) / G) * ln2).exp()
        assert at >= half > below, (k, t)


def test_symmetric_exhaustive_grid_against_float64(ora):
    G = ora.pgrid()
    tau = ora.pmap_thresholds(p_mode=1)
    x = np.arange(int(tau[0]) - 200, 201, dtype=np.int64)
    y = 7.0 * np.exp2(x / G)
    frac = np.abs((y + 0.5) - np.round(y + 0.5))
    frac[x == -G] = 1.0
    assert frac.min() > 1e-7
    want = np.clip(np.floor(y + 0.5), 0, 7).astype(np.uint8)
    assert np.array_equal(ora.pmap(x.astype(np.float32), p_mode=1), want)
    xs = np.random.default_rng(6).integers(-25000, 1, size=200).tolist() + [0, -1, -G, -G + 1]
    got = ora.pmap(np.array(xs, np.float32), p_mode=1).astype(int).tolist()
    assert got == [u_decimal_sym(v, G) for v in xs]


def test_symmetric_uses_half_the_codes_of_the_optimized_map(ora):
    """The point of Sec. 4.2: over the same exponents the symmetric map takes 8
    distinct values and the range-optimized one 16, and its step in p is
    1/7 against 1/15."""
    tau = ora.pmap_thresholds()
    x = np.arange(int(tau[0]) - 10, 10, dtype=np.float32)
    assert len(set(ora.pmap(x, p_mode=1).tolist())) == 8
    assert len(set(ora.pmap(x).tolist())) == 16
    assert np.all(np.diff(ora.pmap(x, p_mode=1).astype(int)) >= 0)


def test_symmetric_grid_keeps_clear_of_rounding_boundaries(ora):
    """Margin of the grid from the rounding boundaries of 7 p (the exact tie
    p = 1/2 aside): above 2e-6 relative, an order of magnitude over the
    error of the hardware exp2 form the kernels build their table with."""
    G = ora.pgrid()
    tau = ora.pmap_thresholds(p_mode=1)
    getcontext().prec = 40
    ln2 = Decimal(2).ln()
    worst = Decimal(1)
    for k, t in enumerate(tau.tolist()):
        half = Decimal(k) + Decimal("0.5")
        for x in (t - 1, t):
            y = Decimal(7) * ((Decimal(x) / G) * ln2).exp()
            gap = abs(y - half) / half
            if gap != 0:
                worst = min(worst, gap)
    assert worst > Decimal("2e-6")
