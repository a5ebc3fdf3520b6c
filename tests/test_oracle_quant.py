"""Pins of the oracle's symmetric INT4 quantizers (Q/K per 64-token block,
V per channel).

Page: RotateAttention review, abstract (INT4 Q and K; INT4 FlashAttention) and
PAROAttention review (64-token blocks aligned with the attention tile).
Properties checked: every code is a nearest integer to x/scale in [-7, 7],
the block maximum reaches +-7, the rounding error is at most half a step,
exactly representable inputs round-trip, zero groups give scale 0.
"""
import numpy as np


def _nearest_ok(x, s, code):
    """code is a nearest integer in [-7,7] to x/s (ties either way)."""
    t = x.astype(np.float64) / s
    err = np.abs(t - code)
    alt = np.minimum(np.abs(t - (code - 1)), np.abs(t - (code + 1)))
    return np.all(err <= alt + 1e-6) and np.all(err <= 0.5 + 1e-6)


def test_qk_blocks_properties(ora):
    rng = np.random.default_rng(0)
    N, H, D = 150, 3, 64          # 3 blocks, last one holds 22 tokens
    y = (rng.standard_normal((1, N, H, D)) * rng.uniform(0.1, 5, size=(1, 1, H, 1))).astype(np.float32)
    codes, s = ora.quant_qk(y)
    assert codes.shape == (1, H, N, D) and s.shape == (1, H, 3)
    for h in range(H):
        for blk in range(3):
            n0, n1 = blk * 64, min(N, blk * 64 + 64)
            xb = y[0, n0:n1, h, :]
            cb = codes[0, h, n0:n1, :].astype(np.int64)
            sc = float(s[0, h, blk])
            assert np.isclose(sc * 7, np.abs(xb).max(), rtol=1e-6)
            assert np.abs(cb).max() == 7
            assert _nearest_ok(xb, sc, cb)
            assert np.max(np.abs(xb - sc * cb)) <= sc / 2 * (1 + 1e-5)


def test_partial_block_uses_valid_tokens_only(ora):
    rng = np.random.default_rng(1)
    N, D = 70, 64
    y = rng.standard_normal((1, N, 1, D)).astype(np.float32)
    y[0, 64:] *= 0.01          # tail block of 6 small tokens
    _, s = ora.quant_qk(y)
    assert np.isclose(s[0, 0, 1] * 7, np.abs(y[0, 64:]).max(), rtol=1e-6)


def test_lossless_on_representable_inputs(ora):
    rng = np.random.default_rng(2)
    N, H, D = 128, 2, 64
    ints = rng.integers(-7, 8, size=(1, N, H, D))
    ints[0, 0, :, 0] = 7
    ints[0, 64, :, 0] = -7
    y = (ints * 2.0 ** -3).astype(np.float32)
    codes, s = ora.quant_qk(y)
    assert np.all(s == np.float32(2.0 ** -3))
    assert np.array_equal(codes, np.transpose(ints, (0, 2, 1, 3)).astype(np.int8))
    vc, vs = ora.quant_v(y)
    assert np.all(vs == np.float32(2.0 ** -3))
    assert np.array_equal(vc, np.transpose(ints, (0, 2, 1, 3)).astype(np.int8))


def test_zero_groups(ora):
    y = np.zeros((1, 100, 2, 64), np.float32)
    y[0, :64, 1, :] = 1.0
    codes, s = ora.quant_qk(y)
    assert s[0, 0, 0] == 0 and s[0, 0, 1] == 0 and s[0, 1, 1] == 0
    assert np.all(codes[0, 0] == 0) and np.all(codes[0, 1, 64:] == 0)
    assert np.all(codes[0, 1, :64] == 7)
    vc, vs = ora.quant_v(y)
    assert np.all(vs[0, 0] == 0) and np.all(vc[0, 0] == 0)


def test_v_per_channel(ora):
    rng = np.random.default_rng(3)
    N, H, D = 333, 2, 64
    v = (rng.standard_normal((1, N, H, D)) * np.linspace(0.01, 30, D)).astype(np.float32)
    vc, vs = ora.quant_v(v)
    for h in range(H):
        for d in range(D):
            col = v[0, :, h, d]
            c = vc[0, h, :, d].astype(np.int64)
            sc = float(vs[0, h, d])
            assert np.isclose(sc * 7, np.abs(col).max(), rtol=1e-6)
            assert np.abs(c).max() == 7
            assert _nearest_ok(col, sc, c)


def test_exact_ties_round_to_even(ora):
    """Reading: round-to-nearest-even.  With amax = 7 the step is exactly 1,
    so x = n + 1/2 is an exact tie."""
    x = np.array([7.0, 2.5, -2.5, 0.5, -0.5, 1.5, 3.5, -4.5, 6.5], np.float32)
    y = np.zeros((1, 64, 1, 16), np.float32)
    y[0, : x.size, 0, 0] = x
    codes, s = ora.quant_qk(y)
    assert s[0, 0, 0] == 1.0
    assert codes[0, 0, : x.size, 0].tolist() == [7, 2, -2, 0, 0, 2, 4, -4, 6]
