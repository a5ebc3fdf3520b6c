"""Pins of the oracle's INT4 online-softmax attention.

Page: RotateAttention review -- abstract (P = exp(QK - max(QK)) inside INT4
FlashAttention), Sec. 4.2 (P codes round(15 p) - 8).  Checked against closed
forms that hold exactly (Q = 0, one key, a dominating key, tiles of equal
scores whose weights follow from the running max), against integer matrix
products for the exact integer quantities, and against textbook fp64
attention on well-conditioned data (error reported, loosely bounded).
"""
import numpy as np
import pytest

import brute_int4 as brute
from oracle import ref_fp64 as ref


def _pro(qc, kc, vc, sq=None, sk=None, sv=None):
    """Build oracle inputs for one (b, h) directly from codes [N, D]."""
    N, D = qc.shape
    nblk = (N + 63) // 64
    sq = np.ones(nblk, np.float32) if sq is None else np.asarray(sq, np.float32)
    sk = np.ones(nblk, np.float32) if sk is None else np.asarray(sk, np.float32)
    sv = np.ones(D, np.float32) if sv is None else np.asarray(sv, np.float32)
    return dict(q_codes=qc[None, None].astype(np.int8), s_q=sq[None, None],
                k_codes=kc[None, None].astype(np.int8), s_k=sk[None, None],
                v_codes=vc[None, None].astype(np.int8), s_v=sv[None, None])


def _alpha(D):
    return np.float32(np.log2(np.e) * (1.0 / np.sqrt(D)))


def _rn32(exact):
    """The running max of a step: the scaled max score rounded to nearest."""
    return np.float32(exact)


def _d(S, c, m):
    """The exponent f32(S c - m): the exact value rounded once."""
    return brute.f32_of_exact_sum(np.float64(S) * np.float64(c), -np.float64(m))


def test_zero_queries_give_channel_means(ora):
    rng = np.random.default_rng(0)
    N, D = 150, 64
    vc = rng.integers(-7, 8, size=(N, D))
    sv = rng.uniform(0.1, 2, D).astype(np.float32)
    pro = _pro(np.zeros((N, D)), rng.integers(-7, 8, size=(N, D)), vc, sv=sv)
    o = ora.attention_rows(pro, 0, 0, np.arange(N))
    want = sv.astype(np.float64) * vc.mean(axis=0)
    assert np.allclose(o, want[None, :], rtol=1e-13, atol=1e-13)


def test_single_token(ora):
    rng = np.random.default_rng(1)
    D = 128
    vc = rng.integers(-7, 8, size=(1, D))
    sv = rng.uniform(0.1, 2, D).astype(np.float32)
    pro = _pro(rng.integers(-7, 8, size=(1, D)), rng.integers(-7, 8, size=(1, D)), vc,
               sq=[0.3], sk=[0.7], sv=sv)
    o = ora.attention_rows(pro, 0, 0, [0])
    assert np.allclose(o[0], sv * vc[0], rtol=1e-14)


def test_dominating_key_first(ora):
    """One key 98*c grid steps above the rest: every other key gets u = 0."""
    rng = np.random.default_rng(2)
    N, D = 256, 64
    qc = np.zeros((N, D), int)
    qc[:, 0] = 7
    kc = rng.integers(-7, 8, size=(N, D))
    kc[:, 0] = -7
    kc[5, 0] = 7
    vc = rng.integers(-7, 8, size=(N, D))
    sv = rng.uniform(0.5, 1.5, D).astype(np.float32)
    qc[:, 1:] = 0
    pro = _pro(qc, kc, vc, sv=sv)
    o = ora.attention_rows(pro, 0, 0, np.arange(0, N, 17))
    assert np.allclose(o, (sv * vc[5])[None, :], rtol=1e-14)


@pytest.mark.parametrize("order", ["rising", "falling"])
def test_two_tiles_of_equal_scores(ora, order):
    """Tile 0 keys all score a, tile 1 keys all score b.  With a rising max the
    first tile is reweighted by beta = 2^(m0 - m1); with a falling max the
    second tile's keys get the code of their exponent against m0.  The two
    query blocks carry different Q scales, so each row uses its own block's."""
    D = 64
    N = 128
    a, b = (2, 7) if order == "rising" else (7, 2)
    qc = np.zeros((N, D), int)
    qc[:, 0] = 1
    kc = np.zeros((N, D), int)
    kc[:64, 0] = a
    kc[64:, 0] = b
    rng = np.random.default_rng(3)
    vc = rng.integers(-7, 8, size=(N, D))
    sv = rng.uniform(0.5, 1.5, D).astype(np.float32)
    sq = np.array([1.0, 0.625], np.float32)
    sk = np.array([1.0, 1.0], np.float32)
    pro = _pro(qc, kc, vc, sq=sq, sk=sk, sv=sv)
    o, m = ora.attention_rows(pro, 0, 0, np.arange(N), with_m=True)

    v0 = vc[:64].sum(axis=0).astype(np.float64)
    v1 = vc[64:].sum(axis=0).astype(np.float64)
    for qb in range(2):
        c = np.float32(np.float32(sq[qb] * sk[0]) * _alpha(D))
        m0 = _rn32(a * float(c))
        m1 = _rn32(b * float(c))
        rows = slice(qb * 64, qb * 64 + 64)
        if order == "rising":
            beta = 2.0 ** (float(m0) - float(m1))
            want = (beta * 15 * v0 + 15 * v1) / (beta * 15 * 64 + 15 * 64)
            assert np.all(m[rows] == m1)
        else:
            d = float(_d(b, c, m0))
            u1 = int(np.floor(15 * 2.0 ** d + 0.5))
            assert 0 < u1 < 15
            want = (15 * v0 + u1 * v1) / (15 * 64 + u1 * 64)
            assert np.all(m[rows] == m0)
        assert np.allclose(o[rows], (sv * want)[None, :], rtol=1e-13)


def test_keys_above_the_rounded_max_get_the_top_code(ora):
    """The step max is m = f32(S_max c), rounded to nearest.  With a large
    score scale c it is coarse and may lie below S_max c; the max key then
    has d = f32(S_max c - m) > 0 and still gets the top code 15 - 8 = 7,
    while a key one score lower is mapped against m as usual."""
    D, N = 64, 64
    qc = np.zeros((N, D), int)
    qc[:, 0] = 7
    qc[:, 1] = 1
    kc = np.zeros((N, D), int)
    kc[:, 0] = -7                      # background keys: S = -49
    kc[3, 0] = 7                       # S = 49
    kc[9, 0] = 7
    kc[9, 1] = -1                      # S = 48
    rng = np.random.default_rng(21)
    vc = rng.integers(-7, 8, size=(N, D))
    alpha = _alpha(D)
    picked = None
    for i in range(400):
        s = np.float32(np.sqrt(2.0 ** 14 / (49 * float(alpha))) * (1.0 + i * 1e-4))
        c = np.float32(np.float32(s * s) * alpha)
        exact = 49.0 * float(c)
        m = _rn32(exact)
        if float(m) < exact:
            picked = (s, c, m)
            break
    assert picked is not None
    s, c, m = picked
    pro = _pro(qc, kc, vc, sq=[s], sk=[s])
    t = ora.attention_tile(pro, 0, 0, 0, 0)
    assert np.all(t["m_after"] == m)
    assert np.all(t["d_val"][:, 3] > 0)
    assert np.all(t["p_code"][:, 3] == 7)
    d9 = float(_d(48, c, m))
    assert np.all(t["d_val"][:, 9] == np.float32(d9))
    u9 = int(np.floor(15 * 2.0 ** d9 + 0.5))
    assert np.all(t["p_code"][:, 9] == u9 - 8)
    assert np.all(t["p_code"][:, 0] == -8)


def test_tile_dump_integers(ora):
    rng = np.random.default_rng(4)
    N, D = 200, 128
    qc = rng.integers(-7, 8, size=(N, D))
    kc = rng.integers(-7, 8, size=(N, D))
    vc = rng.integers(-7, 8, size=(N, D))
    pro = _pro(qc, kc, vc, sq=rng.uniform(0.05, 0.2, 4), sk=rng.uniform(0.05, 0.2, 4))
    prev = None
    live = 0
    for kb in range(4):
        t = ora.attention_tile(pro, 0, 0, 1, kb)
        j0, j1 = kb * 64, min(N, kb * 64 + 64)
        S = qc[64:128] @ kc[j0:j1].T
        assert np.array_equal(t["s_int"][:, : j1 - j0], S)
        assert np.abs(S).max() <= 49 * D
        pc = t["p_code"].astype(np.int64)
        assert pc.min() >= -8 and pc.max() <= 7
        assert np.all(pc[:, j1 - j0:] == -8)
        assert np.array_equal(t["pv_int"], pc[:, : j1 - j0] @ vc[j0:j1])
        assert np.abs(t["pv_int"]).max() <= 8 * 7 * 64
        if prev is not None:
            assert np.all(t["m_after"] >= prev)
        prev = t["m_after"]
        # the exponent is S c - m rounded once, and the code its exact rounding
        c = np.float32(np.float32(pro["s_q"][0, 0, 1] * pro["s_k"][0, 0, kb]) * _alpha(D))
        d = _d(S, c, t["m_after"][:, None])
        assert np.array_equal(t["d_val"][:, : j1 - j0].view(np.uint32), d.view(np.uint32))
        u = np.floor(15 * np.exp2(d.astype(np.float64)) + 0.5)
        assert np.array_equal(pc[:, : j1 - j0], u - 8)
        live += int((u > 0).sum())
        # codes are monotone in the score within the tile
        for r in range(0, 64, 9):
            order = np.argsort(S[r], kind="stable")
            assert np.all(np.diff(pc[r, : j1 - j0][order]) >= 0)
    assert live > 100


def test_thread_count_does_not_change_results(ora):
    rng = np.random.default_rng(5)
    N, D = 300, 64
    pro = _pro(rng.integers(-7, 8, size=(N, D)), rng.integers(-7, 8, size=(N, D)),
               rng.integers(-7, 8, size=(N, D)), sq=rng.uniform(0.01, 0.1, 5),
               sk=rng.uniform(0.01, 0.1, 5))
    n0 = ora.get_threads()
    ora.set_threads(1)
    a = ora.attention_rows(pro, 0, 0, np.arange(N))
    ora.set_threads(max(2, n0))
    b = ora.attention_rows(pro, 0, 0, np.arange(N))
    ora.set_threads(n0)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("rot", [0, 1, 2])
def test_close_to_full_precision_on_well_conditioned_data(ora, rot):
    """INT4 attention vs textbook fp64 attention (no outliers): cosine and
    error are reported by the benches; here only a loose bound is asserted."""
    rng = np.random.default_rng(6)
    grid, seg = (2, 5, 12), (24, 20, 20)
    N, H, D = 120, 2, 64
    q = rng.standard_normal((1, N, H, D)).astype(np.float32)
    k = rng.standard_normal((1, N, H, D)).astype(np.float32)
    v = rng.standard_normal((1, N, H, D)).astype(np.float32)
    pro = ora.prologue(q, k, v, grid, seg, 10000.0, rot)
    o = ora.attention_full(pro)
    want = ref.reference_output(q, k, v, grid, seg)
    cos = (o * want).sum() / np.sqrt((o * o).sum() * (want * want).sum())
    assert cos > 0.9


# ---- symmetric P mode (p_mode = 1: code = round(7 p) in [0, 7]) ------------

def test_symmetric_zero_queries_give_channel_means(ora):
    """Q = 0: every p is 1, code 7 for every key; the scale cancels in A/L, so
    the output is again the mean of the dequantized V rows."""
    rng = np.random.default_rng(11)
    N, D = 150, 64
    vc = rng.integers(-7, 8, size=(N, D))
    sv = rng.uniform(0.5, 2.0, D).astype(np.float32)
    pro = _pro(np.zeros((N, D), int), rng.integers(-7, 8, size=(N, D)), vc, sv=sv)
    o = ora.attention_rows(pro, 0, 0, np.arange(N), p_mode=1)
    want = sv.astype(np.float64) * vc.mean(axis=0)
    assert np.allclose(o, want[None, :], rtol=1e-12, atol=1e-12)
    t = ora.attention_tile(pro, 0, 0, 0, 2, p_mode=1)
    nk = N - 128
    assert np.all(t["p_code"][:, :nk] == 7) and np.all(t["p_code"][:, nk:] == 0)


def test_symmetric_tile_codes_agree_with_the_optimized_ones(ora):
    """Both modes round the same p of every key (same scores, running max and
    grid exponent): u7 = round(7 p) and u15 = round(15 p) must bracket a common
    p, i.e. the intervals [(u7 - 1/2)/7, (u7 + 1/2)/7] and
    [(u15 - 1/2)/15, (u15 + 1/2)/15] meet.  PV is the code matrix times V."""
    rng = np.random.default_rng(12)
    N, D = 200, 128
    qc = rng.integers(-7, 8, size=(N, D))
    kc = rng.integers(-7, 8, size=(N, D))
    vc = rng.integers(-7, 8, size=(N, D))
    pro = _pro(qc, kc, vc, sq=rng.uniform(0.001, 0.01, 4), sk=rng.uniform(0.001, 0.01, 4))
    for kb in range(4):
        t1 = ora.attention_tile(pro, 0, 0, 1, kb, p_mode=1)
        t0 = ora.attention_tile(pro, 0, 0, 1, kb)
        j0, j1 = kb * 64, min(N, kb * 64 + 64)
        assert np.array_equal(t1["s_int"], t0["s_int"])
        assert np.array_equal(t1["m_after"].view(np.uint32), t0["m_after"].view(np.uint32))
        u7 = t1["p_code"][:, : j1 - j0].astype(np.float64)
        u15 = t0["p_code"][:, : j1 - j0].astype(np.float64) + 8
        assert u7.min() >= 0 and u7.max() <= 7
        lo = np.maximum((u7 - 0.5) / 7, (u15 - 0.5) / 15)
        hi = np.minimum((u7 + 0.5) / 7, (u15 + 0.5) / 15)
        assert np.all(lo <= hi + 1e-12)
        assert np.all(t1["p_code"][:, j1 - j0:] == 0)
        assert np.array_equal(t1["pv_int"], t1["p_code"][:, : j1 - j0].astype(np.int64) @ vc[j0:j1])


def test_range_optimized_map_is_closer_to_full_precision(ora):
    """[RA] Sec. 4.2's claim on synthetic data: with the rest of the path
    fixed, the full-range P map gives a smaller error against fp64 attention
    than the symmetric map."""
    rng = np.random.default_rng(13)
    grid, seg = (2, 6, 16), (24, 20, 20)
    N, H, D = 192, 2, 64
    q = rng.standard_normal((1, N, H, D)).astype(np.float32)
    k = rng.standard_normal((1, N, H, D)).astype(np.float32)
    v = rng.standard_normal((1, N, H, D)).astype(np.float32)
    pro = ora.prologue(q, k, v, grid, seg, 10000.0, 2)
    want = ref.reference_output(q, k, v, grid, seg)
    e0 = np.abs(ora.attention_full(pro) - want).mean()
    e1 = np.abs(ora.attention_full(pro, p_mode=1) - want).mean()
    assert e0 < e1
