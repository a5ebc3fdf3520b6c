"""GPU parity of the HIP path against the CPU oracle (through the C ABI).

Integer quantities (Q/K/V codes, scales, scores, P codes, PV sums, running
max) must match bit for bit -- in the step-by-step tile dump and, through its
parity variant, in the benchmarked kernel itself; the fp32 output must match
the oracle's binary64 float path within max-abs OUT_TOL (1e-5; the float path
is the rescale by 2^(m_old - m), the fp32 accumulation and the final
division); the error against textbook fp64 attention is printed.  Shapes span several 64-token tiles with ragged
tails; the full-size workloads are checked in test_gpu_fullsize.py.
"""
import numpy as np
import pytest
import torch

from bit_quantized_attention_rope3d_amd import inputs
from bit_quantized_attention_rope3d_amd.api import Plan, attn_fwd, pmap_device
from oracle import ref_fp64

from gpu_helpers import OUT_TOL, bf16_round, cosine, dev, plan_for, say

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

CASES = {
    "tiny": inputs.get("tiny"),
    "tiny_half": inputs.get("tiny").with_(name="tiny_half", rot="half"),
    "tiny_none": inputs.get("tiny").with_(name="tiny_none", rot="none"),
    "small": inputs.small(),                                             # 105 tokens, D128, bf16
    "small_d64": inputs.small("small_d64", heads=2, head_dim=64, grid=(2, 7, 9), rot="interleaved",
                              dtype="f32", seed=12),                     # 126 tokens
    "medium": inputs.small("medium", heads=2, head_dim=128, grid=(3, 17, 23), rot="interleaved",
                           seed=13),                                     # 1173 tokens, tail 21
    "medium_out": inputs.Workload("medium_out", 1, 2, 128, (3, 16, 20), (44, 42, 42), rot="half",
                                  seed=14, outliers_per_segment=(1, 1, 1)),   # 960 tokens
    "batch2": inputs.small("batch2", heads=2, head_dim=128, grid=(2, 9, 11), rot="half", seed=15,
                           batch=2),                                     # 198 tokens, B=2
}


def _prep(ora, w):
    q, k, v, _ = inputs.generate(w)
    pro = ora.prologue(q, k, v, w.grid, w.seg, w.theta, w.rot_id)
    return q, k, v, pro


@pytest.mark.parametrize("p_mode", [0, 1])
def test_pmap_exhaustive(ora, p_mode):
    """Every binary32 exponent d in [T_0 - 1, -0] (about 1.1e9 values, T_0 the
    lowest threshold), plus zeros, small positive d (keys above a rounded
    running max), -inf and far-negative values, through the attention
    kernels' P-map path (table lookup, exact decision of the 15 table cells
    that hold a rounding boundary, operand packing): 0 mismatches against
    the oracle's threshold count, itself pinned to round(15 2^d) in
    test_oracle_pmap.py."""
    T = ora.pmap_thresholds(p_mode)
    lo = int(np.array(np.float32(T[0]) - np.float32(1.0), np.float32).view(np.uint32))
    start = 0x80000000
    chunk = 1 << 26
    total = bad_total = 0
    out = torch.empty(chunk, dtype=torch.uint8, device="cuda")
    for a in range(start, lo + 1, chunk):
        b = min(a + chunk, lo + 1)
        bits = torch.arange(a, b, dtype=torch.int64, device="cuda").to(torch.int32)
        u_gpu = pmap_device(bits.view(torch.float32), p_mode, out=out[: b - a]).cpu().numpy()
        d = np.arange(a, b, dtype=np.uint32).view(np.float32)
        u_ora = ora.pmap(d, p_mode=p_mode)
        bad = np.nonzero(u_gpu != u_ora)[0]
        assert bad.size == 0, (d[bad[:10]], u_gpu[bad[:10]], u_ora[bad[:10]])
        total += b - a
    extra = np.array([-np.inf, -3.0e38, -1.0e30, -2.0 ** 24, -1e9, -8.0, -7.999, -1.0, 0.0, -0.0,
                      1e-30, 1e-7, 0.01, 1.0], np.float32)
    u_gpu = pmap_device(dev(extra), p_mode).cpu().numpy()
    assert np.array_equal(u_gpu, ora.pmap(np.minimum(extra, 0), p_mode=p_mode))
    say("pmap exhaustive (p_mode %d): %d binary32 exponents + %d extremes, 0 mismatches"
        % (p_mode, total, extra.size))
    assert total > 1_000_000_000


@pytest.mark.parametrize("case", list(CASES))
def test_prologue_bit_exact(ora, case):
    w = CASES[case]
    q, k, v, pro = _prep(ora, w)
    p = plan_for(w)
    got = p.debug_prologue(dev(q), dev(k), dev(v))
    for key in ("q_codes", "k_codes", "v_codes"):
        nbad = int((got[key] != pro[key]).sum())
        assert nbad == 0, (case, key, nbad)
    for key in ("s_q", "s_k", "s_v"):
        assert np.array_equal(got[key].view(np.uint32), pro[key].view(np.uint32)), (case, key)
    say("prologue %s: codes and scales bit-exact" % case)


@pytest.mark.parametrize("case", ["tiny", "small", "small_d64", "medium", "medium_out", "batch2"])
def test_tiles_bit_exact(ora, case):
    w = CASES[case]
    q, k, v, pro = _prep(ora, w)
    p = plan_for(w)
    ws = p.workspace()
    p.prologue(dev(q), dev(k), dev(v), ws)
    N = w.tokens
    nb = (N + 63) // 64
    rng = np.random.default_rng(0)
    picks = {(0, 0), (nb - 1, nb - 1), (0, nb - 1), (nb - 1, 0), (nb // 2, nb // 2)}
    picks |= {tuple(rng.integers(0, nb, 2).tolist()) for _ in range(3)}
    for b in range(w.batch):
        for h in sorted({0, w.heads - 1}):
            for qb, kb in sorted(picks):
                g = p.debug_tile(ws, b, h, qb, kb)
                o = ora.attention_tile({kk: vv[b:b + 1] for kk, vv in pro.items()}, 0, h, qb, kb)
                n = o["s_int"].shape[0]
                nk = min(64, N - kb * 64)
                assert np.array_equal(g["s_int"][:n, :nk], o["s_int"][:, :nk]), (case, b, h, qb, kb, "S")
                assert np.array_equal(g["p_code"][:n], o["p_code"]), (case, b, h, qb, kb, "P")
                assert np.array_equal(g["pv_int"][:n], o["pv_int"]), (case, b, h, qb, kb, "PV")
                assert np.array_equal(g["m_after"][:n].view(np.uint32),
                                      o["m_after"].view(np.uint32)), (case, b, h, qb, kb, "m")
    say("tiles %s: %d tiles bit-exact" % (case, len(picks) * w.batch * len({0, w.heads - 1})))


@pytest.mark.parametrize("case", list(CASES))
def test_output_matches_oracle(ora, case):
    w = CASES[case]
    q, k, v, pro = _prep(ora, w)
    p = plan_for(w)
    o = p.forward(dev(q), dev(k), dev(v)).cpu().numpy()
    want = ora.attention_full(pro)
    err = np.abs(o - want).max()
    cos = cosine(o, want)
    ref = ref_fp64.reference_output(ora.as_f32(q), ora.as_f32(k), ora.as_f32(v), w.grid, w.seg, w.theta)
    say("output %s: max|gpu-oracle| %.2e  cos %.7f | vs fp64 attention: max %.3e cos %.5f"
        % (case, err, cos, np.abs(o - ref).max(), cosine(o, ref)))
    assert err <= OUT_TOL and cos >= 0.999999


@pytest.mark.parametrize("case", list(CASES))
def test_production_kernel_integers(ora, case):
    """The benchmarked attention kernel itself (its parity variant: same
    kernel, LDS ring, barriers, peeled steps and workgroup order) against the
    oracle for every query row: final running max bit for bit, and two
    fingerprints of all of the row's P codes (sum of u, and sum of u times a
    hash of the key index, mod 2^32).  Its output is bit-identical to the
    production instantiation's."""
    w = CASES[case]
    q, k, v, pro = _prep(ora, w)
    p = plan_for(w)
    ws = p.workspace()
    p.prologue(dev(q), dev(k), dev(v), ws)
    o_prod = p.main(p.empty_out(), ws).cpu().numpy()
    o_dbg, rows = p.row_digests(ws)
    rows = rows.cpu().numpy().view(np.uint32)
    assert np.array_equal(o_dbg.cpu().numpy().view(np.uint32), o_prod.view(np.uint32))
    N = w.tokens
    for b in range(w.batch):
        for h in range(w.heads):
            sl = {kk: vv[b:b + 1] for kk, vv in pro.items()}
            ds, dh, m = ora.code_digests(sl, 0, h, np.arange(N))
            r = rows[b, h]
            assert np.array_equal(r[:, 0], m.view(np.uint32)), (case, b, h, "m")
            assert np.array_equal(r[:, 1], ds), (case, b, h, "sum u")
            assert np.array_equal(r[:, 2], dh), (case, b, h, "hash u")
    say("production kernel %s: running max and P-code fingerprints of all %d rows bit-exact"
        % (case, w.batch * w.heads * N))


def test_bf16_output_option(ora):
    w = CASES["medium"]
    q, k, v, pro = _prep(ora, w)
    p = plan_for(w, out_dtype="bf16")
    o = p.forward(dev(q), dev(k), dev(v)).float().cpu().numpy()
    want = ora.attention_full(pro).astype(np.float32)
    wb = bf16_round(want)
    ulp = np.maximum(np.abs(wb), 1e-30) * 2.0 ** -7
    assert np.all(np.abs(o - wb) <= ulp + OUT_TOL)


def test_zero_queries_and_single_token(ora):
    w = CASES["small"]
    q, k, v, _ = inputs.generate(w)
    q[:] = 0
    pro = ora.prologue(q, k, v, w.grid, w.seg, w.theta, w.rot_id)
    o = plan_for(w).forward(dev(q), dev(k), dev(v)).cpu().numpy()
    want = pro["s_v"][:, None, :, :] * pro["v_codes"].astype(np.float64).mean(axis=2)[:, None, :, :]
    assert np.abs(o - want).max() <= 1e-5
    w1 = inputs.Workload("one", 1, 3, 128, (1, 1, 1), (44, 42, 42), rot="half", seed=3)
    q, k, v, _ = inputs.generate(w1)
    pro = ora.prologue(q, k, v, w1.grid, w1.seg, w1.theta, w1.rot_id)
    o = plan_for(w1).forward(dev(q), dev(k), dev(v)).cpu().numpy()
    want = pro["s_v"][:, None] * pro["v_codes"].astype(np.float64)[:, :, :1].transpose(0, 2, 1, 3)
    assert np.abs(o - want).max() <= 1e-6


@pytest.mark.parametrize("p_mode", [0, 1])
def test_zero_scale_blocks(ora, p_mode):
    """Scale-0 blocks give c = 0 for their steps: an all-zero K block as the
    ragged last block (every query's last step) and an all-zero Q block (every
    step of those queries).  All valid keys of such a step share one grid
    exponent, and the padded keys of the ragged step must still add nothing
    to the row sum."""
    w = CASES["medium"]
    q, k, v, _ = inputs.generate(w)
    N = w.tokens
    nb = (N + 63) // 64
    k[:, (nb - 1) * 64:] = 0
    q[:, 64:128] = 0
    pro = ora.prologue(q, k, v, w.grid, w.seg, w.theta, w.rot_id)
    assert np.all(pro["s_k"][..., -1] == 0) and np.all(pro["s_q"][..., 1] == 0)
    p = plan_for(w, p_mode=p_mode)
    o = p.forward(dev(q), dev(k), dev(v)).cpu().numpy()
    want = ora.attention_full(pro, p_mode=p_mode)
    err, cos = np.abs(o - want).max(), cosine(o, want)
    say("zero-scale blocks (p_mode %d): max|gpu-oracle| %.2e cos %.7f" % (p_mode, err, cos))
    assert err <= OUT_TOL and cos >= 0.999999
    ws = p.workspace()
    p.prologue(dev(q), dev(k), dev(v), ws)
    for qb, kb in [(0, nb - 1), (1, nb - 1), (1, 0), (nb - 1, nb - 1)]:
        g = p.debug_tile(ws, 0, 1, qb, kb)
        t = ora.attention_tile(pro, 0, 1, qb, kb, p_mode=p_mode)
        n = t["s_int"].shape[0]
        assert np.array_equal(g["p_code"][:n], t["p_code"]), (qb, kb, "P")
        assert np.array_equal(g["pv_int"][:n], t["pv_int"]), (qb, kb, "PV")
        assert np.array_equal(g["m_after"][:n].view(np.uint32), t["m_after"].view(np.uint32)), (qb, kb, "m")


def test_large_scores(ora):
    """Q and K scaled by 16 make the score scale c 256 times larger, so the
    step max m = f32(S_max c) is coarse and can round below S_max c: those
    keys have d > 0 and the top code.  The codes and the running max must
    still match the oracle bit for bit."""
    w = CASES["medium"].with_(name="large", dtype="f32")
    q, k, v, _ = inputs.generate(w)
    q *= np.float32(16.0)
    k *= np.float32(16.0)
    pro = ora.prologue(q, k, v, w.grid, w.seg, w.theta, w.rot_id)
    p = plan_for(w)
    o = p.forward(dev(q), dev(k), dev(v)).cpu().numpy()
    want = ora.attention_full(pro)
    err, cos = np.abs(o - want).max(), cosine(o, want)
    say("large scores: max|gpu-oracle| %.2e cos %.7f" % (err, cos))
    assert err <= OUT_TOL and cos >= 0.999999
    ws = p.workspace()
    p.prologue(dev(q), dev(k), dev(v), ws)
    nb = (w.tokens + 63) // 64
    for qb, kb in [(0, 0), (3, 7), (nb - 1, nb - 1), (5, nb - 1)]:
        g = p.debug_tile(ws, 0, 1, qb, kb)
        t = ora.attention_tile(pro, 0, 1, qb, kb)
        n = t["s_int"].shape[0]
        assert np.array_equal(g["p_code"][:n], t["p_code"]), (qb, kb, "P")
        assert np.array_equal(g["pv_int"][:n], t["pv_int"]), (qb, kb, "PV")
        assert np.array_equal(g["m_after"][:n].view(np.uint32), t["m_after"].view(np.uint32)), (qb, kb, "m")


def test_deterministic(ora):
    w = CASES["medium"]
    q, k, v, _ = inputs.generate(w)
    p = plan_for(w)
    a = p.forward(dev(q), dev(k), dev(v)).cpu().numpy()
    b = p.forward(dev(q), dev(k), dev(v)).cpu().numpy()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_simple_entry_point_matches_plan(ora):
    w = CASES["small"]
    q, k, v, _ = inputs.generate(w)
    a = plan_for(w).forward(dev(q), dev(k), dev(v)).cpu().numpy()
    b = attn_fwd(dev(q), dev(k), dev(v), w.grid, w.seg, rot=w.rot).cpu().numpy()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("case", ["small", "small_d64", "medium", "medium_out"])
def test_bf16_path_vs_fp64(ora, case):
    """The bf16 fallback against fp64 attention on the same bf16-rounded RoPE'd
    Q/K (the fallback's only input rounding); the remaining error is P rounded
    to bf16 and fp32 accumulation.  The error against exact fp64 attention of
    the unrounded inputs is printed as well."""
    w = CASES[case]
    q, k, v, _ = inputs.generate(w)
    o = plan_for(w, prec="bf16").forward(dev(q), dev(k), dev(v)).cpu().numpy()
    qf, kf, vf = ora.as_f32(q), ora.as_f32(k), ora.as_f32(v)
    qr = bf16_round(ref_fp64.rope3d(qf, w.grid, w.seg, w.theta).astype(np.float32))
    kr = bf16_round(ref_fp64.rope3d(kf, w.grid, w.seg, w.theta).astype(np.float32))
    ref = ref_fp64.attention(qr, kr, bf16_round(vf))
    exact = ref_fp64.reference_output(qf, kf, vf, w.grid, w.seg, w.theta)
    err, cos = np.abs(o - ref).max(), cosine(o, ref)
    say("bf16 path %s: vs fp64 on bf16 inputs max %.3e cos %.7f | vs exact fp64 max %.3e cos %.6f"
        % (case, err, cos, np.abs(o - exact).max(), cosine(o, exact)))
    assert cos >= 0.9999 and err <= 2e-2


# ---- symmetric P mode (p_mode = 1) ------------------------------------------

@pytest.mark.parametrize("case", ["tiny", "small", "small_d64", "medium"])
def test_symmetric_mode_matches_oracle(ora, case):
    """p_mode 1 (code = round(7 p), the baseline of [RA] Sec. 4.2) through the
    same kernels: tiles bit-exact, output within tolerance of the oracle's
    float path; errors of both maps against fp64 attention are printed."""
    w = CASES[case]
    q, k, v, pro = _prep(ora, w)
    p = plan_for(w, p_mode=1)
    ws = p.workspace()
    p.prologue(dev(q), dev(k), dev(v), ws)
    N = w.tokens
    nb = (N + 63) // 64
    for b in range(w.batch):
        for h in sorted({0, w.heads - 1}):
            for qb, kb in sorted({(0, 0), (nb - 1, nb - 1), (0, nb - 1), (nb // 2, nb // 2)}):
                g = p.debug_tile(ws, b, h, qb, kb)
                t = ora.attention_tile({kk: vv[b:b + 1] for kk, vv in pro.items()}, 0, h, qb, kb, p_mode=1)
                n = t["s_int"].shape[0]
                assert np.array_equal(g["p_code"][:n], t["p_code"]), (case, b, h, qb, kb, "P")
                assert np.array_equal(g["pv_int"][:n], t["pv_int"]), (case, b, h, qb, kb, "PV")
                assert np.array_equal(g["m_after"][:n].view(np.uint32), t["m_after"].view(np.uint32))
    o = p.forward(dev(q), dev(k), dev(v)).cpu().numpy()
    want = ora.attention_full(pro, p_mode=1)
    err, cos = np.abs(o - want).max(), cosine(o, want)
    ref = ref_fp64.reference_output(ora.as_f32(q), ora.as_f32(k), ora.as_f32(v), w.grid, w.seg, w.theta)
    o0 = plan_for(w).forward(dev(q), dev(k), dev(v)).cpu().numpy()
    say("symmetric %s: max|gpu-oracle| %.2e cos %.7f | vs fp64: symmetric mean %.3e, range-optimized mean %.3e"
        % (case, err, cos, np.abs(o - ref).mean(), np.abs(o0 - ref).mean()))
    assert err <= OUT_TOL and cos >= 0.999999


# ---- V-side Hadamard (v_hadamard = 1) ---------------------------------------

@pytest.mark.parametrize("case", ["tiny", "small", "small_d64", "medium", "batch2"])
def test_v_hadamard_matches_oracle(ora, case):
    """V rows times H = Walsh-Hadamard / sqrt(D) before the per-channel INT4
    quantization (the summary's offline-fused Hadamard on V), output rows
    times H again: V codes and scales bit-exact, tiles bit-exact, output within
    tolerance of the oracle's float path."""
    w = CASES[case]
    q, k, v, _ = inputs.generate(w)
    pro = ora.prologue(q, k, v, w.grid, w.seg, w.theta, w.rot_id, v_hadamard=True)
    p = plan_for(w, v_hadamard=1)
    got = p.debug_prologue(dev(q), dev(k), dev(v))
    assert np.array_equal(got["v_codes"], pro["v_codes"]), case
    assert np.array_equal(got["s_v"].view(np.uint32), pro["s_v"].view(np.uint32)), case
    ws = p.workspace()
    p.prologue(dev(q), dev(k), dev(v), ws)
    nb = (w.tokens + 63) // 64
    for qb, kb in sorted({(0, 0), (nb - 1, nb - 1), (0, nb - 1)}):
        g = p.debug_tile(ws, 0, 0, qb, kb)
        t = ora.attention_tile({kk: vv[0:1] for kk, vv in pro.items()}, 0, 0, qb, kb)
        n = t["s_int"].shape[0]
        assert np.array_equal(g["pv_int"][:n], t["pv_int"]), (case, qb, kb)
    o = p.forward(dev(q), dev(k), dev(v)).cpu().numpy()
    want = ora.attention_full(pro, v_hadamard=True)
    err, cos = np.abs(o - want).max(), cosine(o, want)
    ref = ref_fp64.reference_output(ora.as_f32(q), ora.as_f32(k), ora.as_f32(v), w.grid, w.seg, w.theta)
    o0 = plan_for(w).forward(dev(q), dev(k), dev(v)).cpu().numpy()
    say("v_hadamard %s: max|gpu-oracle| %.2e cos %.7f | vs fp64 mean: with H %.3e, without %.3e"
        % (case, err, cos, np.abs(o - ref).mean(), np.abs(o0 - ref).mean()))
    assert err <= OUT_TOL and cos >= 0.999999


# ---- full rotation (rot = full) ---------------------------------------------

@pytest.mark.parametrize("case", ["tiny", "small", "small_d64", "medium"])
def test_full_rotation_matches_oracle(ora, case):
    """rot = full: the RoPE'd Q/K rows times the Walsh-Hadamard matrix (the
    dense comparator of Figs. 4-6) in the prologue; codes and scales
    bit-exact, output within tolerance of the oracle."""
    w = CASES[case].with_(name=case + "_full", rot="full")
    q, k, v, pro = _prep(ora, w)
    p = plan_for(w)
    got = p.debug_prologue(dev(q), dev(k), dev(v))
    for key in ("q_codes", "k_codes"):
        assert np.array_equal(got[key], pro[key]), (case, key)
    for key in ("s_q", "s_k"):
        assert np.array_equal(got[key].view(np.uint32), pro[key].view(np.uint32)), (case, key)
    o = p.forward(dev(q), dev(k), dev(v)).cpu().numpy()
    want = ora.attention_full(pro)
    err, cos = np.abs(o - want).max(), cosine(o, want)
    ref = ref_fp64.reference_output(ora.as_f32(q), ora.as_f32(k), ora.as_f32(v), w.grid, w.seg, w.theta)
    say("full rotation %s: max|gpu-oracle| %.2e cos %.7f | vs fp64 mean %.3e"
        % (case, err, cos, np.abs(o - ref).mean()))
    assert err <= OUT_TOL and cos >= 0.999999


def test_mfma_peak_probe():
    """The throughput probe runs for every operand type and reports a
    plausible engine clock and a positive rate."""
    from bit_quantized_attention_rope3d_amd.api import PEAK_KINDS, mfma_peak
    for kind in PEAK_KINDS:
        t, ghz = mfma_peak(kind, iters=2000)
        say("mfma probe %s: %.0f T ops/s at %.3f GHz" % (kind, t, ghz))
        assert t > 0 and 0.5 < ghz < 3.5
