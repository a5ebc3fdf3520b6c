"""Seeded random configurations through the C ABI against the oracle (and, for
the bf16 fallback, against fp64 attention of its own rounded inputs).

Each case draws batch, heads, head dim (64 or 128), a 3D grid (ragged token
counts), a valid frame/height/width split of the head dim (even, positive
segments), the rotation (none, Interleaved, Half, full Walsh-Hadamard), the
input dtype, the P mode and the V-side Hadamard, then checks every Q/K/V
code and scale bit for bit against the oracle's prologue and the output
against the oracle's binary64 float path (max-abs 1e-5), and the benchmarked
kernel's running max and P-code fingerprints of every row bit for bit.
"""
import numpy as np
import pytest
import torch

from bit_quantized_attention_rope3d_amd import inputs

from gpu_helpers import OUT_TOL, cosine, dev, plan_for, say

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

ROTS = ["none", "interleaved", "half", "full"]


def random_case(seed):
    rng = np.random.default_rng(seed)
    D = int(rng.choice([64, 128]))
    s0 = 2 * int(rng.integers(1, D // 2 - 1))
    s1 = 2 * int(rng.integers(1, (D - s0) // 2))
    seg = (s0, s1, D - s0 - s1)
    grid = tuple(int(x) for x in rng.integers(1, 7, size=3))
    w = inputs.Workload("rand%d" % seed, int(rng.integers(1, 3)), int(rng.integers(1, 4)), D, grid, seg,
                        rot=ROTS[int(rng.integers(0, 4))], dtype=str(rng.choice(["bf16", "f32"])),
                        seed=100 + seed, outliers_per_segment=(1, 1, 1))
    return w, int(rng.integers(0, 2)), int(rng.integers(0, 2))


@pytest.mark.parametrize("seed", range(16))
def test_random_configuration(ora, seed):
    w, p_mode, vh = random_case(seed)
    say("random %d: B%d H%d D%d grid %s seg %s rot %s %s p_mode %d v_hadamard %d"
        % (seed, w.batch, w.heads, w.head_dim, w.grid, w.seg, w.rot, w.dtype, p_mode, vh))
    assert all(s > 0 and s % 2 == 0 for s in w.seg) and sum(w.seg) == w.head_dim
    q, k, v, _ = inputs.generate(w)
    p = plan_for(w, p_mode=p_mode, v_hadamard=vh)
    qd, kd, vd = dev(q), dev(k), dev(v)
    ws = p.workspace()
    got = p.debug_prologue(qd, kd, vd, ws)
    pro = ora.prologue(q, k, v, w.grid, w.seg, w.theta, w.rot_id, v_hadamard=bool(vh))
    for key in ("q_codes", "k_codes", "v_codes"):
        assert np.array_equal(got[key], pro[key]), key
    for key in ("s_q", "s_k", "s_v"):
        assert np.array_equal(got[key].view(np.uint32), pro[key].view(np.uint32)), key
    o = p.forward(qd, kd, vd, workspace=ws).cpu().numpy()
    want = ora.attention_full(pro, p_mode=p_mode, v_hadamard=bool(vh))
    err, cos = float(np.abs(o - want).max()), cosine(o, want)
    say("random %d: max|gpu-oracle| %.2e cos %.8f" % (seed, err, cos))
    assert err <= OUT_TOL and cos >= 0.999999
    _, dig = p.row_digests(ws)
    dig = dig.cpu().numpy().view(np.uint32)
    for b in range(w.batch):
        for h in range(w.heads):
            sl = {kk: vv[b:b + 1] for kk, vv in pro.items()}
            ds, dh, m = ora.code_digests(sl, 0, h, np.arange(w.tokens), p_mode=p_mode)
            assert np.array_equal(dig[b, h, :, 0], m.view(np.uint32)), (seed, b, h)
            assert np.array_equal(dig[b, h, :, 1], ds) and np.array_equal(dig[b, h, :, 2], dh), (seed, b, h)


@pytest.mark.parametrize("seed", range(8))
def test_random_configuration_bf16_path(ora, seed):
    """The bf16 fallback on the same random shapes, against fp64 attention of
    its own bf16-rounded RoPE'd Q/K and bf16 V (the bf16 path's bar)."""
    from oracle import ref_fp64
    from gpu_helpers import bf16_round
    w, _, _ = random_case(1000 + seed)
    say("random bf16 %d: B%d H%d D%d grid %s seg %s %s" % (seed, w.batch, w.heads, w.head_dim, w.grid, w.seg, w.dtype))
    q, k, v, _ = inputs.generate(w)
    o = plan_for(w, prec="bf16").forward(dev(q), dev(k), dev(v)).cpu().numpy()
    qf, kf, vf = ora.as_f32(q), ora.as_f32(k), ora.as_f32(v)
    qr = bf16_round(ref_fp64.rope3d(qf, w.grid, w.seg, w.theta).astype(np.float32))
    kr = bf16_round(ref_fp64.rope3d(kf, w.grid, w.seg, w.theta).astype(np.float32))
    ref = ref_fp64.attention(qr, kr, bf16_round(vf))
    err, cos = float(np.abs(o - ref).max()), cosine(o, ref)
    say("random bf16 %d: max %.2e cos %.8f" % (seed, err, cos))
    assert err <= 2e-2 and cos >= 0.9999
