"""Parity at the full workload sizes, in the launch configuration bench.py
times (same plan options, bf16 inputs, f32 output).

Every Q/K/V code and scale of the whole tensors is compared bit for bit with
the oracle's prologue.  Output rows are sampled (head 0 and the last head, the
first 64-row block, one interior block and the ragged tail block) and
compared with the oracle's binary64 float path (max-abs 1e-5).  For the same
rows, the benchmarked kernel's parity variant gives the final running max and
fingerprints of every P code over all N keys, compared bit for bit; and the
step-by-step tile dump gives S, P codes, PV and the running max of the first,
a middle and the ragged last key step of those query blocks.
"""
import numpy as np
import pytest
import torch

from bit_quantized_attention_rope3d_amd import inputs

from gpu_helpers import OUT_TOL, cosine, dev, plan_for, say

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)


# A sequence longer than the attention kernel keeps K scales in LDS for
# (5120 key steps): 2 x 165 x 1000 = 330,000 tokens, one head of D = 64, so
# the kernel instantiation that reads them from global memory is checked too.
LONG = inputs.small("long330k", heads=1, head_dim=64, grid=(2, 165, 1000), rot="half", seed=21)


@pytest.mark.parametrize("name", ["wan480", "wan720", "hy720", "long330k"])
def test_fullsize(ora, name):
    w = LONG if name == "long330k" else inputs.get(name)
    say("fullsize %s: generating %d tokens x %d heads" % (name, w.tokens, w.heads))
    q, k, v, _ = inputs.generate(w)
    p = plan_for(w)
    qd, kd, vd = dev(q), dev(k), dev(v)
    ws = p.workspace()
    say("fullsize %s: GPU prologue + debug copy" % name)
    got = p.debug_prologue(qd, kd, vd, ws)
    say("fullsize %s: oracle prologue" % name)
    pro = ora.prologue(q, k, v, w.grid, w.seg, w.theta, w.rot_id)
    del q, k, v
    for key in ("q_codes", "k_codes", "v_codes"):
        nbad = int(np.count_nonzero(got[key] != pro[key]))
        assert nbad == 0, (name, key, nbad)
    for key in ("s_q", "s_k", "s_v"):
        assert np.array_equal(got[key].view(np.uint32), pro[key].view(np.uint32)), (name, key)
    del got
    say("fullsize %s: prologue bit-exact; running forward" % name)
    out = p.forward(qd, kd, vd, workspace=ws)
    N = w.tokens
    nb = (N + 63) // 64
    tail0 = (N - 1) // 64 * 64
    mid = N // 2 // 64 * 64
    rows = np.unique(np.concatenate([np.arange(0, 64), np.arange(mid, mid + 64),
                                     np.arange(tail0, N)])).astype(np.int32)
    o_all = out[0, rows].float().cpu().numpy()
    del out
    say("fullsize %s: parity variant of the attention kernel" % name)
    o_dbg, dig = p.row_digests(ws)
    dig = dig[0].index_select(1, torch.from_numpy(rows.astype(np.int64)).cuda()).cpu().numpy().view(np.uint32)
    assert np.array_equal(o_dbg[0, rows].float().cpu().numpy().view(np.uint32), o_all.view(np.uint32))
    del o_dbg
    for h in sorted({0, w.heads - 1}):
        o = o_all[:, h, :]
        want = ora.attention_rows(pro, 0, h, rows)
        err, cos = float(np.abs(o - want).max()), cosine(o, want)
        say("fullsize %s head %d: %d rows max|gpu-oracle| %.2e cos %.8f" % (name, h, rows.size, err, cos))
        assert err <= OUT_TOL and cos >= 0.999999
        ds, dh, m = ora.code_digests(pro, 0, h, rows)
        assert np.array_equal(dig[h, :, 0], m.view(np.uint32)), (name, h, "running max")
        assert np.array_equal(dig[h, :, 1], ds), (name, h, "sum of u")
        assert np.array_equal(dig[h, :, 2], dh), (name, h, "hash of u")
        say("fullsize %s head %d: running max and P-code fingerprints over all %d keys bit-exact"
            % (name, h, N))
    for h in sorted({0, w.heads - 1}):
        for qb in (0, mid // 64, nb - 1):
            for kb in (0, nb // 2, nb - 1):
                g = p.debug_tile(ws, 0, h, qb, kb)
                t = ora.attention_tile(pro, 0, h, qb, kb)
                n = t["s_int"].shape[0]
                nk = min(64, N - kb * 64)
                assert np.array_equal(g["s_int"][:n, :nk], t["s_int"][:, :nk]), (name, h, qb, kb, "S")
                assert np.array_equal(g["p_code"][:n], t["p_code"]), (name, h, qb, kb, "P")
                assert np.array_equal(g["pv_int"][:n], t["pv_int"]), (name, h, qb, kb, "PV")
                assert np.array_equal(g["m_after"][:n].view(np.uint32), t["m_after"].view(np.uint32))
    say("fullsize %s: %d tile dumps (first, middle, ragged last key step) bit-exact"
        % (name, 9 * len({0, w.heads - 1})))
