"""Parity at the full workload sizes, in the launch configuration bench.py
times (same plan options, bf16 inputs, f32 output).

Every Q/K/V code and scale of the whole tensors is compared bit for bit with
the oracle's prologue; output rows are sampled (head 0 and the last head, the
first 64-row block, one interior block and the ragged tail block) and
compared with the oracle's binary64 float path (max-abs 2e-3, cosine 0.999).
"""
import numpy as np
import pytest
import torch

from bit_quantized_attention_rope3d_amd import inputs

from gpu_helpers import cosine, dev, plan_for, say

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)


@pytest.mark.parametrize("name", ["wan480", "wan720", "hy720"])
def test_fullsize(ora, name):
    w = inputs.get(name)
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
    tail0 = (N - 1) // 64 * 64
    rows = np.unique(np.concatenate([np.arange(0, 64), np.arange(N // 2 // 64 * 64, N // 2 // 64 * 64 + 64),
                                     np.arange(tail0, N)])).astype(np.int32)
    for h in (0, w.heads - 1):
        o = out[0, rows, h, :].float().cpu().numpy()
        want = ora.attention_rows(pro, 0, h, rows)
        err, cos = float(np.abs(o - want).max()), cosine(o, want)
        say("fullsize %s head %d: %d rows max|gpu-oracle| %.2e cos %.8f" % (name, h, rows.size, err, cos))
        assert err <= 2e-3 and cos >= 0.999
