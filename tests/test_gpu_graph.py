"""The forward entry points allocate nothing and never synchronise, so the
very first ra_attn_fwd of a fresh plan can be captured into a HIP graph
(here through torch.cuda.CUDAGraph, which is a hipGraph on ROCm).  The
captured graph is replayed several times, with other eager work and host
synchronisations in between, and every replay's output must equal an eager
call's bit for bit; the captured calls record kernels only (the library
clears its per-channel V maxima with a kernel, not a memset).
"""
import numpy as np
import pytest
import torch

from bit_quantized_attention_rope3d_amd import inputs

from gpu_helpers import dev, plan_for, say

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)


@pytest.mark.parametrize("prec", ["int4", "bf16"])
def test_first_forward_captures_into_a_graph(prec):
    w = inputs.small("graph", heads=2, head_dim=128, grid=(3, 7, 9), rot="half", seed=41)
    q, k, v, _ = inputs.generate(w)
    qd, kd, vd = dev(q), dev(k), dev(v)
    p = plan_for(w, prec=prec)                    # tables go to the device here
    ws = p.workspace()
    out = p.empty_out()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            p.forward(qd, kd, vd, out=out, workspace=ws)   # the plan's first forward
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    ref = plan_for(w, prec=prec).forward(qd, kd, vd).cpu().numpy()
    for i in range(4):
        out.fill_(float("nan"))
        ws.fill_(0xA5)
        junk = (torch.randn(1 << 20, device="cuda") * 2.0).sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), (prec, i)
        del junk
    say("graph %s: first forward captured, 4 replays bit-identical to an eager call" % prec)
