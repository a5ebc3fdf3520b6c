"""ra_attn_fwd_noalloc: the forward pass with the library's fixed
device-resident workspace, for callers that cannot allocate.  Checked
through the C ABI against ra_attn_fwd (its outputs must be bit-identical:
same kernels, same inputs) on two calls in a row, the second with a smaller
input, and for a plan too large for the fixed workspace, the documented
rejection before any device work.  The device's free memory is unchanged
across the calls."""
import ctypes

import numpy as np
import pytest
import torch

from bit_quantized_attention_rope3d_amd import inputs, native
from bit_quantized_attention_rope3d_amd.api import Plan

from gpu_helpers import dev, plan_for, say

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)


def _run(w, prec="int4"):
    q, k, v, _ = inputs.generate(w)
    qd, kd, vd = dev(q), dev(k), dev(v)
    p = plan_for(w, prec=prec)
    assert p.workspace_bytes <= (64 << 20)
    want = p.forward(qd, kd, vd).cpu().numpy()
    out = p.empty_out()
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    got = p.forward_noalloc(qd, kd, vd, out=out)
    torch.cuda.synchronize()
    free1 = torch.cuda.mem_get_info()[0]
    assert free1 == free0, (free0, free1)
    assert np.array_equal(got.cpu().numpy().view(np.uint32), want.view(np.uint32)), w.name
    p.close()


@pytest.mark.parametrize("prec", ["int4", "bf16"])
def test_noalloc_matches_fwd_on_two_calls(prec):
    big = inputs.small("noalloc_big", heads=3, head_dim=128, grid=(3, 17, 23), rot="half", seed=51)
    small = inputs.small("noalloc_small", heads=2, head_dim=64, grid=(2, 5, 7), rot="interleaved",
                         seed=52, dtype="f32")
    _run(big, prec)        # 1173 tokens x 3 heads
    _run(small, prec)      # then 70 tokens x 2 heads, D64: the array keeps the first call's data
    say("noalloc %s: two calls bit-identical to ra_attn_fwd, free memory unchanged" % prec)


def test_noalloc_rejects_plans_beyond_the_fixed_workspace():
    w = inputs.get("wan480")
    p = Plan(w.batch, w.heads, w.head_dim, w.grid, w.seg, rot=w.rot)
    assert p.workspace_bytes > (64 << 20)
    a16 = ctypes.c_void_p(0x10000)
    rc = native.lib().ra_attn_fwd_noalloc(p._h, a16, a16, a16, a16, None)
    assert native.STATUS[rc] == "RA_ERR_WORKSPACE"
    assert "at most" in native.last_error()
    p.close()
