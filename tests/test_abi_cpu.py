"""Host-side tests of the C ABI (no GPU needed): the library loads, exports
every declared entry point, validates its arguments before touching the
device, maps injected failures to the documented codes, builds RoPE tables
equal to the oracle's bit for bit, and implements the step/block schedule
(RotateAttention review, Sec. 5.1) with the printed INT4 fractions."""
import ctypes
import json
import os
import re

import numpy as np
import pytest

from bit_quantized_attention_rope3d_amd import native

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ra_attn.h")
GOLD = json.load(open(os.path.join(ROOT, "tests", "golden", "pages_facts.json")))


@pytest.fixture(scope="module")
def L():
    return native.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ra_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_function(L):
    names = declared_functions()
    assert len(names) >= 18
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(native._SIGS)


def test_status_strings(L):
    for i, name in enumerate(native.STATUS):
        assert native.status_str(i) == name


def test_opts_default(L):
    o = native.make_opts()
    assert (o.rot, o.prec, o.in_dtype, o.out_dtype) == (2, 0, 1, 0)
    assert o.rope_theta == 10000.0 and o.softmax_scale == 0.0 and o.p_mode == 0


def _create(shape, opts):
    h = ctypes.c_void_p()
    rc = native.lib().ra_plan_create(ctypes.byref(shape), ctypes.byref(opts), ctypes.byref(h))
    return rc, h


@pytest.mark.parametrize("kw,code", [
    (dict(head_dim=96, seg=(32, 32, 32)), "RA_ERR_UNSUPPORTED"),
    (dict(head_dim=64, seg=(22, 21, 21)), "RA_ERR_SEGMENTS"),
    (dict(head_dim=64, seg=(24, 20, 22)), "RA_ERR_SEGMENTS"),
    (dict(head_dim=64, seg=(0, 32, 32)), "RA_ERR_SEGMENTS"),
    (dict(grid=(0, 4, 4)), "RA_ERR_SHAPE"),
    (dict(heads=0), "RA_ERR_SHAPE"),
    (dict(batch=-1), "RA_ERR_SHAPE"),
])
def test_shape_validation(L, kw, code):
    a = dict(batch=1, heads=2, head_dim=64, grid=(2, 4, 4), seg=(24, 20, 20))
    a.update(kw)
    rc, h = _create(native.make_shape(a["batch"], a["heads"], a["head_dim"], a["grid"], a["seg"]),
                    native.make_opts())
    assert native.STATUS[rc] == code
    assert not h.value
    assert native.last_error()


@pytest.mark.parametrize("kw,code", [
    (dict(rot=4), "RA_ERR_INVALID_ARG"),
    (dict(v_hadamard=2), "RA_ERR_INVALID_ARG"),
    (dict(prec=2), "RA_ERR_INVALID_ARG"),
    (dict(in_dtype=5), "RA_ERR_DTYPE"),
    (dict(out_dtype=-1), "RA_ERR_DTYPE"),
    (dict(rope_theta=0.0), "RA_ERR_INVALID_ARG"),
    (dict(softmax_scale=-1.0), "RA_ERR_INVALID_ARG"),
    (dict(p_mode=2), "RA_ERR_INVALID_ARG"),
    (dict(p_mode=-1), "RA_ERR_INVALID_ARG"),
])
def test_opts_validation(L, kw, code):
    rc, h = _create(native.make_shape(1, 2, 64, (2, 4, 4), (24, 20, 20)), native.make_opts(**kw))
    assert native.STATUS[rc] == code


def test_workspace_sizes(L):
    from bit_quantized_attention_rope3d_amd.api import Plan
    p = Plan(1, 40, 128, (21, 45, 80), (44, 42, 42), rot="half")
    Npad = 1182 * 64
    codes = 40 * Npad * 128 * 3 // 4 * 3                      # Q, K, V: 6 bits per code
    assert p.workspace_bytes >= codes + 2 * 40 * 1182 * 4 + 2 * 40 * 128 * 4
    assert p.workspace_bytes < codes + 2 * 1024 * 1024
    b = Plan(1, 40, 128, (21, 45, 80), (44, 42, 42), prec="bf16")
    assert b.workspace_bytes >= 3 * 40 * Npad * 128 * 2
    p.close()
    b.close()


@pytest.mark.parametrize("rot,prec", [("interleaved", "int4"), ("half", "int4"), ("none", "int4"),
                                      ("interleaved", "bf16")])
def test_tables_bit_equal_to_oracle(L, ora, rot, prec):
    from bit_quantized_attention_rope3d_amd.api import Plan
    grid, seg = (21, 45, 80), (44, 42, 42)
    p = Plan(1, 2, 128, grid, seg, rot=rot, prec=prec)
    merged = 1 if (rot == "interleaved" and prec == "int4") else 0
    for s in range(3):
        cs, sn = p.tables(s)
        ocs, osn = ora.rope_table(grid[s], seg[s], 10000.0, merged)
        assert np.array_equal(cs.view(np.uint32), ocs.view(np.uint32))
        assert np.array_equal(sn.view(np.uint32), osn.view(np.uint32))
    p.close()


def test_calls_reject_bad_buffers_before_device_work(L):
    from bit_quantized_attention_rope3d_amd.api import Plan
    p = Plan(1, 2, 64, (2, 4, 4), (24, 20, 20))
    fwd = native.lib().ra_attn_fwd
    a16 = ctypes.c_void_p(0x10000)
    ok_ws = p.workspace_bytes
    assert native.STATUS[fwd(p._h, None, a16, a16, a16, a16, ok_ws, None)] == "RA_ERR_INVALID_ARG"
    assert native.STATUS[fwd(p._h, ctypes.c_void_p(0x10004), a16, a16, a16, a16, ok_ws, None)] == "RA_ERR_ALIGNMENT"
    assert native.STATUS[fwd(p._h, a16, a16, a16, a16, a16, ok_ws - 1, None)] == "RA_ERR_WORKSPACE"
    assert native.STATUS[fwd(p._h, a16, a16, a16, a16, None, ok_ws, None)] == "RA_ERR_WORKSPACE"
    assert native.STATUS[fwd(None, a16, a16, a16, a16, a16, ok_ws, None)] == "RA_ERR_INVALID_ARG"
    p.close()


@pytest.mark.parametrize("what,code", [("alloc", "RA_ERR_OOM"), ("launch", "RA_ERR_HIP")])
def test_fault_injection(L, monkeypatch, what, code):
    """The table upload (ra_plan_upload; ra_plan_create on a GPU) maps an
    allocation failure to RA_ERR_OOM, the forward a launch failure to
    RA_ERR_HIP."""
    from bit_quantized_attention_rope3d_amd.api import Plan
    p = Plan(1, 2, 64, (2, 4, 4), (24, 20, 20))
    a16 = ctypes.c_void_p(0x10000)
    monkeypatch.setenv("RA_FAULT_INJECT", what)
    if what == "alloc":
        rc = native.lib().ra_plan_upload(p._h)
    else:
        rc = native.lib().ra_attn_fwd(p._h, a16, a16, a16, a16, a16, p.workspace_bytes, None)
    assert native.STATUS[rc] == code
    assert what in native.last_error()
    p.close()


def test_schedule_matches_printed_fractions(L):
    from bit_quantized_attention_rope3d_amd.api import schedule_pick
    for case in GOLD["schedule"]["cases"]:
        sched = (case["steps_head"], case["steps_tail"], case["blocks_head"], case["blocks_tail"])
        n = sum(schedule_pick(sched, s, 40, b, 40) == "int4" for s in range(40) for b in range(40))
        assert round(n / 1600, 2) == case["int4_fraction_printed"]
    n10 = sum(schedule_pick((2, 2, 4, 4), s, 10, b, 40) == "int4" for s in range(10) for b in range(40))
    assert n10 == 192          # 0.48 of 400 calls
    assert schedule_pick((2, 2, 4, 4), 0, 10, 20, 40) == "bf16"
    assert schedule_pick((2, 2, 4, 4), 5, 10, 3, 40) == "bf16"
    assert schedule_pick((2, 2, 4, 4), 5, 10, 20, 40) == "int4"


def test_schedule_agrees_with_oracle(L, ora):
    from bit_quantized_attention_rope3d_amd.api import schedule_pick
    for sched in ((6, 4, 2, 2), (2, 2, 2, 2), (2, 2, 4, 4), (0, 0, 0, 0), (1, 3, 0, 5)):
        for s in range(12):
            for b in range(9):
                assert (schedule_pick(sched, s, 12, b, 9) == "bf16") == \
                    ora.schedule_full_precision(sched, s, 12, b, 9)


@pytest.mark.parametrize("p_mode", [0, 1])
def test_pmap_thresholds_agree_with_oracle(L, ora, p_mode):
    """The library finds the P map's thresholds its own way (bisection over
    binary32 bit patterns); they equal the oracle's (pinned against 40-digit
    decimal in test_oracle_pmap.py) bit for bit."""
    from bit_quantized_attention_rope3d_amd.api import pmap_thresholds
    got = pmap_thresholds(p_mode)
    want = ora.pmap_thresholds(p_mode)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    assert native.STATUS[L.ra_pmap_thresholds(2, ctypes.c_void_p(0x10000))] == "RA_ERR_INVALID_ARG"
    assert native.STATUS[L.ra_pmap_thresholds(0, None)] == "RA_ERR_INVALID_ARG"


def test_python_wrappers_reject_bad_tensors(L):
    """The binding checks every buffer it hands to a kernel: inputs, output
    and workspace (shape, dtype, contiguity, device), and the one-shot form
    checks k and v against q, before any call into the library."""
    import torch
    from bit_quantized_attention_rope3d_amd.api import Plan, attn_fwd
    p = Plan(1, 2, 64, (2, 4, 4), (24, 20, 20), in_dtype="f32", out_dtype="f32")
    q = torch.zeros(p.io_shape, dtype=torch.float32)
    with pytest.raises(ValueError, match="input must be"):
        p.forward(q, q, q)                                          # not on a GPU
    with pytest.raises(ValueError, match="out must be"):
        p._check_out(torch.zeros(p.io_shape, dtype=torch.bfloat16), q.device)
    with pytest.raises(ValueError, match="out must be"):
        p._check_out(torch.zeros((1, 31, 2, 64), dtype=torch.float32), q.device)
    with pytest.raises(ValueError, match="out must be"):
        p._check_out(torch.zeros((1, 2, 32, 64), dtype=torch.float32).transpose(1, 2), q.device)
    with pytest.raises(ValueError, match="workspace must be"):
        p._ws(torch.zeros(p.workspace_bytes, dtype=torch.int8), q.device)
    with pytest.raises(ValueError, match="k must be"):
        attn_fwd(q, q[:, :31], q, (2, 4, 4), (24, 20, 20))
    with pytest.raises(ValueError, match="v must be"):
        attn_fwd(q, q, q.to(torch.bfloat16), (2, 4, 4), (24, 20, 20))
    with pytest.raises(ValueError, match="must be bfloat16 or float32"):
        attn_fwd(q.double(), q, q, (2, 4, 4), (24, 20, 20))
    p.close()


def test_mfma_peak_probe_validates_before_launch(L):
    a = ctypes.c_void_p(0x10000)
    ops = ctypes.c_double()
    probe = L.ra_bench_mfma_peak
    assert native.STATUS[probe(99, 10, 10, a, a, ctypes.byref(ops), None)] == "RA_ERR_INVALID_ARG"
    assert native.STATUS[probe(0, 0, 10, a, a, ctypes.byref(ops), None)] == "RA_ERR_INVALID_ARG"
    assert native.STATUS[probe(0, 10, 0, a, a, ctypes.byref(ops), None)] == "RA_ERR_INVALID_ARG"
    assert native.STATUS[probe(0, 10, 10, None, a, ctypes.byref(ops), None)] == "RA_ERR_INVALID_ARG"
