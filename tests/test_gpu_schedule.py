"""The mixed-precision step x block schedule, run end to end on the GPU.

Each call of a denoise-step x transformer-block sweep draws fresh seeded
tensors on the device, asks ra_schedule_pick for its precision (bf16 when the
step or the block is in a head/tail set: RotateAttention review, Sec. 5.1, the
FP16 fallback schedule) and runs that plan.  INT4 calls are compared with the
oracle's binary64 float path (max-abs 1e-5), bf16 calls with
fp64 attention on the bf16-rounded RoPE'd inputs (the bf16 path's own bar);
every call's error against exact fp64 attention of the unrounded inputs is
printed, not gated.  The aggregate attention time over the sweep is printed.

Both sweeps run by default: a small one that checks every head and row, and
the full one -- the Wan-like 720p shape (B1, H40, D128, 21x45x80 = 75,600
tokens, Half rotation) over 10 steps x 40 blocks with 2/2 head/tail steps and
4/4 head/tail blocks -- which samples one head x 64 query rows per call (about
five minutes, mostly the CPU checks; progress is printed per step).
"""
import json
import os
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

from bit_quantized_attention_rope3d_amd import inputs
from oracle import ref_fp64

from gpu_helpers import OUT_TOL, bf16_round, cosine, plan_for, say

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)


def _host(x: torch.Tensor) -> np.ndarray:
    """Device tensor -> numpy float32 or bf16 bit patterns (uint16)."""
    if x.dtype == torch.bfloat16:
        return x.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return x.float().cpu().numpy()


def _check_call(ora, w, prec, qh, kh, vh, rows, o):
    """Errors of output rows `o` [rows, D] of one head; qh, kh, vh are that
    head's inputs [1, N, 1, D] as they went to the GPU."""
    qf, kf, vf = ora.as_f32(qh), ora.as_f32(kh), ora.as_f32(vh)
    qr = ref_fp64.rope3d(qf, w.grid, w.seg, w.theta)[0, :, 0]
    kr = ref_fp64.rope3d(kf, w.grid, w.seg, w.theta)[0, :, 0]
    exact = ref_fp64.attention_rows(qr, kr, vf[0, :, 0], rows)
    rec = dict(max_vs_fp64=float(np.abs(o - exact).max()), cos_vs_fp64=cosine(o, exact))
    if prec == "int4":
        pro = ora.prologue(qh, kh, vh, w.grid, w.seg, w.theta, w.rot_id)
        want = ora.attention_rows(pro, 0, 0, rows)
        rec.update(gate="oracle", max=float(np.abs(o - want).max()), cos=cosine(o, want))
        rec["ok"] = rec["max"] <= OUT_TOL and rec["cos"] >= 0.999999
    else:
        qb = bf16_round(qr.astype(np.float32)).astype(np.float64)
        kb = bf16_round(kr.astype(np.float32)).astype(np.float64)
        want = ref_fp64.attention_rows(qb, kb, bf16_round(vf[0, :, 0]), rows)
        rec.update(gate="fp64 on bf16 inputs", max=float(np.abs(o - want).max()), cos=cosine(o, want))
        rec["ok"] = rec["max"] <= 2e-2 and rec["cos"] >= 0.9999
    return rec


def run_sweep(ora, w, n_steps, n_blocks, sched, rows_per_call=None, all_heads=True, workers=4):
    from bit_quantized_attention_rope3d_amd.api import schedule_pick
    plans = {p: plan_for(w, prec=p) for p in ("int4", "bf16")}
    wss = {p: plans[p].workspace() for p in plans}
    outs = {p: plans[p].empty_out() for p in plans}
    stream = torch.cuda.current_stream()
    N, H = w.tokens, w.heads
    records, futures = [], []
    pool = ThreadPoolExecutor(max_workers=workers)
    t_wall = time.perf_counter()
    for step in range(n_steps):
        for block in range(n_blocks):
            prec = schedule_pick(sched, step, n_steps, block, n_blocks)
            want_bf16 = ora.schedule_full_precision(sched, step, n_steps, block, n_blocks)
            assert prec == ("bf16" if want_bf16 else "int4"), (step, block)
            seed = inputs.schedule_seed(step, block, n_blocks)
            q, k, v = inputs.generate_device(w, seed)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            out = plans[prec].forward(q, k, v, out=outs[prec], workspace=wss[prec])
            e1.record(stream)
            heads = range(H) if all_heads else [(step * n_blocks + block) % H]
            rng = np.random.default_rng(seed)
            rows = (np.arange(N) if rows_per_call is None
                    else np.sort(rng.choice(N, size=min(rows_per_call, N), replace=False)))
            rows = rows.astype(np.int32)
            rows_t = torch.from_numpy(rows.astype(np.int64)).to(out.device)
            for h in heads:
                o = out[0].index_select(0, rows_t)[:, h, :].float().cpu().numpy().astype(np.float64)
                sl = slice(h, h + 1)
                qh, kh, vh = _host(q[:, :, sl]), _host(k[:, :, sl]), _host(v[:, :, sl])
                futures.append((step, block, h, prec,
                                pool.submit(_check_call, ora, w, prec, qh, kh, vh, rows, o)))
            torch.cuda.synchronize()
            records.append(dict(step=step, block=block, prec=prec, ms=e0.elapsed_time(e1)))
            del q, k, v
        done = sum(f.done() for *_, f in futures)
        say("sweep %s: step %d of %d launched (%d calls, %d of %d checks done)"
            % (w.name, step + 1, n_steps, len(records), done, len(futures)))
    wall = time.perf_counter() - t_wall
    errs = []
    for i, (step, block, h, prec, f) in enumerate(futures):
        r = f.result()
        r.update(step=step, block=block, head=h, prec=prec)
        errs.append(r)
        say("call step %d block %2d head %2d %-4s: vs %s max %.2e cos %.7f | vs exact fp64 max %.2e cos %.6f"
            % (step, block, h, prec, r["gate"], r["max"], r["cos"], r["max_vs_fp64"], r["cos_vs_fp64"]))
    pool.shutdown()
    n4 = sum(r["prec"] == "int4" for r in records)
    ms = {p: [r["ms"] for r in records if r["prec"] == p] for p in ("int4", "bf16")}
    summary = dict(
        workload=w.name, tokens=N, heads=H, steps=n_steps, blocks=n_blocks, schedule=list(sched),
        calls=len(records), int4_calls=n4, int4_fraction=n4 / len(records),
        aggregate_ms=float(sum(r["ms"] for r in records)),
        mean_ms={p: (float(np.mean(v)) if v else None) for p, v in ms.items()},
        all_bf16_ms_estimate=(float(np.mean(ms["bf16"])) * len(records) if ms["bf16"] else None),
        worst={p: dict(max=max((e["max"] for e in errs if e["prec"] == p), default=None),
                       cos=min((e["cos"] for e in errs if e["prec"] == p), default=None),
                       max_vs_fp64=max((e["max_vs_fp64"] for e in errs if e["prec"] == p), default=None),
                       cos_vs_fp64=min((e["cos_vs_fp64"] for e in errs if e["prec"] == p), default=None))
               for p in ("int4", "bf16")},
        wall_s=wall)
    say("sweep summary " + json.dumps(summary))
    bad = [e for e in errs if not e["ok"]]
    assert not bad, bad[:4]
    return summary


def test_schedule_sweep_small(ora):
    """4 steps x 6 blocks, 1/1 head/tail steps and blocks: 8 INT4 calls of 24,
    every head and row checked."""
    w = inputs.small(name="sweep_small")
    s = run_sweep(ora, w, 4, 6, (1, 1, 1, 1))
    assert s["int4_calls"] == 8 and s["calls"] == 24


@pytest.mark.timeout(1200)
def test_schedule_sweep_wan720(ora):
    w = inputs.get("wan720")
    threads = ora.get_threads()
    ora.set_threads(2)      # eight checking threads share the host cores
    try:
        s = run_sweep(ora, w, 10, 40, (2, 2, 4, 4), rows_per_call=64, all_heads=False, workers=8)
    finally:
        ora.set_threads(threads)
    assert s["calls"] == 400 and s["int4_calls"] == 192
