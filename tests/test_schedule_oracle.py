"""Pin of the mixed-precision schedule reading against the fractions printed
on the RotateAttention review (Sec. 5.1 as quoted in its circularity check):
68% INT4 for FP16 on the first 6 / last 4 steps and first/last 2 blocks, and
81% for first/last 2 steps and blocks."""
import json
import os

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_facts.json")))


def int4_fraction(fp, sched, n_steps, n_blocks):
    n = sum(not fp(sched, s, n_steps, b, n_blocks) for s in range(n_steps) for b in range(n_blocks))
    return n / (n_steps * n_blocks)


def test_printed_fractions(ora):
    for case in GOLD["schedule"]["cases"]:
        sched = (case["steps_head"], case["steps_tail"], case["blocks_head"], case["blocks_tail"])
        f = int4_fraction(ora.schedule_full_precision, sched, 40, 40)
        assert round(f, 2) == case["int4_fraction_printed"], (case, f)


def test_sweep_fractions(ora):
    # 40 blocks x 10 steps with first/last 2 steps and first/last 4 blocks
    assert int4_fraction(ora.schedule_full_precision, (2, 2, 4, 4), 10, 40) == 0.48
    assert int4_fraction(ora.schedule_full_precision, (2, 2, 4, 4), 40, 40) == 0.72
