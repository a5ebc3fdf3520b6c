"""The oracle's pins catch plausible slips: each case below plants one mistake
in a copy of oracle/ra_oracle.c (on the CPU), builds it, points the oracle
test files at that copy (ORA_LIB_PATH) and requires them to fail.

The planted mistakes are the ones an implementation of the definition could
plausibly make: the K scale of the wrong block, the running max started at 0
instead of -inf, the exponent rounded twice instead of once, a strict instead
of an inclusive threshold compare, thresholds one binary32 step off, the
rescale factor inverted, the row sum taken over codes instead of code + 8,
Q/K codes rounded half away from zero, the INT4 scale off by one level, and a
sign slip in the RoPE pair rotation.
"""
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "ra_oracle.c")

MUTATIONS = {
    "k_scale_of_query_block": ("float sqk = sq[qb] * sk[kb];", "float sqk = sq[qb] * sk[qb];"),
    "running_max_starts_at_zero": ("float m = -INFINITY;\n        double A[ORA_MAX_D]",
                                   "float m = 0.0f;\n        double A[ORA_MAX_D]"),
    "exponent_rounded_twice": ("dv[j] = fmaf((float)S[j], c, -mnew);",
                               "dv[j] = (float)S[j] * c - mnew;"),
    "strict_threshold_compare": ("if (d >= T[k]) ++u;", "if (d > T[k]) ++u;"),
    "thresholds_one_step_high": ("T[k] = d;", "T[k] = nextafterf(d, INFINITY);"),
    "rescale_inverted": ("double beta = exp2((double)m - (double)mnew);",
                         "double beta = exp2((double)mnew - (double)m);"),
    "row_sum_of_codes": ("U += u[j];", "U += u[j] - zp;"),
    "qk_round_half_away": ("float q = rintf(t);", "float q = roundf(t);"),
    "scale_off_by_one_level": ("*inv = 7.0f / amax;", "*inv = 8.0f / amax;"),
    "rope_sign_slip": ("tmp[off + 2 * j] = ac - bs;", "tmp[off + 2 * j] = ac + bs;"),
}

TEST_FILES = ["tests/test_oracle_brute.py", "tests/test_oracle_pmap.py", "tests/test_oracle_attention.py",
              "tests/test_oracle_quant.py", "tests/test_oracle_rope.py"]


def _run_mutant(name, tmp):
    old, new = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, (name, src.count(old))
    c = os.path.join(tmp, name + ".c")
    so = os.path.join(tmp, name + ".so")
    with open(c, "w") as f:
        f.write(src.replace(old, new))
    subprocess.run(["gcc", "-O2", "-std=gnu11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
                    "-fPIC", "-shared", c, "-o", so, "-lm"], check=True)
    env = dict(os.environ, ORA_LIB_PATH=so, OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "-k", "not every_f32", *TEST_FILES],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return r.returncode, r.stdout[-2000:]


def test_unmutated_copy_passes():
    """The same harness on an unchanged copy passes (so a failure below is the
    planted mistake's doing)."""
    with tempfile.TemporaryDirectory() as tmp:
        MUTATIONS["_none"] = ("int ora_block(void)", "int ora_block(void)")
        try:
            rc, out = _run_mutant("_none", tmp)
        finally:
            del MUTATIONS["_none"]
    assert rc == 0, out


def test_every_planted_mistake_fails_a_pin():
    names = sorted(MUTATIONS)
    with tempfile.TemporaryDirectory() as tmp, ThreadPoolExecutor(max_workers=4) as ex:
        results = dict(zip(names, ex.map(lambda n: _run_mutant(n, tmp), names)))
    survived = {n: out for n, (rc, out) in results.items() if rc == 0}
    assert not survived, survived
