"""Build libra_attn.so (HIP for gfx950) in-tree with hipcc.

Usage: python -m bit_quantized_attention_rope3d_amd.build
Every HIP source is compiled with -ffp-contract=off (the kernels request each
fused multiply-add explicitly) and with packed-FP32 instruction selection
disabled.  The INT4 attention kernels are also compiled without NaN semantics:
no value they compare or take the maximum of is NaN (scores are finite MFMA
sums or -inf, running maxima finite or -inf), and with them the compiler
would wrap every fmaxf in NaN-quieting copies of its operands.  The one NaN
the P map can form (0 * inf for a masked key of a zero-scale block) goes
through the FMA's clamp bit, which the hardware maps to 0.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libra_attn.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["ra_host.cpp", "ra_prologue.hip", "ra_int4_attn.hip", "ra_bf16_attn.hip", "ra_peak.hip",
           "ra_noalloc.hip"]
EXTRA = {"ra_int4_attn.hip": ["-fno-honor-nans"]}

CFLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
    "-I" + INCLUDE, "-I" + CSRC,
]


def _compile(src: str, extra=()) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *CFLAGS, *EXTRA.get(src, ()), *extra, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    return obj


def build(verbose: bool = False, save_temps: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    extra = ["-save-temps=obj"] if save_temps else []
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra), SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True, save_temps="--save-temps" in sys.argv)
