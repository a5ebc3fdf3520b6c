"""CPU oracle for the RotateAttention INT4 attention forward.

TEST INFRASTRUCTURE ONLY: the test suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` are the only callers.  The product path
(the HIP library and its Python binding) never imports this package.

Contents
  ra_oracle.c   plain C implementation of the method, step by step (exact
                integers, binary32 where a float decides an integer, binary64
                for the final normalisation)
  oracle.py     ctypes wrapper (build + calls)
  ref_fp64.py   textbook full-precision attention with 3D RoPE (numpy fp64),
                used for error reporting and for invariants of the rotations

Parity status: every function is pinned by tests in ``tests/test_oracle_*.py``
against facts fixed by the pages or by mathematics; the one quantity with no
pin is video-level quality, which needs models and prompts that are absent.
"""
from .oracle import *  # noqa: F401,F403
