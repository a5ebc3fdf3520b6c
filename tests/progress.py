"""Progress lines of long GPU tests, written past pytest's output capture.

pytest holds a test's output until the test ends; a long test (the full-size
schedule sweep runs for minutes) would then look silent to whatever watches
the run.  conftest.py stores pytest's capture manager here, and say() prints
with capturing suspended, so each line reaches the terminal at once."""
from __future__ import annotations

import sys

CAPMAN = None


def say(*a):
    if CAPMAN is not None:
        with CAPMAN.global_and_fixture_disabled():
            print(*a, flush=True)
    else:
        print(*a, flush=True)
        sys.stdout.flush()
