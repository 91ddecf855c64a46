"""The library from C alone: tests/c/abi_use.c allocates its 16 rank buffers
with hipMalloc and runs a ring all-reduce, then a one-pass reduce-scatter and
all-gather, through include/ar.h (no Python, no torch), checking every
element on the host against exact sums.  The program is built by
__graft_entry__.build() (tests/c/build.py)."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

BIN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c", "abi_use")


def test_c_program_uses_the_abi():
    if not os.path.exists(BIN):
        pytest.skip("tests/c/abi_use is not built (tests/c/build.py, run by __graft_entry__.build())")
    print("case C ABI program: 16-rank ring all-reduce, reduce-scatter, all-gather", flush=True)
    r = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
