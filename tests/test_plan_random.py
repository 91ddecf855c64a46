"""Randomised planner cases on the CPU: seeded draws of (schedule, ranks,
group, size, dtype, exec mode, assumed cache size) whose launch lists, run
by the numpy interpreter, must equal the oracle bit for bit.  The small
cache sizes force the group-by-group and piece-by-piece launch orders, so
they are exercised together with every dtype, fusion and one-pass fold."""
import numpy as np
import pytest

import oracle
from gradient_all_reduce_ar_amd import _binding as B
from gradient_all_reduce_ar_amd import workloads
from tests import plan_interp

SCHEDS = ["ring", "hierarchical", "rabenseifner", "recursive_doubling", "tree", "double_tree"]
POW2 = {"rabenseifner", "recursive_doubling", "double_tree"}


def _draw(rng):
    sched = SCHEDS[rng.integers(len(SCHEDS))]
    if sched in POW2:
        n = int(2 ** rng.integers(0, 5))
        g = 1
    else:
        n = int(rng.integers(1, 13))
        divisors = [d for d in range(1, n + 1) if n % d == 0]
        g = int(divisors[rng.integers(len(divisors))]) if sched == "hierarchical" else 1
    dtype = ["fp32", "bf16", "bf16_each", "int8_ef"][rng.integers(4)]
    mode = ["steps", "steps_unfused", "onepass"][rng.integers(3)]
    if dtype == "int8_ef":
        count = int(rng.integers(0, 40)) * 128 + int(rng.integers(0, 128))
    else:
        count = int(rng.integers(0, 3000))
    cache = [None, 64, 512, 4096][rng.integers(4)]
    return sched, n, g, dtype, mode, count, cache


@pytest.mark.parametrize("case", range(400))
def test_random_plan_matches_oracle(case):
    rng = np.random.default_rng([2026, case])
    sched, n, g, dtype, mode, count, cache = _draw(rng)
    what = f"{sched} n={n} g={g} {dtype} {mode} count={count} cache={cache}"
    p = B.ar_plan_create(n, g, count, dtype, sched)
    try:
        B.ar_plan_set_exec(p, mode)
        if cache is not None:
            B.ar_plan_set_cache_bytes(p, cache)
        if dtype == "int8_ef":
            xs = [(rng.standard_normal(count) * np.exp(rng.standard_normal(count))).astype(np.float32)
                  for _ in range(n)]
            es = [(rng.standard_normal(count) * 1e-2).astype(np.float32) for _ in range(n)]
            ref_b, ref_e = [x.copy() for x in xs], [e.copy() for e in es]
            oracle.run_int8ef(ref_b, sched, errs=ref_e, group_size=g)
            got_b, got_e = [x.copy() for x in xs], [e.copy() for e in es]
            plan_interp.run_int8(p, got_b, got_e, g)
            for r in range(n):
                np.testing.assert_array_equal(got_b[r].view(np.uint32), ref_b[r].view(np.uint32), err_msg=what)
                np.testing.assert_array_equal(got_e[r].view(np.uint32), ref_e[r].view(np.uint32), err_msg=what)
        else:
            gen = "fp32" if dtype == "fp32" else "bf16"
            xs = workloads.normal_inputs(n, count, seed=case, sigma=1.0, dtype=gen)
            ref = oracle.run([x.copy() for x in xs], dtype, sched, group_size=g)
            got = plan_interp.run(p, [x.copy() for x in xs], dtype, g)
            bv = np.uint32 if dtype == "fp32" else np.uint16
            for r in range(n):
                np.testing.assert_array_equal(got[r].view(bv), ref[r].view(bv), err_msg=what)
    finally:
        B.ar_plan_destroy(p)
