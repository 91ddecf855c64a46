"""The CPU oracle against brute force and against the exact sum.

* Brute force: the oracle's step-by-step simulation must equal the closed-form
  fold of each schedule (tests/folds.py), computed element by element in pure
  Python, for N <= 4 (and 8 for the tree) and tiny buffers including sizes that
  do not divide into N parts.
* Exact sum: integer-valued inputs whose partial sums are exactly
  representable give exactly the integer sum on every rank (the plain
  definition of all-reduce: every rank ends with G_0 + ... + G_{N-1}).
* fp64 bound: fp32 results lie within 1e-5 * sum_r |x_r| of the fp64 sum.
"""
import numpy as np
import pytest

import oracle
from gradient_all_reduce_ar_amd import workloads
from tests import folds

CASES = [("ring", n, 1) for n in (1, 2, 3, 4)] + \
        [("hierarchical", n, g) for n, g in ((2, 1), (2, 2), (4, 2), (4, 1), (4, 4), (6, 3), (6, 2))] + \
        [("rabenseifner", n, 1) for n in (1, 2, 4, 8)]


@pytest.mark.parametrize("schedule,n,g", CASES)
def test_fp32_matches_closed_form(schedule, n, g):
    for count in list(range(0, 12)) + [17, 33]:
        xs = workloads.uniform_inputs(n, count, seed=count)
        want = folds.expected_fp32(xs, schedule, g)
        bufs = [x.copy() for x in xs]
        oracle.run(bufs, "fp32", schedule, group_size=g)
        for r in range(n):
            np.testing.assert_array_equal(bufs[r].view(np.uint32), want.view(np.uint32),
                                          err_msg=f"{schedule} n={n} g={g} count={count} rank={r}")


@pytest.mark.parametrize("schedule,n,g", CASES)
def test_bf16_matches_closed_form(schedule, n, g):
    for count in (0, 1, 5, 9, 16, 33):
        xs = workloads.uniform_inputs(n, count, seed=100 + count, dtype="bf16")
        want = folds.expected_bf16(xs, schedule, g)
        bufs = [x.copy() for x in xs]
        oracle.run(bufs, "bf16", schedule, group_size=g)
        for r in range(n):
            np.testing.assert_array_equal(bufs[r], want,
                                          err_msg=f"{schedule} n={n} g={g} count={count} rank={r}")


def test_orders_really_differ():
    """The three schedules fold in different orders, so their low bits differ
    on generic data (Scaling ML systems ch. 06: reproducibility needs a fixed
    algorithm).  Guards against a fold test that cannot tell orders apart."""
    xs = workloads.normal_inputs(8, 4096, seed=3)
    res = {}
    for sched, g in (("ring", 1), ("rabenseifner", 1), ("hierarchical", 4)):
        bufs = [x.copy() for x in xs]
        oracle.run(bufs, "fp32", sched, group_size=g)
        res[sched] = bufs[0].view(np.uint32).copy()
    assert (res["ring"] != res["rabenseifner"]).any()
    assert (res["ring"] != res["hierarchical"]).any()
    assert (res["rabenseifner"] != res["hierarchical"]).any()


@pytest.mark.parametrize("schedule,n,g", [("ring", 5, 1), ("ring", 16, 8), ("hierarchical", 16, 8),
                                          ("hierarchical", 12, 3), ("rabenseifner", 16, 1),
                                          ("rabenseifner", 64, 1), ("ring", 64, 8)])
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_integer_inputs_give_exact_sum(schedule, n, g, dtype):
    count = 1000 + n
    xs = workloads.integer_inputs(n, count, seed=n, dtype=dtype)
    exact = np.zeros(count, np.float64)
    for x in xs:
        exact += (folds.widen(x) if dtype == "bf16" else x).astype(np.float64)
    if dtype == "bf16":
        assert np.abs(exact).max() < 256  # every partial sum is exact in bf16's 8 bits
    bufs = [x.copy() for x in xs]
    oracle.run(bufs, dtype, schedule, group_size=g)
    for b in bufs:
        got = folds.widen(b) if dtype == "bf16" else b
        np.testing.assert_array_equal(got.astype(np.float64), exact)


@pytest.mark.parametrize("schedule,n,g", [("ring", 16, 8), ("hierarchical", 16, 8),
                                          ("rabenseifner", 16, 1), ("ring", 7, 1)])
def test_fp32_within_fp64_bound(schedule, n, g):
    """Reading of "within 1e-5 relative of an fp64 sum": elementwise
    |y - y64| <= 1e-5 * sum_r |x_r| (a pure relative bound is meaningless
    where the sum cancels)."""
    count = 20000
    xs = workloads.normal_inputs(n, count, seed=11)
    y64 = np.sum([x.astype(np.float64) for x in xs], axis=0)
    absum = np.sum([np.abs(x.astype(np.float64)) for x in xs], axis=0)
    bufs = [x.copy() for x in xs]
    oracle.run(bufs, "fp32", schedule, group_size=g)
    for b in bufs:
        assert np.all(np.abs(b.astype(np.float64) - y64) <= 1e-5 * absum)
        # recursive summation bound (N-1) u sum|x| with u = 2^-24
        assert np.all(np.abs(b.astype(np.float64) - y64) <= (n - 1) * 2.0 ** -24 * absum * (1 + 1e-6))
    assert np.linalg.norm(bufs[0] - y64) / np.linalg.norm(y64) < 1e-6


def test_denormals_are_kept():
    """No flush-to-zero: sums of denormals stay denormal and exact."""
    tiny = np.float32(1e-45)  # smallest positive denormal
    xs = [np.full(8, tiny * (r + 1), np.float32) for r in range(4)]
    for sched in ("ring", "rabenseifner", "hierarchical"):
        bufs = [x.copy() for x in xs]
        oracle.run(bufs, "fp32", sched, group_size=2)
        for b in bufs:
            assert np.all(b == np.float32(tiny * 10))


def test_bf16_rounds_once_not_per_step():
    """bf16 partial sums travel in fp32 and are rounded once: a case where
    per-step rounding would lose the small terms entirely."""
    one = np.float32(1.0)
    small = np.float32(2.0 ** -9)  # half an ulp of bf16 at 1.0 would be 2^-8
    n = 4
    xs32 = [np.full(4, one if r == 0 else small, np.float32) for r in range(n)]
    xs = [folds.to_bf16_bits(x) for x in xs32]
    bufs = [x.copy() for x in xs]
    oracle.run(bufs, "bf16", "ring")
    # exact sum 1 + 3 * 2^-9 = 1.005859375; nearest bf16 is 1 + 2^-7 = 1.0078125
    for b in bufs:
        assert np.all(folds.widen(b) == np.float32(1.0078125))


def test_bf16_round_to_nearest_even_cases():
    """Rounding of fp32 partials to bf16, ties to even, checked on crafted
    two-rank sums against torch's conversion (a library routine)."""
    vals = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 3.0e38, 1e-40,
                     2.0 ** -126, 65504.0], np.float32)
    a = folds.to_bf16_bits(vals)
    zeros = np.zeros_like(a)
    bufs = [a.copy(), zeros.copy()]
    oracle.run(bufs, "bf16", "ring")
    for b in bufs:
        np.testing.assert_array_equal(b, a)
    # sums that land exactly between two bf16 values
    x = folds.to_bf16_bits(np.full(6, 1.0, np.float32))
    y = folds.to_bf16_bits(np.array([2 ** -8, 3 * 2 ** -8, 2 ** -9, -2 ** -8, 2 ** -7, 5 * 2 ** -8],
                                    np.float32))
    bufs = [x.copy(), y.copy()]
    oracle.run(bufs, "bf16", "ring")
    exact = folds.widen(x) + folds.widen(y)  # exact in fp32
    np.testing.assert_array_equal(bufs[0], folds.to_bf16_bits(exact))
