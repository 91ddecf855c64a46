"""Randomised GPU parity: seeded draws of (schedule, ranks, group, size,
dtype, exec mode, assumed cache size), run through the C ABI on cuda:0 and
compared with the oracle bit for bit (results, and residuals for INT8).
Sizes reach a few hundred thousand elements per rank, so ops span many tiles
and end on ragged tails; small assumed caches force the group-by-group and
piece-by-piece launch orders."""
import sys

import numpy as np
import pytest

import oracle
from gradient_all_reduce_ar_amd import _binding as B
from gradient_all_reduce_ar_amd import workloads
from tests.gpu_util import bits_view, to_device, to_host_bits

pytestmark = pytest.mark.gpu

SCHEDS = ["ring", "hierarchical", "rabenseifner", "recursive_doubling", "tree", "double_tree"]
POW2 = {"rabenseifner", "recursive_doubling", "double_tree"}


def _draw(rng):
    sched = SCHEDS[rng.integers(len(SCHEDS))]
    if sched in POW2:
        n = int(2 ** rng.integers(0, 7))
        g = 1
    else:
        n = int(rng.integers(1, 65))
        divisors = [d for d in range(1, n + 1) if n % d == 0]
        g = int(divisors[rng.integers(len(divisors))]) if sched == "hierarchical" else 1
    dtype = ["fp32", "bf16", "bf16_each", "int8_ef"][rng.integers(4)]
    mode = ["steps", "steps_unfused", "onepass"][rng.integers(3)]
    count = int(rng.integers(0, 300000 // max(1, n // 8)))
    cache = [None, None, 1 << 16, 1 << 20][rng.integers(4)]
    return sched, n, g, dtype, mode, count, cache


@pytest.mark.parametrize("batch", range(8))
def test_random_cases(batch):
    import torch

    for k in range(30):
        case = batch * 30 + k
        rng = np.random.default_rng([7, case])
        sched, n, g, dtype, mode, count, cache = _draw(rng)
        what = f"random case {case}: {sched} n={n} g={g} {dtype} {mode} count={count} cache={cache}"
        print(what, flush=True)
        sys.stdout.flush()
        p = B.ar_plan_create(n, g, count, dtype, sched)
        try:
            B.ar_plan_set_exec(p, mode)
            if cache is not None:
                B.ar_plan_set_cache_bytes(p, cache)
            s = torch.cuda.current_stream()
            if dtype == "int8_ef":
                xs = [(rng.standard_normal(count) * np.exp(rng.standard_normal(count))).astype(np.float32)
                      for _ in range(n)]
                es = [(rng.standard_normal(count) * 1e-2).astype(np.float32) for _ in range(n)]
                bufs = [torch.from_numpy(x).to("cuda:0") for x in xs]
                errs = [torch.from_numpy(e).to("cuda:0") for e in es]
                B.ar_allreduce_ef(p, bufs, errs, s)
                torch.cuda.synchronize()
                rb, re_ = [x.copy() for x in xs], [e.copy() for e in es]
                oracle.run_int8ef(rb, sched, errs=re_, group_size=g)
                for r in range(n):
                    assert np.array_equal(bufs[r].cpu().numpy().view(np.uint32), rb[r].view(np.uint32)), what
                    assert np.array_equal(errs[r].cpu().numpy().view(np.uint32), re_[r].view(np.uint32)), what
            else:
                gen = "fp32" if dtype == "fp32" else "bf16"
                xs = workloads.normal_inputs(n, count, seed=case, sigma=1.0, dtype=gen)
                bufs = to_device(xs, dtype)
                B.ar_allreduce(p, bufs, s)
                torch.cuda.synchronize()
                ref = oracle.run([x.copy() for x in xs], dtype, sched, group_size=g)
                got = to_host_bits(bufs, dtype)
                bv = bits_view(dtype)
                for r in range(n):
                    assert np.array_equal(got[r], ref[r].view(bv)), what
        finally:
            B.ar_plan_destroy(p)


HALF_SCHEDS = ["ring", "hierarchical", "rabenseifner"]


def _draw_half(rng):
    sched = HALF_SCHEDS[rng.integers(len(HALF_SCHEDS))]
    if sched == "rabenseifner":
        n, g = int(2 ** rng.integers(0, 7)), 1
    else:
        n = int(rng.integers(1, 65))
        divisors = [d for d in range(1, n + 1) if n % d == 0]
        g = int(divisors[rng.integers(len(divisors))]) if sched == "hierarchical" else 1
    dtype = ["fp32", "bf16", "bf16_each"][rng.integers(3)]
    mode = ["steps", "steps_unfused", "onepass"][rng.integers(3)]
    coll = ["reduce_scatter", "allgather"][rng.integers(2)]
    count = int(rng.integers(0, 300000 // max(1, n // 8)))
    cache = [None, None, 1 << 16, 1 << 20][rng.integers(4)]
    return sched, n, g, dtype, mode, coll, count, cache


@pytest.mark.parametrize("batch", range(4))
def test_random_halves(batch):
    """Seeded draws of reduce-scatter and all-gather plans (schedule, ranks,
    group, size, dtype, exec mode, assumed cache size) against the oracle's
    halves, every element of every rank bit for bit (the one-pass
    reduce-scatter: the oracle's values on the owned ranges, the inputs
    elsewhere)."""
    import torch

    from tests.test_halves_cpu import onepass_reduce_scatter_expected

    for k in range(20):
        case = batch * 20 + k
        rng = np.random.default_rng([11, case])
        sched, n, g, dtype, mode, coll, count, cache = _draw_half(rng)
        what = f"random halves case {case}: {coll} {sched} n={n} g={g} {dtype} {mode} count={count} cache={cache}"
        print(what, flush=True)
        sys.stdout.flush()
        gen = "fp32" if dtype == "fp32" else "bf16"
        xs = workloads.normal_inputs(n, count, seed=1000 + case, sigma=1.0, dtype=gen)
        if coll == "allgather":
            ref = oracle.allgather([x.copy() for x in xs], dtype, sched, group_size=g)
        elif mode == "onepass":
            ref = onepass_reduce_scatter_expected(xs, dtype, sched, g)
        else:
            ref = oracle.reduce_scatter([x.copy() for x in xs], dtype, sched, group_size=g)
        p = B.ar_plan_create_collective(n, g, count, dtype, sched, coll)
        try:
            B.ar_plan_set_exec(p, mode)
            if cache is not None:
                B.ar_plan_set_cache_bytes(p, cache)
            bufs = to_device(xs, dtype)
            (B.ar_reduce_scatter if coll == "reduce_scatter" else B.ar_allgather)(p, bufs, torch.cuda.current_stream())
            torch.cuda.synchronize()
        finally:
            B.ar_plan_destroy(p)
        got = to_host_bits(bufs, dtype)
        bv = bits_view(dtype)
        for r in range(n):
            assert np.array_equal(got[r], ref[r].view(bv)), f"{what}: rank {r}"
