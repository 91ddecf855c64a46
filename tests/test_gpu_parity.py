"""GPU parity: the HIP path against the CPU oracle, bit for bit.

Every case runs the library through its C ABI on cuda:0 and compares every
element of every rank with the oracle's simulation of the same schedule on
the same seeded inputs (fp32 bits, or bf16 bits).  Sizes span several tiles
and ragged tails; the full-size cases are the 16-rank 192 MiB workloads in
the launch configuration the benchmark times.
"""
import sys

import numpy as np
import pytest

import oracle
from gradient_all_reduce_ar_amd import _binding as B
from gradient_all_reduce_ar_amd import workloads
from tests.folds import widen
from tests.gpu_util import bits_view, gpu_allreduce, to_device, to_host_bits

pytestmark = pytest.mark.gpu

MODES = ["steps", "steps_unfused", "onepass"]


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _check(xs, dtype, sched, group, mode, ref=None):
    _say(f"case {sched} n={len(xs)} g={group} count={len(xs[0])} {dtype} {mode}")
    got = gpu_allreduce(xs, dtype, sched, group, mode)
    if ref is None:
        ref = oracle.run([x.copy() for x in xs], dtype, sched, group_size=group)
    bv = bits_view(dtype)
    for r in range(len(xs)):
        if not np.array_equal(got[r], ref[r].view(bv)):
            bad = np.flatnonzero(got[r] != ref[r].view(bv))
            raise AssertionError(f"{sched} {dtype} {mode} n={len(xs)} g={group} rank {r}: "
                                 f"{len(bad)} elements differ, first at {bad[:5]}")
    return got


def test_c1_ring_fp32_n4():
    """N=4 ring, fp32, 4096 elements per rank, U[-1,1) from seed 0."""
    xs = workloads.uniform_inputs(4, 4096, seed=0)
    for mode in MODES:
        _check(xs, "fp32", "ring", 1, mode)


# Up to 64 ranks: the ring's one-pass fold runs full batches of 16 ranks plus
# a predicated remainder (32, 48, 64), and the hierarchical shapes include
# 8 groups of 8 (the 8 nodes x 8 GPUs case of Scaling ML systems ch. 06,
# "Hierarchical bandwidth multiplier") and groups of 16.
SMALL = [("ring", n, 1) for n in (1, 2, 3, 4, 5, 8, 16, 32, 48, 64)] + \
        [("hierarchical", n, g) for n, g in ((4, 2), (6, 3), (8, 4), (16, 8), (16, 4), (12, 3), (8, 8), (8, 1),
                                             (64, 8), (64, 16), (32, 8), (48, 8))] + \
        [("rabenseifner", n, 1) for n in (2, 4, 8, 16, 64)] + \
        [("recursive_doubling", n, 1) for n in (2, 8, 64)] + \
        [("tree", n, 1) for n in (2, 5, 8, 13, 24, 40, 64)] + \
        [("double_tree", n, 1) for n in (2, 8, 16, 64)]


@pytest.mark.parametrize("sched,n,g", SMALL)
@pytest.mark.parametrize("dtype", ["fp32", "bf16", "bf16_each"])
def test_small_sizes_all_modes(sched, n, g, dtype):
    # 0 and tiny sizes, one that is not a multiple of anything, and one that
    # spans several 4096-element tiles per op with a ragged tail
    for count in (0, 1, 5, 4099, 100003):
        xs = workloads.normal_inputs(n, count, seed=count, sigma=1.0, dtype="fp32" if dtype == "fp32" else "bf16")
        ref = oracle.run([x.copy() for x in xs], dtype, sched, group_size=g)
        for mode in MODES:
            _check(xs, dtype, sched, g, mode, ref)


def test_special_values_fp32():
    """Denormals, signed zeros, infinities and overflow follow IEEE binary32
    exactly as in the oracle (no flush to zero, no fast math)."""
    n, count = 4, 4096 + 16
    vals = np.array([1e-45, -1e-45, 1e-40, 0.0, -0.0, np.inf, -np.inf, 3e38, -3e38, 1.0, 2 ** -149],
                    np.float32)
    rng = np.random.default_rng(5)
    xs = [vals[rng.integers(0, len(vals), count)] for _ in range(n)]
    for sched, g in (("ring", 1), ("hierarchical", 2), ("rabenseifner", 1)):
        for mode in MODES:
            _say(f"special fp32 {sched} {mode}")
            got = gpu_allreduce(xs, "fp32", sched, g, mode)
            ref = oracle.run([x.copy() for x in xs], "fp32", sched, group_size=g)
            for r in range(n):
                a, b = got[r].view(np.float32), ref[r]
                same = (got[r] == b.view(np.uint32)) | (np.isnan(a) & np.isnan(b))
                assert same.all(), (sched, mode, r)


@pytest.mark.parametrize("dtype", ["bf16", "bf16_each"])
def test_special_values_bf16(dtype):
    n, count = 4, 4096 + 16
    vals = np.array([1e-40, -1e-40, 0.0, -0.0, np.inf, -np.inf, 3.3e38, 1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8],
                    np.float32)
    rng = np.random.default_rng(6)
    xs = [workloads._to_bf16_bits(vals[rng.integers(0, len(vals), count)]) for _ in range(n)]
    for sched, g in (("ring", 1), ("hierarchical", 2), ("rabenseifner", 1)):
        for mode in MODES:
            _say(f"special {dtype} {sched} {mode}")
            got = gpu_allreduce(xs, dtype, sched, g, mode)
            ref = oracle.run([x.copy() for x in xs], dtype, sched, group_size=g)
            for r in range(n):
                a, b = widen(got[r]), widen(ref[r])
                same = (got[r] == ref[r]) | (np.isnan(a) & np.isnan(b))
                assert same.all(), (sched, mode, r)


SPECIAL_WIDE = [("ring", 16, 1), ("ring", 64, 1), ("hierarchical", 16, 8), ("hierarchical", 64, 8),
                ("rabenseifner", 16, 1), ("rabenseifner", 64, 1), ("recursive_doubling", 4, 1),
                ("recursive_doubling", 16, 1), ("tree", 5, 1), ("tree", 16, 1), ("tree", 40, 1),
                ("double_tree", 4, 1), ("double_tree", 16, 1), ("double_tree", 64, 1)]


@pytest.mark.parametrize("dtype", ["fp32", "bf16", "bf16_each"])
@pytest.mark.parametrize("sched,n,g", SPECIAL_WIDE)
def test_special_values_every_schedule(sched, n, g, dtype):
    """The same special values through every schedule, at the rank counts
    where the one-pass folds change shape: 16 ranks (one rank per wave), 64
    (eight per wave, one unit per lane), and trees whose rank count is not a
    power of two (missing leaves are -0, the identity of IEEE addition)."""
    count = 4096 + 16
    rng = np.random.default_rng(1000 + n)
    if dtype == "fp32":
        vals = np.array([1e-45, -1e-45, 1e-40, 0.0, -0.0, np.inf, -np.inf, 3e38, -3e38, 1.0, 2 ** -149], np.float32)
        xs = [vals[rng.integers(0, len(vals), count)] for _ in range(n)]
    else:
        vals = np.array([1e-40, -1e-40, 0.0, -0.0, np.inf, -np.inf, 3.3e38, 1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8],
                        np.float32)
        xs = [workloads._to_bf16_bits(vals[rng.integers(0, len(vals), count)]) for _ in range(n)]
    ref = oracle.run([x.copy() for x in xs], dtype, sched, group_size=g)
    for mode in MODES:
        _say(f"special {dtype} {sched} n={n} g={g} {mode}")
        got = gpu_allreduce(xs, dtype, sched, g, mode)
        for r in range(n):
            if dtype == "fp32":
                a, b = got[r].view(np.float32), ref[r]
                same = (got[r] == b.view(np.uint32)) | (np.isnan(a) & np.isnan(b))
            else:
                a, b = widen(got[r]), widen(ref[r])
                same = (got[r] == ref[r]) | (np.isnan(a) & np.isnan(b))
            assert same.all(), (sched, n, mode, r, int(np.argmin(same)))


def test_plan_reuse_streams_and_profiling():
    """One plan, several calls on different buffers and on a side stream; the
    profiling log reports one duration per launch per call."""
    import torch

    n, count = 8, 300001
    plan = B.ar_plan_create(n, 4, count, "bf16", "hierarchical")
    try:
        B.ar_plan_set_profiling(plan, 4)
        side = torch.cuda.Stream()
        for seed in (1, 2, 3):
            xs = workloads.normal_inputs(n, count, seed=seed, dtype="bf16")
            bufs = to_device(xs, "bf16")
            torch.cuda.synchronize()
            with torch.cuda.stream(side):
                B.ar_allreduce(plan, bufs, side)
            side.synchronize()
            ref = oracle.run([x.copy() for x in xs], "bf16", "hierarchical", group_size=4)
            got = to_host_bits(bufs, "bf16")
            for r in range(n):
                assert np.array_equal(got[r], ref[r])
        times = B.ar_plan_launch_times(plan)
        assert len(times) == 3 and all(len(t) == B.ar_plan_num_launches(plan) for t in times)
        assert all(ms > 0 for t in times for ms in t)
        # sampled log: period 3 over 3 calls times every launch exactly once
        B.ar_plan_set_profiling_period(plan, 3)
        xs = workloads.normal_inputs(n, count, seed=9, dtype="bf16")
        bufs = to_device(xs, "bf16")
        for _ in range(3):
            B.ar_allreduce(plan, bufs, torch.cuda.current_stream())
        torch.cuda.synchronize()
        times = B.ar_plan_launch_times(plan)
        nl = B.ar_plan_num_launches(plan)
        assert len(times) == 3
        for i in range(nl):
            timed = [t[i] for t in times if t[i] >= 0]
            assert len(timed) == 1 and timed[0] > 0
            assert all(t[i] == -1 for t in times if t[i] < 0)
    finally:
        B.ar_plan_destroy(plan)


def test_plans_on_host_threads():
    """Distinct plans driven from distinct host threads at once, each on its
    own stream (two of them replaying HIP graphs, captured while the other
    threads launch): every call of every thread matches the oracle.  Buffers
    and outputs are allocated before the threads start."""
    import threading

    import torch

    n, count, reps = 8, 200003, 4
    cases = [("ring", "fp32", 1, False), ("hierarchical", "bf16", 4, True), ("rabenseifner", "fp32", 1, True),
             ("tree", "bf16_each", 1, False)]
    work = []
    for k, (sched, dtype, g, graph) in enumerate(cases):
        xs = workloads.normal_inputs(n, count, seed=50 + k, sigma=1.0, dtype="fp32" if dtype == "fp32" else "bf16")
        ref = oracle.run([x.copy() for x in xs], dtype, sched, group_size=g)
        pristine = to_device(xs, dtype)
        bufs = [t.clone() for t in pristine]
        outs = [[torch.empty_like(t) for t in bufs] for _ in range(reps)]
        work.append(dict(sched=sched, dtype=dtype, g=g, graph=graph, ref=ref, pristine=pristine, bufs=bufs,
                         outs=outs, stream=torch.cuda.Stream(), plan=None, err=None))
    torch.cuda.synchronize()

    def body(w):
        try:
            w["plan"] = B.ar_plan_create(n, w["g"], count, w["dtype"], w["sched"])
            B.ar_plan_set_graph(w["plan"], w["graph"])
            s = w["stream"]
            with torch.cuda.stream(s):
                for rep in range(reps):
                    for b, p in zip(w["bufs"], w["pristine"]):
                        b.copy_(p)
                    B.ar_allreduce(w["plan"], w["bufs"], s)
                    for o, b in zip(w["outs"][rep], w["bufs"]):
                        o.copy_(b)
            s.synchronize()
        except Exception as e:  # reported by the main thread
            w["err"] = e

    _say(f"case host threads: {len(cases)} plans, {reps} calls each")
    threads = [threading.Thread(target=body, args=(w,)) for w in work]
    try:
        for t in threads:
            t.start()
        for t in threads:
            t.join()
        torch.cuda.synchronize()
        for w in work:
            assert w["err"] is None, f"{w['sched']} {w['dtype']}: {w['err']}"
            for rep in range(reps):
                got = to_host_bits(w["outs"][rep], w["dtype"])
                for r in range(n):
                    assert np.array_equal(got[r], w["ref"][r].view(bits_view(w["dtype"]))), \
                        (w["sched"], w["dtype"], rep, r)
    finally:
        for w in work:
            if w["plan"] is not None:
                B.ar_plan_destroy(w["plan"])


# ------------------------------------------------------------- full sizes

E32 = workloads.GATE_PROJ_ELEMS
E16 = workloads.BF16_192MIB_ELEMS


def _full(dtype, sched, group, modes, fp64_check=False):
    count = E32 if dtype == "fp32" else E16
    _say(f"full-size inputs {dtype} n=16 count={count}")
    xs = workloads.normal_inputs(16, count, seed=0, dtype="fp32" if dtype == "fp32" else "bf16")
    ref = oracle.run([x.copy() for x in xs], dtype, sched, group_size=group)
    bv = bits_view(dtype)
    for mode in modes:
        _say(f"full-size {sched} {dtype} {mode}")
        got = gpu_allreduce(xs, dtype, sched, group, mode)
        for r in range(16):
            assert np.array_equal(got[r], ref[r].view(bv)), (sched, dtype, mode, r)
        del got
    if fp64_check:
        y64 = np.zeros(count, np.float64)
        ab = np.zeros(count, np.float64)
        for x in xs:
            y64 += x
            ab += np.abs(x)
        err = np.abs(ref[0].astype(np.float64) - y64)
        assert np.all(err <= 1e-5 * ab)
        assert np.linalg.norm(err) / np.linalg.norm(y64) < 1e-6


def test_full_c2_ring_fp32_16x192MiB():
    _full("fp32", "ring", 8, ["steps", "onepass"], fp64_check=True)


def test_full_c3_ring_bf16_16x192MiB():
    _full("bf16", "ring", 8, ["steps", "onepass"])


def test_full_c4_hierarchical_fp32_2x8x192MiB():
    _full("fp32", "hierarchical", 8, ["steps", "onepass"], fp64_check=True)


def test_full_rabenseifner_fp32_16x192MiB():
    _full("fp32", "rabenseifner", 1, ["steps"])


def test_full_recursive_doubling_fp32_16x192MiB():
    _full("fp32", "recursive_doubling", 1, ["steps", "onepass"])


def test_full_double_tree_bf16_16x192MiB():
    _full("bf16", "double_tree", 1, ["steps", "onepass"])


def test_full_ring_bf16_each_step_16x192MiB():
    _full("bf16_each", "ring", 8, ["steps", "onepass"])


def test_full_rabenseifner_bf16_16x192MiB():
    _full("bf16", "rabenseifner", 1, ["steps", "onepass"])
