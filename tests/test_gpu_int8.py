"""GPU parity of the blockwise INT8 all-reduce with error feedback.

The HIP path (through the C ABI, on cuda:0) against the CPU oracle, bit for
bit: every rank's decoded result and every rank's new residual.  Sizes span
several tiles and ragged final blocks; the full-size case is 16 ranks of
192 MiB of fp32 gradients in the launch configuration the benchmark times.
"""
import sys

import numpy as np
import pytest

import oracle
from gradient_all_reduce_ar_amd import _binding as B
from gradient_all_reduce_ar_amd import workloads

pytestmark = pytest.mark.gpu
Q = B.QBLOCK


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _dev(xs):
    import torch

    return [torch.from_numpy(np.ascontiguousarray(x)).to("cuda:0") for x in xs]


def _host(ts):
    return [t.cpu().numpy() for t in ts]


def _gpu(xs, es, sched, g, mode="steps", plan=None, calls=1):
    import torch

    bufs = _dev(xs)
    errs = _dev(es) if es is not None else None
    own = plan is None
    if own:
        plan = B.ar_plan_create(len(xs), g, len(xs[0]), "int8_ef", sched)
        B.ar_plan_set_exec(plan, mode)
    try:
        outs = []
        for _ in range(calls):
            B.ar_allreduce_ef(plan, bufs, errs, torch.cuda.current_stream())
            torch.cuda.synchronize()
            outs.append((_host(bufs), _host(errs) if errs is not None else None))
    finally:
        if own:
            B.ar_plan_destroy(plan)
    return outs


def _compare(got, ref, what):
    for r in range(len(ref)):
        a, b = got[r].view(np.uint32), ref[r].view(np.uint32)
        if not np.array_equal(a, b):
            bad = np.flatnonzero(a != b)
            raise AssertionError(f"{what} rank {r}: {len(bad)} elements differ, first at {bad[:5]} "
                                 f"({got[r][bad[:3]]} vs {ref[r][bad[:3]]})")


def _case(xs, es, sched, g, mode, calls=1):
    _say(f"case int8_ef {sched} n={len(xs)} g={g} count={len(xs[0])} err={es is not None} {mode} calls={calls}")
    outs = _gpu(xs, es, sched, g, mode, calls=calls)
    rb = [x.copy() for x in xs]
    re_ = [e.copy() for e in es] if es is not None else None
    for c in range(calls):
        oracle.run_int8ef(rb, sched, errs=re_, group_size=g)
        gb, ge = outs[c]
        _compare(gb, rb, f"{sched} n={len(xs)} {mode} call {c} result")
        if es is not None:
            _compare(ge, re_, f"{sched} n={len(xs)} {mode} call {c} residual")


def _grads(n, count, seed):
    """Per-element magnitudes spread over decades so that blocks differ in
    scale (heavy-tailed gradients)."""
    rng = np.random.default_rng(seed)
    return [(rng.standard_normal(count) * np.exp(2 * rng.standard_normal(count))).astype(np.float32)
            for _ in range(n)]


SMALL = [("ring", n, 1) for n in (1, 2, 3, 4, 5, 8, 16, 32, 48, 64)] + \
        [("hierarchical", n, g) for n, g in ((4, 2), (6, 3), (16, 8), (16, 4), (8, 1), (8, 8), (64, 8), (64, 16),
                                             (32, 8), (48, 8))] + \
        [("rabenseifner", n, 1) for n in (2, 8, 16, 64)] + \
        [("recursive_doubling", n, 1) for n in (2, 8, 64)] + \
        [("tree", n, 1) for n in (2, 5, 13, 64)] + \
        [("double_tree", n, 1) for n in (2, 8, 64)]


@pytest.mark.parametrize("sched,n,g", SMALL)
def test_small_sizes(sched, n, g):
    for count in (0, 1, 127, 128, 129, 5 * Q + 77, 100003):
        xs = _grads(n, count, seed=count + n)
        es = [(x * np.float32(0.01)).astype(np.float32) for x in _grads(n, count, seed=count + 1000)]
        for mode in ("steps", "steps_unfused", "onepass"):
            _case(xs, es, sched, g, mode)
        _case(xs, None, sched, g, "steps")
        _case(xs, None, sched, g, "onepass")


def test_error_feedback_over_calls():
    """Three calls in a row on the same buffers: each call's residual feeds
    the next, and the rank buffers carry the previous result as the next
    gradient (a plan is reused as in training)."""
    n, count = 8, 64 * Q + 33
    xs = _grads(n, count, seed=7)
    es = [np.zeros(count, np.float32) for _ in range(n)]
    _case(xs, es, "ring", 1, "steps", calls=3)
    _case(xs, es, "ring", 1, "onepass", calls=3)


def test_special_blocks():
    """Zero blocks, one non-zero element per block, denormal scales, exact
    ties of the rounding, values that reach the clamp, and signed zeros (a
    code of -0 decodes to +0; -0 - 0 keeps its sign in the residual)."""
    n, count = 4, 16 * Q + 9
    rng = np.random.default_rng(11)
    xs = [np.zeros(count, np.float32) for _ in range(n)]
    for r in range(n):
        xs[r][Q:2 * Q] = rng.integers(-127, 128, Q).astype(np.float32)       # exact codes
        xs[r][2 * Q] = 3.0                                                    # lone value
        xs[r][3 * Q:4 * Q] = (rng.standard_normal(Q) * 1e-38).astype(np.float32)  # denormal scale
        xs[r][4 * Q:5 * Q] = np.float32(127.0)
        xs[r][4 * Q + 1:4 * Q + 11] = np.arange(10, dtype=np.float32) + np.float32(0.5)  # ties
        xs[r][5 * Q:6 * Q] = (rng.standard_normal(Q) * 1e30).astype(np.float32)
        xs[r][6 * Q:7 * Q] = rng.standard_normal(Q).astype(np.float32)
        xs[r][6 * Q:6 * Q + 40:3] = -0.0                                    # -0 inside a block
        xs[r][7 * Q:8 * Q] = -0.0                                            # a block of -0
    es = [np.zeros(count, np.float32) for _ in range(n)]
    for r in range(n):
        es[r][6 * Q:6 * Q + 40:3] = -0.0                                    # g + e = -0
        es[r][7 * Q:8 * Q] = -0.0
    for sched, g in (("ring", 1), ("hierarchical", 2), ("rabenseifner", 1), ("tree", 1), ("double_tree", 1)):
        for mode in ("steps", "onepass"):
            _case(xs, es, sched, g, mode)


def test_plan_reuse_and_bucketed_error_feedback():
    """A bucket plan with error arenas equals one oracle call per bucket."""
    import torch

    n = 4
    sizes = [3000, 129, 70000, 5, 40000]
    bp = B.ar_bucket_plan_create(n, 1, sizes, "int8_ef", "ring", 256 * 1024)
    try:
        offs, arena = B.ar_bucket_layout(bp, len(sizes))
        xs = _grads(n, arena, seed=3)
        es = [(x * np.float32(0.01)).astype(np.float32) for x in _grads(n, arena, seed=4)]
        bufs, errs = _dev(xs), _dev(es)
        _say(f"case bucketed int8_ef n={n} arena={arena} buckets={B.ar_bucket_count(bp)}")
        B.ar_bucket_allreduce_ef(bp, bufs, errs, torch.cuda.current_stream())
        torch.cuda.synchronize()
        gb, ge = _host(bufs), _host(errs)
        rb = [x.copy() for x in xs]
        re_ = [e.copy() for e in es]
        for b in range(B.ar_bucket_count(bp)):
            off, cnt = B.ar_bucket_range(bp, b)
            sb = [x[off:off + cnt].copy() for x in rb]
            se = [e[off:off + cnt].copy() for e in re_]
            oracle.run_int8ef(sb, "ring", errs=se)
            for r in range(n):
                rb[r][off:off + cnt] = sb[r]
                re_[r][off:off + cnt] = se[r]
        _compare(gb, rb, "bucketed result")
        _compare(ge, re_, "bucketed residual")
    finally:
        B.ar_bucket_plan_destroy(bp)


@pytest.mark.timeout(600)
def test_full_size_ring_16_ranks_192mib():
    """16 ranks x 192 MiB of fp32 gradients (the benchmark's workload), ring,
    steps and one-pass, with error feedback: the whole result and residual of
    every rank against the oracle."""
    n, count = 16, workloads.GATE_PROJ_ELEMS
    _say(f"case full int8_ef ring n={n} count={count}: inputs")
    xs = workloads.normal_inputs(n, count, seed=0, sigma=1.0, dtype="fp32")
    es = workloads.normal_inputs(n, count, seed=1, sigma=0.01, dtype="fp32")
    for mode in ("steps", "onepass"):
        _case(xs, es, "ring", 1, mode)


@pytest.mark.timeout(600)
def test_full_size_hierarchical_and_tree_16_ranks():
    """2 groups x 8 ranks hierarchical and the 16-rank double tree, 192 MiB
    each, one-pass and steps, with error feedback."""
    n, count = 16, workloads.GATE_PROJ_ELEMS
    xs = workloads.normal_inputs(n, count, seed=2, sigma=1.0, dtype="fp32")
    es = workloads.normal_inputs(n, count, seed=3, sigma=0.01, dtype="fp32")
    for sched, g in (("hierarchical", 8), ("double_tree", 1)):
        for mode in ("steps", "onepass"):
            _case(xs, es, sched, g, mode)
