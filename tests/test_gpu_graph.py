"""Graph replay of a plan (ar_plan_set_graph / ar_bucket_set_graph) on the GPU.

Each replay is checked against the oracle bit for bit, with eager device
work and synchronisations between replays, several pointer sets per plan
(cache hits, new captures and eviction of the oldest graph), the bf16
scratch path, the INT8 error-feedback path, and bucketed plans.
"""
import sys

import numpy as np
import pytest

import oracle
from gradient_all_reduce_ar_amd import _binding as B
from gradient_all_reduce_ar_amd import workloads
from tests.gpu_util import bits_view, to_device, to_host_bits

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _refill(bufs, xs, dtype):
    import torch

    for b, x in zip(bufs, xs):
        b.copy_(torch.from_numpy(np.ascontiguousarray(x).view(np.float32 if dtype == "fp32" else np.int16)))


def _eager_noise():
    import torch

    a = torch.randn(1 << 20, device="cuda")
    (a * 2 + 1).sum().item()


@pytest.mark.parametrize("sched,n,g,dtype", [("ring", 8, 1, "fp32"), ("hierarchical", 8, 4, "bf16"),
                                              ("rabenseifner", 8, 1, "bf16_each"), ("double_tree", 8, 1, "fp32")])
def test_replays_match_oracle(sched, n, g, dtype):
    import torch

    count = 100003
    gen = "fp32" if dtype == "fp32" else "bf16"
    xs = workloads.normal_inputs(n, count, seed=5, sigma=1.0, dtype=gen)
    ys = workloads.normal_inputs(n, count, seed=6, sigma=1.0, dtype=gen)
    want_x = oracle.run([x.copy() for x in xs], dtype, sched, group_size=g)
    want_y = oracle.run([y.copy() for y in ys], dtype, sched, group_size=g)
    bv = bits_view(dtype)
    a, b = to_device(xs, dtype), to_device(ys, dtype)
    p = B.ar_plan_create(n, g, count, dtype, sched)
    try:
        B.ar_plan_set_graph(p, True)
        s = torch.cuda.current_stream()
        for rep in range(3):
            for bufs, src, want, name in ((a, xs, want_x, "A"), (b, ys, want_y, "B")):
                _say(f"case graph {sched} {dtype} n={n} rep={rep} set={name}")
                _refill(bufs, src, dtype)
                B.ar_allreduce(p, bufs, s)
                torch.cuda.synchronize()
                got = to_host_bits(bufs, dtype)
                for r in range(n):
                    np.testing.assert_array_equal(got[r], want[r].view(bv), err_msg=f"rep {rep} set {name} rank {r}")
                _eager_noise()
    finally:
        B.ar_plan_destroy(p)


@pytest.mark.parametrize("sched,n,g,dtype", [("ring", 16, 1, "fp32"), ("hierarchical", 16, 8, "bf16"),
                                              ("rabenseifner", 16, 1, "bf16"), ("double_tree", 8, 1, "bf16_each"),
                                              ("tree", 40, 1, "fp32")])
@pytest.mark.parametrize("cold", [False, True])
def test_onepass_replays_match_oracle(sched, n, g, dtype, cold):
    """The LDS-staged one-pass folds replayed as graphs, with the store
    policy of a launch that fits the assumed cache and (the cache assumed
    at 64 KiB) of one that does not."""
    import torch

    count = 20011
    gen = "fp32" if dtype == "fp32" else "bf16"
    xs = workloads.normal_inputs(n, count, seed=n + 3, sigma=1.0, dtype=gen)
    want = oracle.run([x.copy() for x in xs], dtype, sched, group_size=g)
    bv = bits_view(dtype)
    bufs = to_device(xs, dtype)
    p = B.ar_plan_create(n, g, count, dtype, sched)
    try:
        B.ar_plan_set_exec(p, "onepass")
        if cold:
            B.ar_plan_set_cache_bytes(p, 64 << 10)
        shape = B.ar_plan_launch_shape(p, 0)
        assert shape["lds_bytes"] > 0 and shape["cold"] == int(cold)
        B.ar_plan_set_graph(p, True)
        s = torch.cuda.current_stream()
        for rep in range(3):
            _say(f"case graph onepass {sched} {dtype} n={n} cold={cold} rep={rep}")
            _refill(bufs, xs, dtype)
            B.ar_allreduce(p, bufs, s)
            torch.cuda.synchronize()
            got = to_host_bits(bufs, dtype)
            for r in range(n):
                np.testing.assert_array_equal(got[r], want[r].view(bv), err_msg=f"rep {rep} rank {r}")
            _eager_noise()
    finally:
        B.ar_plan_destroy(p)


def test_graph_cache_eviction_and_profiling_fallback():
    """Nine pointer sets on one plan (the first graph is evicted and later
    captured again); with profiling on the calls run eagerly and log every
    launch."""
    import torch

    n, count = 4, 4099
    xs = workloads.normal_inputs(n, count, seed=9, sigma=1.0, dtype="fp32")
    want = oracle.run([x.copy() for x in xs], "fp32", "ring")
    sets = [to_device(xs, "fp32") for _ in range(9)]
    p = B.ar_plan_create(n, 1, count, "fp32", "ring")
    try:
        B.ar_plan_set_graph(p, True)
        s = torch.cuda.current_stream()
        for k in list(range(9)) + [0, 8]:
            _say(f"case graph cache set={k}")
            _refill(sets[k], xs, "fp32")
            B.ar_allreduce(p, sets[k], s)
            torch.cuda.synchronize()
            got = to_host_bits(sets[k], "fp32")
            for r in range(n):
                np.testing.assert_array_equal(got[r], want[r].view(np.uint32))
        B.ar_plan_set_profiling(p, 2)
        _refill(sets[0], xs, "fp32")
        B.ar_allreduce(p, sets[0], s)
        torch.cuda.synchronize()
        times = B.ar_plan_launch_times(p)
        assert len(times) == 1 and len(times[0]) == B.ar_plan_num_launches(p)
        got = to_host_bits(sets[0], "fp32")
        for r in range(n):
            np.testing.assert_array_equal(got[r], want[r].view(np.uint32))
    finally:
        B.ar_plan_destroy(p)


def test_int8_error_feedback_replays():
    import torch

    n, count = 8, 50 * 128 + 7
    rng = np.random.default_rng(4)
    xs = [rng.standard_normal(count).astype(np.float32) for _ in range(n)]
    es = [(rng.standard_normal(count) * 0.01).astype(np.float32) for _ in range(n)]
    for mode in ("steps", "onepass"):
        p = B.ar_plan_create(n, 1, count, "int8_ef", "ring")
        try:
            B.ar_plan_set_exec(p, mode)
            B.ar_plan_set_graph(p, True)
            bufs = [torch.from_numpy(x).to("cuda") for x in xs]
            errs = [torch.from_numpy(e).to("cuda") for e in es]
            rb, re_ = [x.copy() for x in xs], [e.copy() for e in es]
            for rep in range(3):
                _say(f"case graph int8_ef {mode} rep={rep}")
                B.ar_allreduce_ef(p, bufs, errs, torch.cuda.current_stream())
                torch.cuda.synchronize()
                oracle.run_int8ef(rb, "ring", errs=re_)
                for r in range(n):
                    np.testing.assert_array_equal(bufs[r].cpu().numpy().view(np.uint32), rb[r].view(np.uint32))
                    np.testing.assert_array_equal(errs[r].cpu().numpy().view(np.uint32), re_[r].view(np.uint32))
                _eager_noise()
        finally:
            B.ar_plan_destroy(p)


def test_bucketed_graph_equals_eager():
    import torch

    n = 8
    sizes = workloads.bucketed_tensor_sizes(elem_bytes=2)[:60]
    outs = []
    for graph in (False, True):
        bp = B.ar_bucket_plan_create(n, 1, sizes, "bf16", "rabenseifner", 4 << 20)
        try:
            B.ar_bucket_set_graph(bp, graph)
            offs, arena = B.ar_bucket_layout(bp, len(sizes))
            host = workloads.bucketed_arenas(n, sizes, offs, arena, dtype="bf16")
            bufs = to_device(host, "bf16")
            for rep in range(3):
                _say(f"case bucketed graph={graph} rep={rep}")
                _refill(bufs, host, "bf16")
                B.ar_bucket_allreduce(bp, bufs, torch.cuda.current_stream())
                torch.cuda.synchronize()
                outs.append((graph, to_host_bits(bufs, "bf16")))
                _eager_noise()
        finally:
            B.ar_bucket_plan_destroy(bp)
    ref = outs[0][1]
    for graph, got in outs[1:]:
        for r in range(n):
            np.testing.assert_array_equal(got[r], ref[r], err_msg=f"graph={graph} rank {r}")
