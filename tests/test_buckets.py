"""Bucket fuser ("Collective communication", Scaling ML systems ch. 06,
"Bucket fusion"): tensors go into buckets in reverse order, each bucket gets
one all-reduce.  The layout rules beyond "reverse order, about 25 MB" are a
reading (parity unpinned by the pages): close a bucket before a tensor that
would exceed the cap, a tensor larger than the cap gets its own bucket,
tensors are packed back to back, buckets start 256-byte aligned."""
import numpy as np
import pytest

import oracle
from gradient_all_reduce_ar_amd import _binding as B
from gradient_all_reduce_ar_amd import workloads

CAP = 25 << 20


def _brute_layout(sizes, cap_elems, align):
    """Independent restatement of the rules, for comparison."""
    buckets, cur = [], []
    for t in reversed(range(len(sizes))):
        if cur and sum(sizes[i] for i in cur) + sizes[t] > cap_elems:
            buckets.append(cur)
            cur = []
        cur.append(t)
    if cur:
        buckets.append(cur)
    offsets, ranges, pos = {}, [], 0
    for b in buckets:
        pos = (pos + align - 1) // align * align
        start = pos
        for t in b:
            offsets[t] = pos
            pos += sizes[t]
        ranges.append((start, pos - start))
    return [offsets[t] for t in range(len(sizes))], ranges, pos


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_layout_matches_rules(dtype):
    eb = 2 if dtype == "bf16" else 4
    for sizes in (workloads.bucketed_tensor_sizes(elem_bytes=eb), [5, 7, 3], [CAP // eb + 1, 3, CAP // eb, 1],
                  [1] * 50, []):
        sizes = [int(s) for s in sizes]
        bp = B.ar_bucket_plan_create(4, 1, sizes, dtype, "ring", CAP)
        try:
            offs, arena = B.ar_bucket_layout(bp, len(sizes))
            ranges = [B.ar_bucket_range(bp, b) for b in range(B.ar_bucket_count(bp))]
            want_offs, want_ranges, want_arena = _brute_layout(sizes, CAP // eb, 256 // eb)
            assert offs == want_offs and ranges == want_ranges and arena == want_arena
            for off, cnt in ranges:
                assert (off * eb) % 256 == 0
                assert cnt * eb <= CAP or cnt == max(sizes)
        finally:
            B.ar_bucket_plan_destroy(bp)


def test_reverse_order_and_c5_shape():
    sizes = [int(s) for s in workloads.bucketed_tensor_sizes()]
    assert len(sizes) == 300 and max(sizes) * 2 == 64 << 20
    bp = B.ar_bucket_plan_create(16, 1, sizes, "bf16", "rabenseifner", CAP)
    try:
        offs, _ = B.ar_bucket_layout(bp, len(sizes))
        # the last tensor (first ready in backward) sits at the arena start
        assert offs[-1] == 0
        assert all(offs[t] > offs[t + 1] for t in range(len(sizes) - 1))
        st = B.ar_bucket_stats(bp)
        nb = B.ar_bucket_count(bp)
        assert st["steps"] == nb * 8
        # 7 launches per bucket (last halving round fused with the first
        # doubling round); a bucket whose first round's fp32 partials (N x
        # half a bucket x 4 B) exceed 256 MiB runs that round and the next,
        # which reads them, in pieces (2 extra launches per extra piece when
        # the second round's output fits)
        first = [16 * (B.ar_bucket_range(bp, b)[1] // 2) * 4 for b in range(nb)]
        small = [f for f in first if f <= 2 * (256 << 20)]
        extra = sum(2 * (-(-f // (256 << 20)) - 1) for f in small)
        big = nb - len(small)  # the 64 MiB bucket: its first three rounds in 4 pieces
        assert big == 1 and st["launches"] == 7 * nb + extra + 3 * 3
        assert st["launches"] < 7 * sum(max(1, -(-f // (256 << 20))) for f in first)
        assert st["count"] == sum(B.ar_bucket_range(bp, b)[1] for b in range(nb)) == sum(sizes)
    finally:
        B.ar_bucket_plan_destroy(bp)


BATCH_CASES = [("ring", 4, 1), ("ring", 5, 1), ("hierarchical", 8, 4), ("hierarchical", 6, 3),
               ("rabenseifner", 8, 1), ("recursive_doubling", 4, 1), ("tree", 5, 1), ("double_tree", 8, 1)]


def _small_bucket_case(seed):
    rng = np.random.default_rng(seed)
    return [int(s) for s in rng.integers(1, 3000, 40)] + [0, 1, 7]


@pytest.mark.parametrize("sched,n,g", BATCH_CASES)
@pytest.mark.parametrize("dtype", ["fp32", "bf16", "bf16_each"])
@pytest.mark.parametrize("mode", ["steps", "steps_unfused", "onepass"])
def test_batched_plan_matches_oracle(sched, n, g, dtype, mode):
    """The batched launch list (every bucket's all-reduce in shared
    launches), run over the whole arenas by the numpy interpreter, equals
    the oracle bucket by bucket, bit for bit, and leaves the gaps alone.
    Several cache sizes make one batch, a few, or one bucket per batch."""
    from tests import plan_interp

    eb = 4 if dtype == "fp32" else 2
    sizes = _small_bucket_case(n * 31 + g)
    bp = B.ar_bucket_plan_create(n, g, sizes, dtype, sched, 8 << 10)
    try:
        B.ar_bucket_set_exec(bp, mode)
        offs, arena = B.ar_bucket_layout(bp, len(sizes))
        nb = B.ar_bucket_count(bp)
        ranges = [B.ar_bucket_range(bp, b) for b in range(nb)]
        gen = "fp32" if dtype == "fp32" else "bf16"
        host = workloads.bucketed_arenas(n, sizes, offs, arena, sigma=1.0, dtype=gen)
        refs = [oracle.run([h[off:off + cnt].copy() for h in host], dtype, sched, group_size=g)
                for off, cnt in ranges]
        per_bucket = B.ar_bucket_stats(bp)["launches"]
        for cache in (None, 3000 * eb, 1):
            if cache is not None:
                B.ar_bucket_set_cache_bytes(bp, cache)
            m = B.ar_bucket_batched_plan(bp)
            nl = B.ar_plan_num_launches(m)
            assert nl <= B.ar_bucket_stats(bp)["launches"]
            if cache == 1 and mode != "onepass":
                assert nl == B.ar_bucket_stats(bp)["launches"]  # one bucket per batch
            if cache is None:
                assert nl < per_bucket or per_bucket <= 1
            got = plan_interp.run(m, [h.copy() for h in host], dtype, g)
            bv = np.uint32 if dtype == "fp32" else np.uint16
            covered = np.zeros(arena, bool)
            for b, (off, cnt) in enumerate(ranges):
                covered[off:off + cnt] = True
                for r in range(n):
                    np.testing.assert_array_equal(got[r][off:off + cnt].view(bv), refs[b][r].view(bv),
                                                  err_msg=f"cache={cache} bucket {b} rank {r}")
            for r in range(n):
                assert np.array_equal(got[r][~covered].view(bv), host[r][~covered].view(bv))
    finally:
        B.ar_bucket_plan_destroy(bp)


def test_batched_plan_c5_launches():
    """C5 shape: 12 buckets of at most 25 MiB at 16 ranks.  In the step mode
    the buckets form batches whose widest round (the fp32 partials, N chunks
    x 4 B) fits 256 MiB; a batch takes the launches of one bucket.  One-pass:
    one launch for everything."""
    sizes = [int(s) for s in workloads.bucketed_tensor_sizes()]
    bp = B.ar_bucket_plan_create(16, 1, sizes, "bf16", "ring", CAP)
    try:
        nb = B.ar_bucket_count(bp)
        cnts = [B.ar_bucket_range(bp, b)[1] for b in range(nb)]
        batches, fill = 1, 0
        for c in cnts:
            w = 4 * c  # a reduce-scatter round writes every element once as an fp32 partial
            if fill and fill + w > 256 << 20:
                batches, fill = batches + 1, 0
            fill += w
        m = B.ar_bucket_batched_plan(bp)
        assert B.ar_bucket_stats(bp)["launches"] == 29 * nb
        assert B.ar_plan_num_launches(m) == 29 * batches and batches < nb
        st = B.ar_plan_stats(m)
        assert st["count"] == B.ar_bucket_layout(bp, len(sizes))[1]
        assert st["bytes_sent_total"] == B.ar_bucket_stats(bp)["bytes_sent_total"]
        assert st["hbm_bytes_model"] == B.ar_bucket_stats(bp)["hbm_bytes_model"]
        B.ar_bucket_set_exec(bp, "onepass")
        assert B.ar_plan_num_launches(B.ar_bucket_batched_plan(bp)) == 1
    finally:
        B.ar_bucket_plan_destroy(bp)


def test_batched_plan_reuses_scratch():
    """The batches run one after another, so the fp32 partial-sum slots of a
    batched bf16 plan span the widest batch, not the whole arena (C5,
    Rabenseifner at 64 ranks: N/2 slots)."""
    sizes = [int(s) for s in workloads.bucketed_tensor_sizes()]
    bp = B.ar_bucket_plan_create(64, 1, sizes, "bf16", "rabenseifner", CAP)
    try:
        _, arena = B.ar_bucket_layout(bp, len(sizes))
        m = B.ar_bucket_batched_plan(bp)
        shifts = sorted({B.ar_plan_launch_scratch(m, i)[0] for i in range(B.ar_plan_num_launches(m))})
        stride = B.ar_plan_launch_scratch(m, 0)[1]
        ranges = [B.ar_bucket_range(bp, b) for b in range(B.ar_bucket_count(bp))]
        assert shifts[0] == 0 and set(shifts) <= {off for off, _ in ranges}
        assert max(c for _, c in ranges) <= stride < arena // 4
        assert B.ar_plan_stats(m)["scratch_bytes"] == 32 * stride * 4
    finally:
        B.ar_bucket_plan_destroy(bp)


@pytest.mark.parametrize("exec_mode", ["steps", "onepass"])
def test_batched_plan_op_cap(exec_mode):
    """Many tiny buckets: a merged launch holds launch i of every bucket of its
    batch, so the batches also close before a launch would exceed 65535 ops
    (the workgroups one launch grid holds along the ops).  The merged plan
    still holds exactly the buckets' ops, shifted to their arena offsets."""
    sizes = [64] * 5000  # 5000 buckets of 256 B, 16 ops per ring round each
    bp = B.ar_bucket_plan_create(16, 1, sizes, "fp32", "ring", 256)
    try:
        B.ar_bucket_set_exec(bp, exec_mode)
        m = B.ar_bucket_batched_plan(bp)
        nl = B.ar_plan_num_launches(m)
        nops = [B.ar_plan_launch_info(m, i)[1] for i in range(nl)]
        assert max(nops) <= 65535
        per_bucket = 29 if exec_mode == "steps" else 1
        assert nl == per_bucket * 2  # 4095 buckets x 16 ops, then the other 905
        assert sum(nops) == 5000 * 16 * per_bucket
        got = set()
        for i in range(nl):
            ops = B.ar_plan_launch_ops(m, i)
            got.update(zip(ops["lo"].tolist(), ops["hi"].tolist(), ops["a"].tolist(), ops["o"].tolist()))
        want = set()
        for b in range(B.ar_bucket_count(bp)):
            off, cnt = B.ar_bucket_range(bp, b)
            p = B.ar_plan_create(16, 1, cnt, "fp32", "ring")
            try:
                B.ar_plan_set_exec(p, exec_mode)
                for i in range(B.ar_plan_num_launches(p)):
                    ops = B.ar_plan_launch_ops(p, i)
                    want.update(zip((ops["lo"] + off).tolist(), (ops["hi"] + off).tolist(), ops["a"].tolist(),
                                    ops["o"].tolist()))
            finally:
                B.ar_plan_destroy(p)
        assert got == want
    finally:
        B.ar_bucket_plan_destroy(bp)


def test_batched_plan_errors():
    bp = B.ar_bucket_plan_create(4, 1, [300, 500], "int8_ef", "ring", CAP)
    try:
        with pytest.raises(B.ArError) as ei:
            B.ar_bucket_batched_plan(bp)
        assert ei.value.status == B.AR_ERR_UNSUPPORTED
    finally:
        B.ar_bucket_plan_destroy(bp)
    bp = B.ar_bucket_plan_create(4, 1, [], "fp32", "ring", CAP)
    try:
        with pytest.raises(B.ArError):
            B.ar_bucket_batched_plan(bp)
    finally:
        B.ar_bucket_plan_destroy(bp)


@pytest.mark.gpu
@pytest.mark.timeout(900)
@pytest.mark.parametrize("n,sched", [(16, "rabenseifner"), (16, "ring"), (64, "rabenseifner"), (64, "ring")])
def test_bucketed_bf16_parity(n, sched):
    """C5: 300 lognormal bf16 tensors per rank, 25 MiB buckets, one
    all-reduce per bucket, batched (the default) and one by one; bit-exact
    per bucket against the oracle, all ranks identical, gaps between buckets
    untouched."""
    import torch

    sizes = [int(s) for s in workloads.bucketed_tensor_sizes()]
    bp = B.ar_bucket_plan_create(n, 1, sizes, "bf16", sched, CAP)
    try:
        offs, arena = B.ar_bucket_layout(bp, len(sizes))
        host = workloads.bucketed_arenas(n, sizes, offs, arena)
        nb = B.ar_bucket_count(bp)
        refs = {}
        # batched and one by one in the step mode; the one-pass mode (every
        # bucket in one launch) as the benchmark's comparison runs it
        for batch, mode in ((True, "steps"), (False, "steps"), (True, "onepass")):
            print(f"case bucketed n={n} {sched} batched={batch} {mode}", flush=True)
            B.ar_bucket_set_batching(bp, batch)
            B.ar_bucket_set_exec(bp, mode)
            bufs = [torch.from_numpy(h.view(np.int16)).to("cuda:0") for h in host]
            B.ar_bucket_allreduce(bp, bufs, torch.cuda.current_stream())
            torch.cuda.synchronize()
            for r in range(1, n):
                assert torch.equal(bufs[r], bufs[0]), f"rank {r} differs from rank 0"
            got = bufs[0].cpu().numpy().view(np.uint16)
            del bufs
            covered = np.zeros(arena, bool)
            for b in range(nb):
                off, cnt = B.ar_bucket_range(bp, b)
                covered[off:off + cnt] = True
                if b not in refs:
                    refs[b] = oracle.run([h[off:off + cnt].copy() for h in host], "bf16", sched)[0]
                assert np.array_equal(got[off:off + cnt], refs[b]), f"bucket {b} batched={batch} {mode}"
            print(f"  {nb} buckets bit-exact", flush=True)
            assert np.all(got[~covered] == 0)
    finally:
        B.ar_bucket_plan_destroy(bp)


@pytest.mark.gpu
@pytest.mark.parametrize("sched,n,g", BATCH_CASES)
@pytest.mark.parametrize("dtype", ["fp32", "bf16", "bf16_each"])
def test_batched_small_gpu(sched, n, g, dtype):
    """Batched buckets on the GPU at small sizes, every exec mode, eager and
    replayed as a graph (three replays, each checked), against the oracle."""
    import torch

    sizes = _small_bucket_case(n * 31 + g)
    bp = B.ar_bucket_plan_create(n, g, sizes, dtype, sched, 8 << 10)
    try:
        offs, arena = B.ar_bucket_layout(bp, len(sizes))
        ranges = [B.ar_bucket_range(bp, b) for b in range(B.ar_bucket_count(bp))]
        gen = "fp32" if dtype == "fp32" else "bf16"
        host = workloads.bucketed_arenas(n, sizes, offs, arena, sigma=1.0, dtype=gen)
        refs = [oracle.run([h[off:off + cnt].copy() for h in host], dtype, sched, group_size=g)
                for off, cnt in ranges]
        sv = np.float32 if dtype == "fp32" else np.int16
        bv = np.uint32 if dtype == "fp32" else np.uint16
        for mode in ("steps", "steps_unfused", "onepass"):
            B.ar_bucket_set_exec(bp, mode)
            for graph in (False, True):
                B.ar_bucket_set_graph(bp, graph)
                for cache in (None, 3000 * (4 if dtype == "fp32" else 2)):
                    if cache is not None:
                        B.ar_bucket_set_cache_bytes(bp, cache)
                    print(f"case batched {sched} n={n} g={g} {dtype} {mode} graph={graph} cache={cache}",
                          flush=True)
                    bufs = [torch.from_numpy(h.view(sv)).to("cuda:0") for h in host]
                    for rep in range(3 if graph else 1):
                        if rep:
                            for t, h in zip(bufs, host):
                                t.copy_(torch.from_numpy(h.view(sv)))
                            torch.cuda.synchronize()
                        B.ar_bucket_allreduce(bp, bufs, torch.cuda.current_stream())
                        torch.cuda.synchronize()
                        got = [t.cpu().numpy().view(bv) for t in bufs]
                        for b, (off, cnt) in enumerate(ranges):
                            for r in range(n):
                                assert np.array_equal(got[r][off:off + cnt], refs[b][r].view(bv)), \
                                    f"bucket {b} rank {r} replay {rep}"
                B.ar_bucket_set_cache_bytes(bp, 256 << 20)
    finally:
        B.ar_bucket_plan_destroy(bp)


@pytest.mark.gpu
def test_many_tiny_buckets_gpu():
    """5000 buckets of 64 fp32 elements at 16 ranks: the batched launches are
    capped at 65535 ops, so the call runs (two batches) and every bucket
    matches the oracle, in the step and the one-pass modes."""
    import torch

    sizes = [64] * 5000
    bp = B.ar_bucket_plan_create(16, 1, sizes, "fp32", "ring", 256)
    try:
        offs, arena = B.ar_bucket_layout(bp, len(sizes))
        ranges = [B.ar_bucket_range(bp, b) for b in range(B.ar_bucket_count(bp))]
        host = workloads.bucketed_arenas(16, sizes, offs, arena, sigma=1.0, dtype="fp32")
        refs = [oracle.run([h[off:off + cnt].copy() for h in host], "fp32", "ring") for off, cnt in ranges]
        for mode in ("steps", "onepass"):
            B.ar_bucket_set_exec(bp, mode)
            print(f"case many tiny buckets fp32 ring n=16 {mode}", flush=True)
            bufs = [torch.from_numpy(h).to("cuda:0") for h in host]
            B.ar_bucket_allreduce(bp, bufs, torch.cuda.current_stream())
            torch.cuda.synchronize()
            got = [t.cpu().numpy().view(np.uint32) for t in bufs]
            for b, (off, cnt) in enumerate(ranges):
                for r in range(16):
                    assert np.array_equal(got[r][off:off + cnt], refs[b][r].view(np.uint32)), f"bucket {b} rank {r}"
    finally:
        B.ar_bucket_plan_destroy(bp)
