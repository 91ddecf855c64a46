"""The library's host planner, checked on the CPU (no GPU needed).

* Its transfers equal the oracle's messages (same rounds, senders, receivers,
  ranges, kinds), and its per-rank bytes, cross-group bytes, step counts and
  alpha-beta times equal the oracle's.
* Its kernel launch list, executed by a numpy interpreter (tests/plan_interp),
  gives bit-for-bit the oracle's result in every exec mode -- this checks the
  lowering (scratch slots, bf16 rounding point, fused forwarding copy,
  one-pass fold orders) before any kernel runs.
* Its byte model matches the closed forms of the step-faithful design.
"""
import numpy as np
import pytest

import oracle
from gradient_all_reduce_ar_amd import _binding as B
from gradient_all_reduce_ar_amd import workloads
from tests import plan_interp

SCHEDS = [("ring", n, 1) for n in (1, 2, 3, 4, 5, 8, 16)] + \
         [("ring", 16, 8), ("ring", 64, 8)] + \
         [("hierarchical", n, g) for n, g in ((2, 1), (4, 2), (4, 4), (6, 3), (6, 2), (8, 4), (16, 8),
                                              (16, 4), (12, 3), (64, 8), (9, 3))] + \
         [("rabenseifner", n, 1) for n in (1, 2, 4, 8, 16, 64)] + \
         [("recursive_doubling", n, 1) for n in (1, 2, 4, 16, 64)] + \
         [("tree", n, 1) for n in (1, 2, 3, 5, 8, 13, 16, 64)] + \
         [("double_tree", n, 1) for n in (2, 4, 8, 16, 64)]


def _plan(n, g, count, dtype, sched):
    return B.ar_plan_create(n, g, count, dtype, sched)


def _sorted(d):
    order = np.lexsort((d["src"], d["step"]))
    return {k: v[order] for k, v in d.items()}


@pytest.mark.parametrize("sched,n,g", SCHEDS)
def test_transfers_equal_oracle(sched, n, g):
    for count in (0, 1, n - 1 if n > 1 else 2, 97, 1000, 4096):
        p = _plan(n, g, count, "fp32", sched)
        try:
            mine = _sorted(B.ar_plan_transfers(p))
            ref = _sorted(oracle.messages(n, count, sched, group_size=g))
            assert len(mine["step"]) == len(ref["step"])
            for k in ("step", "src", "dst", "lo", "hi", "kind"):
                np.testing.assert_array_equal(mine[k], ref[k], err_msg=f"{sched} n={n} g={g} count={count} {k}")
            st = B.ar_plan_stats(p)
            for dt, eb in (("fp32", 4),):
                sent, cross, steps = oracle.stats(n, count, dt, sched, group_size=g)
                assert st["steps"] == steps
                assert st["bytes_sent"] == [int(x) for x in sent]
                assert st["cross_group_bytes_total"] == cross
            t = B.ar_plan_cost_alpha_beta(p, 1e-6, 400e9, 50e9)
            assert t == pytest.approx(oracle.cost(n, count, 4, sched, 1e-6, 400e9, 50e9, group_size=g), rel=1e-12)
        finally:
            B.ar_plan_destroy(p)


@pytest.mark.parametrize("sched,n,g", SCHEDS)
@pytest.mark.parametrize("dtype", ["fp32", "bf16", "bf16_each"])
@pytest.mark.parametrize("mode", ["steps", "steps_unfused", "onepass"])
def test_launch_list_matches_oracle(sched, n, g, dtype, mode):
    for count in (0, 3, 37, 1031):
        xs = workloads.normal_inputs(n, count, seed=count + n, sigma=1.0, dtype="fp32" if dtype == "fp32" else "bf16")
        ref = oracle.run([x.copy() for x in xs], dtype, sched, group_size=g)
        p = _plan(n, g, count, dtype, sched)
        try:
            B.ar_plan_set_exec(p, mode)
            got = plan_interp.run(p, [x.copy() for x in xs], dtype, g)
        finally:
            B.ar_plan_destroy(p)
        for r in range(n):
            np.testing.assert_array_equal(got[r].view(np.uint32 if dtype == "fp32" else np.uint16),
                                          ref[r].view(np.uint32 if dtype == "fp32" else np.uint16),
                                          err_msg=f"{sched} n={n} g={g} {dtype} {mode} count={count} rank={r}")


def test_byte_model_closed_forms():
    """Device bytes per call: step-faithful fp32 moves 5(N-1)S (reduce steps
    read 2 and write 1 slice, copy steps read 1 and write 1); fusing the last
    reduce-scatter step with the first all-gather step saves S; one-pass
    moves 2NS.  bf16 with fp32 partials: (14N-18)E bytes unfused, 2E less
    fused."""
    n, e = 16, 12288 * 4096
    S = 4 * e
    for sched, g in (("ring", 8), ("hierarchical", 8), ("rabenseifner", 1)):
        p = _plan(n, g, e, "fp32", sched)
        try:
            assert B.ar_plan_stats(p)["hbm_bytes_model"] == (5 * n - 6) * S
            B.ar_plan_set_exec(p, "steps_unfused")
            assert B.ar_plan_stats(p)["hbm_bytes_model"] == 5 * (n - 1) * S
            B.ar_plan_set_exec(p, "onepass")
            assert B.ar_plan_stats(p)["hbm_bytes_model"] == 2 * n * S
            assert B.ar_plan_stats(p)["launches"] == 1
        finally:
            B.ar_plan_destroy(p)
    e16 = 2 * e
    p = _plan(n, 8, e16, "bf16_each", "ring")
    try:
        # round-each-step bf16 is fp32's byte model at half the element size
        assert B.ar_plan_stats(p)["hbm_bytes_model"] == (5 * n - 6) * 2 * e16
        assert B.ar_plan_stats(p)["scratch_bytes"] == 0
    finally:
        B.ar_plan_destroy(p)
    p = _plan(n, 8, e16, "bf16", "ring")
    try:
        assert B.ar_plan_stats(p)["hbm_bytes_model"] == (14 * n - 18 - 2) * e16
        B.ar_plan_set_exec(p, "steps_unfused")
        assert B.ar_plan_stats(p)["hbm_bytes_model"] == (14 * n - 18) * e16
        assert B.ar_plan_stats(p)["scratch_bytes"] == 4 * e16
    finally:
        B.ar_plan_destroy(p)


def test_launch_counts():
    for n in (2, 4, 16, 64):
        p = _plan(n, 1, 4096, "fp32", "ring")
        assert B.ar_plan_stats(p)["steps"] == 2 * (n - 1)
        assert B.ar_plan_stats(p)["launches"] == 2 * (n - 1) - 1
        B.ar_plan_destroy(p)
    p = _plan(16, 8, 4096, "fp32", "hierarchical")
    assert B.ar_plan_stats(p)["steps"] == 16 and B.ar_plan_stats(p)["launches"] == 15
    B.ar_plan_destroy(p)
    p = _plan(64, 1, 4096, "bf16", "rabenseifner")
    assert B.ar_plan_stats(p)["steps"] == 12 and B.ar_plan_stats(p)["launches"] == 11
    B.ar_plan_destroy(p)


def test_bf16_scratch_slots():
    """Ring keeps one live partial per chunk (1 slot), hierarchical one per
    group (M slots), Rabenseifner one per pair of ranks (N/2 slots)."""
    e = 1024
    for sched, n, g, slots in (("ring", 16, 8, 1), ("hierarchical", 16, 8, 2), ("hierarchical", 16, 16, 1),
                               ("rabenseifner", 16, 1, 8), ("rabenseifner", 2, 1, 0)):
        p = _plan(n, g, e, "bf16", sched)
        assert B.ar_plan_stats(p)["scratch_bytes"] == slots * 4 * e, sched
        B.ar_plan_destroy(p)


@pytest.mark.parametrize("args,status", [
    ((0, 1, 10, "fp32", "ring"), B.AR_ERR_INVALID_ARG),
    ((1025, 1, 10, "fp32", "ring"), B.AR_ERR_INVALID_ARG),
    ((4, 3, 10, "fp32", "ring"), B.AR_ERR_INVALID_ARG),
    ((4, 0, 10, "fp32", "hierarchical"), B.AR_ERR_INVALID_ARG),
    ((4, 1, 10, 7, "ring"), B.AR_ERR_INVALID_ARG),
    ((4, 1, 10, "fp32", 9), B.AR_ERR_INVALID_ARG),
    ((6, 1, 10, "fp32", "rabenseifner"), B.AR_ERR_UNSUPPORTED),
])
def test_create_errors(args, status):
    with pytest.raises(B.ArError) as ei:
        B.ar_plan_create(*args)
    assert ei.value.status == status
    assert B.ar_last_status() == status
    assert B.ar_last_error()


def test_allreduce_rejects_bad_pointers_without_launching():
    p = B.ar_plan_create(4, 1, 1024, "fp32", "ring")
    try:
        with pytest.raises(B.ArError) as ei:
            B.ar_allreduce(p, [4096, 0, 8192, 12288])
        assert ei.value.status == B.AR_ERR_INVALID_ARG and "NULL" in str(ei.value)
        with pytest.raises(B.ArError) as ei:
            B.ar_allreduce(p, [4096, 8200, 1 << 20, 1 << 21])
        assert "aligned" in str(ei.value)
        with pytest.raises(B.ArError) as ei:
            B.ar_allreduce(p, [1 << 20, (1 << 20) + 1024, 1 << 24, 1 << 25])
        assert "overlap" in str(ei.value)
    finally:
        B.ar_plan_destroy(p)


def test_plan_is_hazard_free_and_each_round_touches_each_chunk_once():
    """Within a launch no op writes what another op reads or writes (the
    planner refuses plans that would); creating every schedule here would
    have raised otherwise."""
    for sched, n, g in SCHEDS:
        for dtype in ("fp32", "bf16", "bf16_each"):
            p = _plan(n, g, 4099, dtype, sched)
            for mode in ("steps", "steps_unfused", "onepass"):
                B.ar_plan_set_exec(p, mode)
            B.ar_plan_destroy(p)


@pytest.mark.parametrize("sched,n,g", [("ring", 16, 8), ("hierarchical", 16, 8), ("hierarchical", 128, 16),
                                       ("hierarchical", 64, 8), ("rabenseifner", 256, 16), ("ring", 128, 1)])
def test_extended_cost_model_equals_oracle(sched, n, g):
    count = 4_000_000_000 // 8 if n >= 128 else 1 << 20
    p = _plan(n, g, count, "bf16", sched)
    try:
        for args in ((0.83e-6, 0.83e-6, 450e9, 50e9, 0.0, 1.0), (1e-6, 5e-6, 450e9, 50e9, 400e9, 8.0),
                     (0.0, 0.0, 900e9, 25e9, 3200e9, 8.0)):
            mine = B.ar_plan_cost_alpha_beta_ex(p, *args)
            ref = oracle.cost_ex(n, count, 2, sched, *args, group_size=g)
            assert mine == pytest.approx(ref, rel=1e-12)
    finally:
        B.ar_plan_destroy(p)


def test_large_plans_describe_but_do_not_run():
    """Plans of up to 1024 ranks give transfers, stats and the cost model;
    running them is refused without touching any device."""
    p = B.ar_plan_create(1024, 8, 1 << 20, "fp32", "ring")
    try:
        st = B.ar_plan_stats(p)
        assert st["steps"] == 2046 and st["launches"] == 0
        assert B.ar_plan_cost_alpha_beta(p, 22e-6, 50e9, 50e9) > 2046 * 22e-6
        with pytest.raises(B.ArError) as ei:
            B.ar_allreduce(p, [1 << 20] * 1024)
        assert ei.value.status == B.AR_ERR_UNSUPPORTED
    finally:
        B.ar_plan_destroy(p)
    mine = B.ar_plan_create(128, 16, 4096, "fp32", "hierarchical")
    try:
        got = _sorted(B.ar_plan_transfers(mine))
        ref = _sorted(oracle.messages(128, 4096, "hierarchical", group_size=16))
        for k in ("step", "src", "dst", "lo", "hi", "kind"):
            np.testing.assert_array_equal(got[k], ref[k])
    finally:
        B.ar_plan_destroy(mine)
    with pytest.raises(B.ArError):
        B.ar_plan_create(1025, 1, 10, "fp32", "ring")


def _oracle_best(n, g, count, eb, cands, args):
    best = None
    for c in cands:
        try:
            t = oracle.cost_ex(n, count, eb, c, *args, group_size=g)
        except oracle.OracleError:
            continue
        if best is None or t < best[1]:
            best = (c, t)
    return best


def test_selector_matches_pages_and_oracle():
    """The selector picks the cheapest candidate by the alpha-beta model:
    Scaling ML systems ch. 06: 1 MB on 64 GPUs (alpha 10 us, beta 10 GB/s),
    tree 1320 us beats ring 1456.9 us; with every schedule allowed the
    butterfly (Rabenseifner) wins; Primer ch. 4: on 128 ranks (22 us, 50 GB/s)
    recursive doubling wins below about 54 MB and the ring above; Data-center
    networks 7.2.1: the 2x8 hierarchical all-reduce (1.3 ms) beats the ring
    (7.6 ms) for the 192 MiB gradient."""
    mb = 1_000_000
    args = (10e-6, 10e-6, 10e9, 10e9, 0.0, 1.0)
    name, t = B.ar_select_schedule(64, 1, mb // 4, "fp32", *args, candidates=["ring", "tree"])
    assert name == "tree" and t * 1e6 == pytest.approx(1320.0)
    name, t = B.ar_select_schedule(64, 1, mb // 4, "fp32", *args)
    assert name == "rabenseifner"
    ob = _oracle_best(64, 1, mb // 4, 4, list(B.SCHEDULES), args)
    assert ob[0] == name and t == pytest.approx(ob[1], rel=1e-12)
    a128 = (22e-6, 22e-6, 50e9, 50e9, 0.0, 1.0)
    for size, want in ((40e6, "recursive_doubling"), (70e6, "ring")):
        name, _ = B.ar_select_schedule(128, 1, int(size) // 4, "fp32", *a128, candidates=["ring", "recursive_doubling"])
        assert name == want
    name, t = B.ar_select_schedule(16, 8, 12288 * 4096, "fp32", 0.83e-6, 0.83e-6, 450e9, 50e9,
                                   candidates=["ring", "hierarchical"])
    assert name == "hierarchical" and t * 1e3 == pytest.approx(1.2995, rel=1e-3)
    # power-of-two schedules are skipped for 12 ranks; none left is an error
    name, _ = B.ar_select_schedule(12, 1, 1 << 20, "fp32", *args, candidates=["rabenseifner", "tree"])
    assert name == "tree"
    with pytest.raises(B.ArError):
        B.ar_select_schedule(12, 1, 1 << 20, "fp32", *args, candidates=["rabenseifner"])


@pytest.mark.parametrize("n", [2, 8, 16, 64, 100, 128, 1024])
def test_selector_agrees_with_oracle_over_sizes(n):
    cands = [c for c in B.SCHEDULES if c != "hierarchical"]
    for size in (1e3, 1e5, 1e7, 1e9):
        count = int(size) // 4
        args = (5e-6, 5e-6, 50e9, 50e9, 0.0, 1.0)
        name, t = B.ar_select_schedule(n, 1, count, "fp32", *args, candidates=cands)
        ob = _oracle_best(n, 1, count, 4, cands, args)
        assert t == pytest.approx(ob[1], rel=1e-12)


HIER_SPLIT = [(16, 8), (16, 4), (8, 4), (6, 3), (9, 3), (12, 3), (64, 8)]


@pytest.mark.parametrize("n,g", HIER_SPLIT)
@pytest.mark.parametrize("dtype", ["fp32", "bf16", "bf16_each"])
@pytest.mark.parametrize("mode", ["steps", "steps_unfused"])
def test_group_by_group_order_matches_oracle(n, g, dtype, mode):
    """With a cache smaller than one round's writes, the hierarchical group
    phases run group by group, and with a cache smaller than one group's
    round the range is also cut into pieces; the results are the oracle's
    bit for bit."""
    m = n // g
    fused = mode == "steps"
    rounds = 2 * m * (g - 1) + 2 * (m - 1) - (1 if fused else 0)  # launches of one piece, group by group
    for count in (37, 1031):
        xs = workloads.normal_inputs(n, count, seed=count + n, sigma=1.0, dtype="fp32" if dtype == "fp32" else "bf16")
        ref = oracle.run([x.copy() for x in xs], dtype, "hierarchical", group_size=g)
        for cache in (64, 1 << 30):
            p = _plan(n, g, count, dtype, "hierarchical")
            try:
                B.ar_plan_set_exec(p, mode)
                B.ar_plan_set_cache_bytes(p, cache)
                got = plan_interp.run(p, [x.copy() for x in xs], dtype, g)
                n_launch = B.ar_plan_num_launches(p)
                one_group = 0  # launches whose receivers all lie in one group (phases 1 and 3)
                for i in range(n_launch):
                    ops = B.ar_plan_launch_ops(p, i)
                    ranks = {int(r) for key in ("a", "b", "o", "o2") for r in ops[key] if 0 <= r < B.LOC_SCRATCH}
                    one_group += len({r // g for r in ranks}) == 1
            finally:
                B.ar_plan_destroy(p)
            bv = np.uint32 if dtype == "fp32" else np.uint16
            for r in range(n):
                np.testing.assert_array_equal(got[r].view(bv), ref[r].view(bv),
                                              err_msg=f"n={n} g={g} {dtype} {mode} cache={cache} r={r}")
            if cache == 64 and m > 1:
                # every group's phase-1 and phase-3 rounds in launches of their own, in every piece
                assert n_launch >= rounds and n_launch % rounds == 0 and one_group >= 2 * m * (g - 1)
            if cache == 1 << 30:
                assert n_launch == 2 * (g - 1) + 2 * (m - 1) - (1 if fused else 0)


def test_group_by_group_order_shape():
    """C4 shape at its real size: the default 256 MiB cache is smaller than a
    phase-1 round's 384 MiB of writes, so group 0's seven rounds come first,
    then group 1's; phase 2 is one fused launch; phase 3 likewise by group.
    A large cache keeps the round-by-round order (15 launches)."""
    p = _plan(16, 8, 12288 * 4096, "fp32", "hierarchical")
    try:
        first_rank = [int(B.ar_plan_launch_ops(p, i)["a"].min()) for i in range(B.ar_plan_num_launches(p))]
        nops = [B.ar_plan_launch_info(p, i)[1] for i in range(B.ar_plan_num_launches(p))]
        assert first_rank == [0] * 7 + [8] * 7 + [0] + [0] * 7 + [8] * 7
        assert nops == [8] * 14 + [16] + [8] * 14
        model = B.ar_plan_stats(p)["hbm_bytes_model"]
        B.ar_plan_set_cache_bytes(p, 1 << 30)
        assert B.ar_plan_num_launches(p) == 15
        assert B.ar_plan_stats(p)["hbm_bytes_model"] == model
    finally:
        B.ar_plan_destroy(p)


@pytest.mark.parametrize("sched,n,g", [s for s in SCHEDS if s[0] != "hierarchical"])
@pytest.mark.parametrize("dtype", ["fp32", "bf16", "bf16_each"])
def test_piece_by_piece_order_matches_oracle(sched, n, g, dtype):
    """With a cache smaller than some rounds' writes, those rounds run on
    element pieces one after another (the others whole); the results are the
    oracle's bit for bit (including pieces that cut through chunks).  The
    cache sizes span every round split, some split, none split."""
    for count in (37, 5000):
        xs = workloads.normal_inputs(n, count, seed=count + n, sigma=1.0, dtype="fp32" if dtype == "fp32" else "bf16")
        ref = oracle.run([x.copy() for x in xs], dtype, sched, group_size=g)
        for mode in ("steps", "steps_unfused"):
            launches = []
            for cache in (2048, 6 * count, 24 * count, 1 << 30):
                p = _plan(n, g, count, dtype, sched)
                try:
                    B.ar_plan_set_exec(p, mode)
                    B.ar_plan_set_cache_bytes(p, cache)
                    got = plan_interp.run(p, [x.copy() for x in xs], dtype, g)
                    launches.append(B.ar_plan_num_launches(p))
                finally:
                    B.ar_plan_destroy(p)
                bv = np.uint32 if dtype == "fp32" else np.uint16
                for r in range(n):
                    np.testing.assert_array_equal(got[r].view(bv), ref[r].view(bv),
                                                  err_msg=f"{sched} n={n} {dtype} {mode} count={count} cache={cache} r={r}")
            # a larger cache never needs more launches
            assert launches == sorted(launches, reverse=True), launches


def test_piece_counts():
    """C3 (bf16 ring): every reduce-scatter round writes 403 MB of fp32
    partials, more than the 256 MiB cache, so the reduce-scatter (with the
    fused first all-gather round) runs on two halves of the range, one after
    the other; the all-gather rounds copy 201 MB of bf16 each and run whole.
    C2 (fp32 ring, 201 MB per round) runs in one piece."""
    p3 = _plan(16, 8, 2 * 12288 * 4096, "bf16", "ring")
    p2 = _plan(16, 8, 12288 * 4096, "fp32", "ring")
    try:
        assert B.ar_plan_num_launches(p2) == 29
        n3 = B.ar_plan_num_launches(p3)
        assert n3 == 2 * 15 + 14
        lo = [int(B.ar_plan_launch_ops(p3, i)["lo"].min()) for i in range(n3)]
        hi = [int(B.ar_plan_launch_ops(p3, i)["hi"].max()) for i in range(n3)]
        kinds = [B.ar_plan_launch_info(p3, i)[0] for i in range(n3)]
        half = (2 * 12288 * 4096 // 2) // 64 * 64
        assert max(hi[:15]) <= half and min(lo[15:30]) >= half
        assert kinds[14] == kinds[29] and kinds[14] & 8  # the fused reduce + copy ends each half
        assert all(k & 0xF00 == B.KIND_COPY for k in kinds[30:])
        assert all(lo[i] == 0 and hi[i] == 2 * 12288 * 4096 for i in range(30, n3))
    finally:
        B.ar_plan_destroy(p3)
        B.ar_plan_destroy(p2)


def test_piece_blocks_follow_round_sizes():
    """Rabenseifner's rounds halve and then double: at 16 x 192 MiB fp32 the
    first halving round writes 1.6 GB, so the halving rounds and the fused
    first doubling round run in 6 pieces (4 launches each), then the doubling
    rounds whose outputs exceed the cache (0.4, 0.8 GB) in 3 pieces, each
    with the round that reads its output; the bytes do not change."""
    p = _plan(16, 1, 12288 * 4096, "fp32", "rabenseifner")
    try:
        assert B.ar_plan_num_launches(p) == 6 * 4 + 3 * 3
        assert B.ar_plan_stats(p)["hbm_bytes_model"] == (5 * 16 - 6) * 4 * 12288 * 4096
        B.ar_plan_set_cache_bytes(p, 1 << 40)
        assert B.ar_plan_num_launches(p) == 7
    finally:
        B.ar_plan_destroy(p)


def test_profiling_period_is_checked_on_the_host():
    p = B.ar_plan_create(4, 1, 1024, "fp32", "ring")
    try:
        B.ar_plan_set_profiling_period(p, 5)
        with pytest.raises(B.ArError) as ei:
            B.ar_plan_set_profiling_period(p, 0)
        assert ei.value.status == B.AR_ERR_INVALID_ARG
    finally:
        B.ar_plan_destroy(p)
