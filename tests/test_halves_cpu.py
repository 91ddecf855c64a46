"""The library's reduce-scatter and all-gather plans against the oracle (no GPU).

Owned ranges, transfers, statistics, and the launch lists run by the numpy
interpreter (every element, bit for bit), plus the calls' refusals.  The
oracle's halves themselves are pinned in test_oracle_halves.py.
"""
import numpy as np
import pytest

import oracle
from gradient_all_reduce_ar_amd import _binding as B
from tests import plan_interp
from tests.test_oracle_halves import CASES, _bits, _half_messages, _inputs, part


def _coll_plan(n, g, count, dtype, sched, coll):
    return B.ar_plan_create_collective(n, g, count, dtype, sched, coll)


@pytest.mark.parametrize("sched,n,g", CASES)
def test_plan_owned_ranges_equal_oracle(sched, n, g):
    for count in (0, 1, n + 1, 1031):
        want = oracle.owned_ranges(n, count, sched, group_size=g)
        for coll in ("allreduce", "reduce_scatter", "allgather"):
            p = _coll_plan(n, g, count, "fp32", sched, coll)
            try:
                assert [B.ar_plan_owned_range(p, r) for r in range(n)] == want
            finally:
                B.ar_plan_destroy(p)


def _sorted(d):
    order = np.lexsort((d["src"], d["step"]))
    return {k: v[order] for k, v in d.items()}


@pytest.mark.parametrize("sched,n,g", CASES)
def test_plan_halves_transfers_and_stats_equal_oracle(sched, n, g):
    for count in (0, 1, 97, 4096):
        k, rs, ag = _half_messages(n, count, sched, g)
        total = oracle.steps(n, sched, count, group_size=g)
        whole = _coll_plan(n, g, count, "fp32", sched, "allreduce")
        try:
            cost_whole = B.ar_plan_cost_alpha_beta(whole, 1e-6, 400e9, 50e9)
        finally:
            B.ar_plan_destroy(whole)
        cost = 0.0
        for coll, ref, rounds in (("reduce_scatter", rs, k), ("allgather", ag, total - k)):
            p = _coll_plan(n, g, count, "fp32", sched, coll)
            try:
                mine = _sorted(B.ar_plan_transfers(p))
                ref = _sorted(ref)
                for key in ("step", "src", "dst", "lo", "hi", "kind"):
                    np.testing.assert_array_equal(mine[key], ref[key], err_msg=f"{sched} n={n} {coll} {key}")
                st = B.ar_plan_stats(p)
                assert st["steps"] == rounds
                sent = np.bincount(ref["src"], weights=(ref["hi"] - ref["lo"]) * 4, minlength=n).astype(np.int64)
                assert st["bytes_sent"] == sent.tolist()
                cost += B.ar_plan_cost_alpha_beta(p, 1e-6, 400e9, 50e9)
            finally:
                B.ar_plan_destroy(p)
        assert cost == pytest.approx(cost_whole, rel=1e-12)  # the rounds split between the halves


def onepass_reduce_scatter_expected(xs, dtype, sched, g):
    """The one-pass reduce-scatter: the oracle's values on each owned range,
    every other element as it was (no partial sum is ever stored)."""
    rs = oracle.reduce_scatter([x.copy() for x in xs], dtype, sched, group_size=g)
    out = [x.copy() for x in xs]
    for r, (lo, hi) in enumerate(oracle.owned_ranges(len(xs), len(xs[0]), sched, group_size=g)):
        out[r][lo:hi] = rs[r][lo:hi]
    return out


@pytest.mark.parametrize("sched,n,g", CASES)
@pytest.mark.parametrize("dtype", ["fp32", "bf16", "bf16_each"])
@pytest.mark.parametrize("mode", ["steps", "steps_unfused", "onepass"])
def test_plan_halves_launch_lists_equal_oracle(sched, n, g, dtype, mode):
    """Reduce-scatter and all-gather launch lists, run by the interpreter,
    give the oracle's halves bit for bit in every element, with a cache that
    splits every round into pieces and with one that splits none.  The
    one-pass reduce-scatter leaves the elements outside the owned ranges
    untouched."""
    for count in (0, 37, 1031):
        xs = _inputs(n, count, dtype, seed=count + 11 * n)
        want_rs = (onepass_reduce_scatter_expected(xs, dtype, sched, g) if mode == "onepass" else
                   oracle.reduce_scatter([x.copy() for x in xs], dtype, sched, group_size=g))
        want_ag = oracle.allgather([x.copy() for x in xs], dtype, sched, group_size=g)
        for cache in (64, 1 << 30):
            for coll, want in (("reduce_scatter", want_rs), ("allgather", want_ag)):
                p = _coll_plan(n, g, count, dtype, sched, coll)
                try:
                    B.ar_plan_set_exec(p, mode)
                    B.ar_plan_set_cache_bytes(p, cache)
                    got = plan_interp.run(p, [x.copy() for x in xs], dtype, g)
                finally:
                    B.ar_plan_destroy(p)
                for r in range(n):
                    np.testing.assert_array_equal(_bits(got[r], dtype), _bits(want[r], dtype),
                                                  err_msg=f"{sched} n={n} {dtype} {mode} {coll} cache={cache} r={r}")


def test_collective_plan_errors():
    for sched in ("recursive_doubling", "tree", "double_tree"):
        with pytest.raises(B.ArError) as e:
            _coll_plan(4, 1, 100, "fp32", sched, "reduce_scatter")
        assert e.value.status == B.AR_ERR_UNSUPPORTED
    with pytest.raises(B.ArError) as e:
        _coll_plan(4, 1, 1024, "int8_ef", "ring", "allgather")
    assert e.value.status == B.AR_ERR_UNSUPPORTED
    with pytest.raises(B.ArError) as e:
        _coll_plan(4, 1, 100, "fp32", "ring", 7)
    assert e.value.status == B.AR_ERR_INVALID_ARG
    rs = _coll_plan(4, 1, 100, "fp32", "ring", "reduce_scatter")
    ar = B.ar_plan_create(4, 1, 100, "fp32", "ring")
    tree = B.ar_plan_create(4, 1, 100, "fp32", "tree")
    try:
        # a plan runs only through the call of its own collective; these
        # refusals happen before any pointer is read or device call made
        lib = B.lib()
        assert lib.ar_allreduce(rs, None, None) == B.AR_ERR_INVALID_ARG
        assert lib.ar_allreduce_ef(rs, None, None, None) == B.AR_ERR_INVALID_ARG
        assert lib.ar_allreduce_noalloc(rs, None, None, None) == B.AR_ERR_INVALID_ARG
        assert lib.ar_allgather(rs, None, None) == B.AR_ERR_INVALID_ARG
        assert lib.ar_reduce_scatter(ar, None, None) == B.AR_ERR_INVALID_ARG
        # owned ranges: ranks outside the plan, schedules without halves
        with pytest.raises(B.ArError) as e:
            B.ar_plan_owned_range(rs, 4)
        assert e.value.status == B.AR_ERR_INVALID_ARG
        with pytest.raises(B.ArError) as e:
            B.ar_plan_owned_range(tree, 0)
        assert e.value.status == B.AR_ERR_UNSUPPORTED
        assert B.ar_plan_owned_range(ar, 0) == (25, 50)
    finally:
        for p in (rs, ar, tree):
            B.ar_plan_destroy(p)


@pytest.mark.parametrize("sched,n,g", [("ring", 16, 1), ("hierarchical", 16, 8), ("rabenseifner", 16, 1),
                                        ("ring", 3, 1), ("rabenseifner", 2, 1)])
def test_onepass_halves_shape_and_bytes(sched, n, g):
    """One launch each.  The reduce-scatter folds every owned range from all
    ranks and writes it to its owner only: (N + 1) * S model bytes; the
    all-gather copies each owned range from its owner to the N - 1 others:
    N * S."""
    count = 16 * 1000
    for coll, kinds, model in (("reduce_scatter", {0x300, 0x400, 0x500}, (n + 1) * count * 4),
                               ("allgather", {B.KIND_FAN}, n * count * 4)):
        p = _coll_plan(n, g, count, "fp32", sched, coll)
        try:
            B.ar_plan_set_exec(p, "onepass")
            assert B.ar_plan_num_launches(p) == 1
            kind, nops = B.ar_plan_launch_info(p, 0)
            assert kind & 0xF00 in kinds and nops == n
            ops = B.ar_plan_launch_ops(p, 0)
            owners = ops["o"] if coll == "reduce_scatter" else ops["a"]
            assert sorted(int(x) for x in owners) == list(range(n))
            for r, lo, hi in zip(owners, ops["lo"], ops["hi"]):
                assert B.ar_plan_owned_range(p, int(r)) == (int(lo), int(hi))
            assert B.ar_plan_stats(p)["hbm_bytes_model"] == model
        finally:
            B.ar_plan_destroy(p)


def test_int8_allreduce_owned_ranges_count_elements():
    """INT8 plans cut on 128-element blocks; the owned range is reported in
    elements, clipped to the buffer."""
    count = 1000  # 8 blocks, the last short
    p = B.ar_plan_create(4, 1, count, "int8_ef", "ring")
    try:
        got = [B.ar_plan_owned_range(p, r) for r in range(4)]
    finally:
        B.ar_plan_destroy(p)
    blocks = [part(8, 4, (r + 1) % 4) for r in range(4)]
    assert got == [(min(lo * 128, count), min(hi * 128, count)) for lo, hi in blocks]


def test_large_halves_describe_but_do_not_run():
    """Reduce-scatter and all-gather plans of more than 64 ranks give their
    transfers, owned ranges and statistics; running them is refused before
    any device call."""
    n, count = 256, 1 << 20
    for coll, call, rounds in (("reduce_scatter", B.ar_reduce_scatter, n - 1), ("allgather", B.ar_allgather, n - 1)):
        p = _coll_plan(n, 8, count, "fp32", "ring", coll)
        try:
            st = B.ar_plan_stats(p)
            assert st["steps"] == rounds and st["launches"] == 0
            assert st["bytes_sent"] == [(n - 1) * (count // n) * 4] * n
            assert [B.ar_plan_owned_range(p, r) for r in (0, n - 1)] == [part(count, n, 1), part(count, n, 0)]
            with pytest.raises(B.ArError) as ei:
                call(p, [1 << 20] * n)
            assert ei.value.status == B.AR_ERR_UNSUPPORTED
        finally:
            B.ar_plan_destroy(p)


def test_random_halves_launch_lists():
    """Seeded draws (schedule, ranks up to 64, group, size, dtype, exec mode,
    assumed cache size, collective): the launch list, run by the interpreter,
    gives the oracle's half bit for bit in every element."""
    scheds = ["ring", "hierarchical", "rabenseifner"]
    for case in range(60):
        rng = np.random.default_rng([13, case])
        sched = scheds[rng.integers(3)]
        if sched == "rabenseifner":
            n, g = int(2 ** rng.integers(0, 7)), 1
        else:
            n = int(rng.integers(1, 65))
            divisors = [d for d in range(1, n + 1) if n % d == 0]
            g = int(divisors[rng.integers(len(divisors))]) if sched == "hierarchical" else 1
        dtype = ["fp32", "bf16", "bf16_each"][rng.integers(3)]
        mode = ["steps", "steps_unfused", "onepass"][rng.integers(3)]
        coll = ["reduce_scatter", "allgather"][rng.integers(2)]
        count = int(rng.integers(0, 3000))
        cache = [None, 1 << 10, 1 << 14][rng.integers(3)]
        what = f"case {case}: {coll} {sched} n={n} g={g} {dtype} {mode} count={count} cache={cache}"
        xs = _inputs(n, count, dtype, seed=2000 + case)
        if coll == "allgather":
            want = oracle.allgather([x.copy() for x in xs], dtype, sched, group_size=g)
        elif mode == "onepass":
            want = onepass_reduce_scatter_expected(xs, dtype, sched, g)
        else:
            want = oracle.reduce_scatter([x.copy() for x in xs], dtype, sched, group_size=g)
        p = _coll_plan(n, g, count, dtype, sched, coll)
        try:
            B.ar_plan_set_exec(p, mode)
            if cache is not None:
                B.ar_plan_set_cache_bytes(p, cache)
            got = plan_interp.run(p, [x.copy() for x in xs], dtype, g)
        finally:
            B.ar_plan_destroy(p)
        for r in range(n):
            np.testing.assert_array_equal(_bits(got[r], dtype), _bits(want[r], dtype), err_msg=f"{what} r={r}")
