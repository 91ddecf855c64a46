"""Launch shapes of the one-pass folds, on the CPU (no kernel runs).

From 4 ranks up the fp32 and bf16 one-pass folds are LDS-staged: a
workgroup of min(N, W) waves (W = 16 for fp32, and for bf16 rounded once
outside the balanced tree, up to 16 ranks; 8 otherwise) stages U 16-byte
units per lane of every rank (U = 2 up to 32 ranks, 1 above), N * U KiB of
LDS, and stores with sc1 when the launch's output fits in the assumed
256 MiB cache, nt + sc1 otherwise.  2 and 3 ranks and the INT8 folds keep
the register kernels (no LDS)."""
import pytest

from gradient_all_reduce_ar_amd import _binding as B


def _shape(n, count, dtype, sched, g=1, cache=None):
    p = B.ar_plan_create(n, g, count, dtype, sched)
    try:
        B.ar_plan_set_exec(p, "onepass")
        if cache is not None:
            B.ar_plan_set_cache_bytes(p, cache)
        assert B.ar_plan_num_launches(p) == 1
        return B.ar_plan_launch_shape(p, 0)
    finally:
        B.ar_plan_destroy(p)


@pytest.mark.parametrize("n,dtype,sched,g,threads,units,waves", [
    (16, "fp32", "ring", 1, 1024, 2, 16),
    (16, "bf16", "ring", 1, 1024, 2, 16),
    (16, "bf16_each", "ring", 1, 512, 2, 8),
    (16, "fp32", "hierarchical", 8, 1024, 2, 16),
    (16, "fp32", "rabenseifner", 1, 1024, 2, 16),
    (16, "bf16", "rabenseifner", 1, 512, 2, 8),   # the bf16 balanced tree: 8 waves
    (16, "bf16", "double_tree", 1, 1024, 2, 16),
    (8, "fp32", "ring", 1, 512, 2, 16),            # min(N, 16) waves
    (5, "bf16", "tree", 1, 320, 2, 8),
    (4, "fp32", "ring", 1, 256, 2, 16),
    (32, "fp32", "ring", 1, 512, 2, 8),
    (48, "bf16", "ring", 1, 512, 1, 8),
    (64, "fp32", "rabenseifner", 1, 512, 1, 8),
])
def test_lds_staged_shapes(n, dtype, sched, g, threads, units, waves):
    es = 4 if dtype == "fp32" else 2
    sh = _shape(n, (1 << 20) // es, dtype, sched, g)  # 1 MiB per rank: fits the cache
    assert sh["threads"] == threads
    assert sh["units"] == units
    assert sh["batch"] == waves
    assert sh["lds_bytes"] == n * units * 1024
    assert sh["cpol"] == 16 and sh["cold"] == 0


def test_store_policy_follows_the_cache():
    """N * S above the assumed cache: nt + sc1; within it: sc1."""
    n = 16
    big = _shape(n, 32 << 18, "fp32", "ring")  # 32 MiB per rank: 512 MiB in all
    assert big["cold"] == 1 and big["cpol"] == 18
    small = _shape(n, 4 << 18, "fp32", "ring")  # 4 MiB per rank: 64 MiB
    assert small["cold"] == 0 and small["cpol"] == 16
    shrunk = _shape(n, 4 << 18, "fp32", "ring", cache=32 << 20)
    assert shrunk["cold"] == 1 and shrunk["cpol"] == 18


@pytest.mark.parametrize("n,dtype,sched", [(2, "fp32", "ring"), (3, "bf16", "tree"), (2, "bf16_each", "double_tree"),
                                           (16, "int8_ef", "ring"), (64, "int8_ef", "rabenseifner")])
def test_register_folds_elsewhere(n, dtype, sched):
    es = 4 if dtype in ("fp32", "int8_ef") else 2
    sh = _shape(n, (1 << 20) // es, dtype, sched)
    assert sh["lds_bytes"] == 0


def test_grid_covers_every_tile():
    """One tile (64 * U * 4 fp32 elements) per workgroup along x, one op per
    chunk along y; a ragged count adds one workgroup for the cut tile."""
    n, count = 16, 16 * 512 * 7 + 3
    p = B.ar_plan_create(n, 1, count, "fp32", "ring")
    try:
        B.ar_plan_set_exec(p, "onepass")
        sh = B.ar_plan_launch_shape(p, 0)
        kind, nops = B.ar_plan_launch_info(p, 0)
        assert nops == n
        ops = B.ar_plan_launch_ops(p, 0)
        tile = 64 * sh["units"] * 4
        need = max((hi + tile - 1) // tile - lo // tile for lo, hi in zip(ops["lo"], ops["hi"]))
        assert sh["grid_x"] == need
    finally:
        B.ar_plan_destroy(p)


def _rs_shape(n, count, dtype, sched, g=1):
    p = B.ar_plan_create_collective(n, g, count, dtype, sched, "reduce_scatter")
    try:
        B.ar_plan_set_exec(p, "onepass")
        assert B.ar_plan_num_launches(p) == 1
        kind, _ = B.ar_plan_launch_info(p, 0)
        return kind, B.ar_plan_launch_shape(p, 0), B.ar_plan_launch_ops(p, 0)
    finally:
        B.ar_plan_destroy(p)


@pytest.mark.parametrize("n,dtype,sched,g,waves,units", [
    (16, "fp32", "ring", 1, 16, 4), (16, "bf16", "ring", 1, 16, 4), (16, "fp32", "hierarchical", 8, 16, 4),
    (12, "bf16", "hierarchical", 3, 16, 4), (16, "fp32", "rabenseifner", 1, 16, 4), (9, "fp32", "ring", 1, 16, 4),
    (16, "bf16_each", "ring", 1, 8, 2),      # 8-wave workgroups keep the class's tiles
    (16, "bf16", "rabenseifner", 1, 8, 2),   # (the bf16 balanced tree: 8 waves)
    (8, "fp32", "ring", 1, 16, 2), (4, "fp32", "ring", 1, 16, 2),  # 8 ranks and fewer too
])
def test_reduce_scatter_tiles(n, dtype, sched, g, waves, units):
    """A one-pass reduce-scatter carries the owner flag; from 9 to 16 ranks
    in 16-wave workgroups it stages 4 units per lane and rank (N * 4 KiB of
    LDS).  Its stores take sc1, or nt + sc1 where its output (one rank's
    size: the owned ranges) overflows the assumed 256 MiB cache.  The grid
    covers every tile of the owned ranges."""
    es = 4 if dtype == "fp32" else 2
    for count, cold in (((1 << 20) // es, 0), ((512 << 20) // es, 1)):  # 1 or 512 MiB per rank
        kind, sh, ops = _rs_shape(n, count, dtype, sched, g)
        assert kind & B.KIND_OWNER
        assert sh["units"] == units and sh["lds_bytes"] == n * units * 1024
        assert sh["batch"] == waves and sh["threads"] == 64 * min(n, waves)
        assert sh["cpol"] == (18 if cold else 16) and sh["cold"] == cold
        tile = 64 * units * (4 if dtype == "fp32" else 8)
        assert sh["grid_x"] == max((hi + tile - 1) // tile - lo // tile for lo, hi in zip(ops["lo"], ops["hi"]))


def test_reduce_scatter_above_16_ranks_keeps_the_class_tiles():
    """Above 16 ranks the reduce-scatter fold stages what the all-reduce's
    size class does (2 units up to 32 ranks, 1 above)."""
    for n, units in ((32, 2), (64, 1)):
        kind, sh, _ = _rs_shape(n, 1 << 18, "fp32", "ring")
        assert kind & B.KIND_OWNER
        assert sh["units"] == units and sh["lds_bytes"] == n * units * 1024


def test_allreduce_and_allgather_carry_no_owner_flag():
    for coll in ("allreduce", "allgather"):
        p = B.ar_plan_create_collective(16, 1, 1 << 18, "fp32", "ring", coll)
        try:
            B.ar_plan_set_exec(p, "onepass")
            kind, _ = B.ar_plan_launch_info(p, 0)
            assert not kind & B.KIND_OWNER
        finally:
            B.ar_plan_destroy(p)


@pytest.mark.parametrize("n,dtype,waves,groups", [
    (16, "fp32", 16, 1), (16, "bf16", 16, 1), (8, "fp32", 8, 1), (2, "bf16", 2, 1),
    (17, "fp32", 16, 2), (32, "fp32", 16, 2), (48, "bf16", 16, 3), (64, "bf16", 16, 4),
])
def test_allgather_fan_tiles(n, dtype, waves, groups):
    """The one-pass all-gather stages 4 KiB of the owner per workgroup, each
    wave storing it into one rank; above 16 ranks the destinations split into
    groups of 16, one workgroup per group and tile, so the grid covers every
    tile of the owned ranges that many times."""
    es = 4 if dtype == "fp32" else 2
    count = (3 << 20) // es + 5
    p = B.ar_plan_create_collective(n, 1, count, dtype, "ring", "allgather")
    try:
        B.ar_plan_set_exec(p, "onepass")
        kind, _ = B.ar_plan_launch_info(p, 0)
        assert kind == B.KIND_FAN | es
        sh = B.ar_plan_launch_shape(p, 0)
        ops = B.ar_plan_launch_ops(p, 0)
    finally:
        B.ar_plan_destroy(p)
    assert sh["units"] == 4 and sh["batch"] == waves and sh["threads"] == 64 * waves
    assert sh["cpol"] == 16 and sh["lds_bytes"] == 32768
    tile = 4 * 64 * (16 // es)
    tiles = max((hi + tile - 1) // tile - lo // tile for lo, hi in zip(ops["lo"], ops["hi"]))
    assert sh["grid_x"] == tiles * groups
