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
