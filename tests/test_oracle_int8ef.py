"""Pins of the oracle's compressed all-reduce (blockwise INT8 + error feedback).

Source: "Collective communication" (Scaling ML systems, ch. 06), section
"Gradient compression": the INT8 quantizer (scale = max|g| / 127, codes =
round(g / scale), decoded as code * scale), "Blockwise quantization" (one
fp32 scale per block of b elements, maximum error half a block scale), and
"Definition: error feedback mechanism" (e_{t+1} = g_t + e_t - v_t, the
telescoping sum, the five-step threshold trace).

What pins what:
  * the page trace (golden fixture) -- the error-feedback update and its sign;
  * telescoping sum over K steps -- the residual carried, not dropped;
  * half-scale bound per block -- the scale, the rounding and the block size;
  * exactly representable cases -- the routing of every block by every
    schedule (a block held by one rank, identical blocks on every rank);
  * block-level brute force -- the order in which each schedule combines and
    re-quantizes partial sums, against the closed folds of tests/folds.py;
  * every rank ends with the same values.
"""
import os

import numpy as np
import pytest

import oracle
from tests import folds

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "error_feedback_trace.txt")
B = oracle.QBLOCK

SCHEDS = [("ring", n, 1) for n in (1, 2, 3, 4, 5)] + \
         [("hierarchical", n, g) for n, g in ((4, 2), (6, 3), (6, 2), (8, 4))] + \
         [("rabenseifner", n, 1) for n in (2, 4, 8)] + \
         [("recursive_doubling", n, 1) for n in (2, 4, 8)] + \
         [("tree", n, 1) for n in (2, 3, 5, 8)] + \
         [("double_tree", n, 1) for n in (2, 4, 8)]


def _golden():
    for line in open(GOLDEN):
        if line.strip() and not line.startswith("#"):
            k, g, naive, ef, resid, true = line.split()
            return int(k), float(g), float(naive), float(ef), float(resid), float(true)


def test_block_size_reading():
    assert B == 128


def test_page_error_feedback_trace():
    """Scale forced to 1 (the block's largest entry is 127), so rounding to
    the nearest code is the page's threshold-0.5 unit compressor."""
    k, g, naive_want, ef_want, resid_want, true_want = _golden()
    grad = np.zeros(B, np.float32)
    grad[0] = 127.0
    grad[1] = g
    e = np.zeros(B, np.float32)
    naive = ef = 0.0
    for _ in range(k):
        b = [grad.copy()]
        oracle.run_int8ef(b, "ring")
        naive += float(b[0][1])
        b = [grad.copy()]
        oracle.run_int8ef(b, "ring", errs=[e])
        ef += float(b[0][1])
        assert b[0][0] == 127.0
    assert naive == naive_want
    assert ef == ef_want
    assert e[1] == pytest.approx(resid_want, abs=1e-6)
    assert k * g == pytest.approx(true_want)
    assert ef + float(e[1]) == pytest.approx(true_want, abs=1e-6)


def test_telescoping_sum():
    """sum_t v_t = sum_t g_t + e_1 - e_{K+1} for one worker over K steps."""
    rng = np.random.default_rng(3)
    count, steps = 5 * B + 37, 25
    e = (rng.standard_normal(count) * 0.01).astype(np.float32)
    e1 = e.copy()
    sent = np.zeros(count, np.float64)
    total = np.zeros(count, np.float64)
    for _ in range(steps):
        g = (rng.standard_normal(count) * np.exp(rng.standard_normal(count))).astype(np.float32)
        total += g
        b = [g.copy()]
        oracle.run_int8ef(b, "ring", errs=[e])
        sent += b[0]
    scale = np.abs(total).max()
    np.testing.assert_allclose(sent, total + e1 - e, rtol=0, atol=1e-5 * scale)


def test_half_scale_bound_per_block():
    """One rank: the result is the round trip of g + e and the new residual
    stays within half the block's own scale (blocks of very different
    magnitude keep their own precision)."""
    rng = np.random.default_rng(5)
    count = 7 * B + 55
    mags = np.repeat(10.0 ** rng.integers(-6, 4, size=8), B)[:count]
    g = (rng.standard_normal(count) * mags).astype(np.float32)
    e = (rng.standard_normal(count) * mags * 1e-3).astype(np.float32)
    x = (g + e).astype(np.float32)
    b = [g.copy()]
    oracle.run_int8ef(b, "ring", errs=[e])
    for blk in range(0, count, B):
        xs = x[blk:blk + B]
        s = np.abs(xs).max() / 127.0
        err = np.abs(b[0][blk:blk + B] - xs)
        assert err.max() <= 0.5 * s * (1 + 1e-5) + 1e-30, blk
        np.testing.assert_array_equal(e[blk:blk + B], (xs - b[0][blk:blk + B]).astype(np.float32))


def test_block_boundary_is_128():
    """A block's scale is set by its own largest entry only: small values in
    the same 128-block as a 127 round to 0, in the next block they survive."""
    g = np.zeros(2 * B, np.float32)
    g[0] = 127.0
    g[64:B] = 0.3
    g[B:] = 0.3
    b = [g.copy()]
    oracle.run_int8ef(b, "ring")
    assert np.all(b[0][64:B] == 0)
    np.testing.assert_allclose(b[0][B:], 0.3, rtol=1e-6)


def test_ties_round_to_even():
    g = np.zeros(B, np.float32)
    g[0] = 127.0
    g[1:7] = [2.5, 3.5, -2.5, -3.5, 0.5, -0.5]
    b = [g.copy()]
    oracle.run_int8ef(b, "ring")
    np.testing.assert_array_equal(b[0][1:7], [2, 4, -2, -4, 0, -0.0])


def test_zero_block_and_empty():
    b = [np.zeros(3 * B, np.float32) for _ in range(4)]
    e = [np.zeros(3 * B, np.float32) for _ in range(4)]
    oracle.run_int8ef(b, "ring", errs=e)
    for r in range(4):
        assert not np.any(b[r]) and not np.any(e[r])
    oracle.run_int8ef([np.zeros(0, np.float32)] * 2, "ring")


def _owner_inputs(n, count, seed):
    """Integer data in [-127, 127]; block k is non-zero on rank k mod n only
    and holds a +-127, so every quantization on its path is exact."""
    rng = np.random.default_rng(seed)
    xs = [np.zeros(count, np.float32) for _ in range(n)]
    for k, lo in enumerate(range(0, count, B)):
        hi = min(count, lo + B)
        v = rng.integers(-127, 128, size=hi - lo).astype(np.float32)
        v[rng.integers(0, hi - lo)] = 127.0 * rng.choice([-1, 1])
        xs[k % n][lo:hi] = v
    return xs


@pytest.mark.parametrize("schedule,n,g", SCHEDS)
def test_exact_when_one_rank_holds_each_block(schedule, n, g):
    for count in (1, B - 1, B, 3 * B + 1, 11 * B + 77):
        xs = _owner_inputs(n, count, seed=count)
        want = np.sum(xs, axis=0, dtype=np.float64).astype(np.float32)
        bufs = [x.copy() for x in xs]
        oracle.run_int8ef(bufs, schedule, group_size=g)
        for r in range(n):
            np.testing.assert_array_equal(bufs[r], want, err_msg=f"{schedule} n={n} count={count} rank={r}")


@pytest.mark.parametrize("schedule,n,g", SCHEDS)
def test_exact_for_identical_blocks(schedule, n, g):
    """Every rank holds the same integer blocks with a +-127 each: any
    partial sum of k ranks is k times the block, its scale k, its codes the
    block itself, so the result is exactly n times the input."""
    count = 9 * B + 3
    x = _owner_inputs(1, count, seed=n)[0]
    bufs = [x.copy() for _ in range(n)]
    oracle.run_int8ef(bufs, schedule, group_size=g)
    for r in range(n):
        np.testing.assert_array_equal(bufs[r], np.float32(n) * x)


@pytest.mark.parametrize("schedule,n,g", SCHEDS)
def test_matches_block_level_closed_form(schedule, n, g):
    rng = np.random.default_rng(n * 10 + g)
    for count in (B + 5, 4 * B, 6 * B + 100):
        xs = [(rng.standard_normal(count) * np.exp(rng.standard_normal(count))).astype(np.float32)
              for _ in range(n)]
        es = [(rng.standard_normal(count) * 1e-2).astype(np.float32) for _ in range(n)]
        want, want_e = folds.expected_int8ef(xs, schedule, es, g)
        bufs = [x.copy() for x in xs]
        errs = [e.copy() for e in es]
        oracle.run_int8ef(bufs, schedule, errs=errs, group_size=g)
        for r in range(n):
            # bit patterns: a decoded zero code is +0 on both sides
            np.testing.assert_array_equal(bufs[r].view(np.uint32), want.view(np.uint32),
                                          err_msg=f"{schedule} n={n} count={count} rank={r}")
            np.testing.assert_array_equal(errs[r].view(np.uint32), want_e[r].view(np.uint32))


@pytest.mark.parametrize("schedule,n,g", SCHEDS)
def test_error_bound_against_exact_sum(schedule, n, g):
    """Each of the 2n-1 quantizations on an element's path (n leaves, n-1
    partial sums) moves it by at most half a block scale, and no partial sum
    exceeds sum_r max|block_r| (1 + small), so
    |result - sum| <= (2n-1) * sum_r max|block_r| / 254 * 1.01."""
    rng = np.random.default_rng(17 + n)
    count = 8 * B + 19
    xs = [rng.standard_normal(count).astype(np.float32) for _ in range(n)]
    exact = np.sum(xs, axis=0, dtype=np.float64)
    bufs = [x.copy() for x in xs]
    oracle.run_int8ef(bufs, schedule, group_size=g)
    for lo in range(0, count, B):
        m = sum(np.abs(x[lo:lo + B]).max() for x in xs)
        bound = (2 * n - 1) * m / 254.0 * 1.01
        assert np.abs(bufs[0][lo:lo + B] - exact[lo:lo + B]).max() <= bound
    for r in range(n):
        np.testing.assert_array_equal(bufs[r], bufs[0])
