"""The CPU oracle against what the pages print.

Every expected value here is transcribed from the pages (fixtures under
tests/golden/, each citing its source) or is a closed form the pages state.
"""
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
MiB = 1 << 20


def _rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]


def _chunk_index(lo, count, n):
    for c in range(n):
        if (c * count) // n == lo:
            return c
    raise AssertionError(lo)


# ---------------------------------------------------------------- ring ----

@pytest.mark.parametrize("schedule,group", [("ring", 1), ("ring", 2), ("hierarchical", 2),
                                            ("hierarchical", 4), ("hierarchical", 1),
                                            ("rabenseifner", 1)])
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_worked_example_four_gpus(schedule, group, dtype):
    """Scaling ML systems ch. 06, "Ring AllReduce: step-by-step trace (4 GPUs)":
    [1,5,3,7] + [2,6,4,8] + [3,7,5,9] + [4,8,6,10] = [10,26,18,34] on every
    rank.  All partial sums are small integers, so every schedule gets the
    exact sum in fp32 and in bf16."""
    rows = _rows("ring_worked_example_n4.txt")
    ins = [np.array(r[1:], np.float32) for r in rows if r[0] == "input"]
    want = np.array([r[1:] for r in rows if r[0] == "sum"][0], np.float32)
    if dtype == "fp32":
        bufs = [x.copy() for x in ins]
    else:
        bufs = [(x.view(np.uint32) >> 16).astype(np.uint16) for x in ins]  # exact: small ints
    oracle.run(bufs, dtype, schedule, group_size=group)
    for b in bufs:
        got = b if dtype == "fp32" else (b.astype(np.uint32) << 16).view(np.float32)
        np.testing.assert_array_equal(got, want)


def test_ring_send_table_n4():
    """Primer ch. 4, Figure 4.2: the chunk each rank sends in each of the six
    steps, (i - s) mod 4 in reduce-scatter and (i + 1 - s) mod 4 in all-gather."""
    m = oracle.messages(4, 4, "ring")
    for row in _rows("ring_send_table_n4.txt"):
        src, dst, chunks = int(row[0]), int(row[1]), [int(v) for v in row[2:]]
        for step, c in enumerate(chunks):
            sel = (m["step"] == step) & (m["src"] == src)
            assert sel.sum() == 1
            j = np.flatnonzero(sel)[0]
            assert m["dst"][j] == dst
            assert _chunk_index(m["lo"][j], 4, 4) == c
            assert m["kind"][j] == (oracle.REDUCE if step < 3 else oracle.COPY)


def test_ring_count_grids_n4():
    """Primer ch. 4, Figure 4.3: the per-(rank, chunk) count grids after each
    of the six steps.  All-ones fp32 input makes the buffers equal the counts."""
    rows = _rows("ring_count_grids_n4.txt")
    grids, k = {}, None
    for r in rows:
        if r[0] == "step":
            k = int(r[1])
            grids[k] = []
        else:
            grids[k].append([float(v) for v in r])
    assert sorted(grids) == list(range(7))
    for k, grid in grids.items():
        bufs = [np.ones(4, np.float32) for _ in range(4)]
        oracle.run(bufs, "fp32", "ring", max_steps=k)
        for rank in range(4):
            np.testing.assert_array_equal(bufs[rank], np.array(grid[rank], np.float32),
                                          err_msg=f"after step {k}, rank {rank}")


def test_ring_ownership_after_reduce_scatter():
    """Primer ch. 4, Figure 4.1: after the three reduce-scatter steps P0 owns
    segment 1, P1 segment 2, P2 segment 3, P3 segment 0; section 4.2 states
    the rule: rank i holds the complete chunk (i + 1) mod N."""
    for n in (4, 5, 8):
        bufs = [np.ones(n, np.float32) for _ in range(n)]
        oracle.run(bufs, "fp32", "ring", max_steps=n - 1)
        for i in range(n):
            assert np.flatnonzero(bufs[i] == n).tolist() == [(i + 1) % n]
    bufs = [np.ones(4, np.float32) for _ in range(4)]
    oracle.run(bufs, "fp32", "ring", max_steps=3)
    assert [int(np.flatnonzero(b == 4)[0]) for b in bufs] == [1, 2, 3, 0]


def test_ring_partial_count_rule():
    """Primer ch. 4, section 4.2: after reduce-scatter step s the chunk rank i
    has just received holds the contributions of s + 2 ranks."""
    n = 6
    m = oracle.messages(n, n, "ring")
    for s in range(n - 1):
        bufs = [np.ones(n, np.float32) for _ in range(n)]
        oracle.run(bufs, "fp32", "ring", max_steps=s + 1)
        sel = m["step"] == s
        for j in np.flatnonzero(sel):
            assert bufs[m["dst"][j]][m["lo"][j]] == s + 2


def test_ring_bytes_and_steps():
    """Ring sends 2(N-1)/N * S per rank in 2(N-1) steps (Primer ch. 4,
    section 4.2; Data-center networks 7.2.1).  For the 16-rank, 192 MiB
    fp32 gradient: 360 MiB per rank, 5760 MiB in total, 30 rounds."""
    count = 12288 * 4096
    sent, cross, steps = oracle.stats(16, count, "fp32", "ring", group_size=8)
    assert steps == 30
    assert all(int(b) == 360 * MiB for b in sent)
    assert int(sent.sum()) == 5760 * MiB
    # contiguous placement on two servers: only 7->8 and 15->0 cross, 360 MiB
    # each, 720 MiB in total (Data-center networks 7.2.1, problem 7.2)
    assert cross == 720 * MiB
    for n in (2, 3, 4, 8, 64):
        e = n * 1000
        sent, _, steps = oracle.stats(n, e, "fp32", "ring")
        assert steps == 2 * (n - 1)
        assert all(int(b) == 2 * (n - 1) * (e // n) * 4 for b in sent)


def test_hierarchical_bytes_and_steps():
    """Data-center networks 7.2.1: 2 servers x 8 ranks, 192 MiB: 7 + 2 + 7 = 16
    rounds; per rank 336 MiB over the local links and 24 MiB across servers;
    384 MiB crosses between servers in total.  Primer ch. 4 section 4.4,
    Animation 4.3: (G-1)/G*S per intra phase and 2(M-1)/M*S/G across."""
    count = 12288 * 4096
    sent, cross, steps = oracle.stats(16, count, "fp32", "hierarchical", group_size=8)
    assert steps == 16
    assert all(int(b) == 360 * MiB for b in sent)
    assert cross == 384 * MiB
    m = oracle.messages(16, count, "hierarchical", group_size=8)
    for r in range(16):
        mine = m["src"] == r
        crossing = (m["src"] // 8) != (m["dst"] // 8)
        local_b = int(((m["hi"] - m["lo"])[mine & ~crossing]).sum()) * 4
        cross_b = int(((m["hi"] - m["lo"])[mine & crossing]).sum()) * 4
        assert local_b == 336 * MiB and cross_b == 24 * MiB
    for n, g in ((8, 4), (16, 4), (32, 8), (64, 8)):
        mg = n // g
        e = n * g * 64
        sent, _, steps = oracle.stats(n, e, "fp32", "hierarchical", group_size=g)
        assert steps == 2 * (g - 1) + 2 * (mg - 1)
        want = (2 * (g - 1) * (e // g) + 2 * (mg - 1) * (e // g // mg)) * 4
        assert all(int(b) == want for b in sent)


def test_hierarchical_slice_ownership():
    """Primer ch. 4, Animation 4.3: the slice order is chosen so that GPU k
    ends phase 1 owning slice k; Figure 4.8: only slice k of GPU k leaves the
    server, and only to GPU k of the other server."""
    n, g = 16, 8
    e = 64
    bufs = [np.ones(e, np.float32) for _ in range(n)]
    oracle.run(bufs, "fp32", "hierarchical", group_size=g, max_steps=g - 1)
    for r in range(n):
        k = r % g
        lo, hi = (k * e) // g, ((k + 1) * e) // g
        assert np.all(bufs[r][lo:hi] == g)
        assert np.all(np.delete(bufs[r], np.arange(lo, hi)) < g)
    m = oracle.messages(n, e, "hierarchical", group_size=g)
    crossing = (m["src"] // g) != (m["dst"] // g)
    for j in np.flatnonzero(crossing):
        k = m["src"][j] % g
        assert m["dst"][j] % g == k
        assert (k * e) // g <= m["lo"][j] and m["hi"][j] <= ((k + 1) * e) // g


def test_rabenseifner_pairs_n8():
    """Scaling ML systems ch. 06, "Recursive halving and doubling": round-k
    partners i xor 2^k; (0,1)(2,3)(4,5)(6,7), then (0,2)(1,3)(4,6)(5,7), ...
    The all-gather runs the same pairs in reverse order (Primer Animation 4.2)."""
    m = oracle.messages(8, 64, "rabenseifner")
    assert oracle.steps(8, "rabenseifner") == 6
    for row in _rows("rabenseifner_pairs_n8.txt"):
        k = int(row[1])
        pairs = {tuple(sorted(map(int, p.split("-")))) for p in row[2:]}
        for step in (k, 5 - k):
            sel = m["step"] == step
            got = {tuple(sorted((int(a), int(b)))) for a, b in zip(m["src"][sel], m["dst"][sel])}
            assert got == pairs
            assert sel.sum() == 8  # both directions of every pair


def test_rabenseifner_ownership_bit_reversal():
    """Primer ch. 4, Animation 4.2: rank i ends the reduce-scatter owning the
    chunk whose index is i with its bits reversed (rank 1 owns chunk E, index
    4, when N = 8); Figure 4.5: counts 1, 2, 4, 8 after each round."""
    def bitrev(i, bits):
        return int(format(i, f"0{bits}b")[::-1], 2) if bits else 0

    for n in (2, 4, 8, 16):
        L = n.bit_length() - 1
        for k in range(L + 1):
            bufs = [np.ones(n, np.float32) for _ in range(n)]
            oracle.run(bufs, "fp32", "rabenseifner", max_steps=k)
            for i in range(n):
                assert bufs[i].max() == 2 ** k
                assert (bufs[i] == 2 ** k).sum() == n >> k
        for i in range(n):
            assert np.flatnonzero(bufs[i] == n).tolist() == [bitrev(i, L)]
    bufs = [np.ones(8, np.float32) for _ in range(8)]
    oracle.run(bufs, "fp32", "rabenseifner", max_steps=3)
    assert int(np.flatnonzero(bufs[1] == 8)[0]) == ord("E") - ord("A")


def test_rabenseifner_bytes_and_steps():
    """Primer ch. 4 section 4.3 and Figure 4.5: 2 log2 N steps; the halving
    reduce-scatter sends 7/8 S on 8 ranks; in total 2(N-1)/N * S per rank."""
    for n in (2, 4, 8, 16, 64):
        e = n * 96
        sent, _, steps = oracle.stats(n, e, "fp32", "rabenseifner")
        assert steps == 2 * (n.bit_length() - 1)
        assert all(int(b) == 2 * (n - 1) * (e // n) * 4 for b in sent)
    m = oracle.messages(8, 8 * 96, "rabenseifner")
    rs = m["kind"] == oracle.REDUCE
    for r in range(8):
        assert int(((m["hi"] - m["lo"])[rs & (m["src"] == r)]).sum()) == 7 * 96
    with pytest.raises(oracle.OracleError):
        oracle.steps(12, "rabenseifner")


def test_every_step_moves_each_chunk_once():
    """Primer ch. 4, Figure 4.2: each column of the send table holds every
    chunk once, so no two transfers of a step touch the same range."""
    for sched, n, g in (("ring", 7, 1), ("hierarchical", 8, 4), ("rabenseifner", 8, 1)):
        m = oracle.messages(n, 840, sched, group_size=g)
        for s in np.unique(m["step"]):
            sel = np.flatnonzero(m["step"] == s)
            written = {}
            for j in sel:
                d = int(m["dst"][j])
                for (lo, hi) in written.get(d, []):
                    assert m["hi"][j] <= lo or hi <= m["lo"][j]
                written.setdefault(d, []).append((int(m["lo"][j]), int(m["hi"][j])))


def test_alpha_beta_times_printed_on_pages():
    """The analytic times of Data-center networks 7.2.1 / 7.6.3 and of
    Scaling ML systems ch. 06 (fixture alpha_beta_pages.txt)."""
    for row in _rows("alpha_beta_pages.txt"):
        name, sched = row[0], row[1]
        n, g, nbytes, eb = (int(v) for v in row[2:6])
        alpha_us, bwi, bwc, want_ms, tol = (float(v) for v in row[6:11])
        t = oracle.cost(n, nbytes // eb, eb, sched, alpha_us * 1e-6, bwi * 1e9, bwc * 1e9,
                        group_size=g)
        assert abs(t * 1e3 - want_ms) <= tol * want_ms, (name, t * 1e3, want_ms)


def test_ring_lower_bound_matches():
    """Scaling ML systems ch. 06, "bandwidth-optimal lower bound":
    T_min = 2(N-1)/N * M / beta; the ring reaches it exactly when alpha = 0."""
    for n in (2, 4, 16):
        e = n * 4096
        t = oracle.cost(n, e, 4, "ring", 0.0, 1e9, 1e9)
        assert t == pytest.approx(2 * (n - 1) / n * e * 4 / 1e9, rel=1e-12)
        t = oracle.cost(n, e, 4, "rabenseifner", 0.0, 1e9, 1e9)
        assert t == pytest.approx(2 * (n - 1) / n * e * 4 / 1e9, rel=1e-12)


def test_hierarchical_gradient_time_and_egress_bytes():
    """Data-center networks 7.6.4 (fixture hierarchical_grad_pages.txt): the
    per-supernode cross bytes V_out = 2 (H-1)/H * 8G and the hierarchical
    gradient time T_grad = 2(q-1)a_L + 2(q-1)G/(q B_L) + 2(H-1)a_R
    + max(2(H-1)G/(H q B_NIC), V_out/B_out) for the printed supernode sizes."""
    G = 8e9  # bytes per GPU shard (bf16)
    for row in _rows("hierarchical_grad_pages.txt"):
        S, q, H = int(row[0]), int(row[1]), int(row[2])
        vout_gb, egress, want_ms, tol = float(row[3]), float(row[4]), float(row[5]), float(row[6])
        n = q * H
        count = int(G) // 2
        _, cross, _ = oracle.stats(n, count, "bf16", "hierarchical", group_size=q)
        # one DP instance's cross bytes per supernode, times 8 TP coordinates
        assert cross / H * 8 == pytest.approx(vout_gb * 1e9, rel=1e-9)
        t = oracle.cost_ex(n, count, 2, "hierarchical", 0.83e-6, 0.83e-6, 450e9, 50e9, egress * 1e9, 8.0,
                           group_size=q)
        assert t * 1e3 == pytest.approx(want_ms, rel=tol), (S, t * 1e3)
    # the cross-domain term for S = 128 is about 17.5 ms, and 52.5 ms when
    # 3:1 oversubscription cuts the egress to a third
    for egress, want in ((128 * 50e9, 17.5e-3), (128 * 50e9 / 3, 52.5e-3)):
        q, H = 16, 8
        full = oracle.cost_ex(q * H, int(G) // 2, 2, "hierarchical", 0.0, 0.0, 450e9, 50e9, egress, 8.0, group_size=q)
        local_only = 2 * (q - 1) * G / (q * 450e9)
        assert full - local_only == pytest.approx(want, rel=0.01)


def test_latency_terms_for_1024_gpus():
    """Primer ch. 4 section 4.3 and Panel 4.3: 1,024 ranks and alpha = 22 us:
    the ring spends 2,046 x 22 us = 45 ms in latency; the doubling tree's 10
    steps take about 0.4 ms for a 1 MB message at 50 GB/s."""
    t = oracle.cost(1024, 0, 4, "ring", 22e-6, 50e9, 50e9)
    assert t == pytest.approx(2046 * 22e-6, rel=1e-12) and round(t * 1e3) == 45
    assert oracle.steps(1024, "ring") == 2046 and oracle.steps(1024, "rabenseifner") == 20



def test_double_tree_structure_n8():
    """Primer ch. 4, Figure 4.6: the reduce messages of the double binary
    tree follow the two printed trees; tree 1 carries the first half of the
    buffer and tree 2 (the mirror) the second; every node forwards in at most
    one tree."""
    m = oracle.messages(8, 64, "double_tree")
    up = m["kind"] == oracle.REDUCE
    got = {(1 if m["lo"][j] == 0 else 2, int(m["src"][j]), int(m["dst"][j])) for j in np.flatnonzero(up)}
    want = {tuple(int(v) for v in row) for row in _rows("double_tree_n8.txt")}
    assert got == want
    inner1 = {p for t, c, p in want if t == 1}
    inner2 = {p for t, c, p in want if t == 2}
    assert inner1 == {0, 2, 4, 6} and inner2 == {1, 3, 5, 7}
    assert oracle.steps(8, "double_tree") == 6


def test_tree_and_doubling_steps_and_bytes():
    """Scaling ML systems ch. 06 "Tree AllReduce": log2 N steps up and log2 N
    down, each carrying the whole message; Primer Figure 4.5: recursive
    doubling sends the whole buffer in each of its log2 N steps (3S for 8
    ranks), against 7S/8 for the halving reduce-scatter."""
    S = 8 * 1024
    assert oracle.steps(64, "tree") == 12 and oracle.steps(8, "recursive_doubling") == 3
    sent, _, _ = oracle.stats(8, S, "fp32", "recursive_doubling")
    assert all(int(b) == 3 * S * 4 for b in sent)
    m = oracle.messages(64, S, "tree")
    assert np.all(m["hi"] - m["lo"] == S)
    with pytest.raises(oracle.OracleError):
        oracle.steps(12, "recursive_doubling")


def test_tree_and_doubling_times_printed_on_pages():
    """Scaling ML systems ch. 06, "Ring-tree crossover" example: 1 MB on 64
    GPUs, alpha = 10 us, beta = 10 GB/s: ring 1456.9 us, tree 1320 us.
    Primer ch. 4, "Two worked examples": 1 MB on 8 GPUs at 450 GB/s with
    alpha = 5 us: ring about 74 us, doubling tree about 22 us; Panel 4.3:
    1 MB on 1,024 GPUs at 50 GB/s, alpha = 22 us: the tree about 0.4 ms."""
    mb = 1_000_000
    assert oracle.cost(64, mb // 4, 4, "ring", 10e-6, 10e9, 10e9) * 1e6 == pytest.approx(1456.9, abs=0.05)
    assert oracle.cost(64, mb // 4, 4, "tree", 10e-6, 10e9, 10e9) * 1e6 == pytest.approx(1320.0, rel=1e-9)
    assert round(oracle.cost(8, mb // 4, 4, "ring", 5e-6, 450e9, 450e9) * 1e6) == 74
    assert round(oracle.cost(8, mb // 4, 4, "recursive_doubling", 5e-6, 450e9, 450e9) * 1e6) == 22
    assert round(oracle.cost(1024, mb // 4, 4, "recursive_doubling", 22e-6, 50e9, 50e9) * 1e3, 1) == 0.4


def _crossover(n, sched_a, sched_b, alpha, bw, lo=1e3, hi=1e12):
    """Message size (bytes, multiple of 4 n) where the two modelled times meet."""
    f = lambda size: (oracle.cost(n, int(size) // 4, 4, sched_a, alpha, bw, bw)
                      - oracle.cost(n, int(size) // 4, 4, sched_b, alpha, bw, bw))
    for _ in range(80):
        mid = (lo * hi) ** 0.5
        if (f(mid) > 0) == (f(lo) > 0):
            lo = mid
        else:
            hi = mid
    return lo


def test_crossovers_printed_on_pages():
    """Primer ch. 4 Figure 4.7: for N = 128, alpha = 22 us, 400 Gb/s the ring
    and doubling curves cross at S* of about 54 MB; Scaling ML systems ch. 06:
    for alpha = 5 us, beta = 50 GB/s, N = 100 the ring-tree crossover is
    about 3.8 MB (the page's approximation N alpha beta / log2 N)."""
    s = _crossover(128, "ring", "recursive_doubling", 22e-6, 50e9)
    assert s / 1e6 == pytest.approx(54.2, rel=0.01)
    s = _crossover(100, "ring", "tree", 5e-6, 50e9)
    assert s / 1e6 == pytest.approx(3.8, rel=0.02)
