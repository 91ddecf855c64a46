"""Closed-form summation orders of the schedules, element by element.

Independent of the oracle's simulation: these folds state, per element, the
sum that each schedule produces, as derived from the pages' index rules.  They
are pure Python over numpy float32 scalars (each + is one binary32 add) and
are only practical for tiny inputs.

  ring          element in chunk c: ((x_c + x_{c+1}) + ...) + x_{c+N-1}
                (ranks mod N; the chunk is first sent by rank c at
                reduce-scatter step 0)
  rabenseifner  the balanced pairwise tree over ranks in index order
  recursive_doubling  the same balanced tree (each pair's sum is commutative)
  tree          binomial tree to rank 0 (left-complete for N not 2^k)
  double_tree   half 0 by tree 1, half 1 by its mirror (see dtree_fold)
  hierarchical  group partial of slice k: ((x_{g,k+1} + x_{g,k+2}) + ...) + x_{g,k};
                then, for sub-chunk j of the slice, a ring fold over groups
                starting at group j
"""
import numpy as np


def part(length, k, c):
    return (c * length) // k, ((c + 1) * length) // k


def chunk_of(e, length, k):
    for c in range(k):
        lo, hi = part(length, k, c)
        if lo <= e < hi:
            return c, lo
    raise ValueError


def add32(a, b):
    return np.float32(np.float32(a) + np.float32(b))


def ring_fold(vals, start, add=add32):
    n = len(vals)
    acc = np.float32(vals[start % n])
    for t in range(1, n):
        acc = add(acc, vals[(start + t) % n])
    return acc


def tree_fold(vals, add=add32):
    level = [np.float32(v) for v in vals]
    while len(level) > 1:
        level = [add(level[2 * m], level[2 * m + 1]) for m in range(len(level) // 2)]
    return level[0]


def binomial_fold(vals, add=add32):
    """Binomial tree to rank 0: blocks of 2^k ranks merge pairwise; a block
    without a right neighbour is carried up unchanged (any N)."""
    level = [np.float32(v) for v in vals]
    while len(level) > 1:
        nxt = []
        for m in range(0, len(level), 2):
            nxt.append(add(level[m], level[m + 1]) if m + 1 < len(level) else level[m])
        level = nxt
    return level[0]


def dtree_fold(vals, half, add=add32):
    """Double binary tree (N = 2^L): half 0 climbs tree 1, rooted at 0 with
    the single child N/2; half 1 climbs its mirror, rooted at N-1 with the
    child N/2 - 1.  A node c whose subtree spans 2b-1 ranks adds its own
    value, then its lower child's (c - b/2), then its higher child's (c + b/2)."""
    n = len(vals)

    def sub(c, b):
        if b == 1:
            return np.float32(vals[c])
        return add(add(vals[c], sub(c - b // 2, b // 2)), sub(c + b // 2, b // 2))

    if n == 1:
        return np.float32(vals[0])
    if half == 0:
        return add(vals[0], sub(n // 2, n // 2))
    return add(vals[n - 1], sub(n // 2 - 1, n // 2))


def fold_at(col, e, count, schedule, group_size=1, add=add32):
    """The sum one schedule forms at position e of `count` positions from
    the per-rank values col[r] (scalars, or equal-length vectors)."""
    n = len(col)
    if n == 1:
        return np.float32(col[0])
    if schedule == "ring":
        c, _ = chunk_of(e, count, n)
        return ring_fold(col, c, add)
    if schedule in ("rabenseifner", "recursive_doubling"):
        return tree_fold(col, add)
    if schedule == "tree":
        return binomial_fold(col, add)
    if schedule == "double_tree":
        return dtree_fold(col, 0 if e < count // 2 else 1, add)
    if schedule == "hierarchical":
        g_sz = group_size
        m_groups = n // g_sz
        k, slo = chunk_of(e, count, g_sz)
        _, shi = part(count, g_sz, k)
        partials = []
        for g in range(m_groups):
            local = [col[g * g_sz + l] for l in range(g_sz)]
            partials.append(ring_fold(local, k + 1, add) if g_sz > 1 else np.float32(local[0]))
        j, _ = chunk_of(e - slo, shi - slo, m_groups)
        return ring_fold(partials, j, add) if m_groups > 1 else partials[0]
    raise ValueError(schedule)


def expected_fp32(xs, schedule, group_size=1, add=add32):
    """xs: list of N float32 arrays.  Returns the float32 result array."""
    n = len(xs)
    count = len(xs[0])
    out = np.zeros(count, np.float32)
    for e in range(count):
        out[e] = fold_at([xs[r][e] for r in range(n)], e, count, schedule, group_size, add)
    return out


def widen(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def to_bf16_bits(x):
    """Round-to-nearest-even via torch's conversion (a library routine)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def expected_bf16(bits_list, schedule, group_size=1):
    """bf16 bits in, bf16 bits out: fp32 fold of the widened inputs, one rounding."""
    n = len(bits_list)
    if n == 1:
        return np.asarray(bits_list[0], np.uint16).copy()
    xs = [widen(b) for b in bits_list]
    return to_bf16_bits(expected_fp32(xs, schedule, group_size))


def add_bf16_each(a, b):
    """One add of the round-each-step mode: fp32 add of bf16 values, then RNE
    to bf16 (torch's conversion), returned widened."""
    return widen(to_bf16_bits(np.array([np.float32(a) + np.float32(b)], np.float32)))[0]


def expected_bf16_each(bits_list, schedule, group_size=1):
    if len(bits_list) == 1:
        return np.asarray(bits_list[0], np.uint16).copy()
    xs = [widen(b) for b in bits_list]
    return to_bf16_bits(expected_fp32(xs, schedule, group_size, add=add_bf16_each))


QBLOCK = 128


def int8_roundtrip(x):
    """Blockwise INT8 encode then decode of one block (float32 vector):
    s = max|x| / 127, q = round-half-even(x / s) clamped to [-127, 127],
    value q * s (a zero code gives +0); a block of zeros stays zero."""
    x = np.asarray(x, np.float32)
    s = np.float32(np.max(np.abs(x)) / np.float32(127.0)) if len(x) else np.float32(0)
    if s == 0:
        return np.zeros_like(x)
    # the code is an integer (int8 has no negative zero), so a zero code
    # decodes to +0
    q = np.clip(np.rint(x / s), -127, 127).astype(np.int8).astype(np.float32)
    return (q * s).astype(np.float32)


def expected_int8ef(xs, schedule, errs=None, group_size=1):
    """Block-level closed form of the compressed all-reduce: every leaf is
    round-tripped g + e, every partial sum of the schedule's fold is
    round-tripped, blocks play the role of elements in the chunk partition.
    Returns (result, new_errors)."""
    n = len(xs)
    count = len(xs[0])
    nblk = (count + QBLOCK - 1) // QBLOCK
    out = np.zeros(count, np.float32)
    new_errs = [np.zeros(count, np.float32) for _ in range(n)]

    def add(a, b):
        return int8_roundtrip((np.asarray(a, np.float32) + np.asarray(b, np.float32)).astype(np.float32))

    for blk in range(nblk):
        lo, hi = blk * QBLOCK, min(count, (blk + 1) * QBLOCK)
        col = []
        for r in range(n):
            x = xs[r][lo:hi] + (errs[r][lo:hi] if errs is not None else np.float32(0))
            x = x.astype(np.float32)
            v = int8_roundtrip(x)
            new_errs[r][lo:hi] = (x - v).astype(np.float32)
            col.append(v)
        out[lo:hi] = fold_at(col, blk, nblk, schedule, group_size, add)
    return out, new_errs
