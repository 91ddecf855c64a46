"""Test-side interpreter of the library's launch list (numpy, CPU).

It executes the ops the planner hands to the GPU -- operand locations, fp32
scratch slots, bf16 flags, fused second outputs, one-pass folds -- with numpy
float32 arithmetic, so that the planner's lowering can be checked against the
oracle on a machine without a GPU.  It is neither the oracle nor a fallback:
nothing in the library calls it.
"""
import numpy as np

from gradient_all_reduce_ar_amd import _binding as B
from tests.folds import to_bf16_bits, widen


def _slot_range(lo, hi, shift, stride):
    """Slot indices of elements [lo, hi): e - shift, which must lie in the slot."""
    assert 0 <= lo - shift and hi - shift <= stride, (lo, hi, shift, stride)
    return lo - shift, hi - shift


def _read(loc, lo, hi, bf_flag, bufs, scratch, fp32_mode, shift=0, stride=None):
    if loc >= B.LOC_SCRATCH:
        a, b = _slot_range(lo, hi, shift, stride)
        return scratch[loc - B.LOC_SCRATCH][a:b].copy()
    if fp32_mode:
        return bufs[loc][lo:hi].copy()
    assert bf_flag, "bf16 plan reads a rank buffer as fp32"
    return widen(bufs[loc][lo:hi])


def _write(loc, lo, hi, vals, out_bf, bufs, scratch, fp32_mode, shift=0, stride=None):
    if loc >= B.LOC_SCRATCH:
        assert not out_bf
        a, b = _slot_range(lo, hi, shift, stride)
        scratch[loc - B.LOC_SCRATCH][a:b] = vals
    elif fp32_mode:
        bufs[loc][lo:hi] = vals
    else:
        assert out_bf, "bf16 plan writes fp32 into a rank buffer"
        bufs[loc][lo:hi] = to_bf16_bits(vals)


def run(plan, bufs, dtype, group_size):
    fp32_mode = dtype == "fp32"
    count = len(bufs[0])
    n = len(bufs)
    stats = B.ar_plan_stats(plan)
    nl = B.ar_plan_num_launches(plan)
    stride = B.ar_plan_launch_scratch(plan, 0)[1] if nl else 0
    nslots = stats["scratch_bytes"] // (4 * stride) if stride else 0
    scratch = [np.full(stride, np.nan, np.float32) for _ in range(nslots)]
    for i in range(nl):
        kind, _ = B.ar_plan_launch_info(plan, i)
        ops = B.ar_plan_launch_ops(plan, i)
        shift, _ = B.ar_plan_launch_scratch(plan, i)
        fam = kind & 0xF00
        for k in range(len(ops["lo"])):
            lo, hi = int(ops["lo"][k]), int(ops["hi"][k])
            a, b, o, o2, aux = (int(ops[x][k]) for x in ("a", "b", "o", "o2", "aux"))
            if fam == B.KIND_REDUCE:
                va = _read(a, lo, hi, kind & 1, bufs, scratch, fp32_mode, shift, stride)
                vb = _read(b, lo, hi, kind & 2, bufs, scratch, fp32_mode, shift, stride)
                s = (va + vb).astype(np.float32)
                _write(o, lo, hi, s, bool(kind & 4), bufs, scratch, fp32_mode, shift, stride)
                if kind & 8:
                    _write(o2, lo, hi, s, bool(kind & 4), bufs, scratch, fp32_mode, shift, stride)
            elif fam == B.KIND_COPY:
                bufs[o][lo:hi] = bufs[a][lo:hi]
            elif fam == B.KIND_FAN:  # one-pass all-gather: rank a's range to every other rank
                for r in range(n):
                    if r != a:
                        bufs[r][lo:hi] = bufs[a][lo:hi]
            else:
                each = (kind & 3) == 2  # bf16 rounded at every add

                def fold(a, b):
                    s_ = (a + b).astype(np.float32)
                    return widen(to_bf16_bits(s_)) if each else s_

                cols = [bufs[r][lo:hi].copy() if fp32_mode else widen(bufs[r][lo:hi]) for r in range(n)]
                if fam == B.KIND_RING:
                    acc = cols[aux % n]
                    for t in range(1, n):
                        acc = fold(acc, cols[(aux + t) % n])
                elif fam == B.KIND_TREE:
                    level = cols
                    while len(level) > 1:
                        level = [fold(level[m], level[m + 1]) if m + 1 < len(level) else level[m]
                                 for m in range(0, len(level), 2)]
                    acc = level[0]
                elif fam == B.KIND_DTREE:
                    def sub(c, b):
                        if b == 1:
                            return cols[c]
                        return fold(fold(cols[c], sub(c - b // 2, b // 2)), sub(c + b // 2, b // 2))
                    acc = fold(cols[0], sub(n // 2, n // 2)) if aux == 0 else fold(cols[n - 1], sub(n // 2 - 1, n // 2))
                else:
                    G = group_size
                    M = n // G
                    ls, j = aux & 0xFF, aux >> 8
                    acc = None
                    for mi in range(M):
                        g = (j + mi) % M
                        part = cols[g * G + ls]
                        for t in range(1, G):
                            part = fold(part, cols[g * G + (ls + t) % G])
                        acc = part if acc is None else fold(acc, part)
                res = acc if fp32_mode else to_bf16_bits(acc)
                for r in (range(n) if o < 0 else (o,)):  # a reduce-scatter stores into the owner only
                    bufs[r][lo:hi] = res
    return bufs


def _q_block(x):
    """Codes and scale of one block (numpy float32 arithmetic)."""
    s = np.float32(np.max(np.abs(x)) / np.float32(127.0)) if len(x) else np.float32(0)
    if s == 0:
        return np.zeros(len(x), np.int8), s
    return np.clip(np.rint(x / s), -127, 127).astype(np.int8), s


def run_int8(plan, bufs, errs=None, group=1):
    """Executes an int8_ef plan's launch list on float32 host arrays."""
    n = len(bufs)
    count = len(bufs[0])
    Q = B.QBLOCK
    nblk = (count + Q - 1) // Q
    codes = [np.zeros(nblk * Q, np.int8) for _ in range(n)]
    scales = [np.full(nblk, np.nan, np.float32) for _ in range(n)]

    def dec(r, blk):
        return (codes[r][blk * Q:(blk + 1) * Q].astype(np.float32) * scales[r][blk]).astype(np.float32)

    def put(r, blk, x):
        q, s = _q_block(x)
        codes[r][blk * Q:(blk + 1) * Q] = q
        scales[r][blk] = s

    for i in range(B.ar_plan_num_launches(plan)):
        kind, _ = B.ar_plan_launch_info(plan, i)
        ops = B.ar_plan_launch_ops(plan, i)
        fam = kind & 0xF00
        for k in range(len(ops["lo"])):
            lo, hi = int(ops["lo"][k]), int(ops["hi"][k])
            a, b, o, o2 = (int(ops[x][k]) for x in ("a", "b", "o", "o2"))
            for blk in range(lo, hi):
                e0, e1 = blk * Q, min(count, (blk + 1) * Q)
                if fam == B.KIND_QENCODE:
                    x = np.zeros(Q, np.float32)
                    x[:e1 - e0] = bufs[a][e0:e1] + (errs[a][e0:e1] if errs is not None else np.float32(0))
                    put(a, blk, x)
                    if errs is not None:
                        errs[a][e0:e1] = (x[:e1 - e0] - dec(a, blk)[:e1 - e0]).astype(np.float32)
                elif fam == B.KIND_QREDUCE:
                    def operand(r, raw):
                        if not raw:
                            return dec(r, blk)
                        # the rank's own g + e, encoded here; residual written back
                        xr = np.zeros(Q, np.float32)
                        xr[:e1 - e0] = bufs[r][e0:e1] + (errs[r][e0:e1] if errs is not None else np.float32(0))
                        v = _roundtrip(xr)
                        if errs is not None:
                            errs[r][e0:e1] = (xr - v)[:e1 - e0]
                        return v
                    x = (operand(a, kind & 1) + operand(b, kind & 2)).astype(np.float32)
                    x[e1 - e0:] = 0
                    outs = [o] + ([o2] if kind & 8 else [])
                    q, sc = _q_block(x)
                    for r in outs:
                        if not kind & 32:  # codes stored unless nothing reads them later
                            codes[r][blk * Q:(blk + 1) * Q] = q
                            scales[r][blk] = sc
                        if kind & 16:      # final codes decoded into the rank's buffer
                            bufs[r][e0:e1] = (q.astype(np.float32) * sc)[:e1 - e0]
                elif fam == B.KIND_QCOPY:
                    q, sc = codes[a][e0:e0 + Q].copy(), scales[a][blk]
                    if not kind & 32:
                        codes[o][e0:e0 + Q] = q
                        scales[o][blk] = sc
                    if kind & 16:
                        bufs[o][e0:e1] = (q.astype(np.float32) * sc)[:e1 - e0]
                elif fam == B.KIND_QDECODE:
                    bufs[a][e0:e1] = dec(a, blk)[:e1 - e0]
                elif fam in (B.KIND_RING, B.KIND_HIER, B.KIND_TREE, B.KIND_DTREE):
                    assert kind & 3 == 3, f"one-pass kind {kind:#x} without the INT8 code"
                    _onepass_block(fam, int(ops["aux"][k]), blk, e0, e1, bufs, errs, group)
                else:
                    raise AssertionError(f"kind {kind:#x} in an int8 plan")
    return bufs


def _roundtrip(x):
    q, s = _q_block(x)
    return (q.astype(np.float32) * s).astype(np.float32)


def _onepass_block(fam, aux, blk, e0, e1, bufs, errs, group):
    """One block of a one-pass INT8 fold, in the order the kernel's aux
    selects (the same orders as the fp32 one-pass kinds)."""
    n = len(bufs)
    Q = B.QBLOCK
    leaves = []
    for r in range(n):
        x = np.zeros(Q, np.float32)
        x[:e1 - e0] = bufs[r][e0:e1] + (errs[r][e0:e1] if errs is not None else np.float32(0))
        v = _roundtrip(x)
        if errs is not None:
            errs[r][e0:e1] = (x - v)[:e1 - e0]
        leaves.append(v)

    def add(a, b):
        return _roundtrip((a + b).astype(np.float32))

    if fam == B.KIND_RING:
        acc = leaves[aux % n]
        for t in range(1, n):
            acc = add(acc, leaves[(aux + t) % n])
    elif fam == B.KIND_HIER:
        G = group
        M = n // G
        ls, j = aux & 0xFF, aux >> 8
        acc = None
        for mi in range(M):
            g = (j + mi) % M
            part = leaves[g * G + ls]
            for t in range(1, G):
                part = add(part, leaves[g * G + (ls + t) % G])
            acc = part if acc is None else add(acc, part)
    elif fam == B.KIND_TREE:
        level = leaves
        while len(level) > 1:
            level = [add(level[m], level[m + 1]) if m + 1 < len(level) else level[m]
                     for m in range(0, len(level), 2)]
        acc = level[0]
    else:
        def sub(c, b):
            if b == 1:
                return leaves[c]
            return add(add(leaves[c], sub(c - b // 2, b // 2)), sub(c + b // 2, b // 2))
        acc = add(leaves[0], sub(n // 2, n // 2)) if aux == 0 else add(leaves[n - 1], sub(n // 2 - 1, n // 2))
    for r in range(n):
        bufs[r][e0:e1] = acc[:e1 - e0]
