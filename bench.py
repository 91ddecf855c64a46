"""Benchmark: 16-rank, 192 MiB-per-rank fp32 ring all-reduce on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c1|c2|c2q|c3|c3e|c4|c5r16|c5g16|c5r64|c5g64|overlap]
                [--exec steps|steps_unfused|onepass]

A step is one whole all-reduce (every launch of the schedule) over the N
virtual ranks' buffers, which are resident in HBM before timing starts.  The
W warm-up calls are untimed; the K timed calls run back to back between two
device synchronisations.  Each call is in place, so values grow by about N
per call; the kernels' work does not depend on the values.

Prints ONE JSON line.  value = busbw = algbw * 2(N-1)/N with algbw = S / T
(S = bytes per rank, GB = 1e9; the nccl-tests convention of the AI training
network primer, ch. 4 section 4.8), from K calls with no profiling.
roofline: from a second run of the same K calls (inputs restored first), the
kernel kind with the largest share of GPU time, its algorithmic bytes per
launch over its mean launch duration (a start and a stop HIP event that the
launches record as part of their dispatch, on the call's stream), against
8 TB/s.  Each call of that run times about four of its launches, in
rotation, so every launch position is timed over the run while the events
barely perturb the calls (config.compare.with_launch_events gives that run's
time per call); config.compare also times the calls replayed as HIP graphs.
cpu_baseline: the CPU oracle (plain single-threaded C) timed on the host on
the same inputs.
"""
import argparse
import hashlib
import itertools
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "effective busbw GB/s and % of HBM peak, 16-rank 192 MiB all-reduce"

WORKLOADS = {
    # name: (description, schedule, nranks, group, dtype, count or None for bucketed)
    "c1": ("ring all-reduce, 4 virtual ranks x 4096 fp32 (16 KiB each), U[-1,1) (a case that stays in cache)",
           "ring", 4, 1, "fp32", 4096),
    "c2": ("ring all-reduce, 16 virtual ranks x 192 MiB fp32 (50,331,648 elements each), N(0,1e-3)",
           "ring", 16, 8, "fp32", 12288 * 4096),
    "c3": ("ring all-reduce, 16 virtual ranks x 192 MiB bf16 (100,663,296 elements each), N(0,1e-3), "
           "fp32 accumulate", "ring", 16, 8, "bf16", 2 * 12288 * 4096),
    "c3e": ("ring all-reduce, 16 virtual ranks x 192 MiB bf16, N(0,1e-3), every partial sum rounded to bf16",
            "ring", 16, 8, "bf16_each", 2 * 12288 * 4096),
    "c2q": ("ring all-reduce, 16 virtual ranks x 192 MiB fp32, blockwise INT8 messages (128-element blocks, "
            "fp32 scales) with error feedback, N(0,1e-3) gradients and residuals",
            "ring", 16, 8, "int8_ef", 12288 * 4096),
    "c4": ("hierarchical all-reduce, 2 groups x 8 ranks x 192 MiB fp32, N(0,1e-3)",
           "hierarchical", 16, 8, "fp32", 12288 * 4096),
    "c5r16": ("Rabenseifner, 16 ranks, bf16, 300 lognormal tensors in 25 MiB buckets", "rabenseifner", 16, 1,
              "bf16", None),
    "c5g16": ("ring, 16 ranks, bf16, 300 lognormal tensors in 25 MiB buckets", "ring", 16, 1, "bf16", None),
    "c5r64": ("Rabenseifner, 64 ranks, bf16, 300 lognormal tensors in 25 MiB buckets", "rabenseifner", 64, 1,
              "bf16", None),
    "c5g64": ("ring, 64 ranks, bf16, 300 lognormal tensors in 25 MiB buckets", "ring", 64, 1, "bf16", None),
}

KIND_NAMES = {0x100: "chunk_reduce", 0x200: "chunk_copy", 0x300: "onepass_ring", 0x400: "onepass_hier",
              0x500: "onepass_tree", 0x600: "onepass_dtree", 0x700: "q_encode", 0x800: "q_reduce", 0x900: "q_copy",
              0xA00: "q_decode", 0xB00: "onepass_fan"}


def kernel_label(kind, shape=None, nranks=None):
    """Kernel name with its template arguments, as rocprofv3 reports it
    (shape: ar_plan_launch_shape of a launch of this kind; without it the
    step kernels are named by their flags only)."""
    fam = kind & 0xF00
    if fam == 0x100:
        if shape:
            return f"chunk_reduce<{kind & 0xF}, {shape['units']}, {shape['cpol']}>"
        return f"chunk_reduce<{kind & 0xF}>"
    if fam == 0x200:
        if shape:
            return f"chunk_copy<{kind & 0xFF}, {shape['units']}, {shape['cpol']}>"
        return f"chunk_copy<{kind & 0xFF}>"
    if fam == 0x800:
        if kind & 0x13:  # fused hop: raw operands or final decode
            return f"q_hop<{kind & 0xFF}>"
        return f"q_reduce<{'true' if kind & 8 else 'false'}>"
    if fam == 0x900 and kind & 16:
        return f"q_copy_dec<{'false' if kind & 32 else 'true'}>"
    if fam == 0xB00 and shape:
        return f"onepass_fan<{kind & 0xFF}, {shape['cpol']}>"
    if fam >= 0x700:
        return KIND_NAMES[fam]
    if kind & 3 == 3:  # one-pass fold of an INT8 plan
        return "q_" + KIND_NAMES[fam]
    bf, each = ("true" if kind & 3 else "false"), ("true" if kind & 3 == 2 else "false")
    if shape and shape.get("lds_bytes") and nranks:  # the LDS-staged fold
        ncls = 16 if nranks <= 16 else 32 if nranks <= 32 else 64  # the rank-count size class
        if fam == 0x500:
            nmax = 1 << max(0, (nranks - 1).bit_length())
            fold, ncls = f"TreeFold<{nmax}, {'true' if nranks < nmax else 'false'}>", max(ncls, nmax)
        elif fam == 0x600:
            fold = f"DTreeFoldOp<{nranks}>"
        else:
            fold = {0x300: "RingFold", 0x400: "HierFold"}[fam]
        if kind & 0x1000 and nranks <= 16:  # a reduce-scatter fold: its own tiles
            fold = f"OwnerTiles<{fold}>"
        return f"onepass_lds<{bf}, {each}, {ncls}, {shape['batch']}, {shape['cpol']}, {fold}>"
    if shape and fam in (0x300, 0x400):
        return f"{KIND_NAMES[fam]}<{bf}, {each}, {shape['units']}, {shape['batch']}>"
    if shape and fam == 0x500 and nranks:
        nmax = 1 << max(0, (nranks - 1).bit_length())
        return f"onepass_tree<{bf}, {each}, {nmax}, {'true' if nranks < nmax else 'false'}, {shape['units']}, " \
               f"{shape['batch']}>"
    if shape and fam == 0x600 and nranks:
        return f"onepass_dtree<{bf}, {each}, {nranks}, {shape['units']}>"
    return f"{KIND_NAMES[fam]}<{'bf16' if kind & 1 else 'fp32'}>"


def read_share(kind, elem):
    """Fraction of a step or one-pass kernel's algorithmic bytes that are reads."""
    fam = kind & 0xF00
    if fam == 0x100:
        if elem == 4:
            rd, wr = 8, 4 * (2 if kind & 8 else 1)
        else:
            rd = (2 if kind & 1 else 4) + (2 if kind & 2 else 4)
            wr = (2 if kind & 4 else 4) * (2 if kind & 8 else 1)
        return rd / (rd + wr)
    return 0.5  # copies and one-pass folds read as much as they write


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def launch_bytes(B, plan, i, nranks, elem, count):
    """Algorithmic device bytes of launch i (read + write of every operand)."""
    kind, _ = B.ar_plan_launch_info(plan, i)
    ops = B.ar_plan_launch_ops(plan, i)
    n = (ops["hi"] - ops["lo"]).astype("int64")
    fam = kind & 0xF00
    if fam < B.KIND_QENCODE and fam not in (B.KIND_REDUCE, B.KIND_COPY) and kind & 3 == 3:
        # one-pass INT8 fold: g, e in; e, result out, per rank; ranges count blocks
        el = int(sum(max(0, min(int(h) * B.QBLOCK, count) - int(lo) * B.QBLOCK)
                     for lo, h in zip(ops["lo"], ops["hi"])))
        return el * 16 * nranks, kind
    if fam >= B.KIND_QENCODE:
        # blockwise INT8: op ranges count 128-element blocks
        blocks = int(n.sum())
        el = int(sum(max(0, min(int(h) * B.QBLOCK, count) - int(lo) * B.QBLOCK)
                     for lo, h in zip(ops["lo"], ops["hi"])))
        if fam == B.KIND_QENCODE:
            return el * 13 + 4 * blocks, kind  # g, e in; codes, e out; scales
        if fam == B.KIND_QREDUCE:
            outs = 2 if kind & 8 else 1
            nb = sum(el * 12 if kind & raw else el + 4 * blocks for raw in (1, 2))  # own g, e / codes in
            if not kind & 32:
                nb += (el + 4 * blocks) * outs  # codes and scales out
            if kind & 16:
                nb += el * 4 * outs  # final values decoded into the buffers
            return nb, kind
        if fam == B.KIND_QCOPY:
            nb = (el + 4 * blocks) * (1 if kind & 32 else 2) + (el * 4 if kind & 16 else 0)
            return nb, kind
        return el * 5 + 4 * blocks, kind  # decode: codes, scales in; fp32 out
    if fam == B.KIND_REDUCE:
        if elem == 4:
            per = 3 * 4 + (4 if kind & 8 else 0)
        else:
            a = 2 if kind & 1 else 4
            b = 2 if kind & 2 else 4
            o = 2 if kind & 4 else 4
            per = a + b + o + (o if kind & 8 else 0)
        return int(n.sum()) * per, kind
    if fam == B.KIND_COPY:
        return int(n.sum()) * 2 * elem, kind
    return int(n.sum()) * 2 * elem * nranks, kind


def kernels_sha256():
    """SHA-256 over the code of the device kernel sources (kernels.hip,
    qkernels.hip, kernels.hpp) with comments and blank space removed, so that
    editing a comment does not invalidate counters taken on the same code."""
    import re

    csrc = os.path.join(ROOT, "gradient_all_reduce_ar_amd", "csrc")
    code = []
    for f in ("kernels.hip", "qkernels.hip", "kernels.hpp"):
        text = open(os.path.join(csrc, f)).read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        code.append(" ".join(text.split()))
    return hashlib.sha256("\n".join(code).encode()).hexdigest()


def traffic_record(kernel_name, workload, exec_mode):
    """Counter-measured HBM bytes per launch from a committed rocprofv3 summary,
    if it was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    digest = kernels_sha256()
    try:
        recs = json.load(open(path))
    except ValueError:
        return None
    for r in recs:
        if (r.get("kernel") == kernel_name and r.get("workload") == workload and r.get("exec") == exec_mode
                and r.get("kernels_sha256") == digest):
            return r.get("bytes_per_launch")
    return None


def probe_best(B, torch, stream, src, dst, nb, reps=5, restore=None, split=False):
    """Best rate over 1, 2, 4 units per thread and the three cache policies
    of the probe on these buffers (median of `reps` launches after two);
    split: each workgroup stores into one destination only."""
    best = None
    for units in (1, 2, 4):
        for policy in ((4, 5, 6) if split else (0, 1, 2)):
            ts = []
            for r in range(reps + 2):
                if restore is not None:
                    restore()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                B.ar_hbm_probe(src, dst, nb, units, policy, stream)
                e1.record(stream)
                torch.cuda.synchronize()
                if r >= 2:
                    ts.append(e0.elapsed_time(e1))
            ts.sort()
            med = ts[len(ts) // 2]
            gbps = (len(src) + len(dst)) * nb / (med * 1e-3) / 1e9
            if best is None or gbps > best["GBps"]:
                best = {"GBps": round(gbps, 1), "ms": round(med, 4), "units": units, "policy": policy,
                        "read_share": len(src) / (len(src) + len(dst)), "bytes": (len(src) + len(dst)) * nb}
    return best


def kernel_streams(kind):
    """(sources, destinations) of a step kernel's launch, or None."""
    fam = kind & 0xF00
    if fam == 0x100:
        return (2, 2) if kind & 8 else (2, 1)
    if fam == 0x200:
        return (1, 1)
    return None


def probe_ceilings(B, torch, dev, stream, rank_bufs=None, rank_bytes=0, restore=None, matched=(), gib=4, reps=5):
    """Attainable HBM bandwidth of this GPU for the kernels' read/write mixes,
    measured with the library's own probe kernel (ar_hbm_probe) on buffers of
    `gib` GiB of random fp32 (far larger than the 256 MB device cache): for
    each mix the best of 1, 2 and 4 units per thread and of the three cache
    policies, each the median of `reps` event-timed launches after two
    untimed ones.  With rank_bufs, also the one-pass mix on the workload's
    own buffers: every buffer read and every buffer written, in place (each
    launch on the inputs restored by `restore`, outside its events).
    matched: (name, sources, destinations, bytes per buffer) mixes measured
    on the first bytes of the same buffers: a step kernel's streams at its
    own launch size, so that the launch's start-up and drain weigh as they
    do in the kernel."""
    nbytes = gib << 30
    bufs = [torch.randn(nbytes // 4, device=dev) for _ in range(4)]
    torch.cuda.synchronize()
    mixes = [("read 1:0", bufs[:1], [], nbytes), ("write 0:1", [], bufs[:1], nbytes),
             ("copy 1:1", bufs[:1], bufs[1:2], nbytes), ("reduce 2:1", bufs[:2], bufs[2:3], nbytes),
             ("reduce 2:2", bufs[:2], bufs[2:4], nbytes)]
    if rank_bufs is not None and len(rank_bufs) <= 64 and rank_bytes % 16 == 0 and rank_bytes >= (64 << 20):
        # the one-pass mix (every rank read, every rank written, in place) and
        # its parts: reads of every rank, writes to every rank, a fold into one
        # rank, a fan-out from one rank to the others
        n = len(rank_bufs)
        mixes += [(f"fold {n}:{n}", rank_bufs, rank_bufs, rank_bytes),
                  (f"read {n}:0", rank_bufs, [], rank_bytes),
                  (f"write 0:{n}", [], rank_bufs, rank_bytes),
                  (f"write 0:{n} split", [], rank_bufs, rank_bytes),
                  (f"fold {n}:1", rank_bufs, rank_bufs[:1], rank_bytes),
                  (f"fan 1:{n - 1}", rank_bufs[:1], rank_bufs[1:], rank_bytes)]
    out = {}
    for name, src, dst, nb in mixes:
        writes_ranks = rank_bufs is not None and any(b is rank_bufs[0] for b in dst)
        out[name] = probe_best(B, torch, stream, src, dst, nb, reps, restore if writes_ranks else None,
                               split=name.endswith(" split"))
    for name, ns, nd, nb in matched:
        out[name] = probe_best(B, torch, stream, bufs[:ns], bufs[ns:ns + nd], min(nb, nbytes), reps)
    del bufs
    torch.cuda.empty_cache()
    return out


def staged_bound(ceil, nranks):
    """GB/s of reading every rank and then writing every rank with each
    workgroup storing one rank, at the probes' rates, one after the other
    (the LDS-staged one-pass folds' two halves), or None."""
    rd, wr = ceil.get(f"read {nranks}:0"), ceil.get(f"write 0:{nranks} split")
    if not rd or not wr:
        return None
    return round(1.0 / (0.5 / rd["GBps"] + 0.5 / wr["GBps"]), 1)


def attainable_for(ceil, kind, elem, nbuf, staged=False):
    """The probe mix with a kernel's streams: two sources into one output for
    a reduce, into two for the fused reduce + forward, one into one for a copy,
    every buffer into every buffer for a register one-pass fold (nbuf: the
    rank buffers, and with error feedback the residual buffers too), the read
    and the split-write probes one after the other for an LDS-staged one
    (staged); otherwise (the INT8 step kernels) the two-buffer mix whose read
    share is nearest the kernel's."""
    fam = kind & 0xF00
    fold = f"fold {nbuf}:{nbuf}"
    if staged and staged_bound(ceil, nbuf):
        return f"read {nbuf}:0 then write 0:{nbuf} split", staged_bound(ceil, nbuf)
    if fam == 0x100:
        name = "reduce 2:2" if kind & 8 else "reduce 2:1"
    elif fam == 0x200:
        name = "copy 1:1"
    elif fam in (0x300, 0x400, 0x500, 0x600) and fold in ceil:
        name = fold
    else:
        share = read_share(kind, elem)
        big = [k for k in ceil if k in ("read 1:0", "write 0:1", "copy 1:1", "reduce 2:1", "reduce 2:2")]
        name = min(big, key=lambda k: abs(ceil[k]["read_share"] - share))
    return name, ceil[name]["GBps"]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="c2", choices=sorted(WORKLOADS) + ["overlap", "latency"])
    ap.add_argument("--compute-ratio", type=float, default=1.5,
                    help="overlap workload: backward compute per bucket as a multiple of its all-reduce time")
    ap.add_argument("--exec", default="steps", choices=["steps", "steps_unfused", "onepass"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the one-pass, graph, cold-cache and ceiling runs")
    ap.add_argument("--calibrate", action="store_true",
                    help="first copy 1 GiB three times with the library's probe kernel (ar_hbm_probe, one "
                         "source, one destination), so that hardware counters of the same run can be scaled "
                         "by a kernel of known traffic (1 GiB read, 1 GiB written per launch)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only: the N virtual ranks live in one GPU's HBM; "
              "there is no multi-GPU path to measure (use --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from gradient_all_reduce_ar_amd import _binding as B
    from gradient_all_reduce_ar_amd import workloads

    if args.workload == "overlap":
        return overlap_main(args, B, workloads, np, torch)
    if args.workload == "latency":
        return latency_main(args, B, np, torch)
    desc, sched, n, group, dtype, count = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    quant = dtype == "int8_ef"
    elem = 4 if dtype in ("fp32", "int8_ef") else 2
    nbuf = 2 * n if quant else n  # buffers a one-pass fold reads and writes in place
    view = np.float32 if elem == 4 else np.int16
    gen_dtype = "fp32" if elem == 4 else "bf16"

    if args.calibrate:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            B.ar_hbm_probe([src], [dst], 1 << 30, 2, 1, torch.cuda.current_stream(dev))
        torch.cuda.synchronize()
        del src, dst
        log("calibration: 3 probe copies of 1 GiB (hbm_probe_kernel<2, 1>: read 1 GiB + write 1 GiB each)")

    # ---- inputs, resident in HBM before timing, with pristine device copies
    t0 = time.time()
    bucketed = count is None
    if bucketed:
        sizes = workloads.bucketed_tensor_sizes(elem_bytes=elem)
        plan = B.ar_bucket_plan_create(n, group, sizes, dtype, sched, 25 << 20)
        B.ar_bucket_set_exec(plan, args.exec)
        offsets, arena = B.ar_bucket_layout(plan, len(sizes))
        host = workloads.bucketed_arenas(n, sizes, offsets, arena, dtype=gen_dtype)
        count_logical = int(sum(int(c) for c in sizes))
        # the buckets' all-reduces in shared launches: the plan that runs them
        lplan = B.ar_bucket_batched_plan(plan)
    else:
        plan = B.ar_plan_create(n, group, count, dtype, sched)
        B.ar_plan_set_exec(plan, args.exec)
        if args.workload == "c1":
            host = workloads.uniform_inputs(n, count, seed=0)
        else:
            host = workloads.normal_inputs(n, count, seed=0, dtype=gen_dtype)
        count_logical = count
        lplan = plan
    bufs = [torch.from_numpy(h.view(view)).to(dev) for h in host]
    pristine = [b.clone() for b in bufs]
    errs = perrs = None
    if quant:
        # every call multiplies the values by about N (in place); 28 calls from
        # N(0, 1e-3) stay finite, the range the quantizer is defined on
        if args.warmup + args.steps > 28:
            print("c2q: warmup + steps must be <= 28 (values grow N-fold per in-place call and must stay "
                  "finite)", file=sys.stderr)
            sys.exit(2)
        err_host = workloads.normal_inputs(n, count, seed=1, dtype="fp32")
        errs = [torch.from_numpy(h).to(dev) for h in err_host]
        perrs = [e.clone() for e in errs]
    torch.cuda.synchronize()

    def reset_inputs():
        """Untimed: restore the initial values from the pristine device copies."""
        for b_, p_ in zip(bufs, pristine):
            b_.copy_(p_)
        if quant:
            for e_, p_ in zip(errs, perrs):
                e_.copy_(p_)
        torch.cuda.synchronize()
    log(f"inputs ready in {time.time() - t0:.1f}s: {desc}")

    stream = torch.cuda.current_stream(dev)
    if bucketed:
        run = lambda: B.ar_bucket_allreduce(plan, bufs, stream)  # noqa: E731
    elif quant:
        run = lambda: B.ar_allreduce_ef(plan, bufs, errs, stream)  # noqa: E731
    else:
        run = lambda: B.ar_allreduce(plan, bufs, stream)  # noqa: E731
    # ---- the timed run: the calls as a user makes them (no profiling), back
    # to back between two device synchronisations
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    ev0.record(stream)
    for c in range(args.steps):
        run()
    ev1.record(stream)
    torch.cuda.synchronize()
    t_end = time.perf_counter()
    wall_ms = (t_end - t_start) * 1e3 / max(args.steps, 1)
    ev_ms = ev0.elapsed_time(ev1) / max(args.steps, 1)
    ms = wall_ms

    # ---- per-call times (the nccl-tests convention): every call on the
    # pristine inputs, restored before it outside the timed interval, timed by
    # a HIP event pair around the call
    call_ms = []
    for c in range(args.steps):
        reset_inputs()
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record(stream)
        run()
        c1.record(stream)
        torch.cuda.synchronize()
        call_ms.append(c0.elapsed_time(c1))
    call_sorted = sorted(call_ms)
    median_ms = call_sorted[len(call_sorted) // 2] if len(call_sorted) % 2 else \
        0.5 * (call_sorted[len(call_sorted) // 2 - 1] + call_sorted[len(call_sorted) // 2])
    min_ms = call_sorted[0]

    # ---- the roofline run: the same calls again (inputs restored, untimed),
    # about four launches per call timed by start/stop events that the
    # launches record as part of their dispatch (every launch over `period`
    # calls), so the events barely perturb the calls they time
    nl = B.ar_plan_num_launches(lplan)
    shapes = [B.ar_plan_launch_shape(lplan, i) for i in range(nl)]
    lb = [launch_bytes(B, lplan, i, n, elem, count) for i in range(nl)]
    keys = [(kind, shapes[i]["cold"], shapes[i]["units"]) for i, (_, kind) in enumerate(lb)]
    labels = {k: kernel_label(k[0], shapes[i], n) for i, k in enumerate(keys)}
    staged_keys = {k for i, k in enumerate(keys) if shapes[i].get("lds_bytes")}  # LDS-staged one-pass folds
    period = max(1, nl // 4)

    def timed_run(evict=None):
        """Per-kernel-shape totals of one profiled run of W + K calls."""
        B.ar_plan_set_profiling(lplan, max(args.steps, 1))
        B.ar_plan_set_profiling_period(lplan, period)
        B.ar_plan_set_profiling_evict(lplan, evict, evict.numel() * 4 if evict is not None else 0)
        reset_inputs()
        for _ in range(args.warmup):
            run()
        torch.cuda.synchronize()
        B.ar_plan_launch_times(lplan)  # clear the warm-up entries
        t_p = time.perf_counter()
        for c in range(args.steps):
            run()
        torch.cuda.synchronize()
        run_ms = (time.perf_counter() - t_p) * 1e3 / max(args.steps, 1)
        times = B.ar_plan_launch_times(lplan)  # -1: launch not timed in that call (sampling)
        per = {}
        for call in times:
            for i, t in enumerate(call):
                if t < 0:
                    continue
                k = per.setdefault(keys[i], {"ms": 0.0, "launches": 0, "bytes": 0})
                k["ms"] += t
                k["launches"] += 1
                k["bytes"] += lb[i][0]
        means = []
        for i in range(nl):
            ts = [call[i] for call in times if call[i] >= 0]
            means.append(sum(ts) / len(ts) if ts else None)
        B.ar_plan_set_profiling_evict(lplan, None, 0)
        B.ar_plan_set_profiling(lplan, 0)
        return per, run_ms, means

    per_kind, prof_ms, means = timed_run()
    per_call_count, per_call_bytes = {}, {}
    for i, k in enumerate(keys):
        per_call_count[k] = per_call_count.get(k, 0) + 1
        per_call_bytes[k] = per_call_bytes.get(k, 0) + lb[i][0]
    # the kernel with the largest share of a call's GPU time
    dom = max(per_kind, key=lambda f: per_kind[f]["ms"] / per_kind[f]["launches"] * per_call_count[f])
    d = per_kind[dom]
    avg_ms = d["ms"] / d["launches"]
    bytes_per_launch = d["bytes"] / d["launches"]
    achieved = bytes_per_launch / (avg_ms * 1e-3) / 1e9
    traffic = traffic_record(labels[dom], args.workload, args.exec)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                "kernel": labels[dom],
                "avg_launch_ms": round(avg_ms, 5), "algorithmic_bytes_per_launch": int(bytes_per_launch),
                "launches_timed": d["launches"], "profiling_period": period}
    sum_launch_ms = sum(means) if all(m is not None for m in means) else None
    extra = {}
    prof_alg = count_logical * elem / (prof_ms * 1e-3) / 1e9
    extra["with_launch_events"] = {"exec": args.exec, "ms_per_step": round(prof_ms, 4),
                                   "busbw_GBps": round(prof_alg * 2 * (n - 1) / n, 1),
                                   "algbw_GBps": round(prof_alg, 1)}

    # ---- cold cache: the same profiled calls with 1 GiB written just before
    # every timed launch, so that the launch reads nothing from the device
    # cache; and the attainable bandwidth of each read/write mix on buffers far
    # larger than the cache
    per_cold, ceil = {}, None
    if not args.no_extra:
        evict = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        per_cold, _, _ = timed_run(evict)
        del evict
        torch.cuda.empty_cache()
        matched = []
        for k in per_call_count:  # each step-kernel shape's streams at its mean launch size
            st_ = kernel_streams(k[0])
            if st_ and per_kind.get(k):
                nb = per_call_bytes[k] // per_call_count[k] // sum(st_) // 16 * 16
                matched.append((f"{labels[k]} size", st_[0], st_[1], nb))
        # the one-pass mixes run on the workload's own buffers: the rank
        # buffers, and with error feedback the residual buffers as well (the
        # INT8 one-pass fold reads and writes both in place)
        ceil = probe_ceilings(B, torch, dev, stream, None if bucketed else bufs + (errs if quant else []),
                              count_logical * elem, reset_inputs, matched)
    per_kernel = []

    def share_of_call(k):
        v = per_kind.get(k)
        return v["ms"] / v["launches"] * per_call_count[k] if v else 0.0

    for k in sorted(per_call_count, key=lambda k: -share_of_call(k)):
        v = per_kind.get(k)
        row = {"kernel": labels[k], "launches_per_call": per_call_count[k], "bytes_per_call": per_call_bytes[k]}
        if not v:  # no launch of this shape was timed (sampling over few calls)
            per_kernel.append(row)
            continue
        rate = v["bytes"] / (v["ms"] * 1e-3) / 1e9
        row.update({"bytes_per_launch": int(v["bytes"] / v["launches"]),
                    "warm_ms": round(v["ms"] / v["launches"], 5), "warm_GBps": round(rate, 1),
                    "warm_frac_of_peak": round(rate / HBM_PEAK_GBPS, 4)})
        c = per_cold.get(k)
        if c:
            crate = c["bytes"] / (c["ms"] * 1e-3) / 1e9
            row.update({"cold_ms": round(c["ms"] / c["launches"], 5), "cold_GBps": round(crate, 1),
                        "cold_frac_of_peak": round(crate / HBM_PEAK_GBPS, 4)})
        if ceil:
            probe, att = attainable_for(ceil, k[0], elem, nbuf, staged=k in staged_keys)
            row.update({"attainable_probe": probe, "attainable_GBps": att,
                        "warm_frac_of_attainable": round(rate / att, 4)})
            if c:
                row["cold_frac_of_attainable"] = round(crate / att, 4)
            sm = ceil.get(f"{labels[k]} size")
            if sm:  # the same streams at this launch's size
                row.update({"size_matched_probe_GBps": sm["GBps"], "warm_frac_of_size_matched": round(rate / sm["GBps"], 4)})
        per_kernel.append(row)
        if k == dom:
            if ceil:
                roofline.update({"attainable_GBps": row["attainable_GBps"], "attainable_probe": probe,
                                 "frac_of_attainable": row["warm_frac_of_attainable"]})
                if "size_matched_probe_GBps" in row:
                    roofline.update({"size_matched_GBps": row["size_matched_probe_GBps"],
                                     "frac_of_size_matched": row["warm_frac_of_size_matched"]})
            if c:
                roofline["cold"] = {"avg_launch_ms": row["cold_ms"], "achieved": row["cold_GBps"],
                                    "frac": row["cold_frac_of_peak"],
                                    "frac_of_attainable": row.get("cold_frac_of_attainable")}
    log("per kernel:", json.dumps(per_kernel))

    # ---- buckets one by one, each with its own launches and a HIP event after
    # it (per-bucket times)
    per_bucket = None
    if bucketed:
        nb = B.ar_bucket_count(plan)
        B.ar_bucket_set_batching(plan, False)
        bucket_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(nb + 1)] for _ in range(args.steps)]
        for call in bucket_ev:
            for e in call:
                e.record(stream)  # creates the underlying events outside the timed region
        reset_inputs()
        for _ in range(args.warmup):
            run()
        torch.cuda.synchronize()
        t_b0 = time.perf_counter()
        for c in range(args.steps):
            bucket_ev[c][0].record(stream)
            B.ar_bucket_allreduce_after(plan, bufs, stream, None, bucket_ev[c][1:])
        torch.cuda.synchronize()
        obo_ms = (time.perf_counter() - t_b0) * 1e3 / max(args.steps, 1)
        B.ar_bucket_set_batching(plan, True)
        per_bucket = []
        for b in range(nb):
            t_b = sorted(call[b].elapsed_time(call[b + 1]) for call in bucket_ev)
            _, cnt = B.ar_bucket_range(plan, b)
            med = t_b[len(t_b) // 2]
            alg_b = cnt * elem / (med * 1e-3) / 1e9
            per_bucket.append({"bucket": b, "bytes_per_rank": cnt * elem, "median_ms": round(med, 4),
                               "algbw_GBps": round(alg_b, 1), "busbw_GBps": round(alg_b * 2 * (n - 1) / n, 1)})
        obo_alg = count_logical * elem / (obo_ms * 1e-3) / 1e9
        extra["buckets_one_by_one"] = {
            "ms_per_step": round(obo_ms, 4), "busbw_GBps": round(obo_alg * 2 * (n - 1) / n, 1),
            "algbw_GBps": round(obo_alg, 1), "launches_per_step": B.ar_bucket_stats(plan)["launches"]}

    S = count_logical * elem
    # ---- one-pass comparison on the same buffers (bit-identical results)
    if not args.no_extra and args.exec != "onepass":
        if bucketed:
            B.ar_bucket_set_exec(plan, "onepass")
            lplan = None  # rebuilt for the new mode
        else:
            B.ar_plan_set_exec(plan, "onepass")
        reset_inputs()
        for _ in range(args.warmup):
            run()
        torch.cuda.synchronize()
        t_a = time.perf_counter()
        for _ in range(args.steps):
            run()
        torch.cuda.synchronize()
        op_ms = (time.perf_counter() - t_a) * 1e3 / max(args.steps, 1)
        op_alg = S / (op_ms * 1e-3) / 1e9
        op_stats = B.ar_plan_stats(B.ar_bucket_batched_plan(plan) if bucketed else plan)
        op_gbps = op_stats["hbm_bytes_model"] / (op_ms * 1e-3) / 1e9
        extra["onepass"] = {"ms_per_step": round(op_ms, 4), "busbw_GBps": round(op_alg * 2 * (n - 1) / n, 1),
                            "algbw_GBps": round(op_alg, 1), "hbm_model_GBps": round(op_gbps, 1),
                            "hbm_model_frac_of_peak": round(op_gbps / HBM_PEAK_GBPS, 4)}
        if ceil:
            fold = [k for k in ceil if k == f"fold {nbuf}:{nbuf}"]
            extra["onepass"]["frac_of_copy_ceiling"] = round(op_gbps / ceil["copy 1:1"]["GBps"], 4)
            if fold:
                extra["onepass"]["frac_of_fold_probe"] = round(op_gbps / ceil[fold[0]]["GBps"], 4)
            staged = staged_bound(ceil, nbuf)
            if staged:  # the LDS-staged fold's two halves at their probe rates
                extra["onepass"]["staged_phases_GBps"] = staged
                extra["onepass"]["frac_of_staged_phases"] = round(op_gbps / staged, 4)

    # ---- the schedule's two halves on their own (ar_reduce_scatter,
    # ar_allgather), step mode, on the same buffers; nccl-tests convention:
    # algbw = S / T with S the bytes of one rank's whole buffer, busbw =
    # algbw * (N-1)/N (each half moves (N-1)/N * S per rank)
    if not args.no_extra and not bucketed and not quant and sched in ("ring", "hierarchical", "rabenseifner"):
        halves = {}
        for (coll, call), hmode in itertools.product((("reduce_scatter", B.ar_reduce_scatter),
                                                      ("allgather", B.ar_allgather)), ("steps", "onepass")):
            hp = B.ar_plan_create_collective(n, group, count, dtype, sched, coll)
            try:
                B.ar_plan_set_exec(hp, hmode)
                reset_inputs()
                for _ in range(args.warmup):
                    call(hp, bufs, stream)
                torch.cuda.synchronize()
                t_h = time.perf_counter()
                for _ in range(args.steps):
                    call(hp, bufs, stream)
                torch.cuda.synchronize()
                h_ms = (time.perf_counter() - t_h) * 1e3 / max(args.steps, 1)
                h_st = B.ar_plan_stats(hp)
            finally:
                B.ar_plan_destroy(hp)
            h_alg = S / (h_ms * 1e-3) / 1e9
            h_gbps = h_st["hbm_bytes_model"] / (h_ms * 1e-3) / 1e9
            halves[coll if hmode == "steps" else coll + "_onepass"] = {"ms_per_call": round(h_ms, 4), "busbw_GBps": round(h_alg * (n - 1) / n, 1),
                            "algbw_GBps": round(h_alg, 1), "launches": h_st["launches"], "rounds": h_st["steps"],
                            "hbm_model_GBps": round(h_gbps, 1),
                            "hbm_model_frac_of_peak": round(h_gbps / HBM_PEAK_GBPS, 4)}
        extra["halves"] = halves
        reset_inputs()

    # ---- the same exec mode replayed as one HIP graph per call
    if not args.no_extra:
        for name, graph in (("graph", True),):
            if bucketed:
                B.ar_bucket_set_exec(plan, args.exec)
                B.ar_bucket_set_graph(plan, graph)
            else:
                B.ar_plan_set_profiling(plan, 0)
                B.ar_plan_set_exec(plan, args.exec)
                B.ar_plan_set_graph(plan, graph)
            reset_inputs()
            for _ in range(args.warmup):
                run()
            torch.cuda.synchronize()
            t_g = time.perf_counter()
            for _ in range(args.steps):
                run()
            torch.cuda.synchronize()
            g_ms = (time.perf_counter() - t_g) * 1e3 / max(args.steps, 1)
            g_alg = S / (g_ms * 1e-3) / 1e9
            extra[name] = {"exec": args.exec, "ms_per_step": round(g_ms, 4),
                           "busbw_GBps": round(g_alg * 2 * (n - 1) / n, 1), "algbw_GBps": round(g_alg, 1)}

    # ---- CPU oracle on the same inputs (single-threaded C)
    cpu = None
    if not args.no_cpu_baseline:
        import oracle

        del bufs, errs, pristine, perrs
        torch.cuda.empty_cache()
        # repeat whole oracle runs (fresh copies of the inputs, copied outside
        # the timing) until about 10 s of CPU work, at most 30 s
        cpu_s, done, reps = 0.0, 0, 0
        nbk = B.ar_bucket_count(plan) if bucketed else 1
        while cpu_s < 10.0 and reps < 64:
            if bucketed:
                off, cnt = B.ar_bucket_range(plan, reps % nbk)
                xs = [h[off:off + cnt].copy() for h in host]
                t_c = time.perf_counter()
                oracle.run(xs, dtype, sched, group_size=group)
            elif quant:
                xs, es = [h.copy() for h in host], [h.copy() for h in err_host]
                t_c = time.perf_counter()
                oracle.run_int8ef(xs, sched, errs=es, group_size=group)
                cnt = count
            else:
                xs = [h.copy() for h in host]
                t_c = time.perf_counter()
                oracle.run(xs, dtype, sched, group_size=group)
                cnt = count
            cpu_s += time.perf_counter() - t_c
            done += cnt
            reps += 1
            del xs
            if cpu_s + cpu_s / reps > 30.0:
                break
        what = "buckets in order" if bucketed else "whole-workload all-reduces"
        if quant:
            what = "whole-workload compressed all-reduces with error feedback"
        sample = f"{reps} {what} ({done} elements per rank in total), timed without the input copies"
        cpu_alg = done * elem / cpu_s / 1e9
        cpu = {"value": round(cpu_alg * 2 * (n - 1) / n, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
               "sample": sample, "seconds": round(cpu_s, 2), "host_cpus": os.cpu_count(),
               "cpu_model": cpu_model(), "threads_used": 1}

    algbw = S / (ms * 1e-3) / 1e9
    busbw = algbw * 2 * (n - 1) / n
    stats = B.ar_plan_stats(B.ar_bucket_batched_plan(plan) if bucketed else plan)
    if bucketed:
        B.ar_bucket_set_exec(plan, args.exec)
        stats = B.ar_plan_stats(B.ar_bucket_batched_plan(plan))
    else:
        B.ar_plan_set_exec(plan, args.exec)
        stats = B.ar_plan_stats(plan)
    model_gbps = stats["hbm_bytes_model"] / (ms * 1e-3) / 1e9
    med_alg = S / (median_ms * 1e-3) / 1e9
    out = {
        "metric": METRIC,
        "value": round(busbw, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"fp32": "f32", "bf16": "bf16 (f32 accumulate)", "bf16_each": "bf16 (rounded each add)",
                  "int8_ef": "int8 codes + f32 block scales (f32 add per hop)"}[dtype],
        "data": "synthetic",
        "config": {
            "workload": desc, "schedule": sched, "nranks": n, "group_size": group, "dtype": dtype,
            "count_per_rank": count_logical, "bytes_per_rank": S, "exec": args.exec,
            "executor": ("buckets batched: every bucket's all-reduce in shared launches, " if bucketed else "")
            + f"eager launches; the roofline from a second run of the same calls, about four launches per "
            f"call timed by HIP events (every launch over {period} calls)",
            "algbw_GBps": round(algbw, 1), "busbw_GBps": round(busbw, 1),
            "median_ms": round(median_ms, 4), "min_ms": round(min_ms, 4),
            "median_busbw_GBps": round(med_alg * 2 * (n - 1) / n, 1),
            "per_call_protocol": f"{args.steps} calls, each on the inputs restored from pristine device copies "
                                 "outside its HIP-event interval",
            "hbm_model_bytes": stats["hbm_bytes_model"], "hbm_model_GBps": round(model_gbps, 1),
            "hbm_model_frac_of_peak": round(model_gbps / HBM_PEAK_GBPS, 4),
            "launches_per_step": stats["launches"], "schedule_steps": stats["steps"],
            "event_ms_per_step": round(ev_ms, 4),
            "kernel_ms_per_step": None if sum_launch_ms is None else round(sum_launch_ms, 4),
            "per_kernel": per_kernel,
        },
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    if ceil:
        out["config"]["hbm_ceiling"] = {k: {"GBps": v["GBps"], "units": v["units"], "policy": v["policy"],
                                            "bytes": v["bytes"]} for k, v in ceil.items()}
    if extra:
        out["config"]["compare"] = extra
    if quant:
        pf = B.ar_plan_create(n, group, count, "fp32", sched)
        sent_f32 = B.ar_plan_stats(pf)["bytes_sent_total"]
        B.ar_plan_destroy(pf)
        out["config"]["wire_bytes_total"] = stats["bytes_sent_total"]
        out["config"]["wire_compression_vs_fp32"] = round(sent_f32 / stats["bytes_sent_total"], 4)
    if bucketed:
        out["config"]["buckets"] = B.ar_bucket_count(plan)
        out["config"]["per_bucket_one_by_one"] = per_bucket
        B.ar_bucket_plan_destroy(plan)
    else:
        B.ar_plan_destroy(plan)
    print(json.dumps(out), flush=True)


def latency_main(args, B, np, torch):
    """Time per all-reduce by message size: 16 ranks of fp32, per rank 4 KiB,
    1 MiB and 16 MiB, for the ring, hierarchical 2 x 8, Rabenseifner and
    recursive doubling, in the step mode (eager, and replayed as a HIP graph)
    and the one-pass mode.  Each figure is the mean over back-to-back calls
    made through a prepared call (arguments checked and marshalled once), so
    it is the library's own cost per call: the launches' host and device
    start-up (the alpha of the pages' cost model on one GPU) plus the bytes.
    The step-mode points are also fitted to launches x alpha + model bytes / B."""
    n = 16
    dev = torch.device("cuda:0")
    s = torch.cuda.current_stream(dev)
    rows = []
    for per_rank in (4096, 1 << 20, 16 << 20):
        count = per_rank // 4
        bufs = [torch.randn(count, device=dev) for _ in range(n)]
        for sched, g in (("ring", 1), ("hierarchical", 8), ("rabenseifner", 1), ("recursive_doubling", 1)):
            for mode, graph in (("steps", False), ("steps", True), ("onepass", False)):
                p = B.ar_plan_create(n, g, count, "fp32", sched)
                B.ar_plan_set_exec(p, mode)
                B.ar_plan_set_graph(p, graph)
                call = B.prepared_call(p, bufs, None, s)
                reps = 400 if per_rank <= (1 << 20) else 100
                for _ in range(20):
                    call()
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                for _ in range(reps):
                    call()
                torch.cuda.synchronize()
                us = (time.perf_counter() - t0) / reps * 1e6
                st = B.ar_plan_stats(p)
                B.ar_plan_destroy(p)
                rows.append({"bytes_per_rank": per_rank, "schedule": sched, "exec": mode, "graph": graph,
                             "launches": st["launches"], "hbm_model_bytes": st["hbm_bytes_model"],
                             "us_per_call": round(us, 2)})
                log(json.dumps(rows[-1]))
        del bufs
    # least squares over the eager step-mode points: us = launches * alpha + bytes / B
    pts = [r for r in rows if r["exec"] == "steps" and not r["graph"]]
    A = np.array([[r["launches"], r["hbm_model_bytes"] / 1e9] for r in pts], dtype=np.float64)
    y = np.array([r["us_per_call"] for r in pts], dtype=np.float64)
    (alpha_us, inv_b), *_ = np.linalg.lstsq(A, y, rcond=None)
    one = [r["us_per_call"] for r in rows if r["exec"] == "onepass" and r["bytes_per_rank"] == 4096]
    out = {"metric": "all-reduce time per call, 16 ranks fp32, 4 KiB per rank, one-pass mode", "value": min(one),
           "unit": "us", "n_gpus": 1, "steps": None, "warmup": 20, "ms_per_step": round(min(one) / 1e3, 5),
           "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
           "config": {"workload": "latency sweep: 16 ranks fp32, 4 KiB / 1 MiB / 16 MiB per rank, ring, "
                                  "hierarchical 2x8, Rabenseifner, recursive doubling; step mode eager and graph, "
                                  "one-pass", "rows": rows,
                      "fit_alpha_us_per_launch": round(float(alpha_us), 3),
                      "fit_bandwidth_GBps": round(1e6 / float(inv_b), 1) if inv_b > 0 else None},
           "roofline": None, "cpu_baseline": None}
    print(json.dumps(out), flush=True)


def overlap_main(args, B, workloads, np, torch):
    """Bucketed all-reduces overlapped with a simulated backward pass.

    The backward of bucket b is a spin kernel on a producer stream lasting
    compute_ratio times the bucket's measured all-reduce time (it uses no
    memory bandwidth, like the non-contending compute of the overlap model),
    after which the bucket's ready event is recorded.  The all-reduces run on
    a second stream, each gated on its ready event (ar_bucket_allreduce_after).
    Reported: the measured communication left after the backward ends, next
    to the overlap model's prediction from the measured ready times and
    per-bucket all-reduce times (Primer ch. 4 section 4.7, Figure 4.15).
    """
    n, sched, dtype = 16, "ring", "bf16"
    sizes = workloads.bucketed_tensor_sizes(elem_bytes=2)
    bp = B.ar_bucket_plan_create(n, 1, sizes, dtype, sched, 25 << 20)
    offsets, arena = B.ar_bucket_layout(bp, len(sizes))
    host = workloads.bucketed_arenas(n, sizes, offsets, arena, dtype="bf16")
    bufs = [torch.from_numpy(h.view(np.int16)).cuda() for h in host]
    nb = B.ar_bucket_count(bp)
    producer, consumer = torch.cuda.Stream(), torch.cuda.Stream()
    # 1) per-bucket all-reduce times, back to back, no gating
    done = [torch.cuda.Event(enable_timing=True) for _ in range(nb)]
    start = torch.cuda.Event(enable_timing=True)
    for _ in range(args.warmup):
        B.ar_bucket_allreduce(bp, bufs, consumer)
    torch.cuda.synchronize()
    comm = np.zeros(nb)
    for _ in range(args.steps):
        start.record(consumer)
        B.ar_bucket_allreduce_after(bp, bufs, consumer, None, done)
        torch.cuda.synchronize()
        prev = start
        for b in range(nb):
            comm[b] += prev.elapsed_time(done[b]) / args.steps
            prev = done[b]
    # 2) spin-kernel cycles per ms
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(producer):
        torch.cuda._sleep(1_000_000)
        t0.record(producer)
        torch.cuda._sleep(20_000_000)
        t1.record(producer)
    torch.cuda.synchronize()
    cycles_per_ms = 20_000_000 / t0.elapsed_time(t1)
    # 3) overlapped runs
    ready = [torch.cuda.Event(enable_timing=True) for _ in range(nb)]
    exposed_meas, exposed_model, step_meas = [], [], []
    for it in range(args.steps + args.warmup):
        torch.cuda.synchronize()
        begin = torch.cuda.Event(enable_timing=True)
        bwd_end = torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(producer):
            begin.record(producer)
            for b in range(nb):
                torch.cuda._sleep(max(1, int(args.compute_ratio * comm[b] * cycles_per_ms)))
                ready[b].record(producer)
            bwd_end.record(producer)
        consumer.wait_event(begin)
        B.ar_bucket_allreduce_after(bp, bufs, consumer, ready, done)
        torch.cuda.synchronize()
        if it < args.warmup:
            continue
        r = [begin.elapsed_time(e) for e in ready]
        comp_end = begin.elapsed_time(bwd_end)
        comm_end = begin.elapsed_time(done[-1])
        exposed_meas.append(max(0.0, comm_end - comp_end))
        step_meas.append(max(comp_end, comm_end))
        _, ex = B.ar_overlap_step_time([x * 1e-3 for x in r], [c * 1e-3 for c in comm], comp_end * 1e-3, 0.0)
        exposed_model.append(ex * 1e3)
    S = int(np.sum(sizes)) * 2
    out = {
        "metric": "exposed all-reduce time after backward (bucketed, overlapped)",
        "value": round(float(np.median(exposed_meas)), 4), "unit": "ms", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(float(np.median(step_meas)), 4), "higher_is_better": False,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16 (f32 accumulate)", "data": "synthetic",
        "config": {"workload": "ring all-reduce, 16 ranks, 300 lognormal bf16 tensors in 25 MiB buckets, each "
                               "gated on its bucket's backward (spin kernel of compute_ratio x its all-reduce time)",
                   "buckets": nb, "bytes_per_rank": S, "compute_ratio": args.compute_ratio,
                   "allreduce_ms_per_bucket": [round(c, 4) for c in comm],
                   "allreduce_ms_total": round(float(comm.sum()), 4),
                   "exposed_ms_model": round(float(np.median(exposed_model)), 4),
                   "backward_ms": round(float(np.median([s_ - e_ for s_, e_ in zip(step_meas, exposed_meas)])), 4),
                   "last_bucket_allreduce_ms": round(float(comm[-1]), 4)},
        "roofline": None, "cpu_baseline": None,
    }
    B.ar_bucket_plan_destroy(bp)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
