"""CPU oracle for the gradient all-reduce schedules (ctypes wrapper).

TEST INFRASTRUCTURE ONLY.  Only tests, the smoke check and the benchmark's
CPU-baseline leg may import this package.  It shares no code with the GPU
library: the simulation itself is plain C in ar_oracle.c.

Schedules and datatypes use the oracle's own numbering:
  schedule: "ring" | "hierarchical" | "rabenseifner" | "recursive_doubling" | "tree" |
            "double_tree"
  dtype:    "fp32" (numpy float32 buffers) | "bf16" (numpy uint16 buffers of bf16 bits,
            fp32 partial sums, one rounding) | "bf16_each" (uint16 buffers, every
            partial sum rounded to bf16 as it is formed)
run_int8ef: the compressed all-reduce (blockwise INT8 messages, error feedback)
            on float32 buffers.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_SCHED = {"ring": 0, "hierarchical": 1, "rabenseifner": 2, "recursive_doubling": 3, "tree": 4,
          "double_tree": 5}
_DTYPE = {"fp32": 0, "bf16": 1, "bf16_each": 2}
_ELEM = {"fp32": 4, "bf16": 2, "bf16_each": 2}
REDUCE, COPY = 0, 1

_lib = None


def lib(path=None):
    """Loads liboracle.so, building it with gcc first if it is missing."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        override = os.environ.get("ARO_LIB")  # used by the mutation test only
        if override:
            _lib = _bind(ctypes.CDLL(override))
        else:
            if not os.path.exists(_build.LIB):
                _build.build()
            _lib = _bind(ctypes.CDLL(_build.LIB))
    return _lib


def _bind(L):
    i64, i32, dbl = ctypes.c_longlong, ctypes.c_int, ctypes.c_double
    P = ctypes.c_void_p
    L.aro_steps.argtypes = [i32, i32, i64, i32]
    L.aro_steps.restype = i32
    L.aro_num_messages.argtypes = [i32, i32, i64, i32]
    L.aro_num_messages.restype = i64
    L.aro_messages.argtypes = [i32, i32, i64, i32, P, P, P, P, P, P, P, i64]
    L.aro_messages.restype = i64
    L.aro_stats.argtypes = [i32, i32, i64, i32, i32, P, P]
    L.aro_stats.restype = i32
    L.aro_cost.argtypes = [i32, i32, i64, i32, i32, dbl, dbl, dbl]
    L.aro_cost.restype = dbl
    L.aro_cost_ex.argtypes = [i32, i32, i64, i32, i32, dbl, dbl, dbl, dbl, dbl, dbl]
    L.aro_cost_ex.restype = dbl
    L.aro_run_int8ef.argtypes = [i32, i32, i64, i32, P, P, i32]
    L.aro_run_int8ef.restype = i32
    L.aro_run.argtypes = [i32, i32, i64, i32, i32, P, i32]
    L.aro_run.restype = i32
    L.aro_run_rounds.argtypes = [i32, i32, i64, i32, i32, P, i32, i32]
    L.aro_run_rounds.restype = i32
    return L


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


class OracleError(RuntimeError):
    pass


def steps(nranks, schedule, count=0, group_size=1, L=None):
    n = (L or lib()).aro_steps(nranks, group_size, count, _SCHED[schedule])
    if n < 0:
        raise OracleError(f"aro_steps failed ({n})")
    return n


def messages(nranks, count, schedule, group_size=1, L=None):
    """Returns the message list as a dict of numpy arrays (one entry per message)."""
    L = L or lib()
    n = L.aro_num_messages(nranks, group_size, count, _SCHED[schedule])
    if n < 0:
        raise OracleError(f"aro_num_messages failed ({n})")
    out = {k: np.zeros(max(n, 1), np.int32) for k in ("step", "src", "dst", "kind", "completes")}
    out.update({k: np.zeros(max(n, 1), np.int64) for k in ("lo", "hi")})
    got = L.aro_messages(nranks, group_size, count, _SCHED[schedule],
                         *[_ptr(out[k]) for k in ("step", "src", "dst", "lo", "hi", "kind", "completes")],
                         n)
    if got != n:
        raise OracleError("aro_messages size mismatch")
    return {k: v[:n] for k, v in out.items()}


def stats(nranks, count, dtype, schedule, group_size=1, L=None):
    """(bytes_sent per rank [uint64 array], cross_group_bytes, steps)."""
    L = L or lib()
    sent = np.zeros(nranks, np.uint64)
    cross = np.zeros(1, np.uint64)
    n = L.aro_stats(nranks, group_size, count, _ELEM[dtype], _SCHED[schedule], _ptr(sent), _ptr(cross))
    if n < 0:
        raise OracleError(f"aro_stats failed ({n})")
    return sent, int(cross[0]), n


def cost(nranks, count_bytes_elems, elem_bytes, schedule, alpha_s, bw_intra, bw_cross,
         group_size=1, L=None):
    """Per-round alpha-beta time in seconds ([DCN] 7.2.1 resource model)."""
    t = (L or lib()).aro_cost(nranks, group_size, count_bytes_elems, elem_bytes, _SCHED[schedule],
                              alpha_s, bw_intra, bw_cross)
    if t < 0:
        raise OracleError(f"aro_cost failed ({t})")
    return t


def cost_ex(nranks, count, elem_bytes, schedule, alpha_intra, alpha_cross, bw_intra, bw_cross,
            bw_egress=0.0, share=1.0, group_size=1, L=None):
    """[DCN] 7.6.4 resource model: per-round start-up by link class, shared group egress."""
    t = (L or lib()).aro_cost_ex(nranks, group_size, count, elem_bytes, _SCHED[schedule], alpha_intra, alpha_cross,
                                 bw_intra, bw_cross, bw_egress, share)
    if t < 0:
        raise OracleError(f"aro_cost_ex failed ({t})")
    return t


def run(bufs, dtype, schedule, group_size=1, max_steps=-1, L=None):
    """Runs the schedule in place on a list of equal-length host arrays."""
    L = L or lib()
    want = np.float32 if dtype == "fp32" else np.uint16
    n = len(bufs)
    count = len(bufs[0]) if n else 0
    for b in bufs:
        if b.dtype != want or not b.flags.c_contiguous or len(b) != count:
            raise OracleError("buffers must be contiguous, equal length, of the dtype's storage type")
    arr = (ctypes.c_void_p * n)(*[b.ctypes.data for b in bufs])
    rc = L.aro_run(n, group_size, count, _DTYPE[dtype], _SCHED[schedule],
                   ctypes.cast(arr, ctypes.c_void_p), max_steps)
    if rc != 0:
        raise OracleError(f"aro_run failed ({rc})")
    return bufs


def run_rounds(bufs, dtype, schedule, group_size=1, first_step=0, end_step=-1, L=None):
    """Runs rounds first_step .. end_step-1 in place (end_step < 0: to the
    last round); the buffers stand for the state the earlier rounds left."""
    L = L or lib()
    want = np.float32 if dtype == "fp32" else np.uint16
    n = len(bufs)
    count = len(bufs[0]) if n else 0
    for b in bufs:
        if b.dtype != want or not b.flags.c_contiguous or len(b) != count:
            raise OracleError("buffers must be contiguous, equal length, of the dtype's storage type")
    arr = (ctypes.c_void_p * max(n, 1))(*[b.ctypes.data for b in bufs])
    rc = L.aro_run_rounds(n, group_size, count, _DTYPE[dtype], _SCHED[schedule],
                          ctypes.cast(arr, ctypes.c_void_p), first_step, end_step)
    if rc != 0:
        raise OracleError(f"aro_run_rounds failed ({rc})")
    return bufs


HALVES = ("ring", "hierarchical", "rabenseifner")


def reduce_scatter_rounds(nranks, schedule, count=0, group_size=1, L=None):
    """Number of leading rounds whose messages are reduces: the
    reduce-scatter half ([PRIMER] 4.2; [SCALING] "Six basic primitives")."""
    if schedule not in HALVES:
        raise OracleError(f"{schedule} has no reduce-scatter half")
    m = messages(nranks, count, schedule, group_size, L=L)
    reduce_steps = sorted({int(s) for s, k in zip(m["step"], m["kind"]) if k == REDUCE})
    if reduce_steps != list(range(len(reduce_steps))) or any(
            k == REDUCE for s, k in zip(m["step"], m["kind"]) if s >= len(reduce_steps)):
        raise OracleError("the reduce rounds are not a prefix of the schedule")
    if any(k != REDUCE for s, k in zip(m["step"], m["kind"]) if s < len(reduce_steps)):
        raise OracleError("a reduce round also copies")
    return len(reduce_steps)


def owned_ranges(nranks, count, schedule, group_size=1, L=None):
    """[(lo, hi)] per rank: the range the receiver of each completing reduce
    holds complete after the reduce-scatter half; everything for one rank."""
    if schedule not in HALVES:
        raise OracleError(f"{schedule} has no reduce-scatter half")
    if nranks == 1:
        return [(0, count)]
    m = messages(nranks, count, schedule, group_size, L=L)
    out = [None] * nranks
    for dst, lo, hi, kind, done in zip(m["dst"], m["lo"], m["hi"], m["kind"], m["completes"]):
        if kind == REDUCE and done:
            if out[dst] is not None:
                raise OracleError(f"rank {dst} completes two ranges")
            out[dst] = (int(lo), int(hi))
    if any(o is None for o in out):
        raise OracleError("a rank completes no range")
    return out


def reduce_scatter(bufs, dtype, schedule, group_size=1, L=None):
    """The reduce-scatter half in place; rank r's owned range then holds the
    all-reduce's values."""
    k = reduce_scatter_rounds(len(bufs), schedule, len(bufs[0]) if bufs else 0, group_size, L=L)
    return run_rounds(bufs, dtype, schedule, group_size, 0, k, L=L)


def allgather(bufs, dtype, schedule, group_size=1, L=None):
    """The all-gather half in place: every rank's owned range goes to every
    other rank."""
    k = reduce_scatter_rounds(len(bufs), schedule, len(bufs[0]) if bufs else 0, group_size, L=L)
    return run_rounds(bufs, dtype, schedule, group_size, k, -1, L=L)


QBLOCK = 128


def run_int8ef(bufs, schedule, errs=None, group_size=1, max_steps=-1, L=None):
    """Blockwise-INT8 all-reduce with error feedback, in place on float32
    host arrays; errs (float32 arrays, updated in place) or None."""
    L = L or lib()
    n = len(bufs)
    count = len(bufs[0]) if n else 0
    for b in list(bufs) + list(errs or []):
        if b.dtype != np.float32 or not b.flags.c_contiguous or len(b) != count:
            raise OracleError("buffers must be contiguous float32 arrays of equal length")
    ab = (ctypes.c_void_p * max(n, 1))(*[b.ctypes.data for b in bufs])
    ae = (ctypes.c_void_p * max(n, 1))(*[e.ctypes.data for e in errs]) if errs is not None else None
    rc = L.aro_run_int8ef(n, group_size, count, _SCHED[schedule], ctypes.cast(ab, ctypes.c_void_p),
                          ctypes.cast(ae, ctypes.c_void_p) if ae is not None else None, max_steps)
    if rc != 0:
        raise OracleError(f"aro_run_int8ef failed ({rc})")
    return bufs
