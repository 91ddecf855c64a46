"""ctypes binding of libar.so: the C ABI of include/ar.h under the same names.

Argument marshalling only: every step of the all-reduce runs in the HIP
kernels of libar.so.  There is no fallback; if the library is missing or
fails to load, every call raises.

Device pointers may be passed as ints or as objects with a ``data_ptr()``
method (torch tensors); streams as ints, None (default stream) or objects
with a ``cuda_stream`` attribute (torch streams).
"""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# AR_LIB names another build of the same sources (the sanitizer build of the
# CPU tests); there is no other implementation to fall back to.
LIB_PATH = os.environ.get("AR_LIB") or os.path.join(_HERE, "libar.so")

AR_OK, AR_ERR_INVALID_ARG, AR_ERR_UNSUPPORTED, AR_ERR_OOM, AR_ERR_HIP, AR_ERR_GUARD = range(6)
AR_FLOAT32, AR_BFLOAT16, AR_BFLOAT16_EACH_STEP, AR_INT8_EF = 0, 1, 2, 3
AR_RING, AR_HIERARCHICAL, AR_RABENSEIFNER, AR_RECURSIVE_DOUBLING, AR_TREE, AR_DOUBLE_TREE = range(6)
AR_EXEC_STEPS, AR_EXEC_STEPS_UNFUSED, AR_EXEC_ONEPASS = 0, 1, 2
AR_MAX_RANKS = 64
AR_MAX_PLAN_RANKS = 1024
AR_NOALLOC_SCRATCH_BYTES = 64 << 20

DTYPES = {"fp32": AR_FLOAT32, "bf16": AR_BFLOAT16, "bf16_each": AR_BFLOAT16_EACH_STEP, "int8_ef": AR_INT8_EF}
SCHEDULES = {"ring": AR_RING, "hierarchical": AR_HIERARCHICAL, "rabenseifner": AR_RABENSEIFNER,
             "recursive_doubling": AR_RECURSIVE_DOUBLING, "tree": AR_TREE, "double_tree": AR_DOUBLE_TREE}
EXECS = {"steps": AR_EXEC_STEPS, "steps_unfused": AR_EXEC_STEPS_UNFUSED, "onepass": AR_EXEC_ONEPASS}
AR_ALLREDUCE, AR_REDUCE_SCATTER, AR_ALLGATHER = range(3)
COLLECTIVES = {"allreduce": AR_ALLREDUCE, "reduce_scatter": AR_REDUCE_SCATTER, "allgather": AR_ALLGATHER}

# kernel kind codes reported by ar_plan_launch_info
KIND_REDUCE, KIND_COPY, KIND_RING, KIND_HIER, KIND_TREE, KIND_DTREE = 0x100, 0x200, 0x300, 0x400, 0x500, 0x600
KIND_QENCODE, KIND_QREDUCE, KIND_QCOPY, KIND_QDECODE = 0x700, 0x800, 0x900, 0xA00
KIND_FAN = 0xB00
KIND_OWNER = 0x1000  # flag: a one-pass fold that stores each op's result into its owner only
QBLOCK = 128
LOC_SCRATCH = 1000


class ArError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"ar status {status}: {message}")
        self.status = status


class ar_cost_params_t(ctypes.Structure):
    _fields_ = [("alpha_intra_s", ctypes.c_double), ("alpha_cross_s", ctypes.c_double),
                ("bw_intra_Bps", ctypes.c_double), ("bw_cross_Bps", ctypes.c_double),
                ("bw_group_egress_Bps", ctypes.c_double), ("egress_share", ctypes.c_double)]


class ar_stats_t(ctypes.Structure):
    _fields_ = [
        ("nranks", ctypes.c_int32), ("group_size", ctypes.c_int32),
        ("steps", ctypes.c_uint32), ("launches", ctypes.c_uint32),
        ("count", ctypes.c_uint64), ("elem_bytes", ctypes.c_uint64),
        ("bytes_sent", ctypes.POINTER(ctypes.c_uint64)),
        ("bytes_sent_max", ctypes.c_uint64), ("bytes_sent_total", ctypes.c_uint64),
        ("cross_group_bytes_total", ctypes.c_uint64),
        ("hbm_bytes_model", ctypes.c_uint64),
        ("scratch_bytes", ctypes.c_uint64),
        ("exec", ctypes.c_int32),
    ]

    def to_dict(self):
        d = {k: getattr(self, k) for k, _ in self._fields_ if k != "bytes_sent"}
        d["bytes_sent"] = [self.bytes_sent[i] for i in range(self.nranks)] if self.bytes_sent else []
        return d


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
        _lib = _declare(ctypes.CDLL(LIB_PATH))
    return _lib


def _declare(L):
    P, i32, i64, u64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64
    sz, dbl = ctypes.c_size_t, ctypes.c_double
    pi32, pi64, pf, psz = (ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int64),
                           ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_size_t))
    sig = {
        "ar_plan_create": ([ctypes.c_int, ctypes.c_int, sz, ctypes.c_int, ctypes.c_int], P),
        "ar_plan_create_collective": ([ctypes.c_int, ctypes.c_int, sz, ctypes.c_int, ctypes.c_int, ctypes.c_int], P),
        "ar_plan_owned_range": ([P, ctypes.c_int, psz, psz], ctypes.c_int),
        "ar_reduce_scatter": ([P, P, P], ctypes.c_int),
        "ar_allgather": ([P, P, P], ctypes.c_int),
        "ar_plan_set_exec": ([P, ctypes.c_int], ctypes.c_int),
        "ar_plan_prepare": ([P], ctypes.c_int),
        "ar_allreduce": ([P, P, P], ctypes.c_int),
        "ar_allreduce_ef": ([P, P, P, P], ctypes.c_int),
        "ar_allreduce_noalloc": ([P, P, P, P], ctypes.c_int),
        "ar_plan_stats": ([P], ar_stats_t),
        "ar_plan_cost_alpha_beta": ([P, dbl, dbl, dbl], dbl),
        "ar_plan_cost_alpha_beta_ex": ([P, ctypes.POINTER(ar_cost_params_t)], dbl),
        "ar_plan_destroy": ([P], None),
        "ar_select_schedule": ([ctypes.c_int, ctypes.c_int, sz, ctypes.c_int, ctypes.POINTER(ar_cost_params_t),
                                ctypes.c_uint32, ctypes.POINTER(ctypes.c_double)], ctypes.c_int),
        "ar_last_error": ([], ctypes.c_char_p),
        "ar_last_status": ([], ctypes.c_int),
        "ar_plan_transfers": ([P, pi32, pi32, pi32, pi64, pi64, pi32, i64], i64),
        "ar_plan_num_launches": ([P], i32),
        "ar_plan_launch_info": ([P, i32, pi32, pi32], ctypes.c_int),
        "ar_plan_launch_ops": ([P, i32, pi64, pi64, pi32, pi32, pi32, pi32, pi32], ctypes.c_int),
        "ar_plan_launch_scratch": ([P, i32, pi64, pi64], ctypes.c_int),
        "ar_plan_set_profiling": ([P, ctypes.c_int], ctypes.c_int),
        "ar_plan_set_profiling_period": ([P, ctypes.c_int], ctypes.c_int),
        "ar_plan_set_profiling_evict": ([P, P, sz], ctypes.c_int),
        "ar_plan_describe": ([P, ctypes.c_char_p, sz], i64),
        "ar_plan_set_guard": ([P, sz], ctypes.c_int),
        "ar_plan_check_guards": ([P], ctypes.c_int),
        "ar_bucket_set_guard": ([P, sz], ctypes.c_int),
        "ar_bucket_check_guards": ([P], ctypes.c_int),
        "ar_plan_launch_shape": ([P, i32, pi32, pi32, pi32, pi32, ctypes.POINTER(ctypes.c_uint32), pi32, pi32],
                                 ctypes.c_int),
        "ar_hbm_probe": ([P, i32, P, i32, sz, i32, i32, P], ctypes.c_int),
        "ar_plan_set_graph": ([P, ctypes.c_int], ctypes.c_int),
        "ar_plan_set_cache_bytes": ([P, sz], ctypes.c_int),
        "ar_bucket_set_graph": ([P, ctypes.c_int], ctypes.c_int),
        "ar_plan_launch_times": ([P, pf, i32, pi32], ctypes.c_int),
        "ar_bucket_plan_create": ([ctypes.c_int, ctypes.c_int, psz, ctypes.c_int, ctypes.c_int, ctypes.c_int, sz], P),
        "ar_bucket_layout": ([P, psz, psz], ctypes.c_int),
        "ar_bucket_count": ([P], i32),
        "ar_bucket_range": ([P, i32, psz, psz], ctypes.c_int),
        "ar_bucket_set_exec": ([P, ctypes.c_int], ctypes.c_int),
        "ar_bucket_set_batching": ([P, ctypes.c_int], ctypes.c_int),
        "ar_bucket_set_cache_bytes": ([P, sz], ctypes.c_int),
        "ar_bucket_batched_plan": ([P], P),
        "ar_bucket_allreduce": ([P, P, P], ctypes.c_int),
        "ar_bucket_allreduce_after": ([P, P, P, P, P], ctypes.c_int),
        "ar_bucket_allreduce_ef": ([P, P, P, P, P, P], ctypes.c_int),
        "ar_overlap_step_time": ([ctypes.c_int, ctypes.POINTER(dbl), ctypes.POINTER(dbl), dbl, dbl,
                                  ctypes.POINTER(dbl)], dbl),
        "ar_bucket_stats": ([P], ar_stats_t),
        "ar_bucket_plan_destroy": ([P], None),
    }
    for name, (args, res) in sig.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = res
    del u64
    return L


def _raise():
    L = lib()
    raise ArError(L.ar_last_status(), L.ar_last_error().decode())


def _check(st):
    if st != AR_OK:
        _raise()


def _ptr(x):
    if x is None:
        return 0
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    return int(x)


def _stream(s):
    if s is None:
        return None
    if hasattr(s, "cuda_stream"):
        return s.cuda_stream
    return int(s)


def _ptr_array(bufs):
    return (ctypes.c_void_p * max(len(bufs), 1))(*[_ptr(b) for b in bufs])


def _check_bufs(bufs, nranks, nbytes, what):
    """The C calls read exactly nranks pointers from the host array and let
    the kernels touch nbytes of each buffer, so a short list or a short
    tensor would make them read or write past the end.  Raises ValueError
    unless there are nranks buffers and every tensor among them is a
    contiguous device tensor of at least nbytes.  Plain integers are device
    addresses whose extent cannot be checked here."""
    if bufs is None:
        raise ValueError(f"{what}s: None")
    if len(bufs) != nranks:
        raise ValueError(f"{len(bufs)} {what}s for a plan of {nranks} ranks")
    for r, b in enumerate(bufs):
        if not hasattr(b, "data_ptr"):
            continue
        if not getattr(b, "is_cuda", False):
            raise ValueError(f"{what} {r} is not a device tensor")
        if not b.is_contiguous():
            raise ValueError(f"{what} {r} is not contiguous")
        have = b.numel() * b.element_size()
        if have < nbytes:
            raise ValueError(f"{what} {r} holds {have} bytes; the plan reads and writes {nbytes}")


def _plan_extent(plan):
    """(nranks, bytes of each rank buffer, bytes of each error buffer)."""
    s = lib().ar_plan_stats(plan)
    return s.nranks, s.count * s.elem_bytes, s.count * 4


def _bucket_extent(bp):
    """(nranks, bytes of each rank arena, bytes of each error arena)."""
    s = lib().ar_bucket_stats(bp)
    arena = ctypes.c_size_t()
    _check(lib().ar_bucket_layout(bp, None, ctypes.byref(arena)))
    return s.nranks, arena.value * s.elem_bytes, arena.value * 4


def _code(table, v):
    return table[v] if isinstance(v, str) else int(v)


# ------------------------------------------------------------------ plans

def ar_plan_create(nranks, group_size, count, dtype, schedule):
    p = lib().ar_plan_create(nranks, group_size, count, _code(DTYPES, dtype), _code(SCHEDULES, schedule))
    if not p:
        _raise()
    return p


def ar_plan_create_collective(nranks, group_size, count, dtype, schedule, collective):
    """collective: "allreduce", "reduce_scatter" or "allgather"."""
    p = lib().ar_plan_create_collective(nranks, group_size, count, _code(DTYPES, dtype), _code(SCHEDULES, schedule),
                                        _code(COLLECTIVES, collective))
    if not p:
        _raise()
    return p


def ar_plan_owned_range(plan, rank):
    """(lo, hi): the elements `rank` holds complete after the reduce-scatter."""
    lo, hi = ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().ar_plan_owned_range(plan, rank, ctypes.byref(lo), ctypes.byref(hi)))
    return lo.value, hi.value


def ar_plan_set_exec(plan, exec_mode):
    _check(lib().ar_plan_set_exec(plan, _code(EXECS, exec_mode)))


def ar_plan_set_cache_bytes(plan, nbytes):
    _check(lib().ar_plan_set_cache_bytes(plan, nbytes))


def ar_plan_set_graph(plan, enable=True):
    _check(lib().ar_plan_set_graph(plan, 1 if enable else 0))


def ar_plan_prepare(plan):
    _check(lib().ar_plan_prepare(plan))


def ar_allreduce(plan, rank_bufs, stream=None):
    if plan:
        n, nbytes, _ = _plan_extent(plan)
        _check_bufs(rank_bufs, n, nbytes, "rank buffer")
    arr = _ptr_array(rank_bufs)
    _check(lib().ar_allreduce(plan, ctypes.cast(arr, ctypes.c_void_p), _stream(stream)))


def ar_reduce_scatter(plan, rank_bufs, stream=None):
    if plan:
        n, nbytes, _ = _plan_extent(plan)
        _check_bufs(rank_bufs, n, nbytes, "rank buffer")
    arr = _ptr_array(rank_bufs)
    _check(lib().ar_reduce_scatter(plan, ctypes.cast(arr, ctypes.c_void_p), _stream(stream)))


def ar_allgather(plan, rank_bufs, stream=None):
    if plan:
        n, nbytes, _ = _plan_extent(plan)
        _check_bufs(rank_bufs, n, nbytes, "rank buffer")
    arr = _ptr_array(rank_bufs)
    _check(lib().ar_allgather(plan, ctypes.cast(arr, ctypes.c_void_p), _stream(stream)))


def ar_allreduce_ef(plan, rank_bufs, error_bufs, stream=None):
    """error_bufs: per-rank fp32 residual buffers, or None (no error feedback)."""
    if plan:
        n, nbytes, ebytes = _plan_extent(plan)
        _check_bufs(rank_bufs, n, nbytes, "rank buffer")
        if error_bufs is not None:
            _check_bufs(error_bufs, n, ebytes, "error buffer")
    arr = _ptr_array(rank_bufs)
    err = ctypes.cast(_ptr_array(error_bufs), ctypes.c_void_p) if error_bufs is not None else None
    _check(lib().ar_allreduce_ef(plan, ctypes.cast(arr, ctypes.c_void_p), err, _stream(stream)))


def ar_allreduce_noalloc(plan, rank_bufs, error_bufs=None, stream=None):
    """The all-reduce with its device workspace in the library's fixed array
    (AR_NOALLOC_SCRATCH_BYTES per GPU): allocates nothing."""
    if plan:
        n, nbytes, ebytes = _plan_extent(plan)
        _check_bufs(rank_bufs, n, nbytes, "rank buffer")
        if error_bufs is not None:
            _check_bufs(error_bufs, n, ebytes, "error buffer")
    arr = _ptr_array(rank_bufs)
    err = ctypes.cast(_ptr_array(error_bufs), ctypes.c_void_p) if error_bufs is not None else None
    _check(lib().ar_allreduce_noalloc(plan, ctypes.cast(arr, ctypes.c_void_p), err, _stream(stream)))


def prepared_call(plan, rank_bufs, error_bufs=None, stream=None, noalloc=False):
    """A zero-argument callable that runs ar_allreduce_ef (or, with noalloc,
    ar_allreduce_noalloc) on these buffers: the arguments are checked and
    marshalled once, for loops that repeat the same call.  The tensors must
    keep their storage while the callable is used (it holds references to
    them)."""
    n, nbytes, ebytes = _plan_extent(plan)
    _check_bufs(rank_bufs, n, nbytes, "rank buffer")
    if error_bufs is not None:
        _check_bufs(error_bufs, n, ebytes, "error buffer")
    arr = ctypes.cast(_ptr_array(rank_bufs), ctypes.c_void_p)
    err = ctypes.cast(_ptr_array(error_bufs), ctypes.c_void_p) if error_bufs is not None else None
    fn = lib().ar_allreduce_noalloc if noalloc else lib().ar_allreduce_ef
    st = _stream(stream)
    keep = (list(rank_bufs), None if error_bufs is None else list(error_bufs), arr, err)

    def call():
        if fn(plan, arr, err, st) != AR_OK:
            _raise()

    call.keep = keep
    return call


def ar_plan_stats(plan):
    s = lib().ar_plan_stats(plan)
    return s.to_dict()


def ar_plan_cost_alpha_beta(plan, alpha_s, bw_intra_Bps, bw_cross_Bps):
    t = lib().ar_plan_cost_alpha_beta(plan, alpha_s, bw_intra_Bps, bw_cross_Bps)
    if t < 0:
        _raise()
    return t


def ar_plan_cost_alpha_beta_ex(plan, alpha_intra_s, alpha_cross_s, bw_intra_Bps, bw_cross_Bps,
                               bw_group_egress_Bps=0.0, egress_share=1.0):
    c = ar_cost_params_t(alpha_intra_s, alpha_cross_s, bw_intra_Bps, bw_cross_Bps, bw_group_egress_Bps, egress_share)
    t = lib().ar_plan_cost_alpha_beta_ex(plan, ctypes.byref(c))
    if t < 0:
        _raise()
    return t


def ar_select_schedule(nranks, group_size, count, dtype, alpha_intra_s, alpha_cross_s, bw_intra_Bps,
                       bw_cross_Bps, bw_group_egress_Bps=0.0, egress_share=1.0, candidates=None):
    """(schedule name, modelled seconds) of the fastest candidate."""
    mask = 0
    for c in (candidates or SCHEDULES):
        mask |= 1 << _code(SCHEDULES, c)
    c = ar_cost_params_t(alpha_intra_s, alpha_cross_s, bw_intra_Bps, bw_cross_Bps, bw_group_egress_Bps, egress_share)
    t = ctypes.c_double()
    best = lib().ar_select_schedule(nranks, group_size, count, _code(DTYPES, dtype), ctypes.byref(c), mask,
                                    ctypes.byref(t))
    if best < 0:
        _raise()
    return {v: k for k, v in SCHEDULES.items()}[best], t.value


def ar_plan_destroy(plan):
    lib().ar_plan_destroy(plan)


def ar_last_error():
    return lib().ar_last_error().decode()


def ar_last_status():
    return lib().ar_last_status()


def ar_plan_transfers(plan):
    import numpy as np

    L = lib()
    n = L.ar_plan_transfers(plan, None, None, None, None, None, None, 0)
    if n < 0:
        _raise()
    cols = {k: np.zeros(max(n, 1), np.int32) for k in ("step", "src", "dst", "kind")}
    cols.update({k: np.zeros(max(n, 1), np.int64) for k in ("lo", "hi")})
    c = lambda a, t: a.ctypes.data_as(ctypes.POINTER(t))  # noqa: E731
    L.ar_plan_transfers(plan, c(cols["step"], ctypes.c_int32), c(cols["src"], ctypes.c_int32),
                        c(cols["dst"], ctypes.c_int32), c(cols["lo"], ctypes.c_int64),
                        c(cols["hi"], ctypes.c_int64), c(cols["kind"], ctypes.c_int32), n)
    return {k: v[:n] for k, v in cols.items()}


def ar_plan_num_launches(plan):
    n = lib().ar_plan_num_launches(plan)
    if n < 0:
        _raise()
    return n


def ar_plan_launch_info(plan, i):
    kind, nops = ctypes.c_int32(), ctypes.c_int32()
    _check(lib().ar_plan_launch_info(plan, i, ctypes.byref(kind), ctypes.byref(nops)))
    return kind.value, nops.value


def ar_plan_launch_ops(plan, i):
    import numpy as np

    _, nops = ar_plan_launch_info(plan, i)
    cols = {k: np.zeros(max(nops, 1), np.int64) for k in ("lo", "hi")}
    cols.update({k: np.zeros(max(nops, 1), np.int32) for k in ("a", "b", "o", "o2", "aux")})
    c = lambda a, t: a.ctypes.data_as(ctypes.POINTER(t))  # noqa: E731
    _check(lib().ar_plan_launch_ops(plan, i, c(cols["lo"], ctypes.c_int64), c(cols["hi"], ctypes.c_int64),
                                    *[c(cols[k], ctypes.c_int32) for k in ("a", "b", "o", "o2", "aux")]))
    return {k: v[:nops] for k, v in cols.items()}


def ar_plan_launch_scratch(plan, i):
    """(shift, slot_stride) of launch i's fp32 scratch addressing."""
    shift, stride = ctypes.c_int64(), ctypes.c_int64()
    _check(lib().ar_plan_launch_scratch(plan, i, ctypes.byref(shift), ctypes.byref(stride)))
    return shift.value, stride.value


def ar_plan_set_profiling(plan, max_calls):
    _check(lib().ar_plan_set_profiling(plan, int(max_calls)))


def ar_plan_set_profiling_period(plan, period):
    _check(lib().ar_plan_set_profiling_period(plan, int(period)))


def ar_plan_describe(plan):
    """The plan's configuration, step list and launches (with mean launch
    times from the profiling log) as a dict."""
    import json

    n = lib().ar_plan_describe(plan, None, 0)
    if n < 0:
        _raise()
    buf = ctypes.create_string_buffer(n + 1)
    lib().ar_plan_describe(plan, buf, n + 1)
    return json.loads(buf.value.decode())


def ar_plan_set_guard(plan, nbytes):
    _check(lib().ar_plan_set_guard(plan, int(nbytes)))


def ar_plan_check_guards(plan):
    _check(lib().ar_plan_check_guards(plan))


def ar_bucket_set_guard(bp, nbytes):
    _check(lib().ar_bucket_set_guard(bp, int(nbytes)))


def ar_bucket_check_guards(bp):
    _check(lib().ar_bucket_check_guards(bp))


def ar_plan_set_profiling_evict(plan, buf, nbytes):
    """Cold-cache timing: every timed launch is preceded by a fill of nbytes of buf."""
    _check(lib().ar_plan_set_profiling_evict(plan, _ptr(buf) or None, int(nbytes)))


def ar_plan_launch_shape(plan, i):
    """dict(cold, units, cpol, batch, grid_x, threads, lds_bytes) of launch i's kernel."""
    v = [ctypes.c_int32() for _ in range(4)]
    gx, th, lds = ctypes.c_uint32(), ctypes.c_int32(), ctypes.c_int32()
    _check(lib().ar_plan_launch_shape(plan, i, *[ctypes.byref(x) for x in v], ctypes.byref(gx), ctypes.byref(th),
                                      ctypes.byref(lds)))
    return {"cold": v[0].value, "units": v[1].value, "cpol": v[2].value, "batch": v[3].value,
            "grid_x": gx.value, "threads": th.value, "lds_bytes": lds.value}


def ar_hbm_probe(srcs, dsts, nbytes, units=2, policy=1, stream=None):
    """Each 16-byte unit of every dst gets the fp32 sum of that unit of every
    src (policy 0 plain, 1 nt loads + sc1 stores, 2 nt loads and stores;
    policy | 4: each workgroup stores one dst only)."""
    sa = (ctypes.c_void_p * max(len(srcs), 1))(*[_ptr(b) for b in srcs])
    da = (ctypes.c_void_p * max(len(dsts), 1))(*[_ptr(b) for b in dsts])
    _check(lib().ar_hbm_probe(ctypes.cast(sa, ctypes.c_void_p), len(srcs), ctypes.cast(da, ctypes.c_void_p),
                              len(dsts), int(nbytes), int(units), int(policy), _stream(stream)))


def ar_plan_launch_times(plan):
    """Per-launch ms of the logged calls, as a list of per-call lists (-1: not timed)."""
    n = ctypes.c_int32()
    _check(lib().ar_plan_launch_times(plan, None, 0, ctypes.byref(n)))
    buf = (ctypes.c_float * max(n.value, 1))()
    _check(lib().ar_plan_launch_times(plan, buf, n.value, ctypes.byref(n)))
    L = ar_plan_num_launches(plan)
    flat = [buf[i] for i in range(n.value)]
    return [flat[c * L:(c + 1) * L] for c in range(n.value // L)] if L else []


# ---------------------------------------------------------------- buckets

def ar_bucket_plan_create(nranks, group_size, tensor_counts, dtype, schedule, bucket_cap_bytes):
    counts = (ctypes.c_size_t * max(len(tensor_counts), 1))(*[int(c) for c in tensor_counts])
    p = lib().ar_bucket_plan_create(nranks, group_size, counts, len(tensor_counts), _code(DTYPES, dtype),
                                    _code(SCHEDULES, schedule), bucket_cap_bytes)
    if not p:
        _raise()
    return p


def ar_bucket_layout(bp, ntensors):
    offs = (ctypes.c_size_t * max(ntensors, 1))()
    arena = ctypes.c_size_t()
    _check(lib().ar_bucket_layout(bp, offs, ctypes.byref(arena)))
    return [offs[i] for i in range(ntensors)], arena.value


def ar_bucket_count(bp):
    n = lib().ar_bucket_count(bp)
    if n < 0:
        _raise()
    return n


def ar_bucket_range(bp, b):
    off, cnt = ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().ar_bucket_range(bp, b, ctypes.byref(off), ctypes.byref(cnt)))
    return off.value, cnt.value


def ar_bucket_set_graph(bp, enable=True):
    _check(lib().ar_bucket_set_graph(bp, 1 if enable else 0))


def ar_bucket_set_exec(bp, exec_mode):
    _check(lib().ar_bucket_set_exec(bp, _code(EXECS, exec_mode)))


def ar_bucket_set_cache_bytes(bp, nbytes):
    _check(lib().ar_bucket_set_cache_bytes(bp, int(nbytes)))


def ar_bucket_set_batching(bp, enable=True):
    _check(lib().ar_bucket_set_batching(bp, 1 if enable else 0))


def ar_bucket_batched_plan(bp):
    """The bucket plan's batched plan (owned by bp: never destroy it)."""
    p = lib().ar_bucket_batched_plan(bp)
    if not p:
        _raise()
    return p


def ar_bucket_allreduce(bp, rank_arenas, stream=None):
    if bp:
        n, nbytes, _ = _bucket_extent(bp)
        _check_bufs(rank_arenas, n, nbytes, "rank arena")
    arr = _ptr_array(rank_arenas)
    _check(lib().ar_bucket_allreduce(bp, ctypes.cast(arr, ctypes.c_void_p), _stream(stream)))


def _event(e):
    if e is None:
        return None
    if hasattr(e, "cuda_event"):
        if not e.cuda_event:
            e.record()  # torch creates the underlying event on its first record
        return e.cuda_event
    return int(e)


def ar_bucket_allreduce_after(bp, rank_arenas, stream=None, ready_events=None, done_events=None):
    """ready_events / done_events: per bucket, torch.cuda.Event, raw hipEvent_t ints, or None."""
    if bp:
        n, nbytes, _ = _bucket_extent(bp)
        _check_bufs(rank_arenas, n, nbytes, "rank arena")
    arr = _ptr_array(rank_arenas)
    nb = ar_bucket_count(bp)

    def evs(lst):
        if lst is None:
            return None
        if len(lst) != nb:
            raise ValueError(f"need {nb} events, got {len(lst)}")
        a = (ctypes.c_void_p * max(nb, 1))(*[_event(e) for e in lst])
        return ctypes.cast(a, ctypes.c_void_p)

    _check(lib().ar_bucket_allreduce_after(bp, ctypes.cast(arr, ctypes.c_void_p), _stream(stream),
                                           evs(ready_events), evs(done_events)))


def ar_bucket_allreduce_ef(bp, rank_arenas, error_arenas, stream=None, ready_events=None, done_events=None):
    if bp:
        n, nbytes, ebytes = _bucket_extent(bp)
        _check_bufs(rank_arenas, n, nbytes, "rank arena")
        if error_arenas is not None:
            _check_bufs(error_arenas, n, ebytes, "error arena")
    arr = _ptr_array(rank_arenas)
    err = ctypes.cast(_ptr_array(error_arenas), ctypes.c_void_p) if error_arenas is not None else None
    nb = ar_bucket_count(bp)

    def evs(lst):
        if lst is None:
            return None
        if len(lst) != nb:
            raise ValueError(f"need {nb} events, got {len(lst)}")
        a = (ctypes.c_void_p * max(nb, 1))(*[_event(e) for e in lst])
        return ctypes.cast(a, ctypes.c_void_p)

    _check(lib().ar_bucket_allreduce_ef(bp, ctypes.cast(arr, ctypes.c_void_p), err, _stream(stream),
                                        evs(ready_events), evs(done_events)))


def ar_overlap_step_time(ready_s, comm_s, compute_end_s, update_s):
    """(step seconds, exposed seconds) of the overlap model."""
    n = len(ready_s)
    r = (ctypes.c_double * max(n, 1))(*ready_s)
    c = (ctypes.c_double * max(n, 1))(*comm_s)
    exp = ctypes.c_double()
    t = lib().ar_overlap_step_time(n, r, c, compute_end_s, update_s, ctypes.byref(exp))
    if t < 0:
        _raise()
    return t, exp.value


def ar_bucket_stats(bp):
    return lib().ar_bucket_stats(bp).to_dict()


def ar_bucket_plan_destroy(bp):
    lib().ar_bucket_plan_destroy(bp)
