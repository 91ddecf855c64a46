// capi.hip -- C ABI (include/ar.h) and executor of the all-reduce library.
//
// A plan is built on the host (plan.cpp).  On first use it uploads its op
// tables to the device and, for bf16, allocates the fp32 partial-sum
// scratch.  ar_allreduce then launches one kernel per launch of the plan on
// the caller's stream, passing the caller's rank pointers by value; nothing
// is allocated or copied on the hot path.  After each call an event is
// recorded on the caller's stream, so that changing or destroying the plan
// waits for the plan's own work only, never for the whole device.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <array>
#include <atomic>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "../../include/ar.h"
#include "kernels.hpp"
#include "plan.hpp"

namespace {

// The value of a C enum argument as an integer, read from its bytes: a
// caller may pass any int, and loading a value outside the enumerators as
// the C++ enum type is undefined behaviour.  The planner validates it.
template <class E>
int32_t raw_enum(const E &v) {
  static_assert(sizeof(E) == sizeof(int32_t), "C enums are int-sized");
  int32_t r;
  std::memcpy(&r, &v, sizeof r);
  return r;
}

thread_local std::string g_err;
thread_local ar_status_t g_status = AR_OK;

ar_status_t fail(ar_status_t st, const std::string &msg) {
  g_status = st;
  g_err = msg;
  return st;
}

ar_status_t hip_fail(hipError_t e, const char *what) {
  return fail(AR_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

}  // namespace

struct ar_plan {
  ar::Plan p;
  int device = -1;
  bool prepared = false;
  ar_dev::DevOp *d_ops = nullptr;
  // Host side of the launches, computed whenever the plan is lowered (no
  // device work): the op table's contents, and per launch its first op in
  // the table, its grid width and kernel shape.  launch_err says why the
  // launches cannot run (empty: they can); table_id names this lowering.
  std::vector<ar_dev::DevOp> host_ops;
  std::vector<int64_t> op_offset;
  std::vector<uint32_t> grid_x;
  std::vector<uint8_t> cold;       // streaming kernel shape
  std::string launch_err;
  uint64_t table_id = 0;
  float *scratch = nullptr;        // owned unless external_scratch
  size_t scratch_bytes = 0;
  char *scratch_alloc = nullptr;   // the allocation holding scratch between its guard zones
  size_t guard_bytes = 0;          // guard zone on each side of the owned scratch
  float *external_scratch = nullptr;
  size_t external_scratch_bytes = 0;
  bool trace = false;              // AR_TRACE: dump the plan and its launch times at destroy
  // Graph replay: one instantiated graph of the whole launch sequence per
  // (rank pointers, error pointers, workspace) seen, at most kMaxGraphs.
  struct GraphEntry {
    std::vector<uintptr_t> key;
    hipGraphExec_t exec;
  };
  static constexpr size_t kMaxGraphs = 8;
  bool use_graph = false;
  std::vector<GraphEntry> graphs;
  hipStream_t own_stream = nullptr;  // non-blocking: op-table upload and graph capture
  int32_t prof_calls = 0;           // capacity of the event log in calls
  int64_t prof_logged = 0;          // calls recorded since the log was last read
  std::vector<hipEvent_t> events;   // prof_calls * launches * 2 (start, stop)
  int32_t prof_period = 1;          // call c times launch i iff (i + c) % period == 0
  std::vector<uint8_t> sampled;     // prof_calls * launches: the launch was timed
  void *evict_buf = nullptr;        // written before every timed launch (cold-cache timing)
  int64_t evict_bytes = 0;
  // Completion marks: for each stream the plan has run on, an event recorded
  // after the last call on that stream (none while the stream is being
  // captured by the caller).
  struct DoneMark {
    hipStream_t stream;
    hipEvent_t event;
  };
  static constexpr size_t kMaxMarks = 16;
  std::vector<DoneMark> marks;
  // The last (rank pointers, error pointers) set that passed the pointer
  // checks (checked_n entries; 0: none); the same set is not checked again.
  std::array<uintptr_t, 2 * ar::kMaxExecRanks> checked{};
  int checked_n = 0;

  // fp32 partial-sum slots, or the INT8 code slots
  size_t need_scratch_bytes() const { return static_cast<size_t>(ar::workspace_bytes(p)); }

  // Waits until every call made on this plan has finished on the device.
  void wait_idle() {
    for (DoneMark &m : marks) (void)hipEventSynchronize(m.event);
  }

  void drop_graphs() {
    if (!graphs.empty()) wait_idle();  // a replay may still be in flight
    for (GraphEntry &g : graphs) (void)hipGraphExecDestroy(g.exec);
    graphs.clear();
  }

  void release_marks() {
    wait_idle();
    for (DoneMark &m : marks) (void)hipEventDestroy(m.event);
    marks.clear();
  }

  // Frees the device tables, scratch, graphs and profiling events, after
  // the plan's calls in flight have finished.
  void release_device() {
    wait_idle();
    drop_graphs();
    if (own_stream) (void)hipStreamDestroy(own_stream);
    own_stream = nullptr;
    if (d_ops) (void)hipFree(d_ops);
    if (scratch_alloc) (void)hipFree(scratch_alloc);
    scratch_alloc = nullptr;
    for (hipEvent_t e : events) (void)hipEventDestroy(e);
    d_ops = nullptr;
    scratch = nullptr;
    scratch_bytes = 0;
    events.clear();
    prepared = false;
  }
};

struct ar_bucket_plan {
  int nranks = 0, group_size = 1;
  ar::Dtype dtype = ar::kF32;
  std::vector<int64_t> tensor_offsets, bucket_offset, bucket_count;
  int64_t arena_count = 0;
  std::vector<ar_plan_t *> plans;
  std::vector<uint64_t> bytes_sent;
  float *scratch = nullptr;
  size_t scratch_bytes = 0;
  char *scratch_alloc = nullptr;  // the allocation holding scratch between its guard zones
  size_t guard_bytes = 0;
  hipStream_t own_stream = nullptr;  // non-blocking: guard fills and checks
  // Batched execution: every bucket's all-reduce in shared launches (one
  // plan over the whole arena, built on first use).
  bool batch = true;
  bool use_graph = false;
  ar_plan_t *merged = nullptr;
};

namespace {

bool is_quant_kind(int32_t kind) {
  const int32_t fam = kind & 0xF00;
  if (fam == ar::kKRing || fam == ar::kKHier || fam == ar::kKTree || fam == ar::kKDTree)
    return (kind & 3) == ar::kI8EF;  // one-pass fold of an INT8 plan
  return fam == ar::kKQEncode || fam == ar::kKQReduce || fam == ar::kKQCopy || fam == ar::kKQDecode;
}

std::atomic<uint64_t> g_next_table_id{1};

// Host side of the launches of pl->p (see ar_plan::host_ops).  Called after
// every change of pl->p; touches no device.
void lower_launches(ar_plan_t *pl) {
  pl->host_ops.clear();
  pl->op_offset.clear();
  pl->grid_x.clear();
  pl->cold.clear();
  pl->launch_err.clear();
  pl->table_id = g_next_table_id.fetch_add(1);
  for (const ar::Launch &L : pl->p.launches) {
    pl->op_offset.push_back(static_cast<int64_t>(pl->host_ops.size()));
    const bool out_scratch = !L.ops.empty() && L.ops[0].o >= ar::kLocScratch;
    const bool quant = is_quant_kind(L.kind);
    const bool cold = !quant && !out_scratch && ar::launch_write_bytes(pl->p, L) > pl->p.cache_bytes;
    pl->cold.push_back(cold);
    const int64_t tile = quant ? ar_dev::q_tile_blocks(L.kind) : ar_dev::tile_elems(L.kind, cold, pl->p.nranks);
    int64_t gx = 0;
    for (const ar::Op &o : L.ops) {
      pl->host_ops.push_back({o.lo, o.hi, o.a, o.b, o.o, o.o2, o.aux, 0});
      gx = std::max(gx, (o.hi + tile - 1) / tile - o.lo / tile);
    }
    if (!quant) {  // blocks that walk several tiles
      const int64_t tpb = ar_dev::tiles_per_block(L.kind, pl->p.nranks);
      gx = (gx + tpb - 1) / tpb;
    }
    // a dispatch holds at most 2^32 - 1 work-items per grid dimension (here
    // 2^31 - 1 along the tiles) and 65535 workgroups along the ops
    const int64_t threads = quant ? ar_dev::q_block_threads(L.kind) : ar_dev::block_threads(L.kind, pl->p.nranks);
    // the LDS-staged folds and the one-pass all-gather walk their op's tiles
    // with the grid's stride, so a grid capped at the dispatch limit still
    // covers every tile; the all-gather's grid is its tiles times its
    // destination groups, and stays a multiple of them
    const bool fan = !quant && (L.kind & 0xF00) == ar::kKFan;
    const int64_t groups = fan ? ar_dev::fan_groups(pl->p.nranks) : 1;
    gx *= groups;
    if (!quant && (ar_dev::lds_staged(L.kind, pl->p.nranks) || fan))
      gx = std::min<int64_t>(gx, 0x7fffffff / threads / groups * groups);
    if (gx * threads > 0x7fffffff || static_cast<int64_t>(L.ops.size()) > ar::kMaxLaunchOps)
      pl->launch_err = "op too large for one launch grid";
    pl->grid_x.push_back(static_cast<uint32_t>(std::min<int64_t>(gx, 0x7fffffff)));
  }
}

// Copies the op table to pl->d_ops on the plan's own stream and waits for it.
hipError_t upload_ops(ar_plan_t *pl) {
  hipError_t e = hipSuccess;
  if (!pl->own_stream) {
    e = hipStreamCreateWithFlags(&pl->own_stream, hipStreamNonBlocking);
    if (e != hipSuccess) return e;
  }
  hipEvent_t done = nullptr;
  e = hipEventCreateWithFlags(&done, hipEventDisableTiming);
  if (e != hipSuccess) return e;
  e = hipMemcpyAsync(pl->d_ops, pl->host_ops.data(), pl->host_ops.size() * sizeof(ar_dev::DevOp),
                     hipMemcpyHostToDevice, pl->own_stream);
  if (e == hipSuccess) e = hipEventRecord(done, pl->own_stream);
  if (e == hipSuccess) e = hipEventSynchronize(done);
  (void)hipEventDestroy(done);
  return e;
}

// Guard zones (a debug aid): a device workspace of `bytes` is allocated with
// `guard` extra bytes on each side, filled with kGuardByte, which no kernel
// may touch.  Fills and checks run on a non-blocking stream of the owner and
// are waited for with an event (see upload_ops).
constexpr unsigned char kGuardByte = 0xA7;

hipError_t wait_on(hipStream_t s) {
  hipEvent_t done = nullptr;
  hipError_t e = hipEventCreateWithFlags(&done, hipEventDisableTiming);
  if (e != hipSuccess) return e;
  e = hipEventRecord(done, s);
  if (e == hipSuccess) e = hipEventSynchronize(done);
  (void)hipEventDestroy(done);
  return e;
}

hipError_t own_stream_of(hipStream_t *s) {
  return *s ? hipSuccess : hipStreamCreateWithFlags(s, hipStreamNonBlocking);
}

hipError_t guarded_alloc(size_t bytes, size_t guard, hipStream_t *s, char **alloc) {
  *alloc = nullptr;
  hipError_t e = hipMalloc(reinterpret_cast<void **>(alloc), bytes + 2 * guard);
  if (e != hipSuccess || guard == 0) return e;
  e = own_stream_of(s);
  if (e == hipSuccess) e = hipMemsetAsync(*alloc, kGuardByte, guard, *s);
  if (e == hipSuccess) e = hipMemsetAsync(*alloc + guard + bytes, kGuardByte, guard, *s);
  if (e == hipSuccess) e = wait_on(*s);
  if (e != hipSuccess) {
    (void)hipFree(*alloc);
    *alloc = nullptr;
  }
  return e;
}

// AR_OK if both guard zones of the allocation still hold kGuardByte.
ar_status_t check_guard(const char *alloc, size_t bytes, size_t guard, hipStream_t *s, const char *what) {
  if (!alloc || guard == 0) return AR_OK;
  std::vector<unsigned char> h(2 * guard);
  hipError_t e = own_stream_of(s);
  if (e == hipSuccess) e = hipMemcpyAsync(h.data(), alloc, guard, hipMemcpyDeviceToHost, *s);
  if (e == hipSuccess) e = hipMemcpyAsync(h.data() + guard, alloc + guard + bytes, guard, hipMemcpyDeviceToHost, *s);
  if (e == hipSuccess) e = wait_on(*s);
  if (e != hipSuccess) return hip_fail(e, "guard read");
  for (size_t i = 0; i < h.size(); ++i)
    if (h[i] != kGuardByte)
      return fail(AR_ERR_GUARD, std::string(what) + ": guard byte " +
                                    (i < guard ? std::to_string(guard - i) + " before the start"
                                               : std::to_string(i - guard) + " after the end") +
                                    " was overwritten");
  return AR_OK;
}

ar_status_t prepare(ar_plan_t *pl) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (pl->prepared) {
    if (dev != pl->device) return fail(AR_ERR_INVALID_ARG, "plan was prepared on another device");
    return AR_OK;
  }
  if (!pl->launch_err.empty()) return fail(AR_ERR_UNSUPPORTED, pl->launch_err);
  pl->release_device();
  pl->device = dev;
  const std::vector<ar_dev::DevOp> &host_ops = pl->host_ops;
  if (!host_ops.empty()) {
    e = hipMalloc(reinterpret_cast<void **>(&pl->d_ops), host_ops.size() * sizeof(ar_dev::DevOp));
    if (e != hipSuccess) {
      (void)hipGetLastError();
      pl->d_ops = nullptr;
      return fail(AR_ERR_OOM, std::string("op table allocation: ") + hipGetErrorString(e));
    }
    // The upload runs on the plan's own non-blocking stream and is waited for
    // with an event: a synchronous hipMemcpy goes through the legacy default
    // stream, which invalidates a graph capture that another host thread has
    // in progress (hipErrorStreamCaptureImplicit, measured on MI355X).
    e = upload_ops(pl);
    if (e != hipSuccess) {
      pl->release_device();
      return hip_fail(e, "op table upload");
    }
  }
  const size_t need = pl->need_scratch_bytes();
  if (need > 0 && !pl->external_scratch) {
    e = guarded_alloc(need, pl->guard_bytes, &pl->own_stream, &pl->scratch_alloc);
    if (e != hipSuccess) {
      (void)hipGetLastError();  // clear the sticky allocation error
      pl->release_device();
      return fail(AR_ERR_OOM, std::string("scratch allocation: ") + hipGetErrorString(e));
    }
    pl->scratch = reinterpret_cast<float *>(pl->scratch_alloc + pl->guard_bytes);
    pl->scratch_bytes = need;
  }
  if (need > 0 && pl->external_scratch && pl->external_scratch_bytes < need) {
    pl->release_device();
    return fail(AR_ERR_INVALID_ARG, "external scratch too small");
  }
  if (pl->prof_calls > 0) {
    pl->sampled.assign(static_cast<size_t>(pl->prof_calls) * pl->p.launches.size(), 0);
    pl->events.resize(static_cast<size_t>(pl->prof_calls) * pl->p.launches.size() * 2);
    for (hipEvent_t &ev : pl->events) {
      e = hipEventCreate(&ev);
      if (e != hipSuccess) {
        ev = nullptr;
        pl->release_device();
        return hip_fail(e, "hipEventCreate");
      }
    }
  }
  pl->prepared = true;
  return AR_OK;
}

// Pointer checks of a call: every rank buffer (count elements of the
// buffer dtype) and every error buffer (count fp32) is non-NULL, 16-byte
// aligned, and overlaps no other buffer of the call.  Overlap is found by
// sorting the buffers by address (O(N log N)).  A set that passed is kept on
// the plan and not checked again, so repeated calls with the same buffers
// cost N pointer compares.
ar_status_t check_pointers(ar_plan_t *pl, void *const *rank_bufs, void *const *error_bufs) {
  if (!rank_bufs) return fail(AR_ERR_INVALID_ARG, "rank_bufs is NULL");
  const int n = pl->p.nranks;
  const uint64_t rbytes =
      static_cast<uint64_t>(pl->p.count) * static_cast<uint64_t>(ar::buffer_elem_bytes(pl->p.dtype));
  if (rbytes == 0) return AR_OK;  // nothing is read or written
  const uint64_t ebytes = static_cast<uint64_t>(pl->p.count) * 4;
  std::array<uintptr_t, 2 * ar::kMaxExecRanks> &key = pl->checked;
  bool same = pl->checked_n == 2 * n;
  for (int r = 0; same && r < n; ++r)
    same = key[r] == reinterpret_cast<uintptr_t>(rank_bufs[r]) &&
           key[n + r] == (error_bufs ? reinterpret_cast<uintptr_t>(error_bufs[r]) : 0);
  if (same) return AR_OK;
  struct Extent {
    uintptr_t lo, hi;
    int idx;  // rank r, or n + r for error buffer r
  };
  std::array<Extent, 2 * ar::kMaxExecRanks> ex;  // on the stack: no allocation on this path
  const int next = error_bufs ? 2 * n : n;
  auto name = [n](int idx) {
    return idx < n ? "rank buffer " + std::to_string(idx) : "error buffer " + std::to_string(idx - n);
  };
  for (int k = 0; k < next; ++k) {
    const uintptr_t v = reinterpret_cast<uintptr_t>(k < n ? rank_bufs[k] : error_bufs[k - n]);
    if (!v) return fail(AR_ERR_INVALID_ARG, name(k) + " is NULL");
    if (v % 16) return fail(AR_ERR_INVALID_ARG, name(k) + " is not 16-byte aligned");
    ex[k] = {v, v + (k < n ? rbytes : ebytes), k};
  }
  std::sort(ex.begin(), ex.begin() + next, [](const Extent &a, const Extent &b) { return a.lo < b.lo; });
  int far = 0;  // the extent reaching furthest among those before i
  for (int i = 1; i < next; ++i) {
    if (ex[i].lo < ex[far].hi) {
      const int a = std::min(ex[far].idx, ex[i].idx), b = std::max(ex[far].idx, ex[i].idx);
      if (b < n)
        return fail(AR_ERR_INVALID_ARG, "rank buffers " + std::to_string(a) + " and " + std::to_string(b) + " overlap");
      if (a >= n)
        return fail(AR_ERR_INVALID_ARG,
                    "error buffers " + std::to_string(a - n) + " and " + std::to_string(b - n) + " overlap");
      return fail(AR_ERR_INVALID_ARG, name(a) + " and " + name(b) + " overlap");
    }
    if (ex[i].hi > ex[far].hi) far = i;
  }
  for (int r = 0; r < n; ++r) {
    key[r] = reinterpret_cast<uintptr_t>(rank_bufs[r]);
    key[n + r] = error_bufs ? reinterpret_cast<uintptr_t>(error_bufs[r]) : 0;
  }
  pl->checked_n = 2 * n;
  return AR_OK;
}

// The completion mark of stream s: the event a call on s records after its
// last launch (see enqueue and replay), created on the plan's first call on
// s.  *ev = NULL while the caller captures s into a graph of its own: such
// work runs when the caller launches that graph.  The event is created with
// timing so that a kernel dispatch can record it.
ar_status_t done_mark(ar_plan_t *pl, hipStream_t s, hipEvent_t *ev) {
  *ev = nullptr;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  hipError_t e = hipStreamIsCapturing(s, &cs);
  if (e != hipSuccess) return hip_fail(e, "hipStreamIsCapturing");
  if (cs != hipStreamCaptureStatusNone) return AR_OK;
  for (ar_plan_t::DoneMark &d : pl->marks)
    if (d.stream == s) {
      *ev = d.event;
      return AR_OK;
    }
  if (pl->marks.size() >= ar_plan_t::kMaxMarks) {  // retire the oldest stream's mark
    (void)hipEventSynchronize(pl->marks.front().event);
    (void)hipEventDestroy(pl->marks.front().event);
    pl->marks.erase(pl->marks.begin());
  }
  e = hipEventCreate(ev);
  if (e != hipSuccess) {
    *ev = nullptr;
    return hip_fail(e, "hipEventCreate");
  }
  pl->marks.push_back({s, *ev});
  return AR_OK;
}

ar_stats_t stats_of(const ar::Plan &p) {
  ar_stats_t s{};
  s.nranks = p.nranks;
  s.group_size = p.group_size;
  s.steps = static_cast<uint32_t>(p.nsteps);
  s.launches = static_cast<uint32_t>(p.launches.size());
  s.count = static_cast<uint64_t>(p.count);
  s.elem_bytes = static_cast<uint64_t>(ar::buffer_elem_bytes(p.dtype));
  s.bytes_sent = p.bytes_sent.data();
  for (uint64_t b : p.bytes_sent) {
    s.bytes_sent_max = std::max(s.bytes_sent_max, b);
    s.bytes_sent_total += b;
  }
  s.cross_group_bytes_total = p.cross_group_bytes;
  s.hbm_bytes_model = p.hbm_bytes;
  s.scratch_bytes = ar::workspace_bytes(p);
  s.exec = p.exec;
  return s;
}

}  // namespace

namespace {

// Launches every kernel of the plan on s (each timed by its own start and
// stop events when prof is set).
// done (if not NULL) is recorded when the call's last kernel ends: by that
// kernel's own dispatch (no packet of its own), or after it when the kernel
// is timed or nothing is launched.
ar_status_t enqueue(ar_plan_t *plan, bool quant, ar_dev::KArgs &args, ar_dev::QArgs &qargs, hipStream_t s,
                    bool prof, const ar_dev::DevOp *table, hipEvent_t done) {
  float *const scratch_base = args.scratch;
  size_t last = plan->p.launches.size();  // the last launch with work
  for (size_t i = 0; i < plan->p.launches.size(); ++i)
    if (plan->grid_x[i] > 0 && !plan->p.launches[i].ops.empty()) last = i;
  bool marked = false;
  hipEvent_t *ev = nullptr;
  uint8_t *mark = nullptr;
  const int64_t call = plan->prof_logged;
  if (prof) {
    const size_t slot = static_cast<size_t>(call % plan->prof_calls);
    ev = plan->events.data() + slot * plan->p.launches.size() * 2;
    mark = plan->sampled.data() + slot * plan->p.launches.size();
  }
  for (size_t i = 0; i < plan->p.launches.size(); ++i) {
    const ar::Launch &L = plan->p.launches[i];
    const dim3 grid = ar_dev::grid_for(plan->grid_x[i], static_cast<uint32_t>(L.ops.size()));
    hipError_t e = hipSuccess;
    const bool timed = prof && (static_cast<int64_t>(i) + call) % plan->prof_period == 0;
    if (prof) mark[i] = timed;
    if (grid.x == 0) {
      if (timed) {  // nothing to launch: an empty interval
        e = hipEventRecord(ev[2 * i], s);
        if (e == hipSuccess) e = hipEventRecord(ev[2 * i + 1], s);
        if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
      }
      continue;
    }
    if (timed && plan->evict_bytes > 0) {
      // evict the device cache, outside the launch's events, with plain
      // stores: on MI355X only stores allocate in the Infinity Cache (a read
      // or a non-temporal fill of 1 GiB left the next launch's time
      // unchanged; a plain-store fill did not)
      e = ar_dev::hbm_probe(nullptr, 0, &plan->evict_buf, 1, plan->evict_bytes, 2, 0, s);
      if (e != hipSuccess) return hip_fail(e, "cache eviction write");
    }
    if (timed) ar_dev::t_launch_events = ar_dev::LaunchEvents{ev[2 * i], ev[2 * i + 1]};
    else if (i == last && done) ar_dev::t_launch_events = ar_dev::LaunchEvents{nullptr, done};
    else ar_dev::t_launch_events = ar_dev::LaunchEvents{};
    marked = marked || (i == last && done && !timed);
    if (quant) {
      qargs.ops = table + plan->op_offset[i];
      qargs.nops = static_cast<int32_t>(L.ops.size());
      e = ar_dev::launch_q(L.kind, grid, qargs, s);
    } else {
      args.ops = table + plan->op_offset[i];
      args.nops = static_cast<int32_t>(L.ops.size());
      // slot index e - shift: the kernels add e to this base (integer
      // arithmetic; every address they form lies inside the scratch)
      args.scratch = reinterpret_cast<float *>(reinterpret_cast<uintptr_t>(scratch_base) -
                                               static_cast<uintptr_t>(L.scratch_shift) * sizeof(float));
      const bool out_scratch = !L.ops.empty() && L.ops[0].o >= ar::kLocScratch;
      e = ar_dev::launch(L.kind, grid, args, s, out_scratch, plan->cold[i]);
    }
    ar_dev::t_launch_events = ar_dev::LaunchEvents{};
    if (e != hipSuccess) return hip_fail(e, "kernel launch");
  }
  if (done && !marked) {
    const hipError_t e = hipEventRecord(done, s);
    if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
  }
  return AR_OK;
}

// Graph replay ([PRIMER] 4.8 / the persistent-collective idea of registering
// an operation once for many calls): the launch sequence is captured once per
// set of buffer pointers into a HIP graph and replayed with one launch.  The
// graph holds kernel nodes only (no memset or copy nodes).
ar_status_t replay(ar_plan_t *plan, bool quant, ar_dev::KArgs &args, ar_dev::QArgs &qargs, void *const *rank_bufs,
                   void *const *error_bufs, hipStream_t s, hipEvent_t mark) {
  std::vector<uintptr_t> key;
  const int n = plan->p.nranks;
  key.reserve(2 * n + 2);
  for (int r = 0; r < n; ++r) key.push_back(reinterpret_cast<uintptr_t>(rank_bufs[r]));
  for (int r = 0; r < n; ++r) key.push_back(error_bufs ? reinterpret_cast<uintptr_t>(error_bufs[r]) : 0);
  key.push_back(reinterpret_cast<uintptr_t>(plan->external_scratch ? plan->external_scratch : plan->scratch));
  key.push_back(reinterpret_cast<uintptr_t>(plan->d_ops));
  for (ar_plan_t::GraphEntry &g : plan->graphs)
    if (g.key == key) {
      hipError_t e = hipGraphLaunch(g.exec, s);
      if (e == hipSuccess && mark) e = hipEventRecord(mark, s);
      return e == hipSuccess ? AR_OK : hip_fail(e, "hipGraphLaunch");
    }
  hipError_t e;
  if (!plan->own_stream) {
    e = hipStreamCreateWithFlags(&plan->own_stream, hipStreamNonBlocking);
    if (e != hipSuccess) return hip_fail(e, "hipStreamCreateWithFlags");
  }
  e = hipStreamBeginCapture(plan->own_stream, hipStreamCaptureModeThreadLocal);
  if (e != hipSuccess) return hip_fail(e, "hipStreamBeginCapture");
  const ar_status_t st = enqueue(plan, quant, args, qargs, plan->own_stream, false, plan->d_ops, nullptr);
  hipGraph_t graph = nullptr;
  e = hipStreamEndCapture(plan->own_stream, &graph);
  if (st != AR_OK) {
    if (graph) (void)hipGraphDestroy(graph);
    return st;
  }
  if (e != hipSuccess) return hip_fail(e, "hipStreamEndCapture");
  hipGraphExec_t exec = nullptr;
  e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
  (void)hipGraphDestroy(graph);
  if (e != hipSuccess) return hip_fail(e, "hipGraphInstantiate");
  if (plan->graphs.size() >= ar_plan_t::kMaxGraphs) {
    plan->wait_idle();  // the oldest graph may still be running
    (void)hipGraphExecDestroy(plan->graphs.front().exec);
    plan->graphs.erase(plan->graphs.begin());
  }
  plan->graphs.push_back({std::move(key), exec});
  e = hipGraphLaunch(exec, s);
  if (e == hipSuccess && mark) e = hipEventRecord(mark, s);
  return e == hipSuccess ? AR_OK : hip_fail(e, "hipGraphLaunch");
}

// Argument checks shared by the all-reduce calls.
ar_status_t check_call(ar_plan_t *plan, void *const *rank_bufs, void *const *error_bufs) {
  if (!plan) return fail(AR_ERR_INVALID_ARG, "plan is NULL");
  if (plan->p.nranks > ar::kMaxExecRanks)
    return fail(AR_ERR_UNSUPPORTED, "plans of more than 64 ranks describe a schedule but cannot run");
  if (error_bufs && plan->p.dtype != ar::kI8EF)
    return fail(AR_ERR_INVALID_ARG, "error feedback needs an AR_INT8_EF plan");
  return check_pointers(plan, rank_bufs, error_bufs);
}

// Kernel arguments of a call: the caller's buffers and the plan's
// workspace (fp32 partial-sum slots, or the INT8 code slots and scales).
void fill_args(const ar_plan_t *plan, void *const *rank_bufs, void *const *error_bufs, float *workspace,
               ar_dev::KArgs &args, ar_dev::QArgs &qargs) {
  if (plan->p.dtype == ar::kI8EF) {
    for (int r = 0; r < plan->p.nranks; ++r) {
      qargs.grad[r] = static_cast<float *>(rank_bufs[r]);
      qargs.err[r] = error_bufs ? static_cast<float *>(error_bufs[r]) : nullptr;
    }
    char *ws = reinterpret_cast<char *>(workspace);
    qargs.codes = reinterpret_cast<int8_t *>(ws);
    qargs.scales = reinterpret_cast<float *>(ws + static_cast<int64_t>(plan->p.nranks) * plan->p.code_stride);
    qargs.code_stride = plan->p.code_stride;
    qargs.scale_stride = plan->p.scale_stride;
    qargs.count = plan->p.count;
    qargs.has_err = error_bufs != nullptr;
    qargs.nranks = plan->p.nranks;
    qargs.group_size = plan->p.group_size;
  } else {
    for (int r = 0; r < plan->p.nranks; ++r) args.rank[r] = rank_bufs[r];
    args.scratch = workspace;
    args.slot_stride = plan->p.slot_stride;
    args.nranks = plan->p.nranks;
    args.group_size = plan->p.group_size;
  }
}

// ---- Allocation-free calls (ar_allreduce_noalloc) ----
//
// Their device workspace is `scratch`, a file-scope device array that each
// GPU holds from the library's load until the process ends: the op table of
// the plan last run on that GPU at its start, then the plan's fp32 partial
// sums or INT8 code slots (256-byte aligned).  In host code `scratch` names
// a host-side stand-in, not the device memory: the device address comes from
// hipGetSymbolAddress, once per device, and only that address is used.
constexpr int kMaxDevices = 64;
static __device__ __align__(256) unsigned char scratch[AR_NOALLOC_SCRATCH_BYTES];

std::mutex g_noalloc_mu;
char *g_noalloc_base[kMaxDevices];                   // per device: the address of `scratch`
std::atomic<uint64_t> g_noalloc_owner[kMaxDevices];  // per device: table_id of the op table held, 0 none

// Device address of `scratch` on device dev (looked up on the first call
// there, with dev current).
ar_status_t noalloc_base(int dev, char **base) {
  if (dev < 0 || dev >= kMaxDevices) return fail(AR_ERR_UNSUPPORTED, "device index beyond the library's table");
  std::lock_guard<std::mutex> lock(g_noalloc_mu);
  if (!g_noalloc_base[dev]) {
    void *ptr = nullptr;
    hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress of the allocation-free scratch");
    if (!ptr || reinterpret_cast<uintptr_t>(ptr) % 256)
      return fail(AR_ERR_HIP, "allocation-free scratch has no 256-byte aligned device address");
    g_noalloc_base[dev] = static_cast<char *>(ptr);
  }
  *base = g_noalloc_base[dev];
  return AR_OK;
}

// Bytes of the op table at the start of the array (a multiple of 256).
uint64_t noalloc_table_bytes(const ar_plan_t *plan) {
  return (plan->host_ops.size() * sizeof(ar_dev::DevOp) + 255) / 256 * 256;
}

const char *const kDtypeNames[] = {"fp32", "bf16", "bf16_each", "int8_ef"};
const char *const kSchedNames[] = {"ring", "hierarchical", "rabenseifner", "recursive_doubling", "tree",
                                   "double_tree"};
const char *const kExecNames[] = {"steps", "steps_unfused", "onepass"};
const char *const kCollNames[] = {"allreduce", "reduce_scatter", "allgather"};

// The plan as JSON: its configuration, its schedule step by step (every
// transfer: sender, receiver, range, 0 reduce / 1 copy) and its launches
// (kernel kind, ops, shape, element range, bytes written, and the mean
// duration in ms over the profiling log's calls that timed the launch, or
// null).
std::string describe(const ar_plan_t *pl) {
  const ar::Plan &p = pl->p;
  std::string j = "{";
  auto kv = [&j](const char *k, const std::string &v, bool comma = true) {
    j += std::string("\"") + k + "\": " + v + (comma ? ", " : "");
  };
  auto q = [](const char *v) { return std::string("\"") + v + "\""; };
  kv("nranks", std::to_string(p.nranks));
  kv("group_size", std::to_string(p.group_size));
  kv("count", std::to_string(p.count));
  kv("dtype", q(kDtypeNames[p.dtype]));
  kv("schedule", q(kSchedNames[p.sched]));
  kv("exec", q(kExecNames[p.exec]));
  kv("collective", q(kCollNames[p.coll]));
  kv("steps", std::to_string(p.nsteps));
  kv("hbm_bytes_model", std::to_string(p.hbm_bytes));
  j += "\"step_list\": [";
  for (size_t i = 0; i < p.xfers.size(); ++i) {
    const ar::Transfer &x = p.xfers[i];
    const bool first = i == 0 || p.xfers[i - 1].step != x.step;
    const bool last = i + 1 == p.xfers.size() || p.xfers[i + 1].step != x.step;
    if (first) j += std::string(i ? ", " : "") + "{\"step\": " + std::to_string(x.step) + ", \"transfers\": [";
    j += "[" + std::to_string(x.src) + ", " + std::to_string(x.dst) + ", " + std::to_string(x.lo) + ", " +
         std::to_string(x.hi) + ", " + std::to_string(x.kind) + "]" + (last ? "]}" : ", ");
  }
  j += "], \"launch_list\": [";
  const size_t L = p.launches.size();
  const int64_t calls = pl->prof_calls > 0 ? std::min<int64_t>(pl->prof_logged, pl->prof_calls) : 0;
  for (size_t i = 0; i < L; ++i) {
    const ar::Launch &la = p.launches[i];
    int64_t lo = INT64_MAX, hi = 0;
    for (const ar::Op &o : la.ops) {
      lo = std::min(lo, o.lo);
      hi = std::max(hi, o.hi);
    }
    double sum = 0;
    int timed = 0;
    for (int64_t c = 0; c < calls && !pl->events.empty(); ++c) {
      const size_t slot = static_cast<size_t>((pl->prof_logged - calls + c) % pl->prof_calls);
      if (!pl->sampled[slot * L + i]) continue;
      float ms = 0;
      if (hipEventElapsedTime(&ms, pl->events[(slot * L + i) * 2], pl->events[(slot * L + i) * 2 + 1]) ==
          hipSuccess) {
        sum += ms;
        ++timed;
      }
    }
    char buf[64];
    std::snprintf(buf, sizeof buf, "%.5f", timed ? sum / timed : 0.0);
    j += std::string(i ? ", " : "") + "{\"launch\": " + std::to_string(i) + ", \"kind\": " +
         std::to_string(la.kind) + ", \"ops\": " + std::to_string(la.ops.size()) + ", \"cold\": " +
         std::to_string(pl->cold[i]) + ", \"grid_x\": " + std::to_string(pl->grid_x[i]) + ", \"lo\": " +
         std::to_string(la.ops.empty() ? 0 : lo) + ", \"hi\": " + std::to_string(hi) + ", \"write_bytes\": " +
         std::to_string(ar::launch_write_bytes(p, la)) + ", \"ms\": " + (timed ? buf : "null") + "}";
  }
  j += "]}";
  return j;
}

// AR_TRACE=1 writes the description of every plan at its destruction to
// stderr; AR_TRACE=<path> appends it to that file, one line per plan.
void trace_dump(const ar_plan_t *pl) {
  const char *t = std::getenv("AR_TRACE");
  if (!t || !*t || std::strcmp(t, "0") == 0) return;
  const std::string j = describe(pl) + "\n";
  if (std::strcmp(t, "1") == 0) {
    std::fputs(j.c_str(), stderr);
    return;
  }
  if (FILE *f = std::fopen(t, "a")) {
    std::fputs(j.c_str(), f);
    std::fclose(f);
  }
}

bool trace_enabled() {
  const char *t = std::getenv("AR_TRACE");
  return t && *t && std::strcmp(t, "0") != 0;
}

// ar_plan_set_exec with the mode as an integer.
ar_status_t set_exec(ar_plan_t *plan, int32_t exec) {
  if (!plan) return fail(AR_ERR_INVALID_ARG, "plan is NULL");
  const ar::Exec mode = static_cast<ar::Exec>(exec);
  if (mode == plan->p.exec && plan->prepared) return AR_OK;
  ar::Plan trial = plan->p;
  const std::string err = ar::relower(trial, mode);
  if (!err.empty()) return fail(AR_ERR_INVALID_ARG, err);
  plan->release_device();  // waits for the plan's calls in flight
  plan->p = std::move(trial);
  lower_launches(plan);
  return AR_OK;
}

// ar_plan_create_collective with the enum arguments as integers.
ar_plan_t *create_plan(int nranks, int group_size, size_t count, int32_t dtype, int32_t schedule,
                       int32_t coll = ar::kAllReduce) {
  if (count > static_cast<size_t>(INT64_MAX / 8)) {
    fail(AR_ERR_INVALID_ARG, "count too large");
    return nullptr;
  }
  ar_plan_t *pl = new (std::nothrow) ar_plan_t;
  if (!pl) {
    fail(AR_ERR_OOM, "host allocation failed");
    return nullptr;
  }
  bool unsupported = false;
  const std::string err = ar::build_plan(pl->p, nranks, group_size, static_cast<int64_t>(count),
                                         static_cast<ar::Dtype>(dtype), static_cast<ar::Sched>(schedule),
                                         ar::kSteps, &unsupported, static_cast<ar::Coll>(coll));
  if (!err.empty()) {
    delete pl;
    fail(unsupported ? AR_ERR_UNSUPPORTED : AR_ERR_INVALID_ARG, err);
    return nullptr;
  }
  lower_launches(pl);
  if (trace_enabled()) {  // per-launch timing of the last 16 calls, dumped at destroy
    pl->trace = true;
    pl->prof_calls = 16;
  }
  g_status = AR_OK;
  return pl;
}

// One call of a plan on these buffers (its collective already checked).
ar_status_t run_call(ar_plan_t *plan, void *const *rank_bufs, void *const *error_bufs, void *stream) {
  ar_status_t st = check_call(plan, rank_bufs, error_bufs);
  if (st != AR_OK) return st;
  st = prepare(plan);
  if (st != AR_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool quant = plan->p.dtype == ar::kI8EF;
  ar_dev::KArgs args{};
  ar_dev::QArgs qargs{};
  fill_args(plan, rank_bufs, error_bufs, plan->external_scratch ? plan->external_scratch : plan->scratch, args,
            qargs);
  const bool prof = plan->prof_calls > 0 && !plan->events.empty();
  hipEvent_t mark = nullptr;
  if (!plan->p.launches.empty()) {
    st = done_mark(plan, s, &mark);
    if (st != AR_OK) return st;
  }
  // per-launch events need eager launches (event records captured into a
  // graph cannot be timed), so profiling keeps calls eager
  st = plan->use_graph && !prof && !plan->p.launches.empty()
           ? replay(plan, quant, args, qargs, rank_bufs, error_bufs, s, mark)
           : enqueue(plan, quant, args, qargs, s, prof, plan->d_ops, mark);
  if (st == AR_OK && prof) ++plan->prof_logged;
  return st;
}

}  // namespace

extern "C" {

const char *ar_last_error(void) { return g_err.c_str(); }
ar_status_t ar_last_status(void) { return g_status; }

ar_plan_t *ar_plan_create(int nranks, int group_size, size_t count, ar_dtype_t dtype, ar_schedule_t schedule) {
  return create_plan(nranks, group_size, count, raw_enum(dtype), raw_enum(schedule));
}

ar_plan_t *ar_plan_create_collective(int nranks, int group_size, size_t count, ar_dtype_t dtype,
                                     ar_schedule_t schedule, ar_collective_t collective) {
  return create_plan(nranks, group_size, count, raw_enum(dtype), raw_enum(schedule), raw_enum(collective));
}

ar_status_t ar_plan_set_exec(ar_plan_t *plan, ar_exec_t exec) { return set_exec(plan, raw_enum(exec)); }

ar_status_t ar_plan_set_cache_bytes(ar_plan_t *plan, size_t bytes) {
  if (!plan) return fail(AR_ERR_INVALID_ARG, "plan is NULL");
  if (bytes > static_cast<size_t>(INT64_MAX)) return fail(AR_ERR_INVALID_ARG, "cache size too large");
  ar::Plan trial = plan->p;
  trial.cache_bytes = static_cast<int64_t>(bytes);
  const std::string err = ar::relower(trial, trial.exec);
  if (!err.empty()) return fail(AR_ERR_INVALID_ARG, err);
  plan->release_device();  // waits for the plan's calls in flight
  plan->p = std::move(trial);
  lower_launches(plan);
  return AR_OK;
}

ar_status_t ar_plan_prepare(ar_plan_t *plan) {
  if (!plan) return fail(AR_ERR_INVALID_ARG, "plan is NULL");
  if (plan->p.nranks > ar::kMaxExecRanks)
    return fail(AR_ERR_UNSUPPORTED, "plans of more than 64 ranks describe a schedule but cannot run");
  return prepare(plan);
}

ar_status_t ar_allreduce_ef(ar_plan_t *plan, void *const *rank_bufs, void *const *error_bufs, void *stream) {
  if (plan && plan->p.coll != ar::kAllReduce)
    return fail(AR_ERR_INVALID_ARG, "this plan runs a reduce-scatter or an all-gather: call ar_reduce_scatter or "
                                    "ar_allgather");
  return run_call(plan, rank_bufs, error_bufs, stream);
}

ar_status_t ar_reduce_scatter(ar_plan_t *plan, void *const *rank_bufs, void *stream) {
  if (plan && plan->p.coll != ar::kReduceScatter)
    return fail(AR_ERR_INVALID_ARG, "this plan does not run a reduce-scatter (ar_plan_create_collective)");
  return run_call(plan, rank_bufs, nullptr, stream);
}

ar_status_t ar_allgather(ar_plan_t *plan, void *const *rank_bufs, void *stream) {
  if (plan && plan->p.coll != ar::kAllGather)
    return fail(AR_ERR_INVALID_ARG, "this plan does not run an all-gather (ar_plan_create_collective)");
  return run_call(plan, rank_bufs, nullptr, stream);
}

ar_status_t ar_plan_owned_range(const ar_plan_t *plan, int rank, size_t *lo, size_t *hi) {
  if (!plan || !lo || !hi) return fail(AR_ERR_INVALID_ARG, "NULL argument");
  int64_t a = 0, b = 0;
  if (!ar::owned_range(plan->p, rank, &a, &b))
    return fail(plan->p.sched == ar::kRing || plan->p.sched == ar::kHier || plan->p.sched == ar::kRaben
                    ? AR_ERR_INVALID_ARG
                    : AR_ERR_UNSUPPORTED,
                "rank out of range, or a schedule without a reduce-scatter half");
  // INT8 plans count blocks of kQBlock elements
  const int64_t scale = plan->p.dtype == ar::kI8EF ? ar::kQBlock : 1;
  *lo = static_cast<size_t>(std::min(a * scale, plan->p.count));
  *hi = static_cast<size_t>(std::min(b * scale, plan->p.count));
  return AR_OK;
}

ar_status_t ar_allreduce_noalloc(ar_plan_t *plan, void *const *rank_bufs, void *const *error_bufs, void *stream) {
  if (plan && plan->p.coll != ar::kAllReduce)
    return fail(AR_ERR_INVALID_ARG, "the allocation-free call runs all-reduce plans");
  ar_status_t st = check_call(plan, rank_bufs, error_bufs);
  if (st != AR_OK) return st;
  if (!plan->launch_err.empty()) return fail(AR_ERR_UNSUPPORTED, plan->launch_err);
  const uint64_t table_bytes = noalloc_table_bytes(plan);
  const uint64_t need = table_bytes + ar::workspace_bytes(plan->p);
  if (need > AR_NOALLOC_SCRATCH_BYTES)
    return fail(AR_ERR_INVALID_ARG, "plan needs " + std::to_string(need) +
                                        " bytes of device workspace (op table and scratch); the allocation-free "
                                        "call holds at most " + std::to_string(AR_NOALLOC_SCRATCH_BYTES));
  if (plan->p.launches.empty() || plan->p.count == 0) return AR_OK;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  char *base = nullptr;
  st = noalloc_base(dev, &base);
  if (st != AR_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  auto *table = reinterpret_cast<ar_dev::DevOp *>(base);
  // The op table is written (by kernels whose arguments carry the ops) when
  // another plan's table is in the array, and always while the caller
  // captures s into a graph, so that the graph carries it.
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  e = hipStreamIsCapturing(s, &cs);
  if (e != hipSuccess) return hip_fail(e, "hipStreamIsCapturing");
  if (cs != hipStreamCaptureStatusNone || g_noalloc_owner[dev].load() != plan->table_id) {
    g_noalloc_owner[dev].store(0);
    e = ar_dev::write_ops(table, plan->host_ops.data(), static_cast<int64_t>(plan->host_ops.size()), s);
    if (e != hipSuccess) return hip_fail(e, "op table write");
    g_noalloc_owner[dev].store(plan->table_id);
  }
  const bool quant = plan->p.dtype == ar::kI8EF;
  ar_dev::KArgs args{};
  ar_dev::QArgs qargs{};
  fill_args(plan, rank_bufs, error_bufs, reinterpret_cast<float *>(base + table_bytes), args, qargs);
  return enqueue(plan, quant, args, qargs, s, false, table, nullptr);
}

ar_status_t ar_allreduce(ar_plan_t *plan, void *const *rank_bufs, void *stream) {
  return ar_allreduce_ef(plan, rank_bufs, nullptr, stream);
}

ar_stats_t ar_plan_stats(const ar_plan_t *plan) {
  if (!plan) {
    fail(AR_ERR_INVALID_ARG, "plan is NULL");
    return ar_stats_t{};
  }
  return stats_of(plan->p);
}

double ar_plan_cost_alpha_beta(const ar_plan_t *plan, double alpha_s, double bw_intra_Bps, double bw_cross_Bps) {
  if (!plan || !(bw_intra_Bps > 0) || !(bw_cross_Bps > 0) || alpha_s < 0) {
    fail(AR_ERR_INVALID_ARG, "bad cost-model arguments");
    return -1.0;
  }
  return ar::cost_alpha_beta(plan->p, alpha_s, bw_intra_Bps, bw_cross_Bps);
}

double ar_plan_cost_alpha_beta_ex(const ar_plan_t *plan, const ar_cost_params_t *c) {
  if (!plan || !c || !(c->bw_intra_Bps > 0) || !(c->bw_cross_Bps > 0) || c->alpha_intra_s < 0 ||
      c->alpha_cross_s < 0 || c->bw_group_egress_Bps < 0 || !(c->egress_share >= 1)) {
    fail(AR_ERR_INVALID_ARG, "bad cost-model arguments");
    return -1.0;
  }
  return ar::cost_alpha_beta_ex(plan->p, c->alpha_intra_s, c->alpha_cross_s, c->bw_intra_Bps, c->bw_cross_Bps,
                                c->bw_group_egress_Bps, c->egress_share);
}

int ar_select_schedule(int nranks, int group_size, size_t count, ar_dtype_t dtype, const ar_cost_params_t *params,
                       uint32_t candidates, double *best_s) {
  if (!params) {
    fail(AR_ERR_INVALID_ARG, "params is NULL");
    return -1;
  }
  int best = -1;
  double best_t = 0;
  for (int sched = AR_RING; sched <= AR_DOUBLE_TREE; ++sched) {
    if (!(candidates & (1u << sched))) continue;
    ar::Plan p;
    bool unsupported = false;
    if (!ar::build_plan(p, nranks, group_size, static_cast<int64_t>(count),
                        static_cast<ar::Dtype>(raw_enum(dtype)), static_cast<ar::Sched>(sched), ar::kSteps,
                        &unsupported).empty())
      continue;
    const double t = ar::cost_alpha_beta_ex(p, params->alpha_intra_s, params->alpha_cross_s, params->bw_intra_Bps,
                                            params->bw_cross_Bps, params->bw_group_egress_Bps,
                                            params->egress_share < 1 ? 1.0 : params->egress_share);
    if (best < 0 || t < best_t) {
      best = sched;
      best_t = t;
    }
  }
  if (best < 0) {
    fail(AR_ERR_INVALID_ARG, "no candidate schedule fits these arguments");
    return -1;
  }
  if (best_s) *best_s = best_t;
  g_status = AR_OK;
  return best;
}

void ar_plan_destroy(ar_plan_t *plan) {
  if (!plan) return;
  if (plan->trace) {
    plan->wait_idle();
    trace_dump(plan);
  }
  plan->release_device();
  plan->release_marks();
  delete plan;
}

int64_t ar_plan_transfers(const ar_plan_t *plan, int32_t *step, int32_t *src, int32_t *dst, int64_t *lo,
                          int64_t *hi, int32_t *kind, int64_t cap) {
  if (!plan) {
    fail(AR_ERR_INVALID_ARG, "plan is NULL");
    return -1;
  }
  const auto &x = plan->p.xfers;
  const int64_t n = static_cast<int64_t>(x.size());
  for (int64_t i = 0; i < std::min(n, cap); ++i) {
    if (step) step[i] = x[i].step;
    if (src) src[i] = x[i].src;
    if (dst) dst[i] = x[i].dst;
    if (lo) lo[i] = x[i].lo;
    if (hi) hi[i] = x[i].hi;
    if (kind) kind[i] = x[i].kind;
  }
  return n;
}

int32_t ar_plan_num_launches(const ar_plan_t *plan) {
  if (!plan) {
    fail(AR_ERR_INVALID_ARG, "plan is NULL");
    return -1;
  }
  return static_cast<int32_t>(plan->p.launches.size());
}

ar_status_t ar_plan_launch_info(const ar_plan_t *plan, int32_t i, int32_t *kind, int32_t *nops) {
  if (!plan || i < 0 || i >= static_cast<int32_t>(plan->p.launches.size()))
    return fail(AR_ERR_INVALID_ARG, "bad plan or launch index");
  if (kind) *kind = plan->p.launches[i].kind;
  if (nops) *nops = static_cast<int32_t>(plan->p.launches[i].ops.size());
  return AR_OK;
}

ar_status_t ar_plan_launch_ops(const ar_plan_t *plan, int32_t i, int64_t *lo, int64_t *hi, int32_t *a, int32_t *b,
                               int32_t *o, int32_t *o2, int32_t *aux) {
  if (!plan || i < 0 || i >= static_cast<int32_t>(plan->p.launches.size()))
    return fail(AR_ERR_INVALID_ARG, "bad plan or launch index");
  const auto &ops = plan->p.launches[i].ops;
  for (size_t k = 0; k < ops.size(); ++k) {
    if (lo) lo[k] = ops[k].lo;
    if (hi) hi[k] = ops[k].hi;
    if (a) a[k] = ops[k].a;
    if (b) b[k] = ops[k].b;
    if (o) o[k] = ops[k].o;
    if (o2) o2[k] = ops[k].o2;
    if (aux) aux[k] = ops[k].aux;
  }
  return AR_OK;
}

ar_status_t ar_plan_launch_scratch(const ar_plan_t *plan, int32_t i, int64_t *shift, int64_t *slot_stride) {
  if (!plan || i < 0 || i >= static_cast<int32_t>(plan->p.launches.size()))
    return fail(AR_ERR_INVALID_ARG, "bad plan or launch index");
  if (shift) *shift = plan->p.launches[i].scratch_shift;
  if (slot_stride) *slot_stride = plan->p.slot_stride;
  return AR_OK;
}

ar_status_t ar_plan_set_graph(ar_plan_t *plan, int enable) {
  if (!plan) return fail(AR_ERR_INVALID_ARG, "plan is NULL");
  plan->use_graph = enable != 0;
  plan->drop_graphs();
  return AR_OK;
}

ar_status_t ar_plan_set_profiling(ar_plan_t *plan, int max_calls) {
  if (!plan || max_calls < 0) return fail(AR_ERR_INVALID_ARG, "bad profiling arguments");
  plan->release_device();  // waits for the plan's calls in flight
  plan->prof_calls = max_calls;
  plan->prof_logged = 0;
  return AR_OK;
}

ar_status_t ar_plan_set_profiling_period(ar_plan_t *plan, int period) {
  if (!plan || period < 1) return fail(AR_ERR_INVALID_ARG, "bad profiling period");
  plan->prof_period = period;
  return AR_OK;
}

int64_t ar_plan_describe(const ar_plan_t *plan, char *buf, size_t cap) {
  if (!plan) {
    fail(AR_ERR_INVALID_ARG, "plan is NULL");
    return -1;
  }
  auto *mut = const_cast<ar_plan_t *>(plan);
  mut->wait_idle();  // the profiling log's events must have completed
  const std::string j = describe(plan);
  if (buf && cap > 0) {
    const size_t n = std::min(cap - 1, j.size());
    std::memcpy(buf, j.data(), n);
    buf[n] = 0;
  }
  return static_cast<int64_t>(j.size());
}

ar_status_t ar_plan_set_guard(ar_plan_t *plan, size_t bytes) {
  if (!plan || bytes % 256 || bytes > (size_t{1} << 30)) return fail(AR_ERR_INVALID_ARG, "bad guard size");
  plan->release_device();  // waits for the plan's calls in flight
  plan->guard_bytes = bytes;
  return AR_OK;
}

ar_status_t ar_plan_check_guards(ar_plan_t *plan) {
  if (!plan) return fail(AR_ERR_INVALID_ARG, "plan is NULL");
  plan->wait_idle();
  return check_guard(plan->scratch_alloc, plan->scratch_bytes, plan->guard_bytes, &plan->own_stream,
                     "plan scratch");
}

ar_status_t ar_plan_set_profiling_evict(ar_plan_t *plan, void *buf, size_t bytes) {
  if (!plan || (bytes > 0 && !buf) || bytes % 16 || bytes > static_cast<size_t>(INT64_MAX))
    return fail(AR_ERR_INVALID_ARG, "bad eviction buffer");
  plan->evict_buf = bytes ? buf : nullptr;
  plan->evict_bytes = static_cast<int64_t>(bytes);
  return AR_OK;
}

ar_status_t ar_plan_launch_shape(const ar_plan_t *plan, int32_t i, int32_t *cold, int32_t *units, int32_t *cpol,
                                 int32_t *batch, uint32_t *grid_x, int32_t *threads, int32_t *lds_bytes) {
  if (!plan || i < 0 || i >= static_cast<int32_t>(plan->p.launches.size()))
    return fail(AR_ERR_INVALID_ARG, "bad plan or launch index");
  const ar::Launch &L = plan->p.launches[i];
  const bool quant = is_quant_kind(L.kind);
  const bool out_scratch = !L.ops.empty() && L.ops[0].o >= ar::kLocScratch;
  const ar_dev::KernelShape ks = quant ? ar_dev::KernelShape{0, 0, 0, 0}
                                       : ar_dev::kernel_shape(L.kind, plan->cold[i] != 0, out_scratch, plan->p.nranks);
  if (cold) *cold = plan->cold[i];
  if (units) *units = ks.units;
  if (cpol) *cpol = ks.cpol;
  if (batch) *batch = ks.batch;
  if (grid_x) *grid_x = plan->grid_x[i];
  if (threads) *threads = quant ? ar_dev::q_block_threads(L.kind) : ar_dev::block_threads(L.kind, plan->p.nranks);
  if (lds_bytes) *lds_bytes = ks.lds_bytes;
  return AR_OK;
}

ar_status_t ar_hbm_probe(const void *const *src, int32_t nsrc, void *const *dst, int32_t ndst, size_t bytes,
                         int32_t units, int32_t policy, void *stream) {
  if (nsrc < 0 || ndst < 0 || nsrc > ar_dev::kProbeMax || ndst > ar_dev::kProbeMax || (nsrc > 0 && !src) ||
      (ndst > 0 && !dst) || bytes % 16 || bytes > static_cast<size_t>(INT64_MAX) ||
      (units != 1 && units != 2 && units != 4) || policy < 0 || (policy & ~7) != 0 || (policy & 3) > 2 ||
      ((policy & 4) && ndst < 1))
    return fail(AR_ERR_INVALID_ARG, "bad probe arguments");
  for (int i = 0; i < nsrc; ++i)
    if (!src[i] || reinterpret_cast<uintptr_t>(src[i]) % 16) return fail(AR_ERR_INVALID_ARG, "bad probe source");
  for (int i = 0; i < ndst; ++i)
    if (!dst[i] || reinterpret_cast<uintptr_t>(dst[i]) % 16) return fail(AR_ERR_INVALID_ARG, "bad probe destination");
  const hipError_t e = ar_dev::hbm_probe(src, nsrc, dst, ndst, static_cast<int64_t>(bytes), units, policy,
                                         static_cast<hipStream_t>(stream));
  return e == hipSuccess ? AR_OK : hip_fail(e, "probe launch");
}

ar_status_t ar_plan_launch_times(ar_plan_t *plan, float *ms, int32_t cap, int32_t *n) {
  if (!plan || !n) return fail(AR_ERR_INVALID_ARG, "bad arguments");
  if (plan->prof_calls <= 0) return fail(AR_ERR_INVALID_ARG, "profiling is off");
  const int64_t L = static_cast<int64_t>(plan->p.launches.size());
  const int64_t calls = std::min<int64_t>(plan->prof_logged, plan->prof_calls);
  *n = static_cast<int32_t>(calls * L);
  if (!ms || cap < *n) return AR_OK;  // size query
  const int64_t first = plan->prof_logged - calls;
  for (int64_t c = 0; c < calls; ++c) {
    const size_t slot = static_cast<size_t>((first + c) % plan->prof_calls);
    const hipEvent_t *ev = plan->events.data() + slot * L * 2;
    const uint8_t *mark = plan->sampled.data() + slot * L;
    for (int64_t i = 0; i < L; ++i) {
      if (!mark[i]) {
        ms[c * L + i] = -1.0f;  // not timed in this call
        continue;
      }
      hipError_t e = hipEventElapsedTime(&ms[c * L + i], ev[2 * i], ev[2 * i + 1]);
      if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
    }
  }
  plan->prof_logged = 0;
  return AR_OK;
}

// ---------------------------------------------------------------- buckets

}  // extern "C"

namespace {

// Frees the scratch the buckets share, after the buckets that used it.
void release_bucket_scratch(ar_bucket_plan_t *bp) {
  if (!bp->scratch_alloc) return;
  for (ar_plan_t *pl : bp->plans) pl->wait_idle();
  (void)hipFree(bp->scratch_alloc);
  bp->scratch_alloc = nullptr;
  bp->scratch = nullptr;
  bp->scratch_bytes = 0;
  for (ar_plan_t *pl : bp->plans) {  // their device state pointed at it
    pl->external_scratch = nullptr;
    pl->external_scratch_bytes = 0;
    pl->prepared = pl->prepared && pl->need_scratch_bytes() == 0;
  }
}

void drop_merged(ar_bucket_plan_t *bp) {
  if (bp->merged) ar_plan_destroy(bp->merged);
  bp->merged = nullptr;
}

// The batched plan of a bucket plan, built on first use (NULL for INT8).
ar_plan_t *merged_plan(ar_bucket_plan_t *bp) {
  if (bp->merged) return bp->merged;
  if (bp->dtype == ar::kI8EF) {
    fail(AR_ERR_UNSUPPORTED, "INT8 buckets run one by one");
    return nullptr;
  }
  std::vector<const ar::Plan *> parts;
  for (ar_plan_t *pl : bp->plans) parts.push_back(&pl->p);
  auto *m = new (std::nothrow) ar_plan_t;
  if (!m) {
    fail(AR_ERR_OOM, "host allocation failed");
    return nullptr;
  }
  const std::string err = ar::merge_segments(m->p, parts, bp->bucket_offset, bp->arena_count);
  if (!err.empty()) {
    delete m;
    fail(AR_ERR_INVALID_ARG, "batched buckets: " + err);
    return nullptr;
  }
  lower_launches(m);
  m->use_graph = bp->use_graph;
  m->guard_bytes = bp->guard_bytes;
  bp->merged = m;
  return m;
}

}  // namespace

extern "C" {

ar_bucket_plan_t *ar_bucket_plan_create(int nranks, int group_size, const size_t *tensor_counts, int ntensors,
                                        ar_dtype_t dtype, ar_schedule_t schedule, size_t bucket_cap_bytes) {
  if (ntensors < 0 || (ntensors > 0 && !tensor_counts) || bucket_cap_bytes == 0) {
    fail(AR_ERR_INVALID_ARG, "bad bucket arguments");
    return nullptr;
  }
  const auto dt = static_cast<ar::Dtype>(raw_enum(dtype));
  if (dt != ar::kF32 && dt != ar::kBF16 && dt != ar::kBF16Each && dt != ar::kI8EF) {
    fail(AR_ERR_INVALID_ARG, "unknown dtype");
    return nullptr;
  }
  auto *bp = new (std::nothrow) ar_bucket_plan_t;
  if (!bp) {
    fail(AR_ERR_OOM, "host allocation failed");
    return nullptr;
  }
  bp->nranks = nranks;
  bp->group_size = group_size;
  bp->dtype = dt;
  const int64_t eb = ar::buffer_elem_bytes(dt);
  std::vector<int64_t> counts(tensor_counts, tensor_counts + ntensors);
  for (int64_t c : counts)
    if (c < 0) {
      delete bp;
      fail(AR_ERR_INVALID_ARG, "negative tensor count");
      return nullptr;
    }
  ar::assign_buckets(counts, static_cast<int64_t>(bucket_cap_bytes) / eb, 256 / eb, bp->tensor_offsets,
                     bp->bucket_offset, bp->bucket_count, bp->arena_count);
  bp->bytes_sent.assign(nranks > 0 ? nranks : 0, 0);
  for (size_t b = 0; b < bp->bucket_count.size(); ++b) {
    ar_plan_t *pl = create_plan(nranks, group_size, static_cast<size_t>(bp->bucket_count[b]), dt,
                                raw_enum(schedule));
    if (!pl) {
      const ar_status_t st = g_status;
      const std::string msg = g_err;
      ar_bucket_plan_destroy(bp);
      fail(st, "bucket " + std::to_string(b) + ": " + msg);
      return nullptr;
    }
    bp->plans.push_back(pl);
  }
  g_status = AR_OK;
  return bp;
}

ar_status_t ar_bucket_layout(const ar_bucket_plan_t *bp, size_t *tensor_offsets, size_t *arena_count) {
  if (!bp) return fail(AR_ERR_INVALID_ARG, "bucket plan is NULL");
  if (tensor_offsets)
    for (size_t t = 0; t < bp->tensor_offsets.size(); ++t) tensor_offsets[t] = static_cast<size_t>(bp->tensor_offsets[t]);
  if (arena_count) *arena_count = static_cast<size_t>(bp->arena_count);
  return AR_OK;
}

int32_t ar_bucket_count(const ar_bucket_plan_t *bp) {
  if (!bp) {
    fail(AR_ERR_INVALID_ARG, "bucket plan is NULL");
    return -1;
  }
  return static_cast<int32_t>(bp->bucket_count.size());
}

ar_status_t ar_bucket_range(const ar_bucket_plan_t *bp, int32_t b, size_t *offset, size_t *count) {
  if (!bp || b < 0 || b >= static_cast<int32_t>(bp->bucket_count.size()))
    return fail(AR_ERR_INVALID_ARG, "bad bucket plan or index");
  if (offset) *offset = static_cast<size_t>(bp->bucket_offset[b]);
  if (count) *count = static_cast<size_t>(bp->bucket_count[b]);
  return AR_OK;
}

ar_status_t ar_bucket_set_graph(ar_bucket_plan_t *bp, int enable) {
  if (!bp) return fail(AR_ERR_INVALID_ARG, "bucket plan is NULL");
  for (ar_plan_t *pl : bp->plans) {
    const ar_status_t st = ar_plan_set_graph(pl, enable);
    if (st != AR_OK) return st;
  }
  bp->use_graph = enable != 0;
  if (bp->merged) return ar_plan_set_graph(bp->merged, enable);
  return AR_OK;
}

ar_status_t ar_bucket_set_exec(ar_bucket_plan_t *bp, ar_exec_t exec) {
  if (!bp) return fail(AR_ERR_INVALID_ARG, "bucket plan is NULL");
  for (ar_plan_t *pl : bp->plans) {
    const ar_status_t st = set_exec(pl, raw_enum(exec));
    if (st != AR_OK) return st;
  }
  drop_merged(bp);  // waits for its launches in flight
  return AR_OK;
}

ar_status_t ar_bucket_set_cache_bytes(ar_bucket_plan_t *bp, size_t bytes) {
  if (!bp) return fail(AR_ERR_INVALID_ARG, "bucket plan is NULL");
  for (ar_plan_t *pl : bp->plans) {
    const ar_status_t st = ar_plan_set_cache_bytes(pl, bytes);
    if (st != AR_OK) return st;
  }
  drop_merged(bp);  // waits for its launches in flight
  return AR_OK;
}

ar_status_t ar_bucket_set_guard(ar_bucket_plan_t *bp, size_t bytes) {
  if (!bp || bytes % 256 || bytes > (size_t{1} << 30)) return fail(AR_ERR_INVALID_ARG, "bad guard size");
  release_bucket_scratch(bp);
  bp->guard_bytes = bytes;
  for (ar_plan_t *pl : bp->plans) {
    const ar_status_t st = ar_plan_set_guard(pl, bytes);
    if (st != AR_OK) return st;
  }
  if (bp->merged) return ar_plan_set_guard(bp->merged, bytes);
  return AR_OK;
}

ar_status_t ar_bucket_check_guards(ar_bucket_plan_t *bp) {
  if (!bp) return fail(AR_ERR_INVALID_ARG, "bucket plan is NULL");
  for (ar_plan_t *pl : bp->plans) pl->wait_idle();
  ar_status_t st = check_guard(bp->scratch_alloc, bp->scratch_bytes, bp->guard_bytes, &bp->own_stream,
                               "bucket scratch");
  for (size_t b = 0; st == AR_OK && b < bp->plans.size(); ++b) st = ar_plan_check_guards(bp->plans[b]);
  if (st == AR_OK && bp->merged) st = ar_plan_check_guards(bp->merged);
  return st;
}

ar_status_t ar_bucket_set_batching(ar_bucket_plan_t *bp, int enable) {
  if (!bp) return fail(AR_ERR_INVALID_ARG, "bucket plan is NULL");
  bp->batch = enable != 0;
  return AR_OK;
}

ar_plan_t *ar_bucket_batched_plan(ar_bucket_plan_t *bp) {
  if (!bp) {
    fail(AR_ERR_INVALID_ARG, "bucket plan is NULL");
    return nullptr;
  }
  if (bp->plans.empty()) {
    fail(AR_ERR_INVALID_ARG, "bucket plan has no buckets");
    return nullptr;
  }
  ar_plan_t *m = merged_plan(bp);
  if (m) g_status = AR_OK;
  return m;
}

ar_status_t ar_bucket_allreduce(ar_bucket_plan_t *bp, void *const *rank_arenas, void *stream) {
  return ar_bucket_allreduce_ef(bp, rank_arenas, nullptr, stream, nullptr, nullptr);
}

ar_status_t ar_bucket_allreduce_after(ar_bucket_plan_t *bp, void *const *rank_arenas, void *stream,
                                      void *const *ready_events, void *const *done_events) {
  return ar_bucket_allreduce_ef(bp, rank_arenas, nullptr, stream, ready_events, done_events);
}

double ar_overlap_step_time(int nchunks, const double *ready_s, const double *comm_s, double compute_end_s,
                            double update_s, double *exposed_s) {
  if (nchunks < 0 || (nchunks > 0 && (!ready_s || !comm_s)) || update_s < 0) {
    fail(AR_ERR_INVALID_ARG, "bad overlap-model arguments");
    return -1.0;
  }
  for (int k = 0; k < nchunks; ++k)
    if (comm_s[k] < 0) {
      fail(AR_ERR_INVALID_ARG, "negative communication time");
      return -1.0;
    }
  return ar::overlap_step_time(nchunks, ready_s, comm_s, compute_end_s, update_s, exposed_s);
}

ar_status_t ar_bucket_allreduce_ef(ar_bucket_plan_t *bp, void *const *rank_arenas, void *const *error_arenas,
                                   void *stream, void *const *ready_events, void *const *done_events) {
  if (!bp || !rank_arenas) return fail(AR_ERR_INVALID_ARG, "bad bucket arguments");
  if (error_arenas && bp->dtype != ar::kI8EF) return fail(AR_ERR_INVALID_ARG, "error feedback needs AR_INT8_EF");
  if (bp->plans.empty()) return AR_OK;
  if (bp->batch && bp->dtype != ar::kI8EF && !ready_events && !done_events) {
    ar_plan_t *m = merged_plan(bp);
    if (!m) return g_status;
    return ar_allreduce(m, rank_arenas, stream);
  }
  // one scratch shared by all buckets: they run one after another on one stream
  size_t need = 0;
  for (ar_plan_t *pl : bp->plans) need = std::max(need, pl->need_scratch_bytes());
  if (need > bp->scratch_bytes) {
    release_bucket_scratch(bp);
    hipError_t e = guarded_alloc(need, bp->guard_bytes, &bp->own_stream, &bp->scratch_alloc);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      return fail(AR_ERR_OOM, std::string("bucket scratch: ") + hipGetErrorString(e));
    }
    bp->scratch = reinterpret_cast<float *>(bp->scratch_alloc + bp->guard_bytes);
    bp->scratch_bytes = need;
  }
  const int64_t eb = ar::buffer_elem_bytes(bp->dtype);
  std::vector<void *> ptrs(static_cast<size_t>(bp->nranks)), eptrs(static_cast<size_t>(bp->nranks));
  for (size_t b = 0; b < bp->plans.size(); ++b) {
    ar_plan_t *pl = bp->plans[b];
    if (pl->external_scratch != bp->scratch) {
      pl->external_scratch = bp->scratch;
      pl->external_scratch_bytes = bp->scratch_bytes;
      pl->prepared = pl->prepared && pl->need_scratch_bytes() == 0;
    }
    pl->external_scratch_bytes = bp->scratch_bytes;
    for (int r = 0; r < bp->nranks; ++r) {
      ptrs[r] = static_cast<char *>(rank_arenas[r]) + bp->bucket_offset[b] * eb;
      if (error_arenas) eptrs[r] = static_cast<char *>(error_arenas[r]) + bp->bucket_offset[b] * eb;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (ready_events && ready_events[b]) {
      hipError_t e = hipStreamWaitEvent(s, static_cast<hipEvent_t>(ready_events[b]), 0);
      if (e != hipSuccess) return hip_fail(e, "hipStreamWaitEvent");
    }
    const ar_status_t st = ar_allreduce_ef(pl, ptrs.data(), error_arenas ? eptrs.data() : nullptr, stream);
    if (st != AR_OK) return fail(st, "bucket " + std::to_string(b) + ": " + g_err);
    if (done_events && done_events[b]) {
      hipError_t e = hipEventRecord(static_cast<hipEvent_t>(done_events[b]), s);
      if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
    }
  }
  return AR_OK;
}

ar_stats_t ar_bucket_stats(const ar_bucket_plan_t *bp) {
  ar_stats_t s{};
  if (!bp) {
    fail(AR_ERR_INVALID_ARG, "bucket plan is NULL");
    return s;
  }
  auto *mut = const_cast<ar_bucket_plan_t *>(bp);
  std::fill(mut->bytes_sent.begin(), mut->bytes_sent.end(), 0);
  for (ar_plan_t *pl : bp->plans) {
    const ar_stats_t t = stats_of(pl->p);
    s.steps += t.steps;
    s.launches += t.launches;
    s.count += t.count;
    s.cross_group_bytes_total += t.cross_group_bytes_total;
    s.hbm_bytes_model += t.hbm_bytes_model;
    s.scratch_bytes = std::max(s.scratch_bytes, t.scratch_bytes);
    s.exec = t.exec;
    for (int r = 0; r < bp->nranks; ++r) mut->bytes_sent[r] += pl->p.bytes_sent[r];
  }
  s.nranks = bp->nranks;
  s.group_size = bp->group_size;
  s.elem_bytes = static_cast<uint64_t>(ar::buffer_elem_bytes(bp->dtype));
  s.bytes_sent = bp->bytes_sent.data();
  for (uint64_t b : bp->bytes_sent) {
    s.bytes_sent_max = std::max(s.bytes_sent_max, b);
    s.bytes_sent_total += b;
  }
  return s;
}

void ar_bucket_plan_destroy(ar_bucket_plan_t *bp) {
  if (!bp) return;
  drop_merged(bp);
  release_bucket_scratch(bp);  // waits for the buckets' calls
  for (ar_plan_t *pl : bp->plans) {
    pl->external_scratch = nullptr;
    ar_plan_destroy(pl);
  }
  if (bp->own_stream) (void)hipStreamDestroy(bp->own_stream);
  delete bp;
}

}  // extern "C"
