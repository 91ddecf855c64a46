// plan.hpp -- host-side schedule planner of the gradient all-reduce library.
//
// The planner turns (nranks, group_size, count, dtype, schedule) into
//   1. the logical transfers of the schedule, round by round, and
//   2. the kernel launches that execute them on one GPU, with every operand
//      resolved to a rank buffer or an fp32 scratch slot.
// It is plain C++17 and touches no device.
#pragma once

#include <cstdint>
#include <string>
#include <utility>
#include <vector>

namespace ar {

// kBF16: fp32 partial sums, one rounding per element; kBF16Each: every
// partial sum rounded to bf16 as it is formed (bf16 on the wire); kI8EF: fp32
// buffers, every message blockwise INT8 codes plus one fp32 scale per block,
// with error feedback (the schedule runs over blocks of kQBlock elements).
enum Dtype : int32_t { kF32 = 0, kBF16 = 1, kBF16Each = 2, kI8EF = 3 };
constexpr int64_t kQBlock = 128;
enum Sched : int32_t { kRing = 0, kHier = 1, kRaben = 2, kRDouble = 3, kTree = 4, kDTree = 5 };
enum Exec : int32_t { kSteps = 0, kStepsUnfused = 1, kOnePass = 2 };
// The collective a plan runs: the whole all-reduce, or one of its halves.
// A reduce-scatter plan holds the schedule's reduce rounds only (after them
// every rank holds one range of the buffer fully reduced), an all-gather
// plan its copy rounds only (they spread each rank's range to every rank).
// Ring, hierarchical and Rabenseifner schedules have both halves.
enum Coll : int32_t { kAllReduce = 0, kReduceScatter = 1, kAllGather = 2 };
enum XferKind : int32_t { kReduce = 0, kCopy = 1 };

// One message of the schedule: in round `step`, rank `src` sends elements
// [lo, hi) to rank `dst`, which adds them to its own copy (kReduce) or stores
// them (kCopy).  `final_sum` marks the reduce that leaves the receiver's
// range complete.
struct Transfer {
  int32_t step, src, dst;
  int64_t lo, hi;
  int32_t kind;
  bool final_sum;
};

// Operand location codes.
constexpr int32_t kLocNone = -1;
constexpr int32_t kLocScratch = 1000;  // 1000 + s: fp32 scratch slot s

// Kernel kind codes.
//   kKReduce | flags: out = A + B (fp32 add), written to o and optionally o2.
//     flag 1: A is bf16, 2: B is bf16, 4: outputs are bf16 (rounded), 8: has o2.
//   kKCopy | elem_bytes: o = a, bit copy.
//   kKRing / kKHier / kKTree / kKDTree | dtype (0 fp32, 1 bf16, 2 bf16
//     rounded each add): one-pass fold over all ranks.  kKTree folds the
//     binomial (left-complete) tree, which is the balanced tree when N is a
//     power of two; kKDTree folds one half by one of the two double trees.
constexpr int32_t kKReduce = 0x100;
constexpr int32_t kKCopy = 0x200;
constexpr int32_t kKRing = 0x300;
constexpr int32_t kKHier = 0x400;
constexpr int32_t kKTree = 0x500;
constexpr int32_t kKDTree = 0x600;
//   kKFan | elem_bytes: one-pass all-gather, op [lo, hi) of rank a copied to
//     every other rank.
//   One-pass folds of a reduce-scatter plan store each op's result only
//   into rank o (o = kLocNone: into every rank) and carry kKOwner, which
//   selects the kernels' wider reduce-scatter tiles.
constexpr int32_t kKFan = 0xB00;
constexpr int32_t kKOwner = 0x1000;
constexpr int32_t kFlagABf = 1, kFlagBBf = 2, kFlagOBf = 4, kFlagO2 = 8;
//   Blockwise INT8 (kI8EF); op ranges count blocks, operands are ranks whose
//   code slots (codes + scales in the plan's workspace) are meant:
//   kKQEncode: codes[a] = Q(g_a + e_a), e_a = g_a + e_a - D(codes[a]).
//   kKQReduce [| kFlagO2]: codes[o] (and codes[o2]) = Q(D(codes[a]) + D(codes[b])).
//   kKQCopy: codes[o] = codes[a] (codes and scales).
//   kKQDecode: g_a = D(codes[a]).
//   Flags of the fused step lowering (no separate encode or decode launch):
//   kQFlagARaw / kQFlagBRaw: that operand is the rank's own g + e, encoded
//   in the kernel (residual written back); kQFlagDec: the outputs are the
//   ranks' final codes and are also decoded into their buffers; kQFlagNoCode:
//   nothing reads those codes later, so they are not stored.
constexpr int32_t kKQEncode = 0x700;
constexpr int32_t kKQReduce = 0x800;
constexpr int32_t kKQCopy = 0x900;
constexpr int32_t kKQDecode = 0xA00;
constexpr int32_t kQFlagARaw = 1, kQFlagBRaw = 2, kQFlagDec = 16, kQFlagNoCode = 32;

struct Op {
  int64_t lo, hi;
  int32_t a, b, o, o2;
  int32_t aux;  // one-pass folds: start rank (ring) or packed starts (hier)
};

struct Launch {
  int32_t kind;
  std::vector<Op> ops;
  // fp32 scratch: element e of a slot lives at index e - scratch_shift
  // (a merged plan's batches reuse the same slot memory one after another)
  int64_t scratch_shift = 0;
};

constexpr int64_t kDefaultCacheBytes = 256ll << 20;  // MI355X Infinity Cache (MALL)
constexpr int32_t kMaxExecRanks = 64;    // ranks a plan can execute on the GPU
constexpr int64_t kMaxLaunchOps = 65535;  // ops of one launch: workgroups along grid y
constexpr int32_t kMaxPlanRanks = 1024;  // ranks a plan can describe (stats, cost)

struct Plan {
  int32_t nranks = 0, group_size = 1;
  int64_t count = 0;
  Dtype dtype = kF32;
  Sched sched = kRing;
  Exec exec = kSteps;
  Coll coll = kAllReduce;
  int32_t nsteps = 0;            // rounds of the plan's collective
  int32_t step0 = 0;             // schedule round of its first round (its transfers keep the schedule's numbering)
  std::vector<Transfer> xfers;   // ordered by step
  std::vector<Launch> launches;  // for `exec`
  int32_t nslots = 0;            // fp32 scratch slots used by `launches`
  int64_t slot_stride = 0;       // elements per slot (multiple of 64)
  int64_t units = 0;             // what transfer ranges count: elements, or blocks (kI8EF)
  int64_t cache_bytes = kDefaultCacheBytes;  // device cache the launch order and shapes assume
  int64_t code_stride = 0;       // kI8EF: bytes of codes per rank slot (multiple of 256)
  int64_t scale_stride = 0;      // kI8EF: fp32 scales per rank slot (multiple of 64)
  std::vector<std::pair<int64_t, int64_t>> owned;  // per rank: owned_range (ring, hierarchical, Rabenseifner)
  std::vector<uint64_t> bytes_sent;
  uint64_t cross_group_bytes = 0;
  uint64_t hbm_bytes = 0;        // algorithmic device bytes of `launches`
};

// Bytes of one element on the wire (kI8EF: the code byte; scales extra).
int64_t elem_bytes(Dtype d);
// Bytes of one element of the caller's rank buffers.
int64_t buffer_elem_bytes(Dtype d);
// Bytes one transfer moves (kI8EF: codes plus 4 bytes of scale per block).
uint64_t xfer_bytes(const Plan &p, const Transfer &x);
// Elements covered by the unit range [lo, hi) of a plan.
int64_t unit_elems(const Plan &p, int64_t lo, int64_t hi);
// Device workspace of the plan in bytes (fp32 scratch, or kI8EF code slots).
uint64_t workspace_bytes(const Plan &p);

// Builds the transfers and the launches for `exec`.  Returns an empty string
// on success, else the reason for failure; *unsupported is set when the
// request is valid but not supported (Rabenseifner with N not 2^k; a
// reduce-scatter or all-gather of a schedule without those halves, of INT8,
// or in the one-pass mode).
std::string build_plan(Plan &p, int nranks, int group_size, int64_t count, Dtype dtype,
                       Sched sched, Exec exec, bool *unsupported, Coll coll = kAllReduce);

// The unit range [*lo, *hi) that `rank` holds complete after the
// reduce-scatter half of the plan's schedule (the receiver of the reduces
// that complete a range), which is also what the all-gather half spreads
// from it.  Ring, hierarchical and Rabenseifner plans; false otherwise.
bool owned_range(const Plan &p, int rank, int64_t *lo, int64_t *hi);

// Re-lowers an existing plan for another exec mode (its cache_bytes kept).
std::string relower(Plan &p, Exec exec);

// Per-round alpha-beta model over the transfers (seconds).
double cost_alpha_beta(const Plan &p, double alpha_s, double bw_intra, double bw_cross);

// The same with separate start-up costs for rounds without and with
// cross-group transfers, and an optional egress resource per group of
// bandwidth bw_egress (0 = unlimited) shared by `egress_share` identical
// instances of the collective (every group's cross-group bytes of a round,
// times egress_share, pass through it).
double cost_alpha_beta_ex(const Plan &p, double alpha_intra, double alpha_cross, double bw_intra, double bw_cross,
                          double bw_egress, double egress_share);

// Bytes one launch writes (both outputs of fused ops; fp32 partials of
// kBF16 reduces; every rank's output of a one-pass fold).
int64_t launch_write_bytes(const Plan &p, const Launch &L);

// Several independent all-reduces of one kind side by side.  Segment k is an
// all-reduce planned as parts[k] (parts[k]->count elements) at element offset
// offsets[k] of every rank buffer; the segments are disjoint and lie within
// [0, count).  Segments are taken in order into batches: in the step modes a
// batch holds as many segments as fit, by their widest launch, in
// cache_bytes (at least one); in the one-pass mode every segment is in one
// batch.  Within a batch the launch lists are merged in order: the next
// merged launch takes the next launch of every segment whose next launch has
// the kind of the first unfinished segment's next launch, so segments with
// equal launch lists share every launch.  Each segment's launches keep their
// order and every element its segment's arithmetic, so the result is that of
// the segments run one after another.  fp32 and bf16 plans only (INT8 blocks
// are counted per segment).  Empty string on success.
std::string merge_segments(Plan &out, const std::vector<const Plan *> &parts, const std::vector<int64_t> &offsets,
                           int64_t count);

// Checks that within every launch no op writes a (location, range) that
// another op of the same launch reads or writes.  Empty string if clean.
std::string check_hazards(const Plan &p);

// Overlap model (see ar_overlap_step_time).
double overlap_step_time(int nchunks, const double *ready, const double *comm, double compute_end, double update,
                         double *exposed);

// Bucket fuser: assigns tensors (element counts) to buckets in reverse
// tensor order under `cap_elems`; fills per-tensor arena offsets, bucket
// ranges and the arena length.  Buckets start on `align_elems` boundaries.
void assign_buckets(const std::vector<int64_t> &tensor_counts, int64_t cap_elems,
                    int64_t align_elems, std::vector<int64_t> &tensor_offsets,
                    std::vector<int64_t> &bucket_offset, std::vector<int64_t> &bucket_count,
                    int64_t &arena_count);

}  // namespace ar
