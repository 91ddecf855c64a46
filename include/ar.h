/*
 * ar.h -- C ABI of the MI355X gradient all-reduce library (libar.so).
 *
 * N virtual ranks' gradient buffers live in one GPU's HBM.  The library runs
 * the chunked reduce and copy schedules of gradient all-reduce on them, in
 * place, with hand-written HIP kernels for gfx950:
 *
 *   AR_RING          ring reduce-scatter followed by ring all-gather.
 *                    "Collective communication: algorithms, cost and the
 *                    library that runs them" (AI training network primer,
 *                    ch. 4), section 4.2, the two index rules and Figures
 *                    4.1-4.3; "Collective communication" (Scaling ML systems,
 *                    ch. 06), the "Ring AllReduce" algorithm box.
 *   AR_HIERARCHICAL  intra-group ring reduce-scatter, all-reduce of each slice
 *                    among the ranks with the same local index across groups,
 *                    intra-group ring all-gather.  Primer ch. 4 section 4.4
 *                    (Figure 4.8, Animation 4.3); "Chapter 7. Data-center
 *                    networks" (AI infrastructure book), section 7.2.1.
 *   AR_RABENSEIFNER  recursive-halving reduce-scatter then recursive-doubling
 *                    all-gather.  Primer ch. 4 section 4.3 (Figure 4.5,
 *                    Animation 4.2); Scaling ML systems ch. 06, "Recursive
 *                    halving and doubling (butterfly)".
 *   AR_RECURSIVE_DOUBLING  log2 N steps; in step k every rank exchanges its
 *                    whole buffer with rank i xor 2^k and both add.  Primer
 *                    ch. 4 section 4.3 ("Trees: latency-optimal,
 *                    bandwidth-poor", Figure 4.5).  N a power of two.
 *   AR_TREE          binary tree: the whole buffer is reduced up a binomial
 *                    tree rooted at rank 0 (in step k, rank m*2^(k+1) adds
 *                    what rank m*2^(k+1) + 2^k sends), then broadcast down
 *                    the same edges.  Scaling ML systems ch. 06, "Tree
 *                    AllReduce".  Any N; ceil(log2 N) steps each way.
 *   AR_DOUBLE_TREE   two complementary binary trees, the second the mirror
 *                    of the first (rank r plays node N-1-r), each reducing
 *                    and broadcasting half of the buffer.  Scaling ML systems
 *                    ch. 06, "Double binary tree"; Primer Figure 4.6 (tree 1
 *                    for N = 8: 0 <- 4 <- {2, 6} <- {1, 3, 5, 7}).  A node
 *                    adds its lower-ranked child's part before the higher.
 *                    N a power of two.
 *
 * Result.  On completion every rank buffer holds G_0 + ... + G_{N-1}
 * (Scaling ML systems ch. 06, the algorithm box's output), summed in the
 * exact per-element order of the chosen schedule: floating-point addition is
 * not associative, so the schedule fixes the low bits.
 *
 * Datatypes.  AR_FLOAT32: one IEEE binary32 add per reduction, denormals
 * kept.  AR_BFLOAT16: inputs widen exactly to fp32, partial sums are kept in
 * fp32 (in plan-owned device scratch), and each element is rounded to bf16
 * (nearest, ties to even; NaN stays NaN with its sign) once, when its chunk
 * is complete; all-gather copies bf16 bits.
 *
 * Partition.  A range of L elements cut into K parts gives part c the
 * elements [floor(c*L/K), floor((c+1)*L/K)).
 *
 * Conventions.  All calls are thread-compatible, not thread-safe per plan.
 * Errors never abort: a failing call returns a status (or NULL / a negative
 * value) and sets a thread-local message readable with ar_last_error().
 */
#ifndef AR_H
#define AR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  AR_OK = 0,
  AR_ERR_INVALID_ARG = 1, /* bad argument: sizes, NULL or misaligned pointers */
  AR_ERR_UNSUPPORTED = 2, /* e.g. Rabenseifner with N not a power of two       */
  AR_ERR_OOM = 3,         /* device scratch or table allocation failed         */
  AR_ERR_HIP = 4,         /* a HIP runtime call or kernel launch failed         */
  AR_ERR_GUARD = 5        /* a guard zone around device workspace was written  */
} ar_status_t;

/* AR_BFLOAT16: fp32 partial sums, each element rounded once (see above).
 * AR_BFLOAT16_EACH_STEP: bf16 buffers whose every partial sum is rounded to
 * bf16 (nearest, ties to even) as it is formed, as when each message of the
 * schedule carries bf16 values; no scratch is used.
 * AR_INT8_EF: compressed all-reduce of fp32 buffers ("Collective
 * communication", Scaling ML systems ch. 06, "Gradient compression":
 * INT8 quantization, "Blockwise quantization", "Definition: error feedback
 * mechanism").  Buffers are cut into blocks of 128 elements (the last may be
 * short); a block x travels as codes q = round(x / s) (nearest, ties to even,
 * clamped to [-127, 127]) and one fp32 scale s = max|x| / 127 (a zero block
 * has s = 0 and codes 0), and is read back as q * s.  Each rank first encodes
 * x = g + e (e = its error buffer, or 0) and, with error feedback, stores
 * e = x - q * s.  Every message of the schedule carries codes and scales: a
 * receiver decodes the message and its own codes, adds in fp32 and
 * re-encodes the sum; forwarding copies codes.  At the end each rank's
 * buffer holds the decoded codes it ends with (identical on every rank).
 * The schedule runs over blocks; in the step modes the codes live in
 * plan-owned device memory (about 1.03 bytes per element per rank), in
 * AR_EXEC_ONEPASS they stay in registers (each block folds every rank's
 * contribution in the schedule's order, re-encoding every partial sum).
 * Inputs must be finite. */
typedef enum { AR_FLOAT32 = 0, AR_BFLOAT16 = 1, AR_BFLOAT16_EACH_STEP = 2, AR_INT8_EF = 3 } ar_dtype_t;

typedef enum {
  AR_RING = 0,
  AR_HIERARCHICAL = 1,
  AR_RABENSEIFNER = 2,
  AR_RECURSIVE_DOUBLING = 3,
  AR_TREE = 4,
  AR_DOUBLE_TREE = 5
} ar_schedule_t;

/*
 * How a plan is executed.  Every mode gives bit-identical results (a
 * reduce-scatter: on its owned ranges).
 *   AR_EXEC_STEPS          one kernel launch per step of the schedule; the
 *                          reduce-scatter step that completes a chunk is fused
 *                          with the all-gather step that first forwards it
 *                          (the receiver writes the finished chunk to itself
 *                          and to the next rank).  Default.
 *   AR_EXEC_STEPS_UNFUSED  one kernel launch per step, no fusion.
 *   AR_EXEC_ONEPASS        one launch for the whole all-reduce: every element
 *                          is read once from each rank, folded in the
 *                          schedule's exact order, and written once to each
 *                          rank.  From 4 ranks up (fp32 and bf16) a workgroup
 *                          stages a tile of every rank in LDS, folds it one
 *                          word per thread, and each wave stores its own
 *                          ranks; otherwise, and for AR_INT8_EF, each thread
 *                          folds in registers and stores into every rank.
 *                          (For reduce-scatter and all-gather plans see
 *                          ar_collective_t.)
 */
typedef enum { AR_EXEC_STEPS = 0, AR_EXEC_STEPS_UNFUSED = 1, AR_EXEC_ONEPASS = 2 } ar_exec_t;

/* Maximum number of virtual ranks a plan can run on the GPU. */
#define AR_MAX_RANKS 64
/* Maximum number of ranks a plan can describe: plans of more than
 * AR_MAX_RANKS ranks give transfers, statistics and the cost model only
 * (ar_allreduce returns AR_ERR_UNSUPPORTED for them). */
#define AR_MAX_PLAN_RANKS 1024

typedef struct ar_plan ar_plan_t;

typedef struct {
  int32_t nranks, group_size;
  uint32_t steps;                   /* sequential rounds of the plan's collective   */
  uint32_t launches;                /* kernel launches per call in the exec mode    */
  uint64_t count, elem_bytes;       /* elem_bytes: of the rank buffers               */
  const uint64_t *bytes_sent;       /* [nranks], plan-owned: logical bytes each rank
                                       sends, in the buffer's dtype (AR_INT8_EF: one
                                       byte per element plus 4 per block)           */
  uint64_t bytes_sent_max, bytes_sent_total;
  uint64_t cross_group_bytes_total; /* bytes whose sender and receiver lie in
                                       different groups of group_size contiguous
                                       ranks (Data-center networks 7.2.1)          */
  uint64_t hbm_bytes_model;         /* device bytes read + written per call in the
                                       exec mode (algorithmic count)               */
  uint64_t scratch_bytes;           /* device workspace the plan owns: fp32 partial
                                       sums, or (AR_INT8_EF) codes and scales       */
  int32_t exec;                     /* ar_exec_t in effect                          */
} ar_stats_t;

/*
 * Builds the schedule for nranks virtual ranks of `count` elements each.
 * Host only: no device memory is touched until the first ar_allreduce (or
 * ar_plan_prepare).  group_size: ranks g*G .. g*G+G-1 form group g; it must
 * divide nranks.  For AR_HIERARCHICAL it sets the intra-group size; for the
 * other schedules it only labels groups for cross_group_bytes_total.
 * Returns NULL on error: nranks outside [1, AR_MAX_PLAN_RANKS], group_size < 1 or
 * not dividing nranks, unknown dtype or schedule (AR_ERR_INVALID_ARG);
 * Rabenseifner, recursive doubling or the double tree with nranks not a
 * power of two (AR_ERR_UNSUPPORTED).
 */
ar_plan_t *ar_plan_create(int nranks, int group_size, size_t count, ar_dtype_t dtype,
                          ar_schedule_t schedule);

/* Selects the execution mode (see ar_exec_t).  Host only. */
ar_status_t ar_plan_set_exec(ar_plan_t *plan, ar_exec_t exec);

/*
 * The device cache capacity (bytes) the plan's launch order and kernel
 * shapes assume; default 256 MiB, MI355X's Infinity Cache.  Every round of a
 * schedule writes what the next round of its chain reads (Primer ch. 4
 * sections 4.2-4.4: each step forwards what the previous one produced), and
 * that output is still cached only if it fits:
 *   - a step launch that writes more than this into rank buffers takes the
 *     streaming kernel shape;
 *   - the hierarchical schedule runs its two group phases group by group
 *     (all rounds of group 0, then group 1, ...) when one round of a phase
 *     would write more than this;
 *   - then, for every schedule, a launch round whose output still exceeds
 *     this runs together with the next round of its chain (the round that
 *     reads it; the last reduce round also with the copy round fused into
 *     it) as one block, and the block runs piece by piece: the element
 *     range is cut into the fewest pieces (multiples of 64 elements, the
 *     same offsets on every rank) whose rounds write at most this.  The
 *     other rounds run whole.
 * Results are bit-identical for any value.  Host only.
 */
ar_status_t ar_plan_set_cache_bytes(ar_plan_t *plan, size_t bytes);

/*
 * Allocates the plan's device op tables and, for bf16, its fp32 scratch on
 * the current HIP device, and uploads the tables (synchronously).  Called
 * implicitly by the first ar_allreduce; call it explicitly before capturing
 * ar_allreduce into a HIP graph.  AR_ERR_OOM / AR_ERR_HIP on failure;
 * AR_ERR_UNSUPPORTED for a plan of more than 64 ranks (planned for its
 * statistics and cost model only) or a launch beyond one dispatch's limits
 * (more than 65535 ops, or one op of more tiles than 2^31 - 1 work-items
 * hold).  A plan is bound to the device current at its first prepare.
 */
ar_status_t ar_plan_prepare(ar_plan_t *plan);

/*
 * All-reduce, in place.  rank_bufs: host array of nranks device pointers,
 * read during the call only; buffer r holds >= count elements of the plan's
 * dtype, is 16-byte aligned and overlaps no other rank's buffer (with
 * count == 0 nothing is touched and the pointers may be NULL).  stream: a
 * hipStream_t (NULL = default stream).  Enqueues the kernels and returns;
 * the result is visible after stream synchronisation (the initiating call of
 * a collective returns before completion -- Scaling ML systems ch. 06).
 * Calls that share a plan must not overlap in time (they share scratch).
 * AR_ERR_INVALID_ARG for NULL/misaligned/overlapping pointers or a
 * different device than the plan's; the errors of ar_plan_prepare on the
 * first call; AR_ERR_HIP if a launch fails.
 */
ar_status_t ar_allreduce(ar_plan_t *plan, void *const *rank_bufs, void *stream);

/*
 * Compressed all-reduce with error feedback (AR_INT8_EF plans; Scaling ML
 * systems ch. 06, "Definition: error feedback mechanism": each worker keeps a
 * residual e, sends C(g + e) and keeps g + e - C(g + e)).  error_bufs: host
 * array of nranks device pointers to fp32 buffers of count elements, 16-byte
 * aligned, disjoint from each other and from the rank buffers; each is read
 * and overwritten with the rank's new residual.  error_bufs == NULL runs the
 * compressed all-reduce without error feedback (as ar_allreduce does).
 * Rank buffers as for ar_allreduce (fp32).  AR_ERR_INVALID_ARG for a plan of
 * another dtype with error_bufs != NULL, and for bad pointers.
 */
ar_status_t ar_allreduce_ef(ar_plan_t *plan, void *const *rank_bufs, void *const *error_bufs, void *stream);

/*
 * The two halves of an all-reduce as collectives of their own.  Scaling ML
 * systems ch. 06, "Six basic primitives": an all-reduce is a reduce-scatter
 * followed by an all-gather, which is how the ring runs; FSDP calls the two
 * halves separately (all-gather of parameter shards before a layer runs,
 * reduce-scatter of gradients after the backward pass, each rank keeping its
 * shard).  Primer ch. 4 section 4.2: after the N-1 reduce-scatter steps rank
 * i holds chunk (i+1) mod N complete; each half sends (N-1)/N * S per rank.
 *
 *   AR_ALLREDUCE       the whole schedule (ar_plan_create).
 *   AR_REDUCE_SCATTER  the schedule's reduce rounds only: ring steps
 *                      0..N-2; hierarchical phase 1 and the reduce half of
 *                      the cross-group ring (Primer 4.4); Rabenseifner's
 *                      recursive halving (Primer 4.3).  Afterwards rank r's
 *                      owned range (ar_plan_owned_range) holds the reduced
 *                      values, with the same bits as the all-reduce gives
 *                      there.  In the step modes its other elements hold
 *                      what the schedule left in them: fp32 and
 *                      AR_BFLOAT16_EACH_STEP partial sums, while AR_BFLOAT16
 *                      keeps its fp32 partials in the plan's scratch and
 *                      leaves those elements unchanged; AR_EXEC_ONEPASS folds
 *                      each owned range from every rank in the schedule's
 *                      order and stores it into its owner only, leaving every
 *                      other element unchanged.
 *   AR_ALLGATHER       the schedule's copy rounds only: the cross-group
 *                      ring's copy half and phase 3 for the hierarchical
 *                      schedule, recursive doubling for Rabenseifner.  Each
 *                      rank's owned range is read from that rank and written
 *                      to every other rank; nothing else is read.
 *                      AR_EXEC_ONEPASS does that in one launch: a workgroup
 *                      reads a tile of an owned range once and each of its
 *                      waves stores it into its own ranks.
 */
typedef enum { AR_ALLREDUCE = 0, AR_REDUCE_SCATTER = 1, AR_ALLGATHER = 2 } ar_collective_t;

/*
 * ar_plan_create for one collective.  AR_REDUCE_SCATTER and AR_ALLGATHER
 * plans take the ring, hierarchical or Rabenseifner schedule and fp32 or
 * bf16 (either mode), and run in every exec mode (AR_EXEC_STEPS and
 * AR_EXEC_STEPS_UNFUSED are the same here: no reduce is followed by a copy);
 * other schedules and AR_INT8_EF give AR_ERR_UNSUPPORTED.  Statistics,
 * the cost models, graphs, profiling and guard zones cover the plan's own
 * rounds.  The plan runs with ar_reduce_scatter or ar_allgather only
 * (ar_allreduce, ar_allreduce_ef and ar_allreduce_noalloc refuse it with
 * AR_ERR_INVALID_ARG); other errors as for ar_plan_create.
 */
ar_plan_t *ar_plan_create_collective(int nranks, int group_size, size_t count, ar_dtype_t dtype,
                                     ar_schedule_t schedule, ar_collective_t collective);

/*
 * The element range [*lo, *hi) that `rank` holds complete after the
 * reduce-scatter half of the plan's schedule: the range the receiver of each
 * completing reduce owns, which the all-gather half spreads from it.  Ring:
 * chunk (rank+1) mod N; Rabenseifner: the chunk whose index is `rank` with
 * its log2 N bits reversed (Primer 4.3, Animation 4.2); hierarchical: within
 * slice l = rank mod G, sub-chunk (g+1) mod M of the cross-group ring of
 * group g = rank / G.  Chunks are part(count, K, c) =
 * [floor(c*count/K), floor((c+1)*count/K)), so a range can be empty.  Any
 * collective of these schedules; host only.  AR_ERR_INVALID_ARG for a rank
 * outside [0, nranks) or NULL pointers, AR_ERR_UNSUPPORTED for other
 * schedules.
 */
ar_status_t ar_plan_owned_range(const ar_plan_t *plan, int rank, size_t *lo, size_t *hi);

/*
 * Reduce-scatter and all-gather, in place, for plans of those collectives.
 * Buffers, stream, errors and completion as for ar_allreduce.  Before
 * ar_allgather each rank's owned range must hold its values; ar_reduce_scatter
 * then ar_allgather on the same buffers give the all-reduce's bits in every
 * element.
 */
ar_status_t ar_reduce_scatter(ar_plan_t *plan, void *const *rank_bufs, void *stream);
ar_status_t ar_allgather(ar_plan_t *plan, void *const *rank_bufs, void *stream);

/* Statistics of the plan (valid until the plan is destroyed or re-moded). */
ar_stats_t ar_plan_stats(const ar_plan_t *plan);

/*
 * Per-round alpha-beta time in seconds (Data-center networks 7.2.1):
 *   T = sum over rounds r of (alpha + max over transfers e of V_{r,e} / B_e),
 * B_e = bw_intra_Bps within a group, bw_cross_Bps across groups; every rank
 * has its own link of each class.  Negative on error.
 */
double ar_plan_cost_alpha_beta(const ar_plan_t *plan, double alpha_s, double bw_intra_Bps,
                               double bw_cross_Bps);

/*
 * Resource model of Data-center networks 7.6.4 (T_grad), a generalisation
 * of the above: a round costs alpha_cross_s if it has any cross-group
 * transfer, else alpha_intra_s, plus the slowest resource of the round:
 * each rank's intra and cross links, and -- when bw_group_egress_Bps > 0 --
 * one egress per group that carries the group's cross-group bytes of the
 * round times egress_share (the number of identical collectives that share
 * the egress, e.g. one per tensor-parallel coordinate).
 */
typedef struct {
  double alpha_intra_s, alpha_cross_s;
  double bw_intra_Bps, bw_cross_Bps;
  double bw_group_egress_Bps; /* 0: no egress limit */
  double egress_share;        /* >= 1 */
} ar_cost_params_t;

double ar_plan_cost_alpha_beta_ex(const ar_plan_t *plan, const ar_cost_params_t *params);

/*
 * Schedule selector (the choice NCCL makes per call from its alpha-beta
 * tables: Primer ch. 4 section 4.3 "crossover"; Scaling ML systems ch. 06,
 * "Algorithm crossover"): the schedule in `candidates` (bit 1 << schedule)
 * with the lowest ar_plan_cost_alpha_beta_ex time for these sizes.
 * Schedules that cannot serve nranks (power-of-two ones) are skipped.
 * Returns the schedule and writes its time to *best_s (if not NULL), or -1
 * on error (no candidate fits, bad arguments).  Host only.
 */
int ar_select_schedule(int nranks, int group_size, size_t count, ar_dtype_t dtype,
                       const ar_cost_params_t *params, uint32_t candidates, double *best_s);

/*
 * All-reduce that allocates nothing, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Same arguments, checks and results as ar_allreduce_ef
 * (error_bufs == NULL for every dtype but AR_INT8_EF with error feedback);
 * bit-identical to ar_allreduce / ar_allreduce_ef on the same plan.
 *
 * The plan's device workspace -- its op table, then its fp32 partial sums
 * (AR_BFLOAT16) or INT8 code slots (AR_INT8_EF) -- lives in one array of
 * AR_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs on,
 * from its load until the process ends, instead of in memory the plan
 * allocates; the call never allocates or frees device memory, creates no
 * event and copies nothing through the copy engines.  The op table is written
 * into the array by small kernel launches when the array holds another
 * plan's table (and always while `stream` is being captured, so a captured
 * graph carries it); no part of the array needs to start at zero.
 *
 * All calls on one GPU share its array and leave their contents in it:
 * allocation-free calls that overlap in time on one GPU race, whatever their
 * plans and streams (run them in one stream or order them), and a captured
 * graph of this call must not overlap another allocation-free call on that
 * GPU either.  Graph replay (ar_plan_set_graph) and the profiling log do not
 * apply: the launches are enqueued eagerly on `stream`.  Destroying or
 * re-moding the plan does not wait for these calls: synchronise `stream`
 * first.
 *
 * Errors: as ar_allreduce_ef; AR_ERR_INVALID_ARG (before any device work)
 * when the op table (40 bytes per op, rounded up to 256) plus the workspace
 * (ar_plan_stats().scratch_bytes) exceed AR_NOALLOC_SCRATCH_BYTES, e.g. a bf16
 * ring plan of more than about 16.7 M elements per rank.
 */
#define AR_NOALLOC_SCRATCH_BYTES (64ull << 20)
ar_status_t ar_allreduce_noalloc(ar_plan_t *plan, void *const *rank_bufs, void *const *error_bufs, void *stream);

/* Releases the plan and its device memory, after waiting for the plan's own
 * calls in flight (ar_allreduce / ar_allreduce_ef / the bucket calls; each
 * call records an event on its stream, except while the caller captures that
 * stream into a graph of its own -- such work, and allocation-free calls,
 * the caller finishes before destroying the plan). */
void ar_plan_destroy(ar_plan_t *plan);

/* Thread-local message and status of the last failing call. */
const char *ar_last_error(void);
ar_status_t ar_last_status(void);

/* ---- Plan inspection (host only; used to check the planner on a CPU) ---- */

/* Logical transfers of the schedule: per transfer its round, sender,
 * receiver, element range and kind (0 = reduce, 1 = copy); for AR_INT8_EF
 * the range counts 128-element blocks.  Returns the total number of
 * transfers (writes at most cap), or -1 on error. */
int64_t ar_plan_transfers(const ar_plan_t *plan, int32_t *step, int32_t *src, int32_t *dst,
                          int64_t *lo, int64_t *hi, int32_t *kind, int64_t cap);

/*
 * Kernel launches of the exec mode.  ar_plan_launch_info gives launch i's
 * kernel kind code and op count.  ar_plan_launch_ops writes its ops: element
 * range [lo, hi), and operand locations a, b (inputs), o, o2 (outputs):
 * a location 0..nranks-1 is that rank's buffer, 1000+s is fp32 scratch slot s,
 * -1 is unused.  aux is the fold start (one-pass kernels).  AR_INT8_EF plans
 * use kinds 0x700 (encode rank a), 0x800 (o [and o2 with flag 8] = re-encoded
 * decode(a) + decode(b)), 0x900 (copy a's codes to o) and 0xA00 (decode a
 * into its buffer), and in one-pass mode the fold kinds with dtype code 3;
 * their ranges count blocks and locations name ranks' code slots.  The
 * one-pass all-gather is kind 0xB00 | element bytes (op range of rank a to
 * every other rank); a one-pass reduce-scatter fold carries flag 0x1000
 * (each op's result goes to rank o only).  Host only.
 */
int32_t ar_plan_num_launches(const ar_plan_t *plan);
ar_status_t ar_plan_launch_info(const ar_plan_t *plan, int32_t i, int32_t *kind, int32_t *nops);
ar_status_t ar_plan_launch_ops(const ar_plan_t *plan, int32_t i, int64_t *lo, int64_t *hi,
                               int32_t *a, int32_t *b, int32_t *o, int32_t *o2, int32_t *aux);
/* Kernel shape of launch i: *cold = 1 for the streaming shape (the launch
 * writes more into rank buffers than the assumed device cache), the units
 * each thread moves per tile (16-byte fp32 or 8-byte bf16 units; for the
 * LDS-staged one-pass folds, 16-byte units per lane and rank), the store
 * cache policy (bits of the store instruction: 2 non-temporal, 16 sc1), the
 * ranks a register one-pass fold loads together or the waves per workgroup
 * at most of an LDS-staged fold (0 otherwise), the
 * workgroups along the tiles, the threads per workgroup and the dynamic LDS
 * bytes per workgroup (nonzero only for the LDS-staged one-pass folds, which
 * stage a tile of every rank in LDS before folding it; INT8 kernels: units,
 * cpol, batch and LDS bytes 0).  The one-pass all-gather reports its tile's
 * 16-byte units per lane of one wave (each wave stores the whole tile into
 * its ranks), its waves per workgroup as batch and its static LDS stage.
 * Any out pointer may be NULL.  Host only. */
ar_status_t ar_plan_launch_shape(const ar_plan_t *plan, int32_t i, int32_t *cold, int32_t *units, int32_t *cpol,
                                 int32_t *batch, uint32_t *grid_x, int32_t *threads, int32_t *lds_bytes);
/* fp32 scratch addressing of launch i: element e of slot s is float
 * s * slot_stride + e - shift of the scratch.  shift is 0 except in a
 * batched bucket plan, whose batches reuse the slots one after another
 * (shift = the batch's first arena element).  Host only. */
ar_status_t ar_plan_launch_scratch(const ar_plan_t *plan, int32_t i, int64_t *shift, int64_t *slot_stride);

/*
 * Graph replay (host call, no device work).  With enable != 0, ar_allreduce
 * and ar_allreduce_ef capture the plan's whole launch sequence into a HIP
 * graph the first time they see a set of buffer pointers, and from then on
 * replay it with one graph launch on the caller's stream (the pages'
 * persistent collectives register an operation once for many calls --
 * Scaling ML systems ch. 06, "collective semantics").  Up to 8 pointer sets are
 * kept per plan; the oldest is dropped (after a device synchronisation) when
 * a ninth appears.  The graphs hold kernel nodes only.  Results are
 * bit-identical to eager calls.  While per-launch profiling is on
 * (ar_plan_set_profiling), calls run eagerly.  Changing the exec mode or the
 * profiling log, or calling this function, drops the cached graphs.
 */
ar_status_t ar_plan_set_graph(ar_plan_t *plan, int enable);

/* ---- Debug aids ---- */

/*
 * The plan as JSON (NUL-terminated, truncated to cap - 1 bytes): its
 * configuration; its schedule step by step ("step_list": per step, every
 * transfer as [sender, receiver, lo, hi, kind], kind 0 reduce / 1 copy, the
 * step list of Primer ch. 4 Figure 4.2 for a ring); and its launches
 * ("launch_list": kernel kind code, ops, streaming shape, grid width,
 * element range, bytes written, and the mean duration in ms over the
 * profiling log's calls that timed it, or null).  Returns the full length
 * (call with cap = 0 to size the buffer), -1 on error.  Waits for the
 * plan's calls in flight.
 * With the environment variable AR_TRACE=1 every plan keeps a profiling log
 * of its last 16 calls (calls run eagerly) and writes this description to
 * stderr when it is destroyed; AR_TRACE=<path> appends it to that file, one
 * line per plan.  Results are unchanged.
 */
int64_t ar_plan_describe(const ar_plan_t *plan, char *buf, size_t cap);

/*
 * Guard zones around the plan's device scratch (fp32 partial sums, INT8
 * code slots): with bytes > 0 (a multiple of 256, at most 1 GiB) the scratch
 * is allocated at the next prepare with `bytes` extra on each side, filled
 * with 0xA7.  ar_plan_check_guards waits for the plan's calls and returns
 * AR_ERR_GUARD, naming the first overwritten byte, if a kernel wrote into
 * either zone.  A debug aid for tests; results are unchanged.
 */
ar_status_t ar_plan_set_guard(ar_plan_t *plan, size_t bytes);
ar_status_t ar_plan_check_guards(ar_plan_t *plan);

/* ---- Timing ---- */

/* Per-launch timing.  With max_calls > 0, each ar_allreduce launches every
 * kernel with a start and a stop HIP event that the dispatch itself records
 * (hipExtLaunchKernel; no extra packet between kernels), into a log holding
 * the events of the last max_calls calls (older calls are overwritten);
 * max_calls = 0 turns it off.  Events are allocated at the next prepare, not
 * on the hot path. */
ar_status_t ar_plan_set_profiling(ar_plan_t *plan, int max_calls);

/* Samples the log: with period P > 1, logged call c times only the launches
 * i with (i + c) mod P == 0 (fewer events per call; over P consecutive calls
 * every launch is timed once).  Default 1: every launch.  Host only. */
ar_status_t ar_plan_set_profiling_period(ar_plan_t *plan, int period);

/* Cold-cache timing: with bytes > 0, every launch that the profiling log
 * times is preceded on the call's stream by a kernel that writes `bytes` of
 * buf with plain stores (device memory the caller owns, 16-byte aligned, a
 * multiple of 16 bytes; make it several times the device cache, e.g.
 * 1 GiB), so that the timed launch finds none of its inputs in the cache
 * (MI355X's 256 MB Infinity Cache, which stores allocate in; reads do not).
 * The fill runs outside the launch's own start and stop events, but the
 * timed launch may still pay for writing back the fill's lines it evicts, so
 * its time is an upper bound of the cold time.  bytes = 0 (default) turns it
 * off.  Results are unchanged.  Host only. */
ar_status_t ar_plan_set_profiling_evict(ar_plan_t *plan, void *buf, size_t bytes);

/* Durations in ms of every launch of the logged calls, oldest call first:
 * ms[c * launches + i] is launch i of logged call c, from the kernel's start
 * to its end, or -1 if the profiling period left it untimed.  The caller must have
 * synchronised the stream.  *n receives calls * launches; the log is then
 * cleared. */
ar_status_t ar_plan_launch_times(ar_plan_t *plan, float *ms, int32_t cap, int32_t *n);

/*
 * HBM probe, the attainable-bandwidth reference of the kernels above (Primer
 * ch. 4 section 4.8 judges a collective against what its path can carry):
 * over `bytes` of every buffer (16-byte aligned pointers, bytes a multiple of
 * 16), each 16-byte unit of each of the ndst destinations receives the fp32
 * sum of that unit of the nsrc sources, with the access pattern of the step
 * kernels (`units` 16-byte units per thread per tile, 1, 2 or 4).  policy 0:
 * plain loads and stores (they allocate in the device caches); 1:
 * non-temporal loads and sc1 stores (the step kernels' policy); 2:
 * non-temporal loads and stores (the one-pass kernels').  policy | 4: each
 * workgroup stores one destination only (workgroup b: tile b / ndst into
 * destination b mod ndst, reading every source for it; ndst >= 1), so each
 * wave writes one buffer, the store pattern of the LDS-staged one-pass
 * folds; without it each workgroup stores its tile into every destination,
 * the pattern of the register folds.  nsrc = 1, ndst = 1 is a copy; 2, 1 a
 * reduce step's mix; 0, 1 a fill (writes zeros); k, 0 only reads.  At most
 * 64 buffers of each kind; a destination may equal a source (in place).
 * Enqueued on `stream`.
 */
ar_status_t ar_hbm_probe(const void *const *src, int32_t nsrc, void *const *dst, int32_t ndst, size_t bytes,
                         int32_t units, int32_t policy, void *stream);

/* ---- Bucket fuser (Scaling ML systems ch. 06, "Bucket fusion") ----
 *
 * Gradient tensors are assigned to buckets in reverse tensor order (the
 * order backward produces them).  A bucket is closed before a tensor that
 * would take it past bucket_cap_bytes; a tensor larger than the cap gets a
 * bucket of its own.  Within a bucket tensors are packed back to back in
 * assignment order; every bucket starts 256-byte aligned in a per-rank
 * arena.  One all-reduce plan runs per bucket, in bucket order, on one
 * stream; the gaps between buckets are never touched.
 *
 * Batched execution (the default for fp32 and bf16 dtypes when no events
 * are given): the buckets' all-reduces share launches.  Buckets are taken in
 * order into batches whose widest round writes at most the plan's assumed
 * device cache (ar_plan_set_cache_bytes; no such limit in the one-pass
 * mode) and whose launches hold at most 65535 ops (the workgroups one
 * launch grid holds along the ops: 4095 buckets at 16 ranks), and launch i
 * of a batch runs launch i of each of its buckets, so a batch costs the
 * launches of one bucket.  Every bucket is
 * still its own all-reduce with its own partition and summation order: the
 * result is bit for bit that of the buckets run one by one.  For bf16 the
 * batched plan owns an fp32 scratch that the batches reuse one after
 * another (nslots x the widest batch's extent x 4 bytes).
 */
typedef struct ar_bucket_plan ar_bucket_plan_t;

ar_bucket_plan_t *ar_bucket_plan_create(int nranks, int group_size, const size_t *tensor_counts,
                                        int ntensors, ar_dtype_t dtype, ar_schedule_t schedule,
                                        size_t bucket_cap_bytes);
/* tensor_offsets[t]: element offset of tensor t in each rank's arena;
 * *arena_count: arena length in elements. */
ar_status_t ar_bucket_layout(const ar_bucket_plan_t *bp, size_t *tensor_offsets,
                             size_t *arena_count);
int32_t ar_bucket_count(const ar_bucket_plan_t *bp);
/* Element offset and length of bucket b in the arena. */
ar_status_t ar_bucket_range(const ar_bucket_plan_t *bp, int32_t b, size_t *offset, size_t *count);
ar_status_t ar_bucket_set_exec(ar_bucket_plan_t *bp, ar_exec_t exec);
/* Graph replay for every bucket's plan and the batched plan (see
 * ar_plan_set_graph). */
ar_status_t ar_bucket_set_graph(ar_bucket_plan_t *bp, int enable);
/* ar_plan_set_cache_bytes for every bucket's plan; the batched plan is
 * rebuilt with the new size on its next use.  Host only. */
ar_status_t ar_bucket_set_cache_bytes(ar_bucket_plan_t *bp, size_t bytes);
/* Guard zones (see ar_plan_set_guard) around the scratch the buckets share
 * when run one by one, and around every bucket's and the batched plan's own
 * scratch; the check covers all of them. */
ar_status_t ar_bucket_set_guard(ar_bucket_plan_t *bp, size_t bytes);
ar_status_t ar_bucket_check_guards(ar_bucket_plan_t *bp);
/* enable = 0: ar_bucket_allreduce runs the buckets one by one, each with its
 * own launches; non-zero (default): batched.  Host only. */
ar_status_t ar_bucket_set_batching(ar_bucket_plan_t *bp, int enable);
/* The batched plan (built on first use, owned by bp, valid until the exec
 * mode changes or bp is destroyed), for inspection, profiling and graph
 * settings through the ar_plan_* calls: its count is the arena length and
 * its launches are what batched ar_bucket_allreduce runs.  NULL, with
 * AR_ERR_UNSUPPORTED, for AR_INT8_EF (INT8 buckets always run one by one);
 * NULL with AR_ERR_INVALID_ARG for a plan without buckets.  Not to be passed
 * to ar_plan_destroy. */
ar_plan_t *ar_bucket_batched_plan(ar_bucket_plan_t *bp);
/* All-reduces every bucket of the nranks arenas (16-byte aligned device
 * pointers of arena_count elements), in place, on `stream` (batched unless
 * turned off or AR_INT8_EF). */
ar_status_t ar_bucket_allreduce(ar_bucket_plan_t *bp, void *const *rank_arenas, void *stream);
/* Overlap with the backward pass (Scaling ML systems ch. 06, "Overlap layer
 * by layer" and "Bucket fusion"; Primer ch. 4 section 4.7): like
 * ar_bucket_allreduce, but bucket b's all-reduce first waits on
 * ready_events[b] (a hipEvent_t the producer of its gradients recorded, on
 * any stream; NULL = ready now), and done_events[b] (if the array and the
 * entry are not NULL) is recorded on `stream` after it.  So each bucket
 * starts when it is ready and the previous bucket's all-reduce is done, as in
 * Figure 4.15.  Both arrays have ar_bucket_count entries.  With either array
 * given, the buckets run one by one (not batched). */
ar_status_t ar_bucket_allreduce_after(ar_bucket_plan_t *bp, void *const *rank_arenas, void *stream,
                                      void *const *ready_events, void *const *done_events);
/* The same for AR_INT8_EF bucket plans with error feedback: error_arenas
 * (NULL = none) are nranks fp32 arenas laid out like the rank arenas, each
 * bucket's range used as that bucket's error buffers (see ar_allreduce_ef).
 * ready_events / done_events as above (either may be NULL). */
ar_status_t ar_bucket_allreduce_ef(ar_bucket_plan_t *bp, void *const *rank_arenas, void *const *error_arenas,
                                   void *stream, void *const *ready_events, void *const *done_events);

/* The overlap model of Primer ch. 4 section 4.7 (Figure 4.15) and
 * Data-center networks 7.6.2: chunk k's collective starts at
 * max(ready_s[k], end of chunk k-1's collective) and lasts comm_s[k]; the
 * step ends update_s after both the compute (compute_end_s) and the last
 * collective are done.  Returns the step time; *exposed_s (if not NULL)
 * receives the communication left after the compute ends.  Host only;
 * negative on bad arguments. */
double ar_overlap_step_time(int nchunks, const double *ready_s, const double *comm_s, double compute_end_s,
                            double update_s, double *exposed_s);

/* Sum of the per-bucket statistics (bytes, steps, launches) of the buckets
 * run one by one (the batched plan's own statistics, launches included,
 * come from ar_plan_stats on ar_bucket_batched_plan). */
ar_stats_t ar_bucket_stats(const ar_bucket_plan_t *bp);
void ar_bucket_plan_destroy(ar_bucket_plan_t *bp);

#ifdef __cplusplus
}
#endif

#endif /* AR_H */
