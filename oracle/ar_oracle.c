/*
 * ar_oracle.c -- plain, slow CPU simulation of gradient all-reduce schedules.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the parity authority for the GPU
 * library.  Only the test suite, the smoke check and the benchmark's CPU
 * baseline may load it; the product path never calls it and shares no code,
 * header, table or helper with it.
 *
 * Sources (cited by short tag throughout):
 *   [PRIMER]  "Collective communication: algorithms, cost and the library that
 *             runs them", chapter 4 of the AI training network primer
 *             (hungchun0201.github.io/ai-training-network-primer).
 *   [SCALING] "Collective communication", chapter 06 of Scaling ML systems
 *             (r007.github.io/AI-Robotics-Rus).
 *   [DCN]     "Chapter 7. Data-center networks" of the AI infrastructure book
 *             (bojieli.github.io/ai-infra-book, Russian and Traditional
 *             Chinese editions).
 *
 * Model.  N virtual ranks each hold a buffer of `count` elements.  Every
 * schedule is a list of steps; a step is a set of messages (src, dst,
 * element range [lo, hi), kind).  A step is simulated literally: first every
 * sender's payload is copied out of the pre-step state into a message
 * buffer, then every message is applied at its receiver -- REDUCE adds the
 * payload to the receiver's copy, COPY overwrites it.
 *
 * Partition (the pages only say "cut into N equal parts"; reading for sizes
 * that do not divide): part(L, K, c) = [floor(c*L/K), floor((c+1)*L/K)).
 *
 * Datatypes.
 *   fp32: each REDUCE is one IEEE-754 binary32 add (round to nearest even,
 *         denormals kept).  Built with -ffp-contract=off, no fast-math.
 *   bf16: inputs are widened exactly to fp32; partial sums travel in fp32;
 *         an element is rounded to bf16 (round to nearest, ties to even) once,
 *         by the receiver of the REDUCE that completes its chunk; COPY
 *         messages carry bf16 bits.  (Reading: the pages do not discuss
 *         reduced precision; fp32 accumulation with one final rounding.)
 *   bf16, rounded each step: every message carries bf16 bits, and every
 *         REDUCE widens both operands, adds in fp32 and rounds the sum to
 *         bf16 at once -- what a wire of bf16 values gives.
 *   INT8 with error feedback (aro_run_int8ef, end of file): fp32 buffers;
 *         every message carries blockwise INT8 codes and fp32 scales, the
 *         schedule runs over 128-element blocks.
 *
 * Parity unpinned: the re-encoding of partial sums at every INT8 hop (how
 * compressed messages are summed is not fixed by the pages); it is pinned
 * only where it is exact, by error bounds, and by a closed form of the same
 * reading.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ARO_FP32 0
#define ARO_BF16 1
#define ARO_BF16_EACH 2

#define ARO_RING 0
#define ARO_HIER 1
#define ARO_RABEN 2
#define ARO_RDOUBLE 3
#define ARO_TREE 4
#define ARO_DTREE 5

#define ARO_REDUCE 0
#define ARO_COPY 1

typedef struct {
  int step;      /* sequential round this message belongs to            */
  int src, dst;  /* sending and receiving virtual rank                  */
  int64_t lo, hi;/* element range, identical on sender and receiver     */
  int kind;      /* ARO_REDUCE or ARO_COPY                              */
  int completes; /* 1 if this REDUCE makes the receiver's range final   */
} aro_msg;

typedef struct {
  aro_msg *m;
  int64_t n, cap;
  int nsteps;
} aro_list;

static int push(aro_list *L, int step, int src, int dst, int64_t lo, int64_t hi,
                int kind, int completes) {
  if (L->n == L->cap) {
    int64_t nc = L->cap ? 2 * L->cap : 256;
    aro_msg *nm = (aro_msg *)realloc(L->m, (size_t)nc * sizeof(aro_msg));
    if (!nm) return -1;
    L->m = nm;
    L->cap = nc;
  }
  aro_msg *x = &L->m[L->n++];
  x->step = step; x->src = src; x->dst = dst; x->lo = lo; x->hi = hi;
  x->kind = kind; x->completes = completes;
  return 0;
}

/* Start of part c when a range of length len is cut into k parts. */
static int64_t part_lo(int64_t len, int64_t k, int64_t c) {
  return (int64_t)(((__int128)c * len) / k);
}

static int mod(int a, int n) { return ((a % n) + n) % n; }

/*
 * Ring all-reduce = ring reduce-scatter then ring all-gather.
 * [PRIMER] section 4.2, the two index rules and Figures 4.1-4.3;
 * [SCALING] "Ring AllReduce" algorithm box.
 *   reduce-scatter step s (s = 0..N-2): rank i sends chunk (i - s) mod N to
 *     rank i+1, which adds its own copy; after N-1 steps rank i holds the
 *     complete chunk (i + 1) mod N.
 *   all-gather step s (s = 0..N-2): rank i sends chunk (i + 1 - s) mod N to
 *     rank i+1, which stores it.
 * `members` maps ring position -> virtual rank; [base, base+len) is the range
 * being reduced, cut into `n` chunks.  `first_step` numbers the rounds.
 * `rs_completes` says whether the last reduce-scatter step finishes the
 * element (false when a later phase still has to add more).
 */
static int build_ring(aro_list *L, const int *members, int n, int64_t base, int64_t len,
                      int first_step, int do_rs, int do_ag, int rs_completes) {
  int step = first_step;
  if (do_rs) {
    for (int s = 0; s <= n - 2; ++s, ++step)
      for (int i = 0; i < n; ++i) {
        int c = mod(i - s, n);
        int64_t lo = base + part_lo(len, n, c), hi = base + part_lo(len, n, c + 1);
        if (push(L, step, members[i], members[(i + 1) % n], lo, hi, ARO_REDUCE,
                 rs_completes && s == n - 2)) return -1;
      }
  }
  if (do_ag) {
    for (int s = 0; s <= n - 2; ++s, ++step)
      for (int i = 0; i < n; ++i) {
        int c = mod(i + 1 - s, n);
        int64_t lo = base + part_lo(len, n, c), hi = base + part_lo(len, n, c + 1);
        if (push(L, step, members[i], members[(i + 1) % n], lo, hi, ARO_COPY, 0)) return -1;
      }
  }
  return step;
}

/*
 * Hierarchical all-reduce, [PRIMER] section 4.4 (three phases, Figure 4.8 and
 * Animation 4.3); [DCN] section 7.2.1 (2 servers x 8 ranks); [SCALING]
 * "Hierarchical AllReduce".  Ranks r = g*G + l: group g, local index l
 * (groups are contiguous blocks of G ranks, as servers are in [DCN] 7.2.1).
 *   phase 1: inside each group, a ring reduce-scatter over G slices in which
 *     local l sends slice (l - 1 - s) mod G to local l+1 at step s; the slice
 *     order is rotated so that local k ends owning slice k (Animation 4.3).
 *   phase 2: for each local index l, the M = N/G ranks {g*G + l} run a flat
 *     ring all-reduce (both halves) on slice l cut into M sub-chunks.
 *     (Reading for M > 2: the pages draw M = 2; section 4.4 calls the phase an
 *     all-reduce among the N/8 ranks holding the same slice, done as a ring.)
 *   phase 3: inside each group, a ring all-gather in which local l sends
 *     slice (l - s) mod G to local l+1 at step s.
 */
static int build_hier(aro_list *L, int N, int G, int64_t count) {
  int M = N / G;
  int step = 0;
  /* phase 1 */
  for (int s = 0; s <= G - 2; ++s, ++step)
    for (int g = 0; g < M; ++g)
      for (int l = 0; l < G; ++l) {
        int k = mod(l - 1 - s, G);
        int64_t lo = part_lo(count, G, k), hi = part_lo(count, G, k + 1);
        if (push(L, step, g * G + l, g * G + (l + 1) % G, lo, hi, ARO_REDUCE,
                 M == 1 && s == G - 2)) return -1;
      }
  /* phase 2: reduce-scatter half for every slice, then all-gather half, so
     that all slices advance in the same rounds. */
  if (M > 1) {
    int *members = (int *)malloc(sizeof(int) * (size_t)M);
    if (!members) return -1;
    int end = step;
    for (int half = 0; half < 2; ++half)
      for (int l = 0; l < G; ++l) {
        for (int m = 0; m < M; ++m) members[m] = m * G + l;
        int64_t base = part_lo(count, G, l), len = part_lo(count, G, l + 1) - base;
        int first = half == 0 ? step : step + (M - 1);
        end = build_ring(L, members, M, base, len, first, half == 0, half == 1, 1);
        if (end < 0) { free(members); return -1; }
      }
    free(members);
    step = end;
  }
  /* phase 3 */
  for (int s = 0; s <= G - 2; ++s, ++step)
    for (int g = 0; g < M; ++g)
      for (int l = 0; l < G; ++l) {
        int k = mod(l - s, G);
        int64_t lo = part_lo(count, G, k), hi = part_lo(count, G, k + 1);
        if (push(L, step, g * G + l, g * G + (l + 1) % G, lo, hi, ARO_COPY, 0)) return -1;
      }
  return step;
}

/*
 * Rabenseifner: recursive-halving reduce-scatter then recursive-doubling
 * all-gather.  [PRIMER] section 4.3 (Figure 4.5, Animation 4.2);
 * [SCALING] "Recursive halving and doubling (butterfly)".
 *   N = 2^L.  Each rank tracks a range [a, b) of chunk indices, initially
 *   [0, N) with chunks = part(count, N, c).
 *   RS round k = 1..L: partner p = i xor 2^(k-1); the range splits at
 *     m = (a + b) / 2; rank i keeps [a, m) if bit k-1 of i is 0, else [m, b);
 *     it sends the other half to p and adds what p sends for the kept half.
 *     (The half choice is fixed by Animation 4.2: rank i ends owning the
 *     chunk whose index is i with its bits reversed; rank 1 owns chunk E,
 *     index 4, when N = 8.)
 *   AG round k = L..1: same partner; each rank sends the whole range it
 *     holds and the partner stores it, so both hold the union.
 */
static int build_raben(aro_list *L, int N, int64_t count) {
  int lg = 0;
  while ((1 << lg) < N) ++lg;
  int *a = (int *)malloc(sizeof(int) * (size_t)N * (size_t)(lg + 1));
  int *b = (int *)malloc(sizeof(int) * (size_t)N * (size_t)(lg + 1));
  if (!a || !b) { free(a); free(b); return -1; }
  /* a[k*N + i], b[k*N + i]: chunk range of rank i after RS round k. */
  for (int i = 0; i < N; ++i) { a[i] = 0; b[i] = N; }
  int step = 0;
  for (int k = 1; k <= lg; ++k, ++step)
    for (int i = 0; i < N; ++i) {
      int p = i ^ (1 << (k - 1));
      int ca = a[(k - 1) * N + i], cb = b[(k - 1) * N + i], cm = (ca + cb) / 2;
      int keep_low = ((i >> (k - 1)) & 1) == 0;
      a[k * N + i] = keep_low ? ca : cm;
      b[k * N + i] = keep_low ? cm : cb;
      /* i sends the half it does not keep; p keeps exactly that half */
      int sa = keep_low ? cm : ca, sb = keep_low ? cb : cm;
      if (push(L, step, i, p, part_lo(count, N, sa), part_lo(count, N, sb), ARO_REDUCE,
               k == lg)) { free(a); free(b); return -1; }
    }
  for (int k = lg; k >= 1; --k, ++step)
    for (int i = 0; i < N; ++i) {
      int p = i ^ (1 << (k - 1));
      int ca = a[k * N + i], cb = b[k * N + i];
      if (push(L, step, i, p, part_lo(count, N, ca), part_lo(count, N, cb), ARO_COPY, 0)) {
        free(a); free(b); return -1;
      }
    }
  free(a); free(b);
  return step;
}

/*
 * Recursive doubling, [PRIMER] section 4.3 ("Trees: latency-optimal,
 * bandwidth-poor", Figure 4.5) and [SCALING] "Tree AllReduce": in step k
 * (k = 0..log2 N - 1) every rank exchanges its whole buffer with rank
 * i xor 2^k and both add; after log2 N steps every rank holds the sum.
 * N must be a power of two.
 */
static int build_rdouble(aro_list *L, int N, int64_t count) {
  int lg = 0;
  while ((1 << lg) < N) ++lg;
  for (int k = 0; k < lg; ++k)
    for (int i = 0; i < N; ++i)
      if (push(L, k, i, i ^ (1 << k), 0, count, ARO_REDUCE, k == lg - 1)) return -1;
  return lg;
}

/*
 * Binary tree all-reduce, [SCALING] "Tree AllReduce": a reduce phase in
 * which values climb to the root in log2 N steps, then a broadcast phase in
 * which the root's result descends in log2 N steps; every message carries
 * the whole buffer ([PRIMER] 4.3, Figure 4.7's table: "up to the root, then
 * back down").  Reading: the binomial tree rooted at rank 0 -- in reduce
 * step k the ranks whose index has bit k set and no lower bit send to
 * i - 2^k, which adds; the broadcast runs the same edges in reverse, parent
 * to child.  Works for any N (ceil(log2 N) steps each way).
 */
static int build_tree(aro_list *L, int N, int64_t count) {
  int lg = 0;
  while ((1 << lg) < N) ++lg;
  int step = 0;
  for (int k = 0; k < lg; ++k, ++step)
    for (int i = 0; i < N; ++i)
      if ((i & ((2 << k) - 1)) == (1 << k))
        if (push(L, step, i, i - (1 << k), 0, count, ARO_REDUCE, k == lg - 1)) return -1;
  for (int k = lg - 1; k >= 0; --k, ++step)
    for (int i = 0; i < N; ++i)
      if ((i & ((2 << k) - 1)) == 0 && i + (1 << k) < N)
        if (push(L, step, i, i + (1 << k), 0, count, ARO_COPY, 0)) return -1;
  return step;
}

/*
 * Double binary tree, [SCALING] "Double binary tree" and [PRIMER] Figure
 * 4.6: two trees, the second the mirror image of the first (node r becomes
 * N-1-r), each reducing and broadcasting half of the buffer at the same
 * time.  Tree 1 (read from Figure 4.6 for N = 8: 0 <- 4 <- {2, 6} <-
 * {1, 3, 5, 7}): rank 0 is the root with the single child N/2; a node r > 0
 * whose lowest set bit is b has children r - b/2 and r + b/2 when b > 1.
 * N must be a power of two.  A node sends up in the round equal to its
 * height (log2 b; the root's child N/2 in round log2 N - 1); the broadcast
 * mirrors the rounds.  Messages are emitted by increasing sender rank, so a
 * node that hears from two children in one round adds the lower-ranked
 * child's part first: ((own + lower child) + higher child).
 */
static int tree1_parent(int r, int N) {
  if (r == N / 2) return 0;
  int b = r & -r;
  return (r & (b << 1)) ? r - b : r + b;
}

static int tree1_height(int r, int N) { /* 0 for leaves; root's child: log2 N - 1 */
  int b = r & -r, h = 0;
  while ((1 << h) < b) ++h;
  (void)N;
  return h;
}

static int build_dtree(aro_list *L, int N, int64_t count) {
  int lg = 0;
  while ((1 << lg) < N) ++lg;
  int64_t half = part_lo(count, 2, 1);
  /* reduce rounds 0..lg-1, broadcast rounds lg..2lg-1 */
  for (int round = 0; round < lg; ++round)
    for (int s = 0; s < N; ++s)
      for (int t = 0; t < 2; ++t) {
        /* in tree 2 the sender s plays the part of node N-1-s of tree 1 */
        int node = t == 0 ? s : N - 1 - s;
        if (node == 0 || tree1_height(node, N) != round) continue;
        int par = tree1_parent(node, N);
        int dst = t == 0 ? par : N - 1 - par;
        int64_t lo = t == 0 ? 0 : half, hi = t == 0 ? half : count;
        if (push(L, round, s, dst, lo, hi, ARO_REDUCE, round == lg - 1)) return -1;
      }
  for (int round = 0; round < lg; ++round)
    for (int s = 0; s < N; ++s)
      for (int t = 0; t < 2; ++t) {
        /* the parent sends down in the mirror of the round its child sent up */
        int node = t == 0 ? s : N - 1 - s;
        for (int c = 1; c < N; ++c) {
          if (tree1_parent(c, N) != node || tree1_height(c, N) != lg - 1 - round) continue;
          int dst = t == 0 ? c : N - 1 - c;
          int64_t lo = t == 0 ? 0 : half, hi = t == 0 ? half : count;
          if (push(L, lg + round, s, dst, lo, hi, ARO_COPY, 0)) return -1;
        }
      }
  return 2 * lg;
}

static int is_pow2(int n) { return n > 0 && (n & (n - 1)) == 0; }

/* Validates arguments and builds the message list.  0 on success. */
static int build(aro_list *L, int N, int G, int64_t count, int schedule) {
  memset(L, 0, sizeof(*L));
  if (N < 1 || count < 0) return -1;
  int end;
  if (schedule == ARO_RING) {
    if (G < 1 || N % G) return -1; /* G only labels groups for the ring */
    int *members = (int *)malloc(sizeof(int) * (size_t)N);
    if (!members) return -1;
    for (int i = 0; i < N; ++i) members[i] = i;
    end = build_ring(L, members, N, 0, count, 0, 1, 1, 1);
    free(members);
  } else if (schedule == ARO_HIER) {
    if (G < 1 || N % G) return -1;
    end = build_hier(L, N, G, count);
  } else if (schedule == ARO_RABEN) {
    if (!is_pow2(N)) return -2;
    if (G < 1 || N % G) return -1;
    end = build_raben(L, N, count);
  } else if (schedule == ARO_RDOUBLE || schedule == ARO_DTREE) {
    if (!is_pow2(N)) return -2;
    if (G < 1 || N % G) return -1;
    end = schedule == ARO_RDOUBLE ? build_rdouble(L, N, count) : build_dtree(L, N, count);
  } else if (schedule == ARO_TREE) {
    if (G < 1 || N % G) return -1;
    end = build_tree(L, N, count);
  } else {
    return -1;
  }
  if (end < 0) { free(L->m); L->m = NULL; return -3; }
  L->nsteps = end;
  /* The hierarchical builder emits phase 2 slice by slice; order all
     messages by round (stable, so each round keeps its emission order). */
  if (L->n > 0) {
    aro_msg *sorted = (aro_msg *)malloc((size_t)L->n * sizeof(aro_msg));
    int64_t *start = (int64_t *)calloc((size_t)end + 1, sizeof(int64_t));
    if (!sorted || !start) { free(sorted); free(start); free(L->m); L->m = NULL; return -3; }
    for (int64_t j = 0; j < L->n; ++j) start[L->m[j].step + 1]++;
    for (int r = 0; r < end; ++r) start[r + 1] += start[r];
    for (int64_t j = 0; j < L->n; ++j) sorted[start[L->m[j].step]++] = L->m[j];
    free(start);
    free(L->m);
    L->m = sorted;
  }
  return 0;
}

/* bf16 helpers, written from the definitions of the formats. */
static float widen_bf16(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

static uint16_t round_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  if ((u & 0x7fffffffu) > 0x7f800000u)        /* NaN: keep sign, force quiet */
    return (uint16_t)((u >> 16) | 0x0040u);
  uint32_t lsb = (u >> 16) & 1u;              /* ties go to the even result */
  return (uint16_t)((u + 0x7fffu + lsb) >> 16);
}

/* ---------------------------------------------------------------------- */
/* Exported C ABI of the oracle.                                          */
/* ---------------------------------------------------------------------- */

/* Number of sequential rounds of a schedule, or a negative error code. */
int aro_steps(int nranks, int group_size, long long count, int schedule) {
  aro_list L;
  int rc = build(&L, nranks, group_size, count, schedule);
  if (rc) return rc;
  free(L.m);
  return L.nsteps;
}

/* Number of messages of a schedule (all steps), or a negative error code. */
long long aro_num_messages(int nranks, int group_size, long long count, int schedule) {
  aro_list L;
  int rc = build(&L, nranks, group_size, count, schedule);
  if (rc) return rc;
  long long n = L.n;
  free(L.m);
  return n;
}

/* Writes the message list (at most cap entries).  Returns the count. */
long long aro_messages(int nranks, int group_size, long long count, int schedule,
                       int *step, int *src, int *dst, long long *lo, long long *hi,
                       int *kind, int *completes, long long cap) {
  aro_list L;
  int rc = build(&L, nranks, group_size, count, schedule);
  if (rc) return rc;
  long long n = L.n < cap ? L.n : cap;
  for (long long j = 0; j < n; ++j) {
    step[j] = L.m[j].step; src[j] = L.m[j].src; dst[j] = L.m[j].dst;
    lo[j] = L.m[j].lo; hi[j] = L.m[j].hi;
    kind[j] = L.m[j].kind; completes[j] = L.m[j].completes;
  }
  free(L.m);
  return L.n;
}

/*
 * Bytes each rank sends (logical payload in the buffer's dtype), and the
 * total over messages whose sender and receiver lie in different groups of
 * group_size contiguous ranks ([DCN] 7.2.1 counts these as cross-server).
 */
int aro_stats(int nranks, int group_size, long long count, int elem_bytes, int schedule,
              unsigned long long *bytes_sent, unsigned long long *cross_group_bytes) {
  aro_list L;
  int rc = build(&L, nranks, group_size, count, schedule);
  if (rc) return rc;
  for (int r = 0; r < nranks; ++r) bytes_sent[r] = 0;
  *cross_group_bytes = 0;
  for (int64_t j = 0; j < L.n; ++j) {
    unsigned long long b = (unsigned long long)(L.m[j].hi - L.m[j].lo) * (unsigned)elem_bytes;
    bytes_sent[L.m[j].src] += b;
    if (L.m[j].src / group_size != L.m[j].dst / group_size) *cross_group_bytes += b;
  }
  free(L.m);
  return L.nsteps;
}

/*
 * Per-round resource model of [DCN] section 7.2.1:
 *   T = sum over rounds r of ( alpha + max over transfers e of V_{r,e} / B_e ),
 * with B_e = bw_intra when sender and receiver share a group and bw_cross
 * otherwise.  Each rank has its own link of each class, so the slowest
 * single message of a round sets the round time.  Seconds; < 0 on error.
 */
double aro_cost(int nranks, int group_size, long long count, int elem_bytes, int schedule,
                double alpha_s, double bw_intra, double bw_cross) {
  aro_list L;
  int rc = build(&L, nranks, group_size, count, schedule);
  if (rc) return (double)rc;
  double *worst = (double *)calloc((size_t)(L.nsteps > 0 ? L.nsteps : 1), sizeof(double));
  if (!worst) { free(L.m); return -3.0; }
  for (int64_t j = 0; j < L.n; ++j) {
    double bytes = (double)(L.m[j].hi - L.m[j].lo) * elem_bytes;
    int cross = L.m[j].src / group_size != L.m[j].dst / group_size;
    double t = bytes / (cross ? bw_cross : bw_intra);
    if (t > worst[L.m[j].step]) worst[L.m[j].step] = t;
  }
  double total = 0.0;
  for (int r = 0; r < L.nsteps; ++r) total += alpha_s + worst[r];
  free(worst);
  free(L.m);
  return total;
}

/*
 * Resource model of [DCN] section 7.6.4 (the hierarchical gradient time
 * T_grad): a round costs alpha_cross if any of its messages crosses between
 * groups, else alpha_intra, plus the largest V/B over the round's resources.
 * Resources are each message's own link (bw_intra or bw_cross) and, when
 * bw_egress > 0, one egress per group carrying all bytes the group sends to
 * other groups in the round, multiplied by `share` (identical collectives
 * running side by side through the same egress).  Seconds; < 0 on error.
 */
double aro_cost_ex(int nranks, int group_size, long long count, int elem_bytes, int schedule,
                   double alpha_intra, double alpha_cross, double bw_intra, double bw_cross,
                   double bw_egress, double share) {
  aro_list L;
  int rc = build(&L, nranks, group_size, count, schedule);
  if (rc) return (double)rc;
  int ngroups = nranks / group_size;
  int nrounds = L.nsteps > 0 ? L.nsteps : 1;
  double *round_t = (double *)calloc((size_t)nrounds, sizeof(double));
  int *round_cross = (int *)calloc((size_t)nrounds, sizeof(int));
  double *out_bytes = (double *)calloc((size_t)nrounds * (size_t)ngroups, sizeof(double));
  if (!round_t || !round_cross || !out_bytes) {
    free(round_t); free(round_cross); free(out_bytes); free(L.m);
    return -3.0;
  }
  for (int64_t j = 0; j < L.n; ++j) {
    const aro_msg *x = &L.m[j];
    double bytes = (double)(x->hi - x->lo) * elem_bytes;
    int gs = x->src / group_size, gd = x->dst / group_size;
    double t = bytes / (gs != gd ? bw_cross : bw_intra);
    if (t > round_t[x->step]) round_t[x->step] = t;
    if (gs != gd) {
      round_cross[x->step] = 1;
      out_bytes[(size_t)x->step * ngroups + gs] += bytes;
    }
  }
  double total = 0.0;
  for (int r = 0; r < L.nsteps; ++r) {
    double t = round_t[r];
    if (bw_egress > 0)
      for (int g = 0; g < ngroups; ++g) {
        double te = out_bytes[(size_t)r * ngroups + g] * share / bw_egress;
        if (te > t) t = te;
      }
    total += (round_cross[r] ? alpha_cross : alpha_intra) + t;
  }
  free(round_t); free(round_cross); free(out_bytes); free(L.m);
  return total;
}

/*
 * Runs rounds first_step .. end_step-1 of the schedule in place on host
 * buffers bufs[0..nranks-1] (float* for fp32, uint16_t* holding bf16 bits
 * for bf16); end_step < 0 runs to the last round.  The rounds before
 * first_step are not simulated: the buffers stand for the state they left.
 * [PRIMER] 4.2 and [SCALING] "Six basic primitives": the reduce rounds of
 * the ring, hierarchical and Rabenseifner schedules are a reduce-scatter
 * and the copy rounds after them an all-gather, so the two halves run as
 * (0, k) and (k, -1) with k the number of reduce rounds.  Returns 0, or a
 * negative code.
 */
int aro_run_rounds(int nranks, int group_size, long long count, int dtype, int schedule,
                   void **bufs, int first_step, int end_step) {
  if (dtype != ARO_FP32 && dtype != ARO_BF16 && dtype != ARO_BF16_EACH) return -1;
  if (first_step < 0) return -1;
  aro_list L;
  int rc = build(&L, nranks, group_size, count, schedule);
  if (rc) return rc;
  int nsteps = (end_step >= 0 && end_step < L.nsteps) ? end_step : L.nsteps;

  /* Working fp32 state of every rank: the buffers themselves for fp32, a
     widened copy for bf16. */
  float **w = (float **)calloc((size_t)nranks, sizeof(float *));
  if (!w) { free(L.m); return -3; }
  int err = 0;
  for (int r = 0; r < nranks && !err; ++r) {
    if (dtype == ARO_FP32) {
      w[r] = (float *)bufs[r];
    } else if (dtype == ARO_BF16_EACH) {
      w[r] = NULL; /* no fp32 state: the buffers are the state */
    } else {
      w[r] = (float *)malloc(sizeof(float) * (size_t)(count > 0 ? count : 1));
      if (!w[r]) { err = 1; break; }
      const uint16_t *h = (const uint16_t *)bufs[r];
      for (int64_t e = 0; e < count; ++e) w[r][e] = widen_bf16(h[e]);
    }
  }

  /* Message payload store, sized once for the largest step. */
  int64_t biggest = 1;
  for (int64_t j = 0, step_total = 0; j < L.n; ++j) {
    step_total = (j > 0 && L.m[j].step == L.m[j - 1].step ? step_total : 0) + (L.m[j].hi - L.m[j].lo);
    if (step_total > biggest) biggest = step_total;
  }
  float *pay = NULL;
  uint16_t *pay16 = NULL;
  if (!err) {
    pay = (float *)malloc(sizeof(float) * (size_t)biggest);
    pay16 = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)biggest);
    if (!pay || !pay16) err = 1;
  }
  int64_t j0 = 0;
  while (j0 < L.n && L.m[j0].step < first_step) ++j0;
  while (!err && j0 < L.n && L.m[j0].step < nsteps) {
    int64_t j1 = j0;
    while (j1 < L.n && L.m[j1].step == L.m[j0].step) ++j1;
    /* 1) every sender copies its payload out of the pre-step state */
    int64_t off = 0;
    for (int64_t j = j0; j < j1; ++j) {
      const aro_msg *x = &L.m[j];
      for (int64_t e = x->lo; e < x->hi; ++e, ++off) {
        if (dtype == ARO_BF16_EACH || (dtype == ARO_BF16 && x->kind == ARO_COPY))
          pay16[off] = ((const uint16_t *)bufs[x->src])[e];
        else
          pay[off] = w[x->src][e];
      }
    }
    /* 2) every receiver applies what arrived */
    off = 0;
    for (int64_t j = j0; j < j1; ++j) {
      const aro_msg *x = &L.m[j];
      for (int64_t e = x->lo; e < x->hi; ++e, ++off) {
        if (dtype == ARO_BF16_EACH) {
          uint16_t *d = (uint16_t *)bufs[x->dst];
          if (x->kind == ARO_REDUCE) {
            float wide = widen_bf16(pay16[off]) + widen_bf16(d[e]);
            d[e] = round_bf16(wide);
          } else {
            d[e] = pay16[off];
          }
        } else if (x->kind == ARO_REDUCE) {
          float sum = pay[off] + w[x->dst][e];
          w[x->dst][e] = sum;
          if (dtype == ARO_BF16 && x->completes)
            ((uint16_t *)bufs[x->dst])[e] = round_bf16(sum);
        } else if (dtype == ARO_BF16) {
          ((uint16_t *)bufs[x->dst])[e] = pay16[off];
        } else {
          w[x->dst][e] = pay[off];
        }
      }
    }
    j0 = j1;
  }
  free(pay); free(pay16);
  if (dtype != ARO_FP32)
    for (int r = 0; r < nranks; ++r) free(w[r]);
  free(w);
  free(L.m);
  return err ? -3 : 0;
}

/* The whole schedule, or its first max_steps rounds when max_steps >= 0
   (used to inspect intermediate states). */
int aro_run(int nranks, int group_size, long long count, int dtype, int schedule,
            void **bufs, int max_steps) {
  return aro_run_rounds(nranks, group_size, count, dtype, schedule, bufs, 0, max_steps);
}


/* ---------------------------------------------------------------------- */
/* Compressed all-reduce: blockwise INT8 with error feedback.             */
/* ---------------------------------------------------------------------- */
/*
 * [SCALING] "Gradient compression": INT8 quantization with a scale
 * s = max|g| / 127, q = round(g / s), decoded as q * s; "Blockwise
 * quantization": one fp32 scale per block of b elements (message
 * d + 4d/b bytes); "Error feedback": every worker keeps e_t and sends
 * v_t = C(g_t + e_t), then e_{t+1} = g_t + e_t - v_t.
 *
 * Readings (the pages leave them open): b = 128; round = to nearest, ties
 * to even; a block of zeros has scale 0 and codes 0.  Every message of the
 * schedule carries codes and scales: a REDUCE receiver decodes the message
 * and its own codes, adds in fp32 and re-encodes the sum; a COPY forwards
 * codes.  The schedule is built over blocks (chunk boundaries fall between
 * blocks).  At the end every rank decodes its codes into its buffer.
 */
#define ARO_QB 128

static void q_encode(const float *x, int n, int8_t *q, float *scale) {
  float m = 0.0f;
  for (int i = 0; i < n; ++i) {
    float a = fabsf(x[i]);
    if (a > m) m = a;
  }
  float s = m / 127.0f;
  *scale = s;
  for (int i = 0; i < n; ++i) {
    if (s == 0.0f) {
      q[i] = 0;
      continue;
    }
    float r = rintf(x[i] / s);
    if (r > 127.0f) r = 127.0f;
    if (r < -127.0f) r = -127.0f;
    q[i] = (int8_t)r;
  }
}

static float q_decode(int8_t q, float s) { return (float)q * s; }

/*
 * bufs[r]: fp32 gradient of rank r (count elements), replaced by the
 * decoded result; errs[r]: its fp32 error accumulator, updated in place
 * (errs == NULL: no error feedback, e = 0).  Returns 0 or a negative code.
 */
int aro_run_int8ef(int nranks, int group_size, long long count, int schedule, float **bufs, float **errs,
                   int max_steps) {
  int64_t nblk = (count + ARO_QB - 1) / ARO_QB;
  aro_list L;
  int rc = build(&L, nranks, group_size, nblk, schedule);
  if (rc) return rc;
  int nsteps = (max_steps >= 0 && max_steps < L.nsteps) ? max_steps : L.nsteps;
  int8_t **q = (int8_t **)calloc((size_t)nranks, sizeof(int8_t *));
  float **sc = (float **)calloc((size_t)nranks, sizeof(float *));
  float *x = (float *)malloc(sizeof(float) * ARO_QB);
  int err = !q || !sc || !x;
  for (int r = 0; r < nranks && !err; ++r) {
    q[r] = (int8_t *)malloc((size_t)(count > 0 ? count : 1));
    sc[r] = (float *)malloc(sizeof(float) * (size_t)(nblk > 0 ? nblk : 1));
    if (!q[r] || !sc[r]) err = 1;
  }
  /* each rank compresses g + e and keeps the residual */
  for (int r = 0; r < nranks && !err; ++r)
    for (int64_t b = 0; b < nblk; ++b) {
      int64_t lo = b * ARO_QB;
      int n = (int)((count - lo) < ARO_QB ? (count - lo) : ARO_QB);
      for (int i = 0; i < n; ++i) x[i] = bufs[r][lo + i] + (errs ? errs[r][lo + i] : 0.0f);
      q_encode(x, n, q[r] + lo, &sc[r][b]);
      if (errs)
        for (int i = 0; i < n; ++i) errs[r][lo + i] = x[i] - q_decode(q[r][lo + i], sc[r][b]);
    }
  /* the schedule over blocks; payload copies first, then the receivers */
  int8_t *pq = NULL;
  float *ps = NULL;
  if (!err) {
    pq = (int8_t *)malloc((size_t)(nranks > 0 ? nranks : 1) * (size_t)(count > 0 ? count : 1));
    ps = (float *)malloc(sizeof(float) * (size_t)(nranks > 0 ? nranks : 1) * (size_t)(nblk > 0 ? nblk : 1));
    if (!pq || !ps) err = 1;
  }
  int64_t j0 = 0;
  while (!err && j0 < L.n && L.m[j0].step < nsteps) {
    int64_t j1 = j0;
    while (j1 < L.n && L.m[j1].step == L.m[j0].step) ++j1;
    int64_t eoff = 0, boff = 0;
    for (int64_t j = j0; j < j1; ++j) {
      const aro_msg *m = &L.m[j];
      int64_t elo = m->lo * ARO_QB, ehi = m->hi * ARO_QB < count ? m->hi * ARO_QB : count;
      memcpy(pq + eoff, q[m->src] + elo, (size_t)(ehi > elo ? ehi - elo : 0));
      memcpy(ps + boff, sc[m->src] + m->lo, sizeof(float) * (size_t)(m->hi - m->lo));
      eoff += ehi > elo ? ehi - elo : 0;
      boff += m->hi - m->lo;
    }
    eoff = 0;
    boff = 0;
    for (int64_t j = j0; j < j1; ++j) {
      const aro_msg *m = &L.m[j];
      for (int64_t b = m->lo; b < m->hi; ++b, ++boff) {
        int64_t lo = b * ARO_QB;
        int n = (int)((count - lo) < ARO_QB ? (count - lo) : ARO_QB);
        if (m->kind == ARO_REDUCE) {
          for (int i = 0; i < n; ++i)
            x[i] = q_decode(pq[eoff + i], ps[boff]) + q_decode(q[m->dst][lo + i], sc[m->dst][b]);
          q_encode(x, n, q[m->dst] + lo, &sc[m->dst][b]);
        } else {
          memcpy(q[m->dst] + lo, pq + eoff, (size_t)n);
          sc[m->dst][b] = ps[boff];
        }
        eoff += n;
      }
    }
    j0 = j1;
  }
  /* every rank decodes what it holds */
  for (int r = 0; r < nranks && !err; ++r)
    for (int64_t b = 0; b < nblk; ++b)
      for (int64_t e = b * ARO_QB; e < count && e < (b + 1) * ARO_QB; ++e) bufs[r][e] = q_decode(q[r][e], sc[r][b]);
  free(pq);
  free(ps);
  for (int r = 0; r < nranks; ++r) {
    if (q) free(q[r]);
    if (sc) free(sc[r]);
  }
  free(q);
  free(sc);
  free(x);
  free(L.m);
  return err ? -3 : 0;
}
