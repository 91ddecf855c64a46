// plan.cpp -- schedule builders, lowering to kernel launches, statistics.
//
// Sources, cited by short tag:
//   [PRIMER]  "Collective communication: algorithms, cost and the library that
//             runs them", AI training network primer, chapter 4.
//   [SCALING] "Collective communication", Scaling ML systems, chapter 06.
//   [DCN]     "Chapter 7. Data-center networks", AI infrastructure book.
#include "plan.hpp"

#include <algorithm>
#include <cstdio>
#include <map>
#include <tuple>

namespace ar {

namespace {
// Elements per fp32 scratch slot: the slot's extent rounded up to 64, so
// every slot starts 256-byte aligned.  (Padding the stride away from powers
// of two, by 256 B to 16 KiB, was measured and changed nothing.)
int64_t slot_stride_for(int64_t elems) { return (elems + 63) / 64 * 64; }
}  // namespace

int64_t elem_bytes(Dtype d) { return d == kF32 ? 4 : d == kI8EF ? 1 : 2; }

int64_t buffer_elem_bytes(Dtype d) { return (d == kF32 || d == kI8EF) ? 4 : 2; }

int64_t unit_elems(const Plan &p, int64_t lo, int64_t hi) {
  if (p.dtype != kI8EF) return hi - lo;
  const int64_t e0 = lo * kQBlock, e1 = std::min(hi * kQBlock, p.count);
  return e1 > e0 ? e1 - e0 : 0;
}

uint64_t xfer_bytes(const Plan &p, const Transfer &x) {
  const uint64_t e = static_cast<uint64_t>(unit_elems(p, x.lo, x.hi)) * static_cast<uint64_t>(elem_bytes(p.dtype));
  return p.dtype == kI8EF ? e + 4 * static_cast<uint64_t>(x.hi - x.lo) : e;
}

uint64_t workspace_bytes(const Plan &p) {
  if (p.dtype == kI8EF && p.exec == kOnePass) return 0;  // codes stay in registers
  if (p.dtype == kI8EF)
    return static_cast<uint64_t>(p.nranks) *
           (static_cast<uint64_t>(p.code_stride) + 4 * static_cast<uint64_t>(p.scale_stride));
  return static_cast<uint64_t>(p.nslots) * static_cast<uint64_t>(p.slot_stride) * 4;
}

namespace {

// Part c of a range [base, base+len) cut into k parts: the floor-balanced
// contiguous split (the pages cut the buffer "into N equal parts"; sizes that
// do not divide are split at floor(c*len/k)).
struct Cut {
  int64_t base, len, k;
  int64_t lo(int64_t c) const { return base + static_cast<int64_t>((static_cast<__int128>(c) * len) / k); }
  int64_t hi(int64_t c) const { return lo(c + 1); }
};

inline int wrap(int v, int n) { return ((v % n) + n) % n; }

// Ring over `ring` (ring position -> rank), data range cut into ring.size()
// chunks.  [PRIMER] 4.2: reduce-scatter step s sends chunk (i - s) mod n from
// position i to i+1, which adds; all-gather step s sends chunk (i + 1 - s)
// mod n and the receiver stores it.  `shift` rotates chunk numbering
// (chunk index = rule index + shift), used by the hierarchical phases.
struct RingPhase {
  std::vector<int> ring;
  Cut cut;
  int shift;
};

void emit_ring_rs(std::vector<Transfer> &out, const RingPhase &r, int step0, bool completes_last) {
  const int n = static_cast<int>(r.ring.size());
  for (int s = 0; s + 1 < n; ++s)
    for (int i = 0; i < n; ++i) {
      const int c = wrap(i - s + r.shift, n);
      out.push_back({step0 + s, r.ring[i], r.ring[(i + 1) % n], r.cut.lo(c), r.cut.hi(c), kReduce,
                     completes_last && s == n - 2});
    }
}

void emit_ring_ag(std::vector<Transfer> &out, const RingPhase &r, int step0) {
  const int n = static_cast<int>(r.ring.size());
  for (int s = 0; s + 1 < n; ++s)
    for (int i = 0; i < n; ++i) {
      const int c = wrap(i + 1 - s + r.shift, n);
      out.push_back({step0 + s, r.ring[i], r.ring[(i + 1) % n], r.cut.lo(c), r.cut.hi(c), kCopy, false});
    }
}

int build_ring(std::vector<Transfer> &out, int n, int64_t count) {
  RingPhase r{{}, Cut{0, count, n}, 0};
  for (int i = 0; i < n; ++i) r.ring.push_back(i);
  emit_ring_rs(out, r, 0, true);
  emit_ring_ag(out, r, n - 1);
  return 2 * (n - 1);
}

// [PRIMER] 4.4 / Animation 4.3, [DCN] 7.2.1.  Group g = ranks g*G .. g*G+G-1.
// Phase 1 is the group ring with chunk numbering shifted by -1 (local l sends
// slice (l - 1 - s) mod G), so local k ends owning slice k.  Phase 2 runs a
// flat ring all-reduce of slice l over the M ranks {m*G + l}.  Phase 3 is the
// group all-gather in which local l first sends slice l.
int build_hier(std::vector<Transfer> &out, int n, int g_size, int64_t count) {
  const int groups = n / g_size;
  const Cut slices{0, count, g_size};
  int step = 0;
  for (int g = 0; g < groups; ++g) {
    RingPhase r{{}, slices, -1};
    for (int l = 0; l < g_size; ++l) r.ring.push_back(g * g_size + l);
    emit_ring_rs(out, r, step, groups == 1);
  }
  step += g_size - 1;
  for (int l = 0; l < g_size; ++l) {
    RingPhase r{{}, Cut{slices.lo(l), slices.hi(l) - slices.lo(l), groups}, 0};
    for (int m = 0; m < groups; ++m) r.ring.push_back(m * g_size + l);
    emit_ring_rs(out, r, step, true);
    emit_ring_ag(out, r, step + groups - 1);
  }
  step += 2 * (groups - 1);
  for (int g = 0; g < groups; ++g) {
    // all-gather rule (i + 1 - s) shifted by -1 gives slice (l - s) mod G
    RingPhase r{{}, slices, -1};
    for (int l = 0; l < g_size; ++l) r.ring.push_back(g * g_size + l);
    emit_ring_ag(out, r, step);
  }
  step += g_size - 1;
  return step;
}

// [PRIMER] 4.3 (Figure 4.5, Animation 4.2), [SCALING] "Recursive halving and
// doubling".  N = 2^L.  Reduce-scatter round k = 1..L pairs i with
// i ^ 2^(k-1); the held chunk range halves, the lower half kept when bit k-1
// of i is 0 (so rank i ends owning chunk bitrev(i)).  The all-gather runs the
// rounds in reverse; each rank sends all it holds and the partner stores it.
int build_raben(std::vector<Transfer> &out, int n, int64_t count) {
  int levels = 0;
  while ((1 << levels) < n) ++levels;
  const Cut chunks{0, count, n};
  // held[k][i] = chunk range [first, last) of rank i after reduce-scatter round k
  std::vector<std::vector<std::pair<int, int>>> held(levels + 1, std::vector<std::pair<int, int>>(n));
  for (int i = 0; i < n; ++i) held[0][i] = {0, n};
  for (int k = 1; k <= levels; ++k) {
    const int bit = 1 << (k - 1);
    for (int i = 0; i < n; ++i) {
      const auto [first, last] = held[k - 1][i];
      const int mid = (first + last) / 2;
      held[k][i] = (i & bit) ? std::make_pair(mid, last) : std::make_pair(first, mid);
    }
    for (int i = 0; i < n; ++i) {
      const int partner = i ^ bit;
      const auto [f, l] = held[k][partner];  // i sends what its partner keeps
      out.push_back({k - 1, i, partner, chunks.lo(f), chunks.lo(l), kReduce, k == levels});
    }
  }
  for (int k = levels; k >= 1; --k) {
    const int step = levels + (levels - k);
    for (int i = 0; i < n; ++i) {
      const auto [f, l] = held[k][i];
      out.push_back({step, i, i ^ (1 << (k - 1)), chunks.lo(f), chunks.lo(l), kCopy, false});
    }
  }
  return 2 * levels;
}

// Recursive doubling ([PRIMER] 4.3, Figure 4.5): in step k every rank and its
// partner i ^ 2^k exchange whole buffers and both add.  N = 2^L.
int build_rdouble(std::vector<Transfer> &out, int n, int64_t count) {
  int levels = 0;
  while ((1 << levels) < n) ++levels;
  for (int k = 0; k < levels; ++k)
    for (int i = 0; i < n; ++i) out.push_back({k, i, i ^ (1 << k), 0, count, kReduce, k + 1 == levels});
  return levels;
}

// Binary tree ([SCALING] "Tree AllReduce"): whole-buffer reduce up a
// binomial tree rooted at rank 0 (in step k, rank r = m * 2^(k+1) receives
// from r + 2^k), then the broadcast down the same edges in reverse.
int build_tree(std::vector<Transfer> &out, int n, int64_t count) {
  int levels = 0;
  while ((1 << levels) < n) ++levels;
  int step = 0;
  for (int k = 0; k < levels; ++k, ++step)
    for (int r = 0; r + (1 << k) < n; r += 2 << k)
      out.push_back({step, r + (1 << k), r, 0, count, kReduce, k + 1 == levels});
  for (int k = levels - 1; k >= 0; --k, ++step)
    for (int r = 0; r + (1 << k) < n; r += 2 << k) out.push_back({step, r, r + (1 << k), 0, count, kCopy, false});
  return step;
}

// Double binary tree ([SCALING] "Double binary tree", [PRIMER] Figure 4.6):
// tree 1 roots at rank 0, whose only child is N/2; the subtree of a node c
// spanning 2b - 1 ranks has the children c - b/2 and c + b/2.  Tree 2 is its
// mirror (rank r plays node N-1-r).  Tree 1 reduces and broadcasts the first
// half of the buffer, tree 2 the second, in the same rounds: a node sends up
// in the round equal to its height and hears from its parent in the mirror
// round.  Children are listed lower rank first, so a node with two children
// adds ((own + lower) + higher).  N = 2^L.
int build_dtree(std::vector<Transfer> &out, int n, int64_t count) {
  int levels = 0;
  while ((1 << levels) < n) ++levels;
  if (n < 2) return 0;
  std::vector<int> parent(n, -1), height(n, 0);
  // walk tree 1 from the root's child down; height of a span-(2b-1) node = log2 b
  std::vector<std::pair<int, int>> stack{{n / 2, n / 2}};
  parent[n / 2] = 0;
  while (!stack.empty()) {
    const auto [c, b] = stack.back();
    stack.pop_back();
    int h = 0;
    while ((1 << h) < b) ++h;
    height[c] = h;
    if (b > 1)
      for (int child : {c - b / 2, c + b / 2}) {
        parent[child] = c;
        stack.push_back({child, b / 2});
      }
  }
  const Cut halves{0, count, 2};
  for (int round = 0; round < levels; ++round)
    for (int tree = 0; tree < 2; ++tree)
      for (int c = 1; c < n; ++c)  // tree-1 node ids, ascending
        if (height[c] == round) {
          const int src = tree == 0 ? c : n - 1 - c, dst = tree == 0 ? parent[c] : n - 1 - parent[c];
          out.push_back({round, src, dst, halves.lo(tree), halves.hi(tree), kReduce, round + 1 == levels});
        }
  // children of a tree-2 node come in descending tree-1 id order; reorder the
  // round's tree-2 reduces so each receiver hears its lower-ranked child first
  for (auto it = out.begin(); it != out.end();) {
    auto end = it;
    while (end != out.end() && end->step == it->step) ++end;
    std::stable_sort(it, end, [](const Transfer &a, const Transfer &b) {
      return a.lo != b.lo ? a.lo < b.lo : a.src < b.src;
    });
    it = end;
  }
  for (int round = 0; round < levels; ++round)
    for (int tree = 0; tree < 2; ++tree)
      for (int c = 1; c < n; ++c)
        if (height[c] == levels - 1 - round) {
          const int dst = tree == 0 ? c : n - 1 - c, src = tree == 0 ? parent[c] : n - 1 - parent[c];
          out.push_back({levels + round, src, dst, halves.lo(tree), halves.hi(tree), kCopy, false});
        }
  return 2 * levels;
}

// Scratch slot holding rank r's fp32 partial sums.  Two ranks share a slot
// only when their partial ranges can never overlap while both are live:
//   ring: one live partial per chunk (it travels round the ring) -> 1 slot;
//   hierarchical: per group, partials of distinct slices           -> M slots;
//   Rabenseifner: ranks 2m and 2m+1 keep disjoint halves from the first halving round on
//                 and later ranges nest inside those halves         -> N/2 slots;
//   recursive doubling and the trees: one slot per rank              -> N slots.
int slot_of(const Plan &p, int r) {
  switch (p.sched) {
    case kRing: return 0;
    case kHier: return (p.group_size == 1 || p.group_size == p.nranks) ? 0 : r / p.group_size;
    case kRaben: return r >> 1;
    default: return r;  // doubling and trees: every rank's partial covers a whole buffer or half
  }
}

// Per-rank record of the element ranges whose current value is an fp32
// partial sum in scratch (bf16 lowering).
struct PartialMap {
  std::vector<std::vector<std::pair<int64_t, int64_t>>> ranges;
  explicit PartialMap(int n) : ranges(n) {}
  // 1: [lo,hi) entirely partial, 0: entirely original input, -1: mixed.
  int state(int r, int64_t lo, int64_t hi) const {
    int64_t covered = 0;
    for (const auto &x : ranges[r]) covered += std::max<int64_t>(0, std::min(hi, x.second) - std::max(lo, x.first));
    if (covered == 0) return 0;
    return covered == hi - lo ? 1 : -1;
  }
  void mark(int r, int64_t lo, int64_t hi) {
    if (state(r, lo, hi) == 0) ranges[r].push_back({lo, hi});
  }
};

// Launch order.  Rounds run in order, and every round of a schedule writes
// what the next one reads.  When a round writes more than the device cache
// holds, that output would stream from DRAM again, so the planner reorders
// (the bits are the same in any of these orders, since each element's fold
// depends only on its own chunk's rounds):
//  * hierarchical: the group phases (1: reduce-scatter, 3: all-gather) are
//    independent across groups and run group by group (every round of group
//    0, then of group 1, ...);
//  * and, when a launch still writes more than the cache, the element range
//    is cut into K pieces at the same offsets on every rank and the rounds
//    concerned run on piece 0, then piece 1, ... (each transfer restricted
//    to the piece), block by block (launch_blocks), the other rounds whole.
struct LaunchKey {
  int32_t phase, group, step;
  bool operator<(const LaunchKey &o) const {
    return phase != o.phase ? phase < o.phase : group != o.group ? group < o.group : step < o.step;
  }
  bool operator==(const LaunchKey &o) const { return phase == o.phase && group == o.group && step == o.step; }
};

// Bytes a round stores per element it writes: fp32 (or fp32 partials of
// kBF16), bf16, or INT8 codes.
int64_t round_write_bytes(const Plan &p) { return p.dtype == kBF16Each ? 2 : p.dtype == kI8EF ? 1 : 4; }

// The same for one transfer: kBF16 reduces store fp32 partials, its copies
// bf16 values.
int64_t transfer_write_bytes(const Plan &p, const Transfer &x) {
  return p.dtype == kBF16 && x.kind != kReduce ? 2 : round_write_bytes(p);
}

bool split_groups(const Plan &p) {
  const int G = p.group_size, M = p.nranks / p.group_size;
  if (p.sched != kHier || G < 2 || M < 2) return false;
  const int64_t slice = unit_elems(p, 0, p.units) / G;  // a phase-1 round: N receivers x one slice
  return static_cast<int64_t>(p.nranks) * slice * round_write_bytes(p) > p.cache_bytes;
}

// The launch a transfer belongs to before any piece cut: its round, and for
// a split hierarchical schedule also its phase and, in phases 1 and 3, its
// group.
LaunchKey group_key(const Plan &p, const Transfer &x, bool split) {
  LaunchKey k{0, 0, x.step};
  if (split) {
    const int G = p.group_size, M = p.nranks / p.group_size;
    const int p2 = G - 1, p3 = G - 1 + 2 * (M - 1);  // first rounds of phases 2 and 3
    k.phase = x.step < p2 ? 0 : x.step < p3 ? 1 : 2;
    if (k.phase != 1) k.group = x.src / G;
  }
  return k;
}

// Pieces a launch round needs so that what it writes fits the cache.
int round_pieces(const Plan &p, int64_t bytes) {
  const int64_t k = p.cache_bytes > 0 ? (bytes + p.cache_bytes - 1) / p.cache_bytes : 64;
  return static_cast<int>(std::min<int64_t>(std::max<int64_t>(k, 1), 64));
}

// Launch rounds (the group keys, in order) in blocks that run piece by
// piece.  A round whose output does not fit the cache shares its block with
// the next round of its chain (same phase and group), which reads that
// output, and the last reduce round with the copy round fused into it; a
// block takes the largest piece count its rounds' outputs need.  A round
// whose output the next round does not read (the last of a chain) needs no
// pieces for it.  A schedule whose rounds shrink and grow, like
// Rabenseifner's, so splits only its wide rounds; the ring, whose rounds are
// all alike, runs piece by piece throughout or not at all.  Maps each launch
// round to its block's piece count and first phase.
std::map<LaunchKey, std::pair<int, int>> launch_blocks(const Plan &p, bool split) {
  std::map<LaunchKey, int64_t> bytes;  // what each launch round writes
  std::map<LaunchKey, bool> reduces;
  for (const Transfer &x : p.xfers) {
    const LaunchKey k = group_key(p, x, split);
    bytes[k] += unit_elems(p, x.lo, x.hi) * transfer_write_bytes(p, x);
    if (x.kind == kReduce) reduces[k] = true;
  }
  std::vector<LaunchKey> order;
  for (const auto &e : bytes) order.push_back(e.first);
  const size_t n = order.size();
  std::vector<int> own(n, 1);
  std::vector<bool> link(n, false);  // round i shares its block with round i + 1
  for (size_t i = 0; i + 1 < n; ++i) {
    if (order[i].phase != order[i + 1].phase || order[i].group != order[i + 1].group) continue;
    own[i] = round_pieces(p, bytes[order[i]]);
    link[i] = own[i] > 1 || (reduces[order[i]] && !reduces[order[i + 1]]);
  }
  std::map<LaunchKey, std::pair<int, int>> out;
  int phase = 0;
  for (size_t i = 0; i < n;) {
    size_t i1 = i;
    int k = own[i];
    while (link[i1]) k = std::max(k, own[++i1]);
    for (size_t q = i; q <= i1; ++q) out[order[q]] = {k, phase};
    phase += k;
    i = i1 + 1;
  }
  return out;
}

std::vector<Transfer> launch_order(const Plan &p, std::vector<LaunchKey> &keys) {
  std::vector<std::pair<LaunchKey, Transfer>> idx;
  const bool split = split_groups(p);
  const std::map<LaunchKey, std::pair<int, int>> blocks = launch_blocks(p, split);
  for (const Transfer &x : p.xfers) {
    const std::pair<int, int> &b = blocks.at(group_key(p, x, split));
    const int k = b.first;
    if (k == 1) {
      idx.push_back({LaunchKey{b.second, 0, x.step}, x});
      continue;
    }
    // piece boundaries on multiples of 64 units: 256-byte aligned for every
    // operand dtype.  A boundary may still fall inside a kernel tile (1024 to
    // 4096 elements); that tile's units inside the piece still move as
    // vectors, so a cut costs one partial tile per op.
    for (int q = 0; q < k; ++q) {
      Transfer y = x;
      y.lo = std::max(x.lo, (p.units * q / k) / 64 * 64);
      y.hi = std::min(x.hi, q + 1 == k ? p.units : (p.units * (q + 1) / k) / 64 * 64);
      if (y.hi > y.lo) idx.push_back({LaunchKey{b.second + q, 0, x.step}, y});
    }
  }
  std::stable_sort(idx.begin(), idx.end(),
                   [](const std::pair<LaunchKey, Transfer> &a, const std::pair<LaunchKey, Transfer> &b) {
                     return a.first < b.first;
                   });
  std::vector<Transfer> out;
  keys.clear();
  for (const auto &e : idx) {
    out.push_back(e.second);
    keys.push_back(e.first);
  }
  return out;
}

std::string lower_steps(Plan &p, bool fuse) {
  p.launches.clear();
  const bool bf = p.dtype == kBF16;  // fp32 partials in scratch
  const bool q = p.dtype == kI8EF;   // INT8 code slots in the workspace
  const int32_t copy_fam = q ? kKQCopy : kKCopy;
  PartialMap partial(p.nranks);
  std::vector<bool> finals;  // per launch: all its reduces complete their range
  int max_slot = -1;
  std::vector<LaunchKey> keys;
  const std::vector<Transfer> xs = launch_order(p, keys);
  size_t j = 0;
  while (j < xs.size()) {
    size_t j1 = j;
    while (j1 < xs.size() && keys[j1] == keys[j]) ++j1;
    // Reduces that exchange the same range in both directions (recursive
    // doubling) become one op writing the sum to both ranks (a + b == b + a
    // bit for bit); the k-th reduce into the same receiver range runs in the
    // round's k-th sub-launch, so a node hearing from two children adds them
    // in order.  Every sub-launch reads only what earlier rounds wrote, or its
    // own receiver's accumulating sum.
    std::vector<size_t> items;
    for (size_t t = j; t < j1; ++t)
      if (xs[t].hi > xs[t].lo) items.push_back(t);
    std::vector<long> partner(items.size(), -1);
    for (size_t u = 0; u < items.size(); ++u) {
      const Transfer &x = xs[items[u]];
      if (x.kind != kReduce || partner[u] >= 0) continue;
      for (size_t v = u + 1; v < items.size(); ++v) {
        const Transfer &y = xs[items[v]];
        if (y.kind == kReduce && partner[v] < 0 && y.src == x.dst && y.dst == x.src && y.lo == x.lo && y.hi == x.hi) {
          partner[u] = static_cast<long>(v);
          partner[v] = static_cast<long>(u);
          break;
        }
      }
    }
    std::map<std::tuple<int, int64_t, int64_t>, int> heard;  // (receiver, range) -> reduces so far
    std::vector<int> sub(items.size(), 0);
    int nsub = 1;
    for (size_t u = 0; u < items.size(); ++u) {
      const Transfer &x = xs[items[u]];
      if (x.kind != kReduce || (partner[u] >= 0 && partner[u] < static_cast<long>(u))) continue;
      int &cnt = heard[{x.dst, x.lo, x.hi}];
      sub[u] = cnt++;
      if (partner[u] >= 0) heard[{x.src, x.lo, x.hi}]++;
      nsub = std::max(nsub, sub[u] + 1);
    }
    for (int sr = 0; sr < nsub; ++sr) {
      // split by (kind, operand types, completion) so each launch is uniform;
      // key bit 16 marks reduces that complete their range
      std::map<int32_t, Launch> by_kind;
      std::vector<std::pair<int, std::pair<int64_t, int64_t>>> to_mark;
      for (size_t u = 0; u < items.size(); ++u) {
        if (sub[u] != sr || (partner[u] >= 0 && partner[u] < static_cast<long>(u))) continue;
        const Transfer &x = xs[items[u]];
        const bool pair = partner[u] >= 0;
        Op op{x.lo, x.hi, kLocNone, kLocNone, kLocNone, kLocNone, 0};
        int32_t kind;
        if (x.kind == kCopy) {
          kind = q ? kKQCopy : kKCopy | static_cast<int32_t>(elem_bytes(p.dtype));
          op.a = x.src;
          op.o = x.dst;
        } else if (q) {
          // blockwise INT8: each rank's code slot holds its running sum
          kind = kKQReduce;
          op.a = x.src;
          op.b = x.dst;
          op.o = x.dst;
          if (pair) {
            op.o2 = x.src;
            kind |= kFlagO2;
          }
        } else if (!bf) {
          // fp32, or bf16 rounded at every add: the rank buffers hold the
          // partial sums themselves
          kind = kKReduce | (p.dtype == kBF16Each ? (kFlagABf | kFlagBBf | kFlagOBf) : 0);
          op.a = x.src;
          op.b = x.dst;
          op.o = x.dst;
          if (pair) {
            op.o2 = x.src;
            kind |= kFlagO2;
          }
        } else {
          const int sa = partial.state(x.src, x.lo, x.hi), sb = partial.state(x.dst, x.lo, x.hi);
          if (sa < 0 || sb < 0) return "internal: reduce over a range that is partly partial";
          kind = kKReduce;
          op.a = sa ? kLocScratch + slot_of(p, x.src) : x.src;
          op.b = sb ? kLocScratch + slot_of(p, x.dst) : x.dst;
          if (!sa) kind |= kFlagABf;
          if (!sb) kind |= kFlagBBf;
          if (sa) max_slot = std::max(max_slot, slot_of(p, x.src));
          if (sb) max_slot = std::max(max_slot, slot_of(p, x.dst));
          if (x.final_sum) {
            kind |= kFlagOBf;
            op.o = x.dst;
            if (pair) op.o2 = x.src;
          } else {
            op.o = kLocScratch + slot_of(p, x.dst);
            max_slot = std::max(max_slot, slot_of(p, x.dst));
            to_mark.push_back({x.dst, {x.lo, x.hi}});
            if (pair) {
              op.o2 = kLocScratch + slot_of(p, x.src);
              max_slot = std::max(max_slot, slot_of(p, x.src));
              to_mark.push_back({x.src, {x.lo, x.hi}});
            }
          }
          if (pair) kind |= kFlagO2;
        }
        const int32_t key = kind | ((x.kind == kReduce && x.final_sum) ? 0x10000 : 0);
        Launch &L = by_kind[key];
        L.kind = kind;
        L.ops.push_back(op);
      }
      // partial sums written by this sub-launch are visible to the next one
      for (const auto &m : to_mark) partial.mark(m.first, m.second.first, m.second.second);
      for (auto &kv : by_kind) {
        finals.push_back((kv.first & 0x10000) != 0 && !(kv.second.kind & kFlagO2));
        p.launches.push_back(std::move(kv.second));
      }
    }
    j = j1;
  }
  p.nslots = max_slot + 1;

  if (fuse) {
    // The reduce that completes a chunk, followed by the copy that first
    // forwards it ([PRIMER] 4.2: all-gather step 0 sends the chunk the
    // sender has just completed), becomes one launch whose ops write the
    // finished value to the receiver and to the next rank.
    std::vector<Launch> fused;
    for (size_t i = 0; i < p.launches.size(); ++i) {
      Launch &L = p.launches[i];
      if (finals[i] && i + 1 < p.launches.size() && (p.launches[i + 1].kind & 0xF00) == copy_fam &&
          p.launches[i + 1].ops.size() == L.ops.size()) {
        Launch trial = L;
        bool ok = true;
        for (const Op &c : p.launches[i + 1].ops) {
          bool found = false;
          for (Op &r : trial.ops)
            if (r.o == c.a && r.lo == c.lo && r.hi == c.hi && r.o2 == kLocNone) {
              r.o2 = c.o;
              found = true;
              break;
            }
          if (!found) { ok = false; break; }
        }
        if (ok) {
          trial.kind |= kFlagO2;
          fused.push_back(std::move(trial));
          ++i;  // the copy launch is absorbed
          continue;
        }
      }
      fused.push_back(std::move(L));
    }
    p.launches = std::move(fused);
  }
  return "";
}

std::string lower_onepass(Plan &p) {
  p.launches.clear();
  p.nslots = 0;
  // INT8 plans encode and decode even on one rank; op ranges count p.units
  // (elements, or blocks for INT8)
  if ((p.nranks == 1 && p.dtype != kI8EF) || p.count == 0) return "";
  const int32_t dt = p.dtype;
  if (p.coll == kAllGather) {
    // every owned range goes from its owner to every other rank in one copy
    Launch L{kKFan | static_cast<int32_t>(elem_bytes(p.dtype)), {}};
    for (int r = 0; r < p.nranks; ++r)
      if (p.owned[r].second > p.owned[r].first)
        L.ops.push_back({p.owned[r].first, p.owned[r].second, r, kLocNone, kLocNone, kLocNone, 0});
    p.launches.push_back(std::move(L));
    return "";
  }
  if (p.sched == kRing || p.nranks == 1) {
    // element in chunk c: ((x_c + x_{c+1}) + ...) + x_{c+N-1} -- chunk c is
    // first sent by rank c at reduce-scatter step 0 and gains one rank per step
    Launch L{kKRing | dt, {}};
    const Cut cut{0, p.units, p.nranks};
    for (int c = 0; c < p.nranks; ++c)
      if (cut.hi(c) > cut.lo(c)) L.ops.push_back({cut.lo(c), cut.hi(c), kLocNone, kLocNone, kLocNone, kLocNone, c});
    p.launches.push_back(std::move(L));
  } else if (p.sched == kHier) {
    // slice k of group g: ((x_{g,k+1} + x_{g,k+2}) + ...) + x_{g,k}; then sub-chunk
    // j of the slice folds the group partials as a ring starting at group j
    const int G = p.group_size, M = p.nranks / p.group_size;
    Launch L{kKHier | dt, {}};
    const Cut slices{0, p.units, G};
    for (int k = 0; k < G; ++k) {
      const Cut sub{slices.lo(k), slices.hi(k) - slices.lo(k), M};
      for (int jj = 0; jj < M; ++jj)
        if (sub.hi(jj) > sub.lo(jj))
          L.ops.push_back({sub.lo(jj), sub.hi(jj), kLocNone, kLocNone, kLocNone, kLocNone,
                           ((k + 1) % G) | (jj << 8)});
    }
    p.launches.push_back(std::move(L));
  } else if (p.sched == kDTree) {
    // half h follows tree h: tree 1 = x_0 + D(N/2, N/2), tree 2 = x_{N-1} +
    // D(N/2 - 1, N/2), D(c, b) = (x_c + D(c - b/2, b/2)) + D(c + b/2, b/2)
    Launch L{kKDTree | dt, {}};
    const Cut halves{0, p.units, 2};
    for (int h = 0; h < 2; ++h)
      if (halves.hi(h) > halves.lo(h))
        L.ops.push_back({halves.lo(h), halves.hi(h), kLocNone, kLocNone, kLocNone, kLocNone, h});
    p.launches.push_back(std::move(L));
  } else {
    // Rabenseifner and recursive doubling: the balanced pairwise tree over
    // ranks in index order, ((x0 + x1) + (x2 + x3)) + ...; the binomial tree
    // gives the same when N is 2^k and a left-complete tree otherwise
    Launch L{kKTree | dt, {}};
    L.ops.push_back({0, p.units, kLocNone, kLocNone, kLocNone, kLocNone, 0});
    p.launches.push_back(std::move(L));
  }
  if (p.coll == kReduceScatter) {
    // a reduce-scatter keeps each range on its owner: every op covers one
    // owned range (the tree fold, one op over everything, is cut into them;
    // its order does not depend on the range) and stores into that rank only
    for (Launch &L : p.launches) {
      L.kind |= kKOwner;
      if ((L.kind & 0xF00) == kKTree) {
        L.ops.clear();
        for (int r = 0; r < p.nranks; ++r)
          if (p.owned[r].second > p.owned[r].first)
            L.ops.push_back({p.owned[r].first, p.owned[r].second, kLocNone, kLocNone, r, kLocNone, 0});
        continue;
      }
      for (Op &op : L.ops) {
        for (int r = 0; r < p.nranks && op.o == kLocNone; ++r)
          if (p.owned[r].first == op.lo && p.owned[r].second == op.hi) op.o = r;
        if (op.o == kLocNone) return "internal: a one-pass op is not an owned range";
      }
    }
  }
  return "";
}

uint64_t loc_bytes(const Plan &p, int32_t loc, bool bf16_flag) {
  if (loc == kLocNone) return 0;
  if (p.dtype == kF32) return 4;
  return bf16_flag ? 2 : 4;  // bf16 operand, or an fp32 partial in scratch
}

void compute_stats(Plan &p) {
  p.bytes_sent.assign(p.nranks, 0);
  p.cross_group_bytes = 0;
  for (const Transfer &x : p.xfers) {
    const uint64_t b = xfer_bytes(p, x);
    p.bytes_sent[x.src] += b;
    if (x.src / p.group_size != x.dst / p.group_size) p.cross_group_bytes += b;
  }
  const uint64_t eb = static_cast<uint64_t>(elem_bytes(p.dtype));
  uint64_t h = 0;
  for (const Launch &L : p.launches) {
    const int32_t fam = L.kind & 0xF00;
    for (const Op &op : L.ops) {
      const uint64_t len = static_cast<uint64_t>(op.hi - op.lo);
      const uint64_t el = static_cast<uint64_t>(unit_elems(p, op.lo, op.hi));
      const uint64_t outs = op.o2 != kLocNone ? 2 : 1;
      if (fam == kKReduce) {
        const bool obf = L.kind & kFlagOBf;
        h += len * (loc_bytes(p, op.a, L.kind & kFlagABf) + loc_bytes(p, op.b, L.kind & kFlagBBf) +
                    loc_bytes(p, op.o, obf) + loc_bytes(p, op.o2, obf));
      } else if (fam == kKCopy) {
        h += len * 2 * eb;
      } else if (fam == kKQEncode) {
        h += el * (4 + 4 + 1 + 4) + 4 * len;  // g, e in; codes, e out; scales
      } else if (fam == kKQReduce) {
        const int32_t f = L.kind;
        for (int32_t raw : {f & kQFlagARaw, f & kQFlagBRaw})
          h += raw ? el * 12 : el + 4 * len;  // own g, e in and e out, or codes and scale in
        if (!(f & kQFlagNoCode)) h += (el + 4 * len) * outs;
        if (f & kQFlagDec) h += el * 4 * outs;
      } else if (fam == kKQCopy) {
        h += el + 4 * len;
        if (!(L.kind & kQFlagNoCode)) h += el + 4 * len;
        if (L.kind & kQFlagDec) h += el * 4;
      } else if (fam == kKQDecode) {
        h += el * (1 + 4) + 4 * len;
      } else if (p.dtype == kI8EF) {
        h += el * 16 * static_cast<uint64_t>(p.nranks);  // g, e in; e, result out, per rank
      } else if (fam == kKFan) {
        h += len * eb * static_cast<uint64_t>(p.nranks);  // the owner's range in, N - 1 copies out
      } else {
        // every rank in; the result out to every rank, or to the owner only
        h += len * eb * (static_cast<uint64_t>(p.nranks) + (op.o != kLocNone ? 1 : static_cast<uint64_t>(p.nranks)));
      }
    }
  }
  p.hbm_bytes = h;
}

// Unit ranges per rank (a small interval list).
struct RangeSet {
  std::vector<std::vector<std::pair<int64_t, int64_t>>> r;
  explicit RangeSet(int n) : r(n) {}
  void add(int q, int64_t lo, int64_t hi) { r[q].push_back({lo, hi}); }
  bool overlaps(int q, int64_t lo, int64_t hi) const {
    for (const auto &x : r[q])
      if (x.first < hi && lo < x.second) return true;
    return false;
  }
  bool covers(int q, int64_t lo, int64_t hi) const {  // union of the ranges covers [lo, hi)
    std::vector<std::pair<int64_t, int64_t>> v = r[q];
    std::sort(v.begin(), v.end());
    int64_t at = lo;
    for (const auto &x : v)
      if (x.first <= at) at = std::max(at, x.second);
    return at >= hi;
  }
};

// Fused INT8 step lowering: the first reduce that touches a rank's range
// encodes g + e itself (the residual is written there), and the last write
// of a rank's range also decodes it into the rank's buffer, so no separate
// encode or decode pass runs.  Returns false (launches untouched) when the
// schedule does not have that shape: an operand range partly consumed, a
// copy of codes never written, fused outputs that disagree, or a rank range
// never consumed or never finished.
bool fuse_quantized(Plan &p) {
  const int n = p.nranks;
  struct Tag {
    int32_t flags;
  };
  std::vector<std::vector<Tag>> tags(p.launches.size());
  PartialMap consumed(n), written(n);
  RangeSet raw_used(n);
  for (size_t i = 0; i < p.launches.size(); ++i) {
    const Launch &L = p.launches[i];
    const int32_t fam = L.kind & 0xF00;
    for (const Op &o : L.ops) {
      int32_t f = 0;
      auto operand = [&](int q, int32_t raw_flag) -> bool {
        if (written.state(q, o.lo, o.hi) == 1) return true;  // codes present
        if (written.state(q, o.lo, o.hi) != 0 || consumed.state(q, o.lo, o.hi) != 0) return false;
        f |= raw_flag;
        return true;
      };
      if (fam == kKQReduce) {
        if (!operand(o.a, kQFlagARaw) || !operand(o.b, kQFlagBRaw)) return false;
      } else if (fam == kKQCopy) {
        if (written.state(o.a, o.lo, o.hi) != 1) return false;
      } else {
        return false;
      }
      tags[i].push_back({f});
    }
    // marks after the launch: its ops are hazard-free among themselves
    for (size_t k = 0; k < L.ops.size(); ++k) {
      const Op &o = L.ops[k];
      if (tags[i][k].flags & kQFlagARaw) {
        consumed.mark(o.a, o.lo, o.hi);
        raw_used.add(o.a, o.lo, o.hi);
      }
      if (tags[i][k].flags & kQFlagBRaw) {
        consumed.mark(o.b, o.lo, o.hi);
        raw_used.add(o.b, o.lo, o.hi);
      }
      written.mark(o.o, o.lo, o.hi);
      if (o.o2 != kLocNone) written.mark(o.o2, o.lo, o.hi);
    }
  }
  // backward: is an output the last write of that range, is it read later?
  RangeSet later_write(n), later_read(n), finished(n);
  for (size_t i = p.launches.size(); i-- > 0;) {
    const Launch &L = p.launches[i];
    const bool reduce = (L.kind & 0xF00) == kKQReduce;
    for (size_t k = 0; k < L.ops.size(); ++k) {
      const Op &o = L.ops[k];
      const bool fin = !later_write.overlaps(o.o, o.lo, o.hi);
      bool need = later_read.overlaps(o.o, o.lo, o.hi);
      if (o.o2 != kLocNone) {
        if (fin != !later_write.overlaps(o.o2, o.lo, o.hi)) return false;
        need = need || later_read.overlaps(o.o2, o.lo, o.hi);  // codes go to both or neither
      }
      if (fin) tags[i][k].flags |= kQFlagDec | (need ? 0 : kQFlagNoCode);
    }
    for (size_t k = 0; k < L.ops.size(); ++k) {
      const Op &o = L.ops[k];
      later_write.add(o.o, o.lo, o.hi);
      if (o.o2 != kLocNone) later_write.add(o.o2, o.lo, o.hi);
      if (tags[i][k].flags & kQFlagDec) {
        finished.add(o.o, o.lo, o.hi);
        if (o.o2 != kLocNone) finished.add(o.o2, o.lo, o.hi);
      }
      if (!reduce || !(tags[i][k].flags & kQFlagARaw)) later_read.add(o.a, o.lo, o.hi);
      if (reduce && !(tags[i][k].flags & kQFlagBRaw)) later_read.add(o.b, o.lo, o.hi);
    }
  }
  for (int q = 0; q < n; ++q)
    if (!raw_used.covers(q, 0, p.units) || !finished.covers(q, 0, p.units)) return false;
  // split each launch into launches of uniform flags
  std::vector<Launch> out;
  for (size_t i = 0; i < p.launches.size(); ++i) {
    std::map<int32_t, Launch> by;
    for (size_t k = 0; k < p.launches[i].ops.size(); ++k) {
      Launch &L = by[tags[i][k].flags];
      L.kind = p.launches[i].kind | tags[i][k].flags;
      L.ops.push_back(p.launches[i].ops[k]);
    }
    for (auto &kv : by) out.push_back(std::move(kv.second));
  }
  p.launches = std::move(out);
  return true;
}

// Blockwise INT8: encode every rank, run the schedule over code slots,
// decode every rank -- or, fused, with the encode and decode folded into the
// schedule's first and last touches of each range.
std::string lower_quantized(Plan &p, bool fuse) {
  std::string err = lower_steps(p, fuse);
  if (!err.empty()) return err;
  p.nslots = 0;
  if (p.count == 0) {
    p.launches.clear();
    return "";
  }
  if (fuse && p.nranks > 1) {
    const std::vector<Launch> keep = p.launches;
    if (fuse_quantized(p)) return "";
    p.launches = keep;
  }
  Launch enc{kKQEncode, {}}, dec{kKQDecode, {}};
  for (int r = 0; r < p.nranks; ++r) {
    enc.ops.push_back({0, p.units, r, kLocNone, r, kLocNone, 0});
    dec.ops.push_back({0, p.units, r, kLocNone, r, kLocNone, 0});
  }
  p.launches.insert(p.launches.begin(), std::move(enc));
  p.launches.push_back(std::move(dec));
  return "";
}

std::string lower(Plan &p, Exec exec) {
  p.exec = exec;
  if (p.nranks > kMaxExecRanks) {  // described (stats, cost model) but not executable
    p.launches.clear();
    p.nslots = 0;
    p.slot_stride = 0;
    compute_stats(p);
    return "";
  }
  std::string err;
  if (exec == kOnePass) err = lower_onepass(p);
  else if (p.dtype == kI8EF) err = lower_quantized(p, exec == kSteps);
  else err = lower_steps(p, exec == kSteps);
  if (!err.empty()) return err;
  p.slot_stride = slot_stride_for(p.count);
  compute_stats(p);
  return check_hazards(p);
}

}  // namespace

std::string build_plan(Plan &p, int nranks, int group_size, int64_t count, Dtype dtype, Sched sched,
                       Exec exec, bool *unsupported, Coll coll) {
  *unsupported = false;
  if (nranks < 1 || nranks > kMaxPlanRanks) return "nranks must be in [1, 1024]";
  if (group_size < 1 || nranks % group_size) return "group_size must be >= 1 and divide nranks";
  if (count < 0) return "count must be >= 0";
  if (dtype != kF32 && dtype != kBF16 && dtype != kBF16Each && dtype != kI8EF) return "unknown dtype";
  if (sched < kRing || sched > kDTree) return "unknown schedule";
  if (exec != kSteps && exec != kStepsUnfused && exec != kOnePass) return "unknown exec mode";
  if (coll != kAllReduce && coll != kReduceScatter && coll != kAllGather) return "unknown collective";
  if ((sched == kRaben || sched == kRDouble || sched == kDTree) && (nranks & (nranks - 1))) {
    *unsupported = true;
    return "this schedule needs a power-of-two number of ranks";
  }
  if (coll != kAllReduce) {
    *unsupported = true;
    if (sched != kRing && sched != kHier && sched != kRaben)
      return "reduce-scatter and all-gather plans need the ring, hierarchical or Rabenseifner schedule";
    if (dtype == kI8EF) return "reduce-scatter and all-gather plans are fp32 or bf16";
    *unsupported = false;
  }
  p = Plan{};
  p.nranks = nranks;
  p.group_size = group_size;
  p.count = count;
  p.dtype = dtype;
  p.sched = sched;
  // [SCALING] "Blockwise quantization": the INT8 schedule moves whole blocks,
  // so its transfers are cut on block boundaries
  const int64_t units = dtype == kI8EF ? (count + kQBlock - 1) / kQBlock : count;
  p.units = units;
  if (dtype == kI8EF) {
    p.code_stride = (units * kQBlock + 255) / 256 * 256;
    p.scale_stride = (units + 63) / 64 * 64;
  }
  if (sched == kRing) p.nsteps = build_ring(p.xfers, nranks, units);
  else if (sched == kHier) p.nsteps = build_hier(p.xfers, nranks, group_size, units);
  else if (sched == kRaben) p.nsteps = build_raben(p.xfers, nranks, units);
  else if (sched == kRDouble) p.nsteps = build_rdouble(p.xfers, nranks, units);
  else if (sched == kTree) p.nsteps = build_tree(p.xfers, nranks, units);
  else p.nsteps = build_dtree(p.xfers, nranks, units);
  std::stable_sort(p.xfers.begin(), p.xfers.end(),
                   [](const Transfer &a, const Transfer &b) { return a.step < b.step; });
  if (sched == kRing || sched == kHier || sched == kRaben) {
    // the receiver of the reduce that completes a range owns it; one rank
    // holds everything when there is no transfer
    p.owned.assign(nranks, {0, nranks == 1 ? units : 0});
    for (const Transfer &x : p.xfers)
      if (x.kind == kReduce && x.final_sum) p.owned[x.dst] = {x.lo, x.hi};
  }
  p.coll = coll;
  if (coll != kAllReduce) {
    // one half of the schedule: its reduce rounds (the reduce-scatter) or its
    // copy rounds (the all-gather), which are consecutive; the transfers keep
    // the schedule's round numbers, so the launch order treats every round
    // as it does in the whole all-reduce
    const int32_t keep = coll == kReduceScatter ? kReduce : kCopy;
    std::vector<Transfer> half;
    for (const Transfer &x : p.xfers)
      if (x.kind == keep) half.push_back(x);
    p.xfers = std::move(half);
    p.step0 = p.xfers.empty() ? 0 : p.xfers.front().step;
    p.nsteps = p.xfers.empty() ? 0 : p.xfers.back().step - p.step0 + 1;
  }
  return lower(p, exec);
}

bool owned_range(const Plan &p, int rank, int64_t *lo, int64_t *hi) {
  if (rank < 0 || rank >= p.nranks || static_cast<int>(p.owned.size()) != p.nranks) return false;
  *lo = p.owned[rank].first;
  *hi = p.owned[rank].second;
  return true;
}

std::string relower(Plan &p, Exec exec) {
  if (exec != kSteps && exec != kStepsUnfused && exec != kOnePass) return "unknown exec mode";
  return lower(p, exec);
}

double cost_alpha_beta(const Plan &p, double alpha_s, double bw_intra, double bw_cross) {
  // [DCN] 7.2.1: rounds run one after another; within a round the slowest
  // transfer sets the time, and every round pays its start-up alpha.
  std::vector<double> slowest(static_cast<size_t>(p.nsteps), 0.0);
  for (const Transfer &x : p.xfers) {
    const bool cross = x.src / p.group_size != x.dst / p.group_size;
    const double t = static_cast<double>(xfer_bytes(p, x)) / (cross ? bw_cross : bw_intra);
    slowest[x.step - p.step0] = std::max(slowest[x.step - p.step0], t);
  }
  double total = 0;
  for (double t : slowest) total += alpha_s + t;
  return total;
}

double cost_alpha_beta_ex(const Plan &p, double alpha_intra, double alpha_cross, double bw_intra, double bw_cross,
                          double bw_egress, double egress_share) {
  // [DCN] 7.2.1: T = sum over rounds of (start-up + max over resources e of
  // V_{r,e} / B_e).  Resources: each rank's own intra and cross links, and,
  // when bw_egress > 0, each group's shared egress ([DCN] 7.6.4, T_grad).
  const int groups = p.nranks / p.group_size;
  std::vector<double> link(static_cast<size_t>(p.nsteps), 0.0);
  std::vector<std::vector<double>> egress(static_cast<size_t>(p.nsteps), std::vector<double>(groups, 0.0));
  std::vector<bool> crosses(static_cast<size_t>(p.nsteps), false);
  for (const Transfer &x : p.xfers) {
    const double bytes = static_cast<double>(xfer_bytes(p, x));
    const bool cross = x.src / p.group_size != x.dst / p.group_size;
    const int r = x.step - p.step0;
    link[r] = std::max(link[r], bytes / (cross ? bw_cross : bw_intra));
    if (cross) {
      crosses[r] = true;
      egress[r][x.src / p.group_size] += bytes * egress_share;
    }
  }
  double total = 0;
  for (int r = 0; r < p.nsteps; ++r) {
    double t = link[r];
    if (bw_egress > 0)
      for (double v : egress[r]) t = std::max(t, v / bw_egress);
    total += (crosses[r] ? alpha_cross : alpha_intra) + t;
  }
  return total;
}

int64_t launch_write_bytes(const Plan &p, const Launch &L) {
  const int32_t fam = L.kind & 0xF00;
  const bool fold = fam == kKRing || fam == kKHier || fam == kKTree || fam == kKDTree;
  int64_t elems = 0;
  for (const Op &o : L.ops) {
    const int64_t e = unit_elems(p, o.lo, o.hi);
    if (fold) elems += e * (o.o != kLocNone ? 1 : p.nranks);  // the owner only, or every rank
    else if (fam == kKFan) elems += e * (p.nranks - 1);
    else elems += e * ((o.o2 != kLocNone) ? 2 : 1);
  }
  int64_t eb = buffer_elem_bytes(p.dtype);
  if (fam == kKReduce && p.dtype == kBF16 && !(L.kind & kFlagOBf)) eb = 4;  // fp32 partials
  if (fam == kKQReduce || fam == kKQCopy || fam == kKQEncode) eb = 1;       // codes
  return elems * eb;
}

std::string merge_segments(Plan &out, const std::vector<const Plan *> &parts, const std::vector<int64_t> &offsets,
                           int64_t count) {
  if (parts.empty() || parts.size() != offsets.size()) return "no segments";
  const Plan &p0 = *parts[0];
  if (p0.dtype == kI8EF) return "INT8 plans are not merged";
  int64_t end = 0;
  for (size_t k = 0; k < parts.size(); ++k) {
    const Plan &q = *parts[k];
    if (q.nranks != p0.nranks || q.group_size != p0.group_size || q.dtype != p0.dtype || q.sched != p0.sched ||
        q.exec != p0.exec)
      return "segments differ in ranks, dtype, schedule or exec mode";
    if (offsets[k] < end || q.count < 0 || offsets[k] > count - q.count) return "segments overlap or exceed the buffer";
    end = offsets[k] + q.count;
  }
  Plan m;
  m.nranks = p0.nranks;
  m.group_size = p0.group_size;
  m.count = count;
  m.units = count;
  m.dtype = p0.dtype;
  m.sched = p0.sched;
  m.exec = p0.exec;
  m.cache_bytes = p0.cache_bytes;
  for (size_t k = 0; k < parts.size(); ++k) {
    m.nsteps = std::max(m.nsteps, parts[k]->nsteps);
    m.nslots = std::max(m.nslots, parts[k]->nslots);
    for (Transfer x : parts[k]->xfers) {
      x.lo += offsets[k];
      x.hi += offsets[k];
      m.xfers.push_back(x);
    }
  }
  std::stable_sort(m.xfers.begin(), m.xfers.end(), [](const Transfer &a, const Transfer &b) { return a.step < b.step; });
  // batches of consecutive segments: the widest rounds of a batch write at
  // most cache_bytes together, and a merged launch carries at most
  // kMaxLaunchOps ops (launch i of a batch holds launch i of each segment)
  std::vector<size_t> first{0};
  int64_t fill = 0, fill_ops = 0;
  for (size_t k = 0; k < parts.size(); ++k) {
    int64_t widest = 0, most_ops = 0;
    for (const Launch &L : parts[k]->launches) {
      widest = std::max(widest, launch_write_bytes(*parts[k], L));
      most_ops = std::max(most_ops, static_cast<int64_t>(L.ops.size()));
    }
    const bool bytes_full = m.exec != kOnePass && fill > 0 && fill + widest > m.cache_bytes;
    if (k > first.back() && (bytes_full || fill_ops + most_ops > kMaxLaunchOps)) {
      first.push_back(k);
      fill = 0;
      fill_ops = 0;
    }
    fill += widest;
    fill_ops += most_ops;
  }
  first.push_back(parts.size());
  int64_t extent = 0;  // widest batch, in elements: the scratch slots hold one batch at a time
  for (size_t b = 0; b + 1 < first.size(); ++b) {
    const int64_t lo = offsets[first[b]];
    int64_t hi = lo;
    for (size_t k = first[b]; k < first[b + 1]; ++k) hi = std::max(hi, offsets[k] + parts[k]->count);
    extent = std::max(extent, hi - lo);
    std::vector<size_t> next(parts.size(), 0);  // next launch of each segment of the batch
    for (;;) {
      int32_t kind = -1;
      for (size_t k = first[b]; k < first[b + 1] && kind < 0; ++k)
        if (next[k] < parts[k]->launches.size()) kind = parts[k]->launches[next[k]].kind;
      if (kind < 0) break;
      Launch L{kind, {}, lo};
      for (size_t k = first[b]; k < first[b + 1]; ++k) {
        if (next[k] >= parts[k]->launches.size() || parts[k]->launches[next[k]].kind != kind) continue;
        for (Op o : parts[k]->launches[next[k]].ops) {
          o.lo += offsets[k];
          o.hi += offsets[k];
          L.ops.push_back(o);
        }
        ++next[k];
      }
      m.launches.push_back(std::move(L));
    }
  }
  m.slot_stride = slot_stride_for(extent);
  compute_stats(m);
  out = std::move(m);
  return "";
}

std::string check_hazards(const Plan &p) {
  struct Acc { int32_t loc; int64_t lo, hi; bool write; };
  for (size_t li = 0; li < p.launches.size(); ++li) {
    const Launch &L = p.launches[li];
    const int32_t fam = L.kind & 0xF00;
    if (fam != kKReduce && fam != kKCopy && fam != kKQReduce && fam != kKQCopy)
      continue;  // one-pass, encode and decode ops touch disjoint ranges by construction
    std::vector<std::vector<Acc>> acc(L.ops.size());
    for (size_t i = 0; i < L.ops.size(); ++i) {
      const Op &o = L.ops[i];
      for (int32_t r : {o.a, o.b})
        if (r != kLocNone) acc[i].push_back({r, o.lo, o.hi, false});
      for (int32_t w : {o.o, o.o2})
        if (w != kLocNone) acc[i].push_back({w, o.lo, o.hi, true});
    }
    for (size_t i = 0; i < acc.size(); ++i)
      for (size_t k = i + 1; k < acc.size(); ++k)
        for (const Acc &x : acc[i])
          for (const Acc &y : acc[k])
            if ((x.write || y.write) && x.loc == y.loc && x.lo < y.hi && y.lo < x.hi) {
              char buf[160];
              std::snprintf(buf, sizeof buf, "hazard in launch %zu: ops %zu and %zu touch location %d", li, i, k,
                            x.loc);
              return buf;
            }
  }
  return "";
}

double overlap_step_time(int nchunks, const double *ready, const double *comm, double compute_end, double update,
                         double *exposed) {
  // [PRIMER] 4.7, Figure 4.15: a chunk's collective starts once backward has
  // produced the chunk and the previous collective is done; the update waits
  // for the compute and for the last collective.
  double end = 0.0;
  for (int k = 0; k < nchunks; ++k) end = std::max(end, ready[k]) + comm[k];
  const double done = std::max(compute_end, end);
  if (exposed) *exposed = std::max(0.0, end - compute_end);
  return done + update;
}

void assign_buckets(const std::vector<int64_t> &tensor_counts, int64_t cap_elems, int64_t align_elems,
                    std::vector<int64_t> &tensor_offsets, std::vector<int64_t> &bucket_offset,
                    std::vector<int64_t> &bucket_count, int64_t &arena_count) {
  // [SCALING] "Bucket fusion": parameters go into buckets in the reverse of
  // their forward order, the order their gradients become ready in backward.
  const int n = static_cast<int>(tensor_counts.size());
  tensor_offsets.assign(n, 0);
  bucket_offset.clear();
  bucket_count.clear();
  int64_t cursor = 0, fill = -1;  // fill < 0: no open bucket
  for (int t = n - 1; t >= 0; --t) {
    const int64_t c = tensor_counts[t];
    if (fill > 0 && fill + c > cap_elems) {  // close the open bucket (a lone tensor may exceed the cap)
      bucket_count.push_back(fill);
      cursor = bucket_offset.back() + fill;
      fill = -1;
    }
    if (fill < 0) {
      cursor = (cursor + align_elems - 1) / align_elems * align_elems;
      bucket_offset.push_back(cursor);
      fill = 0;
    }
    tensor_offsets[t] = bucket_offset.back() + fill;
    fill += c;
  }
  if (fill >= 0) {
    bucket_count.push_back(fill);
    cursor = bucket_offset.back() + fill;
  }
  arena_count = cursor;
}

}  // namespace ar
