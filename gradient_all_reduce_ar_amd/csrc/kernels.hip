// kernels.hip -- HIP kernels for gfx950 (CDNA4) that execute the all-reduce
// schedules over N virtual ranks held in one GPU's HBM.
//
// The work is a stream over HBM (one add per 8-12 bytes moved), so the
// kernels are built for bandwidth: every wavefront instruction moves a
// contiguous 1 KiB (fp32) or 512 B (bf16) span, each thread keeps UNROLL
// independent 16-byte loads in flight, and no LDS or MFMA is involved --
// nothing is reused, so staging through LDS would only add a round trip.
//
// Launch geometry: a block works on one op (one transfer of the step; see
// block_coord) and walks its element range in tiles that are aligned to the
// tile size in absolute element coordinates, so every rank buffer, every
// scratch slot and every vector access of a tile share the same alignment.
// Only the first and last tile of an op can be cut by its range; there the
// vector units inside the op still move as vectors and only the units the
// range cuts go element by element.
//
// Summation order.  Each output element is produced by exactly one thread
// from its inputs in the schedule's order with IEEE binary32 adds (packed
// fp32 ops disabled at build time, no contraction, denormals kept), so the
// bits equal a step-by-step execution of the schedule.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <type_traits>
#include <utility>

#include "kernels.hpp"

namespace ar_dev {

thread_local LaunchEvents t_launch_events;

namespace {

constexpr int kBlock = AR_BLOCK;
constexpr int kOPB = AR_ONEPASS_BLOCK;  // threads per workgroup of the one-pass kernels
constexpr int kCpolOnePassF32 = AR_CPOL_ONEPASS_F32, kCpolOnePassBF16 = AR_CPOL_ONEPASS_BF16;

// Native vector types: 16-byte and 8-byte accesses compile to single
// global_load/store_dwordx4 / dwordx2 instructions.
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Streaming accesses.  Every input byte is read once per kernel, so loads
// carry the non-temporal hint (AR_NTL).  Full-tile stores take a cache
// policy (AR_CPOL_*; measured on MI355X): sc1 into rank buffers and fp32
// scratch written by a step (the next step reads them back through the
// device cache; sc1 was 5% faster than the default policy for a ring
// reduce step and 2% for a copy step, non-temporal stores 7% slower), and
// nt (fp32) or nt + sc1 (bf16) in the one-pass kernels, whose output
// nothing reads back.  The hints never change results.
template <typename T>
__device__ __forceinline__ T ld(const char *p) {
#if AR_NTL
  return __builtin_nontemporal_load(reinterpret_cast<const T *>(p));
#else
  return *reinterpret_cast<const T *>(p);
#endif
}
// Stores v at byte offset `off` (per lane) from the wave-uniform address
// `ubase` with cache policy CPOL.  Policies with sc1 go through a buffer
// store, the one vector store that takes the policy bits from the program;
// its resource is built from ubase (uniform, so it lives in scalar
// registers) and covers 2^31 - 1 bytes, far more than a tile.
constexpr int kBufferRsrcFlags = 0x00020000;  // resource word 3: 32-bit data format
template <int CPOL, typename T>
__device__ __forceinline__ void st_cp(char *ubase, uint32_t off, T v) {
  if constexpr ((CPOL & 16) == 0) {
    if constexpr (CPOL & 2) __builtin_nontemporal_store(v, reinterpret_cast<T *>(ubase + off));
    else *reinterpret_cast<T *>(ubase + off) = v;
  } else {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(ubase, 0, 0x7fffffff, kBufferRsrcFlags);
    if constexpr (sizeof(T) == 16) {
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, CPOL);
    } else {
      static_assert(sizeof(T) == 8, "16- or 8-byte stores");
      __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), r, off, 0, CPOL);
    }
  }
}

// Block -> (op, tile): blockIdx.y is the op and blockIdx.x the first tile; a
// block handles tiles tile, tile + stride, ... of its op (the host launches
// fewer blocks than tiles where a block should walk several).
struct BlockCoord {
  int op;
  int64_t tile, stride;
};
__device__ __forceinline__ BlockCoord block_coord() {
  return {static_cast<int>(blockIdx.y), static_cast<int64_t>(blockIdx.x), static_cast<int64_t>(gridDim.x)};
}

__device__ __forceinline__ const char *src_ptr(const KArgs &a, int32_t loc) {
  return loc >= kLocScratchDev
             ? reinterpret_cast<const char *>(a.scratch + static_cast<int64_t>(loc - kLocScratchDev) * a.slot_stride)
             : static_cast<const char *>(a.rank[loc]);
}
__device__ __forceinline__ char *dst_ptr(const KArgs &a, int32_t loc) {
  return loc >= kLocScratchDev
             ? reinterpret_cast<char *>(a.scratch + static_cast<int64_t>(loc - kLocScratchDev) * a.slot_stride)
             : static_cast<char *>(a.rank[loc]);
}

// bf16 <-> fp32.  Widening is exact (the bf16 bits are the top half of the
// fp32 pattern).  Narrowing rounds to nearest, ties to even, computed on the
// bit pattern: add 0x7fff plus the lowest kept bit, drop the low 16 bits.
// NaN keeps its sign and top payload bits and is forced quiet.
__device__ __forceinline__ float widen(uint32_t h) { return __uint_as_float(h << 16); }

__device__ __forceinline__ uint32_t narrow(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t rounded = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
  return (u & 0x7fffffffu) > 0x7f800000u ? ((u >> 16) | 0x40u) : rounded;
}

// 4-element units: fp32 = 16 B (float4), bf16 = 8 B (uint2).
template <bool BF>
__device__ __forceinline__ float4 load4(const char *base, int64_t e) {
  if constexpr (BF) {
    const u32x2 v = ld<u32x2>(base + e * 2);
    return make_float4(widen(v.x & 0xffffu), widen(v.x >> 16), widen(v.y & 0xffffu), widen(v.y >> 16));
  } else {
    const f32x4 v = ld<f32x4>(base + e * 4);
    return make_float4(v.x, v.y, v.z, v.w);
  }
}

template <bool BF>
__device__ __forceinline__ float load1(const char *base, int64_t e) {
  if constexpr (BF) return widen(*reinterpret_cast<const uint16_t *>(base + e * 2));
  else return *reinterpret_cast<const float *>(base + e * 4);
}

__device__ __forceinline__ u32x2 pack4(float4 v) {
  u32x2 r;
  r.x = narrow(v.x) | (narrow(v.y) << 16);
  r.y = narrow(v.z) | (narrow(v.w) << 16);
  return r;
}

// 4-element units at element tile0 + lane (tile0 wave-uniform, lane per
// lane) of the buffer at base.
template <int CPOL>
__device__ __forceinline__ void store_bits4(char *base, int64_t tile0, uint32_t lane, u32x2 bits) {
  st_cp<CPOL, u32x2>(base + tile0 * 2, lane * 2, bits);
}

template <bool BF, int CPOL>
__device__ __forceinline__ void store4(char *base, int64_t tile0, uint32_t lane, float4 v) {
  if constexpr (BF) {
    store_bits4<CPOL>(base, tile0, lane, pack4(v));
  } else {
    f32x4 w;
    w.x = v.x;
    w.y = v.y;
    w.z = v.z;
    w.w = v.w;
    st_cp<CPOL, f32x4>(base + tile0 * 4, lane * 4, w);
  }
}

template <bool BF>
__device__ __forceinline__ void store1(char *base, int64_t e, float v) {
  if constexpr (BF) *reinterpret_cast<uint16_t *>(base + e * 2) = static_cast<uint16_t>(narrow(v));
  else *reinterpret_cast<float *>(base + e * 4) = v;
}

__device__ __forceinline__ float4 add4(float4 a, float4 b) {
  return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
}

// One fold step of a one-pass kernel; EACH rounds the partial sum to bf16 at
// once (the round-each-step bf16 mode), else it stays fp32.
__device__ __forceinline__ float round_keep(float v) { return widen(narrow(v)); }
template <bool EACH>
__device__ __forceinline__ float4 fold4(float4 a, float4 b) {
  const float4 s = add4(a, b);
  if constexpr (EACH) return make_float4(round_keep(s.x), round_keep(s.y), round_keep(s.z), round_keep(s.w));
  return s;
}
__device__ __forceinline__ float fold1(bool each, float a, float b) {
  const float s = a + b;
  return each ? round_keep(s) : s;
}

// ---------------------------------------------------------------------------
// Chunk reduce: o[e] = a[e] + b[e] over the op's range, optionally also
// written to o2 (the fused forwarding copy of the chunk just completed).
// FLAGS: 1 a is bf16, 2 b is bf16, 4 outputs are bf16 (rounded once), 8 o2.
// CP: cache policy of the full-tile stores (the host picks it for rank or
// scratch outputs).  A thread moves units of E elements: 4 (one 16-byte
// access per fp32 operand, 8 bytes per bf16 one), or 8 when every operand is
// bf16 (16-byte accesses).  An fp32 operand next to a bf16 one stays at 4
// elements per unit: with 8, each of its two 16-byte loads per lane would
// cover only half of every line (a 32-byte lane stride), and such reduces
// ran at half speed on MI355X (C3 reduce-scatter step 71 -> 153 us).
// ---------------------------------------------------------------------------
template <int E>
struct Unit {
  float4 v[E / 4];
};

template <bool BF, int E>
__device__ __forceinline__ Unit<E> load_unit(const char *base, int64_t e) {
  Unit<E> r;
  if constexpr (BF && E == 8) {
    const u32x4 w = ld<u32x4>(base + e * 2);
    r.v[0] = make_float4(widen(w.x & 0xffffu), widen(w.x >> 16), widen(w.y & 0xffffu), widen(w.y >> 16));
    r.v[1] = make_float4(widen(w.z & 0xffffu), widen(w.z >> 16), widen(w.w & 0xffffu), widen(w.w >> 16));
  } else {
#pragma unroll
    for (int k = 0; k < E / 4; ++k) r.v[k] = load4<BF>(base, e + 4 * k);
  }
  return r;
}

template <int E>
__device__ __forceinline__ Unit<E> add_unit(const Unit<E> &a, const Unit<E> &b) {
  Unit<E> r;
#pragma unroll
  for (int k = 0; k < E / 4; ++k) r.v[k] = add4(a.v[k], b.v[k]);
  return r;
}

// Stores a unit at element tile0 + lane (tile0 wave-uniform) with policy CP.
template <bool BF, int E, int CP>
__device__ __forceinline__ void store_unit(char *base, int64_t tile0, uint32_t lane, const Unit<E> &x) {
  if constexpr (BF && E == 8) {
    const u32x2 lo = pack4(x.v[0]), hi = pack4(x.v[1]);
    st_cp<CP, u32x4>(base + tile0 * 2, lane * 2, u32x4{lo.x, lo.y, hi.x, hi.y});
  } else if constexpr (BF) {
    store_bits4<CP>(base, tile0, lane, pack4(x.v[0]));
  } else {
#pragma unroll
    for (int k = 0; k < E / 4; ++k) store4<false, CP>(base, tile0, lane + 4 * k, x.v[k]);
  }
}

constexpr int reduce_unit_elems(int flags) { return (flags & 7) == 7 && AR_BF16_UNIT == 8 ? 8 : 4; }

template <int FLAGS, int UNROLL, int CP>
__global__ __launch_bounds__(kBlock) void chunk_reduce(KArgs args) {
  constexpr bool kABf = FLAGS & 1, kBBf = FLAGS & 2, kOBf = FLAGS & 4, kO2 = FLAGS & 8;
  constexpr int kE = reduce_unit_elems(FLAGS);
  constexpr int64_t kTile = static_cast<int64_t>(kBlock) * kE * UNROLL;
  const BlockCoord bc = block_coord();
  const DevOp op = args.ops[bc.op];
  const int64_t t_end = (op.hi + kTile - 1) / kTile;
  const char *A = src_ptr(args, op.a);
  const char *B = src_ptr(args, op.b);
  char *O = dst_ptr(args, op.o);
  char *O2 = kO2 ? dst_ptr(args, op.o2) : nullptr;
  for (int64_t t = op.lo / kTile + bc.tile; t < t_end; t += bc.stride) {
    const int64_t base = t * kTile;
    if (base >= op.lo && base + kTile <= op.hi) {
      Unit<kE> a[UNROLL], b[UNROLL];
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        const int64_t e = base + (static_cast<int64_t>(u) * kBlock + threadIdx.x) * kE;
        a[u] = load_unit<kABf, kE>(A, e);
        b[u] = load_unit<kBBf, kE>(B, e);
      }
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        const uint32_t lane = (static_cast<uint32_t>(u) * kBlock + threadIdx.x) * kE;
        const Unit<kE> s = add_unit(a[u], b[u]);
        store_unit<kOBf, kE, CP>(O, base, lane, s);
        if constexpr (kO2) store_unit<kOBf, kE, CP>(O2, base, lane, s);
      }
    } else {
      // a tile cut by the op's range: the units inside the op take the
      // vector path, the units it cuts the per-element one
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        const uint32_t lane = (static_cast<uint32_t>(u) * kBlock + threadIdx.x) * kE;
        const int64_t e0 = base + lane;
        if (e0 >= op.lo && e0 + kE <= op.hi) {
          const Unit<kE> s = add_unit(load_unit<kABf, kE>(A, e0), load_unit<kBBf, kE>(B, e0));
          store_unit<kOBf, kE, CP>(O, base, lane, s);
          if constexpr (kO2) store_unit<kOBf, kE, CP>(O2, base, lane, s);
        } else {
#pragma unroll
          for (int k = 0; k < kE; ++k) {
            const int64_t e = e0 + k;
            if (e < op.lo || e >= op.hi) continue;
            const float s = load1<kABf>(A, e) + load1<kBBf>(B, e);
            store1<kOBf>(O, e, s);
            if constexpr (kO2) store1<kOBf>(O2, e, s);
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Chunk copy: o[e] = a[e], bit copy of ES-byte elements in 16-byte units.
// ---------------------------------------------------------------------------
template <int ES, int UNROLL, int CP>
__global__ __launch_bounds__(kBlock) void chunk_copy(KArgs args) {
  constexpr int64_t kPerUnit = 16 / ES;
  constexpr int64_t kTile = static_cast<int64_t>(kBlock) * kPerUnit * UNROLL;
  using Elem = typename std::conditional<ES == 2, uint16_t, uint32_t>::type;
  const BlockCoord bc = block_coord();
  const DevOp op = args.ops[bc.op];
  const int64_t t_end = (op.hi + kTile - 1) / kTile;
  const char *A = src_ptr(args, op.a);
  char *O = dst_ptr(args, op.o);
  for (int64_t t = op.lo / kTile + bc.tile; t < t_end; t += bc.stride) {
    const int64_t base = t * kTile;
    if (base >= op.lo && base + kTile <= op.hi) {
      u32x4 v[UNROLL];
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        const int64_t e = base + (static_cast<int64_t>(u) * kBlock + threadIdx.x) * kPerUnit;
        v[u] = ld<u32x4>(A + e * ES);
      }
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        const uint32_t lane = (static_cast<uint32_t>(u) * kBlock + threadIdx.x) * kPerUnit;
        st_cp<CP, u32x4>(O + base * ES, lane * ES, v[u]);
      }
    } else {
      // a tile cut by the op's range: whole 16-byte units inside the op are
      // copied as units, the units it cuts element by element
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        const uint32_t lane = (static_cast<uint32_t>(u) * kBlock + threadIdx.x) * kPerUnit;
        const int64_t e0 = base + lane;
        if (e0 >= op.lo && e0 + kPerUnit <= op.hi) {
          st_cp<CP, u32x4>(O + base * ES, lane * ES, ld<u32x4>(A + e0 * ES));
        } else {
#pragma unroll
          for (int k = 0; k < kPerUnit; ++k) {
            const int64_t e = e0 + k;
            if (e < op.lo || e >= op.hi) continue;
            *reinterpret_cast<Elem *>(O + e * ES) = *reinterpret_cast<const Elem *>(A + e * ES);
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// One-pass folds: read every rank once, fold in registers in the schedule's
// order, write the finished value to every rank.
// ---------------------------------------------------------------------------

// Loads the 4-element unit at e of rank r for each of UNROLL slots.
template <bool BF, int UNROLL>
__device__ __forceinline__ void load_units(const KArgs &args, int r, int64_t base, float4 (&x)[UNROLL]) {
  const char *p = static_cast<const char *>(args.rank[r]);
#pragma unroll
  for (int u = 0; u < UNROLL; ++u)
    x[u] = load4<BF>(p, base + (static_cast<int64_t>(u) * kOPB + threadIdx.x) * 4);
}

// Ranks a fold's result goes to: every rank, or only `owner` when it is a
// rank (a reduce-scatter keeps each range on the rank that owns it).
__device__ __forceinline__ int first_out(const KArgs &args, int owner) { return owner >= 0 ? owner : 0; }
__device__ __forceinline__ int end_out(const KArgs &args, int owner) { return owner >= 0 ? owner + 1 : args.nranks; }

template <bool BF, int UNROLL>
__device__ __forceinline__ void store_all(const KArgs &args, int64_t base, const float4 (&acc)[UNROLL], int owner) {
  const int r0 = first_out(args, owner), r1 = end_out(args, owner);
  if constexpr (BF) {
    u32x2 bits[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) bits[u] = pack4(acc[u]);
    for (int r = r0; r < r1; ++r) {
      char *p = static_cast<char *>(args.rank[r]);
#pragma unroll
      for (int u = 0; u < UNROLL; ++u)
        store_bits4<kCpolOnePassBF16>(p, base, (static_cast<uint32_t>(u) * kOPB + threadIdx.x) * 4, bits[u]);
    }
  } else {
    for (int r = r0; r < r1; ++r) {
      char *p = static_cast<char *>(args.rank[r]);
#pragma unroll
      for (int u = 0; u < UNROLL; ++u)
        store4<false, kCpolOnePassF32>(p, base, (static_cast<uint32_t>(u) * kOPB + threadIdx.x) * 4, acc[u]);
    }
  }
}

// acc (+)= x_r for r = first, first+1, ... (count ranks, wrapping at `wrap_n`
// inside the block of ranks starting at `rank0`), kFB ranks' loads in flight
// at a time; the adds stay in order.
template <bool BF, bool EACH, int UNROLL, int kFB>
__device__ __forceinline__ void ring_fold_units(const KArgs &args, int rank0, int wrap_n, int first, int count,
                                                int64_t base, float4 (&acc)[UNROLL], bool init) {
  int r = first;
  int t = 0;
  if (init) {
    load_units<BF, UNROLL>(args, rank0 + r, base, acc);
    r = (r + 1 == wrap_n) ? 0 : r + 1;
    t = 1;
  }
  // kFB: ranks whose loads are in flight together
  for (; t + kFB <= count; t += kFB) {
    float4 x[kFB][UNROLL];
    int rr[kFB];
    rr[0] = r;
#pragma unroll
    for (int q = 1; q < kFB; ++q) rr[q] = (rr[q - 1] + 1 == wrap_n) ? 0 : rr[q - 1] + 1;
#pragma unroll
    for (int q = 0; q < kFB; ++q) load_units<BF, UNROLL>(args, rank0 + rr[q], base, x[q]);
#pragma unroll
    for (int q = 0; q < kFB; ++q)
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) acc[u] = fold4<EACH>(acc[u], x[q][u]);
    r = (rr[kFB - 1] + 1 == wrap_n) ? 0 : rr[kFB - 1] + 1;
  }
  const int rem = count - t;  // fewer than kFB ranks left: one predicated batch
  if (rem > 0) {
    float4 x[kFB][UNROLL];
#pragma unroll
    for (int q = 0; q + 1 < kFB; ++q)
      if (q < rem) {
        load_units<BF, UNROLL>(args, rank0 + r, base, x[q]);
        r = (r + 1 == wrap_n) ? 0 : r + 1;
      }
#pragma unroll
    for (int q = 0; q + 1 < kFB; ++q)
      if (q < rem) {
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) acc[u] = fold4<EACH>(acc[u], x[q][u]);
      }
  }
}

__device__ __forceinline__ float ring_fold1(const KArgs &args, bool bf, bool each, int rank0, int wrap_n,
                                            int first, int count, int64_t e) {
  auto ld = [&](int r) {
    const char *p = static_cast<const char *>(args.rank[rank0 + r]);
    return bf ? load1<true>(p, e) : load1<false>(p, e);
  };
  // ranks are loaded 8 at a time (independent loads in flight), then folded
  // in order
  int r = first;
  float acc = 0.0f;
  for (int t = 0; t < count; t += 8) {
    float x[8];
#pragma unroll
    for (int q = 0; q < 8; ++q)
      if (t + q < count) {
        x[q] = ld(r);
        r = (r + 1 == wrap_n) ? 0 : r + 1;
      }
#pragma unroll
    for (int q = 0; q < 8; ++q)
      if (t + q < count) acc = (t + q == 0) ? x[q] : fold1(each, acc, x[q]);
  }
  return acc;
}

__device__ __forceinline__ void store_all1(const KArgs &args, bool bf, int64_t e, float v, int owner) {
  for (int r = first_out(args, owner); r < end_out(args, owner); ++r) {
    char *p = static_cast<char *>(args.rank[r]);
    if (bf) store1<true>(p, e, v);
    else store1<false>(p, e, v);
  }
}

// Ring: element in chunk c is ((x_c + x_{c+1}) + ...) + x_{c+N-1}; aux = c.
template <bool BF, bool EACH, int UNROLL, int FB>
__global__ __launch_bounds__(kOPB) void onepass_ring(KArgs args) {
  constexpr int64_t kTile = static_cast<int64_t>(kOPB) * 4 * UNROLL;
  const BlockCoord bc = block_coord();
  const DevOp op = args.ops[bc.op];
  const int64_t t_end = (op.hi + kTile - 1) / kTile;
  for (int64_t t = op.lo / kTile + bc.tile; t < t_end; t += bc.stride) {
    const int64_t base = t * kTile;
    const int n = args.nranks;
    if (base >= op.lo && base + kTile <= op.hi) {
      float4 acc[UNROLL];
      ring_fold_units<BF, EACH, UNROLL, FB>(args, 0, n, op.aux, n, base, acc, true);
      store_all<BF, UNROLL>(args, base, acc, op.o);
    } else {
      // a partial tile: 4-element units inside the op take the vector fold,
      // the units it cuts take the per-element one
      for (int u = 0; u < UNROLL; ++u) {
        const int64_t ubase = base + static_cast<int64_t>(u) * kOPB * 4;
        const int64_t e0 = ubase + static_cast<int64_t>(threadIdx.x) * 4;
        if (e0 >= op.lo && e0 + 4 <= op.hi) {
          float4 acc[1];
          ring_fold_units<BF, EACH, 1, FB>(args, 0, n, op.aux, n, ubase, acc, true);
          store_all<BF, 1>(args, ubase, acc, op.o);
          continue;
        }
        for (int k = 0; k < 4; ++k) {
          const int64_t e = e0 + k;
          if (e < op.lo || e >= op.hi) continue;
          store_all1(args, BF, e, ring_fold1(args, BF, EACH, 0, n, op.aux, n, e), op.o);
        }
      }
    }
  }
}

// Hierarchical: group partial of slice k, ((x_{g,k+1} + x_{g,k+2}) + ...) +
// x_{g,k}; sub-chunk j folds the group partials P_j + P_{j+1} + ... in ring
// order.  aux = ((k + 1) mod G) | (j << 8).
template <bool BF, bool EACH, int UNROLL, int FB>
__global__ __launch_bounds__(kOPB) void onepass_hier(KArgs args) {
  constexpr int64_t kTile = static_cast<int64_t>(kOPB) * 4 * UNROLL;
  const BlockCoord bc = block_coord();
  const DevOp op = args.ops[bc.op];
  const int64_t t_end = (op.hi + kTile - 1) / kTile;
  for (int64_t t = op.lo / kTile + bc.tile; t < t_end; t += bc.stride) {
    const int64_t base = t * kTile;
    const int G = args.group_size, M = args.nranks / G;
    const int lstart = op.aux & 0xff, j = op.aux >> 8;
    if (base >= op.lo && base + kTile <= op.hi) {
      float4 acc[UNROLL];
      int g = j;
      for (int m = 0; m < M; ++m) {
        float4 part[UNROLL];
        ring_fold_units<BF, EACH, UNROLL, FB>(args, g * G, G, lstart, G, base, part, true);
        if (m == 0) {
#pragma unroll
          for (int u = 0; u < UNROLL; ++u) acc[u] = part[u];
        } else {
#pragma unroll
          for (int u = 0; u < UNROLL; ++u) acc[u] = fold4<EACH>(acc[u], part[u]);
        }
        g = (g + 1 == M) ? 0 : g + 1;
      }
      store_all<BF, UNROLL>(args, base, acc, op.o);
    } else {
      // a partial tile: 4-element units inside the op take the vector fold,
      // the units it cuts take the per-element one
      for (int u = 0; u < UNROLL; ++u) {
        const int64_t ubase = base + static_cast<int64_t>(u) * kOPB * 4;
        const int64_t e0 = ubase + static_cast<int64_t>(threadIdx.x) * 4;
        if (e0 >= op.lo && e0 + 4 <= op.hi) {
          float4 acc[1];
          int g = j;
          for (int m = 0; m < M; ++m) {
            float4 part[1];
            ring_fold_units<BF, EACH, 1, FB>(args, g * G, G, lstart, G, ubase, part, true);
            acc[0] = (m == 0) ? part[0] : fold4<EACH>(acc[0], part[0]);
            g = (g + 1 == M) ? 0 : g + 1;
          }
          store_all<BF, 1>(args, ubase, acc, op.o);
          continue;
        }
        for (int k = 0; k < 4; ++k) {
          const int64_t e = e0 + k;
          if (e < op.lo || e >= op.hi) continue;
          float acc = 0.f;
          int g = j;
          for (int m = 0; m < M; ++m) {
            const float part = ring_fold1(args, BF, EACH, g * G, G, lstart, G, e);
            acc = (m == 0) ? part : fold1(EACH, acc, part);
            g = (g + 1 == M) ? 0 : g + 1;
          }
          store_all1(args, BF, e, acc, op.o);
        }
      }
    }
  }
}

// Tree fold over ranks in index order: blocks of 2^k ranks merge pairwise,
// a block without a right neighbour (ranks >= N) is carried up unchanged.
// For N = 2^L this is the balanced tree of Rabenseifner and recursive
// doubling; otherwise it is the binomial tree's left-complete order.  Formed
// batch by batch (8 ranks at a time); NMAX = N rounded up to a power of two.
// The balanced tree over the ranks in index order, folded as a binary
// counter: leaf r joins, from the nearest outward, the sums of the complete
// aligned blocks that end just before it -- one per trailing one bit of r --
// and the joined block waits in slot k (k = the number of those bits) for
// its right sibling; after leaf NMAX - 1 slot log2(NMAX) holds the root.
// Only log2(NMAX) partial sums are live at a time and every slot index is a
// compile-time constant, so the slots stay in registers.
//
// For N below the power of two NMAX the leaves N .. NMAX-1 are -0, the
// exact identity of IEEE addition (x + -0 = x for every x, signed zeros
// included, and x is already a bf16 value where each add is rounded): a
// block of padding sums to -0 and a block with a valid prefix sums to that
// prefix's subtree, which gives exactly the binomial (left-complete) tree --
// neighbours paired level by level, an unpaired last node carried up.
template <bool EACH, int L, int UNROLL>
__device__ __forceinline__ void tree_push(float4 (&slot)[L + 1][UNROLL], int r, float4 (&x)[UNROLL]) {
#pragma unroll
  for (int k = 0; k <= L; ++k) {
    if ((r >> k) & 1) {
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) x[u] = fold4<EACH>(slot[k][u], x[u]);
    } else {
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) slot[k][u] = x[u];
      return;
    }
  }
}

template <bool EACH, int L>
__device__ __forceinline__ void tree_push1(float (&slot)[L + 1], int r, float x) {
#pragma unroll
  for (int k = 0; k <= L; ++k) {
    if ((r >> k) & 1) {
      x = fold1(EACH, slot[k], x);
    } else {
      slot[k] = x;
      return;
    }
  }
}

constexpr int ilog2(int v) { return v <= 1 ? 0 : 1 + ilog2(v / 2); }

// Makes v's value materialise here (an empty asm that reads and writes it).
__device__ __forceinline__ void pin(float4 &v) {
  asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w));
}

// Calls f(std::integral_constant<int, i>) for i = 0 .. N-1: a loop whose
// index is a compile-time constant in every body, however large the body
// (a long unrolled loop may otherwise stay a loop, and arrays indexed by its
// counter then leave registers).
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F &&f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// One-pass tree fold; NMAX (a power of two) >= args.nranks > NMAX / 2, and
// PAD = (args.nranks < NMAX).  kB ranks' loads are in flight at a time;
// padding leaves load nothing.
template <bool BF, bool EACH, int NMAX, bool PAD, int UNROLL, int kB>
__global__ __launch_bounds__(kOPB) void onepass_tree(KArgs args) {
  constexpr int L = ilog2(NMAX);
  constexpr int kBatch = NMAX < kB ? NMAX : kB;
  constexpr int64_t kTile = static_cast<int64_t>(kOPB) * 4 * UNROLL;
  const int n = args.nranks;
  const BlockCoord bc = block_coord();
  const DevOp op = args.ops[bc.op];
  const int64_t t_end = (op.hi + kTile - 1) / kTile;
  for (int64_t t = op.lo / kTile + bc.tile; t < t_end; t += bc.stride) {
    const int64_t base = t * kTile;
    if (base >= op.lo && base + kTile <= op.hi) {
      float4 slot[L + 1][UNROLL];
      static_for<NMAX / kBatch>([&](auto bic) {
        constexpr int bi = decltype(bic)::value;
        float4 v[kBatch][UNROLL];
        if (!PAD || (bi + 1) * kBatch <= NMAX / 2 || (bi + 1) * kBatch <= n) {
#pragma unroll
          for (int q = 0; q < kBatch; ++q) load_units<BF, UNROLL>(args, bi * kBatch + q, base, v[q]);
        } else if (bi * kBatch < n) {
          // the batch holding leaf n
#pragma unroll
          for (int q = 0; q < kBatch; ++q) {
            if (bi * kBatch + q < n) {
              load_units<BF, UNROLL>(args, bi * kBatch + q, base, v[q]);
            } else {
#pragma unroll
              for (int u = 0; u < UNROLL; ++u) v[q][u] = make_float4(-0.0f, -0.0f, -0.0f, -0.0f);
            }
          }
        } else {  // all padding: nothing to load
#pragma unroll
          for (int q = 0; q < kBatch; ++q)
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) v[q][u] = make_float4(-0.0f, -0.0f, -0.0f, -0.0f);
        }
#pragma unroll
        for (int q = 0; q < kBatch; ++q) tree_push<EACH, L, UNROLL>(slot, bi * kBatch + q, v[q]);
        // Finish this batch's adds before the next batch's loads: the live
        // partial sums (one per set bit of the leaves done) are pinned here,
        // and no load moves above this point.  Otherwise the compiler issues
        // all NMAX loads first and every leaf stays live in registers.
#pragma unroll
        for (int j = 0; j <= L; ++j)
          if ((((bi + 1) * kBatch) >> j) & 1)
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) pin(slot[j][u]);
        __builtin_amdgcn_sched_barrier(0);
      });
      store_all<BF, UNROLL>(args, base, slot[L], op.o);
    } else {
      for (int u = 0; u < UNROLL; ++u)
        for (int k = 0; k < 4; ++k) {
          const int64_t e = base + (static_cast<int64_t>(u) * kOPB + threadIdx.x) * 4 + k;
          if (e < op.lo || e >= op.hi) continue;
          float slot[L + 1];
#pragma unroll
          for (int r = 0; r < NMAX; ++r)
            tree_push1<EACH, L>(slot, r, r < n ? load1<BF>(static_cast<const char *>(args.rank[r]), e) : -0.0f);
          store_all1(args, BF, e, slot[L], op.o);
        }
    }
  }
}

// Double binary tree, one half per op (aux = 0: tree 1, 1: its mirror).
// D(c, b) = (x_c + D(c - b/2, b/2)) + D(c + b/2, b/2), D(c, 1) = x_c; tree 1
// gives x_0 + D(N/2, N/2), tree 2 gives x_{N-1} + D(N/2 - 1, N/2).
template <bool BF, bool EACH, int UNROLL, int C, int B>
struct DTreeFold {
  static __device__ __forceinline__ void run(const KArgs &args, int64_t base, float4 (&out)[UNROLL]) {
    load_units<BF, UNROLL>(args, C, base, out);
    if constexpr (B > 1) {
      float4 lo[UNROLL], hi[UNROLL];
      DTreeFold<BF, EACH, UNROLL, C - B / 2, B / 2>::run(args, base, lo);
      DTreeFold<BF, EACH, UNROLL, C + B / 2, B / 2>::run(args, base, hi);
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) out[u] = fold4<EACH>(fold4<EACH>(out[u], lo[u]), hi[u]);
    }
  }
  static __device__ __forceinline__ float run1(const KArgs &args, int64_t e) {
    const float own = load1<BF>(static_cast<const char *>(args.rank[C]), e);
    if constexpr (B == 1) {
      return own;
    } else {
      const float lo = DTreeFold<BF, EACH, UNROLL, C - B / 2, B / 2>::run1(args, e);
      const float hi = DTreeFold<BF, EACH, UNROLL, C + B / 2, B / 2>::run1(args, e);
      return fold1(EACH, fold1(EACH, own, lo), hi);
    }
  }
};

template <bool BF, bool EACH, int N, int UNROLL>
__global__ __launch_bounds__(kOPB) void onepass_dtree(KArgs args) {
  constexpr int64_t kTile = static_cast<int64_t>(kOPB) * 4 * UNROLL;
  const BlockCoord bc = block_coord();
  const DevOp op = args.ops[bc.op];
  const bool second = op.aux != 0;
  const int64_t t_end = (op.hi + kTile - 1) / kTile;
  for (int64_t t = op.lo / kTile + bc.tile; t < t_end; t += bc.stride) {
    const int64_t base = t * kTile;
    if (base >= op.lo && base + kTile <= op.hi) {
      float4 root[UNROLL], sub[UNROLL];
      if (!second) {
        load_units<BF, UNROLL>(args, 0, base, root);
        DTreeFold<BF, EACH, UNROLL, N / 2, N / 2>::run(args, base, sub);
      } else {
        load_units<BF, UNROLL>(args, N - 1, base, root);
        DTreeFold<BF, EACH, UNROLL, N / 2 - 1, N / 2>::run(args, base, sub);
      }
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) root[u] = fold4<EACH>(root[u], sub[u]);
      store_all<BF, UNROLL>(args, base, root, op.o);
    } else {
      for (int u = 0; u < UNROLL; ++u)
        for (int k = 0; k < 4; ++k) {
          const int64_t e = base + (static_cast<int64_t>(u) * kOPB + threadIdx.x) * 4 + k;
          if (e < op.lo || e >= op.hi) continue;
          float v;
          if (!second)
            v = fold1(EACH, load1<BF>(static_cast<const char *>(args.rank[0]), e),
                      DTreeFold<BF, EACH, UNROLL, N / 2, N / 2>::run1(args, e));
          else
            v = fold1(EACH, load1<BF>(static_cast<const char *>(args.rank[N - 1]), e),
                      DTreeFold<BF, EACH, UNROLL, N / 2 - 1, N / 2>::run1(args, e));
          store_all1(args, BF, e, v, op.o);
        }
    }
  }
}

// ---------------------------------------------------------------------------
// LDS-staged one-pass folds: gather, fold, scatter.
//
// The register folds above store every finished unit into all N ranks from
// the thread that folded it, so each wave issues N stores per unit.  On
// MI355X that store pattern is the limit: 16 buffers of 192 MiB written by
// waves that store into all 16 take 0.55 ms (5.85 TB/s), written by waves
// that each store into one buffer 0.47 ms (6.8 TB/s), with the same
// addresses in flight.  Here a workgroup of min(N, W) waves (W = 16 or 8,
// lds_waves) stages one tile of every rank in LDS:
//   gather:  wave w loads the tile of ranks w, w + W, ... into LDS;
//   fold:    thread j folds 4-byte word j (1 fp32 or 2 bf16 elements) over
//            the ranks, reading LDS, in the schedule's order, and leaves the
//            finished word in rank 0's LDS slot (only thread j touches
//            column j);
//   scatter: wave w stores the finished tile into ranks w, w + W, ...
// Barriers separate the phases.  Each element is still produced by one
// thread with the same adds in the same order as the register folds, so
// the bits are the same.  A tile holds U 16-byte units per lane and rank
// (U KiB per rank; fp32 4 elements per unit, bf16 8), so the staging area is
// N * U KiB, at most 64 KiB.  Tiles that an op's range cuts (its first and
// last) skip LDS: each word inside the op folds from HBM and is stored into
// every rank, and the cut words go element by element through the same fold.
// ---------------------------------------------------------------------------
constexpr int kLdsUnits = AR_LDS_UNITS;  // 16-byte units per lane and rank in a tile, up to 32 ranks
// Store policies of the scatter, measured on MI355X (16 ranks, in-place
// calls back to back): where every rank's output fits in the 256 MB
// Infinity Cache, sc1 stores leave it there for the next reader (fp32 ring
// at 8-16 MiB per rank 50.6 -> 42.4 us and 100.2 -> 80.8 us against nt
// stores); above it nt + sc1 was fastest (192 MiB per rank: 1,023 us
// against 1,041 with nt and 1,061 with sc1).  The policy is a template
// argument: with one kernel branching on a launch flag between the two
// store loops, the balanced-tree folds ran 14% slower at 192 MiB per rank
// (1,155 against 1,010 us) for reasons the code does not show.
constexpr int kCpolLdsWarm = AR_CPOL_LDS_WARM, kCpolLdsCold = AR_CPOL_LDS_COLD;
static_assert(kLdsUnits >= 1 && kLdsUnits * 32 <= 64, "a staged tile of 32 ranks fits in 64 KiB");
// Reduce-scatter folds (kKindOwner: each op's result goes to its owner only)
// of 9 to 16 ranks in 16-wave workgroups (one rank per wave) stage 4 units
// per lane and rank, 64 KiB at 16 ranks: each wave's gather reads 4 KiB runs
// of its rank, and the scatter is one store per tile.  Measured on MI355X at
// 16 x 192 MiB: ring fp32 590 -> 531 us, bf16 626 -> 539, hierarchical 2 x 8
// fp32 647 -> 558, Rabenseifner fp32 578 -> 530; hierarchical 4 x 3 bf16 at
// 96 MiB 284 -> 225.  With 8-wave workgroups (two ranks per wave: bf16
// rounded at each add, the bf16 balanced tree) 4 units were 4-6% slower, at
// 8 ranks within 3% either way.  The all-reduce folds, whose scatter stores
// into every rank, were 5-22% slower with 4 units.
constexpr int kLdsUnitsOwner = 4;
static_assert(kLdsUnitsOwner * 16 <= 64, "a reduce-scatter tile of 16 ranks fits in 64 KiB");

// Size classes by rank count (up to 16, 32 or 64 ranks): units per lane and
// rank in a tile, and the ranks one of W waves gathers and scatters at most.
constexpr int lds_class(int n) { return n <= 16 ? 16 : n <= 32 ? 32 : 64; }
template <int NC, int W>
struct LdsClass {
  static constexpr int kU = NC > 32 ? 1 : kLdsUnits;
  static constexpr int kRanksPerWave = (NC + W - 1) / W;
};

// 16-byte units: fp32 4 elements, bf16 8.
template <bool BF>
struct Unit16 {
  static constexpr int kE = BF ? 8 : 4;   // elements per unit
  static constexpr int kES = BF ? 2 : 4;  // bytes per element
};

// Packets a fold adds: an fp32 word (1 element) or a bf16 word (2), element
// by element with fold1's rule.
template <bool EACH>
__device__ __forceinline__ float fold_p(float a, float b) { return fold1(EACH, a, b); }
template <bool EACH>
__device__ __forceinline__ float2 fold_p(float2 a, float2 b) {
  return make_float2(fold1(EACH, a.x, b.x), fold1(EACH, a.y, b.y));
}
__device__ __forceinline__ void set_neg_zero(float &p) { p = -0.0f; }
__device__ __forceinline__ void set_neg_zero(float2 &p) { p = make_float2(-0.0f, -0.0f); }
__device__ __forceinline__ void pin(float &v) { asm volatile("" : "+v"(v)); }
__device__ __forceinline__ void pin(float2 &v) { asm volatile("" : "+v"(v.x), "+v"(v.y)); }

// Sources of a fold, each giving rank r's packet: word j of the staged tile
// (LDS), the word at element e of the rank buffer (HBM), element e (HBM).
template <bool BF>
__device__ __forceinline__ std::conditional_t<BF, float2, float> word_value(uint32_t w) {
  if constexpr (BF) return make_float2(widen(w & 0xffffu), widen(w >> 16));
  else return __uint_as_float(w);
}
template <bool BF>
struct StagedWord {
  using P = std::conditional_t<BF, float2, float>;
  const uint32_t *words;
  int per_rank;  // words per rank in the tile
  int j;
  __device__ __forceinline__ P operator()(int r) const { return word_value<BF>(words[r * per_rank + j]); }
};
template <bool BF>
struct HbmWord {
  using P = std::conditional_t<BF, float2, float>;
  const KArgs &a;
  int64_t e;
  __device__ __forceinline__ P operator()(int r) const {
    return word_value<BF>(*reinterpret_cast<const uint32_t *>(static_cast<const char *>(a.rank[r]) + e * (BF ? 2 : 4)));
  }
};
template <bool BF>
struct HbmElem {
  using P = float;
  const KArgs &a;
  int64_t e;
  __device__ __forceinline__ float operator()(int r) const { return load1<BF>(static_cast<const char *>(a.rank[r]), e); }
};

// Final bits of a word (bf16: rounded once, to nearest even).
__device__ __forceinline__ uint32_t word_bits(float v) { return __float_as_uint(v); }
__device__ __forceinline__ uint32_t word_bits(float2 v) { return narrow(v.x) | (narrow(v.y) << 16); }

// acc = ((x_first + x_first+1) + ...) over `count` ranks of the block of
// ranks starting at rank0, wrapping at wrap_n; four ranks' packets are read
// together, then added in order.
template <bool EACH, class Src>
__device__ __forceinline__ void ring_fold_src(const Src &src, int rank0, int wrap_n, int first, int count,
                                              typename Src::P &acc) {
  using P = typename Src::P;
  constexpr int kB = 4;
  int r = first;
  acc = src(rank0 + r);
  int t = 1;
  for (; t + kB <= count; t += kB) {
    P x[kB];
#pragma unroll
    for (int q = 0; q < kB; ++q) {
      r = (r + 1 == wrap_n) ? 0 : r + 1;
      x[q] = src(rank0 + r);
    }
#pragma unroll
    for (int q = 0; q < kB; ++q) acc = fold_p<EACH>(acc, x[q]);
  }
  for (; t < count; ++t) {
    r = (r + 1 == wrap_n) ? 0 : r + 1;
    acc = fold_p<EACH>(acc, src(rank0 + r));
  }
}

// The schedules' folds of one packet, in the orders of the register kernels
// above (op.aux as there).
struct RingFold {
  static constexpr int kClassMin = 16;
  static constexpr bool kBalancedTree = false;
  static constexpr bool kHalves = true;  // a reduce-scatter plan's fold too
  static constexpr int kTileUnits = 0;  // the size class's units per lane and rank
  template <bool EACH, class Src>
  static __device__ __forceinline__ void run(const KArgs &a, const DevOp &op, const Src &src, typename Src::P &acc) {
    ring_fold_src<EACH>(src, 0, a.nranks, op.aux, a.nranks, acc);
  }
};

struct HierFold {
  static constexpr int kClassMin = 16;
  static constexpr bool kBalancedTree = false;
  static constexpr bool kHalves = true;
  static constexpr int kTileUnits = 0;
  template <bool EACH, class Src>
  static __device__ __forceinline__ void run(const KArgs &a, const DevOp &op, const Src &src, typename Src::P &acc) {
    const int G = a.group_size, M = a.nranks / G;
    const int lstart = op.aux & 0xff;
    int g = op.aux >> 8;
    ring_fold_src<EACH>(src, g * G, G, lstart, G, acc);
    for (int m = 1; m < M; ++m) {
      g = (g + 1 == M) ? 0 : g + 1;
      typename Src::P part;
      ring_fold_src<EACH>(src, g * G, G, lstart, G, part);
      acc = fold_p<EACH>(acc, part);
    }
  }
};

// Balanced tree over NMAX leaves in index order, folded as the binary
// counter of tree_push (leaf r joins, from the nearest outward, the complete
// aligned blocks that end just before it; the joined block waits in slot k
// for its right sibling); leaves n .. NMAX - 1 are -0 when PAD.  Leaves come
// in batches of 4 whose adds finish (the live partial sums pinned) before
// the next batch's reads, so few packets are live at a time.
template <bool EACH, int L, class P>
__device__ __forceinline__ void tree_push_p(P (&slot)[L + 1], int r, P x) {
#pragma unroll
  for (int k = 0; k <= L; ++k) {
    if ((r >> k) & 1) {
      x = fold_p<EACH>(slot[k], x);
    } else {
      slot[k] = x;
      return;
    }
  }
}

template <int NMAX, bool PAD>
struct TreeFold {
  static constexpr int kClassMin = NMAX;
  static constexpr bool kBalancedTree = true;
  static constexpr bool kHalves = true;
  static constexpr int kTileUnits = 0;
  template <bool EACH, class Src>
  static __device__ __forceinline__ void run(const KArgs &a, const DevOp &, const Src &src, typename Src::P &acc) {
    using P = typename Src::P;
    constexpr int L = ilog2(NMAX), kB = NMAX < 4 ? NMAX : 4;
    P slot[L + 1];
    static_for<NMAX / kB>([&](auto bic) {
      constexpr int bi = decltype(bic)::value;
      P x[kB];
#pragma unroll
      for (int q = 0; q < kB; ++q) {
        if (!PAD || bi * kB + q < a.nranks) x[q] = src(bi * kB + q);
        else set_neg_zero(x[q]);
      }
#pragma unroll
      for (int q = 0; q < kB; ++q) tree_push_p<EACH, L>(slot, bi * kB + q, x[q]);
#pragma unroll
      for (int j = 0; j <= L; ++j)
        if ((((bi + 1) * kB) >> j) & 1) pin(slot[j]);
      __builtin_amdgcn_sched_barrier(0);
    });
    acc = slot[L];
  }
};

// Double binary tree: D(c, b) = (x_c + D(c - b/2, b/2)) + D(c + b/2, b/2).
// x_c + D(c - b/2, b/2) is formed before the right subtree starts, so one
// packet per level is live.  (Pinning finished subtrees as the balanced tree
// does made the compiler spill at 32 and 64 ranks.)
template <bool EACH, int C, int B>
struct DTreeSrc {
  template <class Src>
  static __device__ __forceinline__ void run(const Src &src, typename Src::P &out) {
    out = src(C);
    if constexpr (B > 1) {
      typename Src::P sub;
      DTreeSrc<EACH, C - B / 2, B / 2>::run(src, sub);
      out = fold_p<EACH>(out, sub);
      DTreeSrc<EACH, C + B / 2, B / 2>::run(src, sub);
      out = fold_p<EACH>(out, sub);
    }
  }
};
// op.aux = 0: tree 1, x_0 + D(N/2, N/2); 1: tree 2, x_{N-1} + D(N/2 - 1, N/2).
template <int N>
struct DTreeFoldOp {
  static constexpr int kClassMin = N;
  static constexpr bool kBalancedTree = false;
  static constexpr bool kHalves = false;
  static constexpr int kTileUnits = 0;
  template <bool EACH, class Src>
  static __device__ __forceinline__ void run(const KArgs &, const DevOp &op, const Src &src, typename Src::P &acc) {
    typename Src::P sub;
    if (op.aux == 0) {
      acc = src(0);
      DTreeSrc<EACH, N / 2, N / 2>::run(src, sub);
    } else {
      acc = src(N - 1);
      DTreeSrc<EACH, N / 2 - 1, N / 2>::run(src, sub);
    }
    acc = fold_p<EACH>(acc, sub);
  }
};

// NC: rank-count size class, W: waves per workgroup at most (LdsClass); CP:
// the scatter's store policy (kCpolLdsWarm or kCpolLdsCold); F: the fold,
// whose kTileUnits (unless 0) replaces the class's units per lane and rank.
template <bool BF, bool EACH, int NC, int W, int CP, class F>
__global__ __launch_bounds__(64 * W) void onepass_lds(KArgs args) {
  using U16 = Unit16<BF>;
  constexpr int kE = U16::kE, kES = U16::kES;
  constexpr int U = F::kTileUnits > 0 ? F::kTileUnits : LdsClass<NC, W>::kU;
  constexpr int kRPW = LdsClass<NC, W>::kRanksPerWave;
  constexpr int kUnits = 64 * U;                                // units per rank in a tile
  constexpr int kWords = kUnits * 4;                            // 4-byte words per rank in a tile
  constexpr int64_t kTile = static_cast<int64_t>(kUnits) * kE;  // elements
  extern __shared__ u32x4 stage[];                              // [nranks][kUnits]
  const int n = args.nranks;
  const int waves = static_cast<int>(blockDim.x >> 6);
  // the wave index is uniform across the wave: with it in a scalar register
  // the rank pointers come from scalar loads of the kernel arguments
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int lane = static_cast<int>(threadIdx.x & 63);
  const BlockCoord bc = block_coord();
  const DevOp op = args.ops[bc.op];
  const int64_t t_end = (op.hi + kTile - 1) / kTile;
  for (int64_t t = op.lo / kTile + bc.tile; t < t_end; t += bc.stride) {
    const int64_t base = t * kTile;
    if (base >= op.lo && base + kTile <= op.hi) {
      // gather: every load of this wave in flight before the LDS writes
      u32x4 x[kRPW][U];
#pragma unroll
      for (int k = 0; k < kRPW; ++k) {
        const int r = wave + k * waves;
        if (r < n) {
          const char *p = static_cast<const char *>(args.rank[r]) + base * kES;
#pragma unroll
          for (int u = 0; u < U; ++u) x[k][u] = ld<u32x4>(p + (u * 64 + lane) * 16);
        }
      }
#pragma unroll
      for (int k = 0; k < kRPW; ++k) {
        const int r = wave + k * waves;
        if (r < n) {
#pragma unroll
          for (int u = 0; u < U; ++u) stage[r * kUnits + u * 64 + lane] = x[k][u];
        }
      }
      __syncthreads();
      // fold: word j (4 bytes: 1 fp32 or 2 bf16 elements) of every rank,
      // in the schedule's order, one thread per word
      {
        uint32_t *words = reinterpret_cast<uint32_t *>(stage);
        for (int j = static_cast<int>(threadIdx.x); j < kWords; j += static_cast<int>(blockDim.x)) {
          typename StagedWord<BF>::P acc;
          F::template run<EACH>(args, op, StagedWord<BF>{words, kWords, j}, acc);
          words[j] = word_bits(acc);
        }
      }
      __syncthreads();
      // scatter
      u32x4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = stage[u * 64 + lane];
#pragma unroll
      for (int k = 0; k < kRPW; ++k) {
        const int r = wave + k * waves;
        if (r < n && (op.o < 0 || r == op.o)) {
          char *p = static_cast<char *>(args.rank[r]) + base * kES;
#pragma unroll
          for (int u = 0; u < U; ++u) st_cp<CP, u32x4>(p, static_cast<uint32_t>(u * 64 + lane) * 16, v[u]);
        }
      }
      // the next tile's gather overwrites rank 0's slot, which the scatter
      // just read
      if (t + bc.stride < t_end) __syncthreads();
    } else {
      // a tile the op's range cuts: words inside the op fold from HBM and go
      // to every rank; the words it cuts go element by element
      constexpr int kWE = kE / 4;  // elements per word
      for (int j = static_cast<int>(threadIdx.x); j < kWords; j += static_cast<int>(blockDim.x)) {
        const int64_t e0 = base + static_cast<int64_t>(j) * kWE;
        if (e0 >= op.lo && e0 + kWE <= op.hi) {
          typename HbmWord<BF>::P acc;
          F::template run<EACH>(args, op, HbmWord<BF>{args, e0}, acc);
          const uint32_t bits = word_bits(acc);
          for (int r = first_out(args, op.o); r < end_out(args, op.o); ++r)
            *reinterpret_cast<uint32_t *>(static_cast<char *>(args.rank[r]) + e0 * kES) = bits;
          continue;
        }
        for (int k = 0; k < kWE; ++k) {
          const int64_t e = e0 + k;
          if (e < op.lo || e >= op.hi) continue;
          float acc;
          F::template run<EACH>(args, op, HbmElem<BF>{args, e}, acc);
          store_all1(args, BF, e, acc, op.o);
        }
      }
    }
  }
}

// Step kernels come in two shapes: 2 units per thread, and 1 unit per thread
// (more waves in flight).  The 1-unit shape is faster (measured on MI355X)
// for launches that write more into rank buffers than the 256 MB Infinity
// Cache holds, so that the next step streams from DRAM; the 2-unit shape is
// faster for smaller launches, whose inputs the previous step left in the
// cache (checked again with the sc1 store policy).
constexpr int kUnrollWarm = AR_REDUCE_UNROLL;
constexpr int kUnrollCold = AR_COLD_UNROLL;
// Units per thread of a reduce kind: with every operand bf16 (flags 7, 15) a
// unit is 8 bytes, half an fp32 unit, so twice the units keep as many bytes
// in flight (bf16 rounded at each add, ring 16 x 192 MiB 2.13 -> 2.09 ms,
// 64 ranks 2.52 -> 2.48 ms).
// With 8-element units (a bf16 operand) half as many units keep the same
// elements per thread.
constexpr int reduce_unroll(int flags, bool cold) {
  const int u = (flags & 7) == 7 ? (cold ? AR_COLD_UNROLL_BF16 : AR_REDUCE_UNROLL_BF16) : (cold ? kUnrollCold : kUnrollWarm);
  const int per = reduce_unit_elems(flags) / 4;
  return u / per > 0 ? u / per : 1;
}
// one-pass shapes per dtype (measured): fp32 2 units x 8 ranks in flight,
// bf16 1 unit x 16 ranks
constexpr int kOnePassUnrollF32 = AR_ONEPASS_UNROLL_F32, kFoldBatchF32 = AR_FOLD_BATCH_F32;
constexpr int kOnePassUnrollBF16 = AR_ONEPASS_UNROLL_BF16, kFoldBatchBF16 = AR_FOLD_BATCH_BF16;
// The hierarchical fold runs a ring fold per group (typically 8 ranks): a
// batch wider than the group only adds predicated slots (16 -> 8: bf16 2x8
// at 16 x 192 MiB 1.21 -> 1.12 ms, 64 ranks 1.36 -> 1.26 ms).
constexpr int kFoldBatchHierBF16 = AR_FOLD_BATCH_HIER_BF16;
// tree folds (measured): fp32 2 units x 8 ranks in flight, bf16 1 unit x 16
// ranks (they also hold log2 N partial sums)
constexpr int kTreeUnrollF32 = AR_TREE_UNROLL_F32, kTreeBatchF32 = AR_TREE_BATCH_F32;
constexpr int kTreeUnrollBF16 = AR_TREE_UNROLL_BF16, kTreeBatchBF16 = AR_TREE_BATCH_BF16;
constexpr int kCpolRank = AR_CPOL_RANK;
constexpr int kCpolScratch = AR_CPOL_SCRATCH;

template <int FLAGS, int U>
hipError_t launch_reduce_u(dim3 grid, const KArgs &a, hipStream_t s, bool out_scratch) {
  if (out_scratch)
    AR_LAUNCH((chunk_reduce<FLAGS, U, kCpolScratch>), grid, dim3(kBlock), 0, s, a);
  else
    AR_LAUNCH((chunk_reduce<FLAGS, U, kCpolRank>), grid, dim3(kBlock), 0, s, a);
  return hipGetLastError();
}

template <int FLAGS>
hipError_t launch_reduce(dim3 grid, const KArgs &a, hipStream_t s, bool out_scratch, bool cold) {
  return cold ? launch_reduce_u<FLAGS, reduce_unroll(FLAGS, true)>(grid, a, s, out_scratch)
              : launch_reduce_u<FLAGS, reduce_unroll(FLAGS, false)>(grid, a, s, out_scratch);
}

template <int ES>
hipError_t launch_copy(dim3 grid, const KArgs &a, hipStream_t s, bool cold) {
  if (cold) AR_LAUNCH((chunk_copy<ES, kUnrollCold, kCpolRank>), grid, dim3(kBlock), 0, s, a);
  else AR_LAUNCH((chunk_copy<ES, kUnrollWarm, kCpolRank>), grid, dim3(kBlock), 0, s, a);
  return hipGetLastError();
}

template <bool BF, bool EACH>
hipError_t launch_tree(int n, dim3 grid, const KArgs &a, hipStream_t s) {
  constexpr int U = BF ? kTreeUnrollBF16 : kTreeUnrollF32;
  constexpr int B = BF ? kTreeBatchBF16 : kTreeBatchF32;
  switch (n) {
    case 2: AR_LAUNCH((onepass_tree<BF, EACH, 2, false, U, B>), grid, dim3(kOPB), 0, s, a); break;
    case 4: AR_LAUNCH((onepass_tree<BF, EACH, 4, false, U, B>), grid, dim3(kOPB), 0, s, a); break;
    case 8: AR_LAUNCH((onepass_tree<BF, EACH, 8, false, U, B>), grid, dim3(kOPB), 0, s, a); break;
    case 16: AR_LAUNCH((onepass_tree<BF, EACH, 16, false, U, B>), grid, dim3(kOPB), 0, s, a); break;
    case 32: AR_LAUNCH((onepass_tree<BF, EACH, 32, false, U, B>), grid, dim3(kOPB), 0, s, a); break;
    case 64: AR_LAUNCH((onepass_tree<BF, EACH, 64, false, U, B>), grid, dim3(kOPB), 0, s, a); break;
    default:
      if (n == 3) AR_LAUNCH((onepass_tree<BF, EACH, 4, true, U, B>), grid, dim3(kOPB), 0, s, a);
      else if (n < 8) AR_LAUNCH((onepass_tree<BF, EACH, 8, true, U, B>), grid, dim3(kOPB), 0, s, a);
      else if (n < 16) AR_LAUNCH((onepass_tree<BF, EACH, 16, true, U, B>), grid, dim3(kOPB), 0, s, a);
      else if (n < 32) AR_LAUNCH((onepass_tree<BF, EACH, 32, true, U, B>), grid, dim3(kOPB), 0, s, a);
      else if (n < 64) AR_LAUNCH((onepass_tree<BF, EACH, 64, true, U, B>), grid, dim3(kOPB), 0, s, a);
      else return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <bool BF, bool EACH>
hipError_t launch_dtree(int n, dim3 grid, const KArgs &a, hipStream_t s) {
  constexpr int U = BF ? kOnePassUnrollBF16 : kOnePassUnrollF32;
  switch (n) {
    case 2: AR_LAUNCH((onepass_dtree<BF, EACH, 2, U>), grid, dim3(kOPB), 0, s, a); break;
    case 4: AR_LAUNCH((onepass_dtree<BF, EACH, 4, U>), grid, dim3(kOPB), 0, s, a); break;
    case 8: AR_LAUNCH((onepass_dtree<BF, EACH, 8, U>), grid, dim3(kOPB), 0, s, a); break;
    case 16: AR_LAUNCH((onepass_dtree<BF, EACH, 16, U>), grid, dim3(kOPB), 0, s, a); break;
    case 32: AR_LAUNCH((onepass_dtree<BF, EACH, 32, U>), grid, dim3(kOPB), 0, s, a); break;
    case 64: AR_LAUNCH((onepass_dtree<BF, EACH, 64, U>), grid, dim3(kOPB), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// A reduce-scatter plan's fold F, staged with kLdsUnitsOwner units per lane
// and rank (9 to 16 ranks, 16-wave workgroups).
template <class F>
struct OwnerTiles : F {
  static constexpr int kTileUnits = kLdsUnitsOwner;
};

// Waves per workgroup: 16 (one rank each) for folds of up to 16 ranks in fp32
// and in bf16 with one rounding, except the balanced tree in bf16; 8 waves
// otherwise, so that more workgroups share a CU.  Measured on MI355X with
// 16 x 192 MiB, 32 x 96 MiB and 64 x 48 MiB: fp32 at 16 ranks 5.6-5.7 TB/s
// with 8 waves, 5.9-6.2 with 16; bf16 rounded at each add at 16 ranks
// 5.2-5.6 with 16, 5.6-5.8 with 8; the bf16 tree at 16 ranks 5.2 with 16,
// 5.6 with 8; above 16 ranks 8 waves were as fast or faster (up to 30% at
// 64 ranks in bf16).
int lds_waves(int32_t kind, int n) {
  const int dt = kind & 3;
  const bool tree = (kind & 0xF00) == kKindTree;
  return (n <= 16 && (dt == 0 || (dt == 1 && !tree))) ? 16 : 8;
}
int lds_threads(int32_t kind, int n) { return 64 * std::max(1, std::min(n, lds_waves(kind, n))); }

// LDS-staged folds: units per lane and rank and dynamic LDS bytes (N * U
// KiB); reduce-scatter folds of 9 to 16 ranks in 16-wave workgroups take
// kLdsUnitsOwner.
bool lds_owner_tiles(int32_t kind, int n) {
  return (kind & kKindOwner) != 0 && n > 8 && n <= 16 && lds_waves(kind, n) == 16;
}
int lds_units_of(int32_t kind, int n) {
  if (lds_owner_tiles(kind, n)) return kLdsUnitsOwner;
  return n > 32 ? LdsClass<64, 8>::kU : LdsClass<32, 8>::kU;
}
size_t lds_bytes(int32_t kind, int n) { return static_cast<size_t>(n) * 64 * lds_units_of(kind, n) * 16; }

// F::kClassMin: the smallest size class the fold's rank count may take.
// One-pass all-gather (kKindFan | element bytes): op [lo, hi) of rank op.a
// goes to every other rank.  A workgroup of W = min(N, kFanWaves) waves
// loads a 4 KiB tile of rank a into LDS, and after a barrier each wave
// stores the whole tile into one rank other than a.  Above W ranks the
// destinations are split into G = ceil(N / W) groups of W, and G
// workgroups take each tile, one per group (the owner's tile is read G
// times).  Tiles that the op's range cuts copy element by element.  CP: the
// store policy (kCpolFan).
// Measured on MI355X, ring fp32, against 32 KiB tiles each wave stored into
// N / W ranks: 514 against 618 us at 16 x 192 MiB (bf16 519 against 622),
// 258 against 314 at 8 x 192 MiB, 132 against 140 at 4 x 192 MiB, 88
// against 99 at 16 x 32 MiB, 559 against 616 at 32 x 96 MiB, and within
// 1% at 64 x 48 MiB (605 against 598; without the groups, 4 KiB tiles were
// 2-5% slower there).  2, 1 and 8 KiB tiles were slower than 4 at 16 ranks
// (604, 823 and 602 us), and so were 8 or 4 waves (595 and 607).
constexpr int kFanUnits = AR_LDS_UNITS;
constexpr int kFanWaves = 16;
constexpr int kFanTileUnits = 256;  // 16-byte units per tile
constexpr int kCpolFan = AR_CPOL_LDS_WARM;
static_assert(kFanTileUnits <= kFanWaves * kFanUnits * 64, "the tile fits the stage");
// Workgroups per tile: one per group of `waves` destination ranks.
__host__ __device__ constexpr int fan_groups_of(int n, int waves) { return n > waves ? (n + waves - 1) / waves : 1; }
template <int ES, int CP>
__global__ __launch_bounds__(64 * kFanWaves) void onepass_fan(KArgs args) {
  constexpr int kE = 16 / ES;  // elements per unit
  using E = typename std::conditional<ES == 4, uint32_t, uint16_t>::type;
  __shared__ u32x4 stage[kFanWaves * kFanUnits * 64];
  const int n = args.nranks;
  const int waves = static_cast<int>(blockDim.x >> 6);
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int lane = static_cast<int>(threadIdx.x & 63);
  constexpr int units = kFanTileUnits;
  constexpr int64_t tile = static_cast<int64_t>(units) * kE;
  const BlockCoord bc = block_coord();
  // workgroup x takes tile x / G of the op for destination group x mod G
  // (the grid is G times the tiles)
  // (32-bit: the grid holds fewer than 2^31 workgroups)
  const uint32_t groups = static_cast<uint32_t>(fan_groups_of(n, waves));
  const uint32_t x = static_cast<uint32_t>(bc.tile), gx = static_cast<uint32_t>(bc.stride);
  const int g = groups > 1 ? static_cast<int>(x % groups) : 0;
  const int64_t t0 = groups > 1 ? x / groups : x, stride = groups > 1 ? gx / groups : gx;
  const int r_lo = g * waves, r_hi = r_lo + waves < n ? r_lo + waves : n;
  const DevOp op = args.ops[bc.op];
  const char *src = static_cast<const char *>(args.rank[op.a]);
  const int64_t t_end = (op.hi + tile - 1) / tile;
  for (int64_t t = op.lo / tile + t0; t < t_end; t += stride) {
    const int64_t base = t * tile;
    if (base >= op.lo && base + tile <= op.hi) {
      const char *p = src + base * ES;
      for (int q = static_cast<int>(threadIdx.x); q < units; q += static_cast<int>(blockDim.x))
        stage[q] = ld<u32x4>(p + q * 16);
      __syncthreads();
      for (int r = r_lo + wave; r < r_hi; r += waves) {
        if (r == op.a) continue;
        char *d = static_cast<char *>(args.rank[r]) + base * ES;
        for (int q = lane; q < units; q += 64) st_cp<CP, u32x4>(d, static_cast<uint32_t>(q) * 16, stage[q]);
      }
      // the next tile's loads overwrite the stage this tile's stores read
      if (t + stride < t_end) __syncthreads();
    } else {
      const int64_t e0 = base > op.lo ? base : op.lo, e1 = base + tile < op.hi ? base + tile : op.hi;
      for (int64_t e = e0 + threadIdx.x; e < e1; e += blockDim.x) {
        const E x = *reinterpret_cast<const E *>(src + e * ES);
        for (int r = r_lo; r < r_hi; ++r)
          if (r != op.a) *reinterpret_cast<E *>(static_cast<char *>(args.rank[r]) + e * ES) = x;
      }
    }
  }
}

int fan_threads(int32_t nranks) { return 64 * std::min(std::max(nranks, 1), kFanWaves); }

// Measured at 16 ranks (32 and 192 MiB per rank): sc1 stores were 3% faster
// than nt + sc1 and 1-8% faster than plain nt at both sizes, so the fan-out
// takes them whatever its size.
template <int ES>
hipError_t launch_fan(dim3 grid, const KArgs &a, hipStream_t s) {
  AR_LAUNCH((onepass_fan<ES, kCpolFan>), grid, dim3(fan_threads(a.nranks)), 0, s, a);
  return hipGetLastError();
}

template <bool BF, bool EACH, int NC, int W, class F>
hipError_t launch_lds_cw(int32_t kind, dim3 grid, const KArgs &a, hipStream_t s) {
  constexpr int C = NC > F::kClassMin ? NC : F::kClassMin;
  using LC = LdsClass<C, W>;
  // the staging area holds U units per lane of every rank, and the waves
  // cover every rank
  const int threads = lds_threads(kind, a.nranks);
  if (a.nranks < 1 || a.nranks > C || LC::kU != lds_units_of(kind, a.nranks) || threads > 64 * W ||
      LC::kRanksPerWave * (threads / 64) < a.nranks)
    return hipErrorInvalidValue;
  const size_t lds = lds_bytes(kind, a.nranks);
  if (a.store_cold)
    AR_LAUNCH((onepass_lds<BF, EACH, C, W, kCpolLdsCold, F>), grid, dim3(threads), lds, s, a);
  else
    AR_LAUNCH((onepass_lds<BF, EACH, C, W, kCpolLdsWarm, F>), grid, dim3(threads), lds, s, a);
  return hipGetLastError();
}
// The reduce-scatter fold with its own tiles (16 waves; the store policy as
// for the other folds).
template <bool BF, bool EACH, class F>
hipError_t launch_lds_owner(int32_t kind, dim3 grid, const KArgs &a, hipStream_t s) {
  const int threads = lds_threads(kind, a.nranks);
  if (!lds_owner_tiles(kind, a.nranks) || threads > 64 * 16 ||
      LdsClass<16, 16>::kRanksPerWave * (threads / 64) < a.nranks)
    return hipErrorInvalidValue;
  const size_t lds = lds_bytes(kind, a.nranks);
  if (a.store_cold)
    AR_LAUNCH((onepass_lds<BF, EACH, 16, 16, kCpolLdsCold, OwnerTiles<F>>), grid, dim3(threads), lds, s, a);
  else
    AR_LAUNCH((onepass_lds<BF, EACH, 16, 16, kCpolLdsWarm, OwnerTiles<F>>), grid, dim3(threads), lds, s, a);
  return hipGetLastError();
}
// 16-wave workgroups exist only where lds_waves picks them (up to 16 ranks,
// fp32, or bf16 rounded once outside the balanced tree).
template <bool BF, bool EACH, int NC, class F>
hipError_t launch_lds_c(int32_t kind, dim3 grid, const KArgs &a, hipStream_t s) {
  if constexpr (NC <= 16 && F::kClassMin == 16 && F::kHalves && !EACH && !(BF && F::kBalancedTree)) {
    if (lds_owner_tiles(kind, a.nranks)) return launch_lds_owner<BF, EACH, F>(kind, grid, a, s);
  }
  if constexpr (NC <= 16 && F::kClassMin <= 16 && !EACH && !(BF && F::kBalancedTree)) {
    if (lds_waves(kind, a.nranks) == 16) return launch_lds_cw<BF, EACH, NC, 16, F>(kind, grid, a, s);
  }
  return launch_lds_cw<BF, EACH, NC, 8, F>(kind, grid, a, s);
}

template <bool BF, bool EACH, class F>
hipError_t launch_lds_n(int32_t kind, dim3 grid, const KArgs &a, hipStream_t s) {
  switch (lds_class(a.nranks)) {
    case 16: return launch_lds_c<BF, EACH, 16, F>(kind, grid, a, s);
    case 32: return launch_lds_c<BF, EACH, 32, F>(kind, grid, a, s);
    default: return launch_lds_c<BF, EACH, 64, F>(kind, grid, a, s);
  }
}

template <bool BF, bool EACH>
hipError_t launch_lds_tree(int32_t kind, dim3 grid, const KArgs &a, hipStream_t s) {
  switch (a.nranks) {
    case 2: return launch_lds_c<BF, EACH, 16, TreeFold<2, false>>(kind, grid, a, s);
    case 4: return launch_lds_c<BF, EACH, 16, TreeFold<4, false>>(kind, grid, a, s);
    case 8: return launch_lds_c<BF, EACH, 16, TreeFold<8, false>>(kind, grid, a, s);
    case 16: return launch_lds_c<BF, EACH, 16, TreeFold<16, false>>(kind, grid, a, s);
    case 32: return launch_lds_c<BF, EACH, 32, TreeFold<32, false>>(kind, grid, a, s);
    case 64: return launch_lds_c<BF, EACH, 64, TreeFold<64, false>>(kind, grid, a, s);
    default: break;
  }
  const int n = a.nranks;
  if (n == 3) return launch_lds_c<BF, EACH, 16, TreeFold<4, true>>(kind, grid, a, s);
  if (n < 8) return launch_lds_c<BF, EACH, 16, TreeFold<8, true>>(kind, grid, a, s);
  if (n < 16) return launch_lds_c<BF, EACH, 16, TreeFold<16, true>>(kind, grid, a, s);
  if (n < 32) return launch_lds_c<BF, EACH, 32, TreeFold<32, true>>(kind, grid, a, s);
  if (n < 64) return launch_lds_c<BF, EACH, 64, TreeFold<64, true>>(kind, grid, a, s);
  return hipErrorInvalidValue;
}

template <bool BF, bool EACH>
hipError_t launch_lds_dtree(int32_t kind, dim3 grid, const KArgs &a, hipStream_t s) {
  switch (a.nranks) {
    case 2: return launch_lds_c<BF, EACH, 16, DTreeFoldOp<2>>(kind, grid, a, s);
    case 4: return launch_lds_c<BF, EACH, 16, DTreeFoldOp<4>>(kind, grid, a, s);
    case 8: return launch_lds_c<BF, EACH, 16, DTreeFoldOp<8>>(kind, grid, a, s);
    case 16: return launch_lds_c<BF, EACH, 16, DTreeFoldOp<16>>(kind, grid, a, s);
    case 32: return launch_lds_c<BF, EACH, 32, DTreeFoldOp<32>>(kind, grid, a, s);
    case 64: return launch_lds_c<BF, EACH, 64, DTreeFoldOp<64>>(kind, grid, a, s);
    default: return hipErrorInvalidValue;
  }
}

// The LDS-staged fold of a one-pass kind (fp32 0, bf16 1, bf16 rounded at
// each add 2 in the low bits).
template <bool BF, bool EACH>
hipError_t launch_lds_kind(int32_t kind, dim3 grid, const KArgs &a, hipStream_t s) {
  switch (kind & 0xF00) {
    case kKindRing: return launch_lds_n<BF, EACH, RingFold>(kind, grid, a, s);
    case kKindHier: return launch_lds_n<BF, EACH, HierFold>(kind, grid, a, s);
    case kKindTree: return launch_lds_tree<BF, EACH>(kind, grid, a, s);
    case kKindDTree: return launch_lds_dtree<BF, EACH>(kind, grid, a, s);
  }
  return hipErrorInvalidValue;
}

// HBM probe (see hbm_probe): one block per tile of U 16-byte units per
// thread, sources loaded 8 at a time.  POL 0: plain loads and stores (they
// allocate in the caches); 1: non-temporal loads, sc1 stores (the step
// kernels); 2: non-temporal loads and stores (the fp32 one-pass kernels).
// SPLIT: block b takes tile b / ndst and stores it into destination
// b mod ndst only (reading every source for it), so that each wave stores
// into one buffer, as the LDS-staged one-pass folds do; otherwise a block
// stores its tile into every destination, as the register folds do.
struct ProbeArgs {
  const char *src[kProbeMax];
  char *dst[kProbeMax];
  int32_t nsrc, ndst;
  int64_t units;  // 16-byte units per buffer
};
template <int POL>
__device__ __forceinline__ f32x4 probe_ld(const char *p) {
  if constexpr (POL == 0) return *reinterpret_cast<const f32x4 *>(p);
  else return __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p));
}
template <int U, int POL, bool SPLIT>
__global__ __launch_bounds__(kBlock) void hbm_probe_kernel(ProbeArgs a) {
  constexpr int kCp = POL == 0 ? 0 : POL == 1 ? 16 : 2;
  const int64_t tile = SPLIT ? static_cast<int64_t>(blockIdx.x) / a.ndst : static_cast<int64_t>(blockIdx.x);
  const int d0 = SPLIT ? static_cast<int>(static_cast<int64_t>(blockIdx.x) % a.ndst) : 0;
  const int d1 = SPLIT ? d0 + 1 : a.ndst;
  const int64_t t0 = tile * kBlock * U;
  f32x4 acc[U];
#pragma unroll
  for (int u = 0; u < U; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
  int s = 0;
  for (; s + 8 <= a.nsrc; s += 8) {
    f32x4 x[8][U];
#pragma unroll
    for (int q = 0; q < 8; ++q)
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t i = t0 + static_cast<int64_t>(u) * kBlock + threadIdx.x;
        x[q][u] = i < a.units ? probe_ld<POL>(a.src[s + q] + i * 16) : f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
    for (int q = 0; q < 8; ++q)
#pragma unroll
      for (int u = 0; u < U; ++u) acc[u] += x[q][u];
  }
  for (; s < a.nsrc; ++s)
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = t0 + static_cast<int64_t>(u) * kBlock + threadIdx.x;
      if (i < a.units) acc[u] += probe_ld<POL>(a.src[s] + i * 16);
    }
  for (int d = d0; d < d1; ++d)
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = t0 + static_cast<int64_t>(u) * kBlock + threadIdx.x;
      if (i < a.units) st_cp<kCp, f32x4>(a.dst[d] + t0 * 16, static_cast<uint32_t>(i - t0) * 16, acc[u]);
    }
  if (a.ndst == 0) {  // keep the loads: their sum is used by an empty asm
#pragma unroll
    for (int u = 0; u < U; ++u) asm volatile("" ::"v"(acc[u].x), "v"(acc[u].y), "v"(acc[u].z), "v"(acc[u].w));
  }
}

template <int U, bool SPLIT>
void launch_probe_s(int pol, dim3 grid, const ProbeArgs &a, hipStream_t s) {
  if (pol == 0) AR_LAUNCH((hbm_probe_kernel<U, 0, SPLIT>), grid, dim3(kBlock), 0, s, a);
  else if (pol == 1) AR_LAUNCH((hbm_probe_kernel<U, 1, SPLIT>), grid, dim3(kBlock), 0, s, a);
  else AR_LAUNCH((hbm_probe_kernel<U, 2, SPLIT>), grid, dim3(kBlock), 0, s, a);
}
template <int U>
void launch_probe(int pol, bool split, dim3 grid, const ProbeArgs &a, hipStream_t s) {
  if (split) launch_probe_s<U, true>(pol, grid, a, s);
  else launch_probe_s<U, false>(pol, grid, a, s);
}

// Op-table writer: up to kOpsPerWrite ops travel by value in the kernel
// arguments (1.9 KiB) and thread i stores op i.
constexpr int kOpsPerWrite = 48;
struct OpBatch {
  DevOp ops[kOpsPerWrite];
  int32_t n;
};
__global__ __launch_bounds__(64) void write_op_table(DevOp *dst, OpBatch b) {
  const int i = static_cast<int>(threadIdx.x);
  if (i < b.n) dst[i] = b.ops[i];
}

}  // namespace

hipError_t write_ops(DevOp *dst, const DevOp *src, int64_t n, hipStream_t s) {
  for (int64_t k = 0; k < n; k += kOpsPerWrite) {
    OpBatch b;
    b.n = static_cast<int32_t>(std::min<int64_t>(kOpsPerWrite, n - k));
    for (int32_t i = 0; i < b.n; ++i) b.ops[i] = src[k + i];
    hipLaunchKernelGGL(write_op_table, dim3(1), dim3(64), 0, s, dst + k, b);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t hbm_probe(const void *const *src, int nsrc, void *const *dst, int ndst, int64_t bytes, int units,
                     int policy, hipStream_t s) {
  const int pol = policy & 3;
  const bool split = (policy & 4) != 0;
  if (nsrc < 0 || ndst < 0 || nsrc > kProbeMax || ndst > kProbeMax || bytes < 0 || bytes % 16 || policy < 0 ||
      (policy & ~7) != 0 || pol > 2 || (split && ndst < 1))
    return hipErrorInvalidValue;
  ProbeArgs a{};
  for (int i = 0; i < nsrc; ++i) a.src[i] = static_cast<const char *>(src[i]);
  for (int i = 0; i < ndst; ++i) a.dst[i] = static_cast<char *>(dst[i]);
  a.nsrc = nsrc;
  a.ndst = ndst;
  a.units = bytes / 16;
  const int64_t tile = static_cast<int64_t>(kBlock) * units;
  const int64_t blocks = (a.units + tile - 1) / tile * (split ? ndst : 1);
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffff / kBlock) return hipErrorInvalidValue;
  const dim3 grid(static_cast<uint32_t>(blocks));
  switch (units) {
    case 1: launch_probe<1>(pol, split, grid, a, s); break;
    case 2: launch_probe<2>(pol, split, grid, a, s); break;
    case 4: launch_probe<4>(pol, split, grid, a, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

bool lds_staged(int32_t kind, int32_t nranks) {
  const int32_t fam = kind & 0xF00;
  return (fam == kKindRing || fam == kKindHier || fam == kKindTree || fam == kKindDTree) && (kind & 3) != 3 &&
         nranks >= AR_LDS_MIN_RANKS && nranks <= kMaxRanks;
}

KernelShape kernel_shape(int32_t kind, bool cold, bool out_scratch, int32_t nranks) {
  if (lds_staged(kind, nranks))
    return {lds_units_of(kind, nranks), cold ? kCpolLdsCold : kCpolLdsWarm, lds_waves(kind, nranks),
            static_cast<int>(lds_bytes(kind, nranks))};
  switch (kind & 0xF00) {
    case kKindFan:  // units: the tile's 16-byte units per lane of one wave
      return {kFanTileUnits / 64, kCpolFan, fan_threads(nranks) / 64,
              kFanWaves * kFanUnits * 1024};  // the stage is static: its full size
    case kKindReduce: return {reduce_unroll(kind & 0xF, cold), out_scratch ? kCpolScratch : kCpolRank, 0, 0};
    case kKindCopy: return {cold ? kUnrollCold : kUnrollWarm, kCpolRank, 0, 0};
    case kKindRing:
      return (kind & 3) ? KernelShape{kOnePassUnrollBF16, kCpolOnePassBF16, kFoldBatchBF16, 0}
                        : KernelShape{kOnePassUnrollF32, kCpolOnePassF32, kFoldBatchF32, 0};
    case kKindHier:
      return (kind & 3) ? KernelShape{kOnePassUnrollBF16, kCpolOnePassBF16, kFoldBatchHierBF16, 0}
                        : KernelShape{kOnePassUnrollF32, kCpolOnePassF32, kFoldBatchF32, 0};
    case kKindTree:
      return (kind & 3) ? KernelShape{kTreeUnrollBF16, kCpolOnePassBF16, kTreeBatchBF16, 0}
                        : KernelShape{kTreeUnrollF32, kCpolOnePassF32, kTreeBatchF32, 0};
    case kKindDTree:
      return (kind & 3) ? KernelShape{kOnePassUnrollBF16, kCpolOnePassBF16, 0, 0}
                        : KernelShape{kOnePassUnrollF32, kCpolOnePassF32, 0, 0};
  }
  return {0, 0, 0, 0};
}

dim3 grid_for(uint32_t tiles, uint32_t nops) { return dim3(tiles, nops); }

int fan_groups(int32_t nranks) { return fan_groups_of(nranks, fan_threads(nranks) / 64); }

int block_threads(int32_t kind, int32_t nranks) {
  const int32_t fam = kind & 0xF00;
  if (lds_staged(kind, nranks)) return lds_threads(kind, nranks);
  if (fam == kKindFan) return fan_threads(nranks);
  return (fam == kKindReduce || fam == kKindCopy) ? kBlock : kOPB;
}

int64_t tile_elems(int32_t kind, bool cold, int32_t nranks) {
  const int64_t u = cold ? kUnrollCold : kUnrollWarm;
  if (lds_staged(kind, nranks)) return static_cast<int64_t>(64) * lds_units_of(kind, nranks) * ((kind & 3) ? 8 : 4);
  switch (kind & 0xF00) {
    case kKindReduce: return static_cast<int64_t>(kBlock) * reduce_unit_elems(kind & 0xF) * reduce_unroll(kind & 0xF, cold);
    case kKindCopy: return static_cast<int64_t>(kBlock) * (16 / (kind & 0xFF)) * u;
    case kKindFan: return static_cast<int64_t>(kFanTileUnits) * (16 / (kind & 0xFF));
    case kKindTree: return static_cast<int64_t>(kOPB) * 4 * ((kind & 3) ? kTreeUnrollBF16 : kTreeUnrollF32);
    default: return static_cast<int64_t>(kOPB) * 4 * ((kind & 3) ? kOnePassUnrollBF16 : kOnePassUnrollF32);
  }
}

int64_t tiles_per_block(int32_t kind, int32_t nranks) {
  // Measured on 3 GiB in total: the bf16 ring at 2 ranks (2 KiB per rank and
  // tile) ran 14% faster with blocks of 8 tiles, at 4 ranks 3-8%; fp32 and 8
  // or more ranks did not change, and the tree kernels were slower (4 ranks
  // bf16: 7%), so only the ring and hierarchical folds walk several tiles.
  // The LDS-staged folds take one tile per workgroup (a tile of every rank
  // is at least 8 KiB there).
  const int32_t fam = kind & 0xF00;
  if ((fam != kKindRing && fam != kKindHier) || AR_ONEPASS_MIN_BLOCK_BYTES <= 0 || lds_staged(kind, nranks)) return 1;
  // a one-pass tile reads one tile of every rank
  const int64_t bytes = tile_elems(kind, false, nranks) * ((kind & 3) ? 2 : 4) * std::max(nranks, 1);
  return std::max<int64_t>(1, AR_ONEPASS_MIN_BLOCK_BYTES / bytes);
}

hipError_t launch(int32_t kind, dim3 grid, const KArgs &a, hipStream_t s, bool out_scratch, bool cold) {
  switch (kind & 0xF00) {
    case kKindReduce:
      switch (kind & 0xF) {
        case 0: return launch_reduce<0>(grid, a, s, out_scratch, cold);
        case 1: return launch_reduce<1>(grid, a, s, out_scratch, cold);
        case 2: return launch_reduce<2>(grid, a, s, out_scratch, cold);
        case 3: return launch_reduce<3>(grid, a, s, out_scratch, cold);
        case 4: return launch_reduce<4>(grid, a, s, out_scratch, cold);
        case 5: return launch_reduce<5>(grid, a, s, out_scratch, cold);
        case 6: return launch_reduce<6>(grid, a, s, out_scratch, cold);
        case 7: return launch_reduce<7>(grid, a, s, out_scratch, cold);
        case 8: return launch_reduce<8>(grid, a, s, out_scratch, cold);
        case 9: return launch_reduce<9>(grid, a, s, out_scratch, cold);
        case 10: return launch_reduce<10>(grid, a, s, out_scratch, cold);
        case 11: return launch_reduce<11>(grid, a, s, out_scratch, cold);
        case 12: return launch_reduce<12>(grid, a, s, out_scratch, cold);
        case 13: return launch_reduce<13>(grid, a, s, out_scratch, cold);
        case 14: return launch_reduce<14>(grid, a, s, out_scratch, cold);
        case 15: return launch_reduce<15>(grid, a, s, out_scratch, cold);
      }
      break;
    case kKindCopy:
      if ((kind & 0xFF) == 2) return launch_copy<2>(grid, a, s, cold);
      if ((kind & 0xFF) == 4) return launch_copy<4>(grid, a, s, cold);
      return hipErrorInvalidValue;
    case kKindFan:
      if ((kind & 0xFF) == 2) return launch_fan<2>(grid, a, s);
      if ((kind & 0xFF) == 4) return launch_fan<4>(grid, a, s);
      return hipErrorInvalidValue;
    case kKindRing:
    case kKindHier:
    case kKindTree:
    case kKindDTree:
      if (!lds_staged(kind, a.nranks)) break;
      {
        KArgs b = a;
        b.store_cold = cold ? 1 : 0;
        if ((kind & 3) == 2) return launch_lds_kind<true, true>(kind, grid, b, s);
        if ((kind & 3) == 1) return launch_lds_kind<true, false>(kind, grid, b, s);
        return launch_lds_kind<false, false>(kind, grid, b, s);
      }
  }
  switch (kind & 0xF00) {
    case kKindRing:
      if ((kind & 3) == 2)
        AR_LAUNCH((onepass_ring<true, true, kOnePassUnrollBF16, kFoldBatchBF16>), grid, dim3(kOPB), 0, s, a);
      else if ((kind & 3) == 1)
        AR_LAUNCH((onepass_ring<true, false, kOnePassUnrollBF16, kFoldBatchBF16>), grid, dim3(kOPB), 0, s, a);
      else
        AR_LAUNCH((onepass_ring<false, false, kOnePassUnrollF32, kFoldBatchF32>), grid, dim3(kOPB), 0, s, a);
      return hipGetLastError();
    case kKindHier:
      if ((kind & 3) == 2)
        AR_LAUNCH((onepass_hier<true, true, kOnePassUnrollBF16, kFoldBatchHierBF16>), grid, dim3(kOPB), 0, s, a);
      else if ((kind & 3) == 1)
        AR_LAUNCH((onepass_hier<true, false, kOnePassUnrollBF16, kFoldBatchHierBF16>), grid, dim3(kOPB), 0, s, a);
      else
        AR_LAUNCH((onepass_hier<false, false, kOnePassUnrollF32, kFoldBatchF32>), grid, dim3(kOPB), 0, s, a);
      return hipGetLastError();
    case kKindTree:
      if ((kind & 3) == 2) return launch_tree<true, true>(a.nranks, grid, a, s);
      if ((kind & 3) == 1) return launch_tree<true, false>(a.nranks, grid, a, s);
      return launch_tree<false, false>(a.nranks, grid, a, s);
    case kKindDTree:
      if ((kind & 3) == 2) return launch_dtree<true, true>(a.nranks, grid, a, s);
      if ((kind & 3) == 1) return launch_dtree<true, false>(a.nranks, grid, a, s);
      return launch_dtree<false, false>(a.nranks, grid, a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace ar_dev
