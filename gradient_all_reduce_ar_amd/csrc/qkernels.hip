// qkernels.hip -- blockwise INT8 kernels with error feedback for gfx950.
//
// "Collective communication" (Scaling ML systems, ch. 06), section
// "Gradient compression": a block of b = 128 values x is sent as INT8 codes
// q = round(x / s), s = max|x| / 127, plus its fp32 scale s, and decoded as
// q * s ("Blockwise quantization"); each worker sends C(g + e) and keeps
// e = g + e - C(g + e) ("Definition: error feedback mechanism").
//
// Mapping.  Encode and decode (fp32 side): half a wavefront (32 lanes) owns
// one block, 4 consecutive elements per lane, so a block's fp32 values are
// one 512-byte span (one 16-byte access per lane).  Reduce (codes only): 8
// lanes own one block, 16 codes (one 16-byte access) per lane.  A block's
// maximum is a DPP butterfly within its lanes (row permutes, plus one
// swizzle across the two rows of a half-wave), on the bit patterns of |x|,
// which order like the values.  Tiles are aligned to their block count in
// absolute block coordinates.
//
// Exactness.  The code of x is rint(RN(x / s)) with s = RN(max|x| / 127),
// rounding to nearest even, clamped to [-127, 127]; s comes from an
// fma-corrected product (see make_scale), the rare exact quotients below
// from IEEE division (the library is built with correctly rounded fp32
// division).  The kernels
// reach it through t = x * rcp(s): |x / s| <= 127 (1 + 2^-24) and rcp is
// within 1 ulp, so t is within 2^-22 |x / s| < 3.1e-5 of RN(x / s); when t
// lies more than 2^-12 from a half-integer both round to the same integer,
// otherwise (and when s is outside [2^-125, 2^125], where rcp could leave the
// normal range) the code is taken from the exact division.  Decode is one
// fp32 multiply and every sum one fp32 add, with no contraction: each code
// and scale equals a step-by-step execution of the schedule on the CPU.
// Elements past `count` in the last block count as 0.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kernels.hpp"

#ifndef AR_Q_UNROLL
#define AR_Q_UNROLL 2
#endif
#ifndef AR_Q_ENC_UNROLL
#define AR_Q_ENC_UNROLL 1  // blocks per half-wave of the encode kernel
#endif
#ifndef AR_Q_HOP_UNROLL
#define AR_Q_HOP_UNROLL 1  // blocks per half-wave of the fused hop kernel
#endif
#ifndef AR_Q_COPYDEC_UNROLL
#define AR_Q_COPYDEC_UNROLL 2  // blocks per half-wave of the decoding copy
#endif
#ifndef AR_Q_OP_BLOCK
#define AR_Q_OP_BLOCK 512  // threads per workgroup of the one-pass kernels
#endif
#ifndef AR_Q_FOLD_BATCH
#define AR_Q_FOLD_BATCH 4  // ranks whose inputs the one-pass ring loads ahead
#endif

namespace ar_dev {

namespace {

constexpr int kQB = static_cast<int>(ar::kQBlock);  // elements per block
constexpr int kHalf = 32;                            // lanes per block (encode, decode)
constexpr int kBlocksPerPass = AR_BLOCK / kHalf;     // 8
constexpr int kU = AR_Q_UNROLL;
constexpr int kTileBlocks = kBlocksPerPass * kU;
constexpr int kEU = AR_Q_ENC_UNROLL;
constexpr int kEncTileBlocks = kBlocksPerPass * kEU;
constexpr int kHU = AR_Q_HOP_UNROLL;
constexpr int kHopTileBlocks = kBlocksPerPass * kHU;
constexpr int kCU = AR_Q_COPYDEC_UNROLL;
constexpr int kCopyDecTileBlocks = kBlocksPerPass * kCU;
constexpr int kRLanes = 8;                           // lanes per block (reduce): 16 codes each
constexpr int kRBlocksPerPass = AR_BLOCK / kRLanes;  // 32
constexpr int kRTileBlocks = kRBlocksPerPass * kU;
constexpr int kCopyTileBlocks = AR_BLOCK * 16 / kQB;  // one 16-byte chunk of codes per thread
static_assert(8192 % (kTileBlocks * kQB) == 0 && 8192 % (kEncTileBlocks * kQB) == 0 &&
                  8192 % (kHopTileBlocks * kQB) == 0 && 8192 % (kCopyDecTileBlocks * kQB) == 0 &&
                  8192 % (kRTileBlocks * kQB) == 0 && 8192 % (kCopyTileBlocks * kQB) == 0,
              "every INT8 tile lies inside one aligned store window");
static_assert(kQB == kHalf * 4 && kQB == kRLanes * 16, "lane shapes cover one block");

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// max(v, v of another lane) for a DPP lane pattern (all source lanes are
// active: a block's lanes are live or idle together).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_max(uint32_t v) {
  return max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, 0xF, 0xF, false)));
}
// Over each aligned group of 8 lanes: quad swaps 1 and 2, then the mirror
// within each half-row.
__device__ __forceinline__ uint32_t max8(uint32_t v) {
  v = dpp_max<0xB1>(v);   // quad_perm [1,0,3,2]
  v = dpp_max<0x4E>(v);   // quad_perm [2,3,0,1]
  return dpp_max<0x141>(v);  // row_half_mirror
}
// Over each aligned group of 32 lanes: then the row mirror and a swap of the
// two rows.
__device__ __forceinline__ uint32_t max32(uint32_t v) {
  v = dpp_max<0x140>(max8(v));  // row_mirror
  return max(v, static_cast<uint32_t>(__builtin_amdgcn_ds_swizzle(static_cast<int>(v), 0x401F)));  // lane ^ 16
}

__device__ __forceinline__ uint32_t abs_bits(float x) { return __float_as_uint(x) & 0x7fffffffu; }

// Scale of a block from the maximum |x| (bits) and its fast-path reciprocal.
struct Scale {
  float s, rs;
  bool fast;
};
// s = RN(m / 127) without a division: q0 = RN(m * RN(1/127)) is within an
// ulp, the fma residual m - 127 q0 is exact, and one fma correction rounds
// to RN(m / 127) -- checked for every non-negative finite float m.
__device__ __forceinline__ Scale make_scale(uint32_t max_bits) {
  constexpr float kInv127 = 1.0f / 127.0f;
  const float m = __uint_as_float(max_bits);
  const float q0 = m * kInv127;
  Scale r;
  r.s = __builtin_fmaf(__builtin_fmaf(-q0, 127.0f, m), kInv127, q0);
  r.fast = r.s >= 0x1p-125f && r.s <= 0x1p125f;
  r.rs = __builtin_amdgcn_rcpf(r.s);
  return r;
}

// Codes (as floats, -127..127) of N values under scale sc; s == 0 gives 0.
template <int N>
__device__ __forceinline__ void quantize(const float *x, const Scale &sc, float *k) {
  bool slow = !sc.fast;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const float t = x[i] * sc.rs;
    k[i] = rintf(t);
    slow |= fabsf(fabsf(t - k[i]) - 0.5f) < 0x1p-12f;
  }
  if (__builtin_expect(slow, 0)) {
#pragma unroll
    for (int i = 0; i < N; ++i) k[i] = sc.s == 0.0f ? 0.0f : rintf(x[i] / sc.s);
  }
  // clamp; + 0 turns a code of -0 into +0, as an integer code decodes
#pragma unroll
  for (int i = 0; i < N; ++i) k[i] = __builtin_amdgcn_fmed3f(k[i], -127.0f, 127.0f) + 0.0f;
}

__device__ __forceinline__ uint32_t pack4(const float *k) {
  uint32_t w = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) w |= (static_cast<uint32_t>(static_cast<int>(k[i])) & 0xffu) << (8 * i);
  return w;
}

__device__ __forceinline__ float code(uint32_t w, int k) {
  return static_cast<float>(static_cast<int8_t>((w >> (8 * k)) & 0xffu));
}

// Loads 4 fp32 values at element e0 of a buffer of `count` elements; lanes
// at the ragged end load what exists and 0 for the rest.
__device__ __forceinline__ void load4(const float *p, int64_t e0, int64_t count, float x[4]) {
  if (e0 + 4 <= count) {
    const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p + e0));
    x[0] = v.x;
    x[1] = v.y;
    x[2] = v.z;
    x[3] = v.w;
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) x[k] = e0 + k < count ? p[e0 + k] : 0.0f;
  }
}

// Stores with a cache policy (bits of the store instruction: 2 nt, 16 sc1;
// see the step kernels).  Policies with sc1 go through a buffer store, whose
// resource must be wave-uniform: it is built from the start of the aligned
// window of kStoreWindow elements that holds the lane's element.  Every
// INT8 kernel's tile lies inside one such window (checked below), so all
// lanes of a workgroup share it, and readfirstlane makes that visible to the
// compiler.
constexpr int64_t kStoreWindow = 8192;
constexpr int kQRsrcFlags = 0x00020000;  // resource word 3: 32-bit data format

__device__ __forceinline__ int64_t uniform64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(static_cast<uint64_t>(v) >> 32));
  return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

// T (4 or 16 bytes) at element e0 of the element array p (element size ES).
template <int CPOL, int ES, typename T>
__device__ __forceinline__ void st_q(char *p, int64_t e0, T v) {
  if constexpr ((CPOL & 16) == 0) {
    if constexpr (CPOL & 2) __builtin_nontemporal_store(v, reinterpret_cast<T *>(p + e0 * ES));
    else *reinterpret_cast<T *>(p + e0 * ES) = v;
  } else {
    const int64_t w0 = uniform64(e0 & ~(kStoreWindow - 1));
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(p + w0 * ES, 0, 0x7fffffff, kQRsrcFlags);
    const int off = static_cast<int>((e0 - w0) * ES);
    if constexpr (sizeof(T) == 16) __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, CPOL);
    else __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, off, 0, CPOL);
  }
}

template <int CPOL>
__device__ __forceinline__ void store4(float *p, int64_t e0, int64_t count, const float x[4]) {
  if (e0 + 4 <= count) {
    f32x4 v;
    v.x = x[0];
    v.y = x[1];
    v.z = x[2];
    v.w = x[3];
    st_q<CPOL, 4>(reinterpret_cast<char *>(p), e0, v);
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (e0 + k < count) p[e0 + k] = x[k];
  }
}

// 4 (uint32_t) or 16 (u32x4) codes at element e0 of a code slot.
template <int CPOL, typename T>
__device__ __forceinline__ void store_codes(int8_t *codes, int64_t e0, T w) {
  st_q<CPOL, 1>(reinterpret_cast<char *>(codes), e0, w);
}

// (measured on MI355X, 16 ranks x 192 MiB: sc1 codes, nt + sc1 decoded
// values and residuals took the fused ring steps from 2.55 to 2.36 ms;
// the one-pass kernels are fastest with plain nt)
constexpr int kQCpolCode = AR_QCPOL_CODE, kQCpolDec = AR_QCPOL_DEC, kQCpolRes = AR_QCPOL_RES,
              kQCpolResOnePass = AR_QCPOL_RES_ONEPASS, kQCpolOut = AR_QCPOL_OUT;

// codes[r] = Q(g_r + e_r); e_r = (g_r + e_r) - D(codes[r]).
__global__ void __launch_bounds__(AR_BLOCK) q_encode(QArgs a) {
  const DevOp op = a.ops[blockIdx.y];
  const int lane = threadIdx.x % kHalf, sub = threadIdx.x / kHalf;
  const int r = op.a;
  const float *g = a.grad[r];
  float *e = a.err[r];
  int8_t *codes = a.codes + r * a.code_stride;
  float *scl = a.scales + r * a.scale_stride;
  const int64_t t = op.lo / kEncTileBlocks + blockIdx.x;
  float x[kEU][4];
  bool live[kEU];
#pragma unroll
  for (int u = 0; u < kEU; ++u) {
    const int64_t b = t * kEncTileBlocks + u * kBlocksPerPass + sub;
    live[u] = b >= op.lo && b < op.hi;
    const int64_t e0 = b * kQB + lane * 4;
    if (live[u]) {
      load4(g, e0, a.count, x[u]);
      if (a.has_err) {
        float ev[4];
        load4(e, e0, a.count, ev);
#pragma unroll
        for (int k = 0; k < 4; ++k) x[u][k] = x[u][k] + ev[k];
      }
    }
  }
#pragma unroll
  for (int u = 0; u < kEU; ++u) {
    if (!live[u]) continue;  // uniform over the half-wave
    const int64_t b = t * kEncTileBlocks + u * kBlocksPerPass + sub;
    const int64_t e0 = b * kQB + lane * 4;
    const Scale sc = make_scale(
        max32(max(max(abs_bits(x[u][0]), abs_bits(x[u][1])), max(abs_bits(x[u][2]), abs_bits(x[u][3])))));
    float k[4];
    quantize<4>(x[u], sc, k);
    store_codes<kQCpolCode>(codes, e0, pack4(k));
    if (lane == 0) scl[b] = sc.s;
    if (a.has_err) {
      float res[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) res[i] = x[u][i] - k[i] * sc.s;
      store4<kQCpolRes>(e, e0, a.count, res);
    }
  }
}

// codes[o] (and codes[o2]) = Q(D(codes[a]) + D(codes[b])): the received
// message plus the receiver's own running sum, re-encoded.
template <bool O2>
__global__ void __launch_bounds__(AR_BLOCK) q_reduce(QArgs a) {
  const DevOp op = a.ops[blockIdx.y];
  const int lane = threadIdx.x % kRLanes, sub = threadIdx.x / kRLanes;
  const int8_t *ca = a.codes + op.a * a.code_stride;
  const int8_t *cb = a.codes + op.b * a.code_stride;
  const float *sa = a.scales + op.a * a.scale_stride;
  const float *sb = a.scales + op.b * a.scale_stride;
  const int64_t t = op.lo / kRTileBlocks + blockIdx.x;
  u32x4 wa[kU], wb[kU];
  float fa[kU], fb[kU];
  bool live[kU];
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    const int64_t b = t * kRTileBlocks + u * kRBlocksPerPass + sub;
    live[u] = b >= op.lo && b < op.hi;
    if (live[u]) {
      const int64_t e0 = b * kQB + lane * 16;
      wa[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(ca + e0));
      wb[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(cb + e0));
      fa[u] = sa[b];
      fb[u] = sb[b];
    }
  }
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    if (!live[u]) continue;  // uniform over the block's 8 lanes
    const int64_t b = t * kRTileBlocks + u * kRBlocksPerPass + sub;
    const int64_t e0 = b * kQB + lane * 16;
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = code(wa[u][i / 4], i % 4) * fa[u] + code(wb[u][i / 4], i % 4) * fb[u];
    if (e0 + 16 > a.count) {  // the ragged last block (the code slots are padded to whole blocks)
      const int64_t valid = a.count - e0;
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (i >= valid) x[i] = 0.0f;
    }
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) m = max(m, abs_bits(x[i]));
    const Scale sc = make_scale(max8(m));
    float k[16];
    quantize<16>(x, sc, k);
    u32x4 w;
#pragma unroll
    for (int j = 0; j < 4; ++j) w[j] = pack4(k + 4 * j);
    store_codes<kQCpolCode>(a.codes + op.o * a.code_stride, e0, w);
    if (lane == 0) a.scales[op.o * a.scale_stride + b] = sc.s;
    if constexpr (O2) {
      store_codes<kQCpolCode>(a.codes + op.o2 * a.code_stride, e0, w);
      if (lane == 0) a.scales[op.o2 * a.scale_stride + b] = sc.s;
    }
  }
}

// Fused hop (kQFlag* in F, kFlagO2): an operand is either a rank's codes
// or, raw, the rank's own g + e, encoded here (its residual stored); the
// re-encoded sum goes to o (and o2) as codes unless nothing reads them
// later, and, for a rank's final codes, also decoded into its buffer.  Half a
// wavefront per block, 4 elements per lane (the fp32 side sets the shape).
// The loads of all kHU blocks of a lane are issued before any arithmetic.
struct HopIn {
  float x[4];   // raw: g + e
  uint32_t w;   // coded: 4 codes
  float s;      // coded: the block's scale
};

template <bool RAW>
__device__ __forceinline__ void hop_load(const QArgs &a, int r, int64_t b, int64_t e0, HopIn &in) {
  if constexpr (RAW) {
    load4(a.grad[r], e0, a.count, in.x);
    if (a.has_err) {
      float ev[4];
      load4(a.err[r], e0, a.count, ev);
#pragma unroll
      for (int i = 0; i < 4; ++i) in.x[i] = in.x[i] + ev[i];
    }
  } else {
    in.w = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(a.codes + r * a.code_stride + e0));
    in.s = a.scales[r * a.scale_stride + b];
  }
}

template <bool RAW>
__device__ __forceinline__ void hop_value(const QArgs &a, int r, int64_t e0, const HopIn &in, float v[4]) {
  if constexpr (RAW) {
    const Scale sc = make_scale(
        max32(max(max(abs_bits(in.x[0]), abs_bits(in.x[1])), max(abs_bits(in.x[2]), abs_bits(in.x[3])))));
    float k[4];
    quantize<4>(in.x, sc, k);
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = k[i] * sc.s;
    if (a.has_err) {
      float res[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) res[i] = in.x[i] - v[i];
      store4<kQCpolRes>(a.err[r], e0, a.count, res);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = code(in.w, i) * in.s;
  }
}

template <int F>
__global__ void __launch_bounds__(AR_BLOCK) q_hop(QArgs a) {
  constexpr bool kO2 = F & ar::kFlagO2, kDec = F & ar::kQFlagDec, kCode = !(F & ar::kQFlagNoCode);
  constexpr bool kRawA = F & ar::kQFlagARaw, kRawB = F & ar::kQFlagBRaw;
  const DevOp op = a.ops[blockIdx.y];
  const int lane = threadIdx.x % kHalf, sub = threadIdx.x / kHalf;
  const int64_t t = op.lo / kHopTileBlocks + blockIdx.x;
  HopIn ia[kHU], ib[kHU];
  bool live[kHU];
#pragma unroll
  for (int u = 0; u < kHU; ++u) {
    const int64_t b = t * kHopTileBlocks + u * kBlocksPerPass + sub;
    live[u] = b >= op.lo && b < op.hi;
    if (live[u]) {
      const int64_t e0 = b * kQB + lane * 4;
      hop_load<kRawA>(a, op.a, b, e0, ia[u]);
      hop_load<kRawB>(a, op.b, b, e0, ib[u]);
    }
  }
#pragma unroll
  for (int u = 0; u < kHU; ++u) {
    if (!live[u]) continue;  // uniform over the half-wave
    const int64_t b = t * kHopTileBlocks + u * kBlocksPerPass + sub;
    const int64_t e0 = b * kQB + lane * 4;
    float va[4], vb[4], x[4];
    hop_value<kRawA>(a, op.a, e0, ia[u], va);
    hop_value<kRawB>(a, op.b, e0, ib[u], vb);
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = e0 + i < a.count ? va[i] + vb[i] : 0.0f;
    const Scale sc =
        make_scale(max32(max(max(abs_bits(x[0]), abs_bits(x[1])), max(abs_bits(x[2]), abs_bits(x[3])))));
    float k[4];
    quantize<4>(x, sc, k);
    if constexpr (kCode) {
      const uint32_t w = pack4(k);
      store_codes<kQCpolCode>(a.codes + op.o * a.code_stride, e0, w);
      if (lane == 0) a.scales[op.o * a.scale_stride + b] = sc.s;
      if constexpr (kO2) {
        store_codes<kQCpolCode>(a.codes + op.o2 * a.code_stride, e0, w);
        if (lane == 0) a.scales[op.o2 * a.scale_stride + b] = sc.s;
      }
    }
    if constexpr (kDec) {
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = k[i] * sc.s;
      store4<kQCpolDec>(a.grad[op.o], e0, a.count, v);
      if constexpr (kO2) store4<kQCpolDec>(a.grad[op.o2], e0, a.count, v);
    }
  }
}

// A copy that delivers a rank's final codes: decoded into its buffer, and
// stored as codes too unless nothing forwards them later.
template <bool CODE>
__global__ void __launch_bounds__(AR_BLOCK) q_copy_dec(QArgs a) {
  const DevOp op = a.ops[blockIdx.y];
  const int lane = threadIdx.x % kHalf, sub = threadIdx.x / kHalf;
  const int64_t t = op.lo / kCopyDecTileBlocks + blockIdx.x;
  uint32_t w[kCU];
  float s[kCU];
  bool live[kCU];
#pragma unroll
  for (int u = 0; u < kCU; ++u) {
    const int64_t b = t * kCopyDecTileBlocks + u * kBlocksPerPass + sub;
    live[u] = b >= op.lo && b < op.hi;
    if (live[u]) {
      w[u] = __builtin_nontemporal_load(
          reinterpret_cast<const uint32_t *>(a.codes + op.a * a.code_stride + b * kQB + lane * 4));
      s[u] = a.scales[op.a * a.scale_stride + b];
    }
  }
#pragma unroll
  for (int u = 0; u < kCU; ++u) {
    if (!live[u]) continue;
    const int64_t b = t * kCopyDecTileBlocks + u * kBlocksPerPass + sub;
    const int64_t e0 = b * kQB + lane * 4;
    if constexpr (CODE) {
      store_codes<kQCpolCode>(a.codes + op.o * a.code_stride, e0, w[u]);
      if (lane == 0) a.scales[op.o * a.scale_stride + b] = s[u];
    }
    float x[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) x[k] = code(w[u], k) * s[u];
    store4<kQCpolDec>(a.grad[op.o], e0, a.count, x);
  }
}

template <int F>
void launch_hop(dim3 grid, const QArgs &a, hipStream_t s) {
  AR_LAUNCH(q_hop<F>, grid, dim3(AR_BLOCK), 0, s, a);
}

// The fused hop variants the planner emits: operand encodings x (O2) x
// (decode, with or without stored codes).
hipError_t launch_hop_kind(int32_t f, dim3 grid, const QArgs &a, hipStream_t s) {
  constexpr int R = ar::kQFlagARaw, Rb = ar::kQFlagBRaw, O2 = ar::kFlagO2, D = ar::kQFlagDec,
                N = ar::kQFlagNoCode;
  switch (f) {
#define AR_HOP_CASES(RAW)                                             \
  case (RAW): launch_hop<(RAW)>(grid, a, s); break;                   \
  case (RAW) | O2: launch_hop<(RAW) | O2>(grid, a, s); break;         \
  case (RAW) | D: launch_hop<(RAW) | D>(grid, a, s); break;           \
  case (RAW) | D | O2: launch_hop<(RAW) | D | O2>(grid, a, s); break; \
  case (RAW) | D | N: launch_hop<(RAW) | D | N>(grid, a, s); break;   \
  case (RAW) | D | N | O2: launch_hop<(RAW) | D | N | O2>(grid, a, s); break;
    AR_HOP_CASES(0)
    AR_HOP_CASES(R)
    AR_HOP_CASES(Rb)
    AR_HOP_CASES(R | Rb)
#undef AR_HOP_CASES
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// codes[o] = codes[a]: 16 bytes of codes per thread, one scale per thread
// of the first kCopyTileBlocks threads.
__global__ void __launch_bounds__(AR_BLOCK) q_copy(QArgs a) {
  const DevOp op = a.ops[blockIdx.y];
  const int64_t t = op.lo / kCopyTileBlocks + blockIdx.x;
  const int64_t b = t * kCopyTileBlocks + threadIdx.x / (kQB / 16);
  if (b >= op.lo && b < op.hi) {
    const int64_t off = t * kCopyTileBlocks * kQB + threadIdx.x * 16;
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(a.codes + op.a * a.code_stride + off));
    store_codes<kQCpolCode>(a.codes + op.o * a.code_stride, off, v);
  }
  const int64_t bs = t * kCopyTileBlocks + threadIdx.x;
  if (threadIdx.x < kCopyTileBlocks && bs >= op.lo && bs < op.hi)
    a.scales[op.o * a.scale_stride + bs] = a.scales[op.a * a.scale_stride + bs];
}

// g_r = D(codes[r]).
__global__ void __launch_bounds__(AR_BLOCK) q_decode(QArgs a) {
  const DevOp op = a.ops[blockIdx.y];
  const int lane = threadIdx.x % kHalf, sub = threadIdx.x / kHalf;
  const int r = op.a;
  const int8_t *codes = a.codes + r * a.code_stride;
  const float *sc = a.scales + r * a.scale_stride;
  const int64_t t = op.lo / kTileBlocks + blockIdx.x;
  uint32_t w[kU];
  float s[kU];
  bool live[kU];
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    const int64_t b = t * kTileBlocks + u * kBlocksPerPass + sub;
    live[u] = b >= op.lo && b < op.hi;
    if (live[u]) {
      w[u] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(codes + b * kQB + lane * 4));
      s[u] = sc[b];
    }
  }
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    if (!live[u]) continue;
    const int64_t b = t * kTileBlocks + u * kBlocksPerPass + sub;
    float x[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) x[k] = code(w[u], k) * s[u];
    store4<kQCpolDec>(a.grad[r], b * kQB + lane * 4, a.count, x);
  }
}

// ---------------------------------------------------------------- one pass
//
// The whole compressed all-reduce in one launch: every half-wave owns one
// block and folds the ranks' contributions in the schedule's order with the
// step kernels' arithmetic -- a leaf is the round trip v = D(Q(g + e)) (its
// residual g + e - v is stored), an inner node the round trip D(Q(a + b)) --
// then writes the decoded sum to every rank.  The codes never leave
// registers; each rank's g and e are read once and e and the result written
// once.  Blocks are independent, so evaluating the fold depth first gives
// the values of the round-by-round schedule.

constexpr int kOPBlock = AR_Q_OP_BLOCK;       // threads per workgroup
constexpr int kOPTileBlocks = kOPBlock / kHalf;  // one block per half-wave
static_assert(kStoreWindow % (kOPTileBlocks * kQB) == 0, "every one-pass tile lies inside one store window");

// v = D(Q(x)) in place (4 values per lane, 32 lanes per block).
__device__ __forceinline__ void roundtrip4(float x[4]) {
  const Scale sc =
      make_scale(max32(max(max(abs_bits(x[0]), abs_bits(x[1])), max(abs_bits(x[2]), abs_bits(x[3])))));
  float k[4];
  quantize<4>(x, sc, k);
#pragma unroll
  for (int i = 0; i < 4; ++i) x[i] = k[i] * sc.s;
}

// Loads g_r (+ e_r) of this lane's 4 elements.
__device__ __forceinline__ void leaf_load(const QArgs &a, int r, int64_t e0, float x[4]) {
  load4(a.grad[r], e0, a.count, x);
  if (a.has_err) {
    float ev[4];
    load4(a.err[r], e0, a.count, ev);
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = x[i] + ev[i];
  }
}

// x (= g_r + e_r) becomes v_r; the residual goes to e_r.
__device__ __forceinline__ void leaf_finish(const QArgs &a, int r, int64_t e0, float x[4]) {
  float v[4] = {x[0], x[1], x[2], x[3]};
  roundtrip4(v);
  if (a.has_err) {
    float res[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) res[i] = x[i] - v[i];
    store4<kQCpolResOnePass>(a.err[r], e0, a.count, res);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) x[i] = v[i];
}

__device__ __forceinline__ void leaf(const QArgs &a, int r, int64_t e0, float x[4]) {
  leaf_load(a, r, e0, x);
  leaf_finish(a, r, e0, x);
}

// acc = D(Q(acc + y)).
__device__ __forceinline__ void qadd(float acc[4], const float y[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = acc[i] + y[i];
  roundtrip4(acc);
}

__device__ __forceinline__ void store_result(const QArgs &a, int64_t e0, const float v[4]) {
  for (int r = 0; r < a.nranks; ++r) store4<kQCpolOut>(a.grad[r], e0, a.count, v);
}

// The same for exactly N ranks: every argument index is a compile-time
// constant, so a large unrolled kernel can keep its arguments in registers
// (a runtime index makes the compiler copy the whole argument block to
// private memory and read every pointer back from there).
template <int N>
__device__ __forceinline__ void store_result_n(const QArgs &a, int64_t e0, const float v[4]) {
#pragma unroll
  for (int r = 0; r < N; ++r) store4<kQCpolOut>(a.grad[r], e0, a.count, v);
}

// Block coordinate of this half-wave, or -1 when its block is outside the op.
__device__ __forceinline__ int64_t op_block(const DevOp &op) {
  const int64_t b = (op.lo / kOPTileBlocks + blockIdx.x) * kOPTileBlocks + threadIdx.x / kHalf;
  return b >= op.lo && b < op.hi ? b : -1;
}

// Ring: chunk c's blocks fold ranks c, c+1, ..., c+N-1 (aux = c), the order
// in which the chunk travels round the ring in reduce-scatter.  FB ranks'
// inputs are loaded ahead of their use.
template <int FB>
__global__ void __launch_bounds__(kOPBlock) q_onepass_ring(QArgs a) {
  const DevOp op = a.ops[blockIdx.y];
  const int64_t b = op_block(op);
  if (b < 0) return;  // the whole half-wave
  const int64_t e0 = b * kQB + (threadIdx.x % kHalf) * 4;
  const int n = a.nranks;
  float acc[4];
  int r = op.aux;
  for (int t0 = 0; t0 < n; t0 += FB) {
    float x[FB][4];
    int rr = r;
#pragma unroll
    for (int i = 0; i < FB; ++i) {
      if (t0 + i < n) leaf_load(a, rr, e0, x[i]);
      rr = rr + 1 == n ? 0 : rr + 1;
    }
#pragma unroll
    for (int i = 0; i < FB; ++i) {
      if (t0 + i >= n) break;
      leaf_finish(a, r, e0, x[i]);
      if (t0 + i == 0) {
#pragma unroll
        for (int k = 0; k < 4; ++k) acc[k] = x[i][k];
      } else {
        qadd(acc, x[i]);
      }
      r = r + 1 == n ? 0 : r + 1;
    }
  }
  store_result(a, e0, acc);
}

// Hierarchical (aux = ls | j << 8): for groups g = j, j+1, ... (mod M), the
// group's partial folds local ranks ls, ls+1, ... (mod G); the partials fold
// in that group order.
__global__ void __launch_bounds__(kOPBlock) q_onepass_hier(QArgs a) {
  const DevOp op = a.ops[blockIdx.y];
  const int64_t b = op_block(op);
  if (b < 0) return;
  const int64_t e0 = b * kQB + (threadIdx.x % kHalf) * 4;
  const int G = a.group_size, M = a.nranks / a.group_size;
  const int ls = op.aux & 0xFF, j = op.aux >> 8;
  float acc[4];
  for (int mi = 0; mi < M; ++mi) {
    const int g = (j + mi) % M;
    float part[4];
    leaf(a, g * G + ls, e0, part);
    for (int t = 1; t < G; ++t) {
      float y[4];
      leaf(a, g * G + (ls + t) % G, e0, y);
      qadd(part, y);
    }
    if (mi == 0) {
#pragma unroll
      for (int k = 0; k < 4; ++k) acc[k] = part[k];
    } else {
      qadd(acc, part);
    }
  }
  store_result(a, e0, acc);
}

// Tree over ranks in index order (balanced for N = 2^L, left-complete
// binomial otherwise): batches of 8 ranks merge pairwise, a node without a
// right neighbour is carried up unchanged, then the batch results merge the
// same way.  NMAX = N rounded up to a power of two.
template <int NMAX>
__global__ void __launch_bounds__(kOPBlock) q_onepass_tree(QArgs a) {
  constexpr int kB = NMAX < 8 ? NMAX : 8;
  constexpr int kBatches = NMAX / kB;
  const DevOp op = a.ops[blockIdx.y];
  const int64_t b = op_block(op);
  if (b < 0) return;
  const int64_t e0 = b * kQB + (threadIdx.x % kHalf) * 4;
  const int n = a.nranks;
  float res[kBatches][4];
#pragma unroll
  for (int bi = 0; bi < kBatches; ++bi) {
    if (bi * kB >= n) continue;
    float v[kB][4];
#pragma unroll
    for (int i = 0; i < kB; ++i)
      if (bi * kB + i < n) leaf_load(a, bi * kB + i, e0, v[i]);
#pragma unroll
    for (int i = 0; i < kB; ++i)
      if (bi * kB + i < n) leaf_finish(a, bi * kB + i, e0, v[i]);
#pragma unroll
    for (int w = kB, span = 1; w > 1; w /= 2, span *= 2)
#pragma unroll
      for (int i = 0; i < w / 2; ++i)
        if (bi * kB + (2 * i + 1) * span < n) {
          qadd(v[2 * i], v[2 * i + 1]);
#pragma unroll
          for (int k = 0; k < 4; ++k) v[i][k] = v[2 * i][k];
        } else if (i > 0) {
#pragma unroll
          for (int k = 0; k < 4; ++k) v[i][k] = v[2 * i][k];
        }
#pragma unroll
    for (int k = 0; k < 4; ++k) res[bi][k] = v[0][k];
  }
#pragma unroll
  for (int w = kBatches, span = kB; w > 1; w /= 2, span *= 2)
#pragma unroll
    for (int i = 0; i < w / 2; ++i)
      if ((2 * i + 1) * span < n) {
        qadd(res[2 * i], res[2 * i + 1]);
#pragma unroll
        for (int k = 0; k < 4; ++k) res[i][k] = res[2 * i][k];
      } else if (i > 0 && 2 * i * span < n) {
#pragma unroll
        for (int k = 0; k < 4; ++k) res[i][k] = res[2 * i][k];
      }
  store_result(a, e0, res[0]);
}

// Double binary tree, one half per op (aux = 0: tree 1, 1: its mirror):
// D(c, b) = (v_c + D(c - b/2, b/2)) + D(c + b/2, b/2), D(c, 1) = v_c; tree 1
// gives v_0 + D(N/2, N/2), tree 2 gives v_{N-1} + D(N/2 - 1, N/2).
template <int C, int B>
struct QDTree {
  static __device__ __forceinline__ void run(const QArgs &a, int64_t e0, float out[4]) {
    leaf(a, C, e0, out);
    if constexpr (B > 1) {
      // own + lower child, then + higher child; the higher subtree is
      // evaluated after the first add, so one child's values are live at a time
      float sub[4];
      QDTree<C - B / 2, B / 2>::run(a, e0, sub);
      qadd(out, sub);
      QDTree<C + B / 2, B / 2>::run(a, e0, sub);
      qadd(out, sub);
    }
  }
};

template <int N>
__global__ void __launch_bounds__(kOPBlock) q_onepass_dtree(QArgs a) {
  const DevOp op = a.ops[blockIdx.y];
  const int64_t b = op_block(op);
  if (b < 0) return;
  const int64_t e0 = b * kQB + (threadIdx.x % kHalf) * 4;
  float root[4], sub[4];
  if (op.aux == 0) {
    leaf(a, 0, e0, root);
    QDTree<N / 2, N / 2>::run(a, e0, sub);
  } else {
    leaf(a, N - 1, e0, root);
    QDTree<N / 2 - 1, N / 2>::run(a, e0, sub);
  }
  qadd(root, sub);
  store_result_n<N>(a, e0, root);
}

template <int NMAX>
void launch_q_tree(dim3 grid, const QArgs &a, hipStream_t s) {
  AR_LAUNCH(q_onepass_tree<NMAX>, grid, dim3(kOPBlock), 0, s, a);
}

hipError_t launch_q_onepass(int32_t fam, dim3 grid, const QArgs &a, hipStream_t s) {
  const int n = a.nranks;
  switch (fam) {
    case ar::kKRing: AR_LAUNCH(q_onepass_ring<AR_Q_FOLD_BATCH>, grid, dim3(kOPBlock), 0, s, a); break;
    case ar::kKHier: AR_LAUNCH(q_onepass_hier, grid, dim3(kOPBlock), 0, s, a); break;
    case ar::kKTree:
      if (n <= 2) launch_q_tree<2>(grid, a, s);
      else if (n <= 4) launch_q_tree<4>(grid, a, s);
      else if (n <= 8) launch_q_tree<8>(grid, a, s);
      else if (n <= 16) launch_q_tree<16>(grid, a, s);
      else if (n <= 32) launch_q_tree<32>(grid, a, s);
      else if (n <= 64) launch_q_tree<64>(grid, a, s);
      else return hipErrorInvalidValue;
      break;
    case ar::kKDTree:
      switch (n) {
        case 2: AR_LAUNCH(q_onepass_dtree<2>, grid, dim3(kOPBlock), 0, s, a); break;
        case 4: AR_LAUNCH(q_onepass_dtree<4>, grid, dim3(kOPBlock), 0, s, a); break;
        case 8: AR_LAUNCH(q_onepass_dtree<8>, grid, dim3(kOPBlock), 0, s, a); break;
        case 16: AR_LAUNCH(q_onepass_dtree<16>, grid, dim3(kOPBlock), 0, s, a); break;
        case 32: AR_LAUNCH(q_onepass_dtree<32>, grid, dim3(kOPBlock), 0, s, a); break;
        case 64: AR_LAUNCH(q_onepass_dtree<64>, grid, dim3(kOPBlock), 0, s, a); break;
        default: return hipErrorInvalidValue;
      }
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

int64_t q_tile_blocks(int32_t kind) {
  switch (kind & 0xF00) {
    case ar::kKQCopy: return (kind & ar::kQFlagDec) ? kCopyDecTileBlocks : kCopyTileBlocks;
    case ar::kKQReduce:
      return (kind & (ar::kQFlagARaw | ar::kQFlagBRaw | ar::kQFlagDec)) ? kHopTileBlocks : kRTileBlocks;
    case ar::kKQEncode: return kEncTileBlocks;
    case ar::kKQDecode: return kTileBlocks;
    default: return kOPTileBlocks;
  }
}

int q_block_threads(int32_t kind) {
  switch (kind & 0xF00) {
    case ar::kKQCopy:
    case ar::kKQReduce:
    case ar::kKQEncode:
    case ar::kKQDecode: return AR_BLOCK;
    default: return kOPBlock;
  }
}

hipError_t launch_q(int32_t kind, dim3 grid, const QArgs &a, hipStream_t s) {
  switch (kind & 0xF00) {
    case ar::kKQEncode: AR_LAUNCH(q_encode, grid, dim3(AR_BLOCK), 0, s, a); break;
    case ar::kKQReduce:
      if (kind & (ar::kQFlagARaw | ar::kQFlagBRaw | ar::kQFlagDec)) return launch_hop_kind(kind & 0xFF, grid, a, s);
      if (kind & ar::kFlagO2) AR_LAUNCH(q_reduce<true>, grid, dim3(AR_BLOCK), 0, s, a);
      else AR_LAUNCH(q_reduce<false>, grid, dim3(AR_BLOCK), 0, s, a);
      break;
    case ar::kKQCopy:
      if (kind & ar::kQFlagDec) {
        if (kind & ar::kQFlagNoCode) AR_LAUNCH(q_copy_dec<false>, grid, dim3(AR_BLOCK), 0, s, a);
        else AR_LAUNCH(q_copy_dec<true>, grid, dim3(AR_BLOCK), 0, s, a);
      } else {
        AR_LAUNCH(q_copy, grid, dim3(AR_BLOCK), 0, s, a);
      }
      break;
    case ar::kKQDecode: AR_LAUNCH(q_decode, grid, dim3(AR_BLOCK), 0, s, a); break;
    default: return launch_q_onepass(kind & 0xF00, grid, a, s);
  }
  return hipGetLastError();
}

}  // namespace ar_dev
