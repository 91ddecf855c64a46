// qkernels.hip -- blockwise INT8 kernels with error feedback for gfx950.
//
// "Collective communication" (Scaling ML systems, ch. 06), section
// "Gradient compression": a block of b = 128 values x is sent as INT8 codes
// q = round(x / s), s = max|x| / 127, plus its fp32 scale s, and decoded as
// q * s ("Blockwise quantization"); each worker sends C(g + e) and keeps
// e = g + e - C(g + e) ("Definition: error feedback mechanism").
//
// Mapping.  Half a wavefront (32 lanes) owns one block, 4 consecutive
// elements per lane, so a block's fp32 values are one 512-byte span (one
// 16-byte access per lane) and its codes one 128-byte span (4 bytes per
// lane); the block maximum is a 5-step butterfly within the half-wave.  A
// 256-thread workgroup takes 8 blocks per pass and U passes (a tile of 8U
// blocks), tiles aligned to 8U blocks in absolute block coordinates.
//
// Exactness.  x / s and max|x| / 127 are IEEE divisions (the library is built
// with correctly rounded fp32 division), rounding is rintf (nearest, ties to
// even), decode is one fp32 multiply and every sum one fp32 add, with no
// contraction: each code and scale equals a step-by-step execution of the
// schedule on the CPU.  Elements past `count` in the last block count as 0.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kernels.hpp"

#ifndef AR_Q_UNROLL
#define AR_Q_UNROLL 2
#endif

namespace ar_dev {

namespace {

constexpr int kQB = static_cast<int>(ar::kQBlock);  // elements per block
constexpr int kHalf = 32;                            // lanes per block
constexpr int kBlocksPerPass = AR_BLOCK / kHalf;     // 8
constexpr int kU = AR_Q_UNROLL;
constexpr int kTileBlocks = kBlocksPerPass * kU;
constexpr int kCopyTileBlocks = AR_BLOCK * 16 / kQB;  // one 16-byte chunk of codes per thread
static_assert(kQB == kHalf * 4, "a half-wave covers one block, 4 elements per lane");

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float half_wave_max(float m) {
#pragma unroll
  for (int off = kHalf / 2; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, kHalf));
  return m;
}

__device__ __forceinline__ float abs_max4(const float x[4]) {
  return fmaxf(fmaxf(fabsf(x[0]), fabsf(x[1])), fmaxf(fabsf(x[2]), fabsf(x[3])));
}

// Codes of 4 values under scale s, packed little-endian into one word.
__device__ __forceinline__ uint32_t quant4(const float x[4], float s, int q[4]) {
  uint32_t packed = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    int v = 0;
    if (s != 0.0f) {
      float r = rintf(x[k] / s);
      r = fminf(fmaxf(r, -127.0f), 127.0f);
      v = static_cast<int>(r);
    }
    q[k] = v;
    packed |= (static_cast<uint32_t>(v) & 0xffu) << (8 * k);
  }
  return packed;
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

template <bool NT>
__device__ __forceinline__ void store4(float *p, int64_t e0, int64_t count, const float x[4]) {
  if (e0 + 4 <= count) {
    f32x4 v;
    v.x = x[0];
    v.y = x[1];
    v.z = x[2];
    v.w = x[3];
    if constexpr (NT) __builtin_nontemporal_store(v, reinterpret_cast<f32x4 *>(p + e0));
    else *reinterpret_cast<f32x4 *>(p + e0) = v;
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (e0 + k < count) p[e0 + k] = x[k];
  }
}

// codes[r] = Q(g_r + e_r); e_r = (g_r + e_r) - D(codes[r]).
__global__ void __launch_bounds__(AR_BLOCK) q_encode(QArgs a) {
  const DevOp op = a.ops[blockIdx.y];
  const int lane = threadIdx.x % kHalf, sub = threadIdx.x / kHalf;
  const int r = op.a;
  const float *g = a.grad[r];
  float *e = a.err[r];
  int8_t *codes = a.codes + r * a.code_stride;
  float *sc = a.scales + r * a.scale_stride;
  const int64_t t = op.lo / kTileBlocks + blockIdx.x;
  float x[kU][4];
  bool live[kU];
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    const int64_t b = t * kTileBlocks + u * kBlocksPerPass + sub;
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
  for (int u = 0; u < kU; ++u) {
    if (!live[u]) continue;  // uniform over the half-wave
    const int64_t b = t * kTileBlocks + u * kBlocksPerPass + sub;
    const int64_t e0 = b * kQB + lane * 4;
    const float s = half_wave_max(abs_max4(x[u])) / 127.0f;
    int q[4];
    *reinterpret_cast<uint32_t *>(codes + e0) = quant4(x[u], s, q);
    if (lane == 0) sc[b] = s;
    if (a.has_err) {
      float res[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) res[k] = x[u][k] - static_cast<float>(q[k]) * s;
      store4<true>(e, e0, a.count, res);
    }
  }
}

// codes[o] (and codes[o2]) = Q(D(codes[a]) + D(codes[b])): the received
// message plus the receiver's own running sum, re-encoded.
template <bool O2>
__global__ void __launch_bounds__(AR_BLOCK) q_reduce(QArgs a) {
  const DevOp op = a.ops[blockIdx.y];
  const int lane = threadIdx.x % kHalf, sub = threadIdx.x / kHalf;
  const int8_t *ca = a.codes + op.a * a.code_stride;
  const int8_t *cb = a.codes + op.b * a.code_stride;
  const float *sa = a.scales + op.a * a.scale_stride;
  const float *sb = a.scales + op.b * a.scale_stride;
  const int64_t t = op.lo / kTileBlocks + blockIdx.x;
  uint32_t wa[kU], wb[kU];
  float fa[kU], fb[kU];
  bool live[kU];
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    const int64_t b = t * kTileBlocks + u * kBlocksPerPass + sub;
    live[u] = b >= op.lo && b < op.hi;
    if (live[u]) {
      const int64_t e0 = b * kQB + lane * 4;
      wa[u] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(ca + e0));
      wb[u] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(cb + e0));
      fa[u] = sa[b];
      fb[u] = sb[b];
    }
  }
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    if (!live[u]) continue;
    const int64_t b = t * kTileBlocks + u * kBlocksPerPass + sub;
    const int64_t e0 = b * kQB + lane * 4;
    float x[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) x[k] = e0 + k < a.count ? code(wa[u], k) * fa[u] + code(wb[u], k) * fb[u] : 0.0f;
    const float s = half_wave_max(abs_max4(x)) / 127.0f;
    int q[4];
    const uint32_t w = quant4(x, s, q);
    *reinterpret_cast<uint32_t *>(a.codes + op.o * a.code_stride + e0) = w;
    if (lane == 0) a.scales[op.o * a.scale_stride + b] = s;
    if constexpr (O2) {
      *reinterpret_cast<uint32_t *>(a.codes + op.o2 * a.code_stride + e0) = w;
      if (lane == 0) a.scales[op.o2 * a.scale_stride + b] = s;
    }
  }
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
    *reinterpret_cast<u32x4 *>(a.codes + op.o * a.code_stride + off) = v;
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
    store4<false>(a.grad[r], b * kQB + lane * 4, a.count, x);
  }
}

}  // namespace

int64_t q_tile_blocks(int32_t kind) { return (kind & 0xF00) == ar::kKQCopy ? kCopyTileBlocks : kTileBlocks; }

hipError_t launch_q(int32_t kind, dim3 grid, const QArgs &a, hipStream_t s) {
  switch (kind & 0xF00) {
    case ar::kKQEncode: hipLaunchKernelGGL(q_encode, grid, dim3(AR_BLOCK), 0, s, a); break;
    case ar::kKQReduce:
      if (kind & ar::kFlagO2) hipLaunchKernelGGL(q_reduce<true>, grid, dim3(AR_BLOCK), 0, s, a);
      else hipLaunchKernelGGL(q_reduce<false>, grid, dim3(AR_BLOCK), 0, s, a);
      break;
    case ar::kKQCopy: hipLaunchKernelGGL(q_copy, grid, dim3(AR_BLOCK), 0, s, a); break;
    case ar::kKQDecode: hipLaunchKernelGGL(q_decode, grid, dim3(AR_BLOCK), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace ar_dev
