// kernels.hpp -- interface between the executor and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "plan.hpp"

#ifndef AR_REDUCE_UNROLL
#define AR_REDUCE_UNROLL 4
#endif
#ifndef AR_COPY_UNROLL
#define AR_COPY_UNROLL 4
#endif
#ifndef AR_ONEPASS_UNROLL
#define AR_ONEPASS_UNROLL 2
#endif

namespace ar_dev {

constexpr int kMaxRanks = 64;
constexpr int32_t kLocScratchDev = ar::kLocScratch;
constexpr int32_t kKindReduce = ar::kKReduce;
constexpr int32_t kKindCopy = ar::kKCopy;
constexpr int32_t kKindRing = ar::kKRing;
constexpr int32_t kKindHier = ar::kKHier;
constexpr int32_t kKindTree = ar::kKTree;

// One op of a launch as the kernels read it (device table, 40 bytes).
struct DevOp {
  int64_t lo, hi;
  int32_t a, b, o, o2, aux, pad;
};

// Kernel arguments, passed by value (about 560 bytes of kernarg).
struct KArgs {
  void *rank[kMaxRanks];  // the caller's rank buffers for this call
  float *scratch;         // fp32 partial-sum slots
  int64_t slot_stride;    // elements per slot
  const DevOp *ops;       // this launch's ops
  int32_t nranks, group_size;
};

// Tile (elements per block) of a kernel kind; the grid is
// (max over ops of tiles spanned, number of ops).
int64_t tile_elems(int32_t kind);

// Launches the kernel of `kind` on stream s.
hipError_t launch(int32_t kind, dim3 grid, const KArgs &a, hipStream_t s);

}  // namespace ar_dev
