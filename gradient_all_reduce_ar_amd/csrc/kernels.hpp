// kernels.hpp -- interface between the executor and the HIP kernels.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstdint>

#include "plan.hpp"

#ifndef AR_BLOCK
#define AR_BLOCK 256
#endif
#ifndef AR_ONEPASS_BLOCK
#define AR_ONEPASS_BLOCK AR_BLOCK
#endif
#ifndef AR_NTL
#define AR_NTL 1
#endif
// Cache policy of the vector stores (bits of the store instruction: 2 nt,
// 16 sc1): into rank buffers and fp32 scratch by the step kernels, and into
// rank buffers by the fp32 and bf16 one-pass kernels.
#ifndef AR_CPOL_RANK
#define AR_CPOL_RANK 16
#endif
#ifndef AR_CPOL_SCRATCH
#define AR_CPOL_SCRATCH 16
#endif
// The same for the INT8 kernels: codes (read by the next round), decoded
// values written into the rank buffers by the step kernels, residuals
// written by the step kernels, and the one-pass kernels' residuals and
// results.
#ifndef AR_QCPOL_CODE
#define AR_QCPOL_CODE 16
#endif
#ifndef AR_QCPOL_DEC
#define AR_QCPOL_DEC 18
#endif
#ifndef AR_QCPOL_RES
#define AR_QCPOL_RES 18
#endif
#ifndef AR_QCPOL_RES_ONEPASS
#define AR_QCPOL_RES_ONEPASS 2
#endif
#ifndef AR_QCPOL_OUT
#define AR_QCPOL_OUT 2
#endif
#ifndef AR_CPOL_ONEPASS_F32
#define AR_CPOL_ONEPASS_F32 2
#endif
#ifndef AR_CPOL_ONEPASS_BF16
#define AR_CPOL_ONEPASS_BF16 18
#endif
#ifndef AR_FOLD_BATCH_F32
#define AR_FOLD_BATCH_F32 8
#endif
#ifndef AR_FOLD_BATCH_BF16
#define AR_FOLD_BATCH_BF16 16
#endif
#ifndef AR_FOLD_BATCH_HIER_BF16
#define AR_FOLD_BATCH_HIER_BF16 8
#endif
#ifndef AR_REDUCE_UNROLL
#define AR_REDUCE_UNROLL 2
#endif
// Elements per unit of a reduce whose operands are all bf16: 8 (16-byte
// accesses) or 4 (8-byte).
#ifndef AR_BF16_UNIT
#define AR_BF16_UNIT 8
#endif
#ifndef AR_REDUCE_UNROLL_BF16
#define AR_REDUCE_UNROLL_BF16 4
#endif
#ifndef AR_COLD_UNROLL_BF16
#define AR_COLD_UNROLL_BF16 2
#endif
#ifndef AR_COLD_UNROLL
#define AR_COLD_UNROLL 1
#endif
#ifndef AR_ONEPASS_UNROLL_F32
#define AR_ONEPASS_UNROLL_F32 2
#endif
#ifndef AR_ONEPASS_UNROLL_BF16
#define AR_ONEPASS_UNROLL_BF16 1
#endif
#ifndef AR_ONEPASS_MIN_BLOCK_BYTES  // bytes a one-pass block reads at least (0: one tile per block)
#define AR_ONEPASS_MIN_BLOCK_BYTES 16384
#endif
// LDS-staged one-pass folds (gather every rank's tile into LDS, fold, each
// wave stores into its own ranks): used from AR_LDS_MIN_RANKS ranks up, with
// AR_LDS_UNITS 16-byte units per lane and rank in a tile (1 above 32 ranks),
// and store policies for launches whose output fits in the assumed device
// cache (warm: the next reader finds it there) or not (cold).
#ifndef AR_LDS_MIN_RANKS
#define AR_LDS_MIN_RANKS 4
#endif
#ifndef AR_LDS_UNITS
#define AR_LDS_UNITS 2
#endif
#ifndef AR_CPOL_LDS_WARM
#define AR_CPOL_LDS_WARM 16
#endif
#ifndef AR_CPOL_LDS_COLD
#define AR_CPOL_LDS_COLD 18
#endif
#ifndef AR_TREE_UNROLL_F32
#define AR_TREE_UNROLL_F32 2
#endif
#ifndef AR_TREE_UNROLL_BF16
#define AR_TREE_UNROLL_BF16 1
#endif
#ifndef AR_TREE_BATCH_F32
#define AR_TREE_BATCH_F32 8
#endif
#ifndef AR_TREE_BATCH_BF16
#define AR_TREE_BATCH_BF16 16
#endif

// Kernel launch on stream S that records ar_dev::t_launch_events.
#define AR_LAUNCH(K, G, B, SH, S, ...)                                                                       \
  hipExtLaunchKernelGGL(K, G, B, SH, S, ::ar_dev::t_launch_events.start, ::ar_dev::t_launch_events.stop, 0, \
                        __VA_ARGS__)

namespace ar_dev {

// Events the next kernel launch of this thread records its start and end on
// (both NULL: no timing).  The executor sets them around each launch when the
// profiling log is on; the timestamps come from the dispatch itself, so no
// extra packet sits between two kernels.
struct LaunchEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};
extern thread_local LaunchEvents t_launch_events;

constexpr int kMaxRanks = 64;
constexpr int32_t kLocScratchDev = ar::kLocScratch;
constexpr int32_t kKindReduce = ar::kKReduce;
constexpr int32_t kKindCopy = ar::kKCopy;
constexpr int32_t kKindRing = ar::kKRing;
constexpr int32_t kKindHier = ar::kKHier;
constexpr int32_t kKindTree = ar::kKTree;
constexpr int32_t kKindDTree = ar::kKDTree;
constexpr int32_t kKindFan = ar::kKFan;
constexpr int32_t kKindOwner = ar::kKOwner;

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
  int32_t nops;           // ops in this launch
  int32_t store_cold;     // the launch writes more than the assumed device cache (host side only)
};

// Arguments of the blockwise INT8 kernels (kI8EF plans).  Rank r's code slot
// is codes + r * code_stride (one int8 per element, blocks of 128) and
// scales + r * scale_stride (one fp32 per block).
struct QArgs {
  float *grad[kMaxRanks];  // the caller's fp32 rank buffers
  float *err[kMaxRanks];   // error-feedback buffers (all NULL: none)
  int8_t *codes;
  float *scales;
  int64_t code_stride, scale_stride;
  int64_t count;           // elements per rank
  const DevOp *ops;
  int32_t nops;
  int32_t has_err;
  int32_t nranks, group_size;
};

// Blocks per tile of the INT8 kernels.
int64_t q_tile_blocks(int32_t kind);

// Threads per workgroup of an INT8 kernel kind.
int q_block_threads(int32_t kind);

// Launches one INT8 kernel (encode, reduce, copy, decode, or a one-pass fold
// kind kKRing / kKHier / kKTree / kKDTree) on stream s.
hipError_t launch_q(int32_t kind, dim3 grid, const QArgs &a, hipStream_t s);

// Whether a one-pass kind at nranks runs the LDS-staged fold.
bool lds_staged(int32_t kind, int32_t nranks);

// Tile (elements per block) of a kernel kind in the warm or cold shape.
int64_t tile_elems(int32_t kind, bool cold, int32_t nranks);

// Threads per workgroup of a kernel kind.
int block_threads(int32_t kind, int32_t nranks);

// Workgroups per tile of a one-pass all-gather (kKindFan) at nranks: each
// stores the tile into one group of up to 16 ranks, one rank per wave, so
// its launch grid is that many times its tiles.
int fan_groups(int32_t nranks);

// Tiles each block of a launch walks (the kernels loop over an op's tiles
// with the grid's stride): more than one for the one-pass ring and
// hierarchical folds when a tile of all ranks is little data (bf16 at 2 or 4
// ranks), so a block is not dispatched for a few KiB.
int64_t tiles_per_block(int32_t kind, int32_t nranks);

// Grid of a launch whose ops span at most `tiles` tiles each.
dim3 grid_for(uint32_t tiles, uint32_t nops);

// Writes the n ops at src (host memory) into the device op table at dst with
// kernels whose arguments carry the ops (no copy engine, no staging memory;
// a stream capture records them as kernel nodes).
hipError_t write_ops(DevOp *dst, const DevOp *src, int64_t n, hipStream_t s);

// Template shape of the kernel a launch of `kind` runs: units each thread
// moves per tile (16-byte fp32 or 8-byte bf16 units; 16-byte units per lane
// and rank for the LDS-staged folds), the store cache policy (bits of the
// store instruction: 2 nt, 16 sc1), for the register one-pass folds the
// ranks whose loads are in flight together and for the LDS-staged folds the
// waves per workgroup at most (0 otherwise), and the dynamic LDS bytes per
// workgroup (0 except the LDS-staged folds).
struct KernelShape {
  int units, cpol, batch, lds_bytes;
};
KernelShape kernel_shape(int32_t kind, bool cold, bool out_scratch, int32_t nranks);

// HBM probe: over `bytes` of every buffer (a multiple of 16), each 16-byte
// unit of every destination receives the fp32 sum of that unit of every
// source (nsrc = 0: zeros, a fill; ndst = 0: reads only).  units: 1, 2 or 4
// 16-byte units per thread per tile.  policy 0: plain loads and stores (they
// allocate in the caches); 1: non-temporal loads and sc1 stores (the step
// kernels); 2: non-temporal loads and stores (the fp32 one-pass kernels).
// Up to kProbeMax buffers of each kind.
constexpr int kProbeMax = 64;
hipError_t hbm_probe(const void *const *src, int nsrc, void *const *dst, int ndst, int64_t bytes, int units,
                     int policy, hipStream_t s);

// Launches the kernel of `kind` on stream s.  out_scratch: the launch's
// outputs are fp32 scratch slots (selects the store cache policy); cold: the
// streaming shape, taken by a launch that writes more into rank buffers than
// the device cache holds (the executor decides).
hipError_t launch(int32_t kind, dim3 grid, const KArgs &a, hipStream_t s, bool out_scratch, bool cold);

}  // namespace ar_dev
