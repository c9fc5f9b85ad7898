// Internal declarations shared by the host planner / ABI (zs_abi.cpp) and the gfx950
// kernels (zs_kernels.hip).  Not part of the public C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "zs.h"

namespace zs {

// Streaming-kernel geometry: 256 threads (four wave64s) per workgroup, each thread owns a
// group of 8 consecutive flat elements (one 16-byte load of 2-byte data, two of fp32) and
// kUnroll groups per tile, so a tile is 4096 flat elements and a wave touches 1 KiB of
// 2-byte data per group row.
constexpr int kThreads = 256;
constexpr int kGroup = 8;
constexpr int kUnroll = 2;
constexpr int64_t kTile = int64_t(kThreads) * kGroup * kUnroll;

// Segment map of one flat range (a rank's shard or the whole buffer), in device memory.
// Segment i covers range-relative [seg_begin[i], seg_begin[i+1]) and lies inside tensor
// seg_tensor[i] (-1: alignment gap or tail padding) starting at element seg_local[i] of it.
// tile_first[k] is the segment holding the first element of tile k (k < ntiles) and
// tile_first[ntiles] = nseg - 1, so the segments meeting tile k are
// tile_first[k] .. tile_first[k+1].
struct DevMap {
  const int64_t* seg_begin;   // nseg + 1 entries, last = len
  const int64_t* seg_local;   // nseg
  const int32_t* seg_tensor;  // nseg
  const int32_t* tile_first;  // ntiles + 1
  int64_t len;
  int64_t ntiles;
  int32_t nseg;
};

// Device-resident state: the public host struct followed by internal scratch.
struct DevState {
  zs_state_host h;
  double raw_sumsq;  // sum of squares of the (still scaled) shard, fixed order
  double pad_;
};

// Per-step AdamW hyper-parameters passed by value to the kernel.
struct AdamwArgs {
  double lr, beta1, beta2, eps, weight_decay;
};

enum FlagMode : int { kFlagSet = 0, kFlagOr = 1 };

// Launchers (zs_kernels.hip).  Each enqueues on `s` and returns the launch status.
hipError_t launch_pack(const DevMap& map, const uint64_t* src_ptrs, int src_dt, void* dst, int dst_dt,
                       double* partials, int grid, hipStream_t s);
hipError_t launch_check(const void* shard, int64_t n, int dt, double* partials, int grid, hipStream_t s);
hipError_t launch_flag_finalize(const double* partials, int nparts, DevState* st, const int32_t* ext, int mode,
                                double* local_out, hipStream_t s);
hipError_t launch_norm_finalize(DevState* st, const double* rank_sumsq, int dp_world, int dp_rank,
                                double* local_out, double max_norm, hipStream_t s);
hipError_t launch_adamw(const DevMap& map, const void* shard, int grad_dt, float* master, float* m, float* v,
                        const AdamwArgs& hp, const DevState* st, const uint64_t* param_ptrs, void* flat_out,
                        int param_dt, int grid, hipStream_t s);
hipError_t launch_unpack(const DevMap& map, const void* src, int src_dt, const uint64_t* dst_ptrs, int dst_dt,
                         const DevState* skip, int grid, hipStream_t s);
hipError_t launch_scaler_update(DevState* st, hipStream_t s);

}  // namespace zs
