// Internal declarations shared by the host planner / ABI (zs_abi.cpp) and the gfx950
// kernels (zs_kernels.hip).  Not part of the public C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "zs.h"

namespace zs {

// Streaming-kernel geometry.  Every streaming kernel launches one workgroup of 256 threads
// (four wave64s) per unit of work - no persistent grid-stride loops, which measured slower
// on MI355X for these pure streams.  A thread owns groups of 8 consecutive flat elements
// (one 16-byte access of 2-byte data, two of fp32), and every kernel covers one
// 4096-element tile per workgroup: kUnroll groups per thread in the unpack kernel, two in
// the pack and check passes (kPackBlock, which also leave one fp64 partial sum per
// workgroup), and the same elements regrouped as four-element quads in the AdamW kernel.
constexpr int kThreads = 256;
constexpr int kGroup = 8;
constexpr int kUnroll = 2;
constexpr int64_t kTile = int64_t(kThreads) * kGroup * kUnroll;
constexpr int64_t kPackBlock = int64_t(kThreads) * kGroup * 2;
constexpr int kLevel2 = 1024;  // first-level partial-sum workgroups of the two-level reduction
// A shard of at most this many tiles runs the AdamW kernel with four workgroups per tile.
constexpr int64_t kSplitTiles = 256;

// XCD-aware work order.  The dispatcher deals consecutive workgroups to the eight XCDs in
// turn.  Run length R: 0 keeps that order (XCD x gets every eighth unit); R > 0 gives each
// XCD runs of R consecutive units (the units of each group of 8R are dealt as eight runs);
// kXcdWhole gives each XCD one contiguous eighth of the range.
constexpr int kXcds = 8;
constexpr int64_t kXcdWhole = -1;
constexpr int64_t kXcdRunAdamw = 16;
constexpr int64_t kXcdRunPack = kXcdWhole;
constexpr int64_t kXcdRunCheck = kXcdWhole;
constexpr int64_t kXcdRunUnpack = kXcdWhole;
// Workgroups launched for `units` units of work in the order of run length `run`.
inline int64_t launch_units(int64_t units, int64_t run) {
  if (run == 0) return units;
  const int64_t group = kXcds * (run > 0 ? run : 1);
  return (units + group - 1) / group * group;
}

// Workgroups (and partial sums) of a pack or check pass over len elements.
__host__ __device__ inline int64_t reduction_blocks(int64_t len) { return (len + kPackBlock - 1) / kPackBlock; }

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
  const uint8_t* seg_nodecay;  // nseg flags (1: the segment's tensor takes no weight decay), or null
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
// launch_pack / launch_check write reduction_blocks(len) partial sums when partials != null;
// launch_reduce_finalize folds n partials (via level2 scratch of kLevel2 doubles when n is
// large) into the state's flag and local sum of squares.
// launch_pack covers flat elements [lo, hi) of the map's range (hi < 0: to its end).
hipError_t launch_pack(const DevMap& map, const uint64_t* src_ptrs, int src_dt, void* dst, int dst_dt, bool accumulate,
                       double* partials, hipStream_t s, int64_t lo = 0, int64_t hi = -1);
hipError_t launch_check(const void* shard, int64_t n, int dt, double* partials, hipStream_t s);
hipError_t launch_reduce_finalize(const double* partials, int64_t nparts, double* level2, DevState* st,
                                  const int32_t* ext, int mode, double* local_out, hipStream_t s);
hipError_t launch_norm_finalize(DevState* st, const double* rank_sumsq, int dp_world, int dp_rank,
                                double* local_out, double max_norm, hipStream_t s);
// The single-rank step's finalizers in one launch (after the same first-level fold as
// launch_reduce_finalize): flag and local sum of squares (set mode, no other ranks), norm
// and clip coefficient, a copy of the state to `pre`, then the scaler commit.  The AdamW
// launch of that step takes `pre` as its state.
hipError_t launch_step_finalize(const double* partials, int64_t nparts, double* level2, DevState* st,
                                DevState* pre, double max_norm, hipStream_t s);
// The allocation-free step (zs_step_flat_noalloc): its finalize reads and commits a bare
// zs_state_host in the caller's memory, and its workspace is a fixed device array of the
// library, one per GPU, holding kNoAllocMaxParts first-level partial sums: check passes of
// at most kNoAllocMaxParts * kPackBlock elements.
constexpr int64_t kNoAllocMaxParts = int64_t(1) << 21;
constexpr int kMaxDevices = 64;
struct NoAllocScratch {
  DevState* pre;
  double* level2;    // kLevel2 slots
  double* partials;  // kNoAllocMaxParts slots
};
// The calling thread's current device's scratch (its address is looked up once per device).
hipError_t noalloc_scratch(NoAllocScratch* out);
hipError_t launch_step_finalize_ext(const double* partials, int64_t nparts, double* level2, zs_state_host* st,
                                    DevState* pre, double max_norm, hipStream_t s);
hipError_t launch_adamw(const DevMap& map, const void* shard, int grad_dt, float* master, float* m, float* v,
                        const AdamwArgs& hp, const DevState* st, const uint64_t* param_ptrs, void* flat_out,
                        int param_dt, hipStream_t s);
hipError_t launch_unpack(const DevMap& map, const void* src, int src_dt, const uint64_t* dst_ptrs, int dst_dt,
                         const DevState* skip, hipStream_t s);
hipError_t launch_scaler_update(DevState* st, hipStream_t s);

// Bandwidth yardsticks (zs_probe.hip); sizes already checked: n a multiple of kTile, bytes a
// multiple of 4 * kTile.
hipError_t launch_probe_mix(const void* g, float* p, float* m, float* v, void* out, int64_t n, hipStream_t s);
hipError_t launch_probe_copy(const void* src, void* dst, int64_t bytes, hipStream_t s);
hipError_t launch_probe_read(const void* src, int64_t bytes, uint32_t* sink, hipStream_t s);
hipError_t launch_probe_write(void* dst, int64_t bytes, hipStream_t s);

}  // namespace zs
