// Host planner of the flat buffer: tensor offsets, the shard partition, the segment maps the
// kernels walk, and the gradient buckets.  Plain C++ with no HIP dependency, so it can be
// built and checked on its own.  Internal to libzs.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

namespace zs_planner {

struct Plan {
  std::vector<int64_t> numels;
  std::vector<int64_t> offsets;
  int64_t flat_numel = 0;
  int64_t shard_begin = 0;
  int64_t shard_numel = 0;
  int32_t dp_world = 1;
  int32_t dp_rank = 0;
  int64_t align = 1;
};

// Places the tensors back to back in list order, each at a multiple of `align`, pads the
// tail to a multiple of dp_world * align and gives rank dp_rank the r-th of dp_world equal
// contiguous shards.  Flat buffers of more than max_flat elements are refused.  Returns ""
// on success, else the reason.
std::string make_plan(const int64_t* numels, int32_t n, int32_t dp_world, int32_t dp_rank, int64_t align,
                      int64_t max_flat, Plan* out);

// Segment map of the range [begin, begin + len): maximal pieces inside one tensor
// (seg_tensor >= 0, starting at element seg_local of it) or inside padding (seg_tensor -1);
// tile_first[k] is the segment holding the first element of tile k (tiles of `tile`
// elements), with one extra entry at the end.
struct HostMap {
  std::vector<int64_t> seg_begin;  // nseg + 1, range-relative
  std::vector<int64_t> seg_local;
  std::vector<int32_t> seg_tensor;
  std::vector<int32_t> tile_first;  // ntiles + 1
  int64_t len = 0;
  int64_t ntiles = 0;
};

HostMap build_map(const Plan& p, int64_t begin, int64_t len, int64_t tile);

// Buckets in backward order (last tensor first), each closed once it holds at least
// bucket_numel elements; the first tensor closes the last one.  Writes the
// [tensor_begin, tensor_end) pairs to bounds (room for 2 * n) when not null and returns
// their number.  Arguments must already be valid (n >= 0, sizes >= 0, bucket_numel > 0).
int32_t plan_buckets(const int64_t* numels, int32_t n, int64_t bucket_numel, int32_t* bounds);

// Flat range of the bucket of tensors [t0, t1): from the first tensor's offset to the next
// tensor's offset (flat_numel after the last tensor).  False unless 0 <= t0 < t1 <= n.
bool bucket_range(const Plan& p, int32_t t0, int32_t t1, int64_t* begin, int64_t* end);

}  // namespace zs_planner
