// Host planner of the flat buffer ("Deep dive: Megatron", section "Distributed optimizer":
// a contiguous buffer whose length divides by the number of ranks, each rank owning one
// equal contiguous range; "3.7 Megatron-LM, DeepSpeed & Parallelism in Practice", section
// "DeepSpeed config for this run": gradient buckets of reduce_bucket_size elements).

#include "zs_plan.h"

#include <algorithm>
#include <cstdio>

namespace zs_planner {
namespace {

bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }

int64_t round_up(int64_t x, int64_t m) { return ((x + m - 1) / m) * m; }

std::string format(const char* fmt, long long a, long long b = 0) {
  char buf[256];
  std::snprintf(buf, sizeof buf, fmt, a, b);
  return buf;
}

}  // namespace

std::string make_plan(const int64_t* numels, int32_t n, int32_t dp_world, int32_t dp_rank, int64_t align,
                      int64_t max_flat, Plan* out) {
  if (numels == nullptr) return "numels is NULL";
  if (n < 1) return format("n_tensors must be >= 1 (got %lld)", n);
  if (dp_world < 1) return format("dp_world must be >= 1 (got %lld)", dp_world);
  if (dp_rank < 0 || dp_rank >= dp_world) return format("dp_rank %lld outside [0, %lld)", dp_rank, dp_world);
  if (!is_pow2(align)) return format("align_elems must be a power of two (got %lld)", align);
  if (align > max_flat || int64_t(dp_world) > max_flat / align)
    return format("dp_world * align_elems exceeds the %lld-element launch limit", max_flat);
  Plan p;
  p.numels.assign(numels, numels + n);
  p.offsets.resize(n);
  p.dp_world = dp_world;
  p.dp_rank = dp_rank;
  p.align = align;
  int64_t pos = 0;
  for (int32_t i = 0; i < n; ++i) {
    if (numels[i] < 0) return format("numels[%lld] is negative", i);
    if (numels[i] > max_flat || pos > max_flat)
      return format("flat buffer exceeds the %lld-element launch limit", max_flat);
    pos = round_up(pos, align);
    p.offsets[i] = pos;
    pos += numels[i];
  }
  p.flat_numel = round_up(pos, int64_t(dp_world) * align);
  if (p.flat_numel > max_flat)
    return format("flat buffer of %lld elements exceeds the %lld-element launch limit", p.flat_numel, max_flat);
  p.shard_numel = p.flat_numel / dp_world;
  p.shard_begin = int64_t(dp_rank) * p.shard_numel;
  *out = std::move(p);
  return "";
}

HostMap build_map(const Plan& p, int64_t begin, int64_t len, int64_t tile) {
  HostMap m;
  m.len = len;
  const int64_t end = begin + len;
  int64_t cur = begin;
  for (size_t i = 0; i < p.numels.size(); ++i) {
    const int64_t a = std::max(p.offsets[i], begin);
    const int64_t b = std::min(p.offsets[i] + p.numels[i], end);
    if (a >= b) continue;
    if (a > cur) {
      m.seg_begin.push_back(cur - begin);
      m.seg_local.push_back(0);
      m.seg_tensor.push_back(-1);
    }
    m.seg_begin.push_back(a - begin);
    m.seg_local.push_back(a - p.offsets[i]);
    m.seg_tensor.push_back(static_cast<int32_t>(i));
    cur = b;
  }
  if (cur < end) {
    m.seg_begin.push_back(cur - begin);
    m.seg_local.push_back(0);
    m.seg_tensor.push_back(-1);
  }
  const int64_t nseg = static_cast<int64_t>(m.seg_tensor.size());
  m.seg_begin.push_back(len);
  m.ntiles = (len + tile - 1) / tile;
  m.tile_first.resize(m.ntiles + 1);
  int64_t s = 0;
  for (int64_t k = 0; k < m.ntiles; ++k) {
    const int64_t x = k * tile;
    while (m.seg_begin[s + 1] <= x) ++s;
    m.tile_first[k] = static_cast<int32_t>(s);
  }
  m.tile_first[m.ntiles] = static_cast<int32_t>(nseg > 0 ? nseg - 1 : 0);
  return m;
}

int32_t plan_buckets(const int64_t* numels, int32_t n, int64_t bucket_numel, int32_t* bounds) {
  int32_t nb = 0;
  int32_t hi = n;
  int64_t filled = 0;
  for (int32_t t = n - 1; t >= 0; --t) {
    filled += numels[t];
    if (filled >= bucket_numel || t == 0) {
      if (bounds) {
        bounds[2 * nb] = t;
        bounds[2 * nb + 1] = hi;
      }
      ++nb;
      hi = t;
      filled = 0;
    }
  }
  return nb;
}

bool bucket_range(const Plan& p, int32_t t0, int32_t t1, int64_t* begin, int64_t* end) {
  const int32_t n = static_cast<int32_t>(p.numels.size());
  if (t0 < 0 || t1 > n || t0 >= t1) return false;
  *begin = p.offsets[t0];
  *end = (t1 == n) ? p.flat_numel : p.offsets[t1];
  return true;
}

}  // namespace zs_planner
