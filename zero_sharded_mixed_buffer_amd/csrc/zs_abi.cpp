// Host side of the C ABI: argument validation, the flat-buffer planner, the segment maps
// uploaded once per layout, the device state, and the launch sequence of each entry point.
// Every step entry point only enqueues work on the caller's stream.

#include <hip/hip_runtime.h>
#include <rocprofiler-sdk-roctx/roctx.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "zs.h"
#include "zs_host.h"
#include "zs_probe.h"
#include "zs_internal.h"
#include "zs_plan.h"

using zs::DevMap;
using zs::DevState;

namespace {

thread_local std::string g_last_error;

zs_status fail(zs_status code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

zs_status ok() { return ZS_OK; }

zs_status hip_fail(hipError_t e, const char* what) {
  return fail(ZS_EHIP, "%s: %s", what, hipGetErrorString(e));
}

// A named profiler range around each step entry point, on the calling host thread (shown by
// rocprofv3 --marker-trace; a no-op when no profiler is attached).
class TraceRange {
 public:
  explicit TraceRange(const char* name) { roctxRangePushA(name); }
  ~TraceRange() { roctxRangePop(); }
  TraceRange(const TraceRange&) = delete;
  TraceRange& operator=(const TraceRange&) = delete;
};

bool is_pow2_double(double x) {
  if (!(x > 0.0) || !std::isfinite(x)) return false;
  int e = 0;
  return std::frexp(x, &e) == 0.5;
}

int64_t round_up(int64_t x, int64_t m) { return ((x + m - 1) / m) * m; }

// ---------------------------------------------------------------------------- planner

using zs_planner::HostMap;
using zs_planner::Plan;

// One workgroup of kThreads per kTile-element tile, and a launch holds fewer than 2^32
// work-items: at most 2^24 - 1 tiles (68.7e9 elements, beyond what one GPU can hold beside
// the 6 bytes per element of replicated model state anyway).
constexpr int64_t kMaxFlat = (((int64_t(1) << 32) - 1) / zs::kThreads) * zs::kTile;

zs_status make_plan(const int64_t* numels, int32_t n, int32_t dp_world, int32_t dp_rank, int64_t align,
                    Plan* out) {
  const std::string err = zs_planner::make_plan(numels, n, dp_world, dp_rank, align, kMaxFlat, out);
  if (!err.empty()) return fail(ZS_EINVAL, "%s", err.c_str());
  return ok();
}

HostMap build_map(const Plan& p, int64_t begin, int64_t len) { return zs_planner::build_map(p, begin, len, zs::kTile); }

// One device allocation per map: seg_begin | seg_local | seg_tensor | tile_first.
zs_status upload_map(const HostMap& h, void** mem, DevMap* out) {
  const size_t nseg = h.seg_tensor.size();
  const size_t b0 = 0;
  const size_t b1 = b0 + (nseg + 1) * sizeof(int64_t);
  const size_t b2 = b1 + std::max<size_t>(nseg, 1) * sizeof(int64_t);
  const size_t b3 = b2 + round_up(std::max<size_t>(nseg, 1) * sizeof(int32_t), 16);
  const size_t total = b3 + h.tile_first.size() * sizeof(int32_t);
  void* d = nullptr;
  hipError_t e = hipMalloc(&d, total);
  if (e != hipSuccess) return fail(ZS_ENOMEM, "hipMalloc of %zu bytes for the segment map: %s", total, hipGetErrorString(e));
  std::vector<unsigned char> host(total, 0);
  std::memcpy(host.data() + b0, h.seg_begin.data(), h.seg_begin.size() * sizeof(int64_t));
  if (nseg) {
    std::memcpy(host.data() + b1, h.seg_local.data(), nseg * sizeof(int64_t));
    std::memcpy(host.data() + b2, h.seg_tensor.data(), nseg * sizeof(int32_t));
  }
  std::memcpy(host.data() + b3, h.tile_first.data(), h.tile_first.size() * sizeof(int32_t));
  e = hipMemcpy(d, host.data(), total, hipMemcpyHostToDevice);
  if (e != hipSuccess) {
    (void)hipFree(d);
    return hip_fail(e, "uploading the segment map");
  }
  unsigned char* base = static_cast<unsigned char*>(d);
  out->seg_begin = reinterpret_cast<const int64_t*>(base + b0);
  out->seg_local = reinterpret_cast<const int64_t*>(base + b1);
  out->seg_tensor = reinterpret_cast<const int32_t*>(base + b2);
  out->tile_first = reinterpret_cast<const int32_t*>(base + b3);
  out->seg_nodecay = nullptr;
  out->len = h.len;
  out->ntiles = h.ntiles;
  out->nseg = static_cast<int32_t>(nseg);
  *mem = d;
  return ok();
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool is_half_dtype(int dt) { return dt == ZS_BF16 || dt == ZS_FP16; }
bool is_grad_dtype(int dt) { return dt == ZS_BF16 || dt == ZS_FP16 || dt == ZS_FP32; }
bool grad_aligned(const void* p, int dt) {
  return (reinterpret_cast<uintptr_t>(p) & (dt == ZS_FP32 ? 3u : 1u)) == 0;
}

zs_status check_state_fields(const zs_state_host* s) {
  if (!is_pow2_double(s->loss_scale)) return fail(ZS_EINVAL, "loss_scale must be a positive power of two");
  if (!is_pow2_double(s->scale_floor)) return fail(ZS_EINVAL, "scale_floor must be a positive power of two");
  if (s->growth_interval < 1) return fail(ZS_EINVAL, "growth_interval must be >= 1");
  if (s->dynamic != 0 && s->dynamic != 1) return fail(ZS_EINVAL, "dynamic must be 0 or 1");
  if (s->step_t < 0 || s->growth_tracker < 0 || s->skipped_total < 0)
    return fail(ZS_EINVAL, "step_t, growth_tracker and skipped_total must be >= 0");
  return ok();
}

zs_status check_hparams(const zs_adamw_hparams* hp) {
  if (hp == nullptr) return fail(ZS_EINVAL, "hparams is NULL");
  const double vals[6] = {hp->lr, hp->beta1, hp->beta2, hp->eps, hp->weight_decay, hp->max_norm};
  for (double x : vals)
    if (!std::isfinite(x)) return fail(ZS_EINVAL, "hyper-parameters must be finite");
  if (hp->lr < 0) return fail(ZS_EINVAL, "lr must be >= 0");
  if (hp->beta1 < 0 || hp->beta1 >= 1 || hp->beta2 < 0 || hp->beta2 >= 1)
    return fail(ZS_EINVAL, "betas must lie in [0, 1)");
  if (!(hp->eps > 0)) return fail(ZS_EINVAL, "eps must be > 0");
  if (hp->weight_decay < 0) return fail(ZS_EINVAL, "weight_decay must be >= 0");
  return ok();
}

}  // namespace

// ---------------------------------------------------------------------------- opaque types

struct zs_layout {
  Plan plan;
  int device = 0;
  int num_cu = 0;
  void* mem_shard = nullptr;
  void* mem_full = nullptr;  // null when the shard is the whole buffer (dp_world == 1)
  DevMap map_shard{};
  DevMap map_full{};
  int64_t nparts = 0;  // partial-sum slots: workgroups of the largest pack / check pass
  void* mem_nodecay = nullptr;         // per-segment no-decay flags of the shard map, or null
  std::vector<int64_t> nodecay_runs;   // the same as shard-relative [begin, end) pairs
  // Tables replaced by zs_layout_set_no_decay: work enqueued before the replacement may
  // still read them, so they (and the host copies their uploads read) live until destroy.
  std::vector<void*> retired_tables;
  std::vector<std::vector<uint8_t>> upload_sources;
};

struct zs_state {
  DevState* dev = nullptr;     // the state, then one more DevState: zs_step's pre-commit copy
  double* partials = nullptr;  // nparts slots, then kLevel2 second-level slots
  int64_t nparts = 0;
  int device = 0;
};

namespace {

zs_status check_device(int device) {
  int cur = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (cur != device) return fail(ZS_EINVAL, "current device %d is not the layout's device %d", cur, device);
  return ok();
}

zs_status check_layout(const zs_layout* l) {
  if (l == nullptr) return fail(ZS_EINVAL, "layout is NULL");
  return check_device(l->device);
}

zs_status check_state(const zs_layout* l, const zs_state* s) {
  if (s == nullptr) return fail(ZS_EINVAL, "state is NULL");
  if (s->device != l->device) return fail(ZS_EINVAL, "state and layout live on different devices");
  if (s->nparts < l->nparts) return fail(ZS_EINVAL, "state was created for a smaller layout");
  return ok();
}

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

}  // namespace

// ---------------------------------------------------------------------------- planning ABI

extern "C" zs_status zs_plan(const int64_t* numels, int32_t n_tensors, int32_t dp_world, int32_t dp_rank,
                             int64_t align_elems, int64_t* offsets_out, int64_t* flat_numel_out,
                             int64_t* shard_begin_out, int64_t* shard_numel_out) {
  Plan p;
  zs_status st = make_plan(numels, n_tensors, dp_world, dp_rank, align_elems, &p);
  if (st != ZS_OK) return st;
  if (offsets_out) std::memcpy(offsets_out, p.offsets.data(), p.offsets.size() * sizeof(int64_t));
  if (flat_numel_out) *flat_numel_out = p.flat_numel;
  if (shard_begin_out) *shard_begin_out = p.shard_begin;
  if (shard_numel_out) *shard_numel_out = p.shard_numel;
  return ok();
}

extern "C" zs_status zs_plan_segments(const int64_t* numels, int32_t n_tensors, int32_t dp_world, int32_t dp_rank,
                                      int64_t align_elems, int32_t whole_flat, int64_t* seg_begin,
                                      int32_t* seg_tensor, int64_t* seg_local, int64_t capacity,
                                      int64_t* n_segments) {
  if (n_segments == nullptr) return fail(ZS_EINVAL, "n_segments is NULL");
  if (capacity < 0) return fail(ZS_EINVAL, "capacity is negative");
  Plan p;
  zs_status st = make_plan(numels, n_tensors, dp_world, dp_rank, align_elems, &p);
  if (st != ZS_OK) return st;
  const HostMap m = whole_flat ? build_map(p, 0, p.flat_numel) : build_map(p, p.shard_begin, p.shard_numel);
  const int64_t nseg = static_cast<int64_t>(m.seg_tensor.size());
  *n_segments = nseg;
  const int64_t k = std::min(nseg, capacity);
  for (int64_t i = 0; i < k; ++i) {
    if (seg_begin) seg_begin[i] = m.seg_begin[i];
    if (seg_tensor) seg_tensor[i] = m.seg_tensor[i];
    if (seg_local) seg_local[i] = m.seg_local[i];
  }
  return ok();
}

extern "C" zs_status zs_plan_buckets(const int64_t* numels, int32_t n_tensors, int64_t bucket_numel,
                                     int32_t* bounds_out, int32_t* n_buckets_out) {
  if (n_buckets_out == nullptr) return fail(ZS_EINVAL, "n_buckets_out is NULL");
  if (n_tensors < 0 || (n_tensors > 0 && numels == nullptr)) return fail(ZS_EINVAL, "bad tensor list");
  if (bucket_numel <= 0) return fail(ZS_EINVAL, "bucket_numel must be positive");
  for (int32_t i = 0; i < n_tensors; ++i)
    if (numels[i] < 0) return fail(ZS_EINVAL, "numels[%d] is negative", i);
  const int32_t nb = zs_planner::plan_buckets(numels, n_tensors, bucket_numel, bounds_out);
  *n_buckets_out = nb;
  return ok();
}

// ---------------------------------------------------------------------------- layout / state

extern "C" zs_status zs_layout_create(const int64_t* numels, int32_t n_tensors, int32_t dp_world, int32_t dp_rank,
                                      int64_t align_elems, zs_layout** out) {
  if (out == nullptr) return fail(ZS_EINVAL, "out is NULL");
  *out = nullptr;
  Plan p;
  zs_status st = make_plan(numels, n_tensors, dp_world, dp_rank, align_elems, &p);
  if (st != ZS_OK) return st;
  zs_layout* l = new (std::nothrow) zs_layout();
  if (l == nullptr) return fail(ZS_ENOMEM, "host allocation of the layout failed");
  l->plan = std::move(p);
  hipError_t e = hipGetDevice(&l->device);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&l->num_cu, hipDeviceAttributeMultiprocessorCount, l->device);
  if (e != hipSuccess) {
    delete l;
    return hip_fail(e, "querying the current device");
  }
  const Plan& q = l->plan;
  l->nparts = std::max<int64_t>(1, std::max(zs::reduction_blocks(q.flat_numel), zs::reduction_blocks(q.shard_numel)));
  st = upload_map(build_map(q, q.shard_begin, q.shard_numel), &l->mem_shard, &l->map_shard);
  if (st == ZS_OK) {
    if (q.dp_world == 1) {
      l->map_full = l->map_shard;
    } else {
      st = upload_map(build_map(q, 0, q.flat_numel), &l->mem_full, &l->map_full);
    }
  }
  if (st != ZS_OK) {
    zs_layout_destroy(l);
    return st;
  }
  *out = l;
  return ok();
}

extern "C" void zs_layout_destroy(zs_layout* l) {
  if (l == nullptr) return;
  if (l->mem_shard) (void)hipFree(l->mem_shard);
  if (l->mem_full) (void)hipFree(l->mem_full);
  if (l->mem_nodecay) (void)hipFree(l->mem_nodecay);
  for (void* t : l->retired_tables) (void)hipFree(t);
  delete l;
}

extern "C" zs_status zs_layout_set_no_decay(zs_layout* l, const uint8_t* no_decay, int32_t n_tensors,
                                            void* stream) {
  const TraceRange trace("zs_layout_set_no_decay");
  zs_status st = check_layout(l);
  if (st != ZS_OK) return st;
  const int32_t n = static_cast<int32_t>(l->plan.numels.size());
  if (no_decay != nullptr && n_tensors != n)
    return fail(ZS_EINVAL, "no_decay has %d flags for %d tensors", n_tensors, n);
  // Build the new table on the host first, so that a failure leaves the old one in force.
  std::vector<int64_t> runs;
  std::vector<uint8_t> flags;
  if (no_decay != nullptr) {
    const HostMap m = build_map(l->plan, l->plan.shard_begin, l->plan.shard_numel);
    const size_t nseg = m.seg_tensor.size();
    flags.assign(std::max<size_t>(nseg, 1), 0);
    for (size_t s = 0; s < nseg; ++s) {
      const int32_t t = m.seg_tensor[s];
      if (t < 0 || no_decay[t] == 0) continue;
      flags[s] = 1;
      if (!runs.empty() && runs.back() == m.seg_begin[s]) {
        runs.back() = m.seg_begin[s + 1];  // adjacent runs merge
      } else {
        runs.push_back(m.seg_begin[s]);
        runs.push_back(m.seg_begin[s + 1]);
      }
    }
  }
  void* d = nullptr;
  if (!runs.empty()) {  // some element of this shard takes no decay: upload its table
    hipError_t e = hipMalloc(&d, flags.size());
    if (e != hipSuccess) return fail(ZS_ENOMEM, "hipMalloc for the no-decay table: %s", hipGetErrorString(e));
    l->upload_sources.push_back(std::move(flags));
    const std::vector<uint8_t>& src = l->upload_sources.back();
    e = hipMemcpyAsync(d, src.data(), src.size(), hipMemcpyHostToDevice, as_stream(stream));
    if (e != hipSuccess) {
      l->upload_sources.pop_back();
      (void)hipFree(d);
      return hip_fail(e, "uploading the no-decay table");
    }
  }
  // The kernels take the table's address at launch, so work enqueued earlier keeps reading
  // the previous table; it is retired rather than freed (no device-wide wait here).
  if (l->mem_nodecay) l->retired_tables.push_back(l->mem_nodecay);
  l->mem_nodecay = d;
  l->nodecay_runs = std::move(runs);
  l->map_shard.seg_nodecay = static_cast<const uint8_t*>(d);
  if (l->plan.dp_world == 1) l->map_full.seg_nodecay = l->map_shard.seg_nodecay;
  return ok();
}

extern "C" zs_status zs_layout_info(const zs_layout* l, int64_t* flat_numel, int64_t* shard_begin,
                                    int64_t* shard_numel) {
  if (l == nullptr) return fail(ZS_EINVAL, "layout is NULL");
  if (flat_numel) *flat_numel = l->plan.flat_numel;
  if (shard_begin) *shard_begin = l->plan.shard_begin;
  if (shard_numel) *shard_numel = l->plan.shard_numel;
  return ok();
}

extern "C" zs_status zs_state_create(const zs_layout* l, const zs_state_host* init, zs_state** out) {
  if (out == nullptr) return fail(ZS_EINVAL, "out is NULL");
  *out = nullptr;
  zs_status st = check_layout(l);
  if (st != ZS_OK) return st;
  if (init == nullptr) return fail(ZS_EINVAL, "init is NULL");
  st = check_state_fields(init);
  if (st != ZS_OK) return st;
  zs_state* s = new (std::nothrow) zs_state();
  if (s == nullptr) return fail(ZS_ENOMEM, "host allocation of the state failed");
  s->device = l->device;
  s->nparts = l->nparts;
  hipError_t e = hipMalloc(reinterpret_cast<void**>(&s->dev), 2 * sizeof(DevState));
  const size_t part_bytes = sizeof(double) * static_cast<size_t>(s->nparts + zs::kLevel2);
  if (e == hipSuccess) e = hipMalloc(reinterpret_cast<void**>(&s->partials), part_bytes);
  if (e != hipSuccess) {
    zs_state_destroy(s);
    return fail(ZS_ENOMEM, "hipMalloc for the state: %s", hipGetErrorString(e));
  }
  DevState h[2]{};
  h[0].h = *init;
  e = hipMemcpy(s->dev, h, sizeof h, hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemset(s->partials, 0, part_bytes);
  if (e != hipSuccess) {
    zs_state_destroy(s);
    return hip_fail(e, "initialising the state");
  }
  *out = s;
  return ok();
}

extern "C" void zs_state_destroy(zs_state* s) {
  if (s == nullptr) return;
  if (s->dev) (void)hipFree(s->dev);
  if (s->partials) (void)hipFree(s->partials);
  delete s;
}

extern "C" zs_status zs_state_read(const zs_state* s, zs_state_host* out, void* stream) {
  if (s == nullptr || out == nullptr) return fail(ZS_EINVAL, "state or out is NULL");
  zs_status st = check_device(s->device);
  if (st != ZS_OK) return st;
  DevState h{};
  hipError_t e = hipMemcpyAsync(&h, s->dev, sizeof h, hipMemcpyDeviceToHost, as_stream(stream));
  if (e == hipSuccess) e = hipStreamSynchronize(as_stream(stream));
  if (e != hipSuccess) return hip_fail(e, "reading the state");
  *out = h.h;
  return ok();
}

extern "C" zs_status zs_state_write(zs_state* s, const zs_state_host* in, void* stream) {
  if (s == nullptr || in == nullptr) return fail(ZS_EINVAL, "state or in is NULL");
  zs_status st = check_device(s->device);
  if (st != ZS_OK) return st;
  st = check_state_fields(in);
  if (st != ZS_OK) return st;
  DevState h{};
  h.h = *in;
  hipError_t e = hipMemcpyAsync(s->dev, &h, sizeof h, hipMemcpyHostToDevice, as_stream(stream));
  if (e == hipSuccess) e = hipStreamSynchronize(as_stream(stream));
  if (e != hipSuccess) return hip_fail(e, "writing the state");
  return ok();
}

// ---------------------------------------------------------------------------- step ABI

namespace {

zs_status pack_common(const zs_layout* l, const void* src_ptrs, zs_dtype src_dtype, void* dst, zs_dtype dst_dtype,
                      int32_t whole_flat, bool accumulate, zs_state* fuse_check, void* stream, const char* what) {
  zs_status st = check_layout(l);
  if (st != ZS_OK) return st;
  if (src_ptrs == nullptr || dst == nullptr) return fail(ZS_EINVAL, "%s: src_ptrs or dst is NULL", what);
  if (!is_half_dtype(src_dtype)) return fail(ZS_EINVAL, "%s: src_dtype must be bf16 or fp16", what);
  if (dst_dtype != src_dtype && dst_dtype != ZS_FP32)
    return fail(ZS_EUNSUPPORTED, "%s: the buffer must have the source dtype or fp32", what);
  if (!aligned16(dst)) return fail(ZS_EINVAL, "%s: the flat buffer must be 16-byte aligned", what);
  if (fuse_check != nullptr) {
    st = check_state(l, fuse_check);
    if (st != ZS_OK) return st;
    if (l->plan.dp_world != 1 || !whole_flat)
      return fail(ZS_EINVAL, "%s: fuse_check needs dp_world == 1 and the whole flat buffer", what);
  }
  const DevMap& map = whole_flat ? l->map_full : l->map_shard;
  hipStream_t s = as_stream(stream);
  double* parts = fuse_check ? fuse_check->partials : nullptr;
  hipError_t e = zs::launch_pack(map, static_cast<const uint64_t*>(src_ptrs), src_dtype, dst, dst_dtype, accumulate,
                                 parts, s);
  if (e != hipSuccess) return hip_fail(e, "launching pack");
  if (fuse_check) {
    const int64_t used = zs::reduction_blocks(map.len);
    e = zs::launch_reduce_finalize(parts, used, parts + fuse_check->nparts, fuse_check->dev, nullptr, zs::kFlagSet,
                                   nullptr, s);
    if (e != hipSuccess) return hip_fail(e, "launching the overflow finalize");
  }
  return ok();
}

}  // namespace

extern "C" zs_status zs_pack(const zs_layout* l, const void* src_ptrs, zs_dtype src_dtype, void* dst,
                             zs_dtype dst_dtype, int32_t whole_flat, zs_state* fuse_check, void* stream) {
  const TraceRange trace("zs_pack");
  return pack_common(l, src_ptrs, src_dtype, dst, dst_dtype, whole_flat, false, fuse_check, stream, "zs_pack");
}

extern "C" zs_status zs_pack_accumulate(const zs_layout* l, const void* src_ptrs, zs_dtype src_dtype, void* acc,
                                        zs_dtype acc_dtype, int32_t whole_flat, zs_state* fuse_check, void* stream) {
  const TraceRange trace("zs_pack_accumulate");
  return pack_common(l, src_ptrs, src_dtype, acc, acc_dtype, whole_flat, true, fuse_check, stream,
                     "zs_pack_accumulate");
}

namespace {

zs_status bucket_range(const zs_layout* l, int32_t t0, int32_t t1, int64_t* begin, int64_t* end) {
  if (!zs_planner::bucket_range(l->plan, t0, t1, begin, end))
    return fail(ZS_EINVAL, "bucket [%d, %d) is not a non-empty tensor range of %d", t0, t1,
                static_cast<int32_t>(l->plan.numels.size()));
  return ok();
}

}  // namespace

extern "C" zs_status zs_bucket_range(const zs_layout* l, int32_t tensor_begin, int32_t tensor_end, int64_t* flat_begin,
                                     int64_t* flat_end) {
  if (l == nullptr || flat_begin == nullptr || flat_end == nullptr) return fail(ZS_EINVAL, "NULL argument");
  return bucket_range(l, tensor_begin, tensor_end, flat_begin, flat_end);
}

extern "C" zs_status zs_pack_bucket(const zs_layout* l, const void* src_ptrs, zs_dtype src_dtype, void* flat,
                                    zs_dtype flat_dtype, int32_t tensor_begin, int32_t tensor_end, int32_t accumulate,
                                    void* stream) {
  const TraceRange trace("zs_pack_bucket");
  zs_status st = check_layout(l);
  if (st != ZS_OK) return st;
  if (src_ptrs == nullptr || flat == nullptr) return fail(ZS_EINVAL, "zs_pack_bucket: src_ptrs or flat is NULL");
  if (!is_half_dtype(src_dtype)) return fail(ZS_EINVAL, "zs_pack_bucket: src_dtype must be bf16 or fp16");
  if (flat_dtype != src_dtype && flat_dtype != ZS_FP32)
    return fail(ZS_EUNSUPPORTED, "zs_pack_bucket: the buffer must have the source dtype or fp32");
  if (!aligned16(flat)) return fail(ZS_EINVAL, "zs_pack_bucket: the flat buffer must be 16-byte aligned");
  int64_t lo = 0, hi = 0;
  st = bucket_range(l, tensor_begin, tensor_end, &lo, &hi);
  if (st != ZS_OK) return st;
  hipError_t e = zs::launch_pack(l->map_full, static_cast<const uint64_t*>(src_ptrs), src_dtype, flat, flat_dtype,
                                 accumulate != 0, nullptr, as_stream(stream), lo, hi);
  if (e != hipSuccess) return hip_fail(e, "launching the bucket pack");
  return ok();
}

extern "C" zs_status zs_unscale_check(const zs_layout* l, const void* shard, zs_dtype grad_dtype, zs_state* state,
                                      const int32_t* ext_overflow, double* local_sumsq_out, void* stream) {
  const TraceRange trace("zs_unscale_check");
  zs_status st = check_layout(l);
  if (st != ZS_OK) return st;
  st = check_state(l, state);
  if (st != ZS_OK) return st;
  if (shard == nullptr) return fail(ZS_EINVAL, "shard is NULL");
  if (!is_grad_dtype(grad_dtype)) return fail(ZS_EINVAL, "grad_dtype must be bf16, fp16 or fp32");
  if (!grad_aligned(shard, grad_dtype)) return fail(ZS_EINVAL, "shard is not aligned to its element size");
  hipStream_t s = as_stream(stream);
  const int64_t n = l->plan.shard_numel;
  hipError_t e = zs::launch_check(shard, n, grad_dtype, state->partials, s);
  if (e != hipSuccess) return hip_fail(e, "launching check");
  e = zs::launch_reduce_finalize(state->partials, zs::reduction_blocks(n), state->partials + state->nparts,
                                 state->dev, ext_overflow, zs::kFlagSet, local_sumsq_out, s);
  if (e != hipSuccess) return hip_fail(e, "launching the overflow finalize");
  return ok();
}

extern "C" zs_status zs_grad_norm(const zs_layout* l, const void* shard, zs_dtype grad_dtype, zs_state* state,
                                  const zs_adamw_hparams* hp, const double* rank_sumsq, double* local_sumsq_out,
                                  void* stream) {
  const TraceRange trace("zs_grad_norm");
  zs_status st = check_layout(l);
  if (st != ZS_OK) return st;
  st = check_state(l, state);
  if (st != ZS_OK) return st;
  st = check_hparams(hp);
  if (st != ZS_OK) return st;
  if (l->plan.dp_world > 1 && rank_sumsq == nullptr)
    return fail(ZS_EINVAL, "rank_sumsq is required when dp_world > 1");
  hipStream_t s = as_stream(stream);
  hipError_t e;
  if (shard != nullptr) {
    if (!is_grad_dtype(grad_dtype)) return fail(ZS_EINVAL, "grad_dtype must be bf16, fp16 or fp32");
    if (!grad_aligned(shard, grad_dtype)) return fail(ZS_EINVAL, "shard is not aligned to its element size");
    const int64_t n = l->plan.shard_numel;
    e = zs::launch_check(shard, n, grad_dtype, state->partials, s);
    if (e != hipSuccess) return hip_fail(e, "launching check");
    e = zs::launch_reduce_finalize(state->partials, zs::reduction_blocks(n), state->partials + state->nparts,
                                   state->dev, nullptr, zs::kFlagOr, nullptr, s);
    if (e != hipSuccess) return hip_fail(e, "launching the sum finalize");
  }
  e = zs::launch_norm_finalize(state->dev, rank_sumsq, l->plan.dp_world, l->plan.dp_rank, local_sumsq_out,
                               hp->max_norm, s);
  if (e != hipSuccess) return hip_fail(e, "launching the norm finalize");
  return ok();
}

extern "C" zs_status zs_adamw_step(const zs_layout* l, const void* shard, zs_dtype grad_dtype, float* master,
                                   float* m, float* v, const zs_adamw_hparams* hp, zs_state* state,
                                   const void* param_ptrs, void* flat_param_out, zs_dtype param_dtype,
                                   void* stream) {
  const TraceRange trace("zs_adamw_step");
  zs_status st = check_layout(l);
  if (st != ZS_OK) return st;
  st = check_state(l, state);
  if (st != ZS_OK) return st;
  st = check_hparams(hp);
  if (st != ZS_OK) return st;
  if (shard == nullptr || master == nullptr || m == nullptr || v == nullptr)
    return fail(ZS_EINVAL, "shard, master, m and v must not be NULL");
  if (!is_grad_dtype(grad_dtype) || !is_half_dtype(param_dtype))
    return fail(ZS_EINVAL, "grad_dtype must be bf16, fp16 or fp32 and param_dtype bf16 or fp16");
  if (!grad_aligned(shard, grad_dtype)) return fail(ZS_EINVAL, "shard is not aligned to its element size");
  if (!aligned16(master) || !aligned16(m) || !aligned16(v)) return fail(ZS_EINVAL, "master, m, v must be 16-byte aligned");
  if (flat_param_out != nullptr && !aligned16(flat_param_out))
    return fail(ZS_EINVAL, "flat_param_out must be 16-byte aligned");
  const zs::AdamwArgs a{hp->lr, hp->beta1, hp->beta2, hp->eps, hp->weight_decay};
  hipError_t e = zs::launch_adamw(l->map_shard, shard, grad_dtype, master, m, v, a, state->dev,
                                  static_cast<const uint64_t*>(param_ptrs), flat_param_out, param_dtype,
                                  as_stream(stream));
  if (e != hipSuccess) return hip_fail(e, "launching adamw");
  return ok();
}

extern "C" zs_status zs_unpack(const zs_layout* l, const void* src, zs_dtype src_dtype, int32_t whole_flat,
                               const void* dst_ptrs, zs_dtype dst_dtype, const zs_state* honour_skip,
                               void* stream) {
  const TraceRange trace("zs_unpack");
  zs_status st = check_layout(l);
  if (st != ZS_OK) return st;
  if (src == nullptr || dst_ptrs == nullptr) return fail(ZS_EINVAL, "src or dst_ptrs is NULL");
  if (!is_half_dtype(dst_dtype)) return fail(ZS_EINVAL, "dst_dtype must be bf16 or fp16");
  if (src_dtype != ZS_FP32 && src_dtype != dst_dtype)
    return fail(ZS_EUNSUPPORTED, "unpack reads fp32 or the destination dtype");
  if (src_dtype == ZS_FP32 && !aligned16(src)) return fail(ZS_EINVAL, "an fp32 src must be 16-byte aligned");
  if (honour_skip != nullptr) {
    st = check_state(l, honour_skip);
    if (st != ZS_OK) return st;
  }
  const DevMap& map = whole_flat ? l->map_full : l->map_shard;
  hipError_t e = zs::launch_unpack(map, src, src_dtype, static_cast<const uint64_t*>(dst_ptrs), dst_dtype,
                                   honour_skip ? honour_skip->dev : nullptr, as_stream(stream));
  if (e != hipSuccess) return hip_fail(e, "launching unpack");
  return ok();
}

extern "C" zs_status zs_scaler_update(zs_state* state, void* stream) {
  const TraceRange trace("zs_scaler_update");
  if (state == nullptr) return fail(ZS_EINVAL, "state is NULL");
  zs_status st = check_device(state->device);
  if (st != ZS_OK) return st;
  hipError_t e = zs::launch_scaler_update(state->dev, as_stream(stream));
  if (e != hipSuccess) return hip_fail(e, "launching the scaler update");
  return ok();
}

extern "C" zs_status zs_step(const zs_layout* l, const void* grad_ptrs, zs_dtype grad_dtype, void* flat,
                             zs_state* state, const zs_adamw_hparams* hp, float* master, float* m, float* v,
                             const void* param_ptrs, zs_dtype param_dtype, void* stream) {
  const TraceRange trace("zs_step");
  zs_status st = check_layout(l);
  if (st != ZS_OK) return st;
  st = check_state(l, state);
  if (st != ZS_OK) return st;
  st = check_hparams(hp);
  if (st != ZS_OK) return st;
  if (l->plan.dp_world != 1) return fail(ZS_EINVAL, "zs_step is the single-rank step: dp_world must be 1");
  if (grad_ptrs == nullptr || flat == nullptr || param_ptrs == nullptr)
    return fail(ZS_EINVAL, "grad_ptrs, flat and param_ptrs must not be NULL");
  if (master == nullptr || m == nullptr || v == nullptr) return fail(ZS_EINVAL, "master, m and v must not be NULL");
  if (!is_half_dtype(grad_dtype) || !is_half_dtype(param_dtype))
    return fail(ZS_EINVAL, "grad_dtype and param_dtype must be bf16 or fp16");
  if (!aligned16(flat)) return fail(ZS_EINVAL, "the flat buffer must be 16-byte aligned");
  if (!aligned16(master) || !aligned16(m) || !aligned16(v)) return fail(ZS_EINVAL, "master, m, v must be 16-byte aligned");
  hipStream_t s = as_stream(stream);
  // Three launches: the pack with the check's partial sums; one workgroup that sets the
  // flag, takes the norm, keeps the pre-commit state and commits the scaler; the update,
  // which reads that pre-commit state.  The arithmetic is the four calls', step for step.
  DevState* pre = state->dev + 1;
  hipError_t e = zs::launch_pack(l->map_full, static_cast<const uint64_t*>(grad_ptrs), grad_dtype, flat, grad_dtype,
                                 false, state->partials, s);
  if (e != hipSuccess) return hip_fail(e, "launching pack");
  e = zs::launch_step_finalize(state->partials, zs::reduction_blocks(l->map_full.len), state->partials + state->nparts,
                               state->dev, pre, hp->max_norm, s);
  if (e != hipSuccess) return hip_fail(e, "launching the step finalize");
  const zs::AdamwArgs a{hp->lr, hp->beta1, hp->beta2, hp->eps, hp->weight_decay};
  e = zs::launch_adamw(l->map_shard, flat, grad_dtype, master, m, v, a, pre, static_cast<const uint64_t*>(param_ptrs),
                       nullptr, param_dtype, s);
  if (e != hipSuccess) return hip_fail(e, "launching adamw");
  return ok();
}

extern "C" zs_status zs_step_flat(const zs_layout* l, const void* flat, zs_dtype grad_dtype, zs_state* state,
                                  const zs_adamw_hparams* hp, float* master, float* m, float* v,
                                  void* flat_param_out, zs_dtype param_dtype, void* stream) {
  const TraceRange trace("zs_step_flat");
  zs_status st = check_layout(l);
  if (st != ZS_OK) return st;
  st = check_state(l, state);
  if (st != ZS_OK) return st;
  st = check_hparams(hp);
  if (st != ZS_OK) return st;
  if (l->plan.dp_world != 1) return fail(ZS_EINVAL, "zs_step_flat is the single-rank step: dp_world must be 1");
  if (flat == nullptr || flat_param_out == nullptr || master == nullptr || m == nullptr || v == nullptr)
    return fail(ZS_EINVAL, "flat, flat_param_out, master, m and v must not be NULL");
  if (!is_half_dtype(grad_dtype) || !is_half_dtype(param_dtype))
    return fail(ZS_EINVAL, "grad_dtype and param_dtype must be bf16 or fp16");
  if (!aligned16(flat) || !aligned16(flat_param_out))
    return fail(ZS_EINVAL, "flat and flat_param_out must be 16-byte aligned");
  if (!aligned16(master) || !aligned16(m) || !aligned16(v)) return fail(ZS_EINVAL, "master, m, v must be 16-byte aligned");
  hipStream_t s = as_stream(stream);
  // zs_unscale_check + zs_grad_norm + zs_adamw_step (flat output) + zs_scaler_update in three
  // launches: the check's partial sums, the one-workgroup finalize (which keeps the
  // pre-commit state for the update), and the update.
  DevState* pre = state->dev + 1;
  const int64_t n = l->plan.shard_numel;
  hipError_t e = zs::launch_check(flat, n, grad_dtype, state->partials, s);
  if (e != hipSuccess) return hip_fail(e, "launching check");
  e = zs::launch_step_finalize(state->partials, zs::reduction_blocks(n), state->partials + state->nparts, state->dev,
                               pre, hp->max_norm, s);
  if (e != hipSuccess) return hip_fail(e, "launching the step finalize");
  const zs::AdamwArgs a{hp->lr, hp->beta1, hp->beta2, hp->eps, hp->weight_decay};
  e = zs::launch_adamw(l->map_shard, flat, grad_dtype, master, m, v, a, pre, nullptr, flat_param_out, param_dtype, s);
  if (e != hipSuccess) return hip_fail(e, "launching adamw");
  return ok();
}

extern "C" zs_status zs_step_flat_noalloc(const void* flat, zs_dtype grad_dtype, int64_t n, zs_state_host* state,
                                          const zs_adamw_hparams* hp, float* master, float* m, float* v,
                                          void* flat_param_out, zs_dtype param_dtype, void* stream) {
  const TraceRange trace("zs_step_flat_noalloc");
  zs_status st = check_hparams(hp);
  if (st != ZS_OK) return st;
  if (flat == nullptr || state == nullptr || flat_param_out == nullptr || master == nullptr || m == nullptr ||
      v == nullptr)
    return fail(ZS_EINVAL, "flat, state, flat_param_out, master, m and v must not be NULL");
  if (!is_half_dtype(grad_dtype) || !is_half_dtype(param_dtype))
    return fail(ZS_EINVAL, "grad_dtype and param_dtype must be bf16 or fp16");
  if (n < 1) return fail(ZS_EINVAL, "n must be positive");
  const int64_t max_n = zs::kNoAllocMaxParts * zs::kPackBlock;
  if (n > max_n)
    return fail(ZS_EINVAL, "n = %lld exceeds the %lld elements the fixed scratch of zs_step_flat_noalloc covers",
                static_cast<long long>(n), static_cast<long long>(max_n));
  if (!aligned16(flat) || !aligned16(flat_param_out))
    return fail(ZS_EINVAL, "flat and flat_param_out must be 16-byte aligned");
  if (!aligned16(master) || !aligned16(m) || !aligned16(v)) return fail(ZS_EINVAL, "master, m, v must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(state) & 7u) != 0) return fail(ZS_EINVAL, "state must be 8-byte aligned");
  zs::NoAllocScratch sc{};
  hipError_t e = zs::noalloc_scratch(&sc);
  if (e != hipSuccess) return hip_fail(e, "looking up the scratch of the allocation-free step");
  hipStream_t s = as_stream(stream);
  // The launches of zs_step_flat, with the scratch in place of the state's workspace: the
  // check's partial sums, the finalize (which keeps the pre-commit state for the update), the
  // update into the flat parameter buffer.
  const int64_t parts = zs::reduction_blocks(n);
  e = zs::launch_check(flat, n, grad_dtype, sc.partials, s);
  if (e != hipSuccess) return hip_fail(e, "launching check");
  e = zs::launch_step_finalize_ext(sc.partials, parts, sc.level2, state, sc.pre, hp->max_norm, s);
  if (e != hipSuccess) return hip_fail(e, "launching the step finalize");
  DevMap map{};  // no segment tables: nothing is scattered and every element decays
  map.len = n;
  map.ntiles = (n + zs::kTile - 1) / zs::kTile;
  const zs::AdamwArgs a{hp->lr, hp->beta1, hp->beta2, hp->eps, hp->weight_decay};
  e = zs::launch_adamw(map, flat, grad_dtype, master, m, v, a, sc.pre, nullptr, flat_param_out, param_dtype, s);
  if (e != hipSuccess) return hip_fail(e, "launching adamw");
  return ok();
}

extern "C" const char* zs_last_error(void) { return g_last_error.c_str(); }

// ---------------------------------------------------------------------------- offloaded step

namespace {

zs_status check_host_scalars(const zs_state_host* sc) {
  if (sc == nullptr) return fail(ZS_EINVAL, "scalars is NULL");
  if (!is_pow2_double(sc->loss_scale)) return fail(ZS_EINVAL, "loss_scale must be a positive power of two");
  if (!(sc->clip_coef > 0.0) || !(sc->clip_coef <= 1.0)) return fail(ZS_EINVAL, "clip_coef must lie in (0, 1]");
  if (sc->step_t < 0) return fail(ZS_EINVAL, "step_t must be >= 0");
  return ok();
}

zs_host::Scalars host_scalars(const zs_adamw_hparams* hp, const zs_state_host* sc) {
  return zs_host::step_scalars(hp->lr, hp->beta1, hp->beta2, hp->eps, hp->weight_decay, sc->loss_scale,
                               sc->clip_coef, sc->step_t);
}

size_t dtype_bytes(int dt) { return dt == ZS_FP32 ? 4 : 2; }

}  // namespace

extern "C" zs_status zs_host_adamw_step(const void* grad, zs_dtype grad_dtype, float* master, float* m, float* v,
                                        int64_t count, const zs_adamw_hparams* hp, const zs_state_host* scalars,
                                        void* param_out, zs_dtype param_dtype, int32_t n_threads) {
  const TraceRange trace("zs_host_adamw_step");
  zs_status st = check_hparams(hp);
  if (st != ZS_OK) return st;
  st = check_host_scalars(scalars);
  if (st != ZS_OK) return st;
  if (count < 0) return fail(ZS_EINVAL, "count is negative");
  if (count > 0 && (grad == nullptr || master == nullptr || m == nullptr || v == nullptr))
    return fail(ZS_EINVAL, "grad, master, m and v must not be NULL");
  if (!is_grad_dtype(grad_dtype) || !is_half_dtype(param_dtype))
    return fail(ZS_EINVAL, "grad_dtype must be bf16, fp16 or fp32 and param_dtype bf16 or fp16");
  if (!grad_aligned(grad, grad_dtype) || !grad_aligned(master, ZS_FP32) || !grad_aligned(m, ZS_FP32) ||
      !grad_aligned(v, ZS_FP32) || !grad_aligned(param_out, ZS_BF16))
    return fail(ZS_EINVAL, "arrays must be aligned to their element size");
  if (scalars->overflow != 0) return ok();  // a skipped step changes nothing
  zs_host::adamw(host_scalars(hp, scalars), grad_dtype, grad, master, m, v, param_dtype, param_out, count,
                 n_threads > 0 ? n_threads : zs_host::default_threads());
  return ok();
}

extern "C" zs_status zs_offload_adamw_step(const zs_layout* l, const void* shard, zs_dtype grad_dtype,
                                           zs_state* state, const zs_adamw_hparams* hp, float* master, float* m,
                                           float* v, void* grad_stage, void* param_stage, int64_t chunk_numel,
                                           void* flat_param_out, zs_dtype param_dtype, int32_t n_threads,
                                           void* stream) {
  const TraceRange trace("zs_offload_adamw_step");
  zs_status st = check_layout(l);
  if (st != ZS_OK) return st;
  st = check_state(l, state);
  if (st != ZS_OK) return st;
  st = check_hparams(hp);
  if (st != ZS_OK) return st;
  if (shard == nullptr || master == nullptr || m == nullptr || v == nullptr || grad_stage == nullptr ||
      param_stage == nullptr || flat_param_out == nullptr)
    return fail(ZS_EINVAL, "zs_offload_adamw_step: a required pointer is NULL");
  if (!is_grad_dtype(grad_dtype) || !is_half_dtype(param_dtype))
    return fail(ZS_EINVAL, "grad_dtype must be bf16, fp16 or fp32 and param_dtype bf16 or fp16");
  if (chunk_numel <= 0) return fail(ZS_EINVAL, "chunk_numel must be positive");
  if (!grad_aligned(shard, grad_dtype) || !grad_aligned(flat_param_out, ZS_BF16))
    return fail(ZS_EINVAL, "device arrays must be aligned to their element size");
  hipStream_t s = as_stream(stream);
  // The step's scalars: loss scale, clip coefficient, overflow flag and t, as left on the
  // device by the check and the norm.
  DevState dev{};
  hipError_t e = hipMemcpyAsync(&dev, state->dev, sizeof dev, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "reading the state");
  if (dev.h.overflow != 0) return ok();  // skipped step: the scaler update commits it
  const zs_host::Scalars k = host_scalars(hp, &dev.h);
  const int threads = n_threads > 0 ? n_threads : zs_host::default_threads();
  const int64_t S = l->plan.shard_numel;
  const int64_t nchunks = (S + chunk_numel - 1) / chunk_numel;
  const size_t gb = dtype_bytes(grad_dtype), pb = dtype_bytes(param_dtype);
  char* gstage = static_cast<char*>(grad_stage);
  char* pstage = static_cast<char*>(param_stage);
  const char* gsrc = static_cast<const char*>(shard);
  char* pdst = static_cast<char*>(flat_param_out);
  hipEvent_t ev_g[2] = {nullptr, nullptr}, ev_p[2] = {nullptr, nullptr};
  for (int i = 0; i < 2 && e == hipSuccess; ++i) {
    e = hipEventCreateWithFlags(&ev_g[i], hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&ev_p[i], hipEventDisableTiming);
  }
  auto chunk_len = [&](int64_t c) { return std::min(chunk_numel, S - c * chunk_numel); };
  auto fetch = [&](int64_t c) -> hipError_t {  // gradient chunk c into staging slot c % 2
    const int slot = static_cast<int>(c & 1);
    hipError_t r = hipMemcpyAsync(gstage + slot * chunk_numel * gb, gsrc + c * chunk_numel * gb,
                                  static_cast<size_t>(chunk_len(c)) * gb, hipMemcpyDeviceToHost, s);
    if (r == hipSuccess) r = hipEventRecord(ev_g[slot], s);
    return r;
  };
  // Double-buffered pipeline: the copy of chunk c+1 down and of chunk c-1 up run while the
  // host updates chunk c.
  std::vector<int64_t> runs;
  if (e == hipSuccess && nchunks > 0) e = fetch(0);
  for (int64_t c = 0; c < nchunks && e == hipSuccess; ++c) {
    const int slot = static_cast<int>(c & 1);
    if (c + 1 < nchunks) e = fetch(c + 1);
    if (e == hipSuccess) e = hipEventSynchronize(ev_g[slot]);
    if (e == hipSuccess && c >= 2) e = hipEventSynchronize(ev_p[slot]);  // slot's previous upload done
    if (e != hipSuccess) break;
    const int64_t off = c * chunk_numel, n = chunk_len(c);
    char* pslot = pstage + slot * chunk_numel * pb;
    // this chunk's no-decay runs, chunk-relative
    runs.clear();
    for (size_t r = 0; r + 1 < l->nodecay_runs.size(); r += 2) {
      const int64_t a = std::max(l->nodecay_runs[r], off), b = std::min(l->nodecay_runs[r + 1], off + n);
      if (a < b) {
        runs.push_back(a - off);
        runs.push_back(b - off);
      }
    }
    zs_host::adamw(k, grad_dtype, gstage + slot * chunk_numel * gb, master + off, m + off, v + off, param_dtype,
                   pslot, n, threads, runs.empty() ? nullptr : runs.data(), static_cast<int64_t>(runs.size() / 2));
    e = hipMemcpyAsync(pdst + off * pb, pslot, static_cast<size_t>(n) * pb, hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = hipEventRecord(ev_p[slot], s);
  }
  if (e == hipSuccess)
    e = hipStreamSynchronize(s);
  else
    (void)hipStreamSynchronize(s);  // no copy may still touch the caller's buffers after return
  for (int i = 0; i < 2; ++i) {
    if (ev_g[i]) (void)hipEventDestroy(ev_g[i]);
    if (ev_p[i]) (void)hipEventDestroy(ev_p[i]);
  }
  if (e != hipSuccess) return hip_fail(e, "offloaded step");
  return ok();
}

// ---------------------------------------------------------------------------- bandwidth yardsticks

namespace {

// Workgroups of a probe launch over `units` elements of kTile each: at least one, and fewer
// than 2^24 (a launch holds fewer than 2^32 work-items).
zs_status probe_units(int64_t total, int64_t unit, const char* what) {
  if (total <= 0 || total % unit != 0) return fail(ZS_EINVAL, "%s: size must be a positive multiple of %lld", what,
                                                   static_cast<long long>(unit));
  if (total / unit >= (int64_t(1) << 24)) return fail(ZS_EINVAL, "%s: size exceeds one launch", what);
  return ok();
}

}  // namespace

extern "C" zs_status zs_probe_mix(const void* g, float* p, float* m, float* v, void* out, int64_t n, void* stream) {
  if (g == nullptr || p == nullptr || m == nullptr || v == nullptr || out == nullptr)
    return fail(ZS_EINVAL, "zs_probe_mix: NULL pointer");
  if (!aligned16(g) || !aligned16(p) || !aligned16(m) || !aligned16(v) || !aligned16(out))
    return fail(ZS_EINVAL, "zs_probe_mix: pointers must be 16-byte aligned");
  zs_status st = probe_units(n, zs::kTile, "zs_probe_mix");
  if (st != ZS_OK) return st;
  hipError_t e = zs::launch_probe_mix(g, p, m, v, out, n, as_stream(stream));
  return e == hipSuccess ? ok() : hip_fail(e, "launching the mix probe");
}

extern "C" zs_status zs_probe_copy(const void* src, void* dst, int64_t bytes, void* stream) {
  if (src == nullptr || dst == nullptr) return fail(ZS_EINVAL, "zs_probe_copy: NULL pointer");
  if (!aligned16(src) || !aligned16(dst)) return fail(ZS_EINVAL, "zs_probe_copy: pointers must be 16-byte aligned");
  zs_status st = probe_units(bytes, 4 * zs::kTile, "zs_probe_copy");
  if (st != ZS_OK) return st;
  hipError_t e = zs::launch_probe_copy(src, dst, bytes, as_stream(stream));
  return e == hipSuccess ? ok() : hip_fail(e, "launching the copy probe");
}

extern "C" zs_status zs_probe_read(const void* src, int64_t bytes, uint32_t* sink, void* stream) {
  if (src == nullptr || sink == nullptr) return fail(ZS_EINVAL, "zs_probe_read: NULL pointer");
  if (!aligned16(src)) return fail(ZS_EINVAL, "zs_probe_read: src must be 16-byte aligned");
  zs_status st = probe_units(bytes, 4 * zs::kTile, "zs_probe_read");
  if (st != ZS_OK) return st;
  hipError_t e = zs::launch_probe_read(src, bytes, sink, as_stream(stream));
  return e == hipSuccess ? ok() : hip_fail(e, "launching the read probe");
}

extern "C" zs_status zs_probe_write(void* dst, int64_t bytes, void* stream) {
  if (dst == nullptr) return fail(ZS_EINVAL, "zs_probe_write: NULL pointer");
  if (!aligned16(dst)) return fail(ZS_EINVAL, "zs_probe_write: dst must be 16-byte aligned");
  zs_status st = probe_units(bytes, 4 * zs::kTile, "zs_probe_write");
  if (st != ZS_OK) return st;
  hipError_t e = zs::launch_probe_write(dst, bytes, as_stream(stream));
  return e == hipSuccess ? ok() : hip_fail(e, "launching the write probe");
}
