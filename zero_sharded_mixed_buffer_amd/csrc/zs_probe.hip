// Bandwidth yardsticks (zs_probe.h): the access patterns of the step's update kernel with
// the arithmetic taken away.  Same launch shape as k_adamw: one workgroup of 256 threads
// per 4096 elements, each thread four quads, every wave-wide access one contiguous row,
// non-temporal loads and stores.

#include "zs_internal.h"

namespace zs {
namespace {

typedef unsigned int pv4u __attribute__((ext_vector_type(4)));
typedef unsigned int pv2u __attribute__((ext_vector_type(2)));

constexpr int kProbeQuads = int(kTile / (int64_t(kThreads) * 4));  // 4

__device__ __forceinline__ pv4u ld4(const void* p) { return __builtin_nontemporal_load(static_cast<const pv4u*>(p)); }
__device__ __forceinline__ void st4(void* p, pv4u x) { __builtin_nontemporal_store(x, static_cast<pv4u*>(p)); }
__device__ __forceinline__ pv2u ld2(const void* p) { return __builtin_nontemporal_load(static_cast<const pv2u*>(p)); }
__device__ __forceinline__ void st2(void* p, pv2u x) { __builtin_nontemporal_store(x, static_cast<pv2u*>(p)); }

// Element q of quad u of this thread in the workgroup's 4096-element tile.
__device__ __forceinline__ int64_t quad_index(int u) {
  return int64_t(blockIdx.x) * kTile + int64_t(u) * (kThreads * 4) + int64_t(threadIdx.x) * 4;
}

__global__ __launch_bounds__(kThreads) void k_probe_mix(const uint16_t* __restrict__ g, uint32_t* __restrict__ p,
                                                        uint32_t* __restrict__ m, uint32_t* __restrict__ v,
                                                        uint16_t* __restrict__ out) {
  pv2u gv[kProbeQuads];
  pv4u pq[kProbeQuads], mq[kProbeQuads], vq[kProbeQuads];
#pragma unroll
  for (int u = 0; u < kProbeQuads; ++u) {
    const int64_t q = quad_index(u);
    gv[u] = ld2(g + q);
    pq[u] = ld4(p + q);
    mq[u] = ld4(m + q);
    vq[u] = ld4(v + q);
  }
#pragma unroll
  for (int u = 0; u < kProbeQuads; ++u) {
    const int64_t q = quad_index(u);
    st4(p + q, mq[u]);
    st4(m + q, vq[u]);
    st4(v + q, pq[u]);
    st2(out + q, gv[u]);
  }
}

__global__ __launch_bounds__(kThreads) void k_probe_copy(const uint32_t* __restrict__ src,
                                                         uint32_t* __restrict__ dst) {
  pv4u x[kProbeQuads];
#pragma unroll
  for (int u = 0; u < kProbeQuads; ++u) x[u] = ld4(src + quad_index(u));
#pragma unroll
  for (int u = 0; u < kProbeQuads; ++u) st4(dst + quad_index(u), x[u]);
}

__global__ __launch_bounds__(kThreads) void k_probe_read(const uint32_t* __restrict__ src,
                                                         uint32_t* __restrict__ sink) {
  uint32_t acc = 0;
#pragma unroll
  for (int u = 0; u < kProbeQuads; ++u) {
    const pv4u x = ld4(src + quad_index(u));
    acc ^= x.x ^ x.y ^ x.z ^ x.w;
  }
  if (acc == 0x9E3779B9u) *sink = acc;  // practically never; keeps the loads
}

__global__ __launch_bounds__(kThreads) void k_probe_write(uint32_t* __restrict__ dst) {
#pragma unroll
  for (int u = 0; u < kProbeQuads; ++u) st4(dst + quad_index(u), pv4u{0u, 0u, 0u, 0u});
}

}  // namespace

hipError_t launch_probe_mix(const void* g, float* p, float* m, float* v, void* out, int64_t n, hipStream_t s) {
  hipLaunchKernelGGL(k_probe_mix, dim3(static_cast<unsigned>(n / kTile)), dim3(kThreads), 0, s,
                     static_cast<const uint16_t*>(g), reinterpret_cast<uint32_t*>(p), reinterpret_cast<uint32_t*>(m),
                     reinterpret_cast<uint32_t*>(v), static_cast<uint16_t*>(out));
  return hipGetLastError();
}

hipError_t launch_probe_copy(const void* src, void* dst, int64_t bytes, hipStream_t s) {
  hipLaunchKernelGGL(k_probe_copy, dim3(static_cast<unsigned>(bytes / (kTile * 4))), dim3(kThreads), 0, s,
                     static_cast<const uint32_t*>(src), static_cast<uint32_t*>(dst));
  return hipGetLastError();
}

hipError_t launch_probe_read(const void* src, int64_t bytes, uint32_t* sink, hipStream_t s) {
  hipLaunchKernelGGL(k_probe_read, dim3(static_cast<unsigned>(bytes / (kTile * 4))), dim3(kThreads), 0, s,
                     static_cast<const uint32_t*>(src), sink);
  return hipGetLastError();
}

hipError_t launch_probe_write(void* dst, int64_t bytes, hipStream_t s) {
  hipLaunchKernelGGL(k_probe_write, dim3(static_cast<unsigned>(bytes / (kTile * 4))), dim3(kThreads), 0, s,
                     static_cast<uint32_t*>(dst));
  return hipGetLastError();
}

}  // namespace zs
