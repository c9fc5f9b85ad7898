// gfx950 kernels of the per-rank ZeRO-1/2 mixed-precision optimizer step.
//
// All kernels stream HBM: no data is reused, so the design goals are full 16-byte
// accesses per lane, whole-wave contiguous 1 KiB rows, enough independent loads in flight
// per wave, one short-lived workgroup per unit of work (the hardware dispatcher keeps
// every CU full and the tail short), non-temporal loads and stores for data nobody
// re-reads soon, and no per-tensor launches.  Tensor boundaries are resolved through a
// device segment map (zs_internal.h): a tile of 4096 flat elements that lies inside one
// tensor (every tile of a large tensor) takes a uniform fast path with one base pointer;
// when that tensor's address is not 16-byte aligned (ragged lists), the tile goes through
// LDS and is funnel-shifted into aligned 16-byte chunks.  A whole pack block that meets
// several segments loads each segment's piece into LDS (as 16-byte chunks when the block
// meets at most 16 segments) and reads its groups back; other
// tiles that meet several segments (the update's scatter, the unpack, the edges of a
// bucket's range) look each 8-element group up by binary search over the tile's few
// segments and fall back to 2-byte accesses only where a group straddles a boundary.
//
// Numerics (the pages keep master weights and Adam moments in FP32 and ask for sensitive
// reductions in higher precision - "Deep dive: Megatron", section "Precision"):
//   - the sum of squares is accumulated in fp64 from exact fp16/bf16 -> fp64 widening;
//   - the AdamW update is evaluated in fp64 (CDNA4's fp64 vector rate, half its fp32
//     rate, is far above what this HBM-bound kernel needs) and each stored fp32 value is
//     rounded once;
//   - model-dtype parameters are the round-to-nearest-even cast of the new fp32 master.
// No kernel uses atomics: every reduction has a fixed order, so results are reproducible.

#include <math.h>

#include <mutex>

#include "zs_internal.h"

namespace zs {
namespace {

// ------------------------------------------------------------------ element conversions

template <int DT>
__device__ __forceinline__ float h2f(uint32_t b);
template <>
__device__ __forceinline__ float h2f<ZS_BF16>(uint32_t b) {
  return __uint_as_float(b << 16);
}
template <>
__device__ __forceinline__ float h2f<ZS_FP16>(uint32_t b) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(b)));
}

// fp32 -> 2-byte with IEEE round-to-nearest-even (gfx950 v_cvt_pk_bf16_f32 / v_cvt_f16_f32).
template <int DT>
__device__ __forceinline__ uint32_t f2h(float f);
template <>
__device__ __forceinline__ uint32_t f2h<ZS_BF16>(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}
template <>
__device__ __forceinline__ uint32_t f2h<ZS_FP16>(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
}

// ------------------------------------------------------------------ 8-element groups

struct G16 {  // eight 2-byte values, element j in bits [16*(j&1), +16) of w[j>>1]
  uint32_t w[4];
  __device__ __forceinline__ uint32_t get(int j) const { return (w[j >> 1] >> ((j & 1) * 16)) & 0xFFFFu; }
  __device__ __forceinline__ void set(int j, uint32_t v) {
    const int sh = (j & 1) * 16;
    w[j >> 1] = (w[j >> 1] & ~(0xFFFFu << sh)) | ((v & 0xFFFFu) << sh);
  }
};

__device__ __forceinline__ G16 g16_zero() { return G16{{0u, 0u, 0u, 0u}}; }

__device__ __forceinline__ bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
__device__ __forceinline__ bool aligned8(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 7u) == 0; }

// 16-byte (and 8-byte) accesses of the streamed arrays; every bulk load and store goes
// through these.  All are non-temporal: every byte is touched once per pass, and the
// streams are read again only by the next pass or the next step, long after they would
// have left the caches.
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

__device__ __forceinline__ v4u ld_v4u(const void* p) { return __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p)); }
// The same load through a global-address-space pointer: a global (not flat) load, which the
// compiler can keep in flight across the LDS writes that follow it.
typedef __attribute__((address_space(1))) const v4u gv4u;
__device__ __forceinline__ v4u ld_v4u_global(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<gv4u*>(reinterpret_cast<uintptr_t>(p)));
}
__device__ __forceinline__ void st_v4u(void* p, v4u x) { __builtin_nontemporal_store(x, reinterpret_cast<v4u*>(p)); }
__device__ __forceinline__ v4f ld_v4f(const float* p) { return __builtin_nontemporal_load(reinterpret_cast<const v4f*>(p)); }
__device__ __forceinline__ void st_v4f(float* p, v4f x) { __builtin_nontemporal_store(x, reinterpret_cast<v4f*>(p)); }

typedef unsigned int v2u __attribute__((ext_vector_type(2)));
__device__ __forceinline__ v2u ld_v2u(const void* p) { return __builtin_nontemporal_load(reinterpret_cast<const v2u*>(p)); }
__device__ __forceinline__ void st_v2u(void* p, v2u x) { __builtin_nontemporal_store(x, reinterpret_cast<v2u*>(p)); }

__device__ __forceinline__ G16 ld16_vec(const uint16_t* p) {
  const v4u u = ld_v4u(p);
  return G16{{u.x, u.y, u.z, u.w}};
}
__device__ __forceinline__ G16 ld16_elem(const uint16_t* p, int cnt) {
  G16 g = g16_zero();
#pragma unroll
  for (int j = 0; j < kGroup; ++j)
    if (j < cnt) g.set(j, p[j]);
  return g;
}
__device__ __forceinline__ void st16_vec(uint16_t* p, const G16& g) {
  st_v4u(p, v4u{g.w[0], g.w[1], g.w[2], g.w[3]});
}
__device__ __forceinline__ void st16_elem(uint16_t* p, const G16& g, int cnt) {
#pragma unroll
  for (int j = 0; j < kGroup; ++j)
    if (j < cnt) p[j] = static_cast<uint16_t>(g.get(j));
}

// ------------------------------------------------------------------ fixed-order reductions

__device__ __forceinline__ double wave_sum(double x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

// Sum over the workgroup; the result is valid in thread 0.  Order: lanes by xor-butterfly,
// then waves 0..3 in index order.
__device__ __forceinline__ double block_sum(double x) {
  __shared__ double red[kThreads / 64];
  x = wave_sum(x);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  double r = 0.0;
  if (threadIdx.x == 0) {
#pragma unroll
    for (int i = 0; i < kThreads / 64; ++i) r += red[i];
  }
  return r;
}

// ------------------------------------------------------------------ segment map walking

// Largest segment index s in [lo, hi] with seg_begin[s] <= x.
__device__ __forceinline__ int seg_find(const DevMap& mp, int lo, int hi, int64_t x) {
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (mp.seg_begin[mid] <= x)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}

// Segment context of one tile.  When the whole tile lies in one segment, `base` maps a
// range index q straight to the tensor element (base + q), or is null for padding (and
// when no pointer table is given).
struct TileSeg {
  int lo, hi;
  bool uniform;
  uint16_t* base;
  int64_t seg_b, seg_e;  // range-relative bounds of the segment (uniform tiles)
};

// The same for `span` consecutive tiles from `tile` (a pack block of several tiles): the
// segments meeting them are tile_first[tile] .. tile_first[min(tile + span, ntiles)].
__device__ __forceinline__ TileSeg span_seg(const DevMap& mp, const uint64_t* ptrs, int64_t tile, int64_t span) {
  TileSeg t;
  const int64_t end = (tile + span < mp.ntiles) ? tile + span : mp.ntiles;
  t.lo = mp.tile_first[tile];
  t.hi = mp.tile_first[end];
  t.uniform = (t.lo == t.hi);
  t.base = nullptr;
  t.seg_b = mp.seg_begin[t.lo];
  t.seg_e = mp.seg_begin[t.lo + 1];
  if (t.uniform && ptrs != nullptr) {
    const int32_t tensor = mp.seg_tensor[t.lo];
    if (tensor >= 0) t.base = reinterpret_cast<uint16_t*>(ptrs[tensor]) + (mp.seg_local[t.lo] - t.seg_b);
  }
  return t;
}

__device__ __forceinline__ TileSeg tile_seg(const DevMap& mp, const uint64_t* ptrs, int64_t tile) {
  return span_seg(mp, ptrs, tile, 1);
}

// Elements delta .. delta+7 of the 16-element sequence a | b (a first), delta in 1..7:
// a funnel shift of 2-byte lanes across two aligned 16-byte chunks (v_alignbyte for odd
// shifts).  delta is uniform across the workgroup.
template <int D>
__device__ __forceinline__ G16 funnel16_at(uint32_t x0, uint32_t x1, uint32_t x2, uint32_t x3, uint32_t x4,
                                           uint32_t x5, uint32_t x6, uint32_t x7) {
  const uint32_t x[8] = {x0, x1, x2, x3, x4, x5, x6, x7};
  constexpr int w = D >> 1;
  G16 r;
  if constexpr ((D & 1) == 0) {
    r.w[0] = x[w]; r.w[1] = x[w + 1]; r.w[2] = x[w + 2]; r.w[3] = x[w + 3];
  } else {
    r.w[0] = __builtin_amdgcn_alignbyte(x[w + 1], x[w], 2);
    r.w[1] = __builtin_amdgcn_alignbyte(x[w + 2], x[w + 1], 2);
    r.w[2] = __builtin_amdgcn_alignbyte(x[w + 3], x[w + 2], 2);
    r.w[3] = __builtin_amdgcn_alignbyte(x[w + 4], x[w + 3], 2);
  }
  return r;
}

__device__ __forceinline__ G16 funnel16(const v4u a, const v4u b, int delta) {
  switch (delta) {
    case 1: return funnel16_at<1>(a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w);
    case 2: return funnel16_at<2>(a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w);
    case 3: return funnel16_at<3>(a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w);
    case 4: return funnel16_at<4>(a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w);
    case 5: return funnel16_at<5>(a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w);
    case 6: return funnel16_at<6>(a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w);
    default: return funnel16_at<7>(a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w);
  }
}

// Pointer to the tensor element of range index q in segment s (null for padding).
__device__ __forceinline__ uint16_t* seg_elem(const DevMap& mp, const uint64_t* ptrs, int s, int64_t q) {
  const int32_t tensor = mp.seg_tensor[s];
  if (tensor < 0) return nullptr;
  return reinterpret_cast<uint16_t*>(ptrs[tensor]) + (mp.seg_local[s] + (q - mp.seg_begin[s]));
}

// Read the cnt (<= 8) elements at range indices q.. from the tensors; padding reads as 0.
__device__ __forceinline__ G16 gather16(const DevMap& mp, const uint64_t* ptrs, const TileSeg& ts, int64_t q,
                                        int cnt) {
  const uint16_t* src;
  if (ts.uniform) {
    if (ts.base == nullptr) return g16_zero();
    src = ts.base + q;
  } else {
    int s = seg_find(mp, ts.lo, ts.hi, q);
    if (mp.seg_begin[s + 1] < q + cnt) {  // the group straddles segments
      G16 g = g16_zero();
#pragma unroll
      for (int j = 0; j < kGroup; ++j) {
        if (j >= cnt) break;
        const int64_t e = q + j;
        while (mp.seg_begin[s + 1] <= e) ++s;
        const uint16_t* p = seg_elem(mp, ptrs, s, e);
        if (p != nullptr) g.set(j, *p);
      }
      return g;
    }
    src = seg_elem(mp, ptrs, s, q);
    if (src == nullptr) return g16_zero();
  }
  if (cnt == kGroup && aligned16(src)) return ld16_vec(src);
  return ld16_elem(src, cnt);
}

// Write the cnt (<= W) elements at range indices q.. into the tensors; padding is skipped.
// W = 8: one 16-byte store when the destination allows it; W = 4: one 8-byte store.
template <int W>
__device__ __forceinline__ void scatter(const DevMap& mp, const uint64_t* ptrs, const TileSeg& ts, int64_t q,
                                        int cnt, const G16& g) {
  uint16_t* dst;
  if (ts.uniform) {
    if (ts.base == nullptr) return;
    dst = ts.base + q;
  } else {
    int s = seg_find(mp, ts.lo, ts.hi, q);
    if (mp.seg_begin[s + 1] < q + cnt) {  // the group straddles segments
#pragma unroll
      for (int j = 0; j < W; ++j) {
        if (j >= cnt) break;
        const int64_t e = q + j;
        while (mp.seg_begin[s + 1] <= e) ++s;
        uint16_t* p = seg_elem(mp, ptrs, s, e);
        if (p != nullptr) *p = static_cast<uint16_t>(g.get(j));
      }
      return;
    }
    dst = seg_elem(mp, ptrs, s, q);
    if (dst == nullptr) return;
  }
  if (W == 8 && cnt == 8 && aligned16(dst))
    st16_vec(dst, g);
  else if (W == 4 && cnt == 4 && aligned8(dst))
    st_v2u(dst, v2u{g.w[0], g.w[1]});
  else
    st16_elem(dst, g, cnt);
}

// Work unit (tile or pack block) of this workgroup among `units` in the XCD-aware order of run length RUN
// (launched with launch_units(units, RUN) workgroups); -1 for the workgroups beyond the last
// unit (fewer than one group).  The map is a bijection on the launched range.
template <int64_t RUN>
__device__ __forceinline__ int64_t ordered_unit(int64_t units) {
  const int64_t b = blockIdx.x;
  if constexpr (RUN == 0) {
    return b;
  } else if constexpr (RUN == kXcdWhole) {
    const int64_t per = (units + kXcds - 1) / kXcds;
    const int64_t u = (b % kXcds) * per + b / kXcds;
    return u < units ? u : -1;
  } else {
    constexpr int64_t group = kXcds * RUN;
    const int64_t w = b % group;
    const int64_t u = (b - w) + (w % kXcds) * RUN + w / kXcds;
    return u < units ? u : -1;
  }
}

__device__ __forceinline__ int group_count(int64_t len, int64_t q) {
  const int64_t rem = len - q;
  return rem >= kGroup ? kGroup : (rem > 0 ? static_cast<int>(rem) : 0);
}

template <int DT>
__device__ __forceinline__ double sumsq8(const G16& g) {
  double acc = 0.0;
#pragma unroll
  for (int j = 0; j < kGroup; ++j) {
    const double x = static_cast<double>(h2f<DT>(g.get(j)));
    acc += x * x;
  }
  return acc;
}

// ------------------------------------------------------------------ pack (+ fused check)

// Read the elements q+jlo .. q+jhi-1 (0 <= jlo < jhi <= 8) into positions jlo..jhi-1 of a
// group, one element at a time; nothing outside that range is read.
__device__ __forceinline__ G16 gather16_masked(const DevMap& mp, const uint64_t* ptrs, const TileSeg& ts, int64_t q,
                                               int jlo, int jhi) {
  G16 g = g16_zero();
  int s = seg_find(mp, ts.lo, ts.hi, q + jlo);
#pragma unroll
  for (int j = 0; j < kGroup; ++j) {
    if (j < jlo || j >= jhi) continue;
    const int64_t e = q + j;
    while (mp.seg_begin[s + 1] <= e) ++s;
    const uint16_t* p = seg_elem(mp, ptrs, s, e);
    if (p != nullptr) g.set(j, *p);
  }
  return g;
}

constexpr int kPackGroups = int(kPackBlock / (int64_t(kThreads) * kGroup));
constexpr int kPackChunks = int(kPackBlock / kGroup);  // 16-byte chunks of one block
// A block across at most kMixPieces segments loads its pieces as whole 16-byte chunks: a
// piece of n elements starting d elements into a chunk takes ceil((d + n) / 8) chunks, so
// the pieces of one block take at most kPackChunks + 2 * kMixPieces of them.
constexpr int kMixPieces = 16;
constexpr int kStageChunks = kPackChunks + 2 * kMixPieces;
static_assert(kStageChunks <= 3 * kThreads, "a piece's chunks take at most three loads per lane");
static_assert(kPackChunks % kThreads == 0, "the staged block's chunks split evenly over the lanes");
constexpr int kPadPiece = -(1 << 30);  // a padding piece: its elements are zero

// One block of the pack: elements [block_base, block_base + kPackBlock) of the flat range,
// of which only those in [lo, end) are read from the tensors and written.  EDGE = false
// promises that the whole block lies in [lo, end), so every group is full and needs no
// mask.  Returns this thread's share of the sum of squares of the written values (CHECK).
// `stage` (kStageChunks chunks), `wide` (kPackBlock floats) and the piece tables `mix_lo`,
// `mix_off` (kMixPieces entries) are the block's LDS.
template <int SDT, bool TO_F32, bool ACC, bool CHECK, bool EDGE>
__device__ __forceinline__ double pack_block(const DevMap& mp, const uint64_t* ptrs, void* dst, const TileSeg& ts,
                                             int64_t block_base, int64_t lo, int64_t end, v4u* stage,
                                             float* wide, int* mix_lo, int* mix_off) {
  G16 vals[kPackGroups];
  int jlos[kPackGroups];
  int cnts[kPackGroups];
  // A full block inside one tensor whose source address is not 16-byte aligned: load the
  // aligned chunks that cover it (all inside the tensor segment) through LDS and shift.
  const int delta = (ts.base != nullptr) ? int((reinterpret_cast<uintptr_t>(ts.base + block_base) >> 1) & 7) : 0;
  const bool staged = !EDGE && ts.uniform && ts.base != nullptr && delta != 0 && block_base - delta >= ts.seg_b &&
                      block_base - delta + kPackBlock + kGroup <= ts.seg_e;
  if (staged) {
    // every load issued before the first LDS write: one memory latency per block
    const v4u* chunk = reinterpret_cast<const v4u*>(ts.base + (block_base - delta));
    constexpr int kPer = kPackChunks / kThreads;
    v4u c[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) c[j] = ld_v4u_global(chunk + j * kThreads + threadIdx.x);
    v4u tail = v4u{0u, 0u, 0u, 0u};
    if (threadIdx.x == 0) tail = ld_v4u_global(chunk + kPackChunks);
#pragma unroll
    for (int j = 0; j < kPer; ++j) stage[j * kThreads + threadIdx.x] = c[j];
    if (threadIdx.x == 0) stage[kPackChunks] = tail;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kPackGroups; ++u) {
      const int k = u * kThreads + threadIdx.x;
      jlos[u] = 0;
      cnts[u] = kGroup;
      vals[u] = funnel16(stage[k], stage[k + 1], delta);
    }
  } else if (!EDGE && !ts.uniform && ts.hi - ts.lo < kMixPieces) {
    // A full block across a few segments: load each tensor piece of the block as the
    // aligned 16-byte chunks that cover it (a chunk holding any byte of the piece lies in the
    // piece's page) into LDS, one piece after the other, then give each element of a lane's
    // group the LDS element of its piece (padding reads as zero).  The block's loads stay
    // 16 bytes wide wherever its pieces start.
    const uint16_t* raw = reinterpret_cast<const uint16_t*>(stage);
    int r = 0;  // chunks loaded so far, uniform across the workgroup
    for (int pc = 0; pc <= ts.hi - ts.lo; ++pc) {  // uniform across the workgroup
      const int sg = ts.lo + pc;
      const int64_t sb = mp.seg_begin[sg], se = mp.seg_begin[sg + 1];
      const int64_t a = sb > block_base ? sb : block_base;
      const int64_t b = se < block_base + kPackBlock ? se : block_base + kPackBlock;
      const int32_t tensor = mp.seg_tensor[sg];
      int off = kPadPiece;
      if (tensor >= 0 && a < b) {
        const uint16_t* src = reinterpret_cast<const uint16_t*>(ptrs[tensor]) + mp.seg_local[sg] + (a - sb);
        const uintptr_t c0 = reinterpret_cast<uintptr_t>(src) & ~uintptr_t(15);
        const int d = int((reinterpret_cast<uintptr_t>(src) - c0) >> 1);
        const int nch = int((d + (b - a) + kGroup - 1) / kGroup);
        const v4u* chunks = reinterpret_cast<const v4u*>(c0);
        // nch <= kStageChunks < 3 * kThreads: at most three loads per lane, all issued
        // before the LDS writes
        v4u c[3];
#pragma unroll
        for (int j = 0; j < 3; ++j) {
          const int i = j * kThreads + threadIdx.x;
          if (i < nch) c[j] = ld_v4u_global(chunks + i);
        }
#pragma unroll
        for (int j = 0; j < 3; ++j) {
          const int i = j * kThreads + threadIdx.x;
          if (i < nch) stage[r + i] = c[j];
        }
        off = r * kGroup + d - int(a - block_base);  // LDS element of block element e: off + e
        r += nch;
      }
      if (threadIdx.x == 0) {
        mix_lo[pc] = int(a - block_base);
        mix_off[pc] = off;
      }
    }
    __syncthreads();
    const int np = ts.hi - ts.lo + 1;
#pragma unroll
    for (int u = 0; u < kPackGroups; ++u) {
      const int e0 = (u * kThreads + threadIdx.x) * kGroup;
      int offs[kGroup];
#pragma unroll
      for (int j = 0; j < kGroup; ++j) offs[j] = mix_off[0];
      for (int pc = 1; pc < np; ++pc) {  // uniform across the workgroup
        const int lo_p = mix_lo[pc], off_p = mix_off[pc];
#pragma unroll
        for (int j = 0; j < kGroup; ++j)
          if (e0 + j >= lo_p) offs[j] = off_p;
      }
      G16 g = g16_zero();
#pragma unroll
      for (int j = 0; j < kGroup; ++j)
        if (offs[j] != kPadPiece) g.set(j, raw[offs[j] + e0 + j]);
      jlos[u] = 0;
      cnts[u] = kGroup;
      vals[u] = g;
    }
  } else if (!EDGE && !ts.uniform) {
    // A full block across many segments: copy each segment's piece of the block into LDS in
    // element order (consecutive lanes, consecutive elements; padding as zeros), then read
    // the 8-element groups back.  One pass over the block's segments replaces a segment
    // search per group and 2-byte loads wherever a group's source is misaligned.
    uint16_t* outb = reinterpret_cast<uint16_t*>(stage);
    for (int sg = ts.lo; sg <= ts.hi; ++sg) {  // uniform across the workgroup
      const int64_t sb = mp.seg_begin[sg], se = mp.seg_begin[sg + 1];
      const int64_t a = sb > block_base ? sb : block_base;
      const int64_t b = se < block_base + kPackBlock ? se : block_base + kPackBlock;
      if (a >= b) continue;
      const int32_t tensor = mp.seg_tensor[sg];
      if (tensor < 0) {
        for (int64_t e = a + threadIdx.x; e < b; e += kThreads) outb[e - block_base] = 0;
      } else {
        const uint16_t* src = reinterpret_cast<const uint16_t*>(ptrs[tensor]) + mp.seg_local[sg] + (a - sb);
        for (int64_t e = a + threadIdx.x; e < b; e += kThreads)
          outb[e - block_base] = __builtin_nontemporal_load(src + (e - a));
      }
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kPackGroups; ++u) {
      const v4u x = stage[u * kThreads + threadIdx.x];
      jlos[u] = 0;
      cnts[u] = kGroup;
      vals[u] = G16{{x.x, x.y, x.z, x.w}};
    }
  } else {
#pragma unroll
    for (int u = 0; u < kPackGroups; ++u) {
      const int64_t q = block_base + int64_t(u * kThreads + threadIdx.x) * kGroup;
      if (!EDGE) {
        jlos[u] = 0;
        cnts[u] = kGroup;
        vals[u] = gather16(mp, ptrs, ts, q, kGroup);
        continue;
      }
      // elements [q + jlo, q + cnt) of this group lie in [lo, end)
      const int64_t a = q < lo ? lo : q;
      const int64_t b = q + kGroup < end ? q + kGroup : end;
      const int jlo = (a < b) ? static_cast<int>(a - q) : 0;
      const int cnt = (a < b) ? static_cast<int>(b - q) : 0;
      jlos[u] = jlo;
      cnts[u] = cnt;
      if (cnt <= 0)
        vals[u] = g16_zero();
      else if (jlo == 0)
        vals[u] = gather16(mp, ptrs, ts, q, cnt);
      else
        vals[u] = gather16_masked(mp, ptrs, ts, q, jlo, cnt);
    }
  }
  double acc = 0.0;
  if (TO_F32) {
    // fp32 destination: widen into LDS in element order, then move the block as
    // lane-contiguous 16-byte rows (each wave instruction covers one contiguous 1 KiB, so
    // every cache line is written - and, when accumulating, read - by one instruction).
#pragma unroll
    for (int u = 0; u < kPackGroups; ++u) {
      const int e = (u * kThreads + threadIdx.x) * kGroup;
#pragma unroll
      for (int j = 0; j < kGroup; ++j) wide[e + j] = h2f<SDT>(vals[u].get(j));
    }
    __syncthreads();
    float* d = static_cast<float*>(dst) + block_base;
    const int64_t elo = lo - block_base;  // block-relative kept range [elo, ehi)
    const int64_t ehi = end - block_base;
    constexpr int kRows = int(kPackBlock / (int64_t(kThreads) * 4));
#pragma unroll
    for (int i = 0; i < kRows; ++i) {
      const int e = i * kThreads * 4 + threadIdx.x * 4;
      int jlo = 0, cnt = 4;
      if (EDGE) {
        const int64_t a = e < elo ? elo : e;
        const int64_t b = e + 4 < ehi ? e + 4 : ehi;
        if (a >= b) continue;
        jlo = static_cast<int>(a - e);
        cnt = static_cast<int>(b - e);
      }
      const bool full = !EDGE || (jlo == 0 && cnt == 4);
      float f[4] = {wide[e], wide[e + 1], wide[e + 2], wide[e + 3]};
      if (ACC) {  // one fp32 add: the exact sum rounded once
        if (full) {
          const v4f o = ld_v4f(d + e);
          f[0] += o.x; f[1] += o.y; f[2] += o.z; f[3] += o.w;
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (j >= jlo && j < cnt) f[j] += d[e + j];
        }
      }
      if (CHECK) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const double x = static_cast<double>(f[j]);
          acc += (j >= jlo && j < cnt) ? x * x : 0.0;
        }
      }
      if (full) {
        st_v4f(d + e, v4f{f[0], f[1], f[2], f[3]});
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (j >= jlo && j < cnt) d[e + j] = f[j];
      }
    }
  } else {
#pragma unroll
    for (int u = 0; u < kPackGroups; ++u) {
      const int cnt = cnts[u], jlo = jlos[u];
      if (EDGE && cnt <= 0) continue;
      const bool full = !EDGE || (jlo == 0 && cnt == kGroup);
      const int64_t q = block_base + int64_t(u * kThreads + threadIdx.x) * kGroup;
      uint16_t* d = static_cast<uint16_t*>(dst) + q;
      G16 out = vals[u];
      if (ACC) {  // fp32 add, then one rounding to the 2-byte dtype (the fp32 sum of two
                  // 2-byte values rounds innocuously: fp32 has > 2p+2 significand bits)
        G16 old = g16_zero();
        if (full) {
          old = ld16_vec(d);
        } else {
#pragma unroll
          for (int j = 0; j < kGroup; ++j)
            if (j >= jlo && j < cnt) old.set(j, d[j]);
        }
#pragma unroll
        for (int j = 0; j < kGroup; ++j) out.set(j, f2h<SDT>(h2f<SDT>(old.get(j)) + h2f<SDT>(vals[u].get(j))));
      }
      if (CHECK) acc += sumsq8<SDT>(out);
      if (full) {
        st16_vec(d, out);
      } else {
#pragma unroll
        for (int j = 0; j < kGroup; ++j)
          if (j >= jlo && j < cnt) d[j] = static_cast<uint16_t>(out.get(j));
      }
    }
  }
  return acc;
}

// Gather the tensors into the flat range; padding becomes zero.  kPackBlock elements per
// workgroup (one 8-element group per thread); workgroup b handles block blk0 + b, and only
// flat elements in [lo, hi) are read from the tensors and written (a whole pack passes
// 0, 0, len; a bucket passes its own range).  TO_F32: widen to fp32 (master seeding, fp32
// accumulation buffers).  ACC: add to the buffer instead of overwriting it.  CHECK: also
// write the fp64 sum of squares of this block's resulting values to partials[blockIdx.x]
// (a non-finite element makes that sum non-finite); used only for whole packs.
template <int SDT, bool TO_F32, bool ACC, bool CHECK>
__global__ __launch_bounds__(kThreads) void k_pack(DevMap mp, const uint64_t* __restrict__ ptrs,
                                                   void* __restrict__ dst, double* __restrict__ partials,
                                                   int64_t blk0, int64_t nblk, int64_t lo, int64_t hi) {
  __shared__ v4u stage[kStageChunks];
  __shared__ float wide[TO_F32 ? kPackBlock : 1];
  __shared__ int mix_lo[kMixPieces], mix_off[kMixPieces];
  const int64_t unit = ordered_unit<kXcdRunPack>(nblk);
  if (unit < 0) return;  // uniform across the workgroup
  const int64_t block_base = (blk0 + unit) * kPackBlock;
  const int64_t end = hi < mp.len ? hi : mp.len;
  static_assert(kPackBlock % kTile == 0, "a pack block covers whole tiles");
  const TileSeg ts = span_seg(mp, ptrs, block_base / kTile, kPackBlock / kTile);
  // uniform across the workgroup: no element of the block is clipped
  const bool whole = block_base >= lo && block_base + kPackBlock <= end;
  const double acc = whole
      ? pack_block<SDT, TO_F32, ACC, CHECK, false>(mp, ptrs, dst, ts, block_base, lo, end, stage, wide, mix_lo,
                                                    mix_off)
      : pack_block<SDT, TO_F32, ACC, CHECK, true>(mp, ptrs, dst, ts, block_base, lo, end, stage, wide, mix_lo,
                                                   mix_off);
  if (CHECK) {
    const double r = block_sum(acc);
    if (threadIdx.x == 0) partials[unit] = r;
  }
}

// ------------------------------------------------------------------ check (sum of squares)

template <int DT>
__global__ __launch_bounds__(kThreads) void k_check(const uint16_t* __restrict__ shard, int64_t n,
                                                    double* __restrict__ partials) {
  constexpr int kPackGroups = int(kPackBlock / (int64_t(kThreads) * kGroup));
  const int64_t unit = ordered_unit<kXcdRunCheck>(reduction_blocks(n));
  if (unit < 0) return;  // uniform across the workgroup
  const bool vec_ok = aligned16(shard);
  G16 vals[kPackGroups];
  if (vec_ok && (unit + 1) * kPackBlock <= n) {  // uniform: a full aligned block, loads issued together
    v4u c[kPackGroups];
#pragma unroll
    for (int u = 0; u < kPackGroups; ++u)
      c[u] = ld_v4u_global(shard + unit * kPackBlock + int64_t(u * kThreads + threadIdx.x) * kGroup);
#pragma unroll
    for (int u = 0; u < kPackGroups; ++u) vals[u] = G16{{c[u].x, c[u].y, c[u].z, c[u].w}};
  } else {
#pragma unroll
    for (int u = 0; u < kPackGroups; ++u) {
      const int64_t q = unit * kPackBlock + int64_t(u * kThreads + threadIdx.x) * kGroup;
      const int cnt = group_count(n, q);
      vals[u] = (cnt == kGroup && vec_ok) ? ld16_vec(shard + q) : ld16_elem(shard + q, cnt);
    }
  }
  double acc = 0.0;
#pragma unroll
  for (int u = 0; u < kPackGroups; ++u) acc += sumsq8<DT>(vals[u]);
  const double r = block_sum(acc);
  if (threadIdx.x == 0) partials[unit] = r;
}

// The same pass over an fp32 shard (a gradient-accumulation buffer).
__global__ __launch_bounds__(kThreads) void k_check_f32(const float* __restrict__ shard, int64_t n,
                                                        double* __restrict__ partials) {
  constexpr int kPackGroups = int(kPackBlock / (int64_t(kThreads) * kGroup));
  const int64_t unit = ordered_unit<kXcdRunCheck>(reduction_blocks(n));
  if (unit < 0) return;  // uniform across the workgroup
  const bool vec_ok = aligned16(shard);
  double acc = 0.0;
#pragma unroll
  for (int u = 0; u < kPackGroups; ++u) {
    const int64_t q = unit * kPackBlock + int64_t(u * kThreads + threadIdx.x) * kGroup;
    const int cnt = group_count(n, q);
    float f[kGroup] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (cnt == kGroup && vec_ok) {
      const v4f a = ld_v4f(shard + q), b = ld_v4f(shard + q + 4);
      f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
      f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
    } else {
#pragma unroll
      for (int j = 0; j < kGroup; ++j)
        if (j < cnt) f[j] = shard[q + j];
    }
#pragma unroll
    for (int j = 0; j < kGroup; ++j) {
      const double x = static_cast<double>(f[j]);
      acc += x * x;
    }
  }
  const double r = block_sum(acc);
  if (threadIdx.x == 0) partials[unit] = r;
}

// First level of the fixed-order reduction of many partial sums: workgroup b adds
// partials [b*per, min((b+1)*per, n)) and writes level2[b].
__global__ __launch_bounds__(kThreads) void k_partial_reduce(const double* __restrict__ partials, int64_t n,
                                                             int64_t per, double* __restrict__ level2) {
  const int64_t b0 = int64_t(blockIdx.x) * per;
  const int64_t b1 = (b0 + per < n) ? b0 + per : n;
  double acc = 0.0;
  for (int64_t i = b0 + threadIdx.x; i < b1; i += kThreads) acc += partials[i];
  const double r = block_sum(acc);
  if (threadIdx.x == 0) level2[blockIdx.x] = r;
}

// ------------------------------------------------------------------ finalize kernels

// The fixed-order sum of n partials by one workgroup: per-thread strided sums, then
// block_sum.  The result is valid in thread 0.
__device__ __forceinline__ double fold_partials(const double* __restrict__ partials, int64_t n) {
  double acc = 0.0;
  for (int64_t i = threadIdx.x; i < n; i += kThreads) acc += partials[i];
  return block_sum(acc);
}

// The overflow flag and this rank's unscaled sum of squares from the raw (scaled) sum of
// squares.  Every element is finite iff the sum is finite: a finite fp16/bf16 square is
// below 2^256 and at most 2^63 of them stay far below the fp64 range, while inf or NaN
// anywhere propagates to the sum.
__device__ __forceinline__ void flag_commit(DevState* st, double raw, const int32_t* ext, int mode,
                                            double* local_out) {
  const bool bad = !isfinite(raw);
  const bool other = (ext != nullptr) && (*ext != 0);
  if (mode == kFlagSet)
    st->h.overflow = (bad || other) ? 1 : 0;
  else if (bad)
    st->h.overflow = 1;
  st->raw_sumsq = raw;
  const double inv = 1.0 / st->h.loss_scale;  // exact: the scale is a power of two
  const double local = (raw * inv) * inv;
  st->h.local_sumsq = local;
  if (local_out != nullptr) *local_out = local;
}

// Global sum of squares in rank order, norm and clip coefficient.  A non-finite partial from
// any rank (its overflow) makes the global sum non-finite and sets the flag.
__device__ __forceinline__ void norm_commit(DevState* st, const double* rank_sumsq, int dp_world, int dp_rank,
                                            double* local_out, double max_norm) {
  const double local = st->h.local_sumsq;
  double ss = 0.0;
  for (int q = 0; q < dp_world; ++q) ss += (q == dp_rank) ? local : rank_sumsq[q];
  if (!isfinite(ss)) st->h.overflow = 1;
  const double norm = sqrt(ss);
  double c = 1.0;
  if (max_norm > 0.0) {
    const double r = max_norm / (norm + 1e-6);
    c = (r < 1.0) ? r : 1.0;
  }
  st->h.sumsq = ss;
  st->h.grad_norm = norm;
  st->h.clip_coef = c;
  if (local_out != nullptr) *local_out = local;
}

// Commit the step in the loss scaler: an overflowed step is skipped and halves a dynamic
// scale (not below the floor); an applied one counts and doubles the scale after
// growth_interval of them.
__device__ __forceinline__ void scaler_commit(DevState* st) {
  zs_state_host h = st->h;
  if (h.overflow) {
    h.skipped_total += 1;
    h.growth_tracker = 0;
    if (h.dynamic) {
      const double halved = h.loss_scale * 0.5;
      h.loss_scale = (halved < h.scale_floor) ? h.scale_floor : halved;
    }
  } else {
    h.step_t += 1;
    if (h.dynamic) {
      h.growth_tracker += 1;
      if (h.growth_tracker >= h.growth_interval) {
        h.loss_scale *= 2.0;
        h.growth_tracker = 0;
      }
    }
  }
  st->h = h;
}

// One workgroup: add the block partials in a fixed order, set the overflow flag and this
// rank's unscaled sum of squares.
__global__ __launch_bounds__(kThreads) void k_flag_finalize(const double* __restrict__ partials, int64_t nparts,
                                                            DevState* __restrict__ st,
                                                            const int32_t* __restrict__ ext, int mode,
                                                            double* __restrict__ local_out) {
  const double raw = fold_partials(partials, nparts);
  if (threadIdx.x == 0) flag_commit(st, raw, ext, mode, local_out);
}

// One thread: global sum of squares in rank order, norm and clip coefficient.
__global__ void k_norm_finalize(DevState* __restrict__ st, const double* __restrict__ rank_sumsq, int dp_world,
                                int dp_rank, double* __restrict__ local_out, double max_norm) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  norm_commit(st, rank_sumsq, dp_world, dp_rank, local_out, max_norm);
}

// One thread: commit the step in the loss scaler.
__global__ void k_scaler_update(DevState* __restrict__ st) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  scaler_commit(st);
}

// The single-rank step's three finalizers in one workgroup: the flag and local sum of
// squares, the norm and clip coefficient, then the scaler commit.  The state as it stands
// before the commit (the flag, clip coefficient, scale and step count that the update
// needs) is copied to `pre` first, and the AdamW launch that follows reads `pre`.
__global__ __launch_bounds__(kThreads) void k_step_finalize(const double* __restrict__ partials, int64_t nparts,
                                                            DevState* __restrict__ st, DevState* __restrict__ pre,
                                                            double max_norm) {
  const double raw = fold_partials(partials, nparts);
  if (threadIdx.x == 0) {
    flag_commit(st, raw, nullptr, kFlagSet, nullptr);
    norm_commit(st, nullptr, 1, 0, nullptr, max_norm);
    *pre = *st;
    scaler_commit(st);
  }
}

// The same finalize for a state that lives in the caller's memory as a bare zs_state_host
// (the allocation-free step): the state is read, finalized and committed in registers, the
// pre-commit copy goes to `pre` and the committed fields back to the caller.
__global__ __launch_bounds__(kThreads) void k_step_finalize_ext(const double* __restrict__ partials, int64_t nparts,
                                                                zs_state_host* __restrict__ st,
                                                                DevState* __restrict__ pre, double max_norm) {
  const double raw = fold_partials(partials, nparts);
  if (threadIdx.x == 0) {
    DevState d{};
    d.h = *st;
    flag_commit(&d, raw, nullptr, kFlagSet, nullptr);
    norm_commit(&d, nullptr, 1, 0, nullptr, max_norm);
    *pre = d;
    scaler_commit(&d);
    *st = d.h;
  }
}

// ------------------------------------------------------------------ AdamW + cast + scatter

// Per-step scalars, evaluated in fp64 by every workgroup from the device state.
struct StepScalars {
  double gs, b1, omb1, b2, omb2, a, rbc2, eps, decay;
};

__device__ __forceinline__ StepScalars step_scalars(const AdamwArgs& hp, const DevState* st) {
  StepScalars k;
  const double t = static_cast<double>(st->h.step_t + 1);
  k.gs = st->h.clip_coef / st->h.loss_scale;  // unscale and clip in one exact-by-construction factor
  k.b1 = hp.beta1;
  k.omb1 = 1.0 - hp.beta1;
  k.b2 = hp.beta2;
  k.omb2 = 1.0 - hp.beta2;
  k.a = hp.lr / (1.0 - pow(hp.beta1, t));
  k.rbc2 = 1.0 / (1.0 - pow(hp.beta2, t));
  k.eps = hp.eps;
  k.decay = 1.0 - hp.lr * hp.weight_decay;
  return k;
}

// One element: returns the new (p, m, v) as fp32.  `decay` is the decoupled weight-decay
// multiplier, 1 - lr * wd, or 1 for a tensor without weight decay.
__device__ __forceinline__ void adamw_elem(const StepScalars& k, double decay, float x, float& p, float& m,
                                           float& v) {
#pragma clang fp contract(off)
  const double g = static_cast<double>(x) * k.gs;
  const float m1 = static_cast<float>(k.b1 * static_cast<double>(m) + k.omb1 * g);
  const float v1 = static_cast<float>(k.b2 * static_cast<double>(v) + k.omb2 * (g * g));
  const double den = sqrt(static_cast<double>(v1) * k.rbc2) + k.eps;
  const double upd = k.a * static_cast<double>(m1) / den;
  p = static_cast<float>(static_cast<double>(p) * decay - upd);
  m = m1;
  v = v1;
}

// Quad layout: a workgroup owns one 4096-element tile; thread t handles the four-element
// quads starting at base + u*1024 + 4t for u < 4.  Every wave-wide access of the fp32
// arrays is then one contiguous 1 KiB row (16 bytes per lane) and every access of the
// 2-byte arrays a contiguous 512-byte row (8 bytes per lane), so each instruction covers
// whole cache lines; with the 8-element layout a 16-byte fp32 access per lane left every
// line half-written by two instructions, which the non-temporal write path turned into
// 6 % extra HBM write traffic.
constexpr int kQuadsPerThread = int(kTile / (int64_t(kThreads) * 4));

// Four gradient values of one quad, as fp32 (exact for every input dtype).
template <int GDT>
__device__ __forceinline__ v4f load_grad4(const void* shard, int64_t q, int cnt, bool vec) {
  if constexpr (GDT == ZS_FP32) {
    const float* g = static_cast<const float*>(shard) + q;
    if (cnt == 4 && vec) return ld_v4f(g);
    float t[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (j < cnt) t[j] = g[j];
    return v4f{t[0], t[1], t[2], t[3]};
  } else {
    const uint16_t* g = static_cast<const uint16_t*>(shard) + q;
    G16 x;
    if (cnt == 4 && vec) {
      const v2u w = ld_v2u(g);
      x = G16{{w.x, w.y, 0u, 0u}};
    } else {
      x = ld16_elem(g, cnt < 4 ? cnt : 4);
    }
    return v4f{h2f<GDT>(x.get(0)), h2f<GDT>(x.get(1)), h2f<GDT>(x.get(2)), h2f<GDT>(x.get(3))};
  }
}

// GROUPS: the map carries no-decay flags (a separate instantiation, so that the common
// single-group kernel keeps its registers).  SPLIT: workgroups per tile, each taking
// kTile / SPLIT consecutive elements (one quad per thread at SPLIT = 4).  A small shard
// runs split: its few tiles would otherwise sit on a few CUs, each thread working through
// four quads of fp64 arithmetic in turn.
template <int GDT, int PDT, bool SCATTER, bool FLAT_OUT, bool GROUPS, int SPLIT>
__global__ __launch_bounds__(kThreads) void k_adamw(DevMap mp, const void* __restrict__ shard,
                                                    float* __restrict__ master, float* __restrict__ mom1,
                                                    float* __restrict__ mom2, AdamwArgs hp,
                                                    const DevState* __restrict__ st,
                                                    const uint64_t* __restrict__ ptrs,
                                                    uint16_t* __restrict__ flat_out) {
  static_assert(SPLIT == 1 || SPLIT == kQuadsPerThread, "a split workgroup takes one quad per thread");
  constexpr int kQuads = kQuadsPerThread / SPLIT;
  if (st->h.overflow) return;  // device-side skip: nothing changes on an overflowed step
  const StepScalars k = step_scalars(hp, st);
  const bool g_vec = (GDT == ZS_FP32) ? aligned16(shard) : aligned8(shard);
  const int64_t n = mp.len;
  const int64_t unit = ordered_unit<SPLIT == 1 ? kXcdRunAdamw : 0>(mp.ntiles * SPLIT);
  if (unit < 0) return;  // uniform across the workgroup
  const int64_t tile = unit / SPLIT;
  const int64_t base = tile * kTile + (unit % SPLIT) * (kTile / SPLIT);
  v4f gv[kQuads];
  v4f pv[kQuads], mv[kQuads], vv[kQuads];
  int cnts[kQuads];
#pragma unroll
  for (int u = 0; u < kQuads; ++u) {
    const int64_t q = base + int64_t(u) * (kThreads * 4) + int64_t(threadIdx.x) * 4;
    const int64_t rem = n - q;
    const int cnt = rem >= 4 ? 4 : (rem > 0 ? static_cast<int>(rem) : 0);
    cnts[u] = cnt;
    gv[u] = load_grad4<GDT>(shard, q, cnt, g_vec);
    if (cnt == 4) {
      pv[u] = ld_v4f(master + q);
      mv[u] = ld_v4f(mom1 + q);
      vv[u] = ld_v4f(mom2 + q);
    } else {
      float pt[4] = {0.f, 0.f, 0.f, 0.f}, mt[4] = {0.f, 0.f, 0.f, 0.f}, vt[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (j < cnt) {
          pt[j] = master[q + j];
          mt[j] = mom1[q + j];
          vt[j] = mom2[q + j];
        }
      }
      pv[u] = v4f{pt[0], pt[1], pt[2], pt[3]};
      mv[u] = v4f{mt[0], mt[1], mt[2], mt[3]};
      vv[u] = v4f{vt[0], vt[1], vt[2], vt[3]};
    }
  }
  // No-decay tensors: one multiplier for a tile inside one segment, else per element.
  constexpr bool groups = GROUPS;
  TileSeg ts{};
  if (SCATTER || groups) ts = tile_seg(mp, SCATTER ? ptrs : nullptr, tile);
  const double tile_decay = (groups && ts.uniform && mp.seg_nodecay[ts.lo]) ? 1.0 : k.decay;
  // A full tile inside one parameter tensor whose address is not 16-byte aligned (ragged
  // lists): the cast parameters go through LDS and leave as destination-aligned 16-byte
  // chunks; only the at most 15 elements at the two ends of the tile are written singly.
  __shared__ uint32_t pstage[SPLIT == 1 ? kTile / 2 : 1];
  int pdelta = 0;
  if (SPLIT == 1 && SCATTER && ts.uniform && ts.base != nullptr && base + kTile <= n)
    pdelta = int((reinterpret_cast<uintptr_t>(ts.base + base) >> 1) & 7);
  // The quads of the tile; PER_ELEM (a tile across segments with no-decay flags, rare) looks
  // each element's decay up, every other tile uses the tile's one multiplier.
  auto update_quads = [&](auto per_elem) {
    constexpr bool PER_ELEM = decltype(per_elem)::value;
#pragma unroll
    for (int u = 0; u < kQuads; ++u) {
      const int cnt = cnts[u];
      if (cnt <= 0) continue;
      const int64_t q = base + int64_t(u) * (kThreads * 4) + int64_t(threadIdx.x) * 4;
      float p[4], m[4], v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        p[j] = pv[u][j];
        m[j] = mv[u][j];
        v[j] = vv[u][j];
      }
      double dec[4] = {tile_decay, tile_decay, tile_decay, tile_decay};
      if constexpr (PER_ELEM) {
        int s = seg_find(mp, ts.lo, ts.hi, q);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (j >= cnt) break;
          while (mp.seg_begin[s + 1] <= q + j) ++s;
          dec[j] = mp.seg_nodecay[s] ? 1.0 : k.decay;
        }
      }
      G16 out = g16_zero();
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        adamw_elem(k, dec[j], gv[u][j], p[j], m[j], v[j]);
        out.set(j, f2h<PDT>(p[j]));
      }
      if (cnt == 4) {
        st_v4f(master + q, v4f{p[0], p[1], p[2], p[3]});
        st_v4f(mom1 + q, v4f{m[0], m[1], m[2], m[3]});
        st_v4f(mom2 + q, v4f{v[0], v[1], v[2], v[3]});
        if (FLAT_OUT) st_v2u(flat_out + q, v2u{out.w[0], out.w[1]});
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (j < cnt) {
            master[q + j] = p[j];
            mom1[q + j] = m[j];
            mom2[q + j] = v[j];
          }
        }
        if (FLAT_OUT) st16_elem(flat_out + q, out, cnt);
      }
      if (SCATTER) {
        if (SPLIT == 1 && pdelta != 0) {
          const int e = u * kThreads * 4 + threadIdx.x * 4;  // tile-relative; cnt == 4 here
          pstage[e / 2] = out.w[0];
          pstage[e / 2 + 1] = out.w[1];
        } else {
          scatter<4>(mp, ptrs, ts, q, cnt, out);
        }
      }
    }
  };
  if (groups && !ts.uniform)  // uniform across the workgroup
    update_quads(std::true_type{});
  else
    update_quads(std::false_type{});
  if (SPLIT == 1 && SCATTER && pdelta != 0) {  // uniform across the workgroup
    __syncthreads();
    const v4u* L = reinterpret_cast<const v4u*>(pstage);
    uint16_t* D = ts.base + base;            // destination of tile element 0
    const int e0 = (8 - pdelta) & 7;         // first tile element at a 16-byte boundary
    constexpr int kFull = int(kTile / kGroup) - 1;  // aligned chunks fully inside the tile
    for (int c = threadIdx.x; c < kFull; c += kThreads)
      st16_vec(D + e0 + c * kGroup, funnel16(L[c], L[c + 1], e0));
    if (threadIdx.x < kGroup) {            // head [0, e0) and tail [e0 + 8*kFull, kTile)
      const uint16_t* P = reinterpret_cast<const uint16_t*>(pstage);
      const int h = threadIdx.x;
      if (h < e0) D[h] = P[h];
      const int t = e0 + kFull * kGroup + h;
      if (t < kTile) D[t] = P[t];
    }
  }
}

// ------------------------------------------------------------------ unpack (scatter-back)

// SRC_F32: the source is the fp32 master (cast RNE to DDT); otherwise a DDT flat buffer
// (bit copy).  A set overflow flag in `skip` makes the kernel a no-op.
template <bool SRC_F32, int DDT>
__global__ __launch_bounds__(kThreads) void k_unpack(DevMap mp, const void* __restrict__ src,
                                                     const DevState* __restrict__ skip,
                                                     const uint64_t* __restrict__ ptrs) {
  if (skip != nullptr && skip->h.overflow) return;
  const int64_t tile = ordered_unit<kXcdRunUnpack>(mp.ntiles);
  if (tile < 0) return;  // uniform across the workgroup
  const bool vec_ok = aligned16(src);
  {
    const TileSeg ts = tile_seg(mp, ptrs, tile);
    const int64_t base = tile * kTile;
    G16 vals[kUnroll];
    int cnts[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t q = base + int64_t(u * kThreads + threadIdx.x) * kGroup;
      const int cnt = group_count(mp.len, q);
      cnts[u] = cnt;
      vals[u] = g16_zero();
      if (cnt <= 0) continue;
      if (SRC_F32) {
        const float* s = static_cast<const float*>(src) + q;
        float f[kGroup] = {0.f};
        if (cnt == kGroup) {
          const v4f a = ld_v4f(s);
          const v4f b = ld_v4f(s + 4);
          f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
          f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
        } else {
#pragma unroll
          for (int j = 0; j < kGroup; ++j)
            if (j < cnt) f[j] = s[j];
        }
#pragma unroll
        for (int j = 0; j < kGroup; ++j) vals[u].set(j, f2h<DDT>(f[j]));
      } else {
        const uint16_t* s = static_cast<const uint16_t*>(src) + q;
        vals[u] = (cnt == kGroup && vec_ok) ? ld16_vec(s) : ld16_elem(s, cnt);
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (cnts[u] <= 0) continue;
      const int64_t q = base + int64_t(u * kThreads + threadIdx.x) * kGroup;
      scatter<kGroup>(mp, ptrs, ts, q, cnts[u], vals[u]);
    }
  }
}

}  // namespace

// ------------------------------------------------------------------ launchers

template <int SDT>
static void pack_dispatch(const dim3& G, hipStream_t s, const DevMap& map, const uint64_t* src_ptrs, void* dst,
                          bool f32, bool acc, double* partials, int64_t blk0, int64_t nblk, int64_t lo, int64_t hi) {
  const dim3 B(kThreads);
  const bool chk = (partials != nullptr);
#define ZS_PACK(F, A, C) \
  hipLaunchKernelGGL((k_pack<SDT, F, A, C>), G, B, 0, s, map, src_ptrs, dst, partials, blk0, nblk, lo, hi)
  if (f32) {
    if (acc) {
      if (chk) ZS_PACK(true, true, true); else ZS_PACK(true, true, false);
    } else {
      if (chk) ZS_PACK(true, false, true); else ZS_PACK(true, false, false);
    }
  } else {
    if (acc) {
      if (chk) ZS_PACK(false, true, true); else ZS_PACK(false, true, false);
    } else {
      if (chk) ZS_PACK(false, false, true); else ZS_PACK(false, false, false);
    }
  }
#undef ZS_PACK
}

hipError_t launch_pack(const DevMap& map, const uint64_t* src_ptrs, int src_dt, void* dst, int dst_dt, bool accumulate,
                       double* partials, hipStream_t s, int64_t lo, int64_t hi) {
  if (hi < 0) hi = map.len;
  if (hi <= lo) return hipSuccess;
  const int64_t blk0 = lo / kPackBlock;
  const int64_t nb = (hi + kPackBlock - 1) / kPackBlock - blk0;
  if (nb <= 0) return hipSuccess;
  const dim3 G(static_cast<unsigned>(launch_units(nb, kXcdRunPack)));
  const bool f32 = (dst_dt == ZS_FP32);
  if (src_dt == ZS_BF16)
    pack_dispatch<ZS_BF16>(G, s, map, src_ptrs, dst, f32, accumulate, partials, blk0, nb, lo, hi);
  else
    pack_dispatch<ZS_FP16>(G, s, map, src_ptrs, dst, f32, accumulate, partials, blk0, nb, lo, hi);
  return hipGetLastError();
}

hipError_t launch_check(const void* shard, int64_t n, int dt, double* partials, hipStream_t s) {
  const int64_t nb = reduction_blocks(n);
  if (nb == 0) return hipSuccess;
  const uint16_t* p = static_cast<const uint16_t*>(shard);
  const dim3 G(static_cast<unsigned>(launch_units(nb, kXcdRunCheck))), B(kThreads);
  if (dt == ZS_BF16)
    hipLaunchKernelGGL((k_check<ZS_BF16>), G, B, 0, s, p, n, partials);
  else if (dt == ZS_FP16)
    hipLaunchKernelGGL((k_check<ZS_FP16>), G, B, 0, s, p, n, partials);
  else
    hipLaunchKernelGGL(k_check_f32, G, B, 0, s, static_cast<const float*>(shard), n, partials);
  return hipGetLastError();
}

// Up to 16 partials per thread go straight to the single finalize workgroup; more are
// first folded by up to kLevel2 workgroups, each over a contiguous range, in fixed order.
// Returns the launch status; *partials / *nparts then name what the finalize folds.
static hipError_t reduce_level2(const double** partials, int64_t* nparts, double* level2, hipStream_t s) {
  if (*nparts <= int64_t(kThreads) * 16) return hipSuccess;
  const int64_t per0 = (*nparts + kLevel2 - 1) / kLevel2;
  const int64_t per = per0 < int64_t(kThreads) * 4 ? int64_t(kThreads) * 4 : per0;
  const int64_t nb = (*nparts + per - 1) / per;
  hipLaunchKernelGGL(k_partial_reduce, dim3(static_cast<unsigned>(nb)), dim3(kThreads), 0, s, *partials, *nparts,
                     per, level2);
  *partials = level2;
  *nparts = nb;
  return hipGetLastError();
}

hipError_t launch_reduce_finalize(const double* partials, int64_t nparts, double* level2, DevState* st,
                                  const int32_t* ext, int mode, double* local_out, hipStream_t s) {
  hipError_t e = reduce_level2(&partials, &nparts, level2, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_flag_finalize, dim3(1), dim3(kThreads), 0, s, partials, nparts, st, ext, mode, local_out);
  return hipGetLastError();
}

hipError_t launch_step_finalize(const double* partials, int64_t nparts, double* level2, DevState* st,
                                DevState* pre, double max_norm, hipStream_t s) {
  hipError_t e = reduce_level2(&partials, &nparts, level2, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_step_finalize, dim3(1), dim3(kThreads), 0, s, partials, nparts, st, pre, max_norm);
  return hipGetLastError();
}

hipError_t launch_step_finalize_ext(const double* partials, int64_t nparts, double* level2, zs_state_host* st,
                                    DevState* pre, double max_norm, hipStream_t s) {
  hipError_t e = reduce_level2(&partials, &nparts, level2, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_step_finalize_ext, dim3(1), dim3(kThreads), 0, s, partials, nparts, st, pre, max_norm);
  return hipGetLastError();
}

// Scratch of the allocation-free step, one copy per GPU for the life of the process: the
// pre-commit state, the second-level partial sums, then one first-level partial sum per
// check workgroup.  Every slot a call reads was written earlier in the same call, so nothing
// needs clearing between calls.
constexpr int64_t kNoAllocPre = 32;  // doubles reserved for the pre-commit DevState
static_assert(sizeof(DevState) <= kNoAllocPre * sizeof(double), "pre-commit state slot too small");
constexpr int64_t kNoAllocDoubles = kNoAllocPre + kLevel2 + kNoAllocMaxParts;
static __device__ __align__(256) double scratch[kNoAllocDoubles];

hipError_t noalloc_scratch(NoAllocScratch* out) {
  // The array's name is a host-side stand-in: its device address comes from the runtime, once
  // per device, with that device current.
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = nullptr;
  {
    std::lock_guard<std::mutex> lock(mu);
    if (addr[dev] == nullptr) {
      e = hipGetSymbolAddress(&addr[dev], HIP_SYMBOL(scratch));
      if (e != hipSuccess) {
        addr[dev] = nullptr;
        return e;
      }
    }
    p = addr[dev];
  }
  double* d = static_cast<double*>(p);
  out->pre = reinterpret_cast<DevState*>(d);
  out->level2 = d + kNoAllocPre;
  out->partials = d + kNoAllocPre + kLevel2;
  return hipSuccess;
}

hipError_t launch_norm_finalize(DevState* st, const double* rank_sumsq, int dp_world, int dp_rank,
                                double* local_out, double max_norm, hipStream_t s) {
  hipLaunchKernelGGL(k_norm_finalize, dim3(1), dim3(64), 0, s, st, rank_sumsq, dp_world, dp_rank, local_out,
                     max_norm);
  return hipGetLastError();
}

hipError_t launch_scaler_update(DevState* st, hipStream_t s) {
  hipLaunchKernelGGL(k_scaler_update, dim3(1), dim3(64), 0, s, st);
  return hipGetLastError();
}

template <int GDT, int PDT, bool GROUPS, int SPLIT>
static void adamw_dispatch_s(const dim3& G, hipStream_t s, const DevMap& map, const void* shard, float* master,
                             float* m, float* v, const AdamwArgs& hp, const DevState* st, const uint64_t* ptrs,
                             uint16_t* flat_out) {
  const dim3 B(kThreads);
#define ZS_ADAMW(SC, FO)                                                                                         \
  hipLaunchKernelGGL((k_adamw<GDT, PDT, SC, FO, GROUPS, SPLIT>), G, B, 0, s, map, shard, master, m, v, hp, st, \
                     ptrs, flat_out)
  if (ptrs != nullptr && flat_out != nullptr)
    ZS_ADAMW(true, true);
  else if (ptrs != nullptr)
    ZS_ADAMW(true, false);
  else if (flat_out != nullptr)
    ZS_ADAMW(false, true);
  else
    ZS_ADAMW(false, false);
#undef ZS_ADAMW
}

template <int GDT, int PDT, bool GROUPS>
static void adamw_dispatch_g(const dim3& G, hipStream_t s, const DevMap& map, const void* shard, float* master,
                             float* m, float* v, const AdamwArgs& hp, const DevState* st, const uint64_t* ptrs,
                             uint16_t* flat_out) {
  if (map.ntiles <= kSplitTiles)
    adamw_dispatch_s<GDT, PDT, GROUPS, kQuadsPerThread>(
        dim3(static_cast<unsigned>(launch_units(map.ntiles * kQuadsPerThread, 0))), s, map, shard, master, m,
        v, hp, st, ptrs, flat_out);
  else
    adamw_dispatch_s<GDT, PDT, GROUPS, 1>(dim3(static_cast<unsigned>(launch_units(map.ntiles, kXcdRunAdamw))), s, map,
                                          shard, master, m, v, hp, st, ptrs, flat_out);
}

template <int GDT, int PDT>
static void adamw_dispatch(const dim3& G, hipStream_t s, const DevMap& map, const void* shard, float* master,
                           float* m, float* v, const AdamwArgs& hp, const DevState* st, const uint64_t* ptrs,
                           uint16_t* flat_out) {
  if (map.seg_nodecay != nullptr)
    adamw_dispatch_g<GDT, PDT, true>(G, s, map, shard, master, m, v, hp, st, ptrs, flat_out);
  else
    adamw_dispatch_g<GDT, PDT, false>(G, s, map, shard, master, m, v, hp, st, ptrs, flat_out);
}

template <int GDT>
static void adamw_dispatch_p(int param_dt, const dim3& G, hipStream_t s, const DevMap& map, const void* shard,
                             float* master, float* m, float* v, const AdamwArgs& hp, const DevState* st,
                             const uint64_t* ptrs, uint16_t* flat_out) {
  if (param_dt == ZS_BF16)
    adamw_dispatch<GDT, ZS_BF16>(G, s, map, shard, master, m, v, hp, st, ptrs, flat_out);
  else
    adamw_dispatch<GDT, ZS_FP16>(G, s, map, shard, master, m, v, hp, st, ptrs, flat_out);
}

hipError_t launch_adamw(const DevMap& map, const void* shard, int grad_dt, float* master, float* m, float* v,
                        const AdamwArgs& hp, const DevState* st, const uint64_t* param_ptrs, void* flat_out,
                        int param_dt, hipStream_t s) {
  if (map.ntiles == 0) return hipSuccess;
  const dim3 G(static_cast<unsigned>(map.ntiles));
  uint16_t* fo = static_cast<uint16_t*>(flat_out);
  if (grad_dt == ZS_BF16)
    adamw_dispatch_p<ZS_BF16>(param_dt, G, s, map, shard, master, m, v, hp, st, param_ptrs, fo);
  else if (grad_dt == ZS_FP16)
    adamw_dispatch_p<ZS_FP16>(param_dt, G, s, map, shard, master, m, v, hp, st, param_ptrs, fo);
  else
    adamw_dispatch_p<ZS_FP32>(param_dt, G, s, map, shard, master, m, v, hp, st, param_ptrs, fo);
  return hipGetLastError();
}

hipError_t launch_unpack(const DevMap& map, const void* src, int src_dt, const uint64_t* dst_ptrs, int dst_dt,
                         const DevState* skip, hipStream_t s) {
  if (map.ntiles == 0) return hipSuccess;
  const dim3 G(static_cast<unsigned>(launch_units(map.ntiles, kXcdRunUnpack))), B(kThreads);
  const bool f32 = (src_dt == ZS_FP32);
  if (dst_dt == ZS_BF16) {
    if (f32)
      hipLaunchKernelGGL((k_unpack<true, ZS_BF16>), G, B, 0, s, map, src, skip, dst_ptrs);
    else
      hipLaunchKernelGGL((k_unpack<false, ZS_BF16>), G, B, 0, s, map, src, skip, dst_ptrs);
  } else {
    if (f32)
      hipLaunchKernelGGL((k_unpack<true, ZS_FP16>), G, B, 0, s, map, src, skip, dst_ptrs);
    else
      hipLaunchKernelGGL((k_unpack<false, ZS_FP16>), G, B, 0, s, map, src, skip, dst_ptrs);
  }
  return hipGetLastError();
}

}  // namespace zs
