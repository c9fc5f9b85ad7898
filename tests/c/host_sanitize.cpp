// The library's host-only code (planner, segment maps, buckets, host AdamW update) built
// with AddressSanitizer and UndefinedBehaviorSanitizer and driven over seeded random cases.
// Every result is checked against a brute-force restatement here; any sanitizer report or
// mismatch ends the program with a non-zero status.  Prints "ok" at the end.

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "zs_host.h"
#include "zs_plan.h"

namespace {

uint64_t g_state = 0x9E3779B97F4A7C15ull;
uint64_t next_u64() {  // splitmix64
  uint64_t z = (g_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
int64_t uniform(int64_t lo, int64_t hi) { return lo + static_cast<int64_t>(next_u64() % uint64_t(hi - lo + 1)); }
float unit() { return static_cast<float>(next_u64() >> 40) / static_cast<float>(1 << 24); }

#define CHECK(c)                                                      \
  do {                                                                \
    if (!(c)) {                                                       \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
      std::exit(1);                                                   \
    }                                                                 \
  } while (0)

void check_map(const zs_planner::Plan& p, int64_t begin, int64_t len, int64_t tile) {
  const zs_planner::HostMap m = zs_planner::build_map(p, begin, len, tile);
  const size_t nseg = m.seg_tensor.size();
  CHECK(m.seg_begin.size() == nseg + 1 && m.seg_local.size() == nseg);
  CHECK(m.seg_begin.front() == 0 && m.seg_begin.back() == len);
  for (size_t s = 0; s < nseg; ++s) CHECK(m.seg_begin[s] < m.seg_begin[s + 1]);
  // every element of the range: brute-force owner against the map
  for (int64_t x = 0; x < len; x += std::max<int64_t>(1, len / 997)) {
    int32_t owner = -1;
    int64_t local = 0;
    for (size_t i = 0; i < p.numels.size(); ++i)
      if (begin + x >= p.offsets[i] && begin + x < p.offsets[i] + p.numels[i]) {
        owner = static_cast<int32_t>(i);
        local = begin + x - p.offsets[i];
      }
    size_t s = 0;
    while (m.seg_begin[s + 1] <= x) ++s;
    CHECK(m.seg_tensor[s] == owner);
    if (owner >= 0) CHECK(m.seg_local[s] + (x - m.seg_begin[s]) == local);
  }
  CHECK(m.ntiles == (len + tile - 1) / tile && static_cast<int64_t>(m.tile_first.size()) == m.ntiles + 1);
  for (int64_t k = 0; k < m.ntiles; ++k) {
    const int32_t s = m.tile_first[k];
    CHECK(m.seg_begin[s] <= k * tile && k * tile < m.seg_begin[s + 1]);
  }
}

void planner_cases() {
  for (int c = 0; c < 300; ++c) {
    const int32_t n = static_cast<int32_t>(uniform(1, 40));
    std::vector<int64_t> numels(n);
    for (auto& x : numels) x = (uniform(0, 4) == 0) ? 0 : uniform(1, 1 << uniform(0, 14));
    const int32_t d = static_cast<int32_t>(uniform(1, 8));
    const int32_t r = static_cast<int32_t>(uniform(0, d - 1));
    const int64_t align = int64_t(1) << uniform(0, 7);
    zs_planner::Plan p;
    const std::string err = zs_planner::make_plan(numels.data(), n, d, r, align, int64_t(1) << 36, &p);
    CHECK(err.empty());
    int64_t end = 0;
    for (int32_t i = 0; i < n; ++i) {
      CHECK(p.offsets[i] % align == 0 && p.offsets[i] >= end);
      end = p.offsets[i] + numels[i];
    }
    CHECK(p.flat_numel >= end && p.flat_numel % (int64_t(d) * align) == 0 && p.flat_numel - end < int64_t(d) * align);
    CHECK(p.shard_numel * d == p.flat_numel && p.shard_begin == r * p.shard_numel);
    const int64_t tile = int64_t(1) << uniform(2, 8);
    check_map(p, p.shard_begin, p.shard_numel, tile);
    check_map(p, 0, p.flat_numel, tile);
    // buckets: a partition in backward order, each closed as soon as it is full
    const int64_t size = uniform(1, 5000);
    std::vector<int32_t> bounds(2 * n);
    const int32_t nb = zs_planner::plan_buckets(numels.data(), n, size, bounds.data());
    CHECK(nb >= 1 && bounds[1] == n && bounds[2 * nb - 2] == 0);
    for (int32_t b = 0; b < nb; ++b) {
      const int32_t t0 = bounds[2 * b], t1 = bounds[2 * b + 1];
      CHECK(t0 < t1);
      if (b + 1 < nb) CHECK(bounds[2 * b + 2 + 1] == t0);
      int64_t sum = 0, tail = 0;
      for (int32_t t = t0; t < t1; ++t) sum += numels[t];
      for (int32_t t = t0 + 1; t < t1; ++t) tail += numels[t];
      if (t0 > 0) CHECK(sum >= size);
      CHECK(tail < size);
      int64_t lo = 0, hi = 0;
      CHECK(zs_planner::bucket_range(p, t0, t1, &lo, &hi));
      CHECK(lo == p.offsets[t0] && hi == (t1 == n ? p.flat_numel : p.offsets[t1]));
    }
    int64_t lo = 0, hi = 0;
    CHECK(!zs_planner::bucket_range(p, 0, 0, &lo, &hi) && !zs_planner::bucket_range(p, 0, n + 1, &lo, &hi));
  }
  // refusals
  zs_planner::Plan p;
  const int64_t big[2] = {int64_t(1) << 40, 5};
  CHECK(!zs_planner::make_plan(big, 2, 1, 0, 1, int64_t(1) << 36, &p).empty());
  const int64_t one[1] = {7};
  CHECK(!zs_planner::make_plan(one, 1, 4, 0, int64_t(1) << 62, int64_t(1) << 36, &p).empty());
  CHECK(!zs_planner::make_plan(one, 1, 2, 2, 1, int64_t(1) << 36, &p).empty());
  CHECK(!zs_planner::make_plan(one, 1, 1, 0, 3, int64_t(1) << 36, &p).empty());
}

uint16_t bf16_rne(float f) {  // independent restatement: compare the dropped half with the tie
  uint32_t u;
  std::memcpy(&u, &f, 4);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  const uint32_t lo = u & 0xffffu, hi = u >> 16;
  const bool up = lo > 0x8000u || (lo == 0x8000u && (hi & 1u));
  return static_cast<uint16_t>(hi + (up ? 1u : 0u));
}

void host_step_cases() {
  const int64_t counts[] = {0, 1, 3, 63, 64, 65, 4097, 100003, 300001};
  for (int64_t count : counts) {
    for (int threads : {1, 3, 8}) {
      std::vector<float> g(count), p(count), m(count), v(count);
      for (int64_t i = 0; i < count; ++i) {
        g[i] = (unit() - 0.5f) * 2e-3f;
        p[i] = (unit() - 0.5f) * 0.04f;
        m[i] = (unit() - 0.5f) * 1e-3f;
        v[i] = unit() * 1e-6f;
      }
      std::vector<float> p0 = p, m0 = m, v0 = v;
      std::vector<uint16_t> out(count + 1, 0xAAAA);
      const zs_host::Scalars k = zs_host::step_scalars(1e-3, 0.9, 0.999, 1e-8, 0.01, 4.0, 0.75, 6);
      zs_host::adamw(k, 2, g.data(), p.data(), m.data(), v.data(), 0, out.data(), count, threads);
      CHECK(out[count] == 0xAAAA);  // nothing written past the end
      for (int64_t i = 0; i < count; ++i) {
        const double gg = static_cast<double>(g[i]) * (0.75 / 4.0);
        const float m1 = static_cast<float>(0.9 * static_cast<double>(m0[i]) + (1.0 - 0.9) * gg);
        const float v1 = static_cast<float>(0.999 * static_cast<double>(v0[i]) + (1.0 - 0.999) * (gg * gg));
        const double den = std::sqrt(static_cast<double>(v1) * (1.0 / (1.0 - std::pow(0.999, 7.0)))) + 1e-8;
        const double upd = (1e-3 / (1.0 - std::pow(0.9, 7.0))) * static_cast<double>(m1) / den;
        const float pn = static_cast<float>(static_cast<double>(p0[i]) * (1.0 - 1e-3 * 0.01) - upd);
        CHECK(std::memcmp(&m[i], &m1, 4) == 0 && std::memcmp(&v[i], &v1, 4) == 0 && std::memcmp(&p[i], &pn, 4) == 0);
        CHECK(out[i] == bf16_rne(pn));
      }
    }
  }
}

// No-decay runs: elements inside a run update with a decay multiplier of 1.
void host_runs_cases() {
  for (int c = 0; c < 40; ++c) {
    const int64_t count = uniform(1, 200000);
    std::vector<int64_t> runs;
    int64_t pos = uniform(0, 50);
    while (pos < count) {
      const int64_t len = uniform(1, 30000);
      runs.push_back(pos);
      runs.push_back(std::min(count, pos + len));
      pos += len + uniform(1, 30000);
    }
    std::vector<float> g(count), p(count), m(count, 0.0f), v(count, 0.0f);
    for (int64_t i = 0; i < count; ++i) {
      g[i] = (unit() - 0.5f) * 2e-3f;
      p[i] = (unit() - 0.5f) * 0.04f;
    }
    std::vector<float> a = p, am = m, av = v, b = p, bm = m, bv = v;
    const zs_host::Scalars k = zs_host::step_scalars(1e-2, 0.9, 0.999, 1e-8, 0.3, 1.0, 1.0, 0);
    zs_host::Scalars knd = k;
    knd.decay = 1.0;
    const int threads = static_cast<int>(uniform(1, 6));
    zs_host::adamw(k, 2, g.data(), a.data(), am.data(), av.data(), 0, nullptr, count, threads, runs.data(),
                   static_cast<int64_t>(runs.size() / 2));
    // reference: one call per element range, in order
    int64_t cur = 0;
    for (size_t r = 0; r < runs.size(); r += 2) {
      if (cur < runs[r]) zs_host::adamw(k, 2, g.data() + cur, b.data() + cur, bm.data() + cur, bv.data() + cur, 0,
                                        nullptr, runs[r] - cur, 1);
      zs_host::adamw(knd, 2, g.data() + runs[r], b.data() + runs[r], bm.data() + runs[r], bv.data() + runs[r], 0,
                     nullptr, runs[r + 1] - runs[r], 1);
      cur = runs[r + 1];
    }
    if (cur < count) zs_host::adamw(k, 2, g.data() + cur, b.data() + cur, bm.data() + cur, bv.data() + cur, 0, nullptr,
                                    count - cur, 1);
    CHECK(std::memcmp(a.data(), b.data(), count * 4) == 0 && std::memcmp(am.data(), bm.data(), count * 4) == 0 &&
          std::memcmp(av.data(), bv.data(), count * 4) == 0);
  }
}

}  // namespace

int main() {
  planner_cases();
  host_step_cases();
  host_runs_cases();
  std::printf("ok\n");
  return 0;
}
