// Host-side AdamW update for the offloaded optimizer step: the optimizer state lives in
// host memory and the CPU runs the update, which is memory-bandwidth-bound ("3.7
// Megatron-LM, DeepSpeed & Parallelism in Practice", section "ZeRO-Offload and
// ZeRO-Infinity").  The arithmetic is the GPU kernel's: every value in fp64, each stored
// fp32 value rounded once (to nearest even), the parameter the round-to-nearest-even cast of
// the new master.  Built with -ffp-contract=off so that no multiply-add is fused.
//
// The element loop is written so that the compiler can vectorise it; function clones for
// AVX-512, AVX2 and the baseline are chosen when the library is loaded.

#include "zs_host.h"

#include <unistd.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <condition_variable>
#include <cstdlib>
#include <cstring>
#include <functional>
#include <memory>
#include <mutex>
#include <thread>
#include <vector>

namespace zs_host {
namespace {

inline uint32_t f32_bits(float f) {
  uint32_t u;
  std::memcpy(&u, &f, sizeof u);
  return u;
}

inline float bits_f32(uint32_t u) {
  float f;
  std::memcpy(&f, &u, sizeof f);
  return f;
}

// fp32 -> bf16, round to nearest even; a NaN stays a (quiet) NaN.
inline uint16_t to_bf16(float f) {
  const uint32_t u = f32_bits(f);
  const uint32_t rounded = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
  const uint32_t nan = (u >> 16) | 0x40u;
  return static_cast<uint16_t>((u & 0x7fffffffu) > 0x7f800000u ? nan : rounded);
}

// fp32 -> fp16 (binary16), round to nearest even, with subnormal results, overflow to
// infinity and quiet NaNs.
inline uint16_t to_f16(float f) {
  const uint32_t u = f32_bits(f);
  const uint32_t sign = (u >> 16) & 0x8000u;
  const uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return static_cast<uint16_t>(sign | 0x7e00u | ((a >> 13) & 0x3ffu));
  if (a >= 0x477ff000u) return static_cast<uint16_t>(sign | 0x7c00u);  // 65520 and above round to inf
  if (a >= 0x38800000u) {                                                // a normal half: rebias by 112
    const uint32_t r = a - 0x38000000u;
    return static_cast<uint16_t>(sign | ((r + 0xfffu + ((r >> 13) & 1u)) >> 13));
  }
  const uint32_t e = a >> 23;  // a subnormal half, k * 2^-24: k = mantissa / 2^(126 - e)
  if (e < 102) return static_cast<uint16_t>(sign);
  const uint32_t mant = (a & 0x7fffffu) | 0x800000u;
  const int s = 126 - static_cast<int>(e);  // 14 .. 24
  uint32_t k = mant >> s;
  const uint32_t rem = mant & ((1u << s) - 1u);
  const uint32_t half = 1u << (s - 1);
  if (rem > half || (rem == half && (k & 1u))) ++k;
  return static_cast<uint16_t>(sign | k);
}

// binary16 -> fp32, exact.
inline float from_f16(uint16_t h) {
  const uint32_t sign = static_cast<uint32_t>(h & 0x8000u) << 16;
  const uint32_t e = (h >> 10) & 0x1fu;
  const uint32_t mant = h & 0x3ffu;
  if (e == 0x1f) return bits_f32(sign | 0x7f800000u | (mant << 13));
  if (e != 0) return bits_f32(sign | ((e + 112u) << 23) | (mant << 13));
  const float mag = static_cast<float>(mant) * 0x1p-24f;  // exact: mant < 2^10
  return sign ? -mag : mag;
}

template <int GD>
inline float grad_at(const void* g, int64_t i) {
  if constexpr (GD == 2) {
    return static_cast<const float*>(g)[i];
  } else if constexpr (GD == 0) {
    return bits_f32(static_cast<uint32_t>(static_cast<const uint16_t*>(g)[i]) << 16);
  } else {
    return from_f16(static_cast<const uint16_t*>(g)[i]);
  }
}

// Function clones resolved at load time.  ThreadSanitizer cannot run the resolvers (they
// run before its runtime starts), so a ThreadSanitizer build keeps the baseline only.
#if defined(__SANITIZE_THREAD__)
#define ZS_HOST_CLONES
#else
#define ZS_HOST_CLONES __attribute__((target_clones("avx512f", "avx2", "default")))
#endif

template <int GD, int PD, bool OUT>
ZS_HOST_CLONES void update_range(
    const Scalars& kk, const void* __restrict__ grad, float* __restrict__ master, float* __restrict__ mom1,
    float* __restrict__ mom2, uint16_t* __restrict__ pout, int64_t lo, int64_t hi) {
  const Scalars k = kk;
  for (int64_t i = lo; i < hi; ++i) {
    const double g = static_cast<double>(grad_at<GD>(grad, i)) * k.gs;
    const float m1 = static_cast<float>(k.b1 * static_cast<double>(mom1[i]) + k.omb1 * g);
    const float v1 = static_cast<float>(k.b2 * static_cast<double>(mom2[i]) + k.omb2 * (g * g));
    const double den = std::sqrt(static_cast<double>(v1) * k.rbc2) + k.eps;
    const double upd = k.a * static_cast<double>(m1) / den;
    const float p = static_cast<float>(static_cast<double>(master[i]) * k.decay - upd);
    master[i] = p;
    mom1[i] = m1;
    mom2[i] = v1;
    if constexpr (OUT) pout[i] = (PD == 0) ? to_bf16(p) : to_f16(p);
  }
}

using RangeFn = void (*)(const Scalars&, const void*, float*, float*, float*, uint16_t*, int64_t, int64_t);

template <int GD>
RangeFn pick_out(int param_dt, bool out) {
  if (!out) return update_range<GD, 0, false>;
  return param_dt == 0 ? update_range<GD, 0, true> : update_range<GD, 1, true>;
}

RangeFn pick(int grad_dt, int param_dt, bool out) {
  if (grad_dt == 0) return pick_out<0>(param_dt, out);
  if (grad_dt == 1) return pick_out<1>(param_dt, out);
  return pick_out<2>(param_dt, out);
}

}  // namespace

Scalars step_scalars(double lr, double beta1, double beta2, double eps, double weight_decay, double loss_scale,
                     double clip_coef, int64_t step_t) {
  Scalars k;
  const double t = static_cast<double>(step_t + 1);
  k.gs = clip_coef / loss_scale;
  k.b1 = beta1;
  k.omb1 = 1.0 - beta1;
  k.b2 = beta2;
  k.omb2 = 1.0 - beta2;
  k.a = lr / (1.0 - std::pow(beta1, t));
  k.rbc2 = 1.0 / (1.0 - std::pow(beta2, t));
  k.eps = eps;
  k.decay = 1.0 - lr * weight_decay;
  return k;
}

int default_threads() {
  if (const char* env = std::getenv("OMP_NUM_THREADS")) {
    const int n = std::atoi(env);
    if (n > 0) return std::min(n, 256);
  }
  const unsigned hw = std::thread::hardware_concurrency();
  return hw == 0 ? 1 : static_cast<int>(std::min(hw, 256u));
}

namespace {

// Worker threads kept for the life of the process, so that a pipelined step can hand many
// chunks to the host without starting threads for each.  One job at a time: run() hands
// out the part indices 0..parts-1 to the workers and the calling thread and returns when
// every part is done.  Each job carries its own counters, so a worker that wakes late
// finds its job's indices used up and calls nothing.  A process forked after the pool
// started gets a pool of its own.
class Pool {
 public:
  static Pool& get() {
    static std::mutex make;
    static Pool* pool = nullptr;
    std::lock_guard<std::mutex> lk(make);
    if (pool == nullptr || pool->pid_ != getpid()) pool = new Pool();  // a forked child's old pool has no threads
    return *pool;
  }

  void run(int parts, const std::function<void(int)>& fn) {
    std::lock_guard<std::mutex> one_job(job_mu_);
    grow(parts - 1);
    auto job = std::make_shared<Job>();
    job->fn = &fn;
    job->parts = parts;
    {
      std::lock_guard<std::mutex> lk(mu_);
      current_ = job;
      ++generation_;
    }
    wake_.notify_all();
    work(*job);
    std::unique_lock<std::mutex> lk(mu_);
    finished_.wait(lk, [&] { return job->done.load() == parts; });
    current_.reset();
  }

 private:
  struct Job {
    const std::function<void(int)>* fn = nullptr;
    int parts = 0;
    std::atomic<int> next{0};
    std::atomic<int> done{0};
  };

  Pool() : pid_(getpid()) {}

  void grow(int want) {
    while (n_workers_ < want) {
      std::thread([this] { loop(); }).detach();
      ++n_workers_;
    }
  }

  void loop() {
    uint64_t seen = 0;
    for (;;) {
      std::shared_ptr<Job> job;
      {
        std::unique_lock<std::mutex> lk(mu_);
        wake_.wait(lk, [&] { return generation_ != seen; });
        seen = generation_;
        job = current_;
      }
      if (job) work(*job);
    }
  }

  void work(Job& job) {
    int did = 0;
    for (int i = job.next.fetch_add(1); i < job.parts; i = job.next.fetch_add(1)) {
      (*job.fn)(i);
      ++did;
    }
    if (did > 0 && job.done.fetch_add(did) + did == job.parts) {
      std::lock_guard<std::mutex> lk(mu_);
      finished_.notify_all();
    }
  }

  const pid_t pid_;
  std::mutex job_mu_;
  std::mutex mu_;
  std::condition_variable wake_, finished_;
  std::shared_ptr<Job> current_;
  uint64_t generation_ = 0;
  int n_workers_ = 0;
};

// Elements [lo, hi) of one thread's part: plain runs with `k`, no-decay runs with `knd`.
void update_part(RangeFn fn, const Scalars& k, const Scalars& knd, const void* grad, float* master, float* m,
                 float* v, uint16_t* pout, int64_t lo, int64_t hi, const int64_t* runs, int64_t n_runs) {
  if (runs == nullptr || n_runs == 0) {
    fn(k, grad, master, m, v, pout, lo, hi);
    return;
  }
  // first run ending after lo
  int64_t a = 0, b = n_runs;
  while (a < b) {
    const int64_t mid = (a + b) / 2;
    if (runs[2 * mid + 1] <= lo)
      a = mid + 1;
    else
      b = mid;
  }
  int64_t cur = lo;
  for (int64_t r = a; r < n_runs && cur < hi; ++r) {
    const int64_t rb = std::max(runs[2 * r], cur), re = std::min(runs[2 * r + 1], hi);
    if (rb >= hi) break;
    if (cur < rb) fn(k, grad, master, m, v, pout, cur, rb);
    if (rb < re) fn(knd, grad, master, m, v, pout, rb, re);
    cur = std::max(cur, re);
  }
  if (cur < hi) fn(k, grad, master, m, v, pout, cur, hi);
}

}  // namespace

void adamw(const Scalars& k, int grad_dt, const void* grad, float* master, float* m, float* v, int param_dt,
           void* param_out, int64_t count, int n_threads, const int64_t* nd_runs, int64_t n_runs) {
  if (count <= 0) return;
  const RangeFn fn = pick(grad_dt, param_dt, param_out != nullptr);
  uint16_t* pout = static_cast<uint16_t*>(param_out);
  Scalars knd = k;
  knd.decay = 1.0;
  // One contiguous part per thread, each a multiple of 64 elements so that no two threads
  // write the same cache line of any array; small ranges stay on the calling thread.
  constexpr int64_t kGrain = 1 << 16;
  const int64_t max_parts = (count + kGrain - 1) / kGrain;
  const int parts = static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(n_threads, max_parts)));
  const int64_t per = ((count + parts - 1) / parts + 63) / 64 * 64;
  auto part = [&](int p) {
    const int64_t lo = std::min(count, p * per), hi = std::min(count, (p + 1) * per);
    if (lo < hi) update_part(fn, k, knd, grad, master, m, v, pout, lo, hi, nd_runs, n_runs);
  };
  if (parts == 1) {
    part(0);
    return;
  }
  Pool::get().run(parts, part);
}

}  // namespace zs_host
