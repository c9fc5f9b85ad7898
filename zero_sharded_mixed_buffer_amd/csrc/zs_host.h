// Host-side (CPU) AdamW update used by the offloaded optimizer step.  Internal to libzs.
#pragma once

#include <cstdint>

namespace zs_host {

// Per-step scalars of the update in fp64, the same quantities the GPU kernel uses:
// unscale-and-clip factor, betas and their complements, lr over the first bias correction,
// the reciprocal of the second, eps and the decoupled decay multiplier.
struct Scalars {
  double gs, b1, omb1, b2, omb2, a, rbc2, eps, decay;
};

Scalars step_scalars(double lr, double beta1, double beta2, double eps, double weight_decay, double loss_scale,
                     double clip_coef, int64_t step_t);

// Updates elements [0, count) of master/m/v in place from grad (grad_dt: 0 bf16, 1 fp16,
// 2 fp32) and, when param_out is not null, writes the cast of the new master in param_dt
// (0 bf16, 1 fp16).  Splits the range over n_threads threads (the caller's thread included).
// nd_runs: null, or n_runs sorted, disjoint [begin, end) pairs (2 * n_runs values) of
// elements that take no weight decay.
void adamw(const Scalars& k, int grad_dt, const void* grad, float* master, float* m, float* v, int param_dt,
           void* param_out, int64_t count, int n_threads, const int64_t* nd_runs = nullptr, int64_t n_runs = 0);

// Default worker count: OMP_NUM_THREADS when set, else the hardware threads (at most 256).
int default_threads();

}  // namespace zs_host
