// A consumer of the C ABI with no Python and no torch: HIP runtime calls for device memory
// and a stream, zs.h for everything else.  It reads a problem from a binary file, runs the
// single-rank step on the GPU for every step's gradients, and writes the state, master, m,
// v and the parameters to a binary file that the test compares with the oracle.  Mode
// "tensors": one allocation per parameter and gradient tensor, zs_step (pack + scatter).
// Mode "flat": one contiguous gradient buffer and one contiguous parameter buffer at the
// offsets zs_plan gives, zs_step_flat.
//
// Input (little-endian): int32 n_tensors, int32 dtype (ZS_BF16 / ZS_FP16), int32 steps,
//   int64 numels[n_tensors], double hparams[6] (lr, beta1, beta2, eps, weight_decay,
//   max_norm), double loss_scale, double scale_floor, int32 dynamic, int32 growth_interval,
//   then the parameters (2-byte values of every tensor back to back), then for each step
//   the gradients in the same layout.
// Output: zs_state_host, then S floats each of master, m and v, then the parameters.
// Exit status 0 on success; any failure prints a message and exits non-zero.

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <string>
#include <vector>

#include "zs.h"

namespace {

[[noreturn]] void die(const char* what, const char* detail) {
  std::fprintf(stderr, "abi_gpu: %s: %s\n", what, detail);
  std::exit(1);
}

void zs_ok(zs_status s, const char* what) {
  if (s != ZS_OK) die(what, zs_last_error());
}

void hip_ok(hipError_t e, const char* what) {
  if (e != hipSuccess) die(what, hipGetErrorString(e));
}

template <typename T>
void read_into(std::FILE* f, T* dst, size_t count) {
  if (count && std::fread(dst, sizeof(T), count, f) != count) die("reading the input", "short file");
}

}  // namespace

int main(int argc, char** argv) {
  if (argc != 4) die("usage", "abi_gpu <input> <output> tensors|flat");
  const std::string mode = argv[3];
  if (mode != "tensors" && mode != "flat") die("usage", "the mode is tensors or flat");
  const bool flat_mode = mode == "flat";
  std::FILE* in = std::fopen(argv[1], "rb");
  if (in == nullptr) die("opening the input", argv[1]);
  int32_t n = 0, dtype = 0, steps = 0;
  read_into(in, &n, 1);
  read_into(in, &dtype, 1);
  read_into(in, &steps, 1);
  if (n < 1 || steps < 0 || (dtype != ZS_BF16 && dtype != ZS_FP16)) die("input", "bad header");
  std::vector<int64_t> numels(n);
  read_into(in, numels.data(), numels.size());
  double hpv[6];
  read_into(in, hpv, 6);
  zs_adamw_hparams hp{hpv[0], hpv[1], hpv[2], hpv[3], hpv[4], hpv[5]};
  zs_state_host init{};
  read_into(in, &init.loss_scale, 1);
  read_into(in, &init.scale_floor, 1);
  read_into(in, &init.dynamic, 1);
  read_into(in, &init.growth_interval, 1);
  init.clip_coef = 1.0;
  int64_t total = 0;
  for (int64_t x : numels) total += x;

  zs_layout* layout = nullptr;
  zs_ok(zs_layout_create(numels.data(), n, 1, 0, 1, &layout), "zs_layout_create");
  int64_t flat_numel = 0, shard_begin = 0, shard_numel = 0;
  zs_ok(zs_layout_info(layout, &flat_numel, &shard_begin, &shard_numel), "zs_layout_info");
  zs_state* state = nullptr;
  zs_ok(zs_state_create(layout, &init, &state), "zs_state_create");

  // Mode tensors: one device allocation per tensor, as a framework has them.  Mode flat:
  // every tensor is a slice of one parameter buffer and one gradient buffer.
  std::vector<int64_t> offsets(n, 0);
  zs_ok(zs_plan(numels.data(), n, 1, 0, 1, offsets.data(), nullptr, nullptr, nullptr), "zs_plan");
  void *flat_params = nullptr, *flat = nullptr;
  hip_ok(hipMalloc(&flat, static_cast<size_t>(flat_numel) * 2 + 16), "hipMalloc flat");
  hip_ok(hipMemset(flat, 0, static_cast<size_t>(flat_numel) * 2), "zero flat");
  if (flat_mode) {
    hip_ok(hipMalloc(&flat_params, static_cast<size_t>(flat_numel) * 2 + 16), "hipMalloc flat params");
    hip_ok(hipMemset(flat_params, 0, static_cast<size_t>(flat_numel) * 2), "zero flat params");
  }
  std::vector<void*> params(n, nullptr), grads(n, nullptr);
  std::vector<uint64_t> pptr(n, 0), gptr(n, 0);
  for (int32_t i = 0; i < n; ++i) {
    const size_t bytes = static_cast<size_t>(numels[i] > 0 ? numels[i] : 1) * 2;
    if (flat_mode) {
      params[i] = static_cast<char*>(flat_params) + offsets[i] * 2;
      grads[i] = static_cast<char*>(flat) + offsets[i] * 2;
    } else {
      hip_ok(hipMalloc(&params[i], bytes), "hipMalloc params");
      hip_ok(hipMalloc(&grads[i], bytes), "hipMalloc grads");
    }
    pptr[i] = reinterpret_cast<uint64_t>(params[i]);
    gptr[i] = reinterpret_cast<uint64_t>(grads[i]);
  }
  void *d_pptr = nullptr, *d_gptr = nullptr;
  float *master = nullptr, *m = nullptr, *v = nullptr;
  hip_ok(hipMalloc(&d_pptr, n * sizeof(uint64_t)), "hipMalloc pointer table");
  hip_ok(hipMalloc(&d_gptr, n * sizeof(uint64_t)), "hipMalloc pointer table");
  hip_ok(hipMemcpy(d_pptr, pptr.data(), n * sizeof(uint64_t), hipMemcpyHostToDevice), "upload pointer table");
  hip_ok(hipMemcpy(d_gptr, gptr.data(), n * sizeof(uint64_t), hipMemcpyHostToDevice), "upload pointer table");
  const size_t sbytes = static_cast<size_t>(shard_numel > 0 ? shard_numel : 1) * sizeof(float);
  hip_ok(hipMalloc(reinterpret_cast<void**>(&master), sbytes), "hipMalloc master");
  hip_ok(hipMalloc(reinterpret_cast<void**>(&m), sbytes), "hipMalloc m");
  hip_ok(hipMalloc(reinterpret_cast<void**>(&v), sbytes), "hipMalloc v");
  hip_ok(hipMemset(m, 0, sbytes), "zero m");
  hip_ok(hipMemset(v, 0, sbytes), "zero v");
  hipStream_t stream = nullptr;
  hip_ok(hipStreamCreate(&stream), "hipStreamCreate");

  std::vector<uint16_t> host(static_cast<size_t>(total));
  auto upload = [&](std::vector<void*>& dst) {
    read_into(in, host.data(), host.size());
    size_t off = 0;
    for (int32_t i = 0; i < n; ++i) {
      hip_ok(hipMemcpy(dst[i], host.data() + off, static_cast<size_t>(numels[i]) * 2, hipMemcpyHostToDevice),
             "upload tensor");
      off += static_cast<size_t>(numels[i]);
    }
  };
  upload(params);
  // fp32 master from the parameters: the widening pack of the shard
  zs_ok(zs_pack(layout, d_pptr, static_cast<zs_dtype>(dtype), master, ZS_FP32, 0, nullptr, stream), "zs_pack");
  for (int32_t s = 0; s < steps; ++s) {
    upload(grads);
    if (flat_mode)
      zs_ok(zs_step_flat(layout, flat, static_cast<zs_dtype>(dtype), state, &hp, master, m, v, flat_params,
                         static_cast<zs_dtype>(dtype), stream),
            "zs_step_flat");
    else
      zs_ok(zs_step(layout, d_gptr, static_cast<zs_dtype>(dtype), flat, state, &hp, master, m, v, d_pptr,
                    static_cast<zs_dtype>(dtype), stream),
            "zs_step");
    hip_ok(hipStreamSynchronize(stream), "step");
  }
  std::fclose(in);

  zs_state_host out_state{};
  zs_ok(zs_state_read(state, &out_state, stream), "zs_state_read");
  std::FILE* out = std::fopen(argv[2], "wb");
  if (out == nullptr) die("opening the output", argv[2]);
  std::fwrite(&out_state, sizeof out_state, 1, out);
  std::vector<float> buf(static_cast<size_t>(shard_numel));
  for (float* arr : {master, m, v}) {
    hip_ok(hipMemcpy(buf.data(), arr, buf.size() * sizeof(float), hipMemcpyDeviceToHost), "download state");
    std::fwrite(buf.data(), sizeof(float), buf.size(), out);
  }
  for (int32_t i = 0; i < n; ++i) {
    std::vector<uint16_t> p(static_cast<size_t>(numels[i]));
    hip_ok(hipMemcpy(p.data(), params[i], p.size() * 2, hipMemcpyDeviceToHost), "download params");
    std::fwrite(p.data(), 2, p.size(), out);
  }
  if (std::fclose(out) != 0) die("writing the output", argv[2]);

  hip_ok(hipStreamDestroy(stream), "hipStreamDestroy");
  if (!flat_mode) {
    for (int32_t i = 0; i < n; ++i) {
      (void)hipFree(params[i]);
      (void)hipFree(grads[i]);
    }
  }
  for (void* p : {d_pptr, d_gptr, flat, flat_params, static_cast<void*>(master), static_cast<void*>(m),
                  static_cast<void*>(v)})
    if (p != nullptr) (void)hipFree(p);
  zs_state_destroy(state);
  zs_layout_destroy(layout);
  std::printf("abi_gpu ok (%s): %d tensors, %lld elements, %d steps\n", mode.c_str(), n,
              static_cast<long long>(total), steps);
  return 0;
}
