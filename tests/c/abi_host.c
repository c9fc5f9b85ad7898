/* A plain C (C99) user of the library's host-only entry points: the header must compile as
 * C and the calls must work without Python or a GPU.  Prints one line per result; the test
 * that builds this file compares the lines with the oracle. */
#include <stdio.h>
#include <stdint.h>
#include <string.h>

#include "zs.h"

int main(void) {
  const int64_t numels[5] = {3, 5, 2, 7, 1};
  int64_t offsets[5], flat = 0, sb = 0, sn = 0;
  if (zs_plan(numels, 5, 2, 1, 4, offsets, &flat, &sb, &sn) != ZS_OK) {
    printf("error %s\n", zs_last_error());
    return 1;
  }
  printf("plan %lld %lld %lld", (long long)flat, (long long)sb, (long long)sn);
  for (int i = 0; i < 5; ++i) printf(" %lld", (long long)offsets[i]);
  printf("\n");

  int32_t bounds[10], nb = 0;
  if (zs_plan_buckets(numels, 5, 6, bounds, &nb) != ZS_OK) return 1;
  printf("buckets %d", nb);
  for (int i = 0; i < nb; ++i) printf(" %d:%d", bounds[2 * i], bounds[2 * i + 1]);
  printf("\n");

  /* one AdamW update of four elements on the host: fp32 gradient, bf16 parameter output */
  float grad[4] = {0.5f, -0.25f, 1e-3f, 0.0f};
  float master[4] = {1.0f, -2.0f, 0.5f, 0.25f};
  float m[4] = {0.0f, 0.1f, 0.0f, 0.0f};
  float v[4] = {0.0f, 0.01f, 0.0f, 0.0f};
  uint16_t param[4];
  zs_adamw_hparams hp = {1e-3, 0.9, 0.999, 1e-8, 0.01, 1.0};
  zs_state_host sc;
  memset(&sc, 0, sizeof sc);
  sc.loss_scale = 2.0;
  sc.scale_floor = 1.0;
  sc.growth_interval = 1000;
  sc.clip_coef = 0.5;
  sc.step_t = 2;
  if (zs_host_adamw_step(grad, ZS_FP32, master, m, v, 4, &hp, &sc, param, ZS_BF16, 2) != ZS_OK) {
    printf("error %s\n", zs_last_error());
    return 1;
  }
  for (int i = 0; i < 4; ++i) {
    uint32_t pb, mb, vb;
    memcpy(&pb, &master[i], 4);
    memcpy(&mb, &m[i], 4);
    memcpy(&vb, &v[i], 4);
    printf("adamw %08x %08x %08x %04x\n", pb, mb, vb, param[i]);
  }
  sc.loss_scale = 3.0; /* not a power of two: rejected */
  printf("invalid %d\n", (int)zs_host_adamw_step(grad, ZS_FP32, master, m, v, 4, &hp, &sc, param, ZS_BF16, 1));
  return 0;
}
