/*
 * zs_probe.h - bandwidth yardsticks exported by libzs.so beside the optimizer step (zs.h).
 *
 * They are not part of the step.  A benchmark times them on the same buffers
 * as the step, to learn what the machine delivers for the step's own access patterns with
 * the arithmetic taken away ("3.7 Megatron-LM, DeepSpeed & Parallelism in Practice",
 * section "ZeRO-Offload and ZeRO-Infinity": the optimizer step is bound by memory
 * bandwidth, so its yardstick is the memory system, not the ALUs).
 *
 * Every kernel has the launch shape of the step's update kernel: one workgroup of 256
 * threads per 4096 elements (16 KiB of each fp32 array), 16-byte (8 for 2-byte data)
 * non-temporal accesses per lane, each wave-wide access one contiguous row.
 *
 * Conventions as in zs.h: device pointers owned by the caller, 16-byte aligned; work is
 * only enqueued on `stream`; the buffers' contents are overwritten with meaningless values.
 * Errors: ZS_EINVAL (nothing enqueued) on a NULL pointer, misalignment or a size that is not
 * a whole number of workgroups; ZS_EHIP from the launch.
 */
#ifndef ZS_PROBE_H
#define ZS_PROBE_H

#include <stdint.h>

#include "zs.h"

#ifdef __cplusplus
extern "C" {
#endif

/* The update's byte mix with no arithmetic: read g (2 bytes per element), p, m, v (4 each);
 * write p, m, v (4 each; rotated: p <- m, m <- v, v <- p) and out (2 bytes: g's bits).
 * 28 bytes per element, like zs_adamw_step with a flat parameter output.  n: elements, a
 * positive multiple of 4096. */
zs_status zs_probe_mix(const void* g, float* p, float* m, float* v, void* out, int64_t n, void* stream);

/* One-to-one copy of `bytes` bytes (a positive multiple of 16384): read src, write dst. */
zs_status zs_probe_copy(const void* src, void* dst, int64_t bytes, void* stream);

/* Read-only pass over `bytes` bytes (a positive multiple of 16384).  sink: one device uint32
 * that receives a value only in the rare case that the data fold to a fixed pattern (so the
 * loads cannot be dropped). */
zs_status zs_probe_read(const void* src, int64_t bytes, uint32_t* sink, void* stream);

/* Write-only pass: `bytes` bytes (a positive multiple of 16384) of dst set to zero. */
zs_status zs_probe_write(void* dst, int64_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ZS_PROBE_H */
