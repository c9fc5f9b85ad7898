/*
 * zs.h - C ABI of the per-rank ZeRO-1/2 mixed-precision optimizer step on MI355X (gfx950).
 *
 * One data-parallel rank's optimizer step over a flat gradient buffer:
 *   pack  -> take this rank's shard -> unscale + overflow flag -> global L2 norm + clip
 *   -> AdamW on the fp32 master / m / v shard -> cast + scatter-back -> loss-scaler update.
 *
 * Sources (page title, section):
 *   "nano-deepspeed (Teaching Edition)", section 2 "Current Feature Range": ZeRO stages
 *     1/2, AdamW only, FP16 dynamic loss scaling and a bf16 path, stage-2 communication as
 *     a packed buffer with local scatter-back.
 *   leetllm "Deep dive: Megatron", section "Distributed optimizer: trade replicated state
 *     for collectives": a contiguous gradient buffer, equal contiguous shards (the buffer
 *     length must divide by the number of ranks), each rank updating its FP32 master and
 *     two FP32 Adam moments, then rebuilding the 2-byte parameters.
 *   "3.7 Megatron-LM, DeepSpeed & Parallelism in Practice", sections "ZeRO Stages Recap"
 *     (2-byte params and grads, 12 bytes of fp32 optimizer state per parameter),
 *     "ZeRO-Offload and ZeRO-Infinity" (dynamic loss scale, window 1000, clipping 1.0,
 *     contiguous gradients; the step is memory-bandwidth-bound) and "Initializing a
 *     DeepSpeed Engine" (torch.optim.AdamW, decoupled weight decay).
 *
 * Conventions for every entry point:
 *   - Tensor data pointers are DEVICE pointers on the layout's GPU, owned by the caller
 *     (typically allocated through PyTorch). They must stay valid until the work enqueued
 *     on `stream` has completed. The library does not query the runtime for what a pointer
 *     is (that would cost every call a runtime round trip, and the pointer tables live on
 *     the device anyway): a host pointer passed as device memory is dereferenced by a
 *     kernel and faults the GPU. The Python binding refuses host tensors in these places.
 *   - Pointer tables (`src_ptrs`, `param_ptrs`, `dst_ptrs`) are DEVICE arrays of n_tensors
 *     device pointers (uint64 each), in parameter-list order, owned by the caller; an entry
 *     for a tensor with zero elements is never read through.  The tensors a table writes
 *     (`param_ptrs`, `dst_ptrs`) must not overlap one another or the flat buffers: their
 *     elements are written concurrently, in no fixed order.
 *   - `stream` is a hipStream_t (NULL = the null stream). Every device step call only
 *     enqueues kernels on it and never synchronises the host; results live in device
 *     memory. The calls that synchronise are zs_state_read and zs_state_write (their
 *     stream) and zs_offload_adamw_step (its stream: the host needs the step's scalars);
 *     none synchronises the whole device.
 *   - Flat buffers, shard-sized fp32 arrays and flat parameter outputs must be 16-byte
 *     aligned (any PyTorch allocation is); a shard view into a flat buffer may start at
 *     any element.
 *   - Return values are zs_status codes; no call aborts or throws. Arguments are checked
 *     on the host before anything is enqueued (ZS_EINVAL, nothing enqueued). A HIP error
 *     from a launch is returned as ZS_EHIP; asynchronous device faults surface on a later
 *     call or at zs_state_read. zs_last_error() gives a message for the calling thread.
 *   - Non-finite gradients are data, not errors: they set the overflow flag and make the
 *     AdamW and unpack kernels skip the update.
 *   - The library's only global state is the per-thread error message and the pool of
 *     host threads that the host AdamW update uses (started on first use; calls from
 *     several threads take turns on it). A layout or state must not be used from two
 *     streams at once without ordering them.
 */
#ifndef ZS_H
#define ZS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    ZS_OK = 0,
    ZS_EINVAL = -1,        /* bad argument; nothing was enqueued */
    ZS_EHIP = -2,          /* the HIP runtime reported an error */
    ZS_ENOMEM = -3,        /* device or host allocation failed (create calls only) */
    ZS_EUNSUPPORTED = -4   /* valid but unsupported combination (e.g. dtype pair) */
} zs_status;

typedef enum { ZS_BF16 = 0, ZS_FP16 = 1, ZS_FP32 = 2 } zs_dtype;

/* AdamW hyper-parameters ("Initializing a DeepSpeed Engine": torch.optim.AdamW; the toy
 * configuration uses lr 1e-3, betas (0.9, 0.999), eps 1e-8, weight decay 0.01) and the
 * global clipping threshold ("DeepSpeed config for this run": gradient_clipping 1.0).
 * Requirements: lr >= 0, 0 <= beta1 < 1, 0 <= beta2 < 1, eps > 0, weight_decay >= 0, all
 * finite; max_norm <= 0 disables clipping (clip coefficient 1). */
typedef struct {
    double lr, beta1, beta2, eps, weight_decay, max_norm;
} zs_adamw_hparams;

/* Loss-scaler and step state, as kept on the device (zs_state_read / zs_state_write).
 * loss_scale and scale_floor must be positive powers of two (so unscaling is exact);
 * growth_interval >= 1.  dynamic = 1: an overflow halves the scale (not below the floor)
 * and growth_interval consecutive applied steps double it; dynamic = 0: the scale never
 * changes (the bf16 path) and growth_tracker stays 0.  step_t counts applied updates.
 * The last five fields are results of the most recent check / norm calls. */
typedef struct {
    double loss_scale;
    double scale_floor;
    int32_t dynamic;
    int32_t growth_interval;
    int64_t growth_tracker;
    int64_t step_t;
    int64_t skipped_total;
    int32_t overflow;      /* 1 when the last check found inf/NaN here or on another rank */
    int32_t reserved;
    double local_sumsq;    /* this rank's sum of squares of the unscaled gradient shard */
    double sumsq;          /* global sum of squares (all ranks, rank order) */
    double grad_norm;      /* sqrt(sumsq) */
    double clip_coef;      /* min(1, max_norm / (grad_norm + 1e-6)), or 1 */
} zs_state_host;

typedef struct zs_layout zs_layout;  /* opaque; host plan + device segment tables */
typedef struct zs_state zs_state;    /* opaque; device zs_state_host + reduction workspace */

/* Host-only planning (no GPU needed).  Tensors are placed back to back in list order, each
 * starting at a multiple of align_elems elements (1 = dense concatenation); the tail is
 * zero-padded up to a multiple of dp_world * align_elems, so the flat buffer splits into
 * dp_world equal contiguous shards of S elements and rank r owns [r*S, (r+1)*S)
 * ("Deep dive: Megatron", section "Distributed optimizer": equal contiguous ownership of a
 * divisible buffer).  numels: host array of n_tensors sizes (>= 0, n_tensors >= 1);
 * align_elems: a power of two; offsets_out: optional host array of n_tensors flat offsets.
 * Errors: ZS_EINVAL on a NULL required pointer, n_tensors < 1, a negative size, dp_world
 * < 1, dp_rank outside [0, dp_world), align_elems not a power of two, or a flat buffer
 * above 68,719,472,640 elements (2^24 - 1 tiles of 4096: the largest grid of one launch). */
zs_status zs_plan(const int64_t* numels, int32_t n_tensors, int32_t dp_world, int32_t dp_rank,
                  int64_t align_elems, int64_t* offsets_out, int64_t* flat_numel_out,
                  int64_t* shard_begin_out, int64_t* shard_numel_out);

/* Host-only view of the segment table the kernels walk: the covered range (this rank's
 * shard, or the whole flat buffer when whole_flat != 0) split into maximal pieces that lie
 * in one tensor or in padding.  seg_begin[i] is range-relative, seg_tensor[i] is the tensor
 * index or -1 for padding, seg_local[i] the element offset inside that tensor.  At most
 * `capacity` entries are written; *n_segments receives the full count either way.  Same
 * argument errors as zs_plan. */
zs_status zs_plan_segments(const int64_t* numels, int32_t n_tensors, int32_t dp_world, int32_t dp_rank,
                           int64_t align_elems, int32_t whole_flat, int64_t* seg_begin, int32_t* seg_tensor,
                           int64_t* seg_local, int64_t capacity, int64_t* n_segments);

/* Plan as zs_plan and upload the segment tables to the current HIP device (once; the step
 * calls allocate nothing).  The layout is owned by the library until zs_layout_destroy.
 * Errors: as zs_plan; ZS_ENOMEM / ZS_EHIP from device allocation or upload. */
zs_status zs_layout_create(const int64_t* numels, int32_t n_tensors, int32_t dp_world, int32_t dp_rank,
                           int64_t align_elems, zs_layout** out);
void zs_layout_destroy(zs_layout* layout);
zs_status zs_layout_info(const zs_layout* layout, int64_t* flat_numel, int64_t* shard_begin,
                         int64_t* shard_numel);

/* Tensors without weight decay: a second parameter group that shares every
 * hyper-parameter but takes weight_decay 0, as is usual for biases and normalisation
 * weights ("Initializing a DeepSpeed Engine": torch.optim.AdamW, whose parameter groups
 * carry their own weight_decay).  no_decay: host array of n_tensors flags (non-zero: that
 * tensor's elements update with a decay multiplier of exactly 1), or NULL to make every
 * tensor decay again (the default).  Applies to zs_adamw_step and zs_offload_adamw_step
 * calls made on this layout after it returns.  The new table is uploaded on `stream`
 * without waiting for anything: device steps enqueued later on `stream` use it, steps on
 * another stream must be ordered after `stream` by the caller.  Work enqueued before the
 * call keeps reading the previous table, which the library keeps until
 * zs_layout_destroy (a few bytes per segment), so no wait for it is needed.  Not to be
 * called while another thread uses the layout.
 * Errors: ZS_EINVAL on a NULL layout or n_tensors different from the layout's;
 * ZS_ENOMEM / ZS_EHIP from the upload (the previous table then stays in force). */
zs_status zs_layout_set_no_decay(zs_layout* layout, const uint8_t* no_decay, int32_t n_tensors, void* stream);

/* Device state for one rank (scaler, step count, flag, norm results) and the workspace of
 * the norm reduction, on the layout's device.  `init` gives the starting zs_state_host
 * (loss_scale 2^16 with dynamic = 1 for fp16, 1 with dynamic = 0 for bf16, typically).
 * Errors: ZS_EINVAL on NULL pointers or an invalid init (see zs_state_host); ZS_ENOMEM. */
zs_status zs_state_create(const zs_layout* layout, const zs_state_host* init, zs_state** out);
void zs_state_destroy(zs_state* state);
/* Copy the device state to *out after all work on `stream` (synchronises `stream`). */
zs_status zs_state_read(const zs_state* state, zs_state_host* out, void* stream);
/* Overwrite the device state (resume from a checkpoint); synchronises `stream`.  The
 * result fields are copied as given.  Errors: ZS_EINVAL as zs_state_create. */
zs_status zs_state_write(zs_state* state, const zs_state_host* in, void* stream);

/* Pack per-parameter tensors into a flat buffer ("nano-deepspeed", section 2: packed
 * buffer; "ZeRO-Offload and ZeRO-Infinity": contiguous_gradients).
 *   src_ptrs: device table of the n_tensors source tensors (contiguous, src_dtype).
 *   dst: whole_flat != 0 -> the flat buffer, flat_numel elements; whole_flat == 0 -> this
 *        rank's shard only, shard_numel elements.  Padding elements are written as zero.
 *   dst_dtype == src_dtype: bit copy (the gradient buffer); dst_dtype == ZS_FP32: exact
 *        widening (seeding the fp32 master from the model-dtype parameters, or the first
 *        micro-step of an fp32 gradient-accumulation buffer).
 *   fuse_check: NULL, or a state to receive this pass's overflow flag and sum of squares
 *        of the packed values (what zs_unscale_check(dst) would compute with no other
 *        ranks, up to summation order); allowed only with dp_world == 1 and whole_flat.
 * Errors: ZS_EINVAL on NULL pointers, unaligned dst, src_dtype not bf16/fp16, a disallowed
 * fuse_check; ZS_EUNSUPPORTED for other dtype pairs. */
zs_status zs_pack(const zs_layout* layout, const void* src_ptrs, zs_dtype src_dtype, void* dst,
                  zs_dtype dst_dtype, int32_t whole_flat, zs_state* fuse_check, void* stream);

/* Gradient accumulation across micro-steps: acc += pack(src), element by element, each sum
 * rounded once (to nearest even) to acc_dtype; the optimizer steps only at the boundary
 * ("Initializing a DeepSpeed Engine": accumulation-aware backward and step;
 * gradient_accumulation_steps in the DeepSpeed configs).  acc_dtype is src_dtype or ZS_FP32
 * (an fp32 main-gradient buffer, as in the Megatron distributed optimizer's ledger); the
 * first micro-step of a window is a plain zs_pack into the same buffer.  Arguments, layout
 * and errors as zs_pack; fuse_check receives the flag and sum of squares of the updated
 * buffer, so the last micro-step can carry the check at dp_world == 1. */
zs_status zs_pack_accumulate(const zs_layout* layout, const void* src_ptrs, zs_dtype src_dtype, void* acc,
                             zs_dtype acc_dtype, int32_t whole_flat, zs_state* fuse_check, void* stream);

/* Bucketed packing: communication starts on a bucket of gradients as soon as backward has
 * produced all of them ("Deep dive: Megatron", section "Distributed optimizer": contiguous
 * buffers let communication begin bucket by bucket; "3.7 Megatron-LM, DeepSpeed &
 * Parallelism in Practice", section "DeepSpeed config for this run": reduce_bucket_size of
 * 5e8 elements; "nano-deepspeed", section 2: a packed bucket).
 * A bucket is a contiguous range [tensor_begin, tensor_end) of the parameter list.  It owns
 * the flat range [offset(tensor_begin), offset(tensor_end)), where offset(n_tensors) is
 * flat_numel: the alignment gap after a tensor and the tail padding belong to the bucket
 * before them, so the buckets of any partition of the tensor list tile the flat buffer.
 *
 * zs_plan_buckets: host only, no GPU.  Walks the tensors from last to first (the order in
 *   which backward produces their gradients) and closes a bucket once it holds at least
 *   bucket_numel elements (the first tensor closes the last bucket).  bounds_out (NULL, or
 *   room for 2 * n_tensors int32) receives [tensor_begin, tensor_end) pairs in closing
 *   order; *n_buckets_out their number.  A tensor larger than bucket_numel is a bucket by
 *   itself; a tensor is never split.  Errors: ZS_EINVAL on a NULL n_buckets_out, negative
 *   numels or bucket_numel <= 0.
 * zs_bucket_range: host only.  The flat range a bucket owns.  Errors: ZS_EINVAL unless
 *   0 <= tensor_begin < tensor_end <= n_tensors.
 * zs_pack_bucket: writes the bucket's flat range of the whole flat buffer `flat` (flat_numel
 *   elements of flat_dtype) and nothing else, exactly as zs_pack(whole_flat = 1) or, with
 *   accumulate != 0, zs_pack_accumulate would write that range.  flat_dtype is src_dtype or
 *   ZS_FP32 (an fp32 communication buffer: exact widening).  Buckets with disjoint ranges
 *   may run concurrently on different streams.  No overflow check is fused: the check runs
 *   on the reduced shard (zs_unscale_check).  Errors: as zs_pack, and ZS_EINVAL for a bad
 *   tensor range. */
zs_status zs_plan_buckets(const int64_t* numels, int32_t n_tensors, int64_t bucket_numel, int32_t* bounds_out,
                          int32_t* n_buckets_out);
zs_status zs_bucket_range(const zs_layout* layout, int32_t tensor_begin, int32_t tensor_end, int64_t* flat_begin,
                          int64_t* flat_end);
zs_status zs_pack_bucket(const zs_layout* layout, const void* src_ptrs, zs_dtype src_dtype, void* flat,
                         zs_dtype flat_dtype, int32_t tensor_begin, int32_t tensor_end, int32_t accumulate,
                         void* stream);

/* Overflow check of this rank's gradient shard (the reduce-scatter output; one GPU: the
 * rank's slice of its packed buffer).  Sets state.overflow = (any element of `shard` is
 * +inf, -inf or NaN) OR (*ext_overflow != 0), and records the shard's sum of squares of the
 * unscaled gradient for zs_grad_norm ("nano-deepspeed", section 2: FP16 dynamic loss scaling).
 *   shard: device pointer to shard_numel elements of grad_dtype (bf16, fp16, or fp32 for
 *          an fp32 accumulation buffer), aligned to its element size.
 *   ext_overflow: NULL or a device int32 holding the OR of the other ranks' flags.
 *   local_sumsq_out: NULL or a device double receiving this rank's sum of squares, the
 *          value the ranks exchange before zs_grad_norm (non-finite iff this shard holds a
 *          non-finite element, so exchanging it also exchanges the flag).
 * Errors: ZS_EINVAL on NULL layout/shard/state or a bad dtype. */
zs_status zs_unscale_check(const zs_layout* layout, const void* shard, zs_dtype grad_dtype, zs_state* state,
                           const int32_t* ext_overflow, double* local_sumsq_out, void* stream);

/* Global L2 norm of the unscaled gradient and the clip coefficient ("DeepSpeed config for
 * this run": gradient_clipping 1.0; "Deep dive: Megatron", section "Precision": sensitive
 * reductions in higher precision - accumulated in fp64).
 *   shard: NULL to reuse the sum recorded by zs_unscale_check / a fused zs_pack; otherwise
 *          the shard is summed again (and a non-finite value there also sets the flag).
 *   rank_sumsq: NULL when dp_world == 1; otherwise a device array of dp_world doubles, every
 *          rank's local sum of squares in rank order (entry dp_rank is replaced by this rank's
 *          own value), added in rank order so all ranks compute the same norm.  A non-finite
 *          entry (an overflow on that rank) sets state.overflow here too.  The exchange for
 *          dp_world > 1 is: zs_unscale_check(..., local_sumsq_out = &buf[rank]) on every rank,
 *          an all-gather of buf (8 bytes per rank), then zs_grad_norm(NULL, ..., buf, ...).
 *   local_sumsq_out: NULL or a device double receiving this rank's local sum of squares.
 * Result: state.sumsq, grad_norm, clip_coef = min(1, max_norm / (grad_norm + 1e-6)) (1 if
 * max_norm <= 0).  On an overflowed step the values are not meaningful and are not used.
 * Errors: ZS_EINVAL on NULL layout/state/hp, bad dtype, rank_sumsq NULL with dp_world > 1. */
zs_status zs_grad_norm(const zs_layout* layout, const void* shard, zs_dtype grad_dtype, zs_state* state,
                       const zs_adamw_hparams* hp, const double* rank_sumsq, double* local_sumsq_out,
                       void* stream);

/* AdamW on this rank's fp32 shard, fused with unscale, clip, cast and scatter-back
 * ("nano-deepspeed", section 2: AdamW only, local scatter-back; "Initializing a DeepSpeed
 * Engine": torch.optim.AdamW).  With t = state.step_t + 1, g = clip_coef * x / loss_scale:
 *   m <- beta1 m + (1 - beta1) g;  v <- beta2 v + (1 - beta2) g^2   (stored fp32)
 *   p <- p (1 - lr wd) - lr (m / (1 - beta1^t)) / (sqrt(v / (1 - beta2^t)) + eps)
 * evaluated in fp64 and rounded once to fp32 per stored value; the model-dtype parameter is
 * the round-to-nearest-even cast of the new fp32 master.  If state.overflow is set the call
 * changes nothing (device-side skip).  Does not advance step_t: zs_scaler_update does.
 *   shard: grad shard, shard_numel elements of grad_dtype (bf16, fp16 or fp32), aligned to
 *          its element size.  master / m / v: device fp32 arrays of shard_numel elements,
 *          updated in place.
 *   param_ptrs: NULL, or the device table of the n_tensors parameter tensors (param_dtype);
 *          the elements this rank owns are overwritten with the cast master.
 *   flat_param_out: NULL, or a device buffer of shard_numel param_dtype elements receiving
 *          the cast master in flat order (the all-gather input).
 * Errors: ZS_EINVAL on NULL required pointers, unaligned fp32 arrays / flat_param_out,
 * invalid hyper-parameters, grad_dtype not bf16/fp16/fp32, param_dtype not bf16/fp16. */
zs_status zs_adamw_step(const zs_layout* layout, const void* shard, zs_dtype grad_dtype, float* master, float* m,
                        float* v, const zs_adamw_hparams* hp, zs_state* state, const void* param_ptrs,
                        void* flat_param_out, zs_dtype param_dtype, void* stream);

/* Scatter a flat buffer back into the parameter tensors ("nano-deepspeed", section 2:
 * local scatter-back; "Deep dive: Megatron", section "Distributed optimizer": all-gather
 * rebuilds the 2-byte parameter buffer).
 *   src: whole_flat != 0 -> flat_numel elements (the all-gathered buffer); whole_flat == 0
 *        -> this rank's shard_numel elements.  src_dtype ZS_FP32 (the master; cast with
 *        round-to-nearest-even) or equal to dst_dtype (bit copy).
 *   dst_ptrs: device table of the n_tensors destination tensors (dst_dtype bf16/fp16);
 *        only the covered elements are written.
 *   honour_skip: NULL, or a state whose overflow flag makes the call a no-op.
 * Errors: ZS_EINVAL on NULL pointers, unaligned fp32 src; ZS_EUNSUPPORTED dtype pairs. */
zs_status zs_unpack(const zs_layout* layout, const void* src, zs_dtype src_dtype, int32_t whole_flat,
                    const void* dst_ptrs, zs_dtype dst_dtype, const zs_state* honour_skip, void* stream);

/* Commit the step in the loss scaler ("nano-deepspeed", section 2: FP16 dynamic loss
 * scaling; "ZeRO-Offload and ZeRO-Infinity": loss_scale_window 1000).  On overflow:
 * skipped_total += 1, growth_tracker = 0, and with dynamic scaling loss_scale =
 * max(loss_scale / 2, scale_floor).  Otherwise step_t += 1 and, with dynamic scaling,
 * growth_tracker += 1, doubling loss_scale and resetting the tracker when it reaches
 * growth_interval.  One device thread; no host involvement.
 * Errors: ZS_EINVAL on a NULL state. */
zs_status zs_scaler_update(zs_state* state, void* stream);

/* The whole single-rank step in one call: zs_pack (whole flat buffer, fused check) ->
 * zs_grad_norm -> zs_adamw_step (scatter into the parameters) -> zs_scaler_update ("nano-
 * deepspeed", section 2: the stage-2 packed buffer with local scatter-back and dynamic loss
 * scaling; "Deep dive: Megatron", section "Distributed optimizer" with one rank;
 * "ZeRO-Offload and ZeRO-Infinity": clipping and the loss-scale window), with the same
 * results bit for bit.  It enqueues three kernels instead of five: the pack with the
 * check's partial sums, one workgroup for the flag, the norm and the scaler commit (the
 * update reads a copy of the state taken before the commit), and the update.  A small
 * list's step is bound by launches, so this and the single call through the caller's
 * binding are what it saves.
 *   layout: dp_world must be 1.
 *   grad_ptrs: device pointer table of the gradients, grad_dtype (bf16 or fp16).
 *   flat: device buffer of flat_numel elements of grad_dtype, 16-byte aligned; receives
 *         the packed gradients (and keeps them).
 *   master, m, v: device fp32 arrays of shard_numel elements, 16-byte aligned, updated in
 *         place unless the step overflows.
 *   param_ptrs: device pointer table of the parameters (param_dtype, bf16 or fp16), which
 *         receive the cast of the new master.
 * Errors: ZS_EINVAL on dp_world != 1, NULL pointers, dtypes, misalignment, a state of
 * another layout or invalid hyper-parameters; nothing is enqueued then. */
zs_status zs_step(const zs_layout* layout, const void* grad_ptrs, zs_dtype grad_dtype, void* flat,
                  zs_state* state, const zs_adamw_hparams* hp, float* master, float* m, float* v,
                  const void* param_ptrs, zs_dtype param_dtype, void* stream);

/* The single-rank step over contiguous buffers, in one call: the gradients are already in
 * the flat buffer (backward wrote them there) and the parameters are the flat parameter
 * buffer ("Deep dive: Megatron", section "Distributed optimizer": backward fills a
 * contiguous gradient buffer; the update rebuilds the contiguous 2-byte parameter buffer).
 * The same results, bit for bit, as zs_unscale_check (no other ranks) -> zs_grad_norm ->
 * zs_adamw_step (flat_param_out, no pointer table) -> zs_scaler_update, in three launches:
 * the check's partial sums, one finalize workgroup (flag, norm, a copy of the pre-commit
 * state for the update, scaler commit), and the update.  No pack and no scatter: 30 bytes
 * per element instead of zs_step's 32.
 *   layout: dp_world must be 1.
 *   flat: device buffer of flat_numel elements of grad_dtype (bf16 or fp16), 16-byte
 *         aligned, holding the gradients in the layout's order (zero in the padding).
 *   master, m, v: device fp32 arrays of shard_numel elements, 16-byte aligned.
 *   flat_param_out: device buffer of flat_numel elements of param_dtype (bf16 or fp16),
 *         16-byte aligned; receives the cast of the new master unless the step overflows.
 * Errors: ZS_EINVAL on dp_world != 1, NULL pointers, dtypes, misalignment, a state of
 * another layout or invalid hyper-parameters; nothing is enqueued then. */
zs_status zs_step_flat(const zs_layout* layout, const void* flat, zs_dtype grad_dtype, zs_state* state,
                       const zs_adamw_hparams* hp, float* master, float* m, float* v, void* flat_param_out,
                       zs_dtype param_dtype, void* stream);

/* zs_step_flat for callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  It needs no layout and no zs_state
 * and allocates nothing: the reduction workspace and the pre-commit state are a fixed device
 * array inside the library (about 16.8 MB, one per GPU, held until the process ends).
 * The same launches and arithmetic as zs_step_flat on a single-rank layout of n elements with
 * align 1 and no no-decay tensors, so the same results bit for bit.
 *   flat: n elements of grad_dtype (bf16 or fp16), 16-byte aligned: the gradients.
 *   n: 1 .. 8,589,934,592 elements (2^21 check workgroups of 4096: the array's capacity).
 *   state: DEVICE pointer to a zs_state_host in the caller's memory (8-byte aligned), read and
 *          committed on the device by each call like the state of zs_step_flat; the caller
 *          fills it once with valid starting values (as zs_state_create checks them) and may
 *          read it back like any device buffer.
 *   master, m, v: n fp32 elements each, 16-byte aligned; flat_param_out: n elements of
 *          param_dtype (bf16 or fp16), 16-byte aligned.
 * Every call on a GPU shares that GPU's array, and calls on one GPU that overlap (different
 * streams without ordering, or several host threads) race on it: order them.  The array keeps
 * the last call's contents; each slot a call reads is written earlier in the same call.
 * Errors: ZS_EINVAL on NULL pointers, dtypes, misalignment, invalid hyper-parameters or n
 * outside 1 .. 8,589,934,592 (nothing is enqueued then); ZS_EHIP from the runtime. */
zs_status zs_step_flat_noalloc(const void* flat, zs_dtype grad_dtype, int64_t n, zs_state_host* state,
                               const zs_adamw_hparams* hp, float* master, float* m, float* v, void* flat_param_out,
                               zs_dtype param_dtype, void* stream);

/* Offloaded optimizer step: the fp32 master, m and v live in host memory and the host CPU
 * runs the update, which is bound by memory bandwidth, not by arithmetic ("3.7
 * Megatron-LM, DeepSpeed & Parallelism in Practice", section "ZeRO-Offload and
 * ZeRO-Infinity": optimizer states in CPU RAM, offload_optimizer with pin_memory, the state
 * processed in sub_group_size chunks).  The arithmetic is zs_adamw_step's: fp64 per
 * element, each stored fp32 value rounded once to nearest even, the parameter the
 * round-to-nearest-even cast of the new master.  Neither call changes the device state:
 * zs_scaler_update commits the step as after zs_adamw_step.
 *
 * zs_host_adamw_step: the update of `count` consecutive shard elements, every array in HOST
 *   memory and owned by the caller: grad (grad_dtype bf16, fp16 or fp32; the reduced,
 *   still loss-scaled gradient), master / m / v (fp32, updated in place) and param_out
 *   (NULL, or count elements of param_dtype bf16 / fp16).  `scalars` is the state as
 *   zs_state_read returns it after zs_grad_norm: loss_scale, clip_coef, step_t (the update
 *   uses t = step_t + 1) and overflow (non-zero: nothing is written).  n_threads host
 *   threads share the range (<= 0: OMP_NUM_THREADS, else every hardware thread).  No GPU
 *   is used.  Errors: ZS_EINVAL on NULL arrays (count > 0), bad dtypes, invalid
 *   hyper-parameters or scalars (loss_scale not a power of two, clip_coef outside (0, 1]).
 * zs_offload_adamw_step: the whole update of this rank's shard_numel elements.  Reads the
 *   state (synchronising `stream`), then pipelines chunks of chunk_numel elements: the
 *   gradient chunk is copied from the device shard (grad_dtype) into `grad_stage`, the host
 *   updates master / m / v (host arrays of shard_numel fp32 each; only the CPU reads them,
 *   so they need not be pinned), and the new parameters
 *   go from `param_stage` to the device buffer flat_param_out (shard_numel elements of
 *   param_dtype: the rank's all-gather input, or with dp_world == 1 the source of
 *   zs_unpack).  grad_stage and param_stage hold two chunks each (2 * chunk_numel elements
 *   of grad_dtype and param_dtype) and should be pinned (hipHostMalloc) so that copies
 *   overlap the host work.  On an overflowed step nothing is copied or written.  Returns
 *   after the last copy has completed.  Errors: ZS_EINVAL on NULL pointers, bad dtypes,
 *   chunk_numel <= 0; ZS_EHIP from the copies. */
zs_status zs_host_adamw_step(const void* grad, zs_dtype grad_dtype, float* master, float* m, float* v,
                             int64_t count, const zs_adamw_hparams* hp, const zs_state_host* scalars,
                             void* param_out, zs_dtype param_dtype, int32_t n_threads);
zs_status zs_offload_adamw_step(const zs_layout* layout, const void* shard, zs_dtype grad_dtype, zs_state* state,
                                const zs_adamw_hparams* hp, float* master, float* m, float* v, void* grad_stage,
                                void* param_stage, int64_t chunk_numel, void* flat_param_out,
                                zs_dtype param_dtype, int32_t n_threads, void* stream);

/* Message for the last non-OK status returned on the calling thread ("" if none). */
const char* zs_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* ZS_H */
