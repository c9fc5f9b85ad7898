"""MI355X-native per-rank ZeRO-1/2 mixed-precision optimizer step.

The step runs in hand-written gfx950 HIP kernels behind the C ABI of
include/zs.h (libzs.so, built in-tree by `python -m zero_sharded_mixed_buffer_amd.build`);
this package is its ctypes binding plus a rank-level optimizer object.
"""

from ._abi import (  # noqa: F401
    LIB_PATH,
    ZS_BF16,
    ZS_FP16,
    ZS_FP32,
    AdamwHParams,
    StateHost,
    ZsError,
    ZsInvalidArgument,
    dtype_code,
    hparams,
    lib,
    state_host,
    zs_adamw_step,
    zs_grad_norm,
    zs_host_adamw_step,
    zs_last_error,
    zs_layout_create,
    zs_layout_destroy,
    zs_layout_info,
    zs_layout_set_no_decay,
    zs_offload_adamw_step,
    zs_pack,
    zs_bucket_range,
    zs_pack_accumulate,
    zs_pack_bucket,
    zs_plan_buckets,
    zs_plan,
    zs_plan_segments,
    zs_probe_copy,
    zs_probe_mix,
    zs_probe_read,
    zs_probe_write,
    zs_scaler_update,
    zs_step,
    zs_step_flat,
    zs_step_flat_noalloc,
    zs_state_create,
    zs_state_destroy,
    zs_state_read,
    zs_state_write,
    zs_unpack,
    zs_unscale_check,
)
from .optimizer import ZeroShardedAdamW, pointer_table, reshard_state_dicts  # noqa: F401
