"""CPU oracle for the per-rank ZeRO-1/2 mixed-precision optimizer step.

TEST INFRASTRUCTURE ONLY.  Only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import this package; the product path never
does and shares no code with it.
"""

from .zs_oracle import (  # noqa: F401
    OracleLayout,
    OracleScaler,
    accumulate,
    bucket_range,
    adamw_update,
    cast_to,
    decay_mask,
    clip_coefficient,
    global_sumsq,
    nonfinite_any,
    pack,
    pack_bucket,
    plan_buckets,
    plan_layout,
    scaler_update,
    shard_of,
    sumsq_unscaled,
    unpack,
    OracleRank,
)
