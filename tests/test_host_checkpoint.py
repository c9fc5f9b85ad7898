"""Re-sharding checkpoints across data-parallel group sizes (no GPU): rank state dicts built
from the oracle's ranks, mapped to another group size by reshard_state_dicts(), equal the
oracle's ranks of that group size that took the same steps, bit for bit.  Clipping is off,
so every group size computes the same update (the global norm's summation order differs
between group sizes)."""

import math

import pytest
import torch

import oracle as O
import zero_sharded_mixed_buffer_amd as Z
from zero_sharded_mixed_buffer_amd.optimizer import PERSISTENT_STATE, STATE_FORMAT

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, max_norm=1e9)


def _run(numels, params, d, align, steps, seed):
    gen = torch.Generator().manual_seed(seed)
    ranks = [O.OracleRank(numels, d, r, params, O.OracleScaler(1.0, dynamic=False), HP, align=align)
             for r in range(d)]
    for _ in range(steps):
        grads = [torch.randn(n, generator=gen).mul(1e-3).to(torch.bfloat16) for n in numels]
        flat = O.pack(grads, ranks[0].layout)
        parts = [O.sumsq_unscaled(O.shard_of(flat, r.layout), 1.0) for r in ranks]
        for r in ranks:
            r.step(O.shard_of(flat, r.layout), other_sumsq=parts)
    return ranks


def _state_dict(rank, numels, align):
    lay = rank.layout
    sc = rank.scaler
    state = {"loss_scale": sc.loss_scale, "scale_floor": sc.scale_floor, "dynamic": int(sc.dynamic),
             "growth_interval": sc.growth_interval, "growth_tracker": sc.growth_tracker, "step_t": sc.step_t,
             "skipped_total": sc.skipped_total}
    assert tuple(state) == PERSISTENT_STATE
    return {"format": STATE_FORMAT,
            "layout": {"numels": list(numels), "dp_world": lay.dp_world, "dp_rank": lay.dp_rank, "align": align,
                       "flat_numel": lay.flat_numel, "shard_begin": lay.shard_begin,
                       "shard_numel": lay.shard_numel},
            "state": state, "master": rank.master.clone(), "m": rank.m.clone(), "v": rank.v.clone()}


def _bits(t):
    return t.contiguous().view(torch.int32)


@pytest.mark.parametrize("numels,align,d_from,d_to", [
    ([513, 200, 64, 1000, 3], 1, 2, 1),
    ([513, 200, 64, 1000, 3], 1, 1, 4),
    ([5, 0, 97, 2, 31], 8, 3, 2),
    ([4096, 1, 4095], 64, 4, 3),
])
def test_reshard_equals_the_other_group_size(numels, align, d_from, d_to):
    gen = torch.Generator().manual_seed(5)
    params = [torch.randn(n, generator=gen).mul(0.02).to(torch.bfloat16) for n in numels]
    src = _run(numels, params, d_from, align, 3, seed=17)
    dst = _run(numels, params, d_to, align, 3, seed=17)
    sds = [_state_dict(r, numels, align) for r in src]
    for r in range(d_to):
        out = Z.reshard_state_dicts(reversed(sds), d_to, r)  # any order of the ranks
        lay = dst[r].layout
        assert out["layout"]["shard_begin"] == lay.shard_begin and out["layout"]["shard_numel"] == lay.shard_numel
        assert out["layout"]["flat_numel"] == lay.flat_numel
        assert out["state"]["step_t"] == 3
        for k in ("master", "m", "v"):
            assert torch.equal(_bits(out[k]), _bits(getattr(dst[r], k))), (r, k)


def test_reshard_round_trip_is_identity():
    numels = [7, 300, 0, 129]
    gen = torch.Generator().manual_seed(8)
    params = [torch.randn(n, generator=gen).mul(0.02).to(torch.bfloat16) for n in numels]
    src = _run(numels, params, 3, 4, 2, seed=3)
    sds = [_state_dict(r, numels, 4) for r in src]
    mid = [Z.reshard_state_dicts(sds, 5, r) for r in range(5)]
    back = [Z.reshard_state_dicts(mid, 3, r) for r in range(3)]
    for a, b in zip(sds, back):
        for k in ("master", "m", "v"):
            assert torch.equal(_bits(a[k]), _bits(b[k]))
        assert a["layout"] == b["layout"] and a["state"] == b["state"]


def test_reshard_rejects_incomplete_or_inconsistent_sets():
    numels = [10, 20]
    params = [torch.zeros(n, dtype=torch.bfloat16) for n in numels]
    src = _run(numels, params, 2, 1, 1, seed=1)
    sds = [_state_dict(r, numels, 1) for r in src]
    with pytest.raises(ValueError, match="all 2 ranks"):
        Z.reshard_state_dicts(sds[:1], 1, 0)
    with pytest.raises(ValueError, match="twice"):
        Z.reshard_state_dicts([sds[0], sds[0]], 1, 0)
    other = dict(sds[1], state=dict(sds[1]["state"], step_t=math.inf))
    with pytest.raises(ValueError, match="differ"):
        Z.reshard_state_dicts([sds[0], other], 1, 0)
    with pytest.raises(ValueError, match="state dict"):
        Z.reshard_state_dicts([dict(sds[0], format="x"), sds[1]], 1, 0)
    moved = dict(sds[1], layout=dict(sds[1]["layout"], numels=[10, 21]))
    with pytest.raises(ValueError, match="different layouts"):
        Z.reshard_state_dicts([sds[0], moved], 1, 0)
    with pytest.raises(Z.ZsInvalidArgument):
        Z.reshard_state_dicts(sds, 2, 2)  # no rank 2 in a group of two
