"""Pins of the CPU oracle against values fixed by the pages or by mathematics.

Each test checks the oracle against something other than itself: the worked
example printed on the pages, closed forms of AdamW, brute force with exact
rationals, exhaustive sweeps of every 16-bit pattern, and library routines the
pages name (torch.optim.AdamW, torch.nn.utils.clip_grad_norm_, torch.cat).
"""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, max_norm=1.0)


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _f32(x):
    return torch.tensor(x, dtype=torch.float32)


# ------------------------------------------------------------------------------------------
# The pages' worked example: sharded SGD with two replicas ("Deep dive: Megatron",
# section "Distributed optimizer").  AdamW with beta1 = beta2 = 0, no decay and a huge eps
# is SGD with step lr/eps: with eps = 2^30 and lr = 0.1 * 2^30 the update is
# 0.1 * g * (1 - |g|/(|g| + eps)), within 4e-9 of plain SGD, below half an fp32 ulp of
# the printed results.
# ------------------------------------------------------------------------------------------

def test_page_sharded_sgd_example_through_adamw_limit():
    ex = _load("sharded_sgd_example.json")
    d = ex["dp_world"]
    # The omitted reduce-scatter: an equal-weight mean of the replicas, as on the page.
    reduced = [sum(g[i] for g in ex["replica_gradients"]) / d for i in range(len(ex["parameters"]))]
    hp = dict(lr=ex["lr"] * 2.0 ** 30, beta1=0.0, beta2=0.0, eps=2.0 ** 30, weight_decay=0.0, max_norm=0.0)
    params = [torch.tensor(ex["parameters"], dtype=torch.float16)]
    grads_flat = torch.tensor(reduced, dtype=torch.float16)
    layouts = [O.plan_layout([4], d, r) for r in range(d)]
    owned = []
    parts = [O.sumsq_unscaled(O.shard_of(grads_flat, lay), 1.0) for lay in layouts]
    for r in range(d):
        rank = O.OracleRank([4], d, r, params, O.OracleScaler(1.0, dynamic=False), hp)
        rec = rank.step(O.shard_of(grads_flat, rank.layout), other_sumsq=parts)
        assert not rec["overflow"] and rec["clip"] == 1.0
        owned.append(rank.master)
    # Rank r owns the r-th contiguous half, exactly as the page's ownership list.
    assert torch.equal(owned[0], _f32(ex["updated"][:2]))
    assert torch.equal(owned[1], _f32(ex["updated"][2:]))
    assert torch.equal(torch.cat(owned), _f32(ex["updated"]))


def test_page_divisibility_and_byte_ledger():
    ex = _load("sharded_sgd_example.json")
    led = _load("byte_ledger.json")
    lay = O.plan_layout([4], 2, 1)
    assert (lay.flat_numel, lay.shard_numel, lay.shard_begin) == (4, 2, 2)
    # Replicated 2-byte param + 4-byte main grad, 12 shardable fp32 bytes (master, m, v).
    for d, want in led["bytes_by_group_size"].items():
        d = int(d)
        lay = O.plan_layout([1 << 20], d, 0)
        shard_state_bytes = 3 * 4 * lay.shard_numel          # fp32 master, m, v of one shard
        per_param = led["replicated_bytes"] + shard_state_bytes / (1 << 20)
        assert per_param == want
    assert 6 + 12 / 8 == ex["bytes_per_parameter_at_d8"]
    assert 2 + 2 + 12 == led["bytes_per_param_2byte_grads"]


def test_page_token_weighting_through_sgd_limit():
    """The reduction must match the loss normalisation: 5.0 vs 2.5 and 0.5 vs 0.75."""
    tw = _load("sharded_sgd_example.json")["token_weighting"]
    means, toks = tw["local_means"], tw["valid_tokens"]
    wrong = sum(means) / len(means)
    right = sum(g * c for g, c in zip(means, toks)) / sum(toks)
    assert (wrong, right) == (tw["replica_mean_gradient"], tw["token_weighted_gradient"])
    hp = dict(lr=0.1 * 2.0 ** 30, beta1=0.0, beta2=0.0, eps=2.0 ** 30, weight_decay=0.0, max_norm=0.0)
    for g, want in ((wrong, tw["param_after_replica_mean"]), (right, tw["param_after_token_weighted"])):
        rank = O.OracleRank([1], 1, 0, [torch.tensor([1.0], dtype=torch.float16)], O.OracleScaler(1.0, dynamic=False), hp)
        rank.step(torch.tensor([g], dtype=torch.float16))
        assert rank.master.item() == np.float32(want)


# ------------------------------------------------------------------------------------------
# AdamW: closed forms, and the library routine the pages name (torch.optim.AdamW)
# ------------------------------------------------------------------------------------------

def _run_oracle_adamw(p0, grads, hp, loss_scale=1.0, clip=1.0):
    master = _f32(p0)
    m = torch.zeros_like(master)
    v = torch.zeros_like(master)
    for t, g in enumerate(grads, start=1):
        master, m, v = O.adamw_update(master, m, v, g, loss_scale, clip, t, hp)
    return master, m, v


def test_adamw_closed_form_constant_gradient():
    # Constant g from zero moments: m_hat = g and sqrt(v_hat) = |g| exactly, so
    # p_t = (1-lam)^t p0 - lr * g/(|g|+eps) * sum_{k<t} (1-lam)^k with lam = lr*wd,
    # m_t = g (1 - beta1^t), v_t = g^2 (1 - beta2^t).
    T = 10
    p0 = [1.0, -0.75, 0.02, 3.0]
    gval = [0.5, -0.25, 1e-3, 2.0 ** -10]
    g = torch.tensor(gval, dtype=torch.float32)
    master, m, v = _run_oracle_adamw(p0, [g] * T, HP)
    lam = HP["lr"] * HP["weight_decay"]
    for i in range(4):
        geo = sum((1 - lam) ** k for k in range(T))
        p_cf = (1 - lam) ** T * p0[i] - HP["lr"] * gval[i] / (abs(gval[i]) + HP["eps"]) * geo
        m_cf = gval[i] * (1 - HP["beta1"] ** T)
        v_cf = gval[i] ** 2 * (1 - HP["beta2"] ** T)
        # Each step rounds the stored fp32 values once: a few fp32 ulps over 10 steps.
        assert abs(master[i].item() - p_cf) <= 12 * 2.0 ** -24 * (abs(p_cf) + HP["lr"])
        assert abs(m[i].item() - m_cf) <= 12 * 2.0 ** -24 * abs(m_cf)
        assert abs(v[i].item() - v_cf) <= 12 * 2.0 ** -24 * abs(v_cf)
    # Worked value: p0 = 1, g = 0.5 gives p_10 = 0.98990047 in fp32 (the closed form rounds there too).
    assert master[0].item() == np.float32(0.98990047)


def test_adamw_zero_gradient_is_pure_decoupled_decay():
    master, m, v = _run_oracle_adamw([1.0, -2.0], [torch.zeros(2)] * 10, HP)
    lam = HP["lr"] * HP["weight_decay"]
    assert abs(master[0].item() - (1 - lam) ** 10) <= 10 * 2.0 ** -24
    assert abs(master[1].item() + 2 * (1 - lam) ** 10) <= 20 * 2.0 ** -24
    assert torch.count_nonzero(m) == 0 and torch.count_nonzero(v) == 0


def test_adamw_eps_added_after_the_root():
    # g = eps = 2^-27 with betas 1/2 and 3/4 (every moment exact in fp32): the update is
    # lr * g / (|g| + eps) = lr / 2 exactly at t = 1; eps inside the square root would give
    # lr * 2^-27 / sqrt(2^-54 + 2^-27), about lr * 2^-13.5.
    hp = dict(HP, weight_decay=0.0, beta1=0.5, beta2=0.75, eps=2.0 ** -27)
    master, _, _ = _run_oracle_adamw([0.0], [torch.tensor([2.0 ** -27])], hp)
    assert master.item() == np.float32(-hp["lr"] / 2)


def test_adamw_zero_lr_keeps_params_and_moves_moments():
    hp = dict(HP, lr=0.0)
    gs = [torch.tensor([0.5, -1.0]) for _ in range(3)]
    master, m, v = _run_oracle_adamw([0.25, 0.5], gs, hp)
    assert torch.equal(master, _f32([0.25, 0.5]))
    assert abs(m[0].item() - 0.5 * (1 - 0.9 ** 3)) < 1e-7


def _torch_adamw_one_step(p, m, v, g, t, hp):
    """One step of torch.optim.AdamW in fp64 from a given fp32 state at step count t-1."""
    prm = torch.nn.Parameter(p.double().clone())
    opt = torch.optim.AdamW([prm], lr=hp["lr"], betas=(hp["beta1"], hp["beta2"]), eps=hp["eps"],
                            weight_decay=hp["weight_decay"], foreach=False)
    prm.grad = g.double()
    opt.step()  # creates the state at step 1 ...
    if t > 1:   # ... so redo it from the requested state
        prm.data.copy_(p.double())
        st = opt.state[prm]
        st["exp_avg"].copy_(m.double())
        st["exp_avg_sq"].copy_(v.double())
        st["step"].fill_(t - 1)
        opt.step()
    st = opt.state[prm]
    return prm.detach(), st["exp_avg"], st["exp_avg_sq"]


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_adamw_matches_torch_optim_adamw_step_by_step(seed):
    # torch.optim.AdamW (the optimizer the pages instantiate) run in fp64 for one step from
    # the oracle's fp32 state, at every t = 1..10.  The moments agree to one fp32 ulp (torch
    # forms m by lerp, whose fp64 rounding differs under cancellation, so a few per cent
    # of the roundings land on the neighbouring fp32 value); torch feeds its unrounded
    # fp64 moments into the parameter update where the oracle uses the stored fp32 ones,
    # which moves p by at most lr * 2^-24 * |m_hat/den| beyond half an ulp.
    gen = torch.Generator().manual_seed(seed)
    n = 4096
    hp = dict(HP, weight_decay=0.1 * (seed + 1))
    master = (torch.randn(n, generator=gen) * 0.02).float()
    m = torch.zeros(n)
    v = torch.zeros(n)
    for t in range(1, 11):
        g = (torch.randn(n, generator=gen) * 1e-3).float()
        p_ref, m_ref, v_ref = _torch_adamw_one_step(master, m, v, g, t, hp)
        master, m, v = O.adamw_update(master, m, v, g, 1.0, 1.0, t, hp)
        for a, b in ((m, m_ref), (v, v_ref)):
            ulp = b.abs().mul(2.0 ** -23)
            assert torch.all((a.double() - b).abs() <= ulp)
            assert int((a != b.float()).sum()) <= n // 64
        ratio = (m_ref / (1 - hp["beta1"] ** t)).abs() / ((v_ref / (1 - hp["beta2"] ** t)).sqrt() + hp["eps"])
        bound = p_ref.abs().mul(2.0 ** -24) + hp["lr"] * 2.0 ** -23 * ratio + 1e-30
        assert torch.all((master.double() - p_ref).abs() <= bound)


def test_adamw_unscale_and_clip_enter_as_one_product():
    # Loss scale 2^16 and clip 0.25 are the same as feeding g * 0.25 unscaled.
    gen = torch.Generator().manual_seed(7)
    x = (torch.randn(512, generator=gen) * 3.0).to(torch.float16)
    p0 = [0.01] * 512
    a = _run_oracle_adamw(p0, [x], HP, loss_scale=2.0 ** 16, clip=0.25)
    b = _run_oracle_adamw(p0, [x.double() * 0.25 / 2.0 ** 16], HP)
    for u, w in zip(a, b):
        assert torch.equal(u, w)


# ------------------------------------------------------------------------------------------
# Norm and clip coefficient
# ------------------------------------------------------------------------------------------

def test_sumsq_matches_exact_rationals():
    gen = torch.Generator().manual_seed(3)
    for dtype in (torch.float16, torch.bfloat16):
        x = (torch.randn(257, generator=gen) * 5).to(dtype)
        exact = sum(Fraction(float(v)) ** 2 for v in x.tolist()) / Fraction(2 ** 10) ** 2
        got = O.sumsq_unscaled(x, 2.0 ** 10)
        assert abs(Fraction(got) - exact) <= exact * Fraction(1, 2 ** 45)


def test_sumsq_special_cases_and_invariants():
    assert O.sumsq_unscaled(torch.zeros(100, dtype=torch.bfloat16), 1.0) == 0.0
    one = torch.zeros(1000, dtype=torch.float16)
    one[417] = -3.5
    assert math.sqrt(O.sumsq_unscaled(one, 1.0)) == 3.5
    gen = torch.Generator().manual_seed(4)
    x = (torch.randn(4096, generator=gen)).to(torch.float16)
    # Power-of-two scale: unscaling is exact, so the sum scales exactly.
    assert O.sumsq_unscaled(x, 2.0 ** 8) * 2.0 ** 16 == O.sumsq_unscaled(x, 1.0)
    # Splitting over ranks changes only the fp64 rounding order.
    whole = O.sumsq_unscaled(x, 1.0)
    parts = [O.sumsq_unscaled(x[i * 1024:(i + 1) * 1024], 1.0) for i in range(4)]
    assert abs(O.global_sumsq(parts) - whole) <= 1e-14 * whole


def test_clip_coefficient_matches_clip_grad_norm():
    gen = torch.Generator().manual_seed(5)
    for scale, max_norm in ((1e-3, 1.0), (1.0, 1.0), (0.1, 0.5), (3.0, 2.0)):
        grads = [torch.randn(300, generator=gen, dtype=torch.float64) * scale for _ in range(3)]
        ss = sum(float((g * g).sum()) for g in grads)
        norm, c = O.clip_coefficient(ss, max_norm)
        work = [g.clone() for g in grads]
        ref_norm = torch.nn.utils.clip_grad_norm_(_as_params(work), max_norm)
        assert abs(norm - float(ref_norm)) <= 1e-13 * norm
        ratio = float(work[0][0] / grads[0][0])
        assert abs(c - ratio) <= 1e-15
    assert O.clip_coefficient(4.0, 0.0) == (2.0, 1.0)
    assert O.clip_coefficient(0.0, 1.0) == (0.0, 1.0)


def _as_params(tensors):
    ps = []
    for t in tensors:
        p = torch.nn.Parameter(torch.zeros_like(t))
        p.grad = t
        ps.append(p)
    return ps


# ------------------------------------------------------------------------------------------
# Overflow flag: exhaustive over every 16-bit pattern against torch.isfinite
# ------------------------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
def test_nonfinite_flag_exhaustive(dtype):
    allbits = torch.arange(-32768, 32768, dtype=torch.int32).to(torch.int16).view(dtype)
    fin = torch.isfinite(allbits.float())
    assert O.nonfinite_any(allbits[fin]) is False
    for v in allbits[~fin].tolist()[:: 97] + [math.inf, -math.inf, math.nan]:
        x = torch.zeros(33, dtype=dtype)
        x[17] = v
        assert O.nonfinite_any(x) is True
    assert int((~fin).sum()) == (2 * 1024 if dtype == torch.float16 else 2 * 128)


# ------------------------------------------------------------------------------------------
# Casts: round-to-nearest-even at ties, fp16 overflow
# ------------------------------------------------------------------------------------------

def test_cast_ties_round_to_even():
    # bf16 keeps 7 fraction bits: 1 + 2^-8 is the midpoint of 1 and 1 + 2^-7.
    x = _f32([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 1 + 2 ** -8 + 2 ** -20])
    assert O.cast_to(x, torch.bfloat16).float().tolist() == [1.0, 1 + 2 ** -6, -1.0, 1 + 2 ** -7]
    # fp16 keeps 10 fraction bits.
    y = _f32([1 + 2 ** -11, 1 + 3 * 2 ** -11, 65519.0, 65520.0])
    assert O.cast_to(y, torch.float16).float().tolist() == [1.0, 1 + 2 ** -9, 65504.0, math.inf]


# ------------------------------------------------------------------------------------------
# Layout, pack, unpack
# ------------------------------------------------------------------------------------------

@pytest.mark.parametrize("align", [1, 8, 64])
@pytest.mark.parametrize("dp_world", [1, 2, 3, 4])
def test_layout_pack_unpack_roundtrip(align, dp_world):
    gen = torch.Generator().manual_seed(align * 10 + dp_world)
    numels = [int(x) for x in torch.randint(0, 300, (37,), generator=gen)]
    tensors = [torch.randn(n, generator=gen).to(torch.bfloat16) for n in numels]
    lays = [O.plan_layout(numels, dp_world, r, align) for r in range(dp_world)]
    lay = lays[0]
    assert lay.flat_numel % (dp_world * align) == 0
    assert lay.flat_numel - (lay.offsets[-1] + numels[-1]) < dp_world * align
    assert all(o % align == 0 for o in lay.offsets)
    # Shards tile the buffer exactly, in rank order, with equal sizes.
    assert [x.shard_begin for x in lays] == [r * lay.shard_numel for r in range(dp_world)]
    flat = O.pack(tensors, lay)
    if align == 1:
        assert torch.equal(flat[:sum(numels)], torch.cat(tensors))
    # Gaps and tail are zero: the padded buffer holds exactly the tensors' bits.
    mask = torch.zeros(lay.flat_numel, dtype=torch.bool)
    for off, n in zip(lay.offsets, numels):
        mask[off:off + n] = True
    assert torch.count_nonzero(flat[~mask].float()) == 0
    back = torch.split(flat[mask], numels)
    assert all(torch.equal(a, b) for a, b in zip(back, tensors))
    # Unpack of every shard restores the tensors; fp32 master round trip is exact.
    out = [torch.full_like(t, 7.0) for t in tensors]
    for x in lays:
        master = O.shard_of(O.pack(tensors, x, torch.float32), x)
        out = O.unpack(master, x, out, whole_flat=False)
    assert all(torch.equal(a, b) for a, b in zip(out, tensors))
    out2 = O.unpack(flat, lay, [torch.zeros_like(t) for t in tensors], whole_flat=True)
    assert all(torch.equal(a, b) for a, b in zip(out2, tensors))


def test_pack_widening_to_fp32_is_exact():
    """Seeding the fp32 master widens bf16 and fp16 values exactly: bf16 shares fp32's
    exponent range (values near 2^127 and subnormals down to 2^-133 survive), fp16's
    largest and smallest values are far inside it."""
    bf = [2.0 ** 100, -(2.0 ** -130), 3 * 2.0 ** -133, 1 + 2.0 ** -7, -1.5 * 2.0 ** 127, 0.0]
    hf = [65504.0, -(2.0 ** -24), 1 + 2.0 ** -10, -3 * 2.0 ** -20]
    lay = O.plan_layout([len(bf), len(hf)], 1, 0)
    src = [torch.tensor(bf, dtype=torch.bfloat16), torch.tensor(hf, dtype=torch.float16)]
    assert src[0].double().tolist() == bf and src[1].double().tolist() == hf  # the inputs are exact
    assert O.pack(src, lay, torch.float32).double().tolist() == bf + hf


def test_unpack_rounds_each_shard_to_nearest_even():
    """The scatter-back of fp32 master shards into bf16 and fp16 tensors, by hand: every value
    is rounded to nearest even (ties included), each rank writes only the elements of its own
    shard, and the rest of each tensor keeps its old value."""
    numels = [3, 5]
    lay0, lay1 = O.plan_layout(numels, 2, 0), O.plan_layout(numels, 2, 1)  # shards [0, 4) and [4, 8)
    t = 2 ** -8  # half a bf16 ulp at 1
    master = _f32([1 + t, 1 + 3 * t, -(1 + t), 1 + t + 2 ** -20, 1 + 2 ** -11, 1 + 3 * 2 ** -11, 65519.0, 2.5])
    old = [torch.full((3,), 9.0, dtype=torch.bfloat16), torch.full((5,), 9.0, dtype=torch.float16)]
    out = O.unpack(master[:4], lay0, old, whole_flat=False)
    assert out[0].float().tolist() == [1.0, 1 + 2 ** -6, -1.0]
    # fp16 keeps 10 fraction bits: 1 + 2^-8 + 2^-20 is 4 ulps and a sliver above 1
    assert out[1].float().tolist() == [1 + 2 ** -8, 9.0, 9.0, 9.0, 9.0]
    out = O.unpack(master[4:], lay1, out, whole_flat=False)
    assert out[0].float().tolist() == [1.0, 1 + 2 ** -6, -1.0]
    # 1 + 2^-11 is a tie (to 1), 1 + 3 * 2^-11 rounds up to 1 + 2^-9, 65519 stays below the overflow at 65520
    assert out[1].float().tolist() == [1 + 2 ** -8, 1.0, 1 + 2 ** -9, 65504.0, 2.5]


def test_layout_rejects_bad_arguments():
    with pytest.raises(ValueError):
        O.plan_layout([4], 2, 2)
    with pytest.raises(ValueError):
        O.plan_layout([4], 1, 0, align=3)
    with pytest.raises(ValueError):
        O.plan_layout([], 1, 0)


# ------------------------------------------------------------------------------------------
# Loss scaler: hand-worked sequences of the rule "a skipped step halves the scale, growth
# after a fixed interval of applied steps", dynamic scaling with window W.
# ------------------------------------------------------------------------------------------

def _run_scaler(s, flags):
    seq = []
    for f in flags:
        before = s.loss_scale
        s = O.scaler_update(s, f)
        seq.append((before, s.step_t, s.growth_tracker, s.loss_scale))
    return s, seq


def test_scaler_tiny_config_sequence():
    # fp16, S0 = 2^16, W = 1000, overflow at step 3 of 5.
    s, seq = _run_scaler(O.OracleScaler(2.0 ** 16, growth_interval=1000), [0, 0, 1, 0, 0])
    assert seq == [(2 ** 16, 1, 1, 2 ** 16), (2 ** 16, 2, 2, 2 ** 16), (2 ** 16, 2, 0, 2 ** 15),
                   (2 ** 15, 3, 1, 2 ** 15), (2 ** 15, 4, 2, 2 ** 15)]
    assert s.skipped_total == 1


def test_scaler_growth_and_backoff_sequence():
    s, seq = _run_scaler(O.OracleScaler(2.0 ** 16, growth_interval=2), [0, 0, 0, 1, 0, 0, 0])
    assert [x[0] for x in seq] == [2 ** 16, 2 ** 16, 2 ** 17, 2 ** 17, 2 ** 16, 2 ** 16, 2 ** 17]
    assert [x[1] for x in seq] == [1, 2, 3, 3, 4, 5, 6]
    assert [x[2] for x in seq] == [1, 0, 1, 0, 1, 0, 1]
    assert [x[3] for x in seq] == [2 ** 16, 2 ** 17, 2 ** 17, 2 ** 16, 2 ** 16, 2 ** 17, 2 ** 17]


def test_scaler_floor_and_static():
    s, seq = _run_scaler(O.OracleScaler(2.0, scale_floor=1.0, growth_interval=5), [1, 1, 1])
    assert [x[3] for x in seq] == [1.0, 1.0, 1.0] and s.step_t == 0 and s.skipped_total == 3
    s, seq = _run_scaler(O.OracleScaler(1.0, dynamic=False), [0, 1, 0, 0, 1])
    assert all(x[3] == 1.0 and x[2] == 0 for x in seq) and s.step_t == 3


def test_scaler_doubles_once_per_window():
    s = O.OracleScaler(2.0 ** 4, growth_interval=7)
    s, _ = _run_scaler(s, [0] * (7 * 5 + 3))
    assert s.loss_scale == 2.0 ** 9 and s.growth_tracker == 3 and s.step_t == 38


# ------------------------------------------------------------------------------------------
# Whole rank: a skipped step leaves everything but the scaler untouched; DP split
# ------------------------------------------------------------------------------------------

def test_rank_skip_leaves_state_untouched():
    gen = torch.Generator().manual_seed(9)
    numels = [100, 37, 1]
    params = [torch.randn(n, generator=gen).mul(0.02).to(torch.float16) for n in numels]
    r = O.OracleRank(numels, 1, 0, params, O.OracleScaler(2.0 ** 16), HP)
    x = (torch.randn(138, generator=gen) * 6).to(torch.float16)
    r.step(x)
    snap = (r.master.clone(), r.m.clone(), r.v.clone(), [p.clone() for p in r.params], r.scaler.step_t)
    bad = x.clone()
    bad[50] = math.nan
    rec = r.step(bad)
    assert rec["overflow"] and r.scaler.loss_scale == 2.0 ** 15 and r.scaler.step_t == snap[4]
    assert torch.equal(r.master, snap[0]) and torch.equal(r.m, snap[1]) and torch.equal(r.v, snap[2])
    assert all(torch.equal(a, b) for a, b in zip(r.params, snap[3]))


def test_dp_split_equals_single_rank_when_unclipped():
    gen = torch.Generator().manual_seed(11)
    numels = [513, 200, 64, 1000, 3]
    params = [torch.randn(n, generator=gen).mul(0.02).to(torch.bfloat16) for n in numels]
    hp = dict(HP, max_norm=1e9)   # clip coefficient exactly 1 on every rank
    single = O.OracleRank(numels, 1, 0, params, O.OracleScaler(1.0, dynamic=False), hp)
    d = 4
    ranks = [O.OracleRank(numels, d, r, params, O.OracleScaler(1.0, dynamic=False), hp) for r in range(d)]
    for step in range(3):
        grads = [torch.randn(n, generator=gen).mul(1e-3).to(torch.bfloat16) for n in numels]
        flat1 = O.pack(grads, single.layout)
        single.step(O.shard_of(flat1, single.layout))
        flat = O.pack(grads, ranks[0].layout)
        parts = [O.sumsq_unscaled(O.shard_of(flat, r.layout), 1.0) for r in ranks]
        for r in ranks:
            r.step(O.shard_of(flat, r.layout), other_sumsq=parts)
    n_real = sum(numels)
    cat = torch.cat([r.master for r in ranks])[:n_real]
    assert torch.equal(cat, single.master[:n_real])
    for i in range(len(numels)):
        merged = params[i].clone()
        for r in ranks:
            owned = O.plan_layout(numels, d, ranks.index(r))
            a = max(owned.offsets[i], owned.shard_begin)
            b = min(owned.offsets[i] + numels[i], owned.shard_begin + owned.shard_numel)
            if a < b:
                merged[a - owned.offsets[i]:b - owned.offsets[i]] = r.params[i][a - owned.offsets[i]:b - owned.offsets[i]]
        assert torch.equal(merged, single.params[i])


# ------------------------------------------------------------------------------------------
# The whole rank step, end to end, against torch: a loss-scaled fp16 list whose global norm
# is large enough to clip, through torch.nn.utils.clip_grad_norm_ over every tensor and then
# torch.optim.AdamW ("3.7 Megatron-LM, DeepSpeed & Parallelism in Practice", sections
# "DeepSpeed config for this run": gradient_clipping 1.0, and "Initializing a DeepSpeed
# Engine": torch.optim.AdamW), for one rank and for two ranks that own equal halves of one
# flat buffer and exchange their partial sums ("Deep dive: Megatron", section "Distributed
# optimizer").  This pins the wiring of OracleRank.step: the norm is global, taken on the
# unscaled gradient, and its clip coefficient and the unscale both reach the update.
# ------------------------------------------------------------------------------------------

STEP_NUMELS = [300, 77, 1024, 5, 640, 1]   # 2047 elements: two ranks split tensor 2
STEP_SCALE = 2.0 ** 12
STEP_HP = dict(HP, weight_decay=0.1)


def _step_inputs(seed, steps):
    """fp16 parameters N(0, 0.02) and `steps` lists of fp16 gradients N(0, 0.1) times the
    loss scale: the unscaled norm is about 4.5, so the clip coefficient is about 0.22."""
    gen = torch.Generator().manual_seed(seed)
    params = [(torch.randn(n, generator=gen) * 0.02).to(torch.float16) for n in STEP_NUMELS]
    grads = [[(torch.randn(n, generator=gen) * 0.1 * STEP_SCALE).to(torch.float16) for n in STEP_NUMELS]
             for _ in range(steps)]
    return params, grads


def _torch_clip_adamw_step(masters, ms, vs, grads_unscaled, t, hp):
    """clip_grad_norm_ over every tensor, then one torch.optim.AdamW step, all in fp64, from
    the given fp32 state at step count t - 1.  Returns (norm, params, m, v) as lists."""
    prms = [torch.nn.Parameter(p.double().clone()) for p in masters]
    opt = torch.optim.AdamW(prms, lr=hp["lr"], betas=(hp["beta1"], hp["beta2"]), eps=hp["eps"],
                            weight_decay=hp["weight_decay"], foreach=False)
    for prm, m, v, g in zip(prms, ms, vs, grads_unscaled):
        prm.grad = g.double().clone()
        opt.state[prm] = {"step": torch.tensor(float(t - 1)), "exp_avg": m.double().clone(),
                          "exp_avg_sq": v.double().clone()}
    norm = float(torch.nn.utils.clip_grad_norm_(prms, hp["max_norm"]))
    opt.step()
    return (norm, [p.detach() for p in prms], [opt.state[p]["exp_avg"] for p in prms],
            [opt.state[p]["exp_avg_sq"] for p in prms])


def _split(flat, offsets, numels):
    return [flat[o:o + n] for o, n in zip(offsets, numels)]


def _assert_step_within_torch_bounds(master, m, v, p_ref, m_ref, v_ref, t, hp):
    """The bounds of the single-tensor AdamW pin: moments within one fp32 ulp of torch's
    fp64 moments, parameters within half an ulp plus what torch's unrounded moments move."""
    for a, b in ((m, m_ref), (v, v_ref)):
        assert torch.all((a.double() - b).abs() <= b.abs().mul(2.0 ** -23)), t
    ratio = (m_ref / (1 - hp["beta1"] ** t)).abs() / ((v_ref / (1 - hp["beta2"] ** t)).sqrt() + hp["eps"])
    bound = p_ref.abs().mul(2.0 ** -24) + hp["lr"] * 2.0 ** -23 * ratio + 1e-30
    assert torch.all((master.double() - p_ref).abs() <= bound), t


@pytest.mark.parametrize("seed", [0, 1])
def test_rank_step_matches_torch_clip_and_adamw(seed):
    params, steps = _step_inputs(seed, 5)
    rank = O.OracleRank(STEP_NUMELS, 1, 0, params, O.OracleScaler(STEP_SCALE), STEP_HP)
    offs = rank.layout.offsets
    for t, grads in enumerate(steps, start=1):
        before = [_split(x, offs, STEP_NUMELS) for x in (rank.master, rank.m, rank.v)]
        rec = rank.step(O.shard_of(O.pack(grads, rank.layout), rank.layout))
        unscaled = [g.double() / STEP_SCALE for g in grads]
        norm, p_ref, m_ref, v_ref = _torch_clip_adamw_step(*before, unscaled, t, STEP_HP)
        assert not rec["overflow"] and rec["loss_scale"] == STEP_SCALE
        assert abs(rec["norm"] - norm) <= 1e-13 * norm
        assert rec["clip"] <= 0.5 and abs(rec["clip"] - STEP_HP["max_norm"] / (norm + 1e-6)) <= 1e-14
        _assert_step_within_torch_bounds(rank.master, rank.m, rank.v, torch.cat(p_ref), torch.cat(m_ref),
                                         torch.cat(v_ref), t, STEP_HP)
        assert rank.scaler.step_t == t


def test_two_ranks_exchanging_partials_match_one_torch_run():
    params, steps = _step_inputs(2, 5)
    d = 2
    ranks = [O.OracleRank(STEP_NUMELS, d, r, params, O.OracleScaler(STEP_SCALE), STEP_HP) for r in range(d)]
    lay = ranks[0].layout
    n_real = sum(STEP_NUMELS)
    assert lay.offsets[2] < lay.shard_numel < lay.offsets[3]   # tensor 2 straddles the ranks
    for t, grads in enumerate(steps, start=1):
        whole = [torch.cat([getattr(r, k) for r in ranks])[:n_real] for k in ("master", "m", "v")]
        before = [_split(x, lay.offsets, STEP_NUMELS) for x in whole]
        flat = O.pack(grads, lay)
        shards = [O.shard_of(flat, r.layout) for r in ranks]
        parts = [O.sumsq_unscaled(s, STEP_SCALE) for s in shards]
        recs = [r.step(s, other_sumsq=parts) for r, s in zip(ranks, shards)]
        unscaled = [g.double() / STEP_SCALE for g in grads]
        norm, p_ref, m_ref, v_ref = _torch_clip_adamw_step(*before, unscaled, t, STEP_HP)
        for rec in recs:
            assert abs(rec["norm"] - norm) <= 1e-13 * norm and rec["clip"] <= 0.5
        assert recs[0]["clip"] == recs[1]["clip"]
        after = [torch.cat([getattr(r, k) for r in ranks])[:n_real] for k in ("master", "m", "v")]
        _assert_step_within_torch_bounds(*after, torch.cat(p_ref), torch.cat(m_ref), torch.cat(v_ref), t,
                                         STEP_HP)


# ------------------------------------------------------------------------------------------
# Gradient accumulation into the flat buffer (the step before the path)
# ------------------------------------------------------------------------------------------

def test_accumulate_fp32_matches_exact_sums():
    from fractions import Fraction as F
    gen = torch.Generator().manual_seed(21)
    numels = [37, 100, 5]
    lay = O.plan_layout(numels, 1, 0)
    micro = [[(torch.randn(n, generator=gen) * 10 ** k).to(torch.bfloat16) for n in numels] for k in (-3, 0, 2, -1)]
    acc = O.pack(micro[0], lay, torch.float32)
    for m in micro[1:]:
        acc = O.accumulate(acc, m, lay)
    flat = [O.pack(m, lay, torch.float32) for m in micro]
    for i in range(lay.flat_numel):
        # sequential fp32 accumulation: each step is the exact sum rounded once to fp32
        x = flat[0][i].item()
        for f in flat[1:]:
            x = float(torch.tensor(float(F(x) + F(f[i].item())), dtype=torch.float32))
        assert acc[i].item() == x


def test_accumulate_model_dtype_rounds_to_nearest_even():
    lay = O.plan_layout([4], 1, 0)
    acc = torch.tensor([1.0, 1.0, 1.0 + 2 ** -7, 256.0], dtype=torch.bfloat16)
    g = [torch.tensor([2 ** -8, 3 * 2 ** -8, 2 ** -8, 1.0], dtype=torch.bfloat16)]
    out = O.accumulate(acc, g, lay)
    # 1 + 2^-8 is a tie -> 1.0 (even); 1 + 3*2^-8 -> 1 + 2^-6; (1 + 2^-7) + 2^-8 is a tie -> 1 + 2^-6
    # (even mantissa); 256 + 1 is a tie between 256 and 258 -> 256.
    assert out.float().tolist() == [1.0, 1.0 + 2 ** -6, 1.0 + 2 ** -6, 256.0]


def test_accumulate_then_step_equals_step_on_summed_gradient():
    """G micro-steps accumulated in fp32 then one step == one step on the exactly summed
    gradient, when every partial sum is exact (small integers)."""
    numels = [64, 3]
    lay = O.plan_layout(numels, 1, 0)
    micro = [[torch.full((n,), float(k + 1), dtype=torch.float16) for n in numels] for k in range(4)]
    acc = O.pack(micro[0], lay, torch.float32)
    for m in micro[1:]:
        acc = O.accumulate(acc, m, lay)
    assert torch.equal(acc, torch.full((67,), 10.0))
    hp = dict(HP)
    r1 = O.OracleRank(numels, 1, 0, [torch.zeros(n, dtype=torch.float16) for n in numels],
                      O.OracleScaler(1.0, dynamic=False), hp)
    r2 = O.OracleRank(numels, 1, 0, [torch.zeros(n, dtype=torch.float16) for n in numels],
                      O.OracleScaler(1.0, dynamic=False), hp)
    r1.step(acc)
    r2.step(torch.full((67,), 10.0, dtype=torch.float16))
    assert torch.equal(r1.master, r2.master) and torch.equal(r1.v, r2.v)


def test_nonfinite_flag_fp32_accumulator():
    x = torch.zeros(10)
    assert O.nonfinite_any(x) is False
    for v in (math.inf, -math.inf, math.nan):
        y = x.clone()
        y[3] = v
        assert O.nonfinite_any(y) is True
    big = torch.tensor([3.4e38, -3.4e38, 1e-45])
    assert O.nonfinite_any(big) is False


# ------------------------------------------------------------------------------------------
# Gradient buckets ("Deep dive: Megatron", section "Distributed optimizer": communication
# starts as buckets of the contiguous buffer become ready; "DeepSpeed config for this run":
# reduce_bucket_size).
# ------------------------------------------------------------------------------------------

def test_plan_buckets_hand_tables():
    # Worked by hand: walk 4,3 | 2,5 | 3 from the end with a bucket size of 6.
    assert O.plan_buckets([3, 5, 2, 7, 1], 6) == [(3, 5), (1, 3), (0, 1)]
    assert O.plan_buckets([3, 5, 2, 7, 1], 100) == [(0, 5)]
    assert O.plan_buckets([3, 5, 2, 7, 1], 1) == [(4, 5), (3, 4), (2, 3), (1, 2), (0, 1)]
    # A tensor above the size is a bucket of its own; it is never split.
    assert O.plan_buckets([2, 50, 2], 10) == [(1, 3), (0, 1)]
    # An empty tensor adds nothing and joins the bucket being filled.
    assert O.plan_buckets([4, 0, 4], 4) == [(2, 3), (0, 2)]
    assert O.plan_buckets([7], 3) == [(0, 1)]


@pytest.mark.parametrize("seed", range(6))
def test_plan_buckets_against_suffix_sum_definition(seed):
    # The same split from prefix sums: a bucket ending at `hi` starts at the largest t
    # with numels[t:hi] >= size, or at 0 when there is none.
    rng = np.random.default_rng(seed)
    numels = [int(x) for x in rng.integers(0, 40, size=int(rng.integers(1, 30)))]
    size = int(rng.integers(1, 90))
    pre = np.concatenate([[0], np.cumsum(numels)])
    want, hi = [], len(numels)
    while hi > 0:
        ok = [t for t in range(hi) if pre[hi] - pre[t] >= size]
        lo = max(ok) if ok else 0
        want.append((lo, hi))
        hi = lo
    assert O.plan_buckets(numels, size) == want


def test_bucket_range_hand_table():
    # sizes 5, 3, 10 at a 8-element alignment: offsets 0, 8, 16, flat length 32.  The gap
    # behind a tensor and the tail belong to the bucket in front of them.
    lay = O.plan_layout([5, 3, 10], 1, 0, 8)
    assert (lay.offsets, lay.flat_numel) == ([0, 8, 16], 32)
    assert O.bucket_range(lay, 0, 1) == (0, 8)
    assert O.bucket_range(lay, 1, 2) == (8, 16)
    assert O.bucket_range(lay, 2, 3) == (16, 32)
    assert O.bucket_range(lay, 0, 2) == (0, 16)
    assert O.bucket_range(lay, 0, 3) == (0, 32)


@pytest.mark.parametrize("align,dp_world", [(1, 1), (64, 4), (8, 3)])
def test_bucket_ranges_tile_the_flat_buffer(align, dp_world):
    rng = np.random.default_rng(align + dp_world)
    numels = [int(x) for x in rng.integers(0, 300, size=23)]
    lay = O.plan_layout(numels, dp_world, 0, align)
    cuts = sorted(set(int(c) for c in rng.integers(1, 23, size=6)))
    bounds = list(zip([0] + cuts, cuts + [23]))
    ranges = [O.bucket_range(lay, a, b) for a, b in bounds]
    assert ranges[0][0] == 0 and ranges[-1][1] == lay.flat_numel
    for (b0, e0), (b1, _) in zip(ranges, ranges[1:]):
        assert e0 == b1
    for (a, b), (lo, hi) in zip(bounds, ranges):
        for t in range(a, b):  # every element of a member tensor lies inside its bucket
            assert lo <= lay.offsets[t] and lay.offsets[t] + numels[t] <= hi
    with pytest.raises(ValueError):
        O.bucket_range(lay, 3, 3)


@pytest.mark.parametrize("accumulate_into", [False, True])
def test_buckets_in_any_order_rebuild_the_whole_pack(accumulate_into):
    torch.manual_seed(7)
    numels = [5, 0, 17, 64, 3, 129, 1, 40]
    lay = O.plan_layout(numels, 2, 1, 8)
    ts = [torch.randn(n).to(torch.bfloat16) for n in numels]
    start = torch.randn(lay.flat_numel).to(torch.bfloat16)
    # concatenation with zero gaps, built directly from the offsets
    cat = torch.zeros(lay.flat_numel, dtype=torch.bfloat16)
    for t, off in zip(ts, lay.offsets):
        cat[off:off + t.numel()] = t
    want = (start.double() + cat.double()).to(torch.bfloat16) if accumulate_into else cat
    buf = start.clone()
    for a, b in [(5, 8), (0, 2), (2, 5)]:
        buf = O.pack_bucket(buf, ts, lay, a, b, accumulate_into=accumulate_into)
    assert torch.equal(buf.view(torch.int16), want.view(torch.int16))
    # one bucket touches its own range only
    one = O.pack_bucket(start, ts, lay, 2, 5, accumulate_into=accumulate_into)
    lo, hi = O.bucket_range(lay, 2, 5)
    assert torch.equal(one[:lo].view(torch.int16), start[:lo].view(torch.int16))
    assert torch.equal(one[hi:].view(torch.int16), start[hi:].view(torch.int16))


# ------------------------------------------------------------------------------------------
# No-decay tensors (a second parameter group with weight_decay 0)
# ------------------------------------------------------------------------------------------

def test_no_decay_tensors_closed_form():
    # zero gradients for 10 steps: decayed tensors shrink by (1 - lr*wd)^t, no-decay
    # tensors keep their value exactly
    lay = O.plan_layout([2, 3, 1], 1, 0)
    mask = O.decay_mask(lay, [False, True, False])
    assert mask.tolist() == [True, True, False, False, False, True]
    p = torch.tensor([1.0, -2.0, 0.5, 0.25, -0.75, 3.0])
    m = torch.zeros(6)
    v = torch.zeros(6)
    for t in range(1, 11):
        p, m, v = O.adamw_update(p, m, v, torch.zeros(6), 1.0, 1.0, t, HP, mask)
    lam = HP["lr"] * HP["weight_decay"]
    assert p[2:5].tolist() == [0.5, 0.25, -0.75]
    for i, x0 in ((0, 1.0), (1, -2.0), (5, 3.0)):
        assert abs(p[i].item() - x0 * (1 - lam) ** 10) <= 10 * abs(x0) * 2.0 ** -24


def test_no_decay_mask_follows_the_shard():
    # four ranks over [5, 0, 9, 2] at align 2: the mask of each rank is its slice of the
    # whole-buffer mask
    numels, nd = [5, 0, 9, 2], [True, False, False, True]
    full = O.decay_mask(O.plan_layout(numels, 1, 0, 2), nd)
    whole = torch.ones(O.plan_layout(numels, 4, 0, 2).flat_numel, dtype=torch.bool)
    whole[:full.numel()] = full
    parts = [O.decay_mask(O.plan_layout(numels, 4, r, 2), nd) for r in range(4)]
    assert torch.equal(torch.cat(parts), whole)


def test_no_decay_group_matches_torch_param_groups():
    # torch.optim.AdamW with two parameter groups (weight_decay wd and 0) in fp64, one step
    # from the oracle's fp32 state, for t = 1..5; same bounds as the single-group pin
    gen = torch.Generator().manual_seed(11)
    n1, n2 = 3000, 1096
    hp = dict(HP, weight_decay=0.3)
    lay = O.plan_layout([n1, n2], 1, 0)
    mask = O.decay_mask(lay, [False, True])
    master = (torch.randn(n1 + n2, generator=gen) * 0.02).float()
    m = torch.zeros(n1 + n2)
    v = torch.zeros(n1 + n2)
    for t in range(1, 6):
        g = (torch.randn(n1 + n2, generator=gen) * 1e-3).float()
        refs = []
        for sl, wd in ((slice(0, n1), hp["weight_decay"]), (slice(n1, n1 + n2), 0.0)):
            refs.append(_torch_adamw_one_step(master[sl], m[sl], v[sl], g[sl], t, dict(hp, weight_decay=wd)))
        p_ref, m_ref, v_ref = (torch.cat([r[i] for r in refs]) for i in range(3))
        master, m, v = O.adamw_update(master, m, v, g, 1.0, 1.0, t, hp, mask)
        for a, b in ((m, m_ref), (v, v_ref)):
            assert torch.all((a.double() - b).abs() <= b.abs().mul(2.0 ** -23))
        ratio = (m_ref / (1 - hp["beta1"] ** t)).abs() / ((v_ref / (1 - hp["beta2"] ** t)).sqrt() + hp["eps"])
        bound = p_ref.abs().mul(2.0 ** -24) + hp["lr"] * 2.0 ** -23 * ratio + 1e-30
        assert torch.all((master.double() - p_ref).abs() <= bound)
