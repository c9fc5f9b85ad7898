"""The pins catch plausible mistakes: each test plants one mistake in the oracle (on the CPU,
by monkeypatching) and checks that at least one pin of test_oracle_pins.py then fails."""

import math

import pytest
import torch

import oracle
import oracle.zs_oracle as Z
import test_oracle_pins as P


def _patch(monkeypatch, name, fn):
    monkeypatch.setattr(Z, name, fn)
    monkeypatch.setattr(oracle, name, fn)


def _fails(*tests):
    """True when at least one of the pin functions raises AssertionError."""
    for t in tests:
        try:
            t()
        except AssertionError:
            return True
    return False


ADAMW_PINS = (P.test_adamw_closed_form_constant_gradient, P.test_adamw_zero_gradient_is_pure_decoupled_decay,
              P.test_adamw_eps_added_after_the_root, P.test_page_sharded_sgd_example_through_adamw_limit,
              lambda: P.test_adamw_matches_torch_optim_adamw_step_by_step(0))


def _adamw_variant(kind):
    def f(master, m, v, x, loss_scale, clip, t, hp):
        lr, b1, b2, eps, wd = hp["lr"], hp["beta1"], hp["beta2"], hp["eps"], hp["weight_decay"]
        g = x.double() / loss_scale * clip
        p = master.double()
        if kind == "coupled_decay":
            g = g + wd * p
        m_t = (b1 * m.double() + (1 - b1) * g).float()
        v_t = ((b1 if kind == "beta1_for_v" else b2) * v.double() + (1 - b2) * g * g).float()
        tt = t + 1 if kind == "t_off_by_one" else t
        m_hat = m_t.double() / (1 if kind == "no_bias_correction" else (1 - b1 ** tt))
        v_hat = v_t.double() / (1 if kind == "no_bias_correction" else (1 - b2 ** tt))
        den = (v_hat + eps).sqrt() if kind == "eps_inside_root" else v_hat.sqrt() + eps
        decay = 1.0 if kind == "coupled_decay" else (1 - lr * wd)
        step = lr * m_hat / den
        p_t = (p * decay + step) if kind == "wrong_sign" else (p * decay - step)
        return p_t.float(), m_t, v_t
    return f


@pytest.mark.parametrize("kind", ["no_bias_correction", "eps_inside_root", "coupled_decay", "wrong_sign",
                                  "beta1_for_v", "t_off_by_one"])
def test_adamw_mistakes_are_caught(monkeypatch, kind):
    _patch(monkeypatch, "adamw_update", _adamw_variant(kind))
    assert _fails(*ADAMW_PINS), kind


def test_norm_without_unscale_is_caught(monkeypatch):
    _patch(monkeypatch, "sumsq_unscaled", lambda x, s: float((x.double() ** 2).sum()) if x.numel() else 0.0)
    assert _fails(P.test_sumsq_matches_exact_rationals, P.test_sumsq_special_cases_and_invariants)


@pytest.mark.parametrize("kind", ["no_eps", "no_min"])
def test_clip_mistakes_are_caught(monkeypatch, kind):
    def f(ss, max_norm):
        n = math.sqrt(ss)
        if max_norm <= 0:
            return n, 1.0
        if kind == "no_eps":
            return n, min(1.0, max_norm / n) if n > 0 else 1.0
        return n, max_norm / (n + 1e-6)
    _patch(monkeypatch, "clip_coefficient", f)
    assert _fails(P.test_clip_coefficient_matches_clip_grad_norm)


def test_overflow_only_inf_is_caught(monkeypatch):
    def f(x):
        if x.numel() == 0:
            return False
        return bool(torch.isinf(x.float()).any())
    _patch(monkeypatch, "nonfinite_any", f)
    assert _fails(lambda: P.test_nonfinite_flag_exhaustive(torch.float16),
                  lambda: P.test_nonfinite_flag_exhaustive(torch.bfloat16))


def test_truncating_cast_is_caught(monkeypatch):
    def f(x, dtype):
        # round toward zero: clear the dropped mantissa bits before rounding
        bits = x.float().contiguous().view(torch.int32)
        keep = 16 if dtype == torch.bfloat16 else 13
        return (bits & ~((1 << keep) - 1)).view(torch.float32).to(dtype)
    _patch(monkeypatch, "cast_to", f)
    assert _fails(P.test_cast_ties_round_to_even)


def test_layout_mistake_is_caught(monkeypatch):
    real = Z.plan_layout

    def f(numels, dp_world, dp_rank, align=1):
        lay = real(numels, dp_world, dp_rank, align)
        # pad only the tail to dp_world (forgetting the per-tensor alignment)
        pos = 0
        offs = []
        for n in numels:
            offs.append(pos)
            pos += n
        lay.offsets = offs
        return lay
    _patch(monkeypatch, "plan_layout", f)
    assert _fails(lambda: P.test_layout_pack_unpack_roundtrip(8, 2), lambda: P.test_layout_pack_unpack_roundtrip(64, 3))


@pytest.mark.parametrize("kind", ["grow_late", "no_reset_on_overflow", "no_floor", "t_counts_skips"])
def test_scaler_mistakes_are_caught(monkeypatch, kind):
    def f(s, overflow):
        s = Z.OracleScaler(**s.__dict__)
        if overflow:
            s.skipped_total += 1
            if kind != "no_reset_on_overflow":
                s.growth_tracker = 0
            if kind == "t_counts_skips":
                s.step_t += 1
            if s.dynamic:
                s.loss_scale = s.loss_scale / 2.0 if kind == "no_floor" else max(s.loss_scale / 2.0, s.scale_floor)
        else:
            s.step_t += 1
            if s.dynamic:
                s.growth_tracker += 1
                if s.growth_tracker == s.growth_interval + (1 if kind == "grow_late" else 0):
                    s.loss_scale *= 2.0
                    s.growth_tracker = 0
        return s
    _patch(monkeypatch, "scaler_update", f)
    assert _fails(P.test_scaler_tiny_config_sequence, P.test_scaler_growth_and_backoff_sequence,
                  P.test_scaler_floor_and_static, P.test_scaler_doubles_once_per_window), kind


@pytest.mark.parametrize("kind", ["strict_threshold", "forward_walk", "last_bucket_dropped"])
def test_bucket_plan_mistakes_are_caught(monkeypatch, kind):
    def wrong(numels, size):
        order = range(len(numels)) if kind == "forward_walk" else reversed(range(len(numels)))
        out, members = [], []
        for t in order:
            members.append(t)
            full = sum(numels[i] for i in members)
            closes = full > size if kind == "strict_threshold" else full >= size
            edge = (t == len(numels) - 1) if kind == "forward_walk" else (t == 0)
            if closes or (edge and kind != "last_bucket_dropped"):
                out.append((min(members), max(members) + 1))
                members = []
        return out
    _patch(monkeypatch, "plan_buckets", wrong)
    assert _fails(P.test_plan_buckets_hand_tables, *(lambda s=s: P.test_plan_buckets_against_suffix_sum_definition(s)
                                                    for s in range(6))), kind


@pytest.mark.parametrize("kind", ["end_at_last_element", "begin_after_gap"])
def test_bucket_range_mistakes_are_caught(monkeypatch, kind):
    def wrong(layout, a, b):
        if kind == "end_at_last_element":  # drops the gap behind the last tensor and the tail
            return layout.offsets[a], layout.offsets[b - 1] + layout.numels[b - 1]
        begin = layout.offsets[a] if a == 0 else layout.offsets[a - 1] + layout.numels[a - 1]
        end = layout.flat_numel if b == len(layout.numels) else layout.offsets[b - 1] + layout.numels[b - 1]
        return begin, end
    _patch(monkeypatch, "bucket_range", wrong)
    assert _fails(P.test_bucket_range_hand_table, lambda: P.test_bucket_ranges_tile_the_flat_buffer(64, 4),
                  lambda: P.test_buckets_in_any_order_rebuild_the_whole_pack(False)), kind


@pytest.mark.parametrize("kind", ["ignored", "inverted"])
def test_no_decay_mistakes_are_caught(monkeypatch, kind):
    real = Z.adamw_update

    def wrong(master, m, v, x, loss_scale, clip, t, hp, decay=None):
        if decay is not None:
            decay = None if kind == "ignored" else ~decay
        return real(master, m, v, x, loss_scale, clip, t, hp, decay)
    _patch(monkeypatch, "adamw_update", wrong)
    assert _fails(P.test_no_decay_tensors_closed_form, P.test_no_decay_group_matches_torch_param_groups), kind


ACCUMULATE_PINS = (P.test_accumulate_fp32_matches_exact_sums, P.test_accumulate_model_dtype_rounds_to_nearest_even,
                   P.test_accumulate_then_step_equals_step_on_summed_gradient)


@pytest.mark.parametrize("kind", ["overwrite", "subtract", "truncate", "sum_in_model_dtype_twice"])
def test_accumulate_mistakes_are_caught(monkeypatch, kind):
    real_pack = Z.pack

    def wrong(acc, tensors, layout):
        packed = real_pack(tensors, layout, acc.dtype)
        if kind == "overwrite":
            return packed
        if kind == "subtract":
            return (acc.double() - packed.double()).to(acc.dtype)
        s = acc.double() + packed.double()
        if kind == "truncate":  # round toward zero instead of to nearest even
            f = s.to(acc.dtype)
            over = (f.double().abs() > s.abs())
            step = torch.nextafter(f, torch.zeros_like(f))
            return torch.where(over, step, f)
        # the sum rounded to the model dtype first, then to the buffer's (two roundings)
        return s.to(torch.bfloat16).to(acc.dtype)
    _patch(monkeypatch, "accumulate", wrong)
    assert _fails(*ACCUMULATE_PINS), kind


@pytest.mark.parametrize("kind", ["shifted", "ignores_shard_begin", "truncating_cast"])
def test_unpack_mistakes_are_caught(monkeypatch, kind):
    real_cast = Z.cast_to

    def wrong(src, layout, tensors, whole_flat):
        lo = 0 if (whole_flat or kind == "ignores_shard_begin") else layout.shard_begin
        hi = lo + src.numel()
        out = []
        for t, off, n in zip(tensors, layout.offsets, layout.numels):
            t = t.clone()
            a, b = max(off, lo), min(off + n, hi)
            if kind == "shifted":
                a = min(a + 1, b)
            if a < b:
                x = src[a - lo:b - lo]
                t.view(-1)[a - off:b - off] = x.to(t.dtype) if kind != "truncating_cast" else \
                    (x.view(torch.int32) & ~0xFFFF).view(torch.float32).to(t.dtype) if x.dtype == torch.float32 \
                    else real_cast(x, t.dtype)
            out.append(t)
        return out
    _patch(monkeypatch, "unpack", wrong)
    pins = [lambda: P.test_layout_pack_unpack_roundtrip(1, 2), lambda: P.test_layout_pack_unpack_roundtrip(8, 3),
            P.test_dp_split_equals_single_rank_when_unclipped, P.test_unpack_rounds_each_shard_to_nearest_even]
    assert _fails(*pins), kind


@pytest.mark.parametrize("kind", ["off_by_one", "first_shard_always"])
def test_shard_mistakes_are_caught(monkeypatch, kind):
    def wrong(flat, layout):
        b = 0 if kind == "first_shard_always" else layout.shard_begin + (1 if layout.shard_begin else 0)
        out = flat[b:b + layout.shard_numel]
        if out.numel() < layout.shard_numel:
            out = torch.cat([out, torch.zeros(layout.shard_numel - out.numel(), dtype=flat.dtype)])
        return out
    _patch(monkeypatch, "shard_of", wrong)
    assert _fails(lambda: P.test_layout_pack_unpack_roundtrip(1, 2), P.test_dp_split_equals_single_rank_when_unclipped,
                  P.test_page_sharded_sgd_example_through_adamw_limit), kind


@pytest.mark.parametrize("kind", ["gaps_not_zeroed", "offset_off_by_one", "rounds_on_widening"])
def test_pack_mistakes_are_caught(monkeypatch, kind):
    def wrong(tensors, layout, dtype=None):
        if dtype is None:
            dtype = tensors[0].dtype
        flat = torch.full((layout.flat_numel,), 3.0, dtype=dtype) if kind == "gaps_not_zeroed" else \
            torch.zeros(layout.flat_numel, dtype=dtype)
        for t, off, n in zip(tensors, layout.offsets, layout.numels):
            if n:
                o = off + 1 if (kind == "offset_off_by_one" and off + n < layout.flat_numel) else off
                x = t.reshape(-1)
                if kind == "rounds_on_widening" and dtype == torch.float32:
                    x = x.to(torch.float16)  # a lossy detour for bf16 sources
                flat[o:o + n] = x.to(dtype)
        return flat
    _patch(monkeypatch, "pack", wrong)
    pins = [lambda: P.test_layout_pack_unpack_roundtrip(8, 2), lambda: P.test_layout_pack_unpack_roundtrip(1, 3),
            P.test_page_sharded_sgd_example_through_adamw_limit, P.test_pack_widening_to_fp32_is_exact]
    assert _fails(*pins), kind


@pytest.mark.parametrize("kind", ["whole_pack", "range_one_short"])
def test_pack_bucket_mistakes_are_caught(monkeypatch, kind):
    def wrong(flat, tensors, layout, tensor_begin, tensor_end, accumulate_into=False):
        begin, end = Z.bucket_range(layout, tensor_begin, tensor_end)
        if kind == "whole_pack":
            begin, end = 0, layout.flat_numel
        else:
            end = max(begin, end - 1)
        full = Z.accumulate(flat, tensors, layout) if accumulate_into else Z.pack(tensors, layout, flat.dtype)
        out = flat.clone()
        out[begin:end] = full[begin:end]
        return out
    _patch(monkeypatch, "pack_bucket", wrong)
    assert _fails(lambda: P.test_buckets_in_any_order_rebuild_the_whole_pack(False),
                  lambda: P.test_buckets_in_any_order_rebuild_the_whole_pack(True)), kind


def test_global_sum_dropping_a_rank_is_caught(monkeypatch):
    _patch(monkeypatch, "global_sumsq", lambda parts: sum(parts[1:]))
    assert _fails(P.test_sumsq_special_cases_and_invariants)


def _rank_step_variant(kind):
    """OracleRank.step with one wiring mistake: the norm from this rank's own partial only
    (local_norm), the norm of the still-scaled gradient (scaled_norm), the clip coefficient
    left out of the update (clip_dropped), the update fed the scaled gradient
    (update_not_unscaled), or the bias correction stuck at t = 1 (t_stuck_at_one)."""
    def step(self, shard_x, ext_overflow=False, other_sumsq=None):
        lay = self.layout
        overflow = Z.nonfinite_any(shard_x) or bool(ext_overflow)
        rec = dict(overflow=overflow, loss_scale=self.scaler.loss_scale, local_sumsq=None, sumsq=None, norm=None,
                   clip=None)
        if not overflow:
            scale = self.scaler.loss_scale
            local = Z.sumsq_unscaled(shard_x, 1.0 if kind == "scaled_norm" else scale)
            if kind == "local_norm" or lay.dp_world == 1:
                ss = local
            else:
                ss = Z.global_sumsq([local if q == lay.dp_rank else other_sumsq[q] for q in range(lay.dp_world)])
            norm, c = Z.clip_coefficient(ss, self.hp["max_norm"])
            t = 1 if kind == "t_stuck_at_one" else self.scaler.step_t + 1
            self.master, self.m, self.v = Z.adamw_update(
                self.master, self.m, self.v, shard_x, 1.0 if kind == "update_not_unscaled" else scale,
                1.0 if kind == "clip_dropped" else c, t, self.hp, self.decay)
            self.params = Z.unpack(self.master, lay, self.params, whole_flat=False)
            rec.update(local_sumsq=local, sumsq=ss, norm=norm, clip=c)
        self.scaler = Z.scaler_update(self.scaler, overflow)
        return rec
    return step


@pytest.mark.parametrize("kind", ["local_norm", "scaled_norm", "clip_dropped", "update_not_unscaled",
                                  "t_stuck_at_one"])
def test_rank_step_wiring_mistakes_are_caught(monkeypatch, kind):
    monkeypatch.setattr(Z.OracleRank, "step", _rank_step_variant(kind))
    assert _fails(lambda: P.test_rank_step_matches_torch_clip_and_adamw(0),
                  P.test_two_ranks_exchanging_partials_match_one_torch_run), kind


def test_rank_step_variant_without_mistake_passes(monkeypatch):
    # the mistake-free rewrite passes every pin, so each failure above is the planted mistake's
    monkeypatch.setattr(Z.OracleRank, "step", _rank_step_variant("none"))
    assert not _fails(lambda: P.test_rank_step_matches_torch_clip_and_adamw(0),
                      P.test_two_ranks_exchanging_partials_match_one_torch_run)
