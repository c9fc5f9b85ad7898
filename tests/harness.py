"""Parity harness: run the HIP path and the CPU oracle side by side on one workload.

Inputs (parameters, per-step gradients) are drawn once on the GPU from the seeded
workload generators and copied to the host for the oracle; no oracle input or
expected value comes from the HIP path.  For dp_world > 1 the other ranks are
virtual: every rank's shard is a slice of the same packed buffer (the stand-in for
the reduce-scatter output), the GPU exchanges the ranks' local sums of squares
through zs_unscale_check / zs_grad_norm, and the oracle takes the same partial
sums from its own arithmetic.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

import oracle as O
import zero_sharded_mixed_buffer_amd as Z
from workloads import gen

# Parity contract: master, m and v within a max relative error of 1e-5 after the run, the
# relative error of an element measured against max(|oracle value|, 1e-3 * RMS of the
# array) because an element that cancels to ~0 has no meaningful relative error.
REL_TOL = 1e-5
REL_FLOOR = 1e-3
NORM_RTOL = 1e-12


def rel_err(a: torch.Tensor, b: torch.Tensor) -> float:
    a = a.double()
    b = b.double()
    if b.numel() == 0:
        return 0.0
    rms = float(b.pow(2).mean().sqrt())
    den = torch.clamp(b.abs(), min=REL_FLOOR * rms) if rms > 0 else b.abs()
    d = (a - b).abs()
    ok = den > 0
    if not bool(ok.all()):
        if bool((d[~ok] != 0).any()):
            return math.inf
    return float((d[ok] / den[ok]).max()) if bool(ok.any()) else 0.0


def plain_rel_err(a, b) -> float:
    a = a.double()
    b = b.double()
    nz = b != 0
    if bool((a[~nz] != 0).any()):
        return math.inf
    return float(((a - b).abs()[nz] / b.abs()[nz]).max()) if bool(nz.any()) else 0.0


def bits(x: torch.Tensor) -> torch.Tensor:
    return x.contiguous().view(torch.int16) if x.element_size() == 2 else x.contiguous().view(torch.int32)


@dataclass
class StepReport:
    step: int
    overflow_gpu: int
    overflow_oracle: bool
    scale_gpu: float
    scale_oracle: float
    norm_gpu: float = float("nan")
    norm_oracle: float = float("nan")
    clip_gpu: float = float("nan")
    clip_oracle: float = float("nan")


@dataclass
class RunReport:
    steps: list = field(default_factory=list)
    master_err: float = 0.0
    m_err: float = 0.0
    v_err: float = 0.0
    master_plain: float = 0.0
    n_master_diff: int = 0
    n_m_diff: int = 0
    n_v_diff: int = 0
    n_param_diff: int = 0


def oracle_scaler(wl):
    return O.OracleScaler(wl.init_scale, 1.0, wl.dynamic, wl.growth_interval)


def sample_windows(lay, width=1 << 16, n_random=24, seed=0, centres=()):
    """Deterministic shard windows [a, b) (shard-relative): the first and last `width`
    elements, windows across the first and last four tensor boundaries inside the shard,
    windows centred on the given shard-relative positions, and n_random seeded ones."""
    import random
    S = lay.shard_numel
    lo, hi = lay.shard_begin, lay.shard_begin + S
    w = min(width, S)
    starts = {0, S - w}
    for c in centres:
        starts.add(min(max(c - w // 2, 0), S - w))
    inside = [off for off in lay.offsets if lo < off < hi]
    for off in inside[:4] + inside[-4:]:
        starts.add(min(max(off - lo - w // 2, 0), S - w))
    rng = random.Random(seed)
    for _ in range(n_random):
        starts.add(rng.randrange(0, S - w + 1))
    return sorted((a, a + w) for a in starts)


def _window_values(tensors_cpu, lay, a, b, dtype):
    """Oracle pack of shard window [a, b): the flat values there, zeros in padding."""
    out = torch.zeros(b - a, dtype=dtype)
    lo = lay.shard_begin + a
    hi = lay.shard_begin + b
    for t, off, n in zip(tensors_cpu, lay.offsets, lay.numels):
        x, y = max(off, lo), min(off + n, hi)
        if x < y:
            out[x - lo:y - lo] = t.view(-1)[x - off:y - off]
    return out


def run_parity_sampled(wl, steps=None, log=print, centres=(), n_random=48, views=False):
    """Full-size parity on sampled outputs.  The GPU runs the whole step at the workload's
    real size in the same launch configuration as bench.py; the oracle computes every
    step's flag, scaler and global norm from all gradients (streamed to the host one
    tensor at a time) and the AdamW state only on sampled shard windows, which are
    compared element by element (master, m, v, params, packed buffer).  views=True (one
    rank): the parameters and gradients are views of two flat buffers, the gradients are
    written through the .grad views as backward would, and each step is the single
    zs_step_flat call."""
    steps = wl.steps if steps is None else steps
    d, rank, align = wl.dp_world, wl.dp_rank, wl.align
    dev = torch.device("cuda", 0)
    dt = gen.TORCH_DTYPE[wl.dtype]
    hp = wl.hparams
    lay = O.plan_layout(wl.numels, d, rank, align)
    S = lay.shard_numel
    wins = sample_windows(lay, width=1 << 20, n_random=n_random, seed=wl.seed, centres=centres)
    params = gen.make_params(wl, dev)
    params_cpu0 = [p.cpu() for p in params]
    opt = Z.ZeroShardedAdamW(params, lr=hp["lr"], betas=(hp["beta1"], hp["beta2"]), eps=hp["eps"],
                             weight_decay=hp["weight_decay"], max_norm=hp["max_norm"], dp_world=d, dp_rank=rank,
                             align=align, dynamic_loss_scale=wl.dynamic, init_scale=wl.init_scale,
                             growth_interval=wl.growth_interval, flat_views=views)
    assert not views or d == 1
    scaler = oracle_scaler(wl)
    # Oracle state on the windows only.
    ref = {}
    for a, b in wins:
        p = _window_values(params_cpu0, lay, a, b, torch.float32)
        ref[(a, b)] = [p, torch.zeros_like(p), torch.zeros_like(p)]
    del params_cpu0
    others = {}
    for q in range(d):
        if q != rank:
            lq = Z.zs_layout_create(wl.numels, d, q, align)
            others[q] = (lq, Z.zs_state_create(lq, Z.state_host(wl.init_scale, 1.0, wl.dynamic, wl.growth_interval)))
    exchange = torch.zeros(d, dtype=torch.float64, device=dev)
    # Tensor pieces overlapping each window, found once: tensor index -> [(window, x, y)].
    import bisect
    overlaps = {}
    for (a, b) in wins:
        lo, hi = lay.shard_begin + a, lay.shard_begin + b
        i = max(bisect.bisect_right(lay.offsets, lo) - 1, 0)
        while i < len(lay.offsets) and lay.offsets[i] < hi:
            x, y = max(lay.offsets[i], lo), min(lay.offsets[i] + lay.numels[i], hi)
            if x < y:
                overlaps.setdefault(i, []).append(((a, b), x, y))
            i += 1
    worst = dict(master=0.0, m=0.0, v=0.0)
    ndiff = dict(master=0, m=0, v=0, params=0)
    try:
        for step in range(1, steps + 1):
            scale = scaler.loss_scale
            grads = gen.make_grads(wl, step, scale, dev)
            if views:
                with torch.no_grad():
                    for p, g in zip(params, grads):
                        p.grad.copy_(g)
                opt.step()
                st_before = st = opt.read_state()
            else:
                opt.pack(grads)
            if views:
                pass
            elif d == 1:
                opt.norm()
            else:
                for q in range(d):
                    if q == rank:
                        opt.check(local_sumsq_out=exchange[q:q + 1])
                    else:
                        Z.zs_unscale_check(others[q][0], opt.flat[q * S:(q + 1) * S], dt, others[q][1], None,
                                           exchange[q:q + 1])
                opt.norm(rank_sumsq=exchange)
                for lq, sq in others.values():
                    Z.zs_grad_norm(lq, None, dt, sq, opt.hp, exchange, None)
                    Z.zs_scaler_update(sq)
            if not views:
                st_before = opt.read_state()
                opt.update()
                st = opt.read_state()

            # Oracle: flag and global norm over every gradient element, one tensor at a time.
            overflow = False
            parts = []
            win_x = {w: torch.zeros(w[1] - w[0], dtype=dt) for w in wins}
            for i, (g, off, n) in enumerate(zip(grads, lay.offsets, lay.numels)):
                gc = g.cpu()
                if O.nonfinite_any(gc):
                    overflow = True
                else:
                    parts.append(O.sumsq_unscaled(gc, scale))
                for (a, b), x, y in overlaps.get(i, ()):
                    lo = lay.shard_begin + a
                    win_x[(a, b)][x - lo:y - lo] = gc.view(-1)[x - off:y - off]
                del gc
            assert st_before["overflow"] == int(overflow), f"step {step}: overflow flag differs"
            if not overflow:
                ss = O.global_sumsq(parts)
                norm, c = O.clip_coefficient(ss, hp["max_norm"])
                assert abs(st_before["grad_norm"] - norm) <= NORM_RTOL * norm, \
                    f"step {step}: norm {st_before['grad_norm']!r} vs {norm!r}"
                assert abs(st_before["clip_coef"] - c) <= NORM_RTOL * c
                t = scaler.step_t + 1
            scaler = O.scaler_update(scaler, overflow)
            assert st["loss_scale"] == scaler.loss_scale and st["step_t"] == scaler.step_t
            assert st["growth_tracker"] == scaler.growth_tracker and st["skipped_total"] == scaler.skipped_total
            flat_gpu = opt.flat
            master_gpu, m_gpu, v_gpu = opt.master, opt.m, opt.v
            for (a, b) in wins:
                xw = win_x[(a, b)]
                assert torch.equal(bits(flat_gpu[lay.shard_begin + a:lay.shard_begin + b].cpu()), bits(xw)), \
                    f"step {step}: packed window {a} differs"
                st_ref = ref[(a, b)]
                if not overflow:
                    ref[(a, b)] = list(O.adamw_update(st_ref[0], st_ref[1], st_ref[2], xw, scale, c, t, hp))
                pm = master_gpu[a:b].cpu()
                for name, got, want in (("master", pm, ref[(a, b)][0]), ("m", m_gpu[a:b].cpu(), ref[(a, b)][1]),
                                        ("v", v_gpu[a:b].cpu(), ref[(a, b)][2])):
                    ndiff[name] += int((bits(got) != bits(want)).sum())
                    worst[name] = max(worst[name], rel_err(got, want) if want.abs().max() > 0 else 0.0)
            log(f"[fullsize] {wl.name} step {step}: overflow={int(overflow)} scale={st['loss_scale']} "
                f"norm={st_before['grad_norm']:.9g} worst={worst} ndiff={ndiff}")
        # Parameters at the windows: the cast of the GPU master, bit-exact (unpack as a function).
        for i, pieces in overlaps.items():
            p, off = params[i], lay.offsets[i]
            for (a, b), x, y in pieces:
                lo = lay.shard_begin + a
                pm = opt.master[x - lay.shard_begin:y - lay.shard_begin].cpu()
                got = p.view(-1)[x - off:y - off].cpu()
                want = O.cast_to(pm, p.dtype)
                assert torch.equal(bits(got), bits(want)), f"params of window {a} differ"
                ndiff["params"] += int((bits(got) != bits(O.cast_to(ref[(a, b)][0][x - lo:y - lo], p.dtype))).sum())
        for k in ("master", "m", "v"):
            assert worst[k] <= REL_TOL, f"{k} relative error {worst[k]}"
        return worst, ndiff, wins
    finally:
        for lq, sq in others.values():
            Z.zs_state_destroy(sq)
            Z.zs_layout_destroy(lq)
        opt.close()


def run_parity(wl, steps=None, align=None, dp_rank=None, check_every_step=True, offload=False,
               offload_chunk=1 << 24, no_decay=None, use_step=False):
    """Run `steps` optimizer steps of workload `wl` on cuda:0 and in the oracle, checking
    every stage each step.  offload=True keeps master / m / v in host memory and runs the
    update on the host (zs_offload_adamw_step, in chunks of offload_chunk elements).
    no_decay: per-tensor flags of tensors that take no weight decay (or None).
    use_step=True (one rank): each step is the single zs_step call (ZeroShardedAdamW.step).
    Returns a RunReport; raises AssertionError on a mismatch of the bit-exact quantities."""
    steps = wl.steps if steps is None else steps
    align = wl.align if align is None else align
    rank = wl.dp_rank if dp_rank is None else dp_rank
    d = wl.dp_world
    dev = torch.device("cuda", 0)
    dt = gen.TORCH_DTYPE[wl.dtype]
    hp = wl.hparams

    params_gpu = gen.make_params(wl, dev)
    params_cpu = [p.cpu() for p in params_gpu]
    opt = Z.ZeroShardedAdamW(params_gpu, lr=hp["lr"], betas=(hp["beta1"], hp["beta2"]), eps=hp["eps"],
                             weight_decay=hp["weight_decay"], max_norm=hp["max_norm"], dp_world=d, dp_rank=rank,
                             align=align, dynamic_loss_scale=wl.dynamic, init_scale=wl.init_scale,
                             growth_interval=wl.growth_interval, offload=offload, offload_chunk=offload_chunk,
                             offload_threads=4 if offload else 0, no_decay=no_decay)
    ref = O.OracleRank(wl.numels, d, rank, params_cpu, oracle_scaler(wl), hp, align, no_decay=no_decay)
    lay = ref.layout
    assert (opt.flat_numel, opt.shard_begin, opt.shard_numel) == (lay.flat_numel, lay.shard_begin, lay.shard_numel)
    # Master seeding (pack with widening) is exact.
    assert torch.equal(opt.master.cpu(), ref.master)

    # Virtual ranks: layout + state of every other rank, sharing the packed buffer.
    others = {}
    for q in range(d):
        if q == rank:
            continue
        lq = Z.zs_layout_create(wl.numels, d, q, align)
        sq = Z.zs_state_create(lq, Z.state_host(wl.init_scale, 1.0, wl.dynamic, wl.growth_interval))
        others[q] = (lq, sq)
    exchange = torch.zeros(d, dtype=torch.float64, device=dev)
    S = lay.shard_numel
    report = RunReport()
    try:
        for step in range(1, steps + 1):
            scale = ref.scaler.loss_scale
            grads = gen.make_grads(wl, step, scale, dev)
            grads_cpu = [g.cpu() for g in grads]
            prev_params = [p.cpu() for p in params_gpu]

            # ---- GPU path
            if use_step:
                # the single call: the flag, norm and clip it leaves in the state are the
                # ones the update used (the scaler commit changes only the scale and counts)
                opt.step(grads)
                st_before = st = opt.read_state()
            else:
                opt.pack(grads)
            if use_step:
                pass
            elif d == 1:
                opt.norm()
            else:
                for q in range(d):
                    shard_q = opt.flat[q * S:(q + 1) * S]
                    if q == rank:
                        opt.check(local_sumsq_out=exchange[q:q + 1])
                    else:
                        Z.zs_unscale_check(others[q][0], shard_q, dt, others[q][1], None, exchange[q:q + 1])
                opt.norm(rank_sumsq=exchange)
                # The virtual ranks run the same protocol, so their scalers stay in step.
                for lq, sq in others.values():
                    Z.zs_grad_norm(lq, None, dt, sq, opt.hp, exchange, None)
                    Z.zs_scaler_update(sq)
            if not use_step:
                st_before = opt.read_state()
                opt.update()
                st = opt.read_state()
            for lq, sq in others.values():
                assert Z.zs_state_read(sq).loss_scale == st["loss_scale"]

            # ---- oracle
            flat_ref = O.pack(grads_cpu, lay)
            shard_ref = O.shard_of(flat_ref, lay)
            other = None
            ext = False
            if d > 1:
                other = []
                for q in range(d):
                    sq = flat_ref[q * S:(q + 1) * S]
                    other.append(O.sumsq_unscaled(sq, scale) if not O.nonfinite_any(sq) else math.inf)
                    if q != rank:
                        ext = ext or O.nonfinite_any(sq)
            rec = ref.step(shard_ref, ext_overflow=ext, other_sumsq=other)

            # ---- bit-exact stages: pack, flag, skip, scaler
            assert torch.equal(bits(opt.flat.cpu()), bits(flat_ref)), f"step {step}: packed buffer differs"
            assert st_before["overflow"] == int(rec["overflow"]), f"step {step}: overflow flag differs"
            assert st["loss_scale"] == ref.scaler.loss_scale, f"step {step}: loss scale differs"
            assert st["step_t"] == ref.scaler.step_t and st["growth_tracker"] == ref.scaler.growth_tracker
            assert st["skipped_total"] == ref.scaler.skipped_total
            r = StepReport(step, st_before["overflow"], rec["overflow"], st["loss_scale"], ref.scaler.loss_scale)
            if not rec["overflow"]:
                r.norm_gpu, r.norm_oracle = st_before["grad_norm"], rec["norm"]
                r.clip_gpu, r.clip_oracle = st_before["clip_coef"], rec["clip"]
                assert abs(r.norm_gpu - r.norm_oracle) <= NORM_RTOL * r.norm_oracle + 1e-300, \
                    f"step {step}: norm {r.norm_gpu!r} vs {r.norm_oracle!r}"
                assert abs(r.clip_gpu - r.clip_oracle) <= NORM_RTOL * r.clip_oracle
            report.steps.append(r)

            if check_every_step or step == steps:
                master_gpu = opt.master.cpu()
                params_now = [p.cpu() for p in params_gpu]
                # Cast + scatter-back as a function of the GPU's own master: bit-exact.
                want = prev_params if rec["overflow"] else O.unpack(master_gpu, lay, prev_params, False)
                for i, (a, b) in enumerate(zip(params_now, want)):
                    assert torch.equal(bits(a), bits(b)), f"step {step}: scattered params of tensor {i} differ"
                report.master_err = rel_err(master_gpu, ref.master)
                report.m_err = rel_err(opt.m.cpu(), ref.m)
                report.v_err = rel_err(opt.v.cpu(), ref.v)
                report.master_plain = plain_rel_err(master_gpu, ref.master)
                report.n_master_diff = int((bits(master_gpu) != bits(ref.master)).sum())
                report.n_m_diff = int((bits(opt.m.cpu()) != bits(ref.m)).sum())
                report.n_v_diff = int((bits(opt.v.cpu()) != bits(ref.v)).sum())
                report.n_param_diff = sum(int((bits(a) != bits(b)).sum()) for a, b in zip(params_now, ref.params))
                assert report.master_err <= REL_TOL, f"step {step}: master rel err {report.master_err}"
                assert report.m_err <= REL_TOL, f"step {step}: m rel err {report.m_err}"
                assert report.v_err <= REL_TOL, f"step {step}: v rel err {report.v_err}"
                assert report.n_param_diff <= report.n_master_diff
    finally:
        for lq, sq in others.values():
            Z.zs_state_destroy(sq)
            Z.zs_layout_destroy(lq)
        opt.close()
    return report


def run_parity_accumulation(wl, micro_steps, accum_dtype, steps=None, dp_rank=None, offload=False):
    """Gradient accumulation: `micro_steps` gradient lists per step are packed into the flat
    buffer (first) and added to it (the rest, the last one fused with the check at dp 1),
    in accum_dtype (fp32 or the model dtype); then the step.  Checks the accumulated buffer
    bit-exactly against the oracle's accumulate() and the state against the 1e-5 contract."""
    steps = wl.steps if steps is None else steps
    rank = wl.dp_rank if dp_rank is None else dp_rank
    d, align = wl.dp_world, wl.align
    dev = torch.device("cuda", 0)
    dt = gen.TORCH_DTYPE[wl.dtype]
    hp = wl.hparams
    params = gen.make_params(wl, dev)
    opt = Z.ZeroShardedAdamW(params, lr=hp["lr"], betas=(hp["beta1"], hp["beta2"]), eps=hp["eps"],
                             weight_decay=hp["weight_decay"], max_norm=hp["max_norm"], dp_world=d, dp_rank=rank,
                             align=align, dynamic_loss_scale=wl.dynamic, init_scale=wl.init_scale,
                             growth_interval=wl.growth_interval, accum_dtype=accum_dtype, offload=offload,
                             offload_chunk=50_001, offload_threads=3 if offload else 0)
    ref = O.OracleRank(wl.numels, d, rank, [p.cpu() for p in params], oracle_scaler(wl), hp, align)
    lay = ref.layout
    S = lay.shard_numel
    others = {}
    for q in range(d):
        if q != rank:
            lq = Z.zs_layout_create(wl.numels, d, q, align)
            others[q] = (lq, Z.zs_state_create(lq, Z.state_host(wl.init_scale, 1.0, wl.dynamic, wl.growth_interval)))
    exchange = torch.zeros(d, dtype=torch.float64, device=dev)
    flags = []
    try:
        for step in range(1, steps + 1):
            scale = ref.scaler.loss_scale
            micro = [gen.make_grads(wl, step * 100 + k, scale, dev, with_faults=False) for k in range(micro_steps)]
            for t, kk, val in wl.faults.get(step, []):   # the step's faults land on its last micro-step
                micro[-1][t].view(-1)[kk] = val
            for k, g in enumerate(micro):
                opt.pack(g, accumulate=k > 0, last=k == micro_steps - 1)
            if d == 1:
                opt.norm()
            else:
                for q in range(d):
                    if q == rank:
                        opt.check(local_sumsq_out=exchange[q:q + 1])
                    else:
                        Z.zs_unscale_check(others[q][0], opt.flat[q * S:(q + 1) * S], opt.grad_dtype, others[q][1],
                                           None, exchange[q:q + 1])
                opt.norm(rank_sumsq=exchange)
                for lq, sq in others.values():
                    Z.zs_grad_norm(lq, None, opt.grad_dtype, sq, opt.hp, exchange, None)
                    Z.zs_scaler_update(sq)
            st_before = opt.read_state()
            opt.update()
            st = opt.read_state()
            acc = O.pack([g.cpu() for g in micro[0]], lay, accum_dtype)
            for g in micro[1:]:
                acc = O.accumulate(acc, [x.cpu() for x in g], lay)
            got_acc = opt.flat.cpu()
            # Bit-exact, except that NaN payloads and signs are not part of the contract: any
            # NaN in the buffer skips the step, and the oracle's own casts (torch's CPU
            # kernels) do not fix one NaN encoding.
            differ = (bits(got_acc) != bits(acc)) & ~(torch.isnan(got_acc.float()) & torch.isnan(acc.float()))
            if bool(differ.any()):
                bad = differ.nonzero().flatten()[:8].tolist()
                raise AssertionError(f"step {step}: accumulated buffer differs at {len(bad)}+ positions, e.g. "
                                     f"{[(i, hex(int(bits(got_acc)[i]) & 0xFFFFFFFF), hex(int(bits(acc)[i]) & 0xFFFFFFFF)) for i in bad]}")
            other, ext = None, False
            if d > 1:
                other = []
                for q in range(d):
                    sq_ = acc[q * S:(q + 1) * S]
                    bad = O.nonfinite_any(sq_)
                    other.append(math.inf if bad else O.sumsq_unscaled(sq_, scale))
                    ext = ext or (bad and q != rank)
            rec = ref.step(O.shard_of(acc, lay), ext_overflow=ext, other_sumsq=other)
            assert st_before["overflow"] == int(rec["overflow"]), f"step {step}: overflow differs"
            assert st["loss_scale"] == ref.scaler.loss_scale and st["step_t"] == ref.scaler.step_t
            if not rec["overflow"]:
                assert abs(st_before["grad_norm"] - rec["norm"]) <= NORM_RTOL * rec["norm"]
            assert rel_err(opt.master.cpu(), ref.master) <= REL_TOL
            assert rel_err(opt.m.cpu(), ref.m) <= REL_TOL
            assert rel_err(opt.v.cpu(), ref.v) <= REL_TOL
            want = ref.params
            ndiff = sum(int((bits(a.cpu()) != bits(b)).sum()) for a, b in zip(params, want))
            assert ndiff <= int((bits(opt.master.cpu()) != bits(ref.master)).sum())
            flags.append(int(rec["overflow"]))
        return flags
    finally:
        for lq, sq in others.values():
            Z.zs_state_destroy(sq)
            Z.zs_layout_destroy(lq)
        opt.close()
