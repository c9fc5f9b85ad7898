"""GPU parity of the offloaded step (optimizer state in host memory, update on the
host CPU, zs_offload_adamw_step) against the oracle, through the C ABI.

The device still packs, checks, takes the norm and updates the scaler; the host updates
master / m / v chunk by chunk while the gradient chunks come down and the new parameters
go up.  Same bar as the device path: bit-exact buffer, flags, skips, scale sequence and
scatter-back; master / m / v within the 1e-5 relative contract.
"""

import pytest
import torch

from workloads import WORKLOADS, gen

pytestmark = pytest.mark.gpu


def _z():
    import zero_sharded_mixed_buffer_amd as Z
    Z.lib()
    return Z


@pytest.mark.parametrize("name,chunk", [("tiny", 4099), ("llama_mini", 1 << 20), ("llama_mini", 65_537),
                                        ("ragged_mini", 100_003), ("moe_mini_dp4", 77_777),
                                        ("qwen_mini_dp2", 1 << 24)])
def test_offload_parity(name, chunk):
    from harness import run_parity
    _z()
    wl = WORKLOADS[name]
    steps = min(wl.steps, 6)
    print(f"[case] offload {name} chunk={chunk} steps={steps}", flush=True)
    rep = run_parity(wl, steps=steps, offload=True, offload_chunk=chunk)
    print(f"[offload] {name}: master_err={rep.master_err:.3e} m_err={rep.m_err:.3e} v_err={rep.v_err:.3e} "
          f"diff(master,m,v)=({rep.n_master_diff},{rep.n_m_diff},{rep.n_v_diff}) "
          f"skips={[s.overflow_gpu for s in rep.steps]}", flush=True)
    assert [s.step for s in rep.steps if s.overflow_gpu] == [k for k in sorted(wl.faults) if k <= steps]


@pytest.mark.parametrize("name,accum", [("ragged_mini", torch.float32), ("moe_mini_dp4", None)])
def test_offload_with_gradient_accumulation(name, accum):
    """Micro-steps accumulated on the device (fp32 or model-dtype buffer), then the offloaded
    update reading that buffer."""
    from harness import run_parity_accumulation
    _z()
    wl = WORKLOADS[name]
    acc_dt = accum if accum is not None else gen.TORCH_DTYPE[wl.dtype]
    print(f"[case] offload + accumulation {name} accum={acc_dt}", flush=True)
    flags = run_parity_accumulation(wl, 3, acc_dt, steps=min(wl.steps, 5), offload=True)
    assert flags == [int(k in wl.faults) for k in range(1, min(wl.steps, 5) + 1)]


def test_offload_and_device_steps_agree():
    """The same gradients through the device update and the offloaded update: the states
    and the parameters agree bit for bit (one arithmetic on both sides)."""
    Z = _z()
    wl = WORKLOADS["llama_mini"]
    dev = torch.device("cuda", 0)
    p0 = gen.make_params(wl, dev)
    kw = dict(lr=1e-3, weight_decay=0.01, max_norm=1.0)
    a = Z.ZeroShardedAdamW([p.clone() for p in p0], **kw)
    b = Z.ZeroShardedAdamW([p.clone() for p in p0], offload=True, offload_chunk=1 << 18, **kw)
    for step in range(1, 4):
        grads = gen.make_grads(wl, step, 1.0, dev, with_faults=False)
        a.step(grads)
        b.step(grads)
    torch.cuda.synchronize()
    bits = lambda x: x.view(torch.int32 if x.element_size() == 4 else torch.int16)
    nd = [int((bits(x.cpu()) != bits(y)).sum()) for x, y in ((a.master, b.master), (a.m, b.m), (a.v, b.v))]
    print(f"[offload] device vs host state bit differences (master, m, v): {nd}", flush=True)
    assert nd == [0, 0, 0]
    assert all(torch.equal(bits(x), bits(y)) for x, y in zip(a.params, b.params))
    a.close()
    b.close()


def test_offload_invalid_arguments():
    Z = _z()
    dev = torch.device("cuda", 0)
    lay = Z.zs_layout_create([1000], 1, 0)
    st = Z.zs_state_create(lay, Z.state_host(1.0, 1.0, False))
    shard = torch.zeros(1000, dtype=torch.bfloat16, device=dev)
    host = [torch.zeros(1000) for _ in range(3)]
    stage_g = torch.empty(2000, dtype=torch.bfloat16, pin_memory=True)
    stage_p = torch.empty(2000, dtype=torch.bfloat16, pin_memory=True)
    out = torch.empty(1000, dtype=torch.bfloat16, device=dev)
    hp = Z.hparams()
    for chunk, sh in ((0, shard), (1000, None)):
        with pytest.raises(Z.ZsError) as e:
            Z.zs_offload_adamw_step(lay, sh, torch.bfloat16, st, hp, *host, stage_g, stage_p, chunk, out,
                                    torch.bfloat16)
        assert e.value.status == -1
    Z.zs_state_destroy(st)
    Z.zs_layout_destroy(lay)


def test_every_variant_together():
    """fp16 with a dynamic scale, 4 ranks (this is rank 2), 3 accumulated micro-steps in an
    fp32 buffer packed bucket by bucket, no-decay 1-D tensors and the offloaded update, with
    injected overflows: against the oracle step by step."""
    import math

    import oracle as O
    from harness import REL_TOL, bits, oracle_scaler, rel_err
    Z = _z()
    wl = WORKLOADS["moe_mini_dp4"]
    dev = torch.device("cuda", 0)
    d, r = wl.dp_world, wl.dp_rank
    hp = wl.hparams
    flags = [len(shape) <= 1 for _, shape in wl.shapes]
    params = gen.make_params(wl, dev)
    opt = Z.ZeroShardedAdamW(params, lr=hp["lr"], betas=(hp["beta1"], hp["beta2"]), eps=hp["eps"],
                             weight_decay=hp["weight_decay"], max_norm=hp["max_norm"], dp_world=d, dp_rank=r,
                             dynamic_loss_scale=True, init_scale=wl.init_scale, accum_dtype=torch.float32,
                             offload=True, offload_chunk=50_000, offload_threads=3, no_decay=flags)
    ref = O.OracleRank(wl.numels, d, r, [p.cpu() for p in params], oracle_scaler(wl), hp, no_decay=flags)
    lay = ref.layout
    S = lay.shard_numel
    others = []
    for q in range(d):
        if q != r:
            lq = Z.zs_layout_create(wl.numels, d, q)
            others.append((q, lq, Z.zs_state_create(lq, Z.state_host(wl.init_scale, 1.0, True))))
    exch = torch.zeros(d, dtype=torch.float64, device=dev)
    buckets = opt.buckets(40_000)
    faults = {2: [(0, 5, float("inf"))], 5: [(3, 1, float("nan"))]}
    skipped = []
    try:
        for step in range(1, 7):
            scale = ref.scaler.loss_scale
            micro = [gen.make_grads(wl, step * 10 + k, scale, dev, with_faults=False) for k in range(3)]
            for t, kk, val in faults.get(step, []):
                micro[-1][t].view(-1)[kk] = val
            for k, g in enumerate(micro):
                for b in buckets[::-1] if k % 2 else buckets:
                    opt.pack_bucket(g, b, accumulate=k > 0)
            opt.check(local_sumsq_out=exch[r:r + 1])
            for q, lq, sq in others:
                Z.zs_unscale_check(lq, opt.flat[q * S:(q + 1) * S], torch.float32, sq, None, exch[q:q + 1])
            opt.norm(rank_sumsq=exch)
            for q, lq, sq in others:
                Z.zs_grad_norm(lq, None, torch.float32, sq, opt.hp, exch, None)
                Z.zs_scaler_update(sq)
            prev = [p.cpu() for p in params]
            opt.update()
            torch.cuda.synchronize()
            acc = O.pack([x.cpu() for x in micro[0]], lay, torch.float32)
            for g in micro[1:]:
                acc = O.accumulate(acc, [x.cpu() for x in g], lay)
            got = opt.flat.cpu()
            # bit-exact, NaN payloads aside (any NaN skips the step)
            differ = (bits(got) != bits(acc)) & ~(torch.isnan(got) & torch.isnan(acc))
            assert not bool(differ.any()), f"step {step}: accumulated buffer differs"
            other, ext = [], False
            for q in range(d):
                sq_ = acc[q * S:(q + 1) * S]
                bad = O.nonfinite_any(sq_)
                other.append(math.inf if bad else O.sumsq_unscaled(sq_, scale))
                ext = ext or (bad and q != r)
            rec = ref.step(O.shard_of(acc, lay), ext_overflow=ext, other_sumsq=other)
            st = opt.read_state()
            skipped.append(int(rec["overflow"]))
            assert st["loss_scale"] == ref.scaler.loss_scale and st["step_t"] == ref.scaler.step_t
            assert st["skipped_total"] == ref.scaler.skipped_total
            for a, b in ((opt.master, ref.master), (opt.m, ref.m), (opt.v, ref.v)):
                assert rel_err(a, b) <= REL_TOL
            want = prev if rec["overflow"] else O.unpack(opt.master, lay, prev, False)
            assert all(torch.equal(bits(a.cpu()), bits(b)) for a, b in zip(params, want))
        assert skipped == [0, 1, 0, 0, 1, 0]
    finally:
        for _, lq, sq in others:
            Z.zs_state_destroy(sq)
            Z.zs_layout_destroy(lq)
        opt.close()


@pytest.mark.parametrize("with_out", [False, True])
def test_offload_first_step_skipped_keeps_parameter_shard_valid(with_out):
    """Rank 1 of 2, fp16 at the initial scale 2^16, step 1 overflowing on the other rank.
    The flat parameter shard (the all-gather input) holds the rank's parameters from the
    start; the skip writes neither it nor a caller's flat_param_out; the applied step 2
    writes the cast of the new master into whichever of the two the update targets and
    scatters it, as the device update does."""
    import oracle as O
    from harness import bits
    Z = _z()
    wl = WORKLOADS["tiny"]
    dev = torch.device("cuda", 0)
    hp = wl.hparams
    params = gen.make_params(wl, dev)
    opt = Z.ZeroShardedAdamW(params, lr=hp["lr"], betas=(hp["beta1"], hp["beta2"]), eps=hp["eps"],
                             weight_decay=hp["weight_decay"], max_norm=hp["max_norm"], dp_world=2, dp_rank=1,
                             dynamic_loss_scale=True, init_scale=2.0 ** 16, offload=True, offload_chunk=10_000)
    lay = O.plan_layout(wl.numels, 2, 1)
    S = lay.shard_numel
    p0 = [p.cpu() for p in params]
    torch.cuda.synchronize()
    assert torch.equal(bits(opt.flat_param.cpu()), bits(O.shard_of(O.pack(p0, lay), lay)))
    out = torch.full((S,), 7.0, dtype=torch.float16, device=dev) if with_out else None
    ext = torch.ones(1, dtype=torch.int32, device=dev)
    exch = torch.zeros(2, dtype=torch.float64, device=dev)
    print(f"[case] offload first-step skip, dp 2 rank 1, flat_param_out={with_out}", flush=True)

    def step(k, scale):
        opt.pack(gen.make_grads(wl, k, scale, dev, with_faults=False))
        opt.check(ext_overflow=ext, local_sumsq_out=exch[1:2])
        opt.norm(rank_sumsq=exch)
        opt.update(flat_param_out=out)
        torch.cuda.synchronize()

    step(1, 2.0 ** 16)
    st = opt.read_state()
    assert st["skipped_total"] == 1 and st["step_t"] == 0 and st["loss_scale"] == 2.0 ** 15
    assert torch.equal(bits(opt.flat_param.cpu()), bits(O.shard_of(O.pack(p0, lay), lay)))
    if with_out:
        assert bool((out == 7.0).all())
    assert all(torch.equal(bits(a.cpu()), bits(b)) for a, b in zip(params, p0))
    ext.zero_()
    step(2, 2.0 ** 15)
    st = opt.read_state()
    assert st["skipped_total"] == 1 and st["step_t"] == 1
    dest = out if with_out else opt.flat_param
    assert torch.equal(bits(dest.cpu()), bits(O.cast_to(opt.master, torch.float16)))
    want = O.unpack(opt.master, lay, p0, False)
    assert all(torch.equal(bits(a.cpu()), bits(b)) for a, b in zip(params, want))
    opt.close()


def test_caller_tensors_are_checked_before_any_launch():
    """Tensors handed to check / norm / update that a kernel would misread (another dtype) or
    overrun (too few elements) are refused with nothing enqueued."""
    Z = _z()
    wl = WORKLOADS["qwen_mini_dp2"]
    dev = torch.device("cuda", 0)
    for offload in (False, True):
        opt = Z.ZeroShardedAdamW(gen.make_params(wl, dev), dp_world=2, dp_rank=1, offload=offload,
                                 offload_chunk=1 << 16)
        S = opt.shard_numel
        bad_calls = [
            lambda: opt.check(ext_overflow=torch.zeros(1, dtype=torch.bool, device=dev)),
            lambda: opt.check(ext_overflow=torch.zeros(1, dtype=torch.int32)),
            lambda: opt.check(local_sumsq_out=torch.zeros(1, dtype=torch.float32, device=dev)),
            lambda: opt.norm(rank_sumsq=torch.zeros(2, dtype=torch.float32, device=dev)),
            lambda: opt.norm(rank_sumsq=torch.zeros(1, dtype=torch.float64, device=dev)),
            lambda: opt.update(flat_param_out=torch.zeros(S - 1, dtype=torch.bfloat16, device=dev)),
            lambda: opt.update(flat_param_out=torch.zeros(S, dtype=torch.float32, device=dev)),
            lambda: opt.update(flat_param_out=torch.zeros(2 * S, dtype=torch.bfloat16, device=dev)[::2]),
        ]
        for i, call in enumerate(bad_calls):
            with pytest.raises(ValueError):
                call()
        torch.cuda.synchronize()
        st = opt.read_state()
        assert st["step_t"] == 0 and st["skipped_total"] == 0  # nothing was committed
        opt.close()
