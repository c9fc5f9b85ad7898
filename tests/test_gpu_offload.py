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
