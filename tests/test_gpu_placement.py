"""The measured placement of the optimizer's buffers (ZeroShardedAdamW(placement="tune")):
choosing it changes nothing the caller can see, and the candidate allocations it times are
released.  The parameters are bit-identical after
construction, and the tuned optimizer's steps equal those of one with four separate
allocations bit for bit (the kernels are the same; only where the buffers sit differs)."""

import pytest
import torch

from workloads import WORKLOADS, gen

pytestmark = pytest.mark.gpu


def _z():
    import zero_sharded_mixed_buffer_amd as Z
    Z.lib()
    return Z


def _bits(x):
    return x.view(torch.int32 if x.element_size() == 4 else torch.int16)


@pytest.mark.parametrize("name,views", [("llama_mini", False), ("moe_mini_dp4", False), ("ragged_mini", True)])
def test_tuned_placement_is_invisible(monkeypatch, name, views):
    import zero_sharded_mixed_buffer_amd.optimizer as OPT
    Z = _z()
    monkeypatch.setattr(OPT, "TUNE_MIN_ELEMENTS", 0)  # tune even these small shards
    wl = WORKLOADS[name]
    dev = torch.device("cuda", 0)
    hp = wl.hparams
    p0 = gen.make_params(wl, dev)
    kw = dict(lr=hp["lr"], betas=(hp["beta1"], hp["beta2"]), eps=hp["eps"], weight_decay=hp["weight_decay"],
              max_norm=hp["max_norm"], dp_world=wl.dp_world, dp_rank=wl.dp_rank, align=wl.align,
              dynamic_loss_scale=wl.dynamic, init_scale=wl.init_scale, flat_views=views)
    pa = [p.clone() for p in p0]
    pb = [p.clone() for p in p0]
    a = Z.ZeroShardedAdamW(pa, placement="tune", **kw)
    b = Z.ZeroShardedAdamW(pb, placement="separate", **kw)
    torch.cuda.synchronize()
    print(f"[case] placement {name} views={views}: {a.placement}", flush=True)
    assert a.placement["mode"] == "tuned" and a.placement["candidates"] == 24
    assert a.placement["arenas"] == len(a.placement["arena_ms"]) == OPT.TUNE_MAX_ARENAS
    assert b.placement["mode"] == "separate"
    assert all(torch.equal(_bits(x), _bits(y)) for x, y in zip(pa, p0)), "tuning changed the parameters"
    for opt in (a, b):
        assert torch.equal(_bits(opt.master.cpu()), _bits(b.master.cpu()))
        assert int(torch.count_nonzero(opt.m)) == 0 and int(torch.count_nonzero(opt.v)) == 0
    d, r = wl.dp_world, wl.dp_rank
    S = a.shard_numel
    exch = [torch.zeros(d, dtype=torch.float64, device=dev) for _ in range(2)]
    for step in range(1, 4):
        grads = gen.make_grads(wl, step, wl.init_scale, dev, with_faults=False)
        for opt, params, ex in ((a, pa, exch[0]), (b, pb, exch[1])):
            if views:
                with torch.no_grad():
                    for p, g in zip(params, grads):
                        p.grad.copy_(g)
                opt.step()
            elif d == 1:
                opt.step(grads)
            else:  # this rank's step; the other ranks' partial sums from their shards of the same buffer
                opt.pack(grads)
                opt.check(local_sumsq_out=ex[r:r + 1])
                for q in range(d):
                    if q != r:
                        lq = Z.zs_layout_create(wl.numels, d, q, wl.align)
                        sq = Z.zs_state_create(lq, Z.state_host(wl.init_scale, 1.0, wl.dynamic, wl.growth_interval))
                        Z.zs_unscale_check(lq, opt.flat[q * S:(q + 1) * S], opt.grad_dtype, sq, None, ex[q:q + 1])
                        torch.cuda.synchronize()
                        Z.zs_state_destroy(sq)
                        Z.zs_layout_destroy(lq)
                opt.norm(rank_sumsq=ex)
                opt.update()
        torch.cuda.synchronize()
        for k in ("master", "m", "v"):
            assert torch.equal(_bits(getattr(a, k).cpu()), _bits(getattr(b, k).cpu())), (step, k)
        assert all(torch.equal(_bits(x), _bits(y)) for x, y in zip(pa, pb)), step
        assert a.read_state() == b.read_state()
    a.close()
    b.close()


def test_candidate_allocations_are_released(monkeypatch):
    """The tuning holds several candidate allocations while it times them and keeps one: after
    construction the optimizer holds exactly what it holds when it times a single candidate."""
    import zero_sharded_mixed_buffer_amd.optimizer as OPT
    Z = _z()
    monkeypatch.setattr(OPT, "TUNE_MIN_ELEMENTS", 0)
    wl = WORKLOADS["llama_mini"]
    dev = torch.device("cuda", 0)
    p0 = gen.make_params(wl, dev)
    held = {}
    for k in (1, 5):
        monkeypatch.setattr(OPT, "TUNE_MAX_ARENAS", k)
        params = [p.clone() for p in p0]
        torch.cuda.synchronize()
        before = torch.cuda.memory_allocated(dev)
        opt = Z.ZeroShardedAdamW(params, placement="tune")
        torch.cuda.synchronize()
        held[k] = torch.cuda.memory_allocated(dev) - before
        print(f"[case] candidates {k}: {opt.placement}, holds {held[k]} bytes", flush=True)
        assert opt.placement["mode"] == "tuned"
        if k == 1:
            assert opt.placement["arenas"] == 1 and opt.placement["arena_ms"] == []
        else:
            assert opt.placement["arenas"] == k and len(opt.placement["arena_ms"]) == k
            assert opt.placement["arena_ms"][opt.placement["arena_pick"]] == min(opt.placement["arena_ms"])
        opt.close()
        del opt, params
    assert held[5] == held[1]



@pytest.mark.parametrize("placement", ["tune", "separate"])
def test_owned_allgather_input_matches_flat_param_out(monkeypatch, placement):
    """allgather_input=True: the optimizer's own all-gather input (carved from the tuned
    arena, or allocated apart) starts as the shard's parameters, and update(scatter=False)
    writes it with exactly what update(flat_param_out=...) writes into a caller's buffer,
    step after step."""
    import zero_sharded_mixed_buffer_amd.optimizer as OPT
    Z = _z()
    monkeypatch.setattr(OPT, "TUNE_MIN_ELEMENTS", 0)
    wl = WORKLOADS["moe_mini_dp4"]
    dev = torch.device("cuda", 0)
    hp = wl.hparams
    p0 = gen.make_params(wl, dev)
    kw = dict(lr=hp["lr"], betas=(hp["beta1"], hp["beta2"]), eps=hp["eps"], weight_decay=hp["weight_decay"],
              max_norm=hp["max_norm"], dp_world=wl.dp_world, dp_rank=wl.dp_rank, align=wl.align,
              dynamic_loss_scale=wl.dynamic, init_scale=wl.init_scale)
    a = Z.ZeroShardedAdamW([p.clone() for p in p0], placement=placement, allgather_input=True, **kw)
    b = Z.ZeroShardedAdamW([p.clone() for p in p0], placement="separate", **kw)
    assert b.flat_param is None
    assert a.placement["mode"] == ("tuned" if placement == "tune" else "separate")
    if placement == "tune":
        lo, hi = a._arena.data_ptr(), a._arena.data_ptr() + a._arena.numel()
        assert lo <= a.flat_param.data_ptr() and a.flat_param.data_ptr() + 2 * a.shard_numel <= hi
    offsets = Z.zs_plan(wl.numels, wl.dp_world, wl.dp_rank, wl.align)[0]
    whole = torch.zeros(a.flat_numel, dtype=p0[0].dtype, device=dev)
    for p, off in zip(p0, offsets):
        whole[off:off + p.numel()] = p.reshape(-1)
    torch.cuda.synchronize()
    assert torch.equal(_bits(a.flat_param), _bits(whole[a.shard_begin:a.shard_begin + a.shard_numel]))
    out_b = torch.full((b.shard_numel,), -1.0, dtype=b.param_dtype, device=dev)
    r = wl.dp_rank
    exch = torch.zeros(wl.dp_world, dtype=torch.float64, device=dev)
    for step in range(1, 4):
        grads = gen.make_grads(wl, step, wl.init_scale, dev, with_faults=False)
        for opt in (a, b):  # the other ranks' partial sums stay zero: the same for both
            opt.pack(grads)
            opt.check(local_sumsq_out=exch[r:r + 1])
        a.norm(rank_sumsq=exch)
        b.norm(rank_sumsq=exch)
        a.update(scatter=False)
        b.update(scatter=False, flat_param_out=out_b)
        torch.cuda.synchronize()
        assert torch.equal(_bits(a.flat_param), _bits(out_b)), step
        for k in ("master", "m", "v"):
            assert torch.equal(_bits(getattr(a, k)), _bits(getattr(b, k))), (step, k)
    a.close()
    b.close()


def test_allgather_input_follows_restored_parameters():
    """load_state_dict refills the owned all-gather input from the parameters the model
    restored first, so that a rank resumed at a skipped step hands out its real parameters."""
    Z = _z()
    wl = WORKLOADS["moe_mini_dp4"]
    dev = torch.device("cuda", 0)
    p0 = gen.make_params(wl, dev)
    params = [p.clone() for p in p0]
    kw = dict(dp_world=wl.dp_world, dp_rank=wl.dp_rank, align=wl.align, dynamic_loss_scale=wl.dynamic,
              init_scale=wl.init_scale, allgather_input=True)
    opt = Z.ZeroShardedAdamW(params, **kw)
    sd = opt.state_dict()
    exch = torch.zeros(wl.dp_world, dtype=torch.float64, device=dev)
    grads = gen.make_grads(wl, 1, wl.init_scale, dev, with_faults=False)
    opt.pack(grads)
    opt.check(local_sumsq_out=exch[wl.dp_rank:wl.dp_rank + 1])
    opt.norm(rank_sumsq=exch)
    opt.update(scatter=False)  # the all-gather input now holds the stepped shard
    torch.cuda.synchronize()
    offsets = Z.zs_plan(wl.numels, wl.dp_world, wl.dp_rank, wl.align)[0]
    whole = torch.zeros(opt.flat_numel, dtype=p0[0].dtype, device=dev)
    for p, off in zip(p0, offsets):
        whole[off:off + p.numel()] = p.reshape(-1)
    want = whole[opt.shard_begin:opt.shard_begin + opt.shard_numel]
    assert not torch.equal(_bits(opt.flat_param), _bits(want))
    with torch.no_grad():  # the model restores its parameters, then the optimizer its state
        for p, q in zip(params, p0):
            p.copy_(q)
    opt.load_state_dict(sd)
    assert torch.equal(_bits(opt.flat_param), _bits(want))
    opt.close()


def test_allgather_input_needs_several_ranks_without_views():
    Z = _z()
    wl = WORKLOADS["llama_mini"]
    dev = torch.device("cuda", 0)
    params = gen.make_params(wl, dev)
    with pytest.raises(ValueError, match="allgather_input"):
        Z.ZeroShardedAdamW(params, allgather_input=True)
