"""Checkpoints through ZeroShardedAdamW.state_dict() / load_state_dict(), and re-sharding
them to another data-parallel group size with reshard_state_dicts(): resumed runs equal
uninterrupted ones bit for bit (clipping off where the group size changes, since the global
norm's summation order depends on it).  The other group's ranks run on one GPU, with the
all-gather of the parameter shards done by a concatenation."""

import pytest
import torch

from workloads import WORKLOADS, gen

pytestmark = pytest.mark.gpu


def _z():
    import zero_sharded_mixed_buffer_amd as Z
    Z.lib()
    return Z


def _bits(x):
    return x.contiguous().view(torch.int16) if x.element_size() == 2 else x.contiguous().view(torch.int32)


@pytest.mark.parametrize("name,offload_after", [("llama_mini", False), ("tiny", False), ("ragged_mini", True)])
def test_state_dict_resume_bit_identical(name, offload_after):
    """6 steps straight == 3 steps, state_dict(), a new optimizer over the saved parameters,
    load_state_dict(), 3 more steps (the tiny fp16 list skips a step and changes its scale)."""
    Z = _z()
    wl = WORKLOADS[name]
    dev = torch.device("cuda", 0)
    print(f"[case] checkpoint {name} offload_after={offload_after}", flush=True)
    kw = dict(dynamic_loss_scale=wl.dynamic, init_scale=wl.init_scale, align=wl.align)
    p0 = gen.make_params(wl, dev)
    a = Z.ZeroShardedAdamW([p.clone() for p in p0], **kw)
    b = Z.ZeroShardedAdamW([p.clone() for p in p0], **kw)
    for s in range(1, 7):
        a.step(gen.make_grads(wl, s, a.read_state()["loss_scale"], dev))
        if s <= 3:
            b.step(gen.make_grads(wl, s, b.read_state()["loss_scale"], dev))
    sd = b.state_dict()
    saved_params = [p.clone() for p in b.params]
    b.close()
    c = Z.ZeroShardedAdamW(saved_params, offload=offload_after, offload_chunk=65_537, **kw)
    c.load_state_dict(sd)
    assert c.read_state()["step_t"] == sd["state"]["step_t"]
    for s in range(4, 7):
        c.step(gen.make_grads(wl, s, c.read_state()["loss_scale"], dev))
    torch.cuda.synchronize()
    for k in ("master", "m", "v"):
        assert torch.equal(_bits(getattr(a, k).cpu()), _bits(getattr(c, k).cpu())), k
    assert all(torch.equal(_bits(x), _bits(y)) for x, y in zip(a.params, c.params))
    sa, sc = a.read_state(), c.read_state()
    for k in ("loss_scale", "step_t", "skipped_total", "growth_tracker"):
        assert sa[k] == sc[k], k
    a.close()
    c.close()


@pytest.mark.parametrize("name,d_to", [("llama_mini", 2), ("ragged_mini_a64", 4)])
def test_resharded_resume_equals_single_rank(name, d_to):
    """3 steps at dp 1, then the checkpoint re-sharded to d_to ranks that take 3 more steps
    (each packs, checks its shard, shares its partial sum, updates its slice and scatters the
    concatenated parameter shards): the ranks' master, m and v concatenated, and every rank's
    parameters, equal 6 steps at dp 1 bit for bit, skipped steps included (a non-finite
    partial sum carries one rank's overflow to all)."""
    Z = _z()
    wl = WORKLOADS[name]
    dev = torch.device("cuda", 0)
    print(f"[case] reshard {name} 1 -> {d_to}", flush=True)
    kw = dict(max_norm=0.0, align=wl.align)  # no clipping: the update does not depend on the group size
    p0 = gen.make_params(wl, dev)
    a = Z.ZeroShardedAdamW([p.clone() for p in p0], **kw)
    b = Z.ZeroShardedAdamW([p.clone() for p in p0], **kw)
    for s in range(1, 7):
        a.step(gen.make_grads(wl, s, 1.0, dev))
        if s <= 3:
            b.step(gen.make_grads(wl, s, 1.0, dev))
    sd = b.state_dict()
    ranks = []
    for r in range(d_to):
        opt = Z.ZeroShardedAdamW([p.clone() for p in b.params], dp_world=d_to, dp_rank=r, **kw)
        opt.load_state_dict(Z.reshard_state_dicts([sd], d_to, r))
        ranks.append(opt)
    b.close()
    S = ranks[0].shard_numel
    exchange = torch.zeros(d_to, dtype=torch.float64, device=dev)
    shards = [torch.empty(S, dtype=ranks[0].param_dtype, device=dev) for _ in range(d_to)]
    for s in range(4, 7):
        grads = gen.make_grads(wl, s, 1.0, dev)
        for r, opt in enumerate(ranks):
            opt.pack(grads)
            opt.check(local_sumsq_out=exchange[r:r + 1])
        for r, opt in enumerate(ranks):
            opt.norm(rank_sumsq=exchange)
            opt.update(scatter=False, flat_param_out=shards[r])
        gathered = torch.cat(shards)  # the all-gather
        for opt in ranks:
            Z.zs_unpack(opt.layout, gathered, opt.param_dtype, True, opt.param_ptrs, opt.param_dtype, None)
    torch.cuda.synchronize()
    used = max(o + n for o, n in zip(Z.zs_plan(a.numels, 1, 0, wl.align)[0], a.numels))
    for k in ("master", "m", "v"):
        whole = torch.cat([getattr(opt, k) for opt in ranks])[:used]
        assert torch.equal(_bits(whole.cpu()), _bits(getattr(a, k)[:used].cpu())), k
    sa = a.read_state()
    for opt in ranks:
        so = opt.read_state()
        assert (so["step_t"], so["skipped_total"]) == (sa["step_t"], sa["skipped_total"])
        assert all(torch.equal(_bits(x), _bits(y)) for x, y in zip(a.params, opt.params))
        opt.close()
    a.close()


def test_load_state_dict_rejects_another_layout():
    Z = _z()
    wl = WORKLOADS["tiny"]
    dev = torch.device("cuda", 0)
    p0 = gen.make_params(wl, dev)
    a = Z.ZeroShardedAdamW([p.clone() for p in p0])
    sd = a.state_dict()
    b = Z.ZeroShardedAdamW([p.clone() for p in p0], dp_world=2, dp_rank=1)
    with pytest.raises(ValueError, match="reshard_state_dicts"):
        b.load_state_dict(sd)
    bad = dict(sd, master=sd["master"][:-1])
    with pytest.raises(ValueError, match="master"):
        a.load_state_dict(bad)
    a.close()
    b.close()
