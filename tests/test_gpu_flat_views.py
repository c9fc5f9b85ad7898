"""ZeroShardedAdamW(flat_views=True): parameters and their .grad are views into a contiguous
parameter buffer and a contiguous gradient buffer laid out like the flat buffer ("Deep
dive: Megatron", section "Distributed optimizer": backward fills a contiguous gradient
buffer and the update rebuilds a contiguous 2-byte parameter buffer), so the step needs no
pack and no scatter.  Checked against the oracle at the bar of the other parity tests, and
with autograd writing the gradients through the views."""

import math

import pytest
import torch

import oracle as O
from workloads import WORKLOADS, gen

pytestmark = pytest.mark.gpu


def _z():
    import zero_sharded_mixed_buffer_amd as Z
    Z.lib()
    return Z


@pytest.mark.parametrize("name,offload", [("tiny", False), ("llama_mini", False), ("ragged_mini", False),
                                          ("ragged_mini_a64", False), ("ragged_mini_a64", True),
                                          ("tiny", True)])
def test_flat_views_step_against_the_oracle(name, offload):
    """offload=True: the host update writes the new parameters straight into the parameter
    buffer (no unpack)."""
    from harness import REL_TOL, bits, rel_err
    Z = _z()
    wl = WORKLOADS[name]
    dt = gen.TORCH_DTYPE[wl.dtype]
    hp = wl.hparams
    dev = torch.device("cuda", 0)
    params = gen.make_params(wl, dev)
    ref = O.OracleRank(wl.numels, 1, 0, [p.cpu() for p in params],
                       O.OracleScaler(wl.init_scale, 1.0, wl.dynamic, wl.growth_interval), hp, wl.align)
    opt = Z.ZeroShardedAdamW(params, lr=hp["lr"], betas=(hp["beta1"], hp["beta2"]), eps=hp["eps"],
                             weight_decay=hp["weight_decay"], max_norm=hp["max_norm"], align=wl.align,
                             dynamic_loss_scale=wl.dynamic, init_scale=wl.init_scale,
                             growth_interval=wl.growth_interval, flat_views=True, offload=offload,
                             offload_chunk=50_001, offload_threads=3)
    base = opt.flat_params.data_ptr()
    for p, off in zip(params, ref.layout.offsets):  # every parameter now lives in the buffer
        assert p.data_ptr() == base + 2 * off and p.grad.data_ptr() == opt.flat.data_ptr() + 2 * off
    print(f"[case] flat views {name}: {len(wl.numels)} tensors, align {wl.align}, {wl.steps} steps", flush=True)
    for step in range(1, wl.steps + 1):
        grads = gen.make_grads(wl, step, ref.scaler.loss_scale, dev)
        opt.zero_grad()
        for p, g in zip(params, grads):
            p.grad.add_(g)  # what backward's accumulation into the views does
        opt.step()
        rec = ref.step(O.shard_of(O.pack([g.cpu() for g in grads], ref.layout), ref.layout))
        st = opt.read_state()
        assert st["overflow"] == int(rec["overflow"]) and st["loss_scale"] == ref.scaler.loss_scale
        assert st["step_t"] == ref.scaler.step_t and st["skipped_total"] == ref.scaler.skipped_total
    for got, want, what in ((opt.master, ref.master, "master"), (opt.m, ref.m, "m"), (opt.v, ref.v, "v")):
        err = rel_err(got.cpu(), want)
        assert err <= REL_TOL, f"{what}: {err}"
    if offload:
        assert opt.flat_param.data_ptr() == opt.flat_params.data_ptr()  # no separate output buffer
    # the parameter buffer holds the cast of the master, padding included (zero there)
    assert torch.equal(bits(opt.flat_params.cpu()), bits(O.cast_to(opt.master.cpu(), dt)))
    for p, off, n in zip(params, ref.layout.offsets, ref.layout.numels):
        assert torch.equal(bits(p.detach().reshape(-1).cpu()), bits(opt.flat_params[off:off + n].cpu()))
    opt.close()


def test_flat_views_take_the_gradients_from_autograd():
    """A small bf16 model (elementwise, no matrix products): backward accumulates into the
    .grad views, so the gradient buffer holds exactly the gradients autograd computes for an
    independent copy of the model, and the step then matches the oracle fed those
    gradients."""
    from harness import REL_TOL, bits, rel_err
    Z = _z()
    dev = torch.device("cuda", 0)
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    shapes = [(64, 33), (33,), (1,), (17, 5, 3)]
    init = [torch.randn(s, generator=g, device=dev).to(torch.bfloat16) for s in shapes]
    xs = [torch.randn(s, generator=g, device=dev).to(torch.bfloat16) for s in shapes]

    def loss_of(ps):
        return sum(((p.float() * x.float()) ** 2).sum() * (i + 1) for i, (p, x) in enumerate(zip(ps, xs)))

    model = [torch.nn.Parameter(t.clone()) for t in init]
    twin = [torch.nn.Parameter(t.clone()) for t in init]
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, max_norm=1.0)
    opt = Z.ZeroShardedAdamW(model, lr=hp["lr"], weight_decay=hp["weight_decay"], max_norm=hp["max_norm"],
                             align=8, flat_views=True)
    numels = [t.numel() for t in init]
    ref = O.OracleRank(numels, 1, 0, [t.cpu() for t in init], O.OracleScaler(1.0, dynamic=False), hp, 8)
    for step in range(3):
        opt.zero_grad()
        loss_of(model).backward()
        for p in twin:
            p.grad = None
        loss_of(twin).backward()
        for p, q, off, n in zip(model, twin, ref.layout.offsets, numels):
            assert p.grad.data_ptr() == opt.flat.data_ptr() + 2 * off  # still the view
            assert torch.equal(bits(opt.flat[off:off + n].cpu()), bits(q.grad.reshape(-1).cpu()))
        opt.step()
        ref.step(O.shard_of(O.pack([q.grad.cpu() for q in twin], ref.layout), ref.layout))
        with torch.no_grad():  # the twin follows the oracle's parameters
            for q, r in zip(twin, ref.params):
                q.copy_(r.view(q.shape))
    for got, want in ((opt.master, ref.master), (opt.m, ref.m), (opt.v, ref.v)):
        assert rel_err(got.cpu(), want) <= REL_TOL
    for p, r in zip(model, ref.params):
        assert torch.equal(bits(p.detach().reshape(-1).cpu()), bits(r.reshape(-1)))
    opt.close()


def test_flat_views_reject_what_they_cannot_hold():
    Z = _z()
    dev = torch.device("cuda", 0)
    mixed = [torch.zeros(8, dtype=torch.bfloat16, device=dev), torch.zeros(8, dtype=torch.float16, device=dev)]
    with pytest.raises(ValueError):
        Z.ZeroShardedAdamW(mixed, flat_views=True)
    with pytest.raises(ValueError):
        Z.ZeroShardedAdamW([torch.zeros(8, dtype=torch.bfloat16, device=dev)], flat_views=True,
                           accum_dtype=torch.float32)
    opt = Z.ZeroShardedAdamW([torch.zeros(8, dtype=torch.bfloat16, device=dev)])
    with pytest.raises(ValueError):
        opt.step()  # no gradients and no views
    opt.close()
    twice = torch.zeros(8, dtype=torch.bfloat16, device=dev)
    with pytest.raises(ValueError, match="more than once"):
        Z.ZeroShardedAdamW([twice, twice])
    # a .grad set to None (as a model-level zero_grad does) is refused, and zero_grad() mends it
    ps = [torch.nn.Parameter(torch.ones(8, dtype=torch.bfloat16, device=dev)) for _ in range(2)]
    opt = Z.ZeroShardedAdamW(ps, flat_views=True)
    ps[1].grad = None
    with pytest.raises(ValueError, match="zero_grad"):
        opt.step()
    opt.zero_grad()
    assert ps[1].grad.data_ptr() == opt.flat.data_ptr() + 2 * 8
    opt.step()
    assert opt.read_state()["step_t"] == 1
    opt.close()


@pytest.mark.parametrize("name", ["qwen_mini_dp2", "moe_mini_dp4"])
def test_flat_views_every_virtual_rank_against_the_oracle(name):
    """Several ranks in one process, each with its own copy of the model in flat views.
    Every rank's gradient buffer holds the same gradients, so its shard stands in for the
    reduce-scatter output; the ranks exchange their local sums of squares, each update
    writes its slice of its parameter buffer, and copying every slice into the other ranks'
    buffers stands in for the all-gather.  Every rank's state shard and whole parameter
    buffer match the oracle's ranks."""
    from harness import REL_TOL, bits, rel_err
    Z = _z()
    wl = WORKLOADS[name]
    d = wl.dp_world
    dt = gen.TORCH_DTYPE[wl.dtype]
    hp = wl.hparams
    dev = torch.device("cuda", 0)
    p0 = gen.make_params(wl, dev)
    kw = dict(lr=hp["lr"], betas=(hp["beta1"], hp["beta2"]), eps=hp["eps"], weight_decay=hp["weight_decay"],
              max_norm=hp["max_norm"], dp_world=d, align=wl.align, dynamic_loss_scale=wl.dynamic,
              init_scale=wl.init_scale, growth_interval=wl.growth_interval, flat_views=True)
    models = [[p.clone() for p in p0] for _ in range(d)]
    opts = [Z.ZeroShardedAdamW(models[r], dp_rank=r, **kw) for r in range(d)]
    refs = [O.OracleRank(wl.numels, d, r, [p.cpu() for p in p0],
                         O.OracleScaler(wl.init_scale, 1.0, wl.dynamic, wl.growth_interval), hp, wl.align)
            for r in range(d)]
    S = opts[0].shard_numel
    exchange = torch.zeros(d, dtype=torch.float64, device=dev)
    print(f"[case] flat views {name}: {d} ranks, {wl.steps} steps", flush=True)
    for step in range(1, wl.steps + 1):
        grads = gen.make_grads(wl, step, refs[0].scaler.loss_scale, dev)
        for r in range(d):
            opts[r].zero_grad()
            for p, g in zip(models[r], grads):
                p.grad.add_(g)
            opts[r].check(local_sumsq_out=exchange[r:r + 1])
        for r in range(d):
            opts[r].norm(rank_sumsq=exchange)
            opts[r].update()
        for q in range(d):  # the all-gather's stand-in
            for r in range(d):
                if q != r:
                    opts[q].flat_params[r * S:(r + 1) * S].copy_(opts[r].param_shard)
        # the oracle ranks: every rank's flag and partial sum feed every rank's step
        flat = O.pack([g.cpu() for g in grads], refs[0].layout)
        shards = [O.shard_of(flat, refs[r].layout) for r in range(d)]
        bad = [O.nonfinite_any(x) for x in shards]
        sums = [math.inf if b else O.sumsq_unscaled(x, refs[0].scaler.loss_scale) for b, x in zip(bad, shards)]
        for r in range(d):  # other_sumsq is indexed by rank; the rank's own entry is not read
            rec = refs[r].step(shards[r], ext_overflow=any(bad[q] for q in range(d) if q != r), other_sumsq=sums)
            st = opts[r].read_state()
            assert st["overflow"] == int(rec["overflow"]) and st["loss_scale"] == refs[r].scaler.loss_scale
    for r in range(d):
        for got, want in ((opts[r].master, refs[r].master), (opts[r].m, refs[r].m), (opts[r].v, refs[r].v)):
            assert rel_err(got.cpu(), want) <= REL_TOL
        full = torch.cat([O.cast_to(opts[q].master.cpu(), dt) for q in range(d)])
        assert torch.equal(bits(opts[r].flat_params.cpu()), bits(full))
    for o in opts:
        o.close()


@pytest.mark.parametrize("name", ["tiny", "ragged_mini_a64", "over_one_level"])
def test_step_flat_bit_identical_to_the_call_sequence(name):
    """step() with flat views is the single call zs_step_flat; it equals the four calls
    (check, norm, update into the parameter buffer, scaler commit) bit for bit, through a
    skipped step and scale growth, on both sides of the two-level fold of the partial sums."""
    import dataclasses
    from harness import bits
    from test_gpu_step import CASES
    Z = _z()
    dev = torch.device("cuda", 0)
    wl = dataclasses.replace(CASES[name](), growth_interval=2)
    p0 = gen.make_params(wl, dev)
    kw = dict(align=wl.align, dynamic_loss_scale=wl.dynamic, init_scale=wl.init_scale,
              growth_interval=wl.growth_interval, flat_views=True)
    ma, mb = [p.clone() for p in p0], [p.clone() for p in p0]
    one, seq = Z.ZeroShardedAdamW(ma, **kw), Z.ZeroShardedAdamW(mb, **kw)
    for step in range(1, wl.steps + 1):
        print(f"[case] zs_step_flat {name} step {step}", flush=True)
        grads = gen.make_grads(wl, step, one.read_state()["loss_scale"], dev)
        for opt, model in ((one, ma), (seq, mb)):
            opt.zero_grad()
            for p, g in zip(model, grads):
                p.grad.add_(g)
        one.step()
        seq.check()
        seq.norm()
        seq.update()
        torch.cuda.synchronize()
        for x, y in ((one.master, seq.master), (one.m, seq.m), (one.v, seq.v), (one.flat_params, seq.flat_params)):
            assert torch.equal(bits(x), bits(y)), f"step {step}"
        sa, sb = one.read_state(), seq.read_state()
        for k in sa:
            assert sa[k] == sb[k] or (isinstance(sa[k], float) and math.isnan(sa[k]) and math.isnan(sb[k])), k
    assert one.read_state()["skipped_total"] == len(wl.faults)
    one.close()
    seq.close()


def test_step_flat_replays_in_a_hip_graph():
    """The flat-views step captured once and replayed with new gradients in the buffer each
    time (one replay overflowing), against the four calls run eagerly on a twin."""
    import dataclasses
    from harness import bits
    Z = _z()
    dev = torch.device("cuda", 0)
    wl = dataclasses.replace(WORKLOADS["tiny"], growth_interval=2)
    p0 = gen.make_params(wl, dev)
    kw = dict(dynamic_loss_scale=wl.dynamic, init_scale=wl.init_scale, growth_interval=wl.growth_interval,
              flat_views=True)
    ma, mb = [p.clone() for p in p0], [p.clone() for p in p0]
    gopt, eopt = Z.ZeroShardedAdamW(ma, **kw), Z.ZeroShardedAdamW(mb, **kw)

    def load(model, opt, grads):
        opt.zero_grad()
        for p, g in zip(model, grads):
            p.grad.add_(g)

    grads = gen.make_grads(wl, 1, wl.init_scale, dev, with_faults=False)
    load(ma, gopt, grads)
    load(mb, eopt, grads)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        gopt.step()
    torch.cuda.current_stream().wait_stream(s)
    eopt.check()
    eopt.norm()
    eopt.update()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gopt.step()
    torch.cuda.synchronize()
    for replay in range(5):
        grads = gen.make_grads(wl, 20 + replay, eopt.read_state()["loss_scale"], dev, with_faults=False)
        if replay == 3:
            grads[2].view(-1)[5] = math.inf
        load(ma, gopt, grads)
        load(mb, eopt, grads)
        graph.replay()
        eopt.check()
        eopt.norm()
        eopt.update()
        torch.cuda.synchronize()
        for x, y in ((gopt.master, eopt.master), (gopt.m, eopt.m), (gopt.v, eopt.v),
                     (gopt.flat_params, eopt.flat_params)):
            assert torch.equal(bits(x), bits(y)), f"replay {replay}"
        assert gopt.read_state()["loss_scale"] == eopt.read_state()["loss_scale"]
    assert gopt.read_state()["skipped_total"] == 1 and gopt.read_state()["step_t"] == 5
    gopt.close()
    eopt.close()


def test_flat_views_with_several_ranks_need_align_8():
    """Each rank writes its slice of the parameter buffer with 16-byte stores, so with several
    ranks the slices must start on 16-byte boundaries: align 1 with an odd-sized list is
    refused; align 8 gives every rank an aligned slice."""
    Z = _z()
    dev = torch.device("cuda", 0)
    sizes = (5, 3, 9)  # 17 elements: shards of 9 at align 1
    with pytest.raises(ValueError, match="multiple of 8"):
        Z.ZeroShardedAdamW([torch.zeros(n, dtype=torch.bfloat16, device=dev) for n in sizes], dp_world=2,
                           dp_rank=1, flat_views=True)
    for r in range(2):
        opt = Z.ZeroShardedAdamW([torch.zeros(n, dtype=torch.bfloat16, device=dev) for n in sizes], dp_world=2,
                                 dp_rank=r, align=8, flat_views=True)
        assert opt.param_shard.data_ptr() % 16 == 0 and opt.shard_numel % 8 == 0
        opt.close()
