"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Bar: bit-exact packed buffer, overflow flags, skip decisions, loss-scale sequence and
cast/scatter-back (as a function of the GPU master); norm within 1e-12 relative (fp64
on both sides); master, m, v within the 1e-5 relative-error contract of harness.py.
"""

import json
import math
import os

import pytest
import torch

import oracle as O
from workloads import WORKLOADS, gen

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _z():
    import zero_sharded_mixed_buffer_amd as Z
    Z.lib()
    return Z


def _log(tag, rep):
    print(f"[parity] {tag}: master_err={rep.master_err:.3e} m_err={rep.m_err:.3e} v_err={rep.v_err:.3e} "
          f"plain_master={rep.master_plain:.3e} diff(master,m,v,params)=({rep.n_master_diff},{rep.n_m_diff},"
          f"{rep.n_v_diff},{rep.n_param_diff}) scales={[s.scale_gpu for s in rep.steps]} "
          f"skips={[s.overflow_gpu for s in rep.steps]}", flush=True)


@pytest.mark.parametrize("name", ["tiny", "llama_mini", "ragged_mini", "ragged_mini_a64", "qwen_mini_dp2",
                                  "moe_mini_dp4"])
def test_workload_parity(name):
    from harness import run_parity
    _z()
    wl = WORKLOADS[name]
    print(f"[case] {name} N={wl.n_elems} T={len(wl.numels)} d={wl.dp_world} r={wl.dp_rank} "
          f"align={wl.align} steps={wl.steps}", flush=True)
    rep = run_parity(wl)
    _log(name, rep)
    overflow_steps = sorted(wl.faults.keys())
    assert [s.step for s in rep.steps if s.overflow_gpu] == overflow_steps


def test_tiny_scale_sequence_matches_hand_table():
    """fp16, S0 = 2^16, inf at step 3: skip at 3, scale halves, t = 1,2,2,3,4."""
    from harness import run_parity
    _z()
    rep = run_parity(WORKLOADS["tiny"])
    assert [s.overflow_gpu for s in rep.steps] == [0, 0, 1, 0, 0]
    assert [s.scale_gpu for s in rep.steps] == [2.0 ** 16, 2.0 ** 16, 2.0 ** 15, 2.0 ** 15, 2.0 ** 15]


@pytest.mark.parametrize("name,interval,fault_steps", [("tiny", 2, (4, 9, 10)), ("moe_mini_dp4", 3, (2, 8)),
                                                      ("tiny", 1, (3,))])
def test_scale_growth_and_backoff_sequences(name, interval, fault_steps):
    """Short growth windows, so the scale both doubles and halves within the run: the scale,
    t, tracker and skip count match the oracle's scaler after every step."""
    import dataclasses
    from harness import run_parity
    _z()
    base = WORKLOADS[name]
    faults = {s: [(0, 3, float("inf"))] for s in fault_steps}
    wl = dataclasses.replace(base, growth_interval=interval, steps=12, faults=faults)
    print(f"[case] growth {name} interval={interval} faults={fault_steps}", flush=True)
    rep = run_parity(wl)
    scales = [s.scale_gpu for s in rep.steps]
    print(f"[growth] {name}: scales={scales}", flush=True)
    assert [s.step for s in rep.steps if s.overflow_gpu] == list(fault_steps)
    assert any(b == 2 * a for a, b in zip(scales, scales[1:]))  # the scale did grow
    assert any(b == a / 2 for a, b in zip(scales, scales[1:]))  # and did back off


def test_scale_floor_holds_on_gpu():
    """Overflows in a row from a loss scale of 2 reach the floor of 1 and stay there; growth
    resumes after the window.  Scale, t, tracker and skips match the oracle each step."""
    import dataclasses
    from harness import run_parity
    _z()
    faults = {s: [(0, 1, float("inf"))] for s in (1, 2, 3, 6)}
    wl = dataclasses.replace(WORKLOADS["tiny"], init_scale=2.0, growth_interval=2, steps=9, faults=faults)
    rep = run_parity(wl)
    scales = [s.scale_gpu for s in rep.steps]
    print(f"[floor] scales={scales}", flush=True)
    assert scales == [1.0, 1.0, 1.0, 1.0, 2.0, 1.0, 1.0, 2.0, 2.0]


@pytest.mark.parametrize("rank", [0, 1, 2])
def test_dp_virtual_ranks_every_rank(rank):
    from harness import run_parity
    _z()
    wl = WORKLOADS["moe_mini_dp4"]
    rep = run_parity(wl, steps=5, dp_rank=rank)
    _log(f"moe_mini_dp4 rank {rank}", rep)


def test_page_sharded_sgd_example_on_gpu():
    """The worked example of the Megatron distributed-optimizer section through the HIP path
    (AdamW in its SGD limit, d = 2 virtual ranks): rank 0 owns [0.8, 1.6], rank 1 [2.4, 3.2]."""
    Z = _z()
    with open(os.path.join(GOLDEN, "sharded_sgd_example.json")) as f:
        ex = json.load(f)
    dev = torch.device("cuda", 0)
    d = ex["dp_world"]
    reduced = [sum(g[i] for g in ex["replica_gradients"]) / d for i in range(4)]
    hp = Z.hparams(ex["lr"] * 2.0 ** 30, 0.0, 0.0, 2.0 ** 30, 0.0, 0.0)
    owned = []
    flat = torch.tensor(reduced, dtype=torch.float16, device=dev)
    exch = torch.zeros(d, dtype=torch.float64, device=dev)
    handles = []
    for r in range(d):
        lay = Z.zs_layout_create([4], d, r)
        st = Z.zs_state_create(lay, Z.state_host(1.0, 1.0, False))
        handles.append((lay, st))
        Z.zs_unscale_check(lay, flat[r * 2:(r + 1) * 2], torch.float16, st, None, exch[r:r + 1])
    for r in range(d):
        lay, st = handles[r]
        params = [torch.tensor(ex["parameters"], dtype=torch.float16, device=dev)]
        ptrs = Z.pointer_table(params, dev)
        master = torch.empty(2, dtype=torch.float32, device=dev)
        m = torch.zeros(2, dtype=torch.float32, device=dev)
        v = torch.zeros(2, dtype=torch.float32, device=dev)
        Z.zs_pack(lay, ptrs, torch.float16, master, torch.float32, whole_flat=False)
        Z.zs_grad_norm(lay, None, torch.float16, st, hp, exch, None)
        Z.zs_adamw_step(lay, flat[r * 2:(r + 1) * 2], torch.float16, master, m, v, hp, st, ptrs, None,
                        torch.float16)
        Z.zs_scaler_update(st)
        owned.append(master.cpu())
        assert Z.zs_state_read(st).step_t == 1
    for lay, st in handles:
        Z.zs_state_destroy(st)
        Z.zs_layout_destroy(lay)
    assert torch.equal(owned[0], torch.tensor(ex["updated"][:2], dtype=torch.float32))
    assert torch.equal(owned[1], torch.tensor(ex["updated"][2:], dtype=torch.float32))


def _edge_case(numels, dtype, dp_world=1, dp_rank=0, align=1, steps=3, zero_grads=False, seed=0):
    """Run a small hand-made tensor list through the step and the oracle."""
    from harness import rel_err, bits
    Z = _z()
    dev = torch.device("cuda", 0)
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    params = [torch.randn(n, generator=g, device=dev).mul_(0.02).to(dtype) for n in numels]
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, max_norm=1.0)
    dyn = dtype == torch.float16
    scale = 2.0 ** 16 if dyn else 1.0
    opt = Z.ZeroShardedAdamW(params, dp_world=dp_world, dp_rank=dp_rank, align=align,
                             dynamic_loss_scale=dyn, init_scale=scale)
    ref = O.OracleRank(numels, dp_world, dp_rank, [p.cpu() for p in params], O.OracleScaler(scale, 1.0, dyn), hp,
                       align)
    S = ref.layout.shard_numel
    exch = torch.zeros(dp_world, dtype=torch.float64, device=dev)
    others = [(Z.zs_layout_create(numels, dp_world, q, align)) for q in range(dp_world)]
    ostates = [Z.zs_state_create(others[q], Z.state_host(scale, 1.0, dyn)) for q in range(dp_world)]
    try:
        for step in range(steps):
            grads = [(torch.zeros(n, device=dev) if zero_grads else torch.randn(n, generator=g, device=dev))
                     .mul_(1e-3 * ref.scaler.loss_scale).to(dtype) for n in numels]
            opt.pack(grads)
            if dp_world == 1:
                opt.norm()
            else:
                for q in range(dp_world):
                    if q == dp_rank:
                        opt.check(local_sumsq_out=exch[q:q + 1])
                    else:
                        Z.zs_unscale_check(others[q], opt.flat[q * S:(q + 1) * S], dtype, ostates[q], None,
                                           exch[q:q + 1])
                opt.norm(rank_sumsq=exch)
                for q in range(dp_world):
                    if q != dp_rank:
                        Z.zs_grad_norm(others[q], None, dtype, ostates[q], opt.hp, exch, None)
                        Z.zs_scaler_update(ostates[q])
            prev = [x.cpu() for x in params]
            opt.update()
            flat_ref = O.pack([x.cpu() for x in grads], ref.layout)
            other = [O.sumsq_unscaled(flat_ref[q * S:(q + 1) * S], ref.scaler.loss_scale) for q in range(dp_world)]
            ref.step(O.shard_of(flat_ref, ref.layout), other_sumsq=other if dp_world > 1 else None)
            assert torch.equal(bits(opt.flat.cpu()), bits(flat_ref))
            assert rel_err(opt.master.cpu(), ref.master) <= 1e-5
            assert rel_err(opt.m.cpu(), ref.m) <= 1e-5
            assert rel_err(opt.v.cpu(), ref.v) <= 1e-5
            # cast + scatter-back, as a function of the GPU's own master: bit-exact
            want = O.unpack(opt.master.cpu(), ref.layout, prev, False)
            assert all(torch.equal(bits(a.cpu()), bits(b)) for a, b in zip(params, want))
        st = opt.read_state()
        assert st["step_t"] == ref.scaler.step_t
        return opt, ref
    finally:
        for q in range(dp_world):
            Z.zs_state_destroy(ostates[q])
            Z.zs_layout_destroy(others[q])


@pytest.mark.parametrize("numels,dtype,d,r,align", [
    ([1], torch.bfloat16, 1, 0, 1),                      # a single element
    ([0, 5, 0, 3, 0], torch.float16, 1, 0, 1),          # empty tensors in the list, ragged tail
    ([7, 9, 4097, 1, 8191], torch.bfloat16, 3, 1, 1),   # shard starts at an odd element
    ([7, 9, 4097, 1, 8191], torch.bfloat16, 3, 2, 1),   # last shard, tail padding
    ([4096 * 3 + 5, 11, 2], torch.float16, 2, 1, 8),    # straddling tensor, aligned starts
    ([1000] * 40, torch.bfloat16, 4, 3, 64),            # gaps + padding
    ([255] * 70, torch.bfloat16, 1, 0, 1),              # 16-17 segments per pack block: either side of
                                                        # the chunked path's limit
    ([273] * 60 + [4099, 3], torch.float16, 2, 1, 1),   # 15-16 misaligned segments per pack block
    ([701] * 30, torch.bfloat16, 1, 0, 8),              # misaligned pieces and padding in one pack block
    ([1] * 5000 + [4097], torch.bfloat16, 1, 0, 1),     # thousands of segments per pack block
])
def test_edge_case_lists(numels, dtype, d, r, align):
    print(f"[case] edge numels={numels} d={d} r={r} align={align}", flush=True)
    opt, _ = _edge_case(numels, dtype, d, r, align)
    opt.close()


@pytest.mark.parametrize("seed", range(24))
def test_random_tensor_lists(seed):
    """Seeded random tensor lists: sizes around the 8-element group and the 4096-element
    tile (and empty tensors), both dtypes, random alignment, group size and rank; two steps
    of the whole path against the oracle."""
    import random
    rng = random.Random(1000 + seed)
    numels = [rng.choice([0, 1, 2, 3, 7, 8, 9, 63, 64, 65, 511, 4095, 4096, 4097, rng.randint(1, 20000)])
              for _ in range(rng.randint(1, 60))]
    if sum(numels) == 0:
        numels[0] = 5
    dtype = rng.choice([torch.bfloat16, torch.float16])
    d = rng.choice([1, 2, 3, 4, 8])
    r = rng.randrange(d)
    align = rng.choice([1, 2, 8, 64, 256])
    print(f"[case] random list seed={seed} n={len(numels)} total={sum(numels)} {dtype} d={d} r={r} align={align}",
          flush=True)
    opt, _ = _edge_case(numels, dtype, d, r, align, steps=2, seed=seed)
    opt.close()


def test_zero_gradients_apply_pure_decay():
    opt, ref = _edge_case([333, 4096], torch.bfloat16, zero_grads=True, steps=4)
    st = opt.read_state()
    assert st["grad_norm"] == 0.0 and st["clip_coef"] == 1.0
    assert torch.count_nonzero(opt.m) == 0 and torch.count_nonzero(opt.v) == 0
    opt.close()


def test_determinism_two_runs_bit_identical():
    from harness import bits
    Z = _z()
    wl = WORKLOADS["ragged_mini"]
    dev = torch.device("cuda", 0)
    outs = []
    for _ in range(2):
        params = gen.make_params(wl, dev)
        opt = Z.ZeroShardedAdamW(params, dynamic_loss_scale=False, init_scale=1.0)
        for step in range(1, 4):
            opt.step(gen.make_grads(wl, step, 1.0, dev, with_faults=False))
        outs.append((opt.master.clone(), opt.m.clone(), opt.v.clone(), opt.read_state()))
        opt.close()
    a, b = outs
    for x, y in zip(a[:3], b[:3]):
        assert torch.equal(bits(x), bits(y))
    assert a[3]["sumsq"] == b[3]["sumsq"] and a[3]["clip_coef"] == b[3]["clip_coef"]


@pytest.mark.parametrize("resume_offloaded", [False, True])
def test_checkpoint_resume_bit_identical(resume_offloaded):
    """6 steps straight == 3 steps, save (state + master/m/v + params), restore into a new
    object, 3 steps.  The restored object may also be an offloaded one: the saved device
    state continues on the host with the same bits."""
    from harness import bits
    Z = _z()
    w = WORKLOADS["llama_mini"]
    dev = torch.device("cuda", 0)
    p0 = gen.make_params(w, dev)
    a = Z.ZeroShardedAdamW([p.clone() for p in p0])
    for s in range(1, 7):
        a.step(gen.make_grads(w, s, 1.0, dev))
    b = Z.ZeroShardedAdamW([p.clone() for p in p0])
    for s in range(1, 4):
        b.step(gen.make_grads(w, s, 1.0, dev))
    saved = (b.read_state(), b.master.clone(), b.m.clone(), b.v.clone(), [p.clone() for p in b.params])
    b.close()
    c = Z.ZeroShardedAdamW(saved[4], offload=resume_offloaded, offload_chunk=100_000)
    c.write_state(saved[0])
    c.master.copy_(saved[1])
    c.m.copy_(saved[2])
    c.v.copy_(saved[3])
    for s in range(4, 7):
        c.step(gen.make_grads(w, s, 1.0, dev))
    torch.cuda.synchronize()
    for x, y in ((a.master, c.master), (a.m, c.m), (a.v, c.v)):
        assert torch.equal(bits(x.cpu()), bits(y.cpu()))
    assert all(torch.equal(bits(x), bits(y)) for x, y in zip(a.params, c.params))
    assert a.read_state()["step_t"] == c.read_state()["step_t"] == 6
    a.close()
    c.close()


def test_unpack_whole_flat_and_shard():
    """zs_unpack as the all-gather consumer: a model-dtype flat buffer (bit copy) and an fp32
    shard (RNE cast) scattered into the tensors, against the oracle's unpack."""
    from harness import bits
    Z = _z()
    dev = torch.device("cuda", 0)
    wl = WORKLOADS["ragged_mini"]
    numels = wl.numels
    for d, r, align in ((1, 0, 1), (3, 1, 1), (4, 3, 64)):
        lay = Z.zs_layout_create(numels, d, r, align)
        flat_numel, sb, sn = Z.zs_layout_info(lay)
        olay = O.plan_layout(numels, d, r, align)
        g = torch.Generator(device=dev)
        g.manual_seed(d * 10 + r)
        flat = torch.randn(flat_numel, generator=g, device=dev).to(torch.bfloat16)
        dst = [torch.zeros(n, dtype=torch.bfloat16, device=dev) for n in numels]
        ptrs = Z.pointer_table(dst, dev)
        Z.zs_unpack(lay, flat, torch.bfloat16, True, ptrs, torch.bfloat16)
        want = O.unpack(flat.cpu(), olay, [x.cpu() for x in dst], True)
        assert all(torch.equal(bits(a.cpu()), bits(b)) for a, b in zip(dst, want))
        master = torch.randn(sn, generator=g, device=dev) * 3
        dst2 = [torch.zeros(n, dtype=torch.float16, device=dev) for n in numels]
        ptrs2 = Z.pointer_table(dst2, dev)
        Z.zs_unpack(lay, master, torch.float32, False, ptrs2, torch.float16)
        want2 = O.unpack(master.cpu(), olay, [torch.zeros(n, dtype=torch.float16) for n in numels], False)
        assert all(torch.equal(bits(a.cpu()), bits(b)) for a, b in zip(dst2, want2))
        # Unpacking a flat buffer with a misaligned start (a shard view) is a bit copy too.
        shard_view = flat[sb:sb + sn]
        dst3 = [torch.zeros(n, dtype=torch.bfloat16, device=dev) for n in numels]
        Z.zs_unpack(lay, shard_view, torch.bfloat16, False, Z.pointer_table(dst3, dev), torch.bfloat16)
        want3 = O.unpack(shard_view.cpu(), olay, [torch.zeros(n, dtype=torch.bfloat16) for n in numels], False)
        assert all(torch.equal(bits(a.cpu()), bits(b)) for a, b in zip(dst3, want3))
        Z.zs_layout_destroy(lay)


def test_cast_rounding_ties_on_gpu():
    """Round-to-nearest-even of the fp32 -> bf16 / fp16 casts at exact ties and overflow."""
    from harness import bits
    Z = _z()
    dev = torch.device("cuda", 0)
    vals = torch.tensor([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 1 + 2 ** -11, 1 + 3 * 2 ** -11,
                         65519.0, 65520.0, 1e-30, -0.0, 3.0e38], dtype=torch.float32)
    n = vals.numel()
    for dt in (torch.bfloat16, torch.float16):
        lay = Z.zs_layout_create([n], 1, 0)
        dst = [torch.zeros(n, dtype=dt, device=dev)]
        Z.zs_unpack(lay, vals.to(dev), torch.float32, False, Z.pointer_table(dst, dev), dt)
        assert torch.equal(bits(dst[0].cpu()), bits(O.cast_to(vals, dt)))
        Z.zs_layout_destroy(lay)


def test_master_seeding_widens_extremes_exactly_on_gpu():
    """The pack into fp32 (how the master is seeded) widens bf16 and fp16 extremes exactly:
    values near 2^127, subnormals, signed zeros; the same bits as the oracle's pack."""
    from harness import bits
    Z = _z()
    dev = torch.device("cuda", 0)
    bf = [2.0 ** 100, -(2.0 ** -130), 3 * 2.0 ** -133, 1 + 2.0 ** -7, -1.5 * 2.0 ** 127, 0.0, -0.0, 2.0 ** -126]
    hf = [65504.0, -(2.0 ** -24), 1 + 2.0 ** -10, -3 * 2.0 ** -20, -0.0, 2.0 ** -14]
    for dt, vals in ((torch.bfloat16, bf), (torch.float16, hf)):
        src = [torch.tensor(vals[:3], dtype=dt), torch.tensor(vals[3:], dtype=dt)]
        lay = Z.zs_layout_create([3, len(vals) - 3], 1, 0)
        olay = O.plan_layout([3, len(vals) - 3], 1, 0)
        dsrc = [t.to(dev) for t in src]
        out = torch.full((olay.flat_numel,), 7.0, dtype=torch.float32, device=dev)
        Z.zs_pack(lay, Z.pointer_table(dsrc, dev), dt, out, torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(bits(out.cpu()), bits(O.pack(src, olay, torch.float32))), dt
        Z.zs_layout_destroy(lay)


def test_overflow_forms_nan_inf_neg_inf_and_ext_flag():
    Z = _z()
    dev = torch.device("cuda", 0)
    n = 10_000
    for dt in (torch.bfloat16, torch.float16):
        for bad in (math.nan, math.inf, -math.inf, None):
            lay = Z.zs_layout_create([n], 1, 0)
            st = Z.zs_state_create(lay, Z.state_host(1.0, 1.0, False))
            x = torch.ones(n, dtype=dt, device=dev)
            if bad is not None:
                x[n - 3] = bad
            Z.zs_unscale_check(lay, x, dt, st)
            assert Z.zs_state_read(st).overflow == (0 if bad is None else 1)
            ext = torch.tensor([1 if bad is None else 0], dtype=torch.int32, device=dev)
            Z.zs_unscale_check(lay, x, dt, st, ext)
            assert Z.zs_state_read(st).overflow == 1
            Z.zs_state_destroy(st)
            Z.zs_layout_destroy(lay)


def test_invalid_arguments_rejected_before_launch():
    Z = _z()
    dev = torch.device("cuda", 0)
    lay = Z.zs_layout_create([100], 1, 0)
    st = Z.zs_state_create(lay, Z.state_host(1.0, 1.0, False))
    buf = torch.zeros(128, dtype=torch.float32, device=dev)
    g = torch.zeros(100, dtype=torch.bfloat16, device=dev)
    hp = Z.hparams()
    with pytest.raises(Z.ZsError) as e:
        Z.zs_adamw_step(lay, g, torch.bfloat16, buf[1:], buf, buf, hp, st)   # unaligned master
    assert e.value.status == -1
    with pytest.raises(Z.ZsError):
        Z.zs_adamw_step(lay, g, torch.bfloat16, buf, buf, buf, Z.hparams(beta1=1.0), st)
    with pytest.raises(Z.ZsError):
        Z.zs_state_create(lay, Z.state_host(3.0, 1.0, True))                # scale not a power of two
    with pytest.raises(Z.ZsError):
        Z.zs_grad_norm(Z.zs_layout_create([100], 2, 0), None, torch.bfloat16, st, hp)  # rank_sumsq missing
    Z.zs_state_destroy(st)
    Z.zs_layout_destroy(lay)


@pytest.mark.parametrize("grad_dt,param_dt", [(torch.bfloat16, torch.bfloat16), (torch.float16, torch.float16),
                                              (torch.bfloat16, torch.float16), (torch.float16, torch.bfloat16)])
@pytest.mark.parametrize("scatter,flat_out", [(True, True), (False, True), (False, False)])
def test_adamw_output_variants(grad_dt, param_dt, scatter, flat_out):
    """Every AdamW entry-point variant (fused scatter, flat parameter shard for the all-gather,
    state only) and mixed gradient / parameter dtypes, against the oracle."""
    from harness import bits, rel_err
    Z = _z()
    dev = torch.device("cuda", 0)
    numels = [1000, 7, 4096 * 2 + 3, 129, 64]
    d, r, align = 3, 1, 1
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    params = [torch.randn(n, generator=g, device=dev).mul_(0.02).to(param_dt) for n in numels]
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, max_norm=1.0)
    lay = Z.zs_layout_create(numels, d, r, align)
    flat_numel, sb, sn = Z.zs_layout_info(lay)
    st = Z.zs_state_create(lay, Z.state_host(1.0, 1.0, False))
    olay = O.plan_layout(numels, d, r, align)
    master = torch.empty(sn, dtype=torch.float32, device=dev)
    Z.zs_pack(lay, Z.pointer_table(params, dev), param_dt, master, torch.float32, whole_flat=False)
    m = torch.zeros_like(master)
    v = torch.zeros_like(master)
    ref_master = O.shard_of(O.pack([p.cpu() for p in params], olay, torch.float32), olay).clone()
    assert torch.equal(master.cpu(), ref_master)
    ref_m, ref_v = torch.zeros(sn), torch.zeros(sn)
    ref_params = [p.cpu() for p in params]
    flat_param = torch.zeros(sn, dtype=param_dt, device=dev) if flat_out else None
    ptrs = Z.pointer_table(params, dev)
    for step in range(1, 4):
        grads = [torch.randn(n, generator=g, device=dev).mul_(1e-3).to(grad_dt) for n in numels]
        flat = torch.zeros(flat_numel, dtype=grad_dt, device=dev)
        Z.zs_pack(lay, Z.pointer_table(grads, dev), grad_dt, flat, grad_dt, whole_flat=True)
        exch = torch.zeros(d, dtype=torch.float64, device=dev)
        flat_ref = O.pack([x.cpu() for x in grads], olay)
        for q in range(d):
            exch[q] = O.sumsq_unscaled(flat_ref[q * sn:(q + 1) * sn], 1.0)   # other ranks' partials
        shard = flat[sb:sb + sn]
        Z.zs_unscale_check(lay, shard, grad_dt, st)
        Z.zs_grad_norm(lay, None, grad_dt, st, Z.hparams(**hp), exch, None)
        Z.zs_adamw_step(lay, shard, grad_dt, master, m, v, Z.hparams(**hp), st, ptrs if scatter else None,
                        flat_param, param_dt)
        Z.zs_scaler_update(st)
        norm, c = O.clip_coefficient(O.global_sumsq([float(x) for x in exch.cpu()]), hp["max_norm"])
        ref_master, ref_m, ref_v = O.adamw_update(ref_master, ref_m, ref_v, O.shard_of(flat_ref, olay), 1.0, c,
                                                  step, hp)
        assert rel_err(master.cpu(), ref_master) <= 1e-5 and rel_err(m.cpu(), ref_m) <= 1e-5
        assert rel_err(v.cpu(), ref_v) <= 1e-5
        if scatter:
            ref_params = O.unpack(master.cpu(), olay, ref_params, False)
            assert all(torch.equal(bits(a.cpu()), bits(b)) for a, b in zip(params, ref_params))
        else:
            assert all(torch.equal(bits(a.cpu()), bits(b)) for a, b in zip(params, ref_params))  # untouched
        if flat_out:
            assert torch.equal(bits(flat_param.cpu()), bits(O.cast_to(master.cpu(), param_dt)))
    Z.zs_state_destroy(st)
    Z.zs_layout_destroy(lay)


def test_grad_norm_recompute_path_matches_check_path():
    """zs_grad_norm with a shard argument (sum recomputed there) equals zs_unscale_check followed
    by zs_grad_norm(NULL); a non-finite element seen only by the recompute still sets the flag."""
    Z = _z()
    dev = torch.device("cuda", 0)
    n = 100_003
    lay = Z.zs_layout_create([n], 1, 0)
    s1 = Z.zs_state_create(lay, Z.state_host(2.0 ** 4, 1.0, True))
    s2 = Z.zs_state_create(lay, Z.state_host(2.0 ** 4, 1.0, True))
    g = torch.Generator(device=dev)
    g.manual_seed(3)
    x = torch.randn(n, generator=g, device=dev).mul_(16.0).to(torch.float16)
    hp = Z.hparams(max_norm=0.5)
    Z.zs_unscale_check(lay, x, torch.float16, s1)
    Z.zs_grad_norm(lay, None, torch.float16, s1, hp)
    Z.zs_grad_norm(lay, x, torch.float16, s2, hp)
    a, b = Z.zs_state_read(s1), Z.zs_state_read(s2)
    assert a.sumsq == b.sumsq and a.grad_norm == b.grad_norm and a.clip_coef == b.clip_coef and not a.overflow
    want = O.sumsq_unscaled(x.cpu(), 2.0 ** 4)
    assert abs(a.sumsq - want) <= 1e-12 * want
    assert a.clip_coef == O.clip_coefficient(a.sumsq, 0.5)[1]
    x[n // 3] = math.nan
    Z.zs_grad_norm(lay, x, torch.float16, s2, hp)
    assert Z.zs_state_read(s2).overflow == 1
    Z.zs_state_destroy(s1)
    Z.zs_state_destroy(s2)
    Z.zs_layout_destroy(lay)


@pytest.mark.parametrize("grad_dt", [torch.bfloat16, torch.float16])
def test_no_write_outside_buffers_with_guard_regions(grad_dt):
    """Poisoned guard regions: every tensor is a view at an odd element offset inside one big
    canary-filled buffer, and the flat buffer and fp32 shards carry canaries on both sides.
    After pack, check, norm, AdamW with scatter and flat output, unpack of the whole buffer
    and of the shard, every canary is untouched and the results still match the oracle."""
    from harness import bits
    Z = _z()
    dev = torch.device("cuda", 0)
    gen_ = torch.Generator(device=dev)
    gen_.manual_seed(11)
    numels = [4096 * 3 + 5, 1, 17, 4096, 8191, 3, 12345, 64]
    G = 37                                     # guard elements between and around tensors
    CAN16 = -12345                             # canary bit pattern for 2-byte buffers
    CAN32 = 0x7F7FBEEF

    def carve(dtype, base_dtype_fill):
        total = sum(numels) + G * (len(numels) + 1)
        big = torch.full((total,), 0, dtype=torch.int16, device=dev)
        big.fill_(base_dtype_fill)
        views, off = [], G
        for n in numels:
            views.append(big[off:off + n].view(dtype))
            off += n + G
        return big, views

    gbig, grads = carve(grad_dt, CAN16)
    pbig, params = carve(grad_dt, CAN16)
    for p in params:
        p.copy_(torch.randn(p.numel(), generator=gen_, device=dev).mul_(0.02).to(grad_dt))
    for g in grads:
        g.copy_(torch.randn(g.numel(), generator=gen_, device=dev).mul_(1e-3).to(grad_dt))
    d, r = 2, 1
    lay = Z.zs_layout_create(numels, d, r, 1)
    flat_numel, sb, sn = Z.zs_layout_info(lay)
    olay = O.plan_layout(numels, d, r, 1)
    st = Z.zs_state_create(lay, Z.state_host(1.0, 1.0, False))
    fl_big = torch.full((flat_numel + 2 * 64,), CAN16, dtype=torch.int16, device=dev)
    flat = fl_big[64:64 + flat_numel].view(grad_dt)
    f32 = lambda: torch.full((sn + 2 * 64,), CAN32, dtype=torch.int32, device=dev)
    mbig, m1big, v1big, fobig = f32(), f32(), f32(), torch.full((sn + 2 * 64,), CAN16, dtype=torch.int16, device=dev)
    master, m, v = mbig[64:64 + sn].view(torch.float32), m1big[64:64 + sn].view(torch.float32), v1big[64:64 + sn].view(torch.float32)
    flat_param = fobig[64:64 + sn].view(grad_dt)
    m.zero_()
    v.zero_()
    pp, gp = Z.pointer_table(params, dev), Z.pointer_table(grads, dev)
    params_before = [p.cpu() for p in params]
    Z.zs_pack(lay, pp, grad_dt, master, torch.float32, whole_flat=False)
    Z.zs_pack(lay, gp, grad_dt, flat, grad_dt, whole_flat=True)
    exch = torch.zeros(d, dtype=torch.float64, device=dev)
    for q in range(d):
        lq = Z.zs_layout_create(numels, d, q, 1)
        sq = Z.zs_state_create(lq, Z.state_host(1.0, 1.0, False))
        Z.zs_unscale_check(lq, flat[q * sn:(q + 1) * sn], grad_dt, sq, None, exch[q:q + 1])
        Z.zs_state_destroy(sq)
        Z.zs_layout_destroy(lq)
    shard = flat[sb:sb + sn]
    Z.zs_unscale_check(lay, shard, grad_dt, st)
    hp = Z.hparams()
    Z.zs_grad_norm(lay, None, grad_dt, st, hp, exch, None)
    Z.zs_adamw_step(lay, shard, grad_dt, master, m, v, hp, st, pp, flat_param, grad_dt)
    Z.zs_unpack(lay, flat_param, grad_dt, False, pp, grad_dt)
    Z.zs_unpack(lay, flat, grad_dt, True, gp, grad_dt)
    Z.zs_scaler_update(st)
    torch.cuda.synchronize()

    def guards_ok(big, n_lead, n_body, can):
        b = big.cpu()
        return bool((b[:n_lead] == can).all()) and bool((b[n_lead + n_body:] == can).all())
    assert guards_ok(fl_big, 64, flat_numel, CAN16)
    for big in (mbig, m1big, v1big):
        assert guards_ok(big, 64, sn, CAN32)
    assert guards_ok(fobig, 64, sn, CAN16)
    for big in (gbig, pbig):
        b = big.cpu()
        off = 0
        for n in numels:
            assert bool((b[off:off + G] == CAN16).all())
            off += G + n
        assert bool((b[off:] == CAN16).all())
    # Results still right: packed buffer bit-exact, params = cast of the new master.
    flat_ref = O.pack([x.cpu() for x in grads], olay)
    assert torch.equal(bits(flat.cpu()), bits(flat_ref))
    want = O.unpack(master.cpu(), olay, params_before, False)
    assert all(torch.equal(bits(a.cpu()), bits(b)) for a, b in zip(params, want))
    Z.zs_state_destroy(st)
    Z.zs_layout_destroy(lay)


@pytest.mark.parametrize("name,accum", [("llama_mini", torch.float32), ("ragged_mini", torch.float32),
                                        ("ragged_mini", None), ("moe_mini_dp4", torch.float32),
                                        ("tiny", None), ("qwen_mini_dp2", None)])
def test_gradient_accumulation_parity(name, accum):
    """Gradient accumulation fused into the pack (3 micro-steps per step), in an fp32 buffer
    or in the model dtype, against the oracle's accumulate(); injected faults land on the
    last micro-step and must still skip the step."""
    from harness import run_parity_accumulation
    _z()
    wl = WORKLOADS[name]
    acc_dt = accum if accum is not None else gen.TORCH_DTYPE[wl.dtype]
    print(f"[case] accumulation {name} accum={acc_dt}", flush=True)
    flags = run_parity_accumulation(wl, 3, acc_dt, steps=min(wl.steps, 6))
    assert [i + 1 for i, f in enumerate(flags) if f] == [s for s in sorted(wl.faults) if s <= min(wl.steps, 6)]


@pytest.mark.parametrize("accum", [None, torch.float32])
def test_accumulation_that_overflows_skips_the_step(accum):
    """Finite fp16 micro-step gradients whose sum leaves fp16's range: in a model-dtype buffer
    the accumulated value rounds to inf, the step is skipped and the scale halves; in an
    fp32 buffer the same sum stays finite and the step is applied.  Both against the oracle."""
    from harness import bits
    Z = _z()
    dev = torch.device("cuda", 0)
    numels = [6, 3]
    params = [torch.tensor([0.5, -0.25, 1.0, 0.0, 3.0, 2.0], dtype=torch.float16, device=dev),
              torch.tensor([1.0, -1.0, 0.125], dtype=torch.float16, device=dev)]
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, max_norm=1.0)
    opt = Z.ZeroShardedAdamW(params, dynamic_loss_scale=True, init_scale=2.0 ** 16, accum_dtype=accum)
    ref = O.OracleRank(numels, 1, 0, [p.cpu() for p in params], O.OracleScaler(2.0 ** 16), hp)
    micro = [[torch.tensor([40000.0, 1.0, -3.0, 0.5, 2.0, 60000.0], dtype=torch.float16),
              torch.tensor([7.0, -7.0, 1.0], dtype=torch.float16)],
             [torch.tensor([40000.0, 2.0, 3.0, 0.5, -2.0, 10000.0], dtype=torch.float16),
              torch.tensor([1.0, 1.0, 1.0], dtype=torch.float16)]]
    opt.step([[t.to(dev) for t in m] for m in micro])
    buf_dt = accum if accum is not None else torch.float16
    acc = O.pack(micro[0], ref.layout, buf_dt)
    acc = O.accumulate(acc, micro[1], ref.layout)
    assert torch.equal(bits(opt.flat.cpu()), bits(acc))
    rec = ref.step(O.shard_of(acc, ref.layout))
    st = opt.read_state()
    assert st["overflow"] == int(rec["overflow"]) and rec["overflow"] == (accum is None)
    assert st["loss_scale"] == ref.scaler.loss_scale == (2.0 ** 15 if accum is None else 2.0 ** 16)
    for a, b in ((opt.master, ref.master), (opt.m, ref.m), (opt.v, ref.v)):
        assert torch.equal(bits(a.cpu()), bits(b))
    opt.close()


def test_step_captures_into_a_hip_graph():
    """The step enqueues kernels only (no host synchronisation, no allocation), so the whole
    single-rank step can be captured once and replayed.  Every replay is compared with the
    same steps run eagerly on a second optimizer, with eager work and synchronisations
    between the replays."""
    from harness import bits
    Z = _z()
    dev = torch.device("cuda", 0)
    wl = WORKLOADS["ragged_mini"]
    p0 = gen.make_params(wl, dev)
    graph_opt = Z.ZeroShardedAdamW([p.clone() for p in p0], dynamic_loss_scale=False, init_scale=1.0)
    eager_opt = Z.ZeroShardedAdamW([p.clone() for p in p0], dynamic_loss_scale=False, init_scale=1.0)
    grads = gen.make_grads(wl, 1, 1.0, dev, with_faults=False)
    # warm up on a side stream (torch requires it before capture), then capture one step
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        graph_opt.step(grads)
    torch.cuda.current_stream().wait_stream(s)
    eager_opt.step(grads)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        graph_opt.step(grads)
    for replay in range(4):
        new = gen.make_grads(wl, 10 + replay, 1.0, dev, with_faults=False)
        for dst, src in zip(grads, new):
            dst.copy_(src)
        g.replay()
        eager_opt.step(grads)
        torch.cuda.synchronize()
        for a, b in ((graph_opt.master, eager_opt.master), (graph_opt.m, eager_opt.m), (graph_opt.v, eager_opt.v)):
            assert torch.equal(bits(a), bits(b)), f"replay {replay}"
        assert all(torch.equal(bits(a), bits(b)) for a, b in zip(graph_opt.params, eager_opt.params))
        sa, sb = graph_opt.read_state(), eager_opt.read_state()
        # one warm-up step plus replay + 1 steps (capturing records the step without running it)
        assert sa["step_t"] == sb["step_t"] == replay + 2 and sa["sumsq"] == sb["sumsq"]
    graph_opt.close()
    eager_opt.close()


def test_spaced_state_placement_gives_the_same_results():
    """master, m and v carved from one allocation at a chosen distance (state_spacing) hold
    exactly what three separate allocations hold."""
    from harness import bits
    Z = _z()
    wl = WORKLOADS["llama_mini"]
    dev = torch.device("cuda", 0)
    p0 = gen.make_params(wl, dev)
    a = Z.ZeroShardedAdamW([p.clone() for p in p0])
    b = Z.ZeroShardedAdamW([p.clone() for p in p0], state_spacing=64 << 20)
    assert b.m.data_ptr() - b.master.data_ptr() == 64 << 20
    for step in range(1, 4):
        grads = gen.make_grads(wl, step, 1.0, dev, with_faults=False)
        a.step(grads)
        b.step(grads)
    torch.cuda.synchronize()
    for x, y in ((a.master, b.master), (a.m, b.m), (a.v, b.v)):
        assert torch.equal(bits(x), bits(y))
    assert all(torch.equal(bits(x), bits(y)) for x, y in zip(a.params, b.params))
    a.close()
    b.close()


@pytest.mark.parametrize("d", [1, 2, 4, 8])
def test_device_memory_matches_the_pages_byte_ledger(d):
    """Bytes per parameter on one rank against the page's table of distributed bytes per
    BF16 parameter with an FP32 main gradient (golden byte_ledger.json): the replicated
    2-byte parameter and 4-byte gradient buffer plus 12/d bytes of fp32 master, m and v."""
    Z = _z()
    with open(os.path.join(GOLDEN, "byte_ledger.json")) as f:
        ledger = json.load(f)
    dev = torch.device("cuda", 0)
    n = 1 << 24
    params = [torch.zeros(n - 1000, dtype=torch.bfloat16, device=dev), torch.zeros(1000, dtype=torch.bfloat16,
                                                                                       device=dev)]
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    opt = Z.ZeroShardedAdamW(params, dp_world=d, dp_rank=d - 1, accum_dtype=torch.float32)
    torch.cuda.synchronize()
    added = torch.cuda.memory_allocated() - before
    per_param = (added + 2 * n) / n       # the parameters were there before the optimizer
    want = ledger["bytes_by_group_size"][str(d)]
    print(f"[ledger] d={d}: {per_param:.4f} bytes per parameter, the page's table {want}", flush=True)
    assert abs(per_param - want) <= 0.01 * want
    opt.close()
