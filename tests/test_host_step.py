"""CPU parity of the host (offloaded) AdamW update, zs_host_adamw_step, against the oracle.

The host step runs on the CPU inside libzs, so these tests need no GPU.  They compare it
with oracle.adamw_update and oracle.cast_to under the same scalars (loss scale, clip
coefficient, t), check its fp32 -> bf16 / fp16 casts and its fp16 -> fp32 widening over
large sets of bit patterns against torch's conversions, and check that the thread count
does not change any bit.
"""

import numpy as np
import pytest
import torch

import oracle as O
from workloads import WORKLOADS, gen

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, max_norm=1.0)
REL_TOL = 1e-5


def _z():
    import zero_sharded_mixed_buffer_amd as Z
    try:
        Z.lib()
    except ImportError as e:  # the build step must run first; fail loudly, never skip silently
        pytest.fail(str(e))
    return Z


def _hp(Z, hp):
    return Z.hparams(hp["lr"], hp["beta1"], hp["beta2"], hp["eps"], hp["weight_decay"], hp["max_norm"])


def _scalars(Z, loss_scale, clip, step_t, overflow=0):
    s = Z.state_host(loss_scale, 1.0, False)
    s.clip_coef = clip
    s.step_t = step_t
    s.overflow = overflow
    return s


def _bits(x):
    return x.view({2: torch.int16, 4: torch.int32}[x.element_size()])


def _rel(a, b):
    a, b = a.double(), b.double()
    return float(((a - b).abs() / b.abs().clamp_min(1e-3)).max()) if a.numel() else 0.0


@pytest.mark.parametrize("name", ["tiny", "llama_mini", "ragged_mini", "moe_mini_dp4"])
def test_host_step_matches_oracle_over_steps(name):
    """Several consecutive updates of a workload's shard: the host step, given the oracle's
    loss scale, clip coefficient and t, against oracle.adamw_update (the 1e-5 relative bar
    of the GPU path, and in practice bit for bit)."""
    Z = _z()
    wl = WORKLOADS[name]
    lay = O.plan_layout(list(wl.numels), wl.dp_world, wl.dp_rank, wl.align)
    dt = gen.TORCH_DTYPE[wl.dtype]
    params = gen.make_params(wl)
    master0 = O.shard_of(O.pack(params, lay, torch.float32), lay)
    o_master, o_m, o_v = master0.clone(), torch.zeros_like(master0), torch.zeros_like(master0)
    h_master, h_m, h_v = master0.clone(), torch.zeros_like(master0), torch.zeros_like(master0)
    out = torch.empty(lay.shard_numel, dtype=dt)
    scale = wl.init_scale
    hp = dict(HP)
    n_exact = 0
    for step in range(1, 5):
        x = O.shard_of(O.pack(gen.make_grads(wl, step, scale, with_faults=False), lay), lay)
        norm, clip = O.clip_coefficient(O.sumsq_unscaled(x, scale), hp["max_norm"])
        o_master, o_m, o_v = O.adamw_update(o_master, o_m, o_v, x, scale, clip, step, hp)
        Z.zs_host_adamw_step(x, dt, h_master, h_m, h_v, lay.shard_numel, _hp(Z, hp),
                             _scalars(Z, scale, clip, step - 1), out, dt, 3)
        for a, b in ((h_master, o_master), (h_m, o_m), (h_v, o_v)):
            assert _rel(a, b) <= REL_TOL
            n_exact += int(torch.equal(_bits(a), _bits(b)))
        assert torch.equal(_bits(out), _bits(O.cast_to(h_master, dt)))
    print(f"[host] {name}: {n_exact} of 12 state arrays bit-identical to the oracle")


@pytest.mark.parametrize("gdt", [torch.bfloat16, torch.float16, torch.float32])
@pytest.mark.parametrize("pdt", [torch.bfloat16, torch.float16])
def test_host_step_dtypes_random(gdt, pdt):
    Z = _z()
    g = torch.Generator().manual_seed(3)
    n = 100_003
    scale = 1024.0 if gdt == torch.float16 else 1.0
    x = (torch.randn(n, generator=g) * 1e-2 * scale).to(gdt)
    master = torch.randn(n, generator=g) * 0.02
    m = torch.randn(n, generator=g) * 1e-3
    v = torch.rand(n, generator=g) * 1e-6
    clip, t = 0.37, 5
    hp = dict(HP)
    want = O.adamw_update(master, m, v, x, scale, clip, t, hp)
    hm, hmm, hv = master.clone(), m.clone(), v.clone()
    out = torch.empty(n, dtype=pdt)
    Z.zs_host_adamw_step(x, gdt, hm, hmm, hv, n, _hp(Z, hp), _scalars(Z, scale, clip, t - 1), out, pdt, 4)
    for a, b in zip((hm, hmm, hv), want):
        assert _rel(a, b) <= REL_TOL
    assert torch.equal(_bits(out), _bits(O.cast_to(hm, pdt)))


def _identity_update(Z, master, pdt):
    """lr = 0, zero gradient and moments: the new master equals the old one exactly, so the
    parameter output is the host's cast of `master`."""
    n = master.numel()
    z = torch.zeros(n)
    out = torch.empty(n, dtype=pdt)
    hp = dict(HP, lr=0.0, weight_decay=0.0)
    Z.zs_host_adamw_step(torch.zeros(n), torch.float32, master.clone(), z.clone(), z.clone(), n, _hp(Z, hp),
                         _scalars(Z, 1.0, 1.0, 0), out, pdt, 4)
    return out


@pytest.mark.parametrize("pdt", [torch.bfloat16, torch.float16])
def test_host_casts_match_torch_round_to_nearest_even(pdt):
    Z = _z()
    rng = np.random.default_rng(11)
    pats = [rng.integers(0, 2 ** 32, size=1 << 21, dtype=np.uint64).astype(np.uint32)]
    # every pattern around the binary16 / bfloat16 boundaries: the smallest and largest
    # normals, the subnormal range, the overflow threshold, ties at every exponent
    for base in (0x33000000, 0x33800000, 0x387FC000, 0x38800000, 0x477FE000, 0x477FF000, 0x7F7F0000, 0x7F800000,
                 0x00000000, 0x00800000, 0x3F800000):
        pats.append(np.arange(base - 4096, base + 4096, dtype=np.int64).astype(np.uint32))
    ties = (np.arange(0, 255, dtype=np.uint32) << 23) | 0x00001000  # fp16 tie bits at every exponent
    pats += [ties, ties | 0x00002000, ties | 0x00008000, ties | 0x00010000]
    u = np.concatenate(pats)
    u = np.concatenate([u, u | 0x80000000])
    master = torch.from_numpy(u.view(np.int32).copy()).view(torch.float32)
    got = _identity_update(Z, master, pdt)
    want = master.to(pdt)
    nan = torch.isnan(want)
    assert torch.equal(torch.isnan(got), nan)
    assert torch.equal(_bits(got)[~nan], _bits(want)[~nan])


def test_host_fp16_gradients_widen_exactly():
    """beta1 = 0 and a unit scale make the new first moment the widened gradient itself
    (the old moment, -0, enters as 0 * -0 = -0, which keeps a -0 gradient's sign), so every
    finite fp16 pattern's widening is checked against torch's."""
    Z = _z()
    allh = torch.arange(-32768, 32768, dtype=torch.int32).to(torch.int16).view(torch.float16)
    finite = torch.isfinite(allh)
    x = allh[finite].clone()
    n = x.numel()
    m = torch.full((n,), -0.0)
    hp = dict(HP, beta1=0.0)
    Z.zs_host_adamw_step(x, torch.float16, torch.zeros(n), m, torch.zeros(n), n, _hp(Z, hp), _scalars(Z, 1.0, 1.0, 0),
                         None, torch.bfloat16, 2)
    assert torch.equal(_bits(m), _bits(x.float()))


def test_host_threads_do_not_change_bits():
    Z = _z()
    g = torch.Generator().manual_seed(5)
    n = 1_000_037
    x = torch.randn(n, generator=g).mul(1e-3).to(torch.bfloat16)
    base = [torch.randn(n, generator=g) * 0.02, torch.randn(n, generator=g) * 1e-3, torch.rand(n, generator=g) * 1e-6]
    outs = []
    for threads in (1, 2, 7, 16):
        st = [b.clone() for b in base]
        out = torch.empty(n, dtype=torch.bfloat16)
        Z.zs_host_adamw_step(x, torch.bfloat16, *st, n, _hp(Z, HP), _scalars(Z, 1.0, 0.5, 9), out, torch.bfloat16,
                             threads)
        outs.append([_bits(t) for t in st] + [_bits(out)])
    for o in outs[1:]:
        assert all(torch.equal(a, b) for a, b in zip(o, outs[0]))


def test_host_step_overflow_and_invalid_arguments():
    Z = _z()
    n = 64
    x = torch.ones(n, dtype=torch.bfloat16)
    st = [torch.full((n,), 0.5), torch.zeros(n), torch.zeros(n)]
    before = [t.clone() for t in st]
    out = torch.full((n,), 7.0, dtype=torch.bfloat16)
    Z.zs_host_adamw_step(x, torch.bfloat16, *st, n, _hp(Z, HP), _scalars(Z, 1.0, 1.0, 0, overflow=1), out,
                         torch.bfloat16)
    assert all(torch.equal(a, b) for a, b in zip(st, before)) and bool((out == 7.0).all())
    bad = [
        dict(scalars=_scalars(Z, 3.0, 1.0, 0)),     # loss scale not a power of two
        dict(scalars=_scalars(Z, 1.0, 0.0, 0)),     # clip coefficient outside (0, 1]
        dict(scalars=_scalars(Z, 1.0, 1.5, 0)),
        dict(scalars=_scalars(Z, 1.0, 1.0, -1)),
        dict(hp=dict(HP, beta2=1.0)),
        dict(count=-1),
        dict(grad=None),
    ]
    for case in bad:
        kw = dict(grad=x, scalars=_scalars(Z, 1.0, 1.0, 0), hp=HP, count=n)
        kw.update(case)
        with pytest.raises(Z.ZsError) as e:
            Z.zs_host_adamw_step(kw["grad"], torch.bfloat16, *st, kw["count"], _hp(Z, kw["hp"]), kw["scalars"],
                                 out, torch.bfloat16)
        assert e.value.status == -1
    # zero elements: nothing to do, NULL arrays allowed
    Z.zs_host_adamw_step(None, torch.bfloat16, None, None, None, 0, _hp(Z, HP), _scalars(Z, 1.0, 1.0, 0), None,
                         torch.bfloat16)
