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
