"""GPU parity of tensors without weight decay (zs_layout_set_no_decay) against the oracle's
second parameter group, through the C ABI, on the device update and on the offloaded one.

Same bar as the other parity tests: bit-exact buffer, flags, skips, scale sequence and
scatter-back; master / m / v within the 1e-5 relative contract (bit-identical in practice).
"""

import random

import pytest
import torch

from workloads import WORKLOADS

pytestmark = pytest.mark.gpu


def _z():
    import zero_sharded_mixed_buffer_amd as Z
    Z.lib()
    return Z


def _flags(wl, kind):
    if kind == "1d":  # biases and normalisation weights
        return [len(shape) <= 1 for _, shape in wl.shapes]
    rng = random.Random(len(wl.numels))
    return [rng.random() < 0.5 for _ in wl.numels]


@pytest.mark.parametrize("name,kind,offload", [
    ("llama_mini", "1d", False), ("ragged_mini", "random", False), ("ragged_mini_a64", "random", False),
    ("moe_mini_dp4", "1d", False), ("qwen_mini_dp2", "random", False), ("tiny", "1d", False),
    ("llama_mini", "1d", True), ("ragged_mini", "random", True), ("moe_mini_dp4", "random", True),
])
def test_no_decay_parity(name, kind, offload):
    from harness import run_parity
    _z()
    wl = WORKLOADS[name]
    flags = _flags(wl, kind)
    steps = min(wl.steps, 6)
    print(f"[case] no-decay {name} {kind} offload={offload}: {sum(flags)} of {len(flags)} tensors", flush=True)
    rep = run_parity(wl, steps=steps, no_decay=flags, offload=offload, offload_chunk=70_001)
    print(f"[no-decay] {name}: diff(master,m,v)=({rep.n_master_diff},{rep.n_m_diff},{rep.n_v_diff}) "
          f"master_err={rep.master_err:.3e}", flush=True)


def test_no_decay_changes_only_the_flagged_tensors():
    """Zero gradients: flagged tensors keep their parameters bit for bit, the others decay,
    and clearing the table makes every tensor decay again."""
    Z = _z()
    dev = torch.device("cuda", 0)
    numels = [5000, 3, 4096, 77, 10000]
    flags = [False, True, True, False, True]
    g = torch.Generator(device=dev)
    g.manual_seed(4)
    params = [torch.randn(n, generator=g, device=dev).mul(0.02).to(torch.bfloat16) for n in numels]
    before = [p.clone() for p in params]
    opt = Z.ZeroShardedAdamW(params, lr=0.1, weight_decay=0.5, max_norm=0.0, no_decay=flags)
    zeros = [torch.zeros(n, dtype=torch.bfloat16, device=dev) for n in numels]
    opt.step(zeros)
    torch.cuda.synchronize()
    for p, b, f in zip(params, before, flags):
        assert torch.equal(p, b) == f
    Z.zs_layout_set_no_decay(opt.layout, None)
    snap = [p.clone() for p in params]
    opt.step(zeros)
    torch.cuda.synchronize()
    assert all(not torch.equal(p, b) for p, b in zip(params, snap))
    with pytest.raises(Z.ZsError) as e:
        Z.zs_layout_set_no_decay(opt.layout, flags[:3])
    assert e.value.status == -1
    opt.close()
