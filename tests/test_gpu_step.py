"""The single-call step zs_step (ZeroShardedAdamW.step with one rank and one micro-step).

zs_step enqueues the kernels of zs_pack (fused check), zs_grad_norm, zs_adamw_step and
zs_scaler_update.  Checked here on both sides of 256 tiles (1,048,576 elements), below
which the AdamW kernel runs four workgroups per tile, and of 4096 pack blocks (16,777,216
elements), where the fold of the partial sums switches from one finalize workgroup to two
levels:
- parity with the CPU oracle, at the bar of the other parity tests;
- bit-identity with the four-call sequence, step by step, through overflow skips and
  scale growth;
- replay in a HIP graph.
"""

import dataclasses
import math

import pytest
import torch

from workloads import WORKLOADS, gen
from workloads.configs import Workload

pytestmark = pytest.mark.gpu

FOLD_ELEMS = 4096 * 4096  # the largest pack whose partial sums one finalize workgroup folds
SPLIT_ELEMS = 256 * 4096  # the largest shard whose AdamW runs four workgroups per tile


def _z():
    import zero_sharded_mixed_buffer_amd as Z
    Z.lib()
    return Z


def _sized(name, shapes, dtype="fp16", steps=5, fault_step=2, growth=2, seed=40):
    """A workload of the given shapes: fp16 with a dynamic scale, one +inf at fault_step and
    a growth interval short enough that the scale also doubles within the run."""
    numels = [math.prod(s) for _, s in shapes]
    faults = {fault_step: [(len(numels) - 1, numels[-1] - 1, math.inf)]} if fault_step else {}
    dynamic = dtype == "fp16"
    return Workload(name, tuple(shapes), dtype, 1, 0, dynamic, 2.0 ** 12 if dynamic else 1.0, 1e-3, 0.02, steps,
                    seed, faults=faults, growth_interval=growth)


def _at_one_level():
    return _sized("at_one_level", [("w", (4096, 4095)), ("b", (4096,))])


def _over_one_level():
    return _sized("over_one_level", [("w", (4096, 4096)), ("b", (1000,)), ("c", (7,))], seed=41)


def _at_split():  # 256 tiles of 4096: the largest shard whose AdamW runs four workgroups per tile
    return _sized("at_split", [("w", (1024, 1000)), ("b", (24576,))], seed=42)


def _over_split():
    return _sized("over_split", [("w", (1024, 1000)), ("b", (24577,))], seed=43)


CASES = {
    "tiny": lambda: WORKLOADS["tiny"],
    "llama_mini": lambda: WORKLOADS["llama_mini"],
    "ragged_mini": lambda: WORKLOADS["ragged_mini"],
    "ragged_mini_a64": lambda: WORKLOADS["ragged_mini_a64"],
    "at_split": _at_split,
    "over_split": _over_split,
    "at_one_level": _at_one_level,
    "over_one_level": _over_one_level,
}


@pytest.mark.parametrize("name", list(CASES))
def test_step_parity_with_oracle(name):
    from harness import run_parity
    _z()
    wl = CASES[name]()
    assert (wl.n_elems <= FOLD_ELEMS) == (name != "over_one_level")
    if "split" in name:
        assert (wl.n_elems <= SPLIT_ELEMS) == (name == "at_split")
    print(f"[case] zs_step parity {name} N={wl.n_elems} T={len(wl.numels)} steps={wl.steps}", flush=True)
    rep = run_parity(wl, use_step=True)
    print(f"[parity] {name}: master_err={rep.master_err:.3e} m_err={rep.m_err:.3e} v_err={rep.v_err:.3e} "
          f"scales={[s.scale_gpu for s in rep.steps]} skips={[s.overflow_gpu for s in rep.steps]}", flush=True)
    assert [s.step for s in rep.steps if s.overflow_gpu] == sorted(wl.faults)


def _pair(Z, wl, dev, **extra):
    p0 = gen.make_params(wl, dev)
    kw = dict(dynamic_loss_scale=wl.dynamic, init_scale=wl.init_scale, growth_interval=wl.growth_interval, **extra)
    return (Z.ZeroShardedAdamW([p.clone() for p in p0], **kw), Z.ZeroShardedAdamW([p.clone() for p in p0], **kw))


def _sequence_step(opt, grads):
    opt.pack(grads)
    opt.norm()
    opt.update()


def _assert_same(a, b, tag):
    from harness import bits
    for x, y, what in ((a.master, b.master, "master"), (a.m, b.m, "m"), (a.v, b.v, "v"), (a.flat, b.flat, "flat")):
        assert torch.equal(bits(x), bits(y)), f"{tag}: {what}"
    assert all(torch.equal(bits(x), bits(y)) for x, y in zip(a.params, b.params)), f"{tag}: params"
    sa, sb = a.read_state(), b.read_state()
    assert sa.keys() == sb.keys()
    for k in sa:  # the same value, or NaN on both sides (the norm of an overflowed step)
        same = sa[k] == sb[k] or (isinstance(sa[k], float) and math.isnan(sa[k]) and math.isnan(sb[k]))
        assert same, f"{tag}: state {k} {sa[k]} != {sb[k]}"


@pytest.mark.parametrize("name", ["tiny", "ragged_mini", "at_split", "over_split", "at_one_level", "over_one_level"])
def test_step_bit_identical_to_the_call_sequence(name):
    Z = _z()
    dev = torch.device("cuda", 0)
    wl = CASES[name]()
    if name in ("tiny", "ragged_mini"):  # a short growth interval so the run doubles the scale too
        wl = dataclasses.replace(wl, growth_interval=2)
    one, seq = _pair(Z, wl, dev)
    scales = []
    for step in range(1, wl.steps + 1):
        print(f"[case] {name} step {step}", flush=True)
        grads = gen.make_grads(wl, step, one.read_state()["loss_scale"], dev)
        one.step(grads)
        _sequence_step(seq, grads)
        torch.cuda.synchronize()
        _assert_same(one, seq, f"{name} step {step}")
        scales.append(one.read_state()["loss_scale"])
    st = one.read_state()
    assert st["skipped_total"] == len(wl.faults) and st["step_t"] == wl.steps - len(wl.faults)
    if wl.dynamic:
        assert len(set(scales)) > 1, scales  # the scale moved: backoff and growth both ran
    one.close()
    seq.close()


@pytest.mark.parametrize("name,variant", [("llama_mini", "no_decay"), ("ragged_mini", "no_decay"),
                                          ("tiny", "bf16_params"), ("llama_mini", "fp16_grads")])
def test_step_variants_bit_identical_to_the_call_sequence(name, variant):
    """zs_step with tensors that take no weight decay, and with gradient and parameter dtypes
    that differ, against the four calls on the same optimizer settings."""
    Z = _z()
    dev = torch.device("cuda", 0)
    wl = CASES[name]()
    extra = {}
    if variant == "no_decay":
        extra["no_decay"] = "1d" if name == "llama_mini" else [i % 3 == 0 for i in range(len(wl.numels))]
    one, seq = _pair(Z, wl, dev, **extra)
    if variant != "no_decay":  # parameters in the other 2-byte dtype, gradients as the workload draws them
        pdt = torch.bfloat16 if variant == "bf16_params" else torch.float16
        gdt = gen.TORCH_DTYPE[wl.dtype] if variant == "bf16_params" else torch.float16
        p0 = [p.to(pdt) for p in gen.make_params(wl, dev)]
        kw = dict(dynamic_loss_scale=wl.dynamic or gdt == torch.float16,
                  init_scale=wl.init_scale if wl.dynamic else 2.0 ** 12, growth_interval=2, grad_dtype=gdt)
        one.close()
        seq.close()
        one = Z.ZeroShardedAdamW([p.clone() for p in p0], **kw)
        seq = Z.ZeroShardedAdamW([p.clone() for p in p0], **kw)
    for step in range(1, 5):
        print(f"[case] {name} {variant} step {step}", flush=True)
        scale = one.read_state()["loss_scale"]
        grads = [g.to(one.model_grad_dtype) for g in gen.make_grads(wl, step, scale, dev)]
        one.step(grads)
        _sequence_step(seq, grads)
        torch.cuda.synchronize()
        _assert_same(one, seq, f"{name} {variant} step {step}")
    one.close()
    seq.close()


@pytest.mark.parametrize("name", ["tiny", "over_one_level"])
def test_step_graph_replays_through_skips_and_growth(name):
    """The captured single call replayed five times, one replay overflowing, each replay
    compared with the call sequence run eagerly on a second optimizer; eager work and
    synchronisations sit between the replays."""
    Z = _z()
    dev = torch.device("cuda", 0)
    wl = dataclasses.replace(CASES[name](), growth_interval=2)
    graph_opt, eager_opt = _pair(Z, wl, dev)
    grads = gen.make_grads(wl, 1, wl.init_scale, dev, with_faults=False)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        graph_opt.step(grads)
    torch.cuda.current_stream().wait_stream(s)
    _sequence_step(eager_opt, grads)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        graph_opt.step(grads)
    torch.cuda.synchronize()
    for replay in range(5):
        scale = eager_opt.read_state()["loss_scale"]
        new = gen.make_grads(wl, 10 + replay, scale, dev, with_faults=False)
        if replay == 2:
            new[0].view(-1)[0] = math.inf
        for dst, src in zip(grads, new):
            dst.copy_(src)
        g.replay()
        _sequence_step(eager_opt, grads)
        torch.cuda.synchronize()
        _assert_same(graph_opt, eager_opt, f"{name} replay {replay}")
    st = graph_opt.read_state()
    assert st["skipped_total"] == 1 and st["step_t"] == 5  # the warm-up step and four applied replays
    graph_opt.close()
    eager_opt.close()


def test_step_rejects_bad_arguments():
    Z = _z()
    dev = torch.device("cuda", 0)
    wl = WORKLOADS["llama_mini"]
    opt = Z.ZeroShardedAdamW(gen.make_params(wl, dev))
    grads = gen.make_grads(wl, 1, 1.0, dev)
    gp = opt._grad_table(grads)
    args = dict(layout=opt.layout, grad_ptrs=gp, grad_dtype=torch.bfloat16, flat=opt.flat, state=opt.state,
                hp=opt.hp, master=opt.master, m=opt.m, v=opt.v, param_ptrs=opt.param_ptrs,
                param_dtype=torch.bfloat16)
    for bad in (dict(grad_ptrs=None), dict(flat=None), dict(param_ptrs=None), dict(master=None),
                dict(grad_dtype=torch.float32), dict(param_dtype=torch.float32), dict(flat=opt.flat[1:])):
        with pytest.raises(Z.ZsError):
            Z.zs_step(**{**args, **bad})
    lay2 = Z.zs_layout_create(wl.numels, 2, 0, 1)
    st2 = Z.zs_state_create(lay2, Z.state_host(1.0, 1.0, False, 1000))
    with pytest.raises(Z.ZsError, match="dp_world"):
        Z.zs_step(**{**args, "layout": lay2, "state": st2})
    Z.zs_state_destroy(st2)
    Z.zs_layout_destroy(lay2)
    # tensors the kernels would misread or fault on are refused before any launch
    with pytest.raises(ValueError, match="lives on cpu"):
        opt.step([g.cpu() for g in grads])
    with pytest.raises(ValueError, match="gradients must be"):
        opt.step([g.float() for g in grads])
    params = gen.make_params(wl, dev)
    with pytest.raises(ValueError, match="one dtype"):
        Z.ZeroShardedAdamW(params[:-1] + [params[-1].half()])
    with pytest.raises(ValueError, match="lives on cpu"):
        Z.ZeroShardedAdamW(params[:-1] + [params[-1].cpu()])
    with pytest.raises(ValueError, match="bf16 or fp16"):
        Z.ZeroShardedAdamW([p.float() for p in params])
    torch.cuda.synchronize()
    assert opt.read_state()["step_t"] == 0  # nothing was enqueued
    opt.close()
