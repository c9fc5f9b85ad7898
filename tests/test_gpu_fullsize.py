"""Full-size parity: the workloads at their real sizes, in the launch configuration bench.py
times, against the oracle on sampled shard windows plus every step's global flag, norm and
scaler state (computed by the oracle from all gradients)."""

import time

import pytest

from workloads import WORKLOADS

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,steps", [
    ("qwen3_0.6b_dp2", 10),
    ("moe_3.4b_dp4", 10),
    ("ragged_20k", 20),
    ("llama3_8b", 10),
])
def test_fullsize_sampled_parity(name, steps):
    import zero_sharded_mixed_buffer_amd as Z
    from harness import run_parity_sampled
    Z.lib()
    wl = WORKLOADS[name]
    print(f"[case] fullsize {name}: {len(wl.numels)} tensors, N={wl.n_elems}, d={wl.dp_world}, steps={steps}",
          flush=True)
    t0 = time.time()
    worst, ndiff, wins = run_parity_sampled(wl, steps=steps, log=lambda s: print(s, flush=True))
    print(f"[fullsize] {name}: {len(wins)} windows, worst={worst}, ndiff={ndiff}, {time.time() - t0:.1f} s",
          flush=True)


@pytest.mark.parametrize("name,steps", [("llama3_8b", 2), ("ragged_20k", 3)])
def test_fullsize_flat_views_sampled_parity(name, steps):
    """The flat-views step at full size: gradients written through the .grad views of the
    gradient buffer, one zs_step_flat call per step (check, norm, AdamW into the parameter
    buffer), against the oracle on sampled windows."""
    import zero_sharded_mixed_buffer_amd as Z
    from harness import run_parity_sampled
    Z.lib()
    wl = WORKLOADS[name]
    print(f"[case] fullsize flat views {name}: N={wl.n_elems}, steps={steps}", flush=True)
    t0 = time.time()
    worst, ndiff, wins = run_parity_sampled(wl, steps=steps, log=lambda s: print(s, flush=True), n_random=16,
                                            views=True)
    print(f"[fullsize] flat views {name}: {len(wins)} windows, worst={worst}, ndiff={ndiff}, "
          f"{time.time() - t0:.1f} s", flush=True)


def test_tensor_beyond_int32_element_indices():
    """One tensor of 2^31 + 4099 elements between two small ones: element indices above 2^31
    and fp32 byte offsets above 2^32 in every array.  Sampled windows sit across those
    boundaries (elements 2^30 and 2^31 of the shard) and at the ends; two steps."""
    import math
    import zero_sharded_mixed_buffer_amd as Z
    from harness import run_parity_sampled
    from workloads.configs import Workload
    Z.lib()
    shapes = (("a", (3,)), ("big", (2 ** 31 + 4099,)), ("c", (5,)))
    wl = Workload("beyond_int32", shapes, "bf16", 1, 0, False, 1.0, 1e-3, 0.02, 2, 77)
    print(f"[case] fullsize beyond_int32: N={wl.n_elems}", flush=True)
    t0 = time.time()
    centres = (2 ** 30, 2 ** 31, 2 ** 31 + 3, 2 ** 32 // 3)
    worst, ndiff, wins = run_parity_sampled(wl, log=lambda s: print(s, flush=True), centres=centres, n_random=8)
    assert any(a < 2 ** 31 < b for a, b in wins) and wl.n_elems > 2 ** 31 and not math.isnan(worst["master"])
    print(f"[fullsize] beyond_int32: {len(wins)} windows, worst={worst}, ndiff={ndiff}, {time.time() - t0:.1f} s",
          flush=True)


@pytest.mark.parametrize("name,flat_kind", [("llama3_8b", "model"), ("llama3_8b", "fp32"), ("ragged_20k", "model")])
def test_fullsize_bucketed_pack(name, flat_kind):
    """The full-size gradient list packed in 5e8-element buckets (the pages' reduce_bucket_size),
    in backward order, into a garbage buffer; sampled windows around every bucket boundary
    and at random places equal the oracle's pack of those windows bit for bit, and the
    whole buffer equals the single-launch pack bit for bit."""
    import random

    import torch

    import oracle as O
    import zero_sharded_mixed_buffer_amd as Z
    from workloads import gen
    Z.lib()
    wl = WORKLOADS[name]
    dev = torch.device("cuda", 0)
    dt = gen.TORCH_DTYPE[wl.dtype]
    flat_dt = torch.float32 if flat_kind == "fp32" else dt
    numels = list(wl.numels)
    buckets = Z.zs_plan_buckets(numels, 500_000_000)
    assert buckets == O.plan_buckets(numels, 500_000_000)
    print(f"[case] fullsize buckets {name} flat={flat_dt}: {len(buckets)} buckets", flush=True)
    lay = Z.zs_layout_create(numels, wl.dp_world, wl.dp_rank, wl.align)
    olay = O.plan_layout(numels, wl.dp_world, wl.dp_rank, wl.align)
    grads = gen.make_grads(wl, 1, wl.init_scale, dev, with_faults=False)
    ptrs = Z.pointer_table(grads, dev)
    ibits = torch.int32 if flat_dt == torch.float32 else torch.int16
    flat = torch.full((olay.flat_numel,), -1, dtype=ibits, device=dev).view(flat_dt)  # NaN bits
    for a, b in buckets:
        Z.zs_pack_bucket(lay, ptrs, dt, flat, flat_dt, a, b)
    torch.cuda.synchronize()
    # windows: both sides of every bucket boundary, the ends, random places
    W = 1 << 14
    starts = set()
    for a, b in buckets:
        lo, hi = O.bucket_range(olay, a, b)
        for edge in (lo, hi):
            starts.add(min(max(edge - W // 2, 0), olay.flat_numel - W))
    rng = random.Random(11)
    starts.update(rng.randrange(0, olay.flat_numel - W) for _ in range(24))
    for s0 in sorted(starts):
        want = torch.zeros(W, dtype=flat_dt)
        for t, off, n in zip(grads, olay.offsets, olay.numels):
            x, y = max(off, s0), min(off + n, s0 + W)
            if x < y:
                want[x - s0:y - s0] = t.view(-1)[x - off:y - off].cpu().to(flat_dt)
        got = flat[s0:s0 + W].cpu()
        assert torch.equal(got.view(ibits), want.view(ibits)), f"window at {s0}"
    whole = torch.empty_like(flat)
    Z.zs_pack(lay, ptrs, dt, whole, flat_dt, whole_flat=True)
    torch.cuda.synchronize()
    assert torch.equal(whole.view(ibits), flat.view(ibits))
    print(f"[fullsize] buckets {name} flat={flat_dt}: {len(starts)} windows equal", flush=True)
    del whole, flat, grads
    Z.zs_layout_destroy(lay)
