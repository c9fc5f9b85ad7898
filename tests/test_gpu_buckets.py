"""GPU parity of the bucketed pack (zs_pack_bucket, zs_bucket_range) against the oracle's
bucket functions, through the C ABI.

Bar: bit-exact.  Buckets are packed in shuffled order, alternating between two streams,
into a buffer that starts as garbage (or, for accumulation, as an earlier micro-step);
the result must equal the oracle's whole pack (or accumulate) bit for bit, and elements
outside the packed buckets must keep their garbage.
"""

import random
import zlib

import pytest
import torch

import oracle as O
from workloads import WORKLOADS, gen

pytestmark = pytest.mark.gpu


def _z():
    import zero_sharded_mixed_buffer_amd as Z
    Z.lib()
    return Z


def bits(x):
    return x.view({2: torch.int16, 4: torch.int32}[x.element_size()])


def _random_partition(n, k, rng):
    cuts = sorted(rng.sample(range(1, n), min(k, n - 1))) if n > 1 else []
    return list(zip([0] + cuts, cuts + [n]))


def _garbage(numel, dtype, dev, seed):
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    if dtype == torch.float32:
        return torch.randint(-2 ** 31, 2 ** 31 - 1, (numel,), generator=g, device=dev, dtype=torch.int32).view(dtype)
    return torch.randint(-2 ** 15, 2 ** 15 - 1, (numel,), generator=g, device=dev, dtype=torch.int16).view(dtype)


def _pack_buckets(Z, lay, ptrs, src_dt, flat, flat_dt, buckets, accumulate, streams):
    main = torch.cuda.current_stream()
    for s in streams:
        s.wait_stream(main)
    for i, (a, b) in enumerate(buckets):
        s = streams[i % len(streams)]
        Z.zs_pack_bucket(lay, ptrs, src_dt, flat, flat_dt, a, b, accumulate=accumulate, stream=s)
    for s in streams:
        main.wait_stream(s)
    torch.cuda.synchronize()


CASES = [("llama_mini", "model", False), ("llama_mini", "fp32", False), ("ragged_mini", "model", False),
         ("ragged_mini_a64", "fp32", False), ("moe_mini_dp4", "model", False), ("tiny", "fp32", False),
         ("qwen_mini_dp2", "model", True), ("ragged_mini", "fp32", True), ("moe_mini_dp4", "fp32", True),
         ("ragged_mini_a64", "model", True)]


@pytest.mark.parametrize("name,flat_kind,accumulate", CASES)
def test_buckets_in_any_order_equal_the_oracle_pack(name, flat_kind, accumulate):
    Z = _z()
    wl = WORKLOADS[name]
    dev = torch.device("cuda", 0)
    dt = gen.TORCH_DTYPE[wl.dtype]
    flat_dt = torch.float32 if flat_kind == "fp32" else dt
    numels = list(wl.numels)
    T = len(numels)
    rng = random.Random(zlib.crc32(f"{name}/{flat_kind}/{accumulate}".encode()))
    buckets = _random_partition(T, max(1, T // 4), rng)
    rng.shuffle(buckets)
    print(f"[case] buckets {name} flat={flat_dt} acc={accumulate} T={T} buckets={len(buckets)}", flush=True)
    lay = Z.zs_layout_create(numels, wl.dp_world, wl.dp_rank, wl.align)
    olay = O.plan_layout(numels, wl.dp_world, wl.dp_rank, wl.align)
    flat_numel, _, _ = Z.zs_layout_info(lay)
    assert flat_numel == olay.flat_numel
    for a, b in buckets:
        assert Z.zs_bucket_range(lay, a, b) == O.bucket_range(olay, a, b)
    grads = gen.make_grads(wl, 1, wl.init_scale, dev, with_faults=False)
    grads_cpu = [g.cpu() for g in grads]
    if accumulate:
        earlier = [g.cpu() for g in gen.make_grads(wl, 2, wl.init_scale, dev, with_faults=False)]
        start = O.pack(earlier, olay, flat_dt)
        want = O.accumulate(start, grads_cpu, olay)
        flat = start.to(dev)
    else:
        flat = _garbage(flat_numel, flat_dt, dev, 5)
        want = O.pack(grads_cpu, olay, flat_dt)
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    _pack_buckets(Z, lay, Z.pointer_table(grads, dev), dt, flat, flat_dt, buckets, accumulate, streams)
    assert torch.equal(bits(flat.cpu()), bits(want))
    Z.zs_layout_destroy(lay)


@pytest.mark.parametrize("name,size", [("ragged_mini", 3000), ("ragged_mini_a64", 5000), ("llama_mini", 200_000),
                                       ("moe_mini_dp4", 20_000)])
def test_planned_buckets_touch_only_their_ranges(name, size):
    """Buckets from zs_plan_buckets; every other one is packed into a garbage buffer: those
    ranges equal the oracle pack, everything else keeps its garbage bits."""
    Z = _z()
    wl = WORKLOADS[name]
    dev = torch.device("cuda", 0)
    dt = gen.TORCH_DTYPE[wl.dtype]
    numels = list(wl.numels)
    buckets = Z.zs_plan_buckets(numels, size)
    assert buckets == O.plan_buckets(numels, size)
    print(f"[case] planned buckets {name} size={size} buckets={len(buckets)}", flush=True)
    lay = Z.zs_layout_create(numels, wl.dp_world, wl.dp_rank, wl.align)
    olay = O.plan_layout(numels, wl.dp_world, wl.dp_rank, wl.align)
    grads = gen.make_grads(wl, 3, wl.init_scale, dev, with_faults=False)
    for flat_dt in (dt, torch.float32):
        flat = _garbage(olay.flat_numel, flat_dt, dev, 9)
        before = flat.cpu()
        chosen = buckets[::2]
        _pack_buckets(Z, lay, Z.pointer_table(grads, dev), dt, flat, flat_dt, chosen, False,
                      [torch.cuda.current_stream()])
        full = O.pack([g.cpu() for g in grads], olay, flat_dt)
        want = before.clone()
        for a, b in chosen:
            want = O.pack_bucket(want, [g.cpu() for g in grads], olay, a, b)
            lo, hi = O.bucket_range(olay, a, b)
            assert torch.equal(bits(want[lo:hi]), bits(full[lo:hi]))
        assert torch.equal(bits(flat.cpu()), bits(want))
    Z.zs_layout_destroy(lay)


def test_bucket_edge_cases():
    """Buckets made of empty tensors (an empty flat range), single-element tensors, a bucket
    ending in the tail padding, and misaligned bucket boundaries inside one 4096-element
    block; bad tensor ranges are rejected before anything runs."""
    Z = _z()
    dev = torch.device("cuda", 0)
    numels = [0, 1, 0, 4093, 3, 1, 0, 0, 8191, 2, 5000, 0]
    for align, d in ((1, 1), (64, 4), (8, 3)):
        lay = Z.zs_layout_create(numels, d, 0, align)
        olay = O.plan_layout(numels, d, 0, align)
        g = torch.Generator(device=dev)
        g.manual_seed(align)
        grads = [torch.randn(n, generator=g, device=dev).to(torch.bfloat16) for n in numels]
        for flat_dt in (torch.bfloat16, torch.float32):
            flat = _garbage(olay.flat_numel, flat_dt, dev, align)
            singles = [(t, t + 1) for t in range(len(numels))]
            random.Random(align).shuffle(singles)
            for a, b in singles:
                lo, hi = Z.zs_bucket_range(lay, a, b)
                assert (lo, hi) == O.bucket_range(olay, a, b)
            _pack_buckets(Z, lay, Z.pointer_table(grads, dev), torch.bfloat16, flat, flat_dt, singles, False,
                          [torch.cuda.Stream(), torch.cuda.Stream(), torch.cuda.Stream()])
            want = O.pack([x.cpu() for x in grads], olay, flat_dt)
            assert torch.equal(bits(flat.cpu()), bits(want))
        ptrs = Z.pointer_table(grads, dev)
        for a, b in ((3, 3), (-1, 2), (5, 13), (6, 4)):
            with pytest.raises(Z.ZsError) as e:
                Z.zs_pack_bucket(lay, ptrs, torch.bfloat16, flat, torch.float32, a, b)
            assert e.value.status == -1
        with pytest.raises(Z.ZsError):
            Z.zs_pack_bucket(lay, ptrs, torch.float32, flat, torch.float32, 0, 2)
        Z.zs_layout_destroy(lay)


def test_bucketed_step_equals_whole_pack_step():
    """The optimizer's bucket helpers: a step whose gradients were packed bucket by bucket
    (in backward order) leaves the same master, moments and parameters as one packed whole."""
    Z = _z()
    wl = WORKLOADS["llama_mini"]
    dev = torch.device("cuda", 0)
    p0 = gen.make_params(wl, dev)
    kw = dict(lr=1e-3, weight_decay=0.01, max_norm=0.0)  # no clipping: the two sums of squares
    # are taken in different orders (fused into the pack, or over the shard afterwards)
    a = Z.ZeroShardedAdamW([p.clone() for p in p0], **kw)
    b = Z.ZeroShardedAdamW([p.clone() for p in p0], **kw)
    for step in range(1, 4):
        grads = gen.make_grads(wl, step, 1.0, dev, with_faults=False)
        a.step(grads)
        for bucket in b.buckets(300_000):
            b.pack_bucket(grads, bucket)
        b.check()
        b.norm()
        b.update()
    torch.cuda.synchronize()
    for x, y in ((a.master, b.master), (a.m, b.m), (a.v, b.v)):
        assert torch.equal(bits(x), bits(y))
    assert all(torch.equal(bits(x), bits(y)) for x, y in zip(a.params, b.params))
    a.close()
    b.close()
