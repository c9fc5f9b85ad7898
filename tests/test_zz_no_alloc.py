"""zs_step_flat_noalloc, the allocation-free variant of zs_step_flat (for callers that cannot
allocate device memory), against zs_step_flat itself through the C ABI: bit-identical master,
m, v, parameter buffer and state on consecutive calls whose sizes shrink (the fixed scratch
keeps the earlier, larger call's contents), including a skipped step; the call changes no
free device memory; sizes beyond the scratch are refused."""

import ctypes

import pytest
import torch

pytestmark = pytest.mark.gpu


def _z():
    import zero_sharded_mixed_buffer_amd as Z
    Z.lib()
    return Z


def _state_to_device(Z, hs, dev):
    raw = ctypes.string_at(ctypes.addressof(hs), ctypes.sizeof(hs))
    return torch.tensor(list(raw), dtype=torch.uint8).to(dev)


def _state_from_device(Z, t):
    return Z.StateHost.from_buffer_copy(t.cpu().numpy().tobytes()).as_dict()


def _bits(x):
    return x.view(torch.int32 if x.element_size() == 4 else torch.int16)


@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
def test_noalloc_step_equals_zs_step_flat_on_shrinking_calls(dtype):
    Z = _z()
    dev = torch.device("cuda", 0)
    fp16 = dtype == torch.float16
    scale0 = 2.0 ** 16 if fp16 else 1.0
    hp = Z.hparams(1e-3, 0.9, 0.999, 1e-8, 0.01, 1.0)
    gen = torch.Generator(device=dev).manual_seed(3)
    warm = False
    for n in (3_000_017, 70_001, 5):  # each call smaller than the one before it
        print(f"[case] noalloc {dtype} n={n}", flush=True)
        hs0 = Z.state_host(scale0, 1.0, fp16, 2)  # growth every 2 applied steps
        lay = Z.zs_layout_create([n], 1, 0, 1)
        st = Z.zs_state_create(lay, hs0)
        st_dev = _state_to_device(Z, hs0, dev)
        p0 = (torch.randn(n, generator=gen, device=dev) * 0.02).to(dtype)
        bufs = {}
        for side in ("ref", "noalloc"):
            bufs[side] = dict(master=p0.float(), m=torch.zeros(n, device=dev), v=torch.zeros(n, device=dev),
                              out=torch.zeros(n, dtype=dtype, device=dev))
        scale = scale0
        for step in range(1, 6):
            g = (torch.randn(n, generator=gen, device=dev) * 1e-2 * scale).to(dtype)
            if step == 3:
                g[n // 2] = float("inf")  # a skipped step: the scale halves
            b = bufs["ref"]
            Z.zs_step_flat(lay, g, dtype, st, hp, b["master"], b["m"], b["v"], b["out"], dtype)
            b = bufs["noalloc"]
            if warm:
                torch.cuda.synchronize()
                free0 = torch.cuda.mem_get_info()[0]
            Z.zs_step_flat_noalloc(g, dtype, n, st_dev, hp, b["master"], b["m"], b["v"], b["out"], dtype)
            torch.cuda.synchronize()
            if warm:
                assert torch.cuda.mem_get_info()[0] == free0, "the allocation-free step changed free device memory"
            warm = True
            want = Z.zs_state_read(st).as_dict()
            got = _state_from_device(Z, st_dev)
            assert got == want, (n, step, got, want)
            for k in ("master", "m", "v", "out"):
                a, r = bufs["noalloc"][k].cpu(), bufs["ref"][k].cpu()
                assert torch.equal(_bits(a), _bits(r)), (n, step, k)
            scale = want["loss_scale"]
        assert want["skipped_total"] == 1 and want["step_t"] == 4
        if fp16:
            assert want["loss_scale"] == 2.0 ** 17  # doubled after steps 1-2, halved at 3, doubled after 4-5
        Z.zs_state_destroy(st)
        Z.zs_layout_destroy(lay)


def test_noalloc_step_refuses_sizes_beyond_its_scratch():
    Z = _z()
    dev = torch.device("cuda", 0)
    hp = Z.hparams()
    st_dev = _state_to_device(Z, Z.state_host(1.0, 1.0, False), dev)
    x = torch.zeros(4096, dtype=torch.bfloat16, device=dev)
    f = torch.zeros(4096, device=dev)
    args = [x, torch.bfloat16, 4096, st_dev, hp, f, f.clone(), f.clone(), x.clone(), torch.bfloat16]
    for k, bad in ((2, 2 ** 33 + 1), (2, 0), (3, None), (0, x[1:])):
        call = list(args)
        call[k] = bad
        with pytest.raises(Z.ZsInvalidArgument):
            Z.zs_step_flat_noalloc(*call)
    torch.cuda.synchronize()
    assert _state_from_device(Z, st_dev)["step_t"] == 0  # nothing ran
