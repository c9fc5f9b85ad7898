"""The bandwidth yardsticks of include/zs_probe.h do what their byte counts claim: the mix
probe moves every element of its eight streams (rotating p, m, v and copying g's bits to
out), the copy copies, the write zeroes, and sizes that are not whole workgroups are
refused before anything runs."""

import pytest
import torch

pytestmark = pytest.mark.gpu


def _z():
    import zero_sharded_mixed_buffer_amd as Z
    Z.lib()
    return Z


def test_probes_move_every_byte():
    Z = _z()
    dev = torch.device("cuda", 0)
    n = 3 * 4096
    gen = torch.Generator(device=dev).manual_seed(5)
    g = torch.randn(n, generator=gen, device=dev).to(torch.bfloat16)
    p, m, v = (torch.randn(n, generator=gen, device=dev) for _ in range(3))
    p0, m0, v0 = p.clone(), m.clone(), v.clone()
    out = torch.zeros(n, dtype=torch.bfloat16, device=dev)
    print(f"[case] probes n={n}", flush=True)
    Z.zs_probe_mix(g, p, m, v, out, n)
    torch.cuda.synchronize()
    assert torch.equal(p, m0) and torch.equal(m, v0) and torch.equal(v, p0)
    assert torch.equal(out.view(torch.int16), g.view(torch.int16))
    nb = n * 4
    Z.zs_probe_copy(p0, m, nb)
    torch.cuda.synchronize()
    assert torch.equal(m, p0)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    Z.zs_probe_read(p0, nb, sink)
    Z.zs_probe_write(v, nb)
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(v)) == 0


def test_probes_refuse_partial_workgroups():
    Z = _z()
    dev = torch.device("cuda", 0)
    a = torch.zeros(8192, device=dev)
    b = torch.zeros(8192, device=dev)
    h = torch.zeros(8192, dtype=torch.bfloat16, device=dev)
    for call in (lambda: Z.zs_probe_mix(h, a, b, a, h, 4095), lambda: Z.zs_probe_mix(h, a, b, a, h, 0),
                 lambda: Z.zs_probe_copy(a, b, 16384 + 16), lambda: Z.zs_probe_write(a, -16384),
                 lambda: Z.zs_probe_read(a, 16384, None), lambda: Z.zs_probe_copy(a[1:], b, 16384)):
        with pytest.raises(Z.ZsInvalidArgument):
            call()
    torch.cuda.synchronize()
