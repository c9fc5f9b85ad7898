"""Re-entrancy of the library: several host threads, each with its own optimizer (layout,
state, buffers) and its own stream, step at the same time on one GPU.  ctypes releases the
interpreter lock around every library call, so the calls really overlap.  Each thread's
results must equal the same steps taken alone, bit for bit: the library keeps no shared
state beyond the per-thread error message and the host thread pool (two of the threads
run the offloaded update, which takes turns on that pool)."""

import threading

import pytest
import torch

from workloads import WORKLOADS, gen

pytestmark = pytest.mark.gpu


def _bits(x):
    return x.contiguous().view(torch.int16) if x.element_size() == 2 else x.contiguous().view(torch.int32)


def _run(Z, wl, steps, stream, offload=False):
    dev = torch.device("cuda", 0)
    with torch.cuda.stream(stream):
        params = gen.make_params(wl, dev)
        opt = Z.ZeroShardedAdamW(params, dynamic_loss_scale=wl.dynamic, init_scale=wl.init_scale, align=wl.align,
                                 offload=offload, offload_chunk=65_537)
        for s in range(1, steps + 1):
            grads = gen.make_grads(wl, s, opt.read_state(stream)["loss_scale"], dev)
            opt.step(grads, stream=stream)
        stream.synchronize()
        out = ([t.detach().cpu() for t in (opt.master, opt.m, opt.v)], [p.cpu() for p in opt.params],
               opt.read_state(stream))
        opt.close()
    return out


def test_threads_with_their_own_optimizers_step_concurrently():
    import zero_sharded_mixed_buffer_amd as Z
    Z.lib()
    jobs = [("tiny", True), ("llama_mini", False), ("ragged_mini", False), ("ragged_mini_a64", True)]
    print(f"[case] concurrent threads: {jobs}", flush=True)
    steps = 6
    alone = [_run(Z, WORKLOADS[n], steps, torch.cuda.Stream(), off) for n, off in jobs]
    results, errors = [None] * len(jobs), []

    def work(i, name, off):
        try:
            results[i] = _run(Z, WORKLOADS[name], steps, torch.cuda.Stream(), off)
        except Exception as e:  # reported below; a thread cannot fail the test itself
            errors.append((name, repr(e)))

    threads = [threading.Thread(target=work, args=(i, n, off), daemon=True) for i, (n, off) in enumerate(jobs)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a thread did not finish"
    assert not errors, errors
    for (name, _), a, b in zip(jobs, alone, results):
        for x, y in zip(a[0], b[0]):
            assert torch.equal(_bits(x), _bits(y)), name
        assert all(torch.equal(_bits(x), _bits(y)) for x, y in zip(a[1], b[1])), name
        assert a[2]["step_t"] == b[2]["step_t"] and a[2]["loss_scale"] == b[2]["loss_scale"], name
