"""The C ABI from a C++ program with no Python and no torch (tests/c/abi_gpu.cpp, built by
the package build): it allocates device memory and a stream with the HIP runtime, runs
zs_step for every step (or, in flat mode, zs_step_flat over one gradient buffer and one
parameter buffer), and writes its results, which are compared here with the oracle run on
the same inputs.  Bar: the loss-scale sequence and skip count exactly; master, m and
v within the 1e-5 relative contract; parameters equal to the cast of the program's master
bit for bit."""

import os
import struct
import subprocess

import pytest
import torch

import oracle as O
from workloads import WORKLOADS, gen

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(__file__), "c", "abi_gpu")


@pytest.mark.parametrize("name,mode", [("tiny", "tensors"), ("llama_mini", "tensors"), ("ragged_mini", "tensors"),
                                       ("tiny", "flat"), ("ragged_mini", "flat")])
def test_c_program_runs_the_step_against_the_oracle(name, mode, tmp_path):
    from harness import REL_TOL, bits, rel_err
    assert os.path.exists(EXE), f"{EXE} is missing: python -m zero_sharded_mixed_buffer_amd.build builds it"
    wl = WORKLOADS[name]
    dt = gen.TORCH_DTYPE[wl.dtype]
    hp = wl.hparams
    params = gen.make_params(wl, "cpu")
    ref = O.OracleRank(wl.numels, 1, 0, params, O.OracleScaler(wl.init_scale, 1.0, wl.dynamic, wl.growth_interval),
                       hp)
    # The oracle runs first: each step's gradients are drawn at the loss scale of that step.
    steps = []
    for step in range(1, wl.steps + 1):
        g = gen.make_grads(wl, step, ref.scaler.loss_scale, "cpu")
        steps.append(g)
        ref.step(O.shard_of(O.pack(g, ref.layout), ref.layout))
    code = 0 if dt == torch.bfloat16 else 1
    inp, out = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(inp, "wb") as f:
        f.write(struct.pack("<iii", len(wl.numels), code, wl.steps))
        f.write(struct.pack(f"<{len(wl.numels)}q", *wl.numels))
        f.write(struct.pack("<6d", hp["lr"], hp["beta1"], hp["beta2"], hp["eps"], hp["weight_decay"], hp["max_norm"]))
        f.write(struct.pack("<ddii", wl.init_scale, 1.0, int(wl.dynamic), wl.growth_interval))
        for tensors in [params] + steps:
            for t in tensors:
                f.write(t.contiguous().view(torch.int16).numpy().tobytes())
    print(f"[case] C program {name}: {len(wl.numels)} tensors, {wl.n_elems} elements, {wl.steps} steps", flush=True)
    res = subprocess.run([EXE, str(inp), str(out), mode], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    data = out.read_bytes()
    # zs_state_host: 2 doubles, 2 int32, 3 int64, 2 int32, 4 doubles
    fmt = "<ddiiqqqiidddd"
    st = struct.unpack_from(fmt, data, 0)
    loss_scale, step_t, skipped = st[0], st[5], st[6]
    assert loss_scale == ref.scaler.loss_scale and step_t == ref.scaler.step_t
    assert skipped == ref.scaler.skipped_total == len(wl.faults)
    S = ref.layout.shard_numel
    off = struct.calcsize(fmt)
    arrays = []
    for _ in range(3):
        arrays.append(torch.frombuffer(bytearray(data[off:off + 4 * S]), dtype=torch.float32))
        off += 4 * S
    for got, want, what in zip(arrays, (ref.master, ref.m, ref.v), ("master", "m", "v")):
        err = rel_err(got, want)
        assert err <= REL_TOL, f"{what}: {err}"
    p_got = torch.frombuffer(bytearray(data[off:]), dtype=torch.int16)
    assert p_got.numel() == wl.n_elems
    assert torch.equal(p_got, bits(O.cast_to(arrays[0], dt)))
    print(f"[c_abi] {name}: {res.stdout.strip()}; scale {loss_scale}, step_t {step_t}, skipped {skipped}", flush=True)
