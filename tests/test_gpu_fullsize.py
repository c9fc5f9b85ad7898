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
    ("llama3_8b", 4),
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
