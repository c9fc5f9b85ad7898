"""bench.py's command line on the CPU: more than one GPU is refused with a message (this
library measures one GPU's share of the step), before anything touches a device."""

import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_several_gpus():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120, cwd=ROOT)
    assert res.returncode == 2
    msg = json.loads(res.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"] or "one MI355X" in msg["error"]


def test_fault_schedules_for_longer_runs():
    """bench.py --faults draws a workload's fault schedule for the run's length: the workload's
    own schedule for its own step count, the same kind of draw for other lengths, every
    position inside its tensor."""
    sys.path.insert(0, ROOT)
    from workloads import WORKLOADS
    for name in ("moe_3.4b_dp4", "ragged_20k", "tiny", "llama3_8b"):
        wl = WORKLOADS[name]
        numels = wl.numels
        assert wl.faults_for(wl.steps) == wl.faults
        for steps in (wl.steps, 3 * wl.steps, 100):
            sched = wl.faults_for(steps)
            assert all(1 <= k <= steps for k in sched)
            for items in sched.values():
                for t, idx, _ in items:
                    assert 0 <= idx < numels[t]
    moe = WORKLOADS["moe_3.4b_dp4"].faults_for(100)
    assert 4 in moe  # the forced overflow step
    rag = WORKLOADS["ragged_20k"].faults_for(40)
    assert len(rag) == 4 and all(len(v) == 2000 for v in rag.values())  # 10 % of the steps, 2,000 values each
    assert WORKLOADS["llama3_8b"].faults_for(50) == {}


def test_one_draw_inputs_are_views_of_one_buffer():
    """bench.py --one-draw: every tensor of the list is a view of one buffer per kind, with the
    workload's shapes, each starting on a 512-byte boundary of that buffer."""
    import torch
    sys.path.insert(0, ROOT)
    import bench
    from workloads import WORKLOADS, gen
    wl = WORKLOADS["ragged_mini"]
    params, grads = bench.one_draw_inputs(torch, gen, wl, "cpu")
    for ts in (params, grads):
        base = ts[0].data_ptr()
        assert len(ts) == len(wl.numels)
        for t, (_, shape) in zip(ts, wl.shapes):
            assert tuple(t.shape) == tuple(shape) and t.dtype == torch.bfloat16
            assert (t.data_ptr() - base) % 512 == 0 and t.untyped_storage().data_ptr() == ts[0].untyped_storage().data_ptr()
    assert float(grads[0].float().std()) > 0
