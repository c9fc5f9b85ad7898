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
