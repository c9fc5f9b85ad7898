"""The library's host-only code (planner, segment maps, buckets, host AdamW) built with the
host compiler's sanitizers and run over seeded random cases (tests/c/host_sanitize.cpp):
AddressSanitizer with UndefinedBehaviorSanitizer, then ThreadSanitizer for the host
update's worker threads.  CPU only."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "zero_sharded_mixed_buffer_amd", "csrc")
SOURCES = [os.path.join(ROOT, "tests", "c", "host_sanitize.cpp"), os.path.join(CSRC, "zs_plan.cpp"),
           os.path.join(CSRC, "zs_host.cpp")]


@pytest.mark.parametrize("sanitizers", ["address,undefined", "thread"])
def test_host_code_under_sanitizers(tmp_path, sanitizers):
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.fail("no host C++ compiler")
    exe = str(tmp_path / "host_sanitize")
    flags = ["-std=c++17", "-O1", "-g", f"-fsanitize={sanitizers}", "-fno-sanitize-recover=all",
             "-fno-omit-frame-pointer", "-ffp-contract=off", "-fno-math-errno", "-pthread"]
    subprocess.run([cxx, *flags, "-I", CSRC, *SOURCES, "-o", exe], check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", TSAN_OPTIONS="halt_on_error=1")
    res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert res.returncode == 0, res.stderr[-4000:]
    assert res.stdout.strip() == "ok"
