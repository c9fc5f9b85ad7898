"""CPU tests of the C-ABI library: it loads, exports every declared symbol, and its host-side
planner and argument checks agree with the oracle's layout (no GPU needed, no kernel run)."""

import os
import random
import re

import pytest

import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _z():
    import zero_sharded_mixed_buffer_amd as Z
    try:
        Z.lib()
    except ImportError as e:  # the build step must run first; fail loudly, never skip silently
        pytest.fail(str(e))
    return Z


def _declared_functions():
    names = set()
    inc = os.path.join(ROOT, "include")
    for h in sorted(os.listdir(inc)):
        if h.endswith(".h"):
            with open(os.path.join(inc, h)) as f:
                text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
            names.update(re.findall(r"\b(zs_[a-z_0-9]+)\s*\(", text))
    return sorted(names)


def test_library_exports_every_declared_symbol():
    Z = _z()
    names = _declared_functions()
    assert "zs_pack" in names and "zs_adamw_step" in names and len(names) >= 16
    lib = Z.lib()
    for n in names:
        assert hasattr(lib, n), f"{n} declared in include/ but not exported"


@pytest.mark.parametrize("seed", range(8))
def test_plan_matches_oracle_layout(seed):
    Z = _z()
    rng = random.Random(seed)
    numels = [rng.choice([0, 1, 2, 7, 63, 64, 65, 1000, 4096, 4097, 12345]) for _ in range(rng.randint(1, 60))]
    d = rng.choice([1, 2, 3, 4, 8])
    r = rng.randrange(d)
    align = rng.choice([1, 2, 8, 64, 256])
    offs, flat_numel, sb, sn = Z.zs_plan(numels, d, r, align)
    lay = O.plan_layout(numels, d, r, align)
    assert offs == lay.offsets
    assert (flat_numel, sb, sn) == (lay.flat_numel, lay.shard_begin, lay.shard_numel)


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("whole", [False, True])
def test_segment_map_covers_range_and_maps_elements(seed, whole):
    """Every element of the covered range belongs to exactly one segment; segment (tensor,
    local) pairs reproduce the oracle's offsets element by element."""
    Z = _z()
    rng = random.Random(100 + seed)
    numels = [rng.randint(0, 300) for _ in range(rng.randint(1, 25))]
    d = rng.choice([1, 2, 3, 5])
    r = rng.randrange(d)
    align = rng.choice([1, 4, 16])
    begin, tensor, local = Z.zs_plan_segments(numels, d, r, align, whole)
    lay = O.plan_layout(numels, d, r, align)
    lo = 0 if whole else lay.shard_begin
    hi = lay.flat_numel if whole else lay.shard_begin + lay.shard_numel
    owner = {}
    for i, (off, n) in enumerate(zip(lay.offsets, numels)):
        for k in range(n):
            owner[off + k] = (i, k)
    ends = begin[1:] + [hi - lo]
    assert begin == sorted(begin) and (not begin or begin[0] == 0)
    for b, e, t, loc in zip(begin, ends, tensor, local):
        assert e > b
        for x in range(b, e):
            flat = lo + x
            if t < 0:
                assert flat not in owner
            else:
                assert owner[flat] == (t, loc + (x - b))
    # Maximal pieces: no two neighbours could merge.
    for k in range(len(tensor) - 1):
        same_tensor = tensor[k] == tensor[k + 1] and tensor[k] >= 0
        assert not same_tensor and not (tensor[k] < 0 and tensor[k + 1] < 0)


def test_plan_rejects_bad_arguments():
    Z = _z()
    for args in (([4], 2, 2, 1), ([4], 0, 0, 1), ([4], 1, 0, 3), ([-1], 1, 0, 1)):
        with pytest.raises(Z.ZsError) as e:
            Z.zs_plan(*args)
        assert e.value.status == -1
        assert Z.zs_last_error()
    with pytest.raises(Z.ZsError):
        Z.zs_plan([], 1, 0, 1)


def test_plan_rejects_a_flat_buffer_beyond_one_launch_grid():
    Z = _z()
    limit = ((2 ** 32 - 1) // 256) * 4096
    assert Z.zs_plan([limit], 1, 0)[1] == limit
    assert Z.zs_plan([limit - 5, 5], 1, 0)[1] == limit
    for numels in ([limit + 1], [limit, 1], [2 ** 40]):
        with pytest.raises(Z.ZsError) as e:
            Z.zs_plan(numels, 1, 0)
        assert e.value.status == -1 and "launch limit" in Z.zs_last_error()


def test_page_example_partition():
    Z = _z()
    # Four parameters over two ranks: rank r owns [2r, 2r+2) ("Deep dive: Megatron", distributed optimizer).
    assert Z.zs_plan([4], 2, 0)[1:] == (4, 0, 2)
    assert Z.zs_plan([4], 2, 1)[1:] == (4, 2, 2)


def test_device_calls_fail_cleanly_without_gpu():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    Z = _z()
    with pytest.raises(Z.ZsError) as e:
        Z.zs_layout_create([10], 1, 0)
    assert e.value.status == -2
    with pytest.raises(Z.ZsError) as e:
        Z.zs_pack(None, 0, 0, 0, 0, stream=0)
    assert e.value.status == -1
    with pytest.raises(Z.ZsError) as e:
        Z.zs_step(None, 0, 0, 0, None, Z.hparams(), 0, 0, 0, 0, stream=0)
    assert e.value.status == -1
    with pytest.raises(Z.ZsError) as e:
        Z.zs_step_flat(None, 0, 0, None, Z.hparams(), 0, 0, 0, 0, stream=0)
    assert e.value.status == -1


@pytest.mark.parametrize("seed", range(8))
def test_bucket_plan_matches_oracle(seed):
    Z = _z()
    rng = random.Random(300 + seed)
    numels = [rng.choice([0, 1, 5, 64, 1000, 4096, 70000]) for _ in range(rng.randint(1, 80))]
    size = rng.choice([1, 100, 4096, 50000, 10 ** 6, 10 ** 9])
    assert Z.zs_plan_buckets(numels, size) == O.plan_buckets(numels, size)


def test_bucket_plan_at_the_pages_bucket_size():
    # 5e8-element buckets over an 8-billion-element Llama-3-8B-shaped tensor list.
    Z = _z()
    from workloads import WORKLOADS
    numels = list(WORKLOADS["llama3_8b"].numels)
    got = Z.zs_plan_buckets(numels, 500_000_000)
    assert got == O.plan_buckets(numels, 500_000_000)
    assert got[0][1] == len(numels) and got[-1][0] == 0 and 12 <= len(got) <= 17


def test_bucket_plan_rejects_bad_arguments():
    Z = _z()
    for numels, size in (([4, 5], 0), ([4, -1], 8)):
        with pytest.raises(Z.ZsError) as e:
            Z.zs_plan_buckets(numels, size)
        assert e.value.status == -1
    assert Z.zs_plan_buckets([], 10) == []


def test_plain_c_program_uses_the_host_entry_points(tmp_path):
    """tests/c/abi_host.c, built as C99 against include/zs.h and linked to libzs.so: planning,
    bucket split and one host AdamW update, compared with the oracle."""
    import shutil
    import struct
    import subprocess

    import torch

    Z = _z()
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.fail("no C compiler")
    libdir = os.path.dirname(Z._abi.LIB_PATH)
    exe = str(tmp_path / "abi_host")
    subprocess.run([cc, "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "c", "abi_host.c"), "-o", exe, "-L", libdir, "-lzs",
                    f"-Wl,-rpath,{libdir}"], check=True)
    env = dict(os.environ, LD_LIBRARY_PATH=":".join(filter(None, ["/opt/rocm/lib", os.environ.get("LD_LIBRARY_PATH")])))
    lines = subprocess.run([exe], check=True, capture_output=True, text=True, env=env).stdout.splitlines()
    numels = [3, 5, 2, 7, 1]
    lay = O.plan_layout(numels, 2, 1, 4)
    assert lines[0].split() == ["plan", str(lay.flat_numel), str(lay.shard_begin), str(lay.shard_numel)] + \
        [str(o) for o in lay.offsets]
    want_b = O.plan_buckets(numels, 6)
    assert lines[1].split() == ["buckets", str(len(want_b))] + [f"{a}:{b}" for a, b in want_b]
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, max_norm=1.0)
    f32 = lambda xs: torch.tensor(xs, dtype=torch.float32)
    p, m, v = O.adamw_update(f32([1.0, -2.0, 0.5, 0.25]), f32([0.0, 0.1, 0.0, 0.0]), f32([0.0, 0.01, 0.0, 0.0]),
                             f32([0.5, -0.25, 1e-3, 0.0]), 2.0, 0.5, 3, hp)
    pb = O.cast_to(p, torch.bfloat16).view(torch.int16)
    hexf = lambda x: "%08x" % struct.unpack("<I", struct.pack("<f", float(x)))[0]
    for i in range(4):
        assert lines[2 + i].split() == ["adamw", hexf(p[i]), hexf(m[i]), hexf(v[i]), "%04x" % (int(pb[i]) & 0xFFFF)]
    assert lines[6] == "invalid -1"


def test_invalid_arguments_raise_value_errors():
    Z = _z()
    with pytest.raises(ValueError):
        Z.zs_plan([4], 2, 5, 1)       # rank outside the group
    with pytest.raises(ValueError):
        Z.zs_plan([4], 1, 0, 3)       # alignment not a power of two
    with pytest.raises(Z.ZsError) as e:
        Z.zs_plan_buckets([4, 5], 0)
    assert isinstance(e.value, ValueError) and e.value.status == -1


def test_c_consumer_is_built_and_fails_cleanly_without_gpu(tmp_path):
    """The torch-free C++ consumer of the ABI (tests/c/abi_gpu, built with the library)
    loads libzs.so; without arguments it prints its usage, and with no GPU its first
    device call fails with the library's message instead of crashing."""
    import struct
    import subprocess
    import torch
    exe = os.path.join(os.path.dirname(__file__), "c", "abi_gpu")
    assert os.path.exists(exe), "build the package first"
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 1 and "usage" in r.stderr
    if torch.cuda.is_available():
        return
    inp = tmp_path / "in.bin"
    with open(inp, "wb") as f:
        f.write(struct.pack("<iii", 1, 0, 0) + struct.pack("<q", 4) + struct.pack("<6d", 1e-3, 0.9, 0.999, 1e-8, 0.0, 1.0))
        f.write(struct.pack("<ddii", 1.0, 1.0, 0, 1000) + bytes(8))
    r = subprocess.run([exe, str(inp), str(tmp_path / "out.bin"), "flat"], capture_output=True, text=True,
                       timeout=60)
    assert r.returncode == 1 and "zs_layout_create" in r.stderr, r.stderr


def test_tensors_the_kernels_would_dereference_are_checked_first():
    """Host or wrong-device tensors never reach a pointer table: a kernel would fault on them."""
    import torch

    import zero_sharded_mixed_buffer_amd as Z
    with pytest.raises(ValueError, match="GPU"):
        Z.ZeroShardedAdamW([torch.zeros(4, dtype=torch.bfloat16)])
    with pytest.raises(ValueError, match="lives on cpu"):
        Z.pointer_table([torch.zeros(4, dtype=torch.bfloat16)], torch.device("cuda", 0))
    with pytest.raises(ValueError, match="contiguous"):
        Z.pointer_table([torch.zeros(4, 4, dtype=torch.bfloat16).t()], "cpu")


def test_binding_refuses_tensors_in_the_wrong_memory():
    """A host tensor passed where the library wants device memory (it would be dereferenced
    by a kernel), or a device tensor where it wants host memory, is refused by the binding
    before the library is called."""
    import torch

    import zero_sharded_mixed_buffer_amd as Z
    host = torch.zeros(16)
    hp = Z.hparams()
    for call in (lambda: Z.zs_pack(None, host, torch.bfloat16, host, torch.bfloat16),
                 lambda: Z.zs_unscale_check(None, host, torch.bfloat16, None),
                 lambda: Z.zs_adamw_step(None, host, torch.bfloat16, host, host, host, hp, None),
                 lambda: Z.zs_unpack(None, host, torch.float32, True, host, torch.bfloat16),
                 lambda: Z.zs_step(None, host, torch.bfloat16, host, None, hp, host, host, host, host),
                 lambda: Z.zs_step_flat(None, host, torch.bfloat16, None, hp, host, host, host, host)):
        with pytest.raises(Z.ZsInvalidArgument, match="must be device memory"):
            call()

    class DeviceTensor:  # stands in for a GPU tensor on a machine without one
        is_cuda = True

        def data_ptr(self):
            return 0

    with pytest.raises(Z.ZsInvalidArgument, match="must be host memory"):
        Z.zs_host_adamw_step(DeviceTensor(), torch.bfloat16, host, host, host, 16, hp, Z.state_host())


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """Without libzs.so every entry point raises ImportError: there is no other path."""
    import torch

    import zero_sharded_mixed_buffer_amd as Z
    from zero_sharded_mixed_buffer_amd import _abi
    monkeypatch.setattr(_abi, "LIB_PATH", str(tmp_path / "libzs.so"))
    monkeypatch.setattr(_abi, "_lib", None)
    with pytest.raises(ImportError, match="libzs.so is missing"):
        Z.lib()
    with pytest.raises(ImportError):
        Z.zs_plan([4, 5], 1, 0)
    with pytest.raises(ImportError):
        Z.zs_scaler_update(None, stream=0)
    with pytest.raises(ImportError):
        Z.zs_host_adamw_step(torch.zeros(4, dtype=torch.bfloat16), torch.bfloat16, torch.zeros(4), torch.zeros(4),
                             torch.zeros(4), 4, Z.hparams(), Z.state_host())


def test_error_messages_stay_with_their_thread():
    """zs_last_error is per thread: a rejected call on one thread does not overwrite the
    message another thread reads."""
    import threading

    import zero_sharded_mixed_buffer_amd as Z
    msgs = {}
    barrier = threading.Barrier(2)

    def fail_with(tag, numels):
        try:
            Z.zs_plan(numels, 2, 5)  # dp_rank outside the group
        except Z.ZsInvalidArgument:
            pass
        barrier.wait(timeout=30)
        msgs[tag] = Z.zs_last_error()

    def fail_other(tag):
        try:
            Z.zs_plan([4], 0, 0)  # dp_world < 1
        except Z.ZsInvalidArgument:
            pass
        barrier.wait(timeout=30)
        msgs[tag] = Z.zs_last_error()

    t1 = threading.Thread(target=fail_with, args=("rank", [4, 4]), daemon=True)
    t2 = threading.Thread(target=fail_other, args=("world",), daemon=True)
    t1.start()
    t2.start()
    t1.join(timeout=60)
    t2.join(timeout=60)
    assert msgs["rank"] != msgs["world"], msgs
    assert "rank" in msgs["rank"].lower() and "world" in msgs["world"].lower(), msgs
