"""Benchmark of the per-rank ZeRO-1/2 optimizer step on one MI355X.

One step = the whole hot path over one batch of synthetic gradients already resident in
HBM: pack (fused with the overflow check and fp64 sum of squares), norm + clip finalize,
AdamW on the fp32 master / m / v with cast + scatter-back into the bf16 parameter
tensors, loss-scaler commit.  Default workload: the Llama-3-8B-shaped list (291 tensors,
8,030,261,248 elements, one rank).  Prints one JSON line on stdout.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, AMD published


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def host_info():
    """The host the CPU baseline ran on: CPU model, hardware threads, memory."""
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    ram = None
    try:
        with open("/proc/meminfo") as fh:
            ram = int(fh.readline().split()[1]) * 1024 / 1e9
    except (OSError, ValueError, IndexError):
        pass
    return {"cpu": model, "hardware_threads": os.cpu_count(), "ram_gb": ram}


def cpu_baseline(wl, n_elems, steps, threads=None):
    """Time the CPU oracle (as it stands) on a bounded slice of the workload: one tensor of
    n_elems elements drawn from the workload's distributions, `steps` whole steps, on
    `threads` torch threads (None: torch's default, every core it was given)."""
    import torch

    import oracle as O
    saved = torch.get_num_threads()
    if threads is not None:
        torch.set_num_threads(threads)
    try:
        return _cpu_baseline(torch, O, wl, n_elems, steps)
    finally:
        torch.set_num_threads(saved)


def _cpu_baseline(torch, O, wl, n_elems, steps):
    gen = torch.Generator().manual_seed(wl.seed)
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float16
    params = [torch.randn(n_elems, generator=gen).mul_(wl.param_sigma).to(dt)]
    rank = O.OracleRank([n_elems], 1, 0, params, O.OracleScaler(wl.init_scale, 1.0, wl.dynamic), wl.hparams)
    times = []
    for s in range(steps):
        g = [torch.randn(n_elems, generator=gen).mul_(wl.grad_sigma * rank.scaler.loss_scale).to(dt)]
        t0 = time.perf_counter()
        flat = O.pack(g, rank.layout)
        rank.step(O.shard_of(flat, rank.layout))
        times.append(time.perf_counter() - t0)
    per_step = sum(times) / len(times)
    return {"value": n_elems / per_step, "unit": "elements/s", "cores": torch.get_num_threads(), "kind": "oracle",
            "sample": f"{steps} whole oracle steps (pack, flag, norm, AdamW, cast, scaler) on a {n_elems}-element "
                      f"single-tensor slice with the workload's distributions; elements/s = slice size / mean "
                      f"step time ({per_step:.2f} s)"}


def host_copy_gbps(torch, gib=2, reps=3):
    """Host-memory yardstick: torch's (multi-threaded) copy of a `gib` GiB fp32 tensor,
    read + write bytes over the best time."""
    n = gib * (1 << 30) // 4
    a = torch.ones(n)
    b = torch.empty(n)
    b.copy_(a)
    best = float("inf")
    for _ in range(reps):
        t0 = time.perf_counter()
        b.copy_(a)
        best = min(best, time.perf_counter() - t0)
    del a, b
    return 2 * 4 * n / best / 1e9


def run_offload(args, wl, torch, Z, gen):
    """The offloaded step: pack + check + norm on the GPU, the AdamW update of the fp32 state
    in host memory on the host CPU (chunks copied down and parameters copied up),
    scatter-back and scaler update on the GPU.  Returns the JSON line."""
    dev = torch.device("cuda", 0)
    hp = wl.hparams
    params = gen.make_params(wl, dev)
    grads = gen.make_grads(wl, 1, wl.init_scale, dev, with_faults=False)
    t_setup = time.perf_counter()
    opt = Z.ZeroShardedAdamW(params, lr=hp["lr"], betas=(hp["beta1"], hp["beta2"]), eps=hp["eps"],
                             weight_decay=hp["weight_decay"], max_norm=hp["max_norm"], dynamic_loss_scale=wl.dynamic,
                             init_scale=wl.init_scale, growth_interval=wl.growth_interval, offload=True,
                             offload_chunk=args.offload_chunk, offload_threads=args.offload_threads)
    log(f"offload state allocated and seeded after {time.perf_counter() - t_setup:.1f} s")
    S, N = opt.shard_numel, wl.n_elems
    stream = torch.cuda.current_stream()

    def one_step(times=None):
        opt.pack(grads, stream)
        opt.norm(stream=stream)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        opt.update(stream=stream)  # returns once the new parameters are on the device
        if times is not None:
            times.append(time.perf_counter() - t0)

    for _ in range(args.warmup):
        one_step()
    torch.cuda.synchronize()
    upd = []
    t0 = time.perf_counter()
    for _ in range(args.steps):
        one_step(upd)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    state = opt.read_state()
    assert state["skipped_total"] == 0 and state["step_t"] == args.warmup + args.steps
    threads = opt.offload_threads or int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    opt.close()
    del params, grads, opt
    torch.cuda.empty_cache()
    upd_s = sorted(upd)[len(upd) // 2]
    host_bytes = 28 * S  # read grad 2 + master/m/v 12, write master/m/v 12 + param 2
    host_gbps = host_bytes / upd_s / 1e9
    copy_gbps = host_copy_gbps(torch)
    log(f"offload step {elapsed * 1e3 / args.steps:.1f} ms, host update {upd_s * 1e3:.1f} ms "
        f"({host_gbps:.0f} GB/s host traffic; host copy yardstick {copy_gbps:.0f} GB/s)")
    return {
        "metric": "optimizer-step elements/s and achieved HBM GB/s (% of MI355X peak)",
        "value": S * args.steps / elapsed,
        "unit": "elements/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": elapsed * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f64",
        "storage": "bf16 grads and params on the GPU; fp32 master/m/v in host memory; fp64 update on the host",
        "data": "synthetic: grads N(0,1e-3) and params N(0,0.02) drawn on the GPU, random init, no dataset",
        "config": {"workload": wl.name, "mode": "offload", "tensors": len(wl.numels), "elements": N,
                   "shard_elements": S, "grad_dtype": wl.dtype, "offload_chunk": args.offload_chunk,
                   "host_threads": threads},
        "offload": {"host_update_ms_median": upd_s * 1e3, "host_update_gbps": host_gbps,
                    "host_bytes_per_element": 28, "pcie_bytes_per_element": 4,
                    "host_copy_yardstick_gbps": copy_gbps},
        "roofline": {"bound": "host-dram", "kernel": "host AdamW update (zs_host_adamw_step chunks)",
                     "achieved": host_gbps, "peak": copy_gbps, "unit": "GB/s", "frac": host_gbps / copy_gbps,
                     "traffic": None, "peak_source": "measured host copy on the same machine (no published figure)"},
    }


def one_draw_inputs(torch, gen, wl, dev):
    """Parameters and gradients of the workload as views into one buffer each, every tensor
    starting on a 512-byte boundary (as the caching allocator places separate small
    tensors), each buffer filled by a single draw with the workload's distribution: the same
    tensor list and kernel paths as one draw per tensor, with a handful of dispatches
    instead of thousands (for counter runs)."""
    dt = gen.TORCH_DTYPE[wl.dtype]
    offs, pos = [], 0
    for n in wl.numels:
        offs.append(pos)
        pos += (n + 255) // 256 * 256
    g = torch.Generator(device=dev)
    g.manual_seed(wl.seed)
    bufs = []
    for sigma in (wl.param_sigma, wl.grad_sigma * wl.init_scale):
        x = torch.randn(pos, generator=g, device=dev, dtype=torch.float32)
        bufs.append(x.mul_(sigma).to(dt))
        del x
    views = [[b[o:o + n].view(shape) for o, n, (_, shape) in zip(offs, wl.numels, wl.shapes)] for b in bufs]
    return views[0], views[1]


def _median(xs):
    xs = sorted(xs)
    if not xs:
        return None
    return xs[len(xs) // 2] if len(xs) % 2 else 0.5 * (xs[len(xs) // 2 - 1] + xs[len(xs) // 2])


def kernel_source_sha256():
    """Hash of the kernel sources with comments and blank space removed, so that counter
    summaries stay valid across comment edits and go stale on any code change."""
    import re
    h = hashlib.sha256()
    for f in ("zero_sharded_mixed_buffer_amd/csrc/zs_kernels.hip", "zero_sharded_mixed_buffer_amd/csrc/zs_internal.h"):
        with open(os.path.join(ROOT, f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()


def measured_traffic(workload, kernel="k_adamw"):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE
    summary, scaled by the copy-kernel calibration recorded there; None when there is no
    summary for this workload or the kernel sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"k_adamw_{workload}_hbm_traffic.md")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        text = fh.read()
    if "```json" not in text:
        return None
    summary = json.loads(text.split("```json", 1)[1].split("```", 1)[0])
    if summary.get("source_sha256") != kernel_source_sha256():
        return None
    return summary["kernels"][kernel]["traffic_bytes"]


def ceilings(torch, Z, opt, stream, reps=5):
    """Measured HBM yardsticks on the step's own buffers (same placement in HBM), with the
    library's probe kernels (include/zs_probe.h): the update kernel's launch shape and
    access pattern with no arithmetic.  mix_4r4w reads the flat gradient shard (2 B) and
    master, m, v (12 B) and writes master, m, v (12 B) and a parameter-sized buffer (2 B):
    the 28 B per element of the update; copy is master -> m (one-to-one), read is master,
    write is m.  They overwrite master, m and v, so they run after the timed steps."""
    S = opt.shard_numel
    n = S // 4096 * 4096
    nb = n * 4 // 16384 * 16384
    out = torch.empty(n, dtype=opt.param_dtype, device=opt.device)
    sink = torch.zeros(1, dtype=torch.int32, device=opt.device)
    g = opt.shard
    cases = (("mix_4r4w", lambda: Z.zs_probe_mix(g, opt.master, opt.m, opt.v, out, n, stream), 28 * n),
             ("copy", lambda: Z.zs_probe_copy(opt.master, opt.m, nb, stream), 2 * nb),
             ("read", lambda: Z.zs_probe_read(opt.master, nb, sink, stream), nb),
             ("write", lambda: Z.zs_probe_write(opt.m, nb, stream), nb))
    res = {}
    for name, fn, nbytes in cases:
        fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        res[name] = {"gbps": nbytes / (ms * 1e-3) / 1e9, "ms": ms, "bytes": nbytes}
    del out, sink
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama3_8b")
    ap.add_argument("--cpu-baseline-elems", type=int, default=1 << 27)
    ap.add_argument("--cpu-baseline-steps", type=int, default=6)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--grad-accum", type=int, default=1,
                    help="micro-steps accumulated into the flat buffer before each optimizer step")
    ap.add_argument("--accum-dtype", choices=["fp32", "model"], default="fp32",
                    help="dtype of the accumulation buffer when --grad-accum > 1")
    ap.add_argument("--bucket-numel", type=int, default=0,
                    help="pack the gradients in buckets of at least this many elements, in backward order "
                         "(the pages' reduce_bucket_size is 500000000), then check the shard; 0 = one pack "
                         "with the check fused")
    ap.add_argument("--offload", action="store_true",
                    help="keep master/m/v in host memory and run the update on the host CPU")
    ap.add_argument("--offload-chunk", type=int, default=1 << 24, help="elements per offloaded chunk")
    ap.add_argument("--offload-threads", type=int, default=0, help="host threads (0: OMP_NUM_THREADS or all)")
    ap.add_argument("--no-decay", choices=["none", "1d"], default="none",
                    help="1d: tensors with at most one dimension (biases, norm weights) take no weight decay")
    ap.add_argument("--state-spacing-gib", type=float, default=0.0,
                    help="place master, m and v this many GiB apart in one allocation (0: the --placement policy)")
    ap.add_argument("--placement", choices=["tune", "separate"], default="tune",
                    help="tune: the optimizer carves its gradient buffer and master/m/v from the fastest of several "
                         "candidate allocations, in the order its update measures fastest there (the default); "
                         "separate: four allocations")
    ap.add_argument("--log-steps", type=int, default=0,
                    help="after the timed region, run this many more steps reading the state after each and "
                         "print one [zs_step k] line per step (scale, skips, norm, clip, time)")
    ap.add_argument("--one-draw", action="store_true",
                    help="draw the parameters and gradients as views into one buffer each (one draw per buffer "
                         "instead of one per tensor), for profiler runs that count every dispatch")
    ap.add_argument("--faults", action="store_true",
                    help="apply the workload's fault schedule (non-finite gradients on its fault steps, drawn for "
                         "--steps steps) in the timed steps and report the skipped steps' time separately")
    ap.add_argument("--flat-views", action="store_true",
                    help="parameters and gradients as views into contiguous buffers (backward fills the "
                         "gradient buffer): the step checks the buffer instead of packing, and the update "
                         "writes the parameter buffer instead of scattering")
    ap.add_argument("--graph", action="store_true",
                    help="also time the single-rank step captured once in a HIP graph and replayed, against the "
                         "same step issued call by call (launch-bound small lists)")
    ap.add_argument("--no-ceilings", dest="ceilings", action="store_false",
                    help="skip timing the probe kernels (the update's 4-read/4-write mix, copy, read, write) on the "
                         "step's buffers as bandwidth yardsticks")
    ap.add_argument("--ceilings", dest="ceilings", action="store_true", help=argparse.SUPPRESS)
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark measures one GPU: the per-rank step runs on one MI355X with no "
                                   "collectives, so --gpus must be 1"}))
        sys.exit(2)

    import torch

    import zero_sharded_mixed_buffer_amd as Z
    from workloads import WORKLOADS, gen

    Z.lib()
    wl = WORKLOADS[args.workload]
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    if args.offload:
        if wl.dp_world != 1:
            print(json.dumps({"error": "bench times the single-rank step"}))
            sys.exit(2)
        log(f"workload {wl.name} (offloaded): {len(wl.numels)} tensors, {wl.n_elems} elements")
        out = run_offload(args, wl, torch, Z, gen)
        if not args.no_cpu_baseline:
            log("timing the CPU oracle baseline")
            out["cpu_baseline"] = cpu_baseline(wl, args.cpu_baseline_elems, args.cpu_baseline_steps)
        print(json.dumps(out), flush=True)
        return
    hp = wl.hparams
    log(f"workload {wl.name}: {len(wl.numels)} tensors, {wl.n_elems} elements, dp {wl.dp_world}")
    t_setup = time.perf_counter()
    if args.one_draw:
        params, grads = one_draw_inputs(torch, gen, wl, dev)
    else:
        params = gen.make_params(wl, dev)
        grads = gen.make_grads(wl, 1, wl.init_scale, dev, with_faults=False)
    torch.cuda.synchronize()
    log(f"inputs resident after {time.perf_counter() - t_setup:.1f} s")
    G = max(1, args.grad_accum)
    accum = torch.float32 if (G > 1 and args.accum_dtype == "fp32") else None
    opt = Z.ZeroShardedAdamW(params, lr=hp["lr"], betas=(hp["beta1"], hp["beta2"]), eps=hp["eps"],
                             weight_decay=hp["weight_decay"], max_norm=hp["max_norm"], dp_world=wl.dp_world,
                             dp_rank=wl.dp_rank, align=wl.align, dynamic_loss_scale=wl.dynamic,
                             init_scale=wl.init_scale, growth_interval=wl.growth_interval, accum_dtype=accum,
                             no_decay="1d" if args.no_decay == "1d" else None,
                             state_spacing=int(args.state_spacing_gib * (1 << 30)) or None,
                             flat_views=args.flat_views, placement=args.placement,
                             allgather_input=wl.dp_world > 1 and not args.flat_views)
    log(f"placement of the optimizer's buffers: {opt.placement}")
    # the placement tuning holds candidate allocations for a moment; the steps' peak is counted apart
    construction_peak = torch.cuda.max_memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    views = args.flat_views
    if views:
        if G != 1 or args.bucket_numel or args.graph:
            print(json.dumps({"error": "--flat-views times the step of one micro-step, call by call"}))
            sys.exit(2)
        with torch.no_grad():  # what backward leaves in the gradient buffer
            for p, g in zip(params, grads):
                p.grad.copy_(g)
        torch.cuda.synchronize()
    S = opt.shard_numel
    N = wl.n_elems
    d, r = wl.dp_world, wl.dp_rank
    stream = torch.cuda.current_stream()
    lay, st = opt.layout, opt.state
    buckets = opt.buckets(args.bucket_numel) if args.bucket_numel > 0 else None
    if buckets is not None:
        log(f"{len(buckets)} buckets of >= {args.bucket_numel} elements")
    # With several ranks this is rank r's step: its own pack of the full local gradients, the
    # check of its shard (the reduce-scatter output), the norm over every rank's partial sum
    # and the update writing the rank's slice of the all-gather input.  The other ranks'
    # partial sums come from their shards of the same buffer, computed once beforehand
    # (on a real group the other GPUs compute them).
    exchange = torch.zeros(d, dtype=torch.float64, device=dev) if d > 1 else None
    flat_param = opt.flat_param if d > 1 and not views else None  # the optimizer's all-gather input
    if d > 1:
        if not views:
            opt.pack(grads, stream)
        for q in range(d):
            if q == r:
                continue
            lq = Z.zs_layout_create(wl.numels, d, q, wl.align)
            sq = Z.zs_state_create(lq, Z.state_host(wl.init_scale, 1.0, wl.dynamic, wl.growth_interval))
            Z.zs_unscale_check(lq, opt.flat[q * S:(q + 1) * S], opt.grad_dtype, sq, None, exchange[q:q + 1], stream)
            torch.cuda.synchronize()
            Z.zs_state_destroy(sq)
            Z.zs_layout_destroy(lq)
    separate_check = (buckets is not None or d > 1) and not views
    # --faults: the timed steps follow the workload's fault schedule.  A fault step packs a
    # gradient list whose affected tensors are copies holding the non-finite values, through
    # a pointer table built beforehand; with several ranks, another rank whose shard holds a
    # fault sends a non-finite partial sum, as its own check would.
    schedule, fault_tables, fault_exch, clean_exch = {}, {}, {}, None
    if args.faults:
        if G != 1 or buckets is not None or views or args.graph:
            print(json.dumps({"error": "--faults times the plain step (one micro-step, one pack)"}))
            sys.exit(2)
        schedule = wl.faults_for(args.steps)
        offsets = Z.zs_plan(wl.numels, d, r, wl.align)[0]
        clean_exch = exchange.clone() if d > 1 else None
        for k, items in schedule.items():
            faulty = list(grads)
            for t, idx, val in items:
                if faulty[t] is grads[t]:
                    faulty[t] = grads[t].clone()
                faulty[t].view(-1)[idx] = val
            fault_tables[k] = (faulty, Z.pointer_table(faulty, dev))
            if d > 1:
                ex = clean_exch.clone()
                for t, idx, val in items:
                    q = (offsets[t] + idx) // S
                    if q != r:
                        ex[q] = math.inf
                fault_exch[k] = ex
        torch.cuda.synchronize()
        log(f"fault schedule over {args.steps} steps: steps {sorted(schedule)} "
            f"({sum(len(v) for v in schedule.values())} non-finite values)")
    fault_step = [None]  # the timed step being issued (1-based) when it is a fault step

    def pack_pass(k):
        last = k == G - 1
        if views:  # the gradients are already in the buffer (the shard: after the reduce-scatter)
            opt.check(local_sumsq_out=exchange[r:r + 1] if d > 1 else None, stream=stream)
            return
        if fault_step[0] is not None:
            _, table = fault_tables[fault_step[0]]
            Z.zs_pack(lay, table, opt.model_grad_dtype, opt.flat, opt.grad_dtype, whole_flat=True,
                      fuse_check=st if d == 1 else None, stream=stream)
        elif buckets is None:
            opt.pack(grads, stream, accumulate=k > 0, last=last)
        else:
            for b in buckets:
                opt.pack_bucket(grads, b, stream, accumulate=k > 0)
        if last and separate_check:
            opt.check(local_sumsq_out=exchange[r:r + 1] if d > 1 else None, stream=stream)

    def one_step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        # G micro-steps: the first packs (widening to an fp32 buffer when accumulating in
        # fp32), the rest add; the last pass carries the overflow check and sum of squares
        # (fused into a whole pack, a separate pass over the shard after bucketed packs).
        pack_pass(0)
        if ev is not None:
            ev[4].record(stream)
        for k in range(1, G):
            pack_pass(k)
        if ev is not None:
            ev[1].record(stream)
        opt.norm(rank_sumsq=exchange, stream=stream)
        if ev is not None:
            ev[2].record(stream)
        if views:  # new parameters straight into the rank's slice of the parameter buffer
            Z.zs_adamw_step(lay, opt.shard, opt.grad_dtype, opt.master, opt.m, opt.v, opt.hp, st, None,
                            opt.param_shard, opt.param_dtype, stream)
        else:
            Z.zs_adamw_step(lay, opt.shard, opt.grad_dtype, opt.master, opt.m, opt.v, opt.hp, st,
                            opt.param_ptrs if d == 1 else None, flat_param, opt.param_dtype, stream)
        if ev is not None:
            ev[3].record(stream)
        Z.zs_scaler_update(st, stream)
        if ev is not None:
            ev[5].record(stream)

    for _ in range(args.warmup):
        one_step()
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} steps done")
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        if schedule:
            fault_step[0] = (k + 1) if (k + 1) in schedule else None
            if d > 1 and ((k + 1) in schedule or k in schedule):  # the other ranks' partials
                exchange.copy_(fault_exch[k + 1] if (k + 1) in schedule else clean_exch)
        one_step(evs[k])
    fault_step[0] = None
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    state = opt.read_state()
    n_skip = len(schedule)
    assert state["skipped_total"] == n_skip and state["step_t"] == args.warmup + args.steps - n_skip, state
    if d > 1 and schedule:
        exchange.copy_(clean_exch)
    graph_replay = None
    if args.graph:
        if d != 1 or G != 1 or buckets is not None:
            print(json.dumps({"error": "--graph times the plain single-rank step"}))
            sys.exit(2)
        # capture once (after a warm-up on the capturing side stream), then replay
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            opt.step(grads)
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            opt.step(grads)
        torch.cuda.synchronize()
        t_g = time.perf_counter()
        for _ in range(args.steps):
            graph.replay()
        torch.cuda.synchronize()
        t_g = time.perf_counter() - t_g
        t_e = time.perf_counter()
        for _ in range(args.steps):
            opt.step(grads)  # the single zs_step call
        torch.cuda.synchronize()
        t_e = time.perf_counter() - t_e
        t_s = time.perf_counter()
        for _ in range(args.steps):  # the same kernels as four calls, with no events between them
            opt.pack(grads, stream)
            opt.norm(stream=stream)
            opt.update(stream=stream)
        torch.cuda.synchronize()
        t_s = time.perf_counter() - t_s
        # GPU-only time per step: 50 steps captured in one graph, replayed, timed with events
        # on the replay stream (the host issue cost of the calls drops out)
        gpu_only = {}
        for kind in ("zs_step", "four_calls"):
            g50 = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g50):
                cap = torch.cuda.current_stream()
                for _ in range(50):
                    if kind == "zs_step":
                        opt.step(grads, stream=cap)
                    else:
                        opt.pack(grads, cap)
                        opt.norm(stream=cap)
                        opt.update(stream=cap)
            g50.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(4):
                g50.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            gpu_only[kind] = e0.elapsed_time(e1) / 200
            del g50
        graph_replay = {"ms_per_step": t_g * 1e3 / args.steps, "single_call_ms_per_step": t_e * 1e3 / args.steps,
                        "gpu_only_ms_per_step": gpu_only,
                        "sequence_ms_per_step": t_s * 1e3 / args.steps}
        log(f"graph replay {graph_replay['ms_per_step']:.4f} ms/step, zs_step call by call "
            f"{graph_replay['single_call_ms_per_step']:.4f} ms/step, four-call sequence "
            f"{graph_replay['sequence_ms_per_step']:.4f} ms/step")
        del graph
    # kernel averages over the applied steps (a skipped step's update returns at once)
    applied = [e for k, e in enumerate(evs) if (k + 1) not in schedule]
    pack_ms = sum(e[0].elapsed_time(e[1]) for e in applied) / len(applied)
    first_pack_ms = sum(e[0].elapsed_time(e[4]) for e in applied) / len(applied)
    adamw_ms = sum(e[2].elapsed_time(e[3]) for e in applied) / len(applied)
    ms_per_step = elapsed * 1e3 / args.steps
    step_ms = sorted(e[0].elapsed_time(e[5]) for e in evs)  # per-step HIP-event durations
    step_median = step_ms[len(step_ms) // 2] if len(step_ms) % 2 else 0.5 * (
        step_ms[len(step_ms) // 2 - 1] + step_ms[len(step_ms) // 2])
    step_p90 = step_ms[min(len(step_ms) - 1, int(math.ceil(0.9 * len(step_ms))) - 1)]
    gb = 4 if accum is not None else 2            # bytes per element of the flat gradient buffer
    adamw_bytes = (gb + 26) * S   # read g + master/m/v 12, write master/m/v 12 + param 2
    first_bytes = gb * S if views else (2 + gb) * N  # views: the check reads the shard; else read tensors, write it
    acc_bytes = (2 + 2 * gb) * N  # read the tensors and the buffer, write the buffer
    check_bytes = gb * S if separate_check else 0  # the separate check re-reads the shard
    pack_bytes = first_bytes + (G - 1) * acc_bytes + check_bytes
    step_bytes = pack_bytes + adamw_bytes
    adamw_gbps = adamw_bytes / (adamw_ms * 1e-3) / 1e9
    step_gbps = step_bytes / (ms_per_step * 1e-3) / 1e9
    traffic = measured_traffic(wl.name) if G == 1 else None
    unpack = None
    if d > 1 and not views:  # with views the all-gather fills the parameter buffer: nothing to unpack
        # After the all-gather every rank scatters the whole model-dtype buffer into its
        # parameters: timed on its own, outside the step (4 B per element of the buffer).
        gathered = torch.empty(opt.flat_numel, dtype=opt.param_dtype, device=dev)
        gathered.zero_()
        ue = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        Z.zs_unpack(lay, gathered, opt.param_dtype, True, opt.param_ptrs, opt.param_dtype, None, stream)
        ue[0].record(stream)
        for _ in range(5):
            Z.zs_unpack(lay, gathered, opt.param_dtype, True, opt.param_ptrs, opt.param_dtype, None, stream)
        ue[1].record(stream)
        torch.cuda.synchronize()
        u_ms = ue[0].elapsed_time(ue[1]) / 5
        unpack = {"unpack_whole_ms": u_ms, "gbps": 4 * opt.flat_numel / u_ms / 1e6}
        del gathered
    log(f"step {ms_per_step:.3f} ms ({step_gbps:.0f} GB/s), pack{'+accumulate' if G > 1 else ''} {pack_ms:.3f} ms "
        f"({pack_bytes / pack_ms / 1e6:.0f} GB/s), adamw {adamw_ms:.3f} ms ({adamw_gbps:.0f} GB/s)")
    out = {
        "metric": "optimizer-step elements/s and achieved HBM GB/s (% of MI355X peak)",
        "value": S * args.steps / elapsed,
        "unit": "elements/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "steps_per_s": 1e3 / ms_per_step,
        "step_ms_events": {"median": step_median, "p90": step_p90, "min": step_ms[0], "max": step_ms[-1]},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f64",
        "storage": "bf16 grads and params, fp32 master/m/v; AdamW and norm arithmetic in fp64",
        "data": "synthetic: grads N(0,1e-3) and params N(0,0.02) drawn on the GPU, random init, no dataset",
        "config": {"workload": wl.name, "tensors": len(wl.numels), "elements": N, "dp_world": wl.dp_world,
                   "dp_rank": wl.dp_rank,
                   "shard_elements": S, "grad_dtype": wl.dtype, "align": wl.align, "grad_accum": G,
                   "accum_dtype": ("fp32" if accum is not None else wl.dtype),
                   "bucket_numel": args.bucket_numel or None, "buckets": len(buckets) if buckets else None,
                   "no_decay": args.no_decay, "state_spacing_gib": args.state_spacing_gib or None,
                   "flat_views": views, "placement": opt.placement,
                   "allgather_input_owned": opt.flat_param is not None, "one_draw": args.one_draw},
        "achieved_hbm_gbps": step_gbps,
        "hbm_frac": step_gbps / HBM_PEAK_GBPS,
        "algorithmic_bytes_per_step": step_bytes,
        "kernels_ms": {"pack_check": pack_ms, "adamw_cast_scatter": adamw_ms,
                       "finalize_and_scaler": sum(e[0].elapsed_time(e[5]) for e in applied) / len(applied)
                       - pack_ms - adamw_ms},
        "unpack_after_allgather": unpack,
        "graph_replay": graph_replay,
        "faults": None if not args.faults else {
            "fault_steps": sorted(schedule),
            "non_finite_values": sum(len(v) for v in schedule.values()),
            "skipped_ms_each": [evs[k - 1][0].elapsed_time(evs[k - 1][5]) for k in sorted(schedule)],
            "applied_ms_median": _median([evs[k][0].elapsed_time(evs[k][5]) for k in range(args.steps)
                                          if (k + 1) not in schedule]),
            "skipped_steps_note": "a skipped step runs the pack (or the shard check), the flag and norm finalize, "
                                  "an update kernel that returns at once and the scaler commit"},
        "accumulation": None if G == 1 else {
            "first_pack_ms": first_pack_ms, "first_pack_gbps": first_bytes / first_pack_ms / 1e6,
            "accumulate_ms_each": (pack_ms - first_pack_ms) / (G - 1),
            "accumulate_gbps": acc_bytes * (G - 1) / (pack_ms - first_pack_ms) / 1e6},
        "roofline": {"bound": "hbm", "kernel": "k_adamw (AdamW + unscale + clip + cast + scatter)",
                     "achieved": adamw_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": adamw_gbps / HBM_PEAK_GBPS, "traffic": traffic,
                     "bytes_per_launch": adamw_bytes, "avg_launch_ms": adamw_ms,
                     "traffic_over_algorithmic": None if traffic is None else traffic / adamw_bytes},
    }
    if args.log_steps > 0 and d == 1 and G == 1 and buckets is None:
        # untimed: each step is followed by a synchronising state read
        for k in range(args.log_steps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            one_step()
            e1.record(stream)
            st_k = opt.read_state(stream)
            log(f"[zs_step {st_k['step_t']}] scale={st_k['loss_scale']:g} skipped={st_k['skipped_total']} "
                f"norm={st_k['grad_norm']:.6g} clip={st_k['clip_coef']:.6g} ms={e0.elapsed_time(e1):.3f} "
                f"elems/s={S / (e0.elapsed_time(e1) * 1e-3):.4g}")
    out["memory"] = {"max_allocated_gb": torch.cuda.max_memory_allocated() / 1e9,
                     "construction_peak_gb": construction_peak / 1e9,
                     "device_total_gb": torch.cuda.get_device_properties(0).total_memory / 1e9}
    if args.ceilings:  # on the step's own buffers, which it overwrites: after every timed step
        out["ceilings"] = ceilings(torch, Z, opt, stream)
        mix = out["ceilings"]["mix_4r4w"]["gbps"]
        out["roofline"]["ceiling_mix_4r4w_gbps"] = mix
        out["roofline"]["frac_of_measured_ceiling"] = adamw_gbps / mix
        log(f"ceilings: " + ", ".join(f"{k} {v['gbps']:.0f} GB/s" for k, v in out["ceilings"].items()) +
            f"; adamw at {adamw_gbps / mix:.3f} of the 4R/4W mix")
    opt.close()
    del params, grads, opt
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        log("timing the CPU oracle baseline (all threads, then one)")
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_baseline_elems, args.cpu_baseline_steps)
        out["cpu_baseline_serial"] = cpu_baseline(wl, args.cpu_baseline_elems // 8, 3, threads=1)
        out["cpu_host"] = host_info()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
