"""A rank-level optimizer object over the C ABI.

ZeroShardedAdamW owns the buffers of one data-parallel rank (flat gradient
buffer, fp32 master / m / v of its shard, device pointer tables) and issues the
step as a fixed sequence of ABI calls on one stream:

    zs_pack -> zs_unscale_check -> zs_grad_norm -> zs_adamw_step -> zs_scaler_update
    (dp_world == 1: the check is fused into the pack pass, and a step of one
    micro-step is the single call zs_step)

It makes no decisions of its own and never synchronises; the skip on overflow,
the clip and the scaler all happen on the device.  With offload=True the fp32
master / m / v live in host memory and update() runs the offloaded step
(zs_offload_adamw_step, which synchronises its stream) followed by zs_unpack.
"""

from __future__ import annotations

import operator

import torch

from . import _abi as A


def pointer_table(tensors, device):
    """Device int64 array of the tensors' data pointers (the ABI's pointer tables).  The
    kernels dereference every pointer of a non-empty tensor, so each must be contiguous and
    live on `device` (a host or another GPU's pointer would fault the GPU)."""
    device = torch.device(device)
    for t in tensors:
        if t.numel():
            if not t.is_contiguous():
                raise ValueError("tensors must be contiguous")
            if t.device != device:
                raise ValueError(f"a tensor lives on {t.device}, not on {device}")
    return torch.tensor([t.data_ptr() for t in tensors], dtype=torch.int64, device=device)


# Shards of at least this many elements choose the placement of their buffers by measurement
# (ZeroShardedAdamW._tune_placement); below it the update is too short for placement to show.
TUNE_MIN_ELEMENTS = 1 << 26
# The tuning first times up to this many separate allocations of the buffers, together using
# at most this fraction of the free device memory, and keeps the fastest.
TUNE_MAX_ARENAS = 64
TUNE_ARENA_MEMORY_FRACTION = 0.5


def tune_arena_count(free_bytes, arena_bytes, max_arenas=None, fraction=None):
    """How many candidate arenas of arena_bytes the placement tuning allocates when
    free_bytes of device memory are free: as many as `fraction` of it holds, at most
    `max_arenas`, and always one (the tuning then falls back if even that does not fit)."""
    max_arenas = TUNE_MAX_ARENAS if max_arenas is None else max_arenas
    fraction = TUNE_ARENA_MEMORY_FRACTION if fraction is None else fraction
    if arena_bytes <= 0:
        raise ValueError("arena_bytes must be positive")
    return max(1, min(int(max_arenas), int(free_bytes * fraction) // int(arena_bytes)))

# Checkpoint format of ZeroShardedAdamW.state_dict(), and the state fields it keeps (the
# others are results of the latest check and norm, recomputed by the next step).
STATE_FORMAT = "zs-rank-state-1"
PERSISTENT_STATE = ("loss_scale", "scale_floor", "dynamic", "growth_interval", "growth_tracker", "step_t",
                    "skipped_total")


def reshard_state_dicts(state_dicts, dp_world, dp_rank):
    """The state dict of rank dp_rank of a dp_world-way group, from every rank's
    state_dict() of one checkpoint taken at any other group size (the same tensor list and
    align).  Ranks own equal contiguous slices of one flat buffer whose layout does not
    depend on the group size, only its zero tail padding does ("Deep dive: Megatron",
    section "Distributed optimizer"), so re-sharding concatenates the old shards in rank
    order, re-pads the tail with zeros and slices the new rank's range.  Padding elements
    carry zero master, m and v and keep them: their gradient is zero.  The scaler and step
    counters are replicated, so every rank must hold the same ones."""
    sds = list(state_dicts)
    if not sds:
        raise ValueError("no state dicts")
    for sd in sds:
        if sd.get("format") != STATE_FORMAT:
            raise ValueError(f"not a {STATE_FORMAT} state dict")
    lay0 = sds[0]["layout"]
    numels, align, d_old = list(lay0["numels"]), lay0["align"], lay0["dp_world"]
    by_rank = {}
    for sd in sds:
        lay = sd["layout"]
        if list(lay["numels"]) != numels or lay["align"] != align or lay["dp_world"] != d_old:
            raise ValueError("the state dicts come from different layouts")
        if lay["dp_rank"] in by_rank:
            raise ValueError(f"rank {lay['dp_rank']} appears twice")
        if sd["state"] != sds[0]["state"]:
            raise ValueError("the ranks' scaler and step states differ")
        by_rank[lay["dp_rank"]] = sd
    if sorted(by_rank) != list(range(d_old)):
        raise ValueError(f"need the state dicts of all {d_old} ranks")
    offsets, flat_old, _, _ = A.zs_plan(numels, d_old, 0, align)
    new_offsets, flat_new, begin, count = A.zs_plan(numels, dp_world, dp_rank, align)
    if new_offsets != offsets:  # the planner places tensors independently of the group size
        raise ValueError("tensor offsets differ between the two group sizes")
    used = max((o + n for o, n in zip(offsets, numels)), default=0)
    out = {"format": STATE_FORMAT,
           "layout": {"numels": numels, "dp_world": dp_world, "dp_rank": dp_rank, "align": align,
                      "flat_numel": flat_new, "shard_begin": begin, "shard_numel": count},
           "state": dict(sds[0]["state"])}
    for k in ("master", "m", "v"):
        whole = torch.cat([by_rank[r][k].reshape(-1) for r in range(d_old)])
        if whole.numel() != flat_old:
            raise ValueError(f"{k}: the shards do not add up to the flat buffer")
        new = torch.zeros(flat_new, dtype=torch.float32)
        new[:used] = whole[:used]
        out[k] = new[begin:begin + count].clone()
    return out


class ZeroShardedAdamW:
    """One data-parallel rank's ZeRO-1/2 AdamW over bf16/fp16 parameters on one GPU.

    params: the model-dtype parameter tensors (contiguous, on the GPU), in a fixed order.
    lr, betas, eps, weight_decay: torch.optim.AdamW's; max_norm: global clipping
        threshold (<= 0: no clipping).
    dp_world, dp_rank: the data-parallel group; this object owns shard dp_rank of the
        flat buffer.  align: per-tensor alignment of the flat layout in elements.
    dynamic_loss_scale, init_scale, scale_floor, growth_interval: the loss scaler
        (dynamic by default for fp16, a static scale of 1 for bf16).
    grad_dtype: the dtype of the incoming gradients (default: the parameters').
    accum_dtype: torch.float32 for an fp32 accumulation buffer (default: grad_dtype).
    offload, offload_chunk, offload_threads: keep master / m / v in host memory and run
        the update on the host CPU in chunks.
    no_decay: one flag per tensor (True: no weight decay), or "1d" for every tensor with
        at most one dimension.
    state_spacing: carve master / m / v from one allocation this many bytes apart.
    placement: "tune" (default): a shard of at least TUNE_MIN_ELEMENTS elements carves the
        gradient buffer and master / m / v from one allocation: the fastest of several
        candidates, with the four in the order whose update measured fastest in it (see
        _tune_placement); "separate": four allocations.  While it is built, the candidates
        together hold at most TUNE_ARENA_MEMORY_FRACTION of the free device memory and at
        most TUNE_MAX_ARENAS of them are tried (module constants a caller may lower).
    flat_views: the parameters and their .grad become views into two flat buffers laid out
        like the gradient buffer (a contiguous parameter buffer and a contiguous gradient
        buffer that backward fills in place).  step() with no gradient list then checks the
        buffer and writes the new parameters straight into the parameter buffer: no pack
        and no scatter.
    allgather_input: with dp_world > 1 on the GPU (no flat views, no offload), the optimizer
        owns self.flat_param, this rank's slice of the all-gather input (2 bytes per shard
        element), seeded with the shard's parameters, placed with the tuned buffers and
        written by update(scatter=False).  Without it the caller passes flat_param_out.
    """

    def __init__(self, params, lr=1e-3, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.01, max_norm=1.0,
                 dp_world=1, dp_rank=0, align=1, dynamic_loss_scale=None, init_scale=None, scale_floor=1.0,
                 growth_interval=1000, grad_dtype=None, accum_dtype=None, offload=False,
                 offload_chunk=1 << 24, offload_threads=0, no_decay=None, state_spacing=None,
                 flat_views=False, placement="tune", allgather_input=False):
        params = list(params)
        if not params:
            raise ValueError("empty parameter list")
        if len({id(p) for p in params}) != len(params):
            # two segments scattering into one tensor would race
            raise ValueError("a tensor appears more than once in the parameter list")
        self.device = params[0].device
        self.param_dtype = params[0].dtype
        if self.device.type != "cuda":
            raise ValueError("the parameters must live on a GPU")
        if self.param_dtype not in (torch.bfloat16, torch.float16):
            raise ValueError("the parameters must be bf16 or fp16")
        if any(p.dtype != self.param_dtype for p in params):
            raise ValueError("every parameter must have one dtype (the kernels cast to one model dtype)")
        for p in params:
            if p.device != self.device:
                raise ValueError(f"a parameter lives on {p.device}, not on {self.device}")
        self.model_grad_dtype = grad_dtype or self.param_dtype
        # The flat buffer holds the model-dtype gradients, or an fp32 accumulation buffer
        # when accum_dtype=torch.float32 (gradient accumulation over micro-steps).
        self.grad_dtype = accum_dtype or self.model_grad_dtype
        if dynamic_loss_scale is None:
            dynamic_loss_scale = self.model_grad_dtype == torch.float16
        if init_scale is None:
            init_scale = 2.0 ** 16 if dynamic_loss_scale else 1.0
        self.params = params
        self.numels = [p.numel() for p in params]
        self.hp = A.hparams(lr, betas[0], betas[1], eps, weight_decay, max_norm)
        self.dp_world, self.dp_rank, self.align = dp_world, dp_rank, align
        with torch.cuda.device(self.device):
            self.layout = A.zs_layout_create(self.numels, dp_world, dp_rank, align)
            self.flat_numel, self.shard_begin, self.shard_numel = A.zs_layout_info(self.layout)
            self.state = A.zs_state_create(self.layout, A.state_host(init_scale, scale_floor, dynamic_loss_scale,
                                                                     growth_interval))
            # no_decay: one flag per parameter (a second group with weight_decay 0), or
            # "1d" for the usual choice of every tensor with at most one dimension
            if isinstance(no_decay, str):
                if no_decay != "1d":
                    raise ValueError("no_decay is a list of flags or '1d'")
                no_decay = [p.dim() <= 1 for p in params]
            self.no_decay = list(no_decay) if no_decay is not None else None
            if self.no_decay is not None:
                A.zs_layout_set_no_decay(self.layout, self.no_decay)
        dev = self.device
        self.offload = bool(offload)
        if placement not in ("tune", "separate"):
            raise ValueError("placement is 'tune' or 'separate'")
        self.flat_views = bool(flat_views)
        self.flat_params = None
        if self.flat_views:
            if dp_world > 1 and self.shard_numel % 8:
                # each rank's update writes its slice of the parameter buffer, which starts at
                # element rank * S and must lie on a 16-byte boundary; align a multiple of 8
                # makes S one (S is a multiple of align)
                raise ValueError(f"flat_views with several ranks needs a shard size that is a multiple of 8 "
                                 f"elements (it is {self.shard_numel}), so that every rank's slice of the parameter "
                                 f"buffer starts on a 16-byte boundary: use align=8")
            if self.grad_dtype != self.param_dtype:
                raise ValueError("flat_views needs the gradient buffer in the parameter dtype")
            if any(p.dtype != self.param_dtype or p.device != dev for p in params):
                raise ValueError("flat_views needs every parameter in one dtype on one device")
            offsets = A.zs_plan(self.numels, dp_world, dp_rank, align)[0]
            self.flat_params = torch.zeros(self.flat_numel, dtype=self.param_dtype, device=dev)
            with torch.no_grad():
                for p, off, n in zip(params, offsets, self.numels):
                    view = self.flat_params[off:off + n].view(p.shape)
                    view.copy_(p)
                    p.data = view
        self.param_ptrs = pointer_table(params, dev)
        self.local_sumsq = torch.zeros(1, dtype=torch.float64, device=dev)
        self._grad_key = None
        self._grad_ptrs = None
        self._grad_objs = []
        S = self.shard_numel
        # the device buffer of the shard's new parameters: offload mode's, or the all-gather
        # input that allgather_input asks for
        self.flat_param = None
        owns_out = bool(allgather_input)
        if owns_out and (dp_world == 1 or self.flat_views or self.offload):
            raise ValueError("allgather_input is for dp_world > 1 on the GPU without flat_views (offload mode and "
                             "flat views have their own parameter shard buffer)")
        self.placement = {"mode": "separate"}
        tune = (placement == "tune" and not self.offload and not state_spacing and S >= TUNE_MIN_ELEMENTS)
        if tune and self._tune_placement(owns_out):
            pass  # flat, master, m, v (and the all-gather input) carved from the arena, master seeded
        elif not self.offload and state_spacing:
            self.flat = torch.zeros(self.flat_numel, dtype=self.grad_dtype, device=dev)
            # master, m and v carved from one allocation, `state_spacing` bytes apart (at
            # least their own size): an explicit placement kept for experiments; measured
            # gaps of 0.125-16 GiB moved the update's rate by no more than the noise, while
            # the memory an allocation receives moved it by up to 13 % (_tune_placement)
            gap = max(int(state_spacing), 4 * S)
            gap = (gap + (1 << 21) - 1) // (1 << 21) * (1 << 21) // 4   # 2 MiB steps, in floats
            self._state_arena = torch.zeros(2 * gap + S, dtype=torch.float32, device=dev)
            self.master = self._state_arena[0:S]
            self.m = self._state_arena[gap:gap + S]
            self.v = self._state_arena[2 * gap:2 * gap + S]
            A.zs_pack(self.layout, self.param_ptrs, self.param_dtype, self.master, torch.float32, whole_flat=False)
            if owns_out:
                self.flat_param = torch.empty(S, dtype=self.param_dtype, device=dev)
                self._seed_flat_param()
        elif not self.offload:
            self.flat = torch.zeros(self.flat_numel, dtype=self.grad_dtype, device=dev)
            self.master = torch.empty(S, dtype=torch.float32, device=dev)
            self.m = torch.zeros(S, dtype=torch.float32, device=dev)
            self.v = torch.zeros(S, dtype=torch.float32, device=dev)
            A.zs_pack(self.layout, self.param_ptrs, self.param_dtype, self.master, torch.float32, whole_flat=False)
            if owns_out:
                self.flat_param = torch.empty(S, dtype=self.param_dtype, device=dev)
                self._seed_flat_param()
        else:
            # Optimizer state in host memory (only the CPU touches it, so it need not be
            # pinned), pinned two-chunk staging buffers for the copies, and the device buffer
            # that receives the new parameters of the shard.
            self.flat = torch.zeros(self.flat_numel, dtype=self.grad_dtype, device=dev)
            self.offload_chunk = int(offload_chunk)
            self.offload_threads = int(offload_threads)
            self.master = torch.empty(S, dtype=torch.float32)
            self.m = torch.zeros(S, dtype=torch.float32)
            self.v = torch.zeros(S, dtype=torch.float32)
            c = min(self.offload_chunk, max(S, 1))
            self.grad_stage = torch.empty(2 * c, dtype=self.grad_dtype, pin_memory=True)
            self.param_stage = torch.empty(2 * c, dtype=self.param_dtype, pin_memory=True)
            # with flat_views the host's new parameters go straight into the parameter buffer
            self.flat_param = self.param_shard if self.flat_views else torch.empty(S, dtype=self.param_dtype,
                                                                                   device=dev)
            # the shard's current parameters, so that the buffer (the all-gather input with
            # several ranks) is valid before the first applied step, and after a skipped one
            self._seed_flat_param()
            seed = torch.empty(S, dtype=torch.float32, device=dev)
            A.zs_pack(self.layout, self.param_ptrs, self.param_dtype, seed, torch.float32, whole_flat=False)
            self.master.copy_(seed)  # synchronous: complete on return
            del seed
        if self.flat_views:  # every .grad a view of the gradient buffer, wherever it was placed
            self._grad_views = []
            for p, off, n in zip(params, A.zs_plan(self.numels, dp_world, dp_rank, align)[0], self.numels):
                p.grad = self.flat[off:off + n].view(p.shape)
                self._grad_views.append(p.grad)

    def _tune_placement(self, owns_out=False):
        """Carve the gradient buffer and master, m, v from one allocation, choosing by
        measurement both the allocation and the order of the four buffers in it, and seed the
        master; with owns_out the rank's slice of the all-gather input follows the four in
        the allocation, and every timing writes it as the step's update does.  On MI355X the update's streams run at rates that depend on the physical
        memory an allocation receives: separate allocations of the same size, held at once,
        measured 5.6-5.8 or 6.3-6.5 TB/s and kept their rate from pass to pass, while the 24
        orders within one allocation moved it by 2-4 %.  So the tuning times up to
        TUNE_MAX_ARENAS candidate allocations (together at most TUNE_ARENA_MEMORY_FRACTION of
        the free memory; one when only one fits), keeps the fastest, releases the others, and
        then times the 24 orders in the one it kept.  Each timing runs the update kernel
        itself at lr = 0 on zero gradients and moments, which writes back the very (finite)
        parameters it reads (the master is the exact fp32 widening of the parameters, and
        their nearest-even cast is the parameters again), so nothing the caller sees
        changes.  Returns False (nothing allocated) when no allocation fits."""
        import itertools
        dev, S = self.device, self.shard_numel
        step = 1 << 21
        gbytes = torch.empty(0, dtype=self.grad_dtype).element_size()
        sizes = {"flat": self.flat_numel * gbytes, "master": 4 * S, "m": 4 * S, "v": 4 * S}
        if owns_out:
            sizes["out"] = S * torch.empty(0, dtype=self.param_dtype).element_size()
        padded = {k: (b + step - 1) // step * step for k, b in sizes.items()}
        total = sum(padded.values())
        free, _ = torch.cuda.mem_get_info(dev)
        n_arenas = tune_arena_count(free, total)
        arenas = []
        for _ in range(n_arenas):
            try:
                arenas.append(torch.empty(total, dtype=torch.uint8, device=dev))
            except torch.cuda.OutOfMemoryError:
                break
        if not arenas:
            return False
        dtypes = {"flat": self.grad_dtype, "master": torch.float32, "m": torch.float32, "v": torch.float32,
                  "out": self.param_dtype}
        numel = {"flat": self.flat_numel, "master": S, "m": S, "v": S, "out": S}

        def carve(arena, order):
            out, off = {}, 0
            for k in (*order, "out") if owns_out else order:
                out[k] = arena[off:off + sizes[k]].view(dtypes[k])[:numel[k]]
                off += padded[k]
            return out

        def seed(b):
            b["flat"].zero_()
            b["m"].zero_()
            b["v"].zero_()
            A.zs_pack(self.layout, self.param_ptrs, self.param_dtype, b["master"], torch.float32,
                      whole_flat=False, stream=stream)

        hp = self.hp
        frozen = A.hparams(0.0, hp.beta1, hp.beta2, hp.eps, hp.weight_decay, hp.max_norm)
        # the update the step makes: into the parameter buffer (views), into the all-gather
        # input (owns_out), or scattered into the parameters
        ptrs = None if (self.flat_views or owns_out) else self.param_ptrs
        stream = torch.cuda.current_stream(dev)

        def update_ms(b):
            """The faster of two timed updates after an untimed one (lr 0, see above)."""
            seed(b)
            shard = b["flat"][self.shard_begin:self.shard_begin + S]
            out_flat = self.param_shard if self.flat_views else b.get("out")
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            for k in range(3):
                if k:
                    ev[k - 1].record(stream)
                A.zs_adamw_step(self.layout, shard, self.grad_dtype, b["master"], b["m"], b["v"], frozen, self.state,
                                ptrs, out_flat, self.param_dtype, stream=stream)
            ev[2].record(stream)
            ev[2].synchronize()
            return min(ev[0].elapsed_time(ev[1]), ev[1].elapsed_time(ev[2]))

        names = ("flat", "master", "m", "v")
        with torch.cuda.device(dev):
            arena_ms = [update_ms(carve(a, names)) for a in arenas] if len(arenas) > 1 else []
            pick = min(range(len(arena_ms)), key=arena_ms.__getitem__) if arena_ms else 0
            arena = arenas[pick]
            del arenas
            if arena_ms:
                torch.cuda.empty_cache()  # hand the candidates not kept back to the device
            times = {}
            for order in itertools.permutations(names):
                times["".join(k[0] if k != "master" else "M" for k in order)] = update_ms(carve(arena, order))
            best = min(times, key=times.get)
            b = carve(arena, [{"f": "flat", "M": "master", "m": "m", "v": "v"}[c] for c in best])
            seed(b)
        self._arena = arena
        self.flat, self.master, self.m, self.v = b["flat"], b["master"], b["m"], b["v"]
        if owns_out:
            self.flat_param = b["out"]
            self._seed_flat_param()
        self.placement = {"mode": "tuned", "order": best, "update_ms": times[best],
                          "update_ms_range": [min(times.values()), max(times.values())], "candidates": len(times),
                          "arenas": max(1, len(arena_ms)), "arena_pick": pick,
                          "arena_ms": [round(t, 4) for t in arena_ms]}
        return True

    def _seed_flat_param(self):
        """Without flat views: copy this rank's parameters (bit for bit) into the flat
        parameter shard that the update writes (offload mode, or allgather_input), so that it
        is valid before the first applied step and after a skipped one."""
        if self.flat_param is not None and not self.flat_views:
            A.zs_pack(self.layout, self.param_ptrs, self.param_dtype, self.flat_param, self.param_dtype,
                      whole_flat=False)

    @property
    def shard(self):
        """This rank's partition of the flat gradient buffer (a view)."""
        return self.flat[self.shard_begin:self.shard_begin + self.shard_numel]

    @property
    def param_shard(self):
        """With flat_views: this rank's partition of the parameter buffer (a view), which its
        update writes and the all-gather of the other ranks' partitions completes."""
        if self.flat_params is None:
            raise ValueError("the optimizer was built without flat_views")
        return self.flat_params[self.shard_begin:self.shard_begin + self.shard_numel]

    def _grad_table(self, grads):
        """Device pointer table of a gradient list, rebuilt (and the list validated) unless it
        holds the very tensor objects validated last time at the same addresses.  The
        optimizer keeps those tensors alive, so their addresses cannot pass to other tensors
        that were never checked."""
        key = tuple(map(torch.Tensor.data_ptr, grads))
        if key != self._grad_key or len(grads) != len(self._grad_objs) or \
                not all(map(operator.is_, grads, self._grad_objs)):
            if len(grads) != len(self.numels) or any(g.numel() != n for g, n in zip(grads, self.numels)):
                raise ValueError("gradients must match the parameter list")
            if any(g.dtype != self.model_grad_dtype for g in grads):
                raise ValueError(f"gradients must be {self.model_grad_dtype}")
            self._grad_ptrs = pointer_table(grads, self.device)
            self._grad_key = key
            self._grad_objs = list(grads)
        return self._grad_ptrs

    def _device_arg(self, t, what, dtype, numel):
        """A caller tensor that a kernel reads or writes: on this GPU, contiguous, of the
        dtype the kernel takes, with at least `numel` elements (exactly, when exact)."""
        if t is None:
            return None
        if not isinstance(t, torch.Tensor):
            raise ValueError(f"{what} must be a torch tensor")
        if t.device != self.device:
            raise ValueError(f"{what} must live on {self.device}, not on {t.device}")
        if t.dtype != dtype:
            raise ValueError(f"{what} must be {dtype}, not {t.dtype}")
        if not t.is_contiguous():
            raise ValueError(f"{what} must be contiguous")
        if t.numel() != numel:
            raise ValueError(f"{what} must have {numel} elements, not {t.numel()}")
        return t

    def pack(self, grads, stream=None, accumulate=False, last=True):
        """Pack the per-parameter gradients into the flat buffer, or add them to it
        (accumulate=True, a later micro-step).  The pass that ends a window (last=True) is
        fused with the overflow check and sum of squares when there is one rank."""
        fuse = self.state if (self.dp_world == 1 and last) else None
        fn = A.zs_pack_accumulate if accumulate else A.zs_pack
        fn(self.layout, self._grad_table(grads), self.model_grad_dtype, self.flat, self.grad_dtype,
           whole_flat=True, fuse_check=fuse, stream=stream)

    def buckets(self, bucket_numel):
        """Tensor ranges [begin, end) of the gradient buckets, in the order backward fills them."""
        return A.zs_plan_buckets(self.numels, bucket_numel)

    def bucket_range(self, bucket):
        """Flat range (begin, end) of the buffer that a bucket owns."""
        return A.zs_bucket_range(self.layout, bucket[0], bucket[1])

    def pack_bucket(self, grads, bucket, stream=None, accumulate=False):
        """Pack (or add) the gradients of one bucket into its range of the flat buffer, as
        soon as backward has produced them; `grads` is the whole gradient list."""
        A.zs_pack_bucket(self.layout, self._grad_table(grads), self.model_grad_dtype, self.flat, self.grad_dtype,
                         bucket[0], bucket[1], accumulate=accumulate, stream=stream)

    def check(self, ext_overflow=None, local_sumsq_out=None, stream=None):
        """Overflow flag and local sum of squares of the shard (after the reduce-scatter);
        local_sumsq_out (a device double) receives the value to exchange with the other ranks."""
        ext_overflow = self._device_arg(ext_overflow, "ext_overflow", torch.int32, 1)
        local_sumsq_out = self._device_arg(local_sumsq_out, "local_sumsq_out", torch.float64, 1)
        A.zs_unscale_check(self.layout, self.shard, self.grad_dtype, self.state, ext_overflow,
                           local_sumsq_out if local_sumsq_out is not None else self.local_sumsq, stream=stream)

    def norm(self, rank_sumsq=None, stream=None):
        """Global norm and clip coefficient; rank_sumsq: device array of every rank's local sum
        of squares in rank order (required when dp_world > 1)."""
        rank_sumsq = self._device_arg(rank_sumsq, "rank_sumsq", torch.float64, self.dp_world)
        A.zs_grad_norm(self.layout, None, self.grad_dtype, self.state, self.hp, rank_sumsq, None, stream=stream)

    def update(self, scatter=True, flat_param_out=None, stream=None):
        """AdamW on the shard, then the new parameters: scattered into the parameter tensors
        (scatter), written to flat_param_out, or with flat_views written into the rank's slice
        of the parameter buffer; then the scaler commit.  With allgather_input,
        scatter=False without flat_param_out writes self.flat_param."""
        flat_param_out = self._device_arg(flat_param_out, "flat_param_out", self.param_dtype, self.shard_numel)
        if self.offload:
            # The host updates the state chunk by chunk; the new parameters of the shard land
            # in flat_param_out when given, else in self.flat_param (the all-gather input with
            # several ranks), and are scattered from there.  An overflowed step writes neither.
            out = flat_param_out if flat_param_out is not None else self.flat_param
            A.zs_offload_adamw_step(self.layout, self.shard, self.grad_dtype, self.state, self.hp, self.master,
                                    self.m, self.v, self.grad_stage, self.param_stage,
                                    min(self.offload_chunk, max(self.shard_numel, 1)), out,
                                    self.param_dtype, self.offload_threads, stream=stream)
            if scatter and not (self.flat_views and out is self.flat_param):
                # views: the parameters are the buffer just written
                A.zs_unpack(self.layout, out, self.param_dtype, False, self.param_ptrs, self.param_dtype,
                            self.state, stream=stream)
        elif self.flat_views and scatter and flat_param_out is None:
            # the parameters are views of the parameter buffer: write the shard's slice of it
            A.zs_adamw_step(self.layout, self.shard, self.grad_dtype, self.master, self.m, self.v, self.hp,
                            self.state, None, self.param_shard, self.param_dtype, stream=stream)
        else:
            out = flat_param_out
            if out is None and not scatter:
                out = self.flat_param  # the owned all-gather input, or None: the state only
            A.zs_adamw_step(self.layout, self.shard, self.grad_dtype, self.master, self.m, self.v, self.hp,
                            self.state, self.param_ptrs if scatter else None, out, self.param_dtype,
                            stream=stream)
        A.zs_scaler_update(self.state, stream=stream)

    def zero_grad(self):
        """Zero the gradient buffer (with flat_views, every parameter's .grad, which is made a
        view of the buffer again if something replaced it), on the current stream."""
        self.flat.zero_()
        if self.flat_views:
            for p, g in zip(self.params, self._grad_views):
                if p.grad is not g:
                    p.grad = g

    def _check_views(self):
        """A parameter whose .grad is no longer its view of the buffer (set to None or
        replaced, e.g. by a model-level zero_grad) would leave stale gradients in the buffer:
        refuse to step."""
        if not all(map(operator.is_, (p.grad for p in self.params), self._grad_views)):
            raise ValueError("a parameter's .grad is no longer a view of the gradient buffer; zero the gradients "
                             "with the optimizer's zero_grad(), which keeps the views")

    def step(self, grads=None, stream=None):
        """Whole single-rank step (dp_world == 1).  `grads` is one gradient list, or a list of
        micro-step gradient lists accumulated into the flat buffer before the step.  With
        flat_views and no `grads`, the gradients are already in the buffer (backward wrote
        them through the .grad views): the step checks the buffer, takes the norm, and the
        update writes the new parameters into the flat parameter buffer."""
        if self.dp_world != 1:
            raise ValueError("step() is the single-rank sequence; call pack/check/norm/update with the "
                             "other ranks' flag and partial sums for dp_world > 1")
        if grads is None:
            if not self.flat_views:
                raise ValueError("step() needs the gradients unless the optimizer was built with flat_views")
            self._check_views()
            if self.offload:
                self.check(stream=stream)
                self.norm(stream=stream)
                self.update(stream=stream)
            else:  # one call: check, norm, update into the parameter buffer, scaler commit
                A.zs_step_flat(self.layout, self.flat, self.grad_dtype, self.state, self.hp, self.master, self.m,
                               self.v, self.flat_params, self.param_dtype, stream=stream)
            return
        micro = grads if (grads and isinstance(grads[0], (list, tuple))) else [grads]
        if len(micro) == 1 and not self.offload and self.grad_dtype == self.model_grad_dtype:
            # one call enqueueing the kernels of the sequence below (same results, fewer calls)
            A.zs_step(self.layout, self._grad_table(micro[0]), self.model_grad_dtype, self.flat, self.state,
                      self.hp, self.master, self.m, self.v, self.param_ptrs, self.param_dtype, stream=stream)
            return
        for i, g in enumerate(micro):
            self.pack(g, stream, accumulate=i > 0, last=i == len(micro) - 1)
        self.norm(stream=stream)
        self.update(stream=stream)

    def set_hparams(self, lr=None, betas=None, eps=None, weight_decay=None, max_norm=None):
        """Change the AdamW hyper-parameters or the clipping threshold for the steps that
        follow, e.g. the learning rate of a warmup-and-decay schedule before each step.
        Every step call hands them to the library when it is enqueued; the library checks
        them there (an invalid value raises ZsInvalidArgument with nothing enqueued)."""
        hp = self.hp
        b1, b2 = (hp.beta1, hp.beta2) if betas is None else betas
        self.hp = A.hparams(hp.lr if lr is None else lr, b1, b2, hp.eps if eps is None else eps,
                            hp.weight_decay if weight_decay is None else weight_decay,
                            hp.max_norm if max_norm is None else max_norm)

    def read_state(self, stream=None):
        return A.zs_state_read(self.state, stream).as_dict()

    def write_state(self, values: dict, stream=None):
        s = A.zs_state_read(self.state, stream)
        for k, v in values.items():
            setattr(s, k, v)
        A.zs_state_write(self.state, s, stream)

    def state_dict(self, stream=None):
        """Host copy of what resuming this rank needs: the scaler and step counters, and the
        fp32 master, m and v of its shard, with the layout they belong to.  The model-dtype
        parameters are the model's to save, as with torch.optim; they are the round-to-
        nearest-even cast of the master.  Synchronises (reads the device state)."""
        st = self.read_state(stream)
        return {
            "format": STATE_FORMAT,
            "layout": {"numels": list(self.numels), "dp_world": self.dp_world, "dp_rank": self.dp_rank,
                       "align": self.align, "flat_numel": self.flat_numel, "shard_begin": self.shard_begin,
                       "shard_numel": self.shard_numel},
            "state": {k: st[k] for k in PERSISTENT_STATE},
            "master": self.master.detach().to("cpu", copy=True),
            "m": self.m.detach().to("cpu", copy=True),
            "v": self.v.detach().to("cpu", copy=True),
        }

    def load_state_dict(self, sd, stream=None):
        """Restore a state_dict() of this rank's layout (the same tensor sizes, dp_world,
        dp_rank and align; reshard_state_dicts() maps a checkpoint taken at another dp_world).
        Writes the scaler and step counters and the master, m and v shard; the model-dtype
        parameters are restored by the model, as with torch.optim, before this call (the
        flat parameter shard of offload=True or allgather_input=True is refilled from them
        here)."""
        if sd.get("format") != STATE_FORMAT:
            raise ValueError(f"not a {STATE_FORMAT} state dict")
        lay = sd["layout"]
        mine = (list(self.numels), self.dp_world, self.dp_rank, self.align)
        theirs = (list(lay["numels"]), lay["dp_world"], lay["dp_rank"], lay["align"])
        if mine != theirs:
            raise ValueError("the state dict belongs to another layout (tensor sizes, dp_world, dp_rank or "
                             "align); map it with reshard_state_dicts()")
        for k in ("master", "m", "v"):
            t = sd[k]
            if t.dtype != torch.float32 or t.numel() != self.shard_numel:
                raise ValueError(f"{k}: expected {self.shard_numel} fp32 elements")
        self.write_state({k: sd["state"][k] for k in PERSISTENT_STATE}, stream)
        for k in ("master", "m", "v"):
            getattr(self, k).copy_(sd[k].reshape(-1))
        # the flat parameter shard (offload, allgather_input) follows the parameters, which the
        # model restores first (restore the model's parameters before the optimizer's state)
        self._seed_flat_param()
        torch.cuda.synchronize(self.device)

    def close(self):
        if getattr(self, "state", None):
            A.zs_state_destroy(self.state)
            self.state = None
        if getattr(self, "layout", None):
            A.zs_layout_destroy(self.layout)
            self.layout = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
