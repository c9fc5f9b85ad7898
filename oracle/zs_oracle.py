"""Plain CPU oracle of the per-rank ZeRO-1/2 mixed-precision optimizer step.

TEST INFRASTRUCTURE ONLY: imported by the tests, the package smoke check and the
benchmark's CPU-baseline leg, never by the product path, and sharing no code with
the HIP library.  Written for clarity, not speed: torch CPU tensors are used as
plain arrays (they carry bf16/fp16 and round-to-nearest-even casts), all
arithmetic on values is fp64, and the optimizer state is stored in fp32 because
the pages keep the master weights and both Adam moments in FP32.

Sources (page title, section):
  [NDS]  "nano-deepspeed (Teaching Edition)", section 2 "Current Feature Range":
         ZeRO stages 0/1/2, AdamW only, FP16 dynamic loss scaling and a bf16 path,
         stage-2 communication as a packed buffer plus local scatter-back.
  [MEG]  leetllm "Deep dive: Megatron", section "Distributed optimizer: trade
         replicated state for collectives": equal contiguous shards of a
         contiguous gradient buffer, each rank updates its FP32 master and Adam
         moments, the sharded-SGD worked example and its divisibility rule.
  [MEGP] same page, section "Precision: FP16, BF16, FP8, and FP4": keep the
         optimizer masters and sensitive reductions in higher precision.
  [BOOK] "3.7 Megatron-LM, DeepSpeed & Parallelism in Practice", sections
         "ZeRO Stages Recap" (fp32 master + two fp32 moments = 12 bytes per
         parameter beside 2-byte params and grads), "ZeRO-Offload and
         ZeRO-Infinity" (dynamic loss scale with a window of 1000, gradient
         clipping 1.0, `contiguous_gradients`) and "Initializing a DeepSpeed
         Engine" (torch.optim.AdamW with decoupled weight decay).

Readings where the pages are silent are marked READING and collected in the
design notes of the repository.

Parity status of each function: every function below is pinned by a CPU test
against values fixed by the pages or by mathematics (worked example, closed
forms, brute force, exhaustive bit-pattern sweeps, library routines).  The
wiring of the stages in OracleRank.step (a global norm over every rank's
partial, taken on the unscaled gradient, whose clip coefficient and unscale
reach the update) is pinned end to end against torch.nn.utils.clip_grad_norm_
followed by torch.optim.AdamW, at one rank and at two ranks sharing one flat
buffer, with clipping active and a loss scale of 2^12.
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import torch

_EXP_MASK = {torch.float16: 0x7C00, torch.bfloat16: 0x7F80, torch.float32: 0x7F800000}


# ----------------------------------------------------------------------------------------------
# Layout and partition  [MEG] equal contiguous ownership, n divisible by d; [NDS] packed buffer
# ----------------------------------------------------------------------------------------------

@dataclass
class OracleLayout:
    numels: list
    offsets: list          # flat index of each tensor's first element
    flat_numel: int        # padded length of the flat buffer (Np)
    dp_world: int
    dp_rank: int
    align: int
    shard_begin: int
    shard_numel: int


def _round_up(x, m):
    return ((x + m - 1) // m) * m


def plan_layout(numels, dp_world, dp_rank, align=1) -> OracleLayout:
    """Place tensors back to back in list order, each starting at a multiple of `align`
    elements (align 1 = dense concatenation), then pad the tail with zeros up to a
    multiple of dp_world * align so that the buffer divides into dp_world equal
    contiguous shards of S elements; rank r owns flat indices [r*S, (r+1)*S).

    READING: the pages require the buffer length to be divisible by the number of
    ranks [MEG] and fix no padding unit; the tail padding is the smallest that makes
    it divisible (and keeps every shard a multiple of `align`).
    """
    if dp_world < 1 or not (0 <= dp_rank < dp_world):
        raise ValueError("rank outside the data-parallel group")
    if align < 1 or (align & (align - 1)):
        raise ValueError("alignment must be a power of two")
    if len(numels) < 1 or any(n < 0 for n in numels):
        raise ValueError("need at least one tensor and non-negative sizes")
    offsets = []
    pos = 0
    for n in numels:
        pos = _round_up(pos, align)
        offsets.append(pos)
        pos += n
    flat_numel = _round_up(pos, dp_world * align)
    shard = flat_numel // dp_world
    return OracleLayout(list(numels), offsets, flat_numel, dp_world, dp_rank, align, dp_rank * shard, shard)


def pack(tensors, layout: OracleLayout, dtype=None) -> torch.Tensor:
    """Copy every tensor into one contiguous flat buffer at its planned offset; gaps and
    the tail are zero.  A bit copy when dtype is the tensors' dtype, an exact widening
    when dtype is float32 (used to seed the fp32 master from the parameters)."""
    if dtype is None:
        dtype = tensors[0].dtype
    flat = torch.zeros(layout.flat_numel, dtype=dtype)
    for t, off, n in zip(tensors, layout.offsets, layout.numels):
        if n:
            flat[off:off + n] = t.reshape(-1).to(dtype)
    return flat


def accumulate(acc: torch.Tensor, tensors, layout: OracleLayout) -> torch.Tensor:
    """Gradient accumulation over micro-steps into the flat buffer: acc + pack(tensors),
    elementwise, rounded once to the buffer's dtype (fp32, or the model dtype).  The
    optimizer steps only at the accumulation boundary ([BOOK] "Initializing a DeepSpeed
    Engine": gradient reduction is accumulation-aware; gradient_accumulation_steps in the
    DeepSpeed configs).  READING: each micro-step's sum is rounded once, to nearest even,
    into the buffer's dtype.  It is evaluated in fp64 here; fp64 carries more than twice
    the significand bits of fp32, bf16 and fp16 plus two, so rounding through fp64 equals
    rounding the exact sum once.  The first micro-step of a window is a plain pack (with
    widening to fp32 if wanted)."""
    packed = pack(tensors, layout, acc.dtype)
    return (acc.double() + packed.double()).to(acc.dtype)


def plan_buckets(numels, bucket_numel):
    """Split the parameter list into gradient buckets.  Backward produces gradients from
    the last tensor to the first; a bucket collects them in that order and is closed (and
    its communication may start) once it holds at least bucket_numel elements; the first
    tensor closes the last bucket.  Returns [tensor_begin, tensor_end) pairs in closing
    order.  ([MEG] contiguous buffers let communication start as buckets become ready;
    [BOOK] "DeepSpeed config for this run": reduce_bucket_size 5e8.)
    READING: the pages give only the size knob; a bucket never splits a tensor, so a
    tensor above the size is a bucket of its own."""
    if bucket_numel <= 0 or any(n < 0 for n in numels):
        raise ValueError("bucket size must be positive and sizes non-negative")
    buckets = []
    members = []
    for t in reversed(range(len(numels))):
        members.append(t)
        if sum(numels[i] for i in members) >= bucket_numel or t == 0:
            buckets.append((min(members), max(members) + 1))
            members = []
    return buckets


def bucket_range(layout: OracleLayout, tensor_begin, tensor_end):
    """Flat range owned by the bucket of tensors [tensor_begin, tensor_end): from the
    offset of its first tensor up to the offset of the tensor after its last one (the end
    of the buffer for the last tensor).  READING: the alignment gap behind a tensor and
    the tail padding go with the bucket in front of them, so the buckets of any split of
    the parameter list cover the flat buffer once."""
    n = len(layout.numels)
    if not (0 <= tensor_begin < tensor_end <= n):
        raise ValueError("not a non-empty tensor range")
    begin = layout.offsets[tensor_begin]
    end = layout.flat_numel if tensor_end == n else layout.offsets[tensor_end]
    return begin, end


def pack_bucket(flat: torch.Tensor, tensors, layout: OracleLayout, tensor_begin, tensor_end, accumulate_into=False):
    """The flat buffer after packing one bucket into it: the bucket's range becomes the
    same range of pack(tensors) (or of accumulate(flat, tensors) with accumulate_into);
    every other element keeps its value."""
    begin, end = bucket_range(layout, tensor_begin, tensor_end)
    full = accumulate(flat, tensors, layout) if accumulate_into else pack(tensors, layout, flat.dtype)
    out = flat.clone()
    out[begin:end] = full[begin:end]
    return out


def shard_of(flat: torch.Tensor, layout: OracleLayout) -> torch.Tensor:
    """This rank's contiguous partition of the flat buffer [MEG]."""
    return flat[layout.shard_begin:layout.shard_begin + layout.shard_numel]


def unpack(src: torch.Tensor, layout: OracleLayout, tensors, whole_flat: bool):
    """Scatter a flat buffer back into the parameter tensors, casting to their dtype with
    round-to-nearest-even [NDS local scatter-back].  `src` is either the whole flat
    buffer (whole_flat) or this rank's shard; only the elements it covers are written,
    the rest of each tensor is left unchanged.  Returns new tensors."""
    lo = 0 if whole_flat else layout.shard_begin
    hi = layout.flat_numel if whole_flat else layout.shard_begin + layout.shard_numel
    assert src.numel() == hi - lo
    out = []
    for t, off, n in zip(tensors, layout.offsets, layout.numels):
        t = t.clone()
        a, b = max(off, lo), min(off + n, hi)
        if a < b:
            t.view(-1)[a - off:b - off] = cast_to(src[a - lo:b - lo], t.dtype)
        out.append(t)
    return out


def cast_to(x: torch.Tensor, dtype) -> torch.Tensor:
    """Round to the model dtype with IEEE round-to-nearest-even (READING: the pages name
    the dtypes, not the rounding; this is torch's Tensor.to)."""
    return x.to(dtype)


# ----------------------------------------------------------------------------------------------
# Unscale + overflow flag  [NDS] FP16 dynamic loss scaling; [BOOK] loss_scale 0 = dynamic
# ----------------------------------------------------------------------------------------------

def nonfinite_any(x: torch.Tensor) -> bool:
    """True when any element is +inf, -inf or NaN, decided on the raw bits: the exponent
    field is all ones.  READING: applied to bf16 as well as fp16 (and to an fp32
    accumulation buffer)."""
    if x.numel() == 0:
        return False
    mask = _EXP_MASK[x.dtype]
    if x.dtype == torch.float32:
        bits = x.contiguous().view(torch.int32).to(torch.int64) & 0xFFFFFFFF
    else:
        bits = x.contiguous().view(torch.int16).to(torch.int32) & 0xFFFF
    return bool(((bits & mask) == mask).any())


# ----------------------------------------------------------------------------------------------
# Global L2 norm and clip coefficient  [BOOK] gradient_clipping 1.0; [MEGP] fp64 reduction
# ----------------------------------------------------------------------------------------------

def sumsq_unscaled(x: torch.Tensor, loss_scale: float) -> float:
    """Sum of squares of the unscaled gradient x / loss_scale, in fp64."""
    if x.numel() == 0:
        return 0.0
    g = x.double() / loss_scale
    return float((g * g).sum())


def global_sumsq(rank_partials) -> float:
    """Add the ranks' partial sums of squares in rank order (every rank gets the same
    value).  READING: the pages fix a global clip but not how partials are combined."""
    total = 0.0
    for p in rank_partials:
        total += p
    return total


def clip_coefficient(sumsq: float, max_norm: float):
    """norm = sqrt(sum of squares); clip coefficient min(1, max_norm / (norm + 1e-6)), the
    convention of torch.nn.utils.clip_grad_norm_; no clipping when max_norm <= 0."""
    norm = math.sqrt(sumsq)
    if max_norm <= 0:
        return norm, 1.0
    return norm, min(1.0, max_norm / (norm + 1e-6))


# ----------------------------------------------------------------------------------------------
# AdamW on the fp32 shard  [NDS] AdamW only; [BOOK] torch.optim.AdamW, 12 bytes of fp32 state
# ----------------------------------------------------------------------------------------------

def adamw_update(master, m, v, x, loss_scale, clip, t, hp, decay=None):
    """One AdamW update of this rank's fp32 master / m / v from its gradient shard x.

    g   = clip * x / loss_scale
    m_t = beta1 * m + (1 - beta1) * g
    v_t = beta2 * v + (1 - beta2) * g^2
    p_t = p * (1 - lr * wd) - lr * (m_t / (1 - beta1^t)) / (sqrt(v_t / (1 - beta2^t)) + eps)

    Decoupled weight decay as in torch.optim.AdamW; t counts applied updates from 1.
    READING: arithmetic in fp64; each of m_t, v_t, p_t is rounded once to fp32 when
    stored, and p_t uses the stored fp32 m_t and v_t.
    decay: None (every element decays), or a bool tensor over the shard that is False for
    the elements of no-decay tensors, which update as if weight_decay were 0.
    Returns new (master, m, v) fp32 tensors.
    """
    lr, b1, b2 = hp["lr"], hp["beta1"], hp["beta2"]
    eps, wd = hp["eps"], hp["weight_decay"]
    g = x.double() / loss_scale * clip
    m_t = (b1 * m.double() + (1.0 - b1) * g).float()
    v_t = (b2 * v.double() + (1.0 - b2) * (g * g)).float()
    m_hat = m_t.double() / (1.0 - b1 ** t)
    v_hat = v_t.double() / (1.0 - b2 ** t)
    mult = torch.full_like(master, 1.0 - lr * wd, dtype=torch.float64)
    if decay is not None:
        mult = torch.where(decay, mult, torch.ones_like(mult))
    p_t = (master.double() * mult - lr * m_hat / (v_hat.sqrt() + eps)).float()
    return p_t, m_t, v_t


def decay_mask(layout: OracleLayout, no_decay):
    """Bool mask over this rank's shard: False on the elements of the tensors listed as
    no-decay, True elsewhere (padding included, where the master stays 0 either way).
    READING: the pages instantiate torch.optim.AdamW with one parameter group ([BOOK]
    "Initializing a DeepSpeed Engine"); the usual second group, biases and normalisation
    weights with weight_decay 0 and every other hyper-parameter shared, is taken as a
    per-tensor flag."""
    mask = torch.ones(layout.shard_numel, dtype=torch.bool)
    lo, hi = layout.shard_begin, layout.shard_begin + layout.shard_numel
    for off, n, nd in zip(layout.offsets, layout.numels, no_decay):
        a, b = max(off, lo), min(off + n, hi)
        if nd and a < b:
            mask[a - lo:b - lo] = False
    return mask


# ----------------------------------------------------------------------------------------------
# Loss scaler  [NDS] dynamic loss scaling; [BOOK] loss_scale_window 1000
# ----------------------------------------------------------------------------------------------

@dataclass
class OracleScaler:
    loss_scale: float
    scale_floor: float = 1.0
    dynamic: bool = True
    growth_interval: int = 1000
    growth_tracker: int = 0
    step_t: int = 0
    skipped_total: int = 0


def scaler_update(s: OracleScaler, overflow: bool) -> OracleScaler:
    """Commit one step.  READING: an overflow skips the update (t unchanged), resets the
    growth tracker and, with dynamic scaling, halves the scale down to the floor; an
    applied update increments t and the tracker, and after growth_interval consecutive
    applied updates the scale doubles and the tracker restarts.  A static scale (bf16)
    never changes and its tracker stays 0."""
    s = OracleScaler(**s.__dict__)
    if overflow:
        s.skipped_total += 1
        s.growth_tracker = 0
        if s.dynamic:
            s.loss_scale = max(s.loss_scale / 2.0, s.scale_floor)
    else:
        s.step_t += 1
        if s.dynamic:
            s.growth_tracker += 1
            if s.growth_tracker == s.growth_interval:
                s.loss_scale *= 2.0
                s.growth_tracker = 0
    return s


# ----------------------------------------------------------------------------------------------
# One rank's whole step, stage by stage in the pages' order
# ----------------------------------------------------------------------------------------------

class OracleRank:
    """One data-parallel rank: layout, fp32 master / m / v of its shard and the scaler."""

    def __init__(self, numels, dp_world, dp_rank, params, scaler: OracleScaler, hp, align=1, no_decay=None):
        self.layout = plan_layout(numels, dp_world, dp_rank, align)
        self.decay = decay_mask(self.layout, no_decay) if no_decay is not None else None
        self.hp = dict(hp)
        self.scaler = scaler
        self.master = shard_of(pack(params, self.layout, torch.float32), self.layout).clone()
        self.m = torch.zeros_like(self.master)
        self.v = torch.zeros_like(self.master)
        self.params = [p.clone() for p in params]

    def step(self, shard_x, ext_overflow=False, other_sumsq=None):
        """shard_x: this rank's (already reduced) gradient shard in the model dtype.
        other_sumsq: the other ranks' partial sums of squares, a list indexed by rank
        (entry dp_rank ignored), or None for a single rank.  Returns a record of the
        step's decisions and scalars."""
        lay = self.layout
        overflow = nonfinite_any(shard_x) or bool(ext_overflow)
        rec = dict(overflow=overflow, loss_scale=self.scaler.loss_scale, local_sumsq=None,
                   sumsq=None, norm=None, clip=None)
        if not overflow:
            local = sumsq_unscaled(shard_x, self.scaler.loss_scale)
            parts = [0.0] * lay.dp_world
            for q in range(lay.dp_world):
                parts[q] = local if q == lay.dp_rank else other_sumsq[q]
            ss = global_sumsq(parts)
            norm, c = clip_coefficient(ss, self.hp["max_norm"])
            t = self.scaler.step_t + 1
            self.master, self.m, self.v = adamw_update(self.master, self.m, self.v, shard_x,
                                                       self.scaler.loss_scale, c, t, self.hp, self.decay)
            self.params = unpack(self.master, lay, self.params, whole_flat=False)
            rec.update(local_sumsq=local, sumsq=ss, norm=norm, clip=c)
        self.scaler = scaler_update(self.scaler, overflow)
        return rec
