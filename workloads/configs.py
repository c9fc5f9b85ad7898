"""Parameter-tensor shape lists and run settings of the optimizer-step workloads.

The shapes stand in for the models the pages train (a GPT-2-style toy model, a
Qwen3-0.6B-shaped list, a ~3.4B MoE list, a Llama-3-8B-shaped list) and a
ragged-size stress list; the optimizer step only sees the tensor sizes, so no
weights or datasets are involved.  Hyper-parameters follow the AdamW settings
of the toy configuration (lr 1e-3, betas (0.9, 0.999), eps 1e-8, weight decay
0.01) with global clipping at 1.0 as in the DeepSpeed configuration on
"Megatron-LM, DeepSpeed & Parallelism in Practice" (section "DeepSpeed config
for this run"), and a loss-scale window of 1000 as in its ZeRO-Offload example.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

HPARAMS = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, max_norm=1.0)
GROWTH_INTERVAL = 1000


def _tiny_gpt2():
    """2 layers, hidden 64, ffn 256, vocab 512, context 128, untied head, with biases."""
    s = [("wte", (512, 64)), ("wpe", (128, 64))]
    for layer in range(2):
        p = f"h{layer}."
        s += [(p + "ln1.w", (64,)), (p + "ln1.b", (64,)),
              (p + "attn.qkv.w", (64, 192)), (p + "attn.qkv.b", (192,)),
              (p + "attn.o.w", (64, 64)), (p + "attn.o.b", (64,)),
              (p + "ln2.w", (64,)), (p + "ln2.b", (64,)),
              (p + "fc.w", (64, 256)), (p + "fc.b", (256,)),
              (p + "proj.w", (256, 64)), (p + "proj.b", (64,))]
    s += [("lnf.w", (64,)), ("lnf.b", (64,)), ("head", (512, 64))]
    return s


def _qwen3_like(layers=28, hidden=1024, ffn=3072, q_heads=16, kv_heads=8, head_dim=128, vocab=151936):
    """Qwen3-style decoder list with a tied embedding (no separate head)."""
    s = [("embed", (vocab, hidden))]
    for layer in range(layers):
        p = f"l{layer}."
        s += [(p + "in_norm", (hidden,)),
              (p + "q", (hidden, q_heads * head_dim)),
              (p + "k", (hidden, kv_heads * head_dim)),
              (p + "v", (hidden, kv_heads * head_dim)),
              (p + "o", (q_heads * head_dim, hidden)),
              (p + "q_norm", (head_dim,)), (p + "k_norm", (head_dim,)),
              (p + "post_norm", (hidden,)),
              (p + "gate", (hidden, ffn)), (p + "up", (hidden, ffn)), (p + "down", (ffn, hidden))]
    s += [("final_norm", (hidden,))]
    return s


def _moe_like(layers=24, hidden=4096, q_heads=32, kv_heads=8, head_dim=128, experts=16, expert_ffn=448,
              vocab=32064):
    """MoE decoder list: GQA attention, a router and 16 three-matrix experts per layer, untied head."""
    s = [("embed", (vocab, hidden))]
    for layer in range(layers):
        p = f"l{layer}."
        s += [(p + "ln1", (hidden,)),
              (p + "q", (hidden, q_heads * head_dim)),
              (p + "k", (hidden, kv_heads * head_dim)),
              (p + "v", (hidden, kv_heads * head_dim)),
              (p + "o", (q_heads * head_dim, hidden)),
              (p + "ln2", (hidden,)),
              (p + "router", (hidden, experts))]
        for e in range(experts):
            s += [(p + f"e{e}.w1", (hidden, expert_ffn)),
                  (p + f"e{e}.w2", (expert_ffn, hidden)),
                  (p + f"e{e}.w3", (hidden, expert_ffn))]
    s += [("final_norm", (hidden,)), ("head", (vocab, hidden))]
    return s


def _llama3_like(layers=32, hidden=4096, ffn=14336, q_heads=32, kv_heads=8, head_dim=128, vocab=128256):
    """Llama-3-style decoder list, untied head, no biases."""
    s = [("embed", (vocab, hidden))]
    for layer in range(layers):
        p = f"l{layer}."
        s += [(p + "in_norm", (hidden,)),
              (p + "q", (hidden, q_heads * head_dim)),
              (p + "k", (hidden, kv_heads * head_dim)),
              (p + "v", (hidden, kv_heads * head_dim)),
              (p + "o", (q_heads * head_dim, hidden)),
              (p + "post_norm", (hidden,)),
              (p + "gate", (hidden, ffn)), (p + "up", (hidden, ffn)), (p + "down", (ffn, hidden))]
    s += [("final_norm", (hidden,)), ("head", (vocab, hidden))]
    return s


def ragged_sizes(seed: int, n_small: int, n_large: int, total: int, small_max: int = 1023):
    """Seeded ragged size list: n_small sizes log-uniform on [1, small_max], n_large sizes
    log-uniform on [small_max + 1, U], with U found by bisection so that the sizes add up to
    `total` (the last large size absorbs the final rounding remainder), then shuffled."""
    rng = np.random.Generator(np.random.PCG64(seed))
    u_small = rng.random(n_small)
    u_large = rng.random(n_large)
    small = np.rint(np.exp(u_small * math.log(small_max))).astype(np.int64)
    small = np.clip(small, 1, small_max)
    lo_edge = small_max + 1
    rest = total - int(small.sum())

    def large(umax):
        return np.rint(lo_edge * np.power(umax / lo_edge, u_large)).astype(np.int64)

    lo, hi = float(lo_edge), float(max(lo_edge * 2, rest))
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if int(large(mid).sum()) < rest:
            lo = mid
        else:
            hi = mid
    big = large(hi)
    big[int(np.argmax(big))] += rest - int(big.sum())
    sizes = np.concatenate([small, big])
    sizes = sizes[rng.permutation(sizes.size)]
    assert int(sizes.sum()) == total and sizes.min() >= 1
    return [int(x) for x in sizes], hi


def _ragged_shapes(seed, n_small, n_large, total):
    sizes, _ = ragged_sizes(seed, n_small, n_large, total)
    return [(f"t{i}", (n,)) for i, n in enumerate(sizes)]


@dataclass(frozen=True)
class Workload:
    """One synthetic optimizer-step workload.

    grads are drawn as N(0, grad_sigma) in fp32, multiplied by the current loss
    scale and rounded to `dtype`; params as N(0, param_sigma) rounded to `dtype`.
    `faults[step]` lists (tensor index, element index, value) overrides applied
    to that step's gradients (steps are numbered from 1).
    """
    name: str
    shapes: tuple
    dtype: str                 # "bf16" or "fp16": grads and params
    dp_world: int
    dp_rank: int
    dynamic: bool              # dynamic loss scaling (fp16) or static scale 1 (bf16)
    init_scale: float
    grad_sigma: float
    param_sigma: float
    steps: int
    seed: int
    align: int = 1
    faults: dict = field(default_factory=dict)
    hparams: dict = field(default_factory=lambda: dict(HPARAMS))
    growth_interval: int = GROWTH_INTERVAL
    fault_spec: tuple = ()     # how `faults` was drawn, to draw the schedule of a longer run

    def faults_for(self, steps):
        """The fault schedule of a run of `steps` steps: `faults` for the workload's own step
        count, otherwise drawn the same way for the longer (or shorter) run."""
        if steps == self.steps or not self.fault_spec:
            return {k: v for k, v in self.faults.items() if k <= steps}
        kind, seed = self.fault_spec[0], self.fault_spec[1]
        if kind == "bernoulli":
            return _faults_bernoulli(seed, steps, self.fault_spec[2], self.fault_spec[3], self.numels)
        n_steps = max(1, round(self.fault_spec[2] * steps))
        return _faults_scattered(seed, steps, n_steps, self.fault_spec[3], self.numels)

    @property
    def numels(self):
        return [int(np.prod(s)) if len(s) else 1 for _, s in self.shapes]

    @property
    def n_elems(self):
        return sum(self.numels)


def _faults_single(step, tensor, index, value):
    return {step: [(tensor, index, value)]}


def _faults_bernoulli(seed, steps, prob, forced_step, numels):
    """Per-step Bernoulli(prob) overflow draws plus one forced overflow step; each
    overflowing step gets one +inf at a numel-weighted random position."""
    rng = np.random.Generator(np.random.PCG64(seed + 1000))
    w = np.asarray(numels, dtype=np.float64)
    w /= w.sum()
    out = {}
    for s in range(1, steps + 1):
        hit = rng.random() < prob
        t = int(rng.choice(len(numels), p=w))
        k = int(rng.integers(0, numels[t]))
        if hit or s == forced_step:
            out[s] = [(t, k, math.inf)]
    return out


def _faults_scattered(seed, steps, n_fault_steps, n_bad, numels):
    """n_fault_steps steps chosen by a seeded permutation; each gets n_bad non-finite
    values (cycling NaN, +inf, -inf) at numel-weighted random positions."""
    rng = np.random.Generator(np.random.PCG64(seed + 2000))
    chosen = sorted(int(x) + 1 for x in rng.permutation(steps)[:n_fault_steps])
    w = np.asarray(numels, dtype=np.float64)
    w /= w.sum()
    vals = [math.nan, math.inf, -math.inf]
    out = {}
    for s in chosen:
        ts = rng.choice(len(numels), size=n_bad, p=w)
        out[s] = [(int(t), int(rng.integers(0, numels[int(t)])), vals[i % 3]) for i, t in enumerate(ts)]
    return out


def _build():
    wl = {}
    tiny = tuple(_tiny_gpt2())
    wl["tiny"] = Workload("tiny", tiny, "fp16", 1, 0, True, 2.0 ** 16, 1e-4, 0.02, 5, 1,
                          faults=_faults_single(3, len(tiny) // 2, 0, math.inf))
    qwen = tuple(_qwen3_like())
    wl["qwen3_0.6b_dp2"] = Workload("qwen3_0.6b_dp2", qwen, "bf16", 2, 0, False, 1.0, 1e-3, 1e-3, 10, 2)
    moe = tuple(_moe_like())
    moe_numels = [int(np.prod(s)) for _, s in moe]
    wl["moe_3.4b_dp4"] = Workload("moe_3.4b_dp4", moe, "fp16", 4, 0, True, 2.0 ** 16, 1e-4, 0.02, 10, 3,
                                  faults=_faults_bernoulli(3, 10, 1e-3, 4, moe_numels),
                                  fault_spec=("bernoulli", 3, 1e-3, 4))
    llama = tuple(_llama3_like())
    wl["llama3_8b"] = Workload("llama3_8b", llama, "bf16", 1, 0, False, 1.0, 1e-3, 0.02, 10, 4)
    rag = tuple(_ragged_shapes(5, 6000, 14000, 2_000_000_000))
    rag_numels = [s[0] for _, s in rag]
    wl["ragged_20k"] = Workload("ragged_20k", rag, "bf16", 1, 0, False, 1.0, 1e-3, 0.02, 20, 5,
                                faults=_faults_scattered(5, 20, 2, 2000, rag_numels),
                                fault_spec=("scattered", 5, 0.1, 2000))

    # Reduced-size variants with the same structure, for parity runs the oracle finishes in seconds.
    mini_rag = tuple(_ragged_shapes(15, 300, 700, 6_000_000))
    mini_numels = [s[0] for _, s in mini_rag]
    wl["ragged_mini"] = Workload("ragged_mini", mini_rag, "bf16", 1, 0, False, 1.0, 1e-3, 0.02, 6, 15,
                                 faults=_faults_scattered(15, 6, 1, 40, mini_numels))
    wl["ragged_mini_a64"] = Workload("ragged_mini_a64", mini_rag, "bf16", 1, 0, False, 1.0, 1e-3, 0.02, 6, 16,
                                     align=64, faults=_faults_scattered(16, 6, 1, 40, mini_numels))
    qwen_mini = tuple(_qwen3_like(layers=2, hidden=256, ffn=768, q_heads=4, kv_heads=2, head_dim=64, vocab=3000))
    wl["qwen_mini_dp2"] = Workload("qwen_mini_dp2", qwen_mini, "bf16", 2, 1, False, 1.0, 1e-3, 1e-3, 10, 12)
    moe_mini = tuple(_moe_like(layers=2, hidden=256, q_heads=4, kv_heads=2, head_dim=64, experts=4, expert_ffn=96,
                               vocab=1003))
    moe_mini_numels = [int(np.prod(s)) for _, s in moe_mini]
    wl["moe_mini_dp4"] = Workload("moe_mini_dp4", moe_mini, "fp16", 4, 2, True, 2.0 ** 16, 1e-4, 0.02, 10, 13,
                                  faults=_faults_bernoulli(13, 10, 1e-3, 4, moe_mini_numels))
    llama_mini = tuple(_llama3_like(layers=2, hidden=256, ffn=896, q_heads=4, kv_heads=2, head_dim=64, vocab=4096))
    wl["llama_mini"] = Workload("llama_mini", llama_mini, "bf16", 1, 0, False, 1.0, 1e-3, 0.02, 10, 14)
    return wl


WORKLOADS = _build()


def get_workload(name: str) -> Workload:
    return WORKLOADS[name]
