"""Seeded generators for parameters and gradients of a workload.

Values come from torch's own generator on the requested device (Philox on the
GPU, the CPU generator otherwise).  A test that compares the GPU path with the
CPU oracle draws the inputs once, on one device, and hands the same tensors
(copied) to both sides.
"""

from __future__ import annotations

import torch

from .configs import Workload

TORCH_DTYPE = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}


def _mix(*xs: int) -> int:
    """Combine small integers into one 63-bit seed (splitmix64 finaliser)."""
    h = 0x9E3779B97F4A7C15
    for x in xs:
        h = (h ^ (int(x) & 0xFFFFFFFFFFFFFFFF)) & 0xFFFFFFFFFFFFFFFF
        h = (h * 0xBF58476D1CE4E5B9) & 0xFFFFFFFFFFFFFFFF
        h ^= h >> 31
        h = (h * 0x94D049BB133111EB) & 0xFFFFFFFFFFFFFFFF
        h ^= h >> 29
    return h & 0x7FFFFFFFFFFFFFFF


def _generator(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def make_params(wl: Workload, device="cpu"):
    """Initial model-dtype parameters, N(0, param_sigma) drawn in fp32 and rounded."""
    gen = _generator(device, _mix(wl.seed, 0xA11))
    dt = TORCH_DTYPE[wl.dtype]
    out = []
    for _, shape in wl.shapes:
        x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
        out.append(x.mul_(wl.param_sigma).to(dt))
    return out


def make_grads(wl: Workload, step: int, loss_scale: float, device="cpu", with_faults=True):
    """Step `step` gradients as the backward pass would leave them: N(0, grad_sigma)
    drawn in fp32, multiplied by the loss scale, rounded to the model dtype, with
    the workload's non-finite injections for that step."""
    gen = _generator(device, _mix(wl.seed, 0x6AD, step))
    dt = TORCH_DTYPE[wl.dtype]
    out = []
    for _, shape in wl.shapes:
        x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
        out.append(x.mul_(wl.grad_sigma * loss_scale).to(dt))
    if with_faults:
        for t, k, val in wl.faults.get(step, []):
            out[t].view(-1)[k] = val
    return out


def fill_grads_(grads, wl: Workload, step: int, loss_scale: float, with_faults=True):
    """In-place variant of make_grads for preallocated tensors on any device."""
    dev = grads[0].device if grads else "cpu"
    gen = _generator(dev, _mix(wl.seed, 0x6AD, step))
    for g in grads:
        x = torch.randn(g.shape, generator=gen, device=dev, dtype=torch.float32)
        g.copy_(x.mul_(wl.grad_sigma * loss_scale))
        del x
    if with_faults:
        for t, k, val in wl.faults.get(step, []):
            grads[t].view(-1)[k] = val
    return grads
