"""Seeded synthetic operands of the target LM head.

For a verify workload ``w`` (its tree rows, vocabulary and attention shape):

* ``hidden`` bf16 [R][H]: the final feature of every tree row, N(0, 1);
* ``weight`` bf16 [V][H]: the head, one row per vocabulary entry,
  N(0, sigma / sqrt(H)), so that a logit has standard deviation about sigma
  (the workload's p_sigma, 3 for the 32K / 128K vocabularies).

H defaults to the model width implied by the attention layer, Hq * D (4096
for the 32-head, 128-dim layers).  The draft side (q logits and the drafted
tokens) is the workload's own: a drafter that reuses no part of this head.
Nothing here evaluates the head; it only draws and lays out numbers.
"""
from __future__ import annotations

import hashlib

import torch


def _gen(device, *parts) -> torch.Generator:
    h = hashlib.sha256(repr(parts).encode()).digest()
    g = torch.Generator(device=device)
    g.manual_seed(int.from_bytes(h[:8], "little") & ((1 << 63) - 1))
    return g


def head_inputs(w, H: int | None = None, sigma: float = 3.0, device: str | None = None,
                tag: int = 0):
    """(hidden [R][H], weight [V][H]) as bf16 tensors on ``device``."""
    device = device or w.device
    H = int(H if H is not None else w.Hq * w.D)
    R, V = w.R, w.V
    hidden = torch.randn((R, H), generator=_gen(device, w.name, R, V, H, tag, "hidden"),
                         device=device, dtype=torch.float32).to(torch.bfloat16)
    weight = torch.empty((V, H), dtype=torch.bfloat16, device=device)
    g = _gen(device, w.name, R, V, H, tag, "weight")
    step = 8192                                   # rows per draw: bounded fp32 staging
    for v0 in range(0, V, step):
        n = min(step, V - v0)
        x = torch.randn((n, H), generator=g, device=device, dtype=torch.float32)
        x.mul_(sigma / H ** 0.5)
        weight[v0:v0 + n] = x.to(torch.bfloat16)
    return hidden, weight
