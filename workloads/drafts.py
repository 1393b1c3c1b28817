"""Seeded synthetic drafter outputs for the dynamic draft-tree builder.

A round of the builder needs, per request and per frontier slot i < K, the
drafter's K candidates (token, probability).  The drafter is not modelled:
tokens are K distinct random ids from the vocabulary, and probabilities are
the K largest entries of a softmax over K + 3 logits ~ N(0, (2 c_b)^2),
sorted descending, where c_b ~ Exp(1) is a per-request confidence (so
requests differ in how peaked their drafts are, as the ECHO section
assumes).  Shapes: tokens int32 and probs float32 [rounds][B][K][K].

Nothing of the builder's arithmetic is here: no products, rankings or
selections.
"""
from __future__ import annotations

import hashlib

import numpy as np
import torch


def _seed(*parts) -> int:
    h = hashlib.sha256(repr(("drafts",) + parts).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def candidates(rounds: int, B: int, K: int, V: int, seed: int = 0, spread: float = 2.0,
               device: str = "cpu"):
    rng = np.random.default_rng(_seed(rounds, B, K, V, seed))
    conf = rng.exponential(1.0, size=B)
    # K distinct ids per node: the first K of a random permutation prefix
    toks = np.empty((rounds, B, K, K), dtype=np.int32)
    for r in range(rounds):
        for b in range(B):
            for i in range(K):
                toks[r, b, i] = rng.choice(V, size=K, replace=False)
    z = rng.standard_normal((rounds, B, K, K + 3)) * (spread * conf)[None, :, None, None]
    p = np.exp(z - z.max(axis=-1, keepdims=True))
    p /= p.sum(axis=-1, keepdims=True)
    probs = -np.sort(-p, axis=-1)[..., :K].astype(np.float32)
    return (torch.from_numpy(toks).to(device), torch.from_numpy(probs).to(device))
