"""Target LM head: the vocabulary logits of every tree row (oracle; test
infrastructure).

Pages followed:

* "投机推理算法的常见优化手段" (cnblogs), tree-mask section: one target
  forward over the flattened tree gives, at every tree node, the logits of the
  next-token distribution in that node's context, and verification starts from
  those logits.
* "万字综述 10+ 种 LLM 投机采样推理加速方案", Medusa and EAGLE sections: the
  model's original LM head sits after its last transformer layer and maps the
  final feature of a position to vocabulary logits (EAGLE's drafter reuses
  that same head).

Readings taken where the pages leave the step open:

H1. The head is a bias-free linear map stored one row per vocabulary entry:
    logits[r][v] = sum_k hidden[r][k] * weight[v][k], with hidden[r] the final
    (already normalised) feature of tree row r.  Both operands are bf16
    values; the sum is evaluated in float64 from those values (every product
    of two bf16 values is exact in float64).
H2. What follows the head is unchanged: the acceptance of ``accept`` runs on
    these logits (temperature, coins and walk as there).

Pinned by tests/test_oracle_lm_head.py: permutation weights (logits are the
hidden entries themselves), small-integer operands against a brute-force
integer sum, and bf16 operands against an exactly rounded sum (math.fsum of
the exact products).
"""
from __future__ import annotations

import numpy as np


def logits(hidden: np.ndarray, weight: np.ndarray) -> np.ndarray:
    """[R][H] x [V][H] -> [R][V] float64 logits (reading H1)."""
    h = np.asarray(hidden, dtype=np.float64)
    w = np.asarray(weight, dtype=np.float64)
    if h.ndim != 2 or w.ndim != 2 or h.shape[1] != w.shape[1]:
        raise ValueError(f"hidden {h.shape} and weight {w.shape} do not share the feature axis")
    return h @ w.T


def row_logits(hidden_row: np.ndarray, weight: np.ndarray) -> np.ndarray:
    """Logits of one tree row, for sampled checks at full vocabulary size."""
    return logits(np.asarray(hidden_row)[None, :], weight)[0]
