"""Pins of the oracle's LM head (logits = hidden . weight^T, reading H1).

* Permutation weights: weight[v] = e_{pi(v)} makes logits[r][v] equal to
  hidden[r][pi(v)] exactly; with H != V and a non-symmetric pi a transposed
  operand or a swapped axis fails.
* Small-integer operands: every product and partial sum is an exact integer in
  float64, checked against a brute-force integer triple loop.
* bf16 operands at a realistic width: every product of two bf16 values is
  exact in float64, so math.fsum of the products is the exactly rounded
  logit; the oracle stays within a few ulps of it.
* The composition with acceptance: greedy acceptance on permutation-weight
  logits equals greedy acceptance on the hidden entries themselves.
"""
import math

import numpy as np
import pytest

from oracle import accept as AC
from oracle import lm_head as LH


def _bf16(x):
    """Round float32 values to bf16 (nearest even), returned as float64."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16 << 16
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def test_permutation_weights_give_hidden_entries():
    rng = np.random.default_rng(1)
    R, H, V = 5, 7, 11
    hidden = rng.standard_normal((R, H))
    pi = rng.integers(0, H, size=V)
    weight = np.zeros((V, H))
    weight[np.arange(V), pi] = 1.0
    z = LH.logits(hidden, weight)
    assert z.shape == (R, V)
    assert np.array_equal(z, hidden[:, pi])
    assert np.array_equal(LH.row_logits(hidden[3], weight), hidden[3, pi])


def test_small_integers_match_brute_force():
    rng = np.random.default_rng(2)
    R, H, V = 3, 9, 6
    hidden = rng.integers(-9, 10, size=(R, H))
    weight = rng.integers(-9, 10, size=(V, H))
    want = [[sum(int(hidden[r][k]) * int(weight[v][k]) for k in range(H)) for v in range(V)]
            for r in range(R)]
    assert np.array_equal(LH.logits(hidden, weight), np.array(want, dtype=np.float64))


def test_bf16_operands_within_ulps_of_exact_sum():
    rng = np.random.default_rng(3)
    R, H, V = 2, 4096, 16
    hidden = _bf16(rng.standard_normal((R, H)))
    weight = _bf16(rng.standard_normal((V, H)) * 3.0 / 64.0)
    z = LH.logits(hidden, weight)
    for r in range(R):
        for v in range(V):
            exact = math.fsum(hidden[r] * weight[v])     # products are exact in float64
            mag = math.fsum(np.abs(hidden[r] * weight[v]))
            assert abs(z[r, v] - exact) <= 64 * np.finfo(np.float64).eps * mag


def test_shape_mismatch_rejected():
    with pytest.raises(ValueError):
        LH.logits(np.zeros((2, 3)), np.zeros((4, 5)))


def test_greedy_acceptance_on_head_logits():
    rng = np.random.default_rng(4)
    H, V = 12, 10
    parents = np.array([-1, 0, 0, 1, 2], dtype=np.int32)
    hidden = rng.standard_normal((len(parents), H))
    pi = rng.permutation(H)[:V]
    weight = np.zeros((V, H))
    weight[np.arange(V), pi] = 1.0
    direct = hidden[:, pi]
    tokens = np.array([0] + [int(np.argmax(direct[p])) for p in parents[1:]], dtype=np.int32)
    a = AC.accept_request(parents, tokens, LH.logits(hidden, weight), None, 0.0, 0, 0, 0)
    b = AC.accept_request(parents, tokens, direct, None, 0.0, 0, 0, 0)
    assert a["accept_len"] == b["accept_len"] == 2
    assert a["path"] == b["path"] and a["tokens"] == b["tokens"]
