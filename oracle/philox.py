"""Philox4x64-10 counter-based uniforms (oracle side; test infrastructure).

The pages draw the acceptance coin with a plain ``random()`` (guijiagi.com
speculative-decoding post, rejection-sampling section).  Both the oracle and
the GPU library replace it by one counter-based generator so the two sides see
the same coins without sharing state: Philox4x64 with 10 rounds, as published
by Salmon, Moraes, Dror and Shaw, "Parallel Random Numbers: As Easy as 1, 2,
3" (SC'11).  Written here from that definition; the CPU tests pin it bit for
bit against ``numpy.random.Philox``.

Round function on a counter (x0, x1, x2, x3) under key (k0, k1):

    (hi0, lo0) = 128-bit product M0 * x0,   (hi1, lo1) = M1 * x2
    x' = (hi1 ^ x1 ^ k0,  lo1,  hi0 ^ x3 ^ k1,  lo0)

and between rounds the key is bumped by the Weyl constants (W0, W1).

Convention used by the verify step: key = (seed, 0); counter =
(step, request, row, purpose) with purpose 0 for the accept coin of a draft
row and 1 for the sampling coin of the node where the walk stops; the uniform
is (word0 >> 11) * 2**-53, a double in [0, 1).
"""
from __future__ import annotations

import numpy as np

M0 = 0xD2E7470EE14C6C93
M1 = 0xCA5A826395121157
W0 = 0x9E3779B97F4A7C15
W1 = 0xBB67AE8584CAA73B
_MASK64 = (1 << 64) - 1
_LO32 = np.uint64(0xFFFFFFFF)
_S32 = np.uint64(32)


def _mulhilo(a: int, b: np.ndarray):
    """128-bit product of constant ``a`` and uint64 array ``b`` as (hi, lo)."""
    a_lo = np.uint64(a & 0xFFFFFFFF)
    a_hi = np.uint64(a >> 32)
    b_lo = b & _LO32
    b_hi = b >> _S32
    ll = a_lo * b_lo
    lh = a_lo * b_hi
    hl = a_hi * b_lo
    hh = a_hi * b_hi
    mid = (ll >> _S32) + (lh & _LO32) + (hl & _LO32)
    lo = (ll & _LO32) | ((mid & _LO32) << _S32)
    hi = hh + (lh >> _S32) + (hl >> _S32) + (mid >> _S32)
    return hi, lo


def philox4x64_10(counter, key):
    """Philox4x64-10 of counters ``counter`` (4 uint64 arrays) under ``key``.

    Returns the four output words as uint64 arrays of the broadcast shape.
    """
    x0, x1, x2, x3 = (np.asarray(c, dtype=np.uint64) for c in counter)
    x0, x1, x2, x3 = np.broadcast_arrays(x0, x1, x2, x3)
    x0, x1, x2, x3 = (a.copy() for a in (x0, x1, x2, x3))
    k0, k1 = int(key[0]) & _MASK64, int(key[1]) & _MASK64
    with np.errstate(over="ignore"):
        for r in range(10):
            if r:
                k0 = (k0 + W0) & _MASK64
                k1 = (k1 + W1) & _MASK64
            hi0, lo0 = _mulhilo(M0, x0)
            hi1, lo1 = _mulhilo(M1, x2)
            x0, x1, x2, x3 = (hi1 ^ x1 ^ np.uint64(k0), lo1,
                              hi0 ^ x3 ^ np.uint64(k1), lo0)
    return x0, x1, x2, x3


def uniform(seed, step, request, row, purpose) -> np.ndarray:
    """Verify-step uniform in [0, 1) for (seed, step, request, row, purpose)."""
    w0, _, _, _ = philox4x64_10((step, request, row, purpose), (seed, 0))
    return (w0 >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)
