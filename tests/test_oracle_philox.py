"""Pin the oracle's Philox4x64-10 to numpy's implementation, bit for bit.

numpy's Philox bit generator advances its 256-bit counter *before* producing
a block, so the block for counter C is ``random_raw`` of a generator started
at C - 1.
"""
import numpy as np
import pytest

from oracle import philox

M64 = (1 << 64) - 1


def _numpy_block(counter, key):
    v = sum(int(c) << (64 * i) for i, c in enumerate(counter))
    v = (v - 1) % (1 << 256)
    cm1 = np.array([(v >> (64 * i)) & M64 for i in range(4)], dtype=np.uint64)
    g = np.random.Philox(key=np.array(key, dtype=np.uint64), counter=cm1)
    return [int(x) for x in g.random_raw(4)]


CASES = [
    ((0, 0, 0, 0), (0, 0)),
    ((0, 0, 0, 1), (0, 0)),
    ((1, 2, 3, 4), (1, 0)),
    ((M64, M64, M64, M64), (M64, M64)),
    ((0, 7, 5, 1), (12345678901234567, 0)),
    ((3, 63, 255, 1), (0xDEADBEEF, 0)),
]


@pytest.mark.parametrize("counter,key", CASES)
def test_philox_matches_numpy(counter, key):
    ours = philox.philox4x64_10([np.uint64(c) for c in counter], key)
    assert [int(x) for x in ours] == _numpy_block(counter, key)


def test_philox_vectorised_matches_numpy_random_counters():
    rng = np.random.default_rng(0)
    n = 64
    ctr = rng.integers(0, 2**63, size=(4, n), dtype=np.uint64) * np.uint64(2) + \
        rng.integers(0, 2, size=(4, n), dtype=np.uint64)
    key = (int(rng.integers(0, 2**63)) * 2 + 1, 0)
    out = philox.philox4x64_10(list(ctr), key)
    for j in range(n):
        assert [int(o[j]) for o in out] == _numpy_block([int(c[j]) for c in ctr], key)


def test_uniform_is_top_53_bits_of_word0():
    rows = np.arange(100, dtype=np.uint64)
    u = philox.uniform(5, 9, 3, rows, 1)
    assert u.dtype == np.float64 and (u >= 0).all() and (u < 1).all()
    for r in (0, 17, 99):
        w0 = _numpy_block((9, 3, r, 1), (5, 0))[0]
        assert u[r] == (w0 >> 11) / float(1 << 53)


def test_uniform_moments():
    rows = np.arange(200000, dtype=np.uint64)
    u = philox.uniform(0, 0, 0, rows, 0)
    assert abs(u.mean() - 0.5) < 0.003
    assert abs(u.var() - 1 / 12) < 0.002
