"""Pins of the oracle's KV commit / rollback.

Brute force: after committing path [0, c1, ..., ca], logical slot L + k holds
the row that was at L + path[k]; prefix slots are untouched; a chain whose
path is its own prefix leaves the cache unchanged; freed blocks are exactly
the logical blocks at or past the new length.
"""
import numpy as np
import pytest

from oracle import kv


@pytest.mark.parametrize("path", [[0], [0, 1, 2], [0, 2, 3], [0, 1, 3, 4], [0, 5, 9, 17]])
def test_commit_is_a_gather(path):
    L, N, D = 7, 20, 3
    rng = np.random.default_rng(len(path))
    rows = rng.standard_normal((L + N, D))
    out = kv.commit(rows, L, path)
    assert out.shape == (L + len(path), D)
    np.testing.assert_array_equal(out[:L], rows[:L])
    for k, p in enumerate(path):
        np.testing.assert_array_equal(out[L + k], rows[L + p])


def test_chain_prefix_path_is_identity():
    rows = np.arange(40.0).reshape(20, 2)
    out = kv.commit(rows, 10, [0, 1, 2, 3])
    np.testing.assert_array_equal(out, rows[:14])


def test_new_length_and_freed_blocks():
    table = np.arange(100, 110)
    # L = 30, tree of 20 rows occupies slots 30..49 -> blocks 0..3 (block 16)
    assert kv.new_length(30, 2) == 33
    assert kv.freed_blocks(table, 30, 20, 2) == [103]          # blocks >= ceil(33/16)=3
    assert kv.freed_blocks(table, 30, 20, 0) == [102, 103]     # new_len 31 -> from block 2
    assert kv.freed_blocks(table, 16, 16, 15) == []            # everything kept
    assert kv.freed_blocks(table, 0, 33, 0) == [101, 102]      # new_len 1: blocks 1, 2
