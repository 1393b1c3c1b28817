"""Pins of the oracle's tree mask, depth and the workload tree builders."""
import os

import numpy as np
import pytest

from conftest import GOLDEN
from oracle import tree as T
from workloads import trees


def _read_mask(path):
    rows = []
    names = []
    for line in open(path, encoding="utf-8"):
        if line.startswith("#") or not line.strip():
            continue
        parts = line.split()
        names.append(parts[0])
        rows.append([int(x) for x in parts[1:]])
    return names, np.array(rows, dtype=bool)


def test_toy_mask_matches_printed_matrix():
    names, M = _read_mask(os.path.join(GOLDEN, "toy_tree_mask.txt"))
    assert names == ["root", "A", "B", "C", "D", "E"]
    assert np.array_equal(T.ancestor_mask(trees.toy_tree()), M)


def test_toy_mask_words_and_depth():
    M = T.ancestor_mask(trees.toy_tree())
    w = T.pack_words(M, 1)[:, 0]
    # bit j of row i set iff column j printed as 1 (E sees root, B, itself)
    assert int(w[5]) == (1 << 0) | (1 << 2) | (1 << 5)
    assert [int(x) for x in w] == [1, 3, 5, 11, 19, 37]
    assert list(T.depth(trees.toy_tree())) == [0, 1, 1, 2, 2, 2]


def _counts():
    out = []
    for line in open(os.path.join(GOLDEN, "tree_counts.txt"), encoding="utf-8"):
        if line.startswith("#") or not line.strip():
            continue
        kind, params, nodes, leaves = line.split()
        out.append((kind, tuple(int(x) for x in params.split(",")), int(nodes), int(leaves)))
    return out


@pytest.mark.parametrize("kind,params,nodes,leaves", _counts())
def test_tree_sizes_stated_by_pages(kind, params, nodes, leaves):
    p = trees.cartesian(params) if kind == "cartesian" else trees.k_schedule(params)
    assert trees.draft_nodes(p) == nodes
    kids = T.children(p)
    assert sum(1 for k in kids if not k) == leaves


def test_eagle2_round_two_has_25_leaves_and_expands_5():
    rng = np.random.default_rng(7)
    ex = trees.Eagle2Expansion(rng, topk=5)
    ex.step()                       # round 1: root -> 5
    bottom = ex.step()              # round 2: 5 x 5 = 25 leaves
    assert len(bottom) == 25
    scores = {u: ex.score[u] for u in bottom}
    ex.step()                       # round 3: only the top-5 leaves grow
    chosen = ex.expanded_per_round[-1]
    assert len(chosen) == 5
    best5 = sorted(bottom, key=lambda u: -scores[u])[:5]
    assert sorted(chosen) == sorted(best5)
    kids = T.children(np.array(ex.parents))
    assert sum(1 for u in bottom if kids[u]) == 5


def _invariants(parents):
    M = T.ancestor_mask(parents)
    d = T.depth(parents)
    n = len(parents)
    assert np.array_equal(M.sum(axis=1), d + 1)           # ancestors + self
    assert not np.triu(M, 1).any()                        # M_ij => j <= i
    assert M.diagonal().all()
    for i in range(1, n):                                 # M_i = M_parent + {i}
        expect = M[parents[i]].copy()
        expect[i] = True
        assert np.array_equal(M[i], expect)


@pytest.mark.parametrize("parents", [
    trees.chain(8), trees.cartesian((3, 5, 7)), trees.k_schedule((3, 2, 2, 1, 1)),
    trees.eagle2_tree(np.random.default_rng(3), 64), trees.eagle2_tree(np.random.default_rng(4), 9),
])
def test_mask_invariants(parents):
    _invariants(parents)


def test_chain_mask_is_lower_triangular():
    M = T.ancestor_mask(trees.chain(8))
    assert np.array_equal(M, np.tril(np.ones((9, 9), dtype=bool)))


def test_pack_words_roundtrip_two_words():
    p = trees.cartesian((3, 5, 7))
    M = T.ancestor_mask(p)
    W = T.pack_words(M, 2)
    back = np.zeros_like(M)
    for i in range(len(p)):
        for j in range(len(p)):
            back[i, j] = (int(W[i, j // 64]) >> (j % 64)) & 1
    assert np.array_equal(back, M)
    # a depth-3 leaf in the second word sees exactly 4 rows
    assert sum(bin(int(x)).count("1") for x in W[123]) == 4


@pytest.mark.parametrize("bad", [[0, 0], [-1, 1], [-1, 0, 2], [-1, -1], [-1, 0, 5]])
def test_invalid_trees_rejected(bad):
    with pytest.raises(T.TreeError):
        T.ancestor_mask(np.array(bad))


def test_echo_budget_sums_and_bounds():
    rng = np.random.default_rng(11)
    n = trees.echo_budget(rng, 64, 1024)
    assert n.sum() == 1024 and n.min() >= 8 and n.max() <= 64
    t = trees.eagle2_tree(np.random.default_rng(1), 64, 5, 8)
    assert len(t) == 64 and T.depth(t).max() <= 8
