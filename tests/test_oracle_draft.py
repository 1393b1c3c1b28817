"""Pins of the oracle's dynamic draft-tree builder (EAGLE-2 rounds, ECHO budget).

* The EAGLE-2 paragraph's count (cnblogs page, draft-tree generation): with
  K = 5 the second round leaves 25 leaves and only 5 of them are expanded.
* Scores are the float32 product of the path's probabilities: recomputed by
  walking each node's path from the root.
* The frontier is the top K of the bottom layer by that product: brute force
  over the layer.
* The selection keeps every root plus the K_max - B best non-root nodes of
  the batch (brute-force pairwise check), never more than max_rows rows per
  request, and each request's rows form a valid flattened tree.
* Checkpoints cut low-confidence branches; confident requests take the
  budget that weak ones leave (ECHO section).
"""
import numpy as np
import pytest

from oracle import draft as DR
from oracle import tree as T


def _cands(rng, rounds, B, K, V=1000, conf=None):
    toks = np.zeros((rounds, B, K, K), dtype=np.int32)
    probs = np.zeros((rounds, B, K, K), dtype=np.float32)
    for r in range(rounds):
        for b in range(B):
            c = 1.0 if conf is None else conf[b]
            for i in range(K):
                toks[r, b, i] = rng.choice(V, size=K, replace=False)
                z = rng.standard_normal(K + 3) * 2.0 * c
                p = np.exp(z - z.max())
                p = np.sort(p / p.sum())[::-1][:K]
                probs[r, b, i] = p.astype(np.float32)
    return toks, probs


def test_eagle2_second_round_has_25_leaves_and_expands_5():
    rng = np.random.default_rng(0)
    K = 5
    toks, probs = _cands(rng, 3, 1, K)
    t = DR.begin(7, capacity=200)
    DR.expand(t, toks[0, 0], probs[0, 0], K)
    assert t.count == 1 + 5 and len(t.frontier) == 5
    DR.expand(t, toks[1, 0], probs[1, 0], K)
    leaves = [v for v in range(t.count) if t.depth[v] == 2]
    assert len(leaves) == 25
    assert len(t.frontier) == 5 and set(t.frontier) <= set(leaves)
    DR.expand(t, toks[2, 0], probs[2, 0], K)
    assert t.count == 1 + 5 + 25 + 25
    assert {t.parent[v] for v in range(31, 56)} == set(
        sorted(leaves, key=lambda v: (-float(t.score[v]), v))[:5])


def test_scores_are_path_products_and_frontier_is_top_k_of_bottom_layer():
    rng = np.random.default_rng(1)
    K, rounds = 4, 6
    toks, probs = _cands(rng, rounds, 1, K)
    t = DR.begin(0, capacity=1000)
    prob_of = {0: None}
    for r in range(rounds):
        front = list(t.frontier)
        first = t.count
        DR.expand(t, toks[r, 0], probs[r, 0], K)
        for i, u in enumerate(front):
            for j in range(K):
                prob_of[first + i * K + j] = probs[r, 0, i, j]
        # brute force: product along the path, root first, in float32
        for v in range(first, t.count):
            path = []
            w = v
            while w != 0:
                path.append(w)
                w = t.parent[w]
            s = np.float32(1)
            for w in reversed(path):
                s = np.float32(s * prob_of[w])
            assert s == t.score[v]
            assert t.token[v] == toks[r, 0, front.index(t.parent[v]), (v - first) % K]
        layer = list(range(first, t.count))
        best = sorted(layer, key=lambda v: (-float(t.score[v]), v))[:K]
        assert t.frontier == best
        # every new node is one deeper than its parent, and the frontier sits on it
        assert all(t.depth[v] == r + 1 for v in layer)


def test_selection_is_the_global_top_and_forms_trees():
    rng = np.random.default_rng(2)
    B, K, rounds = 6, 3, 5
    conf = rng.exponential(1.0, size=B)
    toks, probs = _cands(rng, rounds, B, K, conf=conf)
    for budget, max_rows in [(40, 64), (6, 64), (25, 5), (10 ** 4, 256)]:
        trees, (ro, par, tok, node) = DR.build(np.arange(B), toks, probs, K, 1000, (), budget,
                                              max_rows)
        n = np.diff(ro)
        assert (n >= 1).all() and (n <= max_rows).all()
        total_nodes = sum(min(t.count, max_rows) for t in trees)
        assert ro[-1] == min(budget, total_nodes) if budget >= B else ro[-1] == B
        kept = set()
        for b in range(B):
            p = par[ro[b]:ro[b + 1]]
            T.validate(p)
            nodes = node[ro[b]:ro[b + 1]]
            assert nodes[0] == 0 and list(nodes) == sorted(nodes)
            assert list(tok[ro[b]:ro[b + 1]]) == [trees[b].token[v] for v in nodes]
            for i in range(1, len(nodes)):
                assert nodes[p[i]] == trees[b].parent[nodes[i]]
            kept |= {(b, int(v)) for v in nodes[1:]}
        # pairwise: a kept node outranks every node left out (unless the cap excluded it)
        def key(bv):
            b, v = bv
            return (-float(trees[b].score[v]), b, v)

        def capped(bv):
            b, v = bv
            order = sorted(range(1, trees[b].count), key=lambda w: (-float(trees[b].score[w]), w))
            return order.index(v) >= max_rows - 1
        left = [(b, v) for b in range(B) for v in range(1, trees[b].count) if (b, v) not in kept]
        if kept:
            worst_kept = max(kept, key=key)
            for bv in left:
                assert capped(bv) or key(bv) > key(worst_kept)


def test_checkpoint_cuts_and_budget_moves_to_confident_requests():
    rng = np.random.default_rng(3)
    K, rounds = 3, 6
    toks, probs = _cands(rng, rounds, 2, K)
    # a checkpoint at depth 2 above every score cuts growth there
    trees, _ = DR.build([0, 0], toks, probs, K, 1000, [(2, 1.5)], 10, 64)
    for t in trees:
        assert max(t.depth) == 2 and t.frontier == []
        assert t.count == 1 + K + K * K
    # threshold 0 changes nothing
    a, sa = DR.build([0, 0], toks, probs, K, 1000, [(2, 0.0)], 30, 64)
    b, sb = DR.build([0, 0], toks, probs, K, 1000, (), 30, 64)
    assert all(np.array_equal(x, y) for x, y in zip(sa, sb))
    # request 0 drafts with near-certain probabilities, request 1 with weak ones
    probs2 = probs.copy()
    probs2[:, 0] = np.float32(0.9)
    probs2[:, 1] = np.float32(0.05)
    trees, (ro, *_ ) = DR.build([0, 0], toks, probs2, K, 1000, [(3, 1e-3)], 30, 64)
    n = np.diff(ro)
    assert n[0] == 29 and n[1] == 1
    assert max(trees[1].depth) == 3 and trees[1].frontier == []


def test_capacity_flag_and_probability_clamp():
    K = 2
    t = DR.begin(0, capacity=5)
    DR.expand(t, [[1, 2]], [[np.float32(2.0), np.float32(np.nan)]], K)
    assert t.score[1] == 1.0 and t.score[2] == 0.0          # clamped to [0, 1]
    DR.expand(t, [[3, 4], [5, 6]], [[0.5, 0.4], [0.3, 0.2]], K)   # 3 + 4 > 5
    assert t.flags == DR.FLAG_CAPACITY and t.count == 3 and t.frontier == []
