"""Pins of the oracle's tree attention.

* Tree decoding equals sequence-based decoding: every root-to-leaf branch,
  run as its own causal sequence after the prefix, gives the same outputs at
  its rows (the pages' tree-based vs sequence-based parallel decoding).  The
  sequence side uses torch's CPU scaled_dot_product_attention in float64.
* Closed forms: zero queries average the visible values; with an empty prefix
  the root sees only itself.
"""
import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import tree as T
from workloads import trees


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _sdpa_causal(q, k, v):
    """q [n][D] for the last n positions of k/v [m][D]; causal; float64."""
    n, m = q.shape[0], k.shape[0]
    qi = torch.from_numpy(q)[None, None]
    kk = torch.from_numpy(k)[None, None]
    vv = torch.from_numpy(v)[None, None]
    pos_q = torch.arange(m - n, m)[:, None]
    pos_k = torch.arange(m)[None, :]
    mask = pos_k <= pos_q
    out = torch.nn.functional.scaled_dot_product_attention(qi, kk, vv, attn_mask=mask)
    return out[0, 0].numpy()


def _case(parents, L, Hq, Hkv, D, seed):
    rng = np.random.default_rng(seed)
    N = len(parents)
    return (_rand(rng, N, Hq, D), _rand(rng, Hkv, L, D), _rand(rng, Hkv, L, D),
            _rand(rng, N, Hkv, D), _rand(rng, N, Hkv, D))


@pytest.mark.parametrize("parents,L,Hq,Hkv,D", [
    (trees.toy_tree(), 16, 4, 4, 8),
    (trees.cartesian((2, 3)), 10, 4, 2, 16),
    (trees.k_schedule((3, 2, 1)), 7, 6, 3, 8),
    (trees.eagle2_tree(np.random.default_rng(5), 24), 5, 2, 1, 8),
])
def test_tree_equals_per_branch_sequences(parents, L, Hq, Hkv, D):
    q, kp, vp, kt, vt = _case(parents, L, Hq, Hkv, D, seed=len(parents) + L)
    out = A.tree_attention(q, kp, vp, kt, vt, parents)
    G = Hq // Hkv
    kids = T.children(parents)
    leaves = [i for i in range(len(parents)) if not kids[i]]
    for leaf in leaves:
        path = T.ancestors(parents, leaf)[::-1]           # root .. leaf
        for h in range(Hq):
            kvh = h // G
            keys = np.concatenate([kp[kvh], kt[path, kvh]], axis=0)
            vals = np.concatenate([vp[kvh], vt[path, kvh]], axis=0)
            seq = _sdpa_causal(q[path, h], keys, vals)
            np.testing.assert_allclose(out[path, h], seq, rtol=0, atol=1e-12)


def test_chain_equals_prefix_causal_sdpa():
    parents = trees.chain(8)
    q, kp, vp, kt, vt = _case(parents, 33, 4, 4, 16, seed=1)
    out = A.tree_attention(q, kp, vp, kt, vt, parents)
    for h in range(4):
        keys = np.concatenate([kp[h], kt[:, h]], axis=0)
        vals = np.concatenate([vp[h], vt[:, h]], axis=0)
        np.testing.assert_allclose(out[:, h], _sdpa_causal(q[:, h], keys, vals), atol=1e-12)


def test_zero_query_averages_visible_values():
    parents = trees.toy_tree()
    q, kp, vp, kt, vt = _case(parents, 12, 2, 2, 4, seed=2)
    q[:] = 0
    out = A.tree_attention(q, kp, vp, kt, vt, parents)
    M = T.ancestor_mask(parents)
    for i in range(len(parents)):
        for h in range(2):
            vis = np.concatenate([vp[h], vt[M[i], h]], axis=0)
            np.testing.assert_allclose(out[i, h], vis.mean(axis=0), atol=1e-13)


def test_empty_prefix_root_sees_only_itself():
    parents = trees.cartesian((2, 2))
    q, kp, vp, kt, vt = _case(parents, 0, 2, 1, 8, seed=3)
    out = A.tree_attention(q, kp, vp, kt, vt, parents)
    for h in range(2):
        np.testing.assert_allclose(out[0, h], vt[0, 0], atol=1e-15)


def test_gqa_head_mapping():
    """Query head h uses KV head h // G: swapping KV heads swaps output groups."""
    parents = trees.chain(3)
    q, kp, vp, kt, vt = _case(parents, 9, 4, 2, 8, seed=4)
    out = A.tree_attention(q, kp, vp, kt, vt, parents)
    q2 = q[:, [2, 3, 0, 1]]
    out2 = A.tree_attention(q2, kp[::-1], vp[::-1], kt[:, ::-1], vt[:, ::-1], parents)
    np.testing.assert_allclose(out2[:, [2, 3, 0, 1]], out, atol=1e-13)


# -- arbitrary visibility of the new rows (lookahead-style and random masks) --
from workloads import masks  # noqa: E402


def test_lookahead_mask_counts():
    """Survey page, lookahead decoding 8.2.3 and 8.3.2: with W=5, N=4, G=5 the
    lookahead branch adds W(N-1)-1 rows to "0" and the verify branch G(N-1),
    W(N-1) + G(N-1) = 30 rows in one pass."""
    m = masks.lookahead_visibility(5, 4, 5)
    assert m.shape == (30, 30)
    assert m[:, 0].all()                          # everyone sees "0"
    la = list(range(1, 15))
    ve = list(range(15, 30))
    assert not m[np.ix_(la, ve)].any() and not m[np.ix_(ve, la)].any()
    assert not np.triu(m, 1).any()                # causal


def test_lookahead_mask_equals_two_causal_branches():
    """Each branch, run as its own causal sequence "0", b_1, b_2, ... after the
    prefix, gives the masked outputs at its rows (torch SDPA, float64)."""
    vis = masks.lookahead_visibility(3, 3, 2)     # "0" + 5 lookahead + 4 verify rows
    n = vis.shape[0]
    rng = np.random.default_rng(11)
    Hq, Hkv, D, L = 4, 2, 8, 9
    q, kp, vp = _rand(rng, n, Hq, D), _rand(rng, Hkv, L, D), _rand(rng, Hkv, L, D)
    kt, vt = _rand(rng, n, Hkv, D), _rand(rng, n, Hkv, D)
    out = A.masked_attention(q, kp, vp, kt, vt, vis)
    for rows in ([0, 1, 2, 3, 4, 5], [0, 6, 7, 8, 9]):
        for h in range(Hq):
            kvh = h // (Hq // Hkv)
            keys = np.concatenate([kp[kvh], kt[rows, kvh]], axis=0)
            vals = np.concatenate([vp[kvh], vt[rows, kvh]], axis=0)
            np.testing.assert_allclose(out[rows, h], _sdpa_causal(q[rows, h], keys, vals),
                                       rtol=0, atol=1e-12)


def test_random_mask_zero_query_and_single_key():
    rng = np.random.default_rng(12)
    n, Hq, Hkv, D = 7, 2, 1, 4
    vis = masks.random_visibility(rng, n, 0.4)
    q, kp, vp = np.zeros((n, Hq, D)), _rand(rng, Hkv, 5, D), _rand(rng, Hkv, 5, D)
    kt, vt = _rand(rng, n, Hkv, D), _rand(rng, n, Hkv, D)
    out = A.masked_attention(q, kp, vp, kt, vt, vis)
    for i in range(n):
        visv = np.concatenate([vp[0], vt[vis[i], 0]], axis=0)
        for h in range(Hq):
            np.testing.assert_allclose(out[i, h], visv.mean(axis=0), atol=1e-13)
    # empty prefix, each row seeing exactly one (possibly later) row
    pick = rng.integers(0, n, n)
    one = np.zeros((n, n), dtype=bool)
    one[np.arange(n), pick] = True
    q2 = _rand(rng, n, Hq, D)
    out2 = A.masked_attention(q2, kp[:, :0], vp[:, :0], kt, vt, one)
    for i in range(n):
        for h in range(Hq):
            np.testing.assert_allclose(out2[i, h], vt[pick[i], 0], atol=1e-15)
