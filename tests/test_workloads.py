"""The synthetic input recipes (workloads/): options used by the tests and the
benchmark produce what their docstrings state."""
import numpy as np

import workloads as W


def test_topk_workload_children_are_the_drafters_top_choices():
    w = W.make("medusa", L=64, V=300, Hq=2, Hkv=2, draft="topk")
    q = w.host("q_logits")
    for u in np.nonzero(w.nonleaf)[0]:
        kids = [c for c in range(len(w.parents)) if c > 0 and w.parents[c] == u]
        order = np.argsort(-q[u], kind="stable")
        assert list(w.tokens[kids]) == list(order[:len(kids)])


def test_prefix_lengths_match_make():
    for name, kw in [("dynamic", dict(B=5, L=("uniform", 10, 900), V=100, Hq=2, Hkv=1)),
                     ("specinfer", dict(B=2, L=64, V=100, Hq=2, Hkv=1))]:
        assert np.array_equal(W.gen.prefix_lengths(name, **kw), W.make(name, **kw).prefix_len)


def test_given_trees_and_tokens():
    trees = [np.array([-1, 0, 0, 1]), np.array([-1])]
    w = W.make("dynamic", B=2, L=[5, 7], V=50, Hq=2, Hkv=1, tree=("given", trees),
               given_tokens=np.arange(5))
    assert list(w.parents) == [-1, 0, 0, 1, -1] and list(w.row_offsets) == [0, 4, 5]
    assert list(w.tokens) == [0, 1, 2, 3, 4] and list(w.prefix_len) == [5, 7]


def test_drafter_candidates():
    toks, probs = W.drafts.candidates(3, 4, 5, 1000, seed=9)
    assert toks.shape == probs.shape == (3, 4, 5, 5)
    t, p = toks.numpy(), probs.numpy()
    assert all(len(set(t[r, b, i])) == 5 for r in range(3) for b in range(4) for i in range(5))
    assert (np.diff(p, axis=-1) <= 0).all() and (p > 0).all() and (p.sum(-1) <= 1 + 1e-6).all()
    t2, p2 = W.drafts.candidates(3, 4, 5, 1000, seed=9)
    assert np.array_equal(t, t2.numpy()) and np.array_equal(p, p2.numpy())


def test_head_operands_shapes_scale_and_seeding():
    w = W.make("chain8", L=64, V=3000, Hq=4, Hkv=4)
    h, wt = W.heads.head_inputs(w, H=256)
    assert h.shape == (w.R, 256) and wt.shape == (3000, 256)
    assert h.dtype == wt.dtype and str(h.dtype) == "torch.bfloat16"
    s = float(wt.float().std()) * 256 ** 0.5
    assert 2.8 < s < 3.2
    h2, wt2 = W.heads.head_inputs(w, H=256)
    assert bool((h == h2).all()) and bool((wt == wt2).all())
    assert W.heads.head_inputs(w)[0].shape == (w.R, w.Hq * w.D)
