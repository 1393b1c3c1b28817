"""Pins of the oracle's acceptance walk.

* Closed form (CSDN page, section 7.2): with a constant acceptance rate alpha
  and gamma drafts, E[L] = (1 - alpha^(gamma+1)) / (1 - alpha); alpha -> 1
  gives gamma + 1, alpha -> 0 gives 1.  With context-free P and Q,
  alpha = sum_x min(P(x), Q(x)) (expected value of min(1, p/q) under q).
* Losslessness (CSDN page 7.1, guijiagi post): the emitted token follows p;
  checked by chi-square on a 16-token vocabulary for a chain and for a tree
  with two i.i.d. children per node.
* Mutation tests plant plausible mistakes in a copy of the oracle and check
  that the statistical pins catch them.
* Greedy (survey page 8.1): the path is the longest draft prefix that agrees
  with the target's argmax, found here by brute force over all tree nodes.
"""
import inspect
import types

import numpy as np
import pytest
import scipy.special
import scipy.stats

from oracle import accept as AC
from oracle import philox
from oracle import tree as T
from workloads import trees

V = 16


def _pq(seed, sigma_p=1.5, sigma_q=1.0):
    rng = np.random.default_rng(seed)
    pl = rng.standard_normal(V) * sigma_p
    ql = pl + rng.standard_normal(V) * sigma_q
    return scipy.special.softmax(pl), scipy.special.softmax(ql)


def _run(walk_mod, parents, P, Q, trials, seed, draft_rng_seed):
    """Run ``trials`` independent requests on a context-free P/Q."""
    n = len(parents)
    rng = np.random.default_rng(draft_rng_seed)
    toks = rng.choice(V, size=(trials, n), p=Q)      # drafter: i.i.d. draws from Q
    b = np.arange(trials, dtype=np.uint64)[:, None]
    rows = np.arange(n, dtype=np.uint64)[None, :]
    ca = philox.uniform(seed, 0, b, rows, 0)
    cs = philox.uniform(seed, 0, b, rows, 1)
    Pm = np.broadcast_to(P, (n, V))
    Qm = np.broadcast_to(Q, (n, V))
    out = []
    for t in range(trials):
        out.append(walk_mod.walk_sampling(parents, toks[t], Pm, Qm, ca[t], cs[t]))
    return out


def test_softmax_and_temperature_match_scipy():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((5, 300)) * 4
    np.testing.assert_allclose(AC.softmax(x), scipy.special.softmax(x, axis=1), rtol=1e-14)
    np.testing.assert_allclose(AC.distributions(x, 0.7), scipy.special.softmax(x / 0.7, axis=1),
                               rtol=1e-13)


def test_inverse_cdf_small_cases():
    w = np.array([0.0, 1.0, 0.0, 1.0])
    assert AC.sample_inverse_cdf(w, 0.25)[0] == 1
    assert AC.sample_inverse_cdf(w, 0.5)[0] == 3       # boundary goes to the next index
    assert AC.sample_inverse_cdf(w, 0.0)[0] == 1       # zero weights are never drawn
    rng = np.random.default_rng(1)
    for _ in range(200):
        w = rng.random(37) * (rng.random(37) < 0.6)
        r = rng.random()
        t, _ = AC.sample_inverse_cdf(w, r)
        assert t == np.searchsorted(np.cumsum(w), r * w.sum(), side="right")


def test_expected_length_closed_form_chain():
    gamma = 8
    P, Q = _pq(0)
    alpha = np.minimum(P, Q).sum()
    assert 0.5 < alpha < 0.9
    trials = 200000
    res = _run(AC, trees.chain(gamma), P, Q, trials, seed=11, draft_rng_seed=12)
    L = np.array([r.accept_len + 1 for r in res], dtype=np.float64)
    expect = (1 - alpha ** (gamma + 1)) / (1 - alpha)
    assert abs(L.mean() - expect) / expect < 0.01, (L.mean(), expect)
    # every draw emits exactly accept_len + 1 tokens
    assert all(len(r.tokens) == r.accept_len + 1 for r in res[:1000])


def test_alpha_one_accepts_everything():
    P, _ = _pq(4)
    res = _run(AC, trees.chain(6), P, P, 2000, seed=1, draft_rng_seed=2)
    assert all(r.accept_len == 6 for r in res)


def test_disjoint_support_rejects_first_and_emits_p():
    P = np.zeros(V)
    P[:8] = np.arange(1, 9)
    P /= P.sum()
    Q = np.zeros(V)
    Q[8:] = 1.0 / 8
    res = _run(AC, trees.chain(5), P, Q, 40000, seed=3, draft_rng_seed=4)
    assert all(r.accept_len == 0 for r in res)
    first = np.array([r.tokens[0] for r in res])
    _chi2_ok(first, P)


def _chi2_pvalue(samples, P):
    counts = np.bincount(samples, minlength=V).astype(np.float64)
    exp = P * len(samples)
    keep = exp >= 5
    c = np.append(counts[keep], counts[~keep].sum())
    e = np.append(exp[keep], exp[~keep].sum())
    if e[-1] == 0:
        c, e = c[:-1], e[:-1]
        assert counts[~keep].sum() == 0
    return scipy.stats.chisquare(c, e).pvalue


def _chi2_ok(samples, P):
    p = _chi2_pvalue(samples, P)
    assert p > 1e-3, p


def test_lossless_chain_chi_square():
    P, Q = _pq(5)
    res = _run(AC, trees.chain(4), P, Q, 100000, seed=21, draft_rng_seed=22)
    _chi2_ok(np.array([r.tokens[0] for r in res]), P)


def test_lossless_two_child_tree_chi_square():
    P, Q = _pq(6, sigma_q=1.5)
    res = _run(AC, trees.cartesian((2, 2)), P, Q, 100000, seed=31, draft_rng_seed=32)
    first = np.array([r.tokens[0] for r in res])
    _chi2_ok(first, P)
    # the second child is reached often enough for the residual rule to matter
    assert np.mean([any(k == "accept" and row == 2 for k, row, _ in r.decisions) for r in res]) > 0.1


def _mutant(old, new):
    src = inspect.getsource(AC)
    assert old in src
    mod = types.ModuleType("oracle_accept_mutant")
    mod.__dict__["__name__"] = "oracle.accept_mutant"
    mod.__dict__["__package__"] = "oracle"
    exec(compile(src.replace(old, new), "accept_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("old,new", [
    ("                R = w / Z", "                pass"),                       # no residual
    ("            if r * Qu[x] < R[x]:", "            if r * Qu[x] < P[u][x]:"),  # stale target
    ("w = np.maximum(0.0, R - Qu)", "w = np.abs(R - Qu)"),                        # wrong residual
])
def test_planted_mistakes_fail_the_tree_chi_square(old, new):
    mut = _mutant(old, new)
    P, Q = _pq(6, sigma_q=1.5)
    res = _run(mut, trees.cartesian((2, 2)), P, Q, 100000, seed=31, draft_rng_seed=32)
    assert _chi2_pvalue(np.array([r.tokens[0] for r in res]), P) < 1e-6


def _greedy_brute(parents, tokens, p_logits):
    """Deepest node whose every edge token equals its parent's argmax."""
    n = len(parents)
    best = 0
    for v in range(n):
        path = T.ancestors(parents, v)[::-1]
        ok = all(int(tokens[c]) == int(np.argmax(p_logits[u])) for u, c in zip(path, path[1:]))
        if ok and len(path) > len(T.ancestors(parents, best)):
            best = v
    path = T.ancestors(parents, best)[::-1]
    return path, [int(tokens[c]) for c in path[1:]] + [int(np.argmax(p_logits[best]))]


def test_greedy_is_longest_matching_prefix():
    rng = np.random.default_rng(9)
    for trial in range(200):
        parents = [trees.chain(8), trees.cartesian((3, 3)), trees.k_schedule((3, 2, 1))][trial % 3]
        n = len(parents)
        pl = rng.standard_normal((n, 12))
        kids = T.children(parents)
        tokens = np.zeros(n, dtype=np.int64)
        for u in range(n):
            if kids[u]:
                # distinct sibling tokens; the argmax is among them half the time
                choice = rng.permutation(12)[:len(kids[u])]
                if rng.random() < 0.7:
                    choice[rng.integers(len(choice))] = int(np.argmax(pl[u]))
                    choice = _dedupe(choice, int(np.argmax(pl[u])), rng)
                tokens[kids[u]] = choice
        res = AC.walk_greedy(parents, tokens, pl)
        path, toks = _greedy_brute(parents, tokens, pl)
        assert res.path == path and res.tokens == toks


def _dedupe(choice, keep, rng):
    seen = {keep}
    out = []
    placed = False
    for c in choice:
        if c == keep and not placed:
            out.append(c)
            placed = True
            continue
        while c in seen:
            c = int(rng.integers(12))
        seen.add(c)
        out.append(c)
    return np.array(out)


def test_greedy_duplicate_siblings_take_lowest_row():
    parents = np.array([-1, 0, 0, 1, 2])
    pl = np.zeros((5, 4))
    pl[:, 2] = 1.0
    tokens = np.array([0, 2, 2, 1, 2])     # rows 1 and 2 both match; row 1 chosen
    res = AC.walk_greedy(parents, tokens, pl)
    assert res.path == [0, 1] and res.tokens == [2, 2]


def test_child_probabilities_are_parent_distribution_gathers():
    rng = np.random.default_rng(2)
    parents = trees.cartesian((2, 3))
    n = len(parents)
    pl = rng.standard_normal((n, 50)) * 3
    ql = pl + rng.standard_normal((n, 50))
    tokens = rng.integers(0, 50, size=n)
    out = AC.accept_request(parents, tokens, pl, ql, 1.0, seed=0, step=0, request=0)
    Ps = scipy.special.softmax(pl, axis=1)
    Qs = scipy.special.softmax(ql, axis=1)
    for c in range(1, n):
        u = parents[c]
        assert out["child_p"][c] == pytest.approx(Ps[u, tokens[c]], rel=1e-13)
        assert out["child_q"][c] == pytest.approx(Qs[u, tokens[c]], rel=1e-13)
    assert np.isnan(out["child_p"][0])
    g = AC.accept_request(parents, tokens, pl, None, 0.0, 0, 0, 0)
    assert set(np.unique(g["child_p"][1:])) <= {0.0, 1.0}
