"""Pins of the oracle's walk for deterministic (top-k) children.

Each child is a draft from the point mass at its token; the walk is then
sampling from the target distribution without replacement (oracle reading
10), which fixes these facts independently of the code:

* the first emitted token follows P exactly, whatever the sibling tokens
  (chi-square on a 16-token vocabulary, context-free P);
* child i of the root is taken with probability P(x_i) exactly (distinct
  tokens), so children that cover the vocabulary are always accepted;
* a sibling that repeats a rejected token is never taken;
* on a chain with fixed tokens, E[accepted] = sum_k prod_{i<=k} P(x_i).

Planted mistakes in a copy of the oracle must fail the chi-square pin.
"""
import inspect
import types

import numpy as np
import pytest
import scipy.special
import scipy.stats

from oracle import accept as AC
from oracle import philox
from workloads import trees

V = 16


def _p(seed, sigma=1.5):
    rng = np.random.default_rng(seed)
    return scipy.special.softmax(rng.standard_normal(V) * sigma)


def _run(mod, parents, tokens, P, trials, seed):
    n = len(parents)
    b = np.arange(trials, dtype=np.uint64)[:, None]
    rows = np.arange(n, dtype=np.uint64)[None, :]
    ca = philox.uniform(seed, 0, b, rows, 0)
    cs = philox.uniform(seed, 0, b, rows, 1)
    Pm = np.broadcast_to(P, (n, V))
    return [mod.walk_topk(parents, tokens, Pm, ca[t], cs[t]) for t in range(trials)]


def _topk_tokens(parents, P, offset=0):
    """Children of every node get distinct tokens in descending P order."""
    order = np.argsort(-P, kind="stable")
    kids = [[] for _ in parents]
    for c in range(1, len(parents)):
        kids[parents[c]].append(c)
    tokens = np.zeros(len(parents), dtype=np.int64)
    for u, ks in enumerate(kids):
        for i, c in enumerate(ks):
            tokens[c] = order[(i + offset) % V]
    return tokens


def _chi2_pvalue(samples, P):
    counts = np.bincount(samples, minlength=V).astype(np.float64)
    exp = P * len(samples)
    keep = exp >= 5
    c, e = counts[keep], exp[keep]
    if (~keep).any():
        c = np.append(c, counts[~keep].sum())
        e = np.append(e, exp[~keep].sum())
    return scipy.stats.chisquare(c, e).pvalue


def _binom_ok(hits, trials, p):
    z = (hits - trials * p) / np.sqrt(trials * p * (1 - p))
    assert abs(z) < 4.5, (hits, trials, p, z)


def test_first_token_follows_p_and_children_taken_with_their_mass():
    P = _p(1)
    parents = trees.cartesian((3, 2))
    tokens = _topk_tokens(parents, P)
    trials = 100000
    res = _run(AC, parents, tokens, P, trials, seed=41)
    first = np.array([r.tokens[0] for r in res])
    assert _chi2_pvalue(first, P) > 1e-3
    for c in (1, 2, 3):
        hits = sum(1 for r in res if len(r.path) > 1 and r.path[1] == c)
        _binom_ok(hits, trials, P[tokens[c]])
    # second level: given the walk sits on row 1, its first child follows P too
    on1 = [r for r in res if len(r.path) > 1 and r.path[1] == 1]
    second = np.array([r.tokens[1] for r in on1])
    assert _chi2_pvalue(second, P) > 1e-3


def test_children_covering_the_vocabulary_are_always_accepted():
    P = _p(2)
    parents = np.array([-1] + [0] * V)
    rng = np.random.default_rng(3)
    tokens = np.concatenate([[0], rng.permutation(V)])
    res = _run(AC, parents, tokens, P, 20000, seed=42)
    assert all(r.accept_len == 1 for r in res)
    first = np.array([r.tokens[0] for r in res])
    assert _chi2_pvalue(first, P) > 1e-3


def test_repeated_sibling_token_is_never_taken():
    P = _p(4)
    a, b = int(np.argmax(P)), int(np.argsort(-P)[1])
    parents = np.array([-1, 0, 0, 0])
    tokens = np.array([0, a, a, b])
    trials = 40000
    res = _run(AC, parents, tokens, P, trials, seed=43)
    assert not any(len(r.path) > 1 and r.path[1] == 2 for r in res)
    _binom_ok(sum(1 for r in res if len(r.path) > 1 and r.path[1] == 3), trials, P[b])
    assert _chi2_pvalue(np.array([r.tokens[0] for r in res]), P) > 1e-3


def test_chain_expected_length_closed_form():
    P = np.full(V, 0.2 / (V - 2))
    P[3], P[7] = 0.5, 0.3
    gamma = 6
    tokens = np.array([0, 3, 3, 7, 3, 7, 3])
    trials = 100000
    res = _run(AC, trees.chain(gamma), tokens, P, trials, seed=44)
    L = np.array([r.accept_len for r in res], dtype=np.float64)
    expect = sum(np.prod(P[tokens[1:k + 1]]) for k in range(1, gamma + 1))
    var = L.var()
    assert abs(L.mean() - expect) < 5 * np.sqrt(var / trials), (L.mean(), expect)
    assert all(len(r.tokens) == r.accept_len + 1 for r in res[:1000])


def _mutant(old, new):
    src = inspect.getsource(AC)
    assert old in src
    mod = types.ModuleType("oracle_accept_mutant")
    mod.__dict__["__name__"] = "oracle.accept_mutant"
    mod.__dict__["__package__"] = "oracle"
    exec(compile(src.replace(old, new), "accept_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("old,new", [
    ("            w[x] = max(0.0, R[x] - 1.0)", "            pass"),      # rejected token kept
    ("            if r < R[x]:", "            if r < P[u][x]:"),           # stale target
    ("            R = w / Z\n        if not moved:",
     "            R = w\n        if not moved:"),                          # no renormalisation
])
def test_planted_mistakes_fail_the_chi_square(old, new):
    mut = _mutant(old, new)
    P = _p(1)
    parents = trees.cartesian((3, 2))
    tokens = _topk_tokens(parents, P)
    res = _run(mut, parents, tokens, P, 100000, seed=41)
    assert _chi2_pvalue(np.array([r.tokens[0] for r in res]), P) < 1e-6

