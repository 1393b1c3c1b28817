"""Pins of the acceptance oracle's edge branches and of its near-threshold flags.

* Zero residual (CSDN page "推理加速：推测解码与级联推理", section 7.1): after a
  rejection the next target is norm(max(0, p - q)), which has no value when
  p <= q everywhere.  Reading: keep R and raise the zero-residual flag.  The
  branch is reached exactly when Q_u = P_u (the same logits) and the drafted
  token has P_u(x) = Q_u(x) = 0: r * 0 < 0 fails for every coin, and the
  residual mass sum(max(0, P - Q)) is exactly 0.  With R kept, a second
  child's test is r * Q(x) < P(x) = Q(x), true for every r < 1; with one child
  only, the final token is a draw from P_u.
* Flag windows: the margins the parity comparison uses to decide which
  decisions are too close to their thresholds to compare, checked on hand
  cases where the margin is known in closed form (a coin on a cumulative
  boundary, a coin at the ratio R/Q, probabilities that underflow).

Each pin is checked against planted mistakes in a copy of the oracle: every
mutant must fail it.
"""
import inspect
import types

import numpy as np
import pytest
import scipy.special
import scipy.stats

from oracle import accept as AC
from oracle import philox

V = 16


def _mutant(old, new):
    src = inspect.getsource(AC)
    assert old in src, old
    mod = types.ModuleType("oracle_accept_mutant")
    mod.__dict__["__name__"] = "oracle.accept_mutant"
    mod.__dict__["__package__"] = "oracle"
    exec(compile(src.replace(old, new), "accept_mutant", "exec"), mod.__dict__)
    return mod


# -- zero residual ---------------------------------------------------------------
def _equal_rows(seed, n):
    """n identical target/draft distributions over V tokens; token 0 has logit
    -5000 below the others (probability exactly 0 in float64)."""
    rng = np.random.default_rng(seed)
    logits = rng.standard_normal(V) * 1.5
    logits[0] = -5000.0
    P = AC.distributions(np.tile(logits, (n, 1)), 1.0)
    assert P[0, 0] == 0.0 and (P[0, 1:] > 0).all()
    return P, P.copy()


def _coins(trials, n, seed):
    b = np.arange(trials, dtype=np.uint64)[:, None]
    rows = np.arange(n, dtype=np.uint64)[None, :]
    return philox.uniform(seed, 0, b, rows, 0), philox.uniform(seed, 0, b, rows, 1)


def _check_zero_residual_two_children(mod, trials=400):
    parents = np.array([-1, 0, 0])
    tokens = np.array([0, 0, 5])          # child 1 drafts the zero-probability token
    P, Q = _equal_rows(3, 3)
    ca, cs = _coins(trials, 3, seed=17)
    for t in range(trials):
        res = mod.walk_sampling(parents, tokens, P, Q, ca[t], cs[t])
        assert res.path == [0, 2], res.path
        assert res.tokens[0] == 5
        assert res.zero_residual
        kinds = [(k, row) for k, row, _ in res.decisions]
        assert kinds[:3] == [("accept", 1), ("residual", 1), ("accept", 2)]
        assert res.decisions[1][2] == 0.0            # the residual mass is exactly 0
        # neither the exact rejection nor the exact zero mass is near-threshold
        assert res.first_flag() in (None, len(res.decisions) - 1)


def _check_zero_residual_final_draw(mod, trials=60000):
    """One child, always rejected: the emitted token is a draw from the kept
    R = P_u (chi-square, 15 d.o.f.; P_u(0) = 0 is never drawn)."""
    parents = np.array([-1, 0])
    tokens = np.array([0, 0])
    P, Q = _equal_rows(4, 2)
    ca, cs = _coins(trials, 2, seed=23)
    first = np.empty(trials, dtype=np.int64)
    for t in range(trials):
        res = mod.walk_sampling(parents, tokens, P, Q, ca[t], cs[t])
        assert res.path == [0] and res.zero_residual
        first[t] = res.tokens[0]
    assert (first != 0).all()
    counts = np.bincount(first, minlength=V)[1:].astype(np.float64)
    exp = P[0, 1:] * trials
    assert scipy.stats.chisquare(counts, exp).pvalue > 1e-3


def test_zero_residual_keeps_target_and_raises_flag():
    _check_zero_residual_two_children(AC)


def test_zero_residual_final_draw_follows_target():
    _check_zero_residual_final_draw(AC)


@pytest.mark.parametrize("old,new", [
    # the residual replaces R even when it has no mass
    ("            else:                   # R <= Q_u everywhere: keep R, raise the flag\n"
     "                res.zero_residual = True",
     "            else:\n                R = w\n                res.zero_residual = True"),
    # the flag is forgotten
    ("                res.zero_residual = True", "                pass"),
    # a zero mass is divided by
    ("            if Z > 0:\n                R = w / Z\n            else:                   #",
     "            if Z >= 0:\n                R = w / Z\n            else:                   #"),
    # the draft distribution replaces the kept target
    ("                res.zero_residual = True",
     "                res.zero_residual = True\n                R = np.roll(Qu, 1)"),
])
def test_planted_mistakes_fail_the_zero_residual_pins(old, new):
    mut = _mutant(old, new)
    with np.errstate(all="ignore"):
        with pytest.raises(Exception):
            _check_zero_residual_two_children(mut)
            _check_zero_residual_final_draw(mut, trials=20000)


def test_topk_rejections_always_leave_mass():
    """Point-mass drafts (reading 10): a rejection needs r >= R(x), so R(x) < 1
    and the rest of R keeps positive mass; the branch that would keep R is
    unreachable.  Hammered with a token holding all but ~1e-12 of the mass."""
    rng = np.random.default_rng(5)
    logits = rng.standard_normal(V)
    logits[3] = 30.0                      # P(3) = 1 - O(1e-12)
    P = np.tile(AC.distributions(logits[None, :], 1.0), (3, 1))
    assert 1.0 - P[0, 3] < 1e-11 and P[0, 3] < 1.0
    parents = np.array([-1, 0, 0])
    tokens = np.array([0, 3, 3])
    # coins above R(3) reject child 1; its repeat (child 2) has R(3) = 0
    ca = np.array([0.0, np.nextafter(1.0, 0.0), 0.5])
    res = AC.walk_topk(parents, tokens, P, ca, np.full(3, 0.5))
    assert res.path == [0] and not res.zero_residual
    masses = [m for k, _, m in res.decisions if k == "residual"]
    assert len(masses) == 2 and all(m > 0 for m in masses)


# -- margins ------------------------------------------------------------------------
def _check_draw_margins(mod):
    w = np.array([1.0, 1.0, 2.0])           # cumulative 1, 2, 4; Z = 4
    t, m = mod.sample_inverse_cdf(w, 0.5)   # target 2: on the boundary of rows 1 and 2
    assert t == 2 and m == 0.0
    t, m = mod.sample_inverse_cdf(w, 0.3)   # target 1.2: 0.2 above row 1's lower edge
    assert t == 1 and abs(m - 0.2 / 4) < 1e-15
    t, m = mod.sample_inverse_cdf(w, 0.45)  # target 1.8: 0.2 below its upper edge
    assert t == 1 and abs(m - 0.2 / 4) < 1e-15
    t, m = mod.sample_inverse_cdf(w, 0.0)   # target 0: the lower edge of row 0
    assert t == 0 and m == 0.0
    t, m = mod.sample_inverse_cdf(w, 0.7)   # target 2.8: 0.8 into row 2, 1.2 below its top
    assert t == 2 and abs(m - 0.8 / 4) < 1e-15
    t, m = mod.sample_inverse_cdf(np.array([0.0, 3.0, 0.0]), 0.25)   # zero rows are skipped
    assert t == 1 and abs(m - 0.25) < 1e-15


def _check_accept_margins(mod):
    # R(x) = 0.3, Q(x) = 0.6: threshold r = 0.5 (strict: r = 0.5 rejects)
    assert mod.accept_margin(0.5, 0.3, 0.6) == 0.0
    assert abs(mod.accept_margin(0.2, 0.3, 0.6) - 0.3) < 1e-15
    assert abs(mod.accept_margin(0.5 - 1e-7, 0.3, 0.6) - 1e-7) < 1e-15
    # outcomes no coin can change
    assert mod.accept_margin(0.9, 0.0, 0.0) == np.inf       # rejects always
    assert mod.accept_margin(0.9, 0.25, 0.0) == np.inf      # accepts always
    # probabilities an exponential may flush to zero
    assert mod.accept_margin(0.1, 1e-305, 2e-305) == 0.0
    assert mod.accept_margin(0.1, 0.3, 1e-310) == 0.0
    assert mod.accept_margin(0.1, 1e-310, 0.0) == 0.0
    # R(x) = 0 with Q(x) > 0: rejects unless r < 0, distance r
    assert abs(mod.accept_margin(0.25, 0.0, 0.5) - 0.25) < 1e-15
    # the walk records exactly these margins and takes the strict decision
    parents = np.array([-1, 0])
    P = np.array([[0.3, 0.7], [0.5, 0.5]])
    Q = np.array([[0.6, 0.4], [0.5, 0.5]])
    for r, acc, m in [(0.5, False, 0.0), (0.5 - 1e-7, True, 1e-7), (0.2, True, 0.3)]:
        res = mod.walk_sampling(parents, np.array([0, 0]), P, Q, np.array([0.0, r]),
                                np.array([0.3, 0.3]))
        assert (res.path == [0, 1]) == acc
        kind, row, got = res.decisions[0]
        assert (kind, row) == ("accept", 1) and abs(got - m) < 1e-15
    # after a rejection the margin is taken against the residual: child 1
    # (token 0, coin 0.9) is rejected, R = max(0, P - Q) / 0.3 = [0, 1], and
    # child 2 (token 1, coin 0.5) is 2.5 - 0.5 = 2 from its threshold R/Q
    res = mod.walk_sampling(np.array([-1, 0, 0]), np.array([0, 0, 1]), np.vstack([P, P[:1]]),
                            np.vstack([Q, Q[:1]]), np.array([0.0, 0.9, 0.5]),
                            np.full(3, 0.3))
    assert res.path == [0, 2]
    assert [k for k, _, _ in res.decisions[:3]] == ["accept", "residual", "accept"]
    assert abs(res.decisions[1][2] - 0.3) < 1e-15 and abs(res.decisions[2][2] - 2.0) < 1e-15


def _check_first_flag(mod):
    W = mod.WalkResult
    r = W()
    r.decisions = [("accept", 1, 0.1), ("residual", 1, 0.0), ("sample", 0, 5e-7)]
    assert r.first_flag() is None          # exact zero mass; 5e-7 is outside the draw window
    r.decisions = [("accept", 1, 0.1), ("residual", 1, 1e-9), ("sample", 0, 0.3)]
    assert r.first_flag() == 1             # a positive mass within rounding of zero
    r.decisions = [("accept", 1, 0.1), ("accept", 2, 5e-7), ("sample", 0, 1e-10)]
    assert r.first_flag() == 1             # inside the child-test window
    r.decisions = [("accept", 1, 0.1), ("sample", 0, 1e-10)]
    assert r.first_flag() == 1
    assert r.first_flag(1e-6, 1e-11) is None
    # what the decisions before a flag fix
    r = W()
    r.path, r.tokens = [0, 2, 5], [7, 9, 4]
    r.decisions = [("accept", 1, 0.3), ("residual", 1, 0.4), ("accept", 2, 0.2),
                   ("accept", 5, 1e-8), ("sample", 5, 0.1)]
    assert r.prefix_before(3) == ([0, 2], [7], {1})
    assert r.prefix_before(None) == ([0, 2, 5], [7, 9], {1})
    assert r.prefix_before(0) == ([0], [], set())


def test_draw_margins():
    _check_draw_margins(AC)


def test_accept_margins():
    _check_accept_margins(AC)


def test_first_flag_windows_and_prefix():
    _check_first_flag(AC)


@pytest.mark.parametrize("check,old,new", [
    ("draw", "    margin = min(abs(target - lo), abs(c[t] - target)) / Z if Z > 0 else 0.0",
     "    margin = abs(c[t] - target) / Z if Z > 0 else 0.0"),
    ("draw", "    margin = min(abs(target - lo), abs(c[t] - target)) / Z if Z > 0 else 0.0",
     "    margin = min(abs(target - lo), abs(c[t] - target)) if Z > 0 else 0.0"),
    ("draw", "    lo = c[t - 1] if t > 0 else 0.0", "    lo = c[t] if t > 0 else 0.0"),
    ("accept", "    return abs(r - Rx / Qx)", "    return abs(r * Qx - Rx)"),
    ("accept", "    if 0.0 < Rx < TINY or 0.0 < Qx < TINY:", "    if 0.0 < Rx < TINY:"),
    ("accept", "        return np.inf            # accept iff R(x) > 0, whatever r",
     "        return 0.0 if Rx == 0.0 else np.inf"),
    ("accept", "            res.decisions.append((\"accept\", c, accept_margin(r, R[x], Qu[x])))",
     "            res.decisions.append((\"accept\", c, accept_margin(r, P[u][x], Qu[x])))"),
    ("flag", "                if 0.0 < m < eps_res:", "                if m < eps_res:"),
    ("flag", "            elif m < (eps_draw if kind == \"sample\" else eps):",
     "            elif m < eps:"),
    ("flag", "        accepted = [row for kind, row, _ in decs if kind == \"accept\" and row in self.path]",
     "        accepted = [row for kind, row, _ in self.decisions if kind == \"accept\" and row in self.path]"),
])
def test_planted_mistakes_fail_the_margin_pins(check, old, new):
    mut = _mutant(old, new)
    fn = {"draw": _check_draw_margins, "accept": _check_accept_margins,
          "flag": _check_first_flag}[check]
    with pytest.raises(Exception):
        fn(mut)


# -- comparison up to the first flagged decision ---------------------------------
def _pad(x, S=6):
    return list(x) + [-1] * (S - len(x))


def test_check_outputs_compares_up_to_the_first_flag():
    r = AC.WalkResult()
    r.path, r.tokens = [0, 2, 5], [7, 9, 4]
    r.decisions = [("accept", 1, 0.3), ("residual", 1, 0.4), ("accept", 2, 0.2),
                   ("accept", 5, 1e-8), ("sample", 5, 0.1)]
    assert r.check_outputs(2, _pad([0, 2, 5]), _pad([7, 9, 4])) == (True, True)
    # after the flagged test of row 5: row 5 rejected instead, another final token
    assert r.check_outputs(1, _pad([0, 2]), _pad([7, 11])) == (True, False)
    bad = [(1, [0, 1], [3, 8]),          # continues through row 1, rejected before the flag
           (2, [0, 2, 5], [8, 9, 4]),    # another token for the accepted row 2
           (0, [0], [7]),                # stops before row 2, accepted before the flag
           (2, [0, 3, 5], [7, 9, 4])]    # another accepted row
    for alen, path, toks in bad:
        with pytest.raises(AssertionError):
            r.check_outputs(alen, _pad(path), _pad(toks))
    # a zero residual before the flag must be reported
    r.decisions[1] = ("residual", 1, 0.0)
    r.zero_residual = True
    assert r.check_outputs(2, _pad([0, 2, 5]), _pad([7, 9, 4]), flags=1)[0]
    with pytest.raises(AssertionError):
        r.check_outputs(2, _pad([0, 2, 5]), _pad([7, 9, 4]), flags=0)
    # without a flag every output is compared, flags and accept mask included
    r.decisions[3] = ("accept", 5, 0.2)
    assert r.check_outputs(2, _pad([0, 2, 5]), _pad([7, 9, 4]), flags=1,
                           accept_mask=[1, 0, 1, 0, 0, 1]) == (False, True)
    for kw in (dict(alen=2, path=[0, 2, 5], toks=[7, 9, 3]),
               dict(alen=2, path=[0, 2, 5], toks=[7, 9, 4], flags=0),
               dict(alen=2, path=[0, 2, 5], toks=[7, 9, 4], accept_mask=[1, 1, 1, 0, 0, 1]),
               dict(alen=1, path=[0, 2], toks=[7, 9])):
        with pytest.raises(AssertionError):
            r.check_outputs(kw["alen"], _pad(kw["path"]), _pad(kw["toks"]),
                            flags=kw.get("flags"), accept_mask=kw.get("accept_mask"))
