"""Lossless speculative acceptance over a draft tree (oracle; test infrastructure).

Pages followed:

* "【模型后训练与深度推理】9 推理加速：推测解码与级联推理" (CSDN), section 7.1:
  a draft token x is accepted with probability min(1, p(x)/q(x)); on
  rejection the token is drawn from norm(max(0, p - q)), which makes the
  output follow p exactly.  Section 7.2: the emitted length L counts the final
  corrected or accepted token.
* guijiagi.com speculative-decoding post, rejection-sampling section: drafts
  are tested in order, the first rejection resamples from the residual and
  ends the step; later drafts are discarded.
* "投机推理算法的常见优化手段" (cnblogs), tree-mask section: the target
  forward over the tree gives at node i the distribution of the next token in
  i's context, P(. | ancestors(i)); tree verification checks every token of
  every level instead of one sequence.
* "万字综述 10+ 种 LLM 投机采样推理加速方案", sections 4.3 and 8.1:
  temperature 0 means argmax sampling; greedy verification keeps the longest
  draft prefix that matches the target's own choices.

Readings taken where the pages are silent or garbled:

1. Row u's target logits give the distribution of u's *children* (the page's
   P(i | ancestors(i))); row u's draft logits are the distribution the
   children of u were drafted from.  Leaves' draft rows are never used.
2. A node with several children tests them one after another in ascending
   row order.  Child c (token x, coin r) is accepted iff r * Q_u(x) < R(x),
   where R starts at P_u; after a rejection R <- max(0, R - Q_u) / Z with
   Z = sum(max(0, R - Q_u)) (if Z == 0, R is kept and the step is flagged).
   On a chain this is exactly the pages' rule; with i.i.d. children from Q_u
   it stays lossless.
3. The walk also emits one more token where it stops: after every child of u
   is rejected, a draw from the current residual R; at a leaf, a draw from
   P_leaf (the "bonus" token the emitted-length formula counts).
4. The residual uses the full vectors norm(max(0, P - Q)) (the printed
   pseudo-code keeps only the scalar q(x), which cannot be subtracted from a
   vector; the section 7.1 formula is the reference).
5. Temperature T > 0 divides both target and draft logits; T = 0 is greedy.
6. sample(w, r): inverse CDF in vocabulary order with one uniform: the
   smallest t with sum_{y<=t} w_y > r * sum(w); if rounding leaves none, the
   last t with w_t > 0.
7. Comparison is strict and division-free; Q_u(x) = 0 accepts iff R(x) > 0.
8. Greedy: g = argmax of the target logits (lowest index on ties); move to the
   lowest-numbered child whose token is g, else emit g and stop.
9. Coins: Philox4x64-10, key (seed, 0), counter (step, request, row,
   purpose); purpose 0 = accept coin of draft row c, 1 = sampling coin of the
   node where the walk stops.  This layout is a convention (parity unpinned
   beyond GPU = oracle; the statistics it must produce are pinned).
10. Deterministic children (top-k drafts, as in Medusa or expansion trees;
   the pages give no rule): child c of u is taken as a draft from the point
   mass at its token x, so reading 2 with Q = delta_x accepts c iff r < R(x),
   and a rejection removes x from R (max(0, R - delta_x) / Z).  This is
   sampling from P_u without replacement, so the emitted token still follows
   P_u; no draft logits are used.  A sibling repeating a rejected token has
   R(x) = 0 and is never accepted.

Decisions whose outcome is within rounding of its threshold are reported as
flagged (windows of reading 11 below):

* a child test: |r - R(x)/Q_u(x)| < FLAG_EPS (1e-6), and every child test
  on a probability in (0, TINY), TINY = 1e-300: a float64 exponential may
  flush values below e^-708 (3.3e-308) to zero.  A test on R(x) = Q_u(x) = 0
  (both below e^-745 here, so zero anywhere) rejects for every coin and is
  not flagged, nor is Q_u(x) = 0 with R(x) >= TINY (accepts for every coin);
* a draw: the target r * Z within FLAG_EPS_DRAW * Z (1e-9) of a cumulative
  boundary.  This window is narrower because a vocabulary of 128256 entries
  puts that many boundaries in [0, Z]: a 1e-6 window would flag about a
  quarter of all draws, while a float64 evaluation places the boundaries
  within about 1e-11 * Z;
* a residual after a rejection: a mass Z with 0 < Z < FLAG_EPS_RES (1e-8).
  Renormalising by such a Z multiplies the ~1e-15 absolute rounding of the
  mass into a relative error above 1e-7 in every later test.  A mass of
  exactly 0 is not flagged: it arises only where R <= Q_u entry by entry,
  i.e. where both are the same distribution computed from the same logits,
  which any evaluation reproduces exactly (reading 2 keeps R and raises the
  zero-residual flag).

11. Parity compares a walk only up to its first flagged decision: the
    decisions before it fix the accepted prefix of the path and its tokens.
"""
from __future__ import annotations

import numpy as np

from .tree import children as tree_children
from .tree import validate

FLAG_EPS = 1e-6
FLAG_EPS_DRAW = 1e-9
FLAG_EPS_RES = 1e-8
TINY = 1e-300


def softmax(x: np.ndarray) -> np.ndarray:
    """Softmax of a float64 vector (or of each row of a matrix)."""
    x = np.asarray(x, dtype=np.float64)
    m = np.max(x, axis=-1, keepdims=True)
    e = np.exp(x - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def distributions(logits_rows: np.ndarray, temperature: float) -> np.ndarray:
    """softmax(logits / T) of each row, in float64."""
    return softmax(np.asarray(logits_rows, dtype=np.float64) / float(temperature))


def greedy_token(logits_row: np.ndarray) -> int:
    """argmax with the lowest index winning ties."""
    return int(np.argmax(np.asarray(logits_row, dtype=np.float64)))


def sample_inverse_cdf(w: np.ndarray, r: float):
    """Draw index t from unnormalised weights w with coin r (reading 6).

    Returns (t, margin): margin is the distance of r*Z to the nearest
    boundary of t's cumulative interval, divided by Z.
    """
    w = np.asarray(w, dtype=np.float64)
    Z = float(np.sum(w))
    target = r * Z
    c = np.cumsum(w)
    hit = np.nonzero(c > target)[0]
    if len(hit):
        t = int(hit[0])
    else:
        t = int(np.nonzero(w > 0)[0][-1])
    lo = c[t - 1] if t > 0 else 0.0
    margin = min(abs(target - lo), abs(c[t] - target)) / Z if Z > 0 else 0.0
    return t, margin


def accept_margin(r: float, Rx: float, Qx: float) -> float:
    """Distance of child test r * Q(x) < R(x) from its threshold, in coin
    units (|r - R(x)/Q(x)|); 0 for a test on a probability in (0, TINY),
    infinity for a test whose outcome no coin can change."""
    if 0.0 < Rx < TINY or 0.0 < Qx < TINY:
        return 0.0
    if Qx == 0.0:
        return np.inf            # accept iff R(x) > 0, whatever r
    return abs(r - Rx / Qx)


class WalkResult:
    """Outcome of one request's acceptance walk."""

    def __init__(self):
        self.path = [0]          # accepted rows, root first
        self.tokens = []         # emitted tokens (accepted drafts + final one)
        self.decisions = []      # (kind, row, margin) in walk order
        self.zero_residual = False

    @property
    def accept_len(self) -> int:
        return len(self.path) - 1

    def first_flag(self, eps: float = FLAG_EPS, eps_draw: float = FLAG_EPS_DRAW,
                   eps_res: float = FLAG_EPS_RES):
        """Index into ``decisions`` of the first near-threshold decision, or None.

        Kinds and their margins: "accept" (child row, |r - R(x)/Q(x)|),
        "sample" (node, distance of the target to the nearest cumulative
        boundary over Z), "residual" (rejected child row, the residual mass Z
        itself; flagged only when positive and below ``eps_res``)."""
        for i, (kind, _, m) in enumerate(self.decisions):
            if kind == "residual":
                if 0.0 < m < eps_res:
                    return i
            elif m < (eps_draw if kind == "sample" else eps):
                return i
        return None

    def prefix_before(self, i):
        """What the decisions before index ``i`` fix: (path prefix, tokens of
        that prefix's accepted children, rows rejected by those decisions).
        ``i = None`` means every decision."""
        decs = self.decisions if i is None else self.decisions[:i]
        accepted = [row for kind, row, _ in decs if kind == "accept" and row in self.path]
        rejected = {row for kind, row, _ in decs if kind == "accept" and row not in self.path}
        k = len(accepted)
        assert accepted == self.path[1:1 + k]
        return self.path[:1 + k], self.tokens[:k], rejected

    def check_outputs(self, accept_len, path_row, tokens_row, flags=None, accept_mask=None,
                      flag_eps=None, what=""):
        """Compare another implementation's outputs for this walk (accept_len,
        the path and tokens rows padded with -1, optionally its flags word and
        accept mask) with this result, up to the first flagged decision.

        Raises AssertionError on any difference the unflagged decisions fix:
        the accepted path prefix and its tokens, no continuation through a
        child those decisions rejected, the zero-residual flag if a zero mass
        came before the flag.  Without a flagged decision everything must be
        equal.  Returns (flagged, same): whether a flagged decision exists and
        whether the whole outputs are equal anyway."""
        got_path = [int(x) for x in path_row]
        got_tok = [int(x) for x in tokens_row]
        S = len(got_path)
        exp_path = self.path + [-1] * (S - len(self.path))
        exp_tok = self.tokens + [-1] * (S - len(self.tokens))
        same = int(accept_len) == self.accept_len and got_path == exp_path and got_tok == exp_tok
        flag = self.first_flag(*flag_eps) if flag_eps else self.first_flag()
        if flag is None:
            assert int(accept_len) == self.accept_len, \
                f"{what}: accept_len {int(accept_len)} != {self.accept_len}"
            assert got_path == exp_path, f"{what}: path {got_path} != {exp_path}"
            assert got_tok == exp_tok, f"{what}: tokens {got_tok} != {exp_tok}"
            if flags is not None:
                assert int(flags) == (1 if self.zero_residual else 0), f"{what}: flags {int(flags)}"
            if accept_mask is not None:
                m = np.zeros(len(accept_mask), dtype=np.uint8)
                m[self.path] = 1
                assert np.array_equal(np.asarray(accept_mask, dtype=np.uint8), m), \
                    f"{what}: accept mask"
            return False, True
        pre_path, pre_tok, rejected = self.prefix_before(flag)
        k = len(pre_path)
        assert got_path[:k] == pre_path, \
            f"{what}: path {got_path} does not start with {pre_path} (fixed before the flag)"
        assert got_tok[:k - 1] == pre_tok, \
            f"{what}: tokens {got_tok} do not start with {pre_tok} (fixed before the flag)"
        assert int(accept_len) >= k - 1, f"{what}: accept_len {int(accept_len)} < {k - 1}"
        if int(accept_len) >= k:
            assert got_path[k] not in rejected, \
                f"{what}: continues through row {got_path[k]}, rejected before the flag"
        if flags is not None and any(kd == "residual" and m == 0.0
                                     for kd, _, m in self.decisions[:flag]):
            assert int(flags) & 1, f"{what}: zero residual before the flag, flags {int(flags)}"
        return True, same


def walk_sampling(parents, tokens, P, Q, coin_accept, coin_sample) -> WalkResult:
    """Acceptance walk at temperature > 0 (readings 1-7).

    parents, tokens : local arrays of one request (row 0 = root)
    P, Q            : per-row distributions, P[u] = softmax(p_u/T),
                      Q[u] = softmax(q_u/T) (only non-leaf rows are used)
    coin_accept[c]  : uniform of draft row c (purpose 0)
    coin_sample[u]  : uniform for a draw at node u (purpose 1)
    """
    validate(parents)
    kids = tree_children(parents)
    res = WalkResult()
    u = 0
    while True:
        if not kids[u]:
            t, m = sample_inverse_cdf(P[u], coin_sample[u])
            res.decisions.append(("sample", u, m))
            res.tokens.append(t)
            return res
        R = np.array(P[u], dtype=np.float64)
        Qu = np.asarray(Q[u], dtype=np.float64)
        moved = False
        for c in kids[u]:
            x = int(tokens[c])
            r = float(coin_accept[c])
            res.decisions.append(("accept", c, accept_margin(r, R[x], Qu[x])))
            if r * Qu[x] < R[x]:
                res.path.append(c)
                res.tokens.append(x)
                u = c
                moved = True
                break
            w = np.maximum(0.0, R - Qu)
            Z = float(np.sum(w))
            res.decisions.append(("residual", c, Z))
            if Z > 0:
                R = w / Z
            else:                   # R <= Q_u everywhere: keep R, raise the flag
                res.zero_residual = True
        if not moved:
            t, m = sample_inverse_cdf(R, coin_sample[u])
            res.decisions.append(("sample", u, m))
            res.tokens.append(t)
            return res


def walk_topk(parents, tokens, P, coin_accept, coin_sample) -> WalkResult:
    """Acceptance walk for deterministic children (reading 10)."""
    validate(parents)
    kids = tree_children(parents)
    res = WalkResult()
    u = 0
    while True:
        if not kids[u]:
            t, m = sample_inverse_cdf(P[u], coin_sample[u])
            res.decisions.append(("sample", u, m))
            res.tokens.append(t)
            return res
        R = np.array(P[u], dtype=np.float64)
        moved = False
        for c in kids[u]:
            x = int(tokens[c])
            r = float(coin_accept[c])
            res.decisions.append(("accept", c, accept_margin(r, R[x], 1.0)))
            if r < R[x]:
                res.path.append(c)
                res.tokens.append(x)
                u = c
                moved = True
                break
            w = R.copy()
            w[x] = max(0.0, R[x] - 1.0)
            Z = float(np.sum(w))
            res.decisions.append(("residual", c, Z))
            # Z > 0 always: a rejection needs r >= R(x) with r < 1, so R(x) < 1;
            # R is normalised, and R(x) = w_x / Z_prev < 1 means another entry
            # of w was positive, so it still is.  (The zero-residual case of
            # reading 2 cannot arise for point-mass drafts.)
            assert Z > 0, "unreachable: a rejected point-mass draft leaves mass elsewhere"
            R = w / Z
        if not moved:
            t, m = sample_inverse_cdf(R, coin_sample[u])
            res.decisions.append(("sample", u, m))
            res.tokens.append(t)
            return res


def accept_request_topk(parents, tokens, p_logits, temperature, seed, step, request):
    """Acceptance of one request whose children are deterministic drafts
    (reading 10); temperature > 0.  Returns the same dict as accept_request
    (child_q is NaN everywhere)."""
    parents = np.asarray(parents)
    n = len(parents)
    P = distributions(p_logits, temperature)
    ca, cs = request_coins(seed, step, request, n)
    res = walk_topk(parents, tokens, P, ca, cs)
    child_p = np.full(n, np.nan)
    for c in range(1, n):
        child_p[c] = P[int(parents[c]), int(tokens[c])]
    return dict(path=list(res.path), tokens=list(res.tokens), accept_len=res.accept_len,
                child_p=child_p, child_q=np.full(n, np.nan), result=res)


def walk_greedy(parents, tokens, p_logits) -> WalkResult:
    """Acceptance walk at temperature 0 (reading 8).  Decisions are exact."""
    validate(parents)
    kids = tree_children(parents)
    res = WalkResult()
    u = 0
    while True:
        g = greedy_token(p_logits[u])
        nxt = [c for c in kids[u] if int(tokens[c]) == g]
        res.tokens.append(g)
        if not nxt:
            return res
        res.path.append(nxt[0])
        u = nxt[0]


def request_coins(seed, step, request, n):
    """(coin_accept[n], coin_sample[n]) of one request's rows."""
    from .philox import uniform
    rows = np.arange(n, dtype=np.uint64)
    return (uniform(seed, step, request, rows, 0),
            uniform(seed, step, request, rows, 1))


def accept_request(parents, tokens, p_logits, q_logits, temperature, seed, step, request):
    """Full acceptance of one request: distributions, child probabilities, walk.

    p_logits/q_logits: [n][V] rows of this request (q rows of leaves unused;
    q_logits may be None when temperature == 0).
    Returns dict(path, tokens, accept_len, child_p, child_q, result).
    child_p[c] = P_parent(c)(token c), child_q likewise; NaN at the root.
    At temperature 0, child_p[c] is 1 if token c is the parent's argmax else 0,
    and child_q is NaN.
    """
    parents = np.asarray(parents)
    n = len(parents)
    child_p = np.full(n, np.nan)
    child_q = np.full(n, np.nan)
    if temperature == 0:
        res = walk_greedy(parents, tokens, p_logits)
        for c in range(1, n):
            u = int(parents[c])
            child_p[c] = 1.0 if int(tokens[c]) == greedy_token(p_logits[u]) else 0.0
    else:
        nonleaf = np.zeros(n, dtype=bool)
        nonleaf[parents[1:]] = True
        P = distributions(p_logits, temperature)
        Q = np.full_like(P, np.nan)
        if nonleaf.any():
            Q[nonleaf] = distributions(np.asarray(q_logits)[nonleaf], temperature)
        ca, cs = request_coins(seed, step, request, n)
        res = walk_sampling(parents, tokens, P, Q, ca, cs)
        for c in range(1, n):
            u = int(parents[c])
            child_p[c] = P[u, int(tokens[c])]
            child_q[c] = Q[u, int(tokens[c])]
    return dict(path=list(res.path), tokens=list(res.tokens), accept_len=res.accept_len,
                child_p=child_p, child_q=child_q, result=res)
