"""Draft-tree topologies for the synthetic verify workloads.

These builders produce the *shape* of a draft tree as a parent array in
breadth-first order (row 0 is the root, ``parent[0] == -1`` and
``parent[i] < i``).  They stand in for the drafters the pages describe; none of
the verify method's arithmetic lives here.

Sources (page title, section):

* chain of gamma drafts -- "Speculative decoding" post on guijiagi.com,
  section on the draft-verify paradigm (gamma sequential drafts).
* Cartesian-product tree -- "万字综述 10+ 种 LLM 投机采样推理加速方案",
  section 6.2 (Medusa): k1 x k2 x k3 candidates merged into one token tree,
  3 x 5 x 7 giving 3 + 15 + 105 = 123 tokens.
* expansion tree with a per-step K schedule -- "投机推理算法的常见优化手段",
  section on generating the draft tree (SpecInfer expansion, K = 3, 2, 2, 1, 1
  giving 3 + 6 + 12 + 12 + 12 = 45 tokens).
* dynamic tree -- same page, EAGLE-2 paragraph: each round expands only the
  top-K bottom-layer leaves ranked by the product of probabilities along the
  path (K = 5: 25 leaves after round two, only 5 of them expanded).
* global budget -- same page, section on dynamic draft length (ECHO): one
  verify-token budget Kmax shared by the whole batch.  The pages give no
  allocation algorithm; ``echo_budget`` is a stated stand-in.
"""
from __future__ import annotations

import numpy as np


def toy_tree() -> np.ndarray:
    """The six-node tree root/A/B/C/D/E flattened as [root, A, B, C, D, E]."""
    return np.array([-1, 0, 0, 1, 1, 2], dtype=np.int32)


def chain(gamma: int) -> np.ndarray:
    """A chain of ``gamma`` drafts under the root: gamma + 1 rows."""
    return np.arange(-1, gamma, dtype=np.int32)


def _layered(widths_per_level) -> np.ndarray:
    """BFS tree where every node of level d gets ``widths_per_level[d]`` children."""
    parents = [-1]
    level = [0]
    for k in widths_per_level:
        nxt = []
        for u in level:
            for _ in range(k):
                parents.append(u)
                nxt.append(len(parents) - 1)
        level = nxt
    return np.asarray(parents, dtype=np.int32)


def cartesian(ks) -> np.ndarray:
    """Medusa-style Cartesian tree: head d proposes ks[d] candidates per prefix."""
    return _layered(list(ks))


def k_schedule(ks) -> np.ndarray:
    """SpecInfer expansion tree: at step d every newest node takes top-ks[d]."""
    return _layered(list(ks))


def draft_nodes(parents: np.ndarray) -> int:
    """Number of draft tokens in a tree, i.e. rows excluding the root."""
    return int(len(parents)) - 1


def depths(parents: np.ndarray) -> np.ndarray:
    """Depth of every row (root = 0); needs parent[i] < i."""
    d = np.zeros(len(parents), dtype=np.int32)
    for i in range(1, len(parents)):
        d[i] = d[parents[i]] + 1
    return d


def bfs_relabel(parents: np.ndarray, order_key=None) -> np.ndarray:
    """Relabel an arbitrary rooted tree (root 0) into breadth-first order.

    Children are visited in their original index order (or ``order_key``).
    Returns the new parent array.
    """
    n = len(parents)
    kids = [[] for _ in range(n)]
    for i in range(1, n):
        kids[parents[i]].append(i)
    if order_key is not None:
        for k in kids:
            k.sort(key=lambda j: order_key[j])
    order = [0]
    head = 0
    while head < len(order):
        order.extend(kids[order[head]])
        head += 1
    new_of = {old: new for new, old in enumerate(order)}
    out = np.empty(n, dtype=np.int32)
    out[0] = -1
    for new, old in enumerate(order):
        if new:
            out[new] = new_of[parents[old]]
    return out


class Eagle2Expansion:
    """Dynamic draft tree grown the EAGLE-2 way with synthetic confidences.

    Round 1 gives the root ``topk`` children.  Every later round takes the
    ``topk`` bottom-layer leaves with the largest cumulative score (product of
    per-node confidences along the path) and gives each ``topk`` children.
    Per-node confidences are drawn from ``rng`` (a stand-in for the drafter's
    probabilities) and sorted so siblings come in descending confidence.
    """

    def __init__(self, rng: np.random.Generator, topk: int = 5):
        self.rng = rng
        self.topk = topk
        self.parents = [-1]
        self.score = [1.0]
        self.depth = [0]
        self.bottom = [0]
        self.expanded_per_round = []

    def step(self):
        if len(self.bottom) > self.topk:
            ranked = sorted(self.bottom, key=lambda u: -self.score[u])
            chosen = ranked[: self.topk]
        else:
            chosen = list(self.bottom)
        self.expanded_per_round.append(list(chosen))
        new = []
        for u in chosen:
            conf = np.sort(self.rng.random(self.topk))[::-1]
            for c in conf:
                self.parents.append(u)
                self.score.append(self.score[u] * float(c))
                self.depth.append(self.depth[u] + 1)
                new.append(len(self.parents) - 1)
        self.bottom = new
        return new

    def select(self, rows: int) -> np.ndarray:
        """Keep the root plus the ``rows - 1`` highest-score nodes, BFS order.

        Confidences lie in (0, 1), so a child never outranks its parent and
        the kept set is a connected subtree.
        """
        n = len(self.parents)
        if rows > n:
            raise ValueError("tree smaller than requested rows")
        order = sorted(range(1, n), key=lambda u: (-self.score[u], u))
        keep = [0] + sorted(order[: rows - 1])
        idx = {old: new for new, old in enumerate(keep)}
        par = np.empty(rows, dtype=np.int32)
        par[0] = -1
        for new, old in enumerate(keep):
            if new:
                par[new] = idx[self.parents[old]]
        key = np.array([-self.score[old] for old in keep])
        return bfs_relabel(par, order_key=key)


def eagle2_tree(rng: np.random.Generator, rows: int, topk: int = 5,
                max_depth: int = 8) -> np.ndarray:
    """A dynamic tree of exactly ``rows`` rows (root included), depth <= max_depth."""
    ex = Eagle2Expansion(rng, topk)
    while len(ex.parents) < rows and max(ex.depth) < max_depth:
        ex.step()
    while len(ex.parents) < rows:
        # Depth cap reached but budget left: widen the shallowest layer
        # (the ECHO rule of spending leftover budget on width).
        ex.bottom = [u for u in range(len(ex.parents)) if ex.depth[u] < max_depth]
        ex.step()
    tree = ex.select(rows)
    assert depths(tree).max() <= max_depth
    return tree


def echo_budget(rng: np.random.Generator, batch: int, kmax: int,
                min_rows: int = 8, max_rows: int = 64) -> np.ndarray:
    """Split a global row budget ``kmax`` over ``batch`` requests.

    Stand-in for the ECHO scheduler: every request gets ``min_rows``; the rest
    is shared in proportion to an Exp(1) confidence by largest remainder, with
    a per-request cap of ``max_rows`` and the overflow handed on.  The result
    sums to ``kmax`` exactly.
    """
    if not (batch * min_rows <= kmax <= batch * max_rows):
        raise ValueError("budget outside [batch*min_rows, batch*max_rows]")
    w = rng.exponential(1.0, size=batch)
    n = np.full(batch, min_rows, dtype=np.int64)
    left = kmax - int(n.sum())
    open_ = np.ones(batch, dtype=bool)
    while left > 0:
        ww = np.where(open_, w, 0.0)
        share = ww / ww.sum() * left
        base = np.floor(share).astype(np.int64)
        rem = left - int(base.sum())
        frac = share - base
        order = np.argsort(-frac, kind="stable")
        base[order[:rem]] += 1
        room = max_rows - n
        add = np.minimum(base, room)
        n += add
        left -= int(add.sum())
        open_ = n < max_rows
    assert int(n.sum()) == kmax
    return n.astype(np.int32)
