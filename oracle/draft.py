"""Dynamic draft trees: EAGLE-2 expansion under an ECHO-style global budget.

Oracle side; test infrastructure.  Plain loops over plain Python lists.

Pages followed, both on "投机推理算法的常见优化手段" (cnblogs):

* draft-tree generation section, the EAGLE-2 paragraph: a round does not
  expand every leaf of the bottom layer, only the K most probable ones, where
  a leaf's probability is the product of the node probabilities along its
  path (with K = 5 the second round leaves 25 leaves, of which only 5 are
  expanded);
* dynamic draft length section (ECHO): the batch shares one budget K_max of
  verify tokens; at checkpoint depths fixed offline a branch of low
  confidence is cut; a cut request may still widen at the cut depth when
  budget is left; budget freed by low-confidence requests goes to the
  confident ones.

Readings taken where the pages leave a step open:

D1. A round gives each frontier node (at most K of them, in frontier order)
    the drafter's K candidates (token, probability) in candidate order; the
    new nodes get consecutive ids after the existing ones.  A node's score is
    score(parent) * p rounded to float32 (the product of the path's
    probabilities, accumulated from the root, each step in float32).  The
    drafter's p is clamped to [0, 1] (NaN -> 0), so no score exceeds its
    parent's.
D2. The next frontier is the K highest-scoring nodes of the new layer (ties:
    lower id first).  When the new layer's depth is a checkpoint, its nodes
    scoring below that checkpoint's threshold are not eligible.  An empty
    frontier ends the request's growth (the branch is cut).  A round that
    would overflow the request's node capacity appends nothing, ends its
    growth and raises FLAG_CAPACITY.
D3. Selection: every root is kept, plus the K_max - B highest-scoring
    non-root nodes of the whole batch (ties: lower request, then lower id),
    taken among the nodes ranked below max_rows - 1 in their own request
    (score descending, id ascending).  A child never outscores its parent and
    has the larger id, so each request's kept nodes form a tree.  Widening is
    this selection: every candidate generated at a cut depth stays
    selectable, and the budget goes wherever the scores are highest.
D4. Layout: a request's rows are its root, then its kept nodes in id order
    (breadth-first, since ids grow with depth); parents are remapped to rows.

Every function is pinned by tests/test_oracle_draft.py (the pages' 25-leaf
round, counts, closure, brute-force global ranking, checkpoint cuts).
"""
from __future__ import annotations

import dataclasses

import numpy as np

FLAG_CAPACITY = 1


def clamp_prob(p) -> np.float32:
    p = np.float32(p)
    if not (p >= 0):          # NaN or negative
        return np.float32(0)
    return min(p, np.float32(1))


@dataclasses.dataclass
class DraftTree:
    """One request's growing tree (node 0 is the root)."""
    parent: list
    token: list
    score: list          # np.float32 values
    depth: list
    frontier: list
    capacity: int
    flags: int = 0

    @property
    def count(self):
        return len(self.parent)


def begin(root_token: int, capacity: int) -> DraftTree:
    return DraftTree(parent=[-1], token=[int(root_token)], score=[np.float32(1)], depth=[0],
                     frontier=[0], capacity=int(capacity))


def expand(t: DraftTree, cand_tokens, cand_probs, K: int, gates=()) -> None:
    """One round (D1, D2).  cand_tokens/cand_probs: [K][K], row i for the
    i-th frontier node; gates: (depth, threshold) pairs."""
    if not t.frontier:
        return
    if t.count + len(t.frontier) * K > t.capacity:
        t.flags |= FLAG_CAPACITY
        t.frontier = []
        return
    first = t.count
    for i, u in enumerate(t.frontier):
        for j in range(K):
            t.parent.append(u)
            t.token.append(int(cand_tokens[i][j]))
            t.score.append(np.float32(t.score[u] * clamp_prob(cand_probs[i][j])))
            t.depth.append(t.depth[u] + 1)
    new = list(range(first, t.count))
    d = t.depth[first]
    thr = [float(th) for gd, th in gates if int(gd) == d]
    if thr:
        new = [v for v in new if all(t.score[v] >= np.float32(th) for th in thr)]
    new.sort(key=lambda v: (-float(t.score[v]), v))
    t.frontier = new[:K]


def select(trees, budget_rows: int, max_rows: int):
    """Global budget selection and layout (D3, D4).  Returns
    (row_offsets [B+1], parents [R], tokens [R], node_of_row [R])."""
    B = len(trees)
    eligible = []
    for b, t in enumerate(trees):
        order = sorted(range(1, t.count), key=lambda v: (-float(t.score[v]), v))
        for rank, v in enumerate(order):
            if rank < max_rows - 1:
                eligible.append((-float(t.score[v]), b, v))
    eligible.sort()
    take = max(0, budget_rows - B)
    kept = [set() for _ in range(B)]
    for _, b, v in eligible[:take]:
        kept[b].add(v)
    row_offsets = [0]
    parents, tokens, node_of_row = [], [], []
    for b, t in enumerate(trees):
        nodes = [0] + sorted(kept[b])
        row = {v: i for i, v in enumerate(nodes)}
        for v in nodes:
            parents.append(-1 if v == 0 else row[t.parent[v]])
            tokens.append(t.token[v])
            node_of_row.append(v)
        row_offsets.append(row_offsets[-1] + len(nodes))
    return (np.array(row_offsets, dtype=np.int32), np.array(parents, dtype=np.int32),
            np.array(tokens, dtype=np.int32), np.array(node_of_row, dtype=np.int32))


def build(root_tokens, cand_tokens, cand_probs, K, capacity, gates, budget_rows, max_rows):
    """All rounds, then the selection.  cand_*: [rounds][B][K][K]."""
    trees = [begin(rt, capacity) for rt in root_tokens]
    for r in range(len(cand_tokens)):
        for b, t in enumerate(trees):
            expand(t, cand_tokens[r][b], cand_probs[r][b], K, gates)
    return trees, select(trees, budget_rows, max_rows)
