"""Tree flattening, ancestor mask and depth (oracle side; test infrastructure).

Follows "投机推理算法的常见优化手段" (cnblogs), section on verifying the draft
tree with a tree mask: the tree is flattened depth- or breadth-first into one
sequence, and each token may attend only to its ancestors.

Reading taken where the page is inconsistent: its sentence defines the mask
the transposed way round ("M_ij = 1 when i is an ancestor of j") and without a
diagonal, while its own worked example (B sees the root but not A; C sees A
and the root) and the printed 6x6 matrix have row = attending token, column =
attended token, and ones on the diagonal.  The oracle follows the printed
matrix: M[i][j] = 1 iff j == i or j is an ancestor of i.  Any topological
order is accepted (row 0 is the root, parent[i] < i).

Position ids: the page says position ids must follow the tree; a row's
position is prefix_len + depth(row).
"""
from __future__ import annotations

import numpy as np


class TreeError(ValueError):
    """The parent array is not a flattened rooted tree."""


def validate(parents) -> None:
    """Row 0 is the root (parent -1) and every other row's parent precedes it."""
    parents = np.asarray(parents)
    if len(parents) == 0:
        raise TreeError("empty tree")
    if parents[0] != -1:
        raise TreeError("row 0 must be the root (parent -1)")
    for i in range(1, len(parents)):
        if not (0 <= parents[i] < i):
            raise TreeError(f"row {i}: parent {parents[i]} must be in [0, {i})")


def ancestors(parents, i) -> list:
    """Rows on the path from row i up to the root, i itself first."""
    out = []
    j = int(i)
    while j != -1:
        out.append(j)
        j = int(parents[j])
    return out


def ancestor_mask(parents) -> np.ndarray:
    """Boolean [n][n]: M[i][j] is true iff j is i or an ancestor of i."""
    validate(parents)
    n = len(parents)
    M = np.zeros((n, n), dtype=bool)
    for i in range(n):
        for j in ancestors(parents, i):
            M[i, j] = True
    return M


def depth(parents) -> np.ndarray:
    """Number of strict ancestors of each row (root = 0)."""
    validate(parents)
    return np.array([len(ancestors(parents, i)) - 1 for i in range(len(parents))],
                    dtype=np.int32)


def children(parents) -> list:
    """children[u] = rows whose parent is u, in ascending row order."""
    n = len(parents)
    out = [[] for _ in range(n)]
    for i in range(1, n):
        out[int(parents[i])].append(i)
    return out


def pack_words(M: np.ndarray, words: int) -> np.ndarray:
    """Pack mask rows into uint64 words: bit (j mod 64) of word (j div 64)."""
    n = M.shape[0]
    out = np.zeros((n, words), dtype=np.uint64)
    for i in range(n):
        for j in np.nonzero(M[i])[0]:
            out[i, j // 64] |= np.uint64(1) << np.uint64(j % 64)
    return out
