"""KV-cache append and commit/rollback (oracle side; test infrastructure).

Pages: guijiagi.com speculative-decoding post, KV-cache management section --
the KV of rejected candidates must be rolled back, and with block-wise paged
KV the blocks of rejected tokens are simply freed; the CSDN page's data-flow
section -- the KV cache is reused at verification.

Reading taken: during verification the tree's K/V rows sit in cache slots
[L, L + N) of their request (row i at L + i).  Commit keeps the accepted path
(root first) and compacts it to the front of that range: slot L + k receives
the row that was at L + path[k], k = 0..a.  The new length is L + a + 1 (the
root is the last already-emitted token; the newly emitted final token has no
KV yet).  With paged KV, every logical block lying wholly at or beyond the
new length, up to the blocks the tree occupied, is freed.
"""
from __future__ import annotations

import numpy as np


def append(prefix_rows: np.ndarray, tree_rows: np.ndarray) -> np.ndarray:
    """Logical cache of one request/head after the tree rows are appended."""
    return np.concatenate([prefix_rows, tree_rows], axis=0)


def commit(logical: np.ndarray, L: int, path) -> np.ndarray:
    """Cache rows [0, L + a + 1) after committing accepted ``path`` (root first).

    logical: rows of one request/head, at least L + max(path) + 1 long.
    """
    kept = [logical[L + int(p)] for p in path]
    return np.concatenate([logical[:L], np.stack(kept)], axis=0)


def new_length(L: int, accept_len: int) -> int:
    return int(L) + int(accept_len) + 1


def freed_blocks(block_row, L: int, tree_rows: int, accept_len: int, block: int = 16):
    """Physical blocks released by the commit, in logical order."""
    nl = new_length(L, accept_len)
    first = -(-nl // block)
    end = -(-(L + tree_rows) // block)
    return [int(block_row[j]) for j in range(first, end)]
