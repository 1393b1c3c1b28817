"""Visibility masks of the new rows that are not tree masks (inputs only).

A caller of the attention may pass any per-row visibility of the new rows,
packed as 64-bit words.  Two shapes serve as inputs here:

* lookahead_visibility -- the survey page's lookahead decoding, section
  8.2.3: the current token ("0") plus a lookahead branch of W*(N-1) - 1 rows
  and a verify branch of G*(N-1) rows in one pass; each row sees only rows
  before it (causal), and neither branch sees the other (both see "0").
  Rows are ordered "0", lookahead branch, verify branch.
* random_visibility -- arbitrary bits (rows may see later rows), every row
  seeing itself.
"""
from __future__ import annotations

import numpy as np


def lookahead_visibility(W: int, N: int, G: int) -> np.ndarray:
    la = W * (N - 1) - 1
    ve = G * (N - 1)
    n = 1 + la + ve
    branch = np.array([0] + [1] * la + [2] * ve)
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    return (j <= i) & ((branch[None, :] == branch[:, None]) | (j == 0))


def random_visibility(rng: np.random.Generator, n: int, density: float = 0.5) -> np.ndarray:
    m = rng.random((n, n)) < density
    m[np.arange(n), np.arange(n)] = True
    return m
