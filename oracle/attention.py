"""Tree attention by its definition (oracle side; test infrastructure).

Pages: "投机推理算法的常见优化手段" (cnblogs), tree-mask section -- the
flattened tree goes through one forward pass with the tree mask, the KV
cache and tree position ids; "万字综述 10+ 种 LLM 投机采样推理加速方案"
section 5.2 -- tree-based parallel decoding verifies every branch in one pass
with a dedicated attention mask and gives what sequence-based decoding (each
branch as its own sequence with its own KV) gives.

The pages never write the attention formula.  Reading taken: standard scaled
dot-product attention, softmax(q k^T * scale) v, over the keys a row may see:
the whole KV prefix of its request plus the tree rows j with M[i][j] = 1.
Grouped-query heads: query head h reads KV head h // (Hq / Hkv).  No ALiBi,
soft-capping or dropout; rotary embedding is the caller's business.
"""
from __future__ import annotations

import numpy as np

from .tree import ancestor_mask


def softmax_rows(s: np.ndarray) -> np.ndarray:
    """Row-wise softmax of a float64 matrix; -inf entries get weight 0."""
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def tree_attention(q, k_prefix, v_prefix, k_tree, v_tree, parents, scale=None):
    """Attention output of one request's tree rows.

    q        [N][Hq][D]   queries of the N tree rows (row 0 = root)
    k_prefix [Hkv][L][D]  cached keys before the tree;  v_prefix likewise
    k_tree   [N][Hkv][D]  keys of the tree rows;        v_tree likewise
    parents  [N]          local parent array
    Returns float64 [N][Hq][D].
    """
    return masked_attention(q, k_prefix, v_prefix, k_tree, v_tree, ancestor_mask(parents),
                            scale)


def masked_attention(q, k_prefix, v_prefix, k_tree, v_tree, visible, scale=None):
    """The same attention under any visibility of the new rows.

    visible [N][N] bool: row i sees new row j.  Every row sees the whole
    prefix.  The pages' lookahead decoding (section 8.2.3 of the survey page)
    combines two branches in one pass with such a mask: causal inside each
    branch, no branch seeing the other; tree_attention is the case
    visible = the ancestor mask.
    """
    q = np.asarray(q, dtype=np.float64)
    k_prefix = np.asarray(k_prefix, dtype=np.float64)
    v_prefix = np.asarray(v_prefix, dtype=np.float64)
    k_tree = np.asarray(k_tree, dtype=np.float64)
    v_tree = np.asarray(v_tree, dtype=np.float64)
    N, Hq, D = q.shape
    Hkv, L, _ = k_prefix.shape
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    M = np.asarray(visible, dtype=bool)
    assert M.shape == (N, N)
    visible = np.concatenate([np.ones((N, L), dtype=bool), M], axis=1)
    out = np.empty((N, Hq, D), dtype=np.float64)
    for h in range(Hq):
        kvh = h // G
        keys = np.concatenate([k_prefix[kvh], k_tree[:, kvh, :]], axis=0)
        vals = np.concatenate([v_prefix[kvh], v_tree[:, kvh, :]], axis=0)
        s = (q[:, h, :] @ keys.T) * scale
        s = np.where(visible, s, -np.inf)
        out[:, h, :] = softmax_rows(s) @ vals
    return out


def attention_rows(q_rows, keys, vals, scale):
    """Plain attention of a few query vectors over an explicit key list.

    q_rows [n][D], keys/vals [K][D]; every key visible.  Used to check single
    sampled outputs of large workloads one by one.
    """
    s = (np.asarray(q_rows, np.float64) @ np.asarray(keys, np.float64).T) * scale
    return softmax_rows(s) @ np.asarray(vals, np.float64)
