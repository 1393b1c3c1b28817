"""One verify step over a workload: allocate device buffers, call the library.

``VerifyStep`` owns the output and workspace tensors (torch allocations: the
library itself never allocates) and runs the five C entry points in order on
one stream: build mask -> append tree K/V -> tree attention -> acceptance ->
commit.  It only marshals; every step runs in libspecverify.
"""
from __future__ import annotations

import math

import numpy as np
import torch

from . import _lib as L


def pack_visibility(visibility, row_offsets, words):
    """Mask words [R][words] (int64 view of uint64) from per-request bool
    [n][n] visibility: bit j of row i's words set iff row i sees row j."""
    R = int(row_offsets[-1])
    out = np.zeros((R, words * 8), dtype=np.uint8)
    for b, vis in enumerate(visibility):
        o = int(row_offsets[b])
        vis = np.asarray(vis, dtype=bool)
        packed = np.packbits(vis, axis=1, bitorder="little")
        out[o:o + vis.shape[0], :packed.shape[1]] = packed
    return out.view(np.int64)


class VerifyStep:
    def __init__(self, w, path_stride=None, out_dtype=None, temperature=None, seed=None, step=None,
                 acceptance="sample", head=None, store_head_logits=False):
        """``w`` is any object with the workload fields (see workloads.gen.Workload).
        ``acceptance``: "sample" (children drawn from the draft rows) or "topk"
        (deterministic children: spec_accept_topk, draft rows unused).
        ``head``: optional (hidden [R][H], weight [V][H]) bf16 tensors; the
        target logits then come from the LM head (spec_lm_head_accept) instead
        of ``w.p_logits``, and are kept in ``head_logits`` (at temperature > 0
        the rows of nodes with children; at 0 every row, only with
        ``store_head_logits``)."""
        if acceptance not in ("sample", "topk"):
            raise ValueError(f"acceptance must be 'sample' or 'topk', not {acceptance!r}")
        self.acceptance = acceptance
        dev = w.q.device
        self.w = w
        self.batch = L.Batch(w.row_offsets, w.prefix_len, dev)
        self.parents = torch.from_numpy(np.asarray(w.parents, np.int32)).to(dev)
        self.tokens = torch.from_numpy(np.asarray(w.tokens, np.int32)).to(dev)
        R, B = self.batch.R, self.batch.B
        self.kv = L.Kv(w.k_cache, w.v_cache, w.Hkv, w.D,
                       layout="paged" if w.kv_layout == "paged" else "contig",
                       capacity=getattr(w, "capacity", 0), block_table=w.block_table)
        self.mask = torch.empty((R, self.batch.words), dtype=torch.int64, device=dev)
        # A caller-supplied visibility of the new rows (not a tree mask):
        # packed once here, it replaces the ancestor mask after build_mask.
        self.caller_mask = None
        if getattr(w, "visibility", None) is not None:
            self.caller_mask = torch.from_numpy(
                pack_visibility(w.visibility, w.row_offsets, self.batch.words)).to(dev)
        self.depth = torch.empty(R, dtype=torch.int32, device=dev)
        self.position = torch.empty(R, dtype=torch.int32, device=dev)
        self.err_row = torch.empty(B, dtype=torch.int32, device=dev)
        odt = out_dtype or (torch.float32 if w.dtype == "f32" else torch.bfloat16)
        self.attn_out = torch.empty((R, w.Hq, w.D), dtype=odt, device=dev)
        self.attn_ws = torch.empty(L.spec_tree_attn_workspace_bytes(self.batch, self.kv, w.Hq),
                                   dtype=torch.uint8, device=dev)
        self.scale = 1.0 / math.sqrt(w.D)
        S = path_stride or self.batch.c.max_rows
        self.acc = L.AcceptOut(
            accept_len=torch.empty(B, dtype=torch.int32, device=dev),
            path=torch.empty((B, S), dtype=torch.int32, device=dev),
            tokens=torch.empty((B, S), dtype=torch.int32, device=dev),
            accept_mask=torch.empty(R, dtype=torch.uint8, device=dev),
            child_p=torch.empty(R, dtype=torch.float32, device=dev),
            child_q=torch.empty(R, dtype=torch.float32, device=dev),
            flags=torch.empty(B, dtype=torch.int32, device=dev))
        self.acc_ws = torch.empty(L.spec_accept_workspace_bytes(self.batch, w.V),
                                  dtype=torch.uint8, device=dev)
        self.head = head
        self.store_head_logits = store_head_logits
        if head is not None:
            self.head_ld = int(w.q_logits.stride(0))
            self.head_logits = torch.empty((R, self.head_ld), dtype=torch.float32, device=dev)
            self.head_ws = torch.empty(L.spec_lm_head_accept_workspace_bytes(self.batch, w.V),
                                       dtype=torch.uint8, device=dev)
        self.new_len = torch.empty(B, dtype=torch.int32, device=dev)
        mbps = int(w.block_table.shape[1]) if w.block_table is not None else 1
        self.freed = torch.empty((B, mbps), dtype=torch.int32, device=dev)
        self.temperature = w.temperature if temperature is None else temperature
        self.seed = w.seed if seed is None else seed
        self.step = w.step if step is None else step

    # -- the five calls -------------------------------------------------------
    def build_mask(self, stream=None):
        L.spec_tree_build_mask(self.batch, self.parents, self.mask, self.depth, self.position,
                               self.err_row, stream)
        if self.caller_mask is not None:
            s = stream if stream is not None else torch.cuda.current_stream(self.mask.device)
            with torch.cuda.stream(s):
                self.mask.copy_(self.caller_mask, non_blocking=True)

    def append(self, stream=None):
        L.spec_kv_append(self.batch, self.kv, self.w.k_new, self.w.v_new, stream)

    def attention(self, stream=None):
        L.spec_tree_attn_verify(self.batch, self.kv, self.w.q, self.w.Hq, self.mask, self.scale,
                                self.attn_out, self.attn_ws, stream)

    def accept(self, stream=None):
        if self.head is not None:
            hidden, weight = self.head
            topk = self.acceptance == "topk"
            store = self.temperature > 0 or self.store_head_logits
            q = self.w.q_logits if (self.temperature > 0 and not topk) else None
            L.spec_lm_head_accept(self.batch, self.parents, self.tokens, hidden, weight, q,
                                  self.w.V, self.temperature, self.seed, self.step, self.acc,
                                  self.head_ws, logits=self.head_logits if store else None,
                                  children=L.SPEC_CHILDREN_TOPK if topk else L.SPEC_CHILDREN_SAMPLED,
                                  logits_ld=self.head_ld, stream=stream)
            return
        if self.acceptance == "topk":
            L.spec_accept_topk(self.batch, self.parents, self.tokens, self.w.p_logits, self.w.V,
                               self.temperature, self.seed, self.step, self.acc, self.acc_ws,
                               stream=stream)
            return
        q = self.w.q_logits if self.temperature > 0 else None
        L.spec_accept_sample(self.batch, self.parents, self.tokens, self.w.p_logits, q,
                             self.w.V, self.temperature, self.seed, self.step, self.acc,
                             self.acc_ws, stream=stream)

    def commit(self, stream=None):
        L.spec_kv_commit(self.batch, self.kv, self.acc.accept_len, self.acc.path, self.new_len,
                         self.freed if self.w.kv_layout == "paged" else None, stream)

    def run(self, stream=None, commit=True):
        self.build_mask(stream)
        self.append(stream)
        self.attention(stream)
        self.accept(stream)
        if commit:
            self.commit(stream)
