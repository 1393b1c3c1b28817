"""Speculative-decoding verify step on AMD MI355X (gfx950).

The work happens in ``lib/libspecverify.so`` (hand-written HIP); ``_lib`` is
its ctypes binding (same names as the C entry points) and ``pipeline`` runs
the five calls of one verify step on torch-owned device buffers.
"""
from . import _lib  # noqa: F401  (fails loudly when the library is not built)
from ._lib import (SpecError, Batch, Kv, AcceptOut, spec_tree_build_mask,  # noqa: F401
                   spec_kv_append, spec_tree_attn_workspace_bytes, spec_tree_attn_verify,
                   spec_accept_workspace_bytes, spec_accept_sample, spec_accept_topk, spec_kv_commit,
                   spec_abi_version, spec_status_string, DraftTree, spec_draft_begin,
                   spec_draft_expand, spec_draft_select_workspace_bytes, spec_draft_select,
                   spec_lm_head_accept_workspace_bytes, spec_lm_head_accept,
                   SPEC_CHILDREN_SAMPLED, SPEC_CHILDREN_TOPK)
