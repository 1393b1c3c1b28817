"""ctypes binding of libspecverify.so: argument marshalling only.

Each function has the name of the C entry point it calls and takes torch
tensors (device memory) plus plain numbers; it fills the C structs, passes
raw pointers and the current HIP stream, and raises ``SpecError`` on any
status other than SPEC_OK.  Every step of the verify path runs in the HIP
library; nothing here computes.  If the library has not been built the
import fails loudly -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "lib", "libspecverify.so")

SPEC_OK = 0
SPEC_BF16, SPEC_F32 = 0, 1
SPEC_KV_CONTIGUOUS, SPEC_KV_PAGED = 0, 1
SPEC_MAX_TREE_ROWS = 256
SPEC_FLAG_ZERO_RESIDUAL, SPEC_FLAG_PATH_TRUNCATED, SPEC_FLAG_BAD_TREE = 1, 2, 4
SPEC_FLAG_SYNC_TIMEOUT = 8
SPEC_DRAFT_FLAG_CAPACITY = 1
STATUS_NAMES = {0: "SPEC_OK", 1: "SPEC_ERR_NULL", 2: "SPEC_ERR_SHAPE", 3: "SPEC_ERR_TREE",
                4: "SPEC_ERR_CAPACITY", 5: "SPEC_ERR_DTYPE", 6: "SPEC_ERR_HIP",
                7: "SPEC_ERR_UNSUPPORTED", 8: "SPEC_ERR_WORKSPACE"}

EXPORTS = ["spec_tree_build_mask", "spec_kv_append", "spec_tree_attn_workspace_bytes",
           "spec_tree_attn_verify", "spec_accept_workspace_bytes", "spec_accept_sample",
           "spec_accept_sample_walk_knobs", "spec_accept_sample_noalloc", "spec_test_exp_f64",
           "spec_accept_topk", "spec_kv_commit", "spec_draft_begin", "spec_draft_expand",
           "spec_draft_select_workspace_bytes", "spec_draft_select", "spec_lm_head_accept_workspace_bytes",
           "spec_lm_head_accept", "spec_status_string", "spec_last_error", "spec_abi_version"]
SPEC_CHILDREN_SAMPLED, SPEC_CHILDREN_TOPK = 0, 1


class SpecError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class CBatch(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("max_rows", ctypes.c_int32),
                ("row_offsets_h", ctypes.c_void_p), ("row_offsets_d", ctypes.c_void_p),
                ("prefix_len_h", ctypes.c_void_p), ("prefix_len_d", ctypes.c_void_p)]


class CKv(ctypes.Structure):
    _fields_ = [("layout", ctypes.c_int), ("dtype", ctypes.c_int),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("capacity", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("block_table_d", ctypes.c_void_p), ("max_blocks_per_seq", ctypes.c_int32)]


class CAcceptOut(ctypes.Structure):
    _fields_ = [("accept_len_d", ctypes.c_void_p), ("path_d", ctypes.c_void_p),
                ("tokens_d", ctypes.c_void_p), ("accept_mask_d", ctypes.c_void_p),
                ("child_p_d", ctypes.c_void_p), ("child_q_d", ctypes.c_void_p),
                ("flags_d", ctypes.c_void_p)]


class CLmHead(ctypes.Structure):
    _fields_ = [("hidden_d", ctypes.c_void_p), ("weight_d", ctypes.c_void_p),
                ("hidden_size", ctypes.c_int32), ("logits_d", ctypes.c_void_p)]


class CDraftTree(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("topk", ctypes.c_int32), ("capacity", ctypes.c_int32),
                ("parent_d", ctypes.c_void_p), ("token_d", ctypes.c_void_p),
                ("score_d", ctypes.c_void_p), ("depth_d", ctypes.c_void_p),
                ("count_d", ctypes.c_void_p), ("frontier_d", ctypes.c_void_p),
                ("flags_d", ctypes.c_void_p)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python tree_attention_verification_02_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, u64, f32, sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                  ctypes.c_uint64, ctypes.c_float, ctypes.c_size_t)
    P = ctypes.POINTER
    sig = {
        "spec_tree_build_mask": ([P(CBatch), vp, vp, vp, vp, vp, vp], ctypes.c_int),
        "spec_kv_append": ([P(CBatch), P(CKv), vp, vp, vp], ctypes.c_int),
        "spec_tree_attn_workspace_bytes": ([P(CBatch), P(CKv), i32], sz),
        "spec_tree_attn_verify": ([P(CBatch), P(CKv), vp, i32, vp, f32, vp, ctypes.c_int, vp, sz, vp],
                                  ctypes.c_int),
        "spec_accept_workspace_bytes": ([P(CBatch), i32], sz),
        "spec_accept_sample": ([P(CBatch), vp, vp, vp, vp, i64, i32, f32, u64, u64, i32,
                                P(CAcceptOut), vp, sz, vp], ctypes.c_int),
        "spec_accept_sample_walk_knobs": ([P(CBatch), vp, vp, vp, vp, i64, i32, f32, u64, u64,
                                           i32, P(CAcceptOut), vp, sz, i32, i32, vp],
                                          ctypes.c_int),
        "spec_accept_sample_noalloc": ([P(CBatch), vp, vp, vp, vp, i64, i32, f32, u64, u64, i32,
                                        P(CAcceptOut), vp], ctypes.c_int),
        "spec_test_exp_f64": ([vp, vp, i64, i32, vp], ctypes.c_int),
        "spec_accept_topk": ([P(CBatch), vp, vp, vp, i64, i32, f32, u64, u64, i32,
                              P(CAcceptOut), vp, sz, vp], ctypes.c_int),
        "spec_kv_commit": ([P(CBatch), P(CKv), vp, vp, i32, vp, vp, vp], ctypes.c_int),
        "spec_draft_begin": ([P(CDraftTree), vp, vp], ctypes.c_int),
        "spec_draft_expand": ([P(CDraftTree), vp, vp, i32, vp, vp, vp], ctypes.c_int),
        "spec_draft_select_workspace_bytes": ([i32, i32], sz),
        "spec_draft_select": ([P(CDraftTree), i32, i32, vp, vp, vp, vp, i32, vp, sz, vp],
                              ctypes.c_int),
        "spec_lm_head_accept_workspace_bytes": ([P(CBatch), i32], sz),
        "spec_lm_head_accept": ([P(CBatch), vp, vp, P(CLmHead), vp, i64, i32, f32, i32, u64, u64,
                                 i32, P(CAcceptOut), vp, sz, vp], ctypes.c_int),
        "spec_status_string": ([ctypes.c_int], ctypes.c_char_p),
        "spec_last_error": ([], ctypes.c_char_p),
        "spec_abi_version": ([], ctypes.c_int),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


LIB = _load()


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, np.ndarray):
        return t.ctypes.data
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _check(status):
    if status != SPEC_OK:
        raise SpecError(status, LIB.spec_last_error().decode())


def _need(cond, status, msg):
    if not cond:
        raise SpecError(status, msg)


def _shaped(t, name, dtype, rows=None, cols=None, row_contiguous=True):
    """Checks the binding can make without the library: a 2-D tensor of the
    given dtype, at least `rows` x `cols`, unit stride along its last axis
    (rows may be padded)."""
    _need(isinstance(t, torch.Tensor), 1, f"{name} must be a tensor")
    _need(t.dtype == dtype, 5, f"{name} must be {dtype}, not {t.dtype}")
    _need(t.dim() == 2, 2, f"{name} must be 2-D, not {tuple(t.shape)}")
    _need(not row_contiguous or t.stride(1) == 1, 2, f"{name} rows must be contiguous")
    if rows is not None:
        _need(t.shape[0] >= rows, 2, f"{name} has {t.shape[0]} rows < {rows}")
    if cols is not None:
        _need(t.shape[1] >= cols, 2, f"{name} has {t.shape[1]} columns < {cols}")


def _dtype_code(dt):
    if dt == torch.bfloat16:
        return SPEC_BF16
    if dt == torch.float32:
        return SPEC_F32
    raise SpecError(5, f"unsupported dtype {dt}")


class Batch:
    """Ragged batch metadata: host int32 arrays and their device copies."""

    def __init__(self, row_offsets, prefix_len, device, max_rows=None):
        self.row_offsets_h = np.ascontiguousarray(row_offsets, dtype=np.int32)
        self.prefix_len_h = np.ascontiguousarray(prefix_len, dtype=np.int32)
        self.row_offsets_d = torch.from_numpy(self.row_offsets_h).to(device)
        self.prefix_len_d = torch.from_numpy(self.prefix_len_h).to(device)
        B = len(self.prefix_len_h)
        if max_rows is None:
            max_rows = int(np.diff(self.row_offsets_h).max()) if B else 1
        self.c = CBatch(B, int(max_rows), _ptr(self.row_offsets_h), _ptr(self.row_offsets_d),
                        _ptr(self.prefix_len_h), _ptr(self.prefix_len_d))

    @property
    def B(self):
        return int(self.c.batch)

    @property
    def R(self):
        return int(self.row_offsets_h[-1])

    @property
    def words(self):
        return (int(self.c.max_rows) + 63) // 64


class Kv:
    """View of a caller-owned KV cache (contiguous or paged)."""

    def __init__(self, k, v, num_kv_heads, head_dim, layout="contig", capacity=0,
                 block_table=None):
        self.k, self.v, self.block_table = k, v, block_table
        paged = layout == "paged"
        mbps = int(block_table.shape[1]) if paged else 0
        self.c = CKv(SPEC_KV_PAGED if paged else SPEC_KV_CONTIGUOUS, _dtype_code(k.dtype),
                     int(num_kv_heads), int(head_dim), _ptr(k), _ptr(v), int(capacity),
                     16 if paged else 0, _ptr(block_table) if paged else None, mbps)


def spec_tree_build_mask(batch, parents, mask, depth=None, position=None, err_row=None,
                         stream=None):
    _check(LIB.spec_tree_build_mask(ctypes.byref(batch.c), _ptr(parents), _ptr(mask),
                                    _ptr(depth), _ptr(position), _ptr(err_row), _stream(stream)))


def spec_kv_append(batch, kv, k_new, v_new, stream=None):
    _check(LIB.spec_kv_append(ctypes.byref(batch.c), ctypes.byref(kv.c), _ptr(k_new),
                              _ptr(v_new), _stream(stream)))


def spec_tree_attn_workspace_bytes(batch, kv, num_q_heads):
    n = LIB.spec_tree_attn_workspace_bytes(ctypes.byref(batch.c), ctypes.byref(kv.c),
                                           int(num_q_heads))
    if n == 0:
        raise SpecError(2, LIB.spec_last_error().decode())
    return int(n)


def spec_tree_attn_verify(batch, kv, q, num_q_heads, mask, softmax_scale, out, workspace,
                          stream=None):
    if q.dtype != kv.k.dtype:
        raise SpecError(5, f"q dtype {q.dtype} differs from the cache dtype {kv.k.dtype}")
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(LIB.spec_tree_attn_verify(ctypes.byref(batch.c), ctypes.byref(kv.c), _ptr(q),
                                     int(num_q_heads), _ptr(mask), float(softmax_scale), _ptr(out),
                                     _dtype_code(out.dtype), _ptr(workspace), ws_bytes,
                                     _stream(stream)))


def spec_accept_workspace_bytes(batch, vocab):
    n = LIB.spec_accept_workspace_bytes(ctypes.byref(batch.c), int(vocab))
    if n == 0:
        raise SpecError(2, LIB.spec_last_error().decode())
    return int(n)


class AcceptOut:
    """Output buffers of spec_accept_sample (optional ones may be None)."""

    def __init__(self, accept_len, path, tokens, accept_mask=None, child_p=None, child_q=None,
                 flags=None):
        self.accept_len, self.path, self.tokens = accept_len, path, tokens
        self.accept_mask, self.child_p, self.child_q, self.flags = accept_mask, child_p, child_q, flags
        self.c = CAcceptOut(_ptr(accept_len), _ptr(path), _ptr(tokens), _ptr(accept_mask),
                            _ptr(child_p), _ptr(child_q), _ptr(flags))

    @property
    def path_stride(self):
        return int(self.path.shape[1])


def spec_accept_sample(batch, parents, tokens, p_logits, q_logits, vocab, temperature, seed, step,
                       out, workspace, logits_ld=None, stream=None):
    if logits_ld is None:
        logits_ld = p_logits.stride(0)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(LIB.spec_accept_sample(ctypes.byref(batch.c), _ptr(parents), _ptr(tokens),
                                  _ptr(p_logits), _ptr(q_logits), int(logits_ld), int(vocab),
                                  float(temperature), int(seed), int(step), out.path_stride,
                                  ctypes.byref(out.c), _ptr(workspace), ws_bytes, _stream(stream)))


def spec_test_exp_f64(x, y, variant=0, stream=None):
    """y = the library's fp64 exponential of x (float64 device tensors);
    variant 0 exp_f64, 1 exp_f64_clamped, 2 exp_f64_stream, 3 and 4 the first
    two evaluated two elements at a time."""
    _check(LIB.spec_test_exp_f64(_ptr(x), _ptr(y), int(x.numel()), int(variant),
                                 _stream(stream)))


SPEC_ACCEPT_SCRATCH_BYTES = 8 << 20


def spec_accept_sample_noalloc(batch, parents, tokens, p_logits, q_logits, vocab, temperature,
                               seed, step, out, logits_ld=None, stream=None):
    """spec_accept_sample on the library's own device scratch (no workspace)."""
    if logits_ld is None:
        logits_ld = p_logits.stride(0)
    _check(LIB.spec_accept_sample_noalloc(ctypes.byref(batch.c), _ptr(parents), _ptr(tokens),
                                          _ptr(p_logits), _ptr(q_logits), int(logits_ld),
                                          int(vocab), float(temperature), int(seed), int(step),
                                          out.path_stride, ctypes.byref(out.c), _stream(stream)))


def spec_accept_sample_walk_knobs(batch, parents, tokens, p_logits, q_logits, vocab, temperature,
                                  seed, step, out, workspace, max_slices=0, max_spins=-1,
                                  logits_ld=None, stream=None):
    """spec_accept_sample with the walk's workgroups per request and barrier
    polls set by the caller (tests of the walk's meetings)."""
    if logits_ld is None:
        logits_ld = p_logits.stride(0)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(LIB.spec_accept_sample_walk_knobs(
        ctypes.byref(batch.c), _ptr(parents), _ptr(tokens), _ptr(p_logits), _ptr(q_logits),
        int(logits_ld), int(vocab), float(temperature), int(seed), int(step), out.path_stride,
        ctypes.byref(out.c), _ptr(workspace), ws_bytes, int(max_slices), int(max_spins),
        _stream(stream)))


def spec_accept_topk(batch, parents, tokens, p_logits, vocab, temperature, seed, step, out,
                     workspace, logits_ld=None, stream=None):
    if logits_ld is None:
        logits_ld = p_logits.stride(0)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(LIB.spec_accept_topk(ctypes.byref(batch.c), _ptr(parents), _ptr(tokens),
                                _ptr(p_logits), int(logits_ld), int(vocab), float(temperature),
                                int(seed), int(step), out.path_stride, ctypes.byref(out.c),
                                _ptr(workspace), ws_bytes, _stream(stream)))


def spec_lm_head_accept_workspace_bytes(batch, vocab):
    n = LIB.spec_lm_head_accept_workspace_bytes(ctypes.byref(batch.c), int(vocab))
    if n == 0:
        raise SpecError(2, LIB.spec_last_error().decode())
    return int(n)


def spec_lm_head_accept(batch, parents, tokens, hidden, weight, q_logits, vocab, temperature,
                        seed, step, out, workspace, logits=None, children=SPEC_CHILDREN_SAMPLED,
                        logits_ld=None, stream=None):
    """hidden [R][H] and weight [V][H] bf16; logits [R][ld] fp32 output (None
    allowed at temperature 0); q_logits as spec_accept_sample.  The shapes the
    library cannot see through raw pointers are checked here first."""
    R = batch.R
    _shaped(hidden, "hidden", torch.bfloat16, rows=R)
    H = int(hidden.shape[1])
    _need(hidden.is_contiguous(), 2, "hidden must be contiguous [R][H]")
    _shaped(weight, "weight", torch.bfloat16, rows=int(vocab), cols=H)
    _need(weight.is_contiguous() and int(weight.shape[1]) == H, 2,
          f"weight must be contiguous [V][{H}], not {tuple(weight.shape)}")
    if logits_ld is None:
        ref = logits if logits is not None else q_logits
        logits_ld = ref.stride(0) if ref is not None else ((int(vocab) + 3) // 4) * 4
    named = [("hidden", hidden), ("weight", weight)]
    for name, t in (("logits", logits), ("q_logits", q_logits)):
        if t is not None:
            _shaped(t, name, torch.float32, rows=R, cols=int(vocab))
            _need(t.stride(0) == int(logits_ld), 2,
                  f"{name} row stride {t.stride(0)} differs from logits_ld {int(logits_ld)}")
            named.append((name, t))
    for name, t in named:
        _need(t.is_cuda, 1, f"{name} must be in device memory")
    head = CLmHead(_ptr(hidden), _ptr(weight), int(hidden.shape[1]), _ptr(logits))
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(LIB.spec_lm_head_accept(ctypes.byref(batch.c), _ptr(parents), _ptr(tokens),
                                   ctypes.byref(head), _ptr(q_logits), int(logits_ld), int(vocab),
                                   float(temperature), int(children), int(seed), int(step),
                                   out.path_stride, ctypes.byref(out.c), _ptr(workspace), ws_bytes,
                                   _stream(stream)))


def spec_kv_commit(batch, kv, accept_len, path, new_len, freed_blocks=None, stream=None):
    _check(LIB.spec_kv_commit(ctypes.byref(batch.c), ctypes.byref(kv.c), _ptr(accept_len),
                              _ptr(path), int(path.shape[1]), _ptr(new_len), _ptr(freed_blocks),
                              _stream(stream)))


class DraftTree:
    """Device state of a batch of growing draft trees (torch-owned arrays)."""

    def __init__(self, batch, topk, capacity, device):
        i32 = dict(dtype=torch.int32, device=device)
        self.parent = torch.empty((batch, capacity), **i32)
        self.token = torch.empty((batch, capacity), **i32)
        self.score = torch.empty((batch, capacity), dtype=torch.float32, device=device)
        self.depth = torch.empty((batch, capacity), **i32)
        self.count = torch.empty(batch, **i32)
        self.frontier = torch.empty((batch, topk), **i32)
        self.flags = torch.empty(batch, **i32)
        self.c = CDraftTree(int(batch), int(topk), int(capacity), _ptr(self.parent),
                            _ptr(self.token), _ptr(self.score), _ptr(self.depth),
                            _ptr(self.count), _ptr(self.frontier), _ptr(self.flags))

    @property
    def batch(self):
        return int(self.c.batch)


def spec_draft_begin(tree, root_tokens, stream=None):
    _check(LIB.spec_draft_begin(ctypes.byref(tree.c), _ptr(root_tokens), _stream(stream)))


def spec_draft_expand(tree, cand_tokens, cand_probs, gates=(), stream=None):
    n = len(gates)
    gd = np.ascontiguousarray([int(d) for d, _ in gates] or [0], dtype=np.int32)
    gs = np.ascontiguousarray([float(t) for _, t in gates] or [0.0], dtype=np.float32)
    _check(LIB.spec_draft_expand(ctypes.byref(tree.c), _ptr(cand_tokens), _ptr(cand_probs), n,
                                 _ptr(gd), _ptr(gs), _stream(stream)))


def spec_draft_select_workspace_bytes(batch, max_rows):
    n = LIB.spec_draft_select_workspace_bytes(int(batch), int(max_rows))
    if n == 0:
        raise SpecError(2, LIB.spec_last_error().decode())
    return int(n)


def spec_draft_select(tree, budget_rows, max_rows, row_offsets, parents, tokens, workspace,
                      node_of_row=None, stream=None):
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(LIB.spec_draft_select(ctypes.byref(tree.c), int(budget_rows), int(max_rows),
                                 _ptr(row_offsets), _ptr(parents), _ptr(tokens), _ptr(node_of_row),
                                 int(parents.numel()), _ptr(workspace), ws_bytes, _stream(stream)))


def spec_abi_version():
    return int(LIB.spec_abi_version())


def spec_status_string(status):
    return LIB.spec_status_string(int(status)).decode()
