// C ABI of the verify-step library: host-side validation, planning and
// launches.  Every check runs before anything is enqueued; a failed check
// returns a status and leaves a thread-local message.
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <string>

#include "../../include/spec_verify.h"
#include "launch.hpp"

static_assert(SPEC_MAX_TREE_ROWS == spec::kMaxRows, "row limit");
static_assert(SPEC_KV_BLOCK == spec::kBlock, "block size");
static_assert(SPEC_FLAG_ZERO_RESIDUAL == spec::kFlagZeroResidual, "flag");
static_assert(SPEC_FLAG_PATH_TRUNCATED == spec::kFlagPathTruncated, "flag");
static_assert(SPEC_FLAG_BAD_TREE == spec::kFlagBadTree, "flag");
static_assert(SPEC_FLAG_SYNC_TIMEOUT == spec::kFlagSyncTimeout, "flag");
static_assert(SPEC_ACCEPT_SCRATCH_BYTES == spec::kAcceptScratchBytes, "scratch size");
static_assert(SPEC_DRAFT_FLAG_CAPACITY == spec::kDraftFlagCapacity, "flag");
static_assert(SPEC_DRAFT_FLAG_BAD_STATE == spec::kDraftFlagBadState, "flag");

namespace {

thread_local std::string g_error;

spec_status fail(spec_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_error = buf;
  return st;
}

spec_status ok() {
  g_error.clear();
  return SPEC_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

using spec::kMaxVocab;

spec_status check_batch(const spec_batch* bt, int* R_out) {
  if (!bt) return fail(SPEC_ERR_NULL, "batch is NULL");
  if (bt->batch < 1) return fail(SPEC_ERR_SHAPE, "batch = %d, need >= 1", bt->batch);
  if (bt->max_rows < 1 || bt->max_rows > SPEC_MAX_TREE_ROWS)
    return fail(SPEC_ERR_SHAPE, "max_rows = %d, need 1..%d", bt->max_rows, SPEC_MAX_TREE_ROWS);
  if (!bt->row_offsets_h || !bt->row_offsets_d || !bt->prefix_len_h || !bt->prefix_len_d)
    return fail(SPEC_ERR_NULL, "batch row_offsets/prefix_len (host and device) must be set");
  if (bt->row_offsets_h[0] != 0) return fail(SPEC_ERR_TREE, "row_offsets[0] = %d, need 0", bt->row_offsets_h[0]);
  for (int b = 0; b < bt->batch; ++b) {
    const int n = bt->row_offsets_h[b + 1] - bt->row_offsets_h[b];
    if (n < 1) return fail(SPEC_ERR_TREE, "request %d has %d rows, need >= 1 (its root)", b, n);
    if (n > bt->max_rows) return fail(SPEC_ERR_TREE, "request %d has %d rows > max_rows %d", b, n, bt->max_rows);
    if (bt->prefix_len_h[b] < 0) return fail(SPEC_ERR_SHAPE, "prefix_len[%d] = %d < 0", b, bt->prefix_len_h[b]);
    if ((int64_t)bt->prefix_len_h[b] + n > (1 << 30))
      return fail(SPEC_ERR_SHAPE, "request %d: prefix + rows too long", b);
  }
  if (R_out) *R_out = bt->row_offsets_h[bt->batch];
  return SPEC_OK;
}

int mask_words(const spec_batch* bt) { return (bt->max_rows + 63) / 64; }

spec_status check_kv(const spec_batch* bt, const spec_kv* kv) {
  if (!kv) return fail(SPEC_ERR_NULL, "kv is NULL");
  if (!kv->k || !kv->v) return fail(SPEC_ERR_NULL, "kv->k / kv->v is NULL");
  if (!aligned16(kv->k) || !aligned16(kv->v)) return fail(SPEC_ERR_SHAPE, "kv->k / kv->v must be 16-byte aligned");
  if (kv->dtype != SPEC_BF16 && kv->dtype != SPEC_F32) return fail(SPEC_ERR_DTYPE, "kv->dtype = %d", (int)kv->dtype);
  if (kv->num_kv_heads < 1) return fail(SPEC_ERR_SHAPE, "num_kv_heads = %d", kv->num_kv_heads);
  if (kv->head_dim != 64 && kv->head_dim != 128)
    return fail(SPEC_ERR_UNSUPPORTED, "head_dim = %d, supported: 64, 128", kv->head_dim);
  if (kv->layout == SPEC_KV_CONTIGUOUS) {
    for (int b = 0; b < bt->batch; ++b) {
      const int need = bt->prefix_len_h[b] + bt->row_offsets_h[b + 1] - bt->row_offsets_h[b];
      if (need > kv->capacity)
        return fail(SPEC_ERR_CAPACITY, "request %d needs %d cache slots > capacity %d", b, need, kv->capacity);
    }
  } else if (kv->layout == SPEC_KV_PAGED) {
    if (kv->block_size != SPEC_KV_BLOCK) return fail(SPEC_ERR_UNSUPPORTED, "block_size = %d, supported: 16", kv->block_size);
    if (!kv->block_table_d) return fail(SPEC_ERR_NULL, "paged kv without block_table_d");
    for (int b = 0; b < bt->batch; ++b) {
      const int need = bt->prefix_len_h[b] + bt->row_offsets_h[b + 1] - bt->row_offsets_h[b];
      const int blocks = (need + SPEC_KV_BLOCK - 1) / SPEC_KV_BLOCK;
      if (blocks > kv->max_blocks_per_seq)
        return fail(SPEC_ERR_CAPACITY, "request %d needs %d blocks > max_blocks_per_seq %d", b, blocks, kv->max_blocks_per_seq);
    }
  } else {
    return fail(SPEC_ERR_SHAPE, "kv->layout = %d", (int)kv->layout);
  }
  return SPEC_OK;
}

spec::KvAddr kv_addr(const spec_kv* kv) {
  spec::KvAddr a;
  a.paged = kv->layout == SPEC_KV_PAGED;
  a.hkv = kv->num_kv_heads;
  a.d = kv->head_dim;
  a.capacity = kv->capacity;
  a.block_table = kv->block_table_d;
  a.mbps = kv->max_blocks_per_seq;
  return a;
}

spec::LaunchCtx ctx(const spec_batch* bt, hipStream_t stream) {
  spec::LaunchCtx c;
  c.B = bt->batch;
  c.row_offsets_d = bt->row_offsets_d;
  c.prefix_len_d = bt->prefix_len_d;
  c.stream = stream;
  return c;
}

spec_status launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(SPEC_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
  return ok();
}

int esize(spec_dtype d) { return d == SPEC_BF16 ? 2 : 4; }

}  // namespace

extern "C" {

int spec_abi_version(void) { return SPEC_ABI_VERSION; }

const char* spec_last_error(void) { return g_error.c_str(); }

const char* spec_status_string(spec_status s) {
  switch (s) {
    case SPEC_OK: return "SPEC_OK";
    case SPEC_ERR_NULL: return "SPEC_ERR_NULL";
    case SPEC_ERR_SHAPE: return "SPEC_ERR_SHAPE";
    case SPEC_ERR_TREE: return "SPEC_ERR_TREE";
    case SPEC_ERR_CAPACITY: return "SPEC_ERR_CAPACITY";
    case SPEC_ERR_DTYPE: return "SPEC_ERR_DTYPE";
    case SPEC_ERR_HIP: return "SPEC_ERR_HIP";
    case SPEC_ERR_UNSUPPORTED: return "SPEC_ERR_UNSUPPORTED";
    case SPEC_ERR_WORKSPACE: return "SPEC_ERR_WORKSPACE";
  }
  return "SPEC_ERR_UNKNOWN";
}

spec_status spec_tree_build_mask(const spec_batch* batch, const int32_t* parents_d, uint64_t* mask_d,
                                 int32_t* depth_d, int32_t* position_d, int32_t* err_row_d,
                                 hipStream_t stream) {
  int R = 0;
  spec_status st = check_batch(batch, &R);
  if (st != SPEC_OK) return st;
  if (!parents_d || !mask_d || !err_row_d) return fail(SPEC_ERR_NULL, "parents_d, mask_d and err_row_d are required");
  return launched(spec::launch_build_mask(ctx(batch, stream), parents_d, mask_d, mask_words(batch),
                                          depth_d, position_d, err_row_d),
                  "spec_tree_build_mask");
}

spec_status spec_kv_append(const spec_batch* batch, const spec_kv* kv, const void* k_new_d,
                           const void* v_new_d, hipStream_t stream) {
  int R = 0;
  spec_status st = check_batch(batch, &R);
  if (st != SPEC_OK) return st;
  if ((st = check_kv(batch, kv)) != SPEC_OK) return st;
  if (!k_new_d || !v_new_d) return fail(SPEC_ERR_NULL, "k_new_d / v_new_d is NULL");
  if (!aligned16(k_new_d) || !aligned16(v_new_d)) return fail(SPEC_ERR_SHAPE, "k_new_d / v_new_d must be 16-byte aligned");
  return launched(spec::launch_kv_append(ctx(batch, stream), R, kv_addr(kv), esize(kv->dtype), k_new_d,
                                         v_new_d, kv->k, kv->v),
                  "spec_kv_append");
}

size_t spec_tree_attn_workspace_bytes(const spec_batch* batch, const spec_kv* kv, int32_t num_q_heads) {
  if (check_batch(batch, nullptr) != SPEC_OK || check_kv(batch, kv) != SPEC_OK) return 0;
  if (num_q_heads < 1 || num_q_heads % kv->num_kv_heads) {
    fail(SPEC_ERR_SHAPE, "num_q_heads = %d not a multiple of num_kv_heads = %d", num_q_heads, kv->num_kv_heads);
    return 0;
  }
  if (kv->dtype == SPEC_F32) return 256;
  const spec::AttnPlan p = spec::plan_attention(batch->batch, batch->row_offsets_h, batch->prefix_len_h,
                                                num_q_heads, kv->num_kv_heads);
  if (p.items < 0) {
    fail(SPEC_ERR_UNSUPPORTED, "a request holds more than %lld keys",
         (long long)spec::kMaxAttnKeys);
    return 0;
  }
  return spec::attention_workspace_bytes(p, kv->head_dim);
}

spec_status spec_tree_attn_verify(const spec_batch* batch, const spec_kv* kv, const void* q_d,
                                  int32_t num_q_heads, const uint64_t* mask_d, float softmax_scale,
                                  void* out_d, spec_dtype out_dtype, void* workspace_d,
                                  size_t workspace_bytes, hipStream_t stream) {
  int R = 0;
  spec_status st = check_batch(batch, &R);
  if (st != SPEC_OK) return st;
  if ((st = check_kv(batch, kv)) != SPEC_OK) return st;
  if (!q_d || !mask_d || !out_d) return fail(SPEC_ERR_NULL, "q_d, mask_d and out_d are required");
  if (!aligned16(q_d) || !aligned16(out_d)) return fail(SPEC_ERR_SHAPE, "q_d / out_d must be 16-byte aligned");
  if (num_q_heads < 1 || num_q_heads % kv->num_kv_heads)
    return fail(SPEC_ERR_SHAPE, "num_q_heads = %d not a multiple of num_kv_heads = %d", num_q_heads, kv->num_kv_heads);
  if (out_dtype != SPEC_BF16 && out_dtype != SPEC_F32) return fail(SPEC_ERR_DTYPE, "out_dtype = %d", (int)out_dtype);
  if (!(softmax_scale == softmax_scale) || softmax_scale <= 0.0f || softmax_scale > 1e30f)
    return fail(SPEC_ERR_SHAPE, "softmax_scale must be finite and > 0");
  const spec::KvAddr addr = kv_addr(kv);
  const int out_f32 = out_dtype == SPEC_F32;
  if (kv->dtype == SPEC_F32) {
    return launched(spec::launch_attention_f32(ctx(batch, stream), R, addr, num_q_heads, (const float*)q_d,
                                               mask_d, mask_words(batch), softmax_scale,
                                               (const float*)kv->k, (const float*)kv->v, out_d, out_f32),
                    "spec_tree_attn_verify");
  }
  const spec::AttnPlan p = spec::plan_attention(batch->batch, batch->row_offsets_h, batch->prefix_len_h,
                                                num_q_heads, kv->num_kv_heads);
  if (p.items < 0)
    return fail(SPEC_ERR_UNSUPPORTED, "a request holds more than %lld keys", (long long)spec::kMaxAttnKeys);
  const size_t need = spec::attention_workspace_bytes(p, kv->head_dim);
  if (!workspace_d || workspace_bytes < need)
    return fail(SPEC_ERR_WORKSPACE, "attention workspace %zu bytes < required %zu", workspace_bytes, need);
  if (!aligned16(workspace_d)) return fail(SPEC_ERR_SHAPE, "workspace must be 16-byte aligned");
  return launched(spec::launch_attention_bf16(ctx(batch, stream), p, addr, num_q_heads, q_d, mask_d,
                                              mask_words(batch), softmax_scale, kv->k, kv->v, out_d,
                                              out_f32, workspace_d),
                  "spec_tree_attn_verify");
}

size_t spec_accept_workspace_bytes(const spec_batch* batch, int32_t vocab) {
  int R = 0;
  if (check_batch(batch, &R) != SPEC_OK) return 0;
  if (vocab < 1 || vocab > kMaxVocab) {
    fail(SPEC_ERR_UNSUPPORTED, "vocab = %d, supported 1..%d", vocab, kMaxVocab);
    return 0;
  }
  return spec::accept_workspace_bytes(R, batch->batch, vocab);
}

static spec_status accept_call(const spec_batch* batch, const int32_t* parents_d,
                               const int32_t* tokens_d, const float* p_logits_d,
                               const float* q_logits_d, bool topk, int64_t logits_ld,
                               int32_t vocab, float temperature, uint64_t seed, uint64_t step,
                               int32_t path_stride, const spec_accept_out* out, void* workspace_d,
                               size_t workspace_bytes, hipStream_t stream, const char* name,
                               spec::WalkKnobs knobs = spec::WalkKnobs(),
                               bool use_scratch = false) {
  int R = 0;
  spec_status st = check_batch(batch, &R);
  if (st != SPEC_OK) return st;
  if (!parents_d || !tokens_d || !p_logits_d) return fail(SPEC_ERR_NULL, "parents_d, tokens_d and p_logits_d are required");
  if (!(temperature >= 0.0f) || temperature > 1e30f) return fail(SPEC_ERR_SHAPE, "temperature must be finite and >= 0");
  if (!topk && temperature > 0.0f && !q_logits_d) return fail(SPEC_ERR_NULL, "q_logits_d is required when temperature > 0");
  if (vocab < 1 || vocab > kMaxVocab) return fail(SPEC_ERR_UNSUPPORTED, "vocab = %d, supported 1..%d", vocab, kMaxVocab);
  if (logits_ld < vocab || logits_ld % 4) return fail(SPEC_ERR_SHAPE, "logits_ld = %lld must be >= vocab and a multiple of 4", (long long)logits_ld);
  if (!aligned16(p_logits_d) || (q_logits_d && !aligned16(q_logits_d)))
    return fail(SPEC_ERR_SHAPE, "logits pointers must be 16-byte aligned");
  if (path_stride < 1) return fail(SPEC_ERR_SHAPE, "path_stride = %d, need >= 1", path_stride);
  if (!out || !out->accept_len_d || !out->path_d || !out->tokens_d)
    return fail(SPEC_ERR_NULL, "out, accept_len_d, path_d and tokens_d are required");
  const size_t need = spec::accept_workspace_bytes(R, batch->batch, vocab);
  if (use_scratch) {
    // the library's own device array instead of a caller workspace
    if (need > spec::kAcceptScratchBytes)
      return fail(SPEC_ERR_WORKSPACE,
                  "%s: this batch needs %zu bytes of scratch, more than the %zu it holds "
                  "(spec_accept_sample takes a caller workspace of any size)",
                  name, need, spec::kAcceptScratchBytes);
    const hipError_t e = spec::accept_scratch(&workspace_d);
    if (e != hipSuccess)
      return fail(SPEC_ERR_HIP, "%s: scratch lookup failed: %s", name, hipGetErrorString(e));
    workspace_bytes = spec::kAcceptScratchBytes;
  }
  if (!workspace_d || workspace_bytes < need)
    return fail(SPEC_ERR_WORKSPACE, "accept workspace %zu bytes < required %zu", workspace_bytes, need);
  if (!aligned16(workspace_d)) return fail(SPEC_ERR_SHAPE, "workspace must be 16-byte aligned");
  return launched(spec::launch_accept(ctx(batch, stream), R, parents_d, tokens_d, p_logits_d,
                                      (temperature > 0.0f && !topk) ? q_logits_d : nullptr,
                                      logits_ld, vocab, temperature, seed, step, path_stride,
                                      out->accept_len_d, out->path_d, out->tokens_d,
                                      out->accept_mask_d, out->child_p_d, out->child_q_d,
                                      out->flags_d, workspace_d, knobs),
                  name);
}

spec_status spec_accept_sample(const spec_batch* batch, const int32_t* parents_d, const int32_t* tokens_d,
                               const float* p_logits_d, const float* q_logits_d, int64_t logits_ld,
                               int32_t vocab, float temperature, uint64_t seed, uint64_t step,
                               int32_t path_stride, const spec_accept_out* out, void* workspace_d,
                               size_t workspace_bytes, hipStream_t stream) {
  return accept_call(batch, parents_d, tokens_d, p_logits_d, q_logits_d, false, logits_ld, vocab,
                     temperature, seed, step, path_stride, out, workspace_d, workspace_bytes, stream,
                     "spec_accept_sample");
}

spec_status spec_accept_sample_noalloc(const spec_batch* batch, const int32_t* parents_d,
                                       const int32_t* tokens_d, const float* p_logits_d,
                                       const float* q_logits_d, int64_t logits_ld, int32_t vocab,
                                       float temperature, uint64_t seed, uint64_t step,
                                       int32_t path_stride, const spec_accept_out* out,
                                       hipStream_t stream) {
  return accept_call(batch, parents_d, tokens_d, p_logits_d, q_logits_d, false, logits_ld, vocab,
                     temperature, seed, step, path_stride, out, nullptr, 0, stream,
                     "spec_accept_sample_noalloc", spec::WalkKnobs(), /*use_scratch=*/true);
}

spec_status spec_accept_sample_walk_knobs(const spec_batch* batch, const int32_t* parents_d,
                                          const int32_t* tokens_d, const float* p_logits_d,
                                          const float* q_logits_d, int64_t logits_ld,
                                          int32_t vocab, float temperature, uint64_t seed,
                                          uint64_t step, int32_t path_stride,
                                          const spec_accept_out* out, void* workspace_d,
                                          size_t workspace_bytes, int32_t max_slices,
                                          int32_t max_spins, hipStream_t stream) {
  if (max_slices < 0) return fail(SPEC_ERR_SHAPE, "max_slices = %d, need >= 0", max_slices);
  if (max_spins < -1) return fail(SPEC_ERR_SHAPE, "max_spins = %d, need >= -1", max_spins);
  spec::WalkKnobs k;
  k.max_slices = max_slices;
  k.max_spins = max_spins;
  return accept_call(batch, parents_d, tokens_d, p_logits_d, q_logits_d, false, logits_ld, vocab,
                     temperature, seed, step, path_stride, out, workspace_d, workspace_bytes, stream,
                     "spec_accept_sample_walk_knobs", k);
}

spec_status spec_test_exp_f64(const double* x_d, double* y_d, int64_t n, int32_t variant,
                              hipStream_t stream) {
  if (!x_d || !y_d) return fail(SPEC_ERR_NULL, "x_d and y_d are required");
  if (n < 1 || n > (int64_t)1 << 32) return fail(SPEC_ERR_SHAPE, "n = %lld, need 1..2^32", (long long)n);
  if (variant < 0 || variant > 4) return fail(SPEC_ERR_SHAPE, "variant = %d, need 0..4", variant);
  return launched(spec::launch_exp64_probe(x_d, y_d, n, variant, stream), "spec_test_exp_f64");
}

spec_status spec_accept_topk(const spec_batch* batch, const int32_t* parents_d, const int32_t* tokens_d,
                             const float* p_logits_d, int64_t logits_ld, int32_t vocab,
                             float temperature, uint64_t seed, uint64_t step, int32_t path_stride,
                             const spec_accept_out* out, void* workspace_d, size_t workspace_bytes,
                             hipStream_t stream) {
  return accept_call(batch, parents_d, tokens_d, p_logits_d, nullptr, true, logits_ld, vocab,
                     temperature, seed, step, path_stride, out, workspace_d, workspace_bytes, stream,
                     "spec_accept_topk");
}

size_t spec_lm_head_accept_workspace_bytes(const spec_batch* batch, int32_t vocab) {
  int R = 0;
  if (check_batch(batch, &R) != SPEC_OK || vocab < 1 || vocab > kMaxVocab) return 0;
  return ((spec::accept_workspace_bytes(R, batch->batch, vocab) + 255) & ~(size_t)255) +
         spec::head_tiles_bytes(R, vocab);
}

spec_status spec_lm_head_accept(const spec_batch* batch, const int32_t* parents_d,
                                const int32_t* tokens_d, const spec_lm_head* head,
                                const float* q_logits_d, int64_t logits_ld, int32_t vocab,
                                float temperature, int32_t children, uint64_t seed, uint64_t step,
                                int32_t path_stride, const spec_accept_out* out, void* workspace_d,
                                size_t workspace_bytes, hipStream_t stream) {
  int R = 0;
  spec_status st = check_batch(batch, &R);
  if (st != SPEC_OK) return st;
  if (!parents_d || !tokens_d) return fail(SPEC_ERR_NULL, "parents_d and tokens_d are required");
  if (!head || !head->hidden_d || !head->weight_d)
    return fail(SPEC_ERR_NULL, "head, head->hidden_d and head->weight_d are required");
  if (!aligned16(head->hidden_d) || !aligned16(head->weight_d))
    return fail(SPEC_ERR_SHAPE, "head->hidden_d / head->weight_d must be 16-byte aligned");
  const int H = head->hidden_size;
  if (H < 64 || H > 65536 || H % 64)
    return fail(SPEC_ERR_UNSUPPORTED, "hidden_size = %d, supported: multiples of 64 in 64..65536", H);
  if (!(temperature >= 0.0f) || temperature > 1e30f) return fail(SPEC_ERR_SHAPE, "temperature must be finite and >= 0");
  if (children != SPEC_CHILDREN_SAMPLED && children != SPEC_CHILDREN_TOPK)
    return fail(SPEC_ERR_SHAPE, "children = %d, need SPEC_CHILDREN_SAMPLED or SPEC_CHILDREN_TOPK", children);
  const bool topk = children == SPEC_CHILDREN_TOPK;
  if (!topk && temperature > 0.0f && !q_logits_d) return fail(SPEC_ERR_NULL, "q_logits_d is required when temperature > 0");
  if (temperature > 0.0f && !head->logits_d) return fail(SPEC_ERR_NULL, "head->logits_d is required when temperature > 0");
  if (vocab < 1 || vocab > kMaxVocab) return fail(SPEC_ERR_UNSUPPORTED, "vocab = %d, supported 1..%d", vocab, kMaxVocab);
  if ((int64_t)vocab * H >= (1ll << 31) || (int64_t)R * H >= (1ll << 31))
    return fail(SPEC_ERR_UNSUPPORTED, "vocab * hidden_size and rows * hidden_size must stay below 2^31");
  if (logits_ld < vocab || logits_ld % 4) return fail(SPEC_ERR_SHAPE, "logits_ld = %lld must be >= vocab and a multiple of 4", (long long)logits_ld);
  if ((head->logits_d && !aligned16(head->logits_d)) || (q_logits_d && !aligned16(q_logits_d)))
    return fail(SPEC_ERR_SHAPE, "logits pointers must be 16-byte aligned");
  if (path_stride < 1) return fail(SPEC_ERR_SHAPE, "path_stride = %d, need >= 1", path_stride);
  if (!out || !out->accept_len_d || !out->path_d || !out->tokens_d)
    return fail(SPEC_ERR_NULL, "out, accept_len_d, path_d and tokens_d are required");
  const size_t acc_bytes = (spec::accept_workspace_bytes(R, batch->batch, vocab) + 255) & ~(size_t)255;
  const size_t need = acc_bytes + spec::head_tiles_bytes(R, vocab);
  if (!workspace_d || workspace_bytes < need)
    return fail(SPEC_ERR_WORKSPACE, "LM head workspace %zu bytes < required %zu", workspace_bytes, need);
  if (!aligned16(workspace_d)) return fail(SPEC_ERR_SHAPE, "workspace must be 16-byte aligned");
  spec::HeadTiles tiles = spec::head_tiles((char*)workspace_d + acc_bytes, R, vocab);
  tiles.hidden = (const uint16_t*)head->hidden_d;
  tiles.weight = (const uint16_t*)head->weight_d;
  tiles.H = H;
  hipError_t e = spec::launch_lm_head(R, (const uint16_t*)head->hidden_d, H,
                                      (const uint16_t*)head->weight_d, vocab, temperature,
                                      head->logits_d, logits_ld, tiles, batch->batch,
                                      batch->row_offsets_d, parents_d, stream);
  if (e != hipSuccess) return launched(e, "spec_lm_head_accept (head)");
  return launched(spec::launch_accept(ctx(batch, stream), R, parents_d, tokens_d, head->logits_d,
                                      (temperature > 0.0f && !topk) ? q_logits_d : nullptr,
                                      logits_ld, vocab, temperature, seed, step, path_stride,
                                      out->accept_len_d, out->path_d, out->tokens_d,
                                      out->accept_mask_d, out->child_p_d, out->child_q_d,
                                      out->flags_d, workspace_d, spec::WalkKnobs(), &tiles),
                  "spec_lm_head_accept");
}

spec_status spec_kv_commit(const spec_batch* batch, const spec_kv* kv, const int32_t* accept_len_d,
                           const int32_t* path_d, int32_t path_stride, int32_t* new_len_d,
                           int32_t* freed_blocks_d, hipStream_t stream) {
  int R = 0;
  spec_status st = check_batch(batch, &R);
  if (st != SPEC_OK) return st;
  if ((st = check_kv(batch, kv)) != SPEC_OK) return st;
  if (!accept_len_d || !path_d || !new_len_d) return fail(SPEC_ERR_NULL, "accept_len_d, path_d and new_len_d are required");
  if (path_stride < 1) return fail(SPEC_ERR_SHAPE, "path_stride = %d, need >= 1", path_stride);
  return launched(spec::launch_kv_commit(ctx(batch, stream), kv_addr(kv), esize(kv->dtype), accept_len_d,
                                         path_d, path_stride, kv->k, kv->v, new_len_d,
                                         kv->layout == SPEC_KV_PAGED ? freed_blocks_d : nullptr),
                  "spec_kv_commit");
}

static spec_status check_draft(const spec_draft_tree* t) {
  if (!t) return fail(SPEC_ERR_NULL, "tree is NULL");
  if (t->batch < 1) return fail(SPEC_ERR_SHAPE, "batch = %d, need >= 1", t->batch);
  if (t->topk < 1 || t->topk > spec::kDraftMaxK)
    return fail(SPEC_ERR_UNSUPPORTED, "topk = %d, supported 1..%d", t->topk, spec::kDraftMaxK);
  if (t->capacity < 1 || t->capacity > spec::kDraftMaxNodes)
    return fail(SPEC_ERR_UNSUPPORTED, "capacity = %d, supported 1..%d", t->capacity, spec::kDraftMaxNodes);
  if ((int64_t)t->batch * t->capacity >= (1ll << 32))
    return fail(SPEC_ERR_SHAPE, "batch * capacity must stay below 2^32");
  if (!t->parent_d || !t->token_d || !t->score_d || !t->depth_d || !t->count_d || !t->frontier_d || !t->flags_d)
    return fail(SPEC_ERR_NULL, "every spec_draft_tree array is required");
  return SPEC_OK;
}

static spec::DraftTree draft_of(const spec_draft_tree* t) {
  return spec::DraftTree{t->batch, t->topk, t->capacity, t->parent_d, t->token_d, t->score_d,
                         t->depth_d, t->count_d, t->frontier_d, t->flags_d};
}

spec_status spec_draft_begin(const spec_draft_tree* tree, const int32_t* root_tokens_d, hipStream_t stream) {
  spec_status st = check_draft(tree);
  if (st != SPEC_OK) return st;
  if (!root_tokens_d) return fail(SPEC_ERR_NULL, "root_tokens_d is required");
  return launched(spec::launch_draft_begin(draft_of(tree), root_tokens_d, stream), "spec_draft_begin");
}

spec_status spec_draft_expand(const spec_draft_tree* tree, const int32_t* cand_tokens_d,
                              const float* cand_probs_d, int32_t n_gates, const int32_t* gate_depth_h,
                              const float* gate_score_h, hipStream_t stream) {
  spec_status st = check_draft(tree);
  if (st != SPEC_OK) return st;
  if (!cand_tokens_d || !cand_probs_d) return fail(SPEC_ERR_NULL, "cand_tokens_d and cand_probs_d are required");
  if (n_gates < 0 || n_gates > spec::kDraftMaxGates)
    return fail(SPEC_ERR_UNSUPPORTED, "n_gates = %d, supported 0..%d", n_gates, spec::kDraftMaxGates);
  if (n_gates > 0 && (!gate_depth_h || !gate_score_h)) return fail(SPEC_ERR_NULL, "gate arrays are required when n_gates > 0");
  spec::DraftGates g{};
  g.n = n_gates;
  for (int i = 0; i < n_gates; ++i) {
    if (gate_depth_h[i] < 1) return fail(SPEC_ERR_SHAPE, "gate_depth[%d] = %d, need >= 1", i, gate_depth_h[i]);
    if (!(gate_score_h[i] >= 0.0f) || gate_score_h[i] > 1e30f)
      return fail(SPEC_ERR_SHAPE, "gate_score[%d] must be finite and >= 0", i);
    g.depth[i] = gate_depth_h[i];
    g.score[i] = gate_score_h[i];
  }
  return launched(spec::launch_draft_expand(draft_of(tree), cand_tokens_d, cand_probs_d, g, stream),
                  "spec_draft_expand");
}

size_t spec_draft_select_workspace_bytes(int32_t batch, int32_t max_rows) {
  if (batch < 1 || max_rows < 1) {
    fail(SPEC_ERR_SHAPE, "batch and max_rows must be >= 1");
    return 0;
  }
  return spec::draft_select_workspace_bytes(batch, max_rows);
}

spec_status spec_draft_select(const spec_draft_tree* tree, int32_t budget_rows, int32_t max_rows,
                              int32_t* row_offsets_d, int32_t* parents_d, int32_t* tokens_d,
                              int32_t* node_of_row_d, int32_t rows_capacity, void* workspace_d,
                              size_t workspace_bytes, hipStream_t stream) {
  spec_status st = check_draft(tree);
  if (st != SPEC_OK) return st;
  const int B = tree->batch;
  if (B > spec::kDraftSelMaxB) return fail(SPEC_ERR_UNSUPPORTED, "batch = %d, selection supports up to %d", B, spec::kDraftSelMaxB);
  if (max_rows < 1 || max_rows > SPEC_MAX_TREE_ROWS || max_rows > tree->capacity)
    return fail(SPEC_ERR_SHAPE, "max_rows = %d, need 1..min(%d, capacity %d)", max_rows, SPEC_MAX_TREE_ROWS, tree->capacity);
  if ((int64_t)B * (max_rows - 1) > spec::kDraftSelMax)
    return fail(SPEC_ERR_UNSUPPORTED, "batch * (max_rows - 1) = %lld, supported up to %d",
                (long long)B * (max_rows - 1), spec::kDraftSelMax);
  if (budget_rows < B) return fail(SPEC_ERR_SHAPE, "budget_rows = %d < batch %d (every root takes a row)", budget_rows, B);
  if (!row_offsets_d || !parents_d || !tokens_d) return fail(SPEC_ERR_NULL, "row_offsets_d, parents_d and tokens_d are required");
  const int64_t most = std::min<int64_t>(budget_rows, (int64_t)B * max_rows);
  if (rows_capacity < most)
    return fail(SPEC_ERR_CAPACITY, "rows_capacity = %d < %lld rows the selection may emit", rows_capacity, (long long)most);
  const size_t need = spec::draft_select_workspace_bytes(B, max_rows);
  if (!workspace_d || workspace_bytes < need)
    return fail(SPEC_ERR_WORKSPACE, "select workspace %zu bytes < required %zu", workspace_bytes, need);
  if (!aligned16(workspace_d)) return fail(SPEC_ERR_SHAPE, "workspace must be 16-byte aligned");
  return launched(spec::launch_draft_select(draft_of(tree), budget_rows, max_rows, row_offsets_d, parents_d,
                                            tokens_d, node_of_row_d, workspace_d, stream),
                  "spec_draft_select");
}

}  // extern "C"
