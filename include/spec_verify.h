/*
 * spec_verify.h -- C ABI of the speculative-decoding verify step on one
 * AMD Instinct MI355X (gfx950).
 *
 * The verify step of speculative decoding runs the target model once over a
 * flattened draft tree and keeps the longest draft path the target accepts:
 *
 *   spec_tree_build_mask   parents -> packed ancestor masks, depth, positions
 *   spec_kv_append         tree rows' K/V -> cache slots [L_b, L_b + N_b)
 *   spec_tree_attn_verify  tree attention: prefix + ancestors only
 *   spec_accept_sample     lossless acceptance walk + final token
 *   spec_accept_topk       the same for deterministic (top-k) children
 *   spec_lm_head_accept    target LM head fused with the acceptance statistics,
 *                          then the same walk
 *   spec_draft_begin / spec_draft_expand / spec_draft_select
 *                          build dynamic draft trees under a batch budget
 *   spec_kv_commit         compact the accepted path's K/V, roll back the rest
 *
 * Pages this interface restates (title, section):
 *   [TREE]  "投机推理算法的常见优化手段" (cnblogs) -- generating and verifying
 *           the draft tree: flattening, the tree mask (printed 6x6 matrix),
 *           the forward call with tree mask, position ids and KV cache, and
 *           verifying every token of every level.
 *   [MATH]  "【模型后训练与深度推理】9 推理加速：推测解码与级联推理" (CSDN),
 *           sections 7.1-7.2: accept with probability min(1, p/q), resample
 *           from norm(max(0, p - q)), emitted length counts the final token.
 *   [SD]    guijiagi.com speculative-decoding post: rejection-sampling rule
 *           (stop at the first rejection), batching with divergent progress,
 *           KV rollback by freeing paged blocks, variable-length candidates.
 *   [SURV]  "万字综述 10+ 种 LLM 投机采样推理加速方案", sections 5.2 (tree
 *           based parallel decoding), 6.2 (Cartesian trees), 4.3/8.1
 *           (temperature 0 = argmax; keep the longest matching prefix).
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Batch of B requests; request b owns tree rows [row_offsets[b],
 *    row_offsets[b+1]) of every per-row array (N_b = that count, root first,
 *    1 <= N_b <= max_rows <= SPEC_MAX_TREE_ROWS).  Rows are flattened in any
 *    topological order: local row 0 is the root and parent[i] < i.
 *  - L_b = prefix_len[b] tokens of KV are already cached for request b.
 *  - All pointers named *_d are device memory, *_h host memory.  The caller
 *    owns every buffer; the library never allocates or frees, and keeps no
 *    pointer after a call returns.  Scratch comes from caller workspaces
 *    sized by the *_workspace_bytes queries (which return 0 for invalid
 *    arguments).
 *  - Every call validates its arguments on the host first.  Invalid
 *    arguments return a status != SPEC_OK and launch nothing; the detail is
 *    in spec_last_error() (thread-local).  Valid calls enqueue kernels on
 *    `stream` and return SPEC_OK without waiting.  Errors found on the device
 *    (a bad parent array held in device memory) are reported through the
 *    documented output fields, never by a fault.
 *  - The library is thread-safe and holds no mutable global state apart from
 *    the thread-local error string.
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SPEC_ABI_VERSION 1
#define SPEC_MAX_TREE_ROWS 256   /* rows per request incl. the root: <= 4 mask words */
#define SPEC_KV_BLOCK 16         /* paged KV block size (tokens) */

typedef enum {
  SPEC_OK = 0,
  SPEC_ERR_NULL = 1,         /* a required pointer is NULL */
  SPEC_ERR_SHAPE = 2,        /* sizes, strides or alignment out of range */
  SPEC_ERR_TREE = 3,         /* host-visible tree metadata inconsistent */
  SPEC_ERR_CAPACITY = 4,     /* cache or output too small for the rows */
  SPEC_ERR_DTYPE = 5,        /* unsupported element type combination */
  SPEC_ERR_HIP = 6,          /* a HIP launch failed */
  SPEC_ERR_UNSUPPORTED = 7,  /* valid request this build does not handle */
  SPEC_ERR_WORKSPACE = 8     /* workspace NULL or smaller than required */
} spec_status;

typedef enum { SPEC_BF16 = 0, SPEC_F32 = 1 } spec_dtype;
typedef enum { SPEC_KV_CONTIGUOUS = 0, SPEC_KV_PAGED = 1 } spec_kv_layout;

/* Ragged batch metadata.  Both copies must hold the same values: the host
 * copy sizes grids and is validated, the device copy is read by kernels. */
typedef struct {
  int32_t batch;                  /* B >= 1 */
  int32_t max_rows;               /* >= every N_b, <= SPEC_MAX_TREE_ROWS;
                                     mask words per row W = ceil(max_rows/64) */
  const int32_t *row_offsets_h;   /* [B+1], row_offsets[0] = 0, strictly increasing */
  const int32_t *row_offsets_d;
  const int32_t *prefix_len_h;    /* [B], L_b >= 0 */
  const int32_t *prefix_len_d;
} spec_batch;

/* KV cache of one attention layer (caller-owned).
 *  contiguous: k, v are [B][Hkv][capacity][D]; request b's token t of head h
 *              at ((b*Hkv + h)*capacity + t)*D.
 *  paged:      k, v are [num_blocks][Hkv][16][D]; token t of request b lives
 *              in physical block block_table[b*max_blocks_per_seq + t/16],
 *              slot t%16.  Block ids are trusted (device memory). */
typedef struct {
  spec_kv_layout layout;
  spec_dtype dtype;               /* element type of k and v */
  int32_t num_kv_heads;           /* Hkv >= 1 */
  int32_t head_dim;               /* D: 64 or 128 */
  void *k;
  void *v;
  int32_t capacity;               /* contiguous: token slots per (request, head) */
  int32_t block_size;             /* paged: must be SPEC_KV_BLOCK */
  const int32_t *block_table_d;   /* paged: [B][max_blocks_per_seq] */
  int32_t max_blocks_per_seq;     /* paged */
} spec_kv;

/* ---------------------------------------------------------------------------
 * spec_tree_build_mask -- [TREE] tree-mask section.
 *
 * For every row i of request b: mask word w, bit j (j = 64*w + bit) is 1 iff
 * local row j is i itself or an ancestor of i (row = attending token, column
 * = attended token, diagonal set, as in the printed matrix).  depth_d[i] =
 * number of strict ancestors; position_d[i] = L_b + depth_i (the tree
 * position id).  The parent array is checked on the device: parent[0] must
 * be -1 and 0 <= parent[i] < i.  err_row_d[b] = -1 when request b is valid,
 * else the smallest invalid local row; its mask rows are then all zero and
 * its depth/position entries -1.
 *
 *   parents_d   int32 [R]   local parent index, -1 at each root
 *   mask_d      uint64 [R][W], W = ceil(max_rows/64)           (output)
 *   depth_d     int32 [R]   optional (NULL)                     (output)
 *   position_d  int32 [R]   optional (NULL)                     (output)
 *   err_row_d   int32 [B]                                       (output)
 */
spec_status spec_tree_build_mask(const spec_batch *batch, const int32_t *parents_d,
                                 uint64_t *mask_d, int32_t *depth_d, int32_t *position_d,
                                 int32_t *err_row_d, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * spec_kv_append -- [SURV] 5.2 / [TREE]: during verification the tree's K/V
 * rows occupy cache slots L_b .. L_b + N_b - 1 (row i at slot L_b + i).
 *
 *   k_new_d, v_new_d   [R][Hkv][D] of kv->dtype
 * Contiguous caches need capacity >= L_b + N_b; paged caches need
 * max_blocks_per_seq >= ceil((L_b + N_b)/16) with those blocks mapped.
 */
spec_status spec_kv_append(const spec_batch *batch, const spec_kv *kv,
                           const void *k_new_d, const void *v_new_d, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * spec_tree_attn_verify -- [TREE] forward with tree mask; [SURV] 5.2.
 *
 * out[i][h] = softmax_j(q[i][h] . k_j * softmax_scale) v_j over the keys row
 * i may see: every cached prefix token t < L_b of its request, and tree rows
 * j with mask bit (i, j) set (their K/V at slot L_b + j, see spec_kv_append).
 * Query head h reads KV head h / (Hq / Hkv) (grouped-query attention).
 *
 *   q_d        [R][Hq][D], same dtype as the cache
 *   mask_d     uint64 [R][W]: bit j of row i's words = row i sees new row j of
 *              its request.  Usually from spec_tree_build_mask (the ancestor
 *              mask); any other visibility of the new rows may be passed,
 *              such as the survey page's lookahead decoding mask (section
 *              8.2.3: causal branches that do not see each other) or rows
 *              seeing later rows.  Bits at or past N_b are ignored; a row
 *              must see at least one key (a prefix token or one bit).
 *   out_d      [R][Hq][D] of out_dtype (bf16 or f32)
 *   workspace  >= spec_tree_attn_workspace_bytes(batch, kv, Hq) bytes
 *              (split-KV partial results; contents need no initialisation)
 * bf16 caches run on the MFMA path (fp32 accumulation, fp32 online softmax);
 * f32 caches run on a plain fp32 vector path.
 */
size_t spec_tree_attn_workspace_bytes(const spec_batch *batch, const spec_kv *kv,
                                      int32_t num_q_heads);
spec_status spec_tree_attn_verify(const spec_batch *batch, const spec_kv *kv,
                                  const void *q_d, int32_t num_q_heads,
                                  const uint64_t *mask_d, float softmax_scale,
                                  void *out_d, spec_dtype out_dtype,
                                  void *workspace_d, size_t workspace_bytes,
                                  hipStream_t stream);

/* ---------------------------------------------------------------------------
 * spec_accept_sample -- [MATH] 7.1-7.2, [SD] rejection sampling, [TREE]
 * level-by-level tree verification, [SURV] 4.3/8.1 greedy verification.
 *
 * Row u's target logits p_u give the distribution of u's children; row u's
 * draft logits q_u the distribution u's children were drafted from (only
 * rows that have children are read).  At T > 0 the target row of a leaf is
 * read only if the walk ends at that leaf (its bonus draw); no output needs
 * it otherwise.  With T = temperature > 0,
 * P_u = softmax(p_u/T), Q_u = softmax(q_u/T).  For each request, starting at
 * the root: the children c of the current node u are tried in ascending row
 * order; child c (token x = tokens[c], coin r) is accepted iff
 * r * Q_u(x) < R(x), where R starts as P_u and after each rejected sibling
 * becomes max(0, R - Q_u) / sum(max(0, R - Q_u)) (kept, with a flag, when
 * that sum is 0).  An accepted child becomes the new node.  The walk stops
 * at a leaf (emitting one token drawn from P_leaf) or when every child of u
 * is rejected (emitting one token drawn from the current R).  Draws use the
 * inverse CDF in vocabulary order: the smallest t whose cumulative weight
 * exceeds r * (total weight).  T = 0 is greedy: g = argmax p_u (lowest index
 * on ties), move to the lowest-numbered child whose token is g, else emit g.
 *
 * Coins are Philox4x64-10 (Salmon et al., SC'11) with key (seed, 0) and
 * counter (step, b, local row, purpose): purpose 0 = accept coin of draft row
 * c, purpose 1 = draw at the node where the walk stops;
 * r = (word0 >> 11) * 2^-53.
 *
 *   parents_d            int32 [R] local parents (as for the mask)
 *   tokens_d             int32 [R] draft token of each row (roots ignored)
 *   p_logits_d           f32 [R][logits_ld], first `vocab` columns used
 *   q_logits_d           f32 [R][logits_ld] (may be NULL when T == 0)
 *   logits_ld            row stride in elements, >= vocab, multiple of 4;
 *                        both logits pointers 16-byte aligned
 *   path_stride          entries per request in path/tokens outputs, >= 1
 * Outputs (spec_accept_out):
 *   accept_len_d  [B]  a_b = accepted draft tokens
 *   path_d        [B][path_stride]  accepted local rows, root first (a_b + 1
 *                      entries), then -1
 *   tokens_d      [B][path_stride]  the a_b accepted draft tokens followed by
 *                      the final (corrected or bonus) token, then -1
 *   accept_mask_d [R]  1 on rows of the accepted path (root included), else 0 (optional)
 *   child_p_d     [R]  P_parent(c)(token c); NaN at roots (optional).  At T = 0:
 *                      1 if token c is the parent's argmax, else 0.  At T > 0
 *                      NaN on every row of a request whose tree is invalid.
 *   child_q_d     [R]  Q_parent(c)(token c); NaN at roots and on every row of an
 *                      invalid tree; untouched at T = 0 (optional)
 *   flags_d       [B]  SPEC_FLAG_* bits (optional)
 * workspace >= spec_accept_workspace_bytes(batch, vocab) bytes (no init needed).
 *
 * At T > 0 a request's walk may be shared by several workgroups that meet
 * once per vocabulary pass; the library launches only as many as fit on the
 * device together, in the same launch as the vocabulary statistics they
 * read.  If other work holds the compute units so long that a meeting, or
 * a statistics partial the walk needs, does not complete within a bounded
 * wait (about 2^21 polls), that request comes back with accept_len = -1,
 * path and tokens all -1, an empty accept mask and SPEC_FLAG_SYNC_TIMEOUT;
 * every kernel still ends.  Any other request's outputs are complete and
 * exact.
 */
#define SPEC_FLAG_ZERO_RESIDUAL 1   /* a residual had zero mass; R kept unchanged */
#define SPEC_FLAG_PATH_TRUNCATED 2  /* path longer than path_stride; walk cut short */
#define SPEC_FLAG_BAD_TREE 4        /* parent array invalid on the device; accept_len = -1 */
#define SPEC_FLAG_SYNC_TIMEOUT 8    /* walk workgroups did not meet in time; accept_len = -1 */

typedef struct {
  int32_t *accept_len_d;
  int32_t *path_d;
  int32_t *tokens_d;
  uint8_t *accept_mask_d;
  float *child_p_d;
  float *child_q_d;
  int32_t *flags_d;
} spec_accept_out;

size_t spec_accept_workspace_bytes(const spec_batch *batch, int32_t vocab);
spec_status spec_accept_sample(const spec_batch *batch, const int32_t *parents_d,
                               const int32_t *tokens_d, const float *p_logits_d,
                               const float *q_logits_d, int64_t logits_ld, int32_t vocab,
                               float temperature, uint64_t seed, uint64_t step,
                               int32_t path_stride, const spec_accept_out *out,
                               void *workspace_d, size_t workspace_bytes, hipStream_t stream);

/* spec_accept_sample_noalloc -- for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): spec_accept_sample without a workspace argument.  Its
 * scratch is a device array inside the library, SPEC_ACCEPT_SCRATCH_BYTES
 * (8 MiB) per GPU, held by each GPU the library runs on until the process
 * ends; the call allocates nothing.  A batch whose
 * spec_accept_workspace_bytes exceeds that size is refused with
 * SPEC_ERR_WORKSPACE (e.g. 1024 rows over a 128256-entry vocabulary need
 * about 0.5 MiB).  Every call on one GPU shares that GPU's array: calls that
 * overlap on one GPU (two streams, two host threads) race and must be
 * serialised by the caller.  Other arguments, outputs and errors as
 * spec_accept_sample; the outputs are the same bits. */
#define SPEC_ACCEPT_SCRATCH_BYTES (8u << 20)
spec_status spec_accept_sample_noalloc(const spec_batch *batch, const int32_t *parents_d,
                                       const int32_t *tokens_d, const float *p_logits_d,
                                       const float *q_logits_d, int64_t logits_ld,
                                       int32_t vocab, float temperature, uint64_t seed,
                                       uint64_t step, int32_t path_stride,
                                       const spec_accept_out *out, hipStream_t stream);

/* spec_test_exp_f64 -- for tests of the library's double-precision
 * exponential, which every acceptance decision rests on (the probabilities
 * P_u(x) = exp(p_u(x)/T - lse) of [MATH] 7.1 and every residual and draw
 * weight): y_d[i] = f(x_d[i]) for i < n, both f64 device arrays, with
 *   variant 0  exp_f64:          e^x for -708 <= x <= 709, exactly 0 below -708
 *   variant 1  exp_f64_clamped:  e^max(x, -708) (sums of probability mass)
 *   variant 2  exp_f64_stream:   the unguarded core, -745 <= x <= 709
 *   variant 3  exp_f64 evaluated two at a time (elements 2k, 2k+1 together;
 *              a last odd element paired with itself), as the walk's sums do
 *   variant 4  exp_f64_clamped two at a time, as the statistics sums do
 * Variants 3 and 4 must equal 0 and 1 bit for bit.
 * Errors: NULL pointers, n outside 1..2^32, another variant. */
spec_status spec_test_exp_f64(const double *x_d, double *y_d, int64_t n, int32_t variant,
                              hipStream_t stream);

/* spec_accept_sample with the sampling walk's two launch knobs exposed, for
 * tests of its cross-workgroup meetings (the outputs do not depend on them
 * except through SPEC_FLAG_SYNC_TIMEOUT):
 *   max_slices  > 0: at most this many workgroups share one request's walk
 *               (0: as many as fit, up to 32)
 *   max_spins   polls of a meeting's counter before the wait gives up
 *               (-1: the default of spec_accept_sample; 0 gives up at once
 *               unless every workgroup of the request has already arrived)
 * Other arguments, outputs and errors as spec_accept_sample. */
spec_status spec_accept_sample_walk_knobs(const spec_batch *batch, const int32_t *parents_d,
                                          const int32_t *tokens_d, const float *p_logits_d,
                                          const float *q_logits_d, int64_t logits_ld,
                                          int32_t vocab, float temperature, uint64_t seed,
                                          uint64_t step, int32_t path_stride,
                                          const spec_accept_out *out, void *workspace_d,
                                          size_t workspace_bytes, int32_t max_slices,
                                          int32_t max_spins, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * spec_accept_topk -- acceptance when the children are the drafter's top-k
 * choices (deterministic, as in Medusa heads and expansion or EAGLE trees:
 * [SURV] 5.2 and 6.2, [TREE] tree generation).  The pages give no rule for
 * this case; the one taken here treats child c as a draft from the point
 * mass at its token x, so [MATH] 7.1's test and residual become:
 * child c is accepted iff r < R(x), and a rejection removes x from R,
 * where R starts as P_u and is kept normalised (R = P_u on the tokens not
 * yet rejected at u, divided by N = 1 - their P_u mass).  A sibling that
 * repeats a rejected token is never accepted.  When every child of u is
 * rejected, the final token is drawn from R; at a leaf, from P_leaf.  This
 * is sampling from P_u without replacement, so the emitted tokens follow
 * the target distribution exactly; no draft logits are needed.
 *
 * Arguments, outputs, coins (purpose 0 = accept coin of child c, 1 = draw
 * at the stopping node), flags and workspace are those of
 * spec_accept_sample without q_logits_d; child_q_d, when given, is set to
 * NaN.  temperature == 0 is the greedy walk of spec_accept_sample.  A
 * rejection that would leave no mass (N <= 0) keeps R and sets
 * SPEC_FLAG_ZERO_RESIDUAL.
 */
spec_status spec_accept_topk(const spec_batch *batch, const int32_t *parents_d,
                             const int32_t *tokens_d, const float *p_logits_d, int64_t logits_ld,
                             int32_t vocab, float temperature, uint64_t seed, uint64_t step,
                             int32_t path_stride, const spec_accept_out *out, void *workspace_d,
                             size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * spec_lm_head_accept -- the target LM head feeding the acceptance directly.
 * [TREE] tree-mask section (one target forward over the tree gives every
 * node's next-token logits, and verification starts from them) and [SURV]
 * Medusa / EAGLE sections (the model's original LM head maps a position's
 * final feature to vocabulary logits).
 *
 * Target logits of tree row r: z[r][v] = sum_k hidden[r][k] * weight[v][k]
 * (bias-free), bf16 operands, fp32 accumulation.  The statistics the
 * acceptance needs from the target rows (log-sum-exp of z/T, or the argmax
 * at T = 0) are formed from the fp32 results inside the product, so the
 * logits are not read back for them.  Then the walk runs exactly as
 * spec_accept_sample (children = SPEC_CHILDREN_SAMPLED, q_logits_d the
 * drafter's rows) or spec_accept_topk (SPEC_CHILDREN_TOPK, q_logits_d
 * ignored) would on the stored logits; temperature 0 is the greedy walk.
 *
 *   head->hidden_d   bf16 [R][hidden_size] (row stride hidden_size): the
 *                    final feature of every tree row, in row order
 *   head->weight_d   bf16 [vocab][hidden_size]: one row per vocabulary entry
 *   head->hidden_size  a multiple of 64 in 64 .. 65536, with
 *                    vocab * hidden_size and R * hidden_size below 2^31
 *   head->logits_d   fp32 [R][logits_ld] output.  Required at temperature > 0,
 *                    where the first `vocab` entries of the rows of nodes
 *                    that have children are written (the residual passes and
 *                    draws at those nodes read them back) and every other
 *                    row is left untouched: a walk that ends at a leaf finds
 *                    the 256-entry vocabulary tile of its bonus draw from the
 *                    head's partial statistics and recomputes that tile's
 *                    logits alone.  Optional at temperature 0: written in
 *                    full when given, never written when NULL
 *   q_logits_d       as spec_accept_sample (same logits_ld)
 *   workspace >= spec_lm_head_accept_workspace_bytes(batch, vocab) bytes
 *                    (no init needed; 16-byte aligned)
 *
 * Everything else (outputs, coins, flags) is as spec_accept_sample.  Inputs
 * must be finite.  All pointers are device pointers except batch's host
 * arrays; the caller owns every buffer.
 */
#define SPEC_CHILDREN_SAMPLED 0   /* children drafted from q (spec_accept_sample rule) */
#define SPEC_CHILDREN_TOPK 1      /* deterministic children (spec_accept_topk rule) */

typedef struct {
  const void *hidden_d;
  const void *weight_d;
  int32_t hidden_size;
  float *logits_d;
} spec_lm_head;

size_t spec_lm_head_accept_workspace_bytes(const spec_batch *batch, int32_t vocab);
spec_status spec_lm_head_accept(const spec_batch *batch, const int32_t *parents_d,
                                const int32_t *tokens_d, const spec_lm_head *head,
                                const float *q_logits_d, int64_t logits_ld, int32_t vocab,
                                float temperature, int32_t children, uint64_t seed, uint64_t step,
                                int32_t path_stride, const spec_accept_out *out, void *workspace_d,
                                size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * spec_kv_commit -- [SD] KV-cache management: keep accepted tokens' K/V,
 * roll back the rejected ones (paged: free their blocks).
 *
 * For each request: slot L_b + k receives the K/V row at slot L_b + path[k],
 * k = 0 .. a_b (in place, all heads); new_len_d[b] = L_b + a_b + 1.  With
 * paged caches and freed_blocks_d != NULL, row b of freed_blocks_d
 * ([B][max_blocks_per_seq]) lists the physical blocks of logical blocks
 * ceil(new_len/16) .. ceil((L_b + N_b)/16) - 1, then -1.  A request whose
 * accept_len/path are inconsistent (a_b outside [0, N_b), path[0] != 0, or a
 * path entry not strictly increasing / out of range) is left untouched and
 * gets new_len_d[b] = -1.
 */
spec_status spec_kv_commit(const spec_batch *batch, const spec_kv *kv,
                           const int32_t *accept_len_d, const int32_t *path_d,
                           int32_t path_stride, int32_t *new_len_d,
                           int32_t *freed_blocks_d, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Dynamic draft trees -- [TREE] draft-tree generation (EAGLE-2: each round
 * expands only the K most probable bottom-layer leaves, a leaf's
 * probability being the product of the node probabilities on its path) and
 * dynamic draft length (ECHO: one budget of verify rows shared by the batch,
 * checkpoints at fixed depths that cut low-confidence branches, budget that
 * weak requests leave going to confident ones).  These calls build, on the
 * device, the parents/tokens/row_offsets that the verify calls above take.
 *
 * spec_draft_tree holds each request's nodes in creation order (node 0 is
 * the root).  All arrays are device memory owned by the caller:
 *   parent_d, token_d, depth_d  int32 [batch][capacity]
 *   score_d                     f32   [batch][capacity]  product of the path's
 *                               probabilities, each step rounded to f32
 *   count_d                     int32 [batch]  nodes so far
 *   frontier_d                  int32 [batch][topk]  nodes the next round
 *                               expands, -1 padded
 *   flags_d                     int32 [batch]  SPEC_DRAFT_FLAG_* bits
 * Limits: 1 <= topk <= 16, 1 <= capacity <= 4096.
 *
 * spec_draft_begin: every request gets its root (token root_tokens_d[b],
 * score 1) as the only node and the only frontier entry; flags cleared.
 *
 * spec_draft_expand: one round.  cand_tokens_d int32 / cand_probs_d f32
 * [batch][topk][topk]: row i holds the drafter's topk candidates (token,
 * probability) for the request's i-th frontier node (rows past the frontier
 * are ignored).  Each frontier node gets topk children in that order, ids
 * continuing the count; a child's score is f32(score(parent) * p) with p
 * clamped to [0, 1] (NaN -> 0).  The next frontier is the topk
 * highest-scoring new nodes (ties: lower id), skipping, when the new depth
 * equals gate_depth_h[g], nodes scoring below gate_score_h[g]
 * (checkpoints; n_gates <= 8, host arrays).  An empty frontier ends the
 * request's growth.  A round that does not fit in `capacity` appends
 * nothing, ends growth and sets SPEC_DRAFT_FLAG_CAPACITY; a count outside
 * 1..capacity or a frontier entry that is not an existing node (state not
 * made by these calls) ends growth with SPEC_DRAFT_FLAG_BAD_STATE, never a
 * fault.  cand arrays must hold batch * topk * topk entries.
 *
 * spec_draft_select: keeps every root plus the budget_rows - batch
 * highest-scoring non-root nodes of the whole batch (ties: lower request,
 * then lower id), taken among each request's max_rows - 1 best nodes (score
 * descending, id ascending).  A child never outscores its parent and has
 * the larger id, so each request's kept nodes form a tree.  Outputs:
 *   row_offsets_d  int32 [batch + 1]
 *   parents_d, tokens_d, node_of_row_d (optional)  int32 [rows_capacity]:
 *     request b's rows are its root, then its kept nodes in id order
 *     (breadth-first); parents are local rows (-1 at the root);
 *     node_of_row gives each row's node id.
 * Requires budget_rows >= batch, 1 <= max_rows <= min(SPEC_MAX_TREE_ROWS,
 * capacity), batch <= 4096, batch * (max_rows - 1) <= 16384 and
 * rows_capacity >= min(budget_rows, batch * max_rows).  The verify calls
 * need row_offsets on the host too: copy the batch + 1 entries back.
 * workspace >= spec_draft_select_workspace_bytes(batch, max_rows).
 */
#define SPEC_DRAFT_FLAG_CAPACITY 1   /* a round did not fit; growth ended */
#define SPEC_DRAFT_FLAG_BAD_STATE 2  /* count/frontier not made by begin/expand; growth ended */

typedef struct {
  int32_t batch;
  int32_t topk;
  int32_t capacity;
  int32_t *parent_d;
  int32_t *token_d;
  float *score_d;
  int32_t *depth_d;
  int32_t *count_d;
  int32_t *frontier_d;
  int32_t *flags_d;
} spec_draft_tree;

spec_status spec_draft_begin(const spec_draft_tree *tree, const int32_t *root_tokens_d,
                             hipStream_t stream);
spec_status spec_draft_expand(const spec_draft_tree *tree, const int32_t *cand_tokens_d,
                              const float *cand_probs_d, int32_t n_gates,
                              const int32_t *gate_depth_h, const float *gate_score_h,
                              hipStream_t stream);
size_t spec_draft_select_workspace_bytes(int32_t batch, int32_t max_rows);
spec_status spec_draft_select(const spec_draft_tree *tree, int32_t budget_rows, int32_t max_rows,
                              int32_t *row_offsets_d, int32_t *parents_d, int32_t *tokens_d,
                              int32_t *node_of_row_d, int32_t rows_capacity, void *workspace_d,
                              size_t workspace_bytes, hipStream_t stream);

const char *spec_status_string(spec_status status);
const char *spec_last_error(void);
int spec_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* SPEC_VERIFY_H */
