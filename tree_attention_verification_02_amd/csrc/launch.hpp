// Host-side launchers of the verify-step kernels (called by the C ABI layer
// after it has validated every argument).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace spec {

struct LaunchCtx {
  int B;
  const int32_t* row_offsets_d;
  const int32_t* prefix_len_d;
  hipStream_t stream;
};

// Longest-first dispatch covers batches of up to this many requests (their
// order travels in the kernel arguments).
constexpr int kLptMax = 512;
// Longest request (prefix + tree) the bf16 attention plans for: splits of at
// most 8192 keys, at most 1024 splits per request.
constexpr int64_t kMaxAttnKeys = 8192LL * 1024;

// Split-KV plan of the bf16 tree-attention kernel: every (request, KV head,
// row block, key split) is one workgroup.  With `lpt`, workgroups come in two
// phases: first every split but the last of each request (all of full
// length), then the last split of each request, requests ordered by that
// split's length, longest first (`order`), so that the hardware dispatcher's
// in-order list scheduling ends on the short pieces.
struct AttnPlan {
  int rows_per_block;   // query rows (tree rows x group heads) per workgroup
  int split_keys;       // keys per split (multiple of the key tile)
  int64_t items;        // total workgroups
  int64_t partial_items;// workgroups whose request needs more than one split
  int64_t units;        // (request, KV head, row block) triples
  int max_ns;           // most splits of any request
  int lpt;              // two-phase order in use
  int weighted;         // heavy units get 2/3-length splits (mixed-length batches)
  int64_t items_a;      // workgroups of the first phase
  uint16_t order[kLptMax];  // second phase: requests, longest last split first
  // Combine grid: `comb_chunks` workgroups (32 rows each) per unit, enough
  // for the largest unit.  With comb_nreq > 0 (every request one row block,
  // batches of up to kLptMax), only the units of the requests listed in
  // comb_req (those with more than one split) get workgroups.
  int comb_chunks;
  int comb_nreq;
  uint16_t comb_req[kLptMax];
};

hipError_t launch_build_mask(const LaunchCtx& cx, const int32_t* parents, uint64_t* mask, int words,
                             int32_t* depth, int32_t* pos, int32_t* err_row);
hipError_t launch_kv_append(const LaunchCtx& cx, int R, const KvAddr& addr, int esize,
                            const void* k_new, const void* v_new, void* k_cache, void* v_cache);
hipError_t launch_kv_commit(const LaunchCtx& cx, const KvAddr& addr, int esize,
                            const int32_t* accept_len, const int32_t* path, int path_stride,
                            void* k_cache, void* v_cache, int32_t* new_len, int32_t* freed);

// Attention.
AttnPlan plan_attention(int B, const int32_t* row_offsets_h, const int32_t* prefix_len_h, int hq,
                        int hkv);
size_t attention_workspace_bytes(const AttnPlan& plan, int d);
hipError_t launch_attention_bf16(const LaunchCtx& cx, const AttnPlan& plan, const KvAddr& addr,
                                 int hq, const void* q, const uint64_t* mask, int words,
                                 float scale, const void* k_cache, const void* v_cache, void* out,
                                 int out_f32, void* workspace);
hipError_t launch_attention_f32(const LaunchCtx& cx, int R, const KvAddr& addr, int hq,
                                const float* q, const uint64_t* mask, int words, float scale,
                                const float* k_cache, const float* v_cache, void* out, int out_f32);

// Target LM head: logits = hidden . weight^T (bf16 in, fp32 out) with, per
// (tree row, kHeadTileV-entry vocabulary tile), the partial statistics of the
// acceptance: (reference, sum) at temperature > 0, (max, first argmax) at 0.
constexpr int kHeadTileV = 256;   // vocabulary entries per tile
constexpr int kHeadTileR = 256;   // tree rows per workgroup
struct HeadTiles {
  int ntile;      // vocabulary tiles per row
  double* ref;    // [R][ntile]  temperature > 0
  double* s;
  float* m;       // [R][ntile]  temperature 0 (aliases ref / s)
  int32_t* am;
  uint8_t* kids;  // [R] 1 where the row has children: at T > 0 only those logits are stored
  double* leafz;  // [B][kHeadTileV] a leaf's tile logits as the walk recomputes them (tagged)
  const uint16_t* hidden;   // the head's operands, for that recomputation
  const uint16_t* weight;
  int H;
};
int head_vocab_tiles(int vocab);
size_t head_tiles_bytes(int R, int vocab);
HeadTiles head_tiles(void* base, int R, int vocab);
hipError_t launch_lm_head(int R, const uint16_t* hidden, int H, const uint16_t* weight, int vocab,
                          float temperature, float* logits, int64_t ld, const HeadTiles& tiles,
                          int B, const int32_t* row_offsets, const int32_t* parents,
                          hipStream_t stream);

// Acceptance.  At temperature > 0, q_logits == nullptr selects deterministic
// children (each child a point-mass draft; no draft rows are read).  With
// `head`, the target rows' statistics come from the LM head's tile partials
// (merged here) instead of a pass over p_logits; p_logits may then be null at
// temperature 0.  `walk` caps the sampling walk's workgroups per request
// (max_slices > 0) and the polls of its barrier wait (max_spins >= 0); the
// defaults are as many slices as fit and kWalkMaxSpins.
struct WalkKnobs {
  int max_slices = 0;
  int max_spins = -1;
};
size_t accept_workspace_bytes(int R, int B, int vocab);
hipError_t launch_exp64_probe(const double* x, double* y, int64_t n, int variant,
                              hipStream_t stream);
// The no-allocation entry point's workspace: a device array of this many
// bytes in accept.hip, its address on the current device.
constexpr size_t kAcceptScratchBytes = (size_t)8 << 20;
hipError_t accept_scratch(void** ptr);
hipError_t launch_accept(const LaunchCtx& cx, int R, const int32_t* parents, const int32_t* tokens,
                         const float* p_logits, const float* q_logits, int64_t ld, int vocab,
                         float temperature, uint64_t seed, uint64_t step, int path_stride,
                         int32_t* accept_len, int32_t* path, int32_t* tokens_out,
                         uint8_t* accept_mask, float* child_p, float* child_q, int32_t* flags,
                         void* workspace, WalkKnobs walk = WalkKnobs(),
                         const HeadTiles* head = nullptr);

// Dynamic draft trees (EAGLE-2 rounds, global row budget).
constexpr int kDraftMaxK = 16;          // children per expanded node, nodes expanded per round
constexpr int kDraftMaxNodes = 4096;    // nodes per request (capacity), root included
constexpr int kDraftMaxGates = 8;       // checkpoints
constexpr int kDraftSelPer = 16;        // compact candidates per selection thread
constexpr int kDraftSelMax = 1024 * kDraftSelPer;   // B * (max_rows - 1) limit
constexpr int kDraftSelMaxB = 4096;     // requests per selection
constexpr int kDraftFlagCapacity = 1;
constexpr int kDraftFlagBadState = 2;

struct DraftTree {
  int batch, topk, capacity;
  int32_t* parent;    // [batch][capacity]
  int32_t* token;
  float* score;
  int32_t* depth;
  int32_t* count;     // [batch]
  int32_t* frontier;  // [batch][topk]
  int32_t* flags;     // [batch]
};

struct DraftGates {
  int n;
  int depth[kDraftMaxGates];
  float score[kDraftMaxGates];
};

hipError_t launch_draft_begin(const DraftTree& t, const int32_t* root_tokens, hipStream_t stream);
hipError_t launch_draft_expand(const DraftTree& t, const int32_t* cand_tokens,
                               const float* cand_probs, const DraftGates& g, hipStream_t stream);
size_t draft_select_workspace_bytes(int B, int max_rows);
hipError_t launch_draft_select(const DraftTree& t, int budget_rows, int max_rows,
                               int32_t* row_offsets, int32_t* parents, int32_t* tokens,
                               int32_t* node_of_row, void* workspace, hipStream_t stream);

}  // namespace spec
