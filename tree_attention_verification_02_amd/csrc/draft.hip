// Dynamic draft trees on the device: EAGLE-2 expansion rounds and an
// ECHO-style global row budget.
//
// Pages: cnblogs "投机推理算法的常见优化手段", draft-tree generation (EAGLE-2
// expands only the K most probable bottom-layer leaves, a leaf's probability
// being the product of the node probabilities on its path) and dynamic draft
// length (ECHO: one budget of verify tokens shared by the batch, checkpoints
// at fixed depths that cut low-confidence branches, budget moving from weak
// to confident requests).
//
// State per request: nodes in creation order (node 0 = root); parent, token,
// float32 score (product of the path's probabilities, accumulated from the
// root), depth; the node count and the frontier (nodes to expand next, -1
// padded).  Kernels:
//  * draft_begin: one thread per request.
//  * draft_expand: one workgroup per request; thread t creates child
//    (t / K, t % K) of the frontier, then ranks the new layer (score
//    descending, id ascending) among the nodes that pass the checkpoint of
//    that depth; ranks below K form the next frontier.
//  * draft_rank: one workgroup per request; each non-root node's rank in its
//    request; the best max_rows - 1 go to a compact list as 64-bit keys
//    (~score bits, slot) whose ascending order is score descending, then
//    request, then id.
//  * draft_threshold: one workgroup for the batch; radix select (8 bits per
//    round, an LDS histogram) of the (budget - B)-th smallest key, then each
//    request's kept count: its kept nodes are a prefix of its sorted list.
//  * draft_emit: one workgroup per request; rows = root then kept nodes in id
//    order, parents remapped, the request's row offset summed from the kept
//    counts before it.
#include "common.hpp"
#include "launch.hpp"

namespace spec {

constexpr int kDraftThreads = 256;
constexpr int kSelThreads = 1024;

SPEC_DEVICE float clamp_prob(float p) {
  return (p >= 0.0f) ? fminf(p, 1.0f) : 0.0f;     // NaN and negatives -> 0
}

__global__ void __launch_bounds__(256)
draft_begin_kernel(DraftTree t, const int32_t* __restrict__ root_tokens) {
  const int b = blockIdx.x * 256 + threadIdx.x;
  if (b >= t.batch) return;
  const int64_t base = (int64_t)b * t.capacity;
  t.parent[base] = -1;
  t.token[base] = root_tokens[b];
  t.score[base] = 1.0f;
  t.depth[base] = 0;
  t.count[b] = 1;
  t.flags[b] = 0;
  for (int i = 0; i < t.topk; ++i) t.frontier[(int64_t)b * t.topk + i] = (i == 0) ? 0 : -1;
}

__global__ void __launch_bounds__(kDraftThreads)
draft_expand_kernel(DraftTree t, const int32_t* __restrict__ cand_tokens,
                    const float* __restrict__ cand_probs, DraftGates g) {
  __shared__ int fr[kDraftMaxK];
  __shared__ float s_new[kDraftMaxK * kDraftMaxK];
  __shared__ int s_ok[kDraftMaxK * kDraftMaxK];
  __shared__ int n_ok;
  const int b = blockIdx.x;
  const int K = t.topk;
  const int tid = threadIdx.x;
  const int64_t base = (int64_t)b * t.capacity;
  const int c = t.count[b];
  if (tid < K) fr[tid] = t.frontier[(int64_t)b * K + tid];
  if (tid == 0) n_ok = 0;
  __syncthreads();
  int nf = 0;
  bool bad = c < 1 || c > t.capacity;            // state not made by begin/expand
  for (int i = 0; i < K; ++i) {
    nf += (fr[i] >= 0);
    bad |= fr[i] >= c || (fr[i] >= 0 && i > 0 && fr[i - 1] < 0);
  }
  if (bad) {
    if (tid < K) t.frontier[(int64_t)b * K + tid] = -1;
    if (tid == 0) t.flags[b] |= kDraftFlagBadState;
    return;
  }
  if (nf == 0) return;
  const int n_new = nf * K;
  if (c + n_new > t.capacity) {                  // capacity: no append, growth ends
    if (tid < K) t.frontier[(int64_t)b * K + tid] = -1;
    if (tid == 0) t.flags[b] |= kDraftFlagCapacity;
    return;
  }
  const int d = t.depth[base + fr[0]] + 1;       // the frontier is one layer
  if (tid < n_new) {
    const int i = tid / K, j = tid % K;
    const int u = fr[i];
    const int64_t ci = ((int64_t)b * K + i) * K + j;
    const float s = t.score[base + u] * clamp_prob(cand_probs[ci]);
    const int v = c + tid;
    t.parent[base + v] = u;
    t.token[base + v] = cand_tokens[ci];
    t.score[base + v] = s;
    t.depth[base + v] = d;
    int ok = 1;
    for (int k = 0; k < g.n; ++k)
      if (g.depth[k] == d && !(s >= g.score[k])) ok = 0;
    s_new[tid] = s;
    s_ok[tid] = ok;
    if (ok) atomicAdd(&n_ok, 1);
  }
  __syncthreads();
  if (tid < n_new && s_ok[tid]) {
    const float s = s_new[tid];
    int r = 0;
    for (int w = 0; w < n_new; ++w)
      r += s_ok[w] && (s_new[w] > s || (s_new[w] == s && w < tid));
    if (r < K) t.frontier[(int64_t)b * K + r] = c + tid;
  }
  if (tid < K && tid >= n_ok) t.frontier[(int64_t)b * K + tid] = -1;
  if (tid == 0) t.count[b] = c + n_new;
}

// Compact candidate lists: key = (~score bits) << 32 | (b * capacity + v),
// ascending = score descending, then request, then id (scores are >= 0, so
// their bit patterns are ordered like their values).
struct SelectWs {
  uint64_t* cand;    // [B][max_rows - 1]
  int32_t* n_el;     // [B]
  int32_t* kept;     // [B]
};

__host__ __device__ inline size_t align256d(size_t x) { return (x + 255) & ~(size_t)255; }

__host__ __device__ inline SelectWs select_ws(void* p, int B, int max_rows) {
  char* c = (char*)p;
  SelectWs w;
  w.cand = (uint64_t*)c;
  c += align256d((size_t)B * (max_rows > 1 ? max_rows - 1 : 1) * sizeof(uint64_t));
  w.n_el = (int32_t*)c;
  c += align256d((size_t)B * sizeof(int32_t));
  w.kept = (int32_t*)c;
  return w;
}

size_t draft_select_workspace_bytes(int B, int max_rows) {
  return align256d((size_t)B * (max_rows > 1 ? max_rows - 1 : 1) * sizeof(uint64_t)) +
         2 * align256d((size_t)B * sizeof(int32_t));
}

SPEC_DEVICE uint64_t draft_key(float s, int64_t slot) {
  return ((uint64_t)(~__float_as_uint(s)) << 32) | (uint64_t)(uint32_t)slot;
}

__global__ void __launch_bounds__(kDraftThreads)
draft_rank_kernel(DraftTree t, int max_rows, SelectWs ws) {
  __shared__ float sc[kDraftMaxNodes];
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t base = (int64_t)b * t.capacity;
  const int n = min(max(t.count[b], 1), t.capacity);
  const int lim = max_rows - 1;
  for (int v = tid; v < n; v += kDraftThreads) sc[v] = t.score[base + v];
  if (tid == 0) ws.n_el[b] = min(n - 1, lim);
  __syncthreads();
  for (int v = 1 + tid; v < n; v += kDraftThreads) {
    const float s = sc[v];
    int r = 0;
    for (int w = 1; w < n; ++w) r += (sc[w] > s) || (sc[w] == s && w < v);
    if (r < lim) ws.cand[(int64_t)b * lim + r] = draft_key(s, base + v);
  }
}

// One workgroup: the (take + 1)-th smallest key over all compact lists
// (radix select, 8 bits per round: an LDS histogram, then one wave scans
// the 256 bins), then kept[b] = how many of list b's keys are below it.
// Keys are unique, so exactly `take` keys are kept; once the current digit
// holds a single key, that key is the answer and the rounds stop.
__global__ void __launch_bounds__(kSelThreads)
draft_threshold_kernel(int B, int max_rows, int take, SelectWs ws) {
  __shared__ int hist[256];
  __shared__ int s_digit, s_need, s_count, s_total;
  __shared__ uint64_t s_kth;
  __shared__ int s_kept[kDraftSelMaxB];
  const int tid = threadIdx.x, lane = tid & 63;
  const int lim = max_rows - 1;
  const int slots = B * lim;
  if (tid == 0) s_total = 0;
  for (int i = tid; i < B; i += kSelThreads) s_kept[i] = 0;
  uint64_t key[kDraftSelPer];
#pragma unroll
  for (int k = 0; k < kDraftSelPer; ++k) {
    const int f = tid + k * kSelThreads;
    key[k] = ~0ull;                              // empty slot: never selected
    if (f < slots) {
      const int bb = f / lim, r = f - bb * lim;
      const uint64_t c = ws.cand[f];             // in bounds; used only when r < n_el
      if (r < ws.n_el[bb]) key[k] = c;
    }
  }
  int nv = 0;
#pragma unroll
  for (int k = 0; k < kDraftSelPer; ++k) nv += key[k] != ~0ull;
  nv = wave_sum(nv);
  __syncthreads();                               // s_total cleared
  if (lane == 0) atomicAdd(&s_total, nv);
  __syncthreads();
  const int total = s_total;
  uint64_t kth = ~0ull;                          // keep all
  if (take < total) {
    uint64_t prefix = 0;
    if (tid == 0) s_need = take + 1;             // 1-based rank of the first key not kept
    for (int shift = 56; shift >= 0; shift -= 8) {
      for (int i = tid; i < 256; i += kSelThreads) hist[i] = 0;
      __syncthreads();
      const uint64_t hi_mask = (shift == 56) ? 0ull : (~0ull << (shift + 8));
#pragma unroll
      for (int k = 0; k < kDraftSelPer; ++k)
        if (key[k] != ~0ull && ((key[k] ^ prefix) & hi_mask) == 0)
          atomicAdd(&hist[(int)((key[k] >> shift) & 255)], 1);
      __syncthreads();
      if (tid < 64) {
        const int h0 = hist[4 * lane], h1 = hist[4 * lane + 1];
        const int h2 = hist[4 * lane + 2], h3 = hist[4 * lane + 3];
        const int sum = h0 + h1 + h2 + h3;
        int incl = sum;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const int x = __shfl_up(incl, o, 64);
          if (lane >= o) incl += x;
        }
        const int excl = incl - sum;
        const int need = s_need;
        if (excl < need && need <= incl) {       // exactly one lane
          int n2 = need - excl, d = 4 * lane, hs = h0;
          if (n2 > h0) {
            n2 -= h0; ++d; hs = h1;
            if (n2 > h1) {
              n2 -= h1; ++d; hs = h2;
              if (n2 > h2) { n2 -= h2; ++d; hs = h3; }
            }
          }
          s_digit = d;
          s_need = n2;
          s_count = hs;
        }
      }
      __syncthreads();
      prefix |= (uint64_t)s_digit << shift;
      if (s_count == 1) {                        // one key left under this prefix
        const uint64_t m = ~0ull << shift;
#pragma unroll
        for (int k = 0; k < kDraftSelPer; ++k)
          if (key[k] != ~0ull && ((key[k] ^ prefix) & m) == 0) s_kth = key[k];
        __syncthreads();
        prefix = s_kth;
        break;
      }
    }
    kth = prefix;                                // the (take + 1)-th smallest key
  }
#pragma unroll
  for (int k = 0; k < kDraftSelPer; ++k) {
    const int f = tid + k * kSelThreads;
    if (key[k] != ~0ull && (take >= total || key[k] < kth)) atomicAdd(&s_kept[f / lim], 1);
  }
  __syncthreads();
  for (int i = tid; i < B; i += kSelThreads) ws.kept[i] = s_kept[i];
}

__global__ void __launch_bounds__(kDraftThreads)
draft_emit_kernel(DraftTree t, int max_rows, SelectWs ws, int32_t* __restrict__ row_offsets,
                  int32_t* __restrict__ parents, int32_t* __restrict__ tokens,
                  int32_t* __restrict__ node_of_row) {
  __shared__ int row_of[kDraftMaxNodes];
  __shared__ int nodes[kMaxRows];
  __shared__ int part[kDraftThreads / kWave];
  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lim = max_rows - 1;
  const int64_t base = (int64_t)b * t.capacity;
  const int k = ws.kept[b];
  // row offset: requests before b hold 1 + kept rows each
  int acc = 0;
  for (int i = tid; i < b; i += kDraftThreads) acc += 1 + ws.kept[i];
  acc = wave_sum(acc);
  if (lane == 0) part[wave] = acc;
  const int n = min(max(t.count[b], 1), t.capacity);
  for (int v = tid; v < n; v += kDraftThreads) row_of[v] = -1;
  for (int i = tid; i < k; i += kDraftThreads)
    nodes[i] = (int)((uint32_t)ws.cand[(int64_t)b * lim + i] - (uint32_t)base);
  __syncthreads();
  int o = 0;
  for (int w = 0; w < kDraftThreads / kWave; ++w) o += part[w];
  if (tid == 0) row_of[0] = 0;
  for (int i = tid; i < k; i += kDraftThreads) {
    const int v = nodes[i];
    int r = 1;
    for (int j = 0; j < k; ++j) r += nodes[j] < v;
    row_of[v] = r;
  }
  __syncthreads();
  for (int i = tid; i <= k; i += kDraftThreads) {
    // row i holds the node whose row_of is i: the root, or nodes[j] with rank i
    int v = 0;
    if (i > 0)
      for (int j = 0; j < k; ++j)
        if (row_of[nodes[j]] == i) v = nodes[j];
    int pr = -1;
    if (v > 0) pr = row_of[t.parent[base + v]];
    parents[o + i] = pr;
    tokens[o + i] = t.token[base + v];
    if (node_of_row) node_of_row[o + i] = v;
  }
  if (tid == 0) {
    row_offsets[b] = o;
    if (b == gridDim.x - 1) row_offsets[b + 1] = o + 1 + k;
  }
}

hipError_t launch_draft_begin(const DraftTree& t, const int32_t* root_tokens, hipStream_t stream) {
  hipLaunchKernelGGL(draft_begin_kernel, dim3((t.batch + 255) / 256), dim3(256), 0, stream, t,
                     root_tokens);
  return hipGetLastError();
}

hipError_t launch_draft_expand(const DraftTree& t, const int32_t* cand_tokens,
                               const float* cand_probs, const DraftGates& g, hipStream_t stream) {
  hipLaunchKernelGGL(draft_expand_kernel, dim3(t.batch), dim3(kDraftThreads), 0, stream, t,
                     cand_tokens, cand_probs, g);
  return hipGetLastError();
}

hipError_t launch_draft_select(const DraftTree& t, int budget_rows, int max_rows,
                               int32_t* row_offsets, int32_t* parents, int32_t* tokens,
                               int32_t* node_of_row, void* workspace, hipStream_t stream) {
  SelectWs ws = select_ws(workspace, t.batch, max_rows);
  hipLaunchKernelGGL(draft_rank_kernel, dim3(t.batch), dim3(kDraftThreads), 0, stream, t, max_rows,
                     ws);
  hipLaunchKernelGGL(draft_threshold_kernel, dim3(1), dim3(kSelThreads), 0, stream, t.batch,
                     max_rows, budget_rows - t.batch, ws);
  hipLaunchKernelGGL(draft_emit_kernel, dim3(t.batch), dim3(kDraftThreads), 0, stream, t, max_rows,
                     ws, row_offsets, parents, tokens, node_of_row);
  return hipGetLastError();
}

}  // namespace spec
