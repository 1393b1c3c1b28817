// Lossless speculative acceptance over a draft tree.
//
// Pages: CSDN "推理加速：推测解码与级联推理" sections 7.1-7.2 (accept with
// probability min(1, p/q); on rejection draw from norm(max(0, p - q)); the
// emitted length counts the final token); guijiagi.com speculative-decoding
// post, rejection-sampling section (the first rejection ends the step);
// cnblogs "投机推理算法的常见优化手段", tree-mask section (row i's target
// distribution predicts i's children; every level of the tree is checked).
//
// Residuals in closed form.  With P and Q fixed at a node, the residual after
// any number of rejected siblings is R = max(0, P - t Q) / N for a scalar t:
// starting from (t, N) = (0, 1), a rejection moves to t' = t + N and
// N' = G(t') with G(t) = sum_y max(0, P_y - t Q_y) (and keeps (t, N) when
// G(t') = 0).  So every rejection costs one vocabulary pass at a scalar t,
// and the final draw after the last rejection reuses that pass's sums.  A
// draw from P alone (at a leaf) needs no full pass: the statistics partials
// give each chunk's mass, and only the drawn chunk is passed over.
//
// Kernels:
//  * accept_prep (T > 0): lists the rows whose statistics are read -- the
//    target and draft rows of nodes with children (no output needs a leaf's
//    statistics; a walk that ends at a leaf makes its own pass over the
//    leaf's target row) -- and clears the walk's exchange area and the
//    statistics partials.
//  * accept_sample (T > 0), one launch in two parts.  First one workgroup per
//    listed (row, 16K-logit chunk) item streams its chunk once (16-byte
//    loads) into fp64 partial sums, published with a tag.  After them come
//    S workgroups ("slices", taken by ticket in start order) per request,
//    dispatched as the statistics drain: each loads its tree, merges its
//    request's partials (polling each until it shows its tag) into the rows'
//    log-sum-exps of logits/T and the child probabilities P_u(x_c), Q_u(x_c).
//    Each pass is split over the S slices by 1024-element segments; segment
//    sums go to global memory carrying their pass tag, and every slice reads
//    all of them (bounded polls), sums them in the same order and replays
//    the same scalar decisions, so no further broadcast is needed; slice 0
//    rescans the drawn segment and writes the outputs.  With the LM head's
//    partials, a leaf's logits were never stored: its bonus draw finds the
//    256-entry tile from the head's tile partials and the slices recompute
//    that tile's logits from the hidden row and the weight rows.
//  * accept_argmax (T = 0): the first argmax of every target-row chunk;
//    accept_finalize merges them per row.
//  * accept_greedy: temperature 0, one workgroup per request.
//
// Deterministic children (no draft rows): each child is a draft from the
// point mass at its token, so a rejection removes that token from the
// residual: R = P restricted to the tokens not yet rejected, divided by
// N = 1 - (their P mass).  The sibling tests then need no vocabulary pass;
// the one pass left is the final draw (P without the rejected tokens, or
// P_leaf).  The emitted token follows P exactly (sampling without
// replacement).
//
// Every quantity that decides an integer (accept tests, residual masses,
// inverse-CDF boundaries) is evaluated in fp64, with a table-driven fp64
// exponential, so decisions agree with a float64 reference except within
// ~1e-11 of a threshold.
#include <math.h>

#include <algorithm>
#include <atomic>
#include <mutex>

#include "common.hpp"
#include "exp64.hpp"
#include "launch.hpp"
#include "philox.hpp"

namespace spec {

constexpr int kStatThreads = 256;
constexpr int kStatF4 = 16;                   // float4 per thread per statistics chunk
constexpr int kStatChunkLen = kStatThreads * kStatF4 * 4;   // logits per chunk
constexpr int kWalkThreads = 256;
constexpr int kWalkWaves = kWalkThreads / 64;
constexpr int kSeg = kWalkThreads * 4;        // elements per segment (one float4 per thread)
constexpr int kPassF = 8;                     // segments per pass round (float4 in flight per row)
constexpr int kPassChunk = 64;                // segments per partial-sum flush
constexpr int kMaxSlices = 32;                // more pollers per counter cost more than they save
constexpr int kMaxDevices = 64;
constexpr int kWalkMaxSpins = 1 << 21;       // barrier polls before a walk gives up
constexpr int kMaxSegs = (kMaxVocab + kSeg - 1) / kSeg;
constexpr int kSumLoads = 2;                  // segment sums per lane whose loads go out together

// ---------------------------------------------------------------------------
// Workspace.
struct AcceptWs {
  int32_t* am;      // [R]   first argmax of the target row (greedy)
  int nch;          // statistics chunks per row
  double* part_ref; // [2][R][nch] chunk partials: reference
  double* part_s;   //                     and sum of exp(z - reference)
  float* part_m;    // [R][nch]    chunk max (greedy)
  int32_t* part_am; //                     and its first index
  int32_t* order;   // [2R] rows whose statistics are streamed: [0, R) draft rows (R + r),
                    // [R, 2R) target rows (r), each list in row order
  int32_t* sync;    // [64], own 256 B: [0] the walk's ticket counter, [2] draft rows
                    // listed, [3] target rows listed
  double* seg;      // [B][2][nseg] per-pass segment sums carrying their pass tag
                    // (double-buffered by pass parity; zeroed before every walk)
  double* sref;     // [B][2][kMaxSlices] per-slice references of a leaf's pass (tagged
                    // like the sums, same parity buffers; zeroed before every walk)
};

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

__host__ __device__ inline int stat_chunks(int vocab) {
  return (vocab + kStatChunkLen - 1) / kStatChunkLen;
}

__host__ __device__ inline AcceptWs accept_ws(void* base, int R, int B, int vocab) {
  const int nch = stat_chunks(vocab);
  char* p = (char*)base;
  AcceptWs w;
  w.nch = nch;
  w.am = (int32_t*)p;
  p += align256((size_t)R * sizeof(int32_t));
  w.part_ref = (double*)p;
  p += align256(2 * (size_t)R * nch * sizeof(double));
  w.part_s = (double*)p;
  p += align256(2 * (size_t)R * nch * sizeof(double));
  w.part_m = (float*)p;
  p += align256((size_t)R * nch * sizeof(float));
  w.part_am = (int32_t*)p;
  p += align256((size_t)R * nch * sizeof(int32_t));
  w.order = (int32_t*)p;
  p += align256(2 * (size_t)R * sizeof(int32_t));
  w.sync = (int32_t*)p;
  p += 256;
  w.seg = (double*)p;
  p += align256((size_t)B * 2 * ((vocab + kSeg - 1) / kSeg) * sizeof(double));
  w.sref = (double*)p;
  return w;
}

static int segs_for(int vocab) { return (vocab + kSeg - 1) / kSeg; }

size_t accept_workspace_bytes(int R, int B, int vocab) {
  const int nseg = segs_for(vocab);
  const int nch = stat_chunks(vocab);
  // the layout of accept_ws, field by field
  return align256((size_t)R * sizeof(int32_t)) +
         2 * align256(2 * (size_t)R * nch * sizeof(double)) +
         align256((size_t)R * nch * sizeof(float)) +
         align256((size_t)R * nch * sizeof(int32_t)) +
         align256(2 * (size_t)R * sizeof(int32_t)) +
         256 +
         align256((size_t)B * 2 * nseg * sizeof(double)) +
         align256((size_t)B * 2 * kMaxSlices * sizeof(double));
}

// Before the statistics at T > 0 (accept_prep_kernel): blocks 1.. clear the
// walk's exchange area (every segment sum to tag 0, which no pass uses) and
// the statistics partials (tag 0: not yet written); block 0 resets the
// walk's ticket counter and lists the rows whose statistics are streamed:
// the draft rows (order[0, R)) and the target rows (order[R, 2R)) of the
// nodes that have children (no target rows when the LM head has produced
// their partials).  The children marks live in LDS; beyond its tables every
// row is listed.
constexpr int kPrepThreads = 1024;
constexpr int kPrepMaxRows = 16384;
constexpr int kPrepMaxBatch = 4096;

SPEC_DEVICE int find_request(const int* off, int B, int r) {   // off[b] <= r < off[b + 1]
  int lo = 0, hi = B;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (off[mid] <= r) lo = mid; else hi = mid;
  }
  return lo;
}

__global__ void __launch_bounds__(kPrepThreads)
accept_prep_kernel(const int32_t* __restrict__ row_offsets, int B, int R,
                   const int32_t* __restrict__ parents, AcceptWs ws, int vocab, int list_p,
                   int list_q, int wfirst) {
  __shared__ int s_off[kPrepMaxBatch + 1];
  __shared__ unsigned char s_kids[kPrepMaxRows];
  __shared__ int s_wave[kPrepThreads / 64];
  __shared__ int s_key[kMaxRows + 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (blockIdx.x > 0) {
    const int64_t nseg_all = (int64_t)B * 2 * ((vocab + kSeg - 1) / kSeg);
    const int64_t nsref = (int64_t)B * 2 * kMaxSlices;
    const int64_t nslot = 2 * (int64_t)R * ws.nch;
    const int64_t stride = (int64_t)(gridDim.x - 1) * kPrepThreads;
    for (int64_t i = (int64_t)(blockIdx.x - 1) * kPrepThreads + tid; i < nseg_all; i += stride)
      ws.seg[i] = 0.0;
    for (int64_t i = (int64_t)(blockIdx.x - 1) * kPrepThreads + tid; i < nsref; i += stride)
      ws.sref[i] = 0.0;
    for (int64_t i = (int64_t)(blockIdx.x - 1) * kPrepThreads + tid; i < nslot; i += stride) {
      ws.part_ref[i] = 0.0;
      ws.part_s[i] = 0.0;
    }
    return;
  }
  const int m = (list_q ? 1 : 0) + (list_p ? 1 : 0);   // entries per listed node (walks first)
  if (!list_p && !list_q) {
    if (tid == 0) ws.sync[2] = ws.sync[3] = 0;
  } else if (wfirst && (R > kPrepMaxRows || B > kPrepMaxBatch)) {
    for (int r = tid; r < R; r += kPrepThreads) {
      int j = 0;
      if (list_q) ws.order[m * r + j++] = R + r;
      if (list_p) ws.order[m * r + j] = r;
    }
    if (tid == 0) ws.sync[2] = m * R;
  } else if (wfirst) {
    // Walks first: one list, the draft then the target row of each node that
    // has children, nodes ordered by their index inside their request (all
    // roots, then every request's row 1, ...).  Rows are in tree order (a
    // parent before its children), so the statistics a walk needs next
    // arrive about when it gets there.  A counting sort over the 256 local
    // indices; the order inside one index is immaterial.
    for (int i = tid; i <= B; i += kPrepThreads) s_off[i] = row_offsets[i];
    for (int r = tid; r < R; r += kPrepThreads) s_kids[r] = 0;
    for (int i = tid; i <= kMaxRows; i += kPrepThreads) s_key[i] = 0;
    __syncthreads();
    for (int r = tid; r < R; r += kPrepThreads) {
      const int b = find_request(s_off, B, r);
      const int u = r - s_off[b], pu = parents[r];
      if (u > 0 && pu >= 0 && pu < u) s_kids[s_off[b] + pu] = 1;
    }
    __syncthreads();
    for (int r = tid; r < R; r += kPrepThreads)
      if (s_kids[r]) atomicAdd(&s_key[r - s_off[find_request(s_off, B, r)] + 1], 1);
    __syncthreads();
    // exclusive prefix over the 256 indices: s_key[i] = nodes at indices < i
    int cnt = (tid < kMaxRows) ? s_key[tid + 1] : 0;
    int incl = cnt;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int x = __shfl_up(incl, d, 64);
      if (lane >= d) incl += x;
    }
    if (lane == 63) s_wave[wave] = incl;
    __syncthreads();
    for (int w = 0; w < wave; ++w) incl += s_wave[w];
    if (tid < kMaxRows) s_key[tid + 1] = incl;
    if (tid == kMaxRows - 1) ws.sync[2] = m * incl;
    __syncthreads();
    for (int r = tid; r < R; r += kPrepThreads)
      if (s_kids[r]) {
        const int pos = atomicAdd(&s_key[r - s_off[find_request(s_off, B, r)]], 1);
        int j = 0;
        if (list_q) ws.order[m * pos + j++] = R + r;
        if (list_p) ws.order[m * pos + j] = r;
      }
  } else if (R > kPrepMaxRows || B > kPrepMaxBatch) {
    for (int r = tid; r < R; r += kPrepThreads) {
      ws.order[r] = R + r;
      ws.order[R + r] = r;
    }
    if (tid == 0) {
      ws.sync[2] = list_q ? R : 0;
      ws.sync[3] = list_p ? R : 0;
    }
  } else {
    for (int i = tid; i <= B; i += kPrepThreads) s_off[i] = row_offsets[i];
    for (int r = tid; r < R; r += kPrepThreads) s_kids[r] = 0;
    __syncthreads();
    for (int r = tid; r < R; r += kPrepThreads) {        // mark every node that has a child
      const int b = find_request(s_off, B, r);
      const int u = r - s_off[b], pu = parents[r];
      if (u > 0 && pu >= 0 && pu < u) s_kids[s_off[b] + pu] = 1;
    }
    __syncthreads();
    // thread t lists the marked rows of [t * per, (t + 1) * per) after those
    // of the threads before it (block-wide exclusive prefix of the counts)
    const int per = (R + kPrepThreads - 1) / kPrepThreads;
    const int r0 = min(R, tid * per), r1 = min(R, r0 + per);
    int cnt = 0;
    for (int r = r0; r < r1; ++r) cnt += s_kids[r];
    int incl = cnt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int x = __shfl_up(incl, o, 64);
      if (lane >= o) incl += x;
    }
    if (lane == 63) s_wave[wave] = incl;
    __syncthreads();
    int base = 0, total = 0;
    for (int w = 0; w < kPrepThreads / 64; ++w) {
      if (w < wave) base += s_wave[w];
      total += s_wave[w];
    }
    int pos = base + incl - cnt;
    for (int r = r0; r < r1; ++r)
      if (s_kids[r]) {
        ws.order[pos] = R + r;
        ws.order[R + pos] = r;
        ++pos;
      }
    if (tid == 0) {
      ws.sync[2] = list_q ? total : 0;
      ws.sync[3] = list_p ? total : 0;
    }
  }
  if (tid == 0) ws.sync[0] = 0;
}

// ---------------------------------------------------------------------------
// Statistics.

// Greedy statistics: (max, first argmax) of one target-row chunk per
// workgroup.  A chunk is kStatF4 float4 per thread (16K logits), held in
// registers: rows are cut into ws.nch = ceil(V / 16K) chunks so that rows of
// 128K logits spread over the CUs, and every load of a chunk is in flight at
// once.
__global__ void __launch_bounds__(kStatThreads)
accept_argmax_kernel(const float* __restrict__ p_logits, int64_t ld, int vocab, AcceptWs ws) {
  __shared__ float red_m[kStatThreads / 64];
  __shared__ int red_a[kStatThreads / 64];
  const int nch = ws.nch;
  const int r = blockIdx.x / nch;
  const int chunk = (blockIdx.x - r * nch + r) % nch;    // rotated: see sample_stats_item
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float4* row4 = reinterpret_cast<const float4*>(p_logits + (int64_t)r * ld);
  const int v4 = (vocab + 3) >> 2;
  const int f_begin = chunk * (kStatThreads * kStatF4);
  float4 x[kStatF4];
#pragma unroll
  for (int k = 0; k < kStatF4; ++k) x[k] = row4[min(f_begin + k * kStatThreads + tid, v4 - 1)];
  float m = -INFINITY;
  int am = -1;
#pragma unroll
  for (int k = 0; k < kStatF4; ++k) {              // a thread's indices increase with k
    const int y0 = (f_begin + k * kStatThreads + tid) * 4;
    const float xs[4] = {x[k].x, x[k].y, x[k].z, x[k].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool gt = y0 + j < vocab && xs[j] > m;   // strict: the first index wins ties
      m = gt ? xs[j] : m;
      am = gt ? y0 + j : am;
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1)
    merge_arg(m, am, __shfl_xor(m, off, 64), __shfl_xor(am, off, 64));
  if (lane == 0) {
    red_m[wave] = m;
    red_a[wave] = am;
  }
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < kStatThreads / 64; ++w) merge_arg(m, am, red_m[w], red_a[w]);
    ws.part_m[r * nch + chunk] = m;
    ws.part_am[r * nch + chunk] = am;
  }
}

// Sampling statistics: one workgroup per (listed row, chunk) item, the
// listed draft rows first (entry e < nq is the draft row at list position
// np + e), then the target rows (entry nq + r is target row r, no lookup).
// The grid covers every draft row; workgroups past the list end at once.  Each
// item: (reference, sum of exp(z - reference)) with z = logit / T in fp64
// and the chunk's maximum as the reference, so every exponent is <= 0 and
// the per-logit work is branch-free.
struct StatsArgs {
  const float* p_logits;
  const float* q_logits;
  int64_t ld;
  int vocab, R, np;   // np: target rows listed (R, or 0 when the LM head made their partials)
  int nq;             // draft-row entries in the grid (R, or 0 without draft rows)
  int leafp;          // 1: target partials of leaf rows exist too (the LM head's)
  int wfirst;         // 1: the walk workgroups come first in the grid (one stream list)
  double invT;
};

// The partials are published for the walk workgroups of the same launch: each
// value carries tag 1 in the low 8 bits of its mantissa (0: not yet written;
// the partials are cleared before every call), the reference rounded up to
// 44 mantissa bits before the sum is taken (so it stays >= every z of the
// chunk and carries its tag exactly), the sum rounded to 44 bits (2^-45
// relative).  A reader polls each partial until it shows its tag (a shared
// counter of finished items would serialize ten thousand atomics on one
// address).
SPEC_DEVICE double ref_round_up(double v) {
  const unsigned long long bits = (unsigned long long)__double_as_longlong(v);
  const unsigned long long r = (v > 0.0) ? ((bits + 0xffull) & ~0xffull) : (bits & ~0xffull);
  return __longlong_as_double((long long)r);
}
SPEC_DEVICE void publish_tagged(double* p, double v) {
  const unsigned long long bits =
      (((unsigned long long)__double_as_longlong(v) + 0x80ull) & ~0xffull) | 1ull;
  __hip_atomic_store(reinterpret_cast<unsigned long long*>(p), bits, __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}

SPEC_DEVICE void sample_stats_item(const StatsArgs& a, const AcceptWs& ws, int it, double* s_tab,
                                   float* red_m, double* red_s) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nch = ws.nch;
  int e = it / nch;
  // Consecutive workgroups go to the eight XCDs in turn, so chunk k of every
  // row would land on one XCD; rotating the chunk by the entry spreads each
  // chunk position (the ragged last one in particular) over all of them.
  const int chunk = (it - e * nch + e) % nch;
  // Draft-row entries come first in the grid: the entries past the list
  // (draft rows of leaves) then end at once early on, instead of sitting
  // between the last statistics and the walk workgroups in dispatch order.
  // Target-row entries are taken from the end of their range, so the
  // entries past that list end at once before the live ones, not between
  // the last statistics and the walk workgroups.
  int rr;
  if (a.wfirst) {                                    // one list (walks first)
    if (e >= ws.sync[2]) return;
    rr = ws.order[e];
  } else if (e < a.nq) {
    if (e >= ws.sync[2]) return;                     // past the listed draft rows
    rr = ws.order[e];
  } else {
    const int skip = a.np - ws.sync[3];
    const int ep = e - a.nq;
    if (ep < skip) return;                           // past the listed target rows
    rr = ws.order[a.R + ep - skip];
  }
  load_exp_table(s_tab);
  const int which = rr >= a.R ? 1 : 0;
  const f32x4* row4 = reinterpret_cast<const f32x4*>((which ? a.q_logits : a.p_logits) +
                                                     (int64_t)(rr - which * a.R) * a.ld);
  const int v4 = (a.vocab + 3) >> 2;
  const int f_begin = chunk * (kStatThreads * kStatF4);
  // the whole chunk in flight: clamped (in-bounds) loads, masked to -inf
  // (only the row's last chunk can reach past it).  Non-temporal: the
  // stream should not displace what the walks re-read between passes
  // (acceptance -1 to -6% in an interleaved A/B).
  float4 x[kStatF4];
#pragma unroll
  for (int k = 0; k < kStatF4; ++k) {
    const f32x4 v = __builtin_nontemporal_load(row4 + min(f_begin + k * kStatThreads + tid, v4 - 1));
    x[k] = make_float4(v[0], v[1], v[2], v[3]);
  }
  if ((chunk + 1) * kStatChunkLen > a.vocab) {
#pragma unroll
    for (int k = 0; k < kStatF4; ++k) {
      const int y0 = (f_begin + k * kStatThreads + tid) * 4;
      if (y0 + 0 >= a.vocab) x[k].x = -INFINITY;
      if (y0 + 1 >= a.vocab) x[k].y = -INFINITY;
      if (y0 + 2 >= a.vocab) x[k].z = -INFINITY;
      if (y0 + 3 >= a.vocab) x[k].w = -INFINITY;
    }
  }
  float cm = -INFINITY;
#pragma unroll
  for (int k = 0; k < kStatF4; ++k)
    cm = fmaxf(cm, fmaxf(fmaxf(x[k].x, x[k].y), fmaxf(x[k].z, x[k].w)));
  cm = wave_max(cm);
  if (lane == 0) red_m[wave] = cm;
  __syncthreads();
  for (int w = 0; w < kStatThreads / 64; ++w) cm = fmaxf(cm, red_m[w]);
  const double ref = (cm == -INFINITY) ? 0.0 : ref_round_up((double)cm * a.invT);
  double s = 0.0;
#pragma unroll
  for (int k = 0; k < kStatF4; ++k) {
    double e0, e1, e2, e3;
    exp_f64_clamped2(fma((double)x[k].x, a.invT, -ref), fma((double)x[k].y, a.invT, -ref), s_tab,
                     e0, e1);
    exp_f64_clamped2(fma((double)x[k].z, a.invT, -ref), fma((double)x[k].w, a.invT, -ref), s_tab,
                     e2, e3);
    s += e0;
    s += e1;
    s += e2;
    s += e3;
  }
  s = wave_sum_f64(s);
  if (lane == 0) red_s[wave] = s;
  __syncthreads();
  if (tid == 0) {
    double tot = 0.0;
    for (int w = 0; w < kStatThreads / 64; ++w) tot += red_s[w];
    publish_tagged(ws.part_ref + rr * nch + chunk, ref);
    publish_tagged(ws.part_s + rr * nch + chunk, tot);
  }
}

// Target-row chunk partials from the LM head's tile partials: one wave per
// (row, chunk), one lane per tile of the chunk, merged by a wave reduction
// into the (reference, sum) partials of the statistics items (published
// with their tag) or the (max, first argmax) partials of the greedy path.
constexpr int kTilesPerChunk = kStatChunkLen / kHeadTileV;
static_assert(kStatChunkLen % kHeadTileV == 0 && kTilesPerChunk == kWave,
              "a statistics chunk is one wave of head tiles");

__global__ void __launch_bounds__(256)
accept_head_merge_kernel(int B, int R, HeadTiles t, int greedy, AcceptWs ws, int vocab) {
  __shared__ double s_tab[256];
  const int tid = threadIdx.x, lane = tid & 63;
  if (!greedy) load_exp_table(s_tab);
  __syncthreads();
  const int nch = ws.nch;
  const int idx = blockIdx.x * 4 + (tid >> 6);
  if (idx >= R * nch) return;                         // whole wave
  const int r = idx / nch, c = idx - r * nch;
  const int k = c * kTilesPerChunk + lane;
  const bool has = k < t.ntile;
  const int64_t at = (int64_t)r * t.ntile + k;
  if (greedy) {
    float m = has ? t.m[at] : -INFINITY;
    int am = has ? t.am[at] : -1;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
      merge_arg(m, am, __shfl_xor(m, off, 64), __shfl_xor(am, off, 64));
    if (lane == 0) {
      ws.part_m[idx] = m;
      ws.part_am[idx] = am;
    }
    return;
  }
  const double ref = has ? t.ref[at] : -INFINITY;
  double top = ref;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) top = fmax(top, __shfl_xor(top, off, 64));
  top = (top == -INFINITY) ? 0.0 : ref_round_up(top);
  const double s = (has && ref != -INFINITY) ? t.s[at] * exp_f64(ref - top, s_tab) : 0.0;
  const double tot = wave_sum(s);
  if (lane == 0) {
    publish_tagged(ws.part_ref + idx, top);
    publish_tagged(ws.part_s + idx, tot);
  }
}

// Per-row results from the chunk partials, merged in chunk order (so every
// run gives the same bits): a row's log-sum-exp (the sampling walk merges its
// own rows; the partials are loaded 8 at a time, all in flight together), or
// the target argmax.  accept_finalize (greedy): one thread per row writes the
// argmax and, per child, 1 if its token is the parent's argmax.
SPEC_DEVICE unsigned long long load_partial(const double* p) {
  return __hip_atomic_load(reinterpret_cast<unsigned long long*>(const_cast<double*>(p)),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// False if some partial never showed its tag (the polls gave up; with
// max_spins = 0: not all published yet).
SPEC_DEVICE bool merged_ref_sum(const AcceptWs& ws, int rr, const double* tab, double& lse,
                               int max_spins = kWalkMaxSpins) {
  const int nch = ws.nch;
  const double* pr = ws.part_ref + (int64_t)rr * nch;
  const double* ps = ws.part_s + (int64_t)rr * nch;
  double ref = 0.0, s = 0.0;
  bool ok = true;
  for (int c0 = 0; c0 < nch; c0 += 8) {
    unsigned long long r8[8], s8[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      r8[j] = (c0 + j < nch) ? load_partial(pr + c0 + j) : 1ull;
      s8[j] = (c0 + j < nch) ? load_partial(ps + c0 + j) : 1ull;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (c0 + j >= nch) break;
      int spins = 0;
      while (((r8[j] & s8[j]) & 0xffull) == 0 && ++spins <= max_spins) {
        __builtin_amdgcn_s_sleep(1);
        r8[j] = load_partial(pr + c0 + j);
        s8[j] = load_partial(ps + c0 + j);
      }
      ok &= ((r8[j] & s8[j]) & 0xffull) != 0;
      const double rj = __longlong_as_double((long long)(r8[j] & ~0xffull));
      const double sj = __longlong_as_double((long long)(s8[j] & ~0xffull));
      if (c0 + j == 0) {
        ref = rj;
        s = sj;
      } else {
        merge_ref(ref, s, rj, sj, tab);
      }
    }
  }
  lse = ref + log(s);
  return ok;
}
SPEC_DEVICE int merged_argmax(const AcceptWs& ws, int r) {
  const int nch = ws.nch;
  float m = ws.part_m[r * nch];
  int am = ws.part_am[r * nch];
  for (int c = 1; c < nch; ++c)
    merge_arg(m, am, ws.part_m[r * nch + c], ws.part_am[r * nch + c]);
  return am;
}

__global__ void __launch_bounds__(256)
accept_finalize_kernel(const int32_t* __restrict__ row_offsets, int B, int R,
                       const int32_t* __restrict__ parents, const int32_t* __restrict__ tokens,
                       AcceptWs ws, float* __restrict__ child_p) {
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r >= R) return;
  const int b = request_of_row(row_offsets, B, r);
  const int o = row_offsets[b];
  const int u = r - o;
  ws.am[r] = merged_argmax(ws, r);
  if (!child_p) return;
  const int pu = parents[r];
  if (u == 0 || pu < 0 || pu >= u) {              // root, or invalid tree (reported by the walk)
    child_p[r] = __int_as_float(0x7fc00000);
    return;
  }
  child_p[r] = (tokens[r] == merged_argmax(ws, o + pu)) ? 1.0f : 0.0f;
}

// ---------------------------------------------------------------------------
// Walk.

struct WalkShared {
  alignas(16) int par[kMaxRows];   // read as int4 by load_tree
  int tok[kMaxRows];
  int kid_start[kMaxRows + 1];
  int kid_list[kMaxRows];
  int path[kMaxRows];
  int toks[kMaxRows + 1];
  int rej[kMaxRows];                // deterministic children: tokens rejected at the current node
  double cp[kMaxRows];              // P_parent(x_c), Q_parent(x_c) of each child row
  double cq[kMaxRows];
  double lse[2][kMaxRows];          // log-sum-exp of logits / T: target, draft rows
  double coin[2][kMaxRows];         // row k: coin of the accept test of child k, of the draw at k
  double segsum[kMaxSegs];          // the last pass's segment sums
  double tab[256];
  double wave_tot[kWalkWaves];      // per wave (draw rescan, statistics item)
  float red_m[kWalkWaves];          // per wave (statistics item)
  double part[kPassChunk][kWalkWaves];  // per segment and wave (pass)
  double lane_excl[64];             // prefix of the segment sums, per lane block
  double total;
  double c0;
  double chunk_base, chunk_target;   // P-only draw: mass before the drawn chunk, the target
  double frame;                      // leaf pass: the reference its sums were rescaled to
  int chunk;                         // P-only draw: the chunk holding the target (-1: none)
  unsigned char ready[kMaxRows];     // walks first: node's row statistics merged (lazily)
  int tile;                          // LM-head leaf draw: the 256-entry tile holding the target
  double tile_target;                //   and the target less the mass before that tile
  int found_seg;
  int pick;
  int bad;
  int timeout;
  // walk state (broadcast from thread 0)
  int u, len, ntok, done, accept, flags, nrej;
};

// Unnormalised weight of entry y: max(0, P_y - t Q_y), or P_y alone when
// need_q is false (t = 0 at a leaf).
SPEC_DEVICE double walk_weight(float py, float qy, double invT, double lse_p, double lse_q,
                               double t, bool need_q, const double* tab) {
  double P, Q;
  exp_f64_2((double)py * invT - lse_p, need_q ? (double)qy * invT - lse_q : -INFINITY, tab, P, Q);
  if (!need_q) return P;
  return fmax(0.0, fma(-t, Q, P));
}

SPEC_DEVICE double wave_incl_scan(double v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double x = __shfl_up(v, o, 64);
    if (lane >= o) v += x;
  }
  return v;
}

// Exchange of segment sums between the S workgroups of a request.  Each
// sum is published with a relaxed agent-scope atomic store that carries its
// pass in the low 8 bits of the mantissa (the value rounded to 44 bits,
// 2^-45 relative, far inside every near-threshold window), and read with
// relaxed agent-scope atomic loads polled until the tag is the wanted pass.
// A read that sees the wanted tag holds that pass's value: the protocol
// needs no ordering between different locations, hence no fences, no cache
// writeback or invalidate and no counter.  Tag 0 means cleared (the
// exchange area is zeroed before every walk); passes cycle through 1..255,
// and sums live in two buffers by pass parity, so a slot holds the tag of
// its current pass, of the pass two before, or 0 -- never a stale copy of
// the wanted tag.  A poll loop that exceeds `max_spins` gives up: the walk
// ends for that workgroup, and the request reports a timeout unless slice 0
// read every sum (slice 0 alone writes the outputs, so they are then
// complete).
SPEC_DEVICE int pass_tag(int pass) { return (pass - 1) % 255 + 1; }

SPEC_DEVICE void publish_sum(double* p, double v, int tag) {
  const unsigned long long bits =
      (((unsigned long long)__double_as_longlong(v) + 0x80ull) & ~0xffull) | (unsigned)tag;
  __hip_atomic_store(reinterpret_cast<unsigned long long*>(p), bits, __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
SPEC_DEVICE double tagged_value(unsigned long long bits) {
  return __longlong_as_double((long long)(bits & ~0xffull));
}
SPEC_DEVICE unsigned long long load_tagged(const double* p) {
  return __hip_atomic_load(reinterpret_cast<unsigned long long*>(const_cast<double*>(p)),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// The value of slot p once it carries `tag`; false if polling gave up.
SPEC_DEVICE bool read_sum(const double* p, int tag, int max_spins, double& v) {
  unsigned long long bits = load_tagged(p);
  int spins = 0;
  while ((int)(bits & 0xffull) != tag) {
    if (++spins > max_spins) {
      v = 0.0;
      return false;
    }
    __builtin_amdgcn_s_sleep(1);
    bits = load_tagged(p);
  }
  v = tagged_value(bits);
  return true;
}

struct WalkCtx {
  const float* p;     // target row of the current node
  const float* q;     // draft row of the current node
  double invT, lse_p, lse_q;
  int vocab, nseg, seg_lo, seg_hi, slice, S, max_spins;
  int rd_lo, rd_n;    // segments whose sums the pass exchanges (all, or one chunk's)
  double* seg;        // this request's [2][nseg]
  const int* rej;     // tokens whose weight is 0 (LDS), nrej of them
  int nrej;
};

// Bit j set iff entry y0 + j is one of the excluded tokens.
SPEC_DEVICE int excluded4(const WalkCtx& c, int y0) {
  int ex = 0;
  for (int k = 0; k < c.nrej; ++k) {
    const unsigned d = (unsigned)(c.rej[k] - y0);
    if (d < 4u) ex |= 1 << d;
  }
  return ex;
}

// Sum of the weights of 4 consecutive entries starting at y0: max(0, P - tQ)
// (or P alone, without the excluded tokens), entries past the row masked to
// weight 0.
template <bool kQ>
SPEC_DEVICE double weight4(const WalkCtx& c, float4 pv, float4 qv, int y0, double t,
                           const double* tab) {
  const float pa[4] = {pv.x, pv.y, pv.z, pv.w};
  const float qa[4] = {qv.x, qv.y, qv.z, qv.w};
  const int ex = kQ ? 0 : excluded4(c, y0);
  double acc = 0.0;
  if (kQ) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool in = y0 + j < c.vocab;                 // ragged end
      double P, Q;
      exp_f64_clamped2((double)(in ? pa[j] : -INFINITY) * c.invT - c.lse_p,
                       (double)(in ? qa[j] : -INFINITY) * c.invT - c.lse_q, tab, P, Q);
      acc += fmax(0.0, fma(-t, Q, P));
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; j += 2) {
      const bool in0 = y0 + j < c.vocab && !((ex >> j) & 1);   // ragged end, excluded tokens
      const bool in1 = y0 + j + 1 < c.vocab && !((ex >> (j + 1)) & 1);
      double P0, P1;
      exp_f64_clamped2((double)(in0 ? pa[j] : -INFINITY) * c.invT - c.lse_p,
                       (double)(in1 ? pa[j + 1] : -INFINITY) * c.invT - c.lse_p, tab, P0, P1);
      acc += P0;
      acc += P1;
    }
  }
  return acc;
}

// NR consecutive segments from s0: thread tid takes float4 tid of each (all
// loads in flight at once); each wave's sums go to sh.part[s0 - base + i].
// Indices past the row are clamped (in-bounds loads) and masked.
template <bool kQ, int NR>
SPEC_DEVICE void pass_round(WalkShared& sh, const WalkCtx& c, int s0, int base, double t) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float4* p4 = reinterpret_cast<const float4*>(c.p);
  const float4* q4 = reinterpret_cast<const float4*>(c.q);
  const int v4 = (c.vocab + 3) >> 2;
  float4 pb[NR], qb[NR];
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    const int f = min((s0 + i) * (kSeg / 4) + tid, v4 - 1);
    pb[i] = p4[f];
    qb[i] = kQ ? q4[f] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    const double w = wave_sum_f64(weight4<kQ>(c, pb[i], qb[i], (s0 + i) * kSeg + 4 * tid, t, sh.tab));
    if (lane == 0) sh.part[s0 - base + i][wave] = w;
  }
}

template <bool kQ>
SPEC_DEVICE void pass_segments(WalkShared& sh, const WalkCtx& c, double* seg, double t, int tag) {
  const int tid = threadIdx.x;
  for (int base = c.seg_lo; base < c.seg_hi; base += kPassChunk) {
    const int end = min(c.seg_hi, base + kPassChunk);
    int s0 = base;
    for (; s0 + kPassF <= end; s0 += kPassF) pass_round<kQ, kPassF>(sh, c, s0, base, t);
    if ((end - s0) & 4) { pass_round<kQ, 4>(sh, c, s0, base, t); s0 += 4; }
    if ((end - s0) & 2) { pass_round<kQ, 2>(sh, c, s0, base, t); s0 += 2; }
    if ((end - s0) & 1) pass_round<kQ, 1>(sh, c, s0, base, t);
    __syncthreads();
    if (tid < end - base) {
      double tot = 0.0;
#pragma unroll
      for (int w = 0; w < kWalkWaves; ++w) tot += sh.part[tid][w];
      publish_sum(&seg[base + tid], tot, tag);
    }
    __syncthreads();
  }
}

// One vocabulary pass: this workgroup's segments of max(0, P - tQ) (or P),
// published; then every segment's sum of this pass (waiting for the other
// slices' as they arrive) and their ordered total.
SPEC_DEVICE double walk_pass(WalkShared& sh, const WalkCtx& c, int pass, double t, bool need_q) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  double* seg = c.seg + (pass & 1) * c.nseg;
  const int tag = pass_tag(pass);
  if (need_q) {
    // Residual passes are the walks' critical path; raised priority lets
    // their exponentials go first on SIMDs shared with leaf passes and the
    // last statistics items.
    __builtin_amdgcn_s_setprio(2);
    pass_segments<true>(sh, c, seg, t, tag);
    __builtin_amdgcn_s_setprio(0);
  } else {
    pass_segments<false>(sh, c, seg, t, tag);
  }
  if (wave == 0) {
    const int per = (c.rd_n + 63) / 64;
    double part = 0.0;
    bool late = false;
    // the first kSumLoads sums of the lane in one round trip; a slot that
    // does not show the tag yet is polled
    const double* mine = seg + c.rd_lo + lane * per;
    unsigned long long first[kSumLoads];
#pragma unroll
    for (int k = 0; k < kSumLoads; ++k)
      first[k] = (k < per && lane * per + k < c.rd_n) ? load_tagged(mine + k) : 0ull;
#pragma unroll
    for (int k = 0; k < kSumLoads; ++k) {
      const int sidx = c.rd_lo + lane * per + k;
      if (k < per && lane * per + k < c.rd_n) {
        double v;
        if ((int)(first[k] & 0xffull) == tag)
          v = tagged_value(first[k]);
        else
          late |= !read_sum(mine + k, tag, c.max_spins, v);
        sh.segsum[sidx] = v;
        part += v;
      }
    }
    for (int k = kSumLoads; k < per; ++k) {
      const int sidx = c.rd_lo + lane * per + k;
      if (lane * per + k < c.rd_n) {
        double v;
        late |= !read_sum(&seg[sidx], tag, c.max_spins, v);
        sh.segsum[sidx] = v;
        part += v;
      }
    }
    if (__any(late) && lane == 0) sh.timeout = 1;
    const double incl = wave_incl_scan(part, lane);
    sh.lane_excl[lane] = incl - part;
    if (lane == 63) sh.total = incl;
  }
  __syncthreads();
  return sh.total;
}

// Inverse-CDF draw from the weights of the last pass: the first entry whose
// cumulative weight (over the pass's segments, in order) exceeds `target`.
// Every slice finds the segment from that pass's sums (kept in LDS by
// walk_pass); slice 0 rescans it and returns the token (other slices
// return -1).
SPEC_DEVICE int walk_draw(WalkShared& sh, const WalkCtx& c, double t, bool need_q,
                          double target) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (wave == 0) {
    const int per = (c.rd_n + 63) / 64;
    double cum = sh.lane_excl[lane];
    int hit = -1, pos = -1;
    double hit_c0 = 0.0, pos_c0 = 0.0;
    for (int k = 0; k < per; ++k) {
      const int sidx = c.rd_lo + lane * per + k;
      if (lane * per + k < c.rd_n) {
        const double v = sh.segsum[sidx];
        const double nxt = cum + v;
        if (hit < 0 && nxt > target) {
          hit = sidx;
          hit_c0 = cum;
        }
        if (v > 0.0) {
          pos = sidx;
          pos_c0 = cum;
        }
        cum = nxt;
      }
    }
    const uint64_t ball = __ballot(hit >= 0);
    const uint64_t pball = __ballot(pos >= 0);
    if (lane == 0) sh.pick = -1;
    if (ball) {
      const int first = __ffsll((long long)ball) - 1;
      if (lane == first) {
        sh.found_seg = hit;
        sh.c0 = hit_c0;
      }
    } else if (pball) {
      // rounding left the target past the last cumulative sum: the last
      // segment holding a positive weight, whose rescan then returns its last
      // positive weight (the last one of the row)
      const int lastl = 63 - __clzll((long long)pball);
      if (lane == lastl) {
        sh.found_seg = pos;
        sh.c0 = pos_c0;
      }
    } else if (lane == 0) {
      sh.found_seg = -1;
    }
  }
  __syncthreads();
  const int fs = sh.found_seg;
  if (fs < 0) return -1;                             // no positive weight (not reached)
  if (c.slice != 0) return -1;
  // rescan the segment with the same arithmetic as the pass
  const int y0 = fs * kSeg + 4 * tid;
  const int ex = need_q ? 0 : excluded4(c, y0);
  double w[4] = {0.0, 0.0, 0.0, 0.0};
  double acc = 0.0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (y0 + j < c.vocab && !((ex >> j) & 1)) {
      w[j] = walk_weight(c.p[y0 + j], need_q ? c.q[y0 + j] : 0.f, c.invT, c.lse_p, c.lse_q, t,
                         need_q, sh.tab);
      acc += w[j];
    }
  }
  const double incl = wave_incl_scan(acc, lane);
  if (lane == 63) sh.wave_tot[wave] = incl;
  if (tid == 0) sh.pick = 0x7fffffff;
  __syncthreads();
  double base = sh.c0;
  for (int k = 0; k < wave; ++k) base += sh.wave_tot[k];
  double cum = base + (incl - acc);
  int pick = -1, lastpos = -1;
  for (int j = 0; j < 4; ++j) {
    if (y0 + j >= c.vocab) break;
    if (w[j] > 0.0) lastpos = y0 + j;
    cum += w[j];
    if (cum > target) {
      pick = y0 + j;
      break;
    }
  }
  if (pick >= 0) atomicMin(&sh.pick, pick);
  __syncthreads();
  int res = sh.pick;
  if (res == 0x7fffffff) {
    // rounding inside the segment: last positive weight of the segment
    if (tid == 0) sh.pick = -1;
    __syncthreads();
    if (lastpos >= 0) atomicMax(&sh.pick, lastpos);
    __syncthreads();
    res = sh.pick;
  }
  return res;
}

// The request's tree into LDS (and, with `tab`, the exponential table in the
// same memory round trip): parents, tokens, validity, children lists.
// Needs blockDim.x >= max(n, 256).
SPEC_DEVICE void load_tree(WalkShared& sh, const int32_t* parents, const int32_t* tokens, int o,
                           int n, double* tab = nullptr) {
  const int tid = threadIdx.x, lane = tid & 63;
  int p = -1, tk = 0;
  if (tid < n) {
    p = parents[o + tid];
    tk = tokens[o + tid];
  }
  if (tab && tid < 256) tab[tid] = kExp2Frac[tid];
  const bool ok = tid >= n || ((tid == 0) ? (p == -1) : (p >= 0 && p < tid));
  if (tid < n) {
    sh.par[tid] = p;
    sh.tok[tid] = tk;
  }
  if (__syncthreads_or(!ok)) {
    if (tid == 0) sh.bad = 1;
    __syncthreads();
    return;
  }
  if (tid == 0) sh.bad = 0;
  // children of row tid: rows j > tid with par[j] == tid, read 4 at a time
  // (par is padded with -1 to a multiple of 4)
  if (tid < ((n + 3) & ~3) && tid >= n) sh.par[tid] = -1;
  __syncthreads();
  const int4* par4 = reinterpret_cast<const int4*>(sh.par);
  if (tid < n) {
    int cnt = 0;
    for (int j4 = (tid + 1) >> 2; j4 < (n + 3) >> 2; ++j4) {
      const int4 q = par4[j4];
      cnt += (q.x == tid) + (q.y == tid) + (q.z == tid) + (q.w == tid);
    }
    sh.kid_start[tid + 1] = cnt;
  }
  __syncthreads();
  if (tid < 64) {                       // inclusive prefix of the counts, 4 per lane
    int v[4], t = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = 1 + 4 * lane + j;
      v[j] = (i <= n) ? sh.kid_start[i] : 0;
      t += v[j];
    }
    int incl = t;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int x = __shfl_up(incl, off, 64);
      if (lane >= off) incl += x;
    }
    int run = incl - t;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = 1 + 4 * lane + j;
      run += v[j];
      if (i <= n) sh.kid_start[i] = run;
    }
    if (lane == 0) sh.kid_start[0] = 0;
  }
  __syncthreads();
  if (tid < n) {
    int pos = sh.kid_start[tid];
    for (int j4 = (tid + 1) >> 2; j4 < (n + 3) >> 2; ++j4) {
      const int4 q = par4[j4];
      if (q.x == tid) sh.kid_list[pos++] = 4 * j4;
      if (q.y == tid) sh.kid_list[pos++] = 4 * j4 + 1;
      if (q.z == tid) sh.kid_list[pos++] = 4 * j4 + 2;
      if (q.w == tid) sh.kid_list[pos++] = 4 * j4 + 3;
    }
  }
  __syncthreads();
}

struct WalkOut {
  int32_t* accept_len;
  int32_t* path;
  int32_t* tokens_out;
  uint8_t* accept_mask;
  int32_t* flags;
  int path_stride;
  float* child_p;     // optional fp32 copies of P_u(x_c), Q_u(x_c) (sampling walk)
  float* child_q;
};

// Writes path, tokens (except index `skip`, written by the slice that drew
// the final token), accept mask, length and flags.
SPEC_DEVICE void write_outputs(WalkShared& sh, const WalkOut& w, int b, int o, int n, int skip) {
  const int tid = threadIdx.x;
  const int len = sh.len, nt = sh.ntok;
  for (int k = tid; k < w.path_stride; k += blockDim.x) {
    w.path[(int64_t)b * w.path_stride + k] = (k < len) ? sh.path[k] : -1;
    if (k != skip)
      w.tokens_out[(int64_t)b * w.path_stride + k] = (k < nt) ? sh.toks[k] : -1;
  }
  if (w.accept_mask) {
    for (int i = tid; i < n; i += blockDim.x) w.accept_mask[o + i] = 0;
    __syncthreads();
    for (int k = tid; k < len; k += blockDim.x) w.accept_mask[o + sh.path[k]] = 1;
  }
  if (tid == 0) {
    w.accept_len[b] = len - 1;
    if (w.flags) w.flags[b] = sh.flags;
  }
}

// A request without a result (invalid tree, or a walk barrier that gave
// up): accept_len -1, path and tokens -1, empty accept mask, the flags given.
SPEC_DEVICE void write_abandoned(const WalkOut& w, int b, int o, int n, int flags) {
  const int tid = threadIdx.x;
  for (int k = tid; k < w.path_stride; k += blockDim.x) {
    w.path[(int64_t)b * w.path_stride + k] = -1;
    w.tokens_out[(int64_t)b * w.path_stride + k] = -1;
  }
  if (w.accept_mask)
    for (int i = tid; i < n; i += blockDim.x) w.accept_mask[o + i] = 0;
  if (tid == 0) {
    w.accept_len[b] = -1;
    if (w.flags) w.flags[b] = flags;
  }
}

SPEC_DEVICE double wave_max_f64(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmax(v, __shfl_xor(v, o, 64));
  return v;
}

// The draw at a leaf whose target row was never streamed (its statistics
// are needed for nothing else): one pass in two steps.  Each slice takes
// the largest logit / T of its segments as its reference (rounded up to 44
// bits, published with the pass tag; -1e300 for a slice with nothing in
// range), then publishes its segment sums of exp(z/T - reference).  Every
// slice reads all sums and the references of the slices that made them,
// rescales the sums to the largest reference R and leaves them in LDS for
// walk_draw, whose weights are then exp(z/T - R).  Returns R.
SPEC_DEVICE double leaf_pass(WalkShared& sh, WalkCtx& c, int pass, double* sref_req) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tag = pass_tag(pass);
  double* seg = c.seg + (pass & 1) * c.nseg;
  double* sr = sref_req + (pass & 1) * kMaxSlices;
  const float4* p4 = reinterpret_cast<const float4*>(c.p);
  const int v4 = (c.vocab + 3) >> 2;
  float mx = -INFINITY;
  for (int s0 = c.seg_lo; s0 < c.seg_hi; s0 += kPassF) {
    float4 v[kPassF];
#pragma unroll
    for (int i = 0; i < kPassF; ++i)
      v[i] = p4[min((min(s0 + i, c.seg_hi - 1)) * (kSeg / 4) + tid, v4 - 1)];
#pragma unroll
    for (int i = 0; i < kPassF; ++i) {
      const int y0 = (min(s0 + i, c.seg_hi - 1)) * kSeg + 4 * tid;
      const float a = (y0 + 0 < c.vocab) ? v[i].x : -INFINITY;
      const float b = (y0 + 1 < c.vocab) ? v[i].y : -INFINITY;
      const float d = (y0 + 2 < c.vocab) ? v[i].z : -INFINITY;
      const float e = (y0 + 3 < c.vocab) ? v[i].w : -INFINITY;
      mx = fmaxf(mx, fmaxf(fmaxf(a, b), fmaxf(d, e)));
    }
  }
  mx = wave_max(mx);
  if (lane == 0) sh.red_m[wave] = mx;
  __syncthreads();
  float m = sh.red_m[0];
  for (int w = 1; w < kWalkWaves; ++w) m = fmaxf(m, sh.red_m[w]);
  const double ref = (m == -INFINITY) ? -1e300 : ref_round_up((double)m * c.invT);
  c.lse_p = ref;
  pass_segments<false>(sh, c, seg, 0.0, tag);
  if (tid == 0 && c.seg_lo < c.seg_hi) publish_sum(sr + c.slice, ref, tag);
  if (wave == 0) {
    // the slices' references (lane k < S: slice k's) and this lane's sums,
    // all loads issued together; a slot without the tag yet is polled
    const int per_slice = (c.nseg + c.S - 1) / c.S;
    const bool owns = lane < c.S && lane * per_slice < c.nseg;
    const int per = (c.nseg + 63) / 64;
    const double* mine = seg + lane * per;
    const unsigned long long rbits = owns ? load_tagged(sr + lane) : 0ull;
    unsigned long long first[kSumLoads];
#pragma unroll
    for (int k = 0; k < kSumLoads; ++k)
      first[k] = (k < per && lane * per + k < c.nseg) ? load_tagged(mine + k) : 0ull;
    bool late = false;
    double rf = -INFINITY;
    if (owns) {
      if ((int)(rbits & 0xffull) == tag)
        rf = tagged_value(rbits);
      else
        late |= !read_sum(sr + lane, tag, c.max_spins, rf);
    }
#pragma unroll
    for (int k = 0; k < kSumLoads; ++k) {
      const int sidx = lane * per + k;
      if (k < per && sidx < c.nseg) {
        double v;
        if ((int)(first[k] & 0xffull) == tag)
          v = tagged_value(first[k]);
        else
          late |= !read_sum(mine + k, tag, c.max_spins, v);
        sh.segsum[sidx] = v;
      }
    }
    for (int k = kSumLoads; k < per; ++k) {
      const int sidx = lane * per + k;
      if (sidx < c.nseg) {
        double v;
        late |= !read_sum(&seg[sidx], tag, c.max_spins, v);
        sh.segsum[sidx] = v;
      }
    }
    // every sum to the largest reference, in segment order per lane
    const double top = wave_max_f64(rf);
    double part = 0.0;
    for (int k = 0; k < per; ++k) {
      const int sidx = lane * per + k;
      const double ro = __shfl(rf, min(sidx, c.nseg - 1) / per_slice, 64);
      if (sidx < c.nseg) {
        const double w = sh.segsum[sidx] * exp_f64(ro - top, sh.tab);
        sh.segsum[sidx] = w;
        part += w;
      }
    }
    if (__any(late) && lane == 0) sh.timeout = 1;
    const double incl = wave_incl_scan(part, lane);
    sh.lane_excl[lane] = incl - part;
    if (lane == 63) sh.total = incl;
    if (lane == 0) sh.frame = top;
  }
  __syncthreads();
  return sh.frame;
}

// A draw from P_u alone (at a leaf, or from P_u without the rejected tokens
// once every deterministic child is rejected) locates its chunk of the
// vocabulary from the statistics partials of row u: chunk k holds mass
// s_k exp(ref_k - lse_u), less the P_u of the excluded tokens in it.  The
// target is r times their total; the drawn chunk is the first whose
// cumulative mass exceeds it (rounding past the end: the last chunk with
// mass).  Only that chunk's segments are then passed over, against the
// target less the mass before the chunk.  Wave 0 of every slice computes the
// same values; sh.chunk = -1 (no chunk with mass) falls back to a full pass.
static_assert(kStatChunkLen % kSeg == 0, "a chunk is whole segments");
constexpr int kSegsPerChunk = kStatChunkLen / kSeg;
SPEC_DEVICE void locate_chunk(WalkShared& sh, const AcceptWs& ws, const WalkCtx& c, int row,
                              double r) {
  const int lane = threadIdx.x & 63;
  const int nch = ws.nch;                              // <= 64 (vocabulary <= 2^20)
  double m = 0.0;
  if (lane < nch) {
    const double ref = tagged_value(load_partial(ws.part_ref + (int64_t)row * nch + lane));
    const double sum = tagged_value(load_partial(ws.part_s + (int64_t)row * nch + lane));
    m = sum * exp_f64(ref - c.lse_p, sh.tab);
  }
  // excluded tokens, 64 at a time: lane k loads token k's logit (one round
  // trip for all of them), then each is taken off its chunk in list order
  for (int k0 = 0; k0 < c.nrej; k0 += 64) {
    const int k = k0 + lane;
    const int x = (k < c.nrej) ? c.rej[k] : -1;
    const bool in = x >= 0 && x < c.vocab;
    const double px = in ? exp_f64((double)c.p[x] * c.invT - c.lse_p, sh.tab) : 0.0;
    const int xc = in ? x / kStatChunkLen : -1;
    for (int j = 0; j < 64 && k0 + j < c.nrej; ++j) {
      const int cj = __shfl(xc, j, 64);
      const double pj = __shfl(px, j, 64);
      if (lane == cj) m -= pj;
    }
  }
  m = fmax(m, 0.0);
  const double incl = wave_incl_scan(m, lane);
  const double total = __shfl(incl, 63, 64);
  const double target = r * total;
  const uint64_t hit = __ballot(lane < nch && incl > target && m > 0.0);
  const uint64_t pos = __ballot(m > 0.0);
  int ck = -1;
  if (total > 0.0) ck = hit ? __ffsll((long long)hit) - 1 : 63 - __clzll((long long)pos);
  if (lane == 0) {
    sh.chunk = -1;
    sh.chunk_target = target;
  }
  if (ck >= 0 && lane == ck) {
    sh.chunk = ck;
    sh.chunk_base = incl - m;
  }
}

// The bonus draw at a leaf on the LM-head path, whose logits were not
// stored (only rows with children are).  locate_chunk finds the 16K chunk
// from the merged partials; the head's partials of that chunk's 64 tiles of
// 256 entries, s_k exp(ref_k - lse), find the tile; the tile's logits are
// recomputed from the hidden row and the weight rows (bf16 products summed
// in fp32, as the head does; each slice a share, exchanged with the pass
// tag); slice 0 then draws inside the tile with the walk's weights.  A
// target within rounding of the end of the chunk or tile falls back to the
// last tile or entry with positive weight, as the other draws do.  Returns
// the token (slice 0), -1 in the other slices or on a timeout.
SPEC_DEVICE int head_leaf_draw(WalkShared& sh, const WalkCtx& c, const AcceptWs& ws,
                               const HeadTiles& ht, int row, int b, int tag, double r) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (wave == 0) locate_chunk(sh, ws, c, row, r);
  __syncthreads();
  if (wave == 0) {
    const int ck = sh.chunk < 0 ? 0 : sh.chunk;       // (no mass at all: not reached)
    const int t = ck * kTilesPerChunk + lane;
    double m = 0.0;
    if (t < ht.ntile) {
      const int64_t i = (int64_t)row * ht.ntile + t;
      m = ht.s[i] * exp_f64(ht.ref[i] - c.lse_p, sh.tab);
    }
    const double incl = wave_incl_scan(m, lane);
    const double target = sh.chunk_target - sh.chunk_base;
    const uint64_t hit = __ballot(t < ht.ntile && incl > target && m > 0.0);
    const uint64_t pos = __ballot(m > 0.0);
    const int tk = hit ? __ffsll((long long)hit) - 1 : pos ? 63 - __clzll((long long)pos) : 0;
    if (lane == tk) {
      sh.tile = ck * kTilesPerChunk + tk;
      sh.tile_target = target - (incl - m);
    }
  }
  __syncthreads();
  const int v0 = sh.tile * kHeadTileV;
  const int nv = min(kHeadTileV, c.vocab - v0);
  // this slice's share of the tile: G threads per logit, G a power of two
  const int per = (nv + c.S - 1) / c.S;
  const int j0 = c.slice * per, j1 = min(nv, j0 + per);
  int G = 1;
  while (G < 64 && 2 * G * per <= kWalkThreads) G *= 2;
  const int jl = tid / G, part = tid % G;
  const int j = j0 + jl;
  const bool mine = jl < per && j < j1;
  float z = 0.0f;
  if (mine) {
    const uint4* wr = reinterpret_cast<const uint4*>(ht.weight + (int64_t)(v0 + j) * ht.H);
    const uint4* hr = reinterpret_cast<const uint4*>(ht.hidden + (int64_t)row * ht.H);
    for (int k = part; k < ht.H / 8; k += G) {
      const uint4 wv = wr[k], hv = hr[k];
      const uint32_t wa[4] = {wv.x, wv.y, wv.z, wv.w}, ha[4] = {hv.x, hv.y, hv.z, hv.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        z = fmaf(__uint_as_float(wa[e] << 16), __uint_as_float(ha[e] << 16), z);
        z = fmaf(__uint_as_float(wa[e] & 0xffff0000u), __uint_as_float(ha[e] & 0xffff0000u), z);
      }
    }
  }
  for (int o = G / 2; o > 0; o >>= 1) z += __shfl_xor(z, o, 64);
  double* slot = ht.leafz + (int64_t)b * kHeadTileV;
  if (mine && part == 0) publish_sum(slot + j, (double)z, tag);   // a float: exact in 44 bits
  if (c.slice != 0) return -1;
  double zd = 0.0;
  if (tid < nv && !read_sum(slot + tid, tag, c.max_spins, zd)) sh.timeout = 1;
  __syncthreads();
  if (sh.timeout) return -1;
  const double w = tid < nv ? walk_weight((float)zd, 0.0f, c.invT, c.lse_p, 0.0, 0.0, false, sh.tab)
                            : 0.0;
  const double incl = wave_incl_scan(w, lane);
  if (lane == 63) sh.wave_tot[wave] = incl;
  if (tid == 0) sh.pick = 0x7fffffff;
  __syncthreads();
  double base = 0.0;
  for (int k = 0; k < wave; ++k) base += sh.wave_tot[k];
  if (tid < nv && w > 0.0 && base + incl > sh.tile_target) atomicMin(&sh.pick, v0 + tid);
  __syncthreads();
  int res = sh.pick;
  if (res == 0x7fffffff) {
    // rounding past the tile's last cumulative weight: its last positive entry
    __syncthreads();
    if (tid == 0) sh.pick = -1;
    __syncthreads();
    if (tid < nv && w > 0.0) atomicMax(&sh.pick, v0 + tid);
    __syncthreads();
    res = sh.pick;
  }
  return res;
}

// The statistics of one node, merged when the walk reaches it (walks that
// go first in the grid, while the statistics still stream): the
// log-sum-exps of its rows from their chunk partials (polled until
// published), then P_u(x_c), Q_u(x_c) of its children, with the arithmetic
// of the all-rows form (the children's logits load while the partials are
// polled).  Block-wide; sets sh.timeout if a partial never arrives.  (Also
// merging, in the same round trip, every other row whose partials were
// already in measured slower: the extra loads lengthen each step.)
SPEC_DEVICE void node_stats(WalkShared& sh, const AcceptWs& ws, int R, int o, int u,
                            const float* p_logits, const float* q_logits, int64_t ld, int vocab,
                            double invT, bool topk) {
  const int tid = threadIdx.x;
  const int k0 = sh.kid_start[u], nk = sh.kid_start[u + 1] - k0;
  float lp = 0.0f, lq = 0.0f;
  bool cv = false;
  int ch = -1;
  if (tid < nk) {
    ch = sh.kid_list[k0 + tid];
    const int x = sh.tok[ch];
    if (x >= 0 && x < vocab) {
      cv = true;
      lp = (p_logits + (int64_t)(o + u) * ld)[x];
      if (!topk) lq = (q_logits + (int64_t)(o + u) * ld)[x];
    }
  }
  // (a leaf reaches here only with the LM head's partials, for its draw: its
  // target row alone)
  if (tid < ((topk || nk == 0) ? 1 : 2) &&
      !merged_ref_sum(ws, tid * R + o + u, sh.tab, sh.lse[tid][u]))
    sh.timeout = 1;
  __syncthreads();
  if (tid < nk) {
    sh.cp[ch] = cv ? exp_f64((double)lp * invT - sh.lse[0][u], sh.tab) : 0.0;
    if (!topk) sh.cq[ch] = cv ? exp_f64((double)lq * invT - sh.lse[1][u], sh.tab) : 0.0;
  }
  if (tid == 0) sh.ready[u] = 1;
  __syncthreads();
}

// Per-request walk state, kept in LDS and advanced by thread 0.
struct WalkState {
  int u;            // current node (local row)
  int kidx;         // next child of u to test (index into kid_list)
  double t, N;      // residual R = max(0, P_u - t Q_u) / N
  double pass_t;    // t of the weights the last pass left (-1: none at u)
  int action;       // 0: pass, 1: pass then draw, 2: draw from the last pass, 3: stop,
                    // 4: merge the statistics of node u (walks first)
  double act_t;     // t of the pass to run
  int act_q;        // whether the pass needs the draft row
};

// Thread 0: run sibling tests and moves until a vocabulary pass (or a draw)
// is needed.  Coins (sh.coin): purpose 0 for the accept test of child c,
// purpose 1 for the draw at the node where the walk stops.
SPEC_DEVICE void walk_decide(WalkShared& sh, WalkState& st, int path_stride, bool topk,
                             bool lazy, bool leafp) {
  while (true) {
    const int u = st.u;
    const int k0 = sh.kid_start[u], k1 = sh.kid_start[u + 1];
    if (k1 == k0) {                      // leaf: bonus token from P_u
      st.action = 1;
      st.act_t = 0.0;
      st.act_q = 0;
      return;
    }
    if (st.kidx >= k1 && topk) {         // every child rejected: P without the rejected tokens
      st.action = 1;
      st.act_t = 0.0;
      st.act_q = 0;
      return;
    }
    if (st.kidx >= k1) {                 // every child rejected: draw from the residual
      if (st.pass_t == st.t) {
        st.action = 2;
      } else {
        st.action = 1;
        st.act_t = st.t;
        st.act_q = 1;
      }
      return;
    }
    const int ch = sh.kid_list[st.kidx];
    const int x = sh.tok[ch];
    const double Px = sh.cp[ch], Qx = sh.cq[ch];
    const double r = sh.coin[0][ch];
    bool seen = false;                   // deterministic children: x rejected before has R(x) = 0
    if (topk)
      for (int k = 0; k < sh.nrej; ++k) seen |= (sh.rej[k] == x);
    const double Rx = topk ? (seen ? 0.0 : Px / st.N) : fmax(0.0, fma(-st.t, Qx, Px)) / st.N;
    if (topk ? (r < Rx) : (r * Qx < Rx)) {   // accept: move to the child
      if (sh.len >= path_stride) {
        sh.flags |= kFlagPathTruncated;
        st.action = 3;
        return;
      }
      sh.toks[sh.ntok++] = x;
      sh.path[sh.len++] = ch;
      st.u = ch;
      st.kidx = sh.kid_start[ch];
      st.t = 0.0;
      st.N = 1.0;
      st.pass_t = -1.0;
      sh.nrej = 0;
      if (lazy && !sh.ready[ch] && (leafp || sh.kid_start[ch + 1] > sh.kid_start[ch])) {
        st.action = 4;                   // merge the new node's statistics first
        return;
      }
      continue;
    }
    if (topk) {                          // reject: drop x from the residual
      st.kidx += 1;
      if (seen || Px == 0.0) continue;   // (out-of-range tokens have Px = 0)
      const double N2 = st.N - Px;
      if (N2 > 0.0) {
        st.N = N2;
        sh.rej[sh.nrej++] = x;
      } else {
        sh.flags |= kFlagZeroResidual;
      }
      continue;
    }
    // reject: the next residual needs G(t + N)
    st.action = 0;
    st.act_t = st.t + st.N;
    st.act_q = 1;
    return;
  }
}

// Statistics and walk in one launch.  kLazy = false: blocks [0, nstat) are
// statistics items (sample_stats_item), the B * S after them the walk's
// workgroups, which are dispatched as the statistics drain, take tickets and
// load their trees meanwhile; each then polls the partials of all its rows
// until they are published.  kLazy = true (walks first): blocks [0, B * S)
// are the walk's workgroups, all resident at once, each merging a node's
// partials when its walk reaches the node (node_stats); the statistics items
// follow in the order the walks need them.  Every wait is bounded: a request
// whose partials never arrive reports a timeout.
template <bool kLazy>
__global__ void __launch_bounds__(kWalkThreads, 4)
accept_sample_kernel(StatsArgs sa, int nstat, const int32_t* __restrict__ row_offsets, int B,
                     int R, int S, const int32_t* __restrict__ parents,
                     const int32_t* __restrict__ tokens, const float* __restrict__ p_logits,
                     const float* __restrict__ q_logits, int64_t ld, int vocab,
                     float temperature, uint64_t seed, uint64_t step, AcceptWs ws, WalkOut out,
                     int max_spins, HeadTiles ht) {
  __shared__ WalkShared sh;
  __shared__ WalkState st;
  if (kLazy ? (int)blockIdx.x >= B * S : (int)blockIdx.x < nstat) {
    sample_stats_item(sa, ws, (int)blockIdx.x - (kLazy ? B * S : 0), sh.tab, sh.red_m,
                      sh.wave_tot);
    return;
  }
  // (request, slice) by ticket, in the order the workgroups start running:
  // the lowest unfinished request then always has all its slices running
  // or next in line, so the per-request barriers make progress whenever S
  // workgroups fit on the device at once (no cooperative launch needed).
  // With the walks first, every walk workgroup is resident from the start
  // (B * S <= half the device), so the block id serves.
  __shared__ int s_ticket;
  if (threadIdx.x == 0)
    s_ticket = kLazy ? (int)blockIdx.x                      // every walk workgroup resident
               : (S == 1) ? (int)blockIdx.x - nstat
                          : __hip_atomic_fetch_add(ws.sync, 1, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const int b = s_ticket / S;
  const int slice = s_ticket % S;
  if (b < 0 || b >= B) return;                       // (not reached: B * S walk workgroups)
  const int o = row_offsets[b];
  const int n = row_offsets[b + 1] - o;
  const int tid = threadIdx.x;
  if (tid == 0) sh.timeout = 0;
  // Every coin the walk can use, drawn in parallel: purpose 0 for the accept
  // test of child row k, purpose 1 for the draw at node k.
  if (tid < n) {
    sh.coin[0][tid] = verify_uniform(seed, step, (uint64_t)b, (uint64_t)tid, 0);
    sh.coin[1][tid] = verify_uniform(seed, step, (uint64_t)b, (uint64_t)tid, 1);
  }
  load_tree(sh, parents, tokens, o, n, sh.tab);
  // This request's row statistics: each row's log-sum-exp from its chunk
  // partials (in chunk order), then each child's P_u(x_c), Q_u(x_c) in fp64;
  // `write`: slice 0 writes the fp32 outputs (NaN at roots and at rows whose
  // parent is invalid; Q is NaN everywhere without draft rows).  Thread k
  // takes row k's partials and child k's logit; all of them are loaded at
  // once (one memory round trip), the child logits are held in registers
  // until the parents' log-sum-exps are in LDS.  Walks that go first in the
  // grid merge node by node as they reach them instead (node_stats) and run
  // this at their end, for the outputs.
  const bool topk = q_logits == nullptr;
  const double invT = 1.0 / (double)temperature;
  constexpr bool lazy = kLazy;   // walks first in the grid (then sa.wfirst too)
  auto all_rows = [&](bool write) {
    constexpr int kRowsPerThread = 2 * kMaxRows / kWalkThreads;
    float clog[kRowsPerThread];
    bool cval[kRowsPerThread];
#pragma unroll
    for (int j = 0; j < kRowsPerThread; ++j) {
      const int k = tid + j * kWalkThreads;
      const int which = k >= n ? 1 : 0;
      const int i = k - which * n;
      cval[j] = false;
      clog[j] = 0.0f;
      if (k < 2 * n && !(which && topk)) {
        const int pu = sh.par[i];
        const int x = sh.tok[i];
        if (i > 0 && pu >= 0 && pu < i && x >= 0 && x < vocab) {
          cval[j] = true;
          clog[j] = ((which ? q_logits : p_logits) + (int64_t)(o + pu) * ld)[x];
        }
        // (rows of nodes with children only, and with the LM head every target
        // row: the others are not streamed)
        if (!sh.bad && ((!which && sa.leafp) || sh.kid_start[i + 1] > sh.kid_start[i]) &&
            !merged_ref_sum(ws, which * R + o + i, sh.tab, sh.lse[which][i]))
          sh.timeout = 1;
      }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kRowsPerThread; ++j) {
      const int k = tid + j * kWalkThreads;
      if (k >= 2 * n) continue;
      const int which = k >= n ? 1 : 0;
      const int i = k - which * n;
      float* dst = which ? out.child_q : out.child_p;
      const int pu = sh.par[i];
      double val = __longlong_as_double(0x7ff8000000000000LL);
      if (!sh.bad && i > 0 && pu >= 0 && pu < i && !(which && topk)) {   // (NaN: invalid tree)
        val = cval[j] ? exp_f64((double)clog[j] * invT - sh.lse[which][pu], sh.tab) : 0.0;
        (which ? sh.cq : sh.cp)[i] = val;
      }
      if (dst && write) dst[o + i] = (float)val;
    }
    __syncthreads();
  };
  if (!lazy || sh.bad) {
    all_rows(slice == 0);
  } else if constexpr (lazy) {
    if (tid < n) sh.ready[tid] = 0;
    __syncthreads();
    if (sa.leafp || sh.kid_start[1] > sh.kid_start[0])
      node_stats(sh, ws, R, o, 0, p_logits, q_logits, ld, vocab, invT, topk);
  }
  if (sh.bad) {
    if (slice == 0) write_abandoned(out, b, o, n, kFlagBadTree);
    return;
  }
  if (sh.timeout) {
    if (slice == 0) write_abandoned(out, b, o, n, kFlagSyncTimeout);
    return;
  }
  WalkCtx c;
  c.invT = invT;
  c.vocab = vocab;
  c.nseg = (vocab + kSeg - 1) / kSeg;
  const int per = (c.nseg + S - 1) / S;
  c.seg_lo = min(c.nseg, slice * per);
  c.seg_hi = min(c.nseg, c.seg_lo + per);
  c.slice = slice;
  c.S = S;
  c.max_spins = max_spins;
  c.seg = ws.seg + (size_t)b * 2 * c.nseg;
  c.rd_lo = 0;
  c.rd_n = c.nseg;
  if (tid == 0) {
    sh.len = 1;
    sh.ntok = 0;
    sh.flags = 0;
    sh.path[0] = 0;
    sh.nrej = 0;
    st.u = 0;
    st.kidx = sh.kid_start[0];
    st.t = 0.0;
    st.N = 1.0;
    st.pass_t = -1.0;
  }
  int pass = 0;
  int final_token = -1;
  while (true) {
    if (tid == 0)
      walk_decide(sh, st, out.path_stride, topk, lazy, sa.leafp != 0);
    __syncthreads();
    const int action = st.action;
    if (action == 3) break;
    if (lazy && action == 4) {
      node_stats(sh, ws, R, o, st.u, p_logits, q_logits, ld, vocab, invT, topk);
      if (sh.timeout) break;
      continue;
    }
    const int u = st.u;
    c.p = p_logits + (int64_t)(o + u) * ld;
    c.q = topk ? nullptr : q_logits + (int64_t)(o + u) * ld;
    c.lse_p = sh.lse[0][u];
    c.lse_q = st.act_q ? sh.lse[1][u] : 0.0;
    c.rej = sh.rej;
    c.nrej = topk ? sh.nrej : 0;
    const double act_t = st.act_t;
    const bool act_q = st.act_q != 0;
    if (action == 1 && !act_q && !sa.leafp && sh.kid_start[u + 1] == sh.kid_start[u]) {
      // a leaf, whose target row was not streamed: a self-normalised pass
      c.lse_p = leaf_pass(sh, c, ++pass, ws.sref + (size_t)b * 2 * kMaxSlices);
      if (sh.timeout) break;
      final_token = walk_draw(sh, c, 0.0, false, sh.coin[1][u] * sh.total);
      break;
    }
    if (action == 1 && !act_q && ht.hidden && sh.kid_start[u + 1] == sh.kid_start[u]) {
      // a leaf on the LM-head path: its logits were not stored
      final_token = head_leaf_draw(sh, c, ws, ht, o + u, b, pass_tag(++pass), sh.coin[1][u]);
      break;
    }
    if (action == 1 && !act_q) {                     // a draw from P_u alone
      if ((tid >> 6) == 0) locate_chunk(sh, ws, c, o + u, sh.coin[1][u]);
      __syncthreads();
      const int ck = sh.chunk;
      if (ck >= 0) {
        const int a0 = ck * kSegsPerChunk, a1 = min(c.nseg, a0 + kSegsPerChunk);
        const int per = (a1 - a0 + S - 1) / S;
        c.seg_lo = min(a1, a0 + slice * per);
        c.seg_hi = min(a1, c.seg_lo + per);
        c.rd_lo = a0;
        c.rd_n = a1 - a0;
        walk_pass(sh, c, ++pass, 0.0, false);
        if (sh.timeout) break;
        final_token = walk_draw(sh, c, 0.0, false, sh.chunk_target - sh.chunk_base);
        break;
      }
    }
    if (action != 2) {
      const double G = walk_pass(sh, c, ++pass, act_t, act_q);
      if (sh.timeout) break;
      if (action == 0) {
        if (tid == 0) {
          st.pass_t = act_t;
          if (G > 0.0) {
            st.t = act_t;
            st.N = G;
          } else {
            sh.flags |= kFlagZeroResidual;
          }
          st.kidx += 1;
        }
        __syncthreads();
        continue;
      }
    }
    // draw from the weights the last pass left
    const double r = sh.coin[1][u];
    const double dt = (action == 2) ? st.pass_t : act_t;
    const bool dq = (action == 2) ? true : act_q;
    final_token = walk_draw(sh, c, dt, dq, r * sh.total);
    break;
  }
  // Only slice 0 writes: it passed every barrier of the walk (then every sum
  // it read was complete, whatever the other slices did afterwards) or it
  // gave up at one (then the request reports the timeout).
  if (slice != 0) return;
  __syncthreads();
  if (lazy && !sh.timeout) all_rows(true);     // every child's probabilities, for the outputs
  if (sh.timeout) {
    write_abandoned(out, b, o, n, sh.flags | kFlagSyncTimeout);
    return;
  }
  if (tid == 0 && !(sh.flags & kFlagPathTruncated)) sh.toks[sh.ntok++] = final_token;
  __syncthreads();
  write_outputs(sh, out, b, o, n, -1);
}

// Greedy (temperature 0): one workgroup per request, decisions by thread 0.
__global__ void __launch_bounds__(kWalkThreads)
accept_greedy_kernel(const int32_t* __restrict__ row_offsets, const int32_t* __restrict__ parents,
                     const int32_t* __restrict__ tokens, AcceptWs ws, WalkOut out) {
  __shared__ WalkShared sh;
  const int b = blockIdx.x;
  const int o = row_offsets[b];
  const int n = row_offsets[b + 1] - o;
  load_tree(sh, parents, tokens, o, n);
  if (sh.bad) {
    write_abandoned(out, b, o, n, kFlagBadTree);
    return;
  }
  if (threadIdx.x == 0) {
    int u = 0, len = 1, nt = 0, flags = 0;
    sh.path[0] = 0;
    while (true) {
      const int g = ws.am[o + u];
      int nxt = -1;
      for (int k = sh.kid_start[u]; k < sh.kid_start[u + 1]; ++k)
        if (sh.tok[sh.kid_list[k]] == g) {
          nxt = sh.kid_list[k];
          break;
        }
      if (nxt >= 0 && len >= out.path_stride) {
        flags |= kFlagPathTruncated;
        break;
      }
      sh.toks[nt++] = g;
      if (nxt < 0) break;
      sh.path[len++] = nxt;
      u = nxt;
    }
    sh.len = len;
    sh.ntok = nt;
    sh.flags = flags;
  }
  __syncthreads();
  write_outputs(sh, out, b, o, n, -1);
}

// Workspace of the no-allocation acceptance entry point: a file-scope device
// array (each GPU the library runs on holds its own copy until the process
// ends).  Host code never uses the array's name as an address: its device
// address is looked up once per device with hipGetSymbolAddress, with that
// device current, and kept.  Every call on a device shares its copy; the
// statistics kernel clears the counters that must start at zero, and every
// other byte is written before it is read, so stale contents do not matter,
// but calls that overlap on one device race.
static __device__ __align__(256) unsigned char scratch[kAcceptScratchBytes];

hipError_t accept_scratch(void** ptr) {
  static std::atomic<void*> addr[kMaxDevices];
  static std::mutex lock;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = addr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> g(lock);
    p = addr[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (!p) return hipErrorInvalidSymbol;
      addr[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return hipSuccess;
}

// The fp64 exponentials every decision rests on, evaluated element by element
// for tests: variant 0 exp_f64, 1 exp_f64_clamped, 2 exp_f64_stream; 3 and 4
// the first two evaluated two at a time (elements 2k and 2k + 1 together).
__global__ void __launch_bounds__(256)
exp64_probe_kernel(const double* __restrict__ x, double* __restrict__ y, int64_t n, int variant) {
  __shared__ double tab[256];
  load_exp_table(tab);
  __syncthreads();
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const double v = x[i];
  if (variant >= 3) {
    const int64_t j = (i ^ 1) < n ? (i ^ 1) : i;     // the pair's other element
    const double a = (i & 1) ? x[j] : v, b = (i & 1) ? v : x[j];
    double ya, yb;
    if (variant == 3)
      exp_f64_2(a, b, tab, ya, yb);
    else
      exp_f64_clamped2(a, b, tab, ya, yb);
    y[i] = (i & 1) ? yb : ya;
    return;
  }
  y[i] = (variant == 0) ? exp_f64(v, tab) : (variant == 1) ? exp_f64_clamped(v, tab)
                                                            : exp_f64_stream(v, tab);
}

hipError_t launch_exp64_probe(const double* x, double* y, int64_t n, int variant,
                              hipStream_t stream) {
  hipLaunchKernelGGL(exp64_probe_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                     x, y, n, variant);
  return hipGetLastError();
}

// Walk workgroups that fit on device `dev` at once (CUs x occupancy),
// queried once per device.
static hipError_t walk_capacity(int dev, int* capacity) {
  static std::atomic<int> cached[kMaxDevices];
  if (dev >= 0 && dev < kMaxDevices) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) {
      *capacity = c;
      return hipSuccess;
    }
  }
  int cus = 0, per_cu = 0;
  hipError_t e;
  if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess)
    return e;
  int per_cu_lazy = 0;
  if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, accept_sample_kernel<false>,
                                                        kWalkThreads, 0)) != hipSuccess ||
      (e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu_lazy, accept_sample_kernel<true>,
                                                        kWalkThreads, 0)) != hipSuccess)
    return e;
  *capacity = cus * std::min(per_cu, per_cu_lazy);
  if (dev >= 0 && dev < kMaxDevices) cached[dev].store(*capacity, std::memory_order_relaxed);
  return hipSuccess;
}

int walk_slices(int B, int vocab, int capacity_blocks) {
  const int nseg = segs_for(vocab);
  int S = capacity_blocks / (B > 0 ? B : 1);
  const int want = nseg;                       // at least one segment per slice
  if (S > want) S = want;
  if (S > kMaxSlices) S = kMaxSlices;
  if (S < 1) S = 1;
  return S;
}

constexpr int kWalkFirstMinBatch = 8;    // requests from which the walks go first in the grid

hipError_t launch_accept(const LaunchCtx& cx, int R, const int32_t* parents, const int32_t* tokens,
                         const float* p_logits, const float* q_logits, int64_t ld, int vocab,
                         float temperature, uint64_t seed, uint64_t step, int path_stride,
                         int32_t* accept_len, int32_t* path, int32_t* tokens_out,
                         uint8_t* accept_mask, float* child_p, float* child_q, int32_t* flags,
                         void* workspace, WalkKnobs walk, const HeadTiles* head) {
  static_assert(sizeof(WalkShared) + sizeof(WalkState) <= 160 * 1024 / 4,
                "walk LDS: four workgroups per CU (160 KB of LDS)");
  static_assert(kStatThreads == kWalkThreads, "statistics items run in walk-sized workgroups");
  static_assert(kWalkThreads >= kMaxRows && kWalkThreads >= 256, "load_tree: a thread per row and table entry");
  AcceptWs ws = accept_ws(workspace, R, cx.B, vocab);
  const int nch = ws.nch;
  const bool greedy = temperature == 0.0f;
  // q_logits == nullptr at T > 0: deterministic children, target rows only.
  // With the LM head's partials, the target rows are merged, not streamed.
  hipError_t e;
  int nstat = 0;
  StatsArgs stats_args{p_logits, q_logits, ld, vocab, R, 0, 0, head ? 1 : 0, 0,
                       1.0 / (double)temperature};
  if (!greedy && (!head || q_logits)) {
    stats_args.np = head ? 0 : R;
    stats_args.nq = q_logits ? R : 0;
    nstat = (stats_args.np + stats_args.nq) * nch;
  }
  int S = 1;
  if (!greedy) {
    int dev = 0;
    if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
    int capacity = 0;
    if ((e = walk_capacity(dev, &capacity)) != hipSuccess) return e;
    S = walk_slices(cx.B, vocab, capacity);
    // Walks first in the grid (batches of kWalkFirstMinBatch requests or
    // more): the walk workgroups load their trees and take each node's
    // statistics as they reach it (node_stats), while the statistics stream
    // behind them in the order walks need them (every root first), so the
    // walks' set-ups and root decisions overlap the streaming.  They hold at
    // most half of the device, so every walk workgroup is resident at once
    // (no tickets) and the statistics keep the other half.
    if (nstat > 0 && cx.B >= kWalkFirstMinBatch && cx.B <= capacity / 2 &&
        walk.max_slices <= 0) {
      stats_args.wfirst = 1;
      S = walk_slices(cx.B, vocab, capacity / 2);
    }
    if (walk.max_slices > 0) S = walk.max_slices < S ? walk.max_slices : S;
    // the rows to stream (and the walk's exchange area cleared)
    const int64_t nseg_all = (int64_t)cx.B * 2 * segs_for(vocab);
    const int clear_blocks =
        (int)std::max<int64_t>(1, std::min<int64_t>(256, (nseg_all + kPrepThreads - 1) / kPrepThreads));
    hipLaunchKernelGGL(accept_prep_kernel, dim3(1 + clear_blocks), dim3(kPrepThreads), 0,
                       cx.stream, cx.row_offsets_d, cx.B, R, parents, ws, vocab, head ? 0 : 1,
                       q_logits ? 1 : 0, stats_args.wfirst);
  }
  if (head)
    hipLaunchKernelGGL(accept_head_merge_kernel, dim3((R * nch + 3) / 4), dim3(256), 0,
                       cx.stream, cx.B, R, *head, greedy ? 1 : 0, ws, vocab);
  if (greedy && !head)
    hipLaunchKernelGGL(accept_argmax_kernel, dim3(R * nch), dim3(kStatThreads), 0, cx.stream,
                       p_logits, ld, vocab, ws);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  WalkOut out{accept_len, path, tokens_out, accept_mask, flags, path_stride, child_p, child_q};
  if (temperature == 0.0f) {
    hipLaunchKernelGGL(accept_finalize_kernel, dim3((R + 255) / 256), dim3(256), 0, cx.stream,
                       cx.row_offsets_d, cx.B, R, parents, tokens, ws, child_p);
    hipLaunchKernelGGL(accept_greedy_kernel, dim3(cx.B), dim3(kWalkThreads), 0, cx.stream,
                       cx.row_offsets_d, parents, tokens, ws, out);
    return hipGetLastError();
  }
  const int max_spins = walk.max_spins >= 0 ? walk.max_spins : kWalkMaxSpins;
  // nstat statistics items and B * S walk workgroups: the walks after the
  // statistics, taking tickets (see the kernel), or first in the grid.
  HeadTiles ht{};
  if (head) ht = *head;     // ht.hidden == nullptr: no LM head (every leaf draw reads its row)
  if (stats_args.wfirst)
    hipLaunchKernelGGL(accept_sample_kernel<true>, dim3(nstat + cx.B * S), dim3(kWalkThreads), 0,
                       cx.stream, stats_args, nstat, cx.row_offsets_d, cx.B, R, S, parents,
                       tokens, p_logits, q_logits, ld, vocab, temperature, seed, step, ws, out,
                       max_spins, ht);
  else
    hipLaunchKernelGGL(accept_sample_kernel<false>, dim3(nstat + cx.B * S), dim3(kWalkThreads), 0,
                       cx.stream, stats_args, nstat, cx.row_offsets_d, cx.B, R, S, parents,
                       tokens, p_logits, q_logits, ld, vocab, temperature, seed, step, ws, out,
                       max_spins, ht);
  return hipGetLastError();
}

}  // namespace spec
