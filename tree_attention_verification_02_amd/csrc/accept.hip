// Lossless speculative acceptance over a draft tree.
//
// Pages: CSDN "推理加速：推测解码与级联推理" sections 7.1-7.2 (accept with
// probability min(1, p/q); on rejection draw from norm(max(0, p - q)); the
// emitted length counts the final token); guijiagi.com speculative-decoding
// post, rejection-sampling section (first rejection ends the step);
// cnblogs "投机推理算法的常见优化手段", tree-mask section (row i's target
// distribution predicts i's children; every level of the tree is checked).
//
// Two kernels:
//  * accept_stats: one workgroup per (row, {target, draft}) streams the
//    vocabulary row once with 16-byte loads and keeps, per thread, the
//    running max, the sum of exp((x - max)/T) in fp64 and the first argmax;
//    workgroup reduction, then the child probabilities P_u(x_c), Q_u(x_c) of
//    that row's children are gathered in fp64.  Draft rows of leaves are
//    never read.
//  * accept_walk: one workgroup per request runs the sequential walk.  The
//    sibling tests are scalar fp64; each rejection needs the residual mass
//    Z = sum max(0, R - Q), and each final draw an inverse CDF, both as
//    vocabulary passes in which every wave reduces a contiguous 256-element
//    segment; ordered fp64 segment sums make the draw a two-level search
//    (segment, then element) that re-reads one segment.
#include <math.h>

#include "common.hpp"
#include "launch.hpp"
#include "philox.hpp"

namespace spec {

constexpr int kStatThreads = 512;
constexpr int kWalkThreads = 1024;
constexpr int kWalkWaves = kWalkThreads / 64;
constexpr int kTileElems = kWalkThreads * 4;           // elements per walk tile
constexpr int kMaxSegs = 4096;                          // vocab <= 2^20

struct AcceptWs {
  double* s;      // [2][R] sum of exp((x - m)/T)
  float* m;       // [2][R] row max of the raw logits
  int32_t* am;    // [R] argmax of the target row
};

__host__ __device__ inline AcceptWs accept_ws(void* base, int R) {
  AcceptWs w;
  w.s = (double*)base;
  w.m = (float*)(w.s + 2 * (size_t)R);
  w.am = (int32_t*)(w.m + 2 * (size_t)R);
  return w;
}

size_t accept_workspace_bytes(int R, int B) {
  (void)B;
  return 2 * (size_t)R * sizeof(double) + 2 * (size_t)R * sizeof(float) +
         (size_t)R * sizeof(int32_t) + 256;
}

// (max, sum, argmax) triple merge; sums are relative to their own max.
SPEC_DEVICE void merge_stat(float& m, double& s, int& am, float m2, double s2, int am2, float invT) {
  const float M = fmaxf(m, m2);
  if (M == -INFINITY) {
    am = (am < 0) ? am2 : (am2 < 0 ? am : min(am, am2));
    return;
  }
  const double w1 = (m == -INFINITY) ? 0.0 : exp((double)(m - M) * (double)invT);
  const double w2 = (m2 == -INFINITY) ? 0.0 : exp((double)(m2 - M) * (double)invT);
  int a;
  if (m > m2) a = am;
  else if (m2 > m) a = am2;
  else a = (am < 0) ? am2 : (am2 < 0 ? am : min(am, am2));
  s = s * w1 + s2 * w2;
  m = M;
  am = a;
}

__global__ void __launch_bounds__(kStatThreads)
accept_stats_kernel(const int32_t* __restrict__ row_offsets, int B, int R,
                    const int32_t* __restrict__ parents, const int32_t* __restrict__ tokens,
                    const float* __restrict__ p_logits, const float* __restrict__ q_logits,
                    int64_t ld, int vocab, float temperature, AcceptWs ws,
                    float* __restrict__ child_p, float* __restrict__ child_q) {
  __shared__ float red_m[kStatThreads / 64];
  __shared__ double red_s[kStatThreads / 64];
  __shared__ int red_a[kStatThreads / 64];
  __shared__ int has_kids;
  const int which = blockIdx.x >= R ? 1 : 0;          // 0: target p, 1: draft q
  const int r = blockIdx.x - which * R;
  const int b = request_of_row(row_offsets, B, r);
  const int o = row_offsets[b];
  const int n = row_offsets[b + 1] - o;
  const int u = r - o;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool greedy = temperature == 0.0f;
  if (which == 1) {
    if (tid == 0) has_kids = 0;
    __syncthreads();
    for (int i = tid; i < n; i += kStatThreads)
      if (i > 0 && parents[o + i] == u) has_kids = 1;
    __syncthreads();
    if (!has_kids) return;
  }
  const float invT = greedy ? 1.0f : 1.0f / temperature;
  const float* row = (which ? q_logits : p_logits) + (int64_t)r * ld;
  const float4* row4 = reinterpret_cast<const float4*>(row);
  const int v4 = (vocab + 3) >> 2;

  float m = -INFINITY;
  double s = 0.0;
  int am = -1;
  constexpr int U = 4;
  for (int f0 = tid; f0 < v4; f0 += kStatThreads * U) {
    float4 x[U];
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const int f = f0 + k * kStatThreads;
      x[k] = (f < v4) ? row4[f] : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
    }
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const int y0 = (f0 + k * kStatThreads) * 4;
      const float xs[4] = {x[k].x, x[k].y, x[k].z, x[k].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float xv = (y0 + j < vocab) ? xs[j] : -INFINITY;
        if (xv > m) {
          if (!greedy) s = (m == -INFINITY) ? 0.0 : s * exp((double)(m - xv) * (double)invT);
          m = xv;
          am = y0 + j;
        }
        if (!greedy && xv != -INFINITY) s += (double)expf((xv - m) * invT);
      }
    }
  }
  // wave then workgroup reduction
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const float m2 = __shfl_xor(m, off, 64);
    const double s2 = __shfl_xor(s, off, 64);
    const int a2 = __shfl_xor(am, off, 64);
    merge_stat(m, s, am, m2, s2, a2, invT);
  }
  if (lane == 0) {
    red_m[wave] = m;
    red_s[wave] = s;
    red_a[wave] = am;
  }
  __syncthreads();
  if (wave == 0) {
    m = (lane < kStatThreads / 64) ? red_m[lane] : -INFINITY;
    s = (lane < kStatThreads / 64) ? red_s[lane] : 0.0;
    am = (lane < kStatThreads / 64) ? red_a[lane] : -1;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const float m2 = __shfl_xor(m, off, 64);
      const double s2 = __shfl_xor(s, off, 64);
      const int a2 = __shfl_xor(am, off, 64);
      merge_stat(m, s, am, m2, s2, a2, invT);
    }
    if (lane == 0) {
      ws.m[which * R + r] = m;
      ws.s[which * R + r] = s;
      if (which == 0) ws.am[r] = am;
      red_m[0] = m;
      red_s[0] = s;
      red_a[0] = am;
    }
  }
  __syncthreads();
  m = red_m[0];
  s = red_s[0];
  am = red_a[0];
  float* dst = which ? child_q : child_p;
  if (dst == nullptr || (which == 1 && greedy)) return;
  if (which == 0 && u == 0 && tid == 0) {                          // root: no draft
    if (child_p) child_p[o] = __int_as_float(0x7fc00000);
    if (child_q && !greedy) child_q[o] = __int_as_float(0x7fc00000);
  }
  for (int i = tid; i < n; i += kStatThreads) {
    if (i > 0 && parents[o + i] == u) {
      const int x = tokens[o + i];
      float val;
      if (greedy) {
        val = (x == am) ? 1.0f : 0.0f;
      } else {
        const float lx = (x >= 0 && x < vocab) ? row[x] : -INFINITY;
        val = (float)(exp(((double)lx - (double)m) * (double)invT) / s);
      }
      dst[o + i] = val;
    }
  }
}

// ---------------------------------------------------------------------------
// Walk.

struct WalkRow {
  const float* p;
  const float* q;
  float mp, mq, invT;
  double inv_sp, inv_sq;
};

// Weight of vocabulary entry y after `nres` residual steps.  final_res
// selects max(0, R - Q) (the next residual's mass) instead of R itself.
SPEC_DEVICE double walk_weight(const WalkRow& w, float py, float qy, int nres, const double* zinv,
                               bool final_res) {
  double R = (double)expf((py - w.mp) * w.invT) * w.inv_sp;
  if (nres == 0 && !final_res) return R;
  const double Q = (double)expf((qy - w.mq) * w.invT) * w.inv_sq;
  for (int i = 0; i < nres; ++i) {
    const double rn = fmax(0.0, R - Q);
    R = (zinv[i] > 0.0) ? rn * zinv[i] : R;
  }
  return final_res ? fmax(0.0, R - Q) : R;
}

// Inclusive wave scan (Hillis-Steele) of doubles.
SPEC_DEVICE double wave_incl_scan(double v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double t = __shfl_up(v, o, 64);
    if (lane >= o) v += t;
  }
  return v;
}

struct WalkShared {
  int par[kMaxRows];
  int tok[kMaxRows];
  int kid_start[kMaxRows + 1];
  int kid_list[kMaxRows];
  double seg[kMaxSegs];
  double zinv[kMaxRows];
  double lane_excl[64];
  int last_pos;
  int bad;
  // broadcast slots
  double total;
  double c0;
  int found_seg;
  int pick;
};

// One vocabulary pass: fills seg[] with the ordered segment sums of the
// weights and returns their total (the last inclusive prefix).
SPEC_DEVICE double walk_pass(WalkShared& sh, const WalkRow& w, int vocab, int nres, bool final_res,
                             bool need_q) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ntiles = (vocab + kTileElems - 1) / kTileElems;
  const float4* p4 = reinterpret_cast<const float4*>(w.p);
  const float4* q4 = reinterpret_cast<const float4*>(w.q);
  int last = -1;
  constexpr int U = 2;
  for (int t0 = 0; t0 < ntiles; t0 += U) {
    float4 pv[U], qv[U];
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const int y0 = (t0 + k) * kTileElems + 4 * tid;
      const bool in = (t0 + k < ntiles) && y0 < vocab;
      pv[k] = in ? p4[y0 >> 2] : make_float4(0.f, 0.f, 0.f, 0.f);
      qv[k] = (in && need_q) ? q4[y0 >> 2] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int k = 0; k < U; ++k) {
      if (t0 + k >= ntiles) break;
      const int y0 = (t0 + k) * kTileElems + 4 * tid;
      const float pa[4] = {pv[k].x, pv[k].y, pv[k].z, pv[k].w};
      const float qa[4] = {qv[k].x, qv[k].y, qv[k].z, qv[k].w};
      double acc = 0.0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (y0 + j < vocab) {
          const double wt = walk_weight(w, pa[j], qa[j], nres, sh.zinv, final_res);
          acc += wt;
          if (wt > 0.0) last = y0 + j;
        }
      }
      const double incl = wave_incl_scan(acc, lane);
      if (lane == 63) sh.seg[(t0 + k) * kWalkWaves + wave] = incl;
    }
  }
  // last index with positive weight (fallback of the inverse CDF)
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) last = max(last, __shfl_xor(last, o, 64));
  if (lane == 0) atomicMax(&sh.last_pos, last);
  __syncthreads();
  if (wave == 0) {
    const int nseg = ntiles * kWalkWaves;
    const int per = (nseg + 63) / 64;
    double part = 0.0;
    for (int k = 0; k < per; ++k) {
      const int sidx = lane * per + k;
      if (sidx < nseg) part += sh.seg[sidx];
    }
    const double incl = wave_incl_scan(part, lane);
    if (lane == 63) sh.total = incl;
    sh.lane_excl[lane] = incl - part;
  }
  __syncthreads();
  return sh.total;
}

// Draw from the weights of the last pass with coin r; returns the index.
SPEC_DEVICE int walk_draw(WalkShared& sh, const WalkRow& w, int vocab, int nres, bool final_res,
                          bool need_q, double r) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ntiles = (vocab + kTileElems - 1) / kTileElems;
  const int nseg = ntiles * kWalkWaves;
  const double target = r * sh.total;
  if (wave == 0) {
    const int per = (nseg + 63) / 64;
    double cum = sh.lane_excl[lane];
    int hit_seg = -1;
    double hit_c0 = 0.0;
    for (int k = 0; k < per; ++k) {
      const int sidx = lane * per + k;
      if (sidx < nseg) {
        const double nxt = cum + sh.seg[sidx];
        if (hit_seg < 0 && nxt > target) {
          hit_seg = sidx;
          hit_c0 = cum;
        }
        cum = nxt;
      }
    }
    const uint64_t ball = __ballot(hit_seg >= 0);
    if (lane == 0) {
      sh.found_seg = -1;
      sh.pick = -1;
    }
    if (ball) {
      const int first = __ffsll((long long)ball) - 1;
      if (lane == first) {
        sh.found_seg = hit_seg;
        sh.c0 = hit_c0;
      }
    }
  }
  __syncthreads();
  const int fs = sh.found_seg;
  if (fs >= 0 && wave == 0) {
    const int tile = fs / kWalkWaves, wv = fs % kWalkWaves;
    const int y0 = tile * kTileElems + wv * 256 + 4 * lane;
    float pa[4] = {0.f, 0.f, 0.f, 0.f}, qa[4] = {0.f, 0.f, 0.f, 0.f};
    double wt[4] = {0.0, 0.0, 0.0, 0.0};
    double acc = 0.0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (y0 + j < vocab) {
        pa[j] = w.p[y0 + j];
        if (need_q) qa[j] = w.q[y0 + j];
        wt[j] = walk_weight(w, pa[j], qa[j], nres, sh.zinv, final_res);
        acc += wt[j];
      }
    }
    const double incl = wave_incl_scan(acc, lane);
    const double base = sh.c0;
    const uint64_t ball = __ballot(base + incl > target);
    if (ball) {
      const int first = __ffsll((long long)ball) - 1;
      if (lane == first) {
        double c = base + (incl - acc);
        int pick = -1, lastpos = -1;
        for (int j = 0; j < 4; ++j) {
          if (y0 + j >= vocab) break;
          if (wt[j] > 0.0) lastpos = y0 + j;
          c += wt[j];
          if (c > target) { pick = y0 + j; break; }
        }
        sh.pick = (pick >= 0) ? pick : lastpos;
      }
    }
  }
  __syncthreads();
  int pick = sh.pick;
  if (pick < 0) pick = sh.last_pos;     // rounding left no crossing: last positive weight
  return pick;
}

__global__ void __launch_bounds__(kWalkThreads)
accept_walk_kernel(const int32_t* __restrict__ row_offsets, int R,
                   const int32_t* __restrict__ parents, const int32_t* __restrict__ tokens,
                   const float* __restrict__ p_logits, const float* __restrict__ q_logits,
                   int64_t ld, int vocab, float temperature, uint64_t seed, uint64_t step,
                   int path_stride, AcceptWs ws, int32_t* __restrict__ accept_len,
                   int32_t* __restrict__ path, int32_t* __restrict__ tokens_out,
                   uint8_t* __restrict__ accept_mask, int32_t* __restrict__ flags) {
  __shared__ WalkShared sh;
  __shared__ int s_u, s_done, s_len, s_flags, s_child;
  __shared__ int s_path[kMaxRows];
  __shared__ int s_toks[kMaxRows + 1];
  const int b = blockIdx.x;
  const int o = row_offsets[b];
  const int n = row_offsets[b + 1] - o;
  const int tid = threadIdx.x;
  const bool greedy = temperature == 0.0f;
  const float invT = greedy ? 1.0f : 1.0f / temperature;

  if (tid == 0) sh.bad = 0;
  __syncthreads();
  if (tid < n) {
    sh.par[tid] = parents[o + tid];
    sh.tok[tid] = tokens[o + tid];
    const int p = sh.par[tid];
    const bool ok = (tid == 0) ? (p == -1) : (p >= 0 && p < tid);
    if (!ok) sh.bad = 1;
  }
  __syncthreads();
  if (sh.bad) {
    for (int k = tid; k < path_stride; k += kWalkThreads) {
      path[(int64_t)b * path_stride + k] = -1;
      tokens_out[(int64_t)b * path_stride + k] = -1;
    }
    if (accept_mask)
      for (int i = tid; i < n; i += kWalkThreads) accept_mask[o + i] = 0;
    if (tid == 0) {
      accept_len[b] = -1;
      if (flags) flags[b] = kFlagBadTree;
    }
    return;
  }
  // children lists in ascending row order
  if (tid < n) {
    int c = 0;
    for (int i = tid + 1; i < n; ++i) c += (sh.par[i] == tid);
    sh.kid_start[tid + 1] = c;
  }
  __syncthreads();
  if (tid == 0) {
    sh.kid_start[0] = 0;
    for (int i = 1; i <= n; ++i) sh.kid_start[i] += sh.kid_start[i - 1];
    s_u = 0;
    s_done = 0;
    s_len = 1;
    s_flags = 0;
    s_path[0] = 0;
  }
  __syncthreads();
  if (tid < n) {
    int pos = sh.kid_start[tid];
    for (int i = tid + 1; i < n; ++i)
      if (sh.par[i] == tid) sh.kid_list[pos++] = i;
  }
  __syncthreads();

  int ntok = 0;   // tokens emitted (thread 0's copy is authoritative)
  while (true) {
    const int u = s_u;
    const int k0 = sh.kid_start[u], k1 = sh.kid_start[u + 1];
    if (greedy) {
      if (tid == 0) {
        const int g = ws.am[o + u];
        int nxt = -1;
        for (int k = k0; k < k1; ++k)
          if (sh.tok[sh.kid_list[k]] == g) { nxt = sh.kid_list[k]; break; }
        if (nxt >= 0 && s_len >= path_stride) {
          s_flags |= kFlagPathTruncated;
          s_done = 1;
        } else {
          s_toks[ntok++] = g;
          if (nxt >= 0) {
            s_path[s_len++] = nxt;
            s_u = nxt;
          } else {
            s_done = 1;
          }
        }
      }
      __syncthreads();
      if (s_done) break;
      continue;
    }
    // sampling walk at node u
    WalkRow w;
    w.p = p_logits + (int64_t)(o + u) * ld;
    w.q = q_logits ? q_logits + (int64_t)(o + u) * ld : nullptr;
    w.invT = invT;
    w.mp = ws.m[o + u];
    w.inv_sp = 1.0 / ws.s[o + u];
    const bool leaf = (k1 == k0);
    if (leaf) {
      w.mq = 0.f;
      w.inv_sq = 0.0;
      if (tid == 0) sh.last_pos = -1;
      __syncthreads();
      walk_pass(sh, w, vocab, 0, false, false);
      const double r = verify_uniform(seed, step, (uint64_t)b, (uint64_t)u, 1);
      const int t = walk_draw(sh, w, vocab, 0, false, false, r);
      if (tid == 0) s_toks[ntok++] = t;
      break;
    }
    w.mq = ws.m[R + o + u];
    w.inv_sq = 1.0 / ws.s[R + o + u];
    int nres = 0;
    bool moved = false;
    for (int k = k0; k < k1; ++k) {
      const int c = sh.kid_list[k];
      if (tid == 0) {
        const int x = sh.tok[c];
        const double r = verify_uniform(seed, step, (uint64_t)b, (uint64_t)c, 0);
        double Px = 0.0, Qx = 0.0;
        if (x >= 0 && x < vocab) {
          Px = exp(((double)w.p[x] - (double)w.mp) * (double)invT) * w.inv_sp;
          Qx = exp(((double)w.q[x] - (double)w.mq) * (double)invT) * w.inv_sq;
        }
        double Rx = Px;
        for (int i = 0; i < nres; ++i) {
          const double rn = fmax(0.0, Rx - Qx);
          Rx = (sh.zinv[i] > 0.0) ? rn * sh.zinv[i] : Rx;
        }
        s_child = (r * Qx < Rx) ? 1 : 0;
        if (s_child && s_len >= path_stride) {
          s_flags |= kFlagPathTruncated;
          s_done = 1;
          s_child = 0;
        }
      }
      __syncthreads();
      if (s_done) break;
      if (s_child) {
        if (tid == 0) {
          s_toks[ntok++] = sh.tok[c];
          s_path[s_len++] = c;
          s_u = c;
        }
        moved = true;
        __syncthreads();
        break;
      }
      // rejected: residual mass for the next sibling (or the final draw)
      if (tid == 0) sh.last_pos = -1;
      __syncthreads();
      const double Z = walk_pass(sh, w, vocab, nres, true, true);
      if (tid == 0) {
        sh.zinv[nres] = (Z > 0.0) ? 1.0 / Z : 0.0;
        if (!(Z > 0.0)) s_flags |= kFlagZeroResidual;
      }
      __syncthreads();
      ++nres;
    }
    if (s_done) break;
    if (moved) continue;
    // every child rejected: draw from the current residual R_nres
    const double r = verify_uniform(seed, step, (uint64_t)b, (uint64_t)u, 1);
    int t;
    if (sh.zinv[nres - 1] > 0.0) {
      // weights max(0, R_{nres-1} - Q) of the last pass are R_nres unnormalised
      t = walk_draw(sh, w, vocab, nres - 1, true, true, r);
    } else {
      if (tid == 0) sh.last_pos = -1;
      __syncthreads();
      walk_pass(sh, w, vocab, nres, false, true);
      t = walk_draw(sh, w, vocab, nres, false, true, r);
    }
    if (tid == 0) s_toks[ntok++] = t;
    break;
  }
  __syncthreads();
  // outputs
  if (tid == 0) {
    accept_len[b] = s_len - 1;
    if (flags) flags[b] = s_flags;
    const int nt = s_len - 1 + ((s_flags & kFlagPathTruncated) ? 0 : 1);
    s_child = nt;   // reuse as token count broadcast
  }
  __syncthreads();
  const int len = s_len;
  const int nt = s_child;
  for (int k = tid; k < path_stride; k += kWalkThreads) {
    path[(int64_t)b * path_stride + k] = (k < len) ? s_path[k] : -1;
    tokens_out[(int64_t)b * path_stride + k] = (k < nt) ? s_toks[k] : -1;
  }
  if (accept_mask) {
    for (int i = tid; i < n; i += kWalkThreads) accept_mask[o + i] = 0;
    __syncthreads();
    for (int k = tid; k < len; k += kWalkThreads) accept_mask[o + s_path[k]] = 1;
  }
}

hipError_t launch_accept(const LaunchCtx& cx, int R, const int32_t* parents, const int32_t* tokens,
                         const float* p_logits, const float* q_logits, int64_t ld, int vocab,
                         float temperature, uint64_t seed, uint64_t step, int path_stride,
                         int32_t* accept_len, int32_t* path, int32_t* tokens_out,
                         uint8_t* accept_mask, float* child_p, float* child_q, int32_t* flags,
                         void* workspace) {
  AcceptWs ws = accept_ws(workspace, R);
  const int nblk = (temperature == 0.0f) ? R : 2 * R;
  hipLaunchKernelGGL(accept_stats_kernel, dim3(nblk), dim3(kStatThreads), 0, cx.stream,
                     cx.row_offsets_d, cx.B, R, parents, tokens, p_logits, q_logits, ld, vocab,
                     temperature, ws, child_p, child_q);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(accept_walk_kernel, dim3(cx.B), dim3(kWalkThreads), 0, cx.stream,
                     cx.row_offsets_d, R, parents, tokens, p_logits, q_logits, ld, vocab,
                     temperature, seed, step, path_stride, ws, accept_len, path, tokens_out,
                     accept_mask, flags);
  return hipGetLastError();
}

}  // namespace spec
