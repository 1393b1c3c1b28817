// Tree attention for the verify step.
//
// What is computed (page "投机推理算法的常见优化手段" (cnblogs), tree-mask
// section; "万字综述 10+ 种 LLM 投机采样推理加速方案" section 5.2): every
// flattened tree row i of request b attends, in one pass, to all L_b cached
// prefix tokens and to the tree rows its packed ancestor mask selects (their
// K/V sit at slots L_b + j).  out = softmax(q k^T * scale) v, GQA head h on KV
// head h / G.
//
// bf16 path (MFMA, gfx950):
//  * One workgroup = 4 waves = up to 128 query rows of one (request, KV head);
//    a query row is (tree row, head within the GQA group).  All 128 rows
//    share every K/V tile read from HBM.
//  * Keys are cut into splits (split-KV) so long and short requests spread
//    over all CUs; a second kernel merges split partials by log-sum-exp.
//  * Scores are formed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: each lane then owns one query row (column of
//    S^T), so the online-softmax rescale of that row's output is lane-local,
//    and P^T is already in the B-operand layout of O^T = V^T P^T.
//  * K tiles are kept row-major in LDS; V tiles are transposed on the way in
//    (4 keys x 8 dims per thread, repacked in registers) so the V^T operand
//    is two 8-byte LDS reads per MFMA.  Global loads are 16 B per lane,
//    staged in registers one tile ahead (double-buffered LDS).
//  * Softmax is fp32 in the exp2 domain; masking costs nothing on tiles that
//    lie wholly inside the prefix.
#include <math.h>

#include "common.hpp"
#include "launch.hpp"

namespace spec {

constexpr int kTileKeys = 64;
constexpr int kAttnWaves = 4;
constexpr int kRowsPerWave = 32;
constexpr int kRowsPerBlock = kAttnWaves * kRowsPerWave;
constexpr int kVtStride = kTileKeys + 4;   // bf16 per transposed-V row in LDS (136 B)
constexpr int kMaxSplit = 8192;            // keys per split (block ids kept in LDS)

struct AttnArgs {
  const int32_t* row_offsets;
  const int32_t* prefix_len;
  int B;
  int hq;
  int G;
  int split;
  KvAddr addr;
  const uint16_t* q;
  const uint64_t* mask;
  int words;
  float scale_log2;
  const uint16_t* k;
  const uint16_t* v;
  void* out;
  int out_f32;
  float* part;       // [items][kRowsPerBlock][D] unnormalised outputs
  float* part_ml;    // [items][kRowsPerBlock][2]  (running max, running sum)
};

// Per-request work counts, shared by the planner (host) and kernels (device).
__host__ __device__ inline int attn_row_blocks(int n, int G) {
  return (n * G + kRowsPerBlock - 1) / kRowsPerBlock;
}
__host__ __device__ inline int attn_splits(int keys, int split) {
  return (keys + split - 1) / split;
}

// Wave-parallel search: which request holds item `x`, given per-request
// counts.  Returns b and the first item of b.  Uniform across the wave.
template <bool kUnits>
SPEC_DEVICE void locate(int64_t x, const AttnArgs& a, int& b_out, int64_t& base_out) {
  const int lane = threadIdx.x & 63;
  int64_t running = 0;
  for (int base = 0; base < a.B; base += 64) {
    const int b = base + lane;
    int64_t cnt = 0;
    if (b < a.B) {
      const int n = a.row_offsets[b + 1] - a.row_offsets[b];
      const int nrb = attn_row_blocks(n, a.G);
      cnt = (int64_t)a.addr.hkv * nrb;
      if (!kUnits) cnt *= attn_splits(a.prefix_len[b] + n, a.split);
    }
    int64_t incl = cnt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      int64_t t = __shfl_up(incl, o, 64);
      if (lane >= o) incl += t;
    }
    const int64_t total = __shfl(incl, 63, 64);
    if (x < running + total) {
      const uint64_t hit = __ballot(running + incl > x);
      const int first = __ffsll((long long)hit) - 1;
      const int64_t excl = __shfl(incl - cnt, first, 64);
      b_out = base + first;
      base_out = running + excl;
      return;
    }
    running += total;
  }
  b_out = -1;
  base_out = 0;
}


typedef const __attribute__((address_space(1))) uint16_t* gptr_u16;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef const __attribute__((address_space(1))) u32x4* gptr_u4;

// 16-byte load through an explicitly global pointer (plain global_load, so
// LDS waits in the loop do not also wait on the prefetch).
SPEC_DEVICE uint4 gload16(gptr_u16 p) {
  const u32x4 v = *(gptr_u4)p;
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Element offset of absolute key kk: contiguous rows, or a paged block whose
// id was staged in LDS (s_blk holds the split's block ids from block blk0).
SPEC_DEVICE int64_t kv_key_offset(int kk, bool paged, const int* s_blk, int blk0, int64_t blk_stride,
                                  int d) {
  if (!paged) return (int64_t)kk * d;
  return (int64_t)s_blk[(kk >> 4) - blk0] * blk_stride + (kk & 15) * d;
}

// Global -> registers for one 64-key tile: K as 16-byte row chunks, V as
// 4 consecutive keys x 8 dims per thread (transposed when stored).
template <int D>
SPEC_DEVICE void load_kv_tile(gptr_u16 gk, gptr_u16 gv, int t0, int key_end, bool paged,
                              const int* s_blk, int blk0, int64_t blk_stride, int tid,
                              uint4 (&kreg)[kTileKeys * (D / 8) / 256],
                              uint4 (&vreg)[((kTileKeys / 4) * (D / 8) + 255) / 256][4]) {
  constexpr int DC = D / 8;
  constexpr int KCH = kTileKeys * DC / 256;
  constexpr int VUN = (kTileKeys / 4) * DC;
  constexpr int VPT = (VUN + 255) / 256;
#pragma unroll
  for (int j = 0; j < KCH; ++j) {
    const int c = tid + 256 * j;
    const int kk = t0 + c / DC;
    uint4 val = make_uint4(0, 0, 0, 0);
    if (kk < key_end)
      val = gload16(gk + kv_key_offset(kk, paged, s_blk, blk0, blk_stride, D) + (c % DC) * 8);
    kreg[j] = val;
  }
#pragma unroll
  for (int j = 0; j < VPT; ++j) {
    const int u = tid + 256 * j;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int kk = t0 + (u / DC) * 4 + r;
      uint4 val = make_uint4(0, 0, 0, 0);
      if (u < VUN && kk < key_end)
        val = gload16(gv + kv_key_offset(kk, paged, s_blk, blk0, blk_stride, D) + (u % DC) * 8);
      vreg[j][r] = val;
    }
  }
}

// Registers -> LDS: K row-major (stride D + 8), V transposed to [dim][key].
template <int D>
SPEC_DEVICE void store_kv_tile(uint16_t* ks, uint16_t* vt, int tid,
                               const uint4 (&kreg)[kTileKeys * (D / 8) / 256],
                               const uint4 (&vreg)[((kTileKeys / 4) * (D / 8) + 255) / 256][4]) {
  constexpr int DC = D / 8;
  constexpr int KS = D + 8;
  constexpr int KCH = kTileKeys * DC / 256;
  constexpr int VUN = (kTileKeys / 4) * DC;
  constexpr int VPT = (VUN + 255) / 256;
#pragma unroll
  for (int j = 0; j < KCH; ++j) {
    const int c = tid + 256 * j;
    *reinterpret_cast<uint4*>(&ks[(c / DC) * KS + (c % DC) * 8]) = kreg[j];
  }
#pragma unroll
  for (int j = 0; j < VPT; ++j) {
    const int u = tid + 256 * j;
    if (u < VUN) {
      const int kg = u / DC, dc = u % DC;
      const uint32_t w0[4] = {vreg[j][0].x, vreg[j][0].y, vreg[j][0].z, vreg[j][0].w};
      const uint32_t w1[4] = {vreg[j][1].x, vreg[j][1].y, vreg[j][1].z, vreg[j][1].w};
      const uint32_t w2[4] = {vreg[j][2].x, vreg[j][2].y, vreg[j][2].z, vreg[j][2].w};
      const uint32_t w3[4] = {vreg[j][3].x, vreg[j][3].y, vreg[j][3].z, vreg[j][3].w};
#pragma unroll
      for (int i2 = 0; i2 < 4; ++i2) {
        // dims dc*8 + 2*i2 (low halves) and dc*8 + 2*i2 + 1 (high halves)
        const uint2 lo = make_uint2((w0[i2] & 0xffffu) | (w1[i2] << 16),
                                    (w2[i2] & 0xffffu) | (w3[i2] << 16));
        const uint2 hi = make_uint2((w0[i2] >> 16) | (w1[i2] & 0xffff0000u),
                                    (w2[i2] >> 16) | (w3[i2] & 0xffff0000u));
        const int d0 = dc * 8 + 2 * i2;
        *reinterpret_cast<uint2*>(&vt[d0 * kVtStride + kg * 4]) = lo;
        *reinterpret_cast<uint2*>(&vt[(d0 + 1) * kVtStride + kg * 4]) = hi;
      }
    }
  }
}

template <int D>
__global__ void __launch_bounds__(256, 2) attn_bf16_kernel(AttnArgs a) {
  constexpr int KS = D + 8;                 // bf16 per K row in LDS
  constexpr int DC = D / 8;                 // 16-byte chunks per row
  constexpr int KCH = kTileKeys * DC / 256; // K chunks per thread per tile
  constexpr int VUN = (kTileKeys / 4) * DC; // V transpose units per tile
  constexpr int VPT = (VUN + 255) / 256;    // V units per thread
  constexpr int NKS = D / 16;               // MFMA k-steps for q.k
  constexpr int NDB = D / 32;               // 32-dim output blocks
  __shared__ __attribute__((aligned(16))) uint16_t ks_lds[2][kTileKeys * KS];
  __shared__ __attribute__((aligned(16))) uint16_t vt_lds[2][D * kVtStride];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 31;     // query row within the wave tile
  const int half = lane >> 5;

  int b;
  int64_t ibase;
  const int64_t item = blockIdx.x;
  locate<false>(item, a, b, ibase);
  if (b < 0) return;
  const int o = a.row_offsets[b];
  const int n = a.row_offsets[b + 1] - o;
  const int L = a.prefix_len[b];
  const int total_keys = L + n;
  const int nrb = attn_row_blocks(n, a.G);
  const int ns = attn_splits(total_keys, a.split);
  const int64_t local = item - ibase;
  const int s = (int)(local % ns);
  const int rb = (int)((local / ns) % nrb);
  const int kvh = (int)(local / ((int64_t)ns * nrb));
  const int key_begin = s * a.split;
  const int key_end = min(key_begin + a.split, total_keys);
  const int M = n * a.G;

  // ---- this lane's query row --------------------------------------------
  const int row = rb * kRowsPerBlock + wave * kRowsPerWave + col;
  const bool row_ok = row < M;
  const bool wave_active = rb * kRowsPerBlock + wave * kRowsPerWave < M;
  const int ti = row_ok ? row / a.G : 0;
  const int hh = kvh * a.G + (row_ok ? row % a.G : 0);
  bf16x8 qf[NKS];
  uint64_t mw[kMaxWords] = {0, 0, 0, 0};
  if (row_ok) {
    const uint16_t* qp = a.q + ((int64_t)(o + ti) * a.hq + hh) * D + half * 8;
#pragma unroll
    for (int kk = 0; kk < NKS; ++kk)
      qf[kk] = __builtin_bit_cast(bf16x8, gload16((gptr_u16)(qp + kk * 16)));
    for (int w = 0; w < a.words; ++w) mw[w] = a.mask[(int64_t)(o + ti) * a.words + w];
  } else {
#pragma unroll
    for (int kk = 0; kk < NKS; ++kk)
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[kk][e] = (__bf16)0.0f;
  }

  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[db][e] = 0.0f;
  float m_run = -INFINITY;
  float l_run = 0.0f;

  // ---- tile staging -----------------------------------------------------
  // Paged caches: the block ids of this split are read once into LDS so the
  // tile loads below carry no dependent global lookups.
  __shared__ int s_blk[kMaxSplit / kBlock + 2];
  const int blk0 = key_begin >> 4;
  const uint16_t* kbase;
  const uint16_t* vbase;
  if (a.addr.paged) {
    const int nblk = ((key_end + kBlock - 1) >> 4) - blk0;
    for (int i = tid; i < nblk; i += 256)
      s_blk[i] = a.addr.block_table[(int64_t)b * a.addr.mbps + blk0 + i];
    kbase = a.k + (int64_t)kvh * kBlock * D;
    vbase = a.v + (int64_t)kvh * kBlock * D;
  } else {
    const int64_t off = ((int64_t)b * a.addr.hkv + kvh) * a.addr.capacity * D;
    kbase = a.k + off;
    vbase = a.v + off;
  }
  const int64_t blk_stride = (int64_t)a.addr.hkv * kBlock * D;
  const bool paged = a.addr.paged;
  const gptr_u16 gk = (const gptr_u16)kbase;
  const gptr_u16 gv = (const gptr_u16)vbase;
  uint4 kreg[KCH];
  uint4 vreg[VPT][4];

  const int ntiles = (key_end - key_begin + kTileKeys - 1) / kTileKeys;
  __syncthreads();
  load_kv_tile<D>(gk, gv, key_begin, key_end, paged, s_blk, blk0, blk_stride, tid, kreg, vreg);
  store_kv_tile<D>(ks_lds[0], vt_lds[0], tid, kreg, vreg);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    const int t0 = key_begin + t * kTileKeys;
    if (t + 1 < ntiles)
      load_kv_tile<D>(gk, gv, t0 + kTileKeys, key_end, paged, s_blk, blk0, blk_stride, tid, kreg, vreg);

    if (wave_active) {
      // S^T (64 keys x 32 rows) as two 32x32 blocks.
      f32x16 sc[2];
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
#pragma unroll
        for (int e = 0; e < 16; ++e) sc[kh][e] = 0.0f;
        const uint16_t* kp = &ks_lds[buf][(kh * 32 + col) * KS + half * 8];
#pragma unroll
        for (int kk = 0; kk < NKS; ++kk) {
          const bf16x8 kf = *reinterpret_cast<const bf16x8*>(kp + kk * 16);
          sc[kh] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[kk], sc[kh], 0, 0, 0);
        }
      }
      // scale, mask, running max
      const bool full = (t0 + kTileKeys <= L) && (t0 + kTileKeys <= key_end);
      float mx = -INFINITY;
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          float x = sc[kh][e] * a.scale_log2;
          if (!full) {
            const int kk = t0 + kh * 32 + half * 4 + 8 * (e >> 2) + (e & 3);
            bool vis = kk < key_end;
            if (vis && kk >= L) {
              const int j = kk - L;
              vis = (mw[j >> 6] >> (j & 63)) & 1ull;
            }
            x = vis ? x : -INFINITY;
          }
          sc[kh][e] = x;
          mx = fmaxf(mx, x);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m_run, mx);
      // A row with no visible key yet keeps m = -inf; using 0 as the
      // reference then gives alpha = 0 and p = 0 without a (divergent) branch.
      const float m_ref = (m_new == -INFINITY) ? 0.0f : m_new;
      const float alpha = exp2f(m_run - m_ref);
      float rs = 0.0f;
      bf16x8 pb[2][2];
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float p = exp2f(sc[kh][e] - m_ref);
          rs += p;
          pb[kh][e >> 3][e & 7] = (__bf16)p;
        }
      rs += __shfl_xor(rs, 32, 64);
      l_run = l_run * alpha + rs;
      m_run = m_new;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[db][e] *= alpha;
      // O^T += V^T P^T over the 64 keys: 2 halves x 2 16-key steps
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int mm = 0; mm < 2; ++mm) {
          const int kb = kh * 32 + mm * 16 + half * 4;
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            const uint16_t* vp = &vt_lds[buf][(db * 32 + col) * kVtStride + kb];
            const uint2 lo = *reinterpret_cast<const uint2*>(vp);
            const uint2 hi = *reinterpret_cast<const uint2*>(vp + 8);
            const bf16x8 vf = __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
            acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[kh][mm], acc[db], 0, 0, 0);
          }
        }
    }
    if (t + 1 < ntiles) store_kv_tile<D>(ks_lds[buf ^ 1], vt_lds[buf ^ 1], tid, kreg, vreg);
    __syncthreads();
  }

  if (!row_ok) return;
  // acc[db][4*ai + c] holds output dim db*32 + half*4 + 8*ai + c of this row.
  if (ns == 1) {
    const float inv = 1.0f / l_run;
    const int64_t obase = ((int64_t)(o + ti) * a.hq + hh) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int ai = 0; ai < 4; ++ai) {
        const int d0 = db * 32 + half * 4 + 8 * ai;
        const float v0 = acc[db][4 * ai] * inv, v1 = acc[db][4 * ai + 1] * inv;
        const float v2 = acc[db][4 * ai + 2] * inv, v3 = acc[db][4 * ai + 3] * inv;
        if (a.out_f32) {
          *reinterpret_cast<float4*>((float*)a.out + obase + d0) = make_float4(v0, v1, v2, v3);
        } else {
          uint2 pk;
          pk.x = f32_to_bf16_bits(v0) | ((uint32_t)f32_to_bf16_bits(v1) << 16);
          pk.y = f32_to_bf16_bits(v2) | ((uint32_t)f32_to_bf16_bits(v3) << 16);
          *reinterpret_cast<uint2*>((uint16_t*)a.out + obase + d0) = pk;
        }
      }
  } else {
    const int r_in_block = wave * kRowsPerWave + col;
    float* pp = a.part + (item * kRowsPerBlock + r_in_block) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int ai = 0; ai < 4; ++ai) {
        const int d0 = db * 32 + half * 4 + 8 * ai;
        *reinterpret_cast<float4*>(pp + d0) =
            make_float4(acc[db][4 * ai], acc[db][4 * ai + 1], acc[db][4 * ai + 2], acc[db][4 * ai + 3]);
      }
    if (half == 0) {
      float* ml = a.part_ml + (item * kRowsPerBlock + r_in_block) * 2;
      ml[0] = m_run;
      ml[1] = l_run;
    }
  }
}

// Merge split partials of one (request, KV head, row block).
template <int D>
__global__ void __launch_bounds__(256) attn_combine_kernel(AttnArgs a) {
  int b;
  int64_t ubase;
  locate<true>((int64_t)blockIdx.x, a, b, ubase);
  if (b < 0) return;
  const int o = a.row_offsets[b];
  const int n = a.row_offsets[b + 1] - o;
  const int L = a.prefix_len[b];
  const int ns = attn_splits(L + n, a.split);
  if (ns == 1) return;
  const int nrb = attn_row_blocks(n, a.G);
  const int64_t u = blockIdx.x - ubase;            // kvh * nrb + rb
  const int rb = (int)(u % nrb);
  const int kvh = (int)(u / nrb);
  // first item of this request: same prefix order as the main kernel
  int bb;
  int64_t ibase = 0;
  {
    // items of earlier requests = sum over b' < b; recover via locate on units
    // is not enough, so accumulate directly (wave-parallel).
    const int lane = threadIdx.x & 63;
    int64_t acc = 0;
    for (int base = 0; base < b; base += 64) {
      const int bq = base + lane;
      int64_t cnt = 0;
      if (bq < b) {
        const int nq = a.row_offsets[bq + 1] - a.row_offsets[bq];
        cnt = (int64_t)a.addr.hkv * attn_row_blocks(nq, a.G) * attn_splits(a.prefix_len[bq] + nq, a.split);
      }
      acc += cnt;
    }
    ibase = wave_sum(acc);
    bb = b;
  }
  (void)bb;
  const int64_t item0 = ibase + u * ns;            // split 0 of this unit
  const int M = n * a.G;
  const int rows = min(kRowsPerBlock, M - rb * kRowsPerBlock);
  constexpr int C4 = D / 4;
  for (int w = threadIdx.x; w < rows * C4; w += blockDim.x) {
    const int r = w / C4, c4 = w % C4;
    float mmax = -INFINITY;
    for (int s = 0; s < ns; ++s)
      mmax = fmaxf(mmax, a.part_ml[((item0 + s) * kRowsPerBlock + r) * 2]);
    float lsum = 0.0f;
    float4 accv = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s = 0; s < ns; ++s) {
      const float* ml = a.part_ml + ((item0 + s) * kRowsPerBlock + r) * 2;
      const float wgt = (ml[0] == -INFINITY) ? 0.0f : exp2f(ml[0] - mmax);
      lsum += ml[1] * wgt;
      const float4 pv = *reinterpret_cast<const float4*>(
          a.part + ((item0 + s) * kRowsPerBlock + r) * D + c4 * 4);
      accv.x += pv.x * wgt; accv.y += pv.y * wgt; accv.z += pv.z * wgt; accv.w += pv.w * wgt;
    }
    const float inv = 1.0f / lsum;
    const int grow = rb * kRowsPerBlock + r;
    const int ti = grow / a.G;
    const int hh = kvh * a.G + grow % a.G;
    const int64_t obase = ((int64_t)(o + ti) * a.hq + hh) * D + c4 * 4;
    if (a.out_f32) {
      *reinterpret_cast<float4*>((float*)a.out + obase) =
          make_float4(accv.x * inv, accv.y * inv, accv.z * inv, accv.w * inv);
    } else {
      uint2 pk;
      pk.x = f32_to_bf16_bits(accv.x * inv) | ((uint32_t)f32_to_bf16_bits(accv.y * inv) << 16);
      pk.y = f32_to_bf16_bits(accv.z * inv) | ((uint32_t)f32_to_bf16_bits(accv.w * inv) << 16);
      *reinterpret_cast<uint2*>((uint16_t*)a.out + obase) = pk;
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 path: one workgroup per (tree row, query head); keys in chunks of 256,
// one key per thread for the score, block-wide online softmax, then every
// thread accumulates one output dim over a slice of the chunk's keys.
__global__ void __launch_bounds__(256)
attn_f32_kernel(const int32_t* __restrict__ row_offsets, const int32_t* __restrict__ prefix_len,
                int B, int hq, int G, KvAddr addr, const float* __restrict__ q,
                const uint64_t* __restrict__ mask, int words, float scale,
                const float* __restrict__ kc, const float* __restrict__ vc, void* out,
                int out_f32) {
  __shared__ float qs[128];
  __shared__ float ps[256];
  __shared__ float red[8];
  __shared__ float oacc[256];
  const int D = addr.d;
  const int r = blockIdx.x / hq;
  const int h = blockIdx.x % hq;
  const int kvh = h / G;
  const int b = request_of_row(row_offsets, B, r);
  const int o = row_offsets[b];
  const int n = row_offsets[b + 1] - o;
  const int i = r - o;
  const int L = prefix_len[b];
  const int total = L + n;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  if (tid < D) qs[tid] = q[((int64_t)r * hq + h) * D + tid];
  uint64_t mw[kMaxWords] = {0, 0, 0, 0};
  for (int w = 0; w < words; ++w) mw[w] = mask[(int64_t)r * words + w];
  __syncthreads();
  const int d = tid % D;           // output dim this thread accumulates
  const int part = tid / D;        // which slice of the chunk's keys
  const int nparts = 256 / D;
  float m_run = -INFINITY, l_run = 0.0f, o_d = 0.0f;
  for (int c0 = 0; c0 < total; c0 += 256) {
    const int t = c0 + tid;
    float sc = -INFINITY;
    if (t < total) {
      bool vis = true;
      if (t >= L) {
        const int j = t - L;
        vis = (mw[j >> 6] >> (j & 63)) & 1ull;
      }
      if (vis) {
        const float* kp = kc + addr(b, kvh, t);
        float acc = 0.0f;
        for (int e = 0; e < D; ++e) acc = fmaf(qs[e], kp[e], acc);
        sc = acc * scale;
      }
    }
    float mx = wave_max(sc);
    if (lane == 0) red[wave] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = (m_new == -INFINITY) ? 1.0f : expf(m_run - m_new);
    const float p = (sc == -INFINITY) ? 0.0f : expf(sc - m_new);
    ps[tid] = p;
    float sum = wave_sum(p);
    __syncthreads();
    if (lane == 0) red[4 + wave] = sum;
    __syncthreads();
    sum = red[4] + red[5] + red[6] + red[7];
    l_run = l_run * alpha + sum;
    m_run = m_new;
    o_d *= alpha;
    const int cnt = min(256, total - c0);
    for (int j = part; j < cnt; j += nparts) {
      const float pj = ps[j];
      if (pj != 0.0f) o_d = fmaf(pj, vc[addr(b, kvh, c0 + j) + d], o_d);
    }
    __syncthreads();
  }
  oacc[tid] = o_d;
  __syncthreads();
  if (tid < D) {
    float acc = 0.0f;
    for (int pidx = 0; pidx < nparts; ++pidx) acc += oacc[pidx * D + tid];
    const float val = acc / l_run;
    const int64_t oi = ((int64_t)r * hq + h) * D + tid;
    if (out_f32) ((float*)out)[oi] = val;
    else ((uint16_t*)out)[oi] = f32_to_bf16_bits(val);
  }
}

// ---------------------------------------------------------------------------
AttnPlan plan_attention(int B, const int32_t* row_offsets_h, const int32_t* prefix_len_h, int hq,
                        int hkv) {
  const int G = hq / hkv;
  int64_t work = 0, units = 0;
  for (int b = 0; b < B; ++b) {
    const int n = row_offsets_h[b + 1] - row_offsets_h[b];
    const int nrb = attn_row_blocks(n, G);
    units += (int64_t)hkv * nrb;
    work += (int64_t)hkv * nrb * (prefix_len_h[b] + n);
  }
  // Aim at ~4 workgroups per CU (256 CUs), splits of at least 256 keys.
  const int64_t target = 1024;
  int64_t split = (work + target - 1) / target;
  split = ((split + kTileKeys - 1) / kTileKeys) * kTileKeys;
  if (split < 256) split = 256;
  if (split > kMaxSplit) split = kMaxSplit;
  AttnPlan p;
  p.rows_per_block = kRowsPerBlock;
  p.split_keys = (int)split;
  p.items = 0;
  p.partial_items = 0;
  p.units = units;
  for (int b = 0; b < B; ++b) {
    const int n = row_offsets_h[b + 1] - row_offsets_h[b];
    const int ns = attn_splits(prefix_len_h[b] + n, p.split_keys);
    const int64_t it = (int64_t)hkv * attn_row_blocks(n, G) * ns;
    p.items += it;
    if (ns > 1) p.partial_items += it;
  }
  return p;
}

size_t attention_workspace_bytes(const AttnPlan& plan, int d) {
  if (plan.partial_items == 0) return 256;
  return (size_t)plan.items * kRowsPerBlock * (d + 2) * sizeof(float) + 256;
}

hipError_t launch_attention_bf16(const LaunchCtx& cx, const AttnPlan& plan, const KvAddr& addr,
                                 int hq, const void* q, const uint64_t* mask, int words,
                                 float scale, const void* k_cache, const void* v_cache, void* out,
                                 int out_f32, void* workspace) {
  AttnArgs a;
  a.row_offsets = cx.row_offsets_d;
  a.prefix_len = cx.prefix_len_d;
  a.B = cx.B;
  a.hq = hq;
  a.G = hq / addr.hkv;
  a.split = plan.split_keys;
  a.addr = addr;
  a.q = (const uint16_t*)q;
  a.mask = mask;
  a.words = words;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.k = (const uint16_t*)k_cache;
  a.v = (const uint16_t*)v_cache;
  a.out = out;
  a.out_f32 = out_f32;
  a.part = (float*)workspace;
  a.part_ml = a.part + (size_t)plan.items * kRowsPerBlock * addr.d;
  if (plan.items > 0x7fffffff) return hipErrorInvalidValue;
  if (addr.d == 128) {
    hipLaunchKernelGGL(attn_bf16_kernel<128>, dim3((unsigned)plan.items), dim3(256), 0, cx.stream, a);
    if (plan.partial_items)
      hipLaunchKernelGGL(attn_combine_kernel<128>, dim3((unsigned)plan.units), dim3(256), 0, cx.stream, a);
  } else {
    hipLaunchKernelGGL(attn_bf16_kernel<64>, dim3((unsigned)plan.items), dim3(256), 0, cx.stream, a);
    if (plan.partial_items)
      hipLaunchKernelGGL(attn_combine_kernel<64>, dim3((unsigned)plan.units), dim3(256), 0, cx.stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_attention_f32(const LaunchCtx& cx, int R, const KvAddr& addr, int hq,
                                const float* q, const uint64_t* mask, int words, float scale,
                                const float* k_cache, const float* v_cache, void* out, int out_f32) {
  hipLaunchKernelGGL(attn_f32_kernel, dim3((unsigned)((int64_t)R * hq)), dim3(256), 0, cx.stream,
                     cx.row_offsets_d, cx.prefix_len_d, cx.B, hq, hq / addr.hkv, addr, q, mask,
                     words, scale, k_cache, v_cache, out, out_f32);
  return hipGetLastError();
}

}  // namespace spec
