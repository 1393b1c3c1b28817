// Target LM head with the acceptance statistics of its rows in the epilogue.
//
// What is computed (page "投机推理算法的常见优化手段" (cnblogs), tree-mask
// section: one target forward over the flattened tree yields every node's
// next-token logits, and verification starts from them; "万字综述 10+ 种 LLM
// 投机采样推理加速方案", Medusa and EAGLE sections: the model's original LM
// head maps a position's final feature to vocabulary logits):
//   logits[r][v] = sum_k hidden[r][k] * weight[v][k]
// over bf16 operands with fp32 accumulation, and, for every (tree row,
// 256-entry vocabulary tile), the partial statistics the acceptance needs:
//  * temperature > 0: (reference, sum of exp(z/T - reference)) with the
//    tile's largest logit / T as the reference -- the form the acceptance
//    statistics pass writes, so the walk merges either alike.  The terms are
//    fp32 exponentials of the fp32 logits (the logits already carry the fp32
//    accumulation error; the sums lose about 1e-7 more), added in fp64
//    across lanes.  The logits of the rows that have children are stored
//    (fp32): the residual passes and draws at those nodes read them back.  A
//    leaf's logits are needed only if the walk ends there, for one draw,
//    which finds its 256-entry tile from these partials and recomputes that
//    tile's logits alone; so leaf rows are not stored.
//  * temperature 0: the tile's largest logit and its first index.  Nothing
//    else is needed downstream, so the logits need not be stored.
//
// Design (gfx950):
//  * A workgroup is 8 waves and owns a 256 (vocabulary) x 256 (tree rows)
//    output tile; wave (wv, wr) owns 128 x 64 of it as 4 x 2 blocks of
//    v_mfma_f32_32x32x16_bf16 with the weight rows as the A operand.  Each
//    lane then holds one tree row (the MFMA column) and 64 of its logits, so
//    the row statistics are lane-local until one lane-pair swap and one LDS
//    exchange between the two vocabulary halves.
//  * Both operands are K-contiguous.  K slices of BK columns stream
//    global -> LDS with direct-to-LDS 16-byte loads into a STAGES-deep ring;
//    each load instruction fills 1 KB (RPI rows of BK columns).  Row r keeps
//    its 16-byte chunks permuted (chunk c at slot c ^ ((r / RP) % CPR), RP
//    rows per 256 bytes) so that a fragment read -- 16 consecutive rows at
//    one chunk per LDS cycle -- touches all 64 banks once.
//  * The dispatcher deals workgroup ids round-robin to the 8 XCDs; the ids
//    that land on one XCD walk vocabulary tiles with the row tiles inner, so
//    the row tiles sharing a weight tile run together behind one L2, and the
//    weight (the bulk of the bytes) is fetched from beyond L2 about 1.5 times
//    rather than once per row tile.
#include <math.h>

#include "common.hpp"
#include "exp64.hpp"   // merge_arg
#include "launch.hpp"

namespace spec {

namespace {

typedef const __attribute__((address_space(1))) void* hd_gptr;
typedef __attribute__((address_space(3))) void* hd_lptr;

// s_waitcnt immediates: vmcnt <= n (others at their maxima); lgkmcnt == 0.
#define HEAD_VMCNT(n) ((((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8)))
#define HEAD_LGKMCNT0 0xc07f

constexpr int kBM = kHeadTileV;   // vocabulary entries per workgroup
constexpr int kBN = kHeadTileR;   // tree rows per workgroup
static_assert(kBM == 256 && kBN == 256, "wave layout below assumes a 256 x 256 tile");

struct HeadArgs {
  const uint16_t* hidden;   // [R][H]
  const uint16_t* weight;   // [V][H]
  int R, H, V;
  int nvt, nrt;             // vocabulary tiles, row tiles
  float* logits;            // [R][ld] or null
  const uint8_t* store;     // [R] rows whose logits are stored (null: every row)
  int64_t ld;
  int greedy;
  double inv_t;
  HeadTiles tiles;
};

template <int BK, int WAVES>
struct Geo {
  static constexpr int CPR = BK / 8;              // 16-byte chunks per row
  static constexpr int RPI = 64 / CPR;            // rows per 1 KB load
  static constexpr int RP = 16 / CPR;             // rows per 256 bytes
  static constexpr int TA = kBM * BK * 2;         // bytes of the weight slice
  static constexpr int TB = kBN * BK * 2;         // bytes of the hidden slice
  static constexpr int STAGE = TA + TB;
  static constexpr int HW = WAVES / 2;            // waves per operand / per vocabulary half
  static constexpr int LOADS = STAGE / 1024 / WAVES;  // load instructions per wave per stage
  static constexpr int JT = kBN / HW / 32;        // 32-row MFMA blocks per wave
  static_assert(TA / 1024 == HW * LOADS && TB / 1024 == HW * LOADS, "half the waves load each operand");
};

template <int BK, int STAGES, int WAVES>
__global__ void __launch_bounds__(WAVES * 64, 1) lm_head_kernel(HeadArgs a) {
  using G = Geo<BK, WAVES>;
  constexpr int JT = G::JT;
  // One array per ring slot: separate objects let the compiler see that a
  // refill of one slot never aliases the fragment reads of another, so it
  // does not wait for the refill before reading.
  __shared__ __attribute__((aligned(1024))) char st0[G::STAGE];
  __shared__ __attribute__((aligned(1024))) char st1[G::STAGE];
  __shared__ __attribute__((aligned(1024))) char st2[STAGES > 2 ? G::STAGE : 1024];
  __shared__ __attribute__((aligned(1024))) char st3[STAGES > 3 ? G::STAGE : 1024];
  __shared__ float red_m[2][kBN];
  __shared__ int red_a[2][kBN];
  __shared__ double red_s[2][kBN];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wv = wave & 1, wr = wave >> 1;   // vocabulary half, row block of JT * 32 rows
  const int xcd = blockIdx.x & 7, q = blockIdx.x >> 3;
  const int rt = q % a.nrt;
  const int vt = (q / a.nrt) * 8 + xcd;
  if (vt >= a.nvt) return;                         // whole workgroup, before any barrier
  const int v0 = vt * kBM, r0 = rt * kBN;

  // Loads: the first half of the waves fills the weight slice, the second
  // half the hidden slice; lane l of
  // load instruction gi writes slot l of 1 KB block gi, i.e. row
  // gi * RPI + l / CPR, slot l % CPR, which holds chunk slot ^ f(row).
  const bool is_a = wave < G::HW;
  const uint16_t* gsrc = is_a ? a.weight : a.hidden;
  const int lim = is_a ? a.V - 1 : a.R - 1;
  const int base_row = is_a ? v0 : r0;
  uint32_t goff[G::LOADS];
#pragma unroll
  for (int t = 0; t < G::LOADS; ++t) {
    const int gi = (wave % G::HW) * G::LOADS + t;
    const int row = gi * G::RPI + lane / G::CPR;
    const int c = (lane % G::CPR) ^ ((row / G::RP) % G::CPR);
    goff[t] = (uint32_t)min(base_row + row, lim) * (uint32_t)a.H + (uint32_t)(c * 8);
  }
  const int ldst0 = (is_a ? 0 : G::TA) + (wave % G::HW) * G::LOADS * 1024;

  auto issue = [&](char* slot, int k0) {
#pragma unroll
    for (int t = 0; t < G::LOADS; ++t)
      __builtin_amdgcn_global_load_lds((hd_gptr)(gsrc + goff[t] + k0),
                                       (hd_lptr)(slot + ldst0 + t * 1024), 16, 0, 0);
  };

  // Fragment reads: row rb + (lane & 31) (rb a multiple of 32), chunk
  // 2 kk + lane / 32; the permutation term depends on lane & 31 only.
  const int l31 = lane & 31, half = lane >> 5;
  const int fl = (l31 / G::RP) % G::CPR;
  const int lane_base = l31 * BK * 2;

  f32x16 acc[4][JT];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < JT; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  auto compute = [&](const char* slot) {
    const char* sa = slot;
    const char* sb = sa + G::TA;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int co = lane_base + ((((2 * kk) | half) ^ fl) << 4);
      bf16x8 af[4], bfr[JT];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = *reinterpret_cast<const bf16x8*>(sa + (wv * 128 + i * 32) * BK * 2 + co);
#pragma unroll
      for (int j = 0; j < JT; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8*>(sb + (wr * JT * 32 + j * 32) * BK * 2 + co);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < JT; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
      // Scheduling hint: alternate the 4 + JT fragment reads with as many
      // MFMAs (mask 0x100 = LDS read, 0x008 = MFMA), so a wave's reads for the
      // next K step overlap its multiplies instead of bunching before them.
#pragma unroll
      for (int q = 0; q < 4 + JT; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 4 * JT - (4 + JT), 0);
    }
  };

  // A wave whose rows all lie past the last tree row (the ragged last row
  // tile) loads its share and meets every barrier but skips the multiplies;
  // its SIMD then runs only the other wave's MFMAs.
  const bool active = r0 + wr * JT * 32 < a.R;
  const int nk = a.H / BK;
  issue(st0, 0);
  if (STAGES > 2 && nk > 1) issue(st1, BK);
  if (STAGES > 3 && nk > 2) issue(st2, 2 * BK);

  // Step kt: wait for slice kt (slices issued after it may stay in flight),
  // barrier (every wave's part of slice kt has landed and every wave is done
  // with the slot of slice kt - 1), refill that slot with slice
  // kt + STAGES - 1, then multiply slice kt.
#define HEAD_STEP(KT, CUR, NXT)                                                                   \
  {                                                                                               \
    const int after_ = min(nk - 1 - (KT), STAGES - 2);                                            \
    if (after_ >= 2)                                                                              \
      __builtin_amdgcn_s_waitcnt(HEAD_VMCNT(2 * G::LOADS));                                       \
    else if (after_ == 1)                                                                         \
      __builtin_amdgcn_s_waitcnt(HEAD_VMCNT(G::LOADS));                                           \
    else                                                                                          \
      __builtin_amdgcn_s_waitcnt(HEAD_VMCNT(0));                                                  \
    __builtin_amdgcn_s_barrier();                                                                 \
    if ((KT) + STAGES - 1 < nk) issue(NXT, ((KT) + STAGES - 1) * BK);                             \
    if (active) compute(CUR);                                                                     \
    __builtin_amdgcn_s_waitcnt(HEAD_LGKMCNT0);                                                    \
  }
  static_assert(STAGES >= 2 && STAGES <= 4, "ring depth");
  for (int kt = 0; kt < nk; kt += STAGES) {
    if (STAGES == 2) {
      HEAD_STEP(kt, st0, st1);
      if (kt + 1 >= nk) break;
      HEAD_STEP(kt + 1, st1, st0);
    } else if (STAGES == 3) {
      HEAD_STEP(kt, st0, st2);
      if (kt + 1 >= nk) break;
      HEAD_STEP(kt + 1, st1, st0);
      if (kt + 2 >= nk) break;
      HEAD_STEP(kt + 2, st2, st1);
    } else {
      HEAD_STEP(kt, st0, st3);
      if (kt + 1 >= nk) break;
      HEAD_STEP(kt + 1, st1, st0);
      if (kt + 2 >= nk) break;
      HEAD_STEP(kt + 2, st2, st1);
      if (kt + 3 >= nk) break;
      HEAD_STEP(kt + 3, st3, st2);
    }
  }
#undef HEAD_STEP
  __builtin_amdgcn_s_waitcnt(HEAD_VMCNT(0));

  // Epilogue.  acc[i][j][e] is the logit of vocabulary entry
  // v0 + wv*128 + 32 i + 8 (e / 4) + 4 half + e % 4 for tree row
  // r0 + wr*JT*32 + 32 j + l31; for a fixed lane, v grows with (i, e).
  const int vl0 = v0 + wv * 128 + 4 * half;
  if (a.logits) {
    // Each 32-row block of the wave's tile goes through LDS so that every
    // global store writes whole 512-byte row segments.  In the wave's 16 KB
    // region, 16-byte chunk c (4 logits) of row rr sits at slot c ^ rr of
    // the row's 512 bytes: the writes (16 rows at one chunk) and the row
    // reads (16 chunks of one row) both touch all 64 banks once.
    // which of the tile's rows are stored, read once into LDS
    __shared__ unsigned char s_keep[kBN];
    for (int i = tid; i < kBN; i += WAVES * 64)
      s_keep[i] = (r0 + i < a.R) && (!a.store || a.store[r0 + i]);
    __syncthreads();                                 // every wave is done with the ring
    char* reg = (wave < G::HW ? st0 : st1) + (wave % G::HW) * 16384;
    static_assert(G::HW * 16384 <= G::STAGE, "staging regions fit one ring slot");
    const int vcol = v0 + wv * 128 + 4 * l31;        // this lane's 4 logits in a row
#pragma unroll
    for (int j = 0; j < JT; ++j) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int c = 8 * i + 2 * g + half;
          const f32x4 val = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                             acc[i][j][4 * g + 3]};
          *reinterpret_cast<f32x4*>(reg + l31 * 512 + ((c ^ l31) << 4)) = val;
        }
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        const int rr = 2 * t + half;
        const f32x4 x = *reinterpret_cast<const f32x4*>(reg + rr * 512 + ((l31 ^ rr) << 4));
        const int r = r0 + wr * JT * 32 + 32 * j + rr;
        if (!s_keep[r - r0]) continue;
        float* dst = a.logits + (int64_t)r * a.ld + vcol;
        if (vcol + 3 < a.V) {
          // streaming hint: the walk reads back only a few rows, so the
          // logits should not displace the weight and hidden tiles in L2
          __builtin_nontemporal_store(x, reinterpret_cast<f32x4*>(dst));
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (vcol + e < a.V) dst[e] = x[e];
        }
      }
    }
  }

  if (a.greedy) {
#pragma unroll
    for (int j = 0; j < JT; ++j) {
      float m = -INFINITY;
      int am = -1;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int v = vl0 + 32 * i + 8 * (e >> 2) + (e & 3);
          const float x = acc[i][j][e];
          const bool gt = v < a.V && x > m;          // strict: the lane's first index wins
          m = gt ? x : m;
          am = gt ? v : am;
        }
      merge_arg(m, am, __shfl_xor(m, 32, 64), __shfl_xor(am, 32, 64));
      const int rl = wr * JT * 32 + 32 * j + l31;
      if (half == 0) {
        red_m[wv][rl] = m;
        red_a[wv][rl] = am;
      }
    }
    __syncthreads();
    if (wv == 0 && half == 0) {
#pragma unroll
      for (int j = 0; j < JT; ++j) {
        const int rl = wr * JT * 32 + 32 * j + l31;
        const int r = r0 + rl;
        if (r >= a.R) continue;
        float m = red_m[0][rl];
        int am = red_a[0][rl];
        merge_arg(m, am, red_m[1][rl], red_a[1][rl]);
        a.tiles.m[(int64_t)r * a.nvt + vt] = m;
        a.tiles.am[(int64_t)r * a.nvt + vt] = am;
      }
    }
    return;
  }

#pragma unroll
  for (int j = 0; j < JT; ++j) {
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int v = vl0 + 32 * i + 8 * (e >> 2) + (e & 3);
        if (v < a.V) m = fmaxf(m, acc[i][j][e]);
      }
    m = fmaxf(m, __shfl_xor(m, 32, 64));
    if (half == 0) red_m[wv][wr * JT * 32 + 32 * j + l31] = m;
  }
  __syncthreads();
  const double inv_t = a.inv_t;
#pragma unroll
  for (int j = 0; j < JT; ++j) {
    const int rl = wr * JT * 32 + 32 * j + l31;
    const float m = fmaxf(red_m[0][rl], red_m[1][rl]);
    // exp((z - m) / T) as 2^((z - m) * log2(e) / T) in fp32: the largest
    // terms have the smallest arguments, so the tile sum keeps about 1e-7
    // relative accuracy (64 terms per lane), below the logits' own fp32
    // accumulation error; lanes and waves then add in fp64.
    const float c2 = (float)(inv_t * 1.4426950408889634);
    float sf = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int v = vl0 + 32 * i + 8 * (e >> 2) + (e & 3);
        if (v < a.V) sf += __builtin_amdgcn_exp2f((acc[i][j][e] - m) * c2);
      }
    double s = (double)sf;
    s += __shfl_xor(s, 32, 64);
    if (half == 0) red_s[wv][rl] = s;
  }
  __syncthreads();
  if (wv == 0 && half == 0) {
#pragma unroll
    for (int j = 0; j < JT; ++j) {
      const int rl = wr * JT * 32 + 32 * j + l31;
      const int r = r0 + rl;
      if (r >= a.R) continue;
      const float m = fmaxf(red_m[0][rl], red_m[1][rl]);
      a.tiles.ref[(int64_t)r * a.nvt + vt] = (m == -INFINITY) ? 0.0 : (double)m * inv_t;
      a.tiles.s[(int64_t)r * a.nvt + vt] = red_s[0][rl] + red_s[1][rl];
    }
  }
}

// Which rows have children (one workgroup per request, whose rows are
// contiguous and at most kMaxRows), and the request's slot of recomputed
// leaf logits cleared to tag 0.  Parents outside 0 .. row-1 mark nothing
// (the acceptance reports such a tree as invalid and reads no logits).
__global__ void __launch_bounds__(kHeadTileV)
head_rows_kernel(const int32_t* __restrict__ row_offsets, const int32_t* __restrict__ parents,
                 uint8_t* kids, double* leafz) {
  const int b = blockIdx.x, tid = threadIdx.x;
  const int o = row_offsets[b], n = row_offsets[b + 1] - o;
  for (int i = tid; i < n; i += kHeadTileV) kids[o + i] = 0;
  leafz[(int64_t)b * kHeadTileV + tid] = 0.0;
  __syncthreads();
  for (int i = tid; i < n; i += kHeadTileV) {
    const int p = parents[o + i];
    if (i > 0 && p >= 0 && p < i) kids[o + p] = 1;
  }
}

constexpr int kBK = 64;
constexpr int kStages = 2;
constexpr int kWaves = 8;

}  // namespace

int head_vocab_tiles(int vocab) { return (vocab + kBM - 1) / kBM; }

size_t head_tiles_bytes(int R, int vocab) {
  const size_t n = (size_t)R * head_vocab_tiles(vocab);
  // (ref, s) doubles for sampling; (max, argmax) share the same space at T = 0;
  // then the children marks and the leaf-logit slots (B <= R requests)
  return 2 * ((n * sizeof(double) + 255) & ~(size_t)255) + (((size_t)R + 255) & ~(size_t)255) +
         (size_t)R * kHeadTileV * sizeof(double);
}

HeadTiles head_tiles(void* base, int R, int vocab) {
  const size_t n = (size_t)R * head_vocab_tiles(vocab);
  const size_t half = (n * sizeof(double) + 255) & ~(size_t)255;
  char* p = (char*)base;
  HeadTiles t;
  t.ntile = head_vocab_tiles(vocab);
  t.ref = (double*)p;
  t.s = (double*)(p + half);
  t.m = (float*)p;            // greedy: the reference / sum arrays are unused
  t.am = (int32_t*)(p + half);
  t.kids = (uint8_t*)(p + 2 * half);
  t.leafz = (double*)(p + 2 * half + (((size_t)R + 255) & ~(size_t)255));
  t.hidden = nullptr;
  t.weight = nullptr;
  t.H = 0;
  return t;
}

hipError_t launch_lm_head(int R, const uint16_t* hidden, int H, const uint16_t* weight, int vocab,
                          float temperature, float* logits, int64_t ld, const HeadTiles& tiles,
                          int B, const int32_t* row_offsets, const int32_t* parents,
                          hipStream_t stream) {
  HeadArgs a;
  a.hidden = hidden;
  a.weight = weight;
  a.R = R;
  a.H = H;
  a.V = vocab;
  a.nvt = head_vocab_tiles(vocab);
  a.nrt = (R + kBN - 1) / kBN;
  a.logits = logits;
  a.store = nullptr;
  a.ld = ld;
  a.greedy = temperature == 0.0f;
  if (!a.greedy) {
    hipLaunchKernelGGL(head_rows_kernel, dim3((unsigned)B), dim3(kHeadTileV), 0, stream, row_offsets,
                       parents, tiles.kids, tiles.leafz);
    a.store = tiles.kids;
  }
  a.inv_t = a.greedy ? 0.0 : 1.0 / (double)temperature;
  a.tiles = tiles;
  const int groups = (a.nvt + 7) / 8;
  const int64_t blocks = (int64_t)groups * 8 * a.nrt;
  hipLaunchKernelGGL((lm_head_kernel<kBK, kStages, kWaves>), dim3((unsigned)blocks),
                     dim3(kWaves * 64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace spec
