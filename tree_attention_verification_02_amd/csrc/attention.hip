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
//  * A unit is (request, KV head, row block); its query rows are (tree row,
//    head within the GQA group) pairs, 32 per wave.  One workgroup = 8 waves
//    (256 rows); when some unit has more than 256 rows (the 46-row K-schedule
//    tree x 8 heads of a group = 368) every workgroup takes 12 waves (384
//    rows, three per SIMD), so such a unit still reads each K/V tile once.
//  * Keys are cut into splits (split-KV) so long and short requests spread
//    over all CUs; attn_combine merges split partials by log-sum-exp.  With
//    mixed lengths, heavy units get shorter splits, and workgroups take work
//    items by ticket in start order: first the leading splits, then the last
//    split of every unit longest-first, which evens out ragged prefixes.
//  * Scores are formed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: each lane owns one query row (a column of
//    S^T), so the online-softmax rescale of that row is lane-local, and P^T
//    is already in the B-operand layout of O^T = V^T P^T; row sums and the
//    two 32-lane halves meet through v_permlane32_swap.
//  * K/V tiles of 64 keys go from HBM straight into a 4-stage LDS ring
//    (global_load_lds with 8 waves, buffer loads to LDS with 12), 16 bytes
//    per lane, three tiles in flight while one is consumed; one barrier per
//    tile.  V^T operands come from LDS with ds_read_tr16_b64 (a transposing
//    read), so V needs no repacking.  Scheduling-group hints interleave the
//    LDS reads with the MFMAs.
//  * Softmax is fp32 in the exp2 domain with a lazy reference: a row's
//    maximum only moves when a score exceeds it by more than kLazyMax, so
//    the O / l rescale is rare.  Ancestor masks (packed 64-bit words per row)
//    are applied only on tiles that reach the tree's own keys.
#include <math.h>

#include <algorithm>

#include "common.hpp"
#include "launch.hpp"

namespace spec {

constexpr int kTileKeys = 64;
constexpr int kRowsPerWave = 32;
constexpr int kWaves = 8;                  // waves per bf16 workgroup (wide variant: 12)
constexpr int kWideWaves = 12;
constexpr int kDmaWaves = 8;               // waves that issue the K/V tile loads
constexpr int kStages = 4;                 // LDS ring depth (tiles)
constexpr int kCombineRows = 32;           // query rows per combine workgroup
constexpr float kLazyMax = 8.0f;           // log2 headroom of the softmax reference
constexpr int kMaxSplitsCombine = 1024;    // splits per request the combine handles
constexpr int kMaxSplit = 8192;            // keys per split (block ids kept in LDS)
static_assert((int64_t)kMaxSplit * 1024 == kMaxAttnKeys, "key limit");

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
  int rows_per_block;
  float* part;       // [items][rows_per_block][D] unnormalised outputs
  float* part_ml;    // [items][rows_per_block][2]  (running max, running sum)
  int* unit_desc;    // [units][8]: b, kvh, rb, ns, o, rows of the block (main kernel writes)
  int* unit_items;   // [units][max_ns]: item of each split of the unit
  int max_ns;
  int lpt;           // two-phase (longest-first) item order, see AttnPlan
  unsigned* ticket;  // workgroups take items in start order (null: blockIdx)
  int items;
  int weighted;      // heavy units get shorter splits (attn_split_for)
  int64_t items_a;   // items of the first phase
  uint16_t order[kLptMax];
};

// Per-request work counts, shared by the planner (host) and kernels (device).
__host__ __device__ inline int attn_row_blocks(int n, int G, int rpb) {
  return (n * G + rpb - 1) / rpb;
}
// Splits of a request with `keys` keys: a last piece shorter than a quarter
// split joins the one before it (a tiny workgroup pays its start-up and its
// partial write for little work), unless that piece would exceed kMaxSplit.
// The last split ends at `keys`; every other one is `split` long.
__host__ __device__ inline int attn_splits(int keys, int split) {
  int ns = (keys + split - 1) / split;
  if (ns > 1 && keys - (ns - 1) * split < split / 4 && keys - (ns - 2) * split <= kMaxSplit) --ns;
  return ns;
}
// Keys per split of a request with n tree rows.  With `weighted`, a unit
// (KV head, row block) of more than kWaves / 2 row groups runs one wave per
// group instead of two, and is compute-bound: per-item timing on the
// batched dynamic trees gave ~32 keys/us for such units against ~48 for the
// HBM-bound pair-mode units.  Its splits are 2/3 as long, so that every full
// split takes about the same time.
__host__ __device__ inline int attn_split_for(int split, int n, int G, int rpb, int weighted) {
  const int rows = n * G < rpb ? n * G : rpb;
  if (!weighted || (rows + kRowsPerWave - 1) / kRowsPerWave <= rpb / kRowsPerWave / 2) return split;
  const int s2 = (split * 2 / 3) / kTileKeys * kTileKeys;
  return s2 > kTileKeys ? s2 : kTileKeys;
}

// Workgroup index -> (request, KV head, row block, split).  Phase A: every
// split but the last of each request when `lpt` is set (every split
// otherwise), request by request, then (KV head, row block, split).  Phase B
// (`lpt` only): the last split of each request, requests in `order`, then
// (KV head, row block).  Wave-parallel over requests; uniform results;
// b = -1 past the end.  Also returns the request's first row o, rows n and
// prefix length L from the same loads, and (batches of at most 64 requests)
// its first (KV head, row block) unit `ubase` among all requests in request
// order; ubase = -1 otherwise.
struct ItemLoc {
  int b, kvh, rb, s, o, n, L;
  int64_t ubase;
};
SPEC_DEVICE ItemLoc locate_item(int64_t x, const AttnArgs& a) {
  const int lane = threadIdx.x & 63;
  const int tail = a.lpt;
  const int rpb = a.rows_per_block;
  ItemLoc r;
  r.b = -1;
  r.kvh = r.rb = r.s = r.o = r.n = r.L = 0;
  r.ubase = -1;
  const bool phase_a = x < a.items_a;
  if (!phase_a) x -= a.items_a;
  int64_t running = 0;
  for (int base = 0; base < a.B; base += 64) {
    int bq = -1, nrb = 0, ns = 0, o = 0, n = 0, L = 0;
    int64_t cnt = 0;
    if (base + lane < a.B) {
      bq = phase_a ? base + lane : (int)a.order[base + lane];
      o = a.row_offsets[bq];
      n = a.row_offsets[bq + 1] - o;
      L = a.prefix_len[bq];
      nrb = attn_row_blocks(n, a.G, rpb);
      ns = attn_splits(L + n, attn_split_for(a.split, n, a.G, rpb, a.weighted));
      cnt = (int64_t)a.addr.hkv * nrb * (phase_a ? ns - tail : 1);
    }
    int64_t incl = cnt;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int64_t t = __shfl_up(incl, off, 64);
      if (lane >= off) incl += t;
    }
    const int64_t total = __shfl(incl, 63, 64);
    if (x < running + total) {
      const uint64_t hit = __ballot(running + incl > x);
      const int f = __ffsll((long long)hit) - 1;
      const int64_t local = x - running - __shfl(incl - cnt, f, 64);
      r.b = __shfl(bq, f, 64);
      r.o = __shfl(o, f, 64);
      r.n = __shfl(n, f, 64);
      r.L = __shfl(L, f, 64);
      const int nrb_b = __shfl(nrb, f, 64);
      const int ns_b = __shfl(ns, f, 64);
      if (phase_a) {
        const int nsa = ns_b - tail;
        r.s = (int)(local % nsa);
        r.rb = (int)((local / nsa) % nrb_b);
        r.kvh = (int)(local / ((int64_t)nsa * nrb_b));
      } else {
        r.s = ns_b - 1;
        r.rb = (int)(local % nrb_b);
        r.kvh = (int)(local / nrb_b);
      }
      if (a.B <= 64)      // every request is in this chunk (any order)
        r.ubase = wave_sum(bq >= 0 && bq < r.b ? (int64_t)a.addr.hkv * nrb : (int64_t)0);
      return r;
    }
    running += total;
  }
  return r;
}

typedef const __attribute__((address_space(1))) uint16_t* gptr_u16;
typedef const __attribute__((address_space(1))) void* gptr_void;
typedef __attribute__((address_space(3))) void* lptr_void;
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4* lptr_i16x4;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef const __attribute__((address_space(1))) u32x4* gptr_u4;

// s_waitcnt immediate: vmcnt <= n, expcnt and lgkmcnt left at their maxima.
#define SPEC_VMCNT(n) ((((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8)))
// s_waitcnt immediate: lgkmcnt == 0, vmcnt and expcnt left at their maxima.
#define SPEC_LGKMCNT0 0xc07f

// 16-byte load through an explicitly global pointer.
SPEC_DEVICE uint4 gload16(gptr_u16 p) {
  const u32x4 v = *(gptr_u4)p;
  return make_uint4(v.x, v.y, v.z, v.w);
}

// LDS layout of a 64-key tile (K or V), in 1 KB blocks: block
// (chunk group cg = c / 4, row group rg = row / 16) sits at block index
// cg * 4 + rg; inside it, 16-byte chunk c of key row r (r16 = r % 16) goes
// to slot 4 * r16 + ((c % 4) ^ (r16 / 4)).
//  * One direct-to-LDS instruction fills one block: lane l loads row l / 4 of
//    the group, so each 4-lane quad reads one contiguous 64-byte segment of
//    one key row (in-quad order permuted), which streams close to a plain
//    contiguous read.
//  * The 16-byte K reads (32 rows, one chunk) and the transposed V reads
//    (4 rows x 64 bytes per 32 lanes) both hit every bank exactly once per
//    cycle, and each lane needs only two base addresses (even / odd chunk);
//    everything else is a compile-time offset.
SPEC_DEVICE int tile_slot_bytes(int row, int c) {
  const int r16 = row & 15;
  return ((c >> 2) * 4 + (row >> 4)) * 1024 + (4 * r16 + ((c & 3) ^ (r16 >> 2))) * 16;
}

// Direct-to-LDS load of 16 bytes per lane from a uniform base plus a 32-bit
// per-lane byte offset: a raw buffer resource built in scalar registers for
// the base, so a lane keeps only its offset in a vector register (the same
// offset for every 16-key block of the whole tile).
constexpr int kBufferWord3 = 0x00020000;   // raw (untyped) buffer resource, gfx9 family
SPEC_DEVICE void dma16(gptr_u16 base, int lane_bytes, int scalar_bytes, uint16_t* dst) {
  // the base is the same in every lane; saying so keeps it in scalar
  // registers.  readfirstlane returns int: both halves go back through
  // uint32_t, or a low word with bit 31 set would sign-extend into the high
  // word.
  const uint64_t a = (uint64_t)base;
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  const uint64_t u = ((uint64_t)hi << 32) | lo;
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc((void*)u, 0, 0x7fffffff, kBufferWord3);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lptr_void)dst, 16, lane_bytes, scalar_bytes, 0, 0);
}

// Issue the direct-to-LDS loads of one 64-key K and V tile; each loading
// wave issues PER_WAVE of the tile's 1 KB blocks.  A block is 16 consecutive
// keys (one paged KV block: the tile start is 64-aligned), so its base
// address is uniform; lane l writes LDS slot l and loads the global chunk
// that the layout above puts there.
//  * Whole tiles (the common case): the tile's four block ids come from one
//    16-byte LDS read; per load only a scalar base changes.
//  * A tile that reaches the split end: keys at or past it read the split's
//    last key instead (finite data; they are masked out of the softmax), which
//    keeps every access inside the cache rows the caller owns.
template <int D, bool kBufferDma>
SPEC_DEVICE void issue_tile(uint16_t* ks, uint16_t* vs, gptr_u16 gk, gptr_u16 gv, int t0,
                            int key_end, bool paged, const int* s_blk, int blk0,
                            int64_t blk_stride, int wave, int lane) {
  constexpr int NB = D / 8;                  // 1 KB blocks per K (or V) tile
  constexpr int PER_WAVE = 2 * NB / kDmaWaves;
  if (wave >= kDmaWaves) return;             // wide workgroups: the other waves load nothing
  const int rr = lane >> 2;                  // key row inside the 16-key group
  const int cl = (lane & 3) ^ (lane >> 4);   // chunk inside the 4-chunk group
  const int last = key_end - 1;
  if (t0 + kTileKeys <= key_end) {
    int b0, b1, b2, b3;                      // element offsets / stride of the 4 blocks
    int64_t stride;
    if (paged) {
      const int4 ids = *reinterpret_cast<const int4*>(s_blk + ((t0 >> 4) - blk0));
      b0 = __builtin_amdgcn_readfirstlane(ids.x);
      b1 = __builtin_amdgcn_readfirstlane(ids.y);
      b2 = __builtin_amdgcn_readfirstlane(ids.z);
      b3 = __builtin_amdgcn_readfirstlane(ids.w);
      stride = blk_stride;
    } else {
      b0 = t0 >> 4;
      b1 = b0 + 1;
      b2 = b0 + 2;
      b3 = b0 + 3;
      stride = (int64_t)kBlock * D;
    }
    const int lane_bytes = (rr * D + cl * 8) * 2;    // inside a block
#pragma unroll
    for (int j = 0; j < PER_WAVE; ++j) {
      const int gi = wave * PER_WAVE + j;    // uniform
      const bool isv = gi >= NB;
      const int bi = isv ? gi - NB : gi;
      const int grp = bi & 3;
      const int bid = (grp == 0) ? b0 : (grp == 1) ? b1 : (grp == 2) ? b2 : b3;
      // block base by the block id (changes every tile); the chunk group
      // (bi / 4: 32 elements) as the scalar offset
      const gptr_u16 bb = (isv ? gv : gk) + (int64_t)bid * stride;
      uint16_t* dst = (isv ? vs : ks) + bi * 512;
      if (kBufferDma)
        dma16(bb, lane_bytes, (bi >> 2) * 64, dst);
      else
        __builtin_amdgcn_global_load_lds((gptr_void)(bb + (bi >> 2) * 32 + lane_bytes / 2),
                                         (lptr_void)dst, 16, 0, 0);
    }
    return;
  }
#pragma unroll
  for (int j = 0; j < PER_WAVE; ++j) {
    const int gi = wave * PER_WAVE + j;      // uniform
    const bool isv = gi >= NB;
    const int bi = isv ? gi - NB : gi;
    const int grp = bi & 3;
    const int gs = min(t0 + 16 * grp, last);
    const int blk = gs >> 4;
    const int64_t base =
        paged ? (int64_t)__builtin_amdgcn_readfirstlane(s_blk[blk - blk0]) * blk_stride
              : (int64_t)blk * (kBlock * D);
    const int key = min(t0 + 16 * grp + rr, last);     // same 16-key block as gs
    const int c = (bi >> 2) * 4 + cl;
    const int lb = ((key & 15) * D + c * 8) * 2;
    if (kBufferDma)
      dma16((isv ? gv : gk) + base, lb, 0, (isv ? vs : ks) + bi * 512);
    else
      __builtin_amdgcn_global_load_lds((gptr_void)((isv ? gv : gk) + base + lb / 2),
                                       (lptr_void)((isv ? vs : ks) + bi * 512), 16, 0, 0);
  }
}

// Maximum / sum of the two values a query row holds in lanes l and l ^ 32
// (v_permlane32_swap: each lane ends up with both halves' values).
SPEC_DEVICE float row_pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
SPEC_DEVICE float row_pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Visibility of keys kb0 .. kb0+31 for one query row: a prefix key (< L)
// always, tree key L + j when bit j of the row's ancestor mask is set, and
// nothing at or past key_end.
SPEC_DEVICE uint32_t visible_bits(int kb0, int L, int key_end, uint64_t mw0, uint64_t mw1,
                                  uint64_t mw2, uint64_t mw3) {
  const int r = kb0 - L;
  uint64_t tree;
  if (r >= 0) {
    const int w = r >> 6, s = r & 63;
    const uint64_t lo = (w == 0) ? mw0 : (w == 1) ? mw1 : (w == 2) ? mw2 : mw3;
    const uint64_t hi = (w == 0) ? mw1 : (w == 1) ? mw2 : (w == 2) ? mw3 : 0ull;
    tree = s ? ((lo >> s) | (hi << (64 - s))) : lo;
  } else {
    tree = (r <= -64) ? 0ull : (mw0 << (-r));
  }
  const int np = min(max(L - kb0, 0), 32);
  const uint32_t pre = (np >= 32) ? 0xffffffffu : ((1u << np) - 1u);
  const int nv = min(max(key_end - kb0, 0), 32);
  const uint32_t lim = (nv >= 32) ? 0xffffffffu : ((1u << nv) - 1u);
  return ((uint32_t)tree | pre) & lim;
}

// Pieces of the per-wave tile computation, for one 32-key half (hk) of a
// staged tile and one wave's 32 query rows.
// S^T = K Q^T (a 32x32 block); sc[e] is the score of key
// kb0 + half*4 + 8*(e/4) + e%4 (C layout of S^T).
// Scheduling-group masks (instruction classes) for the lean variants below.
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;

// kLean (12-wave workgroups, three waves per SIMD): the fragment reads are
// kept two MFMAs ahead instead of all hoisted, which holds the registers to
// what three waves per SIMD allow.
template <int D, bool kLean = false>
SPEC_DEVICE f32x16 half_scores(const uint16_t* ks, int hk, int lane,
                               const bf16x8 (&qf)[D / 16]) {
  constexpr int NKS = D / 16;
  const int col = lane & 31, half = lane >> 5;
  f32x16 sc;
#pragma unroll
  for (int e = 0; e < 16; ++e) sc[e] = 0.0f;
  const int krow = hk * 32 + col;
#pragma unroll
  for (int kk = 0; kk < NKS; ++kk) {
    const bf16x8 kf = *reinterpret_cast<const bf16x8*>(reinterpret_cast<const char*>(ks) +
                                                       tile_slot_bytes(krow, kk * 2 + half));
    sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[kk], sc, 0, 0, 0);
  }
  if (kLean) {
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
#pragma unroll
    for (int i = 0; i < NKS - 2; ++i) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 2, 0);
  }
  return sc;
}

// Online softmax in the exp2 domain with a lazily moved reference
// (scale_log2 > 0, so the row maximum commutes with the scaling): a row's
// reference m only moves when a score exceeds it by more than kLazyMax (log2
// units), so p = 2^(s - m) stays <= 2^kLazyMax and the O/l rescale is rare.
// O/l is unchanged by the choice of reference.  Returns whether this lane's
// row moved with O != 0 (then O must be scaled by alpha before the next
// P V^T).
SPEC_DEVICE bool half_softmax(const f32x16& sc, float scale_log2, float& m_run, float& l_run,
                              bf16x8 (&pb)[2], float& alpha) {
  float mx = sc[0];
#pragma unroll
  for (int e = 1; e < 16; ++e) mx = fmaxf(mx, sc[e]);
  mx = row_pair_max(mx);
  const float cand = mx * scale_log2;
  const bool move = cand > m_run + kLazyMax;          // false for a fully masked row
  const float m_new = move ? cand : m_run;
  // A row with no visible key yet keeps m = -inf; 0 as the reference then
  // gives alpha = 0 and p = 0 without a divergent branch.
  const float m_ref = (m_new == -INFINITY) ? 0.0f : m_new;
  alpha = __builtin_amdgcn_exp2f(m_run - m_ref);
  float rs = 0.0f;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const float p = __builtin_amdgcn_exp2f(fmaf(sc[e], scale_log2, -m_ref));
    rs += p;
    pb[e >> 3][e & 7] = (__bf16)p;
  }
  rs = row_pair_sum(rs);
  l_run = l_run * alpha + rs;
  // Rows seen for the first time have O = 0 and need no rescale.
  const bool rescale = move && m_run != -INFINITY;
  m_run = m_new;
  return rescale;
}

template <int D>
SPEC_DEVICE void scale_acc(f32x16 (&acc)[D / 32], float alpha) {
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[db][e] *= alpha;
}

// O^T += V^T P^T.  V^T operand by transposed LDS reads: this lane supplies
// the address of 4 dims of one key; lane 4q+c of each 16-lane group receives
// dim dbase+4q+c of 4 consecutive keys.  The k-slots of P^T (key
// half*4 + 8*(e/4) + e%4 of each 16-key step) and of V^T follow the same
// order.
template <int D, bool kLean = false>
SPEC_DEVICE void half_pv(const uint16_t* vs, int hk, int lane, const bf16x8 (&pb)[2],
                         f32x16 (&acc)[D / 32]) {
  constexpr int NDB = D / 32;
  const int grp = lane >> 4, j = lane & 15;
  const int h = grp >> 1;
  const int dsub = (grp & 1) * 16 + 4 * (j & 3);
  const int ksub = j >> 2;
  const char* vbase = reinterpret_cast<const char*>(vs);
#pragma unroll
  for (int mm = 0; mm < 2; ++mm) {
    const int kb = hk * 32 + mm * 16 + h * 4;
    const int ra = kb + ksub, rb = kb + 8 + ksub;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int dim = db * 32 + dsub;
      const uint16_t* pa =
          reinterpret_cast<const uint16_t*>(vbase + tile_slot_bytes(ra, dim >> 3)) + (dim & 7);
      const uint16_t* pbp =
          reinterpret_cast<const uint16_t*>(vbase + tile_slot_bytes(rb, dim >> 3)) + (dim & 7);
      const i16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lptr_i16x4)pa);
      const i16x4 vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lptr_i16x4)pbp);
      const bf16x8 vf = __builtin_bit_cast(
          bf16x8, make_uint4(__builtin_bit_cast(uint2, va).x, __builtin_bit_cast(uint2, va).y,
                             __builtin_bit_cast(uint2, vb).x, __builtin_bit_cast(uint2, vb).y));
      acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[mm], acc[db], 0, 0, 0);
    }
  }
  if (kLean) {
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 4, 0);
#pragma unroll
    for (int i = 0; i < 2 * NDB - 2; ++i) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 2, 0);
  }
}

// One 32-key half (hk) of a staged tile for one wave's 32 query rows:
// scores, mask (tiles at the tree or split end), online softmax, P V^T.
// kb0 is the absolute index of the half's first key.
template <int D, bool kLean = false>
SPEC_DEVICE void compute_half(const uint16_t* ks, const uint16_t* vs, int hk, int kb0, int lane,
                              int L, int key_end, float scale_log2, const uint64_t* mw,
                              const bf16x8 (&qf)[D / 16],
                              f32x16 (&acc)[D / 32], float& m_run, float& l_run) {
  const int half = lane >> 5;
  f32x16 sc = half_scores<D, kLean>(ks, hk, lane, qf);
  if (kb0 + 32 > min(L, key_end)) {          // uniform: only tiles at the tree or split end
    const uint32_t vis = visible_bits(kb0, L, key_end, mw[0], mw[1], mw[2], mw[3]);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int i = half * 4 + 8 * (e >> 2) + (e & 3);
      sc[e] = ((vis >> i) & 1u) ? sc[e] : -INFINITY;
    }
  }
  bf16x8 pb[2];
  float alpha;
  if (__any(half_softmax(sc, scale_log2, m_run, l_run, pb, alpha))) scale_acc<D>(acc, alpha);
  half_pv<D, kLean>(vs, hk, lane, pb, acc);
}

// A whole tile of prefix keys (no mask) for one wave's 32 rows, pipelined
// inside the wave: both halves' scores are issued first, so the second
// half's MFMAs run while the first half's softmax occupies the vector ALUs,
// and the first half's P V^T runs during the second half's softmax.
template <int D>
SPEC_DEVICE void compute_tile_full(const uint16_t* ks, const uint16_t* vs, int lane,
                                   float scale_log2, const bf16x8 (&qf)[D / 16],
                                   f32x16 (&acc)[D / 32], float& m_run, float& l_run) {
  // Raised priority while the scores are issued: of the two waves sharing a
  // SIMD, the first to get here finishes its MFMAs first and moves on to
  // its softmax while the other one's MFMAs run.
  __builtin_amdgcn_s_setprio(1);
  const f32x16 s0 = half_scores<D>(ks, 0, lane, qf);
  const f32x16 s1 = half_scores<D>(ks, 1, lane, qf);
  __builtin_amdgcn_s_setprio(0);
  bf16x8 p0[2], p1[2];
  float a0, a1;
  if (__any(half_softmax(s0, scale_log2, m_run, l_run, p0, a0))) scale_acc<D>(acc, a0);
  half_pv<D>(vs, 0, lane, p0, acc);
  if (__any(half_softmax(s1, scale_log2, m_run, l_run, p1, a1))) scale_acc<D>(acc, a1);
  half_pv<D>(vs, 1, lane, p1, acc);
}

// First (request, KV head, row block) unit of request b: units of all
// earlier requests, in request order.  Wave-parallel; uniform.
SPEC_DEVICE int64_t unit_base(const AttnArgs& a, int b) {
  const int lane = threadIdx.x & 63;
  int64_t cnt = 0;
  for (int base = 0; base < b; base += 64) {
    const int bq = base + lane;
    if (bq < b)
      cnt += (int64_t)a.addr.hkv *
             attn_row_blocks(a.row_offsets[bq + 1] - a.row_offsets[bq], a.G, a.rows_per_block);
  }
  return wave_sum(cnt);
}

// Main kernel: one workgroup of 8 waves per (request, KV head, block of up
// to 256 query rows, key split).  Query rows form groups of 32 (one wave's
// MFMA columns).  With at most 4 groups, two waves share a group and each
// takes one 32-key half of every tile (their partial softmax states merge at
// the end), so small trees still keep every SIMD busy.  K/V tiles of 64 keys
// stream through a 4-stage LDS ring filled by direct-to-LDS loads, three
// tiles ahead of the compute.
template <int D, int W>
__global__ void __launch_bounds__(W * 64, 1) attn_bf16_kernel(AttnArgs a) {
  constexpr int NKS = D / 16;
  constexpr int NDB = D / 32;
  constexpr int ROWS = W * kRowsPerWave;
  constexpr int TILE = kTileKeys * D;                 // bf16 per K (or V) tile
  constexpr int PER_WAVE = 2 * (D / 8) / kDmaWaves;   // DMA blocks per loading wave per tile
  static_assert(PER_WAVE * 3 < 64, "vmcnt range");
  static_assert(W == kWaves || W == kWideWaves, "workgroup shapes");
  __shared__ __attribute__((aligned(16))) uint16_t k0[TILE], k1[TILE], k2[TILE], k3[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t v0[TILE], v1[TILE], v2[TILE], v3[TILE];
  __shared__ __attribute__((aligned(16))) int s_blk[kMaxSplit / kBlock + 4];
  __shared__ uint64_t s_mask[ROWS * 4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // Items in the order workgroups start, across all XCDs: the dispatcher
  // deals workgroups to the XCDs round-robin, and the XCDs stream at
  // different rates, so a fixed blockIdx -> item map leaves the slow XCDs
  // finishing last.  atomicInc wraps at items - 1, so every item is taken
  // exactly once whatever the counter held (the combine resets it to 0 for
  // the next call, and only a first call on a fresh workspace starts the
  // longest-first order elsewhere); an out-of-range start value is returned
  // once and replaced by 0.
  __shared__ int s_item;
  int64_t item = blockIdx.x;
  if (a.ticket) {
    if (tid == 0) {
      unsigned t = atomicInc(a.ticket, (unsigned)(a.items - 1));
      if (t >= (unsigned)a.items) t = atomicInc(a.ticket, (unsigned)(a.items - 1));
      s_item = (int)t;
    }
    __syncthreads();
    item = s_item;
  }
  const ItemLoc loc = locate_item(item, a);
  // Uniform results of the wave-parallel search.  The wide variant says so
  // (its K/V bases then stay in scalar registers for the buffer-resource
  // loads); the 8-wave one keeps the allocation measured fastest for it.
  const int b = (W > kWaves) ? __builtin_amdgcn_readfirstlane(loc.b) : loc.b;
  if (b < 0) return;
  const int kvh = (W > kWaves) ? __builtin_amdgcn_readfirstlane(loc.kvh) : loc.kvh;
  const int rb = (W > kWaves) ? __builtin_amdgcn_readfirstlane(loc.rb) : loc.rb;
  const int s = (W > kWaves) ? __builtin_amdgcn_readfirstlane(loc.s) : loc.s;
  const int o = __builtin_amdgcn_readfirstlane(loc.o);
  const int n = __builtin_amdgcn_readfirstlane(loc.n);
  const int L = __builtin_amdgcn_readfirstlane(loc.L);
  const int total_keys = L + n;
  const int split = attn_split_for(a.split, n, a.G, ROWS, a.weighted);
  const int ns = attn_splits(total_keys, split);
  const int key_begin = __builtin_amdgcn_readfirstlane(s * split);
  const int key_end = __builtin_amdgcn_readfirstlane(s == ns - 1 ? total_keys : key_begin + split);
  const int M = n * a.G;

  if (a.max_ns > 1) {
    // the combine finds each unit's splits here (no search over requests)
    const int64_t ub = loc.ubase >= 0 ? loc.ubase : unit_base(a, b);
    const int64_t unit = ub + (int64_t)kvh * attn_row_blocks(n, a.G, ROWS) + rb;
    if (tid == 0) {
      a.unit_items[unit * a.max_ns + s] = (int)item;
      if (s == 0) {
        int* d = a.unit_desc + unit * 8;
        d[0] = b;
        d[1] = kvh;
        d[2] = rb;
        d[3] = ns;
        d[4] = o;
        d[5] = min(ROWS, M - rb * ROWS);
      }
    }
  }
  const int groups = (min(ROWS, M - rb * ROWS) + kRowsPerWave - 1) / kRowsPerWave;
  const bool pair = groups <= W / 2;
  const int g = pair ? (wave >> 1) : wave;
  const int h_lo = pair ? (wave & 1) : 0;
  const int h_hi = pair ? h_lo + 1 : 2;
  const bool wave_active = g < groups;

  const int col = lane & 31, half = lane >> 5;
  const int row = rb * ROWS + g * kRowsPerWave + col;
  const bool row_ok = wave_active && row < M;
  const int ti = row_ok ? row / a.G : 0;
  const int hh = kvh * a.G + (row_ok ? row % a.G : 0);
  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[db][e] = 0.0f;
  float m_run = -INFINITY;
  float l_run = 0.0f;

  // Paged caches: the split's block ids go to LDS once.
  const int blk0 = key_begin >> 4;
  const bool paged = a.addr.paged;
  const uint16_t* kbase;
  const uint16_t* vbase;
  if (paged) {
    const int nblk = ((key_end + kBlock - 1) >> 4) - blk0;
    for (int i = tid; i < nblk; i += W * 64)
      s_blk[i] = a.addr.block_table[(int64_t)b * a.addr.mbps + blk0 + i];
    kbase = a.k + (int64_t)kvh * kBlock * D;
    vbase = a.v + (int64_t)kvh * kBlock * D;
  } else {
    const int64_t off = ((int64_t)b * a.addr.hkv + kvh) * a.addr.capacity * D;
    kbase = a.k + off;
    vbase = a.v + off;
  }
  const int64_t blk_stride = (int64_t)a.addr.hkv * kBlock * D;
  const gptr_u16 gk = (gptr_u16)kbase;
  const gptr_u16 gv = (gptr_u16)vbase;
  __syncthreads();

  // Ring of 4 stages: tile t lives in stage t % 4.  Step t waits for this
  // wave's loads of tile t (tiles t+1 and t+2 stay in flight; loads complete
  // in issue order), meets the other waves -- after which all of them are
  // done with tile t-1 -- refills that tile's stage with tile t+3, and
  // computes tile t.  No tile past the split is issued, and the last steps
  // wait for correspondingly fewer loads in flight.
  const int ntiles = (key_end - key_begin + kTileKeys - 1) / kTileKeys;
  issue_tile<D, (W > kWaves)>(k0, v0, gk, gv, key_begin, key_end, paged, s_blk, blk0, blk_stride, wave, lane);
  if (ntiles > 1)
    issue_tile<D, (W > kWaves)>(k1, v1, gk, gv, key_begin + kTileKeys, key_end, paged, s_blk, blk0, blk_stride,
                  wave, lane);
  if (ntiles > 2)
    issue_tile<D, (W > kWaves)>(k2, v2, gk, gv, key_begin + 2 * kTileKeys, key_end, paged, s_blk, blk0,
                  blk_stride, wave, lane);
  // The query rows and mask words load while the first tiles stream in.
  bf16x8 qf[NKS];
  // This lane's row's mask words go to LDS (read only at tiles that need
  // them, by this wave alone; both waves of a pair write the same values).
  uint64_t* mw = s_mask + 4 * (g * kRowsPerWave + col);
  uint64_t mw0 = 0, mw1 = 0, mw2 = 0, mw3 = 0;
  if (row_ok) {
    const uint16_t* qp = a.q + ((int64_t)(o + ti) * a.hq + hh) * D + half * 8;
#pragma unroll
    for (int kk = 0; kk < NKS; ++kk)
      qf[kk] = __builtin_bit_cast(bf16x8, gload16((gptr_u16)(qp + kk * 16)));
    const uint64_t* mrow = a.mask + (int64_t)(o + ti) * a.words;
    mw0 = mrow[0];
    if (a.words > 1) mw1 = mrow[1];
    if (a.words > 2) mw2 = mrow[2];
    if (a.words > 3) mw3 = mrow[3];
  } else {
#pragma unroll
    for (int kk = 0; kk < NKS; ++kk)
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[kk][e] = (__bf16)0.0f;
  }
  if (wave_active && half == 0) {
    mw[0] = mw0;
    mw[1] = mw1;
    mw[2] = mw2;
    mw[3] = mw3;
  }

#define SPEC_ATTN_STEP(KC, VC, KN, VN, T)                                                       \
  {                                                                                              \
    const int t0_ = key_begin + (T) * kTileKeys;                                                 \
    if (W > kDmaWaves && wave >= kDmaWaves)                                                      \
      __builtin_amdgcn_s_waitcnt(SPEC_VMCNT(0));                                                 \
    else if ((T) + 2 < ntiles)                                                                   \
      __builtin_amdgcn_s_waitcnt(SPEC_VMCNT(2 * PER_WAVE));                                      \
    else if ((T) + 1 < ntiles)                                                                   \
      __builtin_amdgcn_s_waitcnt(SPEC_VMCNT(PER_WAVE));                                          \
    else                                                                                         \
      __builtin_amdgcn_s_waitcnt(SPEC_VMCNT(0));                                                 \
    __builtin_amdgcn_s_barrier();                                                                \
    if ((T) + 3 < ntiles)                                                                        \
      issue_tile<D, (W > kWaves)>(KN, VN, gk, gv, t0_ + 3 * kTileKeys, key_end, paged, s_blk, blk0,            \
                    blk_stride, wave, lane);                                                     \
    if (wave_active) {                                                                           \
      if (W == kWaves && !pair && t0_ + kTileKeys <= min(L, key_end)) {                          \
        compute_tile_full<D>(KC, VC, lane, a.scale_log2, qf, acc, m_run, l_run);                 \
      } else {                                                                                   \
        for (int hk = h_lo; hk < h_hi; ++hk)                                                     \
          compute_half<D, (W > kWaves)>(KC, VC, hk, t0_ + 32 * hk, lane, L, key_end,             \
                                        a.scale_log2, mw, qf,                                    \
                          acc, m_run, l_run);                                                    \
      }                                                                                          \
    }                                                                                            \
    __builtin_amdgcn_s_waitcnt(SPEC_LGKMCNT0);                                                   \
  }

  for (int t = 0; t < ntiles; t += kStages) {
    SPEC_ATTN_STEP(k0, v0, k3, v3, t);
    if (t + 1 >= ntiles) break;
    SPEC_ATTN_STEP(k1, v1, k0, v0, t + 1);
    if (t + 2 >= ntiles) break;
    SPEC_ATTN_STEP(k2, v2, k1, v1, t + 2);
    if (t + 3 >= ntiles) break;
    SPEC_ATTN_STEP(k3, v3, k2, v2, t + 3);
  }
#undef SPEC_ATTN_STEP
  // Drain the loads still in flight (clamped tail tiles); then the ring is
  // free for the merge of the two key halves of each row group.
  __builtin_amdgcn_s_waitcnt(SPEC_VMCNT(0));
  __syncthreads();
  constexpr int NV4 = NDB * 4;                         // float4 per lane of acc
  // Pair mode: the odd wave of each group hands its (m, l, O) to the even
  // one through the idle ring (group g in a 16 KB stage buffer, the (m, l)
  // pairs in v0).
  static_assert(W / 2 <= 6, "merge slots");
  if (pair && wave_active && (wave & 1)) {
    uint16_t* slot = (g == 0) ? k0 : (g == 1) ? k1 : (g == 2) ? k2 : (g == 3) ? k3 : (g == 4) ? v1 : v2;
    float4* xs = reinterpret_cast<float4*>(slot);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int ai = 0; ai < 4; ++ai)
        xs[(db * 4 + ai) * 64 + lane] = make_float4(acc[db][4 * ai], acc[db][4 * ai + 1],
                                                    acc[db][4 * ai + 2], acc[db][4 * ai + 3]);
    float2* ml = reinterpret_cast<float2*>(v0) + g * 64 + lane;
    *ml = make_float2(m_run, l_run);
  }
  static_assert(NV4 * 64 * 16 <= TILE * 2, "merge slot size");
  __syncthreads();
  if (pair && (wave & 1)) return;
  if (!row_ok) return;
  if (pair) {
    const uint16_t* slot = (g == 0) ? k0 : (g == 1) ? k1 : (g == 2) ? k2 : (g == 3) ? k3 : (g == 4) ? v1 : v2;
    const float4* xs = reinterpret_cast<const float4*>(slot);
    const float2 ml = reinterpret_cast<const float2*>(v0)[g * 64 + lane];
    const float m_new = fmaxf(m_run, ml.x);
    const float m_ref = (m_new == -INFINITY) ? 0.0f : m_new;
    const float a0 = __builtin_amdgcn_exp2f(m_run - m_ref);
    const float a1 = __builtin_amdgcn_exp2f(ml.x - m_ref);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int ai = 0; ai < 4; ++ai) {
        const float4 x = xs[(db * 4 + ai) * 64 + lane];
        acc[db][4 * ai] = acc[db][4 * ai] * a0 + x.x * a1;
        acc[db][4 * ai + 1] = acc[db][4 * ai + 1] * a0 + x.y * a1;
        acc[db][4 * ai + 2] = acc[db][4 * ai + 2] * a0 + x.z * a1;
        acc[db][4 * ai + 3] = acc[db][4 * ai + 3] * a0 + x.w * a1;
      }
    l_run = l_run * a0 + ml.y * a1;
    m_run = m_new;
  }
  // acc[db][4*ai + c] holds output dim db*32 + half*4 + 8*ai + c of this row.
  if (ns == 1) {
    const float inv = 1.0f / l_run;
    const int64_t obase = ((int64_t)(o + ti) * a.hq + hh) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int ai = 0; ai < 4; ++ai) {
        const int d0 = db * 32 + half * 4 + 8 * ai;
        const float v0f = acc[db][4 * ai] * inv, v1f = acc[db][4 * ai + 1] * inv;
        const float v2f = acc[db][4 * ai + 2] * inv, v3f = acc[db][4 * ai + 3] * inv;
        if (a.out_f32) {
          *reinterpret_cast<float4*>((float*)a.out + obase + d0) = make_float4(v0f, v1f, v2f, v3f);
        } else {
          uint2 pk;
          pk.x = f32_to_bf16_bits(v0f) | ((uint32_t)f32_to_bf16_bits(v1f) << 16);
          pk.y = f32_to_bf16_bits(v2f) | ((uint32_t)f32_to_bf16_bits(v3f) << 16);
          *reinterpret_cast<uint2*>((uint16_t*)a.out + obase + d0) = pk;
        }
      }
  } else if (a.out_f32) {
    const int r_in_block = g * kRowsPerWave + col;
    float* pp = a.part + (item * ROWS + r_in_block) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int ai = 0; ai < 4; ++ai) {
        const int d0 = db * 32 + half * 4 + 8 * ai;
        *reinterpret_cast<float4*>(pp + d0) =
            make_float4(acc[db][4 * ai], acc[db][4 * ai + 1], acc[db][4 * ai + 2], acc[db][4 * ai + 3]);
      }
    if (half == 0) {
      float* ml = a.part_ml + (item * ROWS + r_in_block) * 2;
      ml[0] = m_run;
      ml[1] = l_run;
    }
  } else {
    // bf16 output: the partial is stored normalised, y = O / l in fp16 (a
    // convex combination of V rows, |y| <= max |V|; 2^-11 relative, finer
    // than the bf16 output), half the bytes of the fp32 form.  A row whose
    // largest |y| reaches 2^15 is stored as y * 2^-e instead (e < 128), and
    // e travels in the low 7 bits of its l, which is then stored negated.
    const int r_in_block = g * kRowsPerWave + col;
    const float inv = (l_run > 0.0f) ? 1.0f / l_run : 0.0f;
    float mx = 0.0f;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, fabsf(acc[db][i]));
    mx = row_pair_max(mx * inv);
    int e = 0;
    if (mx >= 32768.0f && mx <= 3.4e38f) {
      int k;
      frexpf(mx, &k);                                // mx < 2^k, k <= 128
      e = k - 15;
    }
    const float sc = e ? ldexpf(inv, -e) : inv;
    _Float16* ph = reinterpret_cast<_Float16*>(a.part) + (item * ROWS + r_in_block) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int ai = 0; ai < 4; ++ai) {
        const int d0 = db * 32 + half * 4 + 8 * ai;
        const _Float16 h0 = (_Float16)(acc[db][4 * ai] * sc), h1 = (_Float16)(acc[db][4 * ai + 1] * sc);
        const _Float16 h2 = (_Float16)(acc[db][4 * ai + 2] * sc), h3 = (_Float16)(acc[db][4 * ai + 3] * sc);
        uint2 pk;
        pk.x = (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
        pk.y = (uint32_t)__builtin_bit_cast(uint16_t, h2) | ((uint32_t)__builtin_bit_cast(uint16_t, h3) << 16);
        *reinterpret_cast<uint2*>(ph + d0) = pk;
      }
    if (half == 0) {
      float* ml = a.part_ml + (item * ROWS + r_in_block) * 2;
      ml[0] = m_run;
      ml[1] = e ? -__uint_as_float((__float_as_uint(l_run) & ~127u) | (uint32_t)e) : l_run;
    }
  }
}

// Arguments of the combine: the main kernel's partials and unit tables, and
// which (unit, 32-row chunk) each workgroup takes.
struct CombineArgs {
  const float* part;
  const float* part_ml;
  const int* unit_desc;
  const int* unit_items;
  int max_ns;
  int hq;
  int G;
  void* out;
  int out_f32;
  unsigned* ticket;   // the main kernel's item counter, reset here for the next call
  int chunks;         // workgroups per unit (enough for its rows)
  int hkv;
  int nreq;           // > 0: only the units of req[0 .. nreq) (unit = b * hkv + KV head)
  uint16_t req[kLptMax];
};

// Merge split partials.  One workgroup per 32 query rows of one (request, KV
// head, row block); each thread merges one 4-wide column of a row over the
// splits in one pass with a running maximum (coalesced rows of partials:
// fp32 O for fp32 output, normalised fp16 O / l for bf16 output; weights
// exp2(m_s - m)).  The grid covers only chunks that can
// hold rows (and, when the requests are listed, only units with partials),
// so few workgroups start just to find nothing to do.
template <int D, int W, bool kHalf>
__global__ void __launch_bounds__(256) attn_combine_kernel(CombineArgs a) {
  constexpr int C4 = D / 4;                        // float4 per row
  constexpr int RPI = 256 / C4;                    // rows per pass of the block
  int64_t unit;
  int chunk;
  if (a.nreq > 0) {
    const int per_req = a.hkv * a.chunks;
    const int i = blockIdx.x / per_req;
    const int rem = blockIdx.x - i * per_req;
    unit = (int64_t)a.req[i] * a.hkv + rem / a.chunks;
    chunk = rem % a.chunks;
  } else {
    unit = blockIdx.x / a.chunks;
    chunk = blockIdx.x % a.chunks;
  }
  const int4 d0 = *reinterpret_cast<const int4*>(a.unit_desc + unit * 8);
  const int2 d1 = *reinterpret_cast<const int2*>(a.unit_desc + unit * 8 + 4);
  const int kvh = d0.y, rb = d0.z, ns = d0.w, o = d1.x, m_blk = d1.y;
  if (blockIdx.x == 0 && threadIdx.x == 0 && a.ticket) *a.ticket = 0u;   // for the next call
  if (ns == 1) return;
  const int r0 = chunk * kCombineRows;             // first row (within the block)
  const int rows = min(kCombineRows, m_blk - r0);
  if (rows <= 0) return;
  // Item of each split of this unit, kept in LDS for the loop below.
  __shared__ int s_item[kMaxSplitsCombine];
  for (int sp = threadIdx.x; sp < ns; sp += blockDim.x) s_item[sp] = a.unit_items[unit * a.max_ns + sp];
  __syncthreads();
  const float2* ml = reinterpret_cast<const float2*>(a.part_ml);
  // One pass over the splits per (row, float4 column), with a running
  // maximum.  A thread owns one column of kCombineRows / RPI rows; their
  // loads are unconditional (row index clamped) so that all of them are in
  // flight together.
  constexpr int NP = kCombineRows / RPI;
  constexpr int ROWS = W * kRowsPerWave;
  const int c4 = threadIdx.x % C4;
  const int rsub = threadIdx.x / C4;
  float mx[NP], l[NP];
  float4 accv[NP];
#pragma unroll
  for (int rp = 0; rp < NP; ++rp) {
    mx[rp] = -INFINITY;
    l[rp] = 0.0f;
    accv[rp] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
#pragma unroll 2
  for (int s = 0; s < ns; ++s) {
    const int64_t base = (int64_t)s_item[s] * ROWS + r0;
#pragma unroll
    for (int rp = 0; rp < NP; ++rp) {
      const int64_t pr = base + min(rp * RPI + rsub, rows - 1);
      const float2 v = ml[pr];
      float4 pv;
      float lw = v.y, yscale = 1.0f;
      if (kHalf) {
        // normalised fp16 partial y = O / l (times 2^-e when l is stored negated)
        const uint2 hv = *reinterpret_cast<const uint2*>(
            reinterpret_cast<const _Float16*>(a.part) + pr * D + c4 * 4);
        pv = make_float4((float)__builtin_bit_cast(_Float16, (uint16_t)(hv.x & 0xffffu)),
                         (float)__builtin_bit_cast(_Float16, (uint16_t)(hv.x >> 16)),
                         (float)__builtin_bit_cast(_Float16, (uint16_t)(hv.y & 0xffffu)),
                         (float)__builtin_bit_cast(_Float16, (uint16_t)(hv.y >> 16)));
        if (lw < 0.0f) {
          lw = -lw;
          yscale = ldexpf(1.0f, (int)(__float_as_uint(lw) & 127u));
        }
        yscale *= lw;
      } else {
        pv = *reinterpret_cast<const float4*>(a.part + pr * D + c4 * 4);
      }
      if (v.x > mx[rp]) {                            // new maximum: rescale what is summed
        const float sc = (mx[rp] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(mx[rp] - v.x);
        accv[rp].x *= sc; accv[rp].y *= sc; accv[rp].z *= sc; accv[rp].w *= sc;
        l[rp] *= sc;
        mx[rp] = v.x;
      }
      const float wgt = (v.x == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(v.x - mx[rp]);
      l[rp] += lw * wgt;
      const float yw = yscale * wgt;                 // fp32 partials: O itself (yscale 1)
      accv[rp].x += pv.x * yw; accv[rp].y += pv.y * yw;
      accv[rp].z += pv.z * yw; accv[rp].w += pv.w * yw;
    }
  }
#pragma unroll
  for (int rp = 0; rp < NP; ++rp) {
    const int r = rp * RPI + rsub;
    if (r >= rows) break;
    const float inv = 1.0f / l[rp];
    const int grow = rb * ROWS + r0 + r;
    const int ti = grow / a.G;
    const int hh = kvh * a.G + grow % a.G;
    const int64_t obase = ((int64_t)(o + ti) * a.hq + hh) * D + c4 * 4;
    const float4 v = accv[rp];
    if (a.out_f32) {
      *reinterpret_cast<float4*>((float*)a.out + obase) =
          make_float4(v.x * inv, v.y * inv, v.z * inv, v.w * inv);
    } else {
      uint2 pk;
      pk.x = f32_to_bf16_bits(v.x * inv) | ((uint32_t)f32_to_bf16_bits(v.y * inv) << 16);
      pk.y = f32_to_bf16_bits(v.z * inv) | ((uint32_t)f32_to_bf16_bits(v.w * inv) << 16);
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
  AttnPlan p;
  // 8 waves of 32 query rows: most (request, KV head) pairs fit in one
  // workgroup, so every KV tile is read once.  A batch with a pair of more
  // than 256 query rows (the 70B-shaped K-schedule trees: 46 rows x 8 heads
  // of a group = 368) takes 12 waves (384 rows, three per SIMD) instead, so
  // that such a pair is still one workgroup reading each tile once.
  int max_unit_rows = 0;
  for (int b = 0; b < B; ++b)
    max_unit_rows = std::max(max_unit_rows, (row_offsets_h[b + 1] - row_offsets_h[b]) * G);
  p.rows_per_block = (max_unit_rows > kWaves * kRowsPerWave ? kWideWaves : kWaves) * kRowsPerWave;
  int64_t work = 0, units = 0, max_keys = 0, min_keys = INT64_MAX;
  for (int b = 0; b < B; ++b) {
    const int n = row_offsets_h[b + 1] - row_offsets_h[b];
    const int nrb = attn_row_blocks(n, G, p.rows_per_block);
    units += (int64_t)hkv * nrb;
    work += (int64_t)hkv * nrb * (prefix_len_h[b] + n);
    max_keys = std::max<int64_t>(max_keys, prefix_len_h[b] + n);
    min_keys = std::min<int64_t>(min_keys, prefix_len_h[b] + n);
  }
  // One workgroup per CU at a time (256 CUs).  Requests of (nearly) equal
  // length: the fewest splits that give every CU one workgroup (each split
  // costs a partial-result round trip).  Otherwise ~2.5 workgroups per CU,
  // so that longest-first dispatch evens out the mixed lengths (measured on
  // the batched dynamic trees with start-order dispatch: 2.5 per CU beat
  // 1.5, 2, 3, 3.5, 4 and 5).  Splits are at least 256 keys and at most
  // kMaxSplitsCombine per request.
  constexpr int64_t kCUs = 256;
  auto round_up = [](int64_t x) { return ((x + kTileKeys - 1) / kTileKeys) * kTileKeys; };
  int64_t split;
  const bool equal = B > 0 && max_keys <= min_keys + min_keys / 8;
  if (equal) {
    const int64_t ns = std::max<int64_t>(1, (kCUs + units - 1) / std::max<int64_t>(units, 1));
    split = std::min<int64_t>(round_up((max_keys + ns - 1) / ns), kMaxSplit);
  } else {
    const int64_t target = 5 * kCUs / 2;
    split = std::min<int64_t>(round_up((work + target - 1) / target), kMaxSplit);
  }
  split = std::max<int64_t>(split, round_up((max_keys + kMaxSplitsCombine - 1) / kMaxSplitsCombine));
  if (split < 256) split = 256;
  p.units = units;
  p.items = 0;
  p.partial_items = 0;
  p.items_a = 0;
  p.lpt = 0;
  p.weighted = 0;
  if (split > kMaxSplit) {          // a request longer than kMaxSplit * kMaxSplitsCombine keys
    p.split_keys = 0;
    p.items = -1;
    return p;
  }
  p.split_keys = (int)split;
  // mixed lengths: heavy units split 2/3 as long, unless that would give a
  // request more splits than the combine takes
  p.weighted = equal ? 0 : 1;
  for (int b = 0; b < B && p.weighted; ++b) {
    const int n = row_offsets_h[b + 1] - row_offsets_h[b];
    const int sp = attn_split_for(p.split_keys, n, G, p.rows_per_block, 1);
    if (attn_splits(prefix_len_h[b] + n, sp) > kMaxSplitsCombine) p.weighted = 0;
  }
  p.lpt = (B <= kLptMax) ? 1 : 0;
  p.max_ns = 1;
  int comb_rows = 0;
  bool one_block = B <= kLptMax;
  p.comb_nreq = 0;
  for (int b = 0; b < B; ++b) {
    const int n = row_offsets_h[b + 1] - row_offsets_h[b];
    const int ns = attn_splits(prefix_len_h[b] + n,
                               attn_split_for(p.split_keys, n, G, p.rows_per_block, p.weighted));
    p.max_ns = std::max(p.max_ns, ns);
    const int nrb = attn_row_blocks(n, G, p.rows_per_block);
    const int64_t per = (int64_t)hkv * nrb;
    p.items += per * ns;
    p.items_a += per * (ns - p.lpt);
    if (ns > 1) p.partial_items += per * ns;
    comb_rows = std::max(comb_rows, std::min(n * G, p.rows_per_block));
    one_block = one_block && nrb == 1;
    if (one_block && ns > 1) p.comb_req[p.comb_nreq++] = (uint16_t)b;
  }
  p.comb_chunks = std::max(1, (comb_rows + kCombineRows - 1) / kCombineRows);
  if (!one_block) p.comb_nreq = 0;
  if (p.lpt) {
    // second phase: requests by the estimated time of their last split,
    // longest first (ties by request index): its keys, 1.5x for heavy units
    // (see attn_split_for), plus ~200 keys' worth of start-up
    int64_t tail_len[kLptMax];
    for (int b = 0; b < B; ++b) {
      const int n = row_offsets_h[b + 1] - row_offsets_h[b];
      const int keys = prefix_len_h[b] + n;
      const int sp = attn_split_for(p.split_keys, n, G, p.rows_per_block, p.weighted);
      const int ns = attn_splits(keys, sp);
      const int64_t len = keys - (int64_t)(ns - 1) * sp;
      tail_len[b] = (sp < p.split_keys ? len * 3 / 2 : len) + 200;
      p.order[b] = (uint16_t)b;
    }
    std::stable_sort(p.order, p.order + B,
                     [&](uint16_t x, uint16_t y) { return tail_len[x] > tail_len[y]; });
  }
  return p;
}

size_t attention_workspace_bytes(const AttnPlan& plan, int d) {
  if (plan.partial_items == 0) return 256;
  return (size_t)plan.items * plan.rows_per_block * (d + 2) * sizeof(float) +
         (size_t)plan.units * (8 + plan.max_ns) * sizeof(int) + 256;
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
  a.rows_per_block = plan.rows_per_block;
  a.part = (float*)workspace;
  a.part_ml = a.part + (size_t)plan.items * plan.rows_per_block * addr.d;
  a.unit_desc = (int*)(a.part_ml + (size_t)plan.items * plan.rows_per_block * 2);
  a.unit_items = a.unit_desc + (size_t)plan.units * 8;
  // the ticket counter follows unit_items (inside the workspace's last 256
  // bytes).  Only mixed-length batches use it (several items per CU); plans
  // without partials have no combine to reset it: blockIdx.
  a.ticket = (plan.partial_items && plan.weighted)
                 ? (unsigned*)(a.unit_items + (size_t)plan.units * plan.max_ns)
                 : nullptr;
  a.items = (int)plan.items;
  a.max_ns = plan.max_ns;
  a.lpt = plan.lpt;
  a.weighted = plan.weighted;
  a.items_a = plan.items_a;
  if (plan.lpt) std::copy(plan.order, plan.order + cx.B, a.order);
  if (plan.items <= 0 || plan.items > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid((unsigned)plan.items);
  const int W = plan.rows_per_block / kRowsPerWave;
  if (W * kRowsPerWave != plan.rows_per_block || (W != kWaves && W != kWideWaves))
    return hipErrorInvalidValue;
  CombineArgs ca;
  ca.part = a.part;
  ca.part_ml = a.part_ml;
  ca.unit_desc = a.unit_desc;
  ca.unit_items = a.unit_items;
  ca.max_ns = a.max_ns;
  ca.hq = hq;
  ca.G = a.G;
  ca.out = out;
  ca.out_f32 = out_f32;
  ca.ticket = a.ticket;
  ca.chunks = plan.comb_chunks;
  ca.hkv = addr.hkv;
  ca.nreq = plan.comb_nreq;
  std::copy(plan.comb_req, plan.comb_req + plan.comb_nreq, ca.req);
  const int64_t cwg = (plan.comb_nreq > 0 ? (int64_t)plan.comb_nreq * addr.hkv : plan.units) *
                      plan.comb_chunks;
  if (plan.partial_items && (cwg <= 0 || cwg > 0x7fffffff)) return hipErrorInvalidValue;
  const dim3 cgrid((unsigned)cwg);
  if (addr.d == 128 && W == kWaves) {
    hipLaunchKernelGGL((attn_bf16_kernel<128, kWaves>), grid, dim3(W * 64), 0, cx.stream, a);
    if (plan.partial_items) {
      if (out_f32)
        hipLaunchKernelGGL((attn_combine_kernel<128, kWaves, false>), cgrid, dim3(256), 0, cx.stream, ca);
      else
        hipLaunchKernelGGL((attn_combine_kernel<128, kWaves, true>), cgrid, dim3(256), 0, cx.stream, ca);
    }
  } else if (addr.d == 128) {
    hipLaunchKernelGGL((attn_bf16_kernel<128, kWideWaves>), grid, dim3(W * 64), 0, cx.stream, a);
    if (plan.partial_items) {
      if (out_f32)
        hipLaunchKernelGGL((attn_combine_kernel<128, kWideWaves, false>), cgrid, dim3(256), 0, cx.stream, ca);
      else
        hipLaunchKernelGGL((attn_combine_kernel<128, kWideWaves, true>), cgrid, dim3(256), 0, cx.stream, ca);
    }
  } else if (W == kWaves) {
    hipLaunchKernelGGL((attn_bf16_kernel<64, kWaves>), grid, dim3(W * 64), 0, cx.stream, a);
    if (plan.partial_items) {
      if (out_f32)
        hipLaunchKernelGGL((attn_combine_kernel<64, kWaves, false>), cgrid, dim3(256), 0, cx.stream, ca);
      else
        hipLaunchKernelGGL((attn_combine_kernel<64, kWaves, true>), cgrid, dim3(256), 0, cx.stream, ca);
    }
  } else {
    hipLaunchKernelGGL((attn_bf16_kernel<64, kWideWaves>), grid, dim3(W * 64), 0, cx.stream, a);
    if (plan.partial_items) {
      if (out_f32)
        hipLaunchKernelGGL((attn_combine_kernel<64, kWideWaves, false>), cgrid, dim3(256), 0, cx.stream, ca);
      else
        hipLaunchKernelGGL((attn_combine_kernel<64, kWideWaves, true>), cgrid, dim3(256), 0, cx.stream, ca);
    }
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
