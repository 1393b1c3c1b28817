// Device helpers shared by the verify-step kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#define SPEC_DEVICE __device__ __forceinline__

namespace spec {

constexpr int kWave = 64;
constexpr int kMaxRows = 256;      // rows per request, root included
constexpr int kMaxWords = 4;       // kMaxRows / 64
constexpr int kBlock = 16;         // paged KV block (tokens)
constexpr int kMaxVocab = 1 << 20;  // vocabulary entries the acceptance supports

// Acceptance flags (same values as SPEC_FLAG_* in the public header).
constexpr int kFlagZeroResidual = 1;
constexpr int kFlagPathTruncated = 2;
constexpr int kFlagBadTree = 4;
constexpr int kFlagSyncTimeout = 8;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

SPEC_DEVICE float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// Round-to-nearest-even float -> bf16 bits (finite inputs; NaN stays NaN).
SPEC_DEVICE uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <typename T>
SPEC_DEVICE T wave_sum(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Sum of a double over the wave without the LDS crossbar: a butterfly within
// each 16-lane row by DPP moves (quad_perm [1,0,3,2], quad_perm [2,3,0,1],
// row_ror 4, row_ror 8), then the four row totals read from lanes 0, 16, 32
// and 48 and added in a fixed order.  Every lane returns the same value.
template <int kCtrl>
SPEC_DEVICE double dpp_f64(double v) {
  const unsigned long long b = (unsigned long long)__double_as_longlong(v);
  const int lo = __builtin_amdgcn_mov_dpp((int)(unsigned)b, kCtrl, 0xf, 0xf, false);
  const int hi = __builtin_amdgcn_mov_dpp((int)(unsigned)(b >> 32), kCtrl, 0xf, 0xf, false);
  return __longlong_as_double(
      (long long)(((unsigned long long)(unsigned)hi << 32) | (unsigned long long)(unsigned)lo));
}
SPEC_DEVICE double readlane_f64(double v, int lane) {
  const unsigned long long b = (unsigned long long)__double_as_longlong(v);
  const unsigned lo = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)b, lane);
  const unsigned hi = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)(b >> 32), lane);
  return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}
SPEC_DEVICE double wave_sum_f64(double v) {
  v += dpp_f64<0xB1>(v);
  v += dpp_f64<0x4E>(v);
  v += dpp_f64<0x124>(v);
  v += dpp_f64<0x128>(v);
  return (readlane_f64(v, 0) + readlane_f64(v, 16)) + (readlane_f64(v, 32) + readlane_f64(v, 48));
}

SPEC_DEVICE float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// Request owning global row `r` (row_offsets is increasing, B entries + 1).
SPEC_DEVICE int request_of_row(const int32_t* row_offsets, int B, int r) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (row_offsets[mid] <= r) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Element offset of token `t`, head `h` of request `b` in a KV cache.
struct KvAddr {
  int paged;
  int hkv;
  int d;
  int capacity;
  const int32_t* block_table;
  int mbps;
  SPEC_DEVICE int64_t operator()(int b, int h, int t) const {
    if (!paged) return (((int64_t)b * hkv + h) * capacity + t) * d;
    int blk = block_table[(int64_t)b * mbps + (t >> 4)];
    return (((int64_t)blk * hkv + h) * kBlock + (t & 15)) * d;
  }
};

}  // namespace spec
