// Philox4x64-10 counter-based generator, device side.
//
// Written from the published definition: Salmon, Moraes, Dror, Shaw,
// "Parallel Random Numbers: As Easy as 1, 2, 3" (SC'11).  Each of the ten
// rounds multiplies words 0 and 2 of the counter by two fixed odd constants
// into 128-bit products and recombines their halves with words 1 and 3 and
// the key; between rounds the key advances by two Weyl constants.
//
// The verify step draws the acceptance coins with key (seed, 0) and counter
// (step, request, row, purpose); the uniform is (word0 >> 11) * 2^-53.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace spec {

struct Philox4x64 {
  static constexpr uint64_t kMul0 = 0xD2E7470EE14C6C93ull;
  static constexpr uint64_t kMul1 = 0xCA5A826395121157ull;
  static constexpr uint64_t kWeyl0 = 0x9E3779B97F4A7C15ull;
  static constexpr uint64_t kWeyl1 = 0xBB67AE8584CAA73Bull;

  __device__ __forceinline__ static void block(uint64_t c[4], uint64_t k0, uint64_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
      uint64_t hi0 = __umul64hi(kMul0, c[0]);
      uint64_t lo0 = kMul0 * c[0];
      uint64_t hi1 = __umul64hi(kMul1, c[2]);
      uint64_t lo1 = kMul1 * c[2];
      uint64_t n0 = hi1 ^ c[1] ^ k0;
      uint64_t n2 = hi0 ^ c[3] ^ k1;
      c[0] = n0;
      c[1] = lo1;
      c[2] = n2;
      c[3] = lo0;
      k0 += kWeyl0;
      k1 += kWeyl1;
    }
  }
};

// Uniform double in [0, 1) for the verify-step coin (seed, step, request, row, purpose).
__device__ __forceinline__ double verify_uniform(uint64_t seed, uint64_t step, uint64_t request,
                                                 uint64_t row, uint64_t purpose) {
  uint64_t c[4] = {step, request, row, purpose};
  Philox4x64::block(c, seed, 0);
  return (double)(c[0] >> 11) * 0x1.0p-53;
}

}  // namespace spec
