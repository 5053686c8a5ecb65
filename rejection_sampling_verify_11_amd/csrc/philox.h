// Philox4x64-10 counter-based generator as a device function.
//
// Written from the definition in Salmon, Moraes, Dror and Shaw, "Parallel
// Random Numbers: As Easy as 1, 2, 3" (SC'11): ten rounds, each taking two
// 64x64 -> 128-bit products of counter words with fixed multipliers, XORing
// the high halves into the other two words together with the round key, and
// bumping the key by two Weyl constants between rounds.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {

struct U64x4 {
  uint64_t w[4];
};

__device__ __forceinline__ U64x4 philox4x64_10(uint64_t c0, uint64_t c1, uint64_t c2,
                                                uint64_t c3, uint64_t k0, uint64_t k1) {
  const uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  const uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t lo0 = M0 * c0, hi0 = __umul64hi(M0, c0);
    const uint64_t lo1 = M1 * c2, hi1 = __umul64hi(M1, c2);
    const uint64_t n0 = hi1 ^ c1 ^ k0;
    const uint64_t n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
    k0 += W0;
    k1 += W1;
  }
  U64x4 r;
  r.w[0] = c0; r.w[1] = c1; r.w[2] = c2; r.w[3] = c3;
  return r;
}

// Uniform in [0, 1) with 24 bits, exact in fp32: counter (row, pos, draw,
// offset), key (seed, 0), top 24 bits of output word 0.
__device__ __forceinline__ double uniform24(uint64_t seed, uint64_t row, uint64_t pos,
                                            uint64_t draw, uint64_t offset) {
  U64x4 o = philox4x64_10(row, pos, draw, offset, seed, 0);
  return (double)(o.w[0] >> 40) * (1.0 / 16777216.0);
}

}  // namespace sv
