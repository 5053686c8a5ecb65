// Wave64 scans and reductions on DPP lane moves (CDNA / gfx9 DPP).
//
// An inclusive scan over the 64 lanes of a wave: four row_shr steps (by 1,
// 2, 4, 8 lanes) scan each row of 16 lanes, then row_bcast:15 adds the last
// lane of rows 0 and 2 into rows 1 and 3, and row_bcast:31 adds lane 31
// into rows 2 and 3.  A lane with no source keeps the identity element.
// These run in the vector ALU with a few cycles of latency each, instead of
// the LDS round trip of a cross-lane permute.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {

enum : int {
  kDppRowShr1 = 0x111,
  kDppRowShr2 = 0x112,
  kDppRowShr4 = 0x114,
  kDppRowShr8 = 0x118,
  kDppRowBcast15 = 0x142,
  kDppRowBcast31 = 0x143,
};

template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v, uint32_t ident) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)ident, (int)v, CTRL, ROWS, 0xf, false);
}

template <int CTRL, int ROWS>
__device__ __forceinline__ double dpp_f64(double v, double ident) {
  const uint64_t b = __double_as_longlong(v), z = __double_as_longlong(ident);
  const uint32_t lo = dpp_u32<CTRL, ROWS>((uint32_t)b, (uint32_t)z);
  const uint32_t hi = dpp_u32<CTRL, ROWS>((uint32_t)(b >> 32), (uint32_t)(z >> 32));
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

struct OpAddU32 {
  __device__ static uint32_t ident() { return 0u; }
  __device__ static uint32_t f(uint32_t a, uint32_t b) { return a + b; }
};
struct OpMaxI32 {
  __device__ static uint32_t ident() { return 0x80000000u; }  // INT_MIN
  __device__ static uint32_t f(uint32_t a, uint32_t b) {
    return (uint32_t)max((int)a, (int)b);
  }
};
struct OpMinI32 {
  __device__ static uint32_t ident() { return 0x7FFFFFFFu; }  // INT_MAX
  __device__ static uint32_t f(uint32_t a, uint32_t b) {
    return (uint32_t)min((int)a, (int)b);
  }
};
struct OpOrU32 {
  __device__ static uint32_t ident() { return 0u; }
  __device__ static uint32_t f(uint32_t a, uint32_t b) { return a | b; }
};

// Inclusive scan of a 32-bit value across the wave with operator Op.
template <class Op>
__device__ __forceinline__ uint32_t wave_scan_u32(uint32_t x) {
  const uint32_t id = Op::ident();
  x = Op::f(x, dpp_u32<kDppRowShr1, 0xf>(x, id));
  x = Op::f(x, dpp_u32<kDppRowShr2, 0xf>(x, id));
  x = Op::f(x, dpp_u32<kDppRowShr4, 0xf>(x, id));
  x = Op::f(x, dpp_u32<kDppRowShr8, 0xf>(x, id));
  x = Op::f(x, dpp_u32<kDppRowBcast15, 0xa>(x, id));
  x = Op::f(x, dpp_u32<kDppRowBcast31, 0xc>(x, id));
  return x;
}

// Inclusive prefix sum of an fp64 value across the wave.
__device__ __forceinline__ double wave_scan_add_f64(double x) {
  x += dpp_f64<kDppRowShr1, 0xf>(x, 0.0);
  x += dpp_f64<kDppRowShr2, 0xf>(x, 0.0);
  x += dpp_f64<kDppRowShr4, 0xf>(x, 0.0);
  x += dpp_f64<kDppRowShr8, 0xf>(x, 0.0);
  x += dpp_f64<kDppRowBcast15, 0xa>(x, 0.0);
  x += dpp_f64<kDppRowBcast31, 0xc>(x, 0.0);
  return x;
}

// Value of lane 63 (after an inclusive scan: the wave total), uniform.
__device__ __forceinline__ uint32_t wave_last_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}
__device__ __forceinline__ double wave_last_f64(double x) {
  const uint64_t b = __double_as_longlong(x);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, 63);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), 63);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

}  // namespace sv
