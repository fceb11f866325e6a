// Helpers shared by the two top-K paths (select_topk.hip, select_large.hip).
#pragma once
#include "common.hpp"

namespace pisa {

// Order-preserving 32-bit key of an fp32 score (larger score, larger key).
__device__ __forceinline__ uint32_t order_key(float s) {
  s = s + 0.0f;                                   // -0 -> +0 so equal scores tie
  const uint32_t u = __float_as_uint(s);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inclusive scan over the 64 lanes of a wave.
__device__ __forceinline__ int wave_inclusive_scan(int x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  return x;
}

}  // namespace pisa
