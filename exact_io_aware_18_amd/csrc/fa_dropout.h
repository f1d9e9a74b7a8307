// Dropout on the attention probabilities, regenerated from a counter-based
// generator so that the backward never stores the mask.
//
// The fused kernel of "Flashattention fast and memory efficient exact
// attention with io awareness" (its figure: matmul, mask, softmax, dropout and
// matmul fused into one kernel) applies dropout between the softmax and the
// product with V, at no extra memory.  The form used here is inverted dropout
// on the normalised probabilities:
//   O = (P o Z) V / (1 - p),  Z_ij in {0, 1} kept with probability 1 - p,
// with lse still the statistic of the undropped softmax.  Its gradient for a
// fixed Z: dV = (P o Z)^T dO / (1 - p), dP = (dO V^T) o Z / (1 - p),
// D_i = dO_i . O_i, dS = P o (dP - D).
//
// Generator: Philox-4x32 with 10 rounds (Salmon, Moraes, Dror and Shaw,
// "Parallel random numbers: as easy as 1, 2, 3", SC 2011), written from that
// definition.  Keep rule:
//   key     = (seed mod 2^32, seed div 2^32)
//   counter = (j / 4, i, b*H + h, 0)   for query i, key j of head (b, h)
//   Z_ij    = [word (j mod 4) of Philox(counter, key) >= T],  T = floor(p 2^32)
// One generator call yields the bits of four consecutive keys of one query.
#pragma once

#include <cstdint>

#include "fa_device.h"

namespace fa {

struct DropArgs {
  uint32_t thresh;   // T = floor(p * 2^32); 0 keeps every element
  uint32_t seed_lo;  // Philox key word 0
  uint32_t seed_hi;  // Philox key word 1
  float keep_scale;  // 1 / (1 - p)
};

constexpr uint32_t kPhiloxM0 = 0xD2511F53u;
constexpr uint32_t kPhiloxM1 = 0xCD9E8D57u;
constexpr uint32_t kPhiloxW0 = 0x9E3779B9u;
constexpr uint32_t kPhiloxW1 = 0xBB67AE85u;

// The three-input XORs of a round are one v_bitop3_b32 each (truth table
// 0x96 = a ^ b ^ c); the compiler would otherwise emit two v_xor_b32.
__device__ __forceinline__ uint32_t xor3(uint32_t a, uint32_t b, uint32_t c) {
  return __builtin_amdgcn_bitop3_b32(a, b, c, 0x96);
}

__device__ __forceinline__ u32x4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                               uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)kPhiloxM0 * c0;
    const uint64_t p1 = (uint64_t)kPhiloxM1 * c2;
    const uint32_t n0 = xor3((uint32_t)(p1 >> 32), c1, k0);
    const uint32_t n2 = xor3((uint32_t)(p0 >> 32), c3, k1);
    c1 = (uint32_t)p1;
    c3 = (uint32_t)p0;
    c0 = n0;
    c2 = n2;
    k0 += kPhiloxW0;
    k1 += kPhiloxW1;
  }
  return u32x4{c0, c1, c2, c3};
}

// Keep bits of keys j0 .. j0+3 (j0 a multiple of 4) for query i of head bh:
// bit u is set when key j0 + u is kept.
__device__ __forceinline__ uint32_t keep4(const DropArgs& dp, int bh, int i, int j0) {
  const u32x4 w = philox4x32_10((uint32_t)j0 >> 2, (uint32_t)i, (uint32_t)bh, 0u, dp.seed_lo,
                                dp.seed_hi);
  return (uint32_t)(w[0] >= dp.thresh) | ((uint32_t)(w[1] >= dp.thresh) << 1) |
         ((uint32_t)(w[2] >= dp.thresh) << 2) | ((uint32_t)(w[3] >= dp.thresh) << 3);
}

// Lanes 4m .. 4m+3 (t = lane & 3) each hold the keep bits of four
// consecutive keys for query i0 + t; returns, for lane t, the keep bits of
// queries i0 .. i0+3 at key 4m + t (bit s for query i0 + s).
__device__ __forceinline__ uint32_t quad_transpose4(uint32_t bits, int t) {
  const uint32_t b0 = (uint32_t)__builtin_amdgcn_mov_dpp((int)bits, 0x00, 0xF, 0xF, false);
  const uint32_t b1 = (uint32_t)__builtin_amdgcn_mov_dpp((int)bits, 0x55, 0xF, 0xF, false);
  const uint32_t b2 = (uint32_t)__builtin_amdgcn_mov_dpp((int)bits, 0xAA, 0xF, 0xF, false);
  const uint32_t b3 = (uint32_t)__builtin_amdgcn_mov_dpp((int)bits, 0xFF, 0xF, 0xF, false);
  return ((b0 >> t) & 1u) | (((b1 >> t) & 1u) << 1) | (((b2 >> t) & 1u) << 2) |
         (((b3 >> t) & 1u) << 3);
}

}  // namespace fa
