// Philox4x32-10 counter-based generator, device side (J. Salmon, M. Moraes,
// R. Dror, D. Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3", SC'11,
// section 3).  Stateless: a block of four 32-bit words is a pure function of
// a 128-bit counter and a 64-bit key, so any thread can draw the word of any
// element without coordination and without a stored random tensor.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace i8mp {

struct u32x4 {
  uint32_t w[4];
};

// a ^ b ^ c in one instruction: gfx950's three-input bitwise operation with
// the truth table of XOR (0x96), where two dependent XORs would take two.
__device__ __forceinline__ uint32_t xor3(uint32_t a, uint32_t b, uint32_t c) {
  return __builtin_amdgcn_bitop3_b32(a, b, c, 0x96);
}

// Ten rounds; the key is bumped by the two Weyl constants between rounds.
// Each round forms the full 64-bit products of counter words 0 and 2 with
// the two round multipliers and mixes their halves into the next counter.
__device__ __forceinline__ u32x4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                               uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int i = 0; i < 10; ++i) {
    const uint64_t p = (uint64_t)0xD2511F53u * c0;
    const uint64_t t = (uint64_t)0xCD9E8D57u * c2;
    const uint32_t n0 = xor3((uint32_t)(t >> 32), c1, k0);
    const uint32_t n2 = xor3((uint32_t)(p >> 32), c3, k1);
    c1 = (uint32_t)t;
    c3 = (uint32_t)p;
    c0 = n0;
    c2 = n2;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  u32x4 r;
  r.w[0] = c0;
  r.w[1] = c1;
  r.w[2] = c2;
  r.w[3] = c3;
  return r;
}

// Block number `block` (64-bit) under key `seed`: counter (lo, hi, 0, 0).
__device__ __forceinline__ u32x4 philox_block(uint64_t seed, uint64_t block) {
  return philox4x32_10((uint32_t)block, (uint32_t)(block >> 32), 0u, 0u, (uint32_t)seed,
                       (uint32_t)(seed >> 32));
}

// The stochastic-rounding uniform of a word in units of 2^-24: its top 24
// bits as a float (exact in binary32).  The uniform itself is that times
// 2^-24, in [0, 1 - 2^-24]; the quantizer applies the factor inside the FMA
// that adds it to the quotient.
__device__ __forceinline__ float word_uniform_units(uint32_t w) { return (float)(w >> 8); }

}  // namespace i8mp
