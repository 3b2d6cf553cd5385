// nvfp4_device.hpp -- device-side arithmetic of the NVFP4 format for gfx950.
//
// Every routine reproduces, bit for bit, the encoding that nvfp4.h states:
// IEEE binary32 round-to-nearest-even for each float operation (this file is
// compiled with -ffp-contract=off, correctly rounded division, denormals
// kept), then integer work for the formats.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

constexpr float kFltMax = 3.40282346638528859812e+38f;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) {
  return __uint_as_float(b16 << 16);
}

// ---- per-tensor scales -------------------------------------------------------
// A (tensor amax) -> S = RN32(2688/A) (1 if A == 0, FLT_MAX on overflow),
// k = RN32(S/6), g = RN32(A/2688); 2688 = 6 (E2M1 max) * 448 (E4M3 max).
struct TensorScales {
  float S, k, g;
};

__device__ __forceinline__ TensorScales tensor_scales(float amax) {
  TensorScales t;
  float s = 1.0f;
  if (amax != 0.0f) {
    s = 2688.0f / amax;
    if (s > kFltMax) s = kFltMax;
  }
  t.S = s;
  t.k = s / 6.0f;
  t.g = amax / 2688.0f;
  return t;
}

// ---- E4M3 block scales -----------------------------------------------------------
// Non-negative finite s -> E4M3 byte, round to nearest even, saturating at
// 448 (0x7E).  Below 2^-6 the grid is m * 2^-9 (codes 0..7, code 8 = 2^-6);
// above, the fp32 significand is rounded to 3 bits on the integer bits, a
// carry moving into the exponent.  The even code is the even mantissa.
__device__ __forceinline__ uint32_t e4m3_encode(float s) {
  if (!(s < 448.0f)) return 0x7Eu;
  if (s < 0.015625f) return (uint32_t)__builtin_rintf(s * 512.0f);
  uint32_t b = __float_as_uint(s);
  uint32_t r = b + 0x7FFFFu + ((b >> 20) & 1u);
  return (((r >> 23) - 120u) << 3) | ((r >> 20) & 7u);
}

// E4M3 byte (sign bit clear) -> fp32, exact.
__device__ __forceinline__ float e4m3_decode(uint32_t e) {
  uint32_t ex = (e >> 3) & 15u, m = e & 7u;
  if (ex == 0) return (float)m * 0.001953125f;  // m * 2^-9
  return __uint_as_float(((ex + 120u) << 23) | (m << 20));
}

// Block reciprocal r = RN32(S / d), 0 when d == 0, FLT_MAX on overflow.
__device__ __forceinline__ float block_recip(float S, float d) {
  if (d == 0.0f) return 0.0f;
  float r = S / d;
  return r > kFltMax ? kFltMax : r;
}

// ---- E2M1 elements -----------------------------------------------------------------
// Round-to-nearest-even onto {0,.5,1,1.5,2,3,4,6}: the magnitude index is the
// number of rounding boundaries at or below |y|; boundaries that are ties
// belong to the even index (closed on the side of 0, 1, 2, 4).
__device__ __forceinline__ uint32_t e2m1_rne(float y) {
  float m = __builtin_fabsf(y);
  uint32_t c = (uint32_t)(m > 0.25f) + (uint32_t)(m >= 0.75f) + (uint32_t)(m > 1.25f) +
               (uint32_t)(m >= 1.75f) + (uint32_t)(m > 2.5f) + (uint32_t)(m >= 3.5f) +
               (uint32_t)(m > 5.0f);
  return c | ((__float_as_uint(y) >> 28) & 8u);
}

// Stochastic rounding: lo = largest grid value <= |y|, round up iff
// u16 < 65536 * (|y| - lo) / step, |y| >= 6 saturating.  sr_value returns
// the chosen grid value (sign of y), which the hardware conversion (round to
// nearest) then encodes exactly.
//
// Worked on B = bits(|y| * 2^-126).  That scaling moves E2M1's boundary
// between its subnormal and normal values (1.0) onto fp32's (2^-126), so for
// every |y| the bits of B from 22 up hold lo's code and the 22 bits below
// hold (|y| - lo) / step as a binary fraction.  For |y| >= 1 the multiply is
// exact (only the exponent moves); for |y| < 1, B is |y| * 2^23 in fixed
// point, rounded to nearest by the multiply and raised by one where that
// rounding went down (B * 2^126 < |y|, exact test), so B is the ceiling, which
// is what the comparison with a multiple of 64 needs.  The rule's test
// u16 * 64 < (B & 0x3FFFFF) holds exactly when adding
// a = (65535 - u16) * 64 + 63 carries into bit 22, so bits 22 and up of B + a
// hold the chosen code; capped at code 7 (6.0) and scaled back by 2^126
// (exact), they are the chosen value.
__device__ __forceinline__ float sr_value(float y, uint32_t a) {
  const float m = __builtin_fabsf(y);
  const float ms = m * 0x1p-126f;
  const uint32_t below = ms * 0x1p126f < m ? 1u : 0u;
  uint32_t s = (__float_as_uint(ms) + a + below) & 0xFFC00000u;
  s = __builtin_elementwise_min(s, 7u << 22);
  return __uint_as_float(s | (__float_as_uint(y) & 0x80000000u)) * 0x1p126f;
}

// The addend a of 16-bit slot 2q (low half of Philox word w) and of slot
// 2q + 1 (high half).
__device__ __forceinline__ uint32_t sr_addend_lo(uint32_t w) { return ((~w & 0xFFFFu) << 6) | 63u; }
__device__ __forceinline__ uint32_t sr_addend_hi(uint32_t w) { return ((~w >> 16) << 6) | 63u; }

// ---- Philox4x32 ----------------------------------------------------------------------
struct Philox4 {
  uint32_t x, y, z, w;
};

__device__ __forceinline__ void philox_round(uint32_t& c0, uint32_t& c1, uint32_t& c2,
                                             uint32_t& c3, uint32_t& k0, uint32_t& k1) {
  // 32 x 32 -> 64-bit products (one v_mad_u64_u32 each)
  const uint64_t p0 = (uint64_t)c0 * 0xD2511F53u, p1 = (uint64_t)c2 * 0xCD9E8D57u;
  const uint32_t lo0 = (uint32_t)p0, hi0 = (uint32_t)(p0 >> 32);
  const uint32_t lo1 = (uint32_t)p1, hi1 = (uint32_t)(p1 >> 32);
  uint32_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
  c0 = n0;
  c1 = lo1;
  c2 = n2;
  c3 = lo0;
  k0 += 0x9E3779B9u;
  k1 += 0xBB67AE85u;
}

__device__ __forceinline__ Philox4 philox4x32(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                              uint32_t k0, uint32_t k1, uint32_t rounds) {
  if (rounds == 5) {  // the default: unrolled
#pragma unroll
    for (int r = 0; r < 5; r++) philox_round(c0, c1, c2, c3, k0, k1);
    return Philox4{c0, c1, c2, c3};
  }
  for (uint32_t r = 0; r < rounds; r++) philox_round(c0, c1, c2, c3, k0, k1);
  return Philox4{c0, c1, c2, c3};
}

// Philox call number n (= 2 * block id + call j) of a stream.
__device__ __forceinline__ Philox4 sr_call(uint64_t n, uint64_t seed, uint64_t offset,
                                           uint32_t rounds) {
  return philox4x32((uint32_t)n, (uint32_t)(n >> 32), (uint32_t)offset,
                    (uint32_t)(offset >> 32), (uint32_t)seed, (uint32_t)(seed >> 32), rounds);
}

// 16-bit slot t (0..7) of one call: word t>>1, low half for even t.
__device__ __forceinline__ uint32_t sr_slot(const Philox4& p, int t) {
  uint32_t w = (t >> 1) == 0 ? p.x : (t >> 1) == 1 ? p.y : (t >> 1) == 2 ? p.z : p.w;
  return (t & 1) ? (w >> 16) : (w & 0xFFFFu);
}

// y[t] -> its stochastically rounded grid value, slot t of the call p.
__device__ __forceinline__ void sr_values8(float y[8], const Philox4& p) {
  const uint32_t w[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
  for (int q = 0; q < 4; q++) {
    y[2 * q] = sr_value(y[2 * q], sr_addend_lo(w[q]));
    y[2 * q + 1] = sr_value(y[2 * q + 1], sr_addend_hi(w[q]));
  }
}

// ---- 16-point Hadamard butterflies -----------------------------------------------
// Sign flips, then strides 1, 2, 4 inside a group of 8 (positions base..+7).
__device__ __forceinline__ void rht_signs_and_low_stages(float v[8], uint32_t mask, int base) {
#pragma unroll
  for (int i = 0; i < 8; i++)
    if ((mask >> (base + i)) & 1u) v[i] = -v[i];
#pragma unroll
  for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 8; i++) {
      if (i & h) continue;
      float a = v[i], b = v[i + h];
      v[i] = a + b;
      v[i + h] = a - b;
    }
  }
}

// The butterflies of the transform alone (strides 1, 2, 4, then 8), without
// the sign flips and the final * 1/4.
__device__ __forceinline__ void hadamard16_unscaled(float v[16]) {
#pragma unroll
  for (int h = 1; h < 16; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 16; i++) {
      if (i & h) continue;
      float a = v[i], b = v[i + h];
      v[i] = a + b;
      v[i + h] = a - b;
    }
  }
}

// Full 16-point transform of one in-register block (stride 8 last, * 1/4).
__device__ __forceinline__ void rht16_inreg(float v[16], uint32_t mask) {
  rht_signs_and_low_stages(v, mask, 0);
  rht_signs_and_low_stages(v + 8, mask, 8);
#pragma unroll
  for (int i = 0; i < 8; i++) {
    float a = v[i], b = v[i + 8];
    v[i] = a + b;
    v[i + 8] = a - b;
  }
#pragma unroll
  for (int i = 0; i < 16; i++) v[i] = v[i] * 0.25f;
}

}  // namespace nvfp4
