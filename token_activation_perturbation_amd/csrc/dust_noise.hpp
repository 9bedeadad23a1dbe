// dust_noise.hpp -- the estimator's noise, evaluated inline on gfx950.
//
// The pages fix no generator; they ask for noise that is a pure function of
// a seed and an index so it never has to be stored ("Scaling To Unfathomable
// Depth", section "MeZO": counter-based generators such as Philox).  Value
// a_t^(n)[c] is:
//   words (w0,w1,w2,w3) = Philox4x32-10(counter (c/4, t, n, 0),
//                                        key (seed low, seed high))
//   (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as 1, 2,
//   3", SC'11), then Box-Muller on (w0,w1) for channels 4q, 4q+1 and on
//   (w2,w3) for 4q+2, 4q+3 with 23-bit uniforms (each word's top 23 bits)
//   u = 1 - (w_even >> 9) 2^-23 in (0,1], v = (w_odd >> 9) 2^-23 in [0,1),
//   a_even = sqrt(-2 ln u) cos(2 pi v), a_odd = sqrt(-2 ln u) sin(2 pi v).
//
// gfx950 notes.  The counter is laid out so that one lane's quad index is the
// only per-lane word: token and noise index are wave-uniform, so the first
// two rounds largely run on the scalar unit or are loop-invariant, and the
// key schedule is scalar.  The 32x32->64 products map to v_mad_u64_u32.  The
// transform uses the hardware transcendental unit directly: v_log_f32 is
// log2, and v_sin_f32 / v_cos_f32 take their argument in revolutions and
// use only its fraction, so 2 pi v needs no range reduction.  A uniform is
// built in a float's bit fields, not converted from an integer: the word's
// top 23 bits under exponent field 127 are the float 1 + m 2^-23 in [1, 2)
// (one funnel shift, v_alignbit_b32), whose fraction is v itself and whose
// difference from 2 is u, where a shift, an integer-to-float conversion (a
// half-rate instruction) and a scaling would cost four issue slots.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dust {

constexpr uint32_t kPhiloxM0 = 0xD2511F53u;
constexpr uint32_t kPhiloxM1 = 0xCD9E8D57u;
constexpr uint32_t kPhiloxW0 = 0x9E3779B9u;
constexpr uint32_t kPhiloxW1 = 0xBB67AE85u;

struct NoiseKey {
  uint32_t k0, k1;
};

__device__ __forceinline__ void mul_wide(uint32_t m, uint32_t x, uint32_t& hi, uint32_t& lo) {
  const uint64_t prod = (uint64_t)m * (uint64_t)x;
  hi = (uint32_t)(prod >> 32);
  lo = (uint32_t)prod;
}

// a ^ b ^ c as one VALU instruction: gfx950's three-input bitwise operation
// with truth table 0x96 (odd parity).  The compiler does not form it from a
// chain of XORs.
__device__ __forceinline__ uint32_t xor3(uint32_t a, uint32_t b, uint32_t c) {
  return __builtin_amdgcn_bitop3_b32(a, b, c, 0x96);
}

__device__ __forceinline__ uint4 philox4x32_10(uint32_t x0, uint32_t x1, uint32_t x2,
                                               uint32_t x3, NoiseKey key) {
  uint32_t k0 = key.k0, k1 = key.k1;
#pragma unroll
  for (int round = 0; round < 10; ++round) {
    uint32_t hi0, lo0, hi1, lo1;
    mul_wide(kPhiloxM0, x0, hi0, lo0);
    mul_wide(kPhiloxM1, x2, hi1, lo1);
    // With the counter (quad, token, noise index, 0) only the quad differs
    // per lane, so early rounds XOR a per-lane word with two wave-uniform
    // ones: plain XORs let the compiler fold those two on the scalar unit
    // (the first two rounds of y0, the first three of y2).  Later, two of
    // the three operands differ per lane.
    const uint32_t y0 = round < 2 ? hi1 ^ x1 ^ k0 : xor3(hi1, x1, k0);
    const uint32_t y2 = round < 3 ? hi0 ^ x3 ^ k1 : xor3(hi0, x3, k1);
    x0 = y0;
    x1 = lo1;
    x2 = y2;
    x3 = lo0;
    k0 += kPhiloxW0;
    k1 += kPhiloxW1;
  }
  return make_uint4(x0, x1, x2, x3);
}

// UNIT: the generator returns each Gaussian in units of sqrt(2 ln 2): with
// log2 u from the hardware, a = sqrt(-2 ln u) cos 2 pi v = kNoiseUnit *
// sqrt(-log2 u) cos 2 pi v, and the constant factor is left to the
// consumers, which apply it once per reduced total or per output (a
// multiply per value saved).  !UNIT: the Gaussians themselves (the
// two-pass loss kernel keeps this form, which measured faster there).
constexpr float kNoiseUnit = 1.17741002251547469101f;   // sqrt(2 ln 2)
constexpr float kNoiseUnit2 = 1.38629436111989061883f;  // 2 ln 2
constexpr float kMinusTwoLn2 = -1.38629436111989061883f;

// The pair (a_even, a_odd), divided by kNoiseUnit when UNIT.
template <bool UNIT = true>
__device__ __forceinline__ float2 box_muller(uint32_t w_even, uint32_t w_odd) {
  // the float 1 + (w >> 9) 2^-23 in [1, 2): exponent field 127, the word's
  // top 23 bits as the mantissa (one funnel shift)
  const float xu = __uint_as_float(__builtin_amdgcn_alignbit(0x7Fu, w_even, 9u));
  const float xv = __uint_as_float(__builtin_amdgcn_alignbit(0x7Fu, w_odd, 9u));
  const float u = 2.0f - xu;  // 1 - (w_even >> 9) 2^-23 in (0, 1], exact
  // log2 u <= 0; its negation is a source modifier of the square root
  const float radius = UNIT ? __builtin_amdgcn_sqrtf(-__builtin_amdgcn_logf(u))
                            : __builtin_amdgcn_sqrtf(kMinusTwoLn2 * __builtin_amdgcn_logf(u));
  // v_sin / v_cos take revolutions and keep only the fraction, so xv itself
  // is the angle v = (w_odd >> 9) 2^-23
  return make_float2(radius * __builtin_amdgcn_cosf(xv), radius * __builtin_amdgcn_sinf(xv));
}

// The four Gaussians of channel quad q of token t under noise index n (in
// units of kNoiseUnit when UNIT).
template <bool UNIT = true>
__device__ __forceinline__ float4 noise_quad(uint32_t q, uint32_t t, uint32_t n, NoiseKey key) {
  const uint4 w = philox4x32_10(q, t, n, 0u, key);
  const float2 a = box_muller<UNIT>(w.x, w.y);
  const float2 b = box_muller<UNIT>(w.z, w.w);
  return make_float4(a.x, a.y, b.x, b.y);
}

// Two noise quads at once, (quad qa, noise index na) and (qb, nb) of token
// t, their Philox rounds advanced together.  The values are those of two
// noise_quad<UNIT> calls; interleaving the two dependency chains gives the
// scheduler independent multiplies to issue while a round's products are in
// flight (each stream alone has only two per round).
template <bool UNIT = true>
__device__ __forceinline__ void noise_quad_x2(uint32_t qa, uint32_t na, uint32_t qb, uint32_t nb,
                                              uint32_t t, NoiseKey key, float4& A, float4& B) {
  uint32_t k0 = key.k0, k1 = key.k1;
  uint32_t a0 = qa, a1 = t, a2 = na, a3 = 0u;
  uint32_t b0 = qb, b1 = t, b2 = nb, b3 = 0u;
#pragma unroll
  for (int round = 0; round < 10; ++round) {
    uint32_t ha0, la0, ha1, la1, hb0, lb0, hb1, lb1;
    mul_wide(kPhiloxM0, a0, ha0, la0);
    mul_wide(kPhiloxM0, b0, hb0, lb0);
    mul_wide(kPhiloxM1, a2, ha1, la1);
    mul_wide(kPhiloxM1, b2, hb1, lb1);
    const uint32_t ya0 = round < 2 ? ha1 ^ a1 ^ k0 : xor3(ha1, a1, k0);
    const uint32_t yb0 = round < 2 ? hb1 ^ b1 ^ k0 : xor3(hb1, b1, k0);
    const uint32_t ya2 = round < 3 ? ha0 ^ a3 ^ k1 : xor3(ha0, a3, k1);
    const uint32_t yb2 = round < 3 ? hb0 ^ b3 ^ k1 : xor3(hb0, b3, k1);
    a0 = ya0;
    a1 = la1;
    a2 = ya2;
    a3 = la0;
    b0 = yb0;
    b1 = lb1;
    b2 = yb2;
    b3 = lb0;
    k0 += kPhiloxW0;
    k1 += kPhiloxW1;
  }
  const float2 a_lo = box_muller<UNIT>(a0, a1), b_lo = box_muller<UNIT>(b0, b1);
  const float2 a_hi = box_muller<UNIT>(a2, a3), b_hi = box_muller<UNIT>(b2, b3);
  A = make_float4(a_lo.x, a_lo.y, a_hi.x, a_hi.y);
  B = make_float4(b_lo.x, b_lo.y, b_hi.x, b_hi.y);
}

}  // namespace dust
