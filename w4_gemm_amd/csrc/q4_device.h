// q4_device.h -- device-side number-format helpers for the gfx950 kernels.
//
// Bit-level encoders/decoders for the narrow formats the library stores:
// E2M1 (grid +-{0,0.5,1,1.5,2,3,4,6}), E4M3 (bias 7, max 448, min normal
// 2^-6, min subnormal 2^-9), E8M0 (power-of-two exponent, bias 127), FP16
// and BF16.  Every rounding is round-to-nearest, ties to the even code.
// (Formats: "Quantization in deployment", format cheat sheet and formats.py;
// "Quantization chains", "E4M3 against E5M2".)
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q4 {

__device__ __forceinline__ uint32_t f2u(float f) { return __builtin_bit_cast(uint32_t, f); }
__device__ __forceinline__ float u2f(uint32_t u) { return __builtin_bit_cast(float, u); }

// bf16 bits -> fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t pair) { return u2f(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return u2f(pair & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = f2u(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Value j (0..7, per lane) of eight, by a three-level select (the values
// come in as separate scalars so the selects stay register moves).
__device__ __forceinline__ float pick8(float a0, float a1, float a2, float a3, float a4, float a5, float a6,
                                       float a7, int j) {
  const bool b0 = j & 1, b1 = j & 2, b2 = j & 4;
  const float v01 = b0 ? a1 : a0, v23 = b0 ? a3 : a2, v45 = b0 ? a5 : a4, v67 = b0 ? a7 : a6;
  const float v03 = b1 ? v23 : v01, v47 = b1 ? v67 : v45;
  return b2 ? v47 : v03;
}

// E2M1 code -> value (sign included).
__device__ __forceinline__ float e2m1_value(uint32_t nib) {
  // magnitudes 0,0.5,1,1.5,2,3,4,6: exponent field e = bits 2:1, mantissa m = bit 0
  uint32_t e = (nib >> 1) & 3u, m = nib & 1u;
  float mag = (e == 0) ? 0.5f * (float)m : (float)(2u + m) * (float)(1u << (e - 1)) * 0.5f;
  return (nib & 8u) ? -mag : mag;
}

// E4M3 code (sign 0) of t in [0, 448].
__device__ __forceinline__ uint32_t e4m3_encode(float t) {
  if (t < 0.015625f) {                        // below 2^-6: subnormal step 2^-9
    return (uint32_t)__builtin_rintf(t * 512.0f);  // 8 -> 0x08, the min normal
  }
  uint32_t u = f2u(t);
  u += 0x7FFFFu + ((u >> 20) & 1u);          // round mantissa to 3 bits
  return (u >> 20) - ((127u - 7u) << 3);     // rebias exponent 127 -> 7
}

// E4M3 code (sign bit ignored) -> fp32, exact and branch-free: the code's
// exponent and mantissa bits placed at the top of an fp32 read as
// 2^(e-127) (1 + m/8), or m 2^-129 for e = 0 (an fp32 subnormal); times
// 2^120 that is 2^(e-7) (1 + m/8), resp. m 2^-9.  Needs fp32 denormals
// preserved, which the kernels are built with.
__device__ __forceinline__ float e4m3_value(uint32_t c) {
  return u2f((c & 0x7Fu) << 20) * 0x1p120f;
}

// FP16 bits (sign 0) of t >= 0; >= 65520 gives +inf.
__device__ __forceinline__ uint32_t fp16_encode(float t) {
  if (t >= 65520.0f) return 0x7C00u;
  if (t < 6.103515625e-05f) {                 // below 2^-14: subnormal step 2^-24
    return (uint32_t)__builtin_rintf(t * 16777216.0f);
  }
  uint32_t u = f2u(t);
  u += 0xFFFu + ((u >> 13) & 1u);             // round mantissa to 10 bits
  return (u >> 13) - ((127u - 15u) << 10);
}

// FP16 bits -> fp32: one v_cvt_f32_f16, exact for every fp16 value
// (subnormals included: the kernels run with fp16 denormals preserved).
__device__ __forceinline__ float fp16_value(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// MXFP4 scale exponent for a block whose absmax is amax (fp32, >= 0):
// floor(log2(max(amax, 1e-12))) - 2, read from the exponent bits (amax is
// normal once clamped).  Returns the biased E8M0 byte.
__device__ __forceinline__ uint32_t mx_e8m0(float amax) {
  float a = fmaxf(amax, 1e-12f);
  uint32_t biased = (f2u(a) >> 23) & 0xFFu;   // floor(log2 a) + 127
  return biased - 2u;
}

// 2^(e - 127) for a biased E8M0 byte e in [1, 254].
__device__ __forceinline__ float e8m0_value(uint32_t e) { return u2f(e << 23); }

}  // namespace q4
