// q4_mma.h -- register-level pieces shared by the W4 matmul kernels on
// gfx950: vector types, 8-code dequantization to bf16 (the "dequantize
// weights to BF16 in registers" step of the W4A16 scheme, "Low-bit
// inference for very large MoE", table "Kernels on different hardware"),
// and the bf16 matrix-core step.
#pragma once

#include "q4_device.h"

namespace q4 {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }
__device__ __forceinline__ uint32_t as_u32(bf16x2_t v) { return __builtin_bit_cast(uint32_t, v); }

// 8 E2M1 codes (nibble j of `w` is element j) times a power-of-two scale
// -> 8 bf16, exact.  v_cvt_scalef32_pk_bf16_fp4 converts the two codes of
// one byte (low nibble first) and applies only the exponent of its fp32
// scale operand (measured on gfx950: a scale of 1.5 acts as 1.0), which is
// exactly an E8M0 scale.
__device__ __forceinline__ bf16x8_t dq8_e2m1(uint32_t w, float scale) {
  u32x4_t r;
  r[0] = as_u32(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0));
  r[1] = as_u32(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1));
  r[2] = as_u32(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2));
  r[3] = as_u32(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3));
  return as_bf16x8(r);
}

// Two fp32 values -> packed bf16 pair (low = a), round to nearest even:
// one v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
  return as_u32(__builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

// Four consecutive bf16 outputs: one 8-byte store where dst is 8-byte
// aligned (the usual case: C 16-byte aligned, ldc a multiple of 4), else
// two 4-byte or four 2-byte stores -- the C ABI accepts any 2-byte
// aligned output and any leading dimension.
__device__ __forceinline__ void store_bf16x4(uint16_t* dst, float v0, float v1, float v2, float v3) {
  const uint32_t lo = pk_bf16(v0, v1), hi = pk_bf16(v2, v3);
  const uintptr_t a = reinterpret_cast<uintptr_t>(dst);
  if ((a & 7) == 0) {
    *reinterpret_cast<uint2*>(dst) = make_uint2(lo, hi);
  } else if ((a & 3) == 0) {
    reinterpret_cast<uint32_t*>(dst)[0] = lo;
    reinterpret_cast<uint32_t*>(dst)[1] = hi;
  } else {
    dst[0] = (uint16_t)lo;
    dst[1] = (uint16_t)(lo >> 16);
    dst[2] = (uint16_t)hi;
    dst[3] = (uint16_t)(hi >> 16);
  }
}

// 8 E2M1 codes times an arbitrary fp32 scale (NVFP4: E4M3 * gs) -> 8 bf16:
// exact fp32 code values, one fp32 multiply, one rounding to bf16.
__device__ __forceinline__ bf16x8_t dq8_e2m1_mul(uint32_t w, float scale) {
  u32x4_t r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f32x2_t v;
    if (j == 0) v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
    else if (j == 1) v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
    else if (j == 2) v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
    else v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
    r[j] = pk_bf16(v[0] * scale, v[1] * scale);
  }
  return as_bf16x8(r);
}

// 8 INT4 codes (two's complement nibbles) -> 8 bf16 of (q + 8) * s + off.
// Offset-binary trick: nibble ^ 8 = q + 8 in 0..15, read as a byte by
// v_cvt_f32_ubyte; with off = -(8 + z) * s this is (q - z) * s, exact in
// fp32 (<= 15 bits), so one fma gives it; then one rounding to bf16.
// Symmetric INT4: z = 0; INT4 with a zero point: z from the group's word.
__device__ __forceinline__ bf16x8_t dq8_int4_off(uint32_t w, float s, float m8) {
  const uint32_t lo = (w & 0x0F0F0F0Fu) ^ 0x08080808u;          // elements 0,2,4,6
  const uint32_t hi = ((w >> 4) & 0x0F0F0F0Fu) ^ 0x08080808u;   // elements 1,3,5,7
  u32x4_t r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float e0 = __builtin_fmaf((float)((lo >> (8 * j)) & 0xFFu), s, m8);
    const float e1 = __builtin_fmaf((float)((hi >> (8 * j)) & 0xFFu), s, m8);
    r[j] = pk_bf16(e0, e1);
  }
  return as_bf16x8(r);
}

__device__ __forceinline__ bf16x8_t dq8_int4(uint32_t w, float s) { return dq8_int4_off(w, s, -8.0f * s); }

// 8 INT4 codes -> 8 bf16 of 128 + (q + 8), exact and without the scale (for
// kernels that apply a group's scale after the matrix step).  bf16 0x4300 is
// 128 with a last place of 1, so the offset-binary nibble q ^ 8 placed in
// the four low mantissa bits reads as 128 + q + 8: one bit-select per pair
// (nibble with its top bit flipped, 0x4300 elsewhere) after a shift.  The
// pairs are (0,4), (1,5), (2,6), (3,7), so the output holds elements
// 0,4,1,5,2,6,3,7 -- the other operand must follow that order
// (x8_int4_order).
__device__ __forceinline__ bf16x8_t dq8_int4_biased(uint32_t w) {
  constexpr uint32_t kNib = 0x000F000Fu, kMagic = 0x43084308u;
  u32x4_t r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t v = w >> (4 * j);
    r[j] = ((v ^ kMagic) & kNib) | (kMagic & ~kNib);
  }
  return as_bf16x8(r);
}

// Eight bf16 in k order (x0..x7) -> the order of dq8_int4_biased:
// x0,x4,x1,x5,x2,x6,x3,x7 (one byte permute per output dword).
__device__ __forceinline__ u32x4_t x8_int4_order(u32x4_t v) {
  return u32x4_t{__builtin_amdgcn_perm(v[2], v[0], 0x05040100u), __builtin_amdgcn_perm(v[2], v[0], 0x07060302u),
                 __builtin_amdgcn_perm(v[3], v[1], 0x05040100u), __builtin_amdgcn_perm(v[3], v[1], 0x07060302u)};
}

// INT4 with a zero point: the group's 32-bit word (fp16 scale, int8 zero
// point in bits 16..23) -> (scale, offset) for dq8_int4_off.
__device__ __forceinline__ void int4zp_scale(uint32_t word, float& s, float& off) {
  s = fp16_value(word & 0xFFFFu);
  off = -(float)(8 + (int)(int8_t)((word >> 16) & 0xFFu)) * s;
}

// bf16 matrix core: C(16x16) += A(16x32) * B(32x16), fp32 accumulation.
// Lane l supplies A[l%16][8(l/16)..+8] and B[8(l/16)..+8][l%16]; the result
// lane l, register r holds C[4(l/16)+r][l%16].
__device__ __forceinline__ f32x4_t mma16x16x32(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

}  // namespace q4
