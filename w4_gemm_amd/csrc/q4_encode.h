// q4_encode.h -- the element encoders of the MXFP4 and NVFP4 quantizers,
// shared by q4_quantize's kernels and the GEMM epilogues that write their
// output quantized, so both produce the same bytes for the same values.
//
// MXFP4 ("Quantization in deployment", formats.py mxfp4 and fp4): codes
// E2M1(clamp(w / 2^e, +-6)) for the block's power-of-two scale.  NVFP4
// (same file, nvfp4): block scale E4M3(min((amax_b / 6) / gs, 448)),
// codes E2M1(clamp(w / fp32(E4M3 * gs), +-6)).  Ties to the even code.
#pragma once

#include "q4_device.h"

// Each function with fp32 arithmetic turns contraction off in its own body
// (a file-level pragma here would reach the kernels that include this).
namespace q4 {

struct Chunk8 {
  float v[8];
};

__device__ __forceinline__ Chunk8 load8(const uint16_t* p, bool valid) {
  Chunk8 c;
  uint4 raw = valid ? *reinterpret_cast<const uint4*>(p) : make_uint4(0, 0, 0, 0);
  c.v[0] = bf16_lo(raw.x); c.v[1] = bf16_hi(raw.x);
  c.v[2] = bf16_lo(raw.y); c.v[3] = bf16_hi(raw.y);
  c.v[4] = bf16_lo(raw.z); c.v[5] = bf16_hi(raw.z);
  c.v[6] = bf16_lo(raw.w); c.v[7] = bf16_hi(raw.w);
  return c;
}

// Eight values -> eight packed E2M1 nibbles (element j in bits 4j..4j+3) of
// value / scale, with scale a power of two.  v_cvt_scalef32_pk_fp4_f32
// divides by 2^floor(log2 scale) (only the exponent of its scale operand is
// used), rounds to the nearest E2M1 value with ties to the even code,
// saturates to +-6 and keeps the sign bit -- the rounding rule of the
// formats here, checked on gfx950 against every multiple of 1/128 in
// [0, 10) including all the midpoints.
__device__ __forceinline__ uint32_t e2m1_pack8(const Chunk8& c, float scale) {
  uint32_t p = 0;
  p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, c.v[0], c.v[1], scale, 0);
  p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, c.v[2], c.v[3], scale, 1);
  p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, c.v[4], c.v[5], scale, 2);
  p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, c.v[6], c.v[7], scale, 3);
  return p;
}

// Division by a block scale.  Each code is a correctly rounded fp32
// quotient w / s (NVFP4: also (amax / 6) / gs for the block scale) put
// through a rounding to a short format (E2M1, E4M3, a clamped integer)
// that is monotone in the value.  Here the quotient is formed as a product
// with a reciprocal, twice, the product nudged down and up by a relative
// 2^-20: the reciprocal (v_rcp_f32, within 1 ulp; an fp32 division, within
// 1/2 ulp) and the products add under 2^-21 relative error in all, and the
// fp32 quotient itself is within 2^-23 of the exact one (two roundings for
// the block scale), so the two nudged products bracket it.  Where both
// round to the same code, so does the quotient; where they differ (a
// quotient within about 2^-20 of a rounding boundary, an exact tie) the
// division is done.  This needs the operands in the normal range: the
// callers take this path only for scales within [2^-100, 2^100]; a product
// that overflows then stands for a quotient that takes the top code on
// both sides, one that underflows for one that rounds to zero on both.
constexpr float kNudgeDown = 1.0f - 0x1p-20f, kNudgeUp = 1.0f + 0x1p-20f;

__device__ __forceinline__ bool in_bracket_range(float s) { return s >= 0x1p-100f && s <= 0x1p100f; }

// Codes p of a chunk whose two bracket products disagreed on the nibbles
// set in diff: each of those values is divided by its scale (eff0 for
// elements 0..3, eff1 for 4..7) and its code replaced, one value per pass
// of the loop.  Exact ties (the fp32 quotient on an E2M1 midpoint) are not
// rare: eff = fp32(E4M3 * gs) often has a short mantissa, and 2688 = 6 * 448
// puts the factors 3 and 7 of many bf16 values into it, so several values
// in a hundred can hit a midpoint.  Dividing only those values, rather than
// the whole chunk whenever any lane of the wave needs one, cut the NVFP4
// block pass on the 28672 x 8192 decode weight from 151 to ~110 us.
__device__ __forceinline__ uint32_t e2m1_fix(const Chunk8& x, float eff0, float eff1, uint32_t p, uint32_t diff) {
#pragma clang fp contract(off)
  while (diff != 0u) {
    const int j = __builtin_ctz(diff) >> 2;
    const float v = pick8(x.v[0], x.v[1], x.v[2], x.v[3], x.v[4], x.v[5], x.v[6], x.v[7], j);
    const float y = v / (j < 4 ? eff0 : eff1);  // fp32 division by the scale as used
    const uint32_t c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, y, 0.0f, 1.0f, 0) & 0xFu;
    const uint32_t m = 0xFu << (4 * j);
    p = (p & ~m) | (c << (4 * j));
    diff &= ~m;
  }
  return p;
}

// E2M1 codes of x[j] / eff.
__device__ __forceinline__ uint32_t e2m1_pack8_div(const Chunk8& x, float eff) {
#pragma clang fp contract(off)
  if (in_bracket_range(eff)) {
    const float r = __builtin_amdgcn_rcpf(eff);
    const float rl = r * kNudgeDown, rh = r * kNudgeUp;
    Chunk8 lo, hi;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      lo.v[j] = x.v[j] * rl;
      hi.v[j] = x.v[j] * rh;
    }
    const uint32_t pl = e2m1_pack8(lo, 1.0f), ph = e2m1_pack8(hi, 1.0f);
    if (__builtin_expect(pl == ph, 1)) return pl;
    return e2m1_fix(x, eff, eff, pl, pl ^ ph);
  }
  Chunk8 y;
#pragma unroll
  for (int j = 0; j < 8; ++j) y.v[j] = x.v[j] / eff;  // fp32 division by the scale as used
  return e2m1_pack8(y, 1.0f);
}

// E4M3 code of min((amax / 6) / gs, 448); rgs = 1 / gs (an fp32 division),
// gs_ok = in_bracket_range(gs).
__device__ __forceinline__ uint32_t nv_scale_code(float amax, float gs, float rgs, bool gs_ok) {
#pragma clang fp contract(off)
  if (gs_ok) {
    const float a = amax * rgs;
    // both bracket values in one v_cvt_pk_fp8_f32 (E4M3, round to nearest
    // even; the inputs are in [0, 448]): bytes 0 and 1
    const uint32_t c2 = __builtin_amdgcn_cvt_pk_fp8_f32(fminf(a * (kNudgeDown / 6.0f), 448.0f),
                                                        fminf(a * (kNudgeUp / 6.0f), 448.0f), 0, false);
    if (__builtin_expect((c2 & 0xFFu) == ((c2 >> 8) & 0xFFu), 1)) return c2 & 0xFFu;
  }
  return e4m3_encode(fminf((amax / 6.0f) / gs, 448.0f));
}

__device__ __forceinline__ float absmax8(const Chunk8& c) {
  float a = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) a = fmaxf(a, fabsf(c.v[j]));
  return a;
}

// NVFP4 codes of eight values whose first four belong to one 16-block
// (scale eff0 = fp32(E4M3 * gs)) and last four to another (eff1): element j
// in bits 4j..4j+3.  A block whose E4M3 scale is 0 (eff 0) keeps only the
// sign bits, as the quantizers store it.
__device__ __forceinline__ uint32_t nv_pack8_halves(const Chunk8& x, float eff0, float eff1) {
#pragma clang fp contract(off)
  uint32_t p = 0;
  if (in_bracket_range(eff0) && in_bracket_range(eff1)) {
    const float r0 = __builtin_amdgcn_rcpf(eff0), r1 = __builtin_amdgcn_rcpf(eff1);
    Chunk8 lo, hi;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float r = j < 4 ? r0 : r1;
      lo.v[j] = x.v[j] * (r * kNudgeDown);
      hi.v[j] = x.v[j] * (r * kNudgeUp);
    }
    const uint32_t pl = e2m1_pack8(lo, 1.0f), ph = e2m1_pack8(hi, 1.0f);
    p = __builtin_expect(pl == ph, 1) ? pl : e2m1_fix(x, eff0, eff1, pl, pl ^ ph);
  } else {
    Chunk8 y;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float e = j < 4 ? eff0 : eff1;
      y.v[j] = e != 0.0f ? x.v[j] / e : 0.0f;
    }
    p = e2m1_pack8(y, 1.0f);
  }
  // zero scales: magnitude codes 0, sign bits kept
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if ((j < 4 ? eff0 : eff1) == 0.0f) p = (p & ~(0xFu << (4 * j))) | (((f2u(x.v[j]) >> 31) << 3) << (4 * j));
  return p;
}

}  // namespace q4
