// q4_qout.h -- the GEMM epilogue that writes C already quantized (MXFP4, or
// NVFP4 under a given tensor scale) instead of bf16, so the next layer's
// W4A4 GEMM reads 4-bit activations without a separate quantization pass
// (the pages compute activation scales at the end of the previous kernel,
// "Quantization in deployment", Exercises, "The cost of block FP8").
//
// The bytes are those q4_quantize writes for the bf16 C the same kernel
// writes otherwise: each accumulator is rounded to bf16 (as the bf16
// output is), then encoded by the quantizer's own encoders (q4_encode.h).
//
// Register layout taken: lane l of a wave holds, for row tile i and column
// tile jj, the 4 consecutive columns n = n0 + 16jj + 4(l/16) + q (q = 0..3)
// of row m = m0 + 16i + l%16 -- the layout of a 16x16 matrix-core result
// whose row operand is the weight.  Column tiles 2b and 2b+1 form one
// 32-column block of a row, spread over the 4 lanes with the same l%16:
// each lane holds 8 of its values.  The block absmax is two cross-lane max
// steps; each lane encodes its 8 values into one 32-bit word; two lane
// exchanges then give lane g = l/16 the dword g of the row's 16 code bytes
// (codes k = 8g .. 8g+7), and 16 lanes (one per row) store their dwords
// side by side: in the tiled layout the 16 rows' pieces are one contiguous
// 256 bytes.
#pragma once

#include "q4_encode.h"
#include "q4_launch.h"
#include "q4_layout.h"
#include "q4_mma.h"

namespace q4 {

__device__ __forceinline__ float absmax4(const Chunk8& x, int h) {
  return fmaxf(fmaxf(fabsf(x.v[4 * h]), fabsf(x.v[4 * h + 1])),
               fmaxf(fabsf(x.v[4 * h + 2]), fabsf(x.v[4 * h + 3])));
}

// Max over the four lanes l%16 == lane%16 (lanes 16 and 32 apart).
__device__ __forceinline__ float max_over_row_lanes(float a) {
  a = fmaxf(a, __shfl_xor(a, 16));
  return fmaxf(a, __shfl_xor(a, 32));
}

// The NVFP4 output's copy of the tensor scale (one thread of the grid).
template <int OFMT>
__device__ __forceinline__ void qout_copy_gs(const QOut& q) {
  if constexpr (OFMT == kOutNvfp4)
    if (blockIdx.x == 0 && threadIdx.x == 0) *q.gs_out = *q.gs_in;
}

// Writes the wave's RT x CT tiles of C quantized.  m0 = the row of this
// lane in row tile 0, nb0 = the first column of the wave's tiles (a
// multiple of 32); N % 32 == 0.  Rows past M are quantized as zeros and
// stored only where the tiled layout pads the last tile.  Every lane of the
// wave must call this (the cross-lane steps need them all).
template <int OFMT, int RT, int CT>
__device__ __forceinline__ void store_quantized(const f32x4_t (&acc)[RT][CT], int m0, int nb0, int M, int N,
                                                const QOut& q, int lane) {
  static_assert(CT % 2 == 0, "32-column blocks are pairs of 16-column tiles");
  const int g = lane >> 4;
  const int srows = q.tiled ? ((M + 15) & ~15) : M;
  float gs = 0.0f, rgs = 0.0f;
  bool gs_ok = false;
  if constexpr (OFMT == kOutNvfp4) {
    gs = *q.gs_in;
    rgs = 1.0f / gs;
    gs_ok = in_bracket_range(gs);
  }
  const int src_a = 16 * (2 * (g & 1)) + (lane & 15), src_b = src_a + 16;
#pragma unroll
  for (int b = 0; b < CT / 2; ++b) {
    const int k0 = nb0 + 32 * b;
    if (k0 >= N) break;  // wave-uniform
#pragma unroll
    for (int i = 0; i < RT; ++i) {
      const int m = m0 + 16 * i;
      Chunk8 x;
      const uint32_t p0 = pk_bf16(acc[i][2 * b][0], acc[i][2 * b][1]);
      const uint32_t p1 = pk_bf16(acc[i][2 * b][2], acc[i][2 * b][3]);
      const uint32_t p2 = pk_bf16(acc[i][2 * b + 1][0], acc[i][2 * b + 1][1]);
      const uint32_t p3 = pk_bf16(acc[i][2 * b + 1][2], acc[i][2 * b + 1][3]);
      const bool live = m < M;
      x.v[0] = live ? bf16_lo(p0) : 0.0f; x.v[1] = live ? bf16_hi(p0) : 0.0f;
      x.v[2] = live ? bf16_lo(p1) : 0.0f; x.v[3] = live ? bf16_hi(p1) : 0.0f;
      x.v[4] = live ? bf16_lo(p2) : 0.0f; x.v[5] = live ? bf16_hi(p2) : 0.0f;
      x.v[6] = live ? bf16_lo(p3) : 0.0f; x.v[7] = live ? bf16_hi(p3) : 0.0f;
      uint32_t packed, sbits;
      if constexpr (OFMT == kOutMxfp4) {
        const uint32_t e = mx_e8m0(max_over_row_lanes(absmax8(x)));
        packed = e2m1_pack8(x, e8m0_value(e));
        sbits = e;
      } else {
        const uint32_t c0 = nv_scale_code(max_over_row_lanes(absmax4(x, 0)), gs, rgs, gs_ok);
        const uint32_t c1 = nv_scale_code(max_over_row_lanes(absmax4(x, 1)), gs, rgs, gs_ok);
        packed = nv_pack8_halves(x, e4m3_value(c0) * gs, e4m3_value(c1) * gs);
        sbits = c0 | (c1 << 8);
      }
      // lane g's word: codes k = 4g..4g+3 (low half) and 16+4g..16+4g+3
      // (high half); dword g of the row's piece is codes 8g..8g+7
      const uint32_t wa = __shfl(packed, src_a), wb = __shfl(packed, src_b);
      const uint32_t d = g < 2 ? ((wa & 0xFFFFu) | (wb << 16)) : ((wa >> 16) | (wb & 0xFFFF0000u));
      if (m < srows) {
        const int64_t off = q.tiled ? code_off8<kLayoutTiled>(m, k0, N) : code_off8<kLayoutRows>(m, k0, N);
        *reinterpret_cast<uint32_t*>(q.codes + off + 4 * g) = d;
        if (g == 0) {
          if constexpr (OFMT == kOutMxfp4) {
            const int64_t so = q.tiled ? scale_off<1, kLayoutTiled>(m, k0, N) : scale_off<1, kLayoutRows>(m, k0, N);
            q.scales[so] = (uint8_t)sbits;
          } else {
            const int64_t so = q.tiled ? scale_off<2, kLayoutTiled>(m, k0, N) : scale_off<2, kLayoutRows>(m, k0, N);
            *reinterpret_cast<uint16_t*>(q.scales + so) = (uint16_t)sbits;
          }
        }
      }
    }
  }
}

}  // namespace q4
