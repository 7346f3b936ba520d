// fp8.hip -- per-token FP8 (E4M3) activations for the W4A8 scheme.
//
// W4A8 keeps INT4 weights and quantizes the activations to FP8 so that the
// products run on FP8 matrix cores ("Low-bit inference for very large MoE",
// table "Kernels on different hardware", row W4A8).  The activation
// quantizer is the per-token one of "Quantization in deployment" (formats.py,
// fp8 with one scale per row): scale = max(amax_row, 1e-12) / 448, every
// value divided by the scale (IEEE fp32 division), clamped to +-448 and
// rounded to the nearest E4M3 value, ties to the even code; the sign bit of
// the input is kept (-0 and negatives that round to zero give 0x80).
//
// Layouts (include/q4.h, format Q4_FP8_ROW): row-major codes [rows][cols],
// or the tiled layout the W4A8 kernel streams, with fp32 scales [rows] in
// both.  Tiled: 16-row x 128-k tiles of 2048 bytes; lane l = 16g + n of a
// tile owns 32 operand bytes for row n, k = 32g .. 32g + 31, and operand
// byte p = 4d + i (dword d = 2w + h) holds k = 32g + 8w + 2i + h, i.e. the
// even elements of each group of eight in one dword and the odd ones in the
// next -- the order in which the W4A8 kernel unpacks INT4 nibble pairs.
// Operand bytes 0..15 of every lane come first (1 KB), then bytes 16..31,
// so each half is one contiguous 64-lane load.
#include "q4_device.h"
#include "q4_launch.h"
#include "q4_layout.h"

namespace q4 {
namespace {

constexpr int kRowsPerBlock = 4;  // one wave per row

// E4M3 code (sign included) of x for the row scale s.
__device__ __forceinline__ uint32_t fp8_code(float x, float s) {
  const float y = x / s;
  const float t = fminf(fabsf(y), 448.0f);
  return ((f2u(y) >> 24) & 0x80u) | e4m3_encode(t);
}

template <int LAYOUT>
__global__ void __launch_bounds__(64 * kRowsPerBlock)
fp8_rows_quantize_kernel(const uint16_t* __restrict__ src, int64_t ld, int64_t rows, int64_t cols,
                         int64_t srows, uint8_t* __restrict__ codes, float* __restrict__ scales) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (r >= srows) return;
  if (r >= rows) {  // padding row of the last tile: zero codes
    for (int64_t k0 = (int64_t)lane * 8; k0 < cols; k0 += 512) {
      *reinterpret_cast<uint32_t*>(codes + fp8_tiled_dword(r, k0, cols, 0)) = 0u;
      *reinterpret_cast<uint32_t*>(codes + fp8_tiled_dword(r, k0, cols, 1)) = 0u;
    }
    return;
  }
  const uint16_t* row = src + r * ld;
  // pass 1: the row's largest magnitude (exact: max of bf16 values)
  float amax = 0.0f;
  for (int64_t k0 = (int64_t)lane * 8; k0 < cols; k0 += 512) {
    const uint4 v = *reinterpret_cast<const uint4*>(row + k0);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(w[j])), fabsf(bf16_hi(w[j]))));
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  const float s = fmaxf(amax, 1e-12f) / 448.0f;
  if (lane == 0) scales[r] = s;
  // pass 2: encode (the row is re-read from cache)
  for (int64_t k0 = (int64_t)lane * 8; k0 < cols; k0 += 512) {
    const uint4 v = *reinterpret_cast<const uint4*>(row + k0);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t e[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      e[2 * j] = fp8_code(bf16_lo(w[j]), s);
      e[2 * j + 1] = fp8_code(bf16_hi(w[j]), s);
    }
    if constexpr (LAYOUT == kLayoutRows) {
      uint2 o;
      o.x = e[0] | (e[1] << 8) | (e[2] << 16) | (e[3] << 24);
      o.y = e[4] | (e[5] << 8) | (e[6] << 16) | (e[7] << 24);
      *reinterpret_cast<uint2*>(codes + r * cols + k0) = o;
    } else {
      *reinterpret_cast<uint32_t*>(codes + fp8_tiled_dword(r, k0, cols, 0)) =
          e[0] | (e[2] << 8) | (e[4] << 16) | (e[6] << 24);
      *reinterpret_cast<uint32_t*>(codes + fp8_tiled_dword(r, k0, cols, 1)) =
          e[1] | (e[3] << 8) | (e[5] << 16) | (e[7] << 24);
    }
  }
}

constexpr int kThreads = 256;

// value = fp32(E4M3 value * row scale); 8 values per thread.
template <int LAYOUT, int OUT>
__global__ void __launch_bounds__(kThreads)
fp8_rows_dequant_kernel(const uint8_t* __restrict__ codes, const float* __restrict__ scales,
                        int64_t rows, int64_t cols, void* __restrict__ dst, int64_t ld) {
  const int64_t cpr = cols >> 3, total = rows * cpr;
  for (int64_t c = (int64_t)blockIdx.x * kThreads + threadIdx.x; c < total;
       c += (int64_t)gridDim.x * kThreads) {
    const int64_t r = c / cpr, k0 = (c - r * cpr) * 8;
    uint32_t e[8];
    if constexpr (LAYOUT == kLayoutRows) {
      const uint2 v = *reinterpret_cast<const uint2*>(codes + r * cols + k0);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        e[j] = (v.x >> (8 * j)) & 0xFFu;
        e[4 + j] = (v.y >> (8 * j)) & 0xFFu;
      }
    } else {
      const uint32_t ev = *reinterpret_cast<const uint32_t*>(codes + fp8_tiled_dword(r, k0, cols, 0));
      const uint32_t od = *reinterpret_cast<const uint32_t*>(codes + fp8_tiled_dword(r, k0, cols, 1));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        e[2 * i] = (ev >> (8 * i)) & 0xFFu;
        e[2 * i + 1] = (od >> (8 * i)) & 0xFFu;
      }
    }
    const float s = scales[r];
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float m = e4m3_value(e[j] & 0x7Fu) * s;
      v[j] = (e[j] & 0x80u) ? -m : m;
    }
    if constexpr (OUT == 0) {
      uint4 o;
      o.x = f32_to_bf16_rne(v[0]) | (f32_to_bf16_rne(v[1]) << 16);
      o.y = f32_to_bf16_rne(v[2]) | (f32_to_bf16_rne(v[3]) << 16);
      o.z = f32_to_bf16_rne(v[4]) | (f32_to_bf16_rne(v[5]) << 16);
      o.w = f32_to_bf16_rne(v[6]) | (f32_to_bf16_rne(v[7]) << 16);
      *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(dst) + r * ld + k0) = o;
    } else {
      float4* o = reinterpret_cast<float4*>(reinterpret_cast<float*>(dst) + r * ld + k0);
      o[0] = make_float4(v[0], v[1], v[2], v[3]);
      o[1] = make_float4(v[4], v[5], v[6], v[7]);
    }
  }
}

}  // namespace

hipError_t launch_fp8_rows_quantize(int layout, const uint16_t* src, int64_t ld, int64_t rows,
                                    int64_t cols, uint8_t* codes, float* scales, hipStream_t stream) {
  const int64_t srows = layout == kLayoutTiled ? ((rows + 15) >> 4) << 4 : rows;
  if (srows == 0 || cols == 0) return hipSuccess;
  const unsigned grid = (unsigned)((srows + kRowsPerBlock - 1) / kRowsPerBlock);
  if (layout == kLayoutTiled)
    fp8_rows_quantize_kernel<kLayoutTiled><<<grid, 64 * kRowsPerBlock, 0, stream>>>(src, ld, rows, cols, srows,
                                                                                  codes, scales);
  else
    fp8_rows_quantize_kernel<kLayoutRows><<<grid, 64 * kRowsPerBlock, 0, stream>>>(src, ld, rows, cols, srows,
                                                                                 codes, scales);
  return hipGetLastError();
}

hipError_t launch_fp8_rows_dequant(int layout, const uint8_t* codes, const float* scales, int64_t rows,
                                   int64_t cols, void* dst, int dst_dtype, int64_t ld, hipStream_t stream) {
  const int64_t chunks = rows * (cols >> 3);
  if (!chunks) return hipSuccess;
  int64_t b = (chunks + kThreads - 1) / kThreads;
  if (b > (1 << 20)) b = 1 << 20;
  const unsigned grid = (unsigned)b;
#define Q4_FP8_DQ(L, O) fp8_rows_dequant_kernel<L, O><<<grid, kThreads, 0, stream>>>(codes, scales, rows, cols, dst, ld)
  if (layout == kLayoutTiled) {
    if (dst_dtype == 0) Q4_FP8_DQ(kLayoutTiled, 0); else Q4_FP8_DQ(kLayoutTiled, 1);
  } else {
    if (dst_dtype == 0) Q4_FP8_DQ(kLayoutRows, 0); else Q4_FP8_DQ(kLayoutRows, 1);
  }
#undef Q4_FP8_DQ
  return hipGetLastError();
}

}  // namespace q4
