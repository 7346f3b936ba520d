// q4_layout.h -- byte offsets of codes and scales in the two layouts of a
// quantized tensor (row-major and 16x128 tiled; the layouts are defined in
// include/q4.h).  Shared by the quantizer, the dequantizer and the matmul
// kernels so every kernel addresses a tensor the same way.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q4 {

constexpr int kLayoutRows = 0;
constexpr int kLayoutTiled = 1;

template <int FMT>
struct FmtTraits {
  static constexpr int G = (FMT == 0 || FMT == 4) ? 128 : (FMT == 1 ? 32 : 16);  // block size along K
};

// Byte offset of the 4 code bytes holding elements k0..k0+7 (k0 % 8 == 0)
// of row r.  K = columns.
template <int LAYOUT>
__host__ __device__ __forceinline__ int64_t code_off8(int64_t r, int64_t k0, int64_t K) {
  if constexpr (LAYOUT == kLayoutRows) {
    return r * (K >> 1) + (k0 >> 1);
  } else {
    const int64_t S = K >> 7;
    const int64_t t = r >> 4, n = r & 15, s = k0 >> 7, g = (k0 >> 5) & 3, piece = (k0 >> 3) & 3;
    return ((t * S + s) << 10) + ((g * 16 + n) << 4) + (piece << 2);
  }
}

// Offset (in scale elements: fp16 for INT4, bytes otherwise) of the scale of
// the block holding element k of row r.
template <int FMT, int LAYOUT>
__host__ __device__ __forceinline__ int64_t scale_off(int64_t r, int64_t k, int64_t K) {
  if constexpr (LAYOUT == kLayoutRows) {
    return r * (K / FmtTraits<FMT>::G) + k / FmtTraits<FMT>::G;
  } else {
    const int64_t Q = K >> 9;
    const int64_t t = r >> 4, n = r & 15, s = k >> 7, q = s >> 2, i = s & 3;
    if constexpr (FMT == 0 || FMT == 4) {  // fp16 scales / 32-bit scale + zero-point words
      return (((t * Q + q) << 4) + n) * 4 + i;
    } else {
      const int64_t g = (k >> 5) & 3;
      const int64_t l = g * 16 + n;
      if constexpr (FMT == 1) return (((t * Q + q) << 6) + l) * 4 + i;
      const int64_t h = (k >> 4) & 1;
      return (((t * Q + q) << 6) + l) * 8 + 2 * i + h;
    }
  }
}

// FP8 activations (per-row E4M3, the W4A8 operand), tiled layout: byte
// offset of the operand dword holding the even (h = 0) or odd (h = 1)
// elements of k0 .. k0 + 7 (k0 % 8 == 0) of row r.  Tiles of 16 rows x 128
// k are 2048 bytes; lane l = 16g + n owns k = 32g .. 32g + 31 of row n as 32
// operand bytes, operand dword 2w + h holding elements 32g + 8w + 2i + h
// (i = 0..3, byte i); operand bytes 0..15 of all lanes come first, then
// bytes 16..31.
__host__ __device__ __forceinline__ int64_t fp8_tiled_dword(int64_t r, int64_t k0, int64_t K, int h) {
  const int64_t S = K >> 7, t = r >> 4, n = r & 15, s = k0 >> 7;
  const int g = (int)((k0 >> 5) & 3), w = (int)((k0 >> 3) & 3);
  return ((t * S + s) << 11) + ((w >> 1) << 10) + ((g * 16 + n) << 4) + (((w & 1) * 2 + h) << 2);
}

// Rows of storage (the tiled layout pads the last tile to 16 rows).
template <int LAYOUT>
__host__ __device__ __forceinline__ int64_t stored_rows(int64_t rows) {
  return LAYOUT == kLayoutRows ? rows : ((rows + 15) >> 4) << 4;
}

}  // namespace q4
