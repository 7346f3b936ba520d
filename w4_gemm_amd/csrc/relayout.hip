// relayout.hip -- a quantized weight moved between the row-major and the
// tiled layout (include/q4.h), bit for bit.
//
// Both layouts hold the same codes and scales; the tiled one only places
// them so that one 64-lane load is one contiguous kilobyte of matrix-core
// operand (a row's 32 codes of one 32-wide k group per lane).  The GEMM
// kernels are built for it: on row-major operands the generic kernels run
// 2.7x (W4A16) to 7x (W4A4) slower, so weights quantized row-major (or
// packed row-major elsewhere) are worth converting once, at load time.
//
// The conversion is a permutation:
//   * codes: 16-byte pieces.  Piece l of tiled block (t, s) is bytes
//     [64s + 16g, +16) of row 16t + n (l = 16g + n).  One thread per piece;
//     the tiled side is contiguous per wave, the row-major side 16 rows x
//     64 bytes.
//   * scales: per tile t, q group q (four super-chunks) and lane the tiled
//     layout keeps the lane's entries of the group together: MXFP4 4 bytes
//     (row-major bytes 16q + 4i + g of the row), NVFP4 8 bytes (32q + 8i +
//     2g + h), INT4 4 fp16 and INT4 with a zero point 4 words (4q + i, for
//     each of the 16 rows of the tile: contiguous on both sides).
//   * rows past the end of the last tile (tiled side only) hold the
//     quantization of zeros: codes 0, scales 0, except MXFP4 whose all-zero
//     block stores the E8M0 exponent of the 1e-12 floor.
// The NVFP4 global scale is copied by the first thread.
#include "q4_device.h"
#include "q4_launch.h"
#include "q4_layout.h"

namespace q4 {
namespace {

constexpr int kThreads = 256;

unsigned grid_of(int64_t items) {
  int64_t b = (items + kThreads - 1) / kThreads;
  if (b < 1) b = 1;
  if (b > (1 << 20)) b = 1 << 20;
  return (unsigned)b;
}

template <bool TO_TILED>
__global__ void __launch_bounds__(kThreads)
relayout_codes_kernel(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst, int64_t rows, int64_t cols) {
  const int64_t S = cols >> 7, RT = (rows + 15) >> 4;
  const int64_t total = RT * S * 64;
  for (int64_t p = (int64_t)blockIdx.x * kThreads + threadIdx.x; p < total; p += (int64_t)gridDim.x * kThreads) {
    const int64_t blk = p >> 6;                 // t * S + s
    const int l = (int)(p & 63), n = l & 15, g = l >> 4;
    const int64_t t = blk / S, s = blk - t * S;
    const int64_t r = t * 16 + n;
    const int64_t roff = r * (cols >> 1) + 64 * s + 16 * g;
    if constexpr (TO_TILED) {
      const uint4 v = r < rows ? *reinterpret_cast<const uint4*>(src + roff) : make_uint4(0u, 0u, 0u, 0u);
      *reinterpret_cast<uint4*>(dst + p * 16) = v;
    } else {
      if (r < rows) *reinterpret_cast<uint4*>(dst + roff) = *reinterpret_cast<const uint4*>(src + p * 16);
    }
  }
}

// FMT: 0 INT4 g128, 1 MXFP4, 2 NVFP4, 4 INT4 with a zero point.  One thread
// per (t, q, lane) for MXFP4 / NVFP4, per (t, q, row of the tile) for the
// INT4 formats.
template <int FMT, bool TO_TILED>
__global__ void __launch_bounds__(kThreads)
relayout_scales_kernel(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst, int64_t rows, int64_t cols,
                       const float* __restrict__ gs_src, float* __restrict__ gs_dst) {
  if (FMT == 2 && blockIdx.x == 0 && threadIdx.x == 0) *gs_dst = *gs_src;
  const int64_t Q = cols >> 9, RT = (rows + 15) >> 4;
  constexpr int kPerTQ = (FMT == 1 || FMT == 2) ? 64 : 16;  // units per (t, q)
  const int64_t total = RT * Q * kPerTQ;
  for (int64_t u = (int64_t)blockIdx.x * kThreads + threadIdx.x; u < total; u += (int64_t)gridDim.x * kThreads) {
    const int64_t tq = u / kPerTQ;
    const int64_t t = tq / Q, q = tq - t * Q;
    const int lu = (int)(u - tq * kPerTQ);
    const int n = lu & 15, g = lu >> 4;        // (g = 0 for the INT4 formats)
    const int64_t r = t * 16 + n;
    const bool live = r < rows;
    if constexpr (FMT == 1) {          // 4 E8M0 bytes: row-major 16q + 4i + g
      const int64_t rb = r * (cols >> 5) + 16 * q + g;
      if constexpr (TO_TILED) {
        uint32_t w;
        if (live) w = src[rb] | (src[rb + 4] << 8) | (src[rb + 8] << 16) | ((uint32_t)src[rb + 12] << 24);
        else w = mx_e8m0(0.0f) * 0x01010101u;
        *reinterpret_cast<uint32_t*>(dst + u * 4) = w;
      } else if (live) {
        const uint32_t w = *reinterpret_cast<const uint32_t*>(src + u * 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[rb + 4 * i] = (uint8_t)(w >> (8 * i));
      }
    } else if constexpr (FMT == 2) {   // 8 E4M3 bytes: row-major 32q + 8i + 2g + h
      const int64_t rb = r * (cols >> 4) + 32 * q + 2 * g;
      if constexpr (TO_TILED) {
        uint32_t w[2] = {0u, 0u};
        if (live) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t pr = src[rb + 8 * i] | ((uint32_t)src[rb + 8 * i + 1] << 8);
            w[i >> 1] |= pr << (16 * (i & 1));
          }
        }
        *reinterpret_cast<uint32_t*>(dst + u * 8) = w[0];
        *reinterpret_cast<uint32_t*>(dst + u * 8 + 4) = w[1];
      } else if (live) {
        const uint32_t w0 = *reinterpret_cast<const uint32_t*>(src + u * 8);
        const uint32_t w1 = *reinterpret_cast<const uint32_t*>(src + u * 8 + 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t pr = ((i >> 1) ? w1 : w0) >> (16 * (i & 1));
          dst[rb + 8 * i] = (uint8_t)pr;
          dst[rb + 8 * i + 1] = (uint8_t)(pr >> 8);
        }
      }
    } else {                           // INT4: 4 fp16 (8 bytes); with a zero point 4 words (16 bytes)
      constexpr int kWords = FMT == 0 ? 2 : 4;
      const uint32_t* rs = reinterpret_cast<const uint32_t*>(src);
      uint32_t* rd = reinterpret_cast<uint32_t*>(dst);
      const int64_t rw = (r * (cols >> 7) + 4 * q) * kWords / 4;  // the row's 4 entries, in words
      const int64_t tw = u * kWords;
#pragma unroll
      for (int i = 0; i < kWords; ++i) {
        if constexpr (TO_TILED) rd[tw + i] = live ? rs[rw + i] : 0u;
        else if (live) rd[rw + i] = rs[tw + i];
      }
    }
  }
}

template <int FMT, bool TO_TILED>
hipError_t run(const uint8_t* sc, const void* ss, const float* sg, uint8_t* dc, void* ds, float* dg, int64_t rows,
               int64_t cols, hipStream_t stream) {
  const int64_t RT = (rows + 15) >> 4, S = cols >> 7, Q = cols >> 9;
  relayout_codes_kernel<TO_TILED><<<grid_of(RT * S * 64), kThreads, 0, stream>>>(sc, dc, rows, cols);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t units = RT * Q * ((FMT == 1 || FMT == 2) ? 64 : 16);
  relayout_scales_kernel<FMT, TO_TILED><<<grid_of(units), kThreads, 0, stream>>>(
      static_cast<const uint8_t*>(ss), static_cast<uint8_t*>(ds), rows, cols, sg, dg);
  return hipGetLastError();
}

template <bool TO_TILED>
hipError_t by_fmt(int fmt, const uint8_t* sc, const void* ss, const float* sg, uint8_t* dc, void* ds, float* dg,
                  int64_t rows, int64_t cols, hipStream_t stream) {
  if (fmt == 0) return run<0, TO_TILED>(sc, ss, sg, dc, ds, dg, rows, cols, stream);
  if (fmt == 1) return run<1, TO_TILED>(sc, ss, sg, dc, ds, dg, rows, cols, stream);
  if (fmt == 2) return run<2, TO_TILED>(sc, ss, sg, dc, ds, dg, rows, cols, stream);
  return run<4, TO_TILED>(sc, ss, sg, dc, ds, dg, rows, cols, stream);
}

}  // namespace

hipError_t launch_relayout(int fmt, int to_layout, const uint8_t* src_codes, const void* src_scales,
                           const float* src_gs, uint8_t* dst_codes, void* dst_scales, float* dst_gs, int64_t rows,
                           int64_t cols, hipStream_t stream) {
  if (to_layout == kLayoutTiled)
    return by_fmt<true>(fmt, src_codes, src_scales, src_gs, dst_codes, dst_scales, dst_gs, rows, cols, stream);
  return by_fmt<false>(fmt, src_codes, src_scales, src_gs, dst_codes, dst_scales, dst_gs, rows, cols, stream);
}

}  // namespace q4
