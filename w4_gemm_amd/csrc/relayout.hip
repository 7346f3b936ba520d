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
//   * scales: per tile t, q group q (four super-chunks) and lane l = 16g + n
//     the tiled layout keeps the lane's entries of the group together: MXFP4
//     4 bytes (row-major bytes 16q + 4i + g of row 16t + n), NVFP4 8 bytes
//     (32q + 8i + 2g + h), INT4 4 fp16 and INT4 with a zero point 4 words
//     (4q + i, for each of the 16 rows of the tile: contiguous on both
//     sides).  When both scale pointers are 16-byte aligned one thread moves
//     a tile row's whole group (one contiguous row-side read or write, the
//     lanes' pieces transposed in registers): 39 us instead of 49 for the
//     MXFP4 28672 x 8192 weight, whose scale bytes were otherwise gathered
//     one at a time from rows 256 bytes apart.
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

// Scales, vector form (both scale pointers 16-byte aligned): one thread per
// (t, q, row n of the tile) moves the row's whole group -- MXFP4 16 bytes,
// NVFP4 32, INT4 8, INT4 with a zero point 16, contiguous on the row-major
// side -- and the four lanes' pieces (g = 0..3) on the tiled side, which
// for MXFP4 and NVFP4 is a 4 x 4 transpose of bytes or 16-bit halves done
// with byte permutes.  FMT: 0 INT4 g128, 1 MXFP4, 2 NVFP4, 4 INT4 with a
// zero point.
__device__ __forceinline__ uint32_t pick_byte(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3, int g) {
  // byte g of each word, in word order
  // selector bytes 0, 1 pick byte g of the low and the high word; 0x0C gives 0
  const uint32_t sel = 0x0C0C0400u + 0x0101u * (uint32_t)g;
  const uint32_t lo = __builtin_amdgcn_perm(w1, w0, sel);
  const uint32_t hi = __builtin_amdgcn_perm(w3, w2, sel);
  return lo | (hi << 16);
}

template <int FMT, bool TO_TILED>
__global__ void __launch_bounds__(kThreads)
relayout_scales_vec_kernel(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst, int64_t rows, int64_t cols,
                           const float* __restrict__ gs_src, float* __restrict__ gs_dst) {
  if (FMT == 2 && blockIdx.x == 0 && threadIdx.x == 0) *gs_dst = *gs_src;
  const int64_t Q = cols >> 9, RT = (rows + 15) >> 4;
  const int64_t total = RT * Q * 16;
  for (int64_t u = (int64_t)blockIdx.x * kThreads + threadIdx.x; u < total; u += (int64_t)gridDim.x * kThreads) {
    const int64_t tq = u >> 4;
    const int n = (int)(u & 15);
    const int64_t t = tq / Q, q = tq - t * Q;
    const int64_t r = t * 16 + n;
    const bool live = r < rows;
    if constexpr (FMT == 1) {          // row bytes 16q + 4i + g  <->  tiled dword (tq, 16g + n), byte i
      uint8_t* const rp = (TO_TILED ? const_cast<uint8_t*>(src) : dst) + r * (cols >> 5) + 16 * q;
      uint32_t* const tp = reinterpret_cast<uint32_t*>((TO_TILED ? dst : const_cast<uint8_t*>(src))) + tq * 64 + n;
      if constexpr (TO_TILED) {
        uint4 w = make_uint4(0u, 0u, 0u, 0u);
        if (live) w = *reinterpret_cast<const uint4*>(rp);
#pragma unroll
        for (int g = 0; g < 4; ++g)
          tp[16 * g] = live ? pick_byte(w.x, w.y, w.z, w.w, g) : mx_e8m0(0.0f) * 0x01010101u;
      } else if (live) {
        const uint32_t v0 = tp[0], v1 = tp[16], v2 = tp[32], v3 = tp[48];
        // row word i = byte i of each lane's dword, g = 0..3
        *reinterpret_cast<uint4*>(rp) = make_uint4(pick_byte(v0, v1, v2, v3, 0), pick_byte(v0, v1, v2, v3, 1),
                                                   pick_byte(v0, v1, v2, v3, 2), pick_byte(v0, v1, v2, v3, 3));
      }
    } else if constexpr (FMT == 2) {   // row halves 16q + 4i + g  <->  tiled (tq, 16g + n), half i
      uint8_t* const rp = (TO_TILED ? const_cast<uint8_t*>(src) : dst) + r * (cols >> 4) + 32 * q;
      uint2* const tp = reinterpret_cast<uint2*>((TO_TILED ? dst : const_cast<uint8_t*>(src))) + tq * 64 + n;
      // half h of word d: the low halves by 0x05040100, the high by 0x07060302
      if constexpr (TO_TILED) {
        uint4 a = make_uint4(0u, 0u, 0u, 0u), b = make_uint4(0u, 0u, 0u, 0u);
        if (live) {
          a = reinterpret_cast<const uint4*>(rp)[0];
          b = reinterpret_cast<const uint4*>(rp)[1];
        }
        // row word j holds halves 2j, 2j + 1; half 4i + g sits in word 2i + g/2
        const uint32_t d[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const uint32_t sel = (g & 1) ? 0x07060302u : 0x05040100u;
          tp[16 * g] = make_uint2(__builtin_amdgcn_perm(d[2 + g / 2], d[g / 2], sel),
                                  __builtin_amdgcn_perm(d[6 + g / 2], d[4 + g / 2], sel));
        }
      } else if (live) {
        uint32_t e[8];                  // e[2g + h/2]: lane g's halves 2(h/2), 2(h/2) + 1
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const uint2 v = tp[16 * g];
          e[2 * g] = v.x;
          e[2 * g + 1] = v.y;
        }
        // row word 2i + c = {half i of lane 2c, half i of lane 2c + 1}
        uint32_t o[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t sel = (i & 1) ? 0x07060302u : 0x05040100u;
#pragma unroll
          for (int c = 0; c < 2; ++c) o[2 * i + c] = __builtin_amdgcn_perm(e[2 * (2 * c + 1) + i / 2], e[2 * (2 * c) + i / 2], sel);
        }
        reinterpret_cast<uint4*>(rp)[0] = make_uint4(o[0], o[1], o[2], o[3]);
        reinterpret_cast<uint4*>(rp)[1] = make_uint4(o[4], o[5], o[6], o[7]);
      }
    } else if constexpr (FMT == 0) {   // 4 fp16 per (row, q): 8 bytes, same order on both sides
      const uint2* s2 = reinterpret_cast<const uint2*>(src);
      uint2* d2 = reinterpret_cast<uint2*>(dst);
      const int64_t ri = r * (cols >> 9) + q;       // the row's entry q, in 8-byte units
      if constexpr (TO_TILED) d2[u] = live ? s2[ri] : make_uint2(0u, 0u);
      else if (live) d2[ri] = s2[u];
    } else {                           // 4 words per (row, q): 16 bytes
      const uint4* s4 = reinterpret_cast<const uint4*>(src);
      uint4* d4 = reinterpret_cast<uint4*>(dst);
      const int64_t ri = r * (cols >> 9) + q;
      if constexpr (TO_TILED) d4[u] = live ? s4[ri] : make_uint4(0u, 0u, 0u, 0u);
      else if (live) d4[ri] = s4[u];
    }
  }
}

// Scales, byte form (any alignment): one thread per (t, q, lane) for MXFP4 /
// NVFP4, per (t, q, row of the tile) for the INT4 formats.
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
  if (((reinterpret_cast<uintptr_t>(ss) | reinterpret_cast<uintptr_t>(ds)) & 15) == 0) {
    relayout_scales_vec_kernel<FMT, TO_TILED><<<grid_of(RT * Q * 16), kThreads, 0, stream>>>(
        static_cast<const uint8_t*>(ss), static_cast<uint8_t*>(ds), rows, cols, sg, dg);
    return hipGetLastError();
  }
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
