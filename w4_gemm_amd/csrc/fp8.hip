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

// Element of a group of eight stored at byte i of the two output words:
// row-major keeps the order; the tiled layout puts the even elements in
// the first word and the odd ones in the second.
template <int LAYOUT>
__device__ __forceinline__ int fp8_slot(int i) {
  return LAYOUT == kLayoutRows ? i : (i & 3) * 2 + (i >> 2);
}

// Four E4M3 codes per word.  v_cvt_pk_fp8_f32 rounds to the nearest E4M3
// value with ties to the even code and keeps the sign (-0 -> 0x80); its
// inputs here are already clamped to +-448.
__device__ __forceinline__ uint2 fp8_cvt8(const float (&f)[8]) {
  uint32_t w0 = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
  w0 = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], w0, true);
  uint32_t w1 = __builtin_amdgcn_cvt_pk_fp8_f32(f[4], f[5], 0, false);
  w1 = __builtin_amdgcn_cvt_pk_fp8_f32(f[6], f[7], w1, true);
  return make_uint2(w0, w1);
}

// Codes of x[0..7] / s in the layout's byte order.  The quotient is
// bracketed by the products with the reciprocal nudged down and up by a
// relative 2^-20 (rl, rh; v_rcp_f32 is within 1 ulp and each product adds
// at most 1/2 ulp, far less than the nudge); the clamp to +-448 and the
// E4M3 rounding are monotone in the value, so where both ends give the
// same codes, so does the quotient.  Otherwise (a quotient within about
// 2^-20 of a rounding boundary, an exact tie) the values whose codes differ
// are divided, and for scales outside [2^-100, 2^100] all eight are.
template <int LAYOUT>
__device__ __forceinline__ uint2 fp8_pack8(const float (&x)[8], float s, float rl, float rh, bool fast) {
  if (fast) {
    float lo[8], hi[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float v = x[fp8_slot<LAYOUT>(i)];
      lo[i] = fminf(fmaxf(v * rl, -448.0f), 448.0f);
      hi[i] = fminf(fmaxf(v * rh, -448.0f), 448.0f);
    }
    const uint2 pl = fp8_cvt8(lo), ph = fp8_cvt8(hi);
    if (__builtin_expect(pl.x == ph.x && pl.y == ph.y, 1)) return pl;
    // only the values whose codes differ are divided, one per pass (exact
    // ties are common: s = amax / 448 has a short mantissa whenever amax's
    // has a factor 7)
    uint32_t w[2] = {pl.x, pl.y}, d[2] = {pl.x ^ ph.x, pl.y ^ ph.y};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      while (d[h] != 0u) {
        const int b = __builtin_ctz(d[h]) >> 3;
        const float v = pick8(x[fp8_slot<LAYOUT>(0)], x[fp8_slot<LAYOUT>(1)], x[fp8_slot<LAYOUT>(2)],
                              x[fp8_slot<LAYOUT>(3)], x[fp8_slot<LAYOUT>(4)], x[fp8_slot<LAYOUT>(5)],
                              x[fp8_slot<LAYOUT>(6)], x[fp8_slot<LAYOUT>(7)], 4 * h + b);
        const uint32_t m = 0xFFu << (8 * b);
        w[h] = (w[h] & ~m) | (fp8_code(v, s) << (8 * b));
        d[h] &= ~m;
      }
    }
    return make_uint2(w[0], w[1]);
  }
  uint32_t e[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) e[i] = fp8_code(x[fp8_slot<LAYOUT>(i)], s);
  return make_uint2(e[0] | (e[1] << 8) | (e[2] << 16) | (e[3] << 24),
                    e[4] | (e[5] << 8) | (e[6] << 16) | (e[7] << 24));
}

template <int LAYOUT>
__device__ __forceinline__ void fp8_store8(uint8_t* codes, int64_t r, int64_t k0, int64_t cols, uint2 w) {
  if constexpr (LAYOUT == kLayoutRows) {
    *reinterpret_cast<uint2*>(codes + r * cols + k0) = w;
  } else {
    *reinterpret_cast<uint32_t*>(codes + fp8_tiled_dword(r, k0, cols, 0)) = w.x;
    *reinterpret_cast<uint32_t*>(codes + fp8_tiled_dword(r, k0, cols, 1)) = w.y;
  }
}

__device__ __forceinline__ void unpack8(const uint4& v, float (&x)[8]) {
  x[0] = bf16_lo(v.x); x[1] = bf16_hi(v.x);
  x[2] = bf16_lo(v.y); x[3] = bf16_hi(v.y);
  x[4] = bf16_lo(v.z); x[5] = bf16_hi(v.z);
  x[6] = bf16_lo(v.w); x[7] = bf16_hi(v.w);
}

__device__ __forceinline__ float absmax_bf16x8(const uint4& v, float a) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) a = fmaxf(a, fmaxf(fabsf(bf16_lo(w[j])), fabsf(bf16_hi(w[j]))));
  return a;
}

// One wave per row, any length: the row is read twice (amax, then encode;
// the second read mostly hits the cache).
template <int LAYOUT>
__global__ void __launch_bounds__(64 * kRowsPerBlock)
fp8_rows_quantize_kernel(const uint16_t* __restrict__ src, int64_t ld, int64_t rows, int64_t cols,
                         int64_t srows, uint8_t* __restrict__ codes, float* __restrict__ scales) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (r >= srows) return;
  if (r >= rows) {  // padding row of the last tile: zero codes
    for (int64_t k0 = (int64_t)lane * 8; k0 < cols; k0 += 512) fp8_store8<LAYOUT>(codes, r, k0, cols, make_uint2(0, 0));
    return;
  }
  const uint16_t* row = src + r * ld;
  float amax = 0.0f;  // the row's largest magnitude (exact: max of bf16 values)
  for (int64_t k0 = (int64_t)lane * 8; k0 < cols; k0 += 512)
    amax = absmax_bf16x8(*reinterpret_cast<const uint4*>(row + k0), amax);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  const float s = fmaxf(amax, 1e-12f) / 448.0f;
  if (lane == 0) scales[r] = s;
  const bool fast = s >= 0x1p-100f && s <= 0x1p100f;
  const float rcp = __builtin_amdgcn_rcpf(s);
  const float rl = rcp * (1.0f - 0x1p-20f), rh = rcp * (1.0f + 0x1p-20f);
  float x[8];
  for (int64_t k0 = (int64_t)lane * 8; k0 < cols; k0 += 512) {
    unpack8(*reinterpret_cast<const uint4*>(row + k0), x);
    fp8_store8<LAYOUT>(codes, r, k0, cols, fp8_pack8<LAYOUT>(x, s, rl, rh, fast));
  }
}

// One workgroup of 256 threads per row of at most 256 * 8 * kWgChunks
// values: thread t holds chunks t, t + 256, ... (each 8 values, 16 bytes)
// in registers, every load issued before the first is used, so the row is
// read from HBM once; the row max is combined over the four waves in LDS.
constexpr int kWgChunks = 4;

template <int LAYOUT>
__global__ void __launch_bounds__(256)
fp8_rows_quantize_wg_kernel(const uint16_t* __restrict__ src, int64_t ld, int64_t rows, int64_t cols,
                            uint8_t* __restrict__ codes, float* __restrict__ scales) {
  const int tid = threadIdx.x;
  const int64_t r = blockIdx.x;
  if (r >= rows) {  // padding row of the last tile: zero codes
    for (int64_t k0 = (int64_t)tid * 8; k0 < cols; k0 += 2048) fp8_store8<LAYOUT>(codes, r, k0, cols, make_uint2(0, 0));
    return;
  }
  const uint16_t* row = src + r * ld;
  // every load unconditional, so that all are in flight together: a chunk
  // past the row's end re-reads the row's first one (cols >= 16), which
  // leaves the max unchanged and is never encoded
  uint4 v[kWgChunks];
#pragma unroll
  for (int i = 0; i < kWgChunks; ++i) {
    const int64_t k0 = (int64_t)(tid + 256 * i) * 8;
    v[i] = *reinterpret_cast<const uint4*>(row + (k0 < cols ? k0 : 0));
  }
  __builtin_amdgcn_sched_barrier(0);  // all loads issued before the first use
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < kWgChunks; ++i) amax = absmax_bf16x8(v[i], amax);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  __shared__ float part[4];
  if ((tid & 63) == 0) part[tid >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(part[0], part[1]), fmaxf(part[2], part[3]));
  const float s = fmaxf(amax, 1e-12f) / 448.0f;
  if (tid == 0) scales[r] = s;
  const bool fast = s >= 0x1p-100f && s <= 0x1p100f;
  const float rcp = __builtin_amdgcn_rcpf(s);
  const float rl = rcp * (1.0f - 0x1p-20f), rh = rcp * (1.0f + 0x1p-20f);
  float x[8];
#pragma unroll
  for (int i = 0; i < kWgChunks; ++i) {
    const int64_t k0 = (int64_t)(tid + 256 * i) * 8;
    if (k0 < cols) {
      unpack8(v[i], x);
      fp8_store8<LAYOUT>(codes, r, k0, cols, fp8_pack8<LAYOUT>(x, s, rl, rh, fast));
    }
  }
}

// The same for rows of at most 8192 values with cols % 32 == 0, each thread
// taking 32 consecutive values (one 32-wide group of the tiled layout): its
// codes are two whole 16-byte operand pieces (tiled) or 32 contiguous bytes
// (row-major), written by two 16-byte stores instead of eight 4-byte ones.
// In the tiled layout the 16 rows of a tile share every 128-byte line of
// its codes (8 rows each), so the rows go to workgroups of one XCD: with
// 128 | srows, workgroup b (on XCD b % 8 in dispatch order) takes row
// (b % 8) * srows/8 + b / 8, and each XCD's L2 sees whole lines written
// instead of 16-byte pieces of lines shared with the other XCDs.
template <int LAYOUT>
__global__ void __launch_bounds__(256)
fp8_rows_quantize_wg32_kernel(const uint16_t* __restrict__ src, int64_t ld, int64_t rows, int64_t cols,
                              uint8_t* __restrict__ codes, float* __restrict__ scales) {
  const int tid = threadIdx.x;
  const int64_t srows = gridDim.x;
  const int64_t r = (LAYOUT == kLayoutTiled && srows % 128 == 0)
                        ? (int64_t)(blockIdx.x % 8) * (srows / 8) + blockIdx.x / 8
                        : (int64_t)blockIdx.x;
  const int64_t k0 = (int64_t)tid * 32;
  const bool live = k0 < cols;
  auto store32 = [&](const uint2 (&w)[4]) {
    if constexpr (LAYOUT == kLayoutRows) {
      uint4* d = reinterpret_cast<uint4*>(codes + r * cols + k0);
      d[0] = make_uint4(w[0].x, w[0].y, w[1].x, w[1].y);
      d[1] = make_uint4(w[2].x, w[2].y, w[3].x, w[3].y);
    } else {
      // chunks 0, 1 fill the group's piece in the first operand half, 2, 3
      // the one in the second
      *reinterpret_cast<uint4*>(codes + fp8_tiled_dword(r, k0, cols, 0)) = make_uint4(w[0].x, w[0].y, w[1].x, w[1].y);
      *reinterpret_cast<uint4*>(codes + fp8_tiled_dword(r, k0 + 16, cols, 0)) = make_uint4(w[2].x, w[2].y, w[3].x, w[3].y);
    }
  };
  if (r >= rows) {  // padding row of the last tile: zero codes
    if (live) {
      const uint2 z[4] = {make_uint2(0, 0), make_uint2(0, 0), make_uint2(0, 0), make_uint2(0, 0)};
      store32(z);
    }
    return;
  }
  const uint16_t* row = src + r * ld;
  // every load unconditional (a thread past the row's end re-reads its first
  // 32 values, which leave the max unchanged and are never encoded)
  uint4 v[4];
  const uint16_t* p = row + (live ? k0 : 0);
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = reinterpret_cast<const uint4*>(p)[i];
  __builtin_amdgcn_sched_barrier(0);  // all loads issued before the first use
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) amax = absmax_bf16x8(v[i], amax);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  __shared__ float part[4];
  if ((tid & 63) == 0) part[tid >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(part[0], part[1]), fmaxf(part[2], part[3]));
  const float s = fmaxf(amax, 1e-12f) / 448.0f;
  if (tid == 0) scales[r] = s;
  if (!live) return;
  const bool fast = s >= 0x1p-100f && s <= 0x1p100f;
  const float rcp = __builtin_amdgcn_rcpf(s);
  const float rl = rcp * (1.0f - 0x1p-20f), rh = rcp * (1.0f + 0x1p-20f);
  float x[8];
  uint2 w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    unpack8(v[i], x);
    w[i] = fp8_pack8<LAYOUT>(x, s, rl, rh, fast);
  }
  store32(w);
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
  if (cols <= 256 * 32 && cols % 32 == 0) {  // a workgroup per row, 32 values per thread
    if (layout == kLayoutTiled)
      fp8_rows_quantize_wg32_kernel<kLayoutTiled><<<(unsigned)srows, 256, 0, stream>>>(src, ld, rows, cols, codes, scales);
    else
      fp8_rows_quantize_wg32_kernel<kLayoutRows><<<(unsigned)srows, 256, 0, stream>>>(src, ld, rows, cols, codes, scales);
  } else if (cols <= 2048 * kWgChunks) {  // a workgroup per row, the row in registers
    if (layout == kLayoutTiled)
      fp8_rows_quantize_wg_kernel<kLayoutTiled><<<(unsigned)srows, 256, 0, stream>>>(src, ld, rows, cols, codes, scales);
    else
      fp8_rows_quantize_wg_kernel<kLayoutRows><<<(unsigned)srows, 256, 0, stream>>>(src, ld, rows, cols, codes, scales);
  } else {  // a wave per row, two passes
    const unsigned grid = (unsigned)((srows + kRowsPerBlock - 1) / kRowsPerBlock);
    if (layout == kLayoutTiled)
      fp8_rows_quantize_kernel<kLayoutTiled><<<grid, 64 * kRowsPerBlock, 0, stream>>>(src, ld, rows, cols, srows,
                                                                                    codes, scales);
    else
      fp8_rows_quantize_kernel<kLayoutRows><<<grid, 64 * kRowsPerBlock, 0, stream>>>(src, ld, rows, cols, srows,
                                                                                   codes, scales);
  }
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
