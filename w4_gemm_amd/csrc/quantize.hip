// quantize.hip -- round-to-nearest absmax block quantization of bf16 rows
// into INT4 g128, MXFP4 and NVFP4, and the matching dequantization.
//
// Method ("LLM quantization", how quantization works step by step: a
// group's largest magnitude sets the scale, each value is divided by the
// scale and rounded; block scaling gives each small group its own scale):
//   INT4 g128  s = fp16(amax/7); code = clamp(rne(w/s), -8, 7)
//              ("Low-bit inference for very large MoE", fake_int4)
//   MXFP4      s = 2^(floor(log2(max(amax,1e-12))) - 2), E8M0 byte;
//              code = E2M1(clamp(w/s, +-6))  ("Quantization in deployment",
//              formats.py mxfp4 and fp4)
//   NVFP4      gs = max(amax_tensor,1e-12)/2688; block code
//              E4M3(min((amax_b/6)/gs, 448)); code = E2M1(clamp(w/(E4M3*gs)))
//              (same file, nvfp4)
//   INT4 + zero point, g128 (format cheat sheet, W4A16 INT4 GPTQ/AWQ row:
//              integers -8..7, one scale per 128, plus a zero point; min-max
//              rounding): lo = min(min, 0), hi = max(max, 0),
//              s = fp16((hi - lo)/15), z = clamp(-8 - rne(lo/s), -8, 7),
//              code = clamp(rne(w/s) + z, -8, 7); word = fp16 s | z << 16
//
// Launch shape: one lane per 8 consecutive values of a row (one 16-byte
// load, one 4-byte store of packed nibbles at the position the layout
// gives).  A block of g values is g/8 adjacent lanes (16 for INT4, 4 for
// MXFP4, 2 for NVFP4); its absmax is a butterfly max over those lanes.
// Every lane of a wave runs the same number of iterations so the cross-lane
// steps see the whole group.  In the tiled layout the padding rows of the
// last tile are quantized as zeros.
#include "q4_device.h"
#include "q4_encode.h"
#include "q4_launch.h"
#include "q4_layout.h"

#include <string.h>

#pragma clang fp contract(off)

namespace q4 {
namespace {

typedef uint32_t nt_u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store16_nt(void* p, uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  __builtin_nontemporal_store(nt_u32x4{a, b, c, d}, reinterpret_cast<nt_u32x4*>(p));
}

constexpr int kThreads = 256;

// INT4 codes, clamp(rne(w / s), -8, 7) or, with a zero point z in [-8, 7],
// clamp(rne(w / s) + z, -8, 7), need no division.  A bf16 value (8
// significant bits) over an fp16 scale (11) is either exactly a
// half-integer or at least 2^-12 away from every half-integer: written
// over a common power of two, a nonzero difference is at least 1/(2b) for
// the scale's integer significand b < 2^11, or, for quotients of magnitude
// 1/2 and up, 1/(2a) for the value's significand a < 2^8.  The product
// y = w (1/s), with v_rcp_f32 (within 1 ulp), is within 2^-18 of the
// quotient wherever |w/s| <= 16.5.  So after clamping y (to [-8, 7], or
// [-16, 16] with a zero point; the bounds are integers, and NaN goes to
// the lower one as fmax drops it), adding 768 rounds it to a multiple of
// 2^-14: exactly the half-integer in the first case, still on the
// quotient's side of it in the second.  Adding 1.5 2^23 - 768 then rounds
// to an integer with ties to even, as rne does to the exact quotient, and
// leaves that integer in the low bits of the sum.  (Checked exhaustively
// for every finite bf16 value and every positive finite fp16 scale, with
// the correctly rounded reciprocal and both its neighbours.)  A scale that
// overflowed fp16 (+inf) is divided by.
template <bool ZP>
__device__ __forceinline__ uint32_t int4_code(float y, int z) {
  const float c = ZP ? fminf(fmaxf(y, -16.0f), 16.0f) : fminf(fmaxf(y, -8.0f), 7.0f);
  const int q = (int)(f2u((c + 768.0f) + 12582144.0f) - 0x4B400000u);
  if constexpr (ZP) return (uint32_t)min(max(q + z, -8), 7) & 0xFu;
  else return (uint32_t)q & 0xFu;
}

// Eight INT4 nibbles (element j in bits 4j..4j+3) of x[j] / s, 0 < s.
template <bool ZP>
__device__ __forceinline__ uint32_t int4_pack8(const Chunk8& x, float s, int z) {
  uint32_t p = 0;
  if (s <= 65504.0f) {
    const float r = __builtin_amdgcn_rcpf(s);
#pragma unroll
    for (int j = 0; j < 8; ++j) p |= int4_code<ZP>(x.v[j] * r, z) << (4 * j);
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) p |= int4_code<ZP>(x.v[j] / s, z) << (4 * j);
  }
  return p;
}

template <int LANES>
__device__ __forceinline__ float group_max(float a) {
#pragma unroll
  for (int m = 1; m < LANES; m <<= 1) a = fmaxf(a, __shfl_xor(a, m));
  return a;
}

template <int LANES>
__device__ __forceinline__ float group_min(float a) {
#pragma unroll
  for (int m = 1; m < LANES; m <<= 1) a = fminf(a, __shfl_xor(a, m));
  return a;
}

__device__ __forceinline__ float min8(const Chunk8& c) {
  float a = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) a = fminf(a, c.v[j]);
  return a;
}

__device__ __forceinline__ float max8(const Chunk8& c) {
  float a = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) a = fmaxf(a, c.v[j]);
  return a;
}

// INT4 with a zero point: the group's scale word and (s, z) from its range
// [lo, hi] (already widened to include 0).
struct ZpParams {
  uint32_t word;
  float s, z;
};
__device__ __forceinline__ ZpParams int4zp_params(float lo, float hi) {
  const uint32_t sbits = fp16_encode((hi - lo) / 15.0f);
  const float s = fp16_value(sbits);
  if (s == 0.0f) return ZpParams{0u, 0.0f, 0.0f};
  const float z = fminf(fmaxf(-8.0f - __builtin_rintf(lo / s), -8.0f), 7.0f);
  return ZpParams{sbits | (((uint32_t)(int)z & 0xFFu) << 16), s, z};
}

// Eight values -> eight INT4 nibbles with the zero point (codes 0 if s == 0).
__device__ __forceinline__ uint32_t int4zp_pack8(const Chunk8& c, const ZpParams& zp) {
  return zp.s != 0.0f ? int4_pack8<true>(c, zp.s, (int)zp.z) : 0u;
}

// FMT: 0 INT4 g128, 1 MXFP4, 2 NVFP4.  For NVFP4, gs_src holds the global
// scale, and gs_out, when not null, receives a copy of it from the first
// lane.
template <int FMT, int LAYOUT>
__global__ void __launch_bounds__(kThreads)
quantize_kernel(const uint16_t* __restrict__ src, int64_t ld, int64_t rows, int64_t cols,
                uint8_t* __restrict__ codes, void* __restrict__ scales,
                const float* gs_src, float* gs_out) {
  constexpr int G = FmtTraits<FMT>::G;
  constexpr int LANES = G / 8;
  const int64_t cpr = cols >> 3;  // chunks of 8 per row
  const int64_t total = stored_rows<LAYOUT>(rows) * cpr;

  float gs = 0.0f;
  if constexpr (FMT == 2) {
    gs = *gs_src;
    if (blockIdx.x == 0 && threadIdx.x == 0 && gs_out) *gs_out = gs;
  }
  const float rgs = FMT == 2 ? 1.0f / gs : 0.0f;
  const bool gs_ok = FMT == 2 && in_bracket_range(gs);

  for (int64_t base = (int64_t)blockIdx.x * kThreads; base < total;
       base += (int64_t)gridDim.x * kThreads) {
    const int64_t c = base + threadIdx.x;
    const bool valid = c < total;
    const int64_t r = valid ? c / cpr : 0;
    const int64_t k0 = valid ? (c - r * cpr) * 8 : 0;
    const bool in_src = valid && r < rows;  // tiled padding rows read as zeros
    Chunk8 x = load8(src + (in_src ? r * ld + k0 : 0), in_src);
    const float amax = FMT == 4 ? 0.0f : group_max<LANES>(absmax8(x));

    uint32_t packed = 0;
    if constexpr (FMT == 0) {
      const uint32_t sbits = fp16_encode(amax / 7.0f);
      const float s = fp16_value(sbits);
      packed = s != 0.0f ? int4_pack8<false>(x, s, 0) : 0u;
      if (valid && (k0 % G) == 0)
        reinterpret_cast<uint16_t*>(scales)[scale_off<FMT, LAYOUT>(r, k0, cols)] = (uint16_t)sbits;
    } else if constexpr (FMT == 4) {
      const ZpParams zp = int4zp_params(group_min<LANES>(min8(x)), group_max<LANES>(max8(x)));
      packed = int4zp_pack8(x, zp);
      if (valid && (k0 % G) == 0)
        reinterpret_cast<uint32_t*>(scales)[scale_off<FMT, LAYOUT>(r, k0, cols)] = zp.word;
    } else if constexpr (FMT == 1) {
      const uint32_t e = mx_e8m0(amax);
      packed = e2m1_pack8(x, e8m0_value(e));
      if (valid && (k0 % G) == 0)
        reinterpret_cast<uint8_t*>(scales)[scale_off<FMT, LAYOUT>(r, k0, cols)] = (uint8_t)e;
    } else {
      const uint32_t sc = nv_scale_code(amax, gs, rgs, gs_ok);
      const float eff = e4m3_value(sc) * gs;
      if (eff == 0.0f) {  // E4M3 scale underflowed to 0: magnitude codes 0, signs kept
#pragma unroll
        for (int j = 0; j < 8; ++j) packed |= ((f2u(x.v[j]) >> 31) << 3) << (4 * j);
      } else {
        packed = e2m1_pack8_div(x, eff);
      }
      if (valid && (k0 % G) == 0)
        reinterpret_cast<uint8_t*>(scales)[scale_off<FMT, LAYOUT>(r, k0, cols)] = (uint8_t)sc;
    }
    if (valid) *reinterpret_cast<uint32_t*>(codes + code_off8<LAYOUT>(r, k0, cols)) = packed;
  }
}

// Block-mapped quantizer for cols % 128 == 0 (every tiled tensor): a
// workgroup of 4 waves takes 16 rows x 512 k.  The rows are first staged in
// LDS with fully coalesced loads (each wave instruction reads 1 KB of one
// row); then lane l = 16g + n of wave s takes row n, k = 128s + 32g .. +32 --
// one MXFP4 block, two NVFP4 blocks, a quarter INT4 group (completed by a
// max over the 4 lanes of the row) -- and writes its 16 code bytes with one
// store.  In the tiled layout those 64 stores are exactly tile s: one
// contiguous kilobyte per wave.  Rows past the end are staged as zeros (the
// tiled padding rows) and not stored in the row-major layout.
template <int FMT, int LAYOUT>
__global__ void __launch_bounds__(kThreads)
quantize_block_kernel(const uint16_t* __restrict__ src, int64_t ld, int64_t rows, int64_t cols,
                      uint8_t* __restrict__ codes, void* __restrict__ scales,
                      const float* gs_src, float* gs_out, int reverse) {
  __shared__ __attribute__((aligned(16))) uint16_t xs[16][512 + 8];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t KB = (cols + 511) >> 9;
  const int64_t b0 = blockIdx.x / KB, kb = blockIdx.x - b0 * KB;
  const int64_t band = reverse ? (int64_t)gridDim.x / KB - 1 - b0 : b0;
  const int64_t r0 = band * 16, k0 = kb * 512;

  float gs = 0.0f;
  if constexpr (FMT == 2) {
    gs = *gs_src;
    if (blockIdx.x == 0 && threadIdx.x == 0 && gs_out) *gs_out = gs;
  }
  const float rgs = FMT == 2 ? 1.0f / gs : 0.0f;
  const bool gs_ok = FMT == 2 && in_bracket_range(gs);

#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = 4 * j + wave;
    const int64_t k = k0 + 8 * lane;
    const bool ok = r0 + row < rows && k < cols;
    const uint4 v = ok ? *reinterpret_cast<const uint4*>(src + (r0 + row) * ld + k) : make_uint4(0, 0, 0, 0);
    *reinterpret_cast<uint4*>(&xs[row][8 * lane]) = v;
  }
  __syncthreads();
  const int64_t S = cols >> 7;
  const int64_t s = kb * 4 + wave;  // super-chunk of this wave
  if (s >= S) return;               // (row-major, cols % 512 != 0); no barrier follows
  const int n = lane & 15, g = lane >> 4;
  const int64_t r = r0 + n;
  Chunk8 x[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 raw = *reinterpret_cast<const uint4*>(&xs[n][128 * wave + 32 * g + 8 * i]);
    x[i].v[0] = bf16_lo(raw.x); x[i].v[1] = bf16_hi(raw.x);
    x[i].v[2] = bf16_lo(raw.y); x[i].v[3] = bf16_hi(raw.y);
    x[i].v[4] = bf16_lo(raw.z); x[i].v[5] = bf16_hi(raw.z);
    x[i].v[6] = bf16_lo(raw.w); x[i].v[7] = bf16_hi(raw.w);
  }
  const bool store = LAYOUT == kLayoutTiled || r < rows;
  const int64_t Q = cols >> 9;
  const int64_t q = s >> 2, si = s & 3;
  uint32_t packed[4];
  if constexpr (FMT == 0) {
    float amax = fmaxf(fmaxf(absmax8(x[0]), absmax8(x[1])), fmaxf(absmax8(x[2]), absmax8(x[3])));
    amax = fmaxf(amax, __shfl_xor(amax, 16));
    amax = fmaxf(amax, __shfl_xor(amax, 32));
    const uint32_t sbits = fp16_encode(amax / 7.0f);
    const float sc = fp16_value(sbits);
#pragma unroll
    for (int i = 0; i < 4; ++i) packed[i] = sc != 0.0f ? int4_pack8<false>(x[i], sc, 0) : 0u;
    if (store && g == 0) {
      uint16_t* sp = reinterpret_cast<uint16_t*>(scales);
      if constexpr (LAYOUT == kLayoutTiled) sp[((band * Q + q) * 16 + n) * 4 + si] = (uint16_t)sbits;
      else sp[r * S + s] = (uint16_t)sbits;
    }
  } else if constexpr (FMT == 4) {
    float lo = fminf(fminf(min8(x[0]), min8(x[1])), fminf(min8(x[2]), min8(x[3])));
    float hi = fmaxf(fmaxf(max8(x[0]), max8(x[1])), fmaxf(max8(x[2]), max8(x[3])));
    lo = fminf(lo, __shfl_xor(lo, 16));
    lo = fminf(lo, __shfl_xor(lo, 32));
    hi = fmaxf(hi, __shfl_xor(hi, 16));
    hi = fmaxf(hi, __shfl_xor(hi, 32));
    const ZpParams zp = int4zp_params(lo, hi);
#pragma unroll
    for (int i = 0; i < 4; ++i) packed[i] = int4zp_pack8(x[i], zp);
    if (store && g == 0) {
      uint32_t* sp = reinterpret_cast<uint32_t*>(scales);
      if constexpr (LAYOUT == kLayoutTiled) sp[((band * Q + q) * 16 + n) * 4 + si] = zp.word;
      else sp[r * S + s] = zp.word;
    }
  } else if constexpr (FMT == 1) {
    const float amax = fmaxf(fmaxf(absmax8(x[0]), absmax8(x[1])), fmaxf(absmax8(x[2]), absmax8(x[3])));
    const uint32_t e = mx_e8m0(amax);
    const float sc = e8m0_value(e);
#pragma unroll
    for (int i = 0; i < 4; ++i) packed[i] = e2m1_pack8(x[i], sc);
    if (store) {
      uint8_t* sp = reinterpret_cast<uint8_t*>(scales);
      if constexpr (LAYOUT == kLayoutTiled) sp[((band * Q + q) * 64 + lane) * 4 + si] = (uint8_t)e;
      else sp[r * (cols >> 5) + 4 * s + g] = (uint8_t)e;
    }
  } else {
    uint32_t sc2[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float amax = fmaxf(absmax8(x[2 * h]), absmax8(x[2 * h + 1]));
      const uint32_t sc = nv_scale_code(amax, gs, rgs, gs_ok);
      const float eff = e4m3_value(sc) * gs;
      sc2[h] = sc;
#pragma unroll
      for (int i = 2 * h; i < 2 * h + 2; ++i) {
        if (eff == 0.0f) {  // E4M3 scale underflowed to 0: magnitude codes 0, signs kept
          uint32_t p = 0;
#pragma unroll
          for (int j = 0; j < 8; ++j) p |= ((f2u(x[i].v[j]) >> 31) << 3) << (4 * j);
          packed[i] = p;
        } else {
          packed[i] = e2m1_pack8_div(x[i], eff);
        }
      }
    }
    if (store) {
      uint16_t* sp = reinterpret_cast<uint16_t*>(scales);  // the lane's two E4M3 bytes, first block low
      const uint16_t pair = (uint16_t)(sc2[0] | (sc2[1] << 8));
      if constexpr (LAYOUT == kLayoutTiled) sp[((band * Q + q) * 64 + lane) * 4 + si] = pair;
      else sp[(r * (cols >> 4) + 8 * s + 2 * g) >> 1] = pair;
    }
  }
  if (store) {
    uint8_t* dst = LAYOUT == kLayoutTiled ? codes + ((band * S + s) << 10) + lane * 16
                                          : codes + r * (cols >> 1) + 64 * s + 16 * g;
    store16_nt(dst, packed[0], packed[1], packed[2], packed[3]);
  }
}

// NVFP4 global scale gs = max(amax, 1e-12) / 2688 of the tensor absmax
// over rows x cols.  gs is monotone in amax, so the max over workgroups of
// each one's gs is the gs of the tensor's amax: each workgroup folds its gs
// into *gs_bits (set beforehand to the gs of amax 0) with an atomic max on
// the fp32 bits (non-negative floats order like their bit patterns, and max
// is exact, so the result does not depend on order).
__global__ void __launch_bounds__(kThreads)
absmax_kernel(const uint16_t* __restrict__ src, int64_t ld, int64_t rows, int64_t cols,
              uint32_t* gs_bits) {
  // rows over workgroups, a row's 16-byte chunks over the threads (no
  // division per element)
  const int cpr = (int)(cols >> 3);
  float a = 0.0f;
  // two rows at a time, their eight loads per thread in flight together
  // (a weight too large for the last-level cache streams from HBM: 28672 x
  // 8192 measured 4% faster than one row at a time), then the remaining row
  int64_t r = blockIdx.x;
  for (; r + (int64_t)gridDim.x < rows; r += 2 * (int64_t)gridDim.x) {
    const uint16_t* rw[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) rw[q] = src + (r + q * (int64_t)gridDim.x) * ld;
    int c = threadIdx.x;
    for (; c + 3 * kThreads < cpr; c += 4 * kThreads) {
      Chunk8 x[2][4];
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int u = 0; u < 4; ++u) x[q][u] = load8(rw[q] + (int64_t)(c + u * kThreads) * 8, true);
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int u = 0; u < 4; ++u) a = fmaxf(a, absmax8(x[q][u]));
    }
    for (; c < cpr; c += kThreads)
#pragma unroll
      for (int q = 0; q < 2; ++q) a = fmaxf(a, absmax8(load8(rw[q] + (int64_t)c * 8, true)));
  }
  for (; r < rows; r += gridDim.x) {
    const uint16_t* row = src + r * ld;
    int c = threadIdx.x;
    for (; c + 3 * kThreads < cpr; c += 4 * kThreads) {
      Chunk8 x[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) x[u] = load8(row + (int64_t)(c + u * kThreads) * 8, true);
#pragma unroll
      for (int u = 0; u < 4; ++u) a = fmaxf(a, absmax8(x[u]));
    }
    for (; c < cpr; c += kThreads) a = fmaxf(a, absmax8(load8(row + (int64_t)c * 8, true)));
  }
  a = group_max<64>(a);
  __shared__ float part[kThreads / 64];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = a;
  __syncthreads();
  if (threadIdx.x == 0) {
    float m = part[0];
#pragma unroll
    for (int i = 1; i < kThreads / 64; ++i) m = fmaxf(m, part[i]);
    atomicMax(gs_bits, f2u(fmaxf(m, 1e-12f) / 2688.0f));
  }
}

__global__ void set_word_kernel(uint32_t* p, uint32_t v) { *p = v; }

// Dequantize the 8 values at (r, k0); OUT 0 = bf16, 1 = fp32.  Every value
// is fp32(code * scale as stored), then (bf16 output) rounded to nearest
// even.  MXFP4 blocks whose E8M0 scale keeps every value in the normal fp32
// range (bytes 2..252) are converted by v_cvt_scalef32_pk_{bf16,f32}_fp4,
// which multiplies the E2M1 value by the power of two exactly -- the same
// bits; other blocks take the plain path.  NVFP4 reads its E2M1 values
// through the same instruction with scale 1 (exact) before the multiply.
// Split in two so that a lane can issue the loads of several chunks before
// it converts the first: dq_load fetches the 8 codes and the raw scale
// field, dq_store converts and writes them.
// Outputs are written with non-temporal stores: dequantized values (470 MB
// of bf16 for the 28672 x 8192 weight: 107 -> 91 us in both layouts) and
// the quantizer's codes (MXFP4 tiled 106 -> 104 us, NVFP4 192 -> 183) are
// not read back by the kernel and would only evict other lines from L2.
struct DqIn {
  uint32_t packed;  // 8 codes, element j in nibble j
  uint32_t sraw;    // the scale field as stored (fp16 bits, E8M0, E4M3, or the INT4-zp word)
};

template <int FMT, int LAYOUT>
__device__ __forceinline__ DqIn dq_load(const uint8_t* __restrict__ codes, const void* __restrict__ scales,
                                        int64_t r, int64_t k0, int64_t cols) {
  DqIn d;
  d.packed = *reinterpret_cast<const uint32_t*>(codes + code_off8<LAYOUT>(r, k0, cols));
  const int64_t si = scale_off<FMT, LAYOUT>(r, k0, cols);
  if constexpr (FMT == 0) d.sraw = reinterpret_cast<const uint16_t*>(scales)[si];
  else if constexpr (FMT == 4) d.sraw = reinterpret_cast<const uint32_t*>(scales)[si];
  else d.sraw = reinterpret_cast<const uint8_t*>(scales)[si];
  return d;
}

template <int FMT, int OUT>
__device__ __forceinline__ void dq_store(DqIn d, float gs, int64_t r, int64_t k0, void* __restrict__ dst,
                                         int64_t ld) {
  const uint32_t packed = d.packed;
  float v[8];
  if constexpr (FMT == 0) {
    const float s = fp16_value(d.sraw);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int q = ((int)(packed << (28 - 4 * j))) >> 28;  // sign-extend nibble j
      v[j] = (float)q * s;
    }
  } else if constexpr (FMT == 4) {
    const float s = fp16_value(d.sraw & 0xFFFFu);
    const int z = (int)(int8_t)((d.sraw >> 16) & 0xFFu);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int q = ((int)(packed << (28 - 4 * j))) >> 28;
      v[j] = (float)(q - z) * s;
    }
  } else if constexpr (FMT == 1) {
    const uint32_t e = d.sraw;
    const float s = e8m0_value(e);
    if (e >= 2u && e <= 252u) {
      if constexpr (OUT == 0) {
        uint4 o;
        o.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(packed, s, 0));
        o.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(packed, s, 1));
        o.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(packed, s, 2));
        o.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(packed, s, 3));
        store16_nt(reinterpret_cast<uint16_t*>(dst) + r * ld + k0, o.x, o.y, o.z, o.w);
      } else {
        const auto p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(packed, s, 0);
        const auto p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(packed, s, 1);
        const auto p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(packed, s, 2);
        const auto p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(packed, s, 3);
        float* o = reinterpret_cast<float*>(dst) + r * ld + k0;
        store16_nt(o, f2u(p0[0]), f2u(p0[1]), f2u(p1[0]), f2u(p1[1]));
        store16_nt(o + 4, f2u(p2[0]), f2u(p2[1]), f2u(p3[0]), f2u(p3[1]));
      }
      return;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = e2m1_value((packed >> (4 * j)) & 0xFu) * s;
  } else {
    const float eff = e4m3_value(d.sraw) * gs;
    const auto p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(packed, 1.0f, 0);
    const auto p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(packed, 1.0f, 1);
    const auto p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(packed, 1.0f, 2);
    const auto p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(packed, 1.0f, 3);
    v[0] = p0[0] * eff; v[1] = p0[1] * eff; v[2] = p1[0] * eff; v[3] = p1[1] * eff;
    v[4] = p2[0] * eff; v[5] = p2[1] * eff; v[6] = p3[0] * eff; v[7] = p3[1] * eff;
  }
  if constexpr (OUT == 0) {
    uint4 o;
    o.x = f32_to_bf16_rne(v[0]) | (f32_to_bf16_rne(v[1]) << 16);
    o.y = f32_to_bf16_rne(v[2]) | (f32_to_bf16_rne(v[3]) << 16);
    o.z = f32_to_bf16_rne(v[4]) | (f32_to_bf16_rne(v[5]) << 16);
    o.w = f32_to_bf16_rne(v[6]) | (f32_to_bf16_rne(v[7]) << 16);
    store16_nt(reinterpret_cast<uint16_t*>(dst) + r * ld + k0, o.x, o.y, o.z, o.w);
  } else {
    float* o = reinterpret_cast<float*>(dst) + r * ld + k0;
    store16_nt(o, f2u(v[0]), f2u(v[1]), f2u(v[2]), f2u(v[3]));
    store16_nt(o + 4, f2u(v[4]), f2u(v[5]), f2u(v[6]), f2u(v[7]));
  }
}

// Dequantization walks the flattened chunks of 8 values.  Each lane takes
// kDqUnroll chunks a grid-stride apart (so that each wave instruction still
// covers consecutive chunks: 1 KB of bf16 per store) and issues all their
// loads before converting the first: decode is bound by the latency of
// those small loads otherwise.  IDX32: the chunk count fits 32 bits, so
// the row comes from a 32-bit division.
constexpr int kDqUnroll = 4;

template <int FMT, int OUT, int LAYOUT, bool IDX32>
__global__ void __launch_bounds__(kThreads)
dequant_kernel(const uint8_t* __restrict__ codes, const void* __restrict__ scales,
               const float* gs_ptr, int64_t rows, int64_t cols, void* __restrict__ dst,
               int64_t ld) {
  const int64_t cpr = cols >> 3;
  const int64_t total = rows * cpr;
  const float gs = (FMT == 2) ? *gs_ptr : 0.0f;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t c0 = (int64_t)blockIdx.x * kThreads + threadIdx.x; c0 < total; c0 += kDqUnroll * stride) {
    DqIn d[kDqUnroll];
    int64_t rr[kDqUnroll], kk[kDqUnroll];
#pragma unroll
    for (int u = 0; u < kDqUnroll; ++u) {
      const int64_t c = min(c0 + u * stride, total - 1);  // past the end: load the last chunk again
      rr[u] = IDX32 ? (int64_t)((uint32_t)c / (uint32_t)cpr) : c / cpr;
      kk[u] = (c - rr[u] * cpr) * 8;
      d[u] = dq_load<FMT, LAYOUT>(codes, scales, rr[u], kk[u], cols);
    }
#pragma unroll
    for (int u = 0; u < kDqUnroll; ++u)
      if (c0 + u * stride < total) dq_store<FMT, OUT>(d[u], gs, rr[u], kk[u], dst, ld);
  }
}

// Tiled layout: a wave takes 16 rows x 512 k (four 1 KB tiles, one scale
// group) -- four whole-kilobyte loads and one load of the group's scale
// bytes -- and stages them in its own LDS space; it then walks the 16 rows,
// lane l converting the 8 codes at k = 8l of the row (4 bytes of LDS) and
// storing them as one 16-byte piece of a contiguous kilobyte of the row, so
// both the reads and the writes are whole kilobytes.
constexpr int kDqtWaves = kThreads / 64;

template <int FMT>
struct DqtScales {  // the scale group of one 16-row tile and 512 k, as stored
  static constexpr int kBytes = FMT == 0 ? 128 : FMT == 2 ? 512 : 256;
  static constexpr int kPerLane = kBytes / 64;  // 2, 4 or 8 bytes
};

template <int FMT, int OUT>
__global__ void __launch_bounds__(kThreads)
dequant_tiled_kernel(const uint8_t* __restrict__ codes, const void* __restrict__ scales,
                     const float* gs_ptr, int64_t rows, int64_t cols, void* __restrict__ dst,
                     int64_t ld) {
  __shared__ __attribute__((aligned(16))) uint8_t stage[kDqtWaves][4096 + 512];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t S = cols >> 7, Q = cols >> 9;
  const int64_t units = ((rows + 15) >> 4) * Q;
  const int64_t unit = (int64_t)blockIdx.x * kDqtWaves + wave;
  if (unit >= units) return;  // wave-uniform; no barrier follows
  const float gs = (FMT == 2) ? *gs_ptr : 0.0f;
  const int64_t t = unit / Q, q = unit - t * Q;
  uint8_t* const sc = stage[wave];
  // four tiles (t, 4q .. 4q+3): 1 KB each
  const uint8_t* const tsrc = codes + ((t * S + 4 * q) << 10) + lane * 16;
  uint4 w[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) w[j] = *reinterpret_cast<const uint4*>(tsrc + j * 1024);
  const uint8_t* const ssrc = reinterpret_cast<const uint8_t*>(scales) +
                              (t * Q + q) * DqtScales<FMT>::kBytes + lane * DqtScales<FMT>::kPerLane;
  if constexpr (DqtScales<FMT>::kPerLane == 2)
    *reinterpret_cast<uint16_t*>(sc + 4096 + lane * 2) = *reinterpret_cast<const uint16_t*>(ssrc);
  else if constexpr (DqtScales<FMT>::kPerLane == 4)
    *reinterpret_cast<uint32_t*>(sc + 4096 + lane * 4) = *reinterpret_cast<const uint32_t*>(ssrc);
  else
    *reinterpret_cast<uint2*>(sc + 4096 + lane * 8) = *reinterpret_cast<const uint2*>(ssrc);
#pragma unroll
  for (int j = 0; j < 4; ++j) *reinterpret_cast<uint4*>(sc + j * 1024 + lane * 16) = w[j];
  __builtin_amdgcn_wave_barrier();  // the wave's LDS writes before its reads (one wave, in order)
  // lane l: k = 8l of the 512, i.e. tile s = l/16, 32-k group g = (l/4)%4, piece p = l%4
  const int s = lane >> 4, g = (lane >> 2) & 3, pc = lane & 3;
  const int64_t k0 = 512 * q + 8 * lane;
  const int nrows = (int)min((int64_t)16, rows - 16 * t);
  for (int n = 0; n < nrows; ++n) {
    const int tl = g * 16 + n;  // the lane of the tile that holds these codes
    DqIn d;
    d.packed = *reinterpret_cast<const uint32_t*>(sc + s * 1024 + tl * 16 + pc * 4);
    if constexpr (FMT == 0) d.sraw = *reinterpret_cast<const uint16_t*>(sc + 4096 + (n * 4 + s) * 2);
    else if constexpr (FMT == 4) d.sraw = *reinterpret_cast<const uint32_t*>(sc + 4096 + (n * 4 + s) * 4);
    else if constexpr (FMT == 1) d.sraw = sc[4096 + tl * 4 + s];
    else d.sraw = sc[4096 + tl * 8 + 2 * s + (pc >> 1)];
    dq_store<FMT, OUT>(d, gs, 16 * t + n, k0, dst, ld);
  }
}

unsigned grid_for(int64_t chunks) {
  int64_t b = (chunks + kThreads - 1) / kThreads;
  if (b < 1) b = 1;
  if (b > (1 << 20)) b = 1 << 20;
  return (unsigned)b;
}

// Quantize kernel launch: the block-mapped kernel when cols % 128 == 0,
// else the lane-per-8-values kernel.
// reverse = 1 walks the row bands last to first (see the NVFP4 path).
template <int FMT, int LAYOUT>
void launch_q(const uint16_t* src, int64_t ld, int64_t rows, int64_t cols, uint8_t* codes,
              void* scales, const float* gs_src, float* gs_out, hipStream_t stream, int reverse = 0) {
  if (cols % 128 == 0) {
    const int64_t blocks = ((stored_rows<LAYOUT>(rows) + 15) / 16) * ((cols + 511) / 512);
    quantize_block_kernel<FMT, LAYOUT><<<(unsigned)blocks, kThreads, 0, stream>>>(
        src, ld, rows, cols, codes, scales, gs_src, gs_out, reverse);
  } else {
    const unsigned grid = grid_for(stored_rows<LAYOUT>(rows) * (cols >> 3));
    quantize_kernel<FMT, LAYOUT><<<grid, kThreads, 0, stream>>>(src, ld, rows, cols, codes, scales,
                                                               gs_src, gs_out);
  }
}

template <int LAYOUT>
hipError_t quantize_layout(int fmt, const uint16_t* src, int64_t ld, int64_t rows, int64_t cols,
                           uint8_t* codes, void* scales, float* gs, const float* gs_in,
                           hipStream_t stream) {
  const int64_t chunks = stored_rows<LAYOUT>(rows) * (cols >> 3);
  if (fmt == 0) {
    if (chunks) launch_q<0, LAYOUT>(src, ld, rows, cols, codes, scales, nullptr, nullptr, stream);
  } else if (fmt == 4) {
    if (chunks) launch_q<4, LAYOUT>(src, ld, rows, cols, codes, scales, nullptr, nullptr, stream);
  } else if (fmt == 1) {
    if (chunks) launch_q<1, LAYOUT>(src, ld, rows, cols, codes, scales, nullptr, nullptr, stream);
  } else {
    if (gs_in) {
      if (chunks) {
        launch_q<2, LAYOUT>(src, ld, rows, cols, codes, scales, gs_in, gs, stream);
      } else {
        // nothing to quantize: still record the caller's gs
        hipError_t e = hipMemcpyAsync(gs, gs_in, sizeof(float), hipMemcpyDeviceToDevice, stream);
        if (e != hipSuccess) return e;
      }
    } else {
      // gs of amax 0 (an empty tensor keeps it), then the absmax pass folds
      // each workgroup's gs into it, and the quantizer reads the result
      const float gs0 = 1e-12f / 2688.0f;
      uint32_t gs0_bits = 0;
      memcpy(&gs0_bits, &gs0, sizeof gs0_bits);
      uint32_t* gs_bits = reinterpret_cast<uint32_t*>(gs);
      set_word_kernel<<<1, 1, 0, stream>>>(gs_bits, gs0_bits);
      if (chunks) {
        if (rows > 0 && cols > 0) {
          // one workgroup per CU: with 2048 workgroups the final atomic max
          // of each one serialized into a tail (8192^2 NVFP4: 82 -> 69 us)
          const unsigned agrid = (unsigned)(rows < 256 ? rows : 256);
          absmax_kernel<<<agrid, kThreads, 0, stream>>>(src, ld, rows, cols, gs_bits);
        }
        // the absmax pass reads the rows first to last, so the last ones
        // are still in the last-level cache: the block pass starts there
        launch_q<2, LAYOUT>(src, ld, rows, cols, codes, scales, gs, nullptr, stream, 1);
      }
    }
  }
  return hipGetLastError();
}

template <int LAYOUT>
hipError_t dequant_layout(int fmt, const uint8_t* codes, const void* scales, const float* gs,
                          int64_t rows, int64_t cols, void* dst, int dst_dtype, int64_t ld,
                          hipStream_t stream) {
  const int64_t chunks = rows * (cols >> 3);
  if (!chunks) return hipSuccess;
  if constexpr (LAYOUT == kLayoutTiled) {
    const int64_t units = ((rows + 15) >> 4) * (cols >> 9);   // 16 rows x 512 k per wave
    const unsigned tgrid = (unsigned)((units + kDqtWaves - 1) / kDqtWaves);
#define Q4_DQT(F, O) dequant_tiled_kernel<F, O><<<tgrid, kThreads, 0, stream>>>(codes, scales, gs, rows, cols, dst, ld)
    if (dst_dtype == 0) {
      if (fmt == 0) { Q4_DQT(0, 0); } else if (fmt == 1) { Q4_DQT(1, 0); } else if (fmt == 4) { Q4_DQT(4, 0); } else { Q4_DQT(2, 0); }
    } else {
      if (fmt == 0) { Q4_DQT(0, 1); } else if (fmt == 1) { Q4_DQT(1, 1); } else if (fmt == 4) { Q4_DQT(4, 1); } else { Q4_DQT(2, 1); }
    }
#undef Q4_DQT
    return hipGetLastError();
  }
  const unsigned grid = grid_for((chunks + kDqUnroll - 1) / kDqUnroll);
  const bool idx32 = chunks <= 0xFFFFFFFFll;
#define Q4_DQ(F, O)                                                                                              \
  if (idx32) dequant_kernel<F, O, LAYOUT, true><<<grid, kThreads, 0, stream>>>(codes, scales, gs, rows, cols, dst, ld); \
  else dequant_kernel<F, O, LAYOUT, false><<<grid, kThreads, 0, stream>>>(codes, scales, gs, rows, cols, dst, ld)
  if (dst_dtype == 0) {
    if (fmt == 0) { Q4_DQ(0, 0); } else if (fmt == 1) { Q4_DQ(1, 0); } else if (fmt == 4) { Q4_DQ(4, 0); } else { Q4_DQ(2, 0); }
  } else {
    if (fmt == 0) { Q4_DQ(0, 1); } else if (fmt == 1) { Q4_DQ(1, 1); } else if (fmt == 4) { Q4_DQ(4, 1); } else { Q4_DQ(2, 1); }
  }
#undef Q4_DQ
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize(int fmt, int layout, const uint16_t* src, int64_t ld, int64_t rows,
                           int64_t cols, uint8_t* codes, void* scales, float* gs,
                           const float* gs_in, hipStream_t stream) {
  if (layout == kLayoutTiled)
    return quantize_layout<kLayoutTiled>(fmt, src, ld, rows, cols, codes, scales, gs, gs_in, stream);
  return quantize_layout<kLayoutRows>(fmt, src, ld, rows, cols, codes, scales, gs, gs_in, stream);
}

hipError_t launch_dequant(int fmt, int layout, const uint8_t* codes, const void* scales,
                          const float* gs, int64_t rows, int64_t cols, void* dst, int dst_dtype,
                          int64_t ld, hipStream_t stream) {
  if (layout == kLayoutTiled)
    return dequant_layout<kLayoutTiled>(fmt, codes, scales, gs, rows, cols, dst, dst_dtype, ld, stream);
  return dequant_layout<kLayoutRows>(fmt, codes, scales, gs, rows, cols, dst, dst_dtype, ld, stream);
}

}  // namespace q4
