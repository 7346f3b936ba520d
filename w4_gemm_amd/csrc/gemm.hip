// gemm.hip -- W4A16 GEMM (prefill), grouped per-expert W4A16 GEMM (MoE) and
// W4A4 MXFP4 GEMM on gfx950 matrix cores.
//
// W4A16 ("Low-bit inference for very large MoE", table "Kernels on
// different hardware", row W4A16): weights are dequantized to bf16 in
// registers and multiplied on bf16 matrix cores (v_mfma_f32_16x16x32_bf16)
// with fp32 accumulation.  The grouped MoE GEMM (same page, "A few
// details": one low-bit weight matrix per expert, rows grouped by routing)
// is the same tile kernel with the A rows gathered through the routing
// permutation and the row range of each expert read from device offsets.
//
// W4A4 (same table, row W4A4): both operands are MXFP4 and enter the
// block-scaled FP4 matrix core v_mfma_scale_f32_16x16x128_f8f6f4 directly.
// Its operand layout (measured on gfx950): lane l holds the 32 codes of row
// l%16 for k in [32(l/16), 32(l/16)+32) -- one MXFP4 block, 16 bytes, low
// nibble first -- plus that block's E8M0 byte; so a 16-byte load of a row's
// packed codes is directly an operand.
//
// Tile shape: a workgroup of 4 waves covers 64 rows (m) x 256 columns (n);
// each wave owns a 64x64 tile = 4x4 matrix-core tiles of 16x16 and walks K
// in super-chunks of 128.  Rows past the end are clamped for loads and
// masked for stores.  A lane's 16 code bytes for a super-chunk are the same
// operand in both layouts; the tiled layout (include/q4.h) just puts the 64
// lanes' pieces next to each other.
#include "q4_launch.h"
#include "q4_layout.h"
#include "q4_mma.h"

namespace q4 {
namespace {

constexpr int MT = 4;   // 16-row tiles per wave (m)
constexpr int NT = 4;   // 16-col tiles per wave (n)
constexpr int WAVES = 4;

// Pointer to this lane's 16 code bytes of super-chunk 0 for row `row`
// (row % 16 is the lane's column n), and the byte step between super-chunks.
template <int LAYOUT>
__device__ __forceinline__ const uint8_t* frag_base(const uint8_t* codes, int64_t row, int lane,
                                                    int64_t K) {
  if constexpr (LAYOUT == kLayoutRows) return codes + row * (K >> 1) + (lane >> 4) * 16;
  else return codes + (row >> 4) * (K >> 7) * 1024 + lane * 16;
}
template <int LAYOUT>
constexpr int frag_step() { return LAYOUT == kLayoutRows ? 64 : 1024; }

// One launch covers either a dense GEMM (offsets == nullptr: rows [0, M),
// W rows [0, N), grid.y = M tiles of 64) or a grouped GEMM (grid.y =
// experts: rows [offsets[e], offsets[e+1]) clamped to [0, P), W rows
// [e*N, (e+1)*N), A rows through gather[]).
template <int FMT, int LAYOUT>
__global__ void __launch_bounds__(WAVES * 64)
w4a16_kernel(const uint16_t* __restrict__ A, int64_t lda, int64_t T,
             const int32_t* __restrict__ gather, const int32_t* __restrict__ offsets,
             int64_t M, const uint8_t* __restrict__ codes, const void* __restrict__ scales,
             const float* __restrict__ gs_ptr, int N, int K, uint16_t* __restrict__ C,
             int64_t ldc) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int n_wave = blockIdx.x * (WAVES * 16 * NT) + wave * (16 * NT);
  if (n_wave >= N) return;  // whole wave outside N; no block-level sync below

  int64_t row_lo, row_hi, wbase;
  if (offsets) {
    const int e = blockIdx.y;
    row_lo = min<int64_t>(max<int64_t>(offsets[e], 0), M);
    row_hi = min<int64_t>(max<int64_t>(offsets[e + 1], row_lo), M);
    wbase = (int64_t)e * N;
  } else {
    row_lo = (int64_t)blockIdx.y * (16 * MT);
    row_hi = min<int64_t>(row_lo + 16 * MT, M);
    wbase = 0;
  }
  const float gs = (FMT == 2) ? *gs_ptr : 0.0f;

  // In the tiled layout rows are clamped within the expert's last tile
  // (N % 16 == 0 there, so tiles never straddle experts).
  const uint8_t* wfrag[NT];
  int64_t wrow[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int n = min(n_wave + 16 * nt + col, N - 1);
    wrow[nt] = wbase + n;
    wfrag[nt] = frag_base<LAYOUT>(codes, wbase + n, lane, K);
  }

  for (int64_t m0 = row_lo; m0 < row_hi; m0 += 16 * MT) {
    const uint16_t* arow[MT];
    bool aval[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int64_t p = m0 + 16 * mt + col;
      int64_t src = p;
      bool ok = p < row_hi;
      if (gather && ok) {
        src = gather[p];
        ok = src >= 0 && src < T;
      }
      aval[mt] = ok;
      arow[mt] = A + (ok ? src : 0) * lda;
    }
    f32x4_t acc[MT][NT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

    for (int k0s = 0; k0s < K; k0s += 128) {
      const int k0 = k0s + (grp << 5);
      u32x4_t wq[NT];
      uint32_t sraw[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        wq[nt] = *reinterpret_cast<const u32x4_t*>(wfrag[nt] + (int64_t)(k0s >> 7) * frag_step<LAYOUT>());
        const int64_t so = scale_off<FMT, LAYOUT>(wrow[nt], k0, K);
        if constexpr (FMT == 0)
          sraw[nt] = reinterpret_cast<const uint16_t*>(scales)[so];
        else if constexpr (FMT == 4)
          sraw[nt] = reinterpret_cast<const uint32_t*>(scales)[so];
        else if constexpr (FMT == 1)
          sraw[nt] = reinterpret_cast<const uint8_t*>(scales)[so];
        else  // the lane's two 16-blocks are adjacent in both layouts
          sraw[nt] = *reinterpret_cast<const uint16_t*>(reinterpret_cast<const uint8_t*>(scales) + so);
      }
      u32x4_t av[MT][4];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          av[mt][i] = aval[mt] ? *reinterpret_cast<const u32x4_t*>(arow[mt] + k0 + 8 * i)
                               : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          bf16x8_t wb;
          if constexpr (FMT == 0) {
            wb = dq8_int4(wq[nt][i], fp16_value(sraw[nt]));
          } else if constexpr (FMT == 4) {
            float sc, off;
            int4zp_scale(sraw[nt], sc, off);
            wb = dq8_int4_off(wq[nt][i], sc, off);
          } else if constexpr (FMT == 1) {
            wb = dq8_e2m1(wq[nt][i], e8m0_value(sraw[nt]));
          } else {
            const uint32_t sb = (i < 2) ? (sraw[nt] & 0xFFu) : (sraw[nt] >> 8);
            wb = dq8_e2m1_mul(wq[nt][i], e4m3_value(sb) * gs);
          }
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
            acc[mt][nt] = mma16x16x32(as_bf16x8(av[mt][i]), wb, acc[mt][nt]);
        }
      }
    }
    // lane l, register r holds (m = 4(l/16) + r, n = l%16) of each tile
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int n = n_wave + 16 * nt + col;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int64_t p = m0 + 16 * mt + 4 * grp + r;
          if (p < row_hi && n < N) {
            bool ok = true;
            if (gather) {
              const int64_t src = gather[p];
              ok = src >= 0 && src < T;
            }
            C[p * ldc + n] = ok ? (uint16_t)f32_to_bf16_rne(acc[mt][nt][r]) : (uint16_t)0;
          }
        }
      }
  }
}

// W4A4: C[m][n] = sum_k a'[m][k] w'[n][k] with both operands MXFP4.
template <int ALAYOUT, int WLAYOUT>
__global__ void __launch_bounds__(WAVES * 64)
w4a4_kernel(const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales, int M,
            const uint8_t* __restrict__ w_codes, const uint8_t* __restrict__ w_scales, int N,
            int K, uint16_t* __restrict__ C, int64_t ldc) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int n_wave = blockIdx.x * (WAVES * 16 * NT) + wave * (16 * NT);
  if (n_wave >= N) return;
  const int m0 = blockIdx.y * (16 * MT);

  const uint8_t* afrag[MT];
  int arow[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    arow[mt] = min(m0 + 16 * mt + col, M - 1);
    afrag[mt] = frag_base<ALAYOUT>(a_codes, arow[mt], lane, K);
  }
  const uint8_t* wfrag[NT];
  int wrow[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    wrow[nt] = min(n_wave + 16 * nt + col, N - 1);
    wfrag[nt] = frag_base<WLAYOUT>(w_codes, wrow[nt], lane, K);
  }
  f32x4_t acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  for (int k0s = 0; k0s < K; k0s += 128) {
    const int s = k0s >> 7;
    const int k = k0s + (grp << 5);  // first k of this lane's MXFP4 block
    i32x8_t aop[MT], wop[NT];
    uint32_t asc[MT], wsc[NT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(afrag[mt] + (int64_t)s * frag_step<ALAYOUT>());
      aop[mt] = i32x8_t{(int)v[0], (int)v[1], (int)v[2], (int)v[3], 0, 0, 0, 0};
      asc[mt] = a_scales[scale_off<1, ALAYOUT>(arow[mt], k, K)];
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(wfrag[nt] + (int64_t)s * frag_step<WLAYOUT>());
      wop[nt] = i32x8_t{(int)v[0], (int)v[1], (int)v[2], (int)v[3], 0, 0, 0, 0};
      wsc[nt] = w_scales[scale_off<1, WLAYOUT>(wrow[nt], k, K)];
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        acc[mt][nt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            aop[mt], wop[nt], acc[mt][nt], 4, 4, 0, asc[mt], 0, wsc[nt]);
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int n = n_wave + 16 * nt + col;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + 16 * mt + 4 * grp + r;
        if (m < M && n < N) C[(int64_t)m * ldc + n] = (uint16_t)f32_to_bf16_rne(acc[mt][nt][r]);
      }
    }
}

template <int FMT, int LAYOUT>
hipError_t run_w4a16(const uint16_t* A, int64_t lda, int64_t T, const int32_t* gather,
                     const int32_t* offsets, int64_t gy, int64_t M, const uint8_t* codes,
                     const void* scales, const float* gs, int64_t N, int64_t K, uint16_t* C,
                     int64_t ldc, hipStream_t stream) {
  const dim3 grid((unsigned)((N + WAVES * 16 * NT - 1) / (WAVES * 16 * NT)), (unsigned)gy);
  w4a16_kernel<FMT, LAYOUT><<<grid, WAVES * 64, 0, stream>>>(A, lda, T, gather, offsets, M, codes,
                                                             scales, gs, (int)N, (int)K, C, ldc);
  return hipGetLastError();
}

template <int LAYOUT>
hipError_t dispatch_fmt(int fmt, const uint16_t* A, int64_t lda, int64_t T, const int32_t* gather,
                        const int32_t* offsets, int64_t gy, int64_t M, const uint8_t* codes,
                        const void* scales, const float* gs, int64_t N, int64_t K, uint16_t* C,
                        int64_t ldc, hipStream_t stream) {
  if (fmt == 0)
    return run_w4a16<0, LAYOUT>(A, lda, T, gather, offsets, gy, M, codes, scales, gs, N, K, C, ldc, stream);
  if (fmt == 1)
    return run_w4a16<1, LAYOUT>(A, lda, T, gather, offsets, gy, M, codes, scales, gs, N, K, C, ldc, stream);
  if (fmt == 4)
    return run_w4a16<4, LAYOUT>(A, lda, T, gather, offsets, gy, M, codes, scales, gs, N, K, C, ldc, stream);
  return run_w4a16<2, LAYOUT>(A, lda, T, gather, offsets, gy, M, codes, scales, gs, N, K, C, ldc, stream);
}

hipError_t dispatch_w4a16(int fmt, int layout, const uint16_t* A, int64_t lda, int64_t T,
                          const int32_t* gather, const int32_t* offsets, int64_t gy, int64_t M,
                          const uint8_t* codes, const void* scales, const float* gs, int64_t N,
                          int64_t K, uint16_t* C, int64_t ldc, hipStream_t stream) {
  if (layout == kLayoutTiled)
    return dispatch_fmt<kLayoutTiled>(fmt, A, lda, T, gather, offsets, gy, M, codes, scales, gs, N, K,
                                      C, ldc, stream);
  return dispatch_fmt<kLayoutRows>(fmt, A, lda, T, gather, offsets, gy, M, codes, scales, gs, N, K, C,
                                   ldc, stream);
}

}  // namespace

hipError_t launch_gemm_w4a16(int fmt, int layout, const uint8_t* codes, const void* scales,
                             const float* gs, int64_t N, int64_t K, const uint16_t* A, int64_t lda,
                             int64_t M, uint16_t* C, int64_t ldc, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  if (layout == kLayoutTiled)
    return launch_gemm_w4a16_tiled(fmt, codes, scales, gs, N, K, A, lda, M, C, ldc, stream);
  const int64_t gy = (M + 16 * MT - 1) / (16 * MT);
  return dispatch_w4a16(fmt, layout, A, lda, M, nullptr, nullptr, gy, M, codes, scales, gs, N, K,
                        C, ldc, stream);
}

hipError_t launch_grouped(int fmt, int layout, const uint16_t* A, int64_t lda, int64_t T,
                          const int32_t* gather, const int32_t* offsets, int32_t E, int64_t P,
                          const uint8_t* codes, const void* scales, const float* gs, int64_t N,
                          int64_t K, uint16_t* C, int64_t ldc, hipStream_t stream) {
  if (E == 0 || N == 0 || P == 0) return hipSuccess;
  if (layout == kLayoutTiled && T > 0)
    return launch_grouped_tiled(fmt, A, lda, T, gather, offsets, E, P, codes, scales, gs, N, K, C, ldc,
                                stream);
  return dispatch_w4a16(fmt, layout, A, lda, T, gather, offsets, E, P, codes, scales, gs, N, K, C,
                        ldc, stream);
}

hipError_t launch_gemm_w4a4(int a_layout, int w_layout, const uint8_t* a_codes,
                            const uint8_t* a_scales, int64_t M, const uint8_t* w_codes,
                            const uint8_t* w_scales, int64_t N, int64_t K, uint16_t* C,
                            int64_t ldc, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  if (a_layout == kLayoutTiled && w_layout == kLayoutTiled)
    return launch_gemm_w4a4_tiled(a_codes, a_scales, M, w_codes, w_scales, N, K, C, ldc, stream);
  const dim3 grid((unsigned)((N + WAVES * 16 * NT - 1) / (WAVES * 16 * NT)),
                  (unsigned)((M + 16 * MT - 1) / (16 * MT)));
#define Q4_W4A4(AL, WL) w4a4_kernel<AL, WL><<<grid, WAVES * 64, 0, stream>>>(a_codes, a_scales, (int)M, w_codes, w_scales, (int)N, (int)K, C, ldc)
  if (a_layout == kLayoutTiled) {
    if (w_layout == kLayoutTiled) Q4_W4A4(kLayoutTiled, kLayoutTiled); else Q4_W4A4(kLayoutTiled, kLayoutRows);
  } else {
    if (w_layout == kLayoutTiled) Q4_W4A4(kLayoutRows, kLayoutTiled); else Q4_W4A4(kLayoutRows, kLayoutRows);
  }
#undef Q4_W4A4
  return hipGetLastError();
}

}  // namespace q4
