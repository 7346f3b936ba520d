// gemv.hip -- W4A16 GEMV for decode: y[b][n] = sum_k x[b][k] * w'[n][k],
// B <= 16, fp32 accumulation, bf16 output.
//
// Decode reads every weight once per token and is limited by those reads
// ("Low-bit inference for very large MoE", table "Kernels on different
// hardware", row W4A16 and the decode bullet of "A few details"), so the
// kernel is built to stream the packed nibbles and scales from HBM at full
// rate and keep everything else off the memory path.
//
// Mapping on gfx950 (64-lane waves, bf16 matrix cores):
//   * one v_mfma_f32_16x16x32_bf16 step multiplies a 16x32 tile of x (batch
//     rows, zero beyond B) by a 32x16 tile of dequantized weights (16 output
//     columns n).  Because a dot product does not care about the order of k,
//     lane (n = l%16, g = l/16) loads the 16 bytes holding 32 consecutive
//     codes of row n -- exactly one MXFP4 block, two NVFP4 blocks, a quarter
//     INT4 group -- and feeds them to four consecutive steps; the x lanes
//     load the same 32 k for their batch row.  So 128 k (one super-chunk)
//     cost one 16-byte weight load and one scale load per lane.
//   * a wave owns RT tiles of 16 rows and reuses each x fragment across them.
//   * the WAVES waves of a workgroup split K; their partial tiles are summed
//     in LDS in a fixed order (deterministic) and written as bf16.
#include "q4_launch.h"
#include "q4_mma.h"

namespace q4 {
namespace {

template <int FMT, int RT, int WAVES>
__global__ void __launch_bounds__(WAVES * 64)
gemv_kernel(const uint8_t* __restrict__ codes, const void* __restrict__ scales,
            const float* __restrict__ gs_ptr, int N, int K,
            const uint16_t* __restrict__ x, int64_t ldx, int B,
            uint16_t* __restrict__ y, int64_t ldy) {
  __shared__ f32x4_t red[WAVES][RT][64];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int n_base = blockIdx.x * (16 * RT);
  const int nsc = K >> 7;
  const int s_begin = (nsc * wave) / WAVES;
  const int s_end = (nsc * (wave + 1)) / WAVES;
  const int64_t row_bytes = K >> 1;

  const uint8_t* wrow[RT];
  int64_t srow[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int n = min(n_base + 16 * rt + col, N - 1);  // clamped: tail lanes load a valid row
    wrow[rt] = codes + (int64_t)n * row_bytes;
    srow[rt] = (int64_t)n * (K / (FMT == 0 ? 128 : (FMT == 1 ? 32 : 16)));
  }
  const bool xlane = col < B;
  const uint16_t* xrow = x + (int64_t)(xlane ? col : 0) * ldx;
  const float gs = (FMT == 2) ? *gs_ptr : 0.0f;

  f32x4_t acc[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) acc[rt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  for (int s = s_begin; s < s_end; ++s) {
    const int k0 = (s << 7) + (grp << 5);
    u32x4_t wq[RT];
    uint32_t sraw[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      wq[rt] = *reinterpret_cast<const u32x4_t*>(wrow[rt] + (k0 >> 1));
      if constexpr (FMT == 0)
        sraw[rt] = reinterpret_cast<const uint16_t*>(scales)[srow[rt] + s];
      else if constexpr (FMT == 1)
        sraw[rt] = reinterpret_cast<const uint8_t*>(scales)[srow[rt] + (k0 >> 5)];
      else
        sraw[rt] = *reinterpret_cast<const uint16_t*>(
            reinterpret_cast<const uint8_t*>(scales) + srow[rt] + (k0 >> 4));
    }
    u32x4_t xv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      xv[i] = xlane ? *reinterpret_cast<const u32x4_t*>(xrow + k0 + 8 * i)
                    : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        bf16x8_t wb;
        if constexpr (FMT == 0) {
          wb = dq8_int4(wq[rt][i], fp16_value(sraw[rt]));
        } else if constexpr (FMT == 1) {
          wb = dq8_e2m1(wq[rt][i], e8m0_value(sraw[rt]));
        } else {
          const uint32_t sb = (i < 2) ? (sraw[rt] & 0xFFu) : (sraw[rt] >> 8);
          wb = dq8_e2m1_mul(wq[rt][i], e4m3_value(sb) * gs);
        }
        acc[rt] = mma16x16x32(as_bf16x8(xv[i]), wb, acc[rt]);
      }
    }
  }

#pragma unroll
  for (int rt = 0; rt < RT; ++rt) red[wave][rt][lane] = acc[rt];
  __syncthreads();
  // lane l, register r of a tile holds (b = 4(l/16) + r, n = l%16)
  for (int idx = threadIdx.x; idx < RT * 256; idx += WAVES * 64) {
    const int rt = idx >> 8;
    const int b = (idx >> 4) & 15;
    const int nn = idx & 15;
    const int src_lane = ((b >> 2) << 4) | nn;
    float v = 0.0f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) v += red[w][rt][src_lane][b & 3];
    const int n = n_base + 16 * rt + nn;
    if (b < B && n < N) y[(int64_t)b * ldy + n] = (uint16_t)f32_to_bf16_rne(v);
  }
}

template <int FMT, int RT, int WAVES>
hipError_t run(const uint8_t* codes, const void* scales, const float* gs, int64_t N, int64_t K,
               const uint16_t* x, int64_t ldx, int64_t B, uint16_t* y, int64_t ldy,
               hipStream_t stream) {
  const unsigned grid = (unsigned)((N + 16 * RT - 1) / (16 * RT));
  gemv_kernel<FMT, RT, WAVES><<<grid, WAVES * 64, 0, stream>>>(
      codes, scales, gs, (int)N, (int)K, x, ldx, (int)B, y, ldy);
  return hipGetLastError();
}

template <int FMT>
hipError_t dispatch(const uint8_t* codes, const void* scales, const float* gs, int64_t N,
                    int64_t K, const uint16_t* x, int64_t ldx, int64_t B, uint16_t* y,
                    int64_t ldy, hipStream_t stream) {
  // Enough workgroups to cover 256 CUs several times, K split 8 ways when
  // there are at least 8 super-chunks of 128.
  if (K >= 1024) {
    if (N >= 16384) return run<FMT, 4, 8>(codes, scales, gs, N, K, x, ldx, B, y, ldy, stream);
    if (N >= 4096) return run<FMT, 2, 8>(codes, scales, gs, N, K, x, ldx, B, y, ldy, stream);
    return run<FMT, 1, 8>(codes, scales, gs, N, K, x, ldx, B, y, ldy, stream);
  }
  return run<FMT, 1, 4>(codes, scales, gs, N, K, x, ldx, B, y, ldy, stream);
}

}  // namespace

hipError_t launch_gemv(int fmt, const uint8_t* codes, const void* scales, const float* gs,
                       int64_t N, int64_t K, const uint16_t* x, int64_t ldx, int64_t B,
                       uint16_t* y, int64_t ldy, hipStream_t stream) {
  if (N == 0 || B == 0) return hipSuccess;
  if (fmt == 0) return dispatch<0>(codes, scales, gs, N, K, x, ldx, B, y, ldy, stream);
  if (fmt == 1) return dispatch<1>(codes, scales, gs, N, K, x, ldx, B, y, ldy, stream);
  return dispatch<2>(codes, scales, gs, N, K, x, ldx, B, y, ldy, stream);
}

}  // namespace q4
