// gemm_w4a16.hip -- W4A16 GEMM (prefill) for weights in the tiled layout:
// C[m][n] = sum_k a[m][k] w'[n][k], A bf16 row-major, W' the dequantized
// INT4 g128 / MXFP4 / NVFP4 weight, fp32 accumulation, bf16 output.
//
// W4A16 keeps activations in bf16 and dequantizes the 4-bit weights in
// registers before a bf16 matrix multiply ("Low-bit inference for very
// large MoE", table "Kernels on different hardware", row W4A16).  On gfx950
// the multiply is v_mfma_f32_16x16x32_bf16.
//
// The k order inside a super-chunk (128 k) is free, since a dot product
// does not depend on it: lane l = 16g + n of a 1 KB weight tile holds the
// 32 codes of row n at k in [32g, 32g+32), and matrix step i (0..3) of the
// super-chunk takes the codes 8i..8i+8 of every lane -- k = 32g + 8i +
// [0, 8).  The activation fragment of lane l for step i is then the 16 bytes
// a[m][32g + 8i + (0..8)] with m = l%16.
//
// Work decomposition:
//   * a workgroup of 8 waves computes a 256 x 256 block of C.  All waves
//     share the 256 activation rows; wave w owns the 32 columns of weight
//     tiles 2w, 2w+1: 16 x 2 matrix-core tiles, 128 fp32 accumulators per
//     lane (two waves per SIMD).  Each dequantized weight fragment feeds 16
//     matrix instructions, which keeps the dequantization (a multiply per
//     value for NVFP4) small next to the matrix work (a 128 x 512 block
//     with 8 x 4 tiles per wave, 8 products per fragment, measured 18%
//     slower on NVFP4 4096 x 8192 x 8192).  The activation fragments are
//     read from LDS four row tiles at a time, one group ahead.
//   * K advances in stages of 64 (half a super-chunk: steps 2h, 2h+1).  The
//     activations of a stage (256 rows x 64 k, 32 KB) are gathered into LDS
//     by direct global->LDS loads in matrix-fragment order -- each load
//     instruction fills one fragment, lane l fetching exactly the 16 bytes
//     it will later read -- so every fragment read is one contiguous,
//     conflict-free kilobyte.  Three buffers, two stages ahead.
//   * the weight tiles of a super-chunk (the wave's own two, 1 KB each) are
//     copied verbatim into LDS one super-chunk ahead (two buffers); the
//     scale words of a group of four super-chunks go straight into registers
//     (two sets).
//   * one barrier per stage: each wave waits (explicit vmcnt) for its own
//     loads of the stage, the barrier makes all activation fragments
//     visible and frees the buffer the next copies overwrite.  The loop is
//     unrolled by 8 (one scale group) so every wait count is a constant.
//     The copies of a stage are issued one part at a time between its
//     groups of products: issued together right after the barrier they
//     held every wave at once (a copy instruction costs the issuing wave
//     far more than a matrix instruction's issue slot).
//   * weights are the matrix instruction's row operand, so a lane ends with
//     4 consecutive columns of one row of C: 8-byte stores, or the
//     quantized-output epilogue (q4_qout.h: C written as MXFP4 / NVFP4).
#include "q4_launch.h"
#include "q4_layout.h"
#include "q4_lds.h"
#include "q4_mma.h"
#include "q4_qout.h"

#include <type_traits>

namespace q4 {
namespace {

constexpr int kWaves = 8;
constexpr int kRowTiles = 16;                   // 16-row activation tiles per block (256 rows)
constexpr int kWTiles = 2;                      // weight tiles per wave
constexpr int kColTiles = kWTiles * kWaves;     // 16-column weight tiles per block (256 cols)
constexpr int kAFrags = 2 * kRowTiles;          // activation fragments per stage
constexpr int kABufs = 3;
constexpr size_t kSmemBytes = kABufs * kAFrags * 1024 + 2 * kColTiles * 1024;  // 128 KB

// Loads issued for running stage v (group v): the stage's activation
// fragments (4 per wave), the weight tiles of super-chunk v/2 when v is
// even (2 per wave), the scale words of scale group v/8 when v % 8 == 0
// (2 per wave).
constexpr int group_loads(int v) {
  return kAFrags / kWaves + (v % 2 == 0 ? kWTiles : 0) + (v % 8 == 0 ? kWTiles : 0);
}

template <int FMT, int OUT>
__global__ void __launch_bounds__(kWaves * 64)
w4a16_tiled_kernel(const uint16_t* __restrict__ A, int64_t lda, int M,
                   const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                   const float* __restrict__ gs_ptr, int N, int K, uint16_t* __restrict__ C,
                   int64_t ldc, QOut qo) {
  qout_copy_gs<OUT>(qo);
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
  uint8_t (*abuf)[kAFrags][1024] = reinterpret_cast<uint8_t (*)[kAFrags][1024]>(smem);
  uint8_t (*wbuf)[kColTiles][1024] =
      reinterpret_cast<uint8_t (*)[kColTiles][1024]>(smem + kABufs * kAFrags * 1024);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int S = K >> 7, Q = K >> 9, S2 = 2 * S;   // super-chunks, scale groups, stages
  const int RTW = (N + 15) >> 4;

  // workgroup -> 256 x 256 block of C: XCD-major, then groups of 4 block rows
  const int TM = (M + 255) >> 8, TN = (N + 255) >> 8, T = TM * TN;
  const int b = blockIdx.x;
  const int lin = (T % 8 == 0) ? (b % 8) * (T / 8) + b / 8 : b;
  const int gsz = 4 * TN, first_m = (lin / gsz) * 4, gm = min(TM - first_m, 4);
  const int bm = first_m + (lin % gsz) % gm, bn = (lin % gsz) / gm;

  // activation copies: this wave fills the fragments of row tiles 2*wave
  // and 2*wave+1 (steps 2h and 2h+1 of each stage); lane l reads row
  // 16*tile + l%16 (clamped) at k = 32(l/16) + 8i within the super-chunk
  const uint16_t* asrc[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int arow = min(bm * 256 + 16 * (2 * wave + t) + (lane & 15), M - 1);
    asrc[t] = A + (int64_t)arow * lda + 32 * (lane >> 4);
  }
  // this wave's weight tiles (copied and multiplied by it alone)
  const int wt0 = bn * kColTiles + kWTiles * wave;
  // (wave-uniform bases; the lane offsets are added at each load)
  const uint8_t* wsrc[kWTiles];
#pragma unroll
  for (int jj = 0; jj < kWTiles; ++jj) wsrc[jj] = codes + (int64_t)min(wt0 + jj, RTW - 1) * S * 1024;
  const int wlane = lane * 16;
  // this lane's scale bytes of a scale group for weight tile jj: MXFP4 4
  // bytes (one per super-chunk), NVFP4 8 (two per super-chunk), INT4 4 fp16
  // of row n = lane%16 (one per super-chunk)
  constexpr int SW = FMT == 1 ? 1 : FMT == 4 ? 4 : 2;  // 32-bit words per tile and group
  const uint8_t* ssrc[kWTiles];
#pragma unroll
  for (int jj = 0; jj < kWTiles; ++jj) {
    const int64_t t = min(wt0 + jj, RTW - 1);
    ssrc[jj] = scales + t * Q * (FMT == 0 ? 128 : FMT == 1 || FMT == 4 ? 256 : 512);
  }
  const int slane = FMT == 0 ? (lane & 15) * 8 : FMT == 4 ? (lane & 15) * 16 : FMT == 1 ? lane * 4 : lane * 8;
  const float gs = (FMT == 2) ? *gs_ptr : 0.0f;

  // scale words of the current scale group and of the next one (loaded
  // with group 8q, moved into place when the group's first stage starts)
  uint32_t scur[kWTiles][SW], snext[kWTiles][SW];
  // group v (jc = v % 8), in six parts issued in this order: 0..3 the
  // activation copies (row tile t = part / 2, step ip = part % 2), 4 the
  // weight tiles, 5 the scale words; part -1 issues all of them
  auto issue = [&](int v, auto jc, int part) {
    constexpr int J = decltype(jc)::value;
    const int vs = min(v, S2 - 1);
    const int s = vs >> 1, h = vs & 1;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int ip = 0; ip < 2; ++ip)
        if (part < 0 || part == 2 * t + ip)
          copy16_to_lds(asrc[t] + 128 * s + 8 * (2 * h + ip), abuf[v % kABufs][2 * (2 * wave + t) + ip]);
    if constexpr (J % 2 == 0) {
      if (part < 0 || part == 4) {
#pragma unroll
        for (int jj = 0; jj < kWTiles; ++jj)
          copy16_to_lds(wsrc[jj] + (int64_t)s * 1024 + wlane, wbuf[(v >> 1) & 1][kWTiles * wave + jj]);
      }
    }
    if constexpr (J == 0) {
      if (part < 0 || part == 5) {
      const int q = min(v >> 3, Q - 1);
#pragma unroll
      for (int jj = 0; jj < kWTiles; ++jj) {
        if constexpr (SW == 1) {
          snext[jj][0] = *reinterpret_cast<const uint32_t*>(ssrc[jj] + (int64_t)q * 256 + slane);
        } else if constexpr (SW == 4) {
          const u32x4_t w4 = *reinterpret_cast<const u32x4_t*>(ssrc[jj] + (int64_t)q * 256 + slane);
#pragma unroll
          for (int w = 0; w < 4; ++w) snext[jj][w] = w4[w];
        } else {
          const uint2 w2 = *reinterpret_cast<const uint2*>(ssrc[jj] + (int64_t)q * (FMT == 0 ? 128 : 512) + slane);
          snext[jj][0] = w2.x;
          snext[jj][1] = w2.y;
        }
      }
      }
    }
  };

  f32x4_t acc[kRowTiles][kWTiles];
#pragma unroll
  for (int i = 0; i < kRowTiles; ++i)
#pragma unroll
    for (int jj = 0; jj < kWTiles; ++jj) acc[i][jj] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  u32x4_t wq[kWTiles];  // the wave's weight fragments of the current super-chunk

  // stage u, J = u % 8: wait until only group u+1 may be outstanding,
  // barrier, multiply, issuing group u+2 (into the buffers stage u-1 used)
  // among the products.  All of group u+2 is issued before stage u+1's
  // wait, so the counts are those of issuing it at once; spread out, the
  // copies no longer stall every wave together right after the barrier
  // (the first group's products go first): 462 -> 430 us on NVFP4
  // 4096 x 8192 x 8192, bit-identical.
  auto iteration = [&](int u, auto jc) {
    constexpr int J = decltype(jc)::value;
    constexpr int H = J & 1;          // half of the super-chunk
    constexpr int SI = J >> 1;        // super-chunk within the scale group
    wait_vmcnt_lgkm0<group_loads(J + 1)>();
    stage_barrier();
    if constexpr (J == 0) {  // group u/8's scale words have landed (group u is done)
#pragma unroll
      for (int jj = 0; jj < kWTiles; ++jj)
#pragma unroll
        for (int w = 0; w < SW; ++w) scur[jj][w] = snext[jj][w];
    }
    if constexpr (H == 0) {
#pragma unroll
      for (int jj = 0; jj < kWTiles; ++jj)
        wq[jj] = *reinterpret_cast<const u32x4_t*>(&wbuf[(u >> 1) & 1][kWTiles * wave + jj][lane * 16]);
    }
#pragma unroll
    for (int ip = 0; ip < 2; ++ip) {
      const int i = 2 * H + ip;      // matrix step within the super-chunk
      bf16x8_t wb[kWTiles];
#pragma unroll
      for (int jj = 0; jj < kWTiles; ++jj) {
        if constexpr (FMT == 0) {
          const uint32_t hw = (scur[jj][SI >> 1] >> (16 * (SI & 1))) & 0xFFFFu;
          wb[jj] = dq8_int4(wq[jj][i], fp16_value(hw));
        } else if constexpr (FMT == 4) {
          float sc, off;
          int4zp_scale(scur[jj][SI], sc, off);
          wb[jj] = dq8_int4_off(wq[jj][i], sc, off);
        } else if constexpr (FMT == 1) {
          wb[jj] = dq8_e2m1(wq[jj][i], e8m0_value((scur[jj][0] >> (8 * SI)) & 0xFFu));
        } else {
          // the lane's 32 k hold two 16-blocks: steps 0,1 the first, 2,3 the second
          const uint32_t sb = (scur[jj][SI >> 1] >> (16 * (SI & 1) + 8 * H)) & 0xFFu;
          wb[jj] = dq8_e2m1_mul(wq[jj][i], e4m3_value(sb) * gs);
        }
      }
      // the activation fragments in groups of four row tiles, one group
      // read ahead of the products (the fences keep the compiler from
      // reading all sixteen at once, which would not fit two waves per SIMD)
      constexpr int RG = 4;
      bf16x8_t af[2][RG];
      auto read_a = [&](bf16x8_t (&dst)[RG], int g) {
#pragma unroll
        for (int q = 0; q < RG; ++q)
          dst[q] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(&abuf[u % kABufs][2 * (RG * g + q) + ip][lane * 16]));
      };
      read_a(af[0], 0);
#pragma unroll
      for (int g = 0; g < kRowTiles / RG; ++g) {
        if (g + 1 < kRowTiles / RG) read_a(af[(g + 1) & 1], g + 1);
        // group u+2: one part after each of the stage's row-tile groups 1..6
        const int seq = (kRowTiles / RG) * ip + g;
        if (seq >= 1 && seq <= 6) issue(u + 2, std::integral_constant<int, (J + 2) % 8>(), seq - 1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int q = 0; q < RG; ++q)
#pragma unroll
          for (int jj = 0; jj < kWTiles; ++jj)
            acc[RG * g + q][jj] = mma16x16x32(wb[jj], af[g & 1][q], acc[RG * g + q][jj]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  issue(0, std::integral_constant<int, 0>(), -1);
  issue(1, std::integral_constant<int, 1>(), -1);
  // K % 512 == 0 in the tiled layout: the stage count is a multiple of 8
  for (int u0 = 0; u0 < S2; u0 += 8) {
    iteration(u0, std::integral_constant<int, 0>());
    iteration(u0 + 1, std::integral_constant<int, 1>());
    iteration(u0 + 2, std::integral_constant<int, 2>());
    iteration(u0 + 3, std::integral_constant<int, 3>());
    iteration(u0 + 4, std::integral_constant<int, 4>());
    iteration(u0 + 5, std::integral_constant<int, 5>());
    iteration(u0 + 6, std::integral_constant<int, 6>());
    iteration(u0 + 7, std::integral_constant<int, 7>());
  }
  wait_vmcnt_lgkm0<0>();  // no copy into LDS may still be running at exit

  // tile (r, jj): lane l, register q holds C[m][n] with m = 16r + l%16 and
  // n = 16jj + 4(l/16) + q -- four consecutive columns of one row
  const int m0 = bm * 256 + (lane & 15);
  if constexpr (OUT != kOutBf16) {
    store_quantized<OUT>(acc, m0, bn * 256 + 16 * kWTiles * wave, M, N, qo, lane);
    return;
  }
  const int n0 = bn * 256 + 16 * kWTiles * wave + 4 * (lane >> 4);
#pragma unroll
  for (int r = 0; r < kRowTiles; ++r) {
    const int m = m0 + 16 * r;
    if (m < M) {
      uint16_t* crow = C + (int64_t)m * ldc;
#pragma unroll
      for (int jj = 0; jj < kWTiles; ++jj) {
        const int n = n0 + 16 * jj;
        const f32x4_t v = acc[r][jj];
        if (n + 3 < N) {
          store_bf16x4(crow + n, v[0], v[1], v[2], v[3]);
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (n + q < N) crow[n + q] = (uint16_t)f32_to_bf16_rne(v[q]);
        }
      }
    }
  }
}

template <int FMT, int OUT = kOutBf16>
hipError_t run(const uint16_t* A, int64_t lda, int64_t M, const uint8_t* codes, const void* scales,
               const float* gs, int64_t N, int64_t K, uint16_t* C, int64_t ldc, hipStream_t stream,
               const QOut& qo = QOut{}) {
  const hipError_t attr = set_max_lds<&w4a16_tiled_kernel<FMT, OUT>>(kSmemBytes);
  if (attr != hipSuccess) return attr;
  const int64_t T = ((M + 255) / 256) * ((N + 255) / 256);
  w4a16_tiled_kernel<FMT, OUT><<<(unsigned)T, kWaves * 64, kSmemBytes, stream>>>(
      A, lda, (int)M, codes, static_cast<const uint8_t*>(scales), gs, (int)N, (int)K, C, ldc, qo);
  return hipGetLastError();
}

template <int OUT>
hipError_t run_qout(int fmt, const uint16_t* A, int64_t lda, int64_t M, const uint8_t* codes, const void* scales,
                    const float* gs, int64_t N, int64_t K, const QOut& qo, hipStream_t stream) {
  if (fmt == 0) return run<0, OUT>(A, lda, M, codes, scales, gs, N, K, nullptr, 0, stream, qo);
  if (fmt == 1) return run<1, OUT>(A, lda, M, codes, scales, gs, N, K, nullptr, 0, stream, qo);
  if (fmt == 4) return run<4, OUT>(A, lda, M, codes, scales, gs, N, K, nullptr, 0, stream, qo);
  return run<2, OUT>(A, lda, M, codes, scales, gs, N, K, nullptr, 0, stream, qo);
}

}  // namespace

hipError_t launch_gemm_w4a16_tiled(int fmt, const uint8_t* codes, const void* scales, const float* gs,
                                   int64_t N, int64_t K, const uint16_t* A, int64_t lda, int64_t M,
                                   uint16_t* C, int64_t ldc, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  if (fmt == 0) return run<0>(A, lda, M, codes, scales, gs, N, K, C, ldc, stream);
  if (fmt == 1) return run<1>(A, lda, M, codes, scales, gs, N, K, C, ldc, stream);
  if (fmt == 4) return run<4>(A, lda, M, codes, scales, gs, N, K, C, ldc, stream);
  return run<2>(A, lda, M, codes, scales, gs, N, K, C, ldc, stream);
}

hipError_t launch_gemm_w4a16_tiled_qout(int w_fmt, int out_fmt, const uint8_t* codes, const void* scales,
                                        const float* gs, int64_t N, int64_t K, const uint16_t* A, int64_t lda,
                                        int64_t M, const QOut& qo, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  if (out_fmt == kOutMxfp4) return run_qout<kOutMxfp4>(w_fmt, A, lda, M, codes, scales, gs, N, K, qo, stream);
  return run_qout<kOutNvfp4>(w_fmt, A, lda, M, codes, scales, gs, N, K, qo, stream);
}

}  // namespace q4
