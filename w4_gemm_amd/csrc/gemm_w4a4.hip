// gemm_w4a4.hip -- W4A4 MXFP4 GEMM for operands in the tiled layout:
// C[m][n] = sum_k a'[m][k] w'[n][k], both operands MXFP4 (E2M1 codes, one
// E8M0 scale per 32 along K), fp32 accumulation, bf16 output.
//
// The W4A4 scheme quantizes the activations to FP4 as well and multiplies
// on FP4 matrix cores directly ("Low-bit inference for very large MoE",
// table "Kernels on different hardware", row W4A4).  On gfx950 that is
// v_mfma_scale_f32_16x16x128_f8f6f4: lane l supplies the 32 codes of row
// l%16, k in [32(l/16), +32) -- one MXFP4 block -- and that block's E8M0,
// i.e. exactly lane l's 16 bytes of a 1 KB tile of the tiled layout
// (include/q4.h) and byte 4l+i of its scale group.
//
// Work decomposition:
//   * a workgroup of 8 waves computes a 256 x 256 block of C; wave (wm, wn),
//     wm in 0..1, wn in 0..3, owns 128 x 64 = 8 x 4 matrix-core tiles (128
//     fp32 accumulators per lane, two waves per SIMD).
//   * K advances in stages of one super-chunk (128 k).  A stage needs 16
//     A tiles and 16 W tiles (32 KB); they are copied verbatim into LDS by
//     direct global->LDS loads (global_load_lds_dwordx4: one 1 KB tile per
//     wave instruction, no registers; 4 per wave), three stages ahead, into
//     four buffers (144 KB of LDS with the scales: one workgroup per CU).
//     Scales are copied per group of four stages (16 x 256 B for each
//     operand) into two buffers.  Every fragment read from LDS is one
//     contiguous kilobyte (conflict-free).
//   * ping-pong schedule: the two waves of each SIMD alternate a memory step
//     (the stage's 12 fragment reads into registers) and a matrix step (its
//     32 products), half a stage apart, with a barrier between phases; the
//     matrix core of every SIMD is fed by one wave while the other reads.
//     The rules that make the LDS reuse safe are stated at the loop.
//   * workgroups are ordered so that the 32 running on one XCD cover a
//     4 x 8 block of C (shared A and W panels stay in that XCD's L2).
//   * the weight is the matrix instruction's row operand (C^T = W' A'^T per
//     16x16 tile), so a lane ends with 4 consecutive columns of one row of
//     C: one 8-byte store of bf16, or the quantized-output epilogue
//     (q4_qout.h), which writes C as MXFP4 / NVFP4 codes and scales.
#include "q4_launch.h"
#include "q4_layout.h"
#include "q4_lds.h"
#include "q4_mma.h"
#include "q4_qout.h"

#include <type_traits>

namespace q4 {
namespace {

constexpr int kBM = 16;          // A tiles (of 16 rows) per workgroup
constexpr int kBN = 16;          // W tiles per workgroup
constexpr int kTiles = kBM + kBN;
constexpr int kWaves = 8;
constexpr int kCopies = kTiles / kWaves;  // code tiles each wave copies per stage
constexpr int kCodeBufs = 4;
constexpr size_t kSmemBytes = kCodeBufs * kTiles * 1024 + 2 * kTiles * 256;  // 144 KB

template <int OUT>
__global__ void __launch_bounds__(kWaves * 64)
w4a4_tiled_kernel(const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales,
                  int M, const uint8_t* __restrict__ w_codes,
                  const uint8_t* __restrict__ w_scales, int N, int K,
                  uint16_t* __restrict__ C, int64_t ldc, QOut qo) {
  qout_copy_gs<OUT>(qo);
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
  uint8_t (*cbuf)[kTiles][1024] = reinterpret_cast<uint8_t (*)[kTiles][1024]>(smem);
  uint8_t (*sbuf)[kTiles][256] =
      reinterpret_cast<uint8_t (*)[kTiles][256]>(smem + kCodeBufs * kTiles * 1024);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  const int S = K >> 7, Q = K >> 9;
  const int RTA = (M + 15) >> 4, RTW = (N + 15) >> 4;

  // workgroup -> 256 x 256 block of C: XCD-major, then groups of 4 block rows
  const int TM = (M + 255) >> 8, TN = (N + 255) >> 8, T = TM * TN;
  const int b = blockIdx.x;
  const int lin = (T % 8 == 0) ? (b % 8) * (T / 8) + b / 8 : b;
  const int GM = 4, gsz = GM * TN;
  const int first_m = (lin / gsz) * GM;
  const int gm = min(TM - first_m, GM);
  const int bm = first_m + (lin % gsz) % gm;
  const int bn = (lin % gsz) / gm;

  // the tiles this wave copies each stage: WG tiles kCopies*wave + k
  // (0..15 are A row tiles bm*16 + i, 16..31 are W row tiles bn*16 + i)
  // (wave-uniform bases; the lane offset is added at each copy)
  const uint8_t* csrc[kCopies];
#pragma unroll
  for (int k = 0; k < kCopies; ++k) {
    const int ti = kCopies * wave + k;
    csrc[k] = ti < kBM ? a_codes + (int64_t)min(bm * kBM + ti, RTA - 1) * S * 1024
                       : w_codes + (int64_t)min(bn * kBN + ti - kBM, RTW - 1) * S * 1024;
  }
  // the scale copy of this wave: the 256-byte groups of tiles 4*wave + 0..3
  // (lane -> tile 4*wave + lane/16, bytes 16*(lane%16) ..)
  const int sti = 4 * wave + (lane >> 4);
  const uint8_t* ssrc = (sti < kBM ? a_scales + (int64_t)min(bm * kBM + sti, RTA - 1) * Q * 256
                                   : w_scales + (int64_t)min(bn * kBN + sti - kBM, RTW - 1) * Q * 256) +
                        (lane & 15) * 16;

  // copy group t: the codes of stage t (kCopies per wave), plus the scales
  // of group t/4 when t % 4 == 0 (1 per wave).  Past the end the last stage /
  // group is copied again (into free buffers) so every group issues the same
  // number of copies.
  auto issue_codes = [&](int t) {
    const int st = min(t, S - 1);
    uint8_t(*dst)[1024] = cbuf[t % kCodeBufs];
#pragma unroll
    for (int k = 0; k < kCopies; ++k)
      copy16_to_lds(csrc[k] + (int64_t)st * 1024 + lane * 16, dst[kCopies * wave + k]);
  };
  auto issue_scales = [&](int t) {
    const int q = min(t >> 2, Q - 1);
    copy16_to_lds(ssrc + (int64_t)q * 256, sbuf[(t >> 2) & 1][4 * wave]);
  };

  f32x4_t acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  // Fragments of the stage a wave multiplies, in registers (one set), and
  // the scale words of the current group of four stages (byte s % 4 of each
  // is stage s's E8M0, picked by the matrix instruction's op_sel).
  u32x4_t a[8], w[4];
  uint32_t sa[8], sw[4];
  auto as8 = [](u32x4_t v) { return i32x8_t{(int)v[0], (int)v[1], (int)v[2], (int)v[3], 0, 0, 0, 0}; };
  // memory step of stage u: its fragments (and at J == 0 its group's scale
  // words) from LDS into registers
  auto load = [&](int u, auto jc) {
    constexpr int J = decltype(jc)::value;
    const uint8_t(*cb)[1024] = cbuf[u % kCodeBufs];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) w[jj] = *reinterpret_cast<const u32x4_t*>(&cb[kBM + wn * 4 + jj][lane * 16]);
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] = *reinterpret_cast<const u32x4_t*>(&cb[wm * 8 + i][lane * 16]);
    if constexpr (J == 0) {
      const uint8_t(*sb)[256] = sbuf[(u >> 2) & 1];
#pragma unroll
      for (int i = 0; i < 8; ++i) sa[i] = *reinterpret_cast<const uint32_t*>(&sb[wm * 8 + i][lane * 4]);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) sw[jj] = *reinterpret_cast<const uint32_t*>(&sb[kBM + wn * 4 + jj][lane * 4]);
    }
  };
  // matrix step of stage u: its 32 products, with this wave's part of copy
  // group u+3 issued after the first four (into the buffer of stage u-1)
  auto compute = [&](int u, auto jc) {
    constexpr int J = decltype(jc)::value;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        acc[i][jj] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(as8(w[jj]), as8(a[i]), acc[i][jj], 4, 4,
                                                                      J, sw[jj], J, sa[i]);
      if (i == 0) {
        issue_codes(u + 3);
        if constexpr (J == 1) issue_scales(u + 3);
      }
    }
  };

  // Ping-pong: the waves of each SIMD (w and w+4) alternate a memory step
  // and a matrix step, so that the matrix core of every SIMD is fed by one
  // wave while the other reads its next fragments.  Every wave runs
  //   load(u) -> wait -> barrier -> compute(u) -> barrier
  // and waves 4..7 start one barrier later: in phase 2u waves 0..3 multiply
  // stage u while waves 4..7 load it, in phase 2u+1 the reverse (waves 0..3
  // loading stage u+1).  The wait at the end of load(u): this wave's LDS
  // reads (its next matrix step needs them) and its part of copy group u+1
  // (only group u+2 may still be in flight).  Stage u+1 is then visible after
  // the barrier that ends load(u) of waves 4..7, before any wave reads it;
  // and copy group u+3 (issued in compute(u), phase 2u or 2u+1) overwrites
  // stage u-1's buffer, whose last reads (load(u-1) of waves 4..7, phase
  // 2u-2) completed before the barrier ending that phase.  Copies in group
  // t: kCopies, plus the scale copy when t % 4 == 0.  (Past the last stage
  // the copies repeat the last stage into free buffers and the last loads
  // read them: in bounds, never used.)
  issue_codes(0);
  issue_scales(0);
  issue_codes(1);
  issue_codes(2);
  wait_vmcnt_lgkm0<0>();
  stage_barrier();
  if (wm == 1) stage_barrier();
  auto stage = [&](int u, auto jc) {
    constexpr int J = decltype(jc)::value;
    load(u, jc);
    wait_vmcnt_lgkm0<kCopies + (J == 2 ? 1 : 0)>();  // group u+2 carries scales when J == 2
    stage_barrier();
    compute(u, jc);
    stage_barrier();
  };
  // The tiled layout has K % 512 == 0, so S is a multiple of 4.
  using J0 = std::integral_constant<int, 0>;
  using J1 = std::integral_constant<int, 1>;
  using J2 = std::integral_constant<int, 2>;
  using J3 = std::integral_constant<int, 3>;
  for (int s0 = 0; s0 < S; s0 += 4) {
    stage(s0, J0());
    stage(s0 + 1, J1());
    stage(s0 + 2, J2());
    stage(s0 + 3, J3());
  }
  if (wm == 0) stage_barrier();  // every wave has passed the same number of barriers
  wait_vmcnt<0>();

  // lane l, register r of tile (i, jj) holds row 16i + l%16, column
  // 16jj + 4(l/16) + r of the wave's 128 x 64 part
  const int m0 = bm * 256 + wm * 128 + (lane & 15);
  const int nw = bn * 256 + wn * 64;
  if constexpr (OUT != kOutBf16) {
    store_quantized<OUT>(acc, m0, nw, M, N, qo, lane);
  } else {
    const int n0 = nw + 4 * (lane >> 4);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int m = m0 + 16 * i;
      if (m < M) {
        uint16_t* crow = C + (int64_t)m * ldc;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int n = n0 + 16 * jj;
          const f32x4_t v = acc[i][jj];
          if (n + 3 < N) {
            store_bf16x4(crow + n, v[0], v[1], v[2], v[3]);
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (n + r < N) crow[n + r] = (uint16_t)f32_to_bf16_rne(v[r]);
          }
        }
      }
    }
  }
}

}  // namespace

namespace {

template <int OUT>
hipError_t run(const uint8_t* a_codes, const uint8_t* a_scales, int64_t M, const uint8_t* w_codes,
               const uint8_t* w_scales, int64_t N, int64_t K, uint16_t* C, int64_t ldc, const QOut& qo,
               hipStream_t stream) {
  const hipError_t attr = set_max_lds<&w4a4_tiled_kernel<OUT>>(kSmemBytes);
  if (attr != hipSuccess) return attr;
  const int64_t T = ((M + 255) / 256) * ((N + 255) / 256);
  w4a4_tiled_kernel<OUT><<<(unsigned)T, kWaves * 64, kSmemBytes, stream>>>(a_codes, a_scales, (int)M, w_codes,
                                                                   w_scales, (int)N, (int)K, C, ldc, qo);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_w4a4_tiled(const uint8_t* a_codes, const uint8_t* a_scales, int64_t M,
                                  const uint8_t* w_codes, const uint8_t* w_scales, int64_t N,
                                  int64_t K, uint16_t* C, int64_t ldc, hipStream_t stream) {
  return run<kOutBf16>(a_codes, a_scales, M, w_codes, w_scales, N, K, C, ldc, QOut{}, stream);
}

hipError_t launch_gemm_w4a4_tiled_qout(int out_fmt, const uint8_t* a_codes, const uint8_t* a_scales, int64_t M,
                                       const uint8_t* w_codes, const uint8_t* w_scales, int64_t N, int64_t K,
                                       const QOut& qo, hipStream_t stream) {
  if (out_fmt == kOutMxfp4)
    return run<kOutMxfp4>(a_codes, a_scales, M, w_codes, w_scales, N, K, nullptr, 0, qo, stream);
  return run<kOutNvfp4>(a_codes, a_scales, M, w_codes, w_scales, N, K, nullptr, 0, qo, stream);
}

}  // namespace q4
