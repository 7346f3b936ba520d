// grouped.hip -- grouped per-expert W4A16 GEMM (MoE) for expert weights in
// the tiled layout: for every expert e and each routed row p in
// [offsets[e], offsets[e+1]): C[p][n] = sum_k a[gather[p]][k] w'_e[n][k]
// (gather == NULL: row p of a).
//
// One low-bit weight matrix per expert with the tokens grouped by expert is
// the MoE case of the W4A16 scheme ("Low-bit inference for very large MoE",
// "A few details" and table "Kernels on different hardware", row W4A16).
// With a few dozen routed rows per expert the work is a batched GEMV: the
// weights are read once and dominate the bytes, so this kernel streams them
// from HBM the way the decode GEMV does and keeps the routed activation rows
// in LDS.
//
// Work decomposition:
//   * a workgroup of 8 waves covers 256 weight rows of one expert (grid.y =
//     expert); wave w owns two adjacent 16-row tiles over the whole K, so
//     every activation fragment read from LDS feeds two matrix instructions.
//     A workgroup needs 74 KB of LDS and ~100 registers per lane, so two
//     run on each CU (16 waves) and one's barrier waits overlap the other's
//     streaming.
//   * the expert's routed rows are taken in chunks of 48 (three batch tiles
//     of 16; a chunk with fewer rows skips the empty batch tiles -- the MoE
//     workload has 17..46 rows per expert, one chunk each).
//   * K advances in stages of one super-chunk (128 k).  The weight tiles of
//     a stage (16 x 1 KB) are copied verbatim into LDS by direct global->LDS
//     loads (each wave its own two tiles), two stages ahead, into a ring of
//     three buffers; with two workgroups per CU, 64 KB of weights per CU
//     stay in flight without holding registers.  Scale words (one group of
//     four stages) are loaded into registers ahead of their group.  The
//     chunk's activation rows for a stage (48 x 128 bf16) are gathered into
//     LDS through registers by waves 0..5 (two LDS buffers), loaded two
//     stages ahead into two register sets.
//   * one barrier per stage; every wait is an explicit vmcnt count (the
//     stage loop is unrolled by four so each count is a constant).
//   * matrix step i of a super-chunk uses codes 8i..8i+8 of every lane of a
//     weight tile (k = 32g + 8i + [0,8) for lane 16g + n); the activation
//     fragment is read for the same k.  Weights are the row operand of
//     v_mfma_f32_16x16x32_bf16, so a lane ends with 4 consecutive columns of
//     one routed row: 8-byte stores.
//   * a row whose gather index is outside [0, T) is staged from row 0 and its
//     output row written as zeros.
#include "q4_launch.h"
#include "q4_layout.h"
#include "q4_lds.h"
#include "q4_mma.h"

namespace q4 {
namespace {

constexpr int kWaves = 8;
constexpr int kTPW = 2;                    // weight tiles per wave
constexpr int kTiles = kWaves * kTPW;      // 16 tiles = 256 weight rows per workgroup
constexpr int kRows = 48;                  // routed rows per chunk
constexpr int kBT = kRows / 16;            // batch tiles per chunk
constexpr int kWBufs = 3;                  // weight stages in LDS (2 in flight)
constexpr int kXRow = 128 + 8;             // padded LDS row of one stage's activations (bf16)
constexpr int kXThreads = kRows * 16 / 2;  // threads staging activations, 2 pieces each (384)
constexpr size_t kWBytes = (size_t)kWBufs * kTiles * 1024;               // 48 KB
constexpr size_t kSmemBytes = kWBytes + 2ull * kRows * kXRow * 2;        // + 25.5 KB
static_assert(kXThreads % 64 == 0 && kXThreads <= kWaves * 64, "staging split");

// raw scale words of one weight tile for one group of four super-chunks
template <int FMT>
struct ScaleW {
  static constexpr int NSW = FMT == 1 ? 1 : FMT == 4 ? 4 : 2;
  uint32_t w[NSW];
};

// SWIGLU: the expert's weight rows alternate 16-row tiles of W_gate and
// W_up (tile 2j = gate rows 16j.., tile 2j+1 = up rows 16j..), so a wave's
// two tiles are the gate and up rows of the same 16 outputs and the
// epilogue writes h = silu(gate) * up (N/2 columns) instead of both.
template <int FMT, bool SWIGLU>
__global__ void __launch_bounds__(kWaves * 64)
grouped_tiled_kernel(const uint16_t* __restrict__ A, int64_t lda, int T,
                     const int32_t* __restrict__ gather, const int32_t* __restrict__ offsets, int P,
                     const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                     const float* __restrict__ gs_ptr, int N, int K, uint16_t* __restrict__ C,
                     int64_t ldc) {
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
  uint8_t (*wbuf)[kTiles][1024] = reinterpret_cast<uint8_t (*)[kTiles][1024]>(smem);
  auto xs = reinterpret_cast<uint16_t(*)[kRows][kXRow]>(smem + kWBytes);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int e = blockIdx.y;
  const int r0 = min(max(offsets[e], 0), P);
  const int r1 = min(max(offsets[e + 1], r0), P);
  if (r0 >= r1) return;  // whole workgroup, before any barrier

  const int NT = N >> 4;                     // weight tiles per expert (N % 16 == 0)
  const int S = K >> 7, Q = K >> 9;
  const int tile0 = blockIdx.x * kTiles + wave * kTPW;  // within the expert
  const float gs = (FMT == 2) ? *gs_ptr : 0.0f;

  // wave-uniform code base of each of the wave's tiles; per-lane scale words
  const uint8_t* wsrc[kTPW];
  const uint8_t* ssrc[kTPW];
#pragma unroll
  for (int t = 0; t < kTPW; ++t) {
    const int64_t gt = (int64_t)e * NT + min(tile0 + t, NT - 1);
    wsrc[t] = codes + gt * S * 1024;
    if constexpr (FMT == 0) ssrc[t] = scales + (gt * Q * 16 + (lane & 15)) * 8;
    else if constexpr (FMT == 4) ssrc[t] = scales + (gt * Q * 16 + (lane & 15)) * 16;
    else if constexpr (FMT == 1) ssrc[t] = scales + (gt * Q * 64 + lane) * 4;
    else ssrc[t] = scales + (gt * Q * 64 + lane) * 8;
  }
  auto issue_w = [&](int st) {  // stage st (clamped) into ring slot st % kWBufs
    const int sc = min(st, S - 1);
#pragma unroll
    for (int t = 0; t < kTPW; ++t)
      copy16_to_lds(uniform_ptr(wsrc[t] + (int64_t)sc * 1024) + lane * 16, wbuf[st % kWBufs][wave * kTPW + t]);
  };
  ScaleW<FMT> snext[kTPW], scur[kTPW];
  auto issue_s = [&](int q) {
    q = min(q, Q - 1);
#pragma unroll
    for (int t = 0; t < kTPW; ++t) {
      if constexpr (FMT == 1) {
        snext[t].w[0] = *reinterpret_cast<const uint32_t*>(ssrc[t] + (int64_t)q * 256);
      } else if constexpr (FMT == 4) {
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(ssrc[t] + (int64_t)q * 256);
#pragma unroll
        for (int w = 0; w < 4; ++w) snext[t].w[w] = v[w];
      } else {
        const uint2 v = *reinterpret_cast<const uint2*>(ssrc[t] + (int64_t)q * (FMT == 0 ? 128 : 512));
        snext[t].w[0] = v.x;
        snext[t].w[1] = v.y;
      }
    }
  };
  constexpr int kSLoads = kTPW;  // one scale load instruction per tile

  const bool xw = tid < kXThreads;           // waves 0..5 stage activations
  const int xrow = (tid >> 4) % kRows;       // this thread's two rows: xrow, xrow + 24
  const int xk = (tid & 15) * 8;             // its 8 k within a stage

  for (int c0 = r0; c0 < r1; c0 += kRows) {
    const int nb = min(kBT, (r1 - c0 + 15) >> 4);  // batch tiles with rows
    int srow[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int p = c0 + xrow + 24 * j;
      const int g = p < r1 ? (gather ? gather[p] : p) : -1;
      srow[j] = (g >= 0 && g < T) ? g : 0;  // invalid rows staged from row 0, output zeroed
    }
    // x(s) is held in register set s % 2 between its load and its write to
    // LDS buffer s % 2
    u32x4_t xr[2][2];
    auto load_x = [&](int st, auto setc) {
      constexpr int X = decltype(setc)::value;
      if (xw) {
        const int k = min(st, S - 1) * 128 + xk;
#pragma unroll
        for (int j = 0; j < 2; ++j)
          xr[X][j] = *reinterpret_cast<const u32x4_t*>(A + (int64_t)srow[j] * lda + k);
      }
    };
    auto store_x = [&](auto setc) {
      constexpr int X = decltype(setc)::value;
      if (xw) {
#pragma unroll
        for (int j = 0; j < 2; ++j) *reinterpret_cast<u32x4_t*>(&xs[X][xrow + 24 * j][xk]) = xr[X][j];
      }
    };
    using X0 = std::integral_constant<int, 0>;
    using X1 = std::integral_constant<int, 1>;

    f32x4_t acc[kTPW][kBT];
#pragma unroll
    for (int t = 0; t < kTPW; ++t)
#pragma unroll
      for (int bt = 0; bt < kBT; ++bt) acc[t][bt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

    // math of stage st; j = st % 4 is its position in the scale group
    auto stage_math = [&](int st, auto jc) {
      constexpr int j = decltype(jc)::value;
      const uint16_t* xb = &xs[st & 1][lane & 15][32 * (lane >> 4)];
      u32x4_t wv[kTPW];
#pragma unroll
      for (int t = 0; t < kTPW; ++t)
        wv[t] = *reinterpret_cast<const u32x4_t*>(&wbuf[st % kWBufs][wave * kTPW + t][lane * 16]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        bf16x8_t wb[kTPW];
#pragma unroll
        for (int t = 0; t < kTPW; ++t) {
          if constexpr (FMT == 0) {
            const uint32_t h = (scur[t].w[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
            wb[t] = dq8_int4(wv[t][i], fp16_value(h));
          } else if constexpr (FMT == 4) {
            float sc, off;
            int4zp_scale(scur[t].w[j], sc, off);
            wb[t] = dq8_int4_off(wv[t][i], sc, off);
          } else if constexpr (FMT == 1) {
            wb[t] = dq8_e2m1(wv[t][i], e8m0_value((scur[t].w[0] >> (8 * j)) & 0xFFu));
          } else {
            const uint32_t sb = (scur[t].w[j >> 1] >> (16 * (j & 1) + 8 * (i >> 1))) & 0xFFu;
            wb[t] = dq8_e2m1_mul(wv[t][i], e4m3_value(sb) * gs);
          }
        }
#pragma unroll
        for (int bt = 0; bt < kBT; ++bt) {
          if (bt < nb) {
            const bf16x8_t a = as_bf16x8(*reinterpret_cast<const u32x4_t*>(xb + bt * 16 * kXRow + 8 * i));
#pragma unroll
            for (int t = 0; t < kTPW; ++t) acc[t][bt] = mma16x16x32(wb[t], a, acc[t][bt]);
          }
        }
      }
    };

    // Copy plan, per iteration st (J = st % 4), in issue order: the x rows of
    // stage st+2 (two loads per thread of waves 0..5, none in waves 6, 7),
    // the weight DMA of stage st+2 (kTPW per wave), and when J == 2 the
    // scale words of group st/4 + 1 (kSLoads, after W(st+2) = the group's
    // first stage).  Loads complete in order, so each wait below is the
    // number of loads issued after the ones it needs:
    //   * top of iteration st: W(st) -- and at J == 0 the scales issued right
    //     after it -- have landed; x(st+1), W(st+1) (and at J == 3 the scales
    //     after W(st+1)) may be in flight.  x(st) is in LDS (written by its
    //     waves before their wait for lgkmcnt 0, visible after the barrier).
    //   * after the math of stage st: x(st+1) (issued before W(st+1)) has
    //     landed, so its waves write it to LDS; W(st+1), W(st+2) and the
    //     x(st+2) loads stay in flight.
    // Prologue: x(0), W(0), scales(0), x(1), W(1).
    constexpr int kNX = 2;  // x loads per thread of a staging wave
    load_x(0, X0());
    issue_w(0);
    issue_s(0);
    load_x(1, X1());
    issue_w(1);
    if (xw) wait_vmcnt<2 * kTPW + kSLoads + kNX>();  // x(0) landed
    store_x(X0());
    auto iteration = [&](int st, auto jc) {
      constexpr int J = decltype(jc)::value;
      constexpr int SA = J == 3 ? kSLoads : 0;  // scales issued after W(st+1)
      constexpr int SB = J == 2 ? kSLoads : 0;  // scales issued after W(st+2)
      if (xw) wait_vmcnt_lgkm0<kNX + kTPW + SA>();
      else wait_vmcnt_lgkm0<kTPW + SA>();
      stage_barrier();
      if constexpr (J == 0) {
#pragma unroll
        for (int t = 0; t < kTPW; ++t) scur[t] = snext[t];
      }
      __builtin_amdgcn_sched_barrier(0);
      if constexpr ((J & 1) == 0) load_x(st + 2, X0());
      else load_x(st + 2, X1());
      issue_w(st + 2);
      if constexpr (J == 2) issue_s((st >> 2) + 1);
      __builtin_amdgcn_sched_barrier(0);
      stage_math(st, jc);
      if (xw) {
        wait_vmcnt<kTPW + SA + kNX + kTPW + SB>();
        if constexpr ((J & 1) == 0) store_x(X1());
        else store_x(X0());
      }
    };
    using J0 = std::integral_constant<int, 0>;
    using J1 = std::integral_constant<int, 1>;
    using J2 = std::integral_constant<int, 2>;
    using J3 = std::integral_constant<int, 3>;
    // K % 512 == 0 in the tiled layout: S is a multiple of 4
    for (int s0 = 0; s0 < S; s0 += 4) {
      iteration(s0, J0());
      iteration(s0 + 1, J1());
      iteration(s0 + 2, J2());
      iteration(s0 + 3, J3());
    }
    wait_vmcnt<0>();

    // tile t, batch tile bt: lane l, register q holds C[p][n] with
    // p = c0 + 16bt + l%16 and n = 16(tile0+t) + 4(l/16) + q
    if constexpr (SWIGLU) {
      static_assert(kTPW == 2, "a wave holds one gate tile and its up tile");
      if (tile0 + 1 < NT) {
        const int n = 8 * tile0 + 4 * (lane >> 4);  // output column: 16 * (gate tile index) + ...
#pragma unroll
        for (int bt = 0; bt < kBT; ++bt) {
          const int p = c0 + 16 * bt + (lane & 15);
          if (bt < nb && p < r1) {
            const int g = gather ? gather[p] : p;
            f32x4_t v = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
            if (g >= 0 && g < T) {
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const float z = acc[0][bt][q];
                v[q] = z / (1.0f + expf(-z)) * acc[1][bt][q];
              }
            }
            store_bf16x4(C + (int64_t)p * ldc + n, v[0], v[1], v[2], v[3]);
          }
        }
      }
    } else {
#pragma unroll
    for (int t = 0; t < kTPW; ++t) {
      if (tile0 + t < NT) {
        const int n = 16 * (tile0 + t) + 4 * (lane >> 4);
#pragma unroll
        for (int bt = 0; bt < kBT; ++bt) {
          const int p = c0 + 16 * bt + (lane & 15);
          if (bt < nb && p < r1) {
            const int g = gather ? gather[p] : p;
            const f32x4_t v = (g >= 0 && g < T) ? acc[t][bt] : f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
            store_bf16x4(C + (int64_t)p * ldc + n, v[0], v[1], v[2], v[3]);
          }
        }
      }
    }
    }
    stage_barrier();  // the next chunk reuses the LDS buffers
  }
}

template <int FMT, bool SWIGLU>
hipError_t run(const uint16_t* A, int64_t lda, int64_t T, const int32_t* gather, const int32_t* offsets,
               int32_t E, int64_t P, const uint8_t* codes, const void* scales, const float* gs,
               int64_t N, int64_t K, uint16_t* C, int64_t ldc, hipStream_t stream) {
  const hipError_t attr = set_max_lds<&grouped_tiled_kernel<FMT, SWIGLU>>(kSmemBytes);
  if (attr != hipSuccess) return attr;
  const int64_t NT = N / 16;
  const dim3 grid((unsigned)((NT + kWaves * kTPW - 1) / (kWaves * kTPW)), (unsigned)E);
  grouped_tiled_kernel<FMT, SWIGLU><<<grid, kWaves * 64, kSmemBytes, stream>>>(
      A, lda, (int)T, gather, offsets, (int)P, codes, static_cast<const uint8_t*>(scales), gs, (int)N,
      (int)K, C, ldc);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_grouped_tiled(int fmt, const uint16_t* A, int64_t lda, int64_t T, const int32_t* gather,
                                const int32_t* offsets, int32_t E, int64_t P, const uint8_t* codes,
                                const void* scales, const float* gs, int64_t N, int64_t K, uint16_t* C,
                                int64_t ldc, hipStream_t stream) {
  if (E == 0 || N == 0 || P == 0) return hipSuccess;
  if (fmt == 0) return run<0, false>(A, lda, T, gather, offsets, E, P, codes, scales, gs, N, K, C, ldc, stream);
  if (fmt == 1) return run<1, false>(A, lda, T, gather, offsets, E, P, codes, scales, gs, N, K, C, ldc, stream);
  if (fmt == 4) return run<4, false>(A, lda, T, gather, offsets, E, P, codes, scales, gs, N, K, C, ldc, stream);
  return run<2, false>(A, lda, T, gather, offsets, E, P, codes, scales, gs, N, K, C, ldc, stream);
}

hipError_t launch_grouped_tiled_swiglu(int fmt, const uint16_t* A, int64_t lda, int64_t T, const int32_t* gather,
                                       const int32_t* offsets, int32_t E, int64_t P, const uint8_t* codes,
                                       const void* scales, const float* gs, int64_t N2, int64_t K, uint16_t* H,
                                       int64_t ldh, hipStream_t stream) {
  if (E == 0 || N2 == 0 || P == 0) return hipSuccess;
  if (fmt == 0) return run<0, true>(A, lda, T, gather, offsets, E, P, codes, scales, gs, N2, K, H, ldh, stream);
  if (fmt == 1) return run<1, true>(A, lda, T, gather, offsets, E, P, codes, scales, gs, N2, K, H, ldh, stream);
  if (fmt == 4) return run<4, true>(A, lda, T, gather, offsets, E, P, codes, scales, gs, N2, K, H, ldh, stream);
  return run<2, true>(A, lda, T, gather, offsets, E, P, codes, scales, gs, N2, K, H, ldh, stream);
}

}  // namespace q4
