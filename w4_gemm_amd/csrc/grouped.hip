// grouped.hip -- grouped per-expert W4A16 GEMM (MoE) for expert weights in
// the tiled layout: for every expert e and each routed row p in
// [offsets[e], offsets[e+1]): C[p][n] = sum_k a[gather[p]][k] w'_e[n][k].
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
//   * a workgroup of 8 waves covers 512 weight rows of one expert (grid.y =
//     expert); wave w streams four adjacent 16-row tiles over the whole K,
//     so every activation fragment read from LDS feeds four matrix
//     instructions (fragment traffic into registers, not HBM, was what held
//     the first version back).
//   * the expert's routed rows are taken in chunks of 48 (three batch tiles
//     of 16; a chunk with fewer rows skips the empty batch tiles -- the MoE
//     workload has 17..46 rows per expert, one chunk each).
//   * K advances in steps of 256 (2 super-chunks): the chunk's activation
//     rows for the step (48 x 256 bf16) are gathered into LDS by the whole
//     workgroup (two buffers), and each wave's weight codes and scales for
//     the next step are loaded into registers while the current step is
//     multiplied -- 8 KB in flight per wave.  Issue order is pinned (next x,
//     next weights, then math) so the x wait never waits for the weights.
//   * matrix step i of a super-chunk uses codes 8i..8i+8 of every lane of a
//     weight tile (k = 32g + 8i + [0,8) for lane 16g + n); the activation
//     fragment is read for the same k.  Weights are the row operand of
//     v_mfma_f32_16x16x32_bf16, so a lane ends with 4 consecutive columns of
//     one routed row: 8-byte stores.
//   * rows whose gather index is outside [0, T) are staged as zeros and so
//     produce zero output rows.
#include "q4_launch.h"
#include "q4_layout.h"
#include "q4_mma.h"

namespace q4 {
namespace {

constexpr int kWaves = 8;
constexpr int kTPW = 4;                 // weight tiles per wave
constexpr int kRows = 48;               // routed rows per chunk
constexpr int kSCS = 2;                 // super-chunks per step
constexpr int kStepK = 128 * kSCS;      // 256
constexpr int kXRow = kStepK + 8;       // padded LDS row (bf16)
constexpr int kBT = kRows / 16;                         // batch tiles per chunk
constexpr int kPPR = kStepK / 8;                        // 16-byte pieces per row and step
constexpr int kXPer = kRows * kPPR / (kWaves * 64);     // pieces per thread and step
constexpr int kRowStride = kWaves * 64 / kPPR;          // rows between a thread's pieces
constexpr size_t kSmemBytes = 2ull * kRows * kXRow * 2;
static_assert(kSCS == 1 || kSCS == 2 || kSCS == 4, "a step lies within one scale group");
static_assert(kRows % 16 == 0 && kRows * kPPR % (kWaves * 64) == 0, "staging split");

// codes and raw scale words of one step of one weight tile
template <int FMT>
struct StepW {
  static constexpr int NSW = FMT == 1 ? 1 : 2;  // words per tile and scale group
  u32x4_t w[kSCS];
  uint32_t sw[NSW];
};

template <int FMT>
__global__ void __launch_bounds__(kWaves * 64)
grouped_tiled_kernel(const uint16_t* __restrict__ A, int64_t lda, int T,
                     const int32_t* __restrict__ gather, const int32_t* __restrict__ offsets, int P,
                     const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                     const float* __restrict__ gs_ptr, int N, int K, uint16_t* __restrict__ C,
                     int64_t ldc) {
  extern __shared__ __attribute__((aligned(16))) uint16_t xs_raw[];
  auto xs = reinterpret_cast<uint16_t(*)[kRows][kXRow]>(xs_raw);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int e = blockIdx.y;
  const int r0 = min(max(offsets[e], 0), P);
  const int r1 = min(max(offsets[e + 1], r0), P);
  if (r0 >= r1) return;  // whole workgroup, before any barrier

  const int NT = N >> 4;                     // weight tiles per expert (N % 16 == 0)
  const int S = K >> 7, Q = K >> 9, nst = K / kStepK;
  const int tile0 = blockIdx.x * (kWaves * kTPW) + wave * kTPW;  // within the expert
  const float gs = (FMT == 2) ? *gs_ptr : 0.0f;

  // this lane's code bytes and scale words of super-chunk 0 / scale group 0
  const uint8_t* wsrc[kTPW];
  const uint8_t* ssrc[kTPW];
#pragma unroll
  for (int t = 0; t < kTPW; ++t) {
    const int64_t gt = (int64_t)e * NT + min(tile0 + t, NT - 1);
    wsrc[t] = codes + gt * S * 1024 + lane * 16;
    if constexpr (FMT == 0) ssrc[t] = scales + (gt * Q * 16 + (lane & 15)) * 8;
    else if constexpr (FMT == 1) ssrc[t] = scales + (gt * Q * 64 + lane) * 4;
    else ssrc[t] = scales + (gt * Q * 64 + lane) * 8;
  }
  // step st covers super-chunks kSCS*st .. +kSCS, all in scale group
  // kSCS*st/4 (the codes' position in the group: (kSCS*st) % 4 + c)
  auto load_w = [&](StepW<FMT> (&f)[kTPW], int st) {
    const int q = min(kSCS * st / 4, Q - 1);
#pragma unroll
    for (int t = 0; t < kTPW; ++t) {
#pragma unroll
      for (int c = 0; c < kSCS; ++c)
        f[t].w[c] = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4_t*>(wsrc[t] + (int64_t)min(kSCS * st + c, S - 1) * 1024));
      if constexpr (FMT == 1) {
        f[t].sw[0] = *reinterpret_cast<const uint32_t*>(ssrc[t] + (int64_t)q * 256);
      } else {
        const uint2 v = *reinterpret_cast<const uint2*>(ssrc[t] + (int64_t)q * (FMT == 0 ? 128 : 512));
        f[t].sw[0] = v.x;
        f[t].sw[1] = v.y;
      }
    }
  };

  for (int c0 = r0; c0 < r1; c0 += kRows) {
    const int nb = min(kBT, (r1 - c0 + 15) >> 4);  // batch tiles with rows
    // the rows this thread stages: row tid/kPPR + kRowStride*j, source or -1
    const int trow = tid / kPPR;
    int srow[kXPer];
#pragma unroll
    for (int j = 0; j < kXPer; ++j) {
      const int p = c0 + trow + kRowStride * j;
      const int g = p < r1 ? gather[p] : -1;
      srow[j] = (g >= 0 && g < T) ? g : -1;
    }
    const int xk = (tid % kPPR) * 8;  // this thread's 8 k within a step
    u32x4_t xr[kXPer];
    auto load_x = [&](int st) {
      const int k = min(st * kStepK + xk, K - 8);
#pragma unroll
      for (int j = 0; j < kXPer; ++j)
        xr[j] = *reinterpret_cast<const u32x4_t*>(A + (int64_t)max(srow[j], 0) * lda + k);
    };
    auto store_x = [&](int buf) {
#pragma unroll
      for (int j = 0; j < kXPer; ++j)
        *reinterpret_cast<u32x4_t*>(&xs[buf][trow + kRowStride * j][xk]) =
            srow[j] >= 0 ? xr[j] : u32x4_t{0u, 0u, 0u, 0u};
    };

    f32x4_t acc[kTPW][kBT];
#pragma unroll
    for (int t = 0; t < kTPW; ++t)
#pragma unroll
      for (int bt = 0; bt < kBT; ++bt) acc[t][bt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

    auto step_math = [&](const StepW<FMT> (&f)[kTPW], int buf, int st) {
      const uint16_t* xb = &xs[buf][lane & 15][32 * (lane >> 4)];
      const int cq0 = (kSCS * st) & 3;  // position of super-chunk 0 of the step in its group
#pragma unroll
      for (int c = 0; c < kSCS; ++c) {
        const int cq = cq0 + c;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          bf16x8_t wb[kTPW];
#pragma unroll
          for (int t = 0; t < kTPW; ++t) {
            if constexpr (FMT == 0) {
              const uint32_t h = (f[t].sw[cq >> 1] >> (16 * (cq & 1))) & 0xFFFFu;
              wb[t] = dq8_int4(f[t].w[c][i], fp16_value(h));
            } else if constexpr (FMT == 1) {
              wb[t] = dq8_e2m1(f[t].w[c][i], e8m0_value((f[t].sw[0] >> (8 * cq)) & 0xFFu));
            } else {
              const uint32_t sb = (f[t].sw[cq >> 1] >> (16 * (cq & 1) + 8 * (i >> 1))) & 0xFFu;
              wb[t] = dq8_e2m1_mul(f[t].w[c][i], e4m3_value(sb) * gs);
            }
          }
#pragma unroll
          for (int bt = 0; bt < kBT; ++bt) {
            if (bt < nb) {
              const bf16x8_t a = as_bf16x8(*reinterpret_cast<const u32x4_t*>(xb + bt * 16 * kXRow + c * 128 + 8 * i));
#pragma unroll
              for (int t = 0; t < kTPW; ++t) acc[t][bt] = mma16x16x32(wb[t], a, acc[t][bt]);
            }
          }
        }
      }
    };

    // Pinned issue order: next x, then next weights, then the math.
    StepW<FMT> fa[kTPW], fb[kTPW];
    auto prefetch = [&](StepW<FMT> (&f)[kTPW], int st) {
      __builtin_amdgcn_sched_barrier(0);
      load_x(st);
      __builtin_amdgcn_sched_barrier(0);
      load_w(f, st);
      __builtin_amdgcn_sched_barrier(0);
    };
    load_x(0);
    load_w(fa, 0);
    store_x(0);
    __syncthreads();
    int st = 0;
    for (; st + 2 < nst; st += 2) {
      prefetch(fb, st + 1);
      step_math(fa, st & 1, st);
      store_x((st + 1) & 1);
      __syncthreads();
      prefetch(fa, st + 2);
      step_math(fb, (st + 1) & 1, st + 1);
      store_x(st & 1);
      __syncthreads();
    }
    if (st + 1 < nst) {  // two steps left
      prefetch(fb, st + 1);
      step_math(fa, st & 1, st);
      store_x((st + 1) & 1);
      __syncthreads();
      step_math(fb, (st + 1) & 1, st + 1);
    } else {             // one step left
      step_math(fa, st & 1, st);
    }

    // tile t, batch tile bt: lane l, register q holds C[p][n] with
    // p = c0 + 16bt + l%16 and n = 16(tile0+t) + 4(l/16) + q
#pragma unroll
    for (int t = 0; t < kTPW; ++t) {
      if (tile0 + t < NT) {
        const int n = 16 * (tile0 + t) + 4 * (lane >> 4);
#pragma unroll
        for (int bt = 0; bt < kBT; ++bt) {
          const int p = c0 + 16 * bt + (lane & 15);
          if (bt < nb && p < r1) {
            const f32x4_t v = acc[t][bt];
            *reinterpret_cast<uint2*>(C + (int64_t)p * ldc + n) = make_uint2(pk_bf16(v[0], v[1]), pk_bf16(v[2], v[3]));
          }
        }
      }
    }
    __syncthreads();  // the next chunk reuses the LDS buffers
  }
}

template <int FMT>
hipError_t run(const uint16_t* A, int64_t lda, int64_t T, const int32_t* gather, const int32_t* offsets,
               int32_t E, int64_t P, const uint8_t* codes, const void* scales, const float* gs,
               int64_t N, int64_t K, uint16_t* C, int64_t ldc, hipStream_t stream) {
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&grouped_tiled_kernel<FMT>), hipFuncAttributeMaxDynamicSharedMemorySize,
      (int)kSmemBytes);
  if (attr != hipSuccess) return attr;
  const int64_t NT = N / 16;
  const dim3 grid((unsigned)((NT + kWaves * kTPW - 1) / (kWaves * kTPW)), (unsigned)E);
  grouped_tiled_kernel<FMT><<<grid, kWaves * 64, kSmemBytes, stream>>>(
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
  if (fmt == 0) return run<0>(A, lda, T, gather, offsets, E, P, codes, scales, gs, N, K, C, ldc, stream);
  if (fmt == 1) return run<1>(A, lda, T, gather, offsets, E, P, codes, scales, gs, N, K, C, ldc, stream);
  return run<2>(A, lda, T, gather, offsets, E, P, codes, scales, gs, N, K, C, ldc, stream);
}

}  // namespace q4
