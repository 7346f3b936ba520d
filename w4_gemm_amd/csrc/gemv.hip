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
//     lane (n = l%16, g = l/16) takes the 16 bytes holding 32 consecutive
//     codes of row n -- exactly one MXFP4 block, two NVFP4 blocks, a quarter
//     INT4 group -- and feeds them to four consecutive steps; x is read for
//     the same 32 k.  So 128 k (a super-chunk) cost one 16-byte code load per
//     lane.  In the tiled layout (include/q4.h) that load is one contiguous
//     kilobyte per wave; in the row-major layout it is 64 bytes of each of 16
//     rows.
//   * each wave owns one tile of 16 rows and walks the whole K in steps of
//     4 super-chunks (512 k: 4 KB of codes and one 4- or 8-byte scale word
//     per lane in the tiled layout).  The tiles of a workgroup's 4 or 8
//     waves are spread over the matrix (tile = wave * workgroups +
//     workgroup).
//   * x is staged in LDS once per step by the whole workgroup (BT rows,
//     double-buffered) and shared by its waves.  In each step the x loads of
//     two steps ahead are issued first, then the code loads of the next step
//     (non-temporal: the weights are streamed once), then the current step's
//     math runs, and only then are the next step's x values -- loaded a step
//     earlier -- written to LDS: loads complete in order, so by then they
//     have landed, and one step of weights is always in flight.  (Loading x
//     only one step ahead left its L2 latency exposed at B = 16: 21.4-22.7
//     against 20.1-20.3 us on the 28672 x 8192 MXFP4 weight.)  The per-step
//     barrier keeps a workgroup's waves in lockstep, which measured faster
//     than letting them drift.
//   * the loop bodies issue their loads unconditionally (the tail steps are
//     peeled, out-of-range x pieces are clamped and zeroed, surplus pieces go
//     to a spare LDS slot) so the compiler's wait counts stay exact and the
//     prefetched loads stay in flight across the math.
//   * two accumulators (even / odd super-chunks) halve the dependent
//     matrix-core chain; they are summed once at the end.
#include "q4_launch.h"
#include "q4_layout.h"
#include "q4_mma.h"

namespace q4 {
namespace {

constexpr int kSCS = 4;              // super-chunks per step
constexpr int kStepK = kSCS * 128;   // k per step

// Registers of one step of one wave: the codes of its 4 super-chunks and the
// raw scale words (row-major: one per super-chunk; tiled: one q group).
template <int FMT, int LAYOUT>
struct StepFrag {
  static constexpr int NSW = LAYOUT == kLayoutRows ? kSCS : (FMT == 1 ? kSCS / 4 : FMT == 4 ? kSCS : kSCS / 2);
  u32x4_t w[kSCS];
  uint32_t sw[NSW];
};

// Row-major scales of one step of one row, loaded whole: 8 bytes (INT4),
// 16 (MXFP4, INT4 with a zero point) or 32 (NVFP4).
struct StepScales {
  u32x4_t v[2];
};

// One wave streaming the codes and scales of one 16-row tile.  SV (row-major
// only): the scales come as whole steps of the row in vector loads issued
// two steps ahead (StepScales), not with the codes.
template <int FMT, int LAYOUT, bool SV = false>
struct TileStream {
  const uint8_t* wbase;  // this lane's code bytes of super-chunk 0
  int64_t wstep;         // bytes between super-chunks
  const uint8_t* sbase;  // this lane's scales
  const uint8_t* srow;   // row-major: the row's scales
  int nsc;               // super-chunks in K
  int nq;                // q groups in K (tiled)
  int grp;               // lane / 16

  TileStream() = default;
  __device__ TileStream(const uint8_t* codes, const void* scales, int tile, int N, int K, int lane) {
    const int col = lane & 15;
    grp = lane >> 4;
    nsc = K >> 7;
    nq = K >> 9;
    if constexpr (LAYOUT == kLayoutRows) {
      const int n = min(tile * 16 + col, N - 1);
      wbase = codes + (int64_t)n * (K >> 1) + grp * 16;
      wstep = 64;
      srow = reinterpret_cast<const uint8_t*>(scales) +
             (int64_t)n * (K / FmtTraits<FMT>::G) * (FMT == 0 ? 2 : FMT == 4 ? 4 : 1);
      sbase = srow;
      if constexpr (FMT == 1) sbase += grp;        // the lane's block in a super-chunk
      if constexpr (FMT == 2) sbase += 2 * grp;    // the lane's two 16-blocks
    } else {
      const int64_t S = nsc, Q = nq;
      wbase = codes + (int64_t)tile * S * 1024 + lane * 16;
      wstep = 1024;
      if constexpr (FMT == 0)
        sbase = reinterpret_cast<const uint8_t*>(scales) + ((int64_t)tile * Q * 16 + col) * 8;
      else if constexpr (FMT == 4)
        sbase = reinterpret_cast<const uint8_t*>(scales) + ((int64_t)tile * Q * 16 + col) * 16;
      else if constexpr (FMT == 1)
        sbase = reinterpret_cast<const uint8_t*>(scales) + ((int64_t)tile * Q * 64 + lane) * 4;
      else
        sbase = reinterpret_cast<const uint8_t*>(scales) + ((int64_t)tile * Q * 64 + lane) * 8;
    }
  }

  // SV: the row's scales of step st (clamped to the last step; K % 512 == 0
  // and the rows' scale runs aligned, checked at launch).
  __device__ __forceinline__ void load_scales(StepScales& q, int st) const {
    const int stc = min(st, (nsc >> 2) - 1);
    if constexpr (FMT == 0) {
      const uint2 v = *reinterpret_cast<const uint2*>(srow + (int64_t)stc * 8);
      q.v[0] = u32x4_t{v.x, v.y, 0u, 0u};
    } else if constexpr (FMT == 2) {
      q.v[0] = *reinterpret_cast<const u32x4_t*>(srow + (int64_t)stc * 32);
      q.v[1] = *reinterpret_cast<const u32x4_t*>(srow + (int64_t)stc * 32 + 16);
    } else {
      q.v[0] = *reinterpret_cast<const u32x4_t*>(srow + (int64_t)stc * 16);
    }
  }
  // ... and this lane's words of them, as load() would have read them
  __device__ __forceinline__ void take_scales(StepFrag<FMT, LAYOUT>& f, const StepScales& q) const {
#pragma unroll
    for (int c = 0; c < kSCS; ++c) {
      if constexpr (FMT == 0) f.sw[c] = (q.v[0][c >> 1] >> (16 * (c & 1))) & 0xFFFFu;
      else if constexpr (FMT == 4) f.sw[c] = q.v[0][c];
      else if constexpr (FMT == 1) f.sw[c] = (q.v[0][c] >> (8 * grp)) & 0xFFu;
      else {  // word 2c + grp/2 of the 32 bytes (c is known at compile time, grp is not)
        const u32x4_t& h = q.v[c >> 1];
        const uint32_t wv = (grp >> 1) ? h[2 * (c & 1) + 1] : h[2 * (c & 1)];
        f.sw[c] = (wv >> (16 * (grp & 1))) & 0xFFFFu;
      }
    }
  }

  // Loads of step st (super-chunks past K are clamped to the last one).
  __device__ __forceinline__ void load(StepFrag<FMT, LAYOUT>& f, int st) const {
#pragma unroll
    for (int c = 0; c < kSCS; ++c) {
      const int sc = min(st * kSCS + c, nsc - 1);
      f.w[c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(wbase + sc * wstep));
      if constexpr (LAYOUT == kLayoutRows && !SV) {
        if constexpr (FMT == 0) f.sw[c] = reinterpret_cast<const uint16_t*>(sbase)[sc];
        else if constexpr (FMT == 4) f.sw[c] = reinterpret_cast<const uint32_t*>(sbase)[sc];
        else if constexpr (FMT == 1) f.sw[c] = sbase[sc * 4];
        else f.sw[c] = *reinterpret_cast<const uint16_t*>(sbase + sc * 8);
      }
    }
    if constexpr (LAYOUT == kLayoutTiled) {
#pragma unroll
      for (int h = 0; h < kSCS / 4; ++h) {  // the step's q groups
        const int q = min((kSCS / 4) * st + h, nq - 1);
        if constexpr (FMT == 1) {
          f.sw[h] = reinterpret_cast<const uint32_t*>(sbase)[q * 64];
        } else if constexpr (FMT == 4) {  // four 32-bit words per row and q group
          const u32x4_t v = *reinterpret_cast<const u32x4_t*>(sbase + (int64_t)q * 256);
          f.sw[4 * h] = v[0];
          f.sw[4 * h + 1] = v[1];
          f.sw[4 * h + 2] = v[2];
          f.sw[4 * h + 3] = v[3];
        } else {
          const int stride = FMT == 0 ? 16 * 8 : 64 * 8;  // bytes per q group
          const uint2 v = *reinterpret_cast<const uint2*>(sbase + (int64_t)q * stride);
          f.sw[2 * h] = v.x;
          f.sw[2 * h + 1] = v.y;
        }
      }
    }
  }
};

// Scale bits of super-chunk c of a step for this lane: MXFP4 E8M0 byte;
// NVFP4 the two E4M3 bytes of the lane's 32 k (first block low); INT4 fp16.
template <int FMT, int LAYOUT>
__device__ __forceinline__ uint32_t step_scale(const StepFrag<FMT, LAYOUT>& f, int c) {
  if constexpr (LAYOUT == kLayoutRows || FMT == 4) return f.sw[c];
  else if constexpr (FMT == 1) return (f.sw[c >> 2] >> (8 * (c & 3))) & 0xFFu;
  else return (f.sw[c >> 1] >> (16 * (c & 1))) & 0xFFFFu;
}

// INT4 with or without a zero point.  A 128-wide group is one super-chunk,
// so the four matrix steps of a super-chunk share one scale (and zero
// point) per output column n, and the scale can be applied after them: the
// steps multiply x (staged in LDS in the order of dq8_int4_biased) by the
// exact bf16 values 128 + q + 8, a fifth product of x with ones gives the
// group's sum X of x per batch row, and the group adds
//   s * (P - (136 + z) * X) = s * sum_k x_k (q_k - z)
// to the fp32 accumulator.  The products are exact; the only roundings are
// fp32 sums (about 2^-17 of sum |x w'| here, against 2^-9 when w' is first
// rounded to bf16), and the VALU work per code drops from about three
// instructions to one.
template <int FMT, int LAYOUT, int TPW>
__device__ __forceinline__ void step_math_int4(const StepFrag<FMT, LAYOUT> (&f)[TPW], const uint16_t* xrow,
                                               f32x4_t (&acc)[TPW][2]) {
  const bf16x8_t ones = as_bf16x8(u32x4_t{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
#pragma unroll
  for (int c = 0; c < kSCS; ++c) {
    f32x4_t xsum = {0.0f, 0.0f, 0.0f, 0.0f};
    f32x4_t p[TPW];
#pragma unroll
    for (int t = 0; t < TPW; ++t) p[t] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const u32x4_t xv = *reinterpret_cast<const u32x4_t*>(xrow + c * 128 + 8 * i);
      xsum = mma16x16x32(as_bf16x8(xv), ones, xsum);
#pragma unroll
      for (int t = 0; t < TPW; ++t) p[t] = mma16x16x32(as_bf16x8(xv), dq8_int4_biased(f[t].w[c][i]), p[t]);
    }
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const uint32_t sb = step_scale<FMT, LAYOUT>(f[t], c);
      const float s = fp16_value(sb & 0xFFFFu);
      const float kz = FMT == 4 ? -(float)(136 + (int)(int8_t)((sb >> 16) & 0xFFu)) : -136.0f;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        acc[t][c & 1][r] = __builtin_fmaf(s, __builtin_fmaf(kz, xsum[r], p[t][r]), acc[t][c & 1][r]);
    }
  }
}

// MXFP4 / NVFP4: dequantize one step of TPW tiles to bf16 and multiply them
// by x read from LDS at xrow (this lane's batch row, already offset to the
// step and to the lane's 32 k; a row of zeros for lanes past the batch);
// each x fragment feeds every tile.
template <int FMT, int LAYOUT, int TPW>
__device__ __forceinline__ void step_math_fp4(const StepFrag<FMT, LAYOUT> (&f)[TPW], const uint16_t* xrow,
                                              float gs, f32x4_t (&acc)[TPW][2]) {
#pragma unroll
  for (int c = 0; c < kSCS; ++c) {
    uint32_t sb[TPW];
#pragma unroll
    for (int t = 0; t < TPW; ++t) sb[t] = step_scale<FMT, LAYOUT>(f[t], c);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const u32x4_t xv = *reinterpret_cast<const u32x4_t*>(xrow + c * 128 + 8 * i);
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        bf16x8_t wb;
        if constexpr (FMT == 1) {
          wb = dq8_e2m1(f[t].w[c][i], e8m0_value(sb[t]));
        } else {
          const uint32_t e = (i < 2) ? (sb[t] & 0xFFu) : (sb[t] >> 8);
          wb = dq8_e2m1_mul(f[t].w[c][i], e4m3_value(e) * gs);
        }
        acc[t][c & 1] = mma16x16x32(as_bf16x8(xv), wb, acc[t][c & 1]);
      }
    }
  }
}

template <int FMT, int LAYOUT, int TPW>
__device__ __forceinline__ void step_math(const StepFrag<FMT, LAYOUT> (&f)[TPW], const uint16_t* xrow,
                                          float gs, f32x4_t (&acc)[TPW][2]) {
  if constexpr (FMT == 0 || FMT == 4) step_math_int4<FMT, LAYOUT, TPW>(f, xrow, acc);
  else step_math_fp4<FMT, LAYOUT, TPW>(f, xrow, gs, acc);
}

// lane l, register r of the accumulator holds (b = 4(l/16) + r, n = l%16)
__device__ __forceinline__ void store_y(f32x4_t acc, int tile, int ntiles, int N, int B, int lane,
                                        uint16_t* y, int64_t ldy) {
  const int n = tile * 16 + (lane & 15);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int b = 4 * (lane >> 4) + r;
    if (b < B && n < N && tile < ntiles) y[(int64_t)b * ldy + n] = (uint16_t)f32_to_bf16_rne(acc[r]);
  }
}

// x staged per step: [2][BT][kStepK + 8] bf16, one spare 16-byte slot, and
// one row of kStepK zeros that the lanes past the batch read (the matrix
// core always takes 16 rows of x).  Each wave owns TPW adjacent row tiles.
template <int FMT, int LAYOUT, int BT, int TPW, int WAVES, bool SV>
__global__ void __launch_bounds__(WAVES * 64)
gemv_kernel(const uint8_t* __restrict__ codes, const void* __restrict__ scales,
            const float* __restrict__ gs_ptr, int N, int K,
            const uint16_t* __restrict__ x, int64_t ldx, int B,
            uint16_t* __restrict__ y, int64_t ldy) {
  constexpr int XROW = kStepK + 8;
  constexpr int XPIECES = BT * kStepK / 8;                  // 16-byte pieces per step
  constexpr int XPER = (XPIECES + 64 * WAVES - 1) / (64 * WAVES);  // per thread
  extern __shared__ __attribute__((aligned(16))) uint16_t xs_raw[];
  auto xs = reinterpret_cast<uint16_t(*)[BT][XROW]>(xs_raw);
  constexpr int W = WAVES;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int ntiles = (N + 15) >> 4;
  const int tile = (wave * gridDim.x + blockIdx.x) * TPW;  // first of the wave's tiles
  const int nst = (K + kStepK - 1) / kStepK;

  // Staging without branches: out-of-range pieces load a clamped address and
  // are zeroed when written to LDS (not at the load: using a loaded value
  // right away would make the wave wait for it); surplus pieces go to the
  // spare slot.  This keeps the compiler's count of outstanding loads exact.
  auto piece = [&](int j) { return min(tid + j * W * 64, XPIECES - 1); };
  auto load_x = [&](u32x4_t (&xr)[XPER], int st) {
#pragma unroll
    for (int j = 0; j < XPER; ++j) {
      const int p = piece(j);
      const int b = p / (kStepK / 8);
      const int k = st * kStepK + (p % (kStepK / 8)) * 8;
      xr[j] = *reinterpret_cast<const u32x4_t*>(x + (int64_t)min(b, B - 1) * ldx + min(k, K - 8));
    }
  };
  auto store_x = [&](const u32x4_t (&xr)[XPER], int buf, int st) {
#pragma unroll
    for (int j = 0; j < XPER; ++j) {
      const int p = tid + j * W * 64;
      const int pc = piece(j);
      const bool ok = pc / (kStepK / 8) < B && st * kStepK + (pc % (kStepK / 8)) * 8 < K;
      uint16_t* dst = p < XPIECES ? &xs[buf][p / (kStepK / 8)][(p % (kStepK / 8)) * 8]
                                  : &xs_raw[2 * BT * XROW];
      const u32x4_t v = (FMT == 0 || FMT == 4) ? x8_int4_order(xr[j]) : xr[j];
      *reinterpret_cast<u32x4_t*>(dst) = ok ? v : u32x4_t{0u, 0u, 0u, 0u};
    }
  };

  TileStream<FMT, LAYOUT, SV> ts[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t)
    ts[t] = TileStream<FMT, LAYOUT, SV>(codes, scales, min(tile + t, ntiles - 1), N, K, lane);
  const float gs = (FMT == 2) ? *gs_ptr : 0.0f;
  // the lane's x row: its batch row in the current buffer, or the zero row
  uint16_t* const xzero = &xs_raw[2 * BT * XROW + 8];
  if (tid < kStepK / 8) *reinterpret_cast<u32x4_t*>(xzero + 8 * tid) = u32x4_t{0u, 0u, 0u, 0u};
  const bool xlane = col < BT;
  const int xoff = col * XROW + grp * 32;
  auto xrow = [&](int buf) -> const uint16_t* {
    return xlane ? &xs[buf][0][0] + xoff : xzero + grp * 32;
  };
  f32x4_t acc[TPW][2];
#pragma unroll
  for (int t = 0; t < TPW; ++t) acc[t][0] = acc[t][1] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  auto load_w = [&](StepFrag<FMT, LAYOUT> (&f)[TPW], int st) {
#pragma unroll
    for (int t = 0; t < TPW; ++t) ts[t].load(f[t], st);
  };

  // two weight buffers; the x loads of step st+2 are issued before the code
  // loads of step st+1
  StepFrag<FMT, LAYOUT> fa[TPW], fb[TPW];
  u32x4_t xr[XPER];
  // Issue order is pinned (scheduling barriers): the compiler would
  // otherwise sink the next steps' loads below the current step's math to
  // save registers -- and then wait for all of them before storing x.
  // SV: the row scales of steps st and st+1 in two sets (by step parity),
  // loaded two steps ahead and taken into the step's fragments just before
  // that step's loads are issued
  StepScales sq[2][TPW];
  auto load_s = [&](int set, int sst) {
    if constexpr (SV) {
#pragma unroll
      for (int t = 0; t < TPW; ++t) ts[t].load_scales(sq[set][t], sst);
    }
  };
  auto take_s = [&](StepFrag<FMT, LAYOUT> (&f)[TPW], int set) {
    if constexpr (SV) {
#pragma unroll
      for (int t = 0; t < TPW; ++t) ts[t].take_scales(f[t], sq[set][t]);
    }
  };
  auto prefetch = [&](u32x4_t (&xd)[XPER], int xst, StepFrag<FMT, LAYOUT> (&f)[TPW], int wst, int sset, int sst) {
    __builtin_amdgcn_sched_barrier(0);
    load_x(xd, xst);
    __builtin_amdgcn_sched_barrier(0);
    load_w(f, wst);
    __builtin_amdgcn_sched_barrier(0);
    load_s(sset, sst);
    __builtin_amdgcn_sched_barrier(0);
  };
  // x is loaded two steps ahead (two register sets, xr and xq): the values
  // written to LDS after step st's math were loaded during step st-1, before
  // the weights that step st's math already waited for (loads complete in
  // order), so the write never waits; weights are loaded one step ahead.
  u32x4_t xq[XPER];
  load_s(0, 0);
  load_s(1, 1);
  load_x(xr, 0);
  load_x(xq, 1);
  load_w(fa, 0);
  store_x(xr, 0, 0);
  __syncthreads();
  int st = 0;
  for (; st + 2 < nst; st += 2) {
    take_s(fa, 0);
    prefetch(xr, st + 2, fb, st + 1, 0, st + 2);
    step_math<FMT, LAYOUT, TPW>(fa, xrow(st & 1), gs, acc);
    store_x(xq, (st + 1) & 1, st + 1);
    __syncthreads();
    take_s(fb, 1);
    prefetch(xq, st + 3, fa, st + 2, 1, st + 3);
    step_math<FMT, LAYOUT, TPW>(fb, xrow((st + 1) & 1), gs, acc);
    store_x(xr, st & 1, st + 2);
    __syncthreads();
  }
  take_s(fa, 0);
  if (st + 1 < nst) {  // two steps left (xq holds step st+1)
    load_w(fb, st + 1);
    step_math<FMT, LAYOUT, TPW>(fa, xrow(st & 1), gs, acc);
    store_x(xq, (st + 1) & 1, st + 1);
    __syncthreads();
    take_s(fb, 1);
    step_math<FMT, LAYOUT, TPW>(fb, xrow((st + 1) & 1), gs, acc);
  } else {             // one step left
    step_math<FMT, LAYOUT, TPW>(fa, xrow(st & 1), gs, acc);
  }

#pragma unroll
  for (int t = 0; t < TPW; ++t) store_y(acc[t][0] + acc[t][1], tile + t, ntiles, N, B, lane, y, ldy);
}

// Launch shape (measured on the 28672 x 8192 decode GEMV): one tile per
// wave and 8 waves per workgroup -- two waves per SIMD hide the x and
// weight load latencies that a single wave per SIMD exposes -- except INT4
// at B = 1, which ran ~4% faster with 4 waves.
template <int FMT, int LAYOUT, int BT, int TPW = 1, int WAVES = (BT == 1 && (FMT == 0 || FMT == 4)) ? 4 : 8>
hipError_t run(const uint8_t* codes, const void* scales, const float* gs, int64_t N, int64_t K,
               const uint16_t* x, int64_t ldx, int64_t B, uint16_t* y, int64_t ldy,
               hipStream_t stream) {
  const int64_t ntiles = (N + 15) / 16;
  const int64_t nwaves = (ntiles + TPW - 1) / TPW;
  const unsigned grid = (unsigned)((nwaves + WAVES - 1) / WAVES);
  const size_t lds = (2ull * BT * (kStepK + 8) + 8 + kStepK) * sizeof(uint16_t);  // + spare slot, zero row
  // Row-major: the scales of a step of a row in one or two vector loads,
  // issued two steps ahead, when every step is whole (K % 512 == 0) and the
  // rows' scale runs are aligned to the vector (8 bytes INT4, else 16).  The
  // per-super-chunk loads, one step ahead, left the row-major GEMV waiting
  // on them: 38.5 -> 30.8 us (MXFP4, B = 1) on the 28672 x 8192 weight, all
  // formats 15-20% faster; the same kernel without any scale loads took 27.
  const uintptr_t sa = reinterpret_cast<uintptr_t>(scales);
  if (LAYOUT == kLayoutRows && K % kStepK == 0 && (sa & (FMT == 0 ? 7u : 15u)) == 0)
    gemv_kernel<FMT, LAYOUT, BT, TPW, WAVES, LAYOUT == kLayoutRows><<<grid, WAVES * 64, lds, stream>>>(
        codes, scales, gs, (int)N, (int)K, x, ldx, (int)B, y, ldy);
  else
    gemv_kernel<FMT, LAYOUT, BT, TPW, WAVES, false><<<grid, WAVES * 64, lds, stream>>>(
        codes, scales, gs, (int)N, (int)K, x, ldx, (int)B, y, ldy);
  return hipGetLastError();
}

template <int FMT, int LAYOUT>
hipError_t by_batch(const uint8_t* codes, const void* scales, const float* gs, int64_t N,
                    int64_t K, const uint16_t* x, int64_t ldx, int64_t B, uint16_t* y,
                    int64_t ldy, hipStream_t stream) {
  // x rows held in LDS: 1, 4 or 16 (the matrix core always computes 16)
  if (B == 1) return run<FMT, LAYOUT, 1>(codes, scales, gs, N, K, x, ldx, B, y, ldy, stream);
  if (B <= 4) return run<FMT, LAYOUT, 4>(codes, scales, gs, N, K, x, ldx, B, y, ldy, stream);
  return run<FMT, LAYOUT, 16>(codes, scales, gs, N, K, x, ldx, B, y, ldy, stream);
}

template <int FMT>
hipError_t dispatch(int layout, const uint8_t* codes, const void* scales, const float* gs,
                    int64_t N, int64_t K, const uint16_t* x, int64_t ldx, int64_t B, uint16_t* y,
                    int64_t ldy, hipStream_t stream) {
  if (layout == kLayoutTiled)
    return by_batch<FMT, kLayoutTiled>(codes, scales, gs, N, K, x, ldx, B, y, ldy, stream);
  return by_batch<FMT, kLayoutRows>(codes, scales, gs, N, K, x, ldx, B, y, ldy, stream);
}

}  // namespace

hipError_t launch_gemv(int fmt, int layout, const uint8_t* codes, const void* scales,
                       const float* gs, int64_t N, int64_t K, const uint16_t* x, int64_t ldx,
                       int64_t B, uint16_t* y, int64_t ldy, hipStream_t stream) {
  if (N == 0 || B == 0) return hipSuccess;
  if (fmt == 0) return dispatch<0>(layout, codes, scales, gs, N, K, x, ldx, B, y, ldy, stream);
  if (fmt == 1) return dispatch<1>(layout, codes, scales, gs, N, K, x, ldx, B, y, ldy, stream);
  if (fmt == 4) return dispatch<4>(layout, codes, scales, gs, N, K, x, ldx, B, y, ldy, stream);
  return dispatch<2>(layout, codes, scales, gs, N, K, x, ldx, B, y, ldy, stream);
}

}  // namespace q4
