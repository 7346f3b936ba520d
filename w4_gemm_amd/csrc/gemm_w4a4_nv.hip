// gemm_w4a4_nv.hip -- W4A4 GEMM with both operands NVFP4:
// C[m][n] = sum_k a'[m][k] w'[n][k], a' and w' each E2M1 codes times an E4M3
// scale per 16 along K times the operand's own fp32 tensor scale gs; fp32
// accumulation, bf16 output.
//
// W4A4 quantizes the activations to FP4 as well ("Low-bit inference for very
// large MoE", table "Kernels on different hardware", row W4A4); NVFP4 is the
// format with an E4M3 scale per 16 and a tensor scale ("Quantization in
// deployment", cheat sheet and formats.py nvfp4()).  gfx950's block-scaled
// FP4 matrix core takes a power-of-two scale per 32, which cannot carry an
// E4M3 scale per 16, so this kernel uses the fp16 matrix core on exactly
// dequantized operands instead:
//   * a code times its E4M3 block scale has at most 5 significant bits and
//     lies in [2^-10, 2688], so it is exact in fp16 (no subnormals): one
//     v_cvt_scalef32_pk_f16_fp4 per two codes (scale 1.0) and one
//     v_pk_mul_f16 by the block scale per two codes;
//   * fp16 x fp16 products are exact in the fp32 accumulation of
//     v_mfma_f32_16x16x32_f16;
//   * the two tensor scales are common to every product and are applied
//     once, to the fp32 sum: C = bf16((acc * gs_a) * gs_w).
// The result equals sum_k a'_k w'_k up to fp32 summation order and the
// roundings of the tensor-scale products (the per-element dequantized value
// is defined as fp32(code * fp32(E4M3 * gs)), which differs from code *
// E4M3 * gs by at most one fp32 rounding).
//
// Two kernels:
//   * both operands in the tiled layout: a workgroup of 2 x 4 waves computes
//     a 256 x 256 block of C, each wave a 128 x 64 part (8 x 4 tiles of
//     16x16); each matrix step dequantizes 8 A and 4 W fragments (8 codes
//     per lane each) for 32 matrix instructions, two waves per SIMD
//     overlapping one's dequantization with the other's matrix work.  The
//     codes are read from LDS one matrix step at a time (a dword per tile),
//     which keeps the registers within two waves per SIMD.  (4 x 2 waves of
//     64 x 64, 8 fragments per 16 matrix instructions, measured 9.5%
//     slower; 128 x 128 per wave does not fit the registers.)  K advances one
//     super-chunk (128 k) per stage; the stage's 32 code tiles (1 KB each)
//     are copied verbatim into LDS by direct global->LDS loads, two stages
//     ahead, into three buffers, and the E4M3 scales (512 bytes per tile and
//     group of four super-chunks) into two buffers -- the copy scheme of the
//     MXFP4 W4A4 kernel.
//   * any other layout combination: a register-tiled kernel (4 waves, 64 x
//     64 of C per wave) loading each lane's 16 code bytes per super-chunk and
//     its two scale bytes directly.
// Matrix step i of a super-chunk uses codes 8i..8i+8 of every lane (k =
// 32g + 8i + [0,8) for lane 16g + n) of both operands, so both take the same
// k; those eight codes lie in the lane's 16-block i/2.
#include "q4_launch.h"
#include "q4_layout.h"
#include "q4_lds.h"
#include "q4_mma.h"

namespace q4 {
namespace {

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));

// The lane's two E4M3 block scales of one super-chunk (byte 0: its first 16
// k, byte 1: the next 16) -> their fp16 values, exact: the E4M3 exponent and
// mantissa bits placed at bit 7 of an fp16 read as 2^(e-15) (1 + m/8), or as
// the fp16 subnormal m 2^-17 for e = 0; times 2^8 that is the E4M3 value
// 2^(e-7) (1 + m/8), resp. m 2^-9 (fp16 denormals are preserved).
__device__ __forceinline__ f16x2_t e4m3x2_to_f16(uint32_t two) {
  const uint32_t v = ((two & 0x7Fu) << 7) | (((two >> 8) & 0x7Fu) << 23);
  return __builtin_bit_cast(f16x2_t, v) * f16x2_t{(_Float16)256.0f, (_Float16)256.0f};
}

// 8 E2M1 codes (nibble j = element j) times one fp16 block scale -> 8 fp16,
// exact.
__device__ __forceinline__ f16x8_t dq8_e2m1_f16(uint32_t w, _Float16 s) {
  const f16x2_t ss = {s, s};
  const f16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * ss;
  const f16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * ss;
  const f16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * ss;
  const f16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * ss;
  return f16x8_t{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// fp16 matrix core: C(16x16) += A(16x32) B(32x16); same lane layout as the
// bf16 step (lane l: A[l%16][8(l/16)..+8], B[8(l/16)..+8][l%16]; result lane
// l, register r = C[4(l/16)+r][l%16]).
__device__ __forceinline__ f32x4_t mma_f16(f16x8_t a, f16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint16_t out_bf16(float acc, float gsa, float gsw) {
  return (uint16_t)f32_to_bf16_rne((acc * gsa) * gsw);
}

// ---------------------------------------------------------------------------
// both operands tiled
// ---------------------------------------------------------------------------
constexpr int kCodeBufs = 3;
constexpr int kScaleGroup = 512;  // scale bytes of one tile and one group of four super-chunks

// Workgroup shape: WM x WN waves, each owning TM x TN tiles of 16x16 of C;
// the workgroup's block is (WM*TM*16) x (WN*TN*16).  Per stage the block
// needs BMT = WM*TM A tiles and BNT = WN*TN W tiles of 1 KB; each wave
// copies (BMT+BNT)/(WM*WN) of them, and per group of four stages
// 2*(BMT+BNT)/(WM*WN) 256-byte scale pieces (4 bytes per lane).
template <int WM, int WN, int TM, int TN>
struct NvShape {
  static constexpr int kWaves = WM * WN;
  static constexpr int kBMT = WM * TM, kBNT = WN * TN, kTiles = kBMT + kBNT;
  static constexpr int kCopies = kTiles / kWaves;
  static constexpr int kScaleCopies = 2 * kTiles / kWaves;
  static constexpr size_t kSmem = (size_t)kCodeBufs * kTiles * 1024 + 2ull * kTiles * kScaleGroup;
  static_assert(kTiles % kWaves == 0, "code copies per wave");
  static_assert(kSmem <= 160 * 1024, "LDS");
};

template <int WM, int WN, int TM, int TN>
__global__ void __launch_bounds__(WM * WN * 64)
w4a4nv_tiled_kernel(const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales,
                    const float* __restrict__ a_gs, int M, const uint8_t* __restrict__ w_codes,
                    const uint8_t* __restrict__ w_scales, const float* __restrict__ w_gs, int N, int K,
                    uint16_t* __restrict__ C, int64_t ldc) {
  using Sh = NvShape<WM, WN, TM, TN>;
  constexpr int kTiles = Sh::kTiles, kBMT = Sh::kBMT, kBNT = Sh::kBNT;
  constexpr int kCopies = Sh::kCopies, kScaleCopies = Sh::kScaleCopies;
  constexpr int BR = kBMT * 16, BC = kBNT * 16;  // block rows (m) and columns (n)
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
  uint8_t (*cbuf)[kTiles][1024] = reinterpret_cast<uint8_t (*)[kTiles][1024]>(smem);
  uint8_t (*sbuf)[kTiles][kScaleGroup] =
      reinterpret_cast<uint8_t (*)[kTiles][kScaleGroup]>(smem + kCodeBufs * kTiles * 1024);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int S = K >> 7, Q = K >> 9;
  const int RTA = (M + 15) >> 4, RTW = (N + 15) >> 4;

  // workgroup -> block of C: XCD-major, then groups of 4 block rows
  const int TMB = (M + BR - 1) / BR, TNB = (N + BC - 1) / BC, T = TMB * TNB;
  const int b = blockIdx.x;
  const int lin = (T % 8 == 0) ? (b % 8) * (T / 8) + b / 8 : b;
  const int GM = 4, gsz = GM * TNB;
  const int first_m = (lin / gsz) * GM;
  const int gm = min(TMB - first_m, GM);
  const int bm = first_m + (lin % gsz) % gm;
  const int bn = (lin % gsz) / gm;

  // workgroup tile ti: 0..kBMT-1 are A row tiles bm*kBMT + ti, then W row
  // tiles bn*kBNT + (ti - kBMT); rows past the end are clamped
  auto tile_codes = [&](int ti) -> const uint8_t* {
    return ti < kBMT ? a_codes + (int64_t)min(bm * kBMT + ti, RTA - 1) * S * 1024
                     : w_codes + (int64_t)min(bn * kBNT + ti - kBMT, RTW - 1) * S * 1024;
  };
  auto tile_scales = [&](int ti) -> const uint8_t* {
    return ti < kBMT ? a_scales + (int64_t)min(bm * kBMT + ti, RTA - 1) * Q * kScaleGroup
                     : w_scales + (int64_t)min(bn * kBNT + ti - kBMT, RTW - 1) * Q * kScaleGroup;
  };
  // this wave's code tiles kCopies*wave + k (wave-uniform bases)
  const uint8_t* csrc[kCopies];
#pragma unroll
  for (int k = 0; k < kCopies; ++k) csrc[k] = tile_codes(kCopies * wave + k);
  // its scale pieces: 256 bytes each, piece c = tile kCopies*wave + c/2,
  // bytes 256*(c%2) + 4*lane
  const uint8_t* ssrc[kScaleCopies];
#pragma unroll
  for (int c = 0; c < kScaleCopies; ++c) ssrc[c] = tile_scales(kCopies * wave + c / 2) + 256 * (c % 2) + 4 * lane;

  // Past the end the last stage / group is copied again (into free
  // buffers), so every stage issues the same number of copies.
  auto issue_codes = [&](int t) {
    const int st = min(t, S - 1);
    uint8_t(*dst)[1024] = cbuf[t % kCodeBufs];
#pragma unroll
    for (int k = 0; k < kCopies; ++k)
      copy16_to_lds(csrc[k] + (int64_t)st * 1024 + lane * 16, dst[kCopies * wave + k]);
  };
  auto issue_scales = [&](int t) {
    const int q = min(t >> 2, Q - 1);
#pragma unroll
    for (int c = 0; c < kScaleCopies; ++c)
      copy4_to_lds(ssrc[c] + (int64_t)q * kScaleGroup, &sbuf[(t >> 2) & 1][kCopies * wave + c / 2][256 * (c % 2)]);
  };

  f32x4_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  // math of stage s (j = s % 4, its place in the scale group, known at
  // compile time)
  auto compute = [&](int s, auto jc) {
    constexpr int j = decltype(jc)::value;
    const uint8_t(*cb)[1024] = cbuf[s % kCodeBufs];
    const uint8_t(*sb)[kScaleGroup] = sbuf[(s >> 2) & 1];
    f16x2_t fa[TM], fw[TN];  // the lane's two block scales of this stage per tile
#pragma unroll
    for (int i = 0; i < TM; ++i)
      fa[i] = e4m3x2_to_f16(*reinterpret_cast<const uint16_t*>(&sb[wm * TM + i][lane * 8 + 2 * j]));
#pragma unroll
    for (int jj = 0; jj < TN; ++jj)
      fw[jj] = e4m3x2_to_f16(*reinterpret_cast<const uint16_t*>(&sb[kBMT + wn * TN + jj][lane * 8 + 2 * j]));
    // the codes are read one matrix step at a time (a dword per tile), so
    // only that step's are held in registers
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      uint32_t ca[TM], cw[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) ca[i] = *reinterpret_cast<const uint32_t*>(&cb[wm * TM + i][lane * 16 + 4 * kk]);
#pragma unroll
      for (int jj = 0; jj < TN; ++jj)
        cw[jj] = *reinterpret_cast<const uint32_t*>(&cb[kBMT + wn * TN + jj][lane * 16 + 4 * kk]);
      f16x8_t wd[TN];
#pragma unroll
      for (int jj = 0; jj < TN; ++jj) wd[jj] = dq8_e2m1_f16(cw[jj], fw[jj][kk >> 1]);
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const f16x8_t ad = dq8_e2m1_f16(ca[i], fa[i][kk >> 1]);
#pragma unroll
        for (int jj = 0; jj < TN; ++jj) acc[i][jj] = mma_f16(ad, wd[jj], acc[i][jj]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // prologue: stages 0 (codes + scales) and 1 (codes)
  issue_codes(0);
  issue_scales(0);
  issue_codes(1);

  // iteration s: wait for stage s (stage s+1 may stay in flight) and for
  // this wave's LDS reads of stage s-1, barrier, issue stage s+2 into the
  // buffers of stage s-1 (no wave reads them any more), compute stage s.  Copies
  // of stage s+1: kCopies, plus kScaleCopies when (s+1) % 4 == 0.  The tiled
  // layout has K % 512 == 0, so S is a multiple of 4.
  using J0 = std::integral_constant<int, 0>;
  using J1 = std::integral_constant<int, 1>;
  using J2 = std::integral_constant<int, 2>;
  using J3 = std::integral_constant<int, 3>;
  for (int s0 = 0; s0 < S; s0 += 4) {
    wait_vmcnt_lgkm0<kCopies>();
    stage_barrier();
    issue_codes(s0 + 2);
    compute(s0, J0());
    wait_vmcnt_lgkm0<kCopies>();
    stage_barrier();
    issue_codes(s0 + 3);
    compute(s0 + 1, J1());
    wait_vmcnt_lgkm0<kCopies>();
    stage_barrier();
    issue_codes(s0 + 4);
    issue_scales(s0 + 4);
    compute(s0 + 2, J2());
    wait_vmcnt_lgkm0<kCopies + kScaleCopies>();
    stage_barrier();
    issue_codes(s0 + 5);
    compute(s0 + 3, J3());
  }
  wait_vmcnt<0>();

  const float gsa = *a_gs, gsw = *w_gs;
  // lane l, register r of tile (i, jj) holds row 4(l/16) + r, column l%16
  const int row0 = bm * BR + wm * TM * 16;
  const int col0 = bn * BC + wn * TN * 16 + (lane & 15);
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int jj = 0; jj < TN; ++jj) {
      const int n = col0 + jj * 16;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = row0 + i * 16 + 4 * (lane >> 4) + r;
        if (m < M && n < N) C[(int64_t)m * ldc + n] = out_bf16(acc[i][jj][r], gsa, gsw);
      }
    }
}

template <int WM, int WN, int TM, int TN>
hipError_t run_tiled(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_gs, int64_t M,
                     const uint8_t* w_codes, const uint8_t* w_scales, const float* w_gs, int64_t N, int64_t K,
                     uint16_t* C, int64_t ldc, hipStream_t stream) {
  using Sh = NvShape<WM, WN, TM, TN>;
  auto* kern = &w4a4nv_tiled_kernel<WM, WN, TM, TN>;
  const hipError_t attr = set_max_lds<&w4a4nv_tiled_kernel<WM, WN, TM, TN>>(Sh::kSmem);
  if (attr != hipSuccess) return attr;
  const int64_t BR = Sh::kBMT * 16, BC = Sh::kBNT * 16;
  const int64_t T = ((M + BR - 1) / BR) * ((N + BC - 1) / BC);
  kern<<<(unsigned)T, Sh::kWaves * 64, Sh::kSmem, stream>>>(a_codes, a_scales, a_gs, (int)M, w_codes, w_scales,
                                                             w_gs, (int)N, (int)K, C, ldc);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// any layouts: register-tiled
// ---------------------------------------------------------------------------
constexpr int kMT = 4;      // 16-row tiles per wave (m)
constexpr int kNT = 4;      // 16-col tiles per wave (n)
constexpr int kGWaves = 4;

// this lane's 16 code bytes of super-chunk 0 for row `row` and the byte
// step between super-chunks
template <int LAYOUT>
__device__ __forceinline__ const uint8_t* frag_base(const uint8_t* codes, int64_t row, int lane, int64_t K) {
  if constexpr (LAYOUT == kLayoutRows) return codes + row * (K >> 1) + (lane >> 4) * 16;
  else return codes + (row >> 4) * (K >> 7) * 1024 + lane * 16;
}
template <int LAYOUT>
constexpr int frag_step() { return LAYOUT == kLayoutRows ? 64 : 1024; }

template <int ALAYOUT, int WLAYOUT>
__global__ void __launch_bounds__(kGWaves * 64)
w4a4nv_kernel(const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales,
              const float* __restrict__ a_gs, int M, const uint8_t* __restrict__ w_codes,
              const uint8_t* __restrict__ w_scales, const float* __restrict__ w_gs, int N, int K,
              uint16_t* __restrict__ C, int64_t ldc) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int n_wave = blockIdx.x * (kGWaves * 16 * kNT) + wave * (16 * kNT);
  if (n_wave >= N) return;
  const int m0 = blockIdx.y * (16 * kMT);

  const uint8_t* afrag[kMT];
  int arow[kMT];
#pragma unroll
  for (int mt = 0; mt < kMT; ++mt) {
    arow[mt] = min(m0 + 16 * mt + col, M - 1);
    afrag[mt] = frag_base<ALAYOUT>(a_codes, arow[mt], lane, K);
  }
  const uint8_t* wfrag[kNT];
  int wrow[kNT];
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt) {
    wrow[nt] = min(n_wave + 16 * nt + col, N - 1);
    wfrag[nt] = frag_base<WLAYOUT>(w_codes, wrow[nt], lane, K);
  }
  f32x4_t acc[kMT][kNT];
#pragma unroll
  for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) acc[mt][nt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  for (int s = 0; s < (K >> 7); ++s) {
    const int k = s * 128 + 32 * grp;  // first k of the lane's two 16-blocks (adjacent scale bytes)
    u32x4_t va[kMT], vw[kNT];
    f16x2_t fa[kMT], fw[kNT];
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt) {
      va[mt] = *reinterpret_cast<const u32x4_t*>(afrag[mt] + (int64_t)s * frag_step<ALAYOUT>());
      fa[mt] = e4m3x2_to_f16(*reinterpret_cast<const uint16_t*>(a_scales + scale_off<2, ALAYOUT>(arow[mt], k, K)));
    }
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
      vw[nt] = *reinterpret_cast<const u32x4_t*>(wfrag[nt] + (int64_t)s * frag_step<WLAYOUT>());
      fw[nt] = e4m3x2_to_f16(*reinterpret_cast<const uint16_t*>(w_scales + scale_off<2, WLAYOUT>(wrow[nt], k, K)));
    }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      f16x8_t wd[kNT];
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt) wd[nt] = dq8_e2m1_f16(vw[nt][kk], fw[nt][kk >> 1]);
#pragma unroll
      for (int mt = 0; mt < kMT; ++mt) {
        const f16x8_t ad = dq8_e2m1_f16(va[mt][kk], fa[mt][kk >> 1]);
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) acc[mt][nt] = mma_f16(ad, wd[nt], acc[mt][nt]);
      }
    }
  }
  const float gsa = *a_gs, gsw = *w_gs;
#pragma unroll
  for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
      const int n = n_wave + 16 * nt + col;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + 16 * mt + 4 * grp + r;
        if (m < M && n < N) C[(int64_t)m * ldc + n] = out_bf16(acc[mt][nt][r], gsa, gsw);
      }
    }
}

}  // namespace

hipError_t launch_gemm_w4a4_nvfp4(int a_layout, int w_layout, const uint8_t* a_codes, const uint8_t* a_scales,
                                  const float* a_gs, int64_t M, const uint8_t* w_codes,
                                  const uint8_t* w_scales, const float* w_gs, int64_t N, int64_t K,
                                  uint16_t* C, int64_t ldc, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  if (a_layout == kLayoutTiled && w_layout == kLayoutTiled)
    return run_tiled<2, 4, 8, 4>(a_codes, a_scales, a_gs, M, w_codes, w_scales, w_gs, N, K, C, ldc, stream);
  const dim3 grid((unsigned)((N + kGWaves * 16 * kNT - 1) / (kGWaves * 16 * kNT)),
                  (unsigned)((M + 16 * kMT - 1) / (16 * kMT)));
#define Q4_W4A4NV(AL, WL)                                                                         \
  w4a4nv_kernel<AL, WL><<<grid, kGWaves * 64, 0, stream>>>(a_codes, a_scales, a_gs, (int)M, w_codes, \
                                                           w_scales, w_gs, (int)N, (int)K, C, ldc)
  if (a_layout == kLayoutTiled) {
    if (w_layout == kLayoutTiled) Q4_W4A4NV(kLayoutTiled, kLayoutTiled); else Q4_W4A4NV(kLayoutTiled, kLayoutRows);
  } else {
    if (w_layout == kLayoutTiled) Q4_W4A4NV(kLayoutRows, kLayoutTiled); else Q4_W4A4NV(kLayoutRows, kLayoutRows);
  }
#undef Q4_W4A4NV
  return hipGetLastError();
}

}  // namespace q4
