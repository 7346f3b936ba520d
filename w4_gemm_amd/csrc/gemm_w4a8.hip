// gemm_w4a8.hip -- W4A8 GEMM: INT4 g128 weights, per-token FP8 (E4M3)
// activations, FP8 matrix cores, fp32 accumulation, bf16 output:
//   C[m][n] = s_a[m] * sum_g s_w[n][g] * sum_{k in group g} a8[m][k] * q[n][k]
// where a8 are the E4M3 activation values, s_a their per-row scales, q the
// INT4 codes (-8..7) and s_w the fp16 group scales (one per 128 k).
//
// The W4A8 scheme dequantizes the INT4 weights to FP8 and runs the products
// on FP8 matrix cores ("Low-bit inference for very large MoE", table
// "Kernels on different hardware", row W4A8).  An INT4 code is an integer of
// magnitude <= 8 and so an exact E4M3 value; its group scale is applied in
// fp32 to the matrix core's partial sum over that group of 128 k, the
// per-block promotion the "Quantization in deployment" exercises describe
// for block-scaled FP8 (products within a 128-wide K block on the matrix
// cores, then the block's scale, then accumulation in fp32).  On gfx950 one
// v_mfma_scale_f32_16x16x128_f8f6f4 (E4M3 x E4M3, unit scales) covers one
// INT4 group exactly.
//
// Tiled kernel (both operands in the tiled layouts, K % 512 == 0):
//   * a workgroup of 8 waves computes a 256 x 256 block of C; wave w owns
//     all 256 rows and the 32 columns of weight tiles 2w, 2w+1 = 16 x 2
//     matrix-core tiles (128 fp32 accumulators), so every weight tile is
//     converted INT4->E4M3 by one wave only and each converted fragment
//     feeds 16 products (a 2 x 4 arrangement of 128 x 64 wave tiles converted
//     every tile twice and measured 6% slower);
//   * K advances in stages of 128: 16 FP8 A tiles (2 KB each) and 16 INT4 W
//     tiles (1 KB) are copied verbatim into LDS by direct global->LDS loads
//     (6 per wave per stage), two stages ahead, into three buffers; the W
//     group scales of four stages (16 x 128 B) are copied once per group of
//     four into two buffers;
//   * one barrier per stage, before it a wait for this wave's copies of the
//     stage (explicit vmcnt) and for all its LDS reads (lgkmcnt 0), so no
//     wave still reads the buffer the next copies overwrite; the stage loop
//     unrolled by four;
//   * the products of a row tile go to a fresh register set and are scaled
//     into its accumulators after the next row tile's products are issued,
//     so the vector FMAs never wait on the matrix core's latency;
//   * workgroups ordered so the 32 running on one XCD share A and W panels.
// Generic kernel (any layout): one thread per output, the same promotion
// order, for the shapes and layouts the tiled kernel does not take.
#include "q4_launch.h"
#include "q4_layout.h"
#include "q4_lds.h"
#include "q4_mma.h"

namespace q4 {
namespace {

// INT4 (two's complement nibbles) -> E4M3 bytes.  v_perm_b32 picks byte
// sel (0..7) of the 64-bit pair {hi, lo}; the positive and the negative
// codes each fit one such 8-entry table indexed by the low three bits, and
// selector values 8..11 replicate the top bit of byte 1, 3, 5 or 7 of the
// pair, which turns the nibbles' sign bits into byte masks.
constexpr uint32_t kPosLo = 0x44403800u;  // E4M3 of 0, 1, 2, 3
constexpr uint32_t kPosHi = 0x4E4C4A48u;  // 4, 5, 6, 7
constexpr uint32_t kNegLo = 0xCACCCED0u;  // -8, -7, -6, -5
constexpr uint32_t kNegHi = 0xB8C0C4C8u;  // -4, -3, -2, -1

// Eight codes (nibble j = element j) -> the E4M3 bytes of elements 0,2,4,6
// (`even`, byte i = element 2i) and 1,3,5,7 (`odd`).
__device__ __forceinline__ void int4x8_to_e4m3(uint32_t x, uint32_t& even, uint32_t& odd) {
  const uint32_t se = x & 0x07070707u;
  const uint32_t so = (x >> 4) & 0x07070707u;
  // sign masks: even nibble e has its sign at bit 8e+3, odd nibble o at 8o+7
  const uint32_t me = __builtin_amdgcn_perm(x << 4, x << 12, 0x0B090A08u);
  const uint32_t mo = __builtin_amdgcn_perm(x, x << 8, 0x0B090A08u);
  const uint32_t pe = __builtin_amdgcn_perm(kPosHi, kPosLo, se);
  const uint32_t ne = __builtin_amdgcn_perm(kNegHi, kNegLo, se);
  const uint32_t po = __builtin_amdgcn_perm(kPosHi, kPosLo, so);
  const uint32_t no = __builtin_amdgcn_perm(kNegHi, kNegLo, so);
  even = (ne & me) | (pe & ~me);
  odd = (no & mo) | (po & ~mo);
}

// One INT4 fragment (16 bytes: 32 codes of one lane) -> FP8 operand in the
// order of the tiled FP8 activation layout (dword 2w + h = the even/odd
// elements of codes 8w .. 8w + 7).
__device__ __forceinline__ i32x8_t int4_frag_to_e4m3(u32x4_t raw) {
  i32x8_t r;
  uint32_t e, o;
  int4x8_to_e4m3(raw[0], e, o); r[0] = (int)e; r[1] = (int)o;
  int4x8_to_e4m3(raw[1], e, o); r[2] = (int)e; r[3] = (int)o;
  int4x8_to_e4m3(raw[2], e, o); r[4] = (int)e; r[5] = (int)o;
  int4x8_to_e4m3(raw[3], e, o); r[6] = (int)e; r[7] = (int)o;
  return r;
}

constexpr int kBM = 16;  // A tiles (16 rows) per workgroup
constexpr int kBN = 16;  // W tiles per workgroup
constexpr int kWaves = 8;
constexpr int kABytes = 2048;  // one FP8 tile (16 rows x 128 k)
constexpr int kWBytes = 1024;  // one INT4 tile
constexpr int kBufs = 3;
constexpr int kSBytes = kBN * 128;  // fp16 W scales of one group of four stages
constexpr int kCopies = (kBM * kABytes + kBN * kWBytes) / 1024 / kWaves;  // 1 KB copies per wave per stage
constexpr size_t kSmemBytes = (size_t)kBufs * (kBM * kABytes + kBN * kWBytes) + 2 * kSBytes;  // 148 KB
static_assert(kCopies == 6, "copy plan");

__global__ void __launch_bounds__(kWaves * 64)
w4a8_tiled_kernel(const uint8_t* __restrict__ a_codes, const float* __restrict__ a_scales, int M,
                  const uint8_t* __restrict__ w_codes, const uint8_t* __restrict__ w_scales, int N,
                  int K, uint16_t* __restrict__ C, int64_t ldc) {
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
  uint8_t (*abuf)[kBM][kABytes] = reinterpret_cast<uint8_t (*)[kBM][kABytes]>(smem);
  uint8_t (*wbuf)[kBN][kWBytes] = reinterpret_cast<uint8_t (*)[kBN][kWBytes]>(smem + kBufs * kBM * kABytes);
  uint8_t (*sbuf)[kSBytes] =
      reinterpret_cast<uint8_t (*)[kSBytes]>(smem + kBufs * (kBM * kABytes + kBN * kWBytes));

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wn = wave;  // the wave's two weight tiles 2wn, 2wn+1; all 16 A tiles
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

  // this wave's copies of a stage: A tile halves 4*wave .. 4*wave+3 (tile
  // c/2, half c%2) and W tiles 2*wave, 2*wave+1; wave-uniform bases
  const uint8_t* asrc[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int c = 4 * wave + k;
    asrc[k] = a_codes + (int64_t)min(bm * kBM + (c >> 1), RTA - 1) * S * kABytes + (c & 1) * 1024;
  }
  const uint8_t* wsrc[2];
#pragma unroll
  for (int k = 0; k < 2; ++k)
    wsrc[k] = w_codes + (int64_t)min(bn * kBN + 2 * wave + k, RTW - 1) * S * kWBytes;
  // W scales: lane -> tile 2*wave + lane/32, bytes 4*(lane%32) of its 128
  const uint8_t* ssrc = w_scales + (int64_t)min(bn * kBN + 2 * wave + (lane >> 5), RTW - 1) * Q * 128 +
                        (lane & 31) * 4;

  auto issue_codes = [&](int t) {
    const int st = min(t, S - 1);
    const int bi = t % kBufs;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int c = 4 * wave + k;
      copy16_to_lds(uniform_ptr(asrc[k] + (int64_t)st * kABytes) + lane * 16, &abuf[bi][c >> 1][(c & 1) * 1024]);
    }
#pragma unroll
    for (int k = 0; k < 2; ++k)
      copy16_to_lds(uniform_ptr(wsrc[k] + (int64_t)st * kWBytes) + lane * 16, wbuf[bi][2 * wave + k]);
  };
  auto issue_scales = [&](int t) {
    const int q = min(t >> 2, Q - 1);
    copy4_to_lds(ssrc + (int64_t)q * 128, &sbuf[(t >> 2) & 1][256 * wave]);
  };

  f32x4_t acc[16][2];
#pragma unroll
  for (int i = 0; i < 16; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  auto compute = [&](int s, int j) {
    const int bi = s % kBufs;
    // A fragment i: operand bytes 0..15 and 16..31 of the lane
    auto load_a = [&](int i) {
      const u32x4_t lo = *reinterpret_cast<const u32x4_t*>(&abuf[bi][i][lane * 16]);
      const u32x4_t hi = *reinterpret_cast<const u32x4_t*>(&abuf[bi][i][1024 + lane * 16]);
      return i32x8_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                     (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    };
    // the weight fragments, converted to E4M3, and the fp16 scale of group
    // 4q + j of the lane's weight column in each (scale tile: [row][group])
    float sw[2];
    i32x8_t wq[2];
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      sw[jj] = fp16_value(*reinterpret_cast<const uint16_t*>(
          &sbuf[(s >> 2) & 1][(wn * 2 + jj) * 128 + (lane & 15) * 8 + j * 2]));
      wq[jj] = int4_frag_to_e4m3(*reinterpret_cast<const u32x4_t*>(&wbuf[bi][wn * 2 + jj][lane * 16]));
    }
    i32x8_t a[2];
    a[0] = load_a(0);
    // One A fragment in flight ahead of the products, and the group-scaled
    // accumulation of row tile i done after the products of tile i+1 have
    // been issued, so it reads results whose latency has passed instead of
    // waiting on them (the fences keep the compiler from hoisting every
    // fragment load, which would not fit the register budget of two waves
    // per SIMD).
    f32x4_t p[2][2];
    auto scale_add = [&](int i) {
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[i][jj][r] = __builtin_fmaf(p[i & 1][jj][r], sw[jj], acc[i][jj][r]);
    };
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (i < 15) a[(i + 1) & 1] = load_a(i + 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
        p[i & 1][jj] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            a[i & 1], wq[jj], f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0, 127, 0, 127);
      if (i > 0) {
        scale_add(i - 1);
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // the two products first,
        __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);  // then the previous tile's 8 FMAs
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    scale_add(15);
  };

  issue_codes(0);
  issue_scales(0);
  issue_codes(1);
  // iteration s: wait for copy group s (group s+1 may stay in flight: its
  // kCopies code copies, plus its scale copy when (s+1) % 4 == 0) and for
  // this wave's LDS reads of stage s-1, barrier, issue group s+2 into the
  // buffers of stage s-1, compute stage s.
  for (int s0 = 0; s0 < S; s0 += 4) {
    wait_vmcnt_lgkm0<kCopies>();
    stage_barrier();
    issue_codes(s0 + 2);
    compute(s0, 0);
    wait_vmcnt_lgkm0<kCopies>();
    stage_barrier();
    issue_codes(s0 + 3);
    compute(s0 + 1, 1);
    wait_vmcnt_lgkm0<kCopies>();
    stage_barrier();
    issue_codes(s0 + 4);
    issue_scales(s0 + 4);
    compute(s0 + 2, 2);
    wait_vmcnt_lgkm0<kCopies + 1>();
    stage_barrier();
    issue_codes(s0 + 5);
    compute(s0 + 3, 3);
  }
  wait_vmcnt<0>();

  // lane l, register r of tile (i, jj) holds row 4(l/16) + r, column l%16
  const int row0 = bm * 256;
  const int col0 = bn * 256 + wn * 32 + (lane & 15);
#pragma unroll
  for (int i = 0; i < 16; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = row0 + i * 16 + 4 * (lane >> 4) + r;
      if (m >= M) continue;
      const float sa = a_scales[m];
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int n = col0 + jj * 16;
        if (n < N) C[(int64_t)m * ldc + n] = (uint16_t)f32_to_bf16_rne(acc[i][jj][r] * sa);
      }
    }
}

// E4M3 code (sign included) -> fp32.
__device__ __forceinline__ float e4m3_signed(uint32_t c) {
  const float v = e4m3_value(c & 0x7Fu);
  return (c & 0x80u) ? -v : v;
}

template <int ALAY, int WLAY>
__global__ void __launch_bounds__(256)
w4a8_generic_kernel(const uint8_t* __restrict__ a_codes, const float* __restrict__ a_scales, int M,
                    const uint8_t* __restrict__ w_codes, const uint16_t* __restrict__ w_scales, int N,
                    int K, uint16_t* __restrict__ C, int64_t ldc) {
  const int64_t tn = (N + 15) >> 4, tiles = tn * ((M + 15) >> 4);
  for (int64_t tile = blockIdx.x; tile < tiles; tile += gridDim.x) {
  const int n = (int)(tile % tn) * 16 + (threadIdx.x & 15);
  const int m = (int)(tile / tn) * 16 + (threadIdx.x >> 4);
  if (m >= M || n >= N) continue;
  float acc = 0.0f;
  for (int g = 0; g < (K >> 7); ++g) {
    float part = 0.0f;
    for (int k0 = g * 128; k0 < g * 128 + 128; k0 += 8) {
      uint32_t a[8];
      if constexpr (ALAY == kLayoutRows) {
        const uint2 v = *reinterpret_cast<const uint2*>(a_codes + (int64_t)m * K + k0);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          a[j] = (v.x >> (8 * j)) & 0xFFu;
          a[4 + j] = (v.y >> (8 * j)) & 0xFFu;
        }
      } else {
        const uint32_t ev = *reinterpret_cast<const uint32_t*>(a_codes + fp8_tiled_dword(m, k0, K, 0));
        const uint32_t od = *reinterpret_cast<const uint32_t*>(a_codes + fp8_tiled_dword(m, k0, K, 1));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          a[2 * i] = (ev >> (8 * i)) & 0xFFu;
          a[2 * i + 1] = (od >> (8 * i)) & 0xFFu;
        }
      }
      const uint32_t w = *reinterpret_cast<const uint32_t*>(w_codes + code_off8<WLAY>(n, k0, K));
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int q = ((int)(w << (28 - 4 * j))) >> 28;  // sign-extend nibble j
        part = __builtin_fmaf(e4m3_signed(a[j]), (float)q, part);
      }
    }
    acc = __builtin_fmaf(part, fp16_value(w_scales[scale_off<0, WLAY>(n, g * 128, K)]), acc);
  }
  C[(int64_t)m * ldc + n] = (uint16_t)f32_to_bf16_rne(acc * a_scales[m]);
  }
}

}  // namespace

hipError_t launch_gemm_w4a8(int a_layout, int w_layout, const uint8_t* a_codes, const float* a_scales,
                            int64_t M, const uint8_t* w_codes, const uint16_t* w_scales, int64_t N,
                            int64_t K, uint16_t* C, int64_t ldc, hipStream_t stream) {
  if (a_layout == kLayoutTiled && w_layout == kLayoutTiled) {
    const hipError_t attr = set_max_lds<&w4a8_tiled_kernel>(kSmemBytes);
    if (attr != hipSuccess) return attr;
    const int64_t T = ((M + 255) / 256) * ((N + 255) / 256);
    w4a8_tiled_kernel<<<(unsigned)T, kWaves * 64, kSmemBytes, stream>>>(
        a_codes, a_scales, (int)M, w_codes, reinterpret_cast<const uint8_t*>(w_scales), (int)N, (int)K, C,
        ldc);
    return hipGetLastError();
  }
  const int64_t tiles = ((N + 15) / 16) * ((M + 15) / 16);
  const unsigned grid = (unsigned)(tiles < (1 << 20) ? tiles : (1 << 20));
#define Q4_W4A8_G(AL, WL)                                                                        \
  w4a8_generic_kernel<AL, WL><<<grid, 256, 0, stream>>>(a_codes, a_scales, (int)M, w_codes, w_scales, \
                                                        (int)N, (int)K, C, ldc)
  if (a_layout == kLayoutTiled) {
    if (w_layout == kLayoutTiled) Q4_W4A8_G(kLayoutTiled, kLayoutTiled); else Q4_W4A8_G(kLayoutTiled, kLayoutRows);
  } else {
    if (w_layout == kLayoutTiled) Q4_W4A8_G(kLayoutRows, kLayoutTiled); else Q4_W4A8_G(kLayoutRows, kLayoutRows);
  }
#undef Q4_W4A8_G
  return hipGetLastError();
}

}  // namespace q4
