// probe.hip -- a plain streaming read of a device buffer: the reference
// against which the decode GEMV's HBM rate is judged.  Decode is bound by
// the weight reads ("Low-bit inference for very large MoE", table "Kernels
// on different hardware", row W4A16), so the best rate at which this part
// can read a buffer of the weight's size, with the same rotation past the
// last-level cache, is the ceiling that GEMV can approach; the published 8
// TB/s is a different figure.
//
// Each wave reads eight contiguous 1 KB pieces per iteration (16 bytes per
// lane, non-temporal, all eight in flight), workgroups of 4 waves stride the
// buffer; the values are folded into one word that is written only if it
// equals a constant no buffer of the probe's callers produces, which keeps
// the loads from being removed.  The shape is the best of a sweep on gfx950
// (pieces in flight 4/8/16, plain / non-temporal / global->LDS loads,
// 512..2048 workgroups).
//
// The second probe is the matrix-core counterpart: the rate at which this
// part sustains one kind of matrix instruction, back to back, on operands
// already in registers.  The operands are pseudo-random bits (as quantized
// weights and activations are): with constant operands the part holds its
// top clock, with random ones it lowers the clock to stay within its power
// limit, so the published peak is not the rate a GEMM on real data can
// approach.  Each wave issues 8 independent instructions per iteration
// (each accumulator is reused 8 instructions later), two waves per SIMD.
// The instructions are written out so that every accumulator stays in
// place: nothing else runs in the loop.
//
// Two more kinds run the FP4 instruction at the same rate with the memory
// instructions of the tiled W4A4 kernel mixed in, per SIMD and 64
// instructions: 8 direct global->LDS copies of 1 KB (kind 4), and those
// plus 24 LDS fragment reads of 16 bytes per lane (kind 5) -- what that
// kernel issues per stage.  The copies read a 64 KB window at the sink
// pointer (L2-resident), each wave into its own ring of four 1 KB LDS
// slots; the reads take a wave's own 4 KB of LDS.  The difference to kind
// 0 is what those instructions cost the matrix core (issue slots, and the
// clock, which power sets).  Kind 6 does the same for the tiled W4A16 GEMM
// on NVFP4 weights: bf16 products with, per wave and 16 of them, one
// weight fragment dequantized by that kernel's own helper (the row operand
// of those 16 products), 8 fragment reads and one copy.
#include "q4_launch.h"
#include "q4_mma.h"

#include <type_traits>

namespace q4 {
namespace {

constexpr int kProbeWaves = 4;
constexpr int kProbeU = 8;
constexpr unsigned kProbeGrid = 1024;
constexpr uint32_t kProbeMagic = 0x9E3779B9u;

__global__ void __launch_bounds__(kProbeWaves * 64)
read_probe_kernel(const uint8_t* __restrict__ p, int64_t nchunks, uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t nw = (int64_t)gridDim.x * kProbeWaves;
  u32x4_t acc = u32x4_t{0u, 0u, 0u, 0u};
  int64_t c = ((int64_t)blockIdx.x * kProbeWaves + wave) * kProbeU;
  for (; c + kProbeU <= nchunks; c += nw * kProbeU) {
    u32x4_t v[kProbeU];
#pragma unroll
    for (int u = 0; u < kProbeU; ++u)
      v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p + (c + u) * 1024 + lane * 16));
#pragma unroll
    for (int u = 0; u < kProbeU; ++u) acc ^= v[u];
  }
  for (; c < nchunks; ++c)  // the last wave's partial group of pieces
    acc ^= __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p + c * 1024 + lane * 16));
  const uint32_t w = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (w == kProbeMagic) sink[0] = w;
}

constexpr int kMfmaProbeWaves = 4;
typedef uint32_t u32x8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ uint32_t probe_hash(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

// KIND: 0 FP4 16x16x128 (scaled), 1 bf16 16x16x32, 2 fp16 16x16x32, 3 FP8 16x16x128 (scaled),
// 4 FP4 with one copy per 8 instructions, 5 FP4 with one copy and three fragment reads per 8,
// 6 bf16 with one dequantized NVFP4 fragment, one copy and eight fragment reads per 16
template <int KIND>
__global__ void __launch_bounds__(kMfmaProbeWaves * 64)
mfma_probe_kernel(int64_t iters, uint32_t seed, uint32_t* __restrict__ sink) {
  constexpr bool kCopy = KIND >= 4, kRead = KIND >= 5, kDq = KIND == 6;
  constexpr int kReads = KIND == 6 ? 4 : 3;  // fragment reads per 8 instructions
  // per wave: four 1 KB copy slots, then 4 KB of fragments to read
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kCopy ? kMfmaProbeWaves * 8192 : 16];
  const uint32_t base = (seed * 0x9E3779B1u) ^ ((blockIdx.x * blockDim.x + threadIdx.x) * 64u);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  u32x4_t x[8], y[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      uint32_t a = probe_hash(base + 8u * i + e), b = probe_hash(base + 8u * i + 4u + e + 0x51ED27u);
      if constexpr (KIND == 1 || KIND == 6) {  // bf16: random signs and mantissas, exponents of [0.5, 1)
        a = (a & 0x807F807Fu) | 0x3F003F00u;
        b = (b & 0x807F807Fu) | 0x3F003F00u;
      } else if constexpr (KIND == 2) {  // fp16: the same
        a = (a & 0x83FF83FFu) | 0x38003800u;
        b = (b & 0x83FF83FFu) | 0x38003800u;
      } else if constexpr (KIND == 3) {  // E4M3 without the NaN codes
        a &= 0xF7F7F7F7u;
        b &= 0xF7F7F7F7u;
      }
      x[i][e] = a;
      y[i][e] = b;
    }
  }
  const uint32_t sc = 0x7C7D7E7Fu ^ (probe_hash(base) & 0x03030303u);  // E8M0 near 1
  u32x8_t x8[KIND == 3 ? 8 : 1], y8[KIND == 3 ? 8 : 1];  // FP8 operands: 32 bytes per lane
  if constexpr (KIND == 3) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      x8[i] = u32x8_t{x[i][0], x[i][1], x[i][2], x[i][3], y[i][0], y[i][1], y[i][2], y[i][3]};
      y8[i] = u32x8_t{y[i][0], y[i][1], y[i][2], y[i][3], x[i][0], x[i][1], x[i][2], x[i][3]};
    }
  }
  f32x4_t c[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) c[i] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  // (the instructions exist in the device pass only: the host pass checks
  // inline-asm operands against the host's registers)
  uint8_t* const ring = lds + (kCopy ? wave * 8192 : 0);
  const uint8_t* const csrc = reinterpret_cast<const uint8_t*>(sink) + lane * 16;
  const int cbase = blockIdx.x * kMfmaProbeWaves + wave;
  u32x4_t r[2][4] = {};
  // kind 6: the NVFP4 codes dequantized per 16 products, and their result
  const uint32_t dcodes = probe_hash(base + 4242u);
  const float dscale = e4m3_value(0x3Fu ^ (probe_hash(base + 99u) & 0x07u)) * 0x1p-9f;
  u32x4_t wq = y[0];
  if constexpr (kRead) {
#pragma unroll
    for (int j = 0; j < 16; ++j) reinterpret_cast<uint32_t*>(ring + 4096)[lane + 64 * j] = probe_hash(base + 977u * j);
  }
#if defined(__HIP_DEVICE_COMPILE__)
  const uint32_t fra = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)(ring + 4096) + lane * 16;
  auto iteration = [&](int64_t it, auto set) {
    constexpr int R = decltype(set)::value;  // register set of this iteration's fragment reads
    if constexpr (kDq) {
      if constexpr (R == 0) {  // this pair of iterations' row operand
        wq = __builtin_bit_cast(u32x4_t, dq8_e2m1_mul(dcodes ^ (uint32_t)it, dscale));
        asm volatile("" : "+v"(wq));
      }
    }
    asm volatile("s_nop 4");  // the operands' last vector writes before the first product
    if constexpr (kRead && kReads == 3)
      asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(r[R ^ 1][0]), "+v"(r[R ^ 1][1]), "+v"(r[R ^ 1][2]) :: "memory");
    if constexpr (kRead && kReads == 4)
      asm volatile("s_waitcnt lgkmcnt(0)"
                   : "+v"(r[R ^ 1][0]), "+v"(r[R ^ 1][1]), "+v"(r[R ^ 1][2]), "+v"(r[R ^ 1][3]) :: "memory");
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if constexpr (kCopy) {
        if (i == 1 && (!kDq || R == 0))
          __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(csrc + ((cbase + it) & 63) * 1024),
                                           (__attribute__((address_space(3))) void*)(ring + (it & 3) * 1024), 16, 0, 0);
      }
      if constexpr (kRead) {
        // three 16-byte reads early in each iteration into register set R;
        // the next iteration starts by waiting for them (long landed) and
        // taking them as read, so their registers stay theirs until then
        if (i < kReads) {
          const uint32_t addr = fra + (uint32_t)(((it + i) & 3) * 1024);
          asm volatile("ds_read_b128 %0, %1" : "=v"(r[R][i]) : "v"(addr) : "memory");
        }
      }
      if constexpr (KIND == 0 || KIND == 4 || KIND == 5)
        asm volatile("v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %3 op_sel_hi:[0,0,0] cbsz:4 blgp:4"
                     : "+v"(c[i]) : "v"(x[i]), "v"(y[i]), "v"(sc));
      else if constexpr (KIND == 1)
        asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(c[i]) : "v"(x[i]), "v"(y[i]));
      else if constexpr (KIND == 6)
        asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(c[i]) : "v"(wq), "v"(x[i]));
      else if constexpr (KIND == 2)
        asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+v"(c[i]) : "v"(x[i]), "v"(y[i]));
      else
        asm volatile("v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %3 op_sel_hi:[0,0,0]"
                     : "+v"(c[i]) : "v"(x8[i]), "v"(y8[i]), "v"(sc));
    }
    if constexpr (kCopy) __builtin_amdgcn_s_waitcnt((1 & 0xF) | (0x7 << 4) | (0xF << 8));  // vmcnt(1): one copy in flight
  };
  int64_t it = 0;
  for (; it + 1 < iters; it += 2) {
    iteration(it, std::integral_constant<int, 0>());
    iteration(it + 1, std::integral_constant<int, 1>());
  }
  if (it < iters) iteration(it, std::integral_constant<int, 0>());
  // the last instructions' results are read only after their passes end
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#endif
  f32x4_t t = c[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) t += c[i];
  uint32_t w = __float_as_uint(t[0]) ^ __float_as_uint(t[1]) ^ __float_as_uint(t[2]) ^ __float_as_uint(t[3]);
  if constexpr (kRead) {
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int j = 0; j < kReads; ++j) w ^= r[s][j][0] ^ r[s][j][1] ^ r[s][j][2] ^ r[s][j][3];
  }
  if constexpr (kDq) w ^= wq[0] ^ wq[3];
  if constexpr (kCopy) w ^= reinterpret_cast<const uint32_t*>(ring)[lane];
  if (w == kProbeMagic) sink[0] = w;
}

}  // namespace

int mfma_probe_grid() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return 2 * cus;  // two workgroups of four waves per compute unit: two waves per SIMD
}

hipError_t launch_mfma_probe(int kind, int64_t iters, uint32_t seed, uint32_t* sink, int grid, hipStream_t stream) {
  const dim3 g((unsigned)grid), b(kMfmaProbeWaves * 64);
  switch (kind) {
    case 0: mfma_probe_kernel<0><<<g, b, 0, stream>>>(iters, seed, sink); break;
    case 1: mfma_probe_kernel<1><<<g, b, 0, stream>>>(iters, seed, sink); break;
    case 2: mfma_probe_kernel<2><<<g, b, 0, stream>>>(iters, seed, sink); break;
    case 3: mfma_probe_kernel<3><<<g, b, 0, stream>>>(iters, seed, sink); break;
    case 4: mfma_probe_kernel<4><<<g, b, 0, stream>>>(iters, seed, sink); break;
    case 5: mfma_probe_kernel<5><<<g, b, 0, stream>>>(iters, seed, sink); break;
    default: mfma_probe_kernel<6><<<g, b, 0, stream>>>(iters, seed, sink); break;
  }
  return hipGetLastError();
}

hipError_t launch_read_probe(const uint8_t* src, int64_t bytes, uint32_t* sink, hipStream_t stream) {
  const int64_t nchunks = bytes / 1024;
  if (nchunks == 0) return hipSuccess;
  const int64_t need = (nchunks + kProbeU * kProbeWaves - 1) / (kProbeU * kProbeWaves);
  const unsigned grid = (unsigned)(need < kProbeGrid ? need : kProbeGrid);
  read_probe_kernel<<<grid, kProbeWaves * 64, 0, stream>>>(src, nchunks, sink);
  return hipGetLastError();
}

}  // namespace q4
