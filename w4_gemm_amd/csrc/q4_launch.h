// q4_launch.h -- host-side launchers of the gfx950 kernels, called by the
// C ABI (api.hip) after it has validated every argument.  Each launcher
// only enqueues work on `stream` and returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace q4 {

// Raises KERNEL's dynamic LDS limit to `bytes` on the current device, once
// per device (the attribute belongs to the kernel on that device; devices
// 0..63 are remembered, others set it on every call).
template <auto KERNEL>
hipError_t set_max_lds(size_t bytes) {
  static std::atomic<uint64_t> done{0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = (dev >= 0 && dev < 64) ? (1ull << dev) : 0ull;
  if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(KERNEL), hipFuncAttributeMaxDynamicSharedMemorySize,
                          (int)bytes);
  if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_acq_rel);
  return e;
}

// Output formats of the GEMMs that can write C quantized (q4_qout.h).
constexpr int kOutBf16 = 0;
constexpr int kOutMxfp4 = 1;
constexpr int kOutNvfp4 = 2;

// A quantized GEMM output (the C ABI's q4_tensor, as the kernels take it).
struct QOut {
  uint8_t* codes;
  uint8_t* scales;
  const float* gs_in;  // NVFP4: the tensor scale to quantize with (device)
  float* gs_out;       // NVFP4: the output's own global-scale word (gets *gs_in)
  int tiled;           // 1: tiled layout, 0: row-major
};

// Plain streaming read of `bytes` (a multiple of 1024) at src (16-byte
// aligned); `sink` (device uint32) is never written by real data.
hipError_t launch_read_probe(const uint8_t* src, int64_t bytes, uint32_t* sink, hipStream_t stream);
// Workgroups the matrix-instruction probe launches on the current device
// (0 if the device cannot be queried).
int mfma_probe_grid();
hipError_t launch_mfma_probe(int kind, int64_t iters, uint32_t seed, uint32_t* sink, int grid, hipStream_t stream);

// Quantize bf16 src [rows][ld] into codes/scales (fmt 0 INT4 g128,
// 1 MXFP4, 2 NVFP4; layout 0 row-major, 1 tiled).  NVFP4: gs receives the
// global scale; gs_in, when not null, supplies it instead of the
// tensor-absmax pass.
hipError_t launch_quantize(int fmt, int layout, const uint16_t* src, int64_t ld, int64_t rows,
                           int64_t cols, uint8_t* codes, void* scales, float* gs,
                           const float* gs_in, hipStream_t stream);

// Dequantize into row-major dst [rows][ld], dst_dtype 0 bf16 / 1 fp32.
hipError_t launch_relayout(int fmt, int to_layout, const uint8_t* src_codes, const void* src_scales,
                           const float* src_gs, uint8_t* dst_codes, void* dst_scales, float* dst_gs, int64_t rows,
                           int64_t cols, hipStream_t stream);
hipError_t launch_dequant(int fmt, int layout, const uint8_t* codes, const void* scales,
                          const float* gs, int64_t rows, int64_t cols, void* dst, int dst_dtype,
                          int64_t ld, hipStream_t stream);

// W4A16 GEMV, 1 <= B <= 16, K % 128 == 0 (row-major) / 512 (tiled).
hipError_t launch_gemv(int fmt, int layout, const uint8_t* codes, const void* scales, const float* gs,
                       int64_t N, int64_t K, const uint16_t* x, int64_t ldx, int64_t B,
                       uint16_t* y, int64_t ldy, hipStream_t stream);

// W4A16 GEMM C [M][ldc] = A [M][lda] . W'^T, K % 128 == 0.
hipError_t launch_gemm_w4a16(int fmt, int layout, const uint8_t* codes, const void* scales, const float* gs,
                             int64_t N, int64_t K, const uint16_t* A, int64_t lda, int64_t M,
                             uint16_t* C, int64_t ldc, hipStream_t stream);

// W4A16 GEMM with the weight in the tiled layout (K % 512 == 0): the
// LDS-staged kernel of gemm_w4a16.hip.
hipError_t launch_gemm_w4a16_tiled(int fmt, const uint8_t* codes, const void* scales, const float* gs,
                                   int64_t N, int64_t K, const uint16_t* A, int64_t lda, int64_t M,
                                   uint16_t* C, int64_t ldc, hipStream_t stream);

// W4A4 MXFP4 GEMM C [M][ldc] = A' . W'^T, both MXFP4, K % 128 == 0.
hipError_t launch_gemm_w4a4(int a_layout, int w_layout, const uint8_t* a_codes, const uint8_t* a_scales, int64_t M,
                            const uint8_t* w_codes, const uint8_t* w_scales, int64_t N, int64_t K,
                            uint16_t* C, int64_t ldc, hipStream_t stream);

// W4A4 with both operands in the tiled layout (K % 512 == 0): the
// LDS-staged kernel of gemm_w4a4.hip.
hipError_t launch_gemm_w4a4_tiled(const uint8_t* a_codes, const uint8_t* a_scales, int64_t M,
                                  const uint8_t* w_codes, const uint8_t* w_scales, int64_t N,
                                  int64_t K, uint16_t* C, int64_t ldc, hipStream_t stream);

// The same two GEMMs with C written quantized (MXFP4 or NVFP4 under the
// tensor scale qo.gs_in, N % 32 == 0) by the epilogue of q4_qout.h.
hipError_t launch_gemm_w4a16_tiled_qout(int w_fmt, int out_fmt, const uint8_t* codes, const void* scales,
                                        const float* gs, int64_t N, int64_t K, const uint16_t* A, int64_t lda,
                                        int64_t M, const QOut& qo, hipStream_t stream);
hipError_t launch_gemm_w4a4_tiled_qout(int out_fmt, const uint8_t* a_codes, const uint8_t* a_scales, int64_t M,
                                       const uint8_t* w_codes, const uint8_t* w_scales, int64_t N, int64_t K,
                                       const QOut& qo, hipStream_t stream);

// W4A4 NVFP4 GEMM C [M][ldc] = A' . W'^T, both NVFP4 (E4M3 per 16, each
// operand's fp32 tensor scale a_gs / w_gs on the device), K % 128 == 0:
// fp16 matrix cores on exactly dequantized operands (gemm_w4a4_nv.hip).
hipError_t launch_gemm_w4a4_nvfp4(int a_layout, int w_layout, const uint8_t* a_codes, const uint8_t* a_scales,
                                  const float* a_gs, int64_t M, const uint8_t* w_codes,
                                  const uint8_t* w_scales, const float* w_gs, int64_t N, int64_t K,
                                  uint16_t* C, int64_t ldc, hipStream_t stream);

// Per-token FP8 (E4M3) quantization of bf16 src [rows][ld] into codes
// (row-major [rows][cols] or the tiled FP8 layout) and fp32 scales [rows].
hipError_t launch_fp8_rows_quantize(int layout, const uint16_t* src, int64_t ld, int64_t rows,
                                    int64_t cols, uint8_t* codes, float* scales, hipStream_t stream);

// FP8 rows -> row-major dst [rows][ld], dst_dtype 0 bf16 / 1 fp32.
hipError_t launch_fp8_rows_dequant(int layout, const uint8_t* codes, const float* scales, int64_t rows,
                                   int64_t cols, void* dst, int dst_dtype, int64_t ld, hipStream_t stream);

// W4A8 GEMM C [M][ldc] = A8' . W'^T: A per-token FP8, W INT4 g128,
// K % 128 == 0 (512 for a tiled operand).
hipError_t launch_gemm_w4a8(int a_layout, int w_layout, const uint8_t* a_codes, const float* a_scales,
                            int64_t M, const uint8_t* w_codes, const uint16_t* w_scales, int64_t N,
                            int64_t K, uint16_t* C, int64_t ldc, hipStream_t stream);

// MoE routing: top-k experts per token (ids, softmax gates) from fp32
// logits [T][ld], then the expert-major dispatch (offsets [E+1], gather
// [T*k], inv [T][k]) in one workgroup whose LDS holds per-expert token
// bitmaps: moe_dispatch_lds_bytes(T, E) <= kMoeDispatchMaxLds.
constexpr size_t kMoeDispatchMaxLds = 160 * 1024;
size_t moe_dispatch_lds_bytes(int64_t T, int32_t E);
hipError_t launch_moe_route(const float* logits, int64_t ld, int64_t T, int32_t E, int32_t k,
                            int32_t* ids, float* weights, int32_t* offsets, int32_t* gather,
                            int32_t* inv, hipStream_t stream);

// h [P][ldh] = silu(gu[:, :I]) * gu[:, I:2I] (bf16), I % 8 == 0.
hipError_t launch_swiglu(const uint16_t* gu, int64_t ld_gu, int64_t P, int64_t I, uint16_t* h, int64_t ldh,
                         hipStream_t stream);

// out [T][ldo] = sum_j w[t][j] * y[inv[t][j]] (bf16), N % 8 == 0.
hipError_t launch_moe_combine(const uint16_t* y, int64_t ldy, const int32_t* inv, const float* w, int64_t T,
                              int32_t k, int64_t N, uint16_t* out, int64_t ldo, hipStream_t stream);

// Grouped expert GEMM with the expert weights in the tiled layout (K % 512
// == 0, N % 16 == 0, T > 0): the weight-streaming kernel of grouped.hip.
hipError_t launch_grouped_tiled(int fmt, const uint16_t* A, int64_t lda, int64_t T, const int32_t* gather,
                                const int32_t* offsets, int32_t E, int64_t P, const uint8_t* codes,
                                const void* scales, const float* gs, int64_t N, int64_t K, uint16_t* C,
                                int64_t ldc, hipStream_t stream);

// The same kernel with the SwiGLU epilogue: each expert's 2I weight rows
// alternate 16-row tiles of W_gate and W_up; writes H [P][ldh] (I columns).
hipError_t launch_grouped_tiled_swiglu(int fmt, const uint16_t* A, int64_t lda, int64_t T, const int32_t* gather,
                                       const int32_t* offsets, int32_t E, int64_t P, const uint8_t* codes,
                                       const void* scales, const float* gs, int64_t N2, int64_t K, uint16_t* H,
                                       int64_t ldh, hipStream_t stream);

// Grouped expert GEMM (W4A16), see q4_grouped_gemm.
hipError_t launch_grouped(int fmt, int layout, const uint16_t* A, int64_t lda, int64_t T,
                          const int32_t* gather, const int32_t* offsets, int32_t E, int64_t P,
                          const uint8_t* codes, const void* scales, const float* gs, int64_t N,
                          int64_t K, uint16_t* C, int64_t ldc, hipStream_t stream);

}  // namespace q4
