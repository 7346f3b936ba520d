// api.hip -- the C ABI of libq4.so (declared in include/q4.h): argument
// validation on the host, then one launcher per call.  No call allocates,
// frees or synchronizes; every error is returned before any HIP call.
#include "../../include/q4.h"

#include <hip/hip_runtime.h>

#include "q4_launch.h"

namespace {

thread_local int g_last_hip_error = 0;

constexpr int64_t kMaxDim = (int64_t)1 << 31;  // kernels index rows/cols in int

int block_of(int fmt) {
  switch (fmt) {
    case Q4_INT4_G128: return 128;
    case Q4_MXFP4: return 32;
    case Q4_NVFP4: return 16;
    case Q4_FP8_ROW: return 16;  // row-major rows are stored in 16-byte pieces
    case Q4_INT4_ZP_G128: return 128;
    default: return 0;
  }
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

q4_status hip_status(hipError_t e) {
  if (e == hipSuccess) return Q4_OK;
  g_last_hip_error = (int)e;
  return Q4_ERR_HIP;
}

// Validates a quantized tensor descriptor: known format and layout, sizes
// in range and multiples of the block (of 512 in the tiled layout), buffers
// present and aligned when the tensor is not empty.
q4_status check_tensor(const q4_tensor* t) {
  if (!t) return Q4_ERR_NULL;
  const int g = block_of(t->fmt);
  if (!g || (t->layout != Q4_LAYOUT_ROWS && t->layout != Q4_LAYOUT_TILED)) return Q4_ERR_FORMAT;
  if (t->rows < 0 || t->cols < 0 || t->rows >= kMaxDim || t->cols >= kMaxDim) return Q4_ERR_SHAPE;
  if (t->cols % (t->layout == Q4_LAYOUT_TILED ? 512 : g)) return Q4_ERR_SHAPE;
  if (t->fmt == Q4_NVFP4) {
    if (!t->global_scale) return Q4_ERR_NULL;
    if (!aligned(t->global_scale, 4)) return Q4_ERR_ALIGN;
  } else if (t->global_scale) {
    return Q4_ERR_FORMAT;
  }
  if (t->rows > 0 && t->cols > 0) {
    if (!t->codes || !t->scales) return Q4_ERR_NULL;
    if (!aligned(t->codes, 16) || !aligned(t->scales, 4)) return Q4_ERR_ALIGN;
  }
  return Q4_OK;
}

// A bf16 matrix argument: rows x cols with leading dimension ld.
q4_status check_bf16(const void* p, int64_t rows, int64_t cols, int64_t ld) {
  if (rows < 0 || cols < 0) return Q4_ERR_SHAPE;
  if (rows == 0 || cols == 0) return Q4_OK;
  if (!p) return Q4_ERR_NULL;
  if (ld < cols) return Q4_ERR_SHAPE;
  if (!aligned(p, 16) || ld % 8) return Q4_ERR_ALIGN;
  return Q4_OK;
}

// An output bf16 matrix written element by element (2-byte alignment).
q4_status check_out_bf16(const void* p, int64_t rows, int64_t cols, int64_t ld) {
  if (rows < 0 || cols < 0) return Q4_ERR_SHAPE;
  if (rows == 0 || cols == 0) return Q4_OK;
  if (!p) return Q4_ERR_NULL;
  if (ld < cols) return Q4_ERR_SHAPE;
  if (!aligned(p, 2)) return Q4_ERR_ALIGN;
  return Q4_OK;
}

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

}  // namespace

extern "C" {

int q4_version(void) { return 102; }

const char* q4_status_string(int status) {
  switch (status) {
    case Q4_OK: return "ok";
    case Q4_ERR_NULL: return "a required pointer is NULL";
    case Q4_ERR_SHAPE: return "invalid size (negative, too large or not a multiple of the block)";
    case Q4_ERR_ALIGN: return "misaligned pointer or leading dimension";
    case Q4_ERR_FORMAT: return "unknown or unsupported format for this call";
    case Q4_ERR_HIP: return "HIP launch failed (see q4_last_hip_error)";
    default: return "unknown status";
  }
}

int q4_last_hip_error(void) { return g_last_hip_error; }

q4_status q4_sizes(int fmt, int layout, int64_t rows, int64_t cols, size_t* codes_bytes,
                   size_t* scales_bytes) {
  const int g = block_of(fmt);
  if (!g || (layout != Q4_LAYOUT_ROWS && layout != Q4_LAYOUT_TILED)) return Q4_ERR_FORMAT;
  if (rows < 0 || cols < 0 || rows >= kMaxDim || cols >= kMaxDim) return Q4_ERR_SHAPE;
  if (cols % (layout == Q4_LAYOUT_TILED ? 512 : g)) return Q4_ERR_SHAPE;
  // the tiled layout stores whole 16-row tiles; per stored row both layouts
  // hold cols/2 code bytes and cols/g scales (fp16 for INT4)
  const size_t srows = layout == Q4_LAYOUT_TILED ? (size_t)((rows + 15) / 16) * 16 : (size_t)rows;
  if (fmt == Q4_FP8_ROW) {  // one byte per value, one fp32 scale per row
    if (codes_bytes) *codes_bytes = srows * (size_t)cols;
    if (scales_bytes) *scales_bytes = (size_t)rows * 4;
    return Q4_OK;
  }
  if (codes_bytes) *codes_bytes = srows * (size_t)cols / 2;
  if (scales_bytes)
    *scales_bytes = srows * (size_t)(cols / g) * (fmt == Q4_INT4_G128 ? 2 : fmt == Q4_INT4_ZP_G128 ? 4 : 1);
  return Q4_OK;
}

q4_status q4_quantize(const void* src_bf16, int64_t ld, const q4_tensor* dst,
                      const float* nv_global_in, void* stream) {
  q4_status st = check_tensor(dst);
  if (st != Q4_OK) return st;
  if (nv_global_in && dst->fmt != Q4_NVFP4) return Q4_ERR_FORMAT;
  if (nv_global_in && !aligned(nv_global_in, 4)) return Q4_ERR_ALIGN;
  st = check_bf16(src_bf16, dst->rows, dst->cols, ld);
  if (st != Q4_OK) return st;
  if (dst->fmt != Q4_NVFP4 && (dst->rows == 0 || dst->cols == 0)) return Q4_OK;
  if (dst->fmt == Q4_FP8_ROW)
    return hip_status(q4::launch_fp8_rows_quantize(dst->layout, static_cast<const uint16_t*>(src_bf16), ld,
                                                   dst->rows, dst->cols, static_cast<uint8_t*>(dst->codes),
                                                   static_cast<float*>(dst->scales), as_stream(stream)));
  return hip_status(q4::launch_quantize(
      dst->fmt, dst->layout, static_cast<const uint16_t*>(src_bf16), ld, dst->rows, dst->cols,
      static_cast<uint8_t*>(dst->codes), dst->scales, dst->global_scale, nv_global_in,
      as_stream(stream)));
}

q4_status q4_dequant(const q4_tensor* src, void* dst, int dst_dtype, int64_t ld, void* stream) {
  q4_status st = check_tensor(src);
  if (st != Q4_OK) return st;
  if (dst_dtype != 0 && dst_dtype != 1) return Q4_ERR_FORMAT;
  if (src->rows == 0 || src->cols == 0) return Q4_OK;
  if (!dst) return Q4_ERR_NULL;
  if (ld < src->cols) return Q4_ERR_SHAPE;
  if (!aligned(dst, 16) || ld % (dst_dtype == 0 ? 8 : 4)) return Q4_ERR_ALIGN;
  if (src->fmt == Q4_FP8_ROW)
    return hip_status(q4::launch_fp8_rows_dequant(src->layout, static_cast<const uint8_t*>(src->codes),
                                                  static_cast<const float*>(src->scales), src->rows,
                                                  src->cols, dst, dst_dtype, ld, as_stream(stream)));
  return hip_status(q4::launch_dequant(src->fmt, src->layout, static_cast<const uint8_t*>(src->codes),
                                       src->scales, src->global_scale, src->rows, src->cols, dst,
                                       dst_dtype, ld, as_stream(stream)));
}

q4_status q4_relayout(const q4_tensor* src, const q4_tensor* dst, void* stream) {
  q4_status st = check_tensor(src);
  if (st != Q4_OK) return st;
  st = check_tensor(dst);
  if (st != Q4_OK) return st;
  if (src->fmt != dst->fmt || src->fmt == Q4_FP8_ROW) return Q4_ERR_FORMAT;
  if (src->rows != dst->rows || src->cols != dst->cols) return Q4_ERR_SHAPE;
  hipStream_t s = as_stream(stream);
  if (src->fmt == Q4_NVFP4 && (src->rows == 0 || src->cols == 0 || src->layout == dst->layout)) {
    const hipError_t e = hipMemcpyAsync(dst->global_scale, src->global_scale, 4, hipMemcpyDeviceToDevice, s);
    if (e != hipSuccess) return hip_status(e);
  }
  if (src->rows == 0 || src->cols == 0) return Q4_OK;
  if (src->layout == dst->layout) {  // same layout: a copy
    size_t cb = 0, sb = 0;
    st = q4_sizes(src->fmt, src->layout, src->rows, src->cols, &cb, &sb);
    if (st != Q4_OK) return st;
    hipError_t e = hipMemcpyAsync(dst->codes, src->codes, cb, hipMemcpyDeviceToDevice, s);
    if (e == hipSuccess) e = hipMemcpyAsync(dst->scales, src->scales, sb, hipMemcpyDeviceToDevice, s);
    return hip_status(e);
  }
  return hip_status(q4::launch_relayout(src->fmt, dst->layout, static_cast<const uint8_t*>(src->codes), src->scales,
                                        src->global_scale, static_cast<uint8_t*>(dst->codes), dst->scales,
                                        dst->global_scale, src->rows, src->cols, s));
}

q4_status q4_gemv(const q4_tensor* W, const void* x_bf16, int64_t B, int64_t ldx, void* y_bf16,
                  int64_t ldy, void* stream) {
  q4_status st = check_tensor(W);
  if (st != Q4_OK) return st;
  if (W->fmt == Q4_FP8_ROW) return Q4_ERR_FORMAT;
  if (B < 0 || B > 16) return Q4_ERR_SHAPE;
  if (W->cols % 128) return Q4_ERR_SHAPE;
  if (B == 0 || W->rows == 0) return Q4_OK;
  if (W->cols == 0) return Q4_ERR_SHAPE;
  st = check_bf16(x_bf16, B, W->cols, ldx);
  if (st != Q4_OK) return st;
  st = check_out_bf16(y_bf16, B, W->rows, ldy);
  if (st != Q4_OK) return st;
  return hip_status(q4::launch_gemv(W->fmt, W->layout, static_cast<const uint8_t*>(W->codes), W->scales,
                                    W->global_scale, W->rows, W->cols,
                                    static_cast<const uint16_t*>(x_bf16), ldx, B,
                                    static_cast<uint16_t*>(y_bf16), ldy, as_stream(stream)));
}

q4_status q4_gemm(int64_t M, const void* A_bf16, int64_t lda, const q4_tensor* A_q,
                  const q4_tensor* W, void* C_bf16, int64_t ldc, void* stream) {
  q4_status st = check_tensor(W);
  if (st != Q4_OK) return st;
  if (W->fmt == Q4_FP8_ROW) return Q4_ERR_FORMAT;
  if (M < 0 || M >= kMaxDim || M > (int64_t)65535 * 64) return Q4_ERR_SHAPE;
  if ((A_bf16 == nullptr) == (A_q == nullptr)) return A_bf16 ? Q4_ERR_FORMAT : Q4_ERR_NULL;
  const int64_t N = W->rows, K = W->cols;
  if (K % 128) return Q4_ERR_SHAPE;
  if (A_q) {
    st = check_tensor(A_q);
    if (st != Q4_OK) return st;
    const bool w4a4 = A_q->fmt == W->fmt && (W->fmt == Q4_MXFP4 || W->fmt == Q4_NVFP4);
    const bool w4a8 = A_q->fmt == Q4_FP8_ROW && W->fmt == Q4_INT4_G128;
    if (!w4a4 && !w4a8) return Q4_ERR_FORMAT;
    if (A_q->rows != M || A_q->cols != K) return Q4_ERR_SHAPE;
  }
  if (M == 0 || N == 0) return Q4_OK;
  if (K == 0) return Q4_ERR_SHAPE;
  if (!A_q) {
    st = check_bf16(A_bf16, M, K, lda);
    if (st != Q4_OK) return st;
  }
  st = check_out_bf16(C_bf16, M, N, ldc);
  if (st != Q4_OK) return st;
  if (A_q && A_q->fmt == Q4_FP8_ROW)
    return hip_status(q4::launch_gemm_w4a8(
        A_q->layout, W->layout, static_cast<const uint8_t*>(A_q->codes), static_cast<const float*>(A_q->scales),
        M, static_cast<const uint8_t*>(W->codes), static_cast<const uint16_t*>(W->scales), N, K,
        static_cast<uint16_t*>(C_bf16), ldc, as_stream(stream)));
  if (A_q && A_q->fmt == Q4_NVFP4)
    return hip_status(q4::launch_gemm_w4a4_nvfp4(
        A_q->layout, W->layout, static_cast<const uint8_t*>(A_q->codes), static_cast<const uint8_t*>(A_q->scales),
        A_q->global_scale, M, static_cast<const uint8_t*>(W->codes), static_cast<const uint8_t*>(W->scales),
        W->global_scale, N, K, static_cast<uint16_t*>(C_bf16), ldc, as_stream(stream)));
  if (A_q)
    return hip_status(q4::launch_gemm_w4a4(
        A_q->layout, W->layout, static_cast<const uint8_t*>(A_q->codes), static_cast<const uint8_t*>(A_q->scales), M,
        static_cast<const uint8_t*>(W->codes), static_cast<const uint8_t*>(W->scales), N, K,
        static_cast<uint16_t*>(C_bf16), ldc, as_stream(stream)));
  return hip_status(q4::launch_gemm_w4a16(W->fmt, W->layout, static_cast<const uint8_t*>(W->codes),
                                          W->scales, W->global_scale, N, K,
                                          static_cast<const uint16_t*>(A_bf16), lda, M,
                                          static_cast<uint16_t*>(C_bf16), ldc,
                                          as_stream(stream)));
}

q4_status q4_gemm_quantized(int64_t M, const void* A_bf16, int64_t lda, const q4_tensor* A_q,
                            const q4_tensor* W, const q4_tensor* C_q, const float* nv_global_in,
                            void* stream) {
  q4_status st = check_tensor(W);
  if (st != Q4_OK) return st;
  st = check_tensor(C_q);
  if (st != Q4_OK) return st;
  if (W->fmt == Q4_FP8_ROW || W->layout != Q4_LAYOUT_TILED) return Q4_ERR_FORMAT;
  if (C_q->fmt != Q4_MXFP4 && C_q->fmt != Q4_NVFP4) return Q4_ERR_FORMAT;
  if (C_q->fmt == Q4_NVFP4) {
    if (!nv_global_in) return Q4_ERR_NULL;
    if (!aligned(nv_global_in, 4)) return Q4_ERR_ALIGN;
  } else if (nv_global_in) {
    return Q4_ERR_FORMAT;
  }
  if (M < 0 || M >= kMaxDim || M > (int64_t)65535 * 64) return Q4_ERR_SHAPE;
  if ((A_bf16 == nullptr) == (A_q == nullptr)) return A_bf16 ? Q4_ERR_FORMAT : Q4_ERR_NULL;
  const int64_t N = W->rows, K = W->cols;
  if (C_q->rows != M || C_q->cols != N || N % 32) return Q4_ERR_SHAPE;
  if (A_q) {
    st = check_tensor(A_q);
    if (st != Q4_OK) return st;
    if (A_q->fmt != Q4_MXFP4 || W->fmt != Q4_MXFP4 || A_q->layout != Q4_LAYOUT_TILED) return Q4_ERR_FORMAT;
    if (A_q->rows != M || A_q->cols != K) return Q4_ERR_SHAPE;
  }
  if (M == 0 || N == 0) return Q4_OK;
  if (K == 0) return Q4_ERR_SHAPE;
  if (!A_q) {
    st = check_bf16(A_bf16, M, K, lda);
    if (st != Q4_OK) return st;
  }
  const q4::QOut qo{static_cast<uint8_t*>(C_q->codes), static_cast<uint8_t*>(C_q->scales), nv_global_in,
                    C_q->global_scale, C_q->layout == Q4_LAYOUT_TILED ? 1 : 0};
  const int out = C_q->fmt == Q4_MXFP4 ? q4::kOutMxfp4 : q4::kOutNvfp4;
  if (A_q)
    return hip_status(q4::launch_gemm_w4a4_tiled_qout(
        out, static_cast<const uint8_t*>(A_q->codes), static_cast<const uint8_t*>(A_q->scales), M,
        static_cast<const uint8_t*>(W->codes), static_cast<const uint8_t*>(W->scales), N, K, qo,
        as_stream(stream)));
  return hip_status(q4::launch_gemm_w4a16_tiled_qout(W->fmt, out, static_cast<const uint8_t*>(W->codes),
                                                     W->scales, W->global_scale, N, K,
                                                     static_cast<const uint16_t*>(A_bf16), lda, M, qo,
                                                     as_stream(stream)));
}

q4_status q4_grouped_gemm(const void* A_bf16, int64_t lda, int64_t T, const int32_t* gather,
                          const int32_t* expert_offsets, int32_t E, int64_t P,
                          const q4_tensor* W, int64_t N, void* C_bf16, int64_t ldc,
                          void* stream) {
  q4_status st = check_tensor(W);
  if (st != Q4_OK) return st;
  if (W->fmt == Q4_FP8_ROW) return Q4_ERR_FORMAT;
  if (E < 0 || E > 65535 || N < 0 || T < 0 || P < 0 || P >= kMaxDim || T >= kMaxDim)
    return Q4_ERR_SHAPE;
  if (W->rows != (int64_t)E * N) return Q4_ERR_SHAPE;
  if (W->layout == Q4_LAYOUT_TILED && N % 16) return Q4_ERR_SHAPE;  // experts own whole tiles
  const int64_t K = W->cols;
  if (K % 128) return Q4_ERR_SHAPE;
  if (E == 0 || N == 0 || P == 0) return Q4_OK;
  if (K == 0) return Q4_ERR_SHAPE;
  if (!expert_offsets) return Q4_ERR_NULL;
  if (!gather && T < P) return Q4_ERR_SHAPE;  // identity gather reads rows 0..P-1 of A
  if ((gather && !aligned(gather, 4)) || !aligned(expert_offsets, 4)) return Q4_ERR_ALIGN;
  st = check_bf16(A_bf16, T, K, lda);
  if (st != Q4_OK) return st;
  st = check_out_bf16(C_bf16, P, N, ldc);
  if (st != Q4_OK) return st;
  return hip_status(q4::launch_grouped(W->fmt, W->layout, static_cast<const uint16_t*>(A_bf16), lda, T,
                                       gather, expert_offsets, E, P,
                                       static_cast<const uint8_t*>(W->codes), W->scales,
                                       W->global_scale, N, K, static_cast<uint16_t*>(C_bf16),
                                       ldc, as_stream(stream)));
}

q4_status q4_grouped_gemm_swiglu(const void* A_bf16, int64_t lda, int64_t T, const int32_t* gather,
                                 const int32_t* expert_offsets, int32_t E, int64_t P, const q4_tensor* W,
                                 int64_t I, void* H_bf16, int64_t ldh, void* stream) {
  q4_status st = check_tensor(W);
  if (st != Q4_OK) return st;
  if (W->fmt == Q4_FP8_ROW || W->layout != Q4_LAYOUT_TILED) return Q4_ERR_FORMAT;
  if (E < 0 || E > 65535 || I < 0 || T < 0 || P < 0 || P >= kMaxDim || T >= kMaxDim) return Q4_ERR_SHAPE;
  if (I % 16 || W->rows != (int64_t)E * 2 * I) return Q4_ERR_SHAPE;
  const int64_t K = W->cols;
  if (E == 0 || I == 0 || P == 0) return Q4_OK;
  if (K == 0 || T == 0) return Q4_ERR_SHAPE;
  if (!expert_offsets) return Q4_ERR_NULL;
  if (!gather && T < P) return Q4_ERR_SHAPE;
  if ((gather && !aligned(gather, 4)) || !aligned(expert_offsets, 4)) return Q4_ERR_ALIGN;
  st = check_bf16(A_bf16, T, K, lda);
  if (st != Q4_OK) return st;
  st = check_bf16(H_bf16, P, I, ldh);
  if (st != Q4_OK) return st;
  return hip_status(q4::launch_grouped_tiled_swiglu(
      W->fmt, static_cast<const uint16_t*>(A_bf16), lda, T, gather, expert_offsets, E, P,
      static_cast<const uint8_t*>(W->codes), W->scales, W->global_scale, 2 * I, K, static_cast<uint16_t*>(H_bf16),
      ldh, as_stream(stream)));
}

q4_status q4_moe_route(const float* logits, int64_t ld, int64_t T, int32_t E, int32_t k, int32_t* topk_ids,
                       float* topk_weights, int32_t* expert_offsets, int32_t* gather, int32_t* inv,
                       void* stream) {
  if (T < 0 || T >= kMaxDim || E < 1 || E > 1024 || k < 1 || k > 32 || k > E) return Q4_ERR_SHAPE;
  if (q4::moe_dispatch_lds_bytes(T, E) > q4::kMoeDispatchMaxLds) return Q4_ERR_SHAPE;
  if (!expert_offsets) return Q4_ERR_NULL;
  if (!aligned(expert_offsets, 4)) return Q4_ERR_ALIGN;
  if (T > 0) {
    if (!logits || !topk_ids || !topk_weights || !gather || !inv) return Q4_ERR_NULL;
    if (ld < E) return Q4_ERR_SHAPE;
    if (!aligned(logits, 4) || !aligned(topk_ids, 4) || !aligned(topk_weights, 4) || !aligned(gather, 4) ||
        !aligned(inv, 4))
      return Q4_ERR_ALIGN;
  }
  return hip_status(q4::launch_moe_route(logits, ld, T, E, k, topk_ids, topk_weights, expert_offsets, gather,
                                         inv, as_stream(stream)));
}

q4_status q4_swiglu(const void* gu_bf16, int64_t ld_gu, int64_t P, int64_t I, void* h_bf16, int64_t ldh,
                    void* stream) {
  if (P < 0 || I < 0 || P >= kMaxDim || I >= kMaxDim) return Q4_ERR_SHAPE;
  if (I % 8) return Q4_ERR_SHAPE;
  if (P == 0 || I == 0) return Q4_OK;
  q4_status st = check_bf16(gu_bf16, P, 2 * I, ld_gu);
  if (st != Q4_OK) return st;
  st = check_bf16(h_bf16, P, I, ldh);
  if (st != Q4_OK) return st;
  return hip_status(q4::launch_swiglu(static_cast<const uint16_t*>(gu_bf16), ld_gu, P, I,
                                      static_cast<uint16_t*>(h_bf16), ldh, as_stream(stream)));
}

q4_status q4_moe_combine(const void* y_bf16, int64_t ldy, const int32_t* inv, const float* weights, int64_t T,
                         int32_t k, int64_t N, void* out_bf16, int64_t ldo, void* stream) {
  if (T < 0 || N < 0 || T >= kMaxDim || N >= kMaxDim || k < 1 || k > 32) return Q4_ERR_SHAPE;
  if (N % 8) return Q4_ERR_SHAPE;
  if (T == 0 || N == 0) return Q4_OK;
  if (!inv || !weights) return Q4_ERR_NULL;
  if (!aligned(inv, 4) || !aligned(weights, 4)) return Q4_ERR_ALIGN;
  q4_status st = check_bf16(y_bf16, 1, N, ldy);
  if (st != Q4_OK) return st;
  st = check_bf16(out_bf16, T, N, ldo);
  if (st != Q4_OK) return st;
  return hip_status(q4::launch_moe_combine(static_cast<const uint16_t*>(y_bf16), ldy, inv, weights, T, k, N,
                                           static_cast<uint16_t*>(out_bf16), ldo, as_stream(stream)));
}

q4_status q4_mfma_probe(int32_t kind, int64_t iters, uint32_t seed, uint32_t* sink, double* flops,
                        void* stream) {
  if (kind < Q4_PROBE_FP4 || kind > Q4_PROBE_BF16_MIX) return Q4_ERR_FORMAT;
  if (iters < 0 || iters > ((int64_t)1 << 24)) return Q4_ERR_SHAPE;
  if (!flops) return Q4_ERR_NULL;
  *flops = 0.0;
  if (iters == 0) return Q4_OK;
  if (!sink) return Q4_ERR_NULL;
  // the instruction-mix kinds copy 16 bytes per lane from the sink window
  if (!aligned(sink, kind >= Q4_PROBE_FP4_COPY ? 16 : 4)) return Q4_ERR_ALIGN;
  const int grid = q4::mfma_probe_grid();
  if (grid <= 0) return hip_status(hipErrorInvalidDevice);
  const double per = (kind == Q4_PROBE_BF16 || kind == Q4_PROBE_F16 || kind == Q4_PROBE_BF16_MIX)
                         ? 2.0 * 16 * 16 * 32 : 2.0 * 16 * 16 * 128;
  const q4_status st = hip_status(q4::launch_mfma_probe(kind, iters, seed, sink, grid, as_stream(stream)));
  if (st == Q4_OK) *flops = (double)grid * 4 * 8 * (double)iters * per;
  return st;
}

q4_status q4_read_probe(const void* src, int64_t bytes, uint32_t* sink, void* stream) {
  if (bytes < 0 || bytes % 1024) return Q4_ERR_SHAPE;
  if (bytes == 0) return Q4_OK;
  if (!src || !sink) return Q4_ERR_NULL;
  if (!aligned(src, 16) || !aligned(sink, 4)) return Q4_ERR_ALIGN;
  return hip_status(q4::launch_read_probe(static_cast<const uint8_t*>(src), bytes, sink, as_stream(stream)));
}

}  // extern "C"
