/*
 * q4.h -- C ABI of libq4.so: 4-bit absmax block quantization of bf16
 * weights (INT4 g128, MXFP4, NVFP4) and the W4 matmuls that consume them,
 * as hand-written HIP kernels for AMD gfx950 (MI355X).
 *
 * Formats (one row of K values is split into blocks of g along K):
 *   Q4_INT4_G128  codes -8..7 (4-bit two's complement), one fp16 scale per
 *                 128 values, scale = fp16(amax/7), code = clamp(rne(w/s)).
 *                 ("Quantization in deployment", format cheat sheet, W4A16
 *                 row; "Low-bit inference for very large MoE", fake_int4;
 *                 "Quantization chains", bits per weight: 4.125.)
 *   Q4_MXFP4      E2M1 codes (grid +-{0,0.5,1,1.5,2,3,4,6}), one E8M0
 *                 power-of-two scale per 32 values,
 *                 scale = 2^(floor(log2(max(amax,1e-12))) - 2).
 *                 ("Quantization in deployment", formats.py mxfp4(); 4.25 bits.)
 *   Q4_NVFP4      E2M1 codes, one E4M3 scale per 16 values plus one fp32
 *                 tensor scale gs = max(amax_tensor,1e-12)/2688;
 *                 block scale = E4M3(min(amax_b/6/gs, 448)), element
 *                 divided by E4M3(scale)*gs.  ("Quantization in deployment",
 *                 formats.py nvfp4(); "Quantization chains", NVFP4 vs MXFP4.)
 *   Q4_INT4_ZP_G128  INT4 with a zero point: codes -8..7 (4-bit two's
 *                 complement), per group of 128 one fp16 scale and one zero
 *                 point z (an integer code), value = (q - z) * scale; min-max
 *                 rounding over the group widened to include 0: lo =
 *                 min(min,0), hi = max(max,0), scale = fp16((hi-lo)/15),
 *                 z = clamp(-8 - rne(lo/scale), -8, 7), q = clamp(rne(w/
 *                 scale) + z, -8, 7).  ("Quantization in deployment",
 *                 format cheat sheet, W4A16 INT4 GPTQ/AWQ row: one scale
 *                 per 128 numbers plus a zero point.)  Scales are 32-bit
 *                 words: fp16 bits | (z & 0xFF) << 16.
 *   Q4_FP8_ROW    the activation operand of W4A8, not a weight format:
 *                 one E4M3 byte per value and one fp32 scale per row
 *                 (token), scale = max(amax_row,1e-12)/448, code =
 *                 E4M3(clamp(x/scale, +-448)).  ("Quantization in
 *                 deployment", formats.py fp8() per row; "Quantization
 *                 chains", "One outlier sets the scale".)
 * Every rounding is to nearest, ties to the even code; E2M1 and E4M3 keep
 * the sign bit of the input; a block whose stored scale is 0 has magnitude
 * codes 0.
 *
 * Layouts of a quantized tensor (q4_tensor); all device memory is owned by
 * the caller.  Within a byte, element k sits in bits 3:0 when k is even and
 * in bits 7:4 when k is odd.  INT4 codes are 4-bit two's complement; an
 * E2M1 code is sign*8 + index into {0,0.5,1,1.5,2,3,4,6}.
 *
 * Q4_LAYOUT_ROWS (row-major, dense):
 *   codes   uint8 [rows][cols/2], 16-byte aligned.
 *   scales  INT4: fp16 bits [rows][cols/128]; MXFP4: biased E8M0 exponent
 *           [rows][cols/32]; NVFP4: E4M3 bits [rows][cols/16]; INT4 with a
 *           zero point: 32-bit words [rows][cols/128].  4-byte aligned.
 *
 * Q4_LAYOUT_TILED (the weights pre-shuffled so that one 64-lane load is one
 * contiguous kilobyte holding a whole matrix-core operand; cols % 512 == 0).
 * Rows are grouped in tiles of 16 (RT = ceil(rows/16) tiles, the last one
 * padded), K in super-chunks of 128 (S = cols/128) and super-chunks in
 * groups of four (Q = S/4).  Lane index l = 16*g + n, n = row in the tile
 * (0..15), g = 32-wide k group in the super-chunk (0..3).
 *   codes   RT*S tiles of 1024 bytes; tile (t, s) starts at byte
 *           (t*S + s)*1024 and its bytes [16l, 16l+16) hold the 32 codes
 *           k = 128s + 32g + j (j = 0..31) of row 16t + n.
 *   scales  MXFP4: byte ((t*Q + q)*64 + l)*4 + i is the E8M0 of row 16t+n,
 *                  32-block 4(4q+i) + g                 (RT*Q*256 bytes);
 *           NVFP4: byte ((t*Q + q)*64 + l)*8 + 2i + h is the E4M3 of row
 *                  16t+n, 16-block 8(4q+i) + 2g + h    (RT*Q*512 bytes);
 *           INT4:  fp16 element ((t*Q + q)*16 + n)*4 + i is the scale of
 *                  row 16t+n, 128-group 4q + i          (RT*Q*128 bytes);
 *           INT4 with a zero point: the 32-bit word at the same element
 *                  index                                (RT*Q*256 bytes).
 *   Padding rows (16t+n >= rows) hold the quantization of zeros.
 *
 * Q4_FP8_ROW in the two layouts (cols % 16 == 0 row-major, % 512 tiled):
 *   row-major  codes uint8 [rows][cols] (E4M3 bytes, sign in bit 7).
 *   tiled      RT*S tiles of 2048 bytes, tile (t, s) at (t*S + s)*2048.
 *              Lane l = 16g + n owns 32 operand bytes of row 16t+n:
 *              operand byte 4d + i (dword d = 2w + h, w = 0..3, h = 0..1,
 *              i = 0..3) holds k = 128s + 32g + 8w + 2i + h.  Operand
 *              bytes 0..15 of lane l sit at tile byte 16l, operand bytes
 *              16..31 at 1024 + 16l.  Padding rows hold code 0.
 *   scales     fp32 [rows] in both layouts; global_scale is NULL.
 *
 *   global_scale  NVFP4 only: device fp32[1], the multiplier gs; else NULL.
 *
 * Conventions for every call:
 *   - Pointers named *_bf16 are device bf16 arrays; leading dimensions (ld*)
 *     are in elements, >= the row length, multiples of 8, and the base
 *     pointers 16-byte aligned.
 *   - `stream` is a hipStream_t (NULL = the default stream).  All device work
 *     is enqueued on it; the call returns after the launch, not after the
 *     work.  The library never allocates, frees or synchronizes.
 *   - Arguments are validated on the host before any HIP call; a bad
 *     argument returns its error code and launches nothing.  A failed launch
 *     returns Q4_ERR_HIP; q4_last_hip_error() gives the hipError_t of the
 *     calling thread's last failure.
 *   - Inputs must be finite.  Calls on distinct outputs may run
 *     concurrently; outputs must not alias inputs.
 *   - The first launch of a kernel that uses more than 64 KB of LDS on a
 *     device raises that kernel's LDS limit there (hipFuncSetAttribute, once
 *     per kernel and device); no other state is kept.
 */
#ifndef Q4_H
#define Q4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum q4_format {
    Q4_INT4_G128 = 0,
    Q4_MXFP4 = 1,
    Q4_NVFP4 = 2,
    Q4_FP8_ROW = 3,
    Q4_INT4_ZP_G128 = 4
} q4_format;

typedef enum q4_layout {
    Q4_LAYOUT_ROWS = 0,
    Q4_LAYOUT_TILED = 1
} q4_layout;

typedef enum q4_status {
    Q4_OK = 0,
    Q4_ERR_NULL = -1,   /* a required pointer is NULL                      */
    Q4_ERR_SHAPE = -2,  /* a size is negative, too large or not a multiple */
    Q4_ERR_ALIGN = -3,  /* a pointer or leading dimension is misaligned    */
    Q4_ERR_FORMAT = -4, /* unknown format, or a format the call rejects    */
    Q4_ERR_HIP = -6     /* the HIP launch failed; see q4_last_hip_error()  */
} q4_status;

typedef struct q4_tensor {
    int32_t fmt;          /* q4_format                                     */
    int32_t layout;       /* q4_layout                                     */
    int64_t rows;         /* N for weights, M for activations              */
    int64_t cols;         /* K, a multiple of the format's block size      */
    void* codes;          /* packed codes, see the layouts above           */
    void* scales;         /* block scales, see the layouts above           */
    float* global_scale;  /* NVFP4: fp32[1]; other formats: NULL           */
} q4_tensor;

/* Library version (major*100 + minor). */
int q4_version(void);

/* Static text for a q4_status value. */
const char* q4_status_string(int status);

/* hipError_t of the calling thread's last Q4_ERR_HIP (0 if none). */
int q4_last_hip_error(void);

/*
 * Bytes of codes and scales for a rows x cols tensor of format fmt in
 * layout `layout` ("Quantization chains", bits per weight: codes are 4 bits,
 * scales 16/128, 8/32 and 8/16 bits per value; the tiled layout adds the
 * padding of the last row tile).  Either output pointer may be NULL.
 * Q4_ERR_SHAPE if rows < 0, cols < 0 or cols is not a multiple of the block
 * (of 512 for the tiled layout); Q4_ERR_FORMAT for an unknown fmt/layout.
 */
q4_status q4_sizes(int fmt, int layout, int64_t rows, int64_t cols, size_t* codes_bytes,
                   size_t* scales_bytes);

/*
 * Moves a quantized tensor from one layout to the other (row-major <->
 * tiled, the layouts above), bit for bit: the same codes and scales at the
 * other layout's positions, the NVFP4 global scale copied.  Tiled padding
 * rows receive the quantization of zeros (as q4_quantize writes them).  The
 * GEMM kernels are built for the tiled layout (its fragments are contiguous
 * kilobytes; "Low-bit inference for very large MoE", "A few details":
 * pre-shuffled weights), so weights quantized or packed row-major are worth
 * converting once, when they are loaded.
 *   src, dst  the same fmt (not Q4_FP8_ROW: Q4_ERR_FORMAT), rows and cols
 *             (else Q4_ERR_SHAPE); each validated like any q4_tensor (the
 *             tiled one needs cols % 512 == 0).  Equal layouts: a copy.
 *   dst must not overlap src.  Empty tensors: only the NVFP4 global scale
 *   is copied.
 */
q4_status q4_relayout(const q4_tensor* src, const q4_tensor* dst, void* stream);

/*
 * Quantize a bf16 matrix src [dst->rows][ld] (first dst->cols columns) into
 * dst, by round-to-nearest absmax block quantization along each row
 * ("LLM quantization", the absmax method: the group's largest magnitude
 * sets the scale, every value is divided by it and rounded).
 * NVFP4: if nv_global_in (device fp32[1]) is not NULL its value is used as
 * gs; otherwise gs is computed from the whole matrix (one extra read pass)
 * and written to dst->global_scale.  nv_global_in must be NULL for the other
 * formats.  rows == 0 or cols == 0 is a no-op (for NVFP4 without
 * nv_global_in, gs is still written: max(0,1e-12)/2688).  Q4_FP8_ROW
 * quantizes each row with its own scale (the W4A8 activations).
 */
q4_status q4_quantize(const void* src_bf16, int64_t ld, const q4_tensor* dst,
                      const float* nv_global_in, void* stream);

/*
 * Dequantize src into dst [src->rows][ld]: value = fp32(code * scale) with
 * the scale as stored (NVFP4: scale = fp32(E4M3 * gs)).  dst_dtype 0 writes
 * bf16 (the fp32 value rounded to nearest even), 1 writes fp32 (ld a
 * multiple of 4 for fp32).  This is the step that multiplies the rounded
 * values back by their scale in the worked example of "LLM quantization".
 * Either layout is read; the output is always row-major.
 */
q4_status q4_dequant(const q4_tensor* src, void* dst, int dst_dtype, int64_t ld, void* stream);

/*
 * W4A16 GEMV for decode: y[b][n] = sum_k x[b][k] * w'[n][k] for b < B,
 * n < W->rows, w' the dequantized weight; fp32 accumulation, bf16 output
 * ("Low-bit inference for very large MoE", table "Kernels on different
 * hardware", row W4A16: weights dequantized in registers, 16-bit compute).
 * x_bf16 [B][ldx], y_bf16 [B][ldy].  1 <= B <= 16; K = W->cols must be a
 * multiple of 128.  B == 0 or W->rows == 0 is a no-op.
 */
q4_status q4_gemv(const q4_tensor* W, const void* x_bf16, int64_t B, int64_t ldx,
                  void* y_bf16, int64_t ldy, void* stream);

/*
 * GEMM C[m][n] = sum_k a'[m][k] * w'[n][k], fp32 accumulation, bf16 output
 * C_bf16 [M][ldc].  Exactly one of A_bf16 / A_q is given:
 *   A_bf16 [M][lda]  -> W4A16: W of any format dequantized to bf16 feeding
 *                       bf16 matrix cores (same table, row W4A16);
 *   A_q (MXFP4, rows M, cols K) with W MXFP4 -> W4A4: both operands enter
 *                       the block-scaled FP4 matrix cores directly (same
 *                       table, row W4A4);
 *   A_q (NVFP4, rows M, cols K) with W NVFP4 -> W4A4 NVFP4: each code times
 *                       its E4M3 block scale is exact in fp16, so both
 *                       operands are dequantized to fp16 in registers and
 *                       multiplied on fp16 matrix cores; the two tensor
 *                       scales are applied to the fp32 sum:
 *                       C = (sum_k (qa sa)(qw sw)) * gs_a * gs_w.  A_q's
 *                       global_scale is its own (q4_quantize of A computes
 *                       it from A's amax, or takes the caller's).  gfx950's
 *                       FP4 matrix cores take E8M0 scales per 32, which
 *                       cannot carry E4M3 per 16 ("Quantization in
 *                       deployment", cheat sheet, NVFP4 and MXFP4 rows);
 *   A_q (Q4_FP8_ROW, rows M, cols K) with W INT4 -> W4A8: the INT4 codes
 *                       become exact E4M3 values, the products run on FP8
 *                       matrix cores, and each 128-wide group's partial sum
 *                       is multiplied by its fp16 weight scale in fp32 (same
 *                       table, row W4A8; "Quantization in deployment", the
 *                       per-block promotion of block-scaled FP8 GEMMs);
 *                       C = s_a[m] * sum_g s_w[n][g] * sum_(k in g) a8*q.
 * Other format pairs, and a Q4_FP8_ROW W: Q4_ERR_FORMAT.
 * K = W->cols must be a multiple of 128.  M == 0 or N == 0 is a no-op.
 */
q4_status q4_gemm(int64_t M, const void* A_bf16, int64_t lda, const q4_tensor* A_q,
                  const q4_tensor* W, void* C_bf16, int64_t ldc, void* stream);

/*
 * The GEMM of q4_gemm with its output written quantized by the kernel's
 * epilogue: C_q receives exactly the codes and scales that q4_quantize(C_q)
 * writes for the bf16 C that q4_gemm writes (each fp32 sum rounded to bf16,
 * then block-quantized), and C is never written in bf16 nor read back.  This
 * is the activation quantization of the next W4A4 layer done at the end of
 * the kernel that produces the activations, which saves a pass that reads
 * and writes them ("Quantization in deployment", Exercises, "The cost of
 * block FP8": activation scales computed at the end of the previous kernel).
 *   C_q  MXFP4, or NVFP4 with the tensor scale taken from nv_global_in
 *        (device fp32[1]; required for NVFP4 and NULL otherwise; its value
 *        is also written to C_q->global_scale: an epilogue cannot wait for
 *        the amax of the whole output, so the scale is the caller's, e.g.
 *        a calibrated one).  C_q->rows == M, C_q->cols == N == W->rows,
 *        N % 32 == 0; either layout (tiled: N % 512 == 0, padding rows
 *        written as the quantization of zeros).
 *   Operands: A_bf16 [M][lda] with W of any weight format in the tiled
 *        layout (W4A16), or A_q MXFP4 tiled with W MXFP4 tiled (W4A4).
 *        Other combinations: Q4_ERR_FORMAT.
 * M == 0 or N == 0 is a no-op.  C_q must not alias the operands.
 */
q4_status q4_gemm_quantized(int64_t M, const void* A_bf16, int64_t lda, const q4_tensor* A_q,
                            const q4_tensor* W, const q4_tensor* C_q, const float* nv_global_in,
                            void* stream);

/*
 * Grouped per-expert GEMM for MoE ("Low-bit inference for very large MoE",
 * "A few details": one low-bit weight matrix per expert, rows grouped by
 * routing).  W holds E experts stacked expert-major: W->rows == E*N, expert
 * e owns rows [e*N, (e+1)*N).  For every expert e and every routed row p in
 * [expert_offsets[e], expert_offsets[e+1]):
 *     C[p][n] = sum_k A[gather[p]][k] * w'[e*N + n][k]
 * A_bf16 [T][lda] (T tokens), gather int32 [P] (device; NULL means the
 * identity, row p reads A[p], and needs T >= P), expert_offsets
 * int32 [E+1] (device, non-decreasing, offsets[0] = 0, offsets[E] = P),
 * C_bf16 [P][ldc].  The kernels read the offsets on the device (no host
 * sync) and clamp every range to [0, P]; a row whose gather index is outside
 * [0, T) is written as zeros.  K = W->cols must be a multiple of 128.
 */
q4_status q4_grouped_gemm(const void* A_bf16, int64_t lda, int64_t T, const int32_t* gather,
                          const int32_t* expert_offsets, int32_t E, int64_t P,
                          const q4_tensor* W, int64_t N, void* C_bf16, int64_t ldc,
                          void* stream);

/*
 * The steps of an MoE layer around q4_grouped_gemm ("Low-bit inference for
 * very large MoE", "A few details": one low-bit matrix per expert, tokens
 * grouped by routing).  A layer is
 *   q4_moe_route -> q4_grouped_gemm (gate/up: W rows [e*2I, (e+1)*2I) =
 *   [W_gate_e; W_up_e]) -> q4_swiglu -> q4_grouped_gemm (down: gather =
 *   0..P-1, W rows [e*K, (e+1)*K)) -> q4_moe_combine.
 */

/*
 * The gate/up expert GEMM with the SwiGLU activation fused into its
 * epilogue: for expert e and routed row p,
 *     H[p][n] = bf16(silu(sum_k a[k] w_gate_e[n][k]) * sum_k a[k] w_up_e[n][k])
 * with a = A[gather[p]] as in q4_grouped_gemm (NULL gather = identity).
 * W (tiled layout only, else Q4_ERR_FORMAT) holds 2I rows per expert that
 * alternate 16-row tiles of W_gate and W_up: rows e*2I + 32j + r are gate
 * row 16j + r and rows e*2I + 32j + 16 + r are up row 16j + r (r < 16);
 * I % 16 == 0.  H_bf16 [P][ldh].  Replaces q4_grouped_gemm + q4_swiglu
 * without writing the gate/up products.
 */
q4_status q4_grouped_gemm_swiglu(const void* A_bf16, int64_t lda, int64_t T, const int32_t* gather,
                                 const int32_t* expert_offsets, int32_t E, int64_t P,
                                 const q4_tensor* W, int64_t I, void* H_bf16, int64_t ldh,
                                 void* stream);

/*
 * Routing of T tokens over E experts from fp32 router logits [T][ld].
 * Token t's experts are its k largest logits, largest first, ties to the
 * lower expert id: topk_ids [T][k]; its gate for each is that expert's
 * softmax probability over all E logits (fp32, not renormalized):
 * topk_weights [T][k].  Routed rows are ordered expert-major and, within an
 * expert, by token: expert_offsets [E+1], gather [T*k] (token of each row)
 * and inv [T][k] (row of each choice).  All int32/fp32 device arrays, 4-byte
 * aligned.  1 <= E <= 1024, 1 <= k <= min(E, 32), and the dispatch runs in
 * one workgroup whose LDS holds a token bitmap per expert:
 * 8*E*(ceil(T/32) + 1) bytes <= 160 KB (E = 64: T <= 10208), else
 * Q4_ERR_SHAPE.  T == 0 writes expert_offsets = 0.  Logits compare as
 * values (-0 equal to +0); a NaN logit, outside the finite-input contract,
 * ranks above +inf (sign bit clear) or below -inf (set), so every token
 * still gets k distinct experts and every output index stays in range.
 */
q4_status q4_moe_route(const float* logits, int64_t ld, int64_t T, int32_t E, int32_t k,
                       int32_t* topk_ids, float* topk_weights, int32_t* expert_offsets,
                       int32_t* gather, int32_t* inv, void* stream);

/*
 * SwiGLU between the expert GEMMs: h[p][n] = bf16(silu(g) * u), g =
 * gu[p][n], u = gu[p][I + n], silu(z) = z / (1 + exp(-z)), fp32 math.
 * gu_bf16 [P][ld_gu] (ld_gu >= 2I), h_bf16 [P][ldh]; I % 8 == 0.
 */
q4_status q4_swiglu(const void* gu_bf16, int64_t ld_gu, int64_t P, int64_t I, void* h_bf16,
                    int64_t ldh, void* stream);

/*
 * Gated combine: out[t][n] = bf16(sum_j weights[t][j] * y[inv[t][j]][n]),
 * fp32 accumulation in choice order.  y_bf16 [P][ldy] (expert outputs in
 * routed-row order), inv/weights [T][k] as q4_moe_route writes them,
 * out_bf16 [T][ldo]; N % 8 == 0.
 */
q4_status q4_moe_combine(const void* y_bf16, int64_t ldy, const int32_t* inv, const float* weights,
                         int64_t T, int32_t k, int64_t N, void* out_bf16, int64_t ldo, void* stream);

/*
 * Measurement helper, not a step of the method: reads `bytes` of device
 * memory at src with a plain streaming kernel (16-byte non-temporal loads,
 * each wave 8 KB in flight) and discards the data.  Decode GEMVs are bound
 * by their weight reads ("Low-bit inference for very large MoE", table
 * "Kernels on different hardware", row W4A16), so timing this read on a
 * buffer of the weight's size gives the rate the GEMV can approach on this
 * part.  src 16-byte aligned, bytes a multiple of 1024 (else Q4_ERR_ALIGN /
 * Q4_ERR_SHAPE); sink: device uint32[1], written only if the folded data
 * equals one fixed 32-bit constant (which keeps the loads alive).
 * bytes == 0 is a no-op.
 */
q4_status q4_read_probe(const void* src, int64_t bytes, uint32_t* sink, void* stream);

/*
 * Measurement helper, not a step of the method: the rate at which this part
 * sustains one kind of matrix instruction, back to back, with operands in
 * registers -- the ceiling a GEMM built on that instruction can approach.
 * The operands are pseudo-random bits drawn from `seed` (as quantized data
 * is): with random operands the part lowers its clock to stay within its
 * power limit, so this rate lies below the published dense peak.
 *   kind   Q4_PROBE_FP4  scaled 16x16x128 with E2M1 operands (the W4A4
 *                        MXFP4 GEMM's instruction)
 *          Q4_PROBE_BF16 16x16x32 bf16 (GEMV, W4A16 GEMM, grouped GEMM)
 *          Q4_PROBE_F16  16x16x32 fp16 (the NVFP4 W4A4 GEMM)
 *          Q4_PROBE_FP8  scaled 16x16x128 with E4M3 operands (W4A8)
 *          Q4_PROBE_FP4_COPY  the FP4 instruction with one direct
 *                        global->LDS copy (1 KB per wave) issued per 8
 *                        instructions: the copy rate per SIMD of the tiled
 *                        W4A4 kernel
 *          Q4_PROBE_FP4_MIX   the same plus three 16-byte-per-lane LDS
 *                        fragment reads per 8 instructions: that kernel's
 *                        whole memory-instruction mix, so the rate its loop
 *                        can approach on this part
 *          Q4_PROBE_BF16_MIX  the bf16 instruction with the tiled W4A16
 *                        GEMM's mix on NVFP4 weights: per 16 instructions
 *                        one weight fragment dequantized (their row
 *                        operand), one copy and eight fragment reads
 *          other values: Q4_ERR_FORMAT
 *   iters  iterations of 8 instructions per wave, 0 .. 2^24 (else
 *          Q4_ERR_SHAPE); the launch runs two waves per SIMD on every
 *          compute unit; iters == 0 is a no-op (*flops = 0)
 *   sink   device uint32[1] (the three mix kinds: 16384 uint32, 16-byte
 *          aligned, else Q4_ERR_ALIGN -- the 64 KB the copies read; their
 *          contents do not matter), written only if the folded sums equal
 *          one fixed constant (which keeps the products alive)
 *   flops  host double: receives the floating-point operations the launch
 *          performs (2*16*16*K per instruction); NULL: Q4_ERR_NULL
 */
typedef enum q4_probe_kind {
    Q4_PROBE_FP4 = 0,
    Q4_PROBE_BF16 = 1,
    Q4_PROBE_F16 = 2,
    Q4_PROBE_FP8 = 3,
    Q4_PROBE_FP4_COPY = 4,
    Q4_PROBE_FP4_MIX = 5,
    Q4_PROBE_BF16_MIX = 6
} q4_probe_kind;

q4_status q4_mfma_probe(int32_t kind, int64_t iters, uint32_t seed, uint32_t* sink, double* flops,
                        void* stream);

#ifdef __cplusplus
}
#endif

#endif /* Q4_H */
