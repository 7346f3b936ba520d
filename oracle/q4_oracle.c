/*
 * q4_oracle.c -- plain, slow, obviously correct CPU reference for 4-bit
 * absmax block quantization (INT4 g128, MXFP4, NVFP4) and dequantization.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or constant with the HIP library; it is written from the
 * pages' statement of each format:
 *
 *   - "Low-bit inference for very large MoE" (anrans ai-infra-handbooks),
 *     section "Why quantization-aware training", function fake_int4:
 *     symmetric INT4, one scale per group of input channels, scale = amax/7,
 *     codes = round(w/scale) clamped to -8..7.
 *   - "Quantization in deployment" (anrans ai-infra-handbooks), section
 *     "Fake quantization", formats.py: the E2M1 value grid
 *     {0,0.5,1,1.5,2,3,4,6}, fp4() (clamp x/scale to +-6, nearest grid
 *     value), mxfp4() (block 32, scale 2^(floor(log2 amax)-2), amax clamped
 *     at 1e-12), nvfp4() (block 16, global scale amax/(448*6), E4M3 block
 *     scale of amax_b/6/global), and the format cheat sheet (INT4 -8..7 with
 *     one scale per 128; E8M0 per 32; E4M3 per 16 plus an FP32 tensor scale).
 *   - "Quantization chains" (inferenceinterviews.com), sections "Bits per
 *     weight", "E4M3 against E5M2" (max 448, min normal 2^-6, min subnormal
 *     2^-9) and "MXFP4 against NVFP4 scales".
 *   - for the W4A8 activations: "Quantization in deployment", formats.py
 *     fp8() / fp8_per_row() (one E4M3 scale per token, amax / 448, clamp to
 *     +-448), and "Quantization chains", "One outlier sets the scale".
 *
 * Readings where the pages leave a step open (each one is listed with its
 * justification in the design notes of the repository):
 *   - every rounding to a narrow format is round-to-nearest, ties to the
 *     code whose last bit is even (the chains page checks its examples with
 *     a round-to-nearest-even library; fake_int4 uses torch.round, which is
 *     half-to-even).  The formats.py fp4() argmin would send exact E2M1
 *     ties toward zero; set_ties_toward_zero(1) reproduces that in the E2M1
 *     encoder only, for tests (formats.py's E4M3 cast keeps ties to even);
 *   - the element is divided by the scale as stored (fp16 for INT4, 2^e for
 *     MXFP4, fp32(E4M3 * global) for NVFP4), as nvfp4() does;
 *   - an INT4 block whose fp16 scale is 0, and an NVFP4 block whose E4M3
 *     scale is 0, store scale 0 and magnitude codes 0;
 *   - the E2M1 sign bit is the sign bit of the input (so -0.0 and small
 *     negatives give code 0x8);
 *   - codes are packed two per byte, even k in bits 3:0, odd k in bits 7:4;
 *     INT4 codes are 4-bit two's complement; an E2M1 code is
 *     sign*8 + index into the grid above;
 *   - scales are stored row-major [rows][cols/g] as raw bytes (fp16 bits for
 *     INT4, the biased E8M0 exponent for MXFP4, E4M3 bits for NVFP4) and the
 *     NVFP4 global scale as the fp32 dequantization multiplier.
 *
 * Arithmetic: every step the GPU must reproduce bit for bit is done in fp32
 * (IEEE, round-to-nearest-even, no contraction: build with
 * -ffp-contract=off on x86-64 SSE).  Inputs are fp32 arrays; bf16 inputs
 * are converted to fp32 exactly by the caller.
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Value tables of the narrow formats, built by decoding every code from its  */
/* bit fields.  Each table is strictly increasing in the code.                */
/* ------------------------------------------------------------------------ */

/* E2M1 magnitudes: the grid printed in the format cheat sheet. */
static const float E2M1_GRID[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};

/* E4M3 ("fn": bias 7, 3 mantissa bits, no infinities, 0x7F is NaN).
 * Codes 0..126 are the finite non-negative values. */
static double e4m3_value(int code)
{
    int e = (code >> 3) & 0xF;
    int m = code & 0x7;
    if (e == 0)
        return ldexp((double)m / 8.0, 1 - 7); /* subnormal: 0.m * 2^-6 */
    return ldexp(1.0 + (double)m / 8.0, e - 7);
}

/* FP16 (IEEE binary16): codes 0..0x7BFF are the finite non-negative values. */
static double fp16_value(int code)
{
    int e = (code >> 10) & 0x1F;
    int m = code & 0x3FF;
    if (e == 0)
        return ldexp((double)m / 1024.0, 1 - 15);
    return ldexp(1.0 + (double)m / 1024.0, e - 15);
}

static int g_ties_toward_zero = 0;

void oracle_set_ties_toward_zero(int on) { g_ties_toward_zero = on ? 1 : 0; }

/* Nearest entry of an increasing table to v (v >= table[0]); on an exact
 * tie between two neighbours, the even code.  Distances are computed in
 * double, where they are exact for every fp32 v and every table value used
 * here.  (The test-only tie switch does not reach this search: formats.py
 * rounds E4M3 with torch's float8_e4m3fn cast, which is round-to-nearest
 * with ties to even; only its fp4() rounds by an argmin.) */
static int nearest_code(double v, double (*value)(int), int ncodes)
{
    int lo = 0, hi = ncodes - 1;
    if (v >= value(hi))
        return hi;
    /* binary search: value(lo) <= v < value(hi) */
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (value(mid) <= v)
            lo = mid;
        else
            hi = mid;
    }
    double dlo = v - value(lo);
    double dhi = value(hi) - v;
    if (dlo < dhi)
        return lo;
    if (dhi < dlo)
        return hi;
    return (lo % 2 == 0) ? lo : hi;
}

static double e2m1_value(int code) { return (double)E2M1_GRID[code]; }

/* E2M1 magnitude code of a in [0, 6]. */
int oracle_e2m1_code(float a)
{
    /* Brute force over the eight grid values: nearest, ties to even code. */
    int best = 0;
    double bestd = fabs((double)a - e2m1_value(0));
    for (int c = 1; c < 8; ++c) {
        double d = fabs((double)a - e2m1_value(c));
        if (d < bestd) {
            best = c;
            bestd = d;
        } else if (d == bestd && !g_ties_toward_zero && (c % 2 == 0)) {
            best = c;
        }
    }
    return best;
}

float oracle_e2m1_value(int code)
{
    float v = E2M1_GRID[code & 7];
    return (code & 8) ? -v : v;
}

/* E4M3 code (sign 0) of t >= 0, t <= 448 after the caller's clamp. */
int oracle_e4m3_code(float t) { return nearest_code((double)t, e4m3_value, 127); }
float oracle_e4m3_value(int code) { return (float)e4m3_value(code & 0x7F); }

/* FP16 code (sign 0) of t >= 0.  Values past the largest finite fp16 are
 * rounded against the next power of two (65536) as IEEE does, and become
 * +inf (0x7C00) when they reach it. */
int oracle_fp16_code(float t)
{
    if ((double)t >= 65520.0) /* midpoint of 65504 and 65536: even -> inf */
        return 0x7C00;
    return nearest_code((double)t, fp16_value, 0x7C00);
}
float oracle_fp16_value(int code)
{
    if ((code & 0x7FFF) == 0x7C00)
        return (code & 0x8000) ? -INFINITY : INFINITY;
    float v = (float)fp16_value(code & 0x7FFF);
    return (code & 0x8000) ? -v : v;
}

/* fp32 -> bf16, round to nearest even on the top 16 bits (finite inputs). */
uint16_t oracle_f32_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7FFFu + lsb;
    return (uint16_t)(u >> 16);
}

static int signbit_f(float x)
{
    uint32_t u;
    memcpy(&u, &x, 4);
    return (int)(u >> 31);
}

static void put_nibble(uint8_t* row_codes, int64_t k, int nib)
{
    uint8_t* b = &row_codes[k / 2];
    if (k % 2 == 0)
        *b = (uint8_t)((*b & 0xF0) | (nib & 0xF));
    else
        *b = (uint8_t)((*b & 0x0F) | ((nib & 0xF) << 4));
}

static int get_nibble(const uint8_t* row_codes, int64_t k)
{
    uint8_t b = row_codes[k / 2];
    return (k % 2 == 0) ? (b & 0xF) : (b >> 4);
}

/* ------------------------------------------------------------------------ */
/* INT4, one fp16 scale per group of g values along a row (g = 128).         */
/* Generic in qmax so the same absmax rule can be checked with qmax = 127.   */
/* ------------------------------------------------------------------------ */

/* Symmetric absmax rounding of one group: returns the fp16 scale code and
 * writes the integer codes (clamped to [-qmax-1, qmax]). */
int oracle_absmax_int_group(const float* w, int64_t n, int qmax, int32_t* q_out)
{
    float amax = 0.0f;
    for (int64_t i = 0; i < n; ++i) {
        float a = fabsf(w[i]);
        if (a > amax)
            amax = a;
    }
    float s32 = amax / (float)qmax;      /* fp32 division */
    int s_code = oracle_fp16_code(s32);  /* scale stored in fp16 */
    float s = oracle_fp16_value(s_code);
    for (int64_t i = 0; i < n; ++i) {
        if (s == 0.0f) {
            q_out[i] = 0;
            continue;
        }
        float r = w[i] / s;               /* divide by the stored scale */
        float qr = rintf(r);              /* half-to-even (default mode) */
        if (qr > (float)qmax)
            qr = (float)qmax;
        if (qr < (float)(-qmax - 1))
            qr = (float)(-qmax - 1);
        q_out[i] = (int32_t)qr;
    }
    return s_code;
}

int oracle_quantize_int4(const float* w, int64_t rows, int64_t cols, int64_t ld, int64_t g,
                         uint8_t* codes, uint16_t* scales)
{
    if (g <= 0 || cols % g != 0 || cols % 2 != 0 || g > 4096)
        return -1;
    int64_t nb = cols / g;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        int32_t q[4096];
        uint8_t* rc = codes + r * (cols / 2);
        for (int64_t b = 0; b < nb; ++b) {
            int s_code = oracle_absmax_int_group(w + r * ld + b * g, g, 7, q);
            scales[r * nb + b] = (uint16_t)s_code;
            for (int64_t i = 0; i < g; ++i)
                put_nibble(rc, b * g + i, q[i] & 0xF);
        }
    }
    return 0;
}

void oracle_dequant_int4(const uint8_t* codes, const uint16_t* scales, int64_t rows, int64_t cols,
                         int64_t g, float* out)
{
    int64_t nb = cols / g;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t k = 0; k < cols; ++k) {
            int nib = get_nibble(codes + r * (cols / 2), k);
            int q = (nib >= 8) ? nib - 16 : nib; /* two's complement */
            float s = oracle_fp16_value(scales[r * nb + k / g]);
            out[r * cols + k] = (float)q * s;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* INT4 with a zero point: integers -8..7, one fp16 scale and one zero point */
/* per group of 128 ("Quantization in deployment", format cheat sheet, row    */
/* W4A16 INT4 GPTQ/AWQ: one scale per 128 numbers, plus a zero point; the   */
/* zero point absorbs a constant offset of the group).  Readings (min-max   */
/* rounding, the rule of the GPTQ/AWQ formats that row names):              */
/*   lo = min(min_group, 0), hi = max(max_group, 0)   (0 stays exact)        */
/*   scale = fp16(fp32(hi - lo) / 15)                                        */
/*   z = clamp(-8 - rne(lo / scale), -8, 7)            (an integer code)     */
/*   q = clamp(rne(w / scale) + z, -8, 7),  value = (q - z) * scale          */
/* A group whose fp16 scale is 0 stores scale 0, zero point 0 and codes 0.   */
/* Storage: codes as INT4 (two's complement nibbles); one 32-bit word per    */
/* group = fp16 scale bits | (z & 0xFF) << 16.                               */
/* ------------------------------------------------------------------------ */

uint32_t oracle_int4zp_group(const float* w, int64_t n, int32_t* q_out)
{
    float lo = 0.0f, hi = 0.0f;
    for (int64_t i = 0; i < n; ++i) {
        if (w[i] < lo)
            lo = w[i];
        if (w[i] > hi)
            hi = w[i];
    }
    float range = hi - lo;                     /* fp32 */
    int s_code = oracle_fp16_code(range / 15.0f);
    float s = oracle_fp16_value(s_code);
    if (s == 0.0f) {
        for (int64_t i = 0; i < n; ++i)
            q_out[i] = 0;
        return 0u;
    }
    float zr = -8.0f - rintf(lo / s);          /* divide by the stored scale */
    if (zr < -8.0f)
        zr = -8.0f;
    if (zr > 7.0f)
        zr = 7.0f;
    int z = (int)zr;
    for (int64_t i = 0; i < n; ++i) {
        float qr = rintf(w[i] / s) + (float)z;
        if (qr > 7.0f)
            qr = 7.0f;
        if (qr < -8.0f)
            qr = -8.0f;
        q_out[i] = (int32_t)qr;
    }
    return (uint32_t)s_code | ((uint32_t)(z & 0xFF) << 16);
}

int oracle_quantize_int4zp(const float* w, int64_t rows, int64_t cols, int64_t ld, uint8_t* codes,
                           uint32_t* scales)
{
    const int64_t g = 128;
    if (cols % g != 0)
        return -1;
    int64_t nb = cols / g;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        int32_t q[128];
        uint8_t* rc = codes + r * (cols / 2);
        for (int64_t b = 0; b < nb; ++b) {
            scales[r * nb + b] = oracle_int4zp_group(w + r * ld + b * g, g, q);
            for (int64_t i = 0; i < g; ++i)
                put_nibble(rc, b * g + i, q[i] & 0xF);
        }
    }
    return 0;
}

/* value = fp32((q - z) * scale), exact (|q - z| <= 15, an fp16 scale). */
void oracle_dequant_int4zp(const uint8_t* codes, const uint32_t* scales, int64_t rows, int64_t cols,
                           float* out)
{
    int64_t nb = cols / 128;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t k = 0; k < cols; ++k) {
            int nib = get_nibble(codes + r * (cols / 2), k);
            int q = (nib >= 8) ? nib - 16 : nib;
            uint32_t word = scales[r * nb + k / 128];
            float s = oracle_fp16_value((int)(word & 0xFFFFu));
            int z = (int)(int8_t)((word >> 16) & 0xFFu);
            out[r * cols + k] = (float)(q - z) * s;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* E2M1 element encode shared by MXFP4 and NVFP4: y = clamp(w/scale, -6, 6),  */
/* nearest grid value; sign bit from w.                                       */
/* ------------------------------------------------------------------------ */
static int e2m1_encode(float w, float scale)
{
    int sign = signbit_f(w);
    if (scale == 0.0f)
        return sign << 3;
    float y = w / scale;
    if (y > 6.0f)
        y = 6.0f;
    if (y < -6.0f)
        y = -6.0f;
    return (sign << 3) | oracle_e2m1_code(fabsf(y));
}

/* ------------------------------------------------------------------------ */
/* MXFP4: block 32, E8M0 scale 2^(floor(log2(max(amax,1e-12))) - 2).         */
/* ------------------------------------------------------------------------ */
int oracle_mx_scale_exponent(float amax)
{
    float a = amax > 1e-12f ? amax : 1e-12f;
    int ex;
    frexpf(a, &ex);          /* a = f * 2^ex, f in [0.5, 1): floor(log2 a) = ex-1 */
    return (ex - 1) - 2;     /* largest E2M1 exponent is 2 */
}

int oracle_quantize_mxfp4(const float* w, int64_t rows, int64_t cols, int64_t ld,
                          uint8_t* codes, uint8_t* scales)
{
    const int64_t g = 32;
    if (cols % g != 0)
        return -1;
    int64_t nb = cols / g;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        uint8_t* rc = codes + r * (cols / 2);
        for (int64_t b = 0; b < nb; ++b) {
            const float* blk = w + r * ld + b * g;
            float amax = 0.0f;
            for (int64_t i = 0; i < g; ++i)
                if (fabsf(blk[i]) > amax)
                    amax = fabsf(blk[i]);
            int e = oracle_mx_scale_exponent(amax);
            scales[r * nb + b] = (uint8_t)(e + 127);
            float scale = ldexpf(1.0f, e);
            for (int64_t i = 0; i < g; ++i)
                put_nibble(rc, b * g + i, e2m1_encode(blk[i], scale));
        }
    }
    return 0;
}

void oracle_dequant_mxfp4(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                          float* out)
{
    int64_t nb = cols / 32;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t k = 0; k < cols; ++k) {
            int nib = get_nibble(codes + r * (cols / 2), k);
            float s = ldexpf(1.0f, (int)scales[r * nb + k / 32] - 127);
            out[r * cols + k] = oracle_e2m1_value(nib) * s;
        }
}

/* ------------------------------------------------------------------------ */
/* NVFP4: block 16, E4M3 block scale, fp32 tensor scale.                     */
/* ------------------------------------------------------------------------ */
float oracle_nv_global_scale(const float* w, int64_t rows, int64_t cols, int64_t ld)
{
    float amax = 0.0f;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t k = 0; k < cols; ++k)
            if (fabsf(w[r * ld + k]) > amax)
                amax = fabsf(w[r * ld + k]);
    float a = amax > 1e-12f ? amax : 1e-12f;
    return a / 2688.0f; /* 448 (E4M3 max) * 6 (E2M1 max) */
}

/* E4M3 block-scale code of one block: E4M3(min((amax_b/6)/gs, 448)). */
int oracle_nv_block_scale_code(float amax_b, float gs)
{
    float t = (amax_b / 6.0f) / gs;
    if (t > 448.0f)
        t = 448.0f;
    return oracle_e4m3_code(t);
}

int oracle_quantize_nvfp4(const float* w, int64_t rows, int64_t cols, int64_t ld,
                          const float* gs_in, uint8_t* codes, uint8_t* scales, float* gs_out)
{
    const int64_t g = 16;
    if (cols % g != 0)
        return -1;
    float gs = gs_in ? *gs_in : oracle_nv_global_scale(w, rows, cols, ld);
    if (!(gs > 0.0f))
        return -2;
    *gs_out = gs;
    int64_t nb = cols / g;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        uint8_t* rc = codes + r * (cols / 2);
        for (int64_t b = 0; b < nb; ++b) {
            const float* blk = w + r * ld + b * g;
            float amax = 0.0f;
            for (int64_t i = 0; i < g; ++i)
                if (fabsf(blk[i]) > amax)
                    amax = fabsf(blk[i]);
            int sc = oracle_nv_block_scale_code(amax, gs);
            scales[r * nb + b] = (uint8_t)sc;
            float eff = oracle_e4m3_value(sc) * gs; /* the scale as used */
            for (int64_t i = 0; i < g; ++i)
                put_nibble(rc, b * g + i, e2m1_encode(blk[i], eff));
        }
    }
    return 0;
}

void oracle_dequant_nvfp4(const uint8_t* codes, const uint8_t* scales, float gs, int64_t rows,
                          int64_t cols, float* out)
{
    int64_t nb = cols / 16;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t k = 0; k < cols; ++k) {
            int nib = get_nibble(codes + r * (cols / 2), k);
            float eff = oracle_e4m3_value(scales[r * nb + k / 16]) * gs;
            out[r * cols + k] = oracle_e2m1_value(nib) * eff;
        }
}

/* ------------------------------------------------------------------------ */
/* FP8 E4M3 with one fp32 scale per row: the activation side of W4A8.        */
/* "Quantization in deployment", formats.py fp8() and fp8_per_row(): each    */
/* row (token) gets scale = max(amax_row, 1e-12) / 448; every value is       */
/* divided by it, clamped to +-448 and rounded to the nearest E4M3 value.    */
/* Readings: rounding is to nearest, ties to the even code (torch's          */
/* float8_e4m3fn cast, which fp8() calls); the sign bit of the input is      */
/* kept, so -0 and negatives that round to 0 give 0x80.                      */
/* ------------------------------------------------------------------------ */

/* Row scale of a row whose largest magnitude is amax. */
float oracle_fp8_row_scale(float amax)
{
    float a = amax > 1e-12f ? amax : 1e-12f;
    return a / 448.0f;
}

/* E4M3 code (with sign) of x for a row scale s. */
int oracle_fp8_code(float x, float s)
{
    float y = x / s;
    float t = fabsf(y);
    if (t > 448.0f)
        t = 448.0f;
    return (signbit_f(y) << 7) | oracle_e4m3_code(t);
}

void oracle_quantize_fp8_rows(const float* w, int64_t rows, int64_t cols, int64_t ld,
                              uint8_t* codes, float* scales)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const float* x = w + r * ld;
        float amax = 0.0f;
        for (int64_t k = 0; k < cols; ++k)
            if (fabsf(x[k]) > amax)
                amax = fabsf(x[k]);
        float s = oracle_fp8_row_scale(amax);
        scales[r] = s;
        for (int64_t k = 0; k < cols; ++k)
            codes[r * cols + k] = (uint8_t)oracle_fp8_code(x[k], s);
    }
}

/* value = fp32(E4M3 value * row scale), the product fp8() returns. */
void oracle_dequant_fp8_rows(const uint8_t* codes, const float* scales, int64_t rows,
                             int64_t cols, float* out)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t k = 0; k < cols; ++k) {
            int c = codes[r * cols + k];
            float v = oracle_e4m3_value(c) * scales[r];
            out[r * cols + k] = (c & 0x80) ? -v : v;
        }
}

/* fp32 array -> bf16 array (round to nearest even). */
void oracle_f32_to_bf16_array(const float* in, int64_t n, uint16_t* out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_f32_to_bf16(in[i]);
}

int oracle_abi_version(void) { return 2; }
