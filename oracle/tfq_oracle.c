/*
 * tfq_oracle.c -- plain, slow, CPU reference for the W8A8 scaled-quantized
 * Linear.  TEST INFRASTRUCTURE ONLY: the product library never links, loads
 * or calls this file; only the tests, the smoke check and the benchmark's CPU
 * baseline do.  It shares no code, header, table or constant with the HIP
 * kernels.
 *
 * Sources (web pages, cited by title and section):
 *   [TF-zh]  TeleFuser "量化" (Chinese quantization docs), sections
 *            "基本原理" (symmetric INT8 formula), "Scaled FP8 checkpoint：W8A8"
 *            (row-wise scaled FP8 formula), "离线转换" (one absmax scale per
 *            output row), "验证方法" (E_max / E_rel).
 *   [TF-en]  TeleFuser "Quantization" (English docs), sections "Core ideas",
 *            "tf-kernel FP8: online W8A8", "Scaled FP8 checkpoints: W8A8",
 *            "Offline conversion", "Validation".
 *   [LX-zh]  LightX2V "模型量化技术", table "量化模式" (fp8-b128-deepgemm:
 *            block-symmetric weights, group-symmetric activations) and section
 *            "MiniMax-H3 FP8 FP16 累加" (row-dynamic activations with
 *            scale = max(abs(x)) / qmax for reduced qmax; 448 is the full
 *            E4M3 range with FP32 accumulation).
 *   [VO-en]  vLLM-Omni "FP8 Quantization", table "Parameters"
 *            (weight_block_size).
 *   E4M3FN itself is the OCP 8-bit floating point format (OFP8 spec): 1 sign
 *   bit, 4 exponent bits with bias 7, 3 mantissa bits, no infinities, NaN =
 *   S.1111.111, max finite 448.
 *
 * Arithmetic contract (the readings of points the pages leave open):
 *   - quantisation runs in IEEE binary32 with round-to-nearest-even and no
 *     denormal flush: s = RN(amax / qmax); t = RN(x / s) (a true division);
 *   - FP8: t is clamped to [-qmax, qmax] and encoded to E4M3FN by
 *     round-to-nearest-even with saturation to +-448; the sign of zero is
 *     kept (-0 -> 0x80);
 *   - INT8: q = clamp(round_half_even(t), -128, 127);
 *   - an all-zero row or group has s = 0 and codes of (signed) zero;
 *   - the GEMM reference sums decoded codes exactly in binary64 (every
 *     E4M3FN or INT8 product is a multiple of 2^-18, bounded by 448^2, so
 *     any binary64 summation order is exact for K <= 2^17) and applies the
 *     scales in binary64;
 *   - the INT8 BF16 output follows one fixed binary32 order:
 *     bf16_RNE(RN(RN(float(acc) * s_row) * s_col) [+ bias]).
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math
 *        -fexcess-precision=standard -fopenmp -shared -fPIC
 * OpenMP only splits independent rows/outputs over threads; it never changes
 * the order of any floating-point sum.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_QTYPE_E4M3FN 0
#define ORC_QTYPE_INT8 1

/* ------------------------------------------------------------------------ */
/* bit casts                                                                 */
/* ------------------------------------------------------------------------ */
static uint32_t f32_bits(float v) { uint32_t u; memcpy(&u, &v, 4); return u; }
static float bits_f32(uint32_t u) { float v; memcpy(&v, &u, 4); return v; }

/* BF16 is the upper half of a binary32; decoding is exact. */
float tfq_oracle_bf16_to_f32(uint16_t h) { return bits_f32((uint32_t)h << 16); }

/* binary32 -> BF16 with round-to-nearest-even on the 16 dropped bits.
 * Inputs are finite (NaN is out of contract). */
uint16_t tfq_oracle_f32_to_bf16(float v)
{
    uint32_t u = f32_bits(v);
    uint32_t upper = u >> 16;
    uint32_t rest = u & 0xFFFFu;
    if (rest > 0x8000u || (rest == 0x8000u && (upper & 1u))) upper += 1u;
    return (uint16_t)upper;
}

/* ------------------------------------------------------------------------ */
/* E4M3FN decode: the closed form of the OCP definition                      */
/* ------------------------------------------------------------------------ */
double tfq_oracle_e4m3fn_value(uint8_t code)
{
    int s = code >> 7, e = (code >> 3) & 0xF, m = code & 7;
    double mag;
    if (e == 15 && m == 7) return NAN;              /* S.1111.111 */
    if (e == 0) mag = ldexp((double)m / 8.0, -6);   /* subnormal: 2^-6 * m/8 */
    else mag = ldexp(1.0 + (double)m / 8.0, e - 7); /* normal */
    return s ? -mag : mag;
}

/* ------------------------------------------------------------------------ */
/* E4M3FN encoder 1: arithmetic on the binary32 fields                        */
/* Round-to-nearest-even on the E4M3FN grid, subnormals kept, saturation to   */
/* +-448, never NaN, sign of zero kept.                                       */
/* ------------------------------------------------------------------------ */
uint8_t tfq_oracle_e4m3fn_encode(float v)
{
    uint32_t u = f32_bits(v);
    uint8_t sign = (uint8_t)((u >> 31) << 7);
    float a = fabsf(v);
    uint32_t code;
    if (a >= 448.0f) return (uint8_t)(sign | 0x7E); /* saturate (RNE of [448,464) is 448 too) */
    if (a < 0.015625f) {
        /* below the smallest normal 2^-6: the grid is m * 2^-9, m = 0..8;
         * a * 512 is exact (scaling by a power of two) and rintf rounds
         * half to even under the default rounding mode. m = 8 is the code
         * of 2^-6 itself, so the carry lands on the right code. */
        code = (uint32_t)rintf(a * 512.0f);
    } else {
        uint32_t au = f32_bits(a);
        int e = (int)((au >> 23) & 0xFF) - 127;   /* -6 .. 8 */
        uint32_t mant = au & 0x7FFFFFu;
        uint32_t keep = mant >> 20;               /* top 3 mantissa bits */
        uint32_t dropped = mant & 0xFFFFFu;       /* 20 dropped bits */
        code = ((uint32_t)(e + 7) << 3) | keep;
        if (dropped > 0x80000u || (dropped == 0x80000u && (code & 1u))) code += 1u;
        /* a carry out of the mantissa moves to the next binade: correct.
         * a < 448 and RNE cannot pass 448 (0x7E), so code <= 0x7E. */
    }
    return (uint8_t)(sign | code);
}

/* ------------------------------------------------------------------------ */
/* E4M3FN encoder 2: nearest finite value by search, ties to the even code.  */
/* Written independently of encoder 1; only used to cross-check it.          */
/* ------------------------------------------------------------------------ */
static double g_pos_values[127]; /* values of codes 0x00..0x7E, increasing */
static int g_pos_ready = 0;

static void init_pos_values(void)
{
    if (g_pos_ready) return;
    for (int c = 0; c < 127; ++c) g_pos_values[c] = tfq_oracle_e4m3fn_value((uint8_t)c);
    g_pos_ready = 1;
}

uint8_t tfq_oracle_e4m3fn_encode_search(float v)
{
    init_pos_values();
    uint8_t sign = (signbit(v) ? 0x80 : 0x00);
    double a = fabs((double)v);
    /* the largest code whose value is <= a (binary search on the sorted table) */
    int lo = 0, hi = 126;
    while (lo < hi) {
        int mid = (lo + hi + 1) / 2;
        if (g_pos_values[mid] <= a) lo = mid; else hi = mid - 1;
    }
    int best = lo;
    if (lo < 126) {
        double dlo = a - g_pos_values[lo], dhi = g_pos_values[lo + 1] - a;
        if (dhi < dlo || (dhi == dlo && ((lo + 1) % 2 == 0))) best = lo + 1;
    }
    /* a above 448: the nearest finite value is 448 (lo == 126): saturation. */
    return (uint8_t)(sign | best);
}

/* Encoder 1 over an array (for cross-checks against library casts). */
void tfq_oracle_e4m3fn_encode_array(const float* in, uint8_t* out, int64_t n)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = tfq_oracle_e4m3fn_encode(in[i]);
}

/* Exhaustive agreement of the two encoders over a range of binary32 bit
 * patterns [first, last] (both signs are tried for each pattern).  Returns
 * the number of disagreements and stores the first offending pattern. */
int64_t tfq_oracle_encoder_mismatches(uint32_t first, uint32_t last, uint32_t* first_bad)
{
    int64_t bad = 0;
    uint32_t fb = 0xFFFFFFFFu;
    init_pos_values();
#pragma omp parallel for schedule(static) reduction(+ : bad)
    for (int64_t p = (int64_t)first; p <= (int64_t)last; ++p) {
        for (int sgn = 0; sgn < 2; ++sgn) {
            uint32_t bits = (uint32_t)p | ((uint32_t)sgn << 31);
            float v = bits_f32(bits);
            if (tfq_oracle_e4m3fn_encode(v) != tfq_oracle_e4m3fn_encode_search(v)) {
                ++bad;
#pragma omp critical
                if (bits < fb) fb = bits;
            }
        }
    }
    if (first_bad) *first_bad = fb;
    return bad;
}

/* ------------------------------------------------------------------------ */
/* One quantisation of a single value with a given scale (row, group or     */
/* block).  [TF-en] "Core ideas" (INT8), "Scaled FP8 checkpoints" (FP8).     */
/* ------------------------------------------------------------------------ */
static uint8_t quantize_value(float x, float s, int qtype, float qmax)
{
    float t;
    if (s == 0.0f) t = copysignf(0.0f, x); /* all-zero row/group: codes are signed zeros */
    else t = x / s;                         /* RN binary32 division */
    if (qtype == ORC_QTYPE_E4M3FN) {
        t = fminf(fmaxf(t, -qmax), qmax);   /* clamp(x/s, f_min, f_max) with f = qmax */
        return tfq_oracle_e4m3fn_encode(t);
    } else {
        float r = rintf(t);                 /* round half to even */
        if (r < -128.0f) r = -128.0f;
        if (r > 127.0f) r = 127.0f;
        int8_t q = (int8_t)(int)r;
        return (uint8_t)q;
    }
}

/* ------------------------------------------------------------------------ */
/* Row-wise (per-token) dynamic quantisation, optionally per group of        */
/* `group` consecutive columns (1 x group token groups).                     */
/*   x      : BF16 bits, row r starts at x + r*ld                            */
/*   q      : codes, dense [rows, cols]                                      */
/*   scale  : FP32, dense [rows, ceil(cols/group)] (group 0 = whole row)     */
/* [TF-en] "Scaled FP8 checkpoints: W8A8" (each input row quantised with its */
/* own absmax), "tf-kernel FP8: online W8A8" (per-token activations);        */
/* [LX-zh] "MiniMax-H3 FP8 FP16 累加" (scale = max(abs(x))/qmax);             */
/* [LX-zh] "量化模式" fp8-b128-deepgemm (group-symmetric activations).        */
/* ------------------------------------------------------------------------ */
void tfq_oracle_quantize_rows(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld,
                              int qtype, float qmax, int64_t group, uint8_t* q, float* scale)
{
    int64_t g = (group <= 0) ? cols : group;
    int64_t ngroups = (cols + g - 1) / g;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const uint16_t* xr = x + r * ld;
        for (int64_t gi = 0; gi < ngroups; ++gi) {
            int64_t c0 = gi * g, c1 = c0 + g < cols ? c0 + g : cols;
            float amax = 0.0f;
            for (int64_t c = c0; c < c1; ++c) {
                float a = fabsf(tfq_oracle_bf16_to_f32(xr[c]));
                if (a > amax) amax = a;
            }
            float s = amax / qmax;
            scale[r * ngroups + gi] = s;
            for (int64_t c = c0; c < c1; ++c)
                q[r * cols + c] = quantize_value(tfq_oracle_bf16_to_f32(xr[c]), s, qtype, qmax);
        }
    }
}

/* Weight quantisation with one scale per (block x block) tile of W [n, k]
 * (block-symmetric weights: [LX-zh] "量化模式" fp8-b128-deepgemm; [VO-en]
 * "Parameters" weight_block_size).  scale is dense [ceil(n/block),
 * ceil(k/block)].  Per-output-channel weights ([TF-en] "Offline conversion":
 * one absmax scale per output row) are tfq_oracle_quantize_rows on W. */
void tfq_oracle_quantize_blocks(const uint16_t* w, int64_t n, int64_t k, int qtype, float qmax,
                                int64_t block, uint8_t* q, float* scale)
{
    int64_t nb = (n + block - 1) / block, kb = (k + block - 1) / block;
#pragma omp parallel for schedule(static)
    for (int64_t bi = 0; bi < nb * kb; ++bi) {
        int64_t br = bi / kb, bc = bi % kb;
        int64_t r0 = br * block, r1 = r0 + block < n ? r0 + block : n;
        int64_t c0 = bc * block, c1 = c0 + block < k ? c0 + block : k;
        float amax = 0.0f;
        for (int64_t r = r0; r < r1; ++r)
            for (int64_t c = c0; c < c1; ++c) {
                float a = fabsf(tfq_oracle_bf16_to_f32(w[r * k + c]));
                if (a > amax) amax = a;
            }
        float s = amax / qmax;
        scale[br * kb + bc] = s;
        for (int64_t r = r0; r < r1; ++r)
            for (int64_t c = c0; c < c1; ++c)
                q[r * k + c] = quantize_value(tfq_oracle_bf16_to_f32(w[r * k + c]), s, qtype, qmax);
    }
}

/* ------------------------------------------------------------------------ */
/* GEMM references.  A codes [M, K] (row-major), B codes [N, K] (row-major,  */
/* one output channel per row): y[m, n] = s_row[m] * s_col[n] * sum_k        */
/* a[m,k] b[n,k]  ([TF-en] "Core ideas": x_hat = s q, so the dequantised     */
/* Linear x_hat w_hat^T factors into this).  Only the rows listed in         */
/* `rows` (nrows of them; NULL = all M) are computed, in that order.         */
/* ------------------------------------------------------------------------ */
static double code_value(uint8_t c, int qtype)
{
    return qtype == ORC_QTYPE_E4M3FN ? tfq_oracle_e4m3fn_value(c) : (double)(int8_t)c;
}

double tfq_oracle_gelu_tanh(double h)
{
    /* GELU, tanh form (Hendrycks & Gimpel, "Gaussian Error Linear Units"). */
    const double pi = 3.14159265358979323846;
    const double c = sqrt(2.0 / pi);
    return 0.5 * h * (1.0 + tanh(c * (h + 0.044715 * h * h * h)));
}

/* Exact dots of selected rows: dot[i, n] = sum_k a[rows[i], k] * b[n, k]. */
void tfq_oracle_dot(const uint8_t* a, const uint8_t* b, int qtype, int64_t M, int64_t N, int64_t K,
                    const int64_t* rows, int64_t nrows, double* dot)
{
    int64_t R = rows ? nrows : M;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < R; ++i) {
        int64_t m = rows ? rows[i] : i;
        double* arow = (double*)malloc(sizeof(double) * (size_t)K);
        for (int64_t k = 0; k < K; ++k) arow[k] = code_value(a[m * K + k], qtype);
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k) acc += arow[k] * code_value(b[n * K + k], qtype);
            dot[i * N + n] = acc;
        }
        free(arow);
    }
}

/* Scaled Linear reference in binary64.
 *   scale_block == 0 : y = dot * s_row[m] * s_col[n]
 *   scale_block  > 0 : y = sum_kb s_row[m, kb] * s_col[n / blk, kb] * dot_kb
 *                      (a_scale [M, K/blk], b_scale [N/blk, K/blk]) -- the
 *                      per-K-block accumulation of block-scaled FP8.
 * then + bias[n] (BF16, may be NULL), then GELU-tanh if epi == 1. */
void tfq_oracle_linear_ref(const uint8_t* a, const float* a_scale, const uint8_t* b,
                           const float* b_scale, int qtype, int64_t M, int64_t N, int64_t K,
                           int64_t scale_block, const uint16_t* bias, int epi,
                           const int64_t* rows, int64_t nrows, double* y)
{
    int64_t R = rows ? nrows : M;
    int64_t nkb = scale_block > 0 ? (K + scale_block - 1) / scale_block : 1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < R; ++i) {
        int64_t m = rows ? rows[i] : i;
        double* arow = (double*)malloc(sizeof(double) * (size_t)K);
        for (int64_t k = 0; k < K; ++k) arow[k] = code_value(a[m * K + k], qtype);
        for (int64_t n = 0; n < N; ++n) {
            double v;
            if (scale_block <= 0) {
                double acc = 0.0;
                for (int64_t k = 0; k < K; ++k) acc += arow[k] * code_value(b[n * K + k], qtype);
                v = acc * (double)a_scale[m] * (double)b_scale[n];
            } else {
                v = 0.0;
                for (int64_t kb = 0; kb < nkb; ++kb) {
                    int64_t k0 = kb * scale_block;
                    int64_t k1 = k0 + scale_block < K ? k0 + scale_block : K;
                    double acc = 0.0;
                    for (int64_t k = k0; k < k1; ++k) acc += arow[k] * code_value(b[n * K + k], qtype);
                    v += (double)a_scale[m * nkb + kb] * (double)b_scale[(n / scale_block) * nkb + kb] * acc;
                }
            }
            if (bias) v += (double)tfq_oracle_bf16_to_f32(bias[n]);
            if (epi == 1) v = tfq_oracle_gelu_tanh(v);
            y[i * N + n] = v;
        }
        free(arow);
    }
}

/* ------------------------------------------------------------------------ */
/* MXFP8 (E4M3FN elements, 32-element blocks along a row, E8M0 block scales) */
/* ------------------------------------------------------------------------ */
/* The pages (TeleFuser "Quantization", converter section; TeleFuser "量化"
 * page, 离线转换) say only that MXFP4/6/8 use 32-value blocks with E8M0
 * scales.  The block rule is read from the OCP Microscaling (MX) format
 * specification v1.0: the shared exponent of a block is
 * floor(log2(max |v|)) - emax_elem, emax_elem = 8 for E4M3 (448 = 1.75 * 2^8),
 * clamped to the E8M0 range [-127, 127] (an all-zero block takes -127); the
 * block scale is X = 2^shared_exp, stored as the E8M0 byte shared_exp + 127;
 * each element is v / X, clamped to +-448 and encoded to E4M3FN (RNE). */

/* E8M0 byte of a block whose largest magnitude is amax (a finite float). */
uint8_t tfq_oracle_mx_scale_code(float amax)
{
    int e;
    if (!(amax > 0.0f)) return 0;            /* zero block: 2^-127 */
    (void)frexpf(amax, &e);                   /* amax = f * 2^e, f in [0.5, 1) */
    int shared = (e - 1) - 8;                 /* floor(log2 amax) - emax_elem */
    if (shared < -127) shared = -127;
    if (shared > 127) shared = 127;
    return (uint8_t)(shared + 127);
}

/* Quantise rows of BF16 x [rows, cols] (cols % 32 == 0, leading dim ld) to
 * MXFP8: codes [rows, cols] and E8M0 scales [rows, cols / 32]. */
void tfq_oracle_quantize_mx(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld,
                            uint8_t* q, uint8_t* scale)
{
    const int64_t nb = cols / 32;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t b = 0; b < nb; ++b) {
            const uint16_t* xb = x + r * ld + b * 32;
            float amax = 0.0f;
            for (int i = 0; i < 32; ++i) {
                float a = fabsf(tfq_oracle_bf16_to_f32(xb[i]));
                if (a > amax) amax = a;
            }
            const uint8_t code = tfq_oracle_mx_scale_code(amax);
            scale[r * nb + b] = code;
            const double X = ldexp(1.0, (int)code - 127);
            for (int i = 0; i < 32; ++i) {
                /* v / X is exact in binary64; rounding it to binary32 is the
                 * only rounding before the E4M3FN encode */
                float t = (float)((double)tfq_oracle_bf16_to_f32(xb[i]) / X);
                t = fminf(fmaxf(t, -448.0f), 448.0f);
                q[r * cols + b * 32 + i] = tfq_oracle_e4m3fn_encode(t);
            }
        }
    }
}

/* MXFP8 Linear reference in binary64 for selected rows:
 *   y[m, n] = sum_kb 2^(ea[m,kb] - 127) * 2^(eb[n,kb] - 127) * dot_kb
 * (dot_kb = the exact binary64 sum of decoded code products over block kb),
 * then + bias[n] (BF16, may be NULL), then GELU-tanh if epi == 1.  Each
 * dot_kb is exact; only the combination over blocks rounds (relative error
 * below K/32 * 2^-53). */
void tfq_oracle_linear_mx_ref(const uint8_t* a, const uint8_t* a_scale, const uint8_t* b,
                              const uint8_t* b_scale, int64_t M, int64_t N, int64_t K,
                              const uint16_t* bias, int epi, const int64_t* rows, int64_t nrows,
                              double* y)
{
    const int64_t R = rows ? nrows : M;
    const int64_t nb = K / 32;
    (void)M;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < R; ++i) {
        const int64_t m = rows ? rows[i] : i;
        double* arow = (double*)malloc(sizeof(double) * (size_t)K);
        for (int64_t k = 0; k < K; ++k) arow[k] = tfq_oracle_e4m3fn_value(a[m * K + k]);
        for (int64_t n = 0; n < N; ++n) {
            double v = 0.0;
            for (int64_t kb = 0; kb < nb; ++kb) {
                double acc = 0.0;
                for (int64_t k = kb * 32; k < kb * 32 + 32; ++k)
                    acc += arow[k] * tfq_oracle_e4m3fn_value(b[n * K + k]);
                v += ldexp(acc, (int)a_scale[m * nb + kb] - 127 + (int)b_scale[n * nb + kb] - 127);
            }
            if (bias) v += (double)tfq_oracle_bf16_to_f32(bias[n]);
            if (epi == 1) v = tfq_oracle_gelu_tanh(v);
            y[i * N + n] = v;
        }
        free(arow);
    }
}

/* ---- MXFP4 ----
 * OCP Microscaling (MX) v1.0 with E2M1 elements: 1 sign bit, 2 exponent
 * bits (bias 1) and 1 mantissa bit, magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6;
 * one E8M0 scale per 32 elements (TeleFuser "Quantization", converter
 * section: MXFP4/6/8 use 32-value blocks and E8M0 scales).  Shared exponent
 * floor(log2(amax)) - 2 (2 = the exponent of E2M1's largest normal, 6 =
 * 1.5 * 2^2), clamped to [-127, 127]; elements v / 2^shared clamped to +-6
 * and rounded to the nearest E2M1 value, ties to the even code.  Two codes
 * per byte, the element with the lower index in the low nibble. */
static const double kE2M1Mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

double tfq_oracle_e2m1_value(uint8_t code)
{
    const double v = kE2M1Mag[code & 7];
    return (code & 8) ? -v : v;
}

/* Nearest E2M1 code of t (saturating at 6; ties to the even code; the sign
 * is kept, also for results of zero). */
uint8_t tfq_oracle_e2m1_encode(float t)
{
    const int neg = signbit(t) != 0;
    double a = fabs((double)t);
    if (a > 6.0) a = 6.0;
    int best = 0;
    double bd = INFINITY;
    for (int c = 0; c < 8; ++c) {
        const double d = fabs(a - kE2M1Mag[c]);
        if (d < bd || (d == bd && (c & 1) == 0)) {
            best = c;
            bd = d;
        }
    }
    return (uint8_t)(best | (neg ? 8 : 0));
}

uint8_t tfq_oracle_mx4_scale_code(float amax)
{
    int e;
    if (!(amax > 0.0f)) return 0;            /* zero block: 2^-127 */
    (void)frexpf(amax, &e);                   /* amax = f * 2^e, f in [0.5, 1) */
    int shared = (e - 1) - 2;                 /* floor(log2 amax) - emax_elem */
    if (shared < -127) shared = -127;
    if (shared > 127) shared = 127;
    return (uint8_t)(shared + 127);
}

/* Quantise rows of BF16 x [rows, cols] (cols % 32 == 0, leading dim ld) to
 * MXFP4: packed codes [rows, cols / 2] and E8M0 scales [rows, cols / 32]. */
void tfq_oracle_quantize_mx4(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld,
                             uint8_t* q, uint8_t* scale)
{
    const int64_t nb = cols / 32;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t i = 0; i < cols / 2; ++i) q[r * (cols / 2) + i] = 0;
        for (int64_t b = 0; b < nb; ++b) {
            const uint16_t* xb = x + r * ld + b * 32;
            float amax = 0.0f;
            for (int i = 0; i < 32; ++i) {
                float a = fabsf(tfq_oracle_bf16_to_f32(xb[i]));
                if (a > amax) amax = a;
            }
            const uint8_t code = tfq_oracle_mx4_scale_code(amax);
            scale[r * nb + b] = code;
            const double X = ldexp(1.0, (int)code - 127);
            for (int i = 0; i < 32; ++i) {
                const float t = (float)((double)tfq_oracle_bf16_to_f32(xb[i]) / X);
                const int64_t e = b * 32 + i;
                q[r * (cols / 2) + e / 2] |= (uint8_t)(tfq_oracle_e2m1_encode(t) << (4 * (e & 1)));
            }
        }
    }
}

/* MXFP4 Linear reference in binary64 for selected rows (codes packed two
 * per byte; as tfq_oracle_linear_mx_ref otherwise). */
void tfq_oracle_linear_mx4_ref(const uint8_t* a, const uint8_t* a_scale, const uint8_t* b,
                               const uint8_t* b_scale, int64_t M, int64_t N, int64_t K,
                               const uint16_t* bias, int epi, const int64_t* rows, int64_t nrows,
                               double* y)
{
    const int64_t R = rows ? nrows : M;
    const int64_t nb = K / 32, kb2 = K / 2;
    (void)M;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < R; ++i) {
        const int64_t m = rows ? rows[i] : i;
        double* arow = (double*)malloc(sizeof(double) * (size_t)K);
        for (int64_t k = 0; k < K; ++k)
            arow[k] = tfq_oracle_e2m1_value((uint8_t)(a[m * kb2 + k / 2] >> (4 * (k & 1))));
        for (int64_t n = 0; n < N; ++n) {
            double v = 0.0;
            for (int64_t kb = 0; kb < nb; ++kb) {
                double acc = 0.0;
                for (int64_t k = kb * 32; k < kb * 32 + 32; ++k)
                    acc += arow[k] *
                           tfq_oracle_e2m1_value((uint8_t)(b[n * kb2 + k / 2] >> (4 * (k & 1))));
                v += ldexp(acc, (int)a_scale[m * nb + kb] - 127 + (int)b_scale[n * nb + kb] - 127);
            }
            if (bias) v += (double)tfq_oracle_bf16_to_f32(bias[n]);
            if (epi == 1) v = tfq_oracle_gelu_tanh(v);
            y[i * N + n] = v;
        }
        free(arow);
    }
}

/* ---- MXFP6 ----
 * OCP MX v1.0 with FP6 elements: E2M3 (1 sign, 2 exponent bits with bias 1,
 * 3 mantissa bits; largest 7.5 = 1.875 * 2^2) or E3M2 (3 exponent bits with
 * bias 3, 2 mantissa bits; largest 28 = 1.75 * 2^4), no infinities or NaN.
 * Shared exponent floor(log2(amax)) - emax (2 for E2M3, 4 for E3M2); the
 * elements are rounded to the nearest value, ties to the even code, clamped
 * at the largest.  Six-bit codes are packed as a little-endian bit stream:
 * element i of a row takes bits 6 i .. 6 i + 5 of the row's bytes (four
 * elements per three bytes). */
static void fp6_params(int fmt, int* ebits, int* mbits, int* bias)
{
    if (fmt == 0) { *ebits = 2; *mbits = 3; *bias = 1; }   /* E2M3 */
    else { *ebits = 3; *mbits = 2; *bias = 3; }             /* E3M2 */
}

/* Value of a 6-bit code (sign in bit 5). */
double tfq_oracle_fp6_value(int fmt, uint8_t code)
{
    int eb, mb, bias;
    fp6_params(fmt, &eb, &mb, &bias);
    const int e = (code >> mb) & ((1 << eb) - 1);
    const int m = code & ((1 << mb) - 1);
    double v = e == 0 ? ldexp((double)m, 1 - bias - mb)
                      : ldexp(1.0 + ldexp((double)m, -mb), e - bias);
    return (code & 32) ? -v : v;
}

/* Nearest FP6 code of t, searched over all 32 magnitudes (saturating at the
 * largest; ties to the even code; sign kept, also for zero). */
uint8_t tfq_oracle_fp6_encode(int fmt, float t)
{
    const int neg = signbit(t) != 0;
    const double a = fabs((double)t);
    int best = 0;
    double bd = INFINITY;
    for (int c = 0; c < 32; ++c) {
        const double d = fabs(a - tfq_oracle_fp6_value(fmt, (uint8_t)c));
        if (d < bd || (d == bd && (c & 1) == 0)) {
            best = c;
            bd = d;
        }
    }
    return (uint8_t)(best | (neg ? 32 : 0));
}

uint8_t tfq_oracle_mx6_scale_code(int fmt, float amax)
{
    int e;
    if (!(amax > 0.0f)) return 0;
    (void)frexpf(amax, &e);
    int shared = (e - 1) - (fmt == 0 ? 2 : 4);
    if (shared < -127) shared = -127;
    if (shared > 127) shared = 127;
    return (uint8_t)(shared + 127);
}

static void put6(uint8_t* row, int64_t i, uint8_t code)
{
    const int64_t bit = 6 * i;
    const uint32_t v = (uint32_t)(code & 63) << (bit & 7);
    row[bit >> 3] |= (uint8_t)v;
    if ((bit & 7) > 2) row[(bit >> 3) + 1] |= (uint8_t)(v >> 8);
}

static uint8_t get6(const uint8_t* row, int64_t i)
{
    const int64_t bit = 6 * i;
    uint32_t v = row[bit >> 3];
    if ((bit & 7) > 2) v |= (uint32_t)row[(bit >> 3) + 1] << 8;
    return (uint8_t)((v >> (bit & 7)) & 63);
}

/* Quantise rows of BF16 x [rows, cols] (cols % 32 == 0) to MXFP6: packed
 * codes [rows, 3 cols / 4] bytes and E8M0 scales [rows, cols / 32]. */
void tfq_oracle_quantize_mx6(int fmt, const uint16_t* x, int64_t rows, int64_t cols, int64_t ld,
                             uint8_t* q, uint8_t* scale)
{
    const int64_t nb = cols / 32, rb = cols * 3 / 4;
    int eb, mb, bias;
    fp6_params(fmt, &eb, &mb, &bias);
    const float maxv = (float)tfq_oracle_fp6_value(fmt, 31);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        uint8_t* qr = q + r * rb;
        for (int64_t i = 0; i < rb; ++i) qr[i] = 0;
        for (int64_t b = 0; b < nb; ++b) {
            const uint16_t* xb = x + r * ld + b * 32;
            float amax = 0.0f;
            for (int i = 0; i < 32; ++i) {
                float a = fabsf(tfq_oracle_bf16_to_f32(xb[i]));
                if (a > amax) amax = a;
            }
            const uint8_t code = tfq_oracle_mx6_scale_code(fmt, amax);
            scale[r * nb + b] = code;
            const double X = ldexp(1.0, (int)code - 127);
            for (int i = 0; i < 32; ++i) {
                float t = (float)((double)tfq_oracle_bf16_to_f32(xb[i]) / X);
                t = fminf(fmaxf(t, -maxv), maxv);
                put6(qr, b * 32 + i, tfq_oracle_fp6_encode(fmt, t));
            }
        }
    }
}

/* MXFP6 Linear reference in binary64 for selected rows. */
void tfq_oracle_linear_mx6_ref(int fmt, const uint8_t* a, const uint8_t* a_scale, const uint8_t* b,
                               const uint8_t* b_scale, int64_t M, int64_t N, int64_t K,
                               const uint16_t* bias, int epi, const int64_t* rows, int64_t nrows,
                               double* y)
{
    const int64_t R = rows ? nrows : M;
    const int64_t nb = K / 32, rb = K * 3 / 4;
    (void)M;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < R; ++i) {
        const int64_t m = rows ? rows[i] : i;
        double* arow = (double*)malloc(sizeof(double) * (size_t)K);
        for (int64_t k = 0; k < K; ++k) arow[k] = tfq_oracle_fp6_value(fmt, get6(a + m * rb, k));
        for (int64_t n = 0; n < N; ++n) {
            double v = 0.0;
            for (int64_t kb = 0; kb < nb; ++kb) {
                double acc = 0.0;
                for (int64_t k = kb * 32; k < kb * 32 + 32; ++k)
                    acc += arow[k] * tfq_oracle_fp6_value(fmt, get6(b + n * rb, k));
                v += ldexp(acc, (int)a_scale[m * nb + kb] - 127 + (int)b_scale[n * nb + kb] - 127);
            }
            if (bias) v += (double)tfq_oracle_bf16_to_f32(bias[n]);
            if (epi == 1) v = tfq_oracle_gelu_tanh(v);
            y[i * N + n] = v;
        }
        free(arow);
    }
}

/* INT8 W8A8: exact INT32 accumulators (held in int64 here; the caller keeps
 * K small enough that they fit INT32) and the fixed-order BF16 output.
 * acc and y_bf16 may each be NULL. */
void tfq_oracle_int8_linear(const int8_t* a, const float* a_scale, const int8_t* b,
                            const float* b_scale, int64_t M, int64_t N, int64_t K,
                            const uint16_t* bias, const int64_t* rows, int64_t nrows,
                            int64_t* acc, uint16_t* y_bf16)
{
    int64_t R = rows ? nrows : M;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < R; ++i) {
        int64_t m = rows ? rows[i] : i;
        for (int64_t n = 0; n < N; ++n) {
            int64_t sum = 0;
            for (int64_t k = 0; k < K; ++k) sum += (int64_t)a[m * K + k] * (int64_t)b[n * K + k];
            if (acc) acc[i * N + n] = sum;
            if (y_bf16) {
                float f = (float)sum;          /* RN int -> binary32 */
                f = f * a_scale[m];            /* RN */
                f = f * b_scale[n];            /* RN */
                if (bias) f = f + tfq_oracle_bf16_to_f32(bias[n]);
                y_bf16[i * N + n] = tfq_oracle_f32_to_bf16(f);
            }
        }
    }
}

/* Array forms of two steps above, for references that form the exact dots
 * with a library matmul (the exact-dot property: any binary64 summation
 * order gives the same sum for K <= 2^17): GELU-tanh of n values in place,
 * and the INT8 BF16 epilogue of tfq_oracle_int8_linear on given INT sums
 * (sums [R, N] of rows `rows`, or of rows 0..R-1 when rows is NULL). */
void tfq_oracle_gelu_tanh_array(double* v, int64_t n)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) v[i] = tfq_oracle_gelu_tanh(v[i]);
}

void tfq_oracle_int8_epilogue(const int64_t* sums, const float* a_scale, const float* b_scale,
                              int64_t R, int64_t N, const uint16_t* bias, const int64_t* rows,
                              uint16_t* y_bf16)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < R; ++i) {
        int64_t m = rows ? rows[i] : i;
        for (int64_t n = 0; n < N; ++n) {
            float f = (float)sums[i * N + n]; /* RN int -> binary32 */
            f = f * a_scale[m];               /* RN */
            f = f * b_scale[n];               /* RN */
            if (bias) f = f + tfq_oracle_bf16_to_f32(bias[n]);
            y_bf16[i * N + n] = tfq_oracle_f32_to_bf16(f);
        }
    }
}

/* Operator error measures of [TF-en] "Validation": E_max = max|y_q - y| and
 * E_rel = ||y_q - y||_2 / ||y||_2 over n values. */
void tfq_oracle_error_measures(const double* yq, const double* y, int64_t n, double* e_max,
                               double* e_rel)
{
    double mx = 0.0, num = 0.0, den = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        double d = fabs(yq[i] - y[i]);
        if (d > mx) mx = d;
        num += (yq[i] - y[i]) * (yq[i] - y[i]);
        den += y[i] * y[i];
    }
    *e_max = mx;
    *e_rel = den > 0.0 ? sqrt(num) / sqrt(den) : 0.0;
}

/* Threads the OpenMP runtime will use (for the CPU-baseline report). */
int tfq_oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
