/*
 * CPU oracle for the LLM.int8() mixed-precision linear layer Y = X.W.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load this library. The GPU library never links it and
 * shares no code, header or table with it.
 *
 * Plain, single-threaded, obviously-correct C. Every function follows one step
 * of the method as the pages state it:
 *
 *   [P2] "8-bit quantization of giant language models: LLM.int8()" (2kiu.com)
 *        section 2.1 (vector-wise scales: per-column for W, per-row for X),
 *        section 2.3 (outlier columns of X by a threshold on the column's
 *        absolute maximum, default 6.0; X_outlier.W_outlier in 16-bit, the rest
 *        in int8 with row/column scales), section 4.2 (the whole column goes
 *        the 16-bit way).
 *   [P5] "LLM.int8() pitfalls: why your 8-bit model collapses" (codearts)
 *        section 1 (scale_factor = 127 / max|x|, q = round(x * scale_factor)),
 *        section 2 (worked example), section 3.3 (dequantize the 8-bit result
 *        and ADD it to the 16-bit result).
 *   [P3] "Large-model quantization in practice: from INT8 to QLoRA" (cnnetsun)
 *        section 3.2 (round, then clamp, then cast; compute in float32) and
 *        section 3.3 (symmetric: zero point 0, clamp to [-127, 127]).
 *   [P1] "8-Bit LLM Quantization with Lightning Fabric" (aicoding) section 2.2
 *        (int8 x int8 -> int32 matmul, then rescale by scale_x * scale_w and
 *        add the bias), section 3.12 (per-layer quantization error as the
 *        mean absolute difference from the 16-bit output).
 *   [P2] also section 2.4 (int8 weights take half the memory of fp16 ones)
 *        and section 6 (the int8 weights are kept and reused; the fp16 ones
 *        need not be).
 *   [P5] also section 2 (the traditional 8-bit quantization uses one scale for
 *        the whole matrix).
 *   [P4] "INT8 vs FP8 vs GPTQ" page (mlqm.cn) sections 2 and 4 (二, 四)
 *        (FP8 E4M3: 4 exponent bits, 3 mantissa bits, largest value about 448;
 *        an alternative to INT8 at the same 8-bit size; wide-ranged activations
 *        need a scale before the cast).
 *
 * Readings taken where the pages are silent or disagree:
 *   - outlier test is |x| >= threshold (inclusive); a column is an outlier when
 *     any of its entries passes it;
 *   - the row absmax of X excludes outlier columns; outlier columns of Xq are 0;
 *   - a NaN entry never passes the threshold test and never sets an absmax
 *     (every comparison with NaN is false); its int8 code is 0;
 *   - the column absmax of W runs over all K rows (W is quantized once, at load);
 *   - the scale is applied as x * fl32(127 / absmax): one IEEE fp32 division,
 *     one fp32 multiply, round-half-to-even, clamp to [-127, 127], cast;
 *   - an all-zero row/column has absmax 0 and quantizes to all zeros;
 *   - merge is a sum; the 16-bit product and the merge are evaluated in fp64
 *     here (the most exact reading of "fp32-accumulated"; the GPU's fp16 output
 *     is compared against it with a tolerance).
 *   - FP8 variant: E4M3 as in the OCP 8-bit formats (bias 7, subnormals, no
 *     infinities, 0x7f and 0xff are NaN, largest finite 448); the same absmax
 *     scaling with 448 in place of 127: t = x * fl32(448 / absmax) in fp32,
 *     then the nearest E4M3 value, ties to the even code, magnitudes above 448
 *     saturating to 448; dequantization divides by 448^2; the fp8 matmul sums
 *     the exact products in fp64.
 *
 * Build: gcc -O2 -ffp-contract=off -std=c11 -shared -fPIC (no fast-math).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* IEEE 754 binary16 -> binary32. Exact for every pattern (binary32 holds every
 * binary16 value, including subnormals, as a normal or zero value). */
static float ora_half(uint16_t h)
{
    unsigned sign = h >> 15;
    int e = (h >> 10) & 0x1f;
    unsigned f = h & 0x3ffu;
    float v;
    if (e == 0)
        v = ldexpf((float)f, -24);                   /* f * 2^-24 */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexpf((float)(f | 0x400u), e - 25);     /* (1024 + f) * 2^(e-25) */
    return sign ? -v : v;
}

void ora_half_to_float(const uint16_t *h, int64_t n, float *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = ora_half(h[i]);
}

/* The symmetric absmax quantizer of [P5] section 1 with the round/clamp/cast
 * order of [P3] section 3.2: q = clamp(round_half_even(x * inv), -127, 127).
 * A NaN entry (the pages do not say; inputs are meant to be finite) codes as 0
 * here, so that the cast below is always defined. */
static int8_t ora_quant(float x, float inv)
{
    float v = x * inv;
    if (isnan(v))
        return 0;
    float r = rintf(v);                 /* default mode: round half to even */
    if (r > 127.0f)
        r = 127.0f;
    if (r < -127.0f)
        r = -127.0f;
    return (int8_t)r;
}

/* Weight side, run once per weight ([P2] section 2.1: one scale per column of
 * W, i.e. per output channel; [P2] section 6: quantized at load and reused).
 * W is [K x N] row-major (leading dimension ldw). Output Wq is [N x K]
 * (row n holds output channel n, K-contiguous), s[n] = max_k |W[k, n]|. */
void ora_quantize_colwise(const uint16_t *W, int64_t K, int64_t N, int64_t ldw,
                          int8_t *Wq, float *s)
{
    /* s[n] = max over all K rows of |W[k, n]| (rows visited in memory order) */
    for (int64_t n = 0; n < N; ++n)
        s[n] = 0.0f;
    for (int64_t k = 0; k < K; ++k)
        for (int64_t n = 0; n < N; ++n) {
            float a = fabsf(ora_half(W[k * ldw + n]));
            if (a > s[n])
                s[n] = a;
        }
    float *inv = malloc((size_t)N * sizeof(float));
    for (int64_t n = 0; n < N; ++n)
        inv[n] = s[n] > 0.0f ? 127.0f / s[n] : 0.0f;
    for (int64_t k = 0; k < K; ++k)
        for (int64_t n = 0; n < N; ++n)
            Wq[n * K + k] = s[n] > 0.0f ? ora_quant(ora_half(W[k * ldw + n]), inv[n]) : 0;
    free(inv);
}

/* Outlier columns of X ([P2] section 2.3 and 4.2): column k is an outlier when
 * some row i has |X[i, k]| >= threshold. Writes the ascending list of such k
 * into idx (capacity K) and returns how many there are. */
int32_t ora_find_outliers(const uint16_t *X, int64_t M, int64_t K, int64_t ldx,
                          float threshold, int32_t *idx)
{
    unsigned char *hit = calloc((size_t)(K > 0 ? K : 1), 1);
    for (int64_t i = 0; i < M; ++i)
        for (int64_t k = 0; k < K; ++k)
            if (fabsf(ora_half(X[i * ldx + k])) >= threshold)
                hit[k] = 1;
    int32_t count = 0;
    for (int64_t k = 0; k < K; ++k)
        if (hit[k])
            idx[count++] = (int32_t)k;
    free(hit);
    return count;
}

/* Activation side ([P2] section 2.1 and 2.3: one scale per row of the
 * non-outlier part X_normal). m[i] = max over non-outlier k of |X[i, k]|;
 * Xq[i, k] = 0 on outlier columns, else the quantized value. Xq is [M x K],
 * K-contiguous. */
void ora_quantize_rowwise(const uint16_t *X, int64_t M, int64_t K, int64_t ldx,
                          const int32_t *idx, int32_t count, int8_t *Xq, float *m)
{
    unsigned char *is_out = calloc((size_t)(K > 0 ? K : 1), 1);
    for (int32_t p = 0; p < count; ++p)
        is_out[idx[p]] = 1;
    for (int64_t i = 0; i < M; ++i) {
        float mi = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            if (is_out[k])
                continue;
            float a = fabsf(ora_half(X[i * ldx + k]));
            if (a > mi)
                mi = a;
        }
        m[i] = mi;
        float inv = mi > 0.0f ? 127.0f / mi : 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            if (is_out[k] || mi == 0.0f)
                Xq[i * K + k] = 0;
            else
                Xq[i * K + k] = ora_quant(ora_half(X[i * ldx + k]), inv);
        }
    }
    free(is_out);
}

/* The int8 matmul with int32 accumulation ([P1] section 2.2): C[i, n] =
 * sum_k Xq[i, k] * Wq[n, k]. Accumulates in int64 and reports (returns 1)
 * if a result would not fit in int32; it never does for K <= 133144. */
int ora_gemm_i8(const int8_t *Xq, const int8_t *Wq, int64_t M, int64_t N, int64_t K,
                int32_t *C)
{
    int overflow = 0;
    for (int64_t i = 0; i < M; ++i)
        for (int64_t n = 0; n < N; ++n) {
            int64_t acc = 0;
            for (int64_t k = 0; k < K; ++k)
                acc += (int64_t)Xq[i * K + k] * (int64_t)Wq[n * K + k];
            if (acc > INT32_MAX || acc < INT32_MIN)
                overflow = 1;
            C[i * N + n] = (int32_t)acc;
        }
    return overflow;
}

/* The 16-bit outlier product and the merge ([P2] section 2.3; [P5] section
 * 3.3): Y[i, n] = C[i, n] * m[i] * s[n] / 127^2 + sum_{k in O} X[i, k] W[k, n].
 * Evaluated in fp64, outlier terms summed in ascending k. */
void ora_merge(const int32_t *C, const float *m, const float *s,
               const uint16_t *X, int64_t ldx, const uint16_t *W, int64_t ldw,
               const int32_t *idx, int32_t count, int64_t M, int64_t N, double *Y)
{
    double *yo = malloc((size_t)(N > 0 ? N : 1) * sizeof(double));
    for (int64_t i = 0; i < M; ++i) {
        for (int64_t n = 0; n < N; ++n)
            yo[n] = 0.0;
        /* outlier terms of every Y[i, n] summed in ascending k */
        for (int32_t p = 0; p < count; ++p) {
            int64_t k = idx[p];
            double x = (double)ora_half(X[i * ldx + k]);
            for (int64_t n = 0; n < N; ++n)
                yo[n] += x * (double)ora_half(W[k * ldw + n]);
        }
        for (int64_t n = 0; n < N; ++n)
            Y[i * N + n] = (double)C[i * N + n] * (double)m[i] * (double)s[n] / 16129.0 + yo[n];
    }
    free(yo);
}

/* One whole layer call, step by step in the order the pages give: find the
 * outlier columns, quantize X by rows, int8 matmul, 16-bit outlier product,
 * dequantize and add. Wq/s come from ora_quantize_colwise (load time). The
 * intermediates are returned through the caller's buffers. Returns the outlier
 * count, or -1 if an int32 accumulator would overflow. */
int32_t ora_linear(const uint16_t *X, int64_t M, int64_t K, int64_t ldx,
                   const uint16_t *W, int64_t ldw, int64_t N,
                   const int8_t *Wq, const float *s, float threshold,
                   int32_t *idx, int8_t *Xq, float *m, int32_t *C, double *Y)
{
    int32_t count = ora_find_outliers(X, M, K, ldx, threshold, idx);
    ora_quantize_rowwise(X, M, K, ldx, idx, count, Xq, m);
    if (ora_gemm_i8(Xq, Wq, M, N, K, C))
        return -1;
    ora_merge(C, m, s, X, ldx, W, ldw, idx, count, M, N, Y);
    return count;
}

/* Int8-only weight residency ([P2] sections 2.4 and 6: only Wq and s are
 * kept). The 16-bit outlier product then takes the outlier rows of W from the
 * dequantized codes, W_O[k, n] = Wq[n, k] * s[n] / 127, instead of the fp16
 * rows. Otherwise as ora_merge: fp64, outlier terms in ascending k. */
void ora_merge_int8w(const int32_t *C, const float *m, const float *s,
                     const uint16_t *X, int64_t ldx, const int8_t *Wq, int64_t K,
                     const int32_t *idx, int32_t count, int64_t M, int64_t N, double *Y)
{
    double *yo = malloc((size_t)(N > 0 ? N : 1) * sizeof(double));
    for (int64_t i = 0; i < M; ++i) {
        for (int64_t n = 0; n < N; ++n)
            yo[n] = 0.0;
        for (int32_t p = 0; p < count; ++p) {
            int64_t k = idx[p];
            double x = (double)ora_half(X[i * ldx + k]);
            for (int64_t n = 0; n < N; ++n)
                yo[n] += x * ((double)Wq[n * K + k] * (double)s[n] / 127.0);
        }
        for (int64_t n = 0; n < N; ++n)
            Y[i * N + n] = (double)C[i * N + n] * (double)m[i] * (double)s[n] / 16129.0 + yo[n];
    }
    free(yo);
}

/* The traditional 8-bit comparison ([P5] section 2: one scale for the whole
 * matrix; section 1: scale = 127 / max|x|): one absmax over all of W, the same
 * quantizer. Wq is [N x K] as in ora_quantize_colwise. Returns the absmax. */
float ora_quantize_tensorwise(const uint16_t *W, int64_t K, int64_t N, int64_t ldw, int8_t *Wq)
{
    float sw = 0.0f;
    for (int64_t k = 0; k < K; ++k)
        for (int64_t n = 0; n < N; ++n) {
            float a = fabsf(ora_half(W[k * ldw + n]));
            if (a > sw)
                sw = a;
        }
    float inv = sw > 0.0f ? 127.0f / sw : 0.0f;
    for (int64_t k = 0; k < K; ++k)
        for (int64_t n = 0; n < N; ++n)
            Wq[n * K + k] = sw > 0.0f ? ora_quant(ora_half(W[k * ldw + n]), inv) : 0;
    return sw;
}

/* The traditional 8-bit linear layer: one absmax over all of X, the int8
 * matmul, and Y = C * sx * sw / 127^2 (fp64). No outlier decomposition. Xq is
 * [M x K]; returns sx. */
float ora_linear_tensorwise(const uint16_t *X, int64_t M, int64_t K, int64_t ldx,
                            const int8_t *Wq, float sw, int64_t N, int8_t *Xq, int32_t *C,
                            double *Y)
{
    float sx = 0.0f;
    for (int64_t i = 0; i < M; ++i)
        for (int64_t k = 0; k < K; ++k) {
            float a = fabsf(ora_half(X[i * ldx + k]));
            if (a > sx)
                sx = a;
        }
    float inv = sx > 0.0f ? 127.0f / sx : 0.0f;
    for (int64_t i = 0; i < M; ++i)
        for (int64_t k = 0; k < K; ++k)
            Xq[i * K + k] = sx > 0.0f ? ora_quant(ora_half(X[i * ldx + k]), inv) : 0;
    ora_gemm_i8(Xq, Wq, M, N, K, C);
    for (int64_t i = 0; i < M; ++i)
        for (int64_t n = 0; n < N; ++n)
            Y[i * N + n] = (double)C[i * N + n] * (double)sx * (double)sw / 16129.0;
    return sx;
}

/* The bias of the layer, added after the rescale ([P1] section 2.2):
 * Y[i, n] += b[n] with b an fp16 vector of N entries. */
void ora_add_bias(double *Y, int64_t M, int64_t N, const uint16_t *bias)
{
    for (int64_t i = 0; i < M; ++i)
        for (int64_t n = 0; n < N; ++n)
            Y[i * N + n] += (double)ora_half(bias[n]);
}

/* ---- FP8 (E4M3) variant of the decomposition ([P4] sections 2 and 4) ---- */

/* Value of an E4M3 code: sign, 4-bit exponent field e (bias 7), 3-bit mantissa
 * field f. e = 0 is subnormal (f/8 * 2^-6); otherwise (1 + f/8) * 2^(e-7).
 * e = 15, f = 7 is NaN (the format has no infinities). */
double ora_e4m3_value(uint8_t c)
{
    unsigned e = (c >> 3) & 0xfu, f = c & 7u;
    double v;
    if (e == 15 && f == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)f, -9);
    else
        v = ldexp((double)(8u + f), (int)e - 10);
    return (c & 0x80u) ? -v : v;
}

/* Nearest E4M3 code to a finite fp32 value: the 127 non-negative finite codes
 * 0x00 .. 0x7e are in increasing order of value, so a binary search brackets
 * |t| between two neighbours; the nearer one wins and a tie goes to the even
 * code (even mantissa). |t| above 448 gives 448. The sign is copied (so -0 and
 * small negative values that round to zero give 0x80). */
uint8_t ora_e4m3_encode(float t)
{
    double a = fabs((double)t);
    uint8_t sign = signbit(t) ? 0x80u : 0u;
    if (a >= 448.0)
        return sign | 0x7eu;
    unsigned lo = 0, hi = 0x7e; /* value(lo) <= a < value(hi) */
    while (hi - lo > 1) {
        unsigned mid = (lo + hi) / 2;
        if (ora_e4m3_value((uint8_t)mid) <= a)
            lo = mid;
        else
            hi = mid;
    }
    double dlo = a - ora_e4m3_value((uint8_t)lo), dhi = ora_e4m3_value((uint8_t)hi) - a;
    unsigned c = dlo < dhi ? lo : dhi < dlo ? hi : ((lo & 1u) ? hi : lo);
    return sign | (uint8_t)c;
}

void ora_e4m3_encode_array(const float *t, int64_t n, uint8_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = ora_e4m3_encode(t[i]);
}

void ora_e4m3_value_array(const uint8_t *c, int64_t n, double *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = ora_e4m3_value(c[i]);
}

/* The E4M3 code of x under absmax a: x * fl32(448 / a) in fp32, then encoded;
 * a = 0 gives code 0. */
static uint8_t ora_quant_fp8(float x, float a)
{
    if (!(a > 0.0f))
        return 0;
    float inv = 448.0f / a;
    float t = x * inv;
    return ora_e4m3_encode(t);
}

/* Weight side of the FP8 variant: s[n] = max_k |W[k, n]| over all K rows;
 * Wq8 [N x K] holds the E4M3 codes of W[k, n] under s[n]. */
void ora_quantize_colwise_fp8(const uint16_t *W, int64_t K, int64_t N, int64_t ldw,
                              uint8_t *Wq8, float *s)
{
    for (int64_t n = 0; n < N; ++n)
        s[n] = 0.0f;
    for (int64_t k = 0; k < K; ++k)
        for (int64_t n = 0; n < N; ++n) {
            float a = fabsf(ora_half(W[k * ldw + n]));
            if (a > s[n])
                s[n] = a;
        }
    for (int64_t k = 0; k < K; ++k)
        for (int64_t n = 0; n < N; ++n)
            Wq8[n * K + k] = ora_quant_fp8(ora_half(W[k * ldw + n]), s[n]);
}

/* Activation side of the FP8 variant: m[i] = max over non-outlier k of
 * |X[i, k]|; Xq8 [M x K] holds the E4M3 codes under m[i], 0 on outlier
 * columns. */
void ora_quantize_rowwise_fp8(const uint16_t *X, int64_t M, int64_t K, int64_t ldx,
                              const int32_t *idx, int32_t count, uint8_t *Xq8, float *m)
{
    unsigned char *is_out = calloc((size_t)(K > 0 ? K : 1), 1);
    for (int32_t p = 0; p < count; ++p)
        is_out[idx[p]] = 1;
    for (int64_t i = 0; i < M; ++i) {
        float mi = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            float a = fabsf(ora_half(X[i * ldx + k]));
            if (!is_out[k] && a > mi)
                mi = a;
        }
        m[i] = mi;
        for (int64_t k = 0; k < K; ++k)
            Xq8[i * K + k] = is_out[k] ? 0 : ora_quant_fp8(ora_half(X[i * ldx + k]), mi);
    }
    free(is_out);
}

/* The fp8 matmul: C[i, n] = sum_k value(Xq8[i, k]) * value(Wq8[n, k]) in fp64
 * (every product is exact), ascending k. */
void ora_gemm_fp8(const uint8_t *Xq8, const uint8_t *Wq8, int64_t M, int64_t N, int64_t K,
                  double *C)
{
    double value[256]; /* ora_e4m3_value of every code, looked up below */
    for (int c = 0; c < 256; ++c)
        value[c] = ora_e4m3_value((uint8_t)c);
    double *xv = malloc((size_t)(K > 0 ? K : 1) * sizeof(double));
    for (int64_t i = 0; i < M; ++i) {
        for (int64_t k = 0; k < K; ++k)
            xv[k] = value[Xq8[i * K + k]];
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k)
                acc += xv[k] * value[Wq8[n * K + k]];
            C[i * N + n] = acc;
        }
    }
    free(xv);
}

/* Merge of the FP8 variant: Y[i, n] = C[i, n] * m[i] * s[n] / 448^2 + the
 * 16-bit outlier product over the fp16 rows of W (as ora_merge), fp64. */
void ora_merge_fp8(const double *C, const float *m, const float *s,
                   const uint16_t *X, int64_t ldx, const uint16_t *W, int64_t ldw,
                   const int32_t *idx, int32_t count, int64_t M, int64_t N, double *Y)
{
    double *yo = malloc((size_t)(N > 0 ? N : 1) * sizeof(double));
    for (int64_t i = 0; i < M; ++i) {
        for (int64_t n = 0; n < N; ++n)
            yo[n] = 0.0;
        for (int32_t p = 0; p < count; ++p) {
            int64_t k = idx[p];
            double x = (double)ora_half(X[i * ldx + k]);
            for (int64_t n = 0; n < N; ++n)
                yo[n] += x * (double)ora_half(W[k * ldw + n]);
        }
        for (int64_t n = 0; n < N; ++n)
            Y[i * N + n] = C[i * N + n] * (double)m[i] * (double)s[n] / 200704.0 + yo[n];
    }
    free(yo);
}
