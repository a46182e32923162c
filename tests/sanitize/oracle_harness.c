/*
 * Sanitizer harness for the CPU oracle (built with AddressSanitizer and
 * UndefinedBehaviorSanitizer, no recovery): drives every oracle entry point on
 * seeded small shapes and the edge cases of the method, so that an
 * out-of-bounds access, a use of freed memory or an undefined operation in any
 * of them aborts the run. It also checks a few facts that hold for every
 * input: codes within [-127, 127], outlier columns coded 0, ascending outlier
 * indices and C within 127^2 (K - |O|) in magnitude.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

void ora_half_to_float(const uint16_t *h, int64_t n, float *out);
void ora_quantize_colwise(const uint16_t *W, int64_t K, int64_t N, int64_t ldw, int8_t *Wq,
                          float *s);
int32_t ora_find_outliers(const uint16_t *X, int64_t M, int64_t K, int64_t ldx, float threshold,
                          int32_t *idx);
void ora_quantize_rowwise(const uint16_t *X, int64_t M, int64_t K, int64_t ldx,
                          const int32_t *idx, int32_t count, int8_t *Xq, float *m);
int ora_gemm_i8(const int8_t *Xq, const int8_t *Wq, int64_t M, int64_t N, int64_t K, int32_t *C);
void ora_merge(const int32_t *C, const float *m, const float *s, const uint16_t *X, int64_t ldx,
               const uint16_t *W, int64_t ldw, const int32_t *idx, int32_t count, int64_t M,
               int64_t N, double *Y);
void ora_merge_int8w(const int32_t *C, const float *m, const float *s, const uint16_t *X,
                     int64_t ldx, const int8_t *Wq, int64_t K, const int32_t *idx, int32_t count,
                     int64_t M, int64_t N, double *Y);
int32_t ora_linear(const uint16_t *X, int64_t M, int64_t K, int64_t ldx, const uint16_t *W,
                   int64_t ldw, int64_t N, const int8_t *Wq, const float *s, float threshold,
                   int32_t *idx, int8_t *Xq, float *m, int32_t *C, double *Y);
float ora_quantize_tensorwise(const uint16_t *W, int64_t K, int64_t N, int64_t ldw, int8_t *Wq);
float ora_linear_tensorwise(const uint16_t *X, int64_t M, int64_t K, int64_t ldx,
                            const int8_t *Wq, float sw, int64_t N, int8_t *Xq, int32_t *C,
                            double *Y);
void ora_add_bias(double *Y, int64_t M, int64_t N, const uint16_t *bias);
void ora_e4m3_encode_array(const float *t, int64_t n, uint8_t *out);
void ora_e4m3_value_array(const uint8_t *c, int64_t n, double *out);
void ora_quantize_colwise_fp8(const uint16_t *W, int64_t K, int64_t N, int64_t ldw,
                              uint8_t *Wq8, float *s);
void ora_quantize_rowwise_fp8(const uint16_t *X, int64_t M, int64_t K, int64_t ldx,
                              const int32_t *idx, int32_t count, uint8_t *Xq8, float *m);
void ora_gemm_fp8(const uint8_t *Xq8, const uint8_t *Wq8, int64_t M, int64_t N, int64_t K,
                  double *C);
void ora_merge_fp8(const double *C, const float *m, const float *s, const uint16_t *X,
                   int64_t ldx, const uint16_t *W, int64_t ldw, const int32_t *idx,
                   int32_t count, int64_t M, int64_t N, double *Y);

static uint64_t state = 0x9e3779b97f4a7c15ull;
static uint32_t next(void)
{ /* xorshift64*: any fixed sequence will do */
    state ^= state >> 12;
    state ^= state << 25;
    state ^= state >> 27;
    return (uint32_t)((state * 0x2545f4914f6cdd1dull) >> 32);
}

/* fp16 patterns: mostly small normal values, some large, zeros, subnormals,
 * and (when asked) infinities and NaNs */
static uint16_t rand_half(int specials)
{
    uint32_t r = next() % 100;
    uint16_t sign = (uint16_t)((next() & 1u) << 15);
    if (r < 5)
        return sign;                                   /* +-0 */
    if (r < 10)
        return sign | (uint16_t)(next() % 0x400u);     /* subnormal */
    if (specials && r < 12)
        return sign | 0x7c00u;                         /* inf */
    if (specials && r < 14)
        return sign | (uint16_t)(0x7c01u + next() % 0x3ffu); /* NaN */
    if (r < 20)
        return sign | (uint16_t)(0x4600u + next() % 0x1800u); /* 6 .. 2^15 */
    return sign | (uint16_t)(0x2000u + next() % 0x2400u);   /* about 2^-7 .. 4 */
}

static int failures = 0;
#define CHECK(c) do { if (!(c)) { fprintf(stderr, "check failed line %d: %s\n", __LINE__, #c); ++failures; } } while (0)

static void one_case(int64_t M, int64_t K, int64_t N, float threshold, int specials)
{
    int64_t ldx = K + (next() % 2) * 8, ldw = N + (next() % 2) * 8;
    uint16_t *X = malloc(sizeof(uint16_t) * (size_t)(M * ldx));
    uint16_t *W = malloc(sizeof(uint16_t) * (size_t)(K * ldw));
    uint16_t *bias = malloc(sizeof(uint16_t) * (size_t)N);
    for (int64_t i = 0; i < M * ldx; ++i)
        X[i] = rand_half(specials);
    for (int64_t i = 0; i < K * ldw; ++i)
        W[i] = rand_half(0);
    for (int64_t i = 0; i < N; ++i)
        bias[i] = rand_half(0);
    if (M > 1)
        memset(X, 0, sizeof(uint16_t) * (size_t)K); /* a zero row */
    int8_t *Wq = malloc((size_t)(N * K));
    float *s = malloc(sizeof(float) * (size_t)N);
    int32_t *idx = malloc(sizeof(int32_t) * (size_t)K);
    int8_t *Xq = malloc((size_t)(M * K));
    float *m = malloc(sizeof(float) * (size_t)M);
    int32_t *C = malloc(sizeof(int32_t) * (size_t)(M * N));
    double *Y = malloc(sizeof(double) * (size_t)(M * N));
    float *f = malloc(sizeof(float) * (size_t)(M * ldx));

    ora_half_to_float(X, M * ldx, f);
    ora_quantize_colwise(W, K, N, ldw, Wq, s);
    int32_t count = ora_linear(X, M, K, ldx, W, ldw, N, Wq, s, threshold, idx, Xq, m, C, Y);
    CHECK(count >= 0 && count <= K);
    for (int32_t p = 1; p < count; ++p)
        CHECK(idx[p] > idx[p - 1]);
    for (int64_t i = 0; i < M * K; ++i)
        CHECK(Xq[i] >= -127 && Xq[i] <= 127);
    for (int64_t i = 0; i < M; ++i)
        for (int32_t p = 0; p < count; ++p)
            CHECK(Xq[i * K + idx[p]] == 0);
    for (int64_t i = 0; i < M * N; ++i)
        CHECK(llabs((long long)C[i]) <= 16129LL * (K - count));
    ora_merge_int8w(C, m, s, X, ldx, Wq, K, idx, count, M, N, Y);
    ora_add_bias(Y, M, N, bias);
    CHECK(ora_find_outliers(X, M, K, ldx, threshold, idx) == count);
    ora_quantize_rowwise(X, M, K, ldx, idx, count, Xq, m);
    CHECK(ora_gemm_i8(Xq, Wq, M, N, K, C) == 0);
    ora_merge(C, m, s, X, ldx, W, ldw, idx, count, M, N, Y);

    float sw = ora_quantize_tensorwise(W, K, N, ldw, Wq);
    ora_linear_tensorwise(X, M, K, ldx, Wq, sw, N, Xq, C, Y);

    uint8_t *Wq8 = malloc((size_t)(N * K));
    uint8_t *Xq8 = malloc((size_t)(M * K));
    double *C8 = malloc(sizeof(double) * (size_t)(M * N));
    ora_quantize_colwise_fp8(W, K, N, ldw, Wq8, s);
    ora_quantize_rowwise_fp8(X, M, K, ldx, idx, count, Xq8, m);
    ora_gemm_fp8(Xq8, Wq8, M, N, K, C8);
    ora_merge_fp8(C8, m, s, X, ldx, W, ldw, idx, count, M, N, Y);
    uint8_t codes[256];
    double vals[256];
    float t[256];
    for (int c = 0; c < 256; ++c) {
        codes[c] = (uint8_t)c;
        t[c] = ldexpf((float)(int)(next() % 2000) - 1000.0f, (int)(next() % 20) - 12);
    }
    ora_e4m3_value_array(codes, 256, vals);
    ora_e4m3_encode_array(t, 256, codes);
    free(Wq8); free(Xq8); free(C8);
    free(X); free(W); free(bias); free(Wq); free(s); free(idx); free(Xq); free(m); free(C);
    free(Y); free(f);
}

int main(void)
{
    const float thresholds[] = {6.0f, 0.0f, -1.0f, INFINITY, 2.5f, 1e-3f};
    int cases = 0;
    for (int rep = 0; rep < 60; ++rep) {
        int64_t M = 1 + next() % 40, K = 16 * (1 + next() % 12), N = 8 * (1 + next() % 10);
        float thr = thresholds[next() % 6];
        one_case(M, K, N, thr, rep % 3 == 0);
        ++cases;
    }
    /* edge shapes: one row, one 16-column chunk, every column an outlier */
    one_case(1, 16, 8, 6.0f, 0);
    one_case(1, 16, 8, 0.0f, 0);
    one_case(3, 16, 8, INFINITY, 1);
    one_case(64, 256, 8, 0.0f, 1);
    cases += 4;
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("oracle harness: %d cases clean\n", cases);
    return 0;
}
