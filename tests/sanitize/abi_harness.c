/*
 * Sanitizer harness for the argument checks of the C ABI (include/llmint8.h).
 * Built with AddressSanitizer and UndefinedBehaviorSanitizer on the host side
 * of both this program and the library, it calls every entry point with
 * arguments that must be rejected before any HIP call (null and misaligned
 * pointers, bad sizes and pitches, K past the int32 bound, NaN thresholds,
 * short workspaces, bad option structs) and the size queries at extreme
 * shapes, and checks each status. The pointers are never dereferenced: a
 * rejected call enqueues nothing, so no device is needed (the run hides them).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "llmint8.h"

static int failures = 0;

static void expect(const char *what, int got, int want)
{
    if (got != want) {
        fprintf(stderr, "%s: status %d, expected %d\n", what, got, want);
        ++failures;
    }
}

#define P(x) ((void *)(uintptr_t)(x))
#define A P(0x100000)
#define B P(0x200000)
#define MIS P(0x300008)

int main(void)
{
    const float inf = INFINITY, nan = NAN;
    const int64_t big = (int64_t)1 << 40;
    /* quantize_colwise */
    expect("colwise null W", llmint8_quantize_colwise(NULL, 64, 32, 32, B, A, NULL), 1);
    expect("colwise K 0", llmint8_quantize_colwise(A, 0, 32, 32, B, A, NULL), 1);
    expect("colwise huge K", llmint8_quantize_colwise(A, big, 32, 32, B, A, NULL), 1);
    expect("colwise huge N", llmint8_quantize_colwise(A, 64, big, big, B, A, NULL), 1);
    expect("colwise ld short", llmint8_quantize_colwise(A, 64, 32, 16, B, A, NULL), 1);
    expect("colwise misaligned", llmint8_quantize_colwise(MIS, 64, 32, 32, B, A, NULL), 2);
    expect("colwise K past bound", llmint8_quantize_colwise(A, 133152, 32, 32, B, A, NULL), 3);
    expect("colwise INT64_MAX",
           llmint8_quantize_colwise(A, INT64_MAX, INT64_MAX, INT64_MAX, B, A, NULL), 1);
    expect("colwise INT64_MIN", llmint8_quantize_colwise(A, INT64_MIN, 32, 32, B, A, NULL), 1);
    /* find_outliers */
    expect("find nan", llmint8_find_outliers(A, 4, 64, 64, nan, B, B, A, 0, NULL), 1);
    expect("find small ws", llmint8_find_outliers(A, 4, 64, 64, 6.f, B, B, A, 16, NULL), 4);
    expect("find huge M", llmint8_find_outliers(A, INT64_MAX, 64, 64, 6.f, B, B, A, 0, NULL), 1);
    expect("find negative ld", llmint8_find_outliers(A, 4, 64, -64, 6.f, B, B, A, 0, NULL), 1);
    /* quantize_rowwise */
    expect("rowq idx without count",
           llmint8_quantize_rowwise(A, 4, 64, 64, A, NULL, B, A, NULL), 1);
    expect("rowq misaligned m", llmint8_quantize_rowwise(A, 4, 64, 64, NULL, NULL, B, MIS, NULL), 2);
    expect("rowq K past bound",
           llmint8_quantize_rowwise(A, 4, 200000, 200000, NULL, NULL, B, A, NULL), 3);
    /* linear */
    expect("linear null W finite",
           llmint8_linear(A, 4, 64, 64, B, A, NULL, 32, 32, 6.f, B, 32, NULL, NULL, A, 0, NULL), 1);
    expect("linear null W inf, small ws",
           llmint8_linear(A, 4, 64, 64, B, A, NULL, 32, 32, inf, B, 32, NULL, NULL, A, 0, NULL), 4);
    expect("linear nan", llmint8_linear(A, 4, 64, 64, B, A, A, 32, 32, nan, B, 32, NULL, NULL,
                                        A, 0, NULL), 1);
    expect("linear ldy short", llmint8_linear(A, 4, 64, 64, B, A, A, 32, 32, 6.f, B, 8, NULL,
                                              NULL, A, 0, NULL), 1);
    expect("linear huge sizes", llmint8_linear(A, INT64_MAX, 64, 64, B, A, A, 32, INT64_MAX,
                                               6.f, B, INT64_MAX, NULL, NULL, A, 0, NULL), 1);
    expect("linear ldy past tile bound",
           llmint8_linear(A, 4, 64, 64, B, A, A, 32, 32, 6.f, B, (int64_t)1 << 21, NULL, NULL,
                          A, (size_t)1 << 40, NULL), 2);
    expect("linear misaligned C_debug",
           llmint8_linear(A, 4, 64, 64, B, A, A, 32, 32, 6.f, B, 32, NULL, MIS, A,
                          (size_t)1 << 40, NULL), 2);
    llmint8_linear_opts o;
    memset(&o, 0, sizeof o);
    o.struct_size = sizeof o - 8;
    expect("linear_ex old struct", llmint8_linear_ex(A, 4, 64, 64, B, A, A, 32, 32, 6.f, B, 32,
                                                     NULL, NULL, A, 0, NULL, &o), 1);
    o.struct_size = sizeof o;
    o.outlier_weights = 7;
    expect("linear_ex bad mode", llmint8_linear_ex(A, 4, 64, 64, B, A, A, 32, 32, 6.f, B, 32,
                                                   NULL, NULL, A, 0, NULL, &o), 1);
    o.outlier_weights = LLMINT8_OUTLIER_W_INT8;
    o.bias = MIS;
    expect("linear_ex misaligned bias", llmint8_linear_ex(A, 4, 64, 64, B, A, NULL, 32, 32, 6.f,
                                                          B, 32, NULL, NULL, A, 0, NULL, &o), 2);
    o.bias = NULL;
    expect("linear_ex int8 weights small ws",
           llmint8_linear_ex(A, 4, 64, 64, B, A, NULL, 32, 32, 6.f, B, 32, NULL, NULL, A, 0,
                             NULL, &o), 4);
    /* the allocation-free layer: every check first, then the scratch size */
    expect("noalloc null X", llmint8_linear_noalloc(NULL, 4, 64, 64, B, A, A, 32, 32, 6.f, B, 32,
                                                    NULL, NULL, NULL), 1);
    expect("noalloc nan", llmint8_linear_noalloc(A, 4, 64, 64, B, A, A, 32, 32, nan, B, 32, NULL,
                                                 NULL, NULL), 1);
    expect("noalloc beyond scratch",
           llmint8_linear_noalloc(A, 2048, 4096, 4096, B, A, A, 11008, 11008, 6.f, B, 11008,
                                  NULL, NULL, NULL), 4);
    expect("noalloc huge", llmint8_linear_noalloc(A, ((int64_t)1 << 31) - 1, 133136, 133136, B,
                                                  A, A, 65536, 65536, 6.f, B, 65536, NULL, NULL,
                                                  NULL), 4);
    /* per-tensor and FP8 */
    expect("qtw small ws", llmint8_quantize_tensorwise(A, 64, 32, 32, B, A, A, 16, NULL), 4);
    expect("ltw ldy short", llmint8_linear_tensorwise(A, 4, 64, 64, B, A, 32, NULL, B, 16, NULL,
                                                      NULL, A, 0, NULL), 1);
    expect("cfp8 N not mult 8", llmint8_quantize_colwise_fp8(A, 64, 30, 32, B, A, NULL), 2);
    expect("rfp8 misaligned", llmint8_quantize_rowwise_fp8(A, 4, 64, 64, NULL, NULL, MIS, A,
                                                           NULL), 2);
    o.outlier_weights = LLMINT8_OUTLIER_W_INT8;
    expect("lfp8 int8 weights", llmint8_linear_fp8(A, 4, 64, 64, B, A, A, 32, 32, 6.f, B, 32,
                                                   NULL, NULL, A, (size_t)1 << 40, NULL, &o), 1);
    /* size queries: zero for impossible shapes, no overflow at the largest ones */
    expect("ws zero M", (int)(llmint8_workspace_size(0, 64, 64) != 0), 0);
    expect("ws K past bound", (int)(llmint8_workspace_size(4, 133160, 64) != 0), 0);
    expect("ws max", (int)(llmint8_workspace_size(((int64_t)1 << 31) - 1, 133136,
                                                  ((int64_t)1 << 31) - 1) == 0), 0);
    expect("find ws max", (int)(llmint8_find_outliers_workspace_size(((int64_t)1 << 31) - 1,
                                                                      133136) == 0), 0);
    expect("fp8 ws max", (int)(llmint8_linear_fp8_workspace_size(65, 133136,
                                                                 ((int64_t)1 << 31) - 1) == 0), 0);
    expect("ltw ws max", (int)(llmint8_linear_tensorwise_workspace_size(
                                   ((int64_t)1 << 31) - 1, 133136, ((int64_t)1 << 31) - 1) == 0),
           0);
    for (int st = -1; st < 8; ++st)
        if (!llmint8_status_string(st) || strncmp(llmint8_status_string(st), "LLMINT8", 7) != 0)
            ++failures;
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("abi harness: clean\n");
    return 0;
}
