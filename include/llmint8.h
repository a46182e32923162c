/*
 * llmint8.h - C ABI of the MI355X (gfx950) LLM.int8() mixed-precision linear layer.
 *
 * The layer computes Y = X . W for an fp16 activation X [M x K] and an fp16
 * weight W [K x N] the way LLM.int8() does ("8-bit quantization of giant
 * language models: LLM.int8()" walkthrough, 2kiu.com, sections 2.1 and 2.3;
 * "LLM.int8() pitfalls" page, codearts.csdn.net, sections 1 and 3):
 *
 *   1. the outlier columns O of X are those with some |X[i, k]| >= threshold;
 *   2. X without those columns is quantized per row:   m[i] = max_{k not in O} |X[i, k]|,
 *      Xq[i, k] = clamp(rint(X[i, k] * fl32(127 / m[i])), -127, 127), Xq[i, O] = 0;
 *   3. W is quantized per column (output channel):     s[n] = max_k |W[k, n]|,
 *      Wq[n, k] = clamp(rint(W[k, n] * fl32(127 / s[n])), -127, 127);
 *   4. C = Xq . Wq^T with int32 accumulation (exact);
 *   5. Y[i, n] = fp16( C[i, n] * m[i] * s[n] / 127^2 + sum_{k in O} X[i, k] W[k, n] ),
 *      the second term an fp16 product with fp32 accumulation.
 * rint rounds half to even; a zero absmax gives an all-zero row/column.
 *
 * Conventions shared by every call:
 *   - Every pointer is a DEVICE pointer unless stated otherwise. fp16 data is
 *     passed as uint16_t IEEE binary16 bit patterns. `stream` is a hipStream_t
 *     (NULL = the default stream).
 *   - Matrices are row-major with an explicit leading dimension in elements.
 *   - The caller owns and allocates every buffer, including the workspace. The
 *     library never allocates device memory, keeps no state between calls and
 *     is re-entrant; calls that share a workspace must be ordered on one stream.
 *     The one exception is llmint8_linear_noalloc, whose workspace is a fixed
 *     scratch array the library holds on each GPU (see there).
 *   - Calls are asynchronous: they enqueue kernels on `stream` and return.
 *     Results are valid once the caller synchronizes with the stream. Inputs
 *     and outputs must not overlap.
 *   - Shape/alignment rules (else LLMINT8_ERR_UNSUPPORTED): every pointer is
 *     16-byte aligned; K is a multiple of 16; N is a multiple of 8; ldx, ldw and
 *     ldy are multiples of 8. M >= 1 is otherwise unrestricted. An empty input
 *     (M, K or N below 1) is LLMINT8_ERR_INVALID_ARG.
 *   - Arguments are validated before any HIP call is made. A failed check
 *     enqueues nothing and leaves every output untouched. Device faults surface
 *     at the caller's next synchronization.
 *   - Inputs are meant to be finite. An infinite entry of X makes its column an
 *     outlier. A NaN entry of X is never an outlier and never sets a row
 *     absmax, on every path; its own code, and so the row of C and Y it lies
 *     in, are unspecified. Other rows are unaffected.
 */
#ifndef LLMINT8_H_
#define LLMINT8_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every int-returning call. */
#define LLMINT8_OK 0
#define LLMINT8_ERR_INVALID_ARG 1  /* NULL required pointer, size <= 0, ld < row length, NaN threshold */
#define LLMINT8_ERR_UNSUPPORTED 2  /* alignment / multiple-of rule above is broken */
#define LLMINT8_ERR_OVERFLOW 3     /* K > LLMINT8_MAX_K: an int32 accumulator could overflow */
#define LLMINT8_ERR_WORKSPACE 4    /* workspace NULL or smaller than the size query returns */
#define LLMINT8_ERR_HIP 5          /* a HIP launch or runtime call failed */

/* Largest K for which 127 * 127 * K fits in int32. */
#define LLMINT8_MAX_K 133144

/*
 * Weight quantization, run once per weight at load time (walkthrough page,
 * section 2.1: one scale per column of W; section 6: quantize once, reuse).
 *   W          [K x N] fp16, row-major, leading dimension ldw >= N.
 *   Wq         [N x K] int8 output: row n is output channel n, K-contiguous.
 *   col_absmax [N] fp32 output: s[n] = max_k |W[k, n]| over all K rows.
 * Bit-exact with the definition above (fp32 scale, round half to even).
 */
int llmint8_quantize_colwise(const uint16_t *W, int64_t K, int64_t N, int64_t ldw,
                             int8_t *Wq, float *col_absmax, void *stream);

/*
 * Outlier-column detection (walkthrough page, sections 2.3 and 4.2: a column
 * whose absolute maximum reaches the threshold, default 6.0, goes the 16-bit
 * way; rescanned on every call).
 *   X         [M x K] fp16, leading dimension ldx >= K.
 *   threshold  host float; +inf gives no outliers, <= 0 makes every column one.
 *   idx       [K] int32 output: the outlier columns in ascending order in
 *             idx[0 .. *count); entries beyond *count are unspecified.
 *   count     [1] int32 output (device): |O|.
 *   workspace  device scratch of at least llmint8_find_outliers_workspace_size(M, K) bytes.
 */
size_t llmint8_find_outliers_workspace_size(int64_t M, int64_t K);
int llmint8_find_outliers(const uint16_t *X, int64_t M, int64_t K, int64_t ldx, float threshold,
                          int32_t *idx, int32_t *count, void *workspace, size_t workspace_bytes,
                          void *stream);

/*
 * Row-wise (per-token) quantization of X without its outlier columns
 * (walkthrough page, sections 2.1 and 2.3; codearts page, section 1).
 *   X          [M x K] fp16, leading dimension ldx >= K.
 *   idx, count outlier columns as produced by llmint8_find_outliers (device):
 *              idx holds K entries (the first *count are used; the call may
 *              read all K). Both NULL means no outlier columns.
 *   Xq         [M x K] int8 output, leading dimension K; outlier columns are 0.
 *   row_absmax [M] fp32 output: m[i] = max over non-outlier k of |X[i, k]|.
 */
int llmint8_quantize_rowwise(const uint16_t *X, int64_t M, int64_t K, int64_t ldx,
                             const int32_t *idx, const int32_t *count, int8_t *Xq,
                             float *row_absmax, void *stream);

/*
 * The whole layer: detection, row quantization of X, int8 GEMM with int32
 * accumulation, fp16 outlier product and the dequantize-and-add merge, on one
 * stream with no host synchronization (the outlier count never leaves the GPU).
 *   X          [M x K] fp16, leading dimension ldx >= K.
 *   Wq, col_absmax  from llmint8_quantize_colwise (Wq [N x K], K-contiguous).
 *   W          [K x N] fp16, leading dimension ldw >= N: the original weight,
 *              whose rows k in O feed the 16-bit product. May be NULL only when
 *              threshold is +inf.
 *   threshold  host float, default in the pages 6.0.
 *   Y          [M x N] fp16 output, leading dimension ldy >= N.
 *   outlier_count_out  optional [1] int32 output (device): |O|.
 *   C_debug    optional [M x N] int32 output (leading dimension N): the exact
 *              int32 accumulators of step 4.
 *   workspace  device scratch of at least llmint8_workspace_size(M, K, N) bytes.
 * When the outlier share is large, the int8 GEMM runs over the K - |O| kept
 * columns only (compacted operands); when a large-M call's output tiles
 * (128 x 256 or 256 x 256) number fewer than the GPU's 256 CUs, each tile's
 * k range is split into parts whose int32 sums meet in the workspace. Up to
 * 64 rows, and up to 256 when the shape lets the small-M kernels stream K in
 * one pass, the call takes the small-M kernels. The result is identical
 * either way.
 */
size_t llmint8_workspace_size(int64_t M, int64_t K, int64_t N);
int llmint8_linear(const uint16_t *X, int64_t M, int64_t K, int64_t ldx,
                   const int8_t *Wq, const float *col_absmax,
                   const uint16_t *W, int64_t ldw, int64_t N, float threshold,
                   uint16_t *Y, int64_t ldy, int32_t *outlier_count_out, int32_t *C_debug,
                   void *workspace, size_t workspace_bytes, void *stream);

/*
 * llmint8_linear without a workspace argument, for callers that cannot
 * allocate device memory: code being captured into a HIP graph, tight serving
 * loops, harnesses that forbid hipMalloc. Same arguments, results and checks
 * as llmint8_linear otherwise; the call itself allocates nothing.
 * Its workspace is a static device array of LLMINT8_NOALLOC_SCRATCH_BYTES
 * (32 MiB) inside the library, one per GPU, held until the process ends; its
 * address is looked up on the first call on each device (the only HIP call
 * besides the launches). It never splits the k range of its GEMM tiles, so
 * it needs llmint8_workspace_size(M, K, N) less the split-K area; a call
 * whose need exceeds the scratch returns LLMINT8_ERR_WORKSPACE before any HIP
 * call: in practice this covers the small-M (decode) shapes, M <= 256, and
 * small large-M ones. Every call on one GPU
 * shares its scratch, so calls that may overlap on one GPU (different
 * streams, or host threads without ordering) race; order them on one stream.
 * Nothing in the scratch needs to start at zero: every call writes what it
 * reads.
 */
#define LLMINT8_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int llmint8_linear_noalloc(const uint16_t *X, int64_t M, int64_t K, int64_t ldx,
                           const int8_t *Wq, const float *col_absmax,
                           const uint16_t *W, int64_t ldw, int64_t N, float threshold,
                           uint16_t *Y, int64_t ldy, int32_t *outlier_count_out,
                           int32_t *C_debug, void *stream);

/* Where the 16-bit outlier product takes its weight rows from. */
#define LLMINT8_OUTLIER_W_FP16 0 /* rows k in O of the fp16 weight W */
#define LLMINT8_OUTLIER_W_INT8 1 /* the dequantized codes Wq[n, k] * col_absmax[n] / 127 */

/*
 * Options of llmint8_linear_ex. Zero-initialize, set struct_size =
 * sizeof(llmint8_linear_opts), then fill the fields you use; zero and NULL
 * fields are off. The struct is read during the call only; pointers in it are
 * device pointers, 16-byte aligned.
 *   gemm_begin_event, gemm_end_event  optional hipEvent_t handles (created by
 *       the caller) that the GEMM kernel's own dispatch on `stream` stamps when
 *       the kernel starts and when it completes (no separate stream commands),
 *       so a caller can time the dominant kernel of the layer with
 *       hipEventElapsedTime.
 *   outlier_weights  LLMINT8_OUTLIER_W_FP16 (default) or LLMINT8_OUTLIER_W_INT8:
 *       keep only the int8 weight (walkthrough page, sections 2.4 and 6: the
 *       int8 weights replace the fp16 ones); W may then be NULL at any
 *       threshold. Any other value is LLMINT8_ERR_INVALID_ARG.
 *   bias         optional [N] fp16, added to every row of Y after the rescale
 *       (Lightning Fabric page, section 2.2).
 *   y_col_absmax optional [N] fp32 output: max over the M rows of |Y[i, n]| as
 *       stored (fp16). The next layer can pass it as its x_col_absmax, which
 *       spares its outlier scan a pass over its X.
 *   x_col_absmax optional [K] fp32 input: max over the M rows of |X[i, k]|. The
 *       outlier columns are then taken as those with x_col_absmax[k] >=
 *       threshold, without a scan of X; the caller vouches that it is X's
 *       column absmax (the result follows the values given).
 */
typedef struct llmint8_linear_opts {
  size_t struct_size;
  void *gemm_begin_event;
  void *gemm_end_event;
  int outlier_weights;
  const uint16_t *bias;
  float *y_col_absmax;
  const float *x_col_absmax;
} llmint8_linear_opts;

/* llmint8_linear with options; opts == NULL is exactly llmint8_linear. A
 * struct_size other than sizeof(llmint8_linear_opts) is LLMINT8_ERR_INVALID_ARG. */
int llmint8_linear_ex(const uint16_t *X, int64_t M, int64_t K, int64_t ldx,
                      const int8_t *Wq, const float *col_absmax,
                      const uint16_t *W, int64_t ldw, int64_t N, float threshold,
                      uint16_t *Y, int64_t ldy, int32_t *outlier_count_out, int32_t *C_debug,
                      void *workspace, size_t workspace_bytes, void *stream,
                      const llmint8_linear_opts *opts);

/*
 * The traditional 8-bit layer that LLM.int8() is measured against ("LLM.int8()
 * pitfalls" page, section 2: one scale for the whole matrix; section 1: scale =
 * 127 / max|x|). No outlier decomposition: an outlier sets the scale of every
 * entry. Same conventions and shape rules as the calls above.
 *
 * llmint8_quantize_tensorwise: W [K x N] fp16 (ldw >= N) ->
 *   Wq       [N x K] int8 output, Wq[n, k] = clamp(rint(W[k, n] * fl32(127 / sw)), -127, 127);
 *   w_absmax [1] fp32 output (device): sw = max over all of W of |W[k, n]|.
 *   workspace at least llmint8_quantize_tensorwise_workspace_size(K, N) bytes.
 * Bit-exact with that definition; sw = 0 gives all-zero codes.
 */
size_t llmint8_quantize_tensorwise_workspace_size(int64_t K, int64_t N);
int llmint8_quantize_tensorwise(const uint16_t *W, int64_t K, int64_t N, int64_t ldw,
                                int8_t *Wq, float *w_absmax, void *workspace,
                                size_t workspace_bytes, void *stream);

/*
 * llmint8_linear_tensorwise: Y = fp16( C * sx * sw / 127^2 [+ bias] ) with
 *   sx = max over all of X of |X[i, k]|, Xq = clamp(rint(X * fl32(127 / sx)), -127, 127),
 *   C = Xq . Wq^T (int32, exact).
 *   X          [M x K] fp16, leading dimension ldx >= K.
 *   Wq, w_absmax  from llmint8_quantize_tensorwise.
 *   bias       optional [N] fp16, added after the rescale (Lightning Fabric
 *              page, section 2.2).
 *   Y          [M x N] fp16 output, leading dimension ldy >= N.
 *   x_absmax   optional [1] fp32 output (device): sx.
 *   C_debug    optional [M x N] int32 output (leading dimension N): C.
 *   workspace  at least llmint8_linear_tensorwise_workspace_size(M, K, N) bytes.
 */
size_t llmint8_linear_tensorwise_workspace_size(int64_t M, int64_t K, int64_t N);
int llmint8_linear_tensorwise(const uint16_t *X, int64_t M, int64_t K, int64_t ldx,
                              const int8_t *Wq, const float *w_absmax, int64_t N,
                              const uint16_t *bias, uint16_t *Y, int64_t ldy, float *x_absmax,
                              int32_t *C_debug, void *workspace, size_t workspace_bytes,
                              void *stream);

/*
 * FP8 (E4M3) variant of the decomposition: the same outlier split, with the
 * 8-bit part coded in E4M3 instead of int8 (the "INT8 vs FP8 vs GPTQ" page,
 * mlqm.cn, sections 2 and 4: FP8 E4M3 has 4 exponent and 3 mantissa bits, its
 * largest value is about 448, and wide-ranged inputs need a scale before the
 * cast). E4M3 here
 * is the OCP 8-bit format: bias 7, subnormals, no infinities, 0x7f/0xff NaN.
 *   codes:  q = e4m3(x * fl32(448 / absmax)), nearest value, ties to even;
 *           absmax per row of X (outlier columns excluded) and per column of W,
 *           exactly as in steps 2 and 3 above; a zero absmax gives code 0.
 *   matmul: C = value(Xq8) . value(Wq8)^T, products exact, summed by the
 *           E4M3 MFMA into fp32 accumulators;
 *   merge:  Y = fp16( C * m[i] * s[n] / 448^2 + X_O . W_O ).
 * The codes are bit-exact with that definition. C is not: one MFMA adds 64
 * products keeping fewer bits than fp32 (errors up to about 2^-13 of the sum
 * of the magnitudes measured on MI355X).
 *
 * llmint8_quantize_colwise_fp8: as llmint8_quantize_colwise, E4M3 codes.
 *   Wq8 [N x K] uint8 E4M3 codes; col_absmax [N] fp32.
 * llmint8_quantize_rowwise_fp8: as llmint8_quantize_rowwise, E4M3 codes.
 *   Xq8 [M x K] uint8 E4M3 codes (0 on outlier columns); row_absmax [M] fp32.
 * llmint8_linear_fp8: the whole FP8 layer (small-M and large-M paths as for
 *   llmint8_linear, without the single-kernel one), with the arguments of
 *   llmint8_linear_ex except:
 *   Wq8, col_absmax  from llmint8_quantize_colwise_fp8;
 *   C_debug    optional [M x N] fp32 output (leading dimension N): C;
 *   workspace  at least llmint8_linear_fp8_workspace_size(M, K, N) bytes;
 *   opts       may be NULL; outlier_weights must be LLMINT8_OUTLIER_W_FP16
 *              (else LLMINT8_ERR_INVALID_ARG); the events, bias,
 *              y_col_absmax and x_col_absmax act as for llmint8_linear_ex.
 */
int llmint8_quantize_colwise_fp8(const uint16_t *W, int64_t K, int64_t N, int64_t ldw,
                                 uint8_t *Wq8, float *col_absmax, void *stream);
int llmint8_quantize_rowwise_fp8(const uint16_t *X, int64_t M, int64_t K, int64_t ldx,
                                 const int32_t *idx, const int32_t *count, uint8_t *Xq8,
                                 float *row_absmax, void *stream);
size_t llmint8_linear_fp8_workspace_size(int64_t M, int64_t K, int64_t N);
int llmint8_linear_fp8(const uint16_t *X, int64_t M, int64_t K, int64_t ldx,
                       const uint8_t *Wq8, const float *col_absmax,
                       const uint16_t *W, int64_t ldw, int64_t N, float threshold,
                       uint16_t *Y, int64_t ldy, int32_t *outlier_count_out, float *C_debug,
                       void *workspace, size_t workspace_bytes, void *stream,
                       const llmint8_linear_opts *opts);

/* Human-readable name of a status code (static storage, never NULL). */
const char *llmint8_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* LLMINT8_H_ */
