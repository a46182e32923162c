// Internal launchers of the gfx950 kernels. Each returns hipSuccess or the
// error of its launch; none synchronizes.
#pragma once

#include "common.hpp"

namespace llmint8 {

// What the layer's epilogue adds beyond Y = dequant(C) + X_O . W_O.
struct EpilogueOpts {
  int int8w;             // W_O from the int8 codes, Wq[n, k] * s[n] / 127
  const uint16_t *bias;  // optional [N] fp16, added to every row
  float *ycmax;          // optional [N]: max over rows of |Y[i, n]| as stored
};

// Column maxima of |Y| combined across blocks with an integer max on the float
// bits (non-negative floats order like their patterns): the result does not
// depend on the order.
__device__ inline void ycmax_update(float *ycmax, int64_t n, float v) {
  atomicMax((unsigned int *)(ycmax + n), __builtin_bit_cast(unsigned int, v));
}

// |Y| as stored: the fp16 rounding of v, as a float.
__device__ inline float stored_abs(float v) { return __builtin_fabsf(h2f(f2h(v))); }

// Outlier detection is split over row chunks: each (column tile, row chunk)
// block writes one partial column bitmask; a single block ORs them.
struct DetectPlan {
  int row_chunks;
  int rows_per_chunk;
  int col_tiles;
  int64_t kw;  // 32-bit mask words covering K columns
};
DetectPlan detect_plan(int64_t M, int64_t K);

struct DetectOut {
  const float *xcmax;  // optional [K]: column absmax of X supplied by the caller
  float threshold;
  float *ycmax;        // optional [N], zeroed here for the epilogue's maxima
  int64_t N;
  uint32_t *pmask;   // [row_chunks x kw] partial masks (scratch)
  uint32_t *omask;   // [kw] outlier bitmask, bit k%32 of word k/32
  int32_t *wprefix;  // [kw] outliers in words before w
  int32_t *idx;      // [K] ascending outlier columns
  int32_t *count;    // [1]
  int32_t *count_copy;  // optional second copy of the count
  uint32_t *sem;        // optional [nsem] arrival counters of the split-K GEMM, zeroed here
  int64_t nsem;
};

hipError_t launch_detect(const uint16_t *X, int64_t M, int64_t K, int64_t ldx, float threshold,
                         const DetectPlan &plan, const DetectOut &out, hipStream_t stream);

// Row quantization for the public call: outlier columns from an index list.
// Codec (CodecI8 or CodecE4M3) picks the 8-bit encoding of every quantizer.
template <class Codec>
hipError_t launch_rowquant_idx(const uint16_t *X, int64_t M, int64_t K, int64_t ldx,
                               const int32_t *idx, const int32_t *count, uint8_t *Xq, float *m,
                               hipStream_t stream);

// Column absmax + quantize + transpose of W [K x N] into Wq [N x K]; the two
// halves also run alone (s: column maxima out, then the scales the codes use).
template <class Codec>
hipError_t launch_colwise(const uint16_t *W, int64_t K, int64_t N, int64_t ldw, uint8_t *Wq,
                          float *s, hipStream_t stream);
hipError_t launch_colwise_absmax(const uint16_t *W, int64_t K, int64_t N, int64_t ldw, float *s,
                                 hipStream_t stream);
template <class Codec>
hipError_t launch_colwise_quant(const uint16_t *W, int64_t K, int64_t N, int64_t ldw,
                                const float *s, uint8_t *Wq, hipStream_t stream);

// Weight side of a large-M call, one launch: W_O^T [N x ldo] fp16, whose row n
// holds W[idx[p], n] for p < |O| (or, with W null, the int8 codes Wq[n, idx[p]],
// exact in fp16; the epilogue applies s[n] / 127), zeros up to the next
// multiple of 64; and, when the outlier share calls for it, the compacted copy
// Wqc [N x ldq] of Wq without the outlier columns.
struct WeightSideArgs {
  const uint16_t *W;      // fp16 weight [K x N] (null: gather the int8 codes)
  int64_t ldw;
  const int8_t *Wq;       // [N x K]
  int64_t M, K, N;
  const int32_t *idx;     // ascending outlier columns
  const int32_t *count;   // [1]
  uint16_t *wot;
  int64_t ldo;
  const uint32_t *omask;  // outlier bitmask
  const int32_t *wprefix; // outliers in the mask words before w
  int8_t *wqc;
  int64_t ldq;
  int64_t gather_blocks;  // set by the launcher
};

// Row quantization inside the layer: outlier columns from the detection
// bitmask; also gathers the outlier columns into xo [M x ldo] and, when the
// outlier share calls for it, writes compacted rows (K - |O| kept columns).
// Xq rows have pitch ldq (a multiple of 128) and are zero past their last
// column up to the next multiple of 128; xo rows have pitch ldo (a multiple of
// 64) and are zero from |O| up to the next multiple of 64.
struct RowQuantArgs {
  const uint16_t *X;
  int64_t M, K, ldx;
  const uint32_t *omask;
  const int32_t *wprefix;
  const int32_t *count;
  uint8_t *Xq;
  int64_t ldq;
  float *m;
  uint16_t *xo;
  int64_t ldo;
};

// Row quantization and the weight side of a large-M call in one launch
// (gather: the outlier product needs W_O^T).
template <class Codec>
hipError_t launch_layer_prep(const RowQuantArgs &r, const WeightSideArgs &w, bool gather,
                             hipStream_t stream);

struct GemmArgs {
  const int8_t *xq;      // [M x ldq] int8 (compacted rows when compaction is on)
  const int8_t *wq;      // [N x K] int8, caller's
  const int8_t *wqc;     // [N x ldq] int8 compacted copy (workspace)
  const float *m;        // [M]
  const float *s;        // [N]
  const uint16_t *xo;    // [M x ldo] fp16 gathered outlier columns
  const uint16_t *wot;   // [N x ldo] fp16 outlier rows of W, transposed
  const uint16_t *w;     // non-null when the outlier product runs (rows gathered in wot)
  const int32_t *count;  // [1]
  uint16_t *y;           // [M x ldy] fp16
  int32_t *cdbg;         // optional [M x N] int32
  int64_t M, N, K, ldq, ldo, ldw, ldy;
  EpilogueOpts ep;
  int fp8;               // xq and wq hold E4M3 codes instead of int8 ones
  int64_t ldc;           // row pitch of cdbg (0: N)
  // Split-K tiles (int8 only; null part: never split). Each part of a tile
  // stores its int32 sums in one slot of part and counts itself in sem[tile];
  // the last to arrive adds the other slots and runs the epilogue. sem must be
  // zero when the GEMM starts.
  int32_t *part;         // [tiles x ksplit slots of split_slot_bytes(bm) each]
  uint32_t *sem;         // [tiles] arrival counters
  int64_t part_bytes;    // bytes available at part
  int ksplit;            // set by the launcher on the split-K tiles
};

// Bytes of one part's int32 sums of a bm x 256 tile.
inline int64_t split_slot_bytes(int bm) { return (int64_t)bm * 256 * 4; }

// Split-K plan of the large-M GEMM: each of its `tiles` bm x 256 tiles cuts
// its k range into ksplit parts (ksplit = 1: whole tiles, no split).
struct GemmSplitPlan {
  int64_t tiles;
  int ksplit;
  int bm;
};
GemmSplitPlan gemm_split_plan(int64_t M, int64_t K, int64_t N);

// Caller-supplied events (may be null) that the GEMM kernel's own dispatch
// stamps when the kernel starts and when it ends.
struct GemmEvents {
  void *begin;
  void *end;
};

// Large-M tiled GEMM with the fused dequantize + outlier epilogue; picks the
// tile shapes (256x256, 256x128, or whole waves of 256x256 tiles and the
// remaining columns in 128x256 tiles, in one launch) from the problem size.
hipError_t launch_gemm(const GemmArgs &args, const GemmEvents &ev, hipStream_t stream);
hipError_t launch_gemm_wide(const GemmArgs &args, const GemmEvents &ev, hipStream_t stream);
hipError_t launch_gemm_narrow(const GemmArgs &args, const GemmEvents &ev, hipStream_t stream);
hipError_t launch_gemm_pair(const GemmArgs &a1, const GemmArgs &a2, const GemmEvents &ev,
                            hipStream_t stream);
hipError_t launch_gemm_split(const GemmArgs &a, int bm, const GemmEvents &ev, hipStream_t stream);

// Small-M (decode) path: a detection kernel and a split-K GEMM that quantizes
// its slice of X itself.
struct DecodeDetectArgs {
  const uint16_t *X;
  int M;
  int64_t K, ldx, kw;
  float threshold;
  uint32_t *omask;    // [kw] outlier bitmask
  float *pmax;        // [det_blocks x M] row absmax over each block's kept columns
  const float *xcmax; // optional [K]: column absmax of X supplied by the caller
  float *ycmax;       // optional [N], zeroed here for the epilogue's maxima
  int64_t N;
};

struct DecodeGemmArgs {
  const uint16_t *X;
  const int8_t *wq;
  const float *s;
  const uint32_t *omask;
  const float *pmax;
  const uint16_t *w;
  int32_t *part;      // [kb x M x N] int32 partial sums
  float *m;           // [M] row absmax
  int32_t *count_out; // optional [1] outlier count
  uint16_t *y;
  int32_t *cdbg;
  int64_t M, N, K, kw, kc, ldx, ldw, ldy;
  int det_blocks;
  int kb;             // K splits (partial sums per output)
  EpilogueOpts ep;
  int fp8;            // E4M3 codes of X and Wq (fp32 partial sums) instead of int8
};

struct DecodePlan {
  int tiles;       // 64-column tiles
  int kb;          // K splits
  int det_blocks;  // detection blocks (256 columns each)
  int64_t kc;      // k bytes per split (multiple of 64)
};
DecodePlan decode_plan(int64_t M, int64_t K, int64_t N);
// Whether a layer call of this shape takes the small-M kernels (M <= 64
// always; up to kDecodeMaxM = 256 rows when their plan streams every K range
// in one pass).
bool use_decode_path(int64_t M, int64_t K, int64_t N);

hipError_t launch_decode(const DecodeDetectArgs &det, const DecodeGemmArgs &gemm,
                         const DecodePlan &plan, const GemmEvents &ev, hipStream_t stream);

// Single-kernel small-M path (no workspace): for the shapes fused_decode_fits
// accepts, one kernel detects, quantizes, multiplies and writes Y.
struct FusedArgs {
  const uint16_t *X;
  const int8_t *wq;
  const float *s;
  const uint16_t *w;   // null only when no column can be an outlier
  uint16_t *y;
  int32_t *cdbg;       // optional [M x N] int32
  int32_t *count_out;  // optional [1]
  int64_t ldx, ldw, ldy;
  int M, K, N;
  int tiles;           // 16-column output tiles
  uint32_t tcut;       // smallest fp16 magnitude pattern whose value reaches the threshold
  float threshold;
  const float *xcmax;  // optional [K]: column absmax of X supplied by the caller
  EpilogueOpts ep;
};
bool fused_decode_fits(int64_t M, int64_t K, int64_t ldx);
hipError_t launch_decode_fused(const FusedArgs &a, const GemmEvents &ev, hipStream_t stream);

// The per-tensor int8 layer (one absmax for all of X, one for all of W).
// scratch holds N floats.
hipError_t launch_quantize_tensorwise(const uint16_t *W, int64_t K, int64_t N, int64_t ldw,
                                      int8_t *Wq, float *w_absmax, float *scratch,
                                      hipStream_t stream);

constexpr int kTensorAbsBlocks = 512;  // blocks of the partial max|X| pass

struct TensorwiseLayout {
  float *partial;  // [kTensorAbsBlocks]
  float *m;        // [M], every entry max|X|
  float *s;        // [N], every entry max|W|
  int32_t *count;  // [1], zero: no outlier product
  int8_t *xq;      // [M x ldq], zero past column K
  int64_t ldq;
};
hipError_t launch_linear_tensorwise(const uint16_t *X, int64_t M, int64_t K, int64_t ldx,
                                    const int8_t *Wq, const float *w_absmax, int64_t N,
                                    uint16_t *Y, int64_t ldy, const uint16_t *bias,
                                    float *x_absmax, int32_t *cdbg, const TensorwiseLayout &L,
                                    const GemmEvents &ev, hipStream_t stream);

}  // namespace llmint8
