// C ABI of the LLM.int8() linear layer: argument checks, workspace layout and
// the launch sequence. Every check runs before the first HIP call, so a
// rejected call enqueues nothing.
#include <cmath>
#include <cstdint>
#include <mutex>

#include "internal.hpp"
#include "llmint8.h"

#define LLMINT8_EXPORT extern "C" __attribute__((visibility("default")))

using namespace llmint8;

namespace {

constexpr int64_t kMaxDim = (int64_t)1 << 31;
constexpr int64_t kMaxTileLd = (int64_t)1 << 21;  // 256 rows x 4 bytes x 2^21 = 2^31

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
size_t up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Row pitches of the padded int8 (bytes) and fp16 outlier (elements) copies of X.
int64_t pitch_q(int64_t K) { return (K + 127) / 128 * 128; }
int64_t pitch_o(int64_t K) { return (K + 63) / 64 * 64; }

// Offsets (bytes) of the regions a call carves out of its workspace.
struct Layout {
  size_t pmask, omask, wprefix, idx, count, xq, m, xo, wqc, wot, part, sem, kpart, kpart_bytes,
      total;
};

// Small-M layer calls: preparation outputs, split-K partial sums, counters.
Layout make_decode_layout(int64_t M, int64_t K, int64_t N) {
  const DecodePlan p = decode_plan(M, K, N);
  Layout L{};
  size_t o = 0;
  L.omask = o;
  o += up((size_t)((K + 31) / 32) * 4);
  L.pmask = o;  // partial row maxima [det_blocks x M] fp32
  o += up((size_t)p.det_blocks * (size_t)M * 4);
  L.m = o;
  o += up((size_t)M * 4);
  L.part = o;
  o += up((size_t)p.kb * (size_t)M * (size_t)N * 4);
  L.total = o;
  return L;
}

// split: room for the large-M GEMM's split-K tiles (int8 layer calls that may
// allocate; the FP8 layer and the allocation-free call run without them).
Layout make_layout(int64_t M, int64_t K, int64_t N, bool layer, bool any_m_prefill = false,
                   bool split = false) {
  if (layer && !any_m_prefill && use_decode_path(M, K, N)) return make_decode_layout(M, K, N);
  const DetectPlan p = detect_plan(M, K);
  Layout L{};
  size_t o = 0;
  L.pmask = o;
  o += up((size_t)p.row_chunks * (size_t)p.kw * 4);
  L.omask = o;
  o += up((size_t)p.kw * 4);
  L.wprefix = o;
  o += up((size_t)p.kw * 4);
  if (layer) {
    L.idx = o;
    o += up((size_t)K * 4);
    L.count = o;
    o += up(64);
    const size_t ldq = (size_t)pitch_q(K), ldo = (size_t)pitch_o(K);
    L.xq = o;
    o += up((size_t)M * ldq);
    L.m = o;
    o += up((size_t)M * 4);
    L.xo = o;
    o += up((size_t)M * ldo * 2);
    L.wqc = o;
    o += up((size_t)N * ldq);
    L.wot = o;
    o += up((size_t)N * ldo * 2);
    const GemmSplitPlan sp = split ? gemm_split_plan(M, K, N) : GemmSplitPlan{0, 1, 256};
    if (sp.ksplit > 1) {
      L.sem = o;
      o += up((size_t)sp.tiles * 4);
      L.kpart = o;
      L.kpart_bytes = (size_t)sp.tiles * (size_t)sp.ksplit * (size_t)split_slot_bytes(sp.bm);
      o += up(L.kpart_bytes);
    }
  }
  L.total = o;
  return L;
}

// Shape rules shared by the calls that read an fp16 [rows x cols] matrix.
int check_matrix(const void *p, int64_t rows, int64_t cols, int64_t ld) {
  if (!p || rows <= 0 || cols <= 0 || ld < cols) return LLMINT8_ERR_INVALID_ARG;
  if (rows >= kMaxDim || cols >= kMaxDim || ld >= kMaxDim) return LLMINT8_ERR_INVALID_ARG;
  if (!aligned16(p) || ld % 8 != 0) return LLMINT8_ERR_UNSUPPORTED;
  return LLMINT8_OK;
}

int check_k(int64_t K) {
  if (K > LLMINT8_MAX_K) return LLMINT8_ERR_OVERFLOW;
  if (K % 16 != 0) return LLMINT8_ERR_UNSUPPORTED;
  return LLMINT8_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? LLMINT8_OK : LLMINT8_ERR_HIP; }

// Value of a non-negative binary16 pattern (0 .. 0x7c00 = +inf), exactly.
float half_value(uint32_t p) {
  if (p >= 0x7c00u) return INFINITY;
  if (p < 0x400u) return std::ldexp((float)p, -24);
  return std::ldexp((float)(1024u + (p & 0x3ffu)), (int)(p >> 10) - 25);
}

// Smallest binary16 magnitude pattern whose value is >= threshold, so that for
// every fp16 x, |x| >= threshold exactly when (bits(x) & 0x7fff) >= the result
// (non-negative fp16 values are ordered like their patterns).
uint32_t fp16_threshold_bits(float threshold) {
  if (!(threshold > 0.f)) return 0u;
  uint32_t lo = 0u, hi = 0x7c00u;  // half_value(hi) >= threshold always holds
  while (lo < hi) {
    const uint32_t mid = (lo + hi) / 2;
    if (half_value(mid) >= threshold)
      hi = mid;
    else
      lo = mid + 1;
  }
  return lo;
}

// The large-M layer sequence: detection, row quantization with the outlier
// gather, K-compaction when it pays, the W_O^T gather and the GEMM with the
// fused epilogue. fp8 selects E4M3 codes for Xq and Wq.
hipError_t prefill_layer(const uint16_t *X, int64_t M, int64_t K, int64_t ldx, const int8_t *Wq,
                         const float *col_absmax, const uint16_t *Wf, int64_t ldw, int64_t N,
                         float threshold, uint16_t *Y, int64_t ldy, int32_t *outlier_count_out,
                         int32_t *C_debug, uint8_t *ws, const Layout &L,
                         const llmint8_linear_opts &o, const GemmEvents &ev,
                         const EpilogueOpts &ep, bool fp8, hipStream_t s) {
  const DetectPlan plan = detect_plan(M, K);
  uint32_t *omask = (uint32_t *)(ws + L.omask);
  int32_t *wprefix = (int32_t *)(ws + L.wprefix);
  int32_t *idx = (int32_t *)(ws + L.idx);
  int32_t *count = (int32_t *)(ws + L.count);
  int8_t *xq = (int8_t *)(ws + L.xq);
  float *m = (float *)(ws + L.m);
  uint16_t *xo = (uint16_t *)(ws + L.xo);
  int8_t *wqc = (int8_t *)(ws + L.wqc);
  const bool int8w = ep.int8w != 0;

  // split-K tiles only on int8 calls whose layout has room for them
  const bool split = L.kpart_bytes > 0 && !fp8;
  uint32_t *sem = split ? (uint32_t *)(ws + L.sem) : nullptr;
  int32_t *kpart = split ? (int32_t *)(ws + L.kpart) : nullptr;
  const GemmSplitPlan sp = split ? gemm_split_plan(M, K, N) : GemmSplitPlan{0, 1, 256};
  DetectOut d{o.x_col_absmax, threshold, o.y_col_absmax, N, (uint32_t *)(ws + L.pmask), omask,
              wprefix, idx, count, outlier_count_out, sem, sp.tiles};
  const int64_t ldq = pitch_q(K), ldo = pitch_o(K);
  uint16_t *wot = (uint16_t *)(ws + L.wot);
  hipError_t e = launch_detect(X, M, K, ldx, threshold, plan, d, s);
  if (e == hipSuccess) {
    const RowQuantArgs r{X, M, K, ldx, omask, wprefix, count, (uint8_t *)xq, ldq, m, xo, ldo};
    const WeightSideArgs w{Wf, ldw, Wq, M, K, N, idx, count, wot, ldo, omask, wprefix, wqc, ldq, 0};
    e = fp8 ? launch_layer_prep<CodecE4M3>(r, w, Wf || int8w, s)
            : launch_layer_prep<CodecI8>(r, w, Wf || int8w, s);
  }
  if (e == hipSuccess) {
    // the GEMM's outlier product runs when it has weight rows (gathered above)
    const uint16_t *wo_src = (Wf || int8w) ? wot : nullptr;
    GemmArgs g{xq, Wq, wqc, m, col_absmax, xo, wot, wo_src ? (const uint16_t *)wot : nullptr,
               count, Y, C_debug, M, N, K, ldq, ldo, ldw, ldy, ep, fp8 ? 1 : 0, 0,
               kpart, sem, split ? (int64_t)L.kpart_bytes : 0, 1};
    e = launch_gemm(g, ev, s);
  }
  return e;
}

}  // namespace

LLMINT8_EXPORT const char *llmint8_status_string(int status) {
  switch (status) {
    case LLMINT8_OK: return "LLMINT8_OK";
    case LLMINT8_ERR_INVALID_ARG: return "LLMINT8_ERR_INVALID_ARG: null pointer, bad size or NaN threshold";
    case LLMINT8_ERR_UNSUPPORTED: return "LLMINT8_ERR_UNSUPPORTED: alignment or multiple-of rule broken";
    case LLMINT8_ERR_OVERFLOW: return "LLMINT8_ERR_OVERFLOW: K too large for int32 accumulation";
    case LLMINT8_ERR_WORKSPACE: return "LLMINT8_ERR_WORKSPACE: workspace missing or too small";
    case LLMINT8_ERR_HIP: return "LLMINT8_ERR_HIP: HIP launch or runtime error";
    default: return "LLMINT8: unknown status";
  }
}

LLMINT8_EXPORT int llmint8_quantize_colwise(const uint16_t *W, int64_t K, int64_t N, int64_t ldw,
                                            int8_t *Wq, float *col_absmax, void *stream) {
  int st = check_matrix(W, K, N, ldw);
  if (st) return st;
  if (!Wq || !col_absmax) return LLMINT8_ERR_INVALID_ARG;
  if ((st = check_k(K))) return st;
  if (N % 8 != 0 || !aligned16(Wq) || !aligned16(col_absmax)) return LLMINT8_ERR_UNSUPPORTED;
  return hip_status(
      launch_colwise<CodecI8>(W, K, N, ldw, (uint8_t *)Wq, col_absmax, (hipStream_t)stream));
}

LLMINT8_EXPORT size_t llmint8_find_outliers_workspace_size(int64_t M, int64_t K) {
  if (M <= 0 || K <= 0 || M >= kMaxDim || K > LLMINT8_MAX_K) return 0;
  return make_layout(M, K, 0, false).total;
}

LLMINT8_EXPORT int llmint8_find_outliers(const uint16_t *X, int64_t M, int64_t K, int64_t ldx,
                                         float threshold, int32_t *idx, int32_t *count,
                                         void *workspace, size_t workspace_bytes, void *stream) {
  int st = check_matrix(X, M, K, ldx);
  if (st) return st;
  if (!idx || !count || std::isnan(threshold)) return LLMINT8_ERR_INVALID_ARG;
  if ((st = check_k(K))) return st;
  if (!aligned16(idx) || !aligned16(count)) return LLMINT8_ERR_UNSUPPORTED;
  const Layout L = make_layout(M, K, 0, false);
  if (!workspace || workspace_bytes < L.total) return LLMINT8_ERR_WORKSPACE;
  if (!aligned16(workspace)) return LLMINT8_ERR_UNSUPPORTED;
  uint8_t *ws = (uint8_t *)workspace;
  DetectOut d{nullptr, threshold, nullptr, 0, (uint32_t *)(ws + L.pmask),
              (uint32_t *)(ws + L.omask), (int32_t *)(ws + L.wprefix), idx, count, nullptr};
  return hip_status(launch_detect(X, M, K, ldx, threshold, detect_plan(M, K), d,
                                  (hipStream_t)stream));
}

LLMINT8_EXPORT int llmint8_quantize_rowwise(const uint16_t *X, int64_t M, int64_t K, int64_t ldx,
                                            const int32_t *idx, const int32_t *count, int8_t *Xq,
                                            float *row_absmax, void *stream) {
  int st = check_matrix(X, M, K, ldx);
  if (st) return st;
  if (!Xq || !row_absmax || (!idx) != (!count)) return LLMINT8_ERR_INVALID_ARG;
  if ((st = check_k(K))) return st;
  if (!aligned16(Xq) || !aligned16(row_absmax)) return LLMINT8_ERR_UNSUPPORTED;
  if (idx && (!aligned16(idx) || !aligned16(count))) return LLMINT8_ERR_UNSUPPORTED;
  return hip_status(
      launch_rowquant_idx<CodecI8>(X, M, K, ldx, idx, count, (uint8_t *)Xq, row_absmax,
                                   (hipStream_t)stream));
}

LLMINT8_EXPORT size_t llmint8_workspace_size(int64_t M, int64_t K, int64_t N) {
  if (M <= 0 || K <= 0 || N <= 0 || M >= kMaxDim || N >= kMaxDim || K > LLMINT8_MAX_K) return 0;
  return make_layout(M, K, N, true, false, true).total;
}

namespace {

// Every check of llmint8_linear_ex except the workspace one; makes no HIP call.
int check_linear(const uint16_t *X, int64_t M, int64_t K, int64_t ldx, const int8_t *Wq,
                 const float *col_absmax, const uint16_t *W, int64_t ldw, int64_t N,
                 float threshold, uint16_t *Y, int64_t ldy, int32_t *outlier_count_out,
                 int32_t *C_debug, const llmint8_linear_opts &o) {
  if (o.outlier_weights != LLMINT8_OUTLIER_W_FP16 && o.outlier_weights != LLMINT8_OUTLIER_W_INT8)
    return LLMINT8_ERR_INVALID_ARG;
  const bool int8w = o.outlier_weights == LLMINT8_OUTLIER_W_INT8;
  if ((o.bias && !aligned16(o.bias)) || (o.y_col_absmax && !aligned16(o.y_col_absmax)) ||
      (o.x_col_absmax && !aligned16(o.x_col_absmax)))
    return LLMINT8_ERR_UNSUPPORTED;
  int st = check_matrix(X, M, K, ldx);
  if (st) return st;
  if ((st = check_matrix(Y, M, N, ldy))) return st;
  if (!Wq || !col_absmax || std::isnan(threshold)) return LLMINT8_ERR_INVALID_ARG;
  if (!W && !int8w && !(std::isinf(threshold) && threshold > 0)) return LLMINT8_ERR_INVALID_ARG;
  if (W && (st = check_matrix(W, K, N, ldw))) return st;
  if ((st = check_k(K))) return st;
  if (N % 8 != 0 || !aligned16(Wq) || !aligned16(col_absmax)) return LLMINT8_ERR_UNSUPPORTED;
  if ((outlier_count_out && !aligned16(outlier_count_out)) || (C_debug && !aligned16(C_debug)))
    return LLMINT8_ERR_UNSUPPORTED;
  // the GEMM addresses a 256-row output tile with 32-bit byte offsets
  if (ldy >= kMaxTileLd || N >= kMaxTileLd) return LLMINT8_ERR_UNSUPPORTED;
  return LLMINT8_OK;
}

// The layer after check_linear: the workspace check, then the launches.
int run_linear(const uint16_t *X, int64_t M, int64_t K, int64_t ldx, const int8_t *Wq,
               const float *col_absmax, const uint16_t *W, int64_t ldw, int64_t N,
               float threshold, uint16_t *Y, int64_t ldy, int32_t *outlier_count_out,
               int32_t *C_debug, void *workspace, size_t workspace_bytes, hipStream_t s,
               const llmint8_linear_opts &o, bool split) {
  const Layout L = make_layout(M, K, N, true, false, split);
  if (!workspace || workspace_bytes < L.total) return LLMINT8_ERR_WORKSPACE;
  if (!aligned16(workspace)) return LLMINT8_ERR_UNSUPPORTED;

  const bool int8w = o.outlier_weights == LLMINT8_OUTLIER_W_INT8;
  uint8_t *ws = (uint8_t *)workspace;
  const GemmEvents ev{o.gemm_begin_event, o.gemm_end_event};
  // with int8 outlier weights the fp16 weight is not read at all
  const uint16_t *Wf = int8w ? nullptr : W;
  const EpilogueOpts ep{int8w ? 1 : 0, o.bias, o.y_col_absmax};

  if (fused_decode_fits(M, K, ldx)) {
    const FusedArgs f{X, Wq, col_absmax, Wf, Y, C_debug, outlier_count_out, ldx, ldw, ldy,
                      (int)M, (int)K, (int)N, (int)((N + 15) / 16), fp16_threshold_bits(threshold),
                      threshold, o.x_col_absmax, ep};
    return hip_status(launch_decode_fused(f, ev, s));
  }
  if (use_decode_path(M, K, N)) {
    const DecodePlan dp = decode_plan(M, K, N);
    const int64_t kw = (K + 31) / 32;
    uint32_t *omask = (uint32_t *)(ws + L.omask);
    float *pmax = (float *)(ws + L.pmask);
    DecodeDetectArgs det{X, (int)M, K, ldx, kw, threshold, omask, pmax, o.x_col_absmax,
                         o.y_col_absmax, N};
    DecodeGemmArgs g{X, Wq, col_absmax, omask, pmax, Wf, (int32_t *)(ws + L.part),
                     (float *)(ws + L.m), outlier_count_out, Y, C_debug,
                     M, N, K, kw, dp.kc, ldx, ldw, ldy, dp.det_blocks, dp.kb, ep};
    return hip_status(launch_decode(det, g, dp, ev, s));
  }

  return hip_status(prefill_layer(X, M, K, ldx, Wq, col_absmax, Wf, ldw, N, threshold, Y, ldy,
                                  outlier_count_out, C_debug, ws, L, o, ev, ep, false, s));
}

// Scratch of llmint8_linear_noalloc: one copy per GPU the library runs on,
// held until the process ends. Host code never uses the array's name as an
// address (on the host it is only a handle); it uses the device address that
// hipGetSymbolAddress returns for the current device, kept per device.
constexpr size_t kScratchBytes = LLMINT8_NOALLOC_SCRATCH_BYTES;
__device__ __attribute__((aligned(256))) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void *scratch_ptr[kMaxDevices];

// Device address of this GPU's scratch, looked up once per device with that
// device current.
int scratch_of(hipStream_t s, void **out) {
  int dev = 0;
  hipError_t e = s ? hipStreamGetDevice(s, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) return LLMINT8_ERR_HIP;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    int cur = 0;
    if (hipGetDevice(&cur) != hipSuccess) return LLMINT8_ERR_HIP;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return LLMINT8_ERR_HIP;
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev && hipSetDevice(cur) != hipSuccess) return LLMINT8_ERR_HIP;
    if (e != hipSuccess || !p) return LLMINT8_ERR_HIP;
    scratch_ptr[dev] = p;
  }
  *out = scratch_ptr[dev];
  return LLMINT8_OK;
}

}  // namespace

LLMINT8_EXPORT int llmint8_linear_ex(const uint16_t *X, int64_t M, int64_t K, int64_t ldx,
                                     const int8_t *Wq, const float *col_absmax, const uint16_t *W,
                                     int64_t ldw, int64_t N, float threshold, uint16_t *Y,
                                     int64_t ldy, int32_t *outlier_count_out, int32_t *C_debug,
                                     void *workspace, size_t workspace_bytes, void *stream,
                                     const llmint8_linear_opts *opts) {
  if (opts && opts->struct_size != sizeof(llmint8_linear_opts)) return LLMINT8_ERR_INVALID_ARG;
  const llmint8_linear_opts o = opts ? *opts : llmint8_linear_opts{};
  const int st = check_linear(X, M, K, ldx, Wq, col_absmax, W, ldw, N, threshold, Y, ldy,
                              outlier_count_out, C_debug, o);
  if (st) return st;
  return run_linear(X, M, K, ldx, Wq, col_absmax, W, ldw, N, threshold, Y, ldy,
                    outlier_count_out, C_debug, workspace, workspace_bytes, (hipStream_t)stream,
                    o, true);
}

LLMINT8_EXPORT int llmint8_linear_noalloc(const uint16_t *X, int64_t M, int64_t K, int64_t ldx,
                                          const int8_t *Wq, const float *col_absmax,
                                          const uint16_t *W, int64_t ldw, int64_t N,
                                          float threshold, uint16_t *Y, int64_t ldy,
                                          int32_t *outlier_count_out, int32_t *C_debug,
                                          void *stream) {
  const llmint8_linear_opts o{};
  int st = check_linear(X, M, K, ldx, Wq, col_absmax, W, ldw, N, threshold, Y, ldy,
                        outlier_count_out, C_debug, o);
  if (st) return st;
  if (make_layout(M, K, N, true).total > kScratchBytes) return LLMINT8_ERR_WORKSPACE;
  void *ws = nullptr;
  if ((st = scratch_of((hipStream_t)stream, &ws))) return st;
  return run_linear(X, M, K, ldx, Wq, col_absmax, W, ldw, N, threshold, Y, ldy,
                    outlier_count_out, C_debug, ws, kScratchBytes, (hipStream_t)stream, o,
                    false);
}

LLMINT8_EXPORT size_t llmint8_quantize_tensorwise_workspace_size(int64_t K, int64_t N) {
  if (K <= 0 || N <= 0 || N >= kMaxDim || K > LLMINT8_MAX_K) return 0;
  return up((size_t)N * 4);
}

LLMINT8_EXPORT int llmint8_quantize_tensorwise(const uint16_t *W, int64_t K, int64_t N,
                                               int64_t ldw, int8_t *Wq, float *w_absmax,
                                               void *workspace, size_t workspace_bytes,
                                               void *stream) {
  int st = check_matrix(W, K, N, ldw);
  if (st) return st;
  if (!Wq || !w_absmax) return LLMINT8_ERR_INVALID_ARG;
  if ((st = check_k(K))) return st;
  if (N % 8 != 0 || !aligned16(Wq) || !aligned16(w_absmax)) return LLMINT8_ERR_UNSUPPORTED;
  if (!workspace || workspace_bytes < up((size_t)N * 4)) return LLMINT8_ERR_WORKSPACE;
  if (!aligned16(workspace)) return LLMINT8_ERR_UNSUPPORTED;
  return hip_status(launch_quantize_tensorwise(W, K, N, ldw, Wq, w_absmax, (float *)workspace,
                                               (hipStream_t)stream));
}

namespace {

// Workspace of llmint8_linear_tensorwise: partial maxima, broadcast scales,
// a zero outlier count, the padded int8 copy of X.
struct TensorwiseOffsets {
  size_t partial, m, s, count, xq, total;
};

TensorwiseOffsets tensorwise_offsets(int64_t M, int64_t K, int64_t N) {
  TensorwiseOffsets L{};
  size_t o = 0;
  L.partial = o;
  o += up((size_t)kTensorAbsBlocks * 4);
  L.m = o;
  o += up((size_t)M * 4);
  L.s = o;
  o += up((size_t)N * 4);
  L.count = o;
  o += up(64);
  L.xq = o;
  o += up((size_t)M * (size_t)pitch_q(K));
  L.total = o;
  return L;
}

}  // namespace

LLMINT8_EXPORT size_t llmint8_linear_tensorwise_workspace_size(int64_t M, int64_t K, int64_t N) {
  if (M <= 0 || K <= 0 || N <= 0 || M >= kMaxDim || N >= kMaxDim || K > LLMINT8_MAX_K) return 0;
  return tensorwise_offsets(M, K, N).total;
}

LLMINT8_EXPORT int llmint8_linear_tensorwise(const uint16_t *X, int64_t M, int64_t K,
                                             int64_t ldx, const int8_t *Wq,
                                             const float *w_absmax, int64_t N,
                                             const uint16_t *bias, uint16_t *Y, int64_t ldy,
                                             float *x_absmax, int32_t *C_debug, void *workspace,
                                             size_t workspace_bytes, void *stream) {
  int st = check_matrix(X, M, K, ldx);
  if (st) return st;
  if ((st = check_matrix(Y, M, N, ldy))) return st;
  if (!Wq || !w_absmax) return LLMINT8_ERR_INVALID_ARG;
  if ((st = check_k(K))) return st;
  if (N % 8 != 0 || !aligned16(Wq) || !aligned16(w_absmax)) return LLMINT8_ERR_UNSUPPORTED;
  if ((bias && !aligned16(bias)) || (x_absmax && !aligned16(x_absmax)) ||
      (C_debug && !aligned16(C_debug)))
    return LLMINT8_ERR_UNSUPPORTED;
  if (ldy >= kMaxTileLd || N >= kMaxTileLd) return LLMINT8_ERR_UNSUPPORTED;
  const TensorwiseOffsets o = tensorwise_offsets(M, K, N);
  if (!workspace || workspace_bytes < o.total) return LLMINT8_ERR_WORKSPACE;
  if (!aligned16(workspace)) return LLMINT8_ERR_UNSUPPORTED;
  uint8_t *ws = (uint8_t *)workspace;
  const TensorwiseLayout L{(float *)(ws + o.partial), (float *)(ws + o.m), (float *)(ws + o.s),
                           (int32_t *)(ws + o.count), (int8_t *)(ws + o.xq), pitch_q(K)};
  return hip_status(launch_linear_tensorwise(X, M, K, ldx, Wq, w_absmax, N, Y, ldy, bias,
                                             x_absmax, C_debug, L, GemmEvents{nullptr, nullptr},
                                             (hipStream_t)stream));
}

LLMINT8_EXPORT int llmint8_linear(const uint16_t *X, int64_t M, int64_t K, int64_t ldx,
                                  const int8_t *Wq, const float *col_absmax, const uint16_t *W,
                                  int64_t ldw, int64_t N, float threshold, uint16_t *Y,
                                  int64_t ldy, int32_t *outlier_count_out, int32_t *C_debug,
                                  void *workspace, size_t workspace_bytes, void *stream) {
  return llmint8_linear_ex(X, M, K, ldx, Wq, col_absmax, W, ldw, N, threshold, Y, ldy,
                           outlier_count_out, C_debug, workspace, workspace_bytes, stream, nullptr);
}

// ---- FP8 (E4M3) variant --------------------------------------------------------------

LLMINT8_EXPORT int llmint8_quantize_colwise_fp8(const uint16_t *W, int64_t K, int64_t N,
                                                int64_t ldw, uint8_t *Wq8, float *col_absmax,
                                                void *stream) {
  int st = check_matrix(W, K, N, ldw);
  if (st) return st;
  if (!Wq8 || !col_absmax) return LLMINT8_ERR_INVALID_ARG;
  if ((st = check_k(K))) return st;
  if (N % 8 != 0 || !aligned16(Wq8) || !aligned16(col_absmax)) return LLMINT8_ERR_UNSUPPORTED;
  return hip_status(launch_colwise<CodecE4M3>(W, K, N, ldw, Wq8, col_absmax, (hipStream_t)stream));
}

LLMINT8_EXPORT int llmint8_quantize_rowwise_fp8(const uint16_t *X, int64_t M, int64_t K,
                                                int64_t ldx, const int32_t *idx,
                                                const int32_t *count, uint8_t *Xq8,
                                                float *row_absmax, void *stream) {
  int st = check_matrix(X, M, K, ldx);
  if (st) return st;
  if (!Xq8 || !row_absmax || (!idx) != (!count)) return LLMINT8_ERR_INVALID_ARG;
  if ((st = check_k(K))) return st;
  if (!aligned16(Xq8) || !aligned16(row_absmax)) return LLMINT8_ERR_UNSUPPORTED;
  if (idx && (!aligned16(idx) || !aligned16(count))) return LLMINT8_ERR_UNSUPPORTED;
  return hip_status(launch_rowquant_idx<CodecE4M3>(X, M, K, ldx, idx, count, Xq8, row_absmax,
                                                   (hipStream_t)stream));
}

LLMINT8_EXPORT size_t llmint8_linear_fp8_workspace_size(int64_t M, int64_t K, int64_t N) {
  if (M <= 0 || K <= 0 || N <= 0 || M >= kMaxDim || N >= kMaxDim || K > LLMINT8_MAX_K) return 0;
  return make_layout(M, K, N, true).total;
}

LLMINT8_EXPORT int llmint8_linear_fp8(const uint16_t *X, int64_t M, int64_t K, int64_t ldx,
                                      const uint8_t *Wq8, const float *col_absmax,
                                      const uint16_t *W, int64_t ldw, int64_t N, float threshold,
                                      uint16_t *Y, int64_t ldy, int32_t *outlier_count_out,
                                      float *C_debug, void *workspace, size_t workspace_bytes,
                                      void *stream, const llmint8_linear_opts *opts) {
  if (opts && opts->struct_size != sizeof(llmint8_linear_opts)) return LLMINT8_ERR_INVALID_ARG;
  const llmint8_linear_opts o = opts ? *opts : llmint8_linear_opts{};
  if (o.outlier_weights != LLMINT8_OUTLIER_W_FP16) return LLMINT8_ERR_INVALID_ARG;
  if ((o.bias && !aligned16(o.bias)) || (o.y_col_absmax && !aligned16(o.y_col_absmax)) ||
      (o.x_col_absmax && !aligned16(o.x_col_absmax)))
    return LLMINT8_ERR_UNSUPPORTED;
  int st = check_matrix(X, M, K, ldx);
  if (st) return st;
  if ((st = check_matrix(Y, M, N, ldy))) return st;
  if (!Wq8 || !col_absmax || std::isnan(threshold)) return LLMINT8_ERR_INVALID_ARG;
  if (!W && !(std::isinf(threshold) && threshold > 0)) return LLMINT8_ERR_INVALID_ARG;
  if (W && (st = check_matrix(W, K, N, ldw))) return st;
  if ((st = check_k(K))) return st;
  if (N % 8 != 0 || !aligned16(Wq8) || !aligned16(col_absmax)) return LLMINT8_ERR_UNSUPPORTED;
  if ((outlier_count_out && !aligned16(outlier_count_out)) || (C_debug && !aligned16(C_debug)))
    return LLMINT8_ERR_UNSUPPORTED;
  if (ldy >= kMaxTileLd || N >= kMaxTileLd) return LLMINT8_ERR_UNSUPPORTED;
  const Layout L = make_layout(M, K, N, true);
  if (!workspace || workspace_bytes < L.total) return LLMINT8_ERR_WORKSPACE;
  if (!aligned16(workspace)) return LLMINT8_ERR_UNSUPPORTED;
  const GemmEvents ev{o.gemm_begin_event, o.gemm_end_event};
  const EpilogueOpts ep{0, o.bias, o.y_col_absmax};
  hipStream_t s = (hipStream_t)stream;
  uint8_t *ws = (uint8_t *)workspace;
  if (use_decode_path(M, K, N)) {
    const DecodePlan dp = decode_plan(M, K, N);
    const int64_t kw = (K + 31) / 32;
    uint32_t *omask = (uint32_t *)(ws + L.omask);
    float *pmax = (float *)(ws + L.pmask);
    DecodeDetectArgs det{X, (int)M, K, ldx, kw, threshold, omask, pmax, o.x_col_absmax,
                         o.y_col_absmax, N};
    DecodeGemmArgs g{X, (const int8_t *)Wq8, col_absmax, omask, pmax, W, (int32_t *)(ws + L.part),
                     (float *)(ws + L.m), outlier_count_out, Y, (int32_t *)C_debug,
                     M, N, K, kw, dp.kc, ldx, ldw, ldy, dp.det_blocks, dp.kb, ep, 1};
    return hip_status(launch_decode(det, g, dp, ev, s));
  }
  return hip_status(prefill_layer(X, M, K, ldx, (const int8_t *)Wq8, col_absmax, W, ldw, N,
                                  threshold, Y, ldy, outlier_count_out, (int32_t *)C_debug,
                                  ws, L, o, ev, ep, true, s));
}
