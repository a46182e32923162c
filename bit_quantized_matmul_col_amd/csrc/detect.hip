// Outlier-column detection for gfx950.
//
// A column k of X [M x K] is an outlier when some row has |X[i, k]| >= threshold
// ("8-bit quantization of giant language models: LLM.int8()" walkthrough,
// sections 2.3 and 4.2). HBM-bound: X is read once, 2MK bytes.
//
// Pass 1 (k_detect_partial): a block owns 512 columns (64 lanes x one 16-byte
// chunk of 8 fp16) of one row chunk; its 8 waves stride over the chunk's rows,
// so every wave load is a fully coalesced 1 KB row segment. The running column
// maxima are compared with the threshold once at the end (max >= t is the same
// test as "some entry >= t") and stored as 16 mask words per row chunk.
// Pass 2 (k_detect_finish): one block ORs the row-chunk masks into LDS (all
// partial-mask loads in flight at once), scans the per-word popcounts and writes
// the ascending outlier list, the per-word prefix and the count. When
// the caller supplies the column absmax of X, pass 1 is skipped and pass 2
// compares it with the threshold instead.
#include "internal.hpp"

namespace llmint8 {

namespace {

constexpr int kTileCols = 512;
constexpr int kMaxRowChunks = 64;
constexpr int kRowPhases = 8;  // waves per detection block, each on every 8th row

__global__ __launch_bounds__(64 * kRowPhases) void k_detect_partial(
    const uint16_t *__restrict__ X, int64_t M, int64_t K, int64_t ldx, float threshold,
    int rows_per_chunk, int64_t kw, uint32_t *__restrict__ pmask) {
  const int t = threadIdx.x;
  const int c = t & 63;   // 16-byte chunk within the tile
  const int rp = t >> 6;  // row phase 0 .. kRowPhases - 1
  const int64_t col = (int64_t)blockIdx.x * kTileCols + (int64_t)c * 8;
  const int64_t r0 = (int64_t)blockIdx.y * rows_per_chunk;
  const int64_t r1 = (r0 + rows_per_chunk < M) ? r0 + rows_per_chunk : M;
  constexpr int P = kRowPhases;

  float mx[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (col < K) {
    const uint16_t *p = X + col;
    int64_t r = r0 + rp;
    for (; r + 3 * P < r1; r += 4 * P) {
      u32x4 v0 = *(const u32x4 *)(p + r * ldx);
      u32x4 v1 = *(const u32x4 *)(p + (r + P) * ldx);
      u32x4 v2 = *(const u32x4 *)(p + (r + 2 * P) * ldx);
      u32x4 v3 = *(const u32x4 *)(p + (r + 3 * P) * ldx);
      absmax8(v0, mx);
      absmax8(v1, mx);
      absmax8(v2, mx);
      absmax8(v3, mx);
    }
    for (; r < r1; r += P) absmax8(*(const u32x4 *)(p + r * ldx), mx);
  }
  unsigned bits = 0;
  if (col < K && rp < r1 - r0) {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (mx[e] >= threshold) bits |= 1u << e;
  }
  __shared__ uint8_t sb[P][64];
  sb[rp][c] = (uint8_t)bits;
  __syncthreads();
  if (t < kTileCols / 32) {
    uint32_t word = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int ch = 4 * t + j;
      uint32_t b = 0;
#pragma unroll
      for (int q = 0; q < P; ++q) b |= sb[q][ch];
      word |= b << (8 * j);
    }
    const int64_t w = (int64_t)blockIdx.x * (kTileCols / 32) + t;
    if (w < kw) pmask[(int64_t)blockIdx.y * kw + w] = word;
  }
}

template <int KB>
__global__ __launch_bounds__(1024) void k_detect_finish(const uint32_t *__restrict__ pmask,
                                                        int row_chunks, int64_t K, int64_t kw,
                                                        DetectOut out) {
  extern __shared__ uint32_t smask[];  // [kw]
  const int t = threadIdx.x;
  if (out.ycmax)  // the epilogue's column maxima start from zero
    for (int64_t n = t; n < out.N; n += 1024) out.ycmax[n] = 0.f;
  if (out.sem)  // so do the split-K GEMM's arrival counters
    for (int64_t i = t; i < out.nsem; i += 1024) out.sem[i] = 0u;
  if (out.xcmax) {
    // outlier bits straight from the caller's column absmax of X
    for (int64_t w = t; w < kw; w += 1024) {
      uint32_t bits = 0u;
      for (int j = 0; j < 8; ++j) {
        const int64_t k = 32 * w + 4 * j;
        if (k >= K) break;
        const f32x4 v = *(const f32x4 *)(out.xcmax + k);
#pragma unroll
        for (int e = 0; e < 4; ++e) bits |= (v[e] >= out.threshold ? 1u : 0u) << (4 * j + e);
      }
      smask[w] = bits;
    }
    __syncthreads();
  } else {
    for (int64_t w = t; w < kw; w += 1024) smask[w] = 0u;
    __syncthreads();
    // OR the row-chunk masks: every thread issues a batch of KB independent
    // loads (the launch sizes KB so that one batch covers all the words), then
    // merges the non-zero words (rare) into LDS. Words past the end read as
    // zero through the buffer resource.
    const int64_t total_words = (int64_t)row_chunks * kw;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)pmask, (short)0, (int)(total_words * 4), 0x00020000);
    for (int64_t base = 0; base < total_words; base += 1024 * KB) {
      uint32_t v[KB];
#pragma unroll
      for (int u = 0; u < KB; ++u)
        v[u] = __builtin_amdgcn_raw_buffer_load_b32(rs, (int)(4 * (base + t + 1024 * u)), 0, 0);
#pragma unroll
      for (int u = 0; u < KB; ++u)
        if (v[u]) atomicOr(&smask[(base + t + 1024 * u) % kw], v[u]);
    }
    __syncthreads();
  }

  const int64_t per = (kw + 1023) / 1024;
  const int64_t w0 = (int64_t)t * per;
  const int64_t w1 = (w0 + per < kw) ? w0 + per : kw;
  int local = 0;
  for (int64_t w = w0; w < w1; ++w) {
    uint32_t v = smask[w];
    const int64_t valid = K - 32 * w;  // columns of this word inside K
    if (valid < 32) v &= (1u << valid) - 1u;
    smask[w] = v;
    out.omask[w] = v;
    local += __builtin_popcount(v);
  }

  // Block-wide exclusive scan of the per-thread counts.
  __shared__ int wsum[16];
  const int lane = t & 63, wv = t >> 6;
  int incl = local;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int y = __shfl_up(incl, off, 64);
    if (lane >= off) incl += y;
  }
  if (lane == 63) wsum[wv] = incl;
  __syncthreads();
  int before = 0, total = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    before += (i < wv) ? wsum[i] : 0;
    total += wsum[i];
  }
  int pos = before + incl - local;

  for (int64_t w = w0; w < w1; ++w) {
    uint32_t v = smask[w];
    out.wprefix[w] = pos;
    while (v) {  // the set bits of the word, ascending
      out.idx[pos++] = (int32_t)(32 * w + __builtin_ctz(v));
      v &= v - 1u;
    }
  }
  if (t == 0) {
    *out.count = total;
    if (out.count_copy) *out.count_copy = total;
  }
}

}  // namespace

DetectPlan detect_plan(int64_t M, int64_t K) {
  DetectPlan p;
  p.kw = (K + 31) / 32;
  p.col_tiles = (int)((K + kTileCols - 1) / kTileCols);
  // Aim for >= 4 rows per block phase and at most kMaxRowChunks partial masks.
  int64_t chunks = (M + 31) / 32;
  if (chunks > kMaxRowChunks) chunks = kMaxRowChunks;
  if (chunks < 1) chunks = 1;
  p.rows_per_chunk = (int)((M + chunks - 1) / chunks);
  p.row_chunks = (int)((M + p.rows_per_chunk - 1) / p.rows_per_chunk);
  return p;
}

hipError_t launch_detect(const uint16_t *X, int64_t M, int64_t K, int64_t ldx, float threshold,
                         const DetectPlan &plan, const DetectOut &out, hipStream_t stream) {
  // a caller-supplied column absmax replaces the scan of X
  if (!out.xcmax) {
    hipLaunchKernelGGL(k_detect_partial, dim3(plan.col_tiles, plan.row_chunks),
                       dim3(64 * kRowPhases), 0,
                       stream, X, M, K, ldx, threshold, plan.rows_per_chunk, plan.kw, out.pmask);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // one batch of partial-mask loads per thread covers all the words
  const int64_t words = out.xcmax ? 0 : (int64_t)plan.row_chunks * plan.kw;
  const size_t lds = (size_t)plan.kw * 4;
  const uint32_t *pm = (const uint32_t *)out.pmask;
  if (words <= 1024 * 8)
    hipLaunchKernelGGL(k_detect_finish<8>, dim3(1), dim3(1024), lds, stream, pm, plan.row_chunks,
                       K, plan.kw, out);
  else if (words <= 1024 * 16)
    hipLaunchKernelGGL(k_detect_finish<16>, dim3(1), dim3(1024), lds, stream, pm,
                       plan.row_chunks, K, plan.kw, out);
  else
    hipLaunchKernelGGL(k_detect_finish<32>, dim3(1), dim3(1024), lds, stream, pm,
                       plan.row_chunks, K, plan.kw, out);
  return hipGetLastError();
}

}  // namespace llmint8
