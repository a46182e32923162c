// Small-M (decode-shaped) path of the LLM.int8() linear layer on gfx950.
//
// With M <= 256 rows the layer is bound by streaming the int8 weight Wq from
// HBM (the decode regime of the INT8-vs-FP8 page, section one: every step
// re-reads all weights). The path is three kernels. None communicates across
// blocks inside a kernel (on gfx950 each XCD has its own L2, so an agent-scope
// fence writes back and invalidates a whole L2; stream order between kernels
// is the cheap handoff), and every load of a kernel is issued unconditionally
// (clamped address, result masked afterwards) so that all of a thread's loads are in
// flight before its first wait.
//
// k_decode_detect: block b owns 128 columns of X over all M rows. It writes the
//   outlier bits of its columns (4 mask words) and, per row, the absmax over
//   its kept columns; the row absmax over all kept columns is the max of these.
// k_decode_gemm: block (tile, kb) owns 64 output columns and one K range. It
//   reduces the partial maxima to m[i], quantizes its slice of X into LDS while
//   its Wq loads are in flight, runs 16x16x64 int8 MFMAs and stores int32
//   partial sums.
// k_decode_epilogue: adds the K-split partial sums in a fixed order (exact
//   integers), dequantizes, adds the fp16 outlier terms and writes Y.
#include "internal.hpp"

namespace llmint8 {

namespace {

constexpr int kDetCols = 128;      // columns per detection block (256: 1.2 us slower per step)
constexpr int kDetChunks = kDetCols / 8;            // 16-byte column chunks per block
constexpr int kDetRows = 256 / kDetChunks;          // row phases per detection block
constexpr int kDetRowIters = kDecodeMaxM / kDetRows;  // rows per thread up to kDecodeMaxM
constexpr int kTileN = 64;         // output columns per GEMM / epilogue block
constexpr int kSubK = 512;         // k bytes staged per GEMM stage
constexpr int kXPitch = kSubK + 16;
constexpr int kPmaxUnroll = 8;     // detection partials per thread loaded up front
constexpr int kTargetBlocks = 256; // GEMM blocks aimed for (one per CU)
constexpr int kOnePassBlocks = 768;  // most blocks for K ranges of at most two stages
constexpr int kWideBlocks = 512;     // blocks aimed for when that does not fit
constexpr int kGroupedOneRangeBlocks = 384;  // most blocks for 3-4 row groups over all of K
constexpr int kMaxSplits = 16;
constexpr int kListWords = 256;    // mask words scanned per epilogue window
constexpr int kOutBatch = 32;      // outlier columns staged per epilogue round
constexpr int kEpilogueFillBlocks = 256;  // epilogue blocks that fill the CUs

__device__ inline u32x4 zero4() { return (u32x4){0u, 0u, 0u, 0u}; }

// RI rows per thread: the launch takes the fewest that cover M (loads of rows
// past M, clamped to row 0, cost 0.3 us per call at M = 32 when RI covered 64)
template <int RI>
__global__ __launch_bounds__(256) void k_decode_detect(DecodeDetectArgs a) {
  static_assert(kDetCols % 64 == 0, "whole waves of column flags");
  __shared__ float scol[kDetRows][kDetCols];
  __shared__ uint32_t sflag[kDetCols / 32];
  const int t = threadIdx.x;
  const int c = t % kDetChunks, ph = t / kDetChunks;
  const int64_t col0 = (int64_t)blockIdx.x * kDetCols + c * 8;
  const bool colok = col0 < a.K;
  const uint16_t *base = a.X + (colok ? col0 : 0);
  if (a.ycmax)  // the epilogue's column maxima start from zero
    for (int64_t n = (int64_t)blockIdx.x * 256 + t; n < a.N; n += (int64_t)gridDim.x * 256)
      a.ycmax[n] = 0.f;
  // a caller-supplied column absmax decides the outlier columns
  float xc = 0.f;
  if (a.xcmax && t < kDetCols) {
    const int64_t col = (int64_t)blockIdx.x * kDetCols + t;
    xc = a.xcmax[col < a.K ? col : 0];
  }

  u32x4 v[RI];
#pragma unroll
  for (int j = 0; j < RI; ++j) {
    const int row = ph + kDetRows * j;
    const bool ok = colok && row < a.M;
    const u32x4 x = *(const u32x4 *)(base + (ok ? (int64_t)row * a.ldx : 0));
    v[j] = ok ? x : zero4();
  }
  float cm[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < RI; ++j) absmax8(v[j], cm);
#pragma unroll
  for (int e = 0; e < 8; ++e) scol[ph][c * 8 + e] = cm[e];
  __syncthreads();

  // column t of the block: outlier when its max over all rows reaches the threshold
  if (t < kDetCols) {  // whole waves
    float mx = 0.f;
#pragma unroll
    for (int p = 0; p < kDetRows; ++p) mx = __builtin_fmaxf(mx, scol[p][t]);
    const int64_t col = (int64_t)blockIdx.x * kDetCols + t;
    const bool flag = col < a.K && (a.xcmax ? xc : mx) >= a.threshold;
    const uint64_t bal = __ballot(flag);
    if ((t & 63) == 0) {
      sflag[(t >> 5)] = (uint32_t)bal;
      sflag[(t >> 5) + 1] = (uint32_t)(bal >> 32);
    }
  }
  __syncthreads();
  if (t < kDetCols / 32) {
    const int64_t w = (int64_t)blockIdx.x * (kDetCols / 32) + t;
    if (w < a.kw) a.omask[w] = sflag[t];
  }

  // per-row max over the block's kept columns; the kDetChunks lanes of a row
  // phase (consecutive lanes) reduce
  const unsigned ob = (sflag[c >> 2] >> ((c & 3) * 8)) & 0xffu;
#pragma unroll
  for (int j = 0; j < RI; ++j) {
    const int row = ph + kDetRows * j;
    float mx = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = (e & 1) ? fp16_hi(v[j][e >> 1]) : fp16_lo(v[j][e >> 1]);
      mx = ((ob >> e) & 1u) ? mx : __builtin_fmaxf(mx, __builtin_fabsf(x));
    }
#pragma unroll
    for (int off = kDetChunks / 2; off > 0; off >>= 1)
      mx = __builtin_fmaxf(mx, __shfl_xor(mx, off, 64));
    if (c == 0 && row < a.M) a.pmax[(int64_t)blockIdx.x * a.M + row] = mx;
  }
}

// Four int8 codes of the fp16 pairs (w0, w1) for the scale inv, packed in
// byte order. The fp32 product x * inv is rounded first (fp16_lo_mul /
// fp16_hi_mul; the sign of a zero product does not matter); adding 1.5 * 2^23 then
// rounds it to the nearest integer, ties to even (the sum's unit in the last
// place is 1), and leaves that integer in two's complement in the low bits of
// the sum. The product never exceeds 127 in magnitude by more than a few ulps
// (|x| <= absmax of its row), so no clamp is needed.
__device__ inline uint32_t codes4(uint32_t w0, uint32_t w1, float inv) {
#pragma clang fp contract(off)
  const float kMagic = 12582912.0f;
  const uint32_t q0 = __builtin_bit_cast(uint32_t, fp16_lo_mul(w0, inv) + kMagic);
  const uint32_t q1 = __builtin_bit_cast(uint32_t, fp16_hi_mul(w0, inv) + kMagic);
  const uint32_t q2 = __builtin_bit_cast(uint32_t, fp16_lo_mul(w1, inv) + kMagic);
  const uint32_t q3 = __builtin_bit_cast(uint32_t, fp16_hi_mul(w1, inv) + kMagic);
  return (q0 & 0xffu) | ((q1 & 0xffu) << 8) | ((q2 & 0xffu) << 16) | (q3 << 24);
}

// 0xff in byte e of the result when bit e of the low four bits of n is clear.
__device__ inline uint32_t keep_bytes(uint32_t n4) {
  return ~(((n4 * 0x00204081u) & 0x01010101u) * 0xffu);
}

// One GEMM stage: a 512-byte K range of X (all rows of the block) and of the
// wave's 16 Wq rows. Loads past the end of the range read clamped addresses
// and are neutralised afterwards: their X codes are masked to zero (so the
// Wq bytes they meet do not matter), rows past M have a zero scale.
template <int MB>
struct DecodeStage {
  u32x4 x[4 * MB];       // X chunk: row wv + 4 u, columns k0 + 8 lane .. + 8
  u32x4 b[kSubK / 64];   // Wq bytes k0 + 64 j + 16 g .. + 16 of column ncol
  uint32_t mw;           // outlier mask word of column k0 + 8 lane
  bool kok;              // column k0 + 8 lane lies inside the K range
};

// r0: the first row of the block's row group (rows past M read row 0).
template <int MB>
__device__ inline void decode_load_x(const DecodeGemmArgs &a, DecodeStage<MB> &st, int64_t k0,
                                     int64_t k_end, int r0, int wv, int lane) {
  const int64_t kx = k0 + 8 * lane;
  st.kok = kx < k_end;
  const int64_t kxc = st.kok ? kx : 0;
  st.mw = a.omask[kxc >> 5];
#pragma unroll
  for (int u = 0; u < 4 * MB; ++u) {
    const int row = r0 + wv + 4 * u;
    st.x[u] = *(const u32x4 *)(a.X + (int64_t)(row < a.M ? row : 0) * a.ldx + kxc);
  }
}

template <int MB>
__device__ inline void decode_load_b(DecodeStage<MB> &st, int64_t k0, int64_t k_end,
                                     const int8_t *brow, int g) {
#pragma unroll
  for (int j = 0; j < kSubK / 64; ++j) {
    const int64_t k = k0 + 64 * j + 16 * g;
    st.b[j] = *(const u32x4 *)(brow + (k < k_end ? k : 0));
  }
}

template <int MB>
__device__ inline void decode_load(const DecodeGemmArgs &a, DecodeStage<MB> &st, int64_t k0,
                                   int64_t k_end, const int8_t *brow, int r0, int wv, int lane,
                                   int g) {
  decode_load_x<MB>(a, st, k0, k_end, r0, wv, lane);
  decode_load_b<MB>(st, k0, k_end, brow, g);
}

// Four E4M3 codes of the fp16 pairs (w0, w1) for the scale inv = fl32(448 /
// absmax): the fp32 products, then the hardware conversion (nearest, ties to
// even). A zero product always codes as +0 here, where a plain multiply would
// give -0 for a negative x on a row of scale zero; the sums are the same.
__device__ inline uint32_t codes4_e4m3(uint32_t w0, uint32_t w1, float inv) {
#pragma clang fp contract(off)
  const float t[4] = {fp16_lo_mul(w0, inv), fp16_hi_mul(w0, inv), fp16_lo_mul(w1, inv),
                      fp16_hi_mul(w1, inv)};
  return CodecE4M3::code4(t);
}

// Quantize the stage's X chunks into the LDS buffer sx.
template <int MB, bool F8>
__device__ inline void decode_quant(const DecodeStage<MB> &st, uint8_t *sx, const float *sinv,
                                    int wv, int lane) {
  const uint32_t ob = st.kok ? (st.mw >> (8 * (lane & 3))) & 0xffu : 0xffu;
  const uint32_t keep_lo = keep_bytes(ob & 0xfu), keep_hi = keep_bytes(ob >> 4);
#pragma unroll
  for (int u = 0; u < 4 * MB; ++u) {
    const int row = wv + 4 * u;
    const float inv = sinv[row];
    u32x2 out;
    if constexpr (F8) {
      out[0] = codes4_e4m3(st.x[u][0], st.x[u][1], inv) & keep_lo;
      out[1] = codes4_e4m3(st.x[u][2], st.x[u][3], inv) & keep_hi;
    } else {
      out[0] = codes4(st.x[u][0], st.x[u][1], inv) & keep_lo;
      out[1] = codes4(st.x[u][2], st.x[u][3], inv) & keep_hi;
    }
    *(u32x2 *)(sx + row * kXPitch + 8 * lane) = out;
  }
}

// Contract the stage's X codes in sx with its Wq bytes.
// F8: E4M3 codes and v_mfma_f32_16x16x128_f8f6f4, which takes the Wq bytes of
// two consecutive int8 steps (j = 2 jj, 2 jj + 1) per lane and the X codes of
// the same k, so both operands see the same k in every slot; the fp32 sums
// are kept as raw bits in the int32 accumulators.
template <int MB, bool F8>
__device__ inline void decode_mma(const DecodeStage<MB> &st, const uint8_t *sx, i32x4 *acc,
                                  int c16, int g) {
  if constexpr (F8) {
#pragma unroll
    for (int jj = 0; jj < kSubK / 128; ++jj) {
      i32x8 bv;
      bv.lo = __builtin_bit_cast(i32x4, st.b[2 * jj]);
      bv.hi = __builtin_bit_cast(i32x4, st.b[2 * jj + 1]);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const uint8_t *xr = sx + (mb * 16 + c16) * kXPitch + 16 * g;
        i32x8 av;
        av.lo = *(const i32x4 *)(xr + 128 * jj);
        av.hi = *(const i32x4 *)(xr + 128 * jj + 64);
        acc[mb] = __builtin_bit_cast(
            i32x4, __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                       av, bv, __builtin_bit_cast(f32x4, acc[mb]), 0, 0, 0, 0, 0, 0));
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < kSubK / 64; ++j)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const i32x4 av = *(const i32x4 *)(sx + (mb * 16 + c16) * kXPitch + 64 * j + 16 * g);
        acc[mb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, __builtin_bit_cast(i32x4, st.b[j]),
                                                         acc[mb], 0, 0, 0);
      }
  }
}

// One stage through a single LDS buffer: quantize, then contract.
template <int MB, bool F8>
__device__ inline void decode_step(const DecodeStage<MB> &st, uint8_t *sx, const float *sinv,
                                   i32x4 *acc, int wv, int lane, int c16, int g) {
  __syncthreads();  // sinv ready; the previous stage's MFMAs are done with sx
  decode_quant<MB, F8>(st, sx, sinv, wv, lane);
  __syncthreads();
  decode_mma<MB, F8>(st, sx, acc, c16, g);
}

// Block (tile, kb). Wave w owns 16 output columns; lane (c16 = l % 16,
// g = l / 16) supplies, for MFMA step j, the 16 Wq bytes at k = 64 j + 16 g of
// its column and reads the matching Xq bytes from LDS. MB 16-row blocks cover M.
// NST is the number of 512-byte stages of the block's K range when it is 1 or
// 2 (straight-line code, all loads issued before the first wait), 0 for any
// count. With two stages, both are quantized into LDS buffers of their own
// before either is contracted, so only the MFMAs wait for the Wq stream. For
// any count, two register stages alternate so that the next stage's loads are
// in flight while the current one is quantized and contracted. No load is
// issued under a branch that the following waits would have to merge.
// RG: the launch has row groups (M > 64); without them the block covers rows
// 0 .. M - 1 and the group arithmetic folds away.
template <int MB, int NST, bool F8, bool RG>
__global__ __launch_bounds__(256) void k_decode_gemm(DecodeGemmArgs a) {
  constexpr int kStageBytes = MB * 16 * kXPitch;
  __shared__ __attribute__((aligned(16))) uint8_t sx[(NST == 2 ? 2 : 1) * kStageBytes];
  __shared__ float spart[4][64];
  __shared__ float sinv[64];
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int c16 = lane & 15, g = lane >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * kTileN;
  const int kb = blockIdx.y;
  const int64_t K = a.K;
  const int64_t k_begin = (int64_t)kb * a.kc;
  const int64_t k_end = (k_begin + a.kc < K) ? k_begin + a.kc : K;
  const int64_t ncol = n0 + wv * 16 + c16;
  const int8_t *brow = a.wq + ((ncol < a.N) ? ncol : a.N - 1) * K;
  // row group: rows r0 .. r0 + 63 (the blocks of the groups of one tile and
  // K split are 256 or more block ids apart, a multiple of the 8 XCDs, so they
  // run on one XCD and its L2 serves the second read of their Wq bytes)
  const int r0 = RG ? kDecodeGroupRows * (int)blockIdx.z : 0;
  const int mg = !RG ? (int)a.M
                     : (a.M - r0 < kDecodeGroupRows) ? (int)(a.M - r0) : kDecodeGroupRows;

  // detection partials of row r0 + `lane`, blocks wv + 4 i (first kPmaxUnroll up front)
  const int prow = lane < mg ? r0 + lane : 0;
  float pv[kPmaxUnroll];
#pragma unroll
  for (int i = 0; i < kPmaxUnroll; ++i) {
    const int s = wv + 4 * i;
    const float p = a.pmax[(int64_t)(s < a.det_blocks ? s : 0) * a.M + prow];
    pv[i] = s < a.det_blocks ? p : 0.f;
  }

  DecodeStage<MB> s0, s1;
  if constexpr (NST == 2) {
    // both X stages ahead of the Wq bytes: loads complete in issue order, so
    // the X codes of both stages can be formed while Wq is still streaming
    decode_load_x<MB>(a, s0, k_begin, k_end, r0, wv, lane);
    decode_load_x<MB>(a, s1, k_begin + kSubK, k_end, r0, wv, lane);
    decode_load_b<MB>(s0, k_begin, k_end, brow, g);
    decode_load_b<MB>(s1, k_begin + kSubK, k_end, brow, g);
  } else {
    decode_load<MB>(a, s0, k_begin, k_end, brow, r0, wv, lane, g);
  }
  __builtin_amdgcn_sched_barrier(0);  // every load above is issued before the first wait

  float pm = 0.f;
#pragma unroll
  for (int i = 0; i < kPmaxUnroll; ++i) pm = __builtin_fmaxf(pm, pv[i]);
  for (int s = wv + 4 * kPmaxUnroll; s < a.det_blocks; s += 4)
    pm = __builtin_fmaxf(pm, a.pmax[(int64_t)s * a.M + prow]);
  spart[wv][lane] = pm;
  __syncthreads();
  if (t < 64) {
    const float mx = __builtin_fmaxf(__builtin_fmaxf(spart[0][t], spart[1][t]),
                                     __builtin_fmaxf(spart[2][t], spart[3][t]));
    sinv[t] = (t < mg && mx > 0.f) ? (F8 ? inv_scale_of<CodecE4M3>(mx) : inv_scale(mx)) : 0.f;
    if (kb == 0 && blockIdx.x == 0 && t < mg) a.m[r0 + t] = mx;
  }

  i32x4 acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = (i32x4){0, 0, 0, 0};

  if constexpr (NST == 1) {
    decode_step<MB, F8>(s0, sx, sinv, acc, wv, lane, c16, g);
  } else if constexpr (NST == 2) {
    __syncthreads();  // sinv ready
    decode_quant<MB, F8>(s0, sx, sinv, wv, lane);
    decode_quant<MB, F8>(s1, sx + kStageBytes, sinv, wv, lane);
    __syncthreads();
    decode_mma<MB, F8>(s0, sx, acc, c16, g);
    decode_mma<MB, F8>(s1, sx + kStageBytes, acc, c16, g);
  } else {
    const int nst = (int)((k_end - k_begin + kSubK - 1) / kSubK);
    int64_t k0 = k_begin;
    int i = 0;
    for (; i + 2 < nst; i += 2, k0 += 2 * kSubK) {  // stages i + 1 and i + 2 exist
      decode_load<MB>(a, s1, k0 + kSubK, k_end, brow, r0, wv, lane, g);
      decode_step<MB, F8>(s0, sx, sinv, acc, wv, lane, c16, g);
      decode_load<MB>(a, s0, k0 + 2 * kSubK, k_end, brow, r0, wv, lane, g);
      decode_step<MB, F8>(s1, sx, sinv, acc, wv, lane, c16, g);
    }
    if (nst - i == 2) {
      decode_load<MB>(a, s1, k0 + kSubK, k_end, brow, r0, wv, lane, g);
      decode_step<MB, F8>(s0, sx, sinv, acc, wv, lane, c16, g);
      decode_step<MB, F8>(s1, sx, sinv, acc, wv, lane, c16, g);
    } else {
      decode_step<MB, F8>(s0, sx, sinv, acc, wv, lane, c16, g);
    }
  }

  // partial sums: lane holds rows 4g + r of each 16-row block, column ncol.
  // Nontemporal stores: the epilogue kernel reads them once, and lines left
  // dirty in L2 would only lengthen the write-back at the end of this kernel
  // (measured 0.08 us per decode call).
  if (ncol < a.N) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = mb * 16 + 4 * g + r;
        if (row < mg)
          __builtin_nontemporal_store(acc[mb][r],
                                      &a.part[((int64_t)kb * a.M + r0 + row) * a.N + ncol]);
      }
  }
}

// Block (tile, row block of ER = 16 or 8): 64 columns x ER rows, ER / 4
// outputs per thread (rows wv + 4 i, column lane). KB is the number of K
// splits; F8: the partial sums are fp32 (added in split order) and the
// dequantization is / 448^2.
template <int KB, bool F8, int ER>
__global__ __launch_bounds__(256) void k_decode_epilogue(DecodeGemmArgs a) {
  constexpr int kEpiI = ER / 4;                 // outputs per thread
  constexpr int kEpiXH = ER * kOutBatch / 256;  // X entries per thread and batch
  static_assert(kEpiXH >= 1, "one X entry per thread at least");
  __shared__ int slist[kListWords * 32];             // outlier columns of one window
  __shared__ int swsum[4];
  __shared__ float sxo[ER][kOutBatch];               // [row][p]
  __shared__ __attribute__((aligned(16))) uint16_t swo[kOutBatch * kTileN];  // [p][col]
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int64_t n0 = (int64_t)blockIdx.x * kTileN;
  const int64_t col = n0 + lane;
  const bool colok = col < a.N;
  const int64_t colc = colok ? col : 0;
  const int rbase = blockIdx.y * ER;

  // every independent load first, the first mask window ahead of the rest:
  // the outlier chain (mask, list, W rows and X entries) is the longest
  // dependent path of the block, and loads complete in issue order
  const __amdgpu_buffer_rsrc_t mrs =
      __builtin_amdgcn_make_buffer_rsrc((void *)a.omask, (short)0, (int)(a.kw * 4), 0x00020000);
  uint32_t mw = __builtin_amdgcn_raw_buffer_load_b32(mrs, 4 * t, 0, 0);

  int pp[kEpiI][KB];
  float mrow[kEpiI];
#pragma unroll
  for (int i = 0; i < kEpiI; ++i) {
    const int row = rbase + wv + 4 * i;
    const int rowc = row < a.M ? row : 0;
#pragma unroll
    for (int k = 0; k < KB; ++k) pp[i][k] = a.part[((int64_t)k * a.M + rowc) * a.N + colc];
    mrow[i] = a.m[rowc];
  }
  const float scol = a.s[colc];
  // loads without a condition (a bias-less call reads its bias bits from s):
  // a load under a branch is waited for at once, and with it every earlier one
  const uint16_t braw = (a.ep.bias ? a.ep.bias : (const uint16_t *)a.s)[colc];
  // wait for the mask word alone here (the partial sums stay in flight); left
  // to itself the compiler sinks its load below all the others
  asm volatile("" ::"v"(mw));
  // the outlier product runs with fp16 weight rows or with the int8 codes
  const bool i8w = a.ep.int8w != 0;
  const bool outl = a.w || i8w;
  float yo[kEpiI];
#pragma unroll
  for (int i = 0; i < kEpiI; ++i) yo[i] = 0.f;
  // fp16 outlier terms, outlier columns in ascending order (yo: with int8
  // weight codes they are scaled by s / 127 at the end); the partial sums are
  // added after them, so the chain does not wait for the partial sums
  int total_all = 0;
  if (outl) {
    for (int64_t w0 = 0; w0 < a.kw; w0 += kListWords) {
      if (w0 > 0) {
        __syncthreads();  // the previous window's list is consumed
        mw = __builtin_amdgcn_raw_buffer_load_b32(mrs, (int)(4 * (w0 + t)), 0, 0);
      }
      // block-wide exclusive scan of the per-word outlier counts
      const int cnt = __builtin_popcount(mw);
      int incl = cnt;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int yv = __shfl_up(incl, off, 64);
        if (lane >= off) incl += yv;
      }
      if (lane == 63) swsum[wv] = incl;
      __syncthreads();
      int before = 0, total = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        before += (i < wv) ? swsum[i] : 0;
        total += swsum[i];
      }
      int pos = before + incl - cnt;
      uint32_t mm = mw;
      while (mm) {
        slist[pos++] = (int)(32 * (w0 + t) + __builtin_ctz(mm));
        mm &= mm - 1u;
      }
      total_all += total;
      __syncthreads();
      for (int p0 = 0; p0 < total; p0 += kOutBatch) {
        const int np = (total - p0 < kOutBatch) ? total - p0 : kOutBatch;
        // W rows and X entries of the batch, all loaded before the first LDS
        // store so that they share one round trip. Entries past the batch,
        // past N or past M read clamped addresses: they only reach outputs
        // never stored or terms never summed.
        {  // X entries first (16 rows x 32 outliers, two per thread), then the
           // W rows (32 rows x 8 chunks of 8 columns, one per thread)
          uint32_t xe[kEpiXH];
          int xr[kEpiXH], xp[kEpiXH];
#pragma unroll
          for (int h = 0; h < kEpiXH; ++h) {
            const int q = t + 256 * h;
            xr[h] = q >> 5;
            xp[h] = q & 31;
            const int row = rbase + xr[h];
            const int64_t kk = slist[p0 + (xp[h] < np ? xp[h] : np - 1)];
            xe[h] = a.X[(int64_t)(row < a.M ? row : a.M - 1) * a.ldx + kk];
          }
          const int p = t >> 3, ch = t & 7;
          const int64_t cc = n0 + 8 * ch;
          const int64_t kk = slist[p0 + (p < np ? p : np - 1)];
          u32x4 v;
          if (i8w) {  // codes Wq[n, kk] of the 8 columns, as fp16 (exact)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int64_t c0 = cc + 2 * e, c1 = c0 + 1;
              const int q0 = a.wq[(c0 < a.N ? c0 : a.N - 1) * a.K + kk];
              const int q1 = a.wq[(c1 < a.N ? c1 : a.N - 1) * a.K + kk];
              v[e] = (uint32_t)f2h((float)q0) | ((uint32_t)f2h((float)q1) << 16);
            }
          } else {
            v = *(const u32x4 *)(a.w + kk * a.ldw + (cc < a.N ? cc : a.N - 8));
          }
          *(u32x4 *)(swo + p * kTileN + 8 * ch) = v;
#pragma unroll
          for (int h = 0; h < kEpiXH; ++h) sxo[xr[h]][xp[h]] = h2f((uint16_t)xe[h]);
        }
        __syncthreads();
        for (int p = 0; p < np; ++p) {
          const float wval = h2f(swo[p * kTileN + lane]);
#pragma unroll
          for (int i = 0; i < kEpiI; ++i) yo[i] += sxo[wv + 4 * i][p] * wval;
        }
        __syncthreads();
      }
    }
    if (blockIdx.x == 0 && blockIdx.y == 0 && t == 0 && a.count_out) *a.count_out = total_all;
  } else if (blockIdx.x == 0 && blockIdx.y == 0 && a.count_out) {
    // no outlier product: count the mask bits only
    __shared__ int scount[4];
    int cnt = 0;
    for (int64_t w = t; w < a.kw; w += 256) cnt += __builtin_popcount(a.omask[w]);
    cnt = wave_sum(cnt);
    if (lane == 0) scount[wv] = cnt;
    __syncthreads();
    if (t == 0) *a.count_out = scount[0] + scount[1] + scount[2] + scount[3];
  }

  float y[kEpiI];
  const float sd = scol * (F8 ? 1.0f / 200704.0f : 1.0f / 16129.0f);
#pragma unroll
  for (int i = 0; i < kEpiI; ++i) {
    int cacc = 0;
    float cf = 0.f;
#pragma unroll
    for (int k = 0; k < KB; ++k) {
      if constexpr (F8)
        cf += __builtin_bit_cast(float, pp[i][k]);
      else
        cacc += pp[i][k];
    }
    const int row = rbase + wv + 4 * i;
    if (a.cdbg && row < a.M && colok)
      a.cdbg[(int64_t)row * a.N + col] = F8 ? __builtin_bit_cast(int, cf) : cacc;
    y[i] = (F8 ? cf : (float)cacc) * (mrow[i] * sd);
  }

  const float oscale = i8w ? scol * (1.0f / 127.0f) : 1.0f;
  const float bcol = a.ep.bias ? h2f(braw) : 0.f;
  float cmax = 0.f;  // |Y| of this column over the block's rows
#pragma unroll
  for (int i = 0; i < kEpiI; ++i) {
    const int row = rbase + wv + 4 * i;
    const float v = y[i] + yo[i] * oscale + bcol;
    if (colok && row < a.M) a.y[(int64_t)row * a.ldy + col] = f2h(v);
    cmax = row < a.M ? __builtin_fmaxf(cmax, stored_abs(v)) : cmax;
  }
  if (a.ep.ycmax) {
    __shared__ float scm[4][kTileN];
    scm[wv][lane] = cmax;
    __syncthreads();
    if (t < kTileN && n0 + t < a.N) {
      const float mx = __builtin_fmaxf(__builtin_fmaxf(scm[0][t], scm[1][t]),
                                       __builtin_fmaxf(scm[2][t], scm[3][t]));
      ycmax_update(a.ep.ycmax, n0 + t, mx);
    }
  }
}

template <int MB, bool F8, bool RG>
hipError_t launch_decode_gemm_rg(const DecodeGemmArgs &a, int tiles, int kb, const GemmEvents &ev,
                                 hipStream_t stream) {
  const int64_t nst = (a.kc + kSubK - 1) / kSubK;
  const hipEvent_t b = (hipEvent_t)ev.begin, e = (hipEvent_t)ev.end;
  const dim3 grid(tiles, kb, (unsigned)((a.M + kDecodeGroupRows - 1) / kDecodeGroupRows));
  if (nst == 1)
    hipExtLaunchKernelGGL((k_decode_gemm<MB, 1, F8, RG>), grid, dim3(256), 0, stream, b, e, 0u, a);
  else if (nst == 2)
    hipExtLaunchKernelGGL((k_decode_gemm<MB, 2, F8, RG>), grid, dim3(256), 0, stream, b, e, 0u, a);
  else
    hipExtLaunchKernelGGL((k_decode_gemm<MB, 0, F8, RG>), grid, dim3(256), 0, stream, b, e, 0u, a);
  return hipGetLastError();
}

template <int MB, bool F8>
hipError_t launch_decode_gemm(const DecodeGemmArgs &a, int tiles, int kb, const GemmEvents &ev,
                              hipStream_t stream) {
  if constexpr (MB == kDecodeGroupRows / 16) {
    if (a.M > kDecodeGroupRows) return launch_decode_gemm_rg<MB, F8, true>(a, tiles, kb, ev, stream);
  }
  return launch_decode_gemm_rg<MB, F8, false>(a, tiles, kb, ev, stream);
}

// 8-row blocks when 16-row blocks would leave CUs idle: graph-replayed,
// 32x4096x4096 11.4-11.5 -> 11.3 us and 24x4096x4096 11.3 -> 11.0 us, while
// with enough 16-row blocks the 8-row ones cost more (64x4096x11008 25.3 ->
// 26.6 us, 128x4096x4096 20.6 -> 20.9 us).
template <int KB, bool F8>
hipError_t launch_decode_epilogue(const DecodeGemmArgs &a, int tiles, hipStream_t stream) {
  const int64_t blocks16 = (int64_t)tiles * ((a.M + 15) / 16);
  if (blocks16 < kEpilogueFillBlocks)
    hipLaunchKernelGGL((k_decode_epilogue<KB, F8, 8>), dim3(tiles, (unsigned)((a.M + 7) / 8)),
                       dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((k_decode_epilogue<KB, F8, 16>), dim3(tiles, (unsigned)((a.M + 15) / 16)),
                       dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <bool F8>
hipError_t launch_decode_kernels(const DecodeGemmArgs &gemm, const DecodePlan &plan,
                                 const GemmEvents &ev, hipStream_t stream) {
  hipError_t e;
  // MB 16-row blocks cover one row group
  const int64_t rows = gemm.M < kDecodeGroupRows ? gemm.M : kDecodeGroupRows;
  switch ((int)((rows + 15) / 16)) {
    case 1: e = launch_decode_gemm<1, F8>(gemm, plan.tiles, plan.kb, ev, stream); break;
    case 2: e = launch_decode_gemm<2, F8>(gemm, plan.tiles, plan.kb, ev, stream); break;
    case 3: e = launch_decode_gemm<3, F8>(gemm, plan.tiles, plan.kb, ev, stream); break;
    default: e = launch_decode_gemm<4, F8>(gemm, plan.tiles, plan.kb, ev, stream); break;
  }
  if (e != hipSuccess) return e;
  switch (plan.kb) {
    case 1: return launch_decode_epilogue<1, F8>(gemm, plan.tiles, stream);
    case 2: return launch_decode_epilogue<2, F8>(gemm, plan.tiles, stream);
    case 4: return launch_decode_epilogue<4, F8>(gemm, plan.tiles, stream);
    case 8: return launch_decode_epilogue<8, F8>(gemm, plan.tiles, stream);
    default: return launch_decode_epilogue<16, F8>(gemm, plan.tiles, stream);
  }
}

}  // namespace

DecodePlan decode_plan(int64_t M, int64_t K, int64_t N) {
  DecodePlan p;
  p.tiles = (int)((N + kTileN - 1) / kTileN);
  // blocks per K split: tiles x row groups
  const int64_t per = (int64_t)p.tiles * ((M + kDecodeGroupRows - 1) / kDecodeGroupRows);
  p.det_blocks = (int)((K + kDetCols - 1) / kDetCols);
  // K splits: a power of two, about kTargetBlocks blocks in all, and at least
  // one full stage of K per split
  auto splits_for = [&](int64_t target) {
    int b = 1;
    while (b < kMaxSplits && per * (b * 2) <= target && K / (b * 2) >= kSubK)
      b *= 2;
    return b;
  };
  int kb = splits_for(kTargetBlocks);
  // A K range of at most two stages issues all of its loads before its first
  // wait; a longer one streams through two register stages, one ahead. With
  // more than 16 rows, when the ranges are longer than that, split further if
  // it takes at most kOnePassBlocks blocks, else aim for kWideBlocks blocks.
  // Measured under graph replay (same weights each call): 64x4096x11008
  // 35.7 -> 25.8 us, 32x4096x11008 22.7 -> 20.0 us (one-pass ranges);
  // 32x5120x13824 28.2 -> 25.7 us, 48x8192x4096 22.1 -> 21.1 us (more
  // blocks); splitting 32x11008x4096 into one-pass ranges (1024 blocks) took
  // 31.7 us against 24.7, and with one or two rows the extra splits cost
  // more than they gain (1x12288x1032 13.8 -> 15.5 us).
  if (M > 16 && (K + kb - 1) / kb > 2 * kSubK) {
    int b = kb;
    while (b < kMaxSplits && (K + b - 1) / b > 2 * kSubK) b *= 2;
    kb = ((K + b - 1) / b <= 2 * kSubK && per * b <= kOnePassBlocks)
             ? b
             : splits_for(kWideBlocks);
  }
  int64_t kc = (K + kb - 1) / kb;
  kc = (kc + 63) / 64 * 64;
  p.kc = kc;
  p.kb = kb;  // a trailing split may be empty; its partial sums are zero
  return p;
}

// Up to 64 rows the small-M kernels always run. With 65 to 256 rows (two to
// four row groups, whose blocks read the same Wq bytes) they run only when the
// plan reaches K ranges of at most two stages within kOnePassBlocks blocks;
// the large-M path is faster otherwise. Graph-replayed (same weights each
// call): 65x4096x4096 33.1 -> 19.2 us, 128x4096x4096 33.6 -> 21.3 us,
// 192x4096x4096 33.9 -> 28.9 us, 192x2048x2048 31.5 -> 17.7 us on this path;
// 128x4096x11008 35.3 against 66.2 us and 128x8192x8192 40.7 against 67.9 us
// stay on the large-M path, and with a 1024-block budget 256x4096x4096 ran
// level with it (34.5 us). With three or four row groups and one K range per
// block (K <= 1024, where the large-M path costs least, about 25 us) the
// small-M kernels lose beyond kGroupedOneRangeBlocks blocks: 160x1024x11008
// 29.9 against 25.1 us, 256x1024x8192 26.7 against 25.4 us, 160x1024x14336
// 31.3 against 25.6 us, while 192x1024x8192 (384 blocks) ran 24.5 against
// 25.1 us and 160x1024x8192 23.2 against 25.2 us.
bool use_decode_path(int64_t M, int64_t K, int64_t N) {
  if (M <= kDecodeGroupRows) return true;
  if (M > kDecodeMaxM) return false;
  const DecodePlan p = decode_plan(M, K, N);
  const int64_t groups = (M + kDecodeGroupRows - 1) / kDecodeGroupRows;
  const int64_t blocks = (int64_t)p.tiles * groups * p.kb;
  if (p.kc > 2 * kSubK || blocks > kOnePassBlocks) return false;
  return groups <= 2 || p.kb > 1 || blocks <= kGroupedOneRangeBlocks;
}

hipError_t launch_decode(const DecodeDetectArgs &det, const DecodeGemmArgs &gemm,
                         const DecodePlan &plan, const GemmEvents &ev, hipStream_t stream) {
  static_assert(kDetRowIters == 16, "detection row iterations");
  if (det.M <= kDetRows)
    hipLaunchKernelGGL(k_decode_detect<1>, dim3(plan.det_blocks), dim3(256), 0, stream, det);
  else if (det.M <= 2 * kDetRows)
    hipLaunchKernelGGL(k_decode_detect<2>, dim3(plan.det_blocks), dim3(256), 0, stream, det);
  else if (det.M <= 4 * kDetRows)
    hipLaunchKernelGGL(k_decode_detect<4>, dim3(plan.det_blocks), dim3(256), 0, stream, det);
  else if (det.M <= 8 * kDetRows)
    hipLaunchKernelGGL(k_decode_detect<8>, dim3(plan.det_blocks), dim3(256), 0, stream, det);
  else
    hipLaunchKernelGGL(k_decode_detect<16>, dim3(plan.det_blocks), dim3(256), 0, stream, det);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return gemm.fp8 ? launch_decode_kernels<true>(gemm, plan, ev, stream)
                  : launch_decode_kernels<false>(gemm, plan, ev, stream);
}

}  // namespace llmint8
