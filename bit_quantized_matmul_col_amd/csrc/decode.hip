// Small-M (decode-shaped) path of the LLM.int8() linear layer on gfx950.
//
// With M <= 64 rows the layer is bound by streaming the int8 weight Wq from
// HBM (the decode regime of the INT8-vs-FP8 page, section one: every step
// re-reads all weights). The path is three kernels; none waits on a chain of
// dependent loads and none communicates across blocks inside a kernel (on
// gfx950 each XCD has its own L2, so an agent-scope fence writes back and
// invalidates a whole L2; stream order between kernels is the cheap handoff).
//
// k_decode_detect: block b owns 256 columns of X over all M rows. It writes the
//   outlier bits of its columns (8 mask words) and, per row, the absmax over
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

constexpr int kDetCols = 256;      // columns per detection block
constexpr int kDetRows = 8;        // row phases per detection block (32 x 8 threads)
constexpr int kTileN = 64;         // output columns per GEMM / epilogue block
constexpr int kSubK = 512;         // k bytes staged per GEMM block iteration
constexpr int kXPitch = kSubK + 16;
constexpr int kOutBatch = 16;      // outlier columns staged per epilogue round

__global__ __launch_bounds__(256) void k_decode_detect(DecodeDetectArgs a) {
  __shared__ float scol[kDetRows][kDetCols];
  __shared__ uint32_t sflag[kDetCols / 32];
  const int t = threadIdx.x;
  const int c = t & 31, ph = t >> 5;
  const int64_t col0 = (int64_t)blockIdx.x * kDetCols + c * 8;
  const bool colok = col0 < a.K;

  // every (row phase, chunk) load of the block is in flight at once
  u32x4 v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int row = ph + kDetRows * j;
    v[j] = (u32x4){0u, 0u, 0u, 0u};
    if (colok && row < a.M) v[j] = *(const u32x4 *)(a.X + (int64_t)row * a.ldx + col0);
  }
  float cm[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < 8; ++j) absmax8(v[j], cm);
#pragma unroll
  for (int e = 0; e < 8; ++e) scol[ph][c * 8 + e] = cm[e];
  __syncthreads();

  // column t of the block: outlier when its max over all rows reaches the threshold
  {
    float mx = 0.f;
#pragma unroll
    for (int p = 0; p < kDetRows; ++p) mx = __builtin_fmaxf(mx, scol[p][t]);
    const int64_t col = (int64_t)blockIdx.x * kDetCols + t;
    const bool flag = col < a.K && mx >= a.threshold;
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

  // per-row max over the block's kept columns; the 32 lanes of a row phase reduce
  const unsigned ob = (sflag[c >> 2] >> ((c & 3) * 8)) & 0xffu;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int row = ph + kDetRows * j;
    float mx = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = (e & 1) ? fp16_hi(v[j][e >> 1]) : fp16_lo(v[j][e >> 1]);
      if (!((ob >> e) & 1u)) mx = __builtin_fmaxf(mx, __builtin_fabsf(x));
    }
#pragma unroll
    for (int off = 16; off > 0; off >>= 1) mx = __builtin_fmaxf(mx, __shfl_xor(mx, off, 64));
    if (c == 0 && row < a.M) a.pmax[(int64_t)blockIdx.x * a.M + row] = mx;
  }
}

// Block (tile, kb). Wave w owns 16 output columns; lane (c16 = l % 16,
// g = l / 16) loads, for MFMA step j, the 16 bytes at k = 64 j + 16 g of its
// Wq row, and reads the matching Xq bytes from LDS. MB 16-row blocks cover M.
template <int MB>
__global__ __launch_bounds__(256) void k_decode_gemm(DecodeGemmArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t sx[MB * 16 * kXPitch];
  __shared__ float sinv[MB * 16];
  __shared__ int s_cnt[4];
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int c16 = lane & 15, g = lane >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * kTileN;
  const int kb = blockIdx.y;
  const int64_t K = a.K;
  const int64_t k_begin = (int64_t)kb * a.kc;
  const int64_t k_end = (k_begin + a.kc < K) ? k_begin + a.kc : K;
  const int64_t ncol = n0 + wv * 16 + c16;
  const int8_t *brow = a.wq + ((ncol < a.N) ? ncol : a.N - 1) * K;

  // row absmax over all kept columns = max of the detection blocks' partials
  if (t < a.M) {
    float mx = 0.f;
    int s = 0;
    for (; s + 4 <= a.det_blocks; s += 4) {
      const float p0 = a.pmax[(int64_t)s * a.M + t], p1 = a.pmax[(int64_t)(s + 1) * a.M + t];
      const float p2 = a.pmax[(int64_t)(s + 2) * a.M + t], p3 = a.pmax[(int64_t)(s + 3) * a.M + t];
      mx = __builtin_fmaxf(mx, __builtin_fmaxf(__builtin_fmaxf(p0, p1), __builtin_fmaxf(p2, p3)));
    }
    for (; s < a.det_blocks; ++s) mx = __builtin_fmaxf(mx, a.pmax[(int64_t)s * a.M + t]);
    sinv[t] = (mx > 0.f) ? inv_scale(mx) : 0.f;
    if (kb == 0 && blockIdx.x == 0) a.m[t] = mx;
  }
  if (kb == 0 && blockIdx.x == 0 && a.count_out) {
    int cnt = 0;
    for (int64_t w = t; w < a.kw; w += 256) cnt += __builtin_popcount(a.omask[w]);
    cnt = wave_sum(cnt);
    if (lane == 0) s_cnt[wv] = cnt;
    __syncthreads();
    if (t == 0) *a.count_out = s_cnt[0] + s_cnt[1] + s_cnt[2] + s_cnt[3];
  }

  i32x4 acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = (i32x4){0, 0, 0, 0};

  constexpr int XCH = MB * 16 * (kSubK / 8) / 256;  // fp16 chunks of X per thread
  for (int64_t k0 = k_begin; k0 < k_end; k0 += kSubK) {
    u32x4 b[kSubK / 64];
#pragma unroll
    for (int j = 0; j < kSubK / 64; ++j) {
      const int64_t k = k0 + 64 * j + 16 * g;
      b[j] = (k < k_end) ? *(const u32x4 *)(brow + k) : (u32x4){0u, 0u, 0u, 0u};
    }
    u32x4 xv[XCH];
#pragma unroll
    for (int u = 0; u < XCH; ++u) {
      const int q = t + 256 * u;
      const int row = q / (kSubK / 8);
      const int64_t k = k0 + 8 * (q % (kSubK / 8));
      xv[u] = (u32x4){0u, 0u, 0u, 0u};
      if (row < a.M && k < k_end) xv[u] = *(const u32x4 *)(a.X + (int64_t)row * a.ldx + k);
    }
    __syncthreads();  // sinv ready; previous iteration done with sx
#pragma unroll
    for (int u = 0; u < XCH; ++u) {
      const int q = t + 256 * u;
      const int row = q / (kSubK / 8), cc = q % (kSubK / 8);
      const int64_t k = k0 + 8 * cc;
      u32x2 out = {0u, 0u};
      if (row < a.M && k < k_end) {
        const unsigned ob = (a.omask[k >> 5] >> (k & 31)) & 0xffu;
        const float inv = sinv[row];
        if (inv != 0.f) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float x = (e & 1) ? fp16_hi(xv[u][e >> 1]) : fp16_lo(xv[u][e >> 1]);
            const int qv = ((ob >> e) & 1u) ? 0 : quant_i8(x, inv);
            out[e >> 2] |= ((uint32_t)qv & 0xffu) << (8 * (e & 3));
          }
        }
      }
      *(u32x2 *)(sx + row * kXPitch + 8 * cc) = out;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kSubK / 64; ++j)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const i32x4 av = *(const i32x4 *)(sx + (mb * 16 + c16) * kXPitch + 64 * j + 16 * g);
        acc[mb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, __builtin_bit_cast(i32x4, b[j]),
                                                         acc[mb], 0, 0, 0);
      }
  }

  // partial sums: lane holds rows 4g + r of each 16-row block, column ncol
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = mb * 16 + 4 * g + r;
      if (row < a.M && ncol < a.N) a.part[((int64_t)kb * a.M + row) * a.N + ncol] = acc[mb][r];
    }
}

// Block (tile, row group of 16): 64 columns x 16 rows, 4 outputs per thread.
__global__ __launch_bounds__(256) void k_decode_epilogue(DecodeGemmArgs a) {
  __shared__ int slist[2048];                        // outlier columns of one round
  __shared__ uint16_t sxo[16 * kOutBatch];           // [row][p]
  __shared__ uint16_t swo[kOutBatch * kTileN];       // [p][col]
  __shared__ int s_total;
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int64_t n0 = (int64_t)blockIdx.x * kTileN;
  const int64_t col = n0 + lane;
  const int rbase = blockIdx.y * 16;

  float y[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = rbase + wv + 4 * i;
    y[i] = 0.f;
    if (row < a.M && col < a.N) {
      int cacc = 0;
      for (int k = 0; k < a.kb; ++k) cacc += a.part[((int64_t)k * a.M + row) * a.N + col];
      if (a.cdbg) a.cdbg[(int64_t)row * a.N + col] = cacc;
      y[i] = (float)cacc * (a.m[row] * (a.s[col] * (1.0f / 16129.0f)));
    }
  }

  // fp16 outlier terms, outlier columns in ascending order, kOutBatch at a time
  if (a.w) {
    for (int64_t w0 = 0; w0 < a.kw; w0 += 64) {
      if (wv == 0) {  // wave 0 lists the outlier columns of 64 mask words
        const uint32_t mw = (w0 + lane < a.kw) ? a.omask[w0 + lane] : 0u;
        const int cnt = __builtin_popcount(mw);
        int incl = cnt;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const int yv = __shfl_up(incl, off, 64);
          if (lane >= off) incl += yv;
        }
        int pos = incl - cnt;
        uint32_t mm = mw;
        while (mm) {
          slist[pos++] = (int)(32 * (w0 + lane) + __builtin_ctz(mm));
          mm &= mm - 1u;
        }
        if (lane == 63) s_total = incl;
      }
      __syncthreads();
      const int total = s_total;
      for (int p0 = 0; p0 < total; p0 += kOutBatch) {
        const int np = (total - p0 < kOutBatch) ? total - p0 : kOutBatch;
        {
          const int row = rbase + (t >> 4), p = t & 15;  // 16 x 16 = 256 entries
          sxo[t] = (row < a.M && p < np) ? a.X[(int64_t)row * a.ldx + slist[p0 + p]] : 0;
        }
        for (int q = t; q < kOutBatch * kTileN; q += 256) {
          const int p = q / kTileN;
          const int64_t cc = n0 + (q % kTileN);
          swo[q] = (p < np && cc < a.N) ? a.w[(int64_t)slist[p0 + p] * a.ldw + cc] : 0;
        }
        __syncthreads();
        for (int p = 0; p < np; ++p) {
          const float wval = h2f(swo[p * kTileN + lane]);
#pragma unroll
          for (int i = 0; i < 4; ++i) y[i] += h2f(sxo[(wv + 4 * i) * kOutBatch + p]) * wval;
        }
        __syncthreads();
      }
    }
  }
  if (col < a.N) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = rbase + wv + 4 * i;
      if (row < a.M) a.y[(int64_t)row * a.ldy + col] = f2h(y[i]);
    }
  }
}

template <int MB>
hipError_t launch_decode_gemm(const DecodeGemmArgs &a, int tiles, int kb, hipStream_t stream) {
  hipLaunchKernelGGL((k_decode_gemm<MB>), dim3(tiles, kb), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

DecodePlan decode_plan(int64_t M, int64_t K, int64_t N) {
  (void)M;
  DecodePlan p;
  p.tiles = (int)((N + kTileN - 1) / kTileN);
  p.det_blocks = (int)((K + kDetCols - 1) / kDetCols);
  int64_t kb = (512 + p.tiles - 1) / p.tiles;  // aim for ~512 GEMM blocks
  const int64_t kmax = (K + 255) / 256;         // at least 256 k bytes per block
  if (kb > kmax) kb = kmax;
  if (kb > 16) kb = 16;
  if (kb < 1) kb = 1;
  int64_t kc = (K + kb - 1) / kb;
  kc = (kc + 63) / 64 * 64;
  p.kc = kc;
  p.kb = (int)((K + kc - 1) / kc);
  return p;
}

hipError_t launch_decode(const DecodeDetectArgs &det, const DecodeGemmArgs &gemm,
                         const DecodePlan &plan, const GemmEvents &ev, hipStream_t stream) {
  hipLaunchKernelGGL(k_decode_detect, dim3(plan.det_blocks), dim3(256), 0, stream, det);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (ev.begin && (e = hipEventRecord((hipEvent_t)ev.begin, stream)) != hipSuccess) return e;
  const int mb = (int)((gemm.M + 15) / 16);
  switch (mb) {
    case 1: e = launch_decode_gemm<1>(gemm, plan.tiles, plan.kb, stream); break;
    case 2: e = launch_decode_gemm<2>(gemm, plan.tiles, plan.kb, stream); break;
    case 3: e = launch_decode_gemm<3>(gemm, plan.tiles, plan.kb, stream); break;
    default: e = launch_decode_gemm<4>(gemm, plan.tiles, plan.kb, stream); break;
  }
  if (e != hipSuccess) return e;
  if (ev.end && (e = hipEventRecord((hipEvent_t)ev.end, stream)) != hipSuccess) return e;
  hipLaunchKernelGGL(k_decode_epilogue, dim3(plan.tiles, (unsigned)((gemm.M + 15) / 16)),
                     dim3(256), 0, stream, gemm);
  return hipGetLastError();
}

}  // namespace llmint8
