// Large-M GEMM dispatch (tile shape choice) and the W_O^T gather kernel.
#include "gemm_core.hpp"

namespace llmint8 {

namespace {

// waves along N of a 256x256 tile (4: two waves per SIMD) and k bytes per
// stage (128; 64-byte stages with a four-deep ring measured 7-9% slower)
constexpr int kWideWavesN = 4;
constexpr int kWideStageK = 128;

// W_O^T [N x ldo] (fp16): row n holds W[idx[p], n] for p < |O|, zeros up to the
// next multiple of 64. Block b covers 64 columns of W, 64 outlier rows per
// step, transposed through LDS.
__device__ void gather_wot_block(int64_t b, const WeightSideArgs &a) {
  __shared__ __attribute__((aligned(16))) uint16_t st[64 * 72];  // [n][p], pitch 72
  const int count = *a.count;
  const int t = threadIdx.x;
  const int64_t n0 = b * 64;
  const int64_t pad = (count + 63) / 64 * 64;
  for (int64_t p0 = 0; p0 < pad; p0 += 64) {
    u32x4 v[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int q = t + 256 * u;
      const int p = q >> 3, ch = q & 7;  // 64 rows x 8 chunks of 8 fp16
      const int64_t n = n0 + ch * 8;
      const bool ok = p0 + p < count && n < a.N;
      const int64_t src = ok ? (int64_t)a.idx[p0 + p] * a.ldw + n : 0;
      const u32x4 x = *(const u32x4 *)(a.W + src);
      v[u] = ok ? x : (u32x4){0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int q = t + 256 * u;
      const int p = q >> 3, ch = q & 7;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t w = v[u][e >> 1];
        st[(ch * 8 + e) * 72 + p] = (e & 1) ? (uint16_t)(w >> 16) : (uint16_t)(w & 0xffffu);
      }
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int q = t + 256 * u;
      const int nl = q >> 3, ch = q & 7;  // 64 output rows x 8 chunks
      const int64_t n = n0 + nl;
      if (n < a.N)
        *(u32x4 *)(a.wot + n * a.ldo + p0 + ch * 8) = *(const u32x4 *)(st + nl * 72 + ch * 8);
    }
    __syncthreads();
  }
}

// The int8 outlier-weight form of W_O^T [N x ldo]: row n holds the codes
// Wq[n, idx[p]] as fp16 (exact) for p < |O|, zeros up to the next multiple of
// 64. Block b covers 64 rows of Wq; a row's codes are gathered by 4 threads.
__device__ void gather_codes_block(int64_t b, const WeightSideArgs &a) {
  const int count = *a.count;
  const int t = threadIdx.x;
  const int64_t n = b * 64 + (t >> 2);
  if (n >= a.N) return;
  const int pad = (count + 63) / 64 * 64;
  const int8_t *row = a.Wq + n * a.K;
  for (int p = t & 3; p < pad; p += 4) {
    const int q = p < count ? row[a.idx[p]] : 0;
    a.wot[n * a.ldo + p] = f2h((float)q);
  }
}

// Compacted copy Wqc of the Wq rows without the outlier columns, when the
// outlier share calls for it. Block b of nb takes rows b, b + nb, ...: each
// thread compresses 32 bytes (one mask word) into LDS, then the row goes out
// with 16-byte stores, its tail zeroed up to the 128-byte pitch.
__device__ void compact_block(int64_t b, int64_t nb, const WeightSideArgs &a, uint8_t *srow) {
  const int count = *a.count;
  if (!use_compaction(count, a.K, a.M)) return;
  const int t = threadIdx.x;
  const int64_t K = a.K;
  const int64_t kw = (K + 31) / 32;
  const int64_t kk = K - count;
  const int64_t kpad = (kk + 127) / 128 * 128;
  for (int64_t n = b; n < a.N; n += nb) {
    const int8_t *row = a.Wq + n * K;
    for (int64_t w = t; w < kw; w += 256) {
      const uint32_t v = a.omask[w];
      int64_t dst = 32 * w - a.wprefix[w];
      const int nbytes = (K - 32 * w < 32) ? (int)(K - 32 * w) : 32;
      for (int h = 0; h < nbytes; h += 16) {
        const u32x4 d = *(const u32x4 *)(row + 32 * w + h);
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          if (!((v >> (h + e)) & 1u)) {
            srow[dst] = (uint8_t)((d[e >> 2] >> (8 * (e & 3))) & 0xffu);
            ++dst;
          }
        }
      }
    }
    for (int64_t k = kk + t; k < kpad; k += 256) srow[k] = 0;
    __syncthreads();
    int8_t *out = a.wqc + n * a.ldq;
    for (int64_t c16 = t; c16 < kpad / 16; c16 += 256)
      *(u32x4 *)(out + c16 * 16) = *(const u32x4 *)(srow + c16 * 16);
    __syncthreads();
  }
}

// The weight-side preparation of a large-M call in one launch: blocks
// [0, gather_blocks) gather W_O^T, the rest compact Wq.
__global__ __launch_bounds__(256) void k_weight_side(WeightSideArgs a) {
  extern __shared__ u32x4 srow_v[];
  const int64_t b = blockIdx.x;
  if (b < a.gather_blocks) {
    if (a.W)
      gather_wot_block(b, a);
    else
      gather_codes_block(b, a);
  } else {
    compact_block(b - a.gather_blocks, gridDim.x - a.gather_blocks, a, (uint8_t *)srow_v);
  }
}

// Share of the CU slots that the tiles fill over all waves (one block per CU).
double wave_fill(int64_t M, int64_t N, int64_t bm, int64_t bn, int64_t cus) {
  const int64_t tiles = ((M + bm - 1) / bm) * ((N + bn - 1) / bn);
  const int64_t waves = (tiles + cus - 1) / cus;
  return (double)tiles / (double)(waves * cus);
}

// 256x256 tiles (8 waves) unless their last wave leaves most of the chip idle
// and 256x128 tiles fill the waves much better. A 256x128 tile moves 1.5x the
// operand bytes per MFMA and runs 4 waves; measured on the 7B, 13B and 70B
// shapes it is 3-10% slower even where its waves are 90% full against 67%,
// so it is taken as 30% slower.
int cu_count() {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    cus = 256;
  return cus;
}

bool narrow_tiles(int64_t M, int64_t N, int cus) {
  return 0.7 * wave_fill(M, N, 256, 128, cus) > wave_fill(M, N, 256, 256, cus);
}

// Columns [0, n1) of the output in whole waves of 256x256 tiles, or 0 when
// splitting does not pay. The last wave of a 256x256 launch runs
// tiles % cus blocks while the rest of the chip idles; putting the columns of
// those tiles into a second launch of 128x256 tiles (half the work each, still
// two waves per SIMD, in one wave) turns that wave into about half a wave plus
// the launch gap. (256x128 tiles with one wave per SIMD measured 0.63 of a
// full wave for the same half of the work.)
int64_t wide_columns(int64_t M, int64_t N, int cus) {
  const int64_t tm = (M + 255) / 256, tn = (N + 255) / 256;
  const int64_t tiles = tm * tn, full_waves = tiles / cus;
  if (full_waves == 0 || tiles % cus == 0) return 0;
  const int64_t tn1 = full_waves * cus / tm;  // tile columns of the full waves
  if (tn1 <= 0 || tn1 >= tn) return 0;
  const int64_t n1 = tn1 * 256;
  const int64_t tail_blocks = ((M + 127) / 128) * ((N - n1 + 255) / 256);
  return tail_blocks <= cus ? n1 : 0;
}

// The same GEMM restricted to output columns [n0, n0 + ncols).
GemmArgs column_slice(const GemmArgs &a, int64_t n0, int64_t ncols) {
  GemmArgs b = a;
  b.wq = a.wq + n0 * a.K;
  b.wqc = a.wqc ? a.wqc + n0 * a.ldq : nullptr;
  b.s = a.s + n0;
  b.wot = a.wot ? a.wot + n0 * a.ldo : nullptr;
  b.y = a.y + n0;
  b.cdbg = a.cdbg ? a.cdbg + n0 : nullptr;
  if (a.ep.bias) b.ep.bias = a.ep.bias + n0;
  if (a.ep.ycmax) b.ep.ycmax = a.ep.ycmax + n0;
  b.N = ncols;
  return b;
}

}  // namespace

hipError_t launch_weight_side(const WeightSideArgs &args, bool gather, hipStream_t stream) {
  WeightSideArgs a = args;
  a.gather_blocks = gather ? (a.N + 63) / 64 : 0;
  // compaction never applies when even |O| = K would not pay (M below ~313)
  const int64_t cblocks = use_compaction((int)a.K, a.K, a.M) ? (a.N < 1024 ? a.N : 1024) : 0;
  const int64_t blocks = a.gather_blocks + cblocks;
  if (blocks == 0) return hipSuccess;
  const size_t lds = cblocks ? (size_t)a.ldq : 0;
  hipLaunchKernelGGL(k_weight_side, dim3((unsigned)blocks), dim3(256), lds, stream, a);
  return hipGetLastError();
}

hipError_t launch_gemm_wide(const GemmArgs &a, const GemmEvents &ev, hipStream_t stream) {
  using namespace gemm_detail;
  constexpr int W = kWideWavesN, S = kWideStageK;
  if (a.fp8)
    return a.cdbg ? launch_prefill<256, 256, W, S, true, true>(a, ev, stream)
                  : launch_prefill<256, 256, W, S, false, true>(a, ev, stream);
  return a.cdbg ? launch_prefill<256, 256, W, S, true, false>(a, ev, stream)
                : launch_prefill<256, 256, W, S, false, false>(a, ev, stream);
}

hipError_t launch_gemm(const GemmArgs &args, const GemmEvents &ev, hipStream_t stream) {
  GemmArgs a = args;
  if (a.ldc == 0) a.ldc = a.N;
  const int cus = cu_count();
  if (narrow_tiles(a.M, a.N, cus)) return launch_gemm_narrow(a, ev, stream);
  const int64_t n1 = wide_columns(a.M, a.N, cus);
  if (n1 == 0) return launch_gemm_wide(a, ev, stream);
  // the begin event goes with the first launch, the end event with the second
  const hipError_t e =
      launch_gemm_wide(column_slice(a, 0, n1), GemmEvents{ev.begin, nullptr}, stream);
  if (e != hipSuccess) return e;
  return launch_gemm_tail(column_slice(a, n1, a.N - n1), GemmEvents{nullptr, ev.end}, stream);
}

}  // namespace llmint8
