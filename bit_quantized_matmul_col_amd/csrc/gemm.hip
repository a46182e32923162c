// int8 GEMM + fused epilogue of the LLM.int8() linear layer on gfx950 MFMA.
//
// C = Xq . Wq^T with int32 accumulation (the int8 x int8 -> int32 matmul of the
// "8-Bit LLM Quantization with Lightning Fabric" page, section 2.2), then
// Y = C * m[i] * s[n] / 127^2 + X_O . W_O, the 16-bit outlier product added to
// the dequantized int8 result ("LLM.int8() pitfalls" page, section 3.3;
// "LLM.int8()" walkthrough, section 2.3). Both operands of the int8 product are
// K-contiguous, so both stream into LDS with 16-byte loads.
//
// MFMA lane layouts (gfx950, checked on hardware): for v_mfma_*_32x32x32_i8 and
// v_mfma_f32_32x32x16_f16 lane l supplies row (A) / column (B) l % 32 and the
// k-group l / 32 of 16 bytes (8 fp16); the 32x32 result sits in 16 registers,
// register r of lane l holding row 8(r/4) + 4(l/32) + r%4, column l % 32. The
// 16x16x64_i8 form has lane l supply row/column l % 16, k-group l / 16, and
// result register r holding row 4(l/16) + r, column l % 16. Only the pairing
// of A and B k-groups matters for an exact integer dot product, and both
// operands use the same one.
#include "internal.hpp"

namespace llmint8 {

namespace {

constexpr int BK = 64;              // int8 k per main-loop step
constexpr int P8 = BK + 16;         // LDS row pitch (bytes) of int8 tiles
constexpr int OKC = 32;             // fp16 outlier columns per chunk
constexpr int P16 = OKC + 8;        // LDS row pitch (fp16 elements) of outlier tiles

__device__ inline u32x4 zero4() { return (u32x4){0u, 0u, 0u, 0u}; }

// Outlier product for one output tile, accumulated into fp32 MFMA registers.
// X_O [BM x 32] comes from the gathered outlier columns; W_O [32 x BN] are the
// fp16 weight rows idx[p], transposed into LDS so both operands are k-contiguous.
template <int BM, int BN, int WM, int WN>
__device__ inline void outlier_product(const GemmArgs &a, int count, int64_t m0, int64_t n0,
                                       int wm, int wn, uint16_t *sXO, uint16_t *sWO,
                                       f32x16 (&accf)[WM / 32][WN / 32]) {
  constexpr int MI = WM / 32, NI = WN / 32;
  const int t = threadIdx.x, lane = t & 63;
  for (int p0 = 0; p0 < count; p0 += OKC) {
    for (int q = t; q < BM * (OKC / 8); q += 256) {
      const int row = q / (OKC / 8), pc = q % (OKC / 8);
      const int64_t gm = m0 + row;
      const int p = p0 + pc * 8;
      u32x4 v = zero4();
      if (gm < a.M && p < count) {
        v = *(const u32x4 *)(a.xo + gm * a.ldo + p);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (p + e >= count) v[e >> 1] &= (e & 1) ? 0x0000ffffu : 0xffff0000u;
      }
      *(u32x4 *)(sXO + row * P16 + pc * 8) = v;
    }
    for (int q = t; q < OKC * (BN / 8); q += 256) {
      const int pr = q / (BN / 8), c = q % (BN / 8);
      const int p = p0 + pr;
      const int64_t n = n0 + c * 8;
      u32x4 v = zero4();
      if (p < count && n < a.N) v = *(const u32x4 *)(a.w + (int64_t)a.idx[p] * a.ldw + n);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t w = v[e >> 1];
        sWO[(c * 8 + e) * P16 + pr] = (e & 1) ? (uint16_t)(w >> 16) : (uint16_t)(w & 0xffffu);
      }
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < OKC; kk += 16) {
      f16x8 xa[MI], wb[NI];
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
        xa[mi] = *(const f16x8 *)(sXO + (wm * WM + mi * 32 + (lane & 31)) * P16 + kk +
                                  8 * (lane >> 5));
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
        wb[ni] = *(const f16x8 *)(sWO + (wn * WN + ni * 32 + (lane & 31)) * P16 + kk +
                                  8 * (lane >> 5));
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
          accf[mi][ni] =
              __builtin_amdgcn_mfma_f32_32x32x16_f16(xa[mi], wb[ni], accf[mi][ni], 0, 0, 0);
    }
    __syncthreads();
  }
}

// Tiled kernel for prefill shapes: a 256-thread block computes a BM x BN tile,
// its 4 waves a WM x WN sub-tile each from 32x32 MFMA blocks. Operand tiles
// are double-buffered in LDS; the next tile's global loads are in flight while
// the current one feeds the MFMAs.
template <int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(256) void k_gemm_tile(GemmArgs a) {
  constexpr int WGN = BN / WN;
  static_assert((BM / WM) * (BN / WN) == 4, "four waves per block");
  constexpr int MI = WM / 32, NI = WN / 32;
  constexpr int CPR = BK / 16;                // 16-byte chunks per tile row
  constexpr int A_CH = BM * CPR / 256;
  constexpr int B_CH = BN * CPR / 256;
  extern __shared__ u32x4 smem_v[];
  uint8_t *smem = (uint8_t *)smem_v;
  uint8_t *sA = smem;
  uint8_t *sB = smem + 2 * BM * P8;

  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int wm = wv / WGN, wn = wv % WGN;
  const int64_t tiles_m = (a.M + BM - 1) / BM;
  const int64_t m0 = (int64_t)(blockIdx.x % tiles_m) * BM;
  const int64_t n0 = (int64_t)(blockIdx.x / tiles_m) * BN;

  const int count = *a.count;
  const bool compact = use_compaction(count, a.K, a.M);
  const int8_t *B = compact ? a.wqc : a.wq;
  const int64_t K = a.K;
  const int64_t Kl = compact ? K - count : K;

  i32x16 acc[MI][NI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = (i32x16){};

  u32x4 ra[A_CH], rb[B_CH];
  auto gload = [&](int64_t k0) {
#pragma unroll
    for (int u = 0; u < A_CH; ++u) {
      const int q = t + 256 * u;
      const int64_t gm = m0 + q / CPR, gk = k0 + (q % CPR) * 16;
      ra[u] = (gm < a.M && gk < Kl) ? *(const u32x4 *)(a.xq + gm * K + gk) : zero4();
    }
#pragma unroll
    for (int u = 0; u < B_CH; ++u) {
      const int q = t + 256 * u;
      const int64_t gn = n0 + q / CPR, gk = k0 + (q % CPR) * 16;
      rb[u] = (gn < a.N && gk < Kl) ? *(const u32x4 *)(B + gn * K + gk) : zero4();
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int u = 0; u < A_CH; ++u) {
      const int q = t + 256 * u;
      *(u32x4 *)(sA + (buf * BM + q / CPR) * P8 + (q % CPR) * 16) = ra[u];
    }
#pragma unroll
    for (int u = 0; u < B_CH; ++u) {
      const int q = t + 256 * u;
      *(u32x4 *)(sB + (buf * BN + q / CPR) * P8 + (q % CPR) * 16) = rb[u];
    }
  };

  const int64_t nk = (Kl + BK - 1) / BK;
  if (nk > 0) {
    gload(0);
    sstore(0);
  }
  __syncthreads();
  for (int64_t it = 0; it < nk; ++it) {
    const int buf = (int)(it & 1);
    if (it + 1 < nk) gload((it + 1) * BK);
#pragma unroll
    for (int kk = 0; kk < BK; kk += 32) {
      i32x4 af[MI], bf[NI];
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
        af[mi] = *(const i32x4 *)(sA + (buf * BM + wm * WM + mi * 32 + (lane & 31)) * P8 + kk +
                                  16 * (lane >> 5));
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
        bf[ni] = *(const i32x4 *)(sB + (buf * BN + wn * WN + ni * 32 + (lane & 31)) * P8 + kk +
                                  16 * (lane >> 5));
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
          acc[mi][ni] =
              __builtin_amdgcn_mfma_i32_32x32x32_i8(af[mi], bf[ni], acc[mi][ni], 0, 0, 0);
    }
    if (it + 1 < nk) sstore(buf ^ 1);
    __syncthreads();
  }

  // Dequantize: C * m[i] * s[n] / 127^2 (exact int32 kept for the debug copy).
  f32x16 accf[MI][NI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
      const int64_t col = n0 + wn * WN + ni * 32 + (lane & 31);
      const float sc = (col < a.N) ? a.s[col] * (1.0f / 16129.0f) : 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + wm * WM + mi * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const float mr = (row < a.M) ? a.m[row] : 0.f;
        if (a.cdbg && row < a.M && col < a.N) a.cdbg[row * a.N + col] = acc[mi][ni][r];
        accf[mi][ni][r] = (float)acc[mi][ni][r] * (mr * sc);
      }
    }

  if (count > 0 && a.w) {
    uint16_t *sXO = (uint16_t *)smem;
    uint16_t *sWO = sXO + BM * P16;
    outlier_product<BM, BN, WM, WN>(a, count, m0, n0, wm, wn, sXO, sWO, accf);
  }

#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
      const int64_t col = n0 + wn * WN + ni * 32 + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + wm * WM + mi * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (row < a.M && col < a.N) a.y[row * a.ldy + col] = f2h(accf[mi][ni][r]);
      }
    }
}

}  // namespace

hipError_t launch_gemm(const GemmArgs &a, hipStream_t stream) {
  constexpr int BM = 128, BN = 128;
  const int64_t tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  const size_t lds = 2 * (BM + BN) * P8;
  hipLaunchKernelGGL((k_gemm_tile<BM, BN, 64, 64>), dim3((unsigned)tiles), dim3(256), lds, stream,
                     a);
  return hipGetLastError();
}

}  // namespace llmint8
