// The traditional per-tensor int8 linear layer, the comparison the pitfalls
// page draws against LLM.int8() (sections 1 and 2: one scale, 127 / max|x|,
// for the whole matrix; no outlier decomposition). It reuses the column
// quantizer and the large-M GEMM with broadcast scales: the GEMM's epilogue
// multiplies C by m[i] * s[n] / 127^2, so m[] filled with max|X| and s[] with
// max|W| give Y = C * sx * sw / 127^2.
#include "internal.hpp"

namespace llmint8 {

namespace {

// Partial max of |x| over X: 16-byte chunks, grid-strided, one value per block.
__global__ __launch_bounds__(256) void k_absmax_partial(const uint16_t *__restrict__ X, int64_t M,
                                                        int64_t K, int64_t ldx,
                                                        float *__restrict__ partial) {
  __shared__ float red[4];
  const int t = threadIdx.x;
  const int64_t chunks = K / 8;  // K is a multiple of 16
  const int64_t total = M * chunks;
  float mx[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int64_t q = (int64_t)blockIdx.x * 256 + t; q < total; q += (int64_t)gridDim.x * 256) {
    const int64_t r = q / chunks, c = q % chunks;
    absmax8(*(const u32x4 *)(X + r * ldx + 8 * c), mx);
  }
  float v = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) v = __builtin_fmaxf(v, mx[e]);
  v = wave_max(v);
  if ((t & 63) == 0) red[t >> 6] = v;
  __syncthreads();
  if (t == 0)
    partial[blockIdx.x] = __builtin_fmaxf(__builtin_fmaxf(red[0], red[1]),
                                          __builtin_fmaxf(red[2], red[3]));
}

// max over n values of src, written to *out; dst[0 .. nd) = that max (dst may
// be src); fill[0 .. nf) = *fill_from when fill is set; *zero = 0 when set.
__global__ __launch_bounds__(1024) void k_absmax_finish(const float *src, int64_t n,
                                                        float *out, float *dst, int64_t nd,
                                                        float *fill, int64_t nf,
                                                        const float *fill_from, int32_t *zero) {
  __shared__ float red[16];
  const int t = threadIdx.x;
  float v = 0.f;
  for (int64_t i = t; i < n; i += 1024) v = __builtin_fmaxf(v, src[i]);
  v = wave_max(v);
  if ((t & 63) == 0) red[t >> 6] = v;
  __syncthreads();
  float mx = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) mx = __builtin_fmaxf(mx, red[i]);
  __syncthreads();  // every thread has read src before dst (possibly src) is written
  if (t == 0 && out) *out = mx;
  for (int64_t i = t; i < nd; i += 1024) dst[i] = mx;
  if (fill) {
    const float f = *fill_from;
    for (int64_t i = t; i < nf; i += 1024) fill[i] = f;
  }
  if (zero && t == 0) *zero = 0;
}

// Codes of row blockIdx.x of X with the one scale fl32(127 / sx) (zero for
// sx = 0), zero from column K up to the row pitch ldq.
__global__ __launch_bounds__(256) void k_quant_tensor(const uint16_t *__restrict__ X, int64_t K,
                                                      int64_t ldx, const float *__restrict__ sx,
                                                      int8_t *__restrict__ Xq, int64_t ldq) {
  const float a = *sx;
  const float inv = a > 0.f ? inv_scale(a) : 0.f;
  const int64_t r = blockIdx.x;
  const uint16_t *row = X + r * ldx;
  int8_t *out = Xq + r * ldq;
  for (int64_t c = threadIdx.x; c < ldq / 8; c += 256) {
    u32x2 q = {0u, 0u};
    if (8 * c < K) {
      const u32x4 v = *(const u32x4 *)(row + 8 * c);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = (e & 1) ? fp16_hi(v[e >> 1]) : fp16_lo(v[e >> 1]);
        q[e >> 2] |= ((uint32_t)quant_i8(x, inv) & 0xffu) << (8 * (e & 3));
      }
    }
    *(u32x2 *)(out + 8 * c) = q;
  }
}

}  // namespace

hipError_t launch_quantize_tensorwise(const uint16_t *W, int64_t K, int64_t N, int64_t ldw,
                                      int8_t *Wq, float *w_absmax, float *scratch,
                                      hipStream_t stream) {
  // per-column maxima, their max, then the column quantizer with that max
  // broadcast to every column
  hipError_t e = launch_colwise_absmax(W, K, N, ldw, scratch, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_absmax_finish, dim3(1), dim3(1024), 0, stream, (const float *)scratch, N,
                     w_absmax, scratch, N, (float *)nullptr, (int64_t)0, (const float *)nullptr,
                     (int32_t *)nullptr);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return launch_colwise_quant<CodecI8>(W, K, N, ldw, scratch, (uint8_t *)Wq, stream);
}

hipError_t launch_linear_tensorwise(const uint16_t *X, int64_t M, int64_t K, int64_t ldx,
                                    const int8_t *Wq, const float *w_absmax, int64_t N,
                                    uint16_t *Y, int64_t ldy, const uint16_t *bias,
                                    float *x_absmax, int32_t *cdbg, const TensorwiseLayout &L,
                                    const GemmEvents &ev, hipStream_t stream) {
  int64_t blocks = (M * (K / 8) + 255) / 256;
  if (blocks > kTensorAbsBlocks) blocks = kTensorAbsBlocks;
  hipLaunchKernelGGL(k_absmax_partial, dim3((unsigned)blocks), dim3(256), 0, stream, X, M, K, ldx,
                     L.partial);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // m[] = max|X| for every row, s[] = max|W| for every column, outlier count 0
  hipLaunchKernelGGL(k_absmax_finish, dim3(1), dim3(1024), 0, stream, (const float *)L.partial,
                     blocks, x_absmax, L.m, M, L.s, N, w_absmax, L.count);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(k_quant_tensor, dim3((unsigned)M), dim3(256), 0, stream, X, K, ldx,
                     (const float *)L.m, L.xq, L.ldq);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const EpilogueOpts ep{0, bias, nullptr};
  const GemmArgs g{L.xq, Wq, nullptr, L.m, L.s, nullptr, nullptr, nullptr, L.count, Y, cdbg,
                   M, N, K, L.ldq, 64, 0, ldy, ep};
  return launch_gemm(g, ev, stream);
}

}  // namespace llmint8
