// Vector-wise int8 quantization kernels for gfx950 (all HBM-bound).
//
// The quantizer is the symmetric absmax one of the "LLM.int8() pitfalls" page
// (codearts), section 1: q = round(x * 127 / absmax), with the round-then-clamp
// order and the [-127, 127] range of the INT8-to-QLoRA page (cnnetsun),
// sections 3.2 and 3.3. Vector-wise scales are per row of X and per column
// (output channel) of W ("LLM.int8()" walkthrough, 2kiu.com, section 2.1); the
// row scale of X ignores the outlier columns, which go the 16-bit way (same
// page, section 2.3).
#include "internal.hpp"

namespace llmint8 {

namespace {

// Reduction of one float per thread to a block-wide max (256 threads).
__device__ inline float block_max256(float v, float *red) {
  v = wave_max(v);
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  if (lane == 0) red[wv] = v;
  __syncthreads();
  float r = __builtin_fmaxf(__builtin_fmaxf(red[0], red[1]), __builtin_fmaxf(red[2], red[3]));
  __syncthreads();
  return r;
}

// Outlier bits of the 8 columns of chunk ch (columns 8ch .. 8ch+7).
__device__ inline unsigned chunk_bits(const uint32_t *mask, int64_t ch) {
  return (mask[ch >> 2] >> ((ch & 3) * 8)) & 0xffu;
}

// Bits of the outlier list entries p0 + t, p0 + t + 256, ... below count set
// in the LDS bitmask (256 threads). Four entries per thread are loaded before
// any is used, so a long list costs few round trips. The loads go through a
// buffer resource over the K-entry list (32-bit offsets, fewer registers;
// entries past K read as 0 and are not used).
__device__ inline void list_to_mask(const int32_t *__restrict__ idx, int count, int64_t K,
                                    int p0, uint32_t *smask) {
  constexpr int kBatch = 4;
  const int t = threadIdx.x;
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc((void *)idx, (short)0, (int)(K * 4), 0x00020000);
  for (int b = p0; b < count; b += 256 * kBatch) {
    int k[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u)
      k[u] = (int)__builtin_amdgcn_raw_buffer_load_b32(rs, 4 * (b + t + 256 * u), 0, 0);
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int p = b + t + 256 * u;
      if (p < count && k[u] >= 0 && k[u] < K) atomicOr(&smask[k[u] >> 5], 1u << (k[u] & 31));
    }
  }
}

// Codes of the 8 fp16 of a chunk, outlier columns (and a zero row) zeroed,
// packed little-endian.
template <class Codec>
__device__ inline u32x2 quant_chunk(const u32x4 &v, unsigned obits, float inv, bool zero_row) {
  float t[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t w = v[e >> 1];
    t[e] = ((e & 1) ? fp16_hi(w) : fp16_lo(w)) * inv;
  }
  u32x2 out = {Codec::code4(t), Codec::code4(t + 4)};
  const unsigned drop = zero_row ? 0xffu : obits;
#pragma unroll
  for (int e = 0; e < 8; ++e)
    if ((drop >> e) & 1u) out[e >> 2] &= ~(0xffu << (8 * (e & 3)));
  return out;
}

// Public row quantization: one block per row; the outlier set is given as an
// index list, turned into an LDS bitmask first.
template <class Codec>
__global__ __launch_bounds__(256) void k_rowquant_idx(const uint16_t *__restrict__ X, int64_t K,
                                                      int64_t ldx, const int32_t *__restrict__ idx,
                                                      const int32_t *__restrict__ count_ptr,
                                                      uint8_t *__restrict__ Xq,
                                                      float *__restrict__ m) {
  extern __shared__ uint32_t smask[];
  __shared__ float red[4];
  const int64_t i = blockIdx.x;
  const int t = threadIdx.x;
  const int64_t kw = (K + 31) / 32;
  for (int64_t w = t; w < kw; w += 256) smask[w] = 0u;
  __syncthreads();
  int count = count_ptr ? *count_ptr : 0;
  if (count > K) count = (int)K;
  list_to_mask(idx, count, K, 0, smask);
  __syncthreads();

  const uint16_t *row = X + i * ldx;
  const int64_t nch = K / 8;
  float mx = 0.f;
  for (int64_t ch = t; ch < nch; ch += 256) {
    const u32x4 v = *(const u32x4 *)(row + ch * 8);
    const unsigned ob = chunk_bits(smask, ch);
    float c8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    absmax8(v, c8);
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (!((ob >> e) & 1u)) mx = __builtin_fmaxf(mx, c8[e]);
  }
  mx = block_max256(mx, red);
  if (t == 0) m[i] = mx;
  const bool zero_row = !(mx > 0.f);
  const float inv = zero_row ? 0.f : inv_scale_of<Codec>(mx);
  uint8_t *qrow = Xq + i * K;
  for (int64_t ch = t; ch < nch; ch += 256) {
    const u32x4 v = *(const u32x4 *)(row + ch * 8);
    *(u32x2 *)(qrow + ch * 8) = quant_chunk<Codec>(v, chunk_bits(smask, ch), inv, zero_row);
  }
}

// Public row quantization for K <= 256 * 8 * CPT (CPT 16-byte chunks of a row
// per thread): block b takes rows R b .. R b + R - 1. A wave's loads complete
// in issue order, so the outlier count and the first kIdxAhead entries of the
// list (read whatever the count, from inside the K-entry list) go out first,
// then the row chunks of all R rows (rows past M re-read row M - 1, chunks
// past K read chunk 0; both are dropped): the LDS bitmask is built while the
// rows are in flight, and only list entries past kIdxAhead wait for them. The
// rows stay in registers between their absmax and their codes; R > 1 builds
// the bitmask once for R rows.
constexpr int kRowChunksMax = 4;
constexpr int kIdxAhead = 2;  // list entries per thread loaded ahead of the rows
template <class Codec, int R, int CPT>
__global__ __launch_bounds__(256) void k_rowquant_rows(const uint16_t *__restrict__ X, int64_t M,
                                                       int64_t K, int64_t ldx,
                                                       const int32_t *__restrict__ idx,
                                                       const int32_t *__restrict__ count_ptr,
                                                       uint8_t *__restrict__ Xq,
                                                       float *__restrict__ m) {
  extern __shared__ uint32_t smask[];
  __shared__ float red[R][4];
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int64_t row0 = (int64_t)blockIdx.x * R;
  const int64_t nch = K / 8;
  // every load goes out unconditionally from a valid address (a load under a
  // branch is waited for at once): without a list, X's first bytes stand in
  const bool has_list = idx != nullptr && count_ptr != nullptr;
  const int32_t *cp = has_list ? count_ptr : (const int32_t *)X;
  const int32_t *ip = has_list ? idx : (const int32_t *)X;
  const int count_word = *cp;
  int ahead[kIdxAhead];
#pragma unroll
  for (int u = 0; u < kIdxAhead; ++u) {
    const int64_t p = t + 256 * u;
    ahead[u] = ip[(has_list && p < K) ? p : 0];
  }
  __builtin_amdgcn_sched_barrier(0);
  u32x4 v[R][CPT];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t row = (row0 + r < M) ? row0 + r : M - 1;
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int64_t ch = t + 256 * j;
      v[r][j] = *(const u32x4 *)(X + row * ldx + (ch < nch ? ch : 0) * 8);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  const int64_t kw = (K + 31) / 32;
  for (int64_t w = t; w < kw; w += 256) smask[w] = 0u;
  __syncthreads();
  const int count_raw = has_list ? count_word : 0;
  const int count = count_raw > K ? (int)K : count_raw;
#pragma unroll
  for (int u = 0; u < kIdxAhead; ++u) {
    const int p = t + 256 * u, k = ahead[u];
    if (p < count && k >= 0 && k < K) atomicOr(&smask[k >> 5], 1u << (k & 31));
  }
  list_to_mask(idx, count, K, 256 * kIdxAhead, smask);
  __syncthreads();

  unsigned ob[CPT];
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    const int64_t ch = t + 256 * j;
    ob[j] = ch < nch ? chunk_bits(smask, ch) : 0xffu;  // absent chunks count as all outliers
  }
  float mx[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    mx[r] = 0.f;
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      float c8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      absmax8(v[r][j], c8);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (!((ob[j] >> e) & 1u)) mx[r] = __builtin_fmaxf(mx[r], c8[e]);
    }
    mx[r] = wave_max(mx[r]);
    if (lane == 0) red[r][wv] = mx[r];
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t row = row0 + r;
    if (row >= M) break;
    const float rm = __builtin_fmaxf(__builtin_fmaxf(red[r][0], red[r][1]),
                                     __builtin_fmaxf(red[r][2], red[r][3]));
    if (t == 0) m[row] = rm;
    const bool zero_row = !(rm > 0.f);
    const float inv = zero_row ? 0.f : inv_scale_of<Codec>(rm);
    uint8_t *qrow = Xq + row * K;
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int64_t ch = t + 256 * j;
      if (ch < nch) *(u32x2 *)(qrow + ch * 8) = quant_chunk<Codec>(v[r][j], ob[j], inv, zero_row);
    }
  }
}

// Row quantization inside the layer, row i (one block). Besides Xq and m it
// gathers the row's outlier entries into xo (position = rank of the column in
// the ascending outlier list) and, in compaction mode, writes the kept codes
// contiguously (staged in LDS so the global stores stay 16-byte wide). Rows of
// Xq (pitch ldq) are zero past their last column up to the next multiple of
// 128 bytes and rows of xo (pitch ldo) from |O| up to the next multiple of 64,
// so the GEMM can run whole 128-byte k stages.
template <class Codec>
__device__ void rowquant_row(int64_t i, const RowQuantArgs &a, uint8_t *srow) {
  __shared__ float red[4];
  const uint16_t *X = a.X;
  const int64_t M = a.M, K = a.K, ldx = a.ldx, ldq = a.ldq, ldo = a.ldo;
  const uint32_t *omask = a.omask;
  const int32_t *wprefix = a.wprefix;
  const int t = threadIdx.x;
  const int count = *a.count;
  const bool compact = use_compaction(count, K, M);
  uint8_t *Xq = a.Xq;
  float *m = a.m;
  uint16_t *xo = a.xo;

  const uint16_t *row = X + i * ldx;
  const int64_t nch = K / 8;
  float mx = 0.f;
  for (int64_t ch = t; ch < nch; ch += 256) {
    const u32x4 v = *(const u32x4 *)(row + ch * 8);
    const unsigned ob = chunk_bits(omask, ch);
    float c8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    absmax8(v, c8);
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (!((ob >> e) & 1u)) mx = __builtin_fmaxf(mx, c8[e]);
  }
  mx = block_max256(mx, red);
  if (t == 0) m[i] = mx;
  const bool zero_row = !(mx > 0.f);
  const float inv = zero_row ? 0.f : inv_scale_of<Codec>(mx);
  uint8_t *qrow = Xq + i * ldq;
  uint16_t *orow = xo + i * ldo;
  const int64_t opad = (count + 63) / 64 * 64;
  for (int64_t p = count + t; p < opad; p += 256) orow[p] = 0;

  for (int64_t ch = t; ch < nch; ch += 256) {
    const u32x4 v = *(const u32x4 *)(row + ch * 8);
    const unsigned ob = chunk_bits(omask, ch);
    const u32x2 q = quant_chunk<Codec>(v, ob, inv, zero_row);
    // rank of column 8ch in the outlier list
    const int64_t wd = ch >> 2;
    const int sh = (int)(ch & 3) * 8;
    int before = wprefix[wd] + __builtin_popcount(sh ? (omask[wd] & ((1u << sh) - 1u)) : 0u);
    if (!compact) *(u32x2 *)(qrow + ch * 8) = q;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int64_t k = ch * 8 + e;
      if ((ob >> e) & 1u) {
        const uint32_t w = v[e >> 1];
        orow[before] = (e & 1) ? (uint16_t)(w >> 16) : (uint16_t)(w & 0xffffu);
        ++before;
      } else if (compact) {
        srow[k - before] = (uint8_t)((q[e >> 2] >> (8 * (e & 3))) & 0xffu);
      }
    }
  }
  if (compact) {
    const int64_t kk = K - count;
    const int64_t kpad = (kk + 127) / 128 * 128;
    for (int64_t k = kk + t; k < kpad; k += 256) srow[k] = 0;
    __syncthreads();
    for (int64_t c16 = t; c16 < kpad / 16; c16 += 256)
      *(u32x4 *)(qrow + c16 * 16) = *(const u32x4 *)(srow + c16 * 16);
  } else {
    for (int64_t c16 = K / 16 + t; c16 < ldq / 16; c16 += 256)
      *(u32x4 *)(qrow + c16 * 16) = (u32x4){0u, 0u, 0u, 0u};
  }
}

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

// The preparation of a large-M call after detection, in one launch: the first
// blocks compact Wq, the next gather_blocks gather W_O^T, the last M quantize
// the rows of X (the block counts are fixed by the host; the work the
// compaction blocks find depends on the outlier count on the device). Blocks
// start roughly in index order, so the compaction blocks, each of which walks
// several rows of Wq one after another, and the gathers, each a chain of
// dependent loads, begin first and overlap the row blocks instead of running
// after them.
template <class Codec>
__global__ __launch_bounds__(256) void k_layer_prep(RowQuantArgs r, WeightSideArgs w) {
  extern __shared__ u32x4 srow_v[];
  uint8_t *srow = (uint8_t *)srow_v;
  const int64_t b = blockIdx.x;
  const int64_t nc = (int64_t)gridDim.x - r.M - w.gather_blocks;  // compaction blocks
  if (b < nc) {
    compact_block(b, nc, w, srow);
  } else if (b < nc + w.gather_blocks) {
    if (w.W)
      gather_wot_block(b - nc, w);
    else
      gather_codes_block(b - nc, w);
  } else {
    rowquant_row<Codec>(b - nc - w.gather_blocks, r, srow);
  }
}

// Column absmax of W [K x N]: a block owns 512 columns of a row chunk, like the
// detection pass; maxima are merged with an integer atomic max on the fp32 bit
// patterns (order-independent for non-negative values, so deterministic).
__global__ __launch_bounds__(256) void k_colabsmax(const uint16_t *__restrict__ W, int64_t K,
                                                   int64_t N, int64_t ldw, int rows_per_chunk,
                                                   unsigned *__restrict__ sbits) {
  const int t = threadIdx.x;
  const int c = t & 63, rp = t >> 6;
  const int64_t col = (int64_t)blockIdx.x * 512 + (int64_t)c * 8;
  const int64_t r0 = (int64_t)blockIdx.y * rows_per_chunk;
  const int64_t r1 = (r0 + rows_per_chunk < K) ? r0 + rows_per_chunk : K;
  float mx[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (col < N) {
    const uint16_t *p = W + col;
    int64_t r = r0 + rp;
    for (; r + 12 < r1; r += 16) {
      u32x4 v0 = *(const u32x4 *)(p + r * ldw);
      u32x4 v1 = *(const u32x4 *)(p + (r + 4) * ldw);
      u32x4 v2 = *(const u32x4 *)(p + (r + 8) * ldw);
      u32x4 v3 = *(const u32x4 *)(p + (r + 12) * ldw);
      absmax8(v0, mx);
      absmax8(v1, mx);
      absmax8(v2, mx);
      absmax8(v3, mx);
    }
    for (; r < r1; r += 4) absmax8(*(const u32x4 *)(p + r * ldw), mx);
  }
  __shared__ float sm[4][512];
#pragma unroll
  for (int e = 0; e < 8; ++e) sm[rp][c * 8 + e] = mx[e];
  __syncthreads();
  for (int j = t; j < 512; j += 256) {
    const int64_t n = (int64_t)blockIdx.x * 512 + j;
    if (n < N) {
      const float v = __builtin_fmaxf(__builtin_fmaxf(sm[0][j], sm[1][j]),
                                      __builtin_fmaxf(sm[2][j], sm[3][j]));
      atomicMax(&sbits[n], __builtin_bit_cast(unsigned, v));
    }
  }
}

__global__ void k_fill_u32(unsigned *__restrict__ p, int64_t n, unsigned v) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// Quantize and transpose a 128 (k) x 64 (n) tile of W into Wq [N x K]: read
// 128-byte row segments of W, transpose the int8 codes through LDS, write
// 128-byte segments of Wq rows.
template <class Codec>
__global__ __launch_bounds__(256) void k_colquant(const uint16_t *__restrict__ W, int64_t K,
                                                  int64_t N, int64_t ldw,
                                                  const float *__restrict__ s,
                                                  uint8_t *__restrict__ Wq) {
  constexpr int TK = 128, TN = 64, PITCH = TK + 16;
  __shared__ __attribute__((aligned(16))) uint8_t st[TN * PITCH];
  __shared__ float sinv[TN];
  __shared__ uint8_t szero[TN];
  const int t = threadIdx.x;
  const int64_t k0 = (int64_t)blockIdx.x * TK;
  const int64_t n0 = (int64_t)blockIdx.y * TN;
  if (t < TN) {
    const int64_t n = n0 + t;
    const float a = (n < N) ? s[n] : 0.f;
    szero[t] = !(a > 0.f);
    sinv[t] = (a > 0.f) ? inv_scale_of<Codec>(a) : 0.f;
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int q = t + 256 * u;
    const int r = q >> 3, ch = q & 7;
    const int64_t k = k0 + r, n = n0 + ch * 8;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (k < K && n < N) v = *(const u32x4 *)(W + k * ldw + n);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int nl = ch * 8 + e;
      const uint32_t w = v[e >> 1];
      const float x = (e & 1) ? fp16_hi(w) : fp16_lo(w);
      const uint32_t code = szero[nl] ? 0u : Codec::code(x * sinv[nl]);
      st[nl * PITCH + r] = (uint8_t)code;
    }
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int q = t + 256 * u;
    const int nl = q >> 3, ch = q & 7;
    const int64_t n = n0 + nl, k = k0 + ch * 16;
    if (n < N && k < K) *(u32x4 *)(Wq + n * K + k) = *(const u32x4 *)(st + nl * PITCH + ch * 16);
  }
}

// Column absmax and codes of W [K x N] with one read of W, for K <= 512 * RPT.
// A block owns a stripe of SC columns (8 or 16: 16 or 32 bytes of every row)
// and holds all of it in registers: thread (rp, c) keeps rows
// RPT*rp .. RPT*rp + RPT - 1 of the stripe's 8-column chunk c. The block
// reduces the stripe's column maxima, codes the values it holds, stages them
// as the stripe's SC rows of Wq [N x K] in LDS and writes those rows whole.
// Two blocks fit on a CU (at most 128 registers per thread and 66 KB of LDS
// each), so one block's loads run while the other codes and writes. Stripes
// are dealt to the XCDs in contiguous runs (blocks go to the 8 XCDs in turn),
// so the stripes that share a 128-byte line of W run on one XCD close together
// in time and the line is fetched from HBM once. Column maxima are the same
// fmax reduction as the two-pass kernels, so the results are bit-identical.
constexpr int kStripeRowPhases = 512;
constexpr int kStripeMaxK = 8192;

template <class Codec, int SC, int RPT>
__global__ __launch_bounds__(kStripeRowPhases * SC / 8) void k_colwise_stripe(
    const uint16_t *__restrict__ W, int64_t K, int64_t N, int64_t ldw, float *__restrict__ s,
    uint8_t *__restrict__ Wq, int64_t stripes, int64_t kp) {
  constexpr int H = SC / 8;                         // 16-byte chunks per row
  constexpr int T = kStripeRowPhases * H;           // threads
  extern __shared__ __attribute__((aligned(16))) uint8_t scode[];  // [SC][kp] codes
  __shared__ float sred[T / 64][SC];
  __shared__ float sinv[SC];
  __shared__ uint8_t szero[SC];
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int c = t % H, rp = t / H;

  // stripe of this block: XCD x = blockIdx.x % 8 takes a contiguous run
  const int64_t bid = blockIdx.x;
  const int64_t x = bid % 8, q = stripes / 8, rem = stripes % 8;
  const int64_t n0 = (x * q + (x < rem ? x : rem) + bid / 8) * SC;
  const int64_t nc = n0 + 8 * c;
  // K is a multiple of 16, so a thread's RPT rows are all inside K or all past it
  const bool ok = nc < N && (int64_t)RPT * rp < K;

  // every row load issued up front; a thread past K or N reads rows 0.. of
  // column 0 instead (a valid address) and its values are dropped
  u32x4 v[RPT];
  {
    const uint16_t *p = W + (ok ? (int64_t)RPT * rp * ldw + nc : 0);
#pragma unroll
    for (int j = 0; j < RPT; ++j) v[j] = *(const u32x4 *)(p + j * ldw);
  }
  float mx[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < RPT; ++j) absmax8(v[j], mx);
#pragma unroll
  for (int e = 0; e < 8; ++e) mx[e] = ok ? mx[e] : 0.f;
  // lanes with the same chunk c hold the same 8 columns
#pragma unroll
  for (int e = 0; e < 8; ++e) {
#pragma unroll
    for (int off = H; off < 64; off <<= 1)
      mx[e] = __builtin_fmaxf(mx[e], __shfl_xor(mx[e], off, 64));
  }
  if (lane < H) {
#pragma unroll
    for (int e = 0; e < 8; ++e) sred[wv][8 * lane + e] = mx[e];
  }
  __syncthreads();
  if (t < SC) {
    float a = 0.f;
#pragma unroll
    for (int w = 0; w < T / 64; ++w) a = __builtin_fmaxf(a, sred[w][t]);
    if (n0 + t < N) s[n0 + t] = a;
    szero[t] = !(a > 0.f);
    sinv[t] = (a > 0.f) ? inv_scale_of<Codec>(a) : 0.f;
  }
  __syncthreads();

  // codes, column by column: the RPT codes of one column are consecutive k
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int nl = 8 * c + e;
    const float si = sinv[nl];
    // a zero column codes to 0 whatever it holds (NaN included)
    const uint32_t keep = szero[nl] ? 0u : 0xffu;
    uint32_t wd[(RPT + 3) / 4];
#pragma unroll
    for (int i = 0; i < (RPT + 3) / 4; ++i) wd[i] = 0u;
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
      const uint32_t w = v[j][e >> 1];
      const float xv = (e & 1) ? fp16_hi(w) : fp16_lo(w);
      wd[j >> 2] |= (Codec::code(xv * si) & keep) << (8 * (j & 3));
    }
    uint8_t *dst = scode + (int64_t)nl * kp + (int64_t)RPT * rp;
    if (ok) {
      if constexpr (RPT == 16)
        *(u32x4 *)dst = u32x4{wd[0], wd[1], wd[2], wd[3]};
      else if constexpr (RPT == 8)
        *(uint2 *)dst = make_uint2(wd[0], wd[1]);
      else if constexpr (RPT == 4)
        *(uint32_t *)dst = wd[0];
      else
        *(uint16_t *)dst = (uint16_t)wd[0];
    }
  }
  __syncthreads();

  // the stripe's rows of Wq, 16 bytes per thread and step
  const int cpr = (int)(K / 16);  // at most 512
  const int rows = (N - n0 < SC) ? (int)(N - n0) : SC;
  uint8_t *dst = Wq + n0 * K;
  for (int qc = t; qc < rows * cpr; qc += T) {
    const int nl = qc / cpr, kc = qc - nl * cpr;
    *(u32x4 *)(dst + (int64_t)nl * K + 16 * kc) = *(const u32x4 *)(scode + nl * (int)kp + 16 * kc);
  }
}

}  // namespace

template <class Codec>
hipError_t launch_rowquant_idx(const uint16_t *X, int64_t M, int64_t K, int64_t ldx,
                               const int32_t *idx, const int32_t *count, uint8_t *Xq, float *m,
                               hipStream_t stream) {
  const size_t lds = (size_t)((K + 31) / 32) * sizeof(uint32_t);
  // 16-byte chunks of a row per thread. The register kernel takes rows that
  // split evenly over the 256 threads: with a ragged split (K = 5120) the
  // threads past the row's end issue a duplicate load each, and the kernel
  // measured slower than reading the row twice.
  const int64_t cpt = (K / 8 + 255) / 256;
  if (cpt <= kRowChunksMax && (K / 8) % 256 == 0) {
    // four rows per block at M >= 8192: the bitmask, built once per block from
    // the outlier list, is then shared by four rows
    const bool four = M >= 8192;
    const dim3 grid((unsigned)(four ? (M + 3) / 4 : M));
    switch ((int)cpt * 2 + (four ? 1 : 0)) {
#define LLMINT8_ROWS(C, F)                                                                      \
  case C * 2 + F:                                                                               \
    hipLaunchKernelGGL((k_rowquant_rows<Codec, F ? 4 : 1, C>), grid, dim3(256), lds, stream, X, \
                       M, K, ldx, idx, count, Xq, m);                                           \
    break;
      LLMINT8_ROWS(1, 0) LLMINT8_ROWS(1, 1) LLMINT8_ROWS(2, 0) LLMINT8_ROWS(2, 1)
      LLMINT8_ROWS(3, 0) LLMINT8_ROWS(3, 1) LLMINT8_ROWS(4, 0) LLMINT8_ROWS(4, 1)
#undef LLMINT8_ROWS
    }
  } else {
    hipLaunchKernelGGL(k_rowquant_idx<Codec>, dim3((unsigned)M), dim3(256), lds, stream, X, K,
                       ldx, idx, count, Xq, m);
  }
  return hipGetLastError();
}
template hipError_t launch_rowquant_idx<CodecI8>(const uint16_t *, int64_t, int64_t, int64_t,
                                                 const int32_t *, const int32_t *, uint8_t *,
                                                 float *, hipStream_t);
template hipError_t launch_rowquant_idx<CodecE4M3>(const uint16_t *, int64_t, int64_t, int64_t,
                                                   const int32_t *, const int32_t *, uint8_t *,
                                                   float *, hipStream_t);

template <class Codec>
hipError_t launch_layer_prep(const RowQuantArgs &r, const WeightSideArgs &args, bool gather,
                             hipStream_t stream) {
  WeightSideArgs w = args;
  w.gather_blocks = gather ? (w.N + 63) / 64 : 0;
  // compaction never applies when even |O| = K would not pay (M below ~313)
  const int64_t cblocks = use_compaction((int)w.K, w.K, w.M) ? (w.N < 1024 ? w.N : 1024) : 0;
  const size_t lds = (r.K <= kCompactMaxK) ? (size_t)r.ldq : 0;
  const int64_t blocks = r.M + w.gather_blocks + cblocks;
  hipLaunchKernelGGL(k_layer_prep<Codec>, dim3((unsigned)blocks), dim3(256), lds, stream, r, w);
  return hipGetLastError();
}
template hipError_t launch_layer_prep<CodecI8>(const RowQuantArgs &, const WeightSideArgs &, bool,
                                               hipStream_t);
template hipError_t launch_layer_prep<CodecE4M3>(const RowQuantArgs &, const WeightSideArgs &,
                                                 bool, hipStream_t);

hipError_t launch_colwise_absmax(const uint16_t *W, int64_t K, int64_t N, int64_t ldw, float *s,
                                 hipStream_t stream) {
  unsigned *sbits = (unsigned *)s;
  hipLaunchKernelGGL(k_fill_u32, dim3((unsigned)((N + 255) / 256)), dim3(256), 0, stream, sbits, N,
                     0u);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int col_tiles = (int)((N + 511) / 512);
  int64_t chunks = (K + 127) / 128;  // ~128 rows per block
  if (chunks > 256) chunks = 256;
  const int rows_per_chunk = (int)((K + chunks - 1) / chunks);
  const int row_chunks = (int)((K + rows_per_chunk - 1) / rows_per_chunk);
  hipLaunchKernelGGL(k_colabsmax, dim3(col_tiles, row_chunks), dim3(256), 0, stream, W, K, N, ldw,
                     rows_per_chunk, sbits);
  return hipGetLastError();
}

template <class Codec>
hipError_t launch_colwise_quant(const uint16_t *W, int64_t K, int64_t N, int64_t ldw,
                                const float *s, uint8_t *Wq, hipStream_t stream) {
  hipLaunchKernelGGL(k_colquant<Codec>,
                     dim3((unsigned)((K + 127) / 128), (unsigned)((N + 63) / 64)), dim3(256), 0,
                     stream, W, K, N, ldw, s, Wq);
  return hipGetLastError();
}
template hipError_t launch_colwise_quant<CodecI8>(const uint16_t *, int64_t, int64_t, int64_t,
                                                  const float *, uint8_t *, hipStream_t);
template hipError_t launch_colwise_quant<CodecE4M3>(const uint16_t *, int64_t, int64_t, int64_t,
                                                    const float *, uint8_t *, hipStream_t);

template <class Codec, int SC, int RPT>
hipError_t launch_colwise_stripe(const uint16_t *W, int64_t K, int64_t N, int64_t ldw,
                                 uint8_t *Wq, float *s, hipStream_t stream) {
  const int64_t stripes = (N + SC - 1) / SC;
  const int64_t kp = K + 16;  // row pitch of the staged codes (bank spread)
  const size_t lds = (size_t)(SC * kp);
  auto *kern = k_colwise_stripe<Codec, SC, RPT>;
  hipError_t e =
      hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)stripes), dim3(kStripeRowPhases * SC / 8), lds, stream,
                     W, K, N, ldw, s, Wq, stripes, kp);
  return hipGetLastError();
}

// The memory-side Infinity Cache of the MI355X. A W that fits in it is read
// by the one-read kernel at 16 or 32 bytes per row without penalty; a larger W
// comes from HBM, where the two-pass kernels' 1 KB row segments use the DRAM
// pages better (measured level or faster at 470 MB, slower at <= 141 MB).
constexpr int64_t kMallBytes = (int64_t)256 << 20;

template <class Codec>
hipError_t launch_colwise(const uint16_t *W, int64_t K, int64_t N, int64_t ldw, uint8_t *Wq,
                          float *s, hipStream_t stream) {
  // one read of W while a stripe of K rows fits in the block's registers and
  // W fits in the Infinity Cache
  if (K <= kStripeMaxK && 2 * K * N <= kMallBytes) {
    if (K <= kStripeMaxK / 8)
      return launch_colwise_stripe<Codec, 16, 2>(W, K, N, ldw, Wq, s, stream);
    if (K <= kStripeMaxK / 4)
      return launch_colwise_stripe<Codec, 16, 4>(W, K, N, ldw, Wq, s, stream);
    if (K <= kStripeMaxK / 2)
      return launch_colwise_stripe<Codec, 16, 8>(W, K, N, ldw, Wq, s, stream);
    // 16 rows per thread: 8-column stripes keep two blocks per CU
    return launch_colwise_stripe<Codec, 8, 16>(W, K, N, ldw, Wq, s, stream);
  }
  const hipError_t e = launch_colwise_absmax(W, K, N, ldw, s, stream);
  if (e != hipSuccess) return e;
  return launch_colwise_quant<Codec>(W, K, N, ldw, s, Wq, stream);
}
template hipError_t launch_colwise<CodecI8>(const uint16_t *, int64_t, int64_t, int64_t,
                                            uint8_t *, float *, hipStream_t);
template hipError_t launch_colwise<CodecE4M3>(const uint16_t *, int64_t, int64_t, int64_t,
                                              uint8_t *, float *, hipStream_t);


}  // namespace llmint8
