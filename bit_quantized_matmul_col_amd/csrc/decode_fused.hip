// Single-kernel small-M path of the LLM.int8() linear layer on gfx950.
//
// For decode-shaped calls with up to 16 rows and K in {1024, 2048, 4096} the
// whole layer runs in one kernel. The layer is bound by streaming the int8
// weight Wq from HBM (the decode regime of the INT8-vs-FP8 page, section one),
// and on gfx950 every extra dependent kernel costs about 3 us. Cross-block
// handoffs through agent-scope fences cost more than a kernel boundary, so this
// kernel needs none: every block recomputes what it needs from X.
//
// Block b (512 threads, persistent over the 16-column tiles b, b + G, ...):
//  1. loads all of X into registers and, once X has arrived, issues the Wq
//     loads of its first tile (they stream while 3-5 run). Loads complete in
//     issue order, so no value loaded after the Wq bytes is used before the
//     tile's MFMAs: a use any earlier would wait for the whole Wq stream;
//  2. X in registers: thread (c, h) holds the 16-byte chunk c
//     (columns 8c .. 8c+7) of rows h, h + R, ... (R = 512 / (K / 8));
//  3. column absmax over all rows with packed 16-bit max on the magnitude bits
//     (for non-negative fp16 the bit patterns order like the values), compared
//     with the smallest fp16 pattern >= threshold: the outlier bits ("LLM.int8()"
//     walkthrough, sections 2.3 and 4.2);
//  4. row absmax over the kept columns the same way, reduced across the block;
//     fl32(127 / m) per row (pitfalls page, section 1);
//  5. int8 codes of the rows below M into LDS (outlier columns zero), once per
//     block;
//  6. per tile: 16x16x64 int8 MFMAs with the wave's eighth of K, a fixed-order
//     sum of the eight wave partials in LDS (exact int32 C), dequantize by
//     m_i * s_j / 127^2, add the fp16 outlier terms X_O . W_O in fp32 (pitfalls
//     page, section 3.3) and store Y.
#include "internal.hpp"

namespace llmint8 {

namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kTileCols = 16;
constexpr int kBatch = 64;     // outlier columns staged per round of the fp16 product

// Four int8 codes of the fp16 pairs (w0, w1) for the scale inv, packed in byte
// order: the fp32 products (fp16_lo_mul / fp16_hi_mul; a zero product's sign
// does not matter here), then adding 1.5 * 2^23 rounds each to the nearest
// integer, ties to even, and leaves it in two's complement in the low bits.
// |x| <= absmax of its row keeps the product within 127 * (1 + 2^-22), so no
// clamp is needed.
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

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
__device__ inline uint32_t pmax16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, a),
                                                                __builtin_bit_cast(u16x2, b)));
}

// Magnitude patterns of the two fp16 in w, with NaN (patterns above 0x7c00)
// taken as 0: a NaN entry never makes its column an outlier and never sets a
// row maximum, as with the fmax-based maxima of the other paths. m + 0x3ff
// reaches bit 15 of its half exactly when m > 0x7c00, and never carries out
// of the half (m <= 0x7fff).
__device__ inline uint32_t mag16(uint32_t w) {
  const uint32_t m = w & 0x7fff7fffu;
  const uint32_t nan = ((m + 0x03ff03ffu) & 0x80008000u) >> 15;
  return m & ~(nan * 0xffffu);
}

// Layout of the dynamic LDS (byte offsets); P = K + 16 is the Xq row pitch
// (16 rows that one MFMA operand reads fall in distinct bank groups).
struct FusedLds {
  int xq, red, list, inv, m, bits, pos, rmax, xo0, ycm, misc, total;
};

__host__ __device__ constexpr FusedLds fused_lds(int K, int MB) {
  FusedLds L{};
  const int P = K + 16;
  int o = 0;
  L.xq = o;
  o += MB * 16 * P;
  o = (o + 15) & ~15;
  L.red = o;  // wave partials [8][MB * 256] int32; also column-max scratch and
  o += kWaves * MB * 256 * 4;  // the fp16 staging of the outlier product
  L.list = o;  // ascending outlier columns, uint16
  o += K * 2;
  o = (o + 15) & ~15;
  L.inv = o;
  o += 64 * 4;
  L.m = o;
  o += 64 * 4;
  L.bits = o;  // outlier bits of each 8-column chunk
  o += K / 8;
  o = (o + 15) & ~15;
  L.pos = o;  // list position of each chunk's first outlier column, uint16
  o += K / 8 * 2;
  o = (o + 15) & ~15;
  L.rmax = o;  // per-wave row maxima [8][32]
  o += kWaves * 32 * 4;
  L.xo0 = o;  // X entries of the first outlier batch [16][64] fp32
  o += 16 * MB * kBatch * 4;
  L.ycm = o;  // per-wave column maxima of |Y| [4][16]
  o += 4 * 16 * 4;
  L.misc = o;
  o += 64;
  L.total = o;
  return L;
}

// Reduce v[0..MR) over the 64 lanes of a wave so that, afterwards, lane l holds
// in v[0] the maximum for row index j(l) = sum of (l bit (5 - s)) * MR / 2^(s+1)
// over the log2(MR) halving steps s (the same value in all lanes sharing those
// bits). Each step halves the values a lane carries and swaps the other half
// with the lane across.
template <int MR>
__device__ inline uint32_t wave_rows_max(uint32_t *v, int lane) {
  int off = 32;
#pragma unroll
  for (int n = MR; n > 1; n >>= 1, off >>= 1) {
    // bitwise selects: a conditional on the two elements would be turned into
    // a run-time index into v, i.e. a compare-and-select over every element
    const uint32_t upm = (lane & off) ? 0xffffffffu : 0u;
#pragma unroll
    for (int i = 0; i < n / 2; ++i) {
      const uint32_t send = (v[i] & upm) | (v[i + n / 2] & ~upm);
      const uint32_t keep = (v[i + n / 2] & upm) | (v[i] & ~upm);
      const uint32_t recv = (uint32_t)__shfl_xor((int)send, off, 64);
      v[i] = keep > recv ? keep : recv;
    }
  }
  uint32_t r = v[0];
  for (; off > 0; off >>= 1) {
    const uint32_t o = (uint32_t)__shfl_xor((int)r, off, 64);
    r = r > o ? r : o;
  }
  return r;
}

template <int K, int MB, bool I8W>
__global__ __launch_bounds__(kThreads) void k_decode_fused(FusedArgs a) {
  constexpr int C = K / 8;               // 16-byte chunks per X row
  constexpr int R = kThreads / C;        // threads sharing a chunk
  constexpr int MR = MB * 16 / R;        // rows per thread
  constexpr int P = K + 16;
  constexpr int KW = K / kWaves;         // k bytes per wave in the MFMA phase
  constexpr int KS = KW / 64;            // MFMA steps per wave
  static_assert(C * R == kThreads && MR * R == MB * 16 && KS * 64 * kWaves == K, "shape");
  static_assert(MR >= 1 && (MR & (MR - 1)) == 0 && MR <= 32, "rows per thread");

  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  constexpr FusedLds L = fused_lds(K, MB);
  uint8_t *sxq = lds + L.xq;
  int32_t *sred = (int32_t *)(lds + L.red);
  uint16_t *slist = (uint16_t *)(lds + L.list);
  float *sinv = (float *)(lds + L.inv);
  float *sm = (float *)(lds + L.m);
  uint8_t *sbits = lds + L.bits;
  uint32_t *srmax = (uint32_t *)(lds + L.rmax);
  int *stotal = (int *)(lds + L.misc);
  uint16_t *spos = (uint16_t *)(lds + L.pos);

  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int c16 = lane & 15, g = lane >> 4;
  const int G = gridDim.x;

  // Per-tile registers: the wave's Wq bytes (wave wv owns k bytes [wv * KW,
  // (wv + 1) * KW)), the column scale and bias bits of the thread's output and
  // the weights of the first batch of outlier columns: 8 fp16 entries of their
  // W rows, or (I8W) two int8 codes. All are loaded without a condition and
  // used only in the tile's epilogue.
  static_assert(MB == 1, "one output per thread");
  struct TileRegs {
    u32x4 b[KS];
    float sc;
    uint32_t braw;
    u32x4 wo;
    int q0, q1;
  };
  // a bias-less call reads its bias bits from s (ignored afterwards)
  const uint16_t *bias_src = a.ep.bias ? a.ep.bias : (const uint16_t *)a.s;
  auto load_cols = [&](TileRegs &tr, int tile) {
    const int no = tile * kTileCols + (t & 15);
    tr.sc = a.s[no < a.N ? no : a.N - 1];
    tr.braw = bias_src[no < a.N ? no : a.N - 1];
  };
  auto load_wq = [&](TileRegs &tr, int tile, int dep) {
    const int n = tile * kTileCols + c16;
    const int8_t *row = a.wq + (int64_t)(n < a.N ? n : a.N - 1) * K + wv * KW + 16 * g + dep;
#pragma unroll
    for (int j = 0; j < KS; ++j) tr.b[j] = *(const u32x4 *)(row + 64 * j);
  };
  auto load_b = [&](TileRegs &tr, int tile) {
    load_wq(tr, tile, 0);
    load_cols(tr, tile);
  };
  // Weights of outlier columns p0 .. p0 + 63 (np of them, at least one) for
  // the tile. fp16: thread t loads row p0 + (t / 2) % 64, columns 8 (t % 2) ..
  // + 8 of the tile (threads t >= 128 repeat the loads of t % 128). I8W: thread
  // t loads the codes Wq[n, k] of outlier p0 + t / 8 for the two columns
  // n = 2 (t % 8), + 1 of the tile.
  auto load_wo = [&](TileRegs &tr, int tile, int p0, int np) {
    if constexpr (I8W) {
      const int p = t >> 3;
      const int64_t kk = slist[p0 + (p < np ? p : np - 1)];
      const int c0 = tile * kTileCols + 2 * (t & 7), c1 = c0 + 1;
      tr.q0 = a.wq[(int64_t)(c0 < a.N ? c0 : a.N - 1) * K + kk];
      tr.q1 = a.wq[(int64_t)(c1 < a.N ? c1 : a.N - 1) * K + kk];
    } else {
      const int p = (t >> 1) & (kBatch - 1), half = t & 1;
      const int64_t kk = slist[p0 + (p < np ? p : np - 1)];
      const int nc = tile * kTileCols + 8 * half;
      tr.wo = *(const u32x4 *)(a.w + kk * a.ldw + (nc < a.N ? nc : a.N - 8));
    }
  };
  // stage the batch's weights as fp16 [kBatch][16] in swo
  auto stage_wo = [&](const TileRegs &tr, uint16_t *swo) {
    if constexpr (I8W) {
      *(uint32_t *)(swo + (t >> 3) * 16 + 2 * (t & 7)) =
          (uint32_t)f2h((float)tr.q0) | ((uint32_t)f2h((float)tr.q1) << 16);
    } else {
      if (t < 2 * kBatch) *(u32x4 *)(swo + (t >> 1) * 16 + 8 * (t & 1)) = tr.wo;
    }
  };
  // 2. X: chunk c of rows h + R j (rows past M read as zero: harmless for every
  //    max, and their codes are replaced by zeros). X is issued before Wq: loads
  //    complete in issue order, and steps 3-5 wait only for X.
  const int c = t % C, h = t / C;
  // a caller-supplied column absmax of X decides the outlier columns
  f32x4 xc0 = {0.f, 0.f, 0.f, 0.f}, xc1 = xc0;
  if (a.xcmax && h == 0) {
    xc0 = *(const f32x4 *)(a.xcmax + 8 * c);
    xc1 = *(const f32x4 *)(a.xcmax + 8 * c + 4);
  }
  // the first tile's scales and bias bits ahead of everything else: they may
  // be used as soon as they arrive
  TileRegs tr0, tr1;
  load_cols(tr0, blockIdx.x);
  u32x4 xv[MR];
  {
    // one buffer resource over rows 0 .. M-1; rows past M are not loaded at
    // all (an out-of-range load reads zero without memory traffic but still
    // takes a load slot: all 16 rows at M = 1 cost 0.6 us per call)
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        (void *)a.X, (short)0, (int)(((int64_t)a.M - 1) * a.ldx * 2 + 2 * K), 0x00020000);
#pragma unroll
    for (int j = 0; j < MR; ++j) {
      const int r = h + R * j;
      xv[j] = (u32x4){0u, 0u, 0u, 0u};
      if (r < a.M)
        xv[j] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(xr, (int)(r * a.ldx * 2 + 16 * c), 0, 0));
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  // 3. column magnitudes, as 16-bit patterns, two per 32-bit word. X is
  // waited for before the Wq loads are issued: measured on this hardware, a
  // load issued together with the Wq stream returns only when the stream is
  // nearly done, and everything up to the MFMAs depends on X.
  uint32_t cm[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int j = 0; j < MR; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) cm[e] = pmax16(cm[e], mag16(xv[j][e]));
  // a zero the compiler cannot see through, computed from the column maxima:
  // added to the Wq addresses, it keeps their loads behind the wait for X
  int xdep = (int)cm[0];
  asm volatile("v_and_b32 %0, 0, %0" : "+v"(xdep));
  load_wq(tr0, blockIdx.x, xdep);
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (R > 1) {
    u32x4 *scm = (u32x4 *)sred;  // [R][C]
    scm[h * C + c] = (u32x4){cm[0], cm[1], cm[2], cm[3]};
    __syncthreads();
    if (h == 0) {
#pragma unroll
      for (int q = 1; q < R; ++q) {
        const u32x4 o = scm[q * C + c];
#pragma unroll
        for (int e = 0; e < 4; ++e) cm[e] = pmax16(cm[e], o[e]);
      }
    }
  }
  if (h == 0) {
    uint32_t bits = 0;
    if (a.xcmax) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        bits |= (xc0[e] >= a.threshold ? 1u : 0u) << e;
        bits |= (xc1[e] >= a.threshold ? 1u : 0u) << (4 + e);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        bits |= ((cm[e] & 0xffffu) >= a.tcut ? 1u : 0u) << (2 * e);
        bits |= ((cm[e] >> 16) >= a.tcut ? 1u : 0u) << (2 * e + 1);
      }
    }
    sbits[c] = (uint8_t)bits;
  }
  __syncthreads();

  // 4. row magnitudes over the kept columns
  const uint32_t ob = sbits[c];
  uint32_t keep16[4];
#pragma unroll
  for (int e = 0; e < 4; ++e)
    keep16[e] = (((ob >> (2 * e)) & 1u) ? 0u : 0x7fffu) |
                (((ob >> (2 * e + 1)) & 1u) ? 0u : 0x7fff0000u);
  {
    uint32_t rm[MR];
#pragma unroll
    for (int j = 0; j < MR; ++j) {
      uint32_t v = 0u;
#pragma unroll
      for (int e = 0; e < 4; ++e) v = pmax16(v, mag16(xv[j][e]) & keep16[e]);
      rm[j] = (v & 0xffffu) > (v >> 16) ? (v & 0xffffu) : (v >> 16);
    }
    const uint32_t r = wave_rows_max<MR>(rm, lane);
    // lane l's result is row index j(l); lanes with the low bits clear publish it
    int j = 0, off = 32;
#pragma unroll
    for (int n = MR; n > 1; n >>= 1, off >>= 1)
      if (lane & off) j += n / 2;
    if ((lane & (off * 2 - 1)) == 0) srmax[wv * 32 + j] = r;
  }
  __syncthreads();
  if (t < MB * 16) {
    // row t is index j = t / R of the waves whose threads have h = t % R
    const int hr = t % R, jr = t / R;
    uint32_t mb = 0u;
#pragma unroll
    for (int w = 0; w < kWaves; ++w)
      if ((w * 64) / C == hr) mb = mb > srmax[w * 32 + jr] ? mb : srmax[w * 32 + jr];
    const float m = h2f((uint16_t)mb);
    const bool live = t < a.M && m > 0.f;
    sinv[t] = live ? inv_scale(m) : 0.f;
    sm[t] = t < a.M ? m : 0.f;
  }
  // outlier list (ascending) from the chunk bits: wave 0, C / 64 chunks per lane
  if (wv == 0) {
    constexpr int CPL = C / 64;
    uint32_t cb[CPL];
    int cnt = 0;
#pragma unroll
    for (int q = 0; q < CPL; ++q) {
      cb[q] = sbits[lane * CPL + q];
      cnt += __builtin_popcount(cb[q]);
    }
    int incl = cnt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o, 64);
      if (lane >= o) incl += y;
    }
    int pos = incl - cnt;
#pragma unroll
    for (int q = 0; q < CPL; ++q) {
      spos[lane * CPL + q] = (uint16_t)pos;
      uint32_t bb = cb[q];
      while (bb) {
        slist[pos++] = (uint16_t)(8 * (lane * CPL + q) + __builtin_ctz(bb));
        bb &= bb - 1u;
      }
    }
    if (lane == 63) {
      *stotal = incl;
      if (blockIdx.x == 0 && a.count_out) *a.count_out = incl;
    }
  }
  __syncthreads();

  // first batch of the outlier product: the weights of the first tile are
  // loaded now (behind the Wq bytes, used after the MFMAs); the X entries come
  // from the registers below
  const int total = *stotal;
  const bool outl = total > 0 && (a.w || I8W);
  const int np0 = total < kBatch ? total : kBatch;
  if (outl) load_wo(tr0, blockIdx.x, 0, np0);

  // 5. int8 codes into LDS for rows below M (the MFMA rows past M only reach
  //    outputs that are never stored, so their LDS rows are left as they are)
  {
    const uint32_t kl = keep_bytes(ob & 0xfu), kh = keep_bytes(ob >> 4);
#pragma unroll
    for (int j = 0; j < MR; ++j) {
      const int r = h + R * j;
      if (r < a.M) {
        const float inv = sinv[r];
        u32x2 out;
        out[0] = codes4(xv[j][0], xv[j][1], inv) & kl;
        out[1] = codes4(xv[j][2], xv[j][3], inv) & kh;
        *(u32x2 *)(sxq + r * P + 8 * c) = out;
      }
    }
  }
  // X entries of the first batch, [16][kBatch] fp32: each thread places the
  // outlier columns of its chunk (list positions from spos)
  float *sxo0 = (float *)(lds + L.xo0);
  if (ob != 0u) {
    uint32_t bb = ob;
    int p = spos[c];
    while (bb && p < kBatch) {
      const int e = __builtin_ctz(bb);
      bb &= bb - 1u;
#pragma unroll
      for (int j = 0; j < MR; ++j) {
        const uint32_t w = xv[j][e >> 1];
        if (h + R * j < a.M)
          sxo0[(h + R * j) * kBatch + p] = h2f((uint16_t)((e & 1) ? (w >> 16) : (w & 0xffffu)));
      }
      ++p;
    }
  }
  __syncthreads();

  // 6. tiles
  auto run_tile = [&](const TileRegs &tr, int tile) {
    const u32x4 *b = tr.b;
    i32x4 acc[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[mb] = (i32x4){0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < KS; ++j)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const i32x4 av =
            *(const i32x4 *)(sxq + (mb * 16 + c16) * P + wv * KW + 64 * j + 16 * g);
        acc[mb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, __builtin_bit_cast(i32x4, b[j]),
                                                         acc[mb], 0, 0, 0);
      }
    // lane holds rows mb * 16 + 4 g + r, column c16
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) sred[wv * MB * 256 + (mb * 16 + 4 * g + r) * 16 + c16] = acc[mb][r];
    __syncthreads();
    // outputs: index q = t + 512 u (u < OPT) is row q / 16, column q % 16 of the tile
    constexpr int OPT = (MB * 256 + kThreads - 1) / kThreads;
    float y[OPT], yo[OPT];
#pragma unroll
    for (int u = 0; u < OPT; ++u) {
      const int q = t + kThreads * u;
      const int orow = q >> 4, n = tile * kTileCols + (q & 15);
      y[u] = 0.f;
      yo[u] = 0.f;
      if (q < MB * 256) {
        int cacc = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) cacc += sred[w * MB * 256 + q];
        const float sc = tr.sc;
        if (a.cdbg && orow < a.M && n < a.N) a.cdbg[(int64_t)orow * a.N + n] = cacc;
        y[u] = (float)cacc * (sm[orow] * (sc * (1.0f / 16129.0f)));
      }
    }
    __syncthreads();  // the partials are consumed; the staging below reuses them
    if (outl) {
      float *sxo = (float *)sred;                                   // [16][kBatch]
      uint16_t *swo = (uint16_t *)(sxo + MB * 16 * kBatch);         // [kBatch][16]
      for (int p0 = 0; p0 < total; p0 += kBatch) {
        const int np = (total - p0 < kBatch) ? total - p0 : kBatch;
        // the first batch was loaded ahead; later ones are loaded here
        const float *xs = p0 == 0 ? sxo0 : sxo;
        if (p0 == 0) {
          stage_wo(tr, swo);
        } else {
          TileRegs tw;
          load_wo(tw, tile, p0, np);
          stage_wo(tw, swo);
        }
        if (p0 > 0) {
          for (int q = t; q < MB * 16 * kBatch; q += kThreads) {  // X entries
            const int r = q / kBatch, p = q % kBatch;
            const int64_t kk = slist[p0 + (p < np ? p : np - 1)];
            sxo[q] = h2f(a.X[(int64_t)(r < a.M ? r : a.M - 1) * a.ldx + kk]);
          }
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < OPT; ++u) {
          const int q = t + kThreads * u;
          if (q < MB * 256)
            for (int p = 0; p < np; ++p)
              yo[u] += xs[(q >> 4) * kBatch + p] * h2f(swo[p * 16 + (q & 15)]);
        }
        __syncthreads();
      }
    }
    // with int8 outlier weights the outlier terms carry the codes: times s / 127
    const float oscale = I8W ? tr.sc * (1.0f / 127.0f) : 1.0f;
    const float bias = a.ep.bias ? h2f((uint16_t)tr.braw) : 0.f;
    float cmax = 0.f;
#pragma unroll
    for (int u = 0; u < OPT; ++u) {
      const int q = t + kThreads * u;
      const int orow = q >> 4, n = tile * kTileCols + (q & 15);
      const float v = y[u] + yo[u] * oscale + bias;
      if (q < MB * 256 && orow < a.M && n < a.N) a.y[(int64_t)orow * a.ldy + n] = f2h(v);
      cmax = (q < MB * 256 && orow < a.M) ? __builtin_fmaxf(cmax, stored_abs(v)) : cmax;
    }
    if (a.ep.ycmax) {
      // the block holds every row of its 16 columns: rows 4 w + l / 16 of
      // column l % 16 in lane l of wave w < 4
      cmax = __builtin_fmaxf(cmax, __shfl_xor(cmax, 16, 64));
      cmax = __builtin_fmaxf(cmax, __shfl_xor(cmax, 32, 64));
      float *sycm = (float *)(lds + L.ycm);  // [4][16]
      if (wv < 4 && lane < 16) sycm[wv * 16 + lane] = cmax;
      __syncthreads();
      const int n = tile * kTileCols + t;
      if (t < 16 && n < a.N)
        a.ep.ycmax[n] = __builtin_fmaxf(__builtin_fmaxf(sycm[t], sycm[16 + t]),
                                        __builtin_fmaxf(sycm[32 + t], sycm[48 + t]));
    }
  };

  for (int tile = blockIdx.x;;) {
    const int t1 = tile + G;
    if (t1 < a.tiles) {
      load_b(tr1, t1);
      if (outl) load_wo(tr1, t1, 0, np0);
    }
    run_tile(tr0, tile);
    if (t1 >= a.tiles) break;
    const int t2 = t1 + G;
    if (t2 < a.tiles) {
      load_b(tr0, t2);
      if (outl) load_wo(tr0, t2, 0, np0);
    }
    run_tile(tr1, t1);
    if (t2 >= a.tiles) break;
    tile = t2;
  }
}

template <int K, int MB, bool I8W>
hipError_t launch_fused_kmb(const FusedArgs &a, const GemmEvents &ev, hipStream_t stream) {
  constexpr FusedLds L = fused_lds(K, MB);
  hipError_t e = hipFuncSetAttribute((const void *)k_decode_fused<K, MB, I8W>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, L.total);
  if (e != hipSuccess) return e;
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    cus = 256;
  const int grid = a.tiles < cus ? a.tiles : cus;
  hipExtLaunchKernelGGL((k_decode_fused<K, MB, I8W>), dim3(grid), dim3(kThreads), L.total, stream,
                        (hipEvent_t)ev.begin, (hipEvent_t)ev.end, 0u, a);
  return hipGetLastError();
}

template <int K>
hipError_t launch_fused_k(const FusedArgs &a, const GemmEvents &ev, hipStream_t stream) {
  return a.ep.int8w ? launch_fused_kmb<K, 1, true>(a, ev, stream)
                    : launch_fused_kmb<K, 1, false>(a, ev, stream);
}

}  // namespace

// Up to 16 rows the single kernel beats the three-kernel path (it replicates X
// into every block, which stops paying beyond one 16-row MFMA block).
bool fused_decode_fits(int64_t M, int64_t K, int64_t ldx) {
  if (M < 1 || M > 16) return false;
  if (M * ldx * 2 >= ((int64_t)1 << 31)) return false;  // 32-bit buffer offsets
  return K == 4096 || K == 2048 || K == 1024;
}

hipError_t launch_decode_fused(const FusedArgs &a, const GemmEvents &ev, hipStream_t stream) {
  switch (a.K) {
    case 4096: return launch_fused_k<4096>(a, ev, stream);
    case 2048: return launch_fused_k<2048>(a, ev, stream);
    case 1024: return launch_fused_k<1024>(a, ev, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace llmint8
