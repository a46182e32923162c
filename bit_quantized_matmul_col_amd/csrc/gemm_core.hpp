// Large-M GEMM of the LLM.int8() linear layer on gfx950 MFMA, with the
// dequantize-and-add epilogue fused in (kernel templates; each tile shape is
// instantiated in its own translation unit).
//
// C = Xq . Wq^T with int32 accumulation (the int8 x int8 -> int32 matmul of the
// "8-Bit LLM Quantization with Lightning Fabric" page, section 2.2); then
// Y = C * m[i] * s[n] / 127^2 + X_O . W_O, the 16-bit outlier product added to
// the dequantized int8 result ("LLM.int8() pitfalls" page, section 3.3;
// "LLM.int8()" walkthrough, section 2.3), accumulated in fp32.
//
// Design (one block per BM x BN output tile, 2 x NWN waves of BM/2 x BN/NWN,
// 32x32 MFMA blocks; 256x256 tiles run 8 waves, two per SIMD, so that one
// wave's MFMAs cover the other's waits):
//  * Operands stream through LDS in stages of 128 bytes of k per row (128 int8
//    or 64 fp16), in a ring of three stages (256x128 tiles) or two (256x256,
//    whose three would not fit in LDS), filled by buffer_load_dwordx4 ... lds: lane
//    l of a wave instruction lands at base + 16 l, so each instruction moves
//    8 rows x 128 B with no register staging. Each operand tile is one buffer
//    resource starting at the tile's first row; a lane keeps one 32-bit offset
//    per 8-row group and the stage's k offset is scalar. Rows past the matrix
//    end lie past the resource's record count and read as zero, so there is no
//    bounds arithmetic in the loop. The loads of a later stage are spread over
//    the k-steps of the current stage's MFMAs.
//  * The 16-byte chunk c of row r is stored at chunk c ^ ((r >> 1) & 7), so the
//    16 rows that lanes 0..15 read for one MFMA operand fall in 16 different
//    bank groups.
//  * The int8 operand Xq is zero from column K (or K - |O|) to its padded
//    pitch, so whatever the other operand holds there adds nothing.
//  * After the int8 k-loop the int32 accumulators are scaled to fp32 in place
//    and a second k-loop with v_mfma_f32_32x32x16_f16 adds X_O . W_O over the
//    gathered outlier columns (X_O [M x ldo] and the pre-transposed W_O^T
//    [N x ldo], both zero-padded to 64 columns).
//  * Blocks are renumbered so each XCD (blocks are dealt to the 8 XCDs round
//    robin) works on a contiguous, M-grouped range of tiles and shares operand
//    stages through its own L2.
//
// MFMA lane layouts (gfx950, checked on hardware): for v_mfma_i32_32x32x32_i8
// and v_mfma_f32_32x32x16_f16 lane l supplies row (A) / column (B) l % 32 and
// k-group l / 32 of 16 bytes; register r of the 32x32 result holds row
// 8(r/4) + 4(l/32) + r%4, column l % 32. Both operands use the same k-groups,
// which is all an exact integer dot product needs.
#pragma once

#include "internal.hpp"

namespace llmint8 {
namespace gemm_detail {

constexpr int kXcds = 8;    // XCDs of the MI355X
constexpr int kGroupM = 8;  // tile rows per ordering group

typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef void __attribute__((address_space(3))) *lptr_t;

// Raw buffer resource over [base, base + bytes): 32-bit word count, data format
// field set as gfx9 raw dword access requires.
__device__ inline rsrc_t make_rsrc(const void *base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void *)base, (short)0, (int)bytes, 0x00020000);
}

// Wait until at most N vector-memory operations of this wave are outstanding
// (they complete in issue order, so the older ones have landed).
template <int N>
__device__ inline void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier for the k-loop. __syncthreads() carries a workgroup fence,
// and the compiler makes that fence wait for every outstanding direct-to-LDS
// load (vmcnt(0)), which would drain the whole ring at each step. In the
// k-loop the only LDS writes are those loads, and each wave has already waited
// for the stage it needs (wait_vm), so the bare barrier is enough; the LDS
// reads of the previous stage have been consumed by its MFMAs.
__device__ inline void ring_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Chunk permutation of row r in a stage of SK bytes per row (SK / 16 chunks of
// 16 bytes). The 16 rows that lanes 0..15 read for one MFMA operand then fall
// in 16 different 16-byte bank groups of the 256-byte bank row: with 128-byte
// rows, rows 2q and 2q + 1 sit in opposite halves and q picks the chunk; with
// 64-byte rows, r % 4 picks the quarter and (r / 4) % 4 the chunk.
template <int SK>
__device__ inline int swz_key(int r) {
  static_assert(SK == 128 || SK == 64, "stage row size");
  return SK == 128 ? (r >> 1) & 7 : (r >> 2) & 3;
}

// Byte offset of logical 16-byte chunk c of row r inside a stage.
template <int SK>
__device__ inline int swz(int r, int c) { return r * SK + 16 * (c ^ swz_key<SK>(r)); }

// One operand tile: ROWS rows from row0 of a row-major matrix, SK bytes of k
// per stage, loaded by NW waves. One wave instruction moves 1 KB = RPI rows;
// wave w loads the row groups w, w + NW, ...; lane l of a group fetches the
// logical chunk that belongs at physical slot l % (SK / 16) of row l / (SK / 16).
template <int ROWS, int NW, int SK>
struct OperandTile {
  static constexpr int RPI = 1024 / SK;            // rows per wave instruction
  static constexpr int G = ROWS / (RPI * NW);      // row groups per wave
  const uint8_t *base;  // first row of the tile
  int bytes;            // bytes from base to the end of the matrix rows in the tile
  int voff[G];

  // k0: the first byte of k the tile reads (the start of a split-K range, a
  // multiple of the stage size); the resource still ends at the end of the
  // last row, so whatever lies past it reads as zero as before.
  __device__ void init(const void *mat, int64_t ld_bytes, int64_t row0, int64_t nrows,
                       int64_t k0 = 0) {
    int64_t rows = nrows - row0;
    rows = rows < ROWS ? rows : ROWS;
    base = (const uint8_t *)mat + row0 * ld_bytes + k0;
    bytes = (int)(rows * ld_bytes - k0);
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const int r = (wv + NW * j) * RPI + lane / (SK / 16);
      const int c = (lane % (SK / 16)) ^ swz_key<SK>(r);
      voff[j] = r * (int)ld_bytes + 16 * c;
    }
  }

  __device__ void load(uint8_t *stage, int kbyte) const {
#pragma unroll
    for (int j = 0; j < G; ++j) load_group(stage, kbyte, j);
  }

  // The j-th of the wave's G row groups of one stage.
  __device__ void load_group(uint8_t *stage, int kbyte, int j) const {
    const int wv = threadIdx.x >> 6;
    const rsrc_t rs = make_rsrc(base, bytes);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lptr_t)(stage + (wv + NW * j) * RPI * SK), 16,
                                              voff[j], kbyte, 0, 0);
  }
};

// BM x BN block tile computed by 2 x NWN waves of WM x WN (NWN = 2: one wave
// per SIMD; NWN = 4: two), staged SK bytes of k at a time.
template <int BM, int BN, int NWN, int SK>
struct TileCfg {
  static constexpr int NW = 2 * NWN, THREADS = 64 * NW;
  static constexpr int WM = BM / 2, WN = BN / NWN;
  static constexpr int MI = WM / 32, NI = WN / 32;
  static constexpr int STAGE = (BM + BN) * SK;
  // stages in the LDS ring: as many as fit in the 160 KB of a CU, up to 4
  static constexpr int SCALES = (BM + 2 * BN) * 4;  // row scales, two column scales
  static constexpr int FIT = (160 * 1024 - SCALES) / STAGE;
  static constexpr int NST = FIT > 4 ? 4 : FIT;
  static_assert(NST >= 2, "two stages must fit");
  static constexpr int LDS = NST * STAGE + SCALES;
};

// Tile coordinates of this block after the XCD-aware renumbering.
__device__ inline void tile_of_block(int64_t bid, int64_t tiles_m, int64_t tiles_n, int64_t &tm,
                                     int64_t &tn) {
  const int64_t nb = tiles_m * tiles_n;
  const int64_t x = bid % kXcds, q = nb / kXcds, rem = nb % kXcds;
  const int64_t v = x * q + (x < rem ? x : rem) + bid / kXcds;
  const int64_t group = kGroupM * tiles_n;
  const int64_t first_m = (v / group) * kGroupM;
  const int64_t gm = (tiles_m - first_m < kGroupM) ? tiles_m - first_m : kGroupM;
  tm = first_m + (v % group) % gm;
  tn = (v % group) / gm;
}

// The MFMAs of one 128-byte stage (4 k-steps of 32 bytes). The operand
// fragments of k-step ks + 1 are read from LDS (into the second of two
// fragment buffers) before the MFMAs of k-step ks are issued; scheduling
// barriers keep the compiler from sinking those reads next to their use, so
// their latency hides behind the current k-step's MFMAs.
template <typename V>
__device__ inline V lds_frag(const uint8_t *p) {
  return *(const V *)p;
}

// Operand fragment of one lane for one k-step: FragChunks<V> consecutive
// logical 16-byte chunks from chunk c0 of a row, each read from its swizzled
// slot.
template <typename V>
struct FragChunks {
  static constexpr int value = 1;
};
template <>
struct FragChunks<i32x8> {
  static constexpr int value = 2;
};

template <int SK, typename V>
__device__ inline void frag(const uint8_t *tile, int row, int c0, V &out) {
  out = lds_frag<V>(tile + swz<SK>(row, c0));
}

template <int SK>
__device__ inline void frag(const uint8_t *tile, int row, int c0, i32x8 &out) {
  out.lo = lds_frag<i32x4>(tile + swz<SK>(row, c0));
  out.hi = lds_frag<i32x4>(tile + swz<SK>(row, c0 + 1));
}

// The MFMAs of one stage of SK bytes of k. A k-step takes 16 * FragChunks<V>
// bytes of k from each of the two lane groups. The operand fragments of k-step ks + 1
// are read from LDS (into the second of two fragment buffers) before the MFMAs
// of k-step ks are issued; scheduling barriers keep the compiler from sinking
// those reads next to their use, so their latency hides behind the current
// k-step's MFMAs. after_kstep(ks, KSTEPS) runs after each k-step's MFMAs.
template <int BM, int WM, int WN, int MI, int NI, int SK, typename V, typename MFMA,
          typename HOOK>
__device__ inline void stage_mfma(const uint8_t *cur, int wm, int wn, int li, int lg,
                                  i32x16 *acc, MFMA mfma, HOOK after_kstep) {
  constexpr int CPL = FragChunks<V>::value;  // chunks per lane per k-step
  constexpr int KSTEPS = SK / (32 * CPL);
  V av[2][MI], bv[2][NI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) frag<SK>(cur, wm * WM + mi * 32 + li, lg * CPL, av[0][mi]);
#pragma unroll
  for (int ni = 0; ni < NI; ++ni) frag<SK>(cur + BM * SK, wn * WN + ni * 32 + li, lg * CPL, bv[0][ni]);
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) {
    const int b = ks & 1;
    if (ks + 1 < KSTEPS) {
      const int c0 = (2 * (ks + 1) + lg) * CPL;
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) frag<SK>(cur, wm * WM + mi * 32 + li, c0, av[b ^ 1][mi]);
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
        frag<SK>(cur + BM * SK, wn * WN + ni * 32 + li, c0, bv[b ^ 1][ni]);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) acc[mi * NI + ni] = mfma(av[b][mi], bv[b][ni], acc[mi * NI + ni]);
    after_kstep(ks, KSTEPS);
    __builtin_amdgcn_sched_barrier(0);
  }
}

struct MfmaI8 {
  __device__ i32x16 operator()(i32x4 a, i32x4 b, i32x16 c) const {
    return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
  }
};

// v_mfma_f32_32x32x64_f8f6f4 with both operands E4M3 (format 0) and no block
// scales: 32 bytes of k per lane, fp32 accumulation (kept as raw bits in the
// int32 accumulator registers).
struct MfmaF8 {
  __device__ i32x16 operator()(i32x8 a, i32x8 b, i32x16 c) const {
    return __builtin_bit_cast(i32x16, __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                                          a, b, __builtin_bit_cast(f32x16, c), 0, 0, 0, 0, 0, 0));
  }
};

struct MfmaF16 {
  __device__ i32x16 operator()(f16x8 a, f16x8 b, i32x16 c) const {
    return __builtin_bit_cast(i32x16, __builtin_amdgcn_mfma_f32_32x32x16_f16(
                                          a, b, __builtin_bit_cast(f32x16, c), 0, 0, 0));
  }
};

// The loads of one stage spread over the k-steps of another stage's MFMAs:
// after k-step ks of ksteps, the row groups j with j * ksteps / G == ks.
template <int BM, int BN, int NW, int SK>
struct SpreadLoads {
  const OperandTile<BM, NW, SK> &A;
  const OperandTile<BN, NW, SK> &B;
  uint8_t *buf;
  int kb;
  bool on;
  __device__ void operator()(int ks, int ksteps) const {
    constexpr int GA = OperandTile<BM, NW, SK>::G, GB = OperandTile<BN, NW, SK>::G;
    if (!on) return;
#pragma unroll
    for (int j = 0; j < GA; ++j)
      if (j * ksteps / GA == ks) A.load_group(buf, kb, j);
#pragma unroll
    for (int j = 0; j < GB; ++j)
      if (j * ksteps / GB == ks) B.load_group(buf + BM * SK, kb, j);
  }
};

// The loads of the next stage in a two-stage ring: the first half of the row
// groups before this stage's MFMAs, the second half after its first k-step.
// Each direct-to-LDS load moves 1 KB through the texture path, and a wave that
// issues all of its loads at once stalls its MFMA issue until they are
// accepted; issued in two halves, they still land well before the next
// stage's wait.
template <int BM, int BN, int NW, int SK>
struct SplitLoads {
  static constexpr int G = OperandTile<BM, NW, SK>::G;
  static_assert(G == OperandTile<BN, NW, SK>::G && G % 2 == 0, "equal, even row groups");
  const OperandTile<BM, NW, SK> &A;
  const OperandTile<BN, NW, SK> &B;
  uint8_t *buf;
  int kb;
  bool on;
  __device__ void groups(int j0, int j1) const {
#pragma unroll
    for (int j = 0; j < G; ++j)
      if (j >= j0 && j < j1) {
        A.load_group(buf, kb, j);
        B.load_group(buf + BM * SK, kb, j);
      }
  }
  __device__ void first_half() const {
    if (on) groups(0, G / 2);
  }
  __device__ void operator()(int ks, int) const {
    if (on && ks == 0) groups(G / 2, G);
  }
};

// What a k-loop multiplies: int8 codes (int32 sums), fp16 (the outlier
// product) or E4M3 codes (fp32 sums).
enum class Op { I8, F16, F8 };

// Pipelined k-loop over nstages 128-byte stages of A and B through a ring of
// NST LDS buffers. At step it the block waits for stage it only (the NST - 2
// younger stages stay in flight), synchronizes (which also frees the buffer of
// stage it - 1), issues stage it + NST - 1 into that buffer and runs the MFMAs
// of stage it.
template <int BM, int BN, int WM, int WN, int MI, int NI, int NST, int NW, int SK, Op OP>
__device__ inline void kloop(uint8_t *smem, const OperandTile<BM, NW, SK> &A,
                             const OperandTile<BN, NW, SK> &B,
                             int64_t nstages, int wm, int wn, int li, int lg,
                             i32x16 *acc) {
  constexpr int STAGE = (BM + BN) * SK;
  constexpr int LPS = OperandTile<BM, NW, SK>::G + OperandTile<BN, NW, SK>::G;  // per lane per stage
  static_assert(NST >= 2 && NST <= 4, "ring depth");
  if (nstages <= 0) return;
#pragma unroll
  for (int st = 0; st < NST - 1; ++st)
    if (st < nstages) {
      A.load(smem + st * STAGE, st * SK);
      B.load(smem + st * STAGE + BM * SK, st * SK);
    }
  for (int64_t it = 0; it < nstages; ++it) {
    // younger stages already issued may stay in flight
    const int64_t ahead = (nstages - 1 - it < NST - 2) ? nstages - 1 - it : NST - 2;
    if (NST >= 4 && ahead >= 2)
      wait_vm<2 * LPS>();
    else if (NST >= 3 && ahead >= 1)
      wait_vm<LPS>();
    else
      wait_vm<0>();
    ring_barrier();
    // The loads of stage it + NST - 1. With three or more buffers they are
    // spread over the k-steps of this stage's MFMAs (they have at least one
    // further stage to land); with two, half go out before the MFMAs and half
    // after the first of the stage's four k-steps, so that the second half
    // still has three quarters of the stage to land. An E4M3 stage has two
    // k-steps, and its second half would have only half a stage (measured
    // slower), so it issues the whole stage up front.
    const int64_t nx = it + NST - 1;
    const bool more = nx < nstages;
    uint8_t *buf = smem + (nx % NST) * STAGE;
    const int kb = (int)(nx * SK);
    const uint8_t *cur = smem + (it % NST) * STAGE;
    auto run = [&](const auto &issue) {
      if constexpr (OP == Op::F16)
        stage_mfma<BM, WM, WN, MI, NI, SK, f16x8>(cur, wm, wn, li, lg, acc, MfmaF16(), issue);
      else if constexpr (OP == Op::F8)
        stage_mfma<BM, WM, WN, MI, NI, SK, i32x8>(cur, wm, wn, li, lg, acc, MfmaF8(), issue);
      else
        stage_mfma<BM, WM, WN, MI, NI, SK, i32x4>(cur, wm, wn, li, lg, acc, MfmaI8(), issue);
    };
    if constexpr (NST == 2 && OP != Op::F8) {
      const SplitLoads<BM, BN, NW, SK> issue{A, B, buf, kb, more};
      issue.first_half();
      run(issue);
    } else if constexpr (NST == 2) {
      if (more) {
        A.load(buf, kb);
        B.load(buf + BM * SK, kb);
      }
      run(SpreadLoads<BM, BN, NW, SK>{A, B, buf, kb, false});
    } else {
      run(SpreadLoads<BM, BN, NW, SK>{A, B, buf, kb, more});
    }
  }
  __syncthreads();  // every wave is done with the ring before it is reused
}

// Split-K handoff of one 256 x 256 tile. Every split stores its int32 sums in
// its own slot of a.part (register r of thread t at word r * TH + t, so each
// store instruction of a wave writes 256 contiguous bytes) and counts itself
// in a.sem[tile]. The split that arrives last adds the other slots to its own
// sums (exact integers, so the order does not matter) and returns true: it
// finishes the tile. The others return false. Nothing waits for another block.
// The slots are written and read with agent-scope atomic stores and loads
// (coherent across the XCDs' L2 caches), and every wave waits for its stores
// to complete before the block counts itself, so no fence is needed: an
// agent-scope fence would write back and invalidate the whole L2 of the XCD,
// costing the other blocks there their staged operand lines.
template <int TH, int NACC>
__device__ inline bool split_merge(const GemmArgs &a, int64_t tile, int split, i32x16 *acc) {
  constexpr int R = NACC * 16;  // int32 sums per thread
  const int t = threadIdx.x;
  const int S = a.ksplit;
  int32_t *slots = a.part + tile * (int64_t)S * R * TH;
  int32_t *mine = slots + (int64_t)split * R * TH;
#pragma unroll
  for (int i = 0; i < NACC; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      __hip_atomic_store(mine + (i * 16 + r) * TH + t, acc[i][r], __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's sums are stored
  __shared__ int s_last;
  __syncthreads();
  if (t == 0)
    s_last = __hip_atomic_fetch_add(a.sem + tile, 1u, __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_AGENT) == (unsigned)(S - 1);
  __syncthreads();
  if (!s_last) return false;
  for (int sp = 0; sp < S; ++sp) {
    if (sp == split) continue;
    const int32_t *other = slots + (int64_t)sp * R * TH;
    // four accumulator blocks (64 loads) in flight at a time
#pragma unroll
    for (int i0 = 0; i0 < NACC; i0 += 4) {
      i32x16 v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          v[i][r] = (i0 + i < NACC) ? __hip_atomic_load(other + ((i0 + i) * 16 + r) * TH + t,
                                                        __ATOMIC_RELAXED,
                                                        __HIP_MEMORY_SCOPE_AGENT)
                                    : 0;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (i0 + i < NACC) acc[i0 + i] += v[i];
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  return true;
}

// One output tile: block bid of the launch's tiles for a. F8: the operands are
// E4M3 codes (fp32 sums, dequantized by 1 / 448^2) instead of int8 codes
// (int32 sums, 1 / 127^2).
// SPLIT: the launch holds a.ksplit blocks per tile, block bid taking k range
// bid / tiles of the tile bid % tiles (so each split's blocks keep the
// XCD-aware tile order); the last split to finish runs the epilogue.
template <int BM, int BN, int NWN, int SK, bool DBG, bool F8, bool SPLIT = false>
__device__ __forceinline__ void prefill_tile(const GemmArgs &a, int64_t bid, uint8_t *smem) {
  static_assert(!SPLIT || ((BM == 256 || BM == 128) && BN == 256 && !F8),
                "split-K: int8 256 x 256 or 128 x 256 tiles");
  using T = TileCfg<BM, BN, NWN, SK>;
  constexpr int NW = T::NW, TH = T::THREADS;
  constexpr int MI = T::MI, NI = T::NI, WM = T::WM, WN = T::WN;
  float *sm = (float *)(smem + T::NST * T::STAGE);
  float *ss = sm + BM;  // column factor of the int8 dequantization
  float *sf = ss + BN;  // column factor applied at the end (int8 outlier weights)

  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int wm = wv / NWN, wn = wv % NWN;
  const int li = lane & 31, lg = lane >> 5;
  int64_t tm, tn;
  const int64_t tiles_m = (a.M + BM - 1) / BM, tiles_n = (a.N + BN - 1) / BN;
  const int64_t tile = SPLIT ? bid % (tiles_m * tiles_n) : bid;
  const int split = SPLIT ? (int)(bid / (tiles_m * tiles_n)) : 0;
  tile_of_block(tile, tiles_m, tiles_n, tm, tn);
  const int64_t m0 = tm * BM, n0 = tn * BN;

  const int count = *a.count;
  const bool compact = use_compaction(count, a.K, a.M);
  const int64_t Kl = compact ? a.K - count : a.K;

  // Y = C m s / 127^2 + X_O W_O. With int8 outlier weights W_O = q s / 127, so
  // Y = s / 127 * (C m / 127 + X_O q): the int8 part is scaled by m / 127
  // before the 16-bit MFMAs add X_O q, and s / 127 is applied last.
  const bool i8w = !F8 && a.ep.int8w != 0;
  constexpr float kDequant = F8 ? 1.0f / 200704.0f : 1.0f / 16129.0f;
  // Rows past M take a NaN row scale. Their values fall outside the Y resource
  // when stored, and fmax ignores a NaN, so the column maxima skip them with no
  // per-row test (per-element row masks would stay live across the store loop).
  for (int i = t; i < BM; i += TH) sm[i] = (m0 + i < a.M) ? a.m[m0 + i] : __builtin_nanf("");
  for (int i = t; i < BN; i += TH) {
    const float sn = (n0 + i < a.N) ? a.s[n0 + i] : 0.f;
    ss[i] = i8w ? 1.0f / 127.0f : sn * kDequant;
    sf[i] = i8w ? sn * (1.0f / 127.0f) : 1.0f;
  }

  i32x16 acc[MI * NI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) acc[mi * NI + ni] = (i32x16){};

  {
    // stages [st0, st1) of the k range: all of them, or this split's share
    const int64_t nst = (Kl + SK - 1) / SK;
    const int64_t st0 = SPLIT ? nst * split / a.ksplit : 0;
    const int64_t st1 = SPLIT ? nst * (split + 1) / a.ksplit : nst;
    OperandTile<BM, NW, SK> A;
    OperandTile<BN, NW, SK> B;
    A.init(a.xq, a.ldq, m0, a.M, st0 * SK);
    if (compact)
      B.init(a.wqc, a.ldq, n0, a.N, st0 * SK);
    else
      B.init(a.wq, a.K, n0, a.N, st0 * SK);
    kloop<BM, BN, WM, WN, MI, NI, T::NST, NW, SK, F8 ? Op::F8 : Op::I8>(
        smem, A, B, st1 - st0, wm, wn, li, lg, acc);
  }
  if constexpr (SPLIT) {
    if (!split_merge<TH, MI * NI>(a, tile, split, acc)) return;
  } else {
    // With no k stage (every column an outlier, compacted) the k-loop has run
    // no barrier, and the scales written to LDS above are not yet visible to
    // every wave. Without this, a wave could read what an earlier block left
    // in LDS (a NaN row scale of rows past M, say) into its dequantization.
    if ((Kl + SK - 1) / SK == 0) __syncthreads();
  }

  // dequantize in place: C * m[i] * s[n] / 127^2 (or / 448^2)
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
      const int cl = wn * WN + ni * 32 + li;
      const float sc = ss[cl];
      // the E4M3 sums are fp32 already (reinterpret the whole vector: a
      // per-element bit cast of the int vector was miscompiled to element 0
      // of each group of four)
      const f32x16 accf = __builtin_bit_cast(f32x16, acc[mi * NI + ni]);
      f32x16 f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int rl = wm * WM + mi * 32 + 8 * (r >> 2) + 4 * lg + (r & 3);
        const float c = F8 ? accf[r] : (float)acc[mi * NI + ni][r];
        f[r] = c * (sm[rl] * sc);
      }
      if constexpr (DBG) {
        const bool colok = n0 + cl < a.N;
        int64_t rows = a.M - m0;
        rows = rows < BM ? rows : BM;
        const rsrc_t rc = make_rsrc(a.cdbg + m0 * a.ldc, rows * a.ldc * 4);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int rl = wm * WM + mi * 32 + 8 * (r >> 2) + 4 * lg + (r & 3);
          if (colok)
            __builtin_amdgcn_raw_buffer_store_b32(acc[mi * NI + ni][r], rc,
                                                  (rl * (int)a.ldc + (int)(n0 + cl)) * 4, 0, 0);
        }
      }
      acc[mi * NI + ni] = __builtin_bit_cast(i32x16, f);
    }

  // fp16 outlier product X_O . W_O over the gathered outlier columns
  if (count > 0 && a.w) {
    OperandTile<BM, NW, SK> A;
    OperandTile<BN, NW, SK> B;
    A.init(a.xo, a.ldo * 2, m0, a.M);
    B.init(a.wot, a.ldo * 2, n0, a.N);
    kloop<BM, BN, WM, WN, MI, NI, T::NST, NW, SK, Op::F16>(smem, A, B, (2 * count + SK - 1) / SK,
                                                           wm, wn, li, lg, acc);
  }

  // store Y (fp16, round to nearest even); rows past M fall outside the resource
  int64_t rows = a.M - m0;
  rows = rows < BM ? rows : BM;
  const rsrc_t ry = make_rsrc(a.y + m0 * a.ldy, rows * a.ldy * 2);
  // the NI column blocks of a row are stored back to back, so that the wave
  // writes whole 128-byte lines of Y (the halves of a line written far apart
  // reached HBM as partial-line writes)
  bool colok[NI];
  float fin[NI], bcol[NI], cmax[NI];  // cmax: |Y| of the column over the wave's rows
#pragma unroll
  for (int ni = 0; ni < NI; ++ni) {
    const int cl = wn * WN + ni * 32 + li;
    colok[ni] = n0 + cl < a.N;
    fin[ni] = sf[cl];
    bcol[ni] = (a.ep.bias && colok[ni]) ? h2f(a.ep.bias[n0 + cl]) : 0.f;
    cmax[ni] = 0.f;
  }
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int rl = wm * WM + mi * 32 + 8 * (r >> 2) + 4 * lg + (r & 3);
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) {
        const int cl = wn * WN + ni * 32 + li;
        const float y = __builtin_bit_cast(f32x16, acc[mi * NI + ni])[r] * fin[ni] + bcol[ni];
        if (colok[ni])
          __builtin_amdgcn_raw_buffer_store_b16(f2h(y), ry,
                                                (rl * (int)a.ldy + (int)(n0 + cl)) * 2, 0, 0);
        cmax[ni] = __builtin_fmaxf(cmax[ni], stored_abs(y));
      }
    }
  if (a.ep.ycmax) {
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
      // lanes l and l + 32 hold the same column
      const float cm = __builtin_fmaxf(cmax[ni], __shfl_xor(cmax[ni], 32, 64));
      if (lg == 0 && colok[ni]) ycmax_update(a.ep.ycmax, n0 + wn * WN + ni * 32 + li, cm);
    }
  }
}

template <int BM, int BN, int NWN, int SK, bool DBG, bool F8>
__global__ __launch_bounds__(128 * NWN, 1) void k_gemm_prefill(GemmArgs a) {
  extern __shared__ u32x4 smem_v[];
  prefill_tile<BM, BN, NWN, SK, DBG, F8>(a, blockIdx.x, (uint8_t *)smem_v);
}

// Two tile shapes with the same wave count in one launch: blocks [0, blocks1)
// take the tiles of a1 (whole waves of large tiles), the rest those of a2 (the
// remaining columns in smaller tiles), which start as soon as CUs free up.
template <int BM1, int BN1, int BM2, int BN2, int NWN, int SK, bool DBG, bool F8>
__global__ __launch_bounds__(128 * NWN, 1) void k_gemm_pair(GemmArgs a1, GemmArgs a2,
                                                           int64_t blocks1) {
  extern __shared__ u32x4 smem_v[];
  const int64_t b = blockIdx.x;
  if (b < blocks1)
    prefill_tile<BM1, BN1, NWN, SK, DBG, F8>(a1, b, (uint8_t *)smem_v);
  else
    prefill_tile<BM2, BN2, NWN, SK, DBG, F8>(a2, b - blocks1, (uint8_t *)smem_v);
}

// Split-K BM x 256 int8 tiles: a.ksplit blocks per tile.
template <int BM, int NWN, int SK, bool DBG>
__global__ __launch_bounds__(128 * NWN, 1) void k_gemm_split(GemmArgs a) {
  extern __shared__ u32x4 smem_v[];
  prefill_tile<BM, 256, NWN, SK, DBG, false, true>(a, blockIdx.x, (uint8_t *)smem_v);
}

template <int BM, int NWN, int SK, bool DBG>
hipError_t launch_split(const GemmArgs &a, const GemmEvents &ev, hipStream_t stream) {
  using T = TileCfg<BM, 256, NWN, SK>;
  auto *kern = k_gemm_split<BM, NWN, SK, DBG>;
  hipError_t e = hipFuncSetAttribute((const void *)kern,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, T::LDS);
  if (e != hipSuccess) return e;
  const int64_t blocks = ((a.M + BM - 1) / BM) * ((a.N + 255) / 256) * a.ksplit;
  hipExtLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(T::THREADS), T::LDS, stream,
                        (hipEvent_t)ev.begin, (hipEvent_t)ev.end, 0u, a);
  return hipGetLastError();
}

template <int BM1, int BN1, int BM2, int BN2, int NWN, int SK, bool DBG, bool F8>
hipError_t launch_pair(const GemmArgs &a1, const GemmArgs &a2, const GemmEvents &ev,
                       hipStream_t stream) {
  using T1 = TileCfg<BM1, BN1, NWN, SK>;
  using T2 = TileCfg<BM2, BN2, NWN, SK>;
  constexpr int LDS = T1::LDS > T2::LDS ? T1::LDS : T2::LDS;
  auto *kern = k_gemm_pair<BM1, BN1, BM2, BN2, NWN, SK, DBG, F8>;
  hipError_t e = hipFuncSetAttribute((const void *)kern,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, LDS);
  if (e != hipSuccess) return e;
  const int64_t blocks1 = ((a1.M + BM1 - 1) / BM1) * ((a1.N + BN1 - 1) / BN1);
  const int64_t blocks2 = ((a2.M + BM2 - 1) / BM2) * ((a2.N + BN2 - 1) / BN2);
  hipExtLaunchKernelGGL(kern, dim3((unsigned)(blocks1 + blocks2)), dim3(T1::THREADS), LDS, stream,
                        (hipEvent_t)ev.begin, (hipEvent_t)ev.end, 0u, a1, a2, blocks1);
  return hipGetLastError();
}

template <int BM, int BN, int NWN, int SK, bool DBG, bool F8>
hipError_t launch_prefill(const GemmArgs &a, const GemmEvents &ev, hipStream_t stream) {
  using T = TileCfg<BM, BN, NWN, SK>;
  hipError_t e = hipFuncSetAttribute((const void *)k_gemm_prefill<BM, BN, NWN, SK, DBG, F8>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, T::LDS);
  if (e != hipSuccess) return e;
  const int64_t tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  hipExtLaunchKernelGGL((k_gemm_prefill<BM, BN, NWN, SK, DBG, F8>), dim3((unsigned)tiles),
                        dim3(T::THREADS), T::LDS, stream, (hipEvent_t)ev.begin,
                        (hipEvent_t)ev.end, 0u, a);
  return hipGetLastError();
}

}  // namespace gemm_detail
}  // namespace llmint8
