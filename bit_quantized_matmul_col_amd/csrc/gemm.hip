// Large-M GEMM dispatch (tile shape choice).
#include "gemm_core.hpp"

namespace llmint8 {

namespace {

// waves along N of a 256x256 tile (4: two waves per SIMD) and k bytes per
// stage (128; 64-byte stages with a four-deep ring measured 7-9% slower)
constexpr int kWideWavesN = 4;
constexpr int kWideStageK = 128;

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
// tiles % cus blocks while the rest of the chip idles; giving the columns of
// those tiles to 128x256 tiles instead (half the work each, still two waves
// per SIMD, at most one wave of them) turns that wave into about half a wave.
// Both shapes run in one launch, the smaller tiles starting as CUs free up.
// (256x128 tiles with one wave per SIMD took 0.63 of a full wave for the same
// half of the work.)
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

// Fewest 128-byte stages of k that a split-K part runs, and most parts. A part
// hands its int32 sums over through memory (256 KB per part, stored and read
// back by the last part); with fewer than 16 stages per part that costs about
// what the split saves.
constexpr int64_t kSplitMinStages = 16;
constexpr int kSplitMax = 8;
// With a short k range (at most 16 stages, K <= 2048) a whole tile is short
// too, and shorter parts pay: 128 x 256 tiles split into parts of at least 4
// stages when there are at most kShortSplitFewTiles tiles, else of at least 8.
// Graph-replayed calls: 300 x 1024 x 4096 25.4 -> 23.5 us, 512 x 1024 x 1024
// 25.5 -> 23.2, 600 x 1024 x 2048 26.2 -> 24.2, 300 x 2048 x 2048 32.9 ->
// 27.6 (4 parts), 768 x 2048 x 4096 35.7 -> 32.2, 400 x 2048 x 8192 35.5 ->
// 32.8. Parts of 4 stages in 128 tiles (1024 x 1024 x 4096, 28.1 -> 30.3 us)
// and 256 x 256 tiles in parts of 4 stages (257 x 1024 x 11008, 26.2 -> 38.2
// us) were slower, so those stay whole.
constexpr int64_t kShortSplitStages = 16;
constexpr int64_t kShortSplitFewTiles = 96;

}  // namespace

// The tiles a split-K launch cuts. When a launch has fewer tiles than CUs (M
// up to several hundred rows at these widths), most of the chip would idle:
// every tile then cuts its k range into as many parts as the CUs take (at most
// kSplitMax, each at least kSplitMinStages stages, fewer for short k ranges). The tiles are 128 x 256
// when that gives a split (a three-stage ring, and no zero rows below M = 128),
// else 256 x 256. Measured on whole calls (best of six interleaved rounds),
// 256 x 256 split tiles against whole ones: 128 x 8192 x 8192 78.4 -> 56.8 us,
// 512 x 8192 x 8192 86.0 -> 72.6 us; 128 x 256 against 256 x 256 split tiles:
// 65 x 4096 x 4096 45.6 -> 33.9 us, 256 x 4096 x 4096 47.2 -> 34.9 us,
// 512 x 8192 x 8192 71.2 -> 62.1 us, 1024 x 4096 x 4096 53.8 -> 44.8 us. A
// partial last wave of a larger launch is left to the paired launch (its
// 128 x 256 tail tiles measured faster than 256 x 256 tiles split in two: 115
// against 124 us at 2048 x 4096 x 11008, 298 against 314 us at
// 4096 x 5120 x 13824). The plan is a function of the shape alone (the
// MI355X's 256 CUs, not a device query), so the workspace size query and the
// launch agree.
GemmSplitPlan gemm_split_plan(int64_t M, int64_t K, int64_t N) {
  constexpr int64_t cus = 256;
  const int64_t nst = (K + 127) / 128;
  const bool short_k = nst <= kShortSplitStages;
  for (const int bm : {128, 256}) {
    if (short_k && bm == 256) break;
    const int64_t tiles = ((M + bm - 1) / bm) * ((N + 255) / 256);
    if (tiles >= cus) continue;
    const int64_t min_st = !short_k ? kSplitMinStages : tiles <= kShortSplitFewTiles ? 4 : 8;
    int64_t S = cus / tiles;
    if (S > kSplitMax) S = kSplitMax;
    while (S > 1 && nst < S * min_st) --S;
    if (S >= 2) return GemmSplitPlan{tiles, (int)S, bm};
  }
  return GemmSplitPlan{0, 1, 256};
}

namespace {

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
  if (a.part && a.sem && !a.fp8) {
    const GemmSplitPlan p = gemm_split_plan(a.M, a.K, a.N);
    if (p.ksplit > 1 && p.tiles * p.ksplit * split_slot_bytes(p.bm) <= a.part_bytes) {
      a.ksplit = p.ksplit;
      return launch_gemm_split(a, p.bm, ev, stream);
    }
  }
  const int cus = cu_count();
  if (narrow_tiles(a.M, a.N, cus)) return launch_gemm_narrow(a, ev, stream);
  const int64_t n1 = wide_columns(a.M, a.N, cus);
  if (n1 == 0) return launch_gemm_wide(a, ev, stream);
  return launch_gemm_pair(column_slice(a, 0, n1), column_slice(a, n1, a.N - n1), ev, stream);
}

}  // namespace llmint8
