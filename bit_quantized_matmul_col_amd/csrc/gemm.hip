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
  const int cus = cu_count();
  if (narrow_tiles(a.M, a.N, cus)) return launch_gemm_narrow(a, ev, stream);
  const int64_t n1 = wide_columns(a.M, a.N, cus);
  if (n1 == 0) return launch_gemm_wide(a, ev, stream);
  return launch_gemm_pair(column_slice(a, 0, n1), column_slice(a, n1, a.N - n1), ev, stream);
}

}  // namespace llmint8
