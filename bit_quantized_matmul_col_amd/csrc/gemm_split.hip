// Split-K instantiations of the large-M GEMM (their own translation unit): when
// a launch has fewer tiles than CUs, each tile's k range is cut into parts
// that run on otherwise idle CUs, in 128 x 256 tiles (a three-stage ring) or
// 256 x 256 ones, as the split plan picks.
#include "gemm_core.hpp"

namespace llmint8 {

hipError_t launch_gemm_split(const GemmArgs &a, int bm, const GemmEvents &ev, hipStream_t stream) {
  using namespace gemm_detail;
  if (bm == 128)
    return a.cdbg ? launch_split<128, 4, 128, true>(a, ev, stream)
                  : launch_split<128, 4, 128, false>(a, ev, stream);
  return a.cdbg ? launch_split<256, 4, 128, true>(a, ev, stream)
                : launch_split<256, 4, 128, false>(a, ev, stream);
}

}  // namespace llmint8
