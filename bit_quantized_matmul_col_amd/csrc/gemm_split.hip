// Split-K instantiation of the large-M GEMM (its own translation unit): when a
// launch has fewer 256x256 tiles than CUs, each tile's k range is cut into
// parts that run on otherwise idle CUs.
#include "gemm_core.hpp"

namespace llmint8 {

hipError_t launch_gemm_split(const GemmArgs &a, const GemmEvents &ev, hipStream_t stream) {
  using namespace gemm_detail;
  return a.cdbg ? launch_split<4, 128, true>(a, ev, stream)
                : launch_split<4, 128, false>(a, ev, stream);
}

}  // namespace llmint8
