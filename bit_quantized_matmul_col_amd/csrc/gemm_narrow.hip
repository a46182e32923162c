// 256x128-tile (4 waves) instantiation of the large-M GEMM and the launch that
// pairs 256x256 and 128x256 tiles (their own translation unit).
#include "gemm_core.hpp"

namespace llmint8 {

hipError_t launch_gemm_narrow(const GemmArgs &a, const GemmEvents &ev, hipStream_t stream) {
  using namespace gemm_detail;
  if (a.fp8)
    return a.cdbg ? launch_prefill<256, 128, 2, 128, true, true>(a, ev, stream)
                  : launch_prefill<256, 128, 2, 128, false, true>(a, ev, stream);
  return a.cdbg ? launch_prefill<256, 128, 2, 128, true, false>(a, ev, stream)
                : launch_prefill<256, 128, 2, 128, false, false>(a, ev, stream);
}

// 256x256 tiles (8 waves) for a1, 128x256 tiles (8 waves) for a2, one launch.
hipError_t launch_gemm_pair(const GemmArgs &a1, const GemmArgs &a2, const GemmEvents &ev,
                            hipStream_t stream) {
  using namespace gemm_detail;
  if (a1.fp8)
    return a1.cdbg ? launch_pair<256, 256, 128, 256, 4, 128, true, true>(a1, a2, ev, stream)
                   : launch_pair<256, 256, 128, 256, 4, 128, false, true>(a1, a2, ev, stream);
  return a1.cdbg ? launch_pair<256, 256, 128, 256, 4, 128, true, false>(a1, a2, ev, stream)
                 : launch_pair<256, 256, 128, 256, 4, 128, false, false>(a1, a2, ev, stream);
}

}  // namespace llmint8
