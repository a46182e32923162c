// 256x128-tile (4 waves) and 128x256-tile (8 waves) instantiations of the
// large-M GEMM (their own translation unit).
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

hipError_t launch_gemm_tail(const GemmArgs &a, const GemmEvents &ev, hipStream_t stream) {
  using namespace gemm_detail;
  if (a.fp8)
    return a.cdbg ? launch_prefill<128, 256, 4, 128, true, true>(a, ev, stream)
                  : launch_prefill<128, 256, 4, 128, false, true>(a, ev, stream);
  return a.cdbg ? launch_prefill<128, 256, 4, 128, true, false>(a, ev, stream)
                : launch_prefill<128, 256, 4, 128, false, false>(a, ev, stream);
}

}  // namespace llmint8
