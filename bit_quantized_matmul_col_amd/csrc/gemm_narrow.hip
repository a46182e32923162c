// 256x128-tile instantiation of the large-M GEMM (its own translation unit).
#include "gemm_core.hpp"

namespace llmint8 {

hipError_t launch_gemm_narrow(const GemmArgs &a, const GemmEvents &ev, hipStream_t stream) {
  return a.cdbg ? gemm_detail::launch_prefill<256, 128, 2, 128, true>(a, ev, stream)
                : gemm_detail::launch_prefill<256, 128, 2, 128, false>(a, ev, stream);
}

}  // namespace llmint8
