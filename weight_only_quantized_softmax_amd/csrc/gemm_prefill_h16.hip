// 128-row grouped dequant GEMM on fp16 matrix cores for 4-bit codes with bf16 block scales
// (gemm_prefill_h16_kernel.h): the instances and their dispatch.
#include "gemm_prefill_h16_kernel.h"

namespace qmoe {

hipError_t launch_gemm_h16_prefill(const GemmArgs& g, int mode, int64_t max_tiles, hipStream_t s) {
  if (max_tiles <= 0) return hipSuccess;
  if (g.bs < 16 || g.bs > 128 || g.K % 8 != 0) return hipErrorInvalidValue;
  if (mode == kModeSwiglu) return launch_h16_mode<kModeSwiglu>(g, max_tiles, s);
  if (mode == kModePlainAct) return launch_h16_mode<kModePlainAct>(g, max_tiles, s);
  return launch_h16_mode<kModeFc2>(g, max_tiles, s);
}

}  // namespace qmoe
