// 128-row grouped dequant GEMM with weights scaled as they are decoded: 8-bit instances.
#include "gemm_prefill_sw_kernel.h"

namespace qmoe {

hipError_t launch_gemm_bf16_prefill_sw8(const GemmArgs& g, int mode, bool scale_bf16,
                                        int64_t max_tiles, hipStream_t s) {
  return scale_bf16 ? launch_sw_t<8, uint16_t>(g, mode, max_tiles, s)
                    : launch_sw_t<8, float>(g, mode, max_tiles, s);
}

}  // namespace qmoe
