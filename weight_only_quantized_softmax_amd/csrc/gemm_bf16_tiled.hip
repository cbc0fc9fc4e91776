// 16-row grouped dequant GEMM (decode shapes), tiled weight layout (qmoe_pack_stack).
#include "gemm_bf16_kernel.h"

namespace qmoe {

hipError_t launch_gemm_bf16_tiled(const GemmArgs& g, int mode, int bits, bool scale_bf16,
                                  int64_t max_tiles, hipStream_t s) {
  return launch_gemm_bf16_layout<true>(g, mode, bits, scale_bf16, max_tiles, s);
}

}  // namespace qmoe
