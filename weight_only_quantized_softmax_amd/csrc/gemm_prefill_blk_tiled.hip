// 128-row block-scale grouped dequant GEMM, tiled weight layout (qmoe_pack_stack).
#include "gemm_prefill_blk_kernel.h"

namespace qmoe {

hipError_t launch_gemm_bf16_prefill_blk_tiled(const GemmArgs& g, int mode, int bits,
                                              bool scale_bf16, int64_t max_tiles, hipStream_t s) {
  return launch_blk_layout<true>(g, mode, bits, scale_bf16, max_tiles, s);
}

}  // namespace qmoe
