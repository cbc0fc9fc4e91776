// 16-row grouped dequant GEMM (decode shapes), rows weight layout; the tiled layout's
// instances live in gemm_bf16_tiled.hip, so that the two halves compile in parallel.
#include "gemm_bf16_kernel.h"

namespace qmoe {

hipError_t launch_gemm_bf16(const GemmArgs& g, int mode, int bits, bool scale_bf16,
                            int64_t max_tiles, hipStream_t s) {
  if (g.packed) return launch_gemm_bf16_tiled(g, mode, bits, scale_bf16, max_tiles, s);
  return launch_gemm_bf16_layout<false>(g, mode, bits, scale_bf16, max_tiles, s);
}

}  // namespace qmoe
