// 128-row block-scale grouped dequant GEMM, rows weight layout; the tiled layout's
// instances live in gemm_prefill_blk_tiled.hip, so that the two halves compile in parallel.
#include "gemm_prefill_blk_kernel.h"

namespace qmoe {

bool prefill_blk_supports(const GemmArgs& g, int bits) {
  if (g.packed) return g.bs > 0;
  return g.bs > 0 && g.K % (bits == 4 ? 128 : 64) == 0 && (bits == 4 || g.bs >= 64);
}

hipError_t launch_gemm_bf16_prefill_blk(const GemmArgs& g, int mode, int bits, bool scale_bf16,
                                        int64_t max_tiles, hipStream_t s) {
  if (g.packed) return launch_gemm_bf16_prefill_blk_tiled(g, mode, bits, scale_bf16, max_tiles, s);
  return launch_blk_layout<false>(g, mode, bits, scale_bf16, max_tiles, s);
}

}  // namespace qmoe
