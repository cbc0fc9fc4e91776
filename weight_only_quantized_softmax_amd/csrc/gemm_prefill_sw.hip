// 128-row grouped dequant GEMM with weights scaled as they are decoded (tiled layout, block
// scales of 16 to 128, MX FP4): 4-bit instances; the 8-bit ones live in
// gemm_prefill_sw8.hip, so that the two halves compile in parallel.
#include "gemm_prefill_sw_kernel.h"

namespace qmoe {

// Blocks of 16 only: there the per-block FMA kernel spends two FMAs per output element per
// 32 k; from blocks of 32 on (and for MX FP4) that kernel measured faster.
bool prefill_sw_supports(const GemmArgs& g) { return g.packed && g.bs == 16 && !g.mx; }

hipError_t launch_gemm_bf16_prefill_sw(const GemmArgs& g, int mode, int bits, bool scale_bf16,
                                       int64_t max_tiles, hipStream_t s) {
  if (max_tiles <= 0) return hipSuccess;
  if (g.mx) return launch_sw_t<4, uint8_t>(g, mode, max_tiles, s);
  if (bits == 8) return launch_gemm_bf16_prefill_sw8(g, mode, scale_bf16, max_tiles, s);
  return scale_bf16 ? launch_sw_t<4, uint16_t>(g, mode, max_tiles, s)
                    : launch_sw_t<4, float>(g, mode, max_tiles, s);
}

}  // namespace qmoe
