// The int8 activation tier's dot at 128-row tiles (v_mfma_i32_16x16x64_i8): dispatch.
#include "gemm_prefill_i8_kernel.h"

namespace qmoe {

bool prefill_i8_supports(const GemmArgs& g, int bits) {
  (void)bits;
  return g.packed && !g.mx && g.M == 128 && (g.bs == 64 || g.bs == 128) && g.K % 64 == 0;
}

hipError_t launch_gemm_i8_prefill(const GemmArgs& g, int mode, int bits, bool scale_bf16,
                                  int64_t max_tiles, hipStream_t s) {
  if (max_tiles <= 0) return hipSuccess;
  if (bits == 4)
    return scale_bf16 ? launch_i8_t<4, uint16_t>(g, mode, max_tiles, s)
                      : launch_i8_t<4, float>(g, mode, max_tiles, s);
  return scale_bf16 ? launch_i8_t<8, uint16_t>(g, mode, max_tiles, s)
                    : launch_i8_t<8, float>(g, mode, max_tiles, s);
}

}  // namespace qmoe
