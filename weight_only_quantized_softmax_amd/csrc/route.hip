// Softmax-top-k routing: one wavefront per token (the per-token routine and its
// tie rule are in route.h).
#include "common.h"
#include "launch.h"
#include "route.h"

namespace qmoe {

template <typename TA, int V>
__global__ __launch_bounds__(256) void route_kernel(const TA* __restrict__ logits, int T, int E,
                                                    int k, int normalize, RouteOpts o,
                                                    int32_t* __restrict__ topk_ids,
                                                    float* __restrict__ topk_w) {
  const int t = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (t >= T) return;  // uniform per wave
  route_token<TA, V>(logits, t, E, k, normalize, o, topk_ids, topk_w);
}

template <typename TA>
static hipError_t launch_route_t(const TA* logits, int T, int E, int k, int normalize,
                                 const RouteOpts& o, int32_t* ids, float* w, hipStream_t s) {
  const int waves_per_block = 4;
  dim3 grid((T + waves_per_block - 1) / waves_per_block), block(64 * waves_per_block);
  const int V = (E + 63) / 64;
  if (V <= 1)
    route_kernel<TA, 1><<<grid, block, 0, s>>>(logits, T, E, k, normalize, o, ids, w);
  else if (V <= 2)
    route_kernel<TA, 2><<<grid, block, 0, s>>>(logits, T, E, k, normalize, o, ids, w);
  else if (V <= 4)
    route_kernel<TA, 4><<<grid, block, 0, s>>>(logits, T, E, k, normalize, o, ids, w);
  else if (V <= 8)
    route_kernel<TA, 8><<<grid, block, 0, s>>>(logits, T, E, k, normalize, o, ids, w);
  else
    route_kernel<TA, 16><<<grid, block, 0, s>>>(logits, T, E, k, normalize, o, ids, w);
  return hipGetLastError();
}

hipError_t launch_route(const void* logits, bool bf16, int T, int E, int k, int normalize,
                        const RouteOpts& o, int32_t* ids, float* w, hipStream_t s) {
  if (bf16)
    return launch_route_t(static_cast<const uint16_t*>(logits), T, E, k, normalize, o, ids, w, s);
  return launch_route_t(static_cast<const float*>(logits), T, E, k, normalize, o, ids, w, s);
}

}  // namespace qmoe
