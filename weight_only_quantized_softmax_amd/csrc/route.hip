// Softmax-top-k routing: one 16-lane row or one wavefront per token (the per-token
// routine and its tie rule are in route.h).
#include "common.h"
#include "launch.h"
#include "route.h"

namespace qmoe {

template <typename TA, int G, int V>
__global__ __launch_bounds__(256) void route_kernel(const TA* __restrict__ logits, int T, int E,
                                                    int k, int normalize, RouteOpts o,
                                                    int32_t* __restrict__ topk_ids,
                                                    float* __restrict__ topk_w) {
  const int wave = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  const int t = wave * (kWave / G) + (threadIdx.x % kWave) / G;
  if (t >= T) return;  // uniform per group of G lanes
  route_token<TA, G, V>(logits, t, E, k, normalize, o, topk_ids, topk_w);
}

template <typename TA, int G>
static void launch_route_g(const TA* logits, int T, int E, int k, int normalize,
                           const RouteOpts& o, int32_t* ids, float* w, hipStream_t s) {
  // below four waves per CU, one wave a block, so that the waves spread over every CU
  const int64_t waves = (static_cast<int64_t>(T) * G + kWave - 1) / kWave;
  const int waves_per_block = waves >= 4 * 256 ? 4 : 1;
  const int tokens_per_block = waves_per_block * (kWave / G);
  dim3 grid((T + tokens_per_block - 1) / tokens_per_block), block(kWave * waves_per_block);
  const int V = (E + G - 1) / G;
  if (V <= 1)
    route_kernel<TA, G, 1><<<grid, block, 0, s>>>(logits, T, E, k, normalize, o, ids, w);
  else if (V <= 2)
    route_kernel<TA, G, 2><<<grid, block, 0, s>>>(logits, T, E, k, normalize, o, ids, w);
  else if (V <= 4)
    route_kernel<TA, G, 4><<<grid, block, 0, s>>>(logits, T, E, k, normalize, o, ids, w);
  else if (V <= 8)
    route_kernel<TA, G, 8><<<grid, block, 0, s>>>(logits, T, E, k, normalize, o, ids, w);
  else
    route_kernel<TA, G, 16><<<grid, block, 0, s>>>(logits, T, E, k, normalize, o, ids, w);
}

template <typename TA>
static hipError_t launch_route_t(const TA* logits, int T, int E, int k, int normalize,
                                 const RouteOpts& o, int32_t* ids, float* w, hipStream_t s) {
  if (route_by_rows(E, k))
    launch_route_g<TA, 16>(logits, T, E, k, normalize, o, ids, w, s);
  else
    launch_route_g<TA, 64>(logits, T, E, k, normalize, o, ids, w, s);
  return hipGetLastError();
}

hipError_t launch_route(const void* logits, bool bf16, int T, int E, int k, int normalize,
                        const RouteOpts& o, int32_t* ids, float* w, hipStream_t s) {
  if (bf16)
    return launch_route_t(static_cast<const uint16_t*>(logits), T, E, k, normalize, o, ids, w, s);
  return launch_route_t(static_cast<const float*>(logits), T, E, k, normalize, o, ids, w, s);
}

}  // namespace qmoe
