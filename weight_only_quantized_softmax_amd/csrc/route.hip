// Softmax-top-k routing: one wavefront per token.
//
// CLIKA "MoE" page: the router picks the top-k experts of each token and the outputs
// combine under the router weights (routing_mode "softmax_topk", renormalize);
// graiphic "QMoE" page: attributes k and normalize_routing_weights.
//
// Lane l holds the logits of experts [l*V, l*V+V), so a lower lane always holds lower
// expert indices. Selection works on an order-preserving integer image of the logit
// (after folding -0 into +0), reduced across the wave with DPP/swizzle max steps; among
// lanes holding the maximum, the lowest lane wins (ballot + count-trailing-zeros), and
// inside a lane the lowest slot, which gives "equal logits: lower index first".
#include "common.h"
#include "launch.h"

namespace qmoe {

__device__ __forceinline__ uint32_t order_key(float f) {
  if (f == 0.0f) f = 0.0f;  // -0 and +0 compare equal
  uint32_t b = __float_as_uint(f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ float key_value(uint32_t k) {
  uint32_t b = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(b);
}

template <typename TA, int V>
__global__ __launch_bounds__(256) void route_kernel(const TA* __restrict__ logits, int T, int E,
                                                    int k, int normalize,
                                                    int32_t* __restrict__ topk_ids,
                                                    float* __restrict__ topk_w) {
  const int lane = lane_id();
  const int t = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (t >= T) return;  // uniform per wave

  float val[V];
  uint32_t key[V];
  const TA* row = logits + static_cast<int64_t>(t) * E;
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const int e = lane * V + v;
    val[v] = e < E ? load_elem(row, e) : -INFINITY;
    key[v] = e < E ? order_key(val[v]) : 0u;  // 0 is below every finite key
  }

  // Softmax over all E: the maximum and the normaliser come first.
  uint32_t best0 = key[0];
#pragma unroll
  for (int v = 1; v < V; ++v) best0 = max(best0, key[v]);
  const float m = key_value(wave_max_u32(best0));
  float part = 0.f;
#pragma unroll
  for (int v = 0; v < V; ++v)
    if (lane * V + v < E) part += expf(val[v] - m);
  const float denom = wave_sum_f32(part);

  int32_t* ids_out = topk_ids + static_cast<int64_t>(t) * k;
  float* w_out = topk_w + static_cast<int64_t>(t) * k;
  float sum = 0.f;
  for (int j = 0; j < k; ++j) {
    uint32_t best = key[0];
    int bslot = 0;
#pragma unroll
    for (int v = 1; v < V; ++v)
      if (key[v] > best) { best = key[v]; bslot = v; }
    const uint32_t wmax = wave_max_u32(best);
    const uint64_t holders = ballot(best == wmax);
    const int src = __builtin_ctzll(holders);
    const int idx = __builtin_amdgcn_readlane(lane * V + bslot, src);
    if (lane == src) {
#pragma unroll
      for (int v = 0; v < V; ++v)
        if (v == bslot) key[v] = 0u;
    }
    const float w = expf(key_value(wmax) - m) / denom;
    sum += w;
    if (lane == 0) {
      ids_out[j] = idx;
      w_out[j] = w;
    }
  }
  if (normalize && lane == 0)
    for (int j = 0; j < k; ++j) w_out[j] = w_out[j] / sum;
}

template <typename TA>
static hipError_t launch_route_t(const TA* logits, int T, int E, int k, int normalize,
                                 int32_t* ids, float* w, hipStream_t s) {
  const int waves_per_block = 4;
  dim3 grid((T + waves_per_block - 1) / waves_per_block), block(64 * waves_per_block);
  const int V = (E + 63) / 64;
  if (V <= 1)
    route_kernel<TA, 1><<<grid, block, 0, s>>>(logits, T, E, k, normalize, ids, w);
  else if (V <= 2)
    route_kernel<TA, 2><<<grid, block, 0, s>>>(logits, T, E, k, normalize, ids, w);
  else if (V <= 4)
    route_kernel<TA, 4><<<grid, block, 0, s>>>(logits, T, E, k, normalize, ids, w);
  else if (V <= 8)
    route_kernel<TA, 8><<<grid, block, 0, s>>>(logits, T, E, k, normalize, ids, w);
  else
    route_kernel<TA, 16><<<grid, block, 0, s>>>(logits, T, E, k, normalize, ids, w);
  return hipGetLastError();
}

hipError_t launch_route(const void* logits, bool bf16, int T, int E, int k, int normalize,
                        int32_t* ids, float* w, hipStream_t s) {
  if (bf16)
    return launch_route_t(static_cast<const uint16_t*>(logits), T, E, k, normalize, ids, w, s);
  return launch_route_t(static_cast<const float*>(logits), T, E, k, normalize, ids, w, s);
}

}  // namespace qmoe
