// Softmax-top-k routing of one token by one wavefront, shared by the routing kernel and
// the fused routing-and-grouping kernel.
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
#pragma once

#include "common.h"

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

// Routes token t (the whole wave calls this with the same t): writes its k expert ids and
// weights to topk_ids[t*k ..] and topk_w[t*k ..] from lane 0.
template <typename TA, int V>
__device__ __forceinline__ void route_token(const TA* logits, int t, int E, int k, int normalize,
                                            int32_t* topk_ids, float* topk_w) {
  const int lane = lane_id();
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

}  // namespace qmoe
