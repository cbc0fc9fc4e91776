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

// Routes token t (the whole wave calls this with the same t): writes its k expert ids and
// weights to topk_ids[t*k ..] and topk_w[t*k ..] from lane 0.
// Routing variants (RouteOpts; CLIKA "MoE" page routing kwargs n_group, topk_group,
// routed_scaling_factor; ClikaRT "QMoEWoQ" page, the aux-free selection bias
// e_score_correction_bias [E]): the bias is added to the logits in fp32 for the selection
// only; with n_group > 1 the experts form n_group groups of E / n_group consecutive
// indices, a group scores the largest selection key of its experts, the topk_group best
// groups (ties to the lower group) are kept and the k experts are chosen among theirs;
// the weights are the softmax over all E logits at the chosen experts, renormalised if
// asked, then multiplied by the scaling factor.
template <typename TA, int V>
__device__ __forceinline__ void route_token(const TA* logits, int t, int E, int k, int normalize,
                                            const RouteOpts& o, int32_t* topk_ids, float* topk_w) {
  const int lane = lane_id();
  float val[V];
  uint32_t key[V];  // selection key per slot
  uint32_t lkmax = 0u;
  const TA* row = logits + static_cast<int64_t>(t) * E;
  const TA* bias = static_cast<const TA*>(o.bias);
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const int e = lane * V + v;
    val[v] = e < E ? load_elem(row, e) : -INFINITY;
    lkmax = max(lkmax, e < E ? order_key(val[v]) : 0u);  // 0 is below every finite key
    const float sel = (bias != nullptr && e < E) ? val[v] + load_elem(bias, e) : val[v];
    key[v] = e < E ? order_key(sel) : 0u;
  }

  // Softmax over all E: the maximum and the normaliser come first.
  const float m = key_value(wave_max_u32(lkmax));
  float part = 0.f;
#pragma unroll
  for (int v = 0; v < V; ++v)
    if (lane * V + v < E) part += expf(val[v] - m);
  const float denom = wave_sum_f32(part);

  if (o.n_group > 1) {
    // group scores (the same in every lane), then the kept groups
    const int gsize = E / o.n_group;
    uint32_t gsc[kMaxGroups];
#pragma unroll
    for (int gi = 0; gi < kMaxGroups; ++gi) {
      if (gi >= o.n_group) break;
      uint32_t local = 0u;
#pragma unroll
      for (int v = 0; v < V; ++v) {
        const int e = lane * V + v;
        if (e < E && e / gsize == gi) local = max(local, key[v]);
      }
      gsc[gi] = wave_max_u32(local);
    }
    uint32_t keep = 0u;
    for (int r = 0; r < o.topk_group; ++r) {
      int bg = -1;
      uint32_t bs = 0u;
#pragma unroll
      for (int gi = 0; gi < kMaxGroups; ++gi) {
        if (gi >= o.n_group) break;
        if (!((keep >> gi) & 1u) && (bg < 0 || gsc[gi] > bs)) { bg = gi; bs = gsc[gi]; }
      }
      keep |= 1u << bg;
    }
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const int e = lane * V + v;
      if (e < E && !((keep >> (e / gsize)) & 1u)) key[v] = 0u;
    }
  }

  int32_t* ids_out = topk_ids + static_cast<int64_t>(t) * k;
  float* w_out = topk_w + static_cast<int64_t>(t) * k;
  float sum = 0.f;
  for (int j = 0; j < k; ++j) {
    uint32_t best = key[0];
    int bslot = 0;
#pragma unroll
    for (int v = 1; v < V; ++v)
      if (key[v] > best) { best = key[v]; bslot = v; }
    float bval = val[0];
#pragma unroll
    for (int v = 1; v < V; ++v)
      if (v == bslot) bval = val[v];
    const uint32_t wmax = wave_max_u32(best);
    const uint64_t holders = ballot(best == wmax);
    const int src = __builtin_ctzll(holders);
    const int idx = __builtin_amdgcn_readlane(lane * V + bslot, src);
    // the chosen expert's own logit (the weight ignores the selection bias)
    const float lv = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(bval), src));
    if (lane == src) {
#pragma unroll
      for (int v = 0; v < V; ++v)
        if (v == bslot) key[v] = 0u;
    }
    const float w = expf(lv - m) / denom;
    sum += w;
    if (lane == 0) {
      ids_out[j] = idx;
      w_out[j] = w;
    }
  }
  if (lane == 0) {
    for (int j = 0; j < k; ++j) {
      float w = normalize ? w_out[j] / sum : w_out[j];
      if (o.scale != 1.0f) w *= o.scale;
      w_out[j] = w;
    }
  }
}

}  // namespace qmoe
