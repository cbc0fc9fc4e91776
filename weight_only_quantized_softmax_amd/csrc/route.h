// Softmax-top-k routing of one token by one wavefront, shared by the routing kernel and
// the fused routing-and-grouping kernel.
//
// CLIKA "MoE" page: each token goes to its top-k experts, whose outputs are summed with the
// routing weights as coefficients (routing_mode "softmax_topk", renormalize);
// graiphic "QMoE" page: attributes k and normalize_routing_weights.
//
// A token is routed by a group of G lanes: a whole wave (G = 64), or one 16-lane DPP row
// (G = 16, four tokens a wave, where E <= 256 and k <= 16). Lane l of the group holds the
// logits of experts [l*V, l*V+V), so a lower lane always holds lower expert indices.
// Selection works on an order-preserving integer image of the logit (after folding -0
// into +0), reduced across the group with DPP max steps (and a swizzle and readlanes for
// the whole wave); among lanes holding the maximum, the lowest lane wins (ballot +
// count-trailing-zeros), and inside a lane the lowest slot, which gives "equal logits:
// lower index first".
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

// Reductions over the G lanes routing one token; every lane of the group gets the result.
template <int G>
__device__ __forceinline__ uint32_t group_max_u32(uint32_t v) {
  static_assert(G == 16 || G == 64, "a token is routed by a DPP row or a wave");
  if constexpr (G == 64) {
    return wave_max_u32(v);
  } else {
    v = max(v, dpp<QMOE_DPP_QUAD_1032>(v));
    v = max(v, dpp<QMOE_DPP_QUAD_2301>(v));
    v = max(v, dpp<QMOE_DPP_ROW_HALF_MIRROR>(v));
    return max(v, dpp<QMOE_DPP_ROW_MIRROR>(v));
  }
}

template <int G>
__device__ __forceinline__ float group_sum_f32(float f) {
  if constexpr (G == 64) return wave_sum_f32(f);
  else return row16_sum_f32(f);
}

// The value of x in lane src (an absolute lane of the caller's group).
template <int G>
__device__ __forceinline__ uint32_t group_read(uint32_t x, int src) {
  if constexpr (G == 64) return __builtin_amdgcn_readlane(x, src);
  else return static_cast<uint32_t>(__shfl(static_cast<int>(x), src));
}

// The logits of one token as its group holds them.
template <int V>
struct TokenLogits {
  float val[V];      // the logits (-inf past E)
  uint32_t key[V];   // selection keys: order_key(logit + bias), 0 past E
  uint32_t lkmax;    // the lane's largest order_key of the logits alone
};

// Loads token t's logits (and the selection bias) into the group's registers.
template <typename TA, int G, int V>
__device__ __forceinline__ void load_token(const TA* logits, int t, int E, const RouteOpts& o,
                                           TokenLogits<V>& r) {
  const int gl = lane_id() & (G - 1);
  const TA* row = logits + static_cast<int64_t>(t) * E;
  const TA* bias = static_cast<const TA*>(o.bias);
  r.lkmax = 0u;
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const int e = gl * V + v;
    r.val[v] = e < E ? load_elem(row, e) : -INFINITY;
    r.lkmax = max(r.lkmax, e < E ? order_key(r.val[v]) : 0u);  // 0 is below every finite key
    const float sel = (bias != nullptr && e < E) ? r.val[v] + load_elem(bias, e) : r.val[v];
    r.key[v] = e < E ? order_key(sel) : 0u;
  }
}

// The sparse mixer routing of token t (graiphic "QMoE" page, use_sparse_mixer; CLIKA "MoE"
// page, sparse_mixer_eps), read from its published definition (the SparseMixer top-2
// router of Phi-3.5-MoE): two picks, the largest logit m1 and then the largest of the
// others m2 (equal logits: the lower index, as in the top-k). Pick j keeps expert e unless
// (mj - l_e) / max(|l_e|, mj) > 2 eps, decided in fp32 with a correctly rounded division
// (0/0 keeps it); pick 2 never keeps pick 1. Pick j's weight is the softmax at the picked
// expert over the experts it keeps, 1 / sum_kept exp(l_e - mj), times the scaling factor.
// Lanes 0 and 1 of the group write the two slots.
template <int G, int V>
__device__ __forceinline__ void route_mixer(TokenLogits<V>& r, int t, int E, const RouteOpts& o,
                                            int32_t* topk_ids, float* topk_w) {
  const int lane = lane_id();
  const int gl = lane & (G - 1);
  const int gbase = lane - gl;
  const uint64_t gmask = G == 64 ? ~0ull : ((1ull << G) - 1ull);
  const float thr = 2.0f * o.mixer_eps;
  float my_w = 0.f;
  int my_id = 0;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    uint32_t best = r.key[0];
    int bslot = 0;
#pragma unroll
    for (int v = 1; v < V; ++v)
      if (r.key[v] > best) { best = r.key[v]; bslot = v; }
    const uint32_t gmax = group_max_u32<G>(best);
    const uint64_t holders = (ballot(best == gmax) >> gbase) & gmask;
    const int src = gbase + __builtin_ctzll(holders);
    const int idx = static_cast<int>(group_read<G>(static_cast<uint32_t>(gl * V + bslot), src));
    const float m = key_value(gmax);  // the pick's logit (-0 read as +0: the same decisions)
    if (lane == src) {
#pragma unroll
      for (int v = 0; v < V; ++v)
        if (v == bslot) r.key[v] = 0u;  // leaves later picks and pick 2's softmax
    }
    // the experts this pick keeps: every expert for pick 1; for pick 2 every expert but
    // pick 1 (whose key is now 0, as are the keys past E)
    float part = 0.f;
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const int e = gl * V + v;
      const bool cand = e < E && (j == 0 || r.key[v] != 0u || e == idx);
      const float l = r.val[v];
      const bool drop = __fdiv_rn(m - l, fmaxf(fabsf(l), m)) > thr;
      if (cand && !drop) part += expf(l - m);
    }
    const float w = 1.0f / group_sum_f32<G>(part);
    if (gl == j) {
      my_w = w;
      my_id = idx;
    }
  }
  if (gl < 2) {
    topk_ids[static_cast<int64_t>(t) * 2 + gl] = my_id;
    topk_w[static_cast<int64_t>(t) * 2 + gl] = o.scale != 1.0f ? my_w * o.scale : my_w;
  }
}

// Routes token t from its loaded logits (all G lanes of the group call this with the same
// t): lanes j < k of the group write its j-th expert id and weight to topk_ids[t*k + j] and
// topk_w[t*k + j].
// Routing variants (RouteOpts; CLIKA "MoE" page routing kwargs n_group, topk_group,
// routed_scaling_factor; ClikaRT "QMoEWoQ" page, e_score_correction_bias [E], a per-expert
// bias for the choice of experts): the bias is added to the logits in fp32 for the selection
// only; with n_group > 1 the experts form n_group groups of E / n_group consecutive
// indices, a group scores the largest selection key of its experts, the topk_group best
// groups (ties to the lower group) are kept and the k experts are chosen among theirs;
// the weights are the softmax over all E logits at the chosen experts, renormalised if
// asked, then multiplied by the scaling factor.
template <int G, int V>
__device__ __forceinline__ void route_loaded(TokenLogits<V>& r, int t, int E, int k,
                                             int normalize, const RouteOpts& o,
                                             int32_t* topk_ids, float* topk_w) {
  if (o.mixer) {
    route_mixer<G, V>(r, t, E, o, topk_ids, topk_w);
    return;
  }
  const int lane = lane_id();
  const int gl = lane & (G - 1);
  const int gbase = lane - gl;
  float* val = r.val;
  uint32_t* key = r.key;

  // Softmax over all E: the maximum and the normaliser come first.
  const float m = key_value(group_max_u32<G>(r.lkmax));
  float part = 0.f;
#pragma unroll
  for (int v = 0; v < V; ++v)
    if (gl * V + v < E) part += expf(val[v] - m);
  const float denom = group_sum_f32<G>(part);

  if (o.n_group > 1) {
    // group scores (the same in every lane), then the kept groups
    const int gsize = E / o.n_group;
    uint32_t gsc[kMaxGroups];
#pragma unroll
    for (int gi = 0; gi < kMaxGroups; ++gi) {
      gsc[gi] = 0u;
      if (gi < o.n_group) {  // uniform: the group's lanes all take it
        uint32_t local = 0u;
#pragma unroll
        for (int v = 0; v < V; ++v) {
          const int e = gl * V + v;
          if (e < E && e / gsize == gi) local = max(local, key[v]);
        }
        gsc[gi] = group_max_u32<G>(local);
      }
    }
    uint32_t keep = 0u;
    for (int rr = 0; rr < o.topk_group; ++rr) {
      int bg = -1;
      uint32_t bs = 0u;
#pragma unroll
      for (int gi = 0; gi < kMaxGroups; ++gi)
        if (gi < o.n_group && !((keep >> gi) & 1u) && (bg < 0 || gsc[gi] > bs)) {
          bg = gi;
          bs = gsc[gi];
        }
      keep |= 1u << bg;
    }
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const int e = gl * V + v;
      if (e < E && !((keep >> (e / gsize)) & 1u)) key[v] = 0u;
    }
  }

  // slot j's id and weight stay in lane j of the group (k <= G), so nothing is read back
  float sum = 0.f, my_w = 0.f;
  int my_id = 0;
  const uint64_t gmask = G == 64 ? ~0ull : ((1ull << G) - 1ull);
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
    const uint32_t gmax = group_max_u32<G>(best);
    const uint64_t holders = (ballot(best == gmax) >> gbase) & gmask;
    const int src = gbase + __builtin_ctzll(holders);
    const int idx = static_cast<int>(group_read<G>(static_cast<uint32_t>(gl * V + bslot), src));
    // the chosen expert's own logit (the weight ignores the selection bias)
    const float lv = __uint_as_float(group_read<G>(__float_as_uint(bval), src));
    if (lane == src) {
#pragma unroll
      for (int v = 0; v < V; ++v)
        if (v == bslot) key[v] = 0u;
    }
    const float w = expf(lv - m) / denom;
    sum += w;
    if (gl == j) {
      my_w = w;
      my_id = idx;
    }
  }
  if (gl < k) {
    float w = normalize ? my_w / sum : my_w;
    if (o.scale != 1.0f) w *= o.scale;
    topk_ids[static_cast<int64_t>(t) * k + gl] = my_id;
    topk_w[static_cast<int64_t>(t) * k + gl] = w;
  }
}

// Loads and routes token t.
template <typename TA, int G, int V>
__device__ __forceinline__ void route_token(const TA* logits, int t, int E, int k, int normalize,
                                            const RouteOpts& o, int32_t* topk_ids, float* topk_w) {
  TokenLogits<V> r;
  load_token<TA, G, V>(logits, t, E, o, r);
  route_loaded<G, V>(r, t, E, k, normalize, o, topk_ids, topk_w);
}

// A token takes one 16-lane row where its experts fit 16 slots a lane and its k slots fit
// the row's lanes; else a whole wave.
inline bool route_by_rows(int E, int k) { return E <= 256 && k <= 16; }

}  // namespace qmoe
