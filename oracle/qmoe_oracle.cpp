/*
 * qmoe_oracle.cpp -- TEST INFRASTRUCTURE ONLY (see qmoe_oracle.h).
 *
 * Plain fp64 evaluation of the weight-only-quantized MoE forward. Every value
 * is widened exactly to double, every product and sum is formed in double in
 * plain ascending loops, and only the final output is rounded (once) to the
 * activation dtype. Speed is not a goal: weights are dequantised element by
 * element from their packed bytes at the point of use.
 *
 * Readings of points the pages leave open (each is also a test in tests/):
 *  - the second forward input holds logits; the softmax is taken here
 *    (ClikaRT "QMoEWoQ" page: the caller computes router logits);
 *  - softmax over all E experts, then the k largest are kept; their weights are
 *    their probabilities, divided by their sum when renormalising;
 *  - selection compares the logit values themselves (IEEE: -0 == +0), larger
 *    first, equal values in ascending expert index; slots keep that order;
 *  - a 4-bit byte holds element 2j in its low nibble and 2j+1 in its high nibble;
 *  - dequant(q) = (q - 2^(bits-1)) * scale, q the unsigned field;
 *  - MX FP4 (E8M0 scales; ClikaRT "QMoEWoQ" page: MXFP4 gpt-oss checkpoints, format
 *    from the OCP Microscaling specification): dequant(q) = e2m1(q) * 2^(e - 127), no
 *    zero point, one scale byte e per 32 k;
 *  - block_size 0: one scale per output row; otherwise scale index floor(k/bs),
 *    with a shorter last block when bs does not divide K;
 *  - interleaved fusion: row 2i is gate, 2i+1 is up; concatenated: rows [0,I)
 *    gate, [I,2I) up; separate stacks: fc1 gate, fc3 up; biases follow rows;
 *  - SwiGLU: g' = min(g, L), u' = clamp(u, -L, L), h = g' * sigmoid(alpha g') * (u' + beta);
 *  - biases are added before the activation (fc1/fc3) and before the routing
 *    weight (fc2); shared_output is added after the weighted sum;
 *  - gelu (graiphic "QMoE" page, activation_type gelu; CLIKA "MoE" page, gelu_mode): the
 *    plain activation x * Phi(x), Phi the standard normal CDF through erf (gelu_mode 0),
 *    or its tanh approximation 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))) (mode 1);
 *  - apply_router_weight_on_input (CLIKA "MoE" page, routing kwargs): the routing weight
 *    multiplies the row that enters the expert, and the expert outputs are then summed
 *    with weight 1; expert_output_scale: multiplies each expert's output (fc2 with its
 *    bias) before the combine (0 means 1);
 *  - the sparse mixer (graiphic "QMoE" page, use_sparse_mixer; CLIKA "MoE" page,
 *    sparse_mixer_eps), read from its published definition (the SparseMixer top-2 router
 *    of the Phi-3.5-MoE model card and GRIN-MoE): k = 2 picks; pick 1 is the largest logit,
 *    pick 2 the largest of the others (ties to the lower index); each pick's weight is
 *    the softmax at the picked expert over the experts the pick keeps, where an expert is
 *    dropped when (m - l) / max(|l|, m) > 2 eps (m the pick's logit, l the expert's; the
 *    second pick also drops the first); the drop decision is taken in fp32, as the
 *    kernel takes it; no renormalisation;
 *  - the int8 block tier (ClikaRT "QMoEWoQ" page, class description) rounds each
 *    block_size run of an activation row to int8 codes under one power-of-two scale 2^e,
 *    e the smallest integer with max|x| <= 127 * 2^e, code = x / 2^e rounded to nearest,
 *    ties to even; the GEMM then takes code * 2^e. It applies to the row x enters fc1
 *    with and to h, after h has been rounded to the activation dtype (the dtype h is held
 *    in between the two GEMMs), so both sides decide the codes from the same values.
 */
#include "qmoe_oracle.h"

#include <algorithm>
#include <cmath>
#include <cstring>
#include <numeric>
#include <vector>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ---- exact widening of stored elements --------------------------------- */

static double widen(const void* base, int32_t dtype, int64_t i) {
  if (dtype == ORACLE_E8M0) {  // a power of two 2^(e - 127); 255 is not a number
    const uint8_t e = static_cast<const uint8_t*>(base)[i];
    return e == 255 ? NAN : std::ldexp(1.0, static_cast<int>(e) - 127);
  }
  if (dtype == ORACLE_F32) {
    float f;
    std::memcpy(&f, static_cast<const char*>(base) + 4 * i, 4);
    return static_cast<double>(f);
  }
  uint16_t h;
  std::memcpy(&h, static_cast<const char*>(base) + 2 * i, 2);
  uint32_t bits = static_cast<uint32_t>(h) << 16;  // a bfloat16 is the top half of a float
  float f;
  std::memcpy(&f, &bits, 4);
  return static_cast<double>(f);
}

/* ---- rounding of the result to bfloat16 (8 significant bits) ----------- */

static uint16_t round_to_bf16(double v) {
  if (std::isnan(v)) return 0x7FC0;
  double r;
  if (v == 0.0) {
    r = v;
  } else {
    int e;
    std::frexp(v, &e);              // |v| = m * 2^e, m in [0.5, 1)
    int q = e - 8;                  // quantum of an 8-significant-bit number
    if (q < -133) q = -133;         // subnormal bfloat16 quantum
    r = std::ldexp(std::nearbyint(std::ldexp(v, -q)), q);  // nearest, ties to even
    if (std::fabs(r) > 3.3895313892515355e38) r = std::copysign(INFINITY, v);
  }
  float f = static_cast<float>(r);  // exact: r has at most 8 significant bits
  uint32_t bits;
  std::memcpy(&bits, &f, 4);
  return static_cast<uint16_t>(bits >> 16);
}

/* Pinned against torch's float32 -> bfloat16 conversion and a single rounding from double. */
void oracle_round_bf16(const double* v, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = round_to_bf16(v[i]);
}

static void store_out(const oracle_params* p, void* dst, int64_t i, double v) {
  if (p->act_dtype == ORACLE_F32) {
    float f = static_cast<float>(v);  // IEEE round-to-nearest-even
    std::memcpy(static_cast<char*>(dst) + 4 * i, &f, 4);
  } else {
    uint16_t h = round_to_bf16(v);
    std::memcpy(static_cast<char*>(dst) + 2 * i, &h, 2);
  }
}

/* ---- the int8 activation tier -------------------------------------------- */

/* The smallest integer e with a <= 127 * 2^e (a >= 0; 0 for an all-zero block). The search
   starts at e0 = ilogb(a) - 6, below the answer since 127 * 2^(e0 - 1) < 2^ilogb(a) <= a. */
static int int8_block_exponent(double a) {
  if (!(a > 0.0)) return 0;
  int e = std::ilogb(a) - 6;
  while (a > 127.0 * std::ldexp(1.0, e)) ++e;
  return e;
}

/* Round one activation row, block by block (a shorter last block when block_size does not
   divide len). */
static void int8_round_row(const oracle_params* p, double* v, int64_t len) {
  const int64_t bs = p->block_size;
  for (int64_t b0 = 0; b0 < len; b0 += bs) {
    const int64_t b1 = std::min(b0 + bs, len);
    double a = 0.0;
    for (int64_t i = b0; i < b1; ++i) a = std::max(a, std::fabs(v[i]));
    const int e = int8_block_exponent(a);
    for (int64_t i = b0; i < b1; ++i)
      v[i] = std::ldexp(std::nearbyint(std::ldexp(v[i], -e)), e);
  }
}

/* v rounded to the activation dtype and widened back. */
static double to_act_dtype(const oracle_params* p, double v) {
  if (p->act_dtype == ORACLE_F32) return static_cast<double>(static_cast<float>(v));
  const uint16_t h = round_to_bf16(v);
  return widen(&h, ORACLE_BF16, 0);
}

/* Pinned by a search over every power of two (tests/bruteforce.py: int8_round), by its
   properties (largest code in [64, 127], error at most half a step, idempotence) and by
   hand-worked blocks including a tie. */
void oracle_int8_round(const oracle_params* p, const void* in, int64_t rows, int64_t cols,
                       void* out) {
  std::vector<double> v(cols);
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t i = 0; i < cols; ++i) v[i] = widen(in, p->act_dtype, r * cols + i);
    int8_round_row(p, v.data(), cols);
    for (int64_t i = 0; i < cols; ++i) store_out(p, out, r * cols + i, v[i]);  // exact
  }
}

/* ---- routing: softmax over all experts, keep the top k ------------------ */

/* The sparse mixer's drop rule for one expert of one pick: its logit l trails the pick's
   logit m by more than 2 eps relative to max(|l|, m), evaluated in fp32 (0/0 keeps it). */
static bool mixer_drops(double m, double l, double eps) {
  const float mf = static_cast<float>(m), lf = static_cast<float>(l);
  const float r = (mf - lf) / std::max(std::fabs(lf), mf);
  return r > 2.0f * static_cast<float>(eps);
}

/* Sparse mixer routing of one token (k = 2): two picks, each weighted by the softmax at the
   picked expert over the experts that pick keeps. Pinned by hand-worked cases and limits
   (eps -> infinity: plain softmaxes; eps = 0 with distinct logits: weights 1). */
static void route_token_mixer(const oracle_params* p, const std::vector<double>& l, int32_t* ids,
                              double* w) {
  const int64_t E = p->E;
  int64_t e1 = 0;
  for (int64_t e = 1; e < E; ++e)
    if (l[e] > l[e1]) e1 = e;
  double s1 = 0.0;
  for (int64_t e = 0; e < E; ++e)
    if (!mixer_drops(l[e1], l[e], p->mixer_eps)) s1 += std::exp(l[e] - l[e1]);
  int64_t e2 = -1;
  for (int64_t e = 0; e < E; ++e)
    if (e != e1 && (e2 < 0 || l[e] > l[e2])) e2 = e;
  double s2 = 0.0;
  for (int64_t e = 0; e < E; ++e)
    if (e != e1 && !mixer_drops(l[e2], l[e], p->mixer_eps)) s2 += std::exp(l[e] - l[e2]);
  const double scale = p->routed_scale != 0.0 ? p->routed_scale : 1.0;
  ids[0] = static_cast<int32_t>(e1);
  ids[1] = static_cast<int32_t>(e2);
  w[0] = scale / s1;  // exp(l[e1] - l[e1]) / s1
  w[1] = scale / s2;
}

/* Softmax-top-k routing of one token, with the selection bias and grouped top-k variants.
   Pinned by the subset brute force (tests/bruteforce.py: select, gates) with many ties,
   scipy's softmax, uniform and one-hot logits. */
static void route_token(const oracle_params* p, const void* logits, int64_t t, int32_t* ids,
                        double* w) {
  const int64_t E = p->E;
  std::vector<double> l(E), key(E);
  for (int64_t e = 0; e < E; ++e) l[e] = widen(logits, p->act_dtype, t * E + e);
  if (p->sparse_mixer) {
    route_token_mixer(p, l, ids, w);
    return;
  }
  // Selection keys: the logits, or with a selection bias their fp32 sum with it (the sum
  // of two stored values, rounded once to float, as the reading of the bias states).
  for (int64_t e = 0; e < E; ++e) {
    if (p->score_bias) {
      const float b = static_cast<float>(widen(p->score_bias, p->act_dtype, e));
      key[e] = static_cast<double>(static_cast<float>(l[e]) + b);
    } else {
      key[e] = l[e];
    }
  }
  // Grouped top-k: groups of E / n_group consecutive experts scored by their largest key;
  // the topk_group best (ties to the lower group) stay selectable.
  std::vector<char> allowed(E, 1);
  if (p->n_group > 1) {
    const int64_t G = p->n_group, gsize = E / G;
    std::vector<double> gs(G);
    for (int64_t g = 0; g < G; ++g)
      gs[g] = *std::max_element(key.begin() + g * gsize, key.begin() + (g + 1) * gsize);
    std::vector<int32_t> gorder(G);
    std::iota(gorder.begin(), gorder.end(), 0);
    std::stable_sort(gorder.begin(), gorder.end(), [&](int32_t a, int32_t b) { return gs[a] > gs[b]; });
    std::vector<char> kept(G, 0);
    for (int64_t r = 0; r < p->topk_group; ++r) kept[gorder[r]] = 1;
    for (int64_t e = 0; e < E; ++e) allowed[e] = kept[e / gsize];
  }

  // Selection: larger key first; a stable sort keeps equal keys in index order.
  std::vector<int32_t> order;
  for (int64_t e = 0; e < E; ++e)
    if (allowed[e]) order.push_back(static_cast<int32_t>(e));
  std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) { return key[a] > key[b]; });

  // Softmax over all E logits (shifted by the maximum for range only; the value is
  // unchanged).
  const double m = *std::max_element(l.begin(), l.end());
  double denom = 0.0;
  for (int64_t e = 0; e < E; ++e) denom += std::exp(l[e] - m);

  double sum = 0.0;
  for (int64_t j = 0; j < p->k; ++j) {
    ids[j] = order[j];
    w[j] = std::exp(l[order[j]] - m) / denom;
    sum += w[j];
  }
  if (p->normalize)
    for (int64_t j = 0; j < p->k; ++j) w[j] /= sum;
  const double scale = p->routed_scale != 0.0 ? p->routed_scale : 1.0;
  for (int64_t j = 0; j < p->k; ++j) w[j] *= scale;
}

/* Pinned as route_token and route_token_mixer are. */
void oracle_route(const oracle_params* p, const void* logits, int32_t* ids, double* w) {
  for (int64_t t = 0; t < p->T; ++t) route_token(p, logits, t, ids + t * p->k, w + t * p->k);
}

/* ---- grouping by expert -------------------------------------------------- */

/* Pinned against numpy's stable argsort with padding (M = 1, 4, 16, 128) and the
   permute-then-unpermute identity. */
int64_t oracle_permute(const oracle_params* p, int32_t M, const int32_t* ids, int32_t* counts,
                       int32_t* padded_offsets, int32_t* sorted_assign, int32_t* assign_pos,
                       int32_t* tiles, int32_t* num_tiles) {
  const int64_t A = p->T * p->k, E = p->E;
  for (int64_t e = 0; e < E; ++e) counts[e] = 0;
  for (int64_t a = 0; a < A; ++a) counts[ids[a]] += 1;

  padded_offsets[0] = 0;
  for (int64_t e = 0; e < E; ++e) {
    int32_t tiles_e = (counts[e] + M - 1) / M;
    padded_offsets[e + 1] = padded_offsets[e] + tiles_e * M;
  }
  for (int64_t r = 0; r < padded_offsets[E]; ++r) sorted_assign[r] = -1;

  // Stable: scan assignments in ascending order once per expert.
  for (int64_t e = 0; e < E; ++e) {
    int32_t pos = padded_offsets[e];
    for (int64_t a = 0; a < A; ++a) {
      if (ids[a] == e) {
        sorted_assign[pos] = static_cast<int32_t>(a);
        assign_pos[a] = pos;
        ++pos;
      }
    }
  }

  int32_t nt = 0;
  for (int64_t e = 0; e < E; ++e) {
    for (int32_t r = 0; r * M < counts[e]; ++r) {
      tiles[2 * nt] = static_cast<int32_t>(e);
      tiles[2 * nt + 1] = std::min(M, counts[e] - r * M);
      ++nt;
    }
  }
  *num_tiles = nt;
  return padded_offsets[E];
}

/* ---- dequantisation of one weight ---------------------------------------- */

static int32_t qfield(const oracle_params* p, const uint8_t* w, int64_t N, int64_t K, int64_t e,
                      int64_t n, int64_t kk) {
  const int64_t row_bytes = K * p->bits / 8;
  const uint8_t* row = w + (e * N + n) * row_bytes;
  if (p->bits == 8) return row[kk];
  uint8_t byte = row[kk / 2];
  return (kk % 2 == 0) ? (byte & 0x0F) : (byte >> 4);
}

/* E2M1: bit 3 the sign, bits 2..1 the exponent (bias 1), bit 0 the mantissa; exponent 0
   is the subnormal range (0 and 0.5). The eight magnitudes as a table. */
static double e2m1(int32_t q) {
  static const double mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
  return (q & 8) ? -mag[q & 7] : mag[q & 7];
}

/* Pinned by the dense numpy dequantisation of the brute force, the hand-worked golden cases
   (nibble order, orientation), E2M1 from its bit fields and the 4-bit/8-bit, per-row/block
   and ragged-block equivalences. */
double oracle_weight(const oracle_params* p, const oracle_stack* st, int64_t N, int64_t K,
                     int64_t e, int64_t n, int64_t kk) {
  if (p->scale_dtype == ORACLE_E8M0) {
    const int64_t nb = (K + p->block_size - 1) / p->block_size;
    const double s = widen(st->s, ORACLE_E8M0, (e * N + n) * nb + kk / p->block_size);
    return e2m1(qfield(p, st->w, N, K, e, n, kk)) * s;
  }
  const int32_t zero = 1 << (p->bits - 1);
  double s;
  if (p->block_size == 0) {
    s = widen(st->s, p->scale_dtype, e * N + n);
  } else {
    const int64_t nb = (K + p->block_size - 1) / p->block_size;
    s = widen(st->s, p->scale_dtype, (e * N + n) * nb + kk / p->block_size);
  }
  return static_cast<double>(qfield(p, st->w, N, K, e, n, kk) - zero) * s;
}

/* One output of a dequantised linear layer: sum_k in[k] * W[n][k] + b[n]. */
static double linear_out(const oracle_params* p, const oracle_stack* st, int64_t N, int64_t K,
                         int64_t e, int64_t n, const double* in) {
  double acc = 0.0;
  for (int64_t kk = 0; kk < K; ++kk) acc += in[kk] * oracle_weight(p, st, N, K, e, n, kk);
  if (st->b) acc += widen(st->b, p->act_dtype, e * N + n);
  return acc;
}

/* ---- activation ---------------------------------------------------------- */

static double sigmoid(double v) { return 1.0 / (1.0 + std::exp(-v)); }

static double swiglu(const oracle_params* p, double g, double u) {
  const double L = p->limit;
  g = std::min(g, L);
  u = std::max(-L, std::min(u, L));
  return g * sigmoid(p->alpha * g) * (u + p->beta);
}

/* The plain activations. gelu is pinned against torch's gelu (both forms) and scipy's
   normal CDF; relu and silu against torch; identity through the exact integer products. */
static double plain_act(const oracle_params* p, double z) {
  switch (p->activation) {
    case ORACLE_ACT_RELU: return z > 0.0 ? z : 0.0;
    case ORACLE_ACT_SILU: return z * sigmoid(z);
    case ORACLE_ACT_GELU:
      if (p->gelu_mode == 0) return 0.5 * z * (1.0 + std::erf(z / std::sqrt(2.0)));
      return 0.5 * z * (1.0 + std::tanh(std::sqrt(2.0 / M_PI) * (z + 0.044715 * z * z * z)));
    default: return z;  // identity
  }
}

/* fc1 (and fc3) followed by the activation for one token row through expert e. */
static void expert_fc1(const oracle_params* p, const oracle_stack* fc1, const oracle_stack* fc3,
                       int64_t e, const double* x, double* h) {
  const int64_t H = p->H, I = p->I;
  if (p->activation != ORACLE_ACT_SWIGLU) {
    for (int64_t i = 0; i < I; ++i) h[i] = plain_act(p, linear_out(p, fc1, I, H, e, i, x));
    return;
  }
  for (int64_t i = 0; i < I; ++i) {
    double g, u;
    if (p->fusion == 1) {         // interleaved: gate row 2i, up row 2i+1
      g = linear_out(p, fc1, 2 * I, H, e, 2 * i, x);
      u = linear_out(p, fc1, 2 * I, H, e, 2 * i + 1, x);
    } else if (p->fusion == 2) {  // concatenated: gate rows [0,I), up rows [I,2I)
      g = linear_out(p, fc1, 2 * I, H, e, i, x);
      u = linear_out(p, fc1, 2 * I, H, e, I + i, x);
    } else {                      // separate stacks: fc1 gate, fc3 up
      g = linear_out(p, fc1, I, H, e, i, x);
      u = linear_out(p, fc3, I, H, e, i, x);
    }
    h[i] = swiglu(p, g, u);
  }
}

static void expert_fc2(const oracle_params* p, const oracle_stack* fc2, int64_t e, const double* h,
                       double* y) {
  for (int64_t m = 0; m < p->H; ++m) y[m] = linear_out(p, fc2, p->H, p->I, e, m, h);
}

static void widen_row(const void* base, int32_t dtype, int64_t row, int64_t len, double* out) {
  for (int64_t i = 0; i < len; ++i) out[i] = widen(base, dtype, row * len + i);
}

static void set_threads(int nthreads) {
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
}

/* fc1 and the activation for given rows (the fc1 stage). Pinned through the forward's
   pins (it is the forward's step) and directly by the layout equivalences. */
void oracle_fc1_rows(const oracle_params* p, const oracle_stack* fc1, const oracle_stack* fc3,
                     const void* x, int64_t n_rows, const int32_t* row_token,
                     const int32_t* row_expert, const double* row_w, double* h, int nthreads) {
  set_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < n_rows; ++r) {
    std::vector<double> xr(p->H);
    widen_row(x, p->act_dtype, row_token[r], p->H, xr.data());
    if (row_w)
      for (int64_t i = 0; i < p->H; ++i) xr[i] *= row_w[r];
    expert_fc1(p, fc1, fc3, row_expert[r], xr.data(), h + r * p->I);
  }
}

/* fc2 for given rows (the fc2 stage); pinned like oracle_fc1_rows. */
void oracle_fc2_rows(const oracle_params* p, const oracle_stack* fc2, const void* h_in,
                     int64_t n_rows, const int32_t* row_index, const int32_t* row_expert,
                     double* y, int nthreads) {
  set_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < n_rows; ++r) {
    std::vector<double> hr(p->I);
    widen_row(h_in, p->act_dtype, row_index[r], p->I, hr.data());
    expert_fc2(p, fc2, row_expert[r], hr.data(), y + r * p->H);
  }
}

/* ---- combine -------------------------------------------------------------- */

/* The combine coefficient of one slot: its routing weight, or 1 when the weight went to the
   expert's input, times the expert output scale. */
static double combine_coef(const oracle_params* p, double w) {
  const double s = p->out_scale != 0.0 ? p->out_scale : 1.0;
  return (p->on_input ? 1.0 : w) * s;
}

/* The combine (stage). Pinned by the zero-weight closed form out = sum_j w_j b2[e_j] and
   the composition test (stages compose to the forward). */
void oracle_combine(const oracle_params* p, const float* y, const int32_t* assign_pos,
                    const float* w, const void* shared, double* out64, void* out_rounded) {
  const int64_t H = p->H, k = p->k;
  for (int64_t t = 0; t < p->T; ++t) {
    for (int64_t m = 0; m < H; ++m) {
      double acc = 0.0;
      for (int64_t j = 0; j < k; ++j)
        acc += combine_coef(p, static_cast<double>(w[t * k + j])) *
               static_cast<double>(y[static_cast<int64_t>(assign_pos[t * k + j]) * H + m]);
      if (shared) acc += widen(shared, p->act_dtype, t * H + m);
      out64[t * H + m] = acc;
      if (out_rounded) store_out(p, out_rounded, t * H + m, acc);
    }
  }
}

/* ---- whole forward, token by token ---------------------------------------- */

/* The whole forward, token by token. Pinned by the dense brute force over all expert
   subsets (tests/bruteforce.py), the closed forms, the linearity and layout equivalences,
   and the hand-worked examples in tests/golden/. */
void oracle_forward(const oracle_params* p, const oracle_stack* fc1, const oracle_stack* fc2,
                    const oracle_stack* fc3, const void* x, const void* logits, const void* shared,
                    int64_t n_sel, const int64_t* sel, double* out64, void* out_rounded,
                    int nthreads) {
  const int64_t H = p->H, I = p->I, k = p->k;
  const int64_t n = sel ? n_sel : p->T;
  set_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < n; ++r) {
    const int64_t t = sel ? sel[r] : r;
    std::vector<int32_t> ids(k);
    std::vector<double> w(k), xr(H), h(I), y(H), acc(H, 0.0);
    route_token(p, logits, t, ids.data(), w.data());
    widen_row(x, p->act_dtype, t, H, xr.data());
    if (p->int8_act) int8_round_row(p, xr.data(), H);
    std::vector<double> xin(H);
    for (int64_t j = 0; j < k; ++j) {
      for (int64_t i = 0; i < H; ++i) xin[i] = p->on_input ? w[j] * xr[i] : xr[i];
      expert_fc1(p, fc1, fc3, ids[j], xin.data(), h.data());
      if (p->int8_act) {
        for (int64_t i = 0; i < I; ++i) h[i] = to_act_dtype(p, h[i]);
        int8_round_row(p, h.data(), I);
      }
      expert_fc2(p, fc2, ids[j], h.data(), y.data());
      const double c = combine_coef(p, w[j]);
      for (int64_t m = 0; m < H; ++m) acc[m] += c * y[m];
    }
    for (int64_t m = 0; m < H; ++m) {
      double v = acc[m] + (shared ? widen(shared, p->act_dtype, t * H + m) : 0.0);
      out64[r * H + m] = v;
      if (out_rounded) store_out(p, out_rounded, r * H + m, v);
    }
  }
}
