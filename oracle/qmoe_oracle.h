/*
 * qmoe_oracle.h -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, fp64 CPU evaluation of the weight-only-quantized MoE block
 * forward. It exists to check the GPU library against; nothing on the product
 * path may include, link or call it. It shares no code with the GPU library.
 *
 * What it computes (the plain definition, step by step):
 *   route    softmax over all E router logits, the k largest logits selected
 *            (ties to the lower expert index), weights = their probabilities,
 *            optionally renormalised to sum to one
 *            (CLIKA "MoE" page, class description and the routing kwargs;
 *             graiphic "QMoE" page, attributes k and normalize_routing_weights)
 *   permute  assignments a = t*k + j grouped by expert, stable in a, each
 *            expert's group padded to a multiple of M rows
 *   fc1      z = x . dequant(W1)^T + b1 per expert, dequant(q) = (q - 2^(bits-1)) * s
 *            (CLIKA "QLinearWoQ" page, class description; graiphic "QMoE" page,
 *             fc1/fc3 inputs, block_size and expert_weight_bits attributes)
 *   act      SwiGLU with alpha, beta and limit (graiphic "QMoE" page,
 *            activation_alpha/beta, swiglu_fusion, swiglu_limit)
 *   fc2      y = h . dequant(W2)^T + b2
 *   combine  out[t] = sum_j w_j * y(t, j) (+ shared_output[t]), rounded once to
 *            the activation dtype (ClikaRT "QMoEWoQ" page, forward)
 *   int8     (optional) x and h rounded to per-block int8 before fc1 and fc2
 *            (ClikaRT "QMoEWoQ" page, class description: the int8 block tier)
 *   variants (optional) gelu, the routing weight on the input, an expert output scale,
 *            the sparse mixer routing (CLIKA "MoE" page, routing kwargs; graiphic "QMoE"
 *            page, activation_type and use_sparse_mixer)
 *
 * What pins each function (tests/test_oracle_pins.py) is listed beside it in
 * qmoe_oracle.cpp.
 */
#ifndef QMOE_ORACLE_H
#define QMOE_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORACLE_F32 = 0, ORACLE_BF16 = 1, ORACLE_E8M0 = 2 /* scales only: 2^(e-127), MX FP4 codes */ };
enum { ORACLE_ACT_SWIGLU = 0, ORACLE_ACT_IDENTITY = 1, ORACLE_ACT_RELU = 2, ORACLE_ACT_SILU = 3,
       ORACLE_ACT_GELU = 4 };

typedef struct {
  int64_t T, H, I, E, k;
  int32_t bits;          /* 4 or 8 */
  int32_t block_size;    /* 0: one scale per output row; else scales per K-block */
  int32_t fusion;        /* 0 separate fc1/fc3, 1 interleaved, 2 gate rows then up rows */
  int32_t activation;    /* ORACLE_ACT_* */
  int32_t normalize;     /* renormalise the k routing weights */
  int32_t act_dtype;     /* ORACLE_F32 / ORACLE_BF16: x, logits, biases, shared, out */
  int32_t scale_dtype;   /* ORACLE_F32 / ORACLE_BF16 / ORACLE_E8M0 (MX FP4 weights) */
  int32_t pad_;
  double alpha, beta, limit; /* limit = +inf: no clamp */
  /* routing variants: grouped top-k (n_group > 1), weight scaling (0 means 1), and the
     selection bias [E] in the activation dtype (NULL: none) */
  int32_t n_group, topk_group;
  double routed_scale;
  const void* score_bias;
  /* 1: the int8 activation tier, x and h rounded to per-block int8 before each GEMM */
  int32_t int8_act;
  int32_t pad2_;
  /* gelu (ORACLE_ACT_GELU): 0 the exact x * Phi(x), 1 the tanh approximation */
  int32_t gelu_mode;
  /* 1: the routing weight multiplies the expert's input row instead of its output */
  int32_t on_input;
  /* multiplies every expert's output (fc2 with its bias) before the combine; 0 means 1 */
  double out_scale;
  /* 1: the sparse mixer routing (k = 2) with threshold mixer_eps */
  int32_t sparse_mixer;
  int32_t pad3_;
  double mixer_eps;
} oracle_params;

typedef struct {
  const uint8_t* w;   /* [E, N, K*bits/8] */
  const void* s;      /* [E, N] or [E, N, ceil(K/block_size)] */
  const void* b;      /* [E, N] in act dtype, or NULL */
} oracle_stack;

/* Routing of every token: ids [T,k], w [T,k] (fp64). */
void oracle_route(const oracle_params* p, const void* logits, int32_t* ids, double* w);

/* Grouping by expert, padded to M. sorted_assign and tiles must hold the worst case
   (T*k + E*(M-1) rows; T*k/M + E tiles, two ints each). Returns the padded row count. */
int64_t oracle_permute(const oracle_params* p, int32_t M, const int32_t* ids, int32_t* counts,
                       int32_t* padded_offsets, int32_t* sorted_assign, int32_t* assign_pos,
                       int32_t* tiles, int32_t* num_tiles);

/* One dequantised weight (fp64) of a stack with N rows and row length K. */
double oracle_weight(const oracle_params* p, const oracle_stack* st, int64_t N, int64_t K,
                     int64_t e, int64_t n, int64_t kk);

/* fc1 + activation for rows: h[r,:] = act(fc1(x[row_token[r]])) through expert row_expert[r];
   with row_w (may be NULL) the input row is x[row_token[r]] * row_w[r]. */
void oracle_fc1_rows(const oracle_params* p, const oracle_stack* fc1, const oracle_stack* fc3,
                     const void* x, int64_t n_rows, const int32_t* row_token,
                     const int32_t* row_expert, const double* row_w, double* h, int nthreads);

/* fc2 for rows: y[r,:] = fc2(h_in[row_index[r]]) through expert row_expert[r]; h_in in act dtype. */
void oracle_fc2_rows(const oracle_params* p, const oracle_stack* fc2, const void* h_in,
                     int64_t n_rows, const int32_t* row_index, const int32_t* row_expert,
                     double* y, int nthreads);

/* Combine: out[t] = sum_j c[t,j] * y[assign_pos[t*k+j]] (+ shared[t]), c = w (or 1 when the
   weight went to the input) times the expert output scale. */
void oracle_combine(const oracle_params* p, const float* y, const int32_t* assign_pos,
                    const float* w, const void* shared, double* out64, void* out_rounded);

/* Whole forward for the selected tokens (sel == NULL: all T tokens, n_sel ignored).
   out64 [n_sel, H] fp64 before rounding; out_rounded [n_sel, H] in act dtype (may be NULL). */
void oracle_forward(const oracle_params* p, const oracle_stack* fc1, const oracle_stack* fc2,
                    const oracle_stack* fc3, const void* x, const void* logits, const void* shared,
                    int64_t n_sel, const int64_t* sel, double* out64, void* out_rounded,
                    int nthreads);

/* The int8 tier's rounding of rows [rows, cols] in the activation dtype: out (same dtype)
   holds code * 2^e per block of block_size (block_size > 0). */
void oracle_int8_round(const oracle_params* p, const void* in, int64_t rows, int64_t cols,
                       void* out);

/* Round fp64 values to bfloat16 bit patterns, nearest-even. */
void oracle_round_bf16(const double* v, int64_t n, uint16_t* out);

#ifdef __cplusplus
}
#endif
#endif
