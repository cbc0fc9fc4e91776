/*
 * qmoe.h -- C ABI of the weight-only-quantized mixture-of-experts forward for
 * AMD Instinct MI355X (gfx950).
 *
 * The operation is the QMoE / QMoEWoQ block forward:
 *   out[t] = sum_{j<k} w[t,j] * FFN_{e[t,j]}(x[t])  (+ shared_output[t])
 * where the router picks the k experts with the largest router logits and
 * weighs them by their softmax probability (optionally renormalised), and
 *   FFN_e(x) = dequant(W2_e) . act(dequant(W1_e) . x + b1_e) + b2_e,
 *   dequant(q) = (q - 2^(bits-1)) * scale   per output row or per K-block.
 * Sources: ClikaRT "QMoEWoQ" page (class description: expert weights stay
 * quantized and are decoded block by block inside the GEMM dot; forward:
 * x [T,H] and router_logits [T,E] give [T,H] in x's dtype, optional
 * shared_output folded into the combine); CLIKA "MoE" page (top-k routing,
 * gated FFN, routing-weighted sum of the expert outputs; routing kwargs); CLIKA
 * "QLinearWoQ" page (y = x·dequant(W)ᵀ + b); graiphic "QMoE" page (input
 * tensors and their shapes; attributes activation_alpha/beta, activation_type,
 * block_size, expert_weight_bits, k, normalize_routing_weights, swiglu_fusion,
 * swiglu_limit).
 *
 * Conventions shared by every entry point:
 *  - Every array argument is a DEVICE pointer owned by the caller, row-major and
 *    densely packed. The library allocates nothing and keeps no state between calls
 *    (apart from the measurement hook of qmoe_time_next_gemm).
 *  - `stream` is a hipStream_t (NULL = the default stream). All work is enqueued
 *    asynchronously on it; no call synchronises with the host.
 *  - Parameters are validated on the host before anything is enqueued; on a
 *    validation failure nothing is launched and the call returns a non-zero
 *    qmoe_status, with a message available from qmoe_last_error().
 *  - A launch failure reported by the HIP runtime returns QMOE_ERR_DEVICE. A
 *    fault inside a kernel surfaces at the caller's next synchronisation.
 *  - num_tokens == 0 is valid: the call returns QMOE_OK and enqueues nothing.
 *  - Calls on different streams with distinct output buffers may run concurrently.
 */
#ifndef QMOE_H
#define QMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  QMOE_OK = 0,
  QMOE_ERR_INVALID = 1,      /* a parameter outside its documented range */
  QMOE_ERR_SHAPE = 2,        /* sizes inconsistent with each other or with the layout */
  QMOE_ERR_DTYPE = 3,        /* an element type combination that is not accepted */
  QMOE_ERR_UNSUPPORTED = 4,  /* valid on the pages but not implemented here */
  QMOE_ERR_UNBOUND = 5,      /* a required pointer is NULL (an unbound weight slot) */
  QMOE_ERR_DEVICE = 6        /* the HIP runtime reported an error */
} qmoe_status;

/* QMOE_E8M0: one unsigned byte e per scale, the power of two 2^(e - 127) (scale_dtype only).
   E8M0 scales select the MX FP4 weight format (ClikaRT "QMoEWoQ" page: the module serves
   block-quantized checkpoints such as MXFP4 gpt-oss): expert_weight_bits 4 and block_size
   32, each 4-bit code an E2M1 value (sign, 2-bit exponent with bias 1, 1-bit mantissa:
   magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6) with no zero point, dequant(q) = e2m1(q) * 2^(e-127);
   bf16 activations and the tiled weight layout only (QMOE_ERR_UNSUPPORTED otherwise).
   Scale bytes 0 and 255 (2^-127 and NaN) and products past the bf16 range are outside
   the tested range. */
typedef enum { QMOE_F32 = 0, QMOE_BF16 = 1, QMOE_E8M0 = 2 } qmoe_dtype;

/* Layout of the expert weight stacks (qmoe_params.weight_layout).
   QMOE_LAYOUT_ROWS: the pages' layout, uint8 [E, N, K*bits/8], row-major.
   QMOE_LAYOUT_TILES: the library's tiled layout, written by qmoe_pack_stack from a
   ROWS stack (see there). Scales and biases keep their layout in both cases. */
typedef enum { QMOE_LAYOUT_ROWS = 0, QMOE_LAYOUT_TILES = 1 } qmoe_layout;

/* Which stack of a forward: fc1 (gate, or fused gate/up), fc2 (down), fc3 (separate up). */
typedef enum { QMOE_FC1 = 1, QMOE_FC2 = 2, QMOE_FC3 = 3 } qmoe_which;

/* activation_type of the graiphic "QMoE" page (relu, gelu, silu, swiglu, identity). gelu is
   the plain activation z * Phi(z) (Phi the standard normal CDF) or its tanh approximation,
   as qmoe_params.gelu_mode selects (CLIKA "MoE" page, routing kwarg gelu_mode). */
typedef enum {
  QMOE_ACT_SWIGLU = 0,
  QMOE_ACT_IDENTITY = 1,
  QMOE_ACT_RELU = 2,
  QMOE_ACT_SILU = 3,
  QMOE_ACT_GELU = 4
} qmoe_act;

typedef struct {
  /* T, H, I, E, k: tokens, hidden_size, inter_size, num_experts, top-k
     (ClikaRT QMoEWoQ::make counts; graiphic QMoE attribute k). 1 <= k <= E <= 512,
     k <= 32 (QMOE_ERR_UNSUPPORTED beyond). */
  int64_t num_tokens, hidden_size, inter_size, num_experts, k;
  /* expert_weight_bits: 4 (two fields per byte, element 2j in the low nibble) or 8. */
  int32_t expert_weight_bits;
  /* block_size: 0 = one scale per output row; else a power of two >= 16, one scale
     per block_size elements along K. A K that block_size does not divide is
     accepted with a shorter last block unless strict_blocks is set. */
  int32_t block_size;
  /* swiglu_fusion: 0 separate gate (fc1) and up (fc3) stacks; 1 fused, row 2i gate and
     row 2i+1 up; 2 fused, rows [0,I) gate and [I,2I) up. Must be 0 unless swiglu. */
  int32_t swiglu_fusion;
  int32_t activation;                /* qmoe_act */
  int32_t normalize_routing_weights; /* non-zero: divide the k weights by their sum */
  /* SwiGLU: h = g' * sigmoid(alpha * g') * (u' + beta), g' = min(g, L),
     u' = clamp(u, -L, L). swiglu_limit <= 0 or +inf means no clamp. */
  float swiglu_alpha, swiglu_beta, swiglu_limit;
  int32_t act_dtype;    /* qmoe_dtype of x, router logits, biases, shared_output, output */
  int32_t scale_dtype;  /* qmoe_dtype of the scales (QMOE_E8M0: MX FP4 weights, above) */
  /* Rows per expert tile of the grouping. 0 = the library's choice for these shapes
     (qmoe_tile_m). bf16 activations take 16, 32 or 128; fp32 activations 1 to 16 rows
     that fit the kernel's LDS. Every call of one forward must use the same value. */
  int32_t tile_m;
  int32_t strict_blocks; /* non-zero: reject a K that block_size does not divide */
  /* qmoe_layout of every weight stack handed to the GEMM and forward entry points.
     QMOE_LAYOUT_TILES requires act_dtype QMOE_BF16. */
  int32_t weight_layout;
  /* Routing variants (CLIKA "MoE" page: routing kwargs n_group, topk_group,
     routed_scaling_factor; ClikaRT "QMoEWoQ" page: e_score_correction_bias [E], a
     per-expert bias used for the choice of experts). All off when zero / NULL.
     n_group > 1: experts form n_group groups of E / n_group consecutive indices (E a
       multiple, n_group <= 16); a group scores the largest selection key of its experts;
       the topk_group best groups are kept (ties to the lower group) and the k experts are
       chosen among theirs (k <= topk_group * E / n_group).
     routed_scaling_factor: multiplies the k routing weights after any renormalisation
       (0 means 1).
     e_score_correction_bias: device [E] in act_dtype, or NULL; the selection key of expert
       e is the fp32 sum logit + bias[e]; the weights use the logits alone. */
  int32_t n_group, topk_group;
  float routed_scaling_factor;
  const void* e_score_correction_bias;
  /* qmoe_compute_mode: QMOE_COMPUTE_FLOAT (0) keeps the activations as they are;
     QMOE_COMPUTE_INT8 (the int8 block tier of the ClikaRT "QMoEWoQ" page) rounds the
     input of each GEMM to per-block int8 first (qmoe_quantize_act): qmoe_forward does so
     for x and h; the GEMM entry points and qmoe_linear_woq take their inputs as given
     (their callers apply qmoe_quantize_act first). Needs block_size > 0
     (QMOE_ERR_INVALID) and bf16 activations (QMOE_ERR_UNSUPPORTED with fp32: the codes
     of h are decided from h, and a last-bit difference in an fp32 h, from summation
     order, can move one code by a step, which is worth more than the fp32 path's bound).
     Where the tiles are prefill-sized (128 rows) in the tiled layout with integer codes,
     blocks of 64 or 128 and H and I multiples of 64, qmoe_forward multiplies the codes on
     the int8 matrix cores (int32 block sums, each scaled once by 2^e times the weight
     scale); elsewhere the rounded activations go through the bf16 kernels. Both give the
     same products exactly; only the fp32 summation order differs. */
  int32_t compute_mode;
  /* The remaining options of the CLIKA "MoE" page's routing kwargs and the graiphic "QMoE"
     page's attributes:
     gelu_mode (activation QMOE_ACT_GELU): 0 = z * Phi(z) through erf, 1 = the tanh
       approximation 0.5 z (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3))).
     expert_output_scale: multiplies every expert's output (fc2 with its bias) before the
       combine, the shared output excepted; 0 means 1. Applied by qmoe_combine.
     apply_router_weight_on_input: non-zero: the routing weight multiplies the row that
       enters the expert (fc1 takes w * x, as its epilogue scales the fp32 sum by w before
       the bias), and the combine sums the expert outputs with weight 1. Not with the int8
       tier (QMOE_ERR_UNSUPPORTED: its codes would depend on each slot's weight).
     use_sparse_mixer: the sparse mixer routing (graiphic use_sparse_mixer; CLIKA
       sparse_mixer_eps), read from its published definition (the SparseMixer top-2 router
       of Phi-3.5-MoE): k must be 2, normalize_routing_weights 0, no grouping and no
       selection bias (QMOE_ERR_INVALID otherwise). Pick 1 is the largest logit m1, pick 2
       the largest of the others m2 (equal logits: lower index); pick j keeps expert e
       unless (mj - l_e) / max(|l_e|, mj) > 2 * sparse_mixer_eps (decided in fp32; pick 2
       never keeps pick 1), and its weight is the softmax at the picked expert over the
       experts it keeps; routed_scaling_factor still applies. sparse_mixer_eps: finite,
       >= 0. */
  int32_t gelu_mode;
  float expert_output_scale;
  int32_t apply_router_weight_on_input;
  int32_t use_sparse_mixer;
  float sparse_mixer_eps;
} qmoe_params;

typedef enum { QMOE_COMPUTE_FLOAT = 0, QMOE_COMPUTE_INT8 = 1 } qmoe_compute_mode;

/* One quantized expert stack (graiphic QMoE fcN_experts_weights / fcN_scales / fcN_experts_bias).
   weights: uint8 [E, N, K*bits/8] (QMOE_LAYOUT_ROWS) or the tiled form from qmoe_pack_stack
   (QMOE_LAYOUT_TILES); scales: scale_dtype [E, N] (block_size 0) or
   [E, N, ceil(K/block_size)]; bias: act_dtype [E, N] or NULL. */
typedef struct {
  const void* weights;
  const void* scales;
  const void* bias;
} qmoe_stack;

/*
 * Tiled weight layout (QMOE_LAYOUT_TILES). The weights of a stack are cut into tiles of
 * 16 rows by S_K elements of K (S_K = 128 for 4-bit, 64 for 8-bit), 1024 bytes each; the
 * GEMM kernels read one tile with one 16-byte load per lane of a 64-lane wavefront, from
 * contiguous memory, in the order in which the matrix-core instructions consume it.
 *   Streams: fc1 with swiglu and swiglu_fusion 1 or 2 has two streams of I rows (stream
 *   0 the gate rows, stream 1 the up rows, wherever the fusion puts them in the ROWS
 *   stack); every other stack has one stream of all its N rows.
 *   Order: tile (e, s, b, t) -- expert e, stream s, rows [16b, 16b+16) of the stream,
 *   K range [t*S_K, t*S_K + S_K) -- starts at byte 1024 * (((e*S + s)*NB + b)*KT + t),
 *   NB = ceil(rows per stream / 16), KT = ceil(K / S_K).
 *   Inside a tile, bytes [16l, 16l+16) belong to lane l = 16*q + n: row 16b + n of the
 *   stream, and for each j < S_K/32 the eight elements k = t*S_K + 32j + 8q + i, i < 8:
 *     4-bit: 32-bit word j (little-endian) holds element i in bits [4p, 4p+4) for
 *            p = (0, 4, 1, 5, 2, 6, 3, 7)[i], i.e. its nibbles hold elements
 *            (0, 2, 4, 6, 1, 3, 5, 7); with E8M0 scales (MX FP4) p = i instead;
 *     8-bit: byte 8j + i holds element i.
 *   Elements past K and rows past the stream's end hold code 0 (their products meet
 *   zero activations or are never stored).
 */

/* Bytes of the tiled form of stack `which` (qmoe_which) for these parameters; 0 when the
   parameters are invalid or the stack does not exist for them (fc3 without separate up
   rows). */
size_t qmoe_packed_stack_size(const qmoe_params* p, int32_t which);

/*
 * Writes the tiled form of one ROWS-layout weight stack (graiphic "QMoE" page:
 * fcN_experts_weights [E, N, K*bits/8]) into `packed` (qmoe_packed_stack_size bytes,
 * caller-owned, 256-byte aligned, not overlapping `weights`). A one-time preparation of
 * the weights, outside the forward; scales and biases are used as they are.
 * p->weight_layout is ignored here.
 */
qmoe_status qmoe_pack_stack(const qmoe_params* p, int32_t which, const void* weights,
                            void* packed, void* stream);

/* Checks the parameters; QMOE_OK when every entry point accepts them. */
qmoe_status qmoe_validate(const qmoe_params* p);

/* The tile height used when p->tile_m == 0, from shapes only (never from routed data). */
int32_t qmoe_tile_m(const qmoe_params* p);

/* Worst-case padded rows and tiles of the grouping for these parameters. */
int64_t qmoe_max_rows(const qmoe_params* p);
int64_t qmoe_max_tiles(const qmoe_params* p);

/* Bytes of device scratch qmoe_permute needs (may be 0). */
size_t qmoe_permute_scratch_size(const qmoe_params* p);

/* Bytes of device workspace qmoe_forward needs (256-byte aligned start required). */
size_t qmoe_workspace_size(const qmoe_params* p);

/*
 * Routing (CLIKA "MoE" page: each token goes to its top-k experts; routing_mode
 * "softmax_topk", renormalize; graiphic "QMoE" page: k, normalize_routing_weights;
 * ClikaRT "QMoEWoQ" page: the caller hands router logits to forward).
 *   router_logits [T, E] act_dtype  ->  topk_ids [T, k] int32, topk_w [T, k] float32.
 * Experts are selected by descending logit, equal logits in ascending expert index
 * (-0 equals +0); slot j holds the j-th selected expert. topk_w = softmax over all
 * E logits at the selected experts, divided by their sum if normalising.
 * Logits must be finite; the result for NaN or Inf logits is unspecified.
 */
qmoe_status qmoe_route(const qmoe_params* p, const void* router_logits, int32_t* topk_ids,
                       float* topk_w, void* stream);

/*
 * Grouping of the T*k assignments a = t*k + j by expert (the per-expert work lists
 * behind the per-expert kernels of the ClikaRT "QMoEWoQ" page).
 *   topk_ids [T*k] int32 in [0, E)  ->
 *   counts [E]              assignments per expert;
 *   padded_offsets [E+1]    first row of each expert; each group padded to a multiple of M;
 *   sorted_assign [max_rows] a at each row, ascending a within an expert, -1 on padding
 *                           (rows beyond padded_offsets[E] are left untouched);
 *   assign_pos [T*k]        row of each assignment (sorted_assign[assign_pos[a]] == a);
 *   tile_list [max_tiles, 2] (expert, valid rows) of tile i, which covers rows [i*M, i*M+M);
 *   num_tiles [1]           number of tiles written.
 * M = qmoe_tile_m(p) or p->tile_m. scratch: qmoe_permute_scratch_size(p) bytes (may be NULL
 * when that size is 0). The result is deterministic and independent of scheduling.
 * Ids outside [0, E) give an unspecified grouping.
 */
qmoe_status qmoe_permute(const qmoe_params* p, const int32_t* topk_ids, int32_t* counts,
                         int32_t* padded_offsets, int32_t* sorted_assign, int32_t* assign_pos,
                         int32_t* tile_list, int32_t* num_tiles, void* scratch,
                         size_t scratch_bytes, void* stream);

/*
 * fc1 (and fc3) grouped GEMM over the quantized expert stacks with the activation
 * fused into its epilogue (graiphic "QMoE" page: fc1/fc3 inputs, activation
 * attributes, swiglu_fusion; ClikaRT "QMoEWoQ" page: each weight block is decoded
 * inside the GEMM dot, never as a dense copy).
 *   x [T, H] act_dtype; sorted_assign, tile_list, num_tiles from qmoe_permute;
 *   fc1: weights [E, f*I, H*bits/8] (f = 2 for fused SwiGLU, else 1);
 *   fc3: separate up stack [E, I, H*bits/8] (only with swiglu and swiglu_fusion 0);
 *   h [max_rows, I] act_dtype (written for every real row of every tile; padding rows
 *   of a tile are written as zeros).
 *   topk_w [T*k] float32 from qmoe_route: read only with apply_router_weight_on_input
 *   (required then, QMOE_ERR_UNBOUND if NULL; may be NULL otherwise).
 * Row r of tile i (expert e, r < valid) computes, for a = sorted_assign[i*M + r] and
 * t = a / k: z = c * (x[t] . dequant(W1_e)^T) + b1_e, with c = topk_w[a] under
 * apply_router_weight_on_input and 1 otherwise, then h = act(z) (SwiGLU on the gate/up
 * pair selected by swiglu_fusion).
 */
qmoe_status qmoe_grouped_gemm_fc1_swiglu(const qmoe_params* p, const void* x,
                                         const int32_t* sorted_assign, const int32_t* tile_list,
                                         const int32_t* num_tiles, const float* topk_w,
                                         qmoe_stack fc1, qmoe_stack fc3, void* h, void* stream);

/*
 * fc2 grouped GEMM (graiphic "QMoE" page: fc2_experts_weights [E, H, I*bits/8],
 * fc2_scales, fc2_experts_bias).
 *   h [max_rows, I] act_dtype (rows of tile i from qmoe_grouped_gemm_fc1_swiglu);
 *   y [max_rows, H] float32: y = h . dequant(W2_e)^T + b2_e for the real rows of each tile.
 */
qmoe_status qmoe_grouped_gemm_fc2(const qmoe_params* p, const void* h, const int32_t* tile_list,
                                  const int32_t* num_tiles, qmoe_stack fc2, float* y,
                                  void* stream);

/*
 * Weighted combine (CLIKA "MoE" page: routing-weighted sum of the expert outputs;
 * ClikaRT "QMoEWoQ" page forward: shared_output folds into the same epilogue and the
 * result takes x's dtype).
 *   out[t, :] = round( sum_{j<k} c[t, j] * y[assign_pos[t*k + j], :] + shared[t, :] )
 * with c = topk_w[t, j] (1 under apply_router_weight_on_input) times expert_output_scale,
 * summed in float32 in slot order j, rounded once (nearest-even) to act_dtype.
 * shared_output [T, H] act_dtype may be NULL. No atomics: each output is written once.
 */
qmoe_status qmoe_combine(const qmoe_params* p, const float* y, const int32_t* assign_pos,
                         const float* topk_w, const void* shared_output, void* output,
                         void* stream);

/*
 * The whole forward: route, permute, fc1 + activation, fc2, combine (ClikaRT
 * "QMoEWoQ" page, forward; graiphic "QMoE" page, the node's inputs and attributes).
 *   input [T, H] act_dtype; router_logits [T, E] act_dtype; shared_output [T, H] or NULL;
 *   output [T, H] act_dtype; fc3 ignored unless swiglu with swiglu_fusion 0.
 *   workspace: at least qmoe_workspace_size(p) bytes, 256-byte aligned; its contents on
 *   entry do not matter and are clobbered.
 * Nothing is synchronised and no device-side count returns to the host, so the call
 * can be captured in a HIP graph.
 */
qmoe_status qmoe_forward(const qmoe_params* p, const void* input, const void* router_logits,
                         qmoe_stack fc1, qmoe_stack fc2, qmoe_stack fc3,
                         const void* shared_output, void* output, void* workspace,
                         size_t workspace_bytes, void* stream);

/* Bytes of the fixed device array that qmoe_forward_noalloc keeps its intermediates in
   (one copy per GPU the library runs on, held until the process ends). */
#define QMOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/*
 * qmoe_forward without a workspace, for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid allocation. Same
 * arguments, results and errors as qmoe_forward, less the workspace; the intermediates go
 * to a fixed array of QMOE_NOALLOC_SCRATCH_BYTES inside the library (one per GPU, taken on
 * the first call on that GPU with hipGetSymbolAddress). The call allocates nothing.
 *   Size limit: parameters whose qmoe_workspace_size exceeds QMOE_NOALLOC_SCRATCH_BYTES are
 *   refused with QMOE_ERR_UNSUPPORTED before anything is enqueued (decode-sized batches fit:
 *   64 tokens at H = I = 2880, E = 32 need about 13 MB).
 *   Concurrency: every call on one GPU shares that GPU's array, which keeps the last call's
 *   contents; calls that overlap on one GPU (different streams, or threads without ordering)
 *   race on it. Calls on different GPUs are independent.
 */
qmoe_status qmoe_forward_noalloc(const qmoe_params* p, const void* input,
                                 const void* router_logits, qmoe_stack fc1, qmoe_stack fc2,
                                 qmoe_stack fc3, const void* shared_output, void* output,
                                 void* stream);

/*
 * Where qmoe_forward keeps each intermediate inside its workspace: byte offsets from the
 * workspace start, in this order, each a multiple of 256. A caller may read the pieces
 * back after the forward has completed on its stream (to inspect the routing and the
 * grouping, say); their contents are those of the entry point named beside each.
 *   topk_ids        int32 [T, k]          qmoe_route (not written when fused_routing is 1)
 *   topk_w          float [T, k]          qmoe_route
 *   counts          int32 [E]             qmoe_permute
 *   padded_offsets  int32 [E + 1]         qmoe_permute
 *   sorted_assign   int32 [qmoe_max_rows]  qmoe_permute (rows past padded_offsets[E] hold
 *                                         whatever the workspace held before)
 *   assign_pos      int32 [T * k]         qmoe_permute
 *   tile_list       int32 [qmoe_max_tiles, 2], num_tiles int32 [1]: qmoe_permute
 *   permute_scratch qmoe_permute_scratch_size bytes
 *   h               act_dtype [qmoe_max_rows, I]   qmoe_grouped_gemm_fc1_swiglu (int8 tier:
 *                                         after its rounding)
 *   y               float [qmoe_max_rows, H]       qmoe_grouped_gemm_fc2
 *   xq              act_dtype [T, H]      the int8 tier's rounded x (0 when compute_mode is
 *                                         QMOE_COMPUTE_FLOAT or the int8 dot runs: no such
 *                                         piece)
 *   xcodes, xfactors, hcodes, hfactors   with the int8 tier on the int8 matrix cores (bf16
 *                   activations, tiled weights with integer codes, 128-row tiles, blocks of
 *                   64 or 128, H and I multiples of 64; 0 otherwise): the rounded x and h as
 *                   int8 codes [rows, K] (within every 64 consecutive k the chunks of 8 in the
 *                   order 0, 4, 1, 5, 2, 6, 3, 7) and float factors 2^e [rows, ceil(K/bs)]
 *   total           == qmoe_workspace_size(p)
 *   fused_routing   1 when this batch is routed and grouped by one kernel (small batches:
 *                   the routed ids stay inside that kernel), else 0.
 *   xsum            float [T]: the sum of each row of x, in fp32, with bf16 activations,
 *                   tiled weights, 128-row tiles, one scale per output row and
 *                   compute_mode QMOE_COMPUTE_FLOAT (fc1 takes the zero point's correction
 *                   from it); 0 otherwise.
 *   x16, xlift, h16, hlift   with 4-bit codes and bf16 block scales of 16 to 128, bf16
 *                   activations, tiled weights, 128-row tiles, compute_mode
 *                   QMOE_COMPUTE_FLOAT, H and I multiples of 8 (0 otherwise): x [T, H] and
 *                   h [qmoe_max_rows, I] as fp16 rows, row r multiplied by 2^lift[r]
 *                   (int32 [T] and [qmoe_max_rows]; the power of two that puts the row's
 *                   largest magnitude in [2^14, 2^15)), which the GEMMs take on fp16 matrix
 *                   cores with each weight (q - 8) * scale exact in one fp16 operand; h16
 *                   holds only the rows of the tiles in use.
 *   hpart           where xsum is formed and the codes are 4-bit (0 otherwise): float
 *                   [qmoe_max_rows, n] with n the column blocks of fc1's 128-row kernel (I / 128
 *                   rounded up with SwiGLU, I / 256 with a plain activation): the sum of each
 *                   row of h over each block of columns, written by fc1; followed by float
 *                   [qmoe_max_rows], their totals per row, from which fc2 takes its zero
 *                   point's correction (rows of tiles in use only).
 * Errors: invalid parameters as qmoe_validate; out NULL -> QMOE_ERR_UNBOUND.
 */
typedef struct {
  size_t topk_ids, topk_w, counts, padded_offsets, sorted_assign, assign_pos, tile_list,
      num_tiles, permute_scratch, h, y, xq, total;
  int32_t fused_routing;
  size_t xcodes, xfactors, hcodes, hfactors;
  size_t xsum;
  size_t x16, xlift, h16, hlift;
  size_t hpart;
} qmoe_workspace_layout;

qmoe_status qmoe_workspace_layout_of(const qmoe_params* p, qmoe_workspace_layout* out);

/*
 * The int8 activation tier's rounding (ClikaRT "QMoEWoQ" page, class description: on the
 * int8 block tier the activation is quantised to int8 per block ahead of the dot product).
 *   in, out: [rows, cols] act_dtype, row-major (out may equal in). Each run of
 *   p->block_size elements of a row (a shorter last one when block_size does not divide
 *   cols) gets the power-of-two scale 2^e, e the smallest integer with
 *   max|x| <= 127 * 2^e, and codes q = rint(x / 2^e) (ties to even, |q| <= 127); out holds
 *   q * 2^e, exact in the activation dtype. Needs block_size > 0.
 *   Ownership: the caller owns both buffers; the call only enqueues one kernel on stream.
 *   Errors: the parameter block is validated first (its shapes need not match rows and
 *   cols); block_size 0 -> QMOE_ERR_INVALID; rows < 0 or cols outside [1, 2^31) ->
 *   QMOE_ERR_SHAPE; rows == 0 -> QMOE_OK with nothing enqueued; NULL in or out ->
 *   QMOE_ERR_UNBOUND; a launch failure -> QMOE_ERR_DEVICE.
 * qmoe_forward with compute_mode QMOE_COMPUTE_INT8 applies it to x (cols = hidden_size)
 * and to h (cols = inter_size); the GEMM entry points and qmoe_linear_woq take their
 * inputs as given.
 */
qmoe_status qmoe_quantize_act(const qmoe_params* p, const void* in, int64_t rows, int64_t cols,
                              void* out, void* stream);

/*
 * Weight-only-quantized linear layer (ClikaRT "QLinearWoQ" page: y = x·dequant(W)ᵀ + b,
 * the weight kept quantized at rest, an activation optionally fused as the epilogue):
 * the grouped GEMM of this library over one expert and no routing.
 *   p: the parameter block read as one layer -- num_experts 1, k 1; num_tokens = rows of
 *      x (T), hidden_size = in_features (K), inter_size = out_features (N); activation
 *      QMOE_ACT_IDENTITY, _RELU, _SILU or _GELU (swiglu is rejected, QMOE_ERR_INVALID;
 *      so is apply_router_weight_on_input, which has no routing weight here);
 *      expert_weight_bits, block_size, scale_dtype, act_dtype, tile_m and weight_layout
 *      as for the expert stacks.
 *   x [T, K] act_dtype; w.weights uint8 [N, K*bits/8] (QMOE_LAYOUT_ROWS, dequant
 *   (q - 2^(bits-1)) * scale) or its tiled form (qmoe_pack_stack with which = QMOE_FC1);
 *   w.scales [N, ceil(K/block_size)] or [N] scale_dtype; w.bias [N] act_dtype or NULL;
 *   y [T, N] act_dtype, written row for row (no padding rows).
 * No workspace. Errors as for the other entry points.
 */
qmoe_status qmoe_linear_woq(const qmoe_params* p, const void* x, qmoe_stack w, void* y,
                            void* stream);

/*
 * Measurement hook, not a step of the method. The next grouped-GEMM kernel that the calling
 * thread launches -- the one launch of qmoe_grouped_gemm_fc1_swiglu or
 * qmoe_grouped_gemm_fc2, or qmoe_forward's fc1 and then its fc2 -- records its own start and
 * end on these HIP events (hipEvent_t, created by the caller, timing enabled; either may
 * be NULL), as hipExtLaunchKernel does, so that hipEventElapsedTime(start, stop) is that
 * kernel's duration alone, without the dispatch gap a separately recorded event holds.
 * Up to four pairs may be armed; each GEMM launch takes the oldest and removes it (arm two
 * before qmoe_forward to time both of its GEMMs). (NULL, NULL) clears every pending pair.
 * Thread-local; never fails (pairs beyond four are ignored).
 */
qmoe_status qmoe_time_next_gemm(void* start_event, void* stop_event);

/* Message of the last failing call on this thread (library-owned, valid until the next
   call on this thread); "" after a successful call. */
const char* qmoe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* QMOE_H */
