// Internal launch interface between the C ABI (api.cpp) and the kernels.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qmoe.h"

namespace qmoe {

// Records msg (and a detail, if non-empty) as the calling thread's qmoe_last_error and
// returns st.
qmoe_status fail_with(qmoe_status st, const char* msg, const char* detail);

// Grouping: one fused block up to this many assignments, otherwise three kernels
// over chunks of kPermChunk assignments.
constexpr int64_t kPermFusedMax = 4096;
constexpr int kPermChunk = 4096;

// K held in LDS per pass by the bf16 grouped GEMM.
constexpr int kGemmChunk = 1024;

enum GemmMode { kModeSwiglu = 0, kModePlainAct = 1, kModeFc2 = 2 };

struct GemmArgs {
  const void* a;               // x [T, K] (fc1) or h [P, K] (fc2), activation dtype
  const int32_t* sorted_assign;  // fc1: assignment of each padded row
  const int32_t* tile_list;    // [tiles, 2] (expert, valid rows)
  const int32_t* num_tiles;
  const uint8_t* w;            // stack [E, N, K*bits/8] (fc1 gate or fused, or fc2)
  const void* s;
  const void* b;
  const uint8_t* w3;           // separate up stack (swiglu_fusion 0)
  const void* s3;
  const void* b3;
  void* out;                   // h [P, ncols] act dtype, or y [P, ncols] f32
  int K;                       // contraction length
  int N;                       // rows of the stack at w
  int ncols;                   // output columns (I for fc1, H for fc2)
  int inter;                   // I (row offset of the up half in concatenated fusion)
  int topk;                    // k, to map an assignment to its token
  int bs;                      // block size, 0 = per output row
  int bs_shift;                // log2(bs) when bs > 0
  int nb;                      // scales per row when bs > 0
  int fusion;
  int act;
  float alpha, beta, limit;
  int M;                       // tile rows
  int64_t a_rows;              // rows of the tensor at a (T for fc1, padded rows for fc2)
  // tiled weight layout (qmoe_pack_stack): 0 = rows [E, N, K*bits/8]
  int packed;
  int kt;                      // tiles along K (ceil(K / S_K))
  int nbk;                     // 16-row blocks per stream
  // single-expert linear layer: the rows of a are the output rows, in consecutive tiles
  // of M rows (no tile list, no gather), and rows past a_rows are never stored
  int linear;
  // MX FP4 weights: E2M1 codes with one E8M0 scale byte per 32 k (tiled layout, natural
  // nibble order); the kernels take them with ST = uint8_t
  int mx;
  // fc1 with the routing weight on the input: the weight of each row's assignment
  // (topk_w, indexed by sorted_assign) scales the row's fp32 sums before the bias; nullptr
  // otherwise
  const float* row_w;
  // the int8 dot: per-block factors 2^e of the rows of a (a then holds int8 codes)
  const float* afac;
  // the 128-row per-row-scale fc1 kernel: the fp32 sum of each row of a (indexed like a's
  // rows), from which the zero point's correction is taken; nullptr: the kernel sums the
  // rows itself
  const float* xsum;
  // the forward with the per-row-scale 128-row kernels (4-bit codes): fc1 also writes, for
  // each row of its tile, the fp32 sum of the bf16 outputs of its column block to
  // hpart[row * hpart_stride + column block] (launch_partsum turns them into h's row sums,
  // which fc2 takes as xsum)
  float* hpart;
  int hpart_stride;
  // the fp16 block-scale kernel (launch_gemm_h16_prefill): a holds fp16 rows, row i lifted
  // by 2^alift[i] (indexed like a's rows); the block scales of weight row n of expert e are
  // lifted by 2^wlift[e * rows + n] (wlift3: the separate up stack); nullptr otherwise
  const int32_t* alift;
  const int32_t* wlift;
  const int32_t* wlift3;
};

// Tiles of a GEMM launch: the grouping's tile list, or the linear layer's row tiles.
__device__ __forceinline__ int gemm_tile_count(const GemmArgs& g) {
  return g.linear ? static_cast<int>((g.a_rows + g.M - 1) / g.M) : *g.num_tiles;
}
// (expert, valid rows) of tile `tile`
__device__ __forceinline__ int2 gemm_tile(const GemmArgs& g, int tile) {
  if (g.linear) {
    const int64_t left = g.a_rows - static_cast<int64_t>(tile) * g.M;
    return make_int2(0, static_cast<int>(left < g.M ? left : g.M));
  }
  return make_int2(g.tile_list[2 * tile], g.tile_list[2 * tile + 1]);
}
// The factor on the fp32 sums of padded row `row` of an fc1-side GEMM (a real row): its
// assignment's routing weight when the weight goes to the expert's input, else 1.
__device__ __forceinline__ float gemm_row_scale(const GemmArgs& g, int64_t row) {
  return g.row_w ? g.row_w[g.sorted_assign[row]] : 1.f;
}
// Row of a that feeds padded row `row` of an fc1-side GEMM (fc2 reads row itself).
__device__ __forceinline__ int64_t gemm_src_row(const GemmArgs& g, int64_t row) {
  return g.linear ? row : g.sorted_assign[row] / g.topk;
}

// Measurement hook: HIP events that the calling thread's next grouped-GEMM launches record
// their own start and end on (hipExtLaunchKernel), one pair per launch in the order the
// pairs were armed. take_gemm_timing returns the oldest pair and removes it (a pair of
// nullptrs when none is armed).
struct GemmTiming {
  hipEvent_t start = nullptr, stop = nullptr;
};
void set_gemm_timing(hipEvent_t start, hipEvent_t stop);
GemmTiming take_gemm_timing();

// Every grouped-GEMM kernel is launched through this: one GemmArgs by value. A launch
// error is left for the caller's hipGetLastError.
inline void launch_gemm_kernel(void (*kernel)(GemmArgs), dim3 grid, dim3 block, size_t lds,
                               hipStream_t s, GemmArgs g) {
  void* args[] = {&g};
  const GemmTiming t = take_gemm_timing();
  if (t.start != nullptr || t.stop != nullptr)
    (void)hipExtLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, args, lds, s,
                             t.start, t.stop, 0);
  else
    (void)hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, args, lds, s);
}

// Tiled layout of one stack: S streams of `rows` rows each, N rows per expert in the
// rows-layout source.
struct PackArgs {
  int E, S, rows, N, K, bits, fusion, NB, KT;
  int natural;  // 4-bit codes keep their order (MX FP4) instead of the decode order
};
hipError_t launch_pack_stack(const uint8_t* src, uint8_t* dst, const PackArgs& a, hipStream_t s);

// Routing variants: selection bias, grouped top-k, weight scaling (route.h).
constexpr int kMaxGroups = 16;
struct RouteOpts {
  const void* bias;     // [E] in the logits' dtype, or nullptr
  int n_group;          // <= 1: no grouping
  int topk_group;
  float scale;          // multiplies the k weights
  bool mixer;           // the sparse mixer (k = 2; no bias, no grouping)
  float mixer_eps;
};

hipError_t launch_route(const void* logits, bool bf16, int T, int E, int k, int normalize,
                        const RouteOpts& o, int32_t* ids, float* w, hipStream_t s);

// One launch for routing and grouping: batches that one 1024-lane block routes in one pass
// (64 tokens when a token takes a 16-lane row, 16 when it takes a wave) and of at most
// kPermFusedMax assignments. The expert ids stay inside the kernel; the weights and the
// grouping are written as by launch_route and launch_permute.
bool route_permute_fits(int64_t T, int64_t A, int64_t E, int64_t k);
hipError_t launch_route_permute(const void* logits, bool bf16, int T, int E, int k, int normalize,
                                const RouteOpts& o, int M, float* w, int32_t* counts,
                                int32_t* padded_offsets, int32_t* sorted_assign,
                                int32_t* assign_pos, int32_t* tile_list, int32_t* num_tiles,
                                hipStream_t s);

size_t permute_scratch_bytes(int64_t A, int E);
hipError_t launch_permute(const int32_t* ids, int64_t A, int E, int M, int32_t* counts,
                          int32_t* padded_offsets, int32_t* sorted_assign, int32_t* assign_pos,
                          int32_t* tile_list, int32_t* num_tiles, void* scratch, hipStream_t s);

// bf16 activations, MFMA 16-row tiles. mode: GemmMode.
hipError_t launch_gemm_bf16(const GemmArgs& g, int mode, int bits, bool scale_bf16,
                            int64_t max_tiles, hipStream_t s);

hipError_t launch_gemm_bf16_tiled(const GemmArgs& g, int mode, int bits, bool scale_bf16,
                                  int64_t max_tiles, hipStream_t s);

// bf16 activations, MFMA 128-row tiles (prefill-sized expert groups).
hipError_t launch_gemm_bf16_prefill(const GemmArgs& g, int mode, int bits, bool scale_bf16,
                                    int64_t max_tiles, hipStream_t s);

// bf16 activations, MFMA 128-row tiles, one scale per output row, K a multiple of 128
// (4-bit) or 64 (8-bit) in the rows layout, any K in the tiled layout: activations loaded
// straight into LDS.
hipError_t launch_gemm_bf16_prefill_rows(const GemmArgs& g, int mode, int bits, bool scale_bf16,
                                         int64_t max_tiles, hipStream_t s);
// Output columns of one workgroup of that kernel's fc1 in mode `mode` (the column blocks
// behind GemmArgs::hpart).
int prefill_rows_fc1_cols(int mode);

// bf16 activations, MFMA 128-row tiles, one scale per output row and K-block. Rows layout:
// K a multiple of 128 (4-bit) or 64 (8-bit), 8-bit blocks of at least 64; tiled layout:
// any block size and K.
bool prefill_blk_supports(const GemmArgs& g, int bits);
hipError_t launch_gemm_bf16_prefill_blk(const GemmArgs& g, int mode, int bits, bool scale_bf16,
                                        int64_t max_tiles, hipStream_t s);
hipError_t launch_gemm_bf16_prefill_blk_tiled(const GemmArgs& g, int mode, int bits,
                                              bool scale_bf16, int64_t max_tiles, hipStream_t s);

// bf16 activations, MFMA 128-row tiles, tiled layout, blocks of 16 to 128 (and MX FP4):
// weights scaled as they are decoded, once per tile.
bool prefill_sw_supports(const GemmArgs& g);
hipError_t launch_gemm_bf16_prefill_sw(const GemmArgs& g, int mode, int bits, bool scale_bf16,
                                       int64_t max_tiles, hipStream_t s);
hipError_t launch_gemm_bf16_prefill_sw8(const GemmArgs& g, int mode, bool scale_bf16,
                                        int64_t max_tiles, hipStream_t s);

// f32 activations, VALU kernel.
hipError_t launch_gemm_f32(const GemmArgs& g, int mode, int bits, bool scale_bf16,
                           int64_t max_tiles, hipStream_t s);

// int8 activation tier: rows x K elements rounded to per-block int8 codes times a power of
// two (quant.hip); in may equal out.
// num_tiles (device, may be null): only the first *num_tiles * tile_m rows are rounded.
hipError_t launch_quantize_blocks(const void* in, void* out, bool bf16, int64_t rows, int K,
                                  int bs, const int32_t* num_tiles, int tile_m, hipStream_t s);

// Combine coefficients: the routing weight (weights = 1) or 1 (weights = 0: the weight went
// to the expert's input), times scale (the expert output scale).
struct CombineOpts {
  int weights;
  float scale;
};
// The same rounding of bf16 rows as int8 codes [rows, K] (the chunks of 8 of every 64-group
// in the order 0, 4, 1, 5, 2, 6, 3, 7) and one factor 2^e per block [rows, ceil(K/bs)] (fp32),
// for the int8 dot. Needs K % 64 == 0, bs in {64, 128}, 16-byte aligned rows.
// The fp32 sum of each of the rows of a bf16 [rows, K] matrix (one wave per row).
hipError_t launch_rowsum(const void* x, float* out, int64_t rows, int K, hipStream_t s);
// The sum of the n fp32 values of each row of parts (row stride n), one wave per row, in a
// fixed order; num_tiles (device): only the first *num_tiles * tile_m rows.
hipError_t launch_partsum(const float* parts, float* out, int64_t rows, int n,
                          const int32_t* num_tiles, int tile_m, hipStream_t s);
hipError_t launch_quantize_codes(const void* in, int8_t* codes, float* fac, int64_t rows, int K,
                                 int bs, const int32_t* num_tiles, int tile_m, hipStream_t s);

// The int8 dot at 128-row tiles (tiled layout, 4- or 8-bit codes, blocks of 64 and 128):
// g.a holds the codes of the rows and g.afac their block factors.
bool prefill_i8_supports(const GemmArgs& g, int bits);
hipError_t launch_gemm_i8_prefill(const GemmArgs& g, int mode, int bits, bool scale_bf16,
                                  int64_t max_tiles, hipStream_t s);

// The fp16 block-scale path (f16prep.hip, gemm_prefill_h16.hip): 4-bit codes with bf16
// block scales of 16 to 128, tiled layout, 128-row tiles, K % 8 == 0.
// Rows of a bf16 [rows, K] matrix to fp16, each lifted by the power of two 2^lift[r] that
// puts its largest magnitude in [2^14, 2^15); num_tiles (device, may be null): only the
// first *num_tiles * tile_m rows.
hipError_t launch_rows_to_f16(const void* in, void* out, int32_t* lift, int64_t rows, int K,
                              const int32_t* num_tiles, int tile_m, hipStream_t s);
// One launch before fc1: for each of up to three scale stacks (scales[i] may be null) of
// rows[i] rows of nb[i] bf16 scales, the power of two 2^lifts[i][r] that puts each row's
// largest scale in [2^12, 2^13); and x [T, H] as rows_to_f16 converts it.
hipError_t launch_prep_f16(const void* const scales[3], int32_t* const lifts[3],
                           const int64_t rows[3], const int nb[3], const void* x, void* x16,
                           int32_t* xlift, int64_t T, int H, hipStream_t s);
// g.a: fp16 rows with g.alift; g.wlift (and g.wlift3) from launch_prep_f16.
hipError_t launch_gemm_h16_prefill(const GemmArgs& g, int mode, int64_t max_tiles, hipStream_t s);

hipError_t launch_combine(const float* y, const int32_t* assign_pos, const float* w,
                          const void* shared, void* out, bool bf16, int T, int H, int k,
                          const CombineOpts& c, hipStream_t s);

}  // namespace qmoe
