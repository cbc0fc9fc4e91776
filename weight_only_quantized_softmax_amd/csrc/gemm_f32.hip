// Grouped dequant GEMM for fp32 activations (VALU, fp32 throughout).
//
// Same operation as the bf16 MFMA kernel (CLIKA "QLinearWoQ" page: x @ dequant(W).T + b,
// per expert; graiphic "QMoE" page: stack and scale shapes), for the fp32 activation type,
// where a bf16 matrix product would not keep fp32 accuracy. The tile's activation rows
// sit in LDS; one wave produces one output column at a time: its lanes split K, decode
// each weight to fp32 in registers as (q - z) * s, and accumulate all tile rows at once;
// a wave-wide sum finishes each row.
#include "common.h"
#include "launch.h"

namespace qmoe {

constexpr int kF32MaxTile = 16;

template <int BITS>
__device__ __forceinline__ int qfield(const uint8_t* row, int k) {
  if (BITS == 8) return row[k];
  const uint8_t b = row[k >> 1];
  return (k & 1) ? (b >> 4) : (b & 0xF);
}

template <int BITS, typename ST>
__device__ __forceinline__ float dequant(const uint8_t* row, const ST* srow, int bs, int k) {
  const float s = load_elem(srow, bs ? k / bs : 0);
  return static_cast<float>(qfield<BITS>(row, k) - (1 << (BITS - 1))) * s;
}

template <int BITS, typename ST, int MODE>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs g) {
  extern __shared__ float xs[];  // [M][K]
  const int tile = blockIdx.y;
  if (tile >= gemm_tile_count(g)) return;
  const int2 tv = gemm_tile(g, tile);
  const int e = tv.x;
  const int valid = tv.y;
  const int M = g.M, K = g.K;
  const int64_t row0 = static_cast<int64_t>(tile) * M;

  for (int f = threadIdx.x; f < M * K; f += blockDim.x) {
    const int m = f / K, kk = f % K;
    float v = 0.f;
    if (m < valid) {
      int64_t src;
      if (MODE == kModeFc2) {
        src = row0 + m;
      } else {
        src = gemm_src_row(g, row0 + m);
      }
      v = static_cast<const float*>(g.a)[src * K + kk];
    }
    xs[f] = v;
  }
  __syncthreads();

  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int col = blockIdx.x * (blockDim.x / kWave) + wave;
  if (col >= g.ncols) return;

  const int64_t row_bytes = static_cast<int64_t>(K) * BITS / 8;
  const int nb = g.bs ? g.nb : 1;
  int rA = col, rB = col;
  const uint8_t* wBb = g.w;
  const ST* sBb = static_cast<const ST*>(g.s);
  const float* bBb = static_cast<const float*>(g.b);
  int NB = g.N;
  if (MODE == kModeSwiglu) {
    if (g.fusion == 1) {
      rA = 2 * col;
      rB = 2 * col + 1;
    } else if (g.fusion == 2) {
      rB = g.inter + col;
    } else {
      wBb = g.w3;
      sBb = static_cast<const ST*>(g.s3);
      bBb = static_cast<const float*>(g.b3);
      NB = g.inter;
    }
  }
  const int64_t gA = static_cast<int64_t>(e) * g.N + rA, gB = static_cast<int64_t>(e) * NB + rB;
  const uint8_t* pA = g.w + gA * row_bytes;
  const uint8_t* pB = wBb + gB * row_bytes;
  const ST* sA = static_cast<const ST*>(g.s) + gA * nb;
  const ST* sB = sBb + gB * nb;

  float accA[kF32MaxTile], accB[kF32MaxTile];
#pragma unroll
  for (int m = 0; m < kF32MaxTile; ++m) accA[m] = accB[m] = 0.f;
  for (int kk = lane; kk < K; kk += kWave) {
    const float wa = dequant<BITS, ST>(pA, sA, g.bs, kk);
    const float wb = (MODE == kModeSwiglu) ? dequant<BITS, ST>(pB, sB, g.bs, kk) : 0.f;
#pragma unroll
    for (int m = 0; m < kF32MaxTile; ++m) {
      if (m < M) {
        const float xv = xs[m * K + kk];
        accA[m] = fmaf(xv, wa, accA[m]);
        if (MODE == kModeSwiglu) accB[m] = fmaf(xv, wb, accB[m]);
      }
    }
  }
  const float biasA = g.b ? static_cast<const float*>(g.b)[gA] : 0.f;
  const float biasB = (MODE == kModeSwiglu && bBb) ? bBb[gB] : 0.f;
#pragma unroll
  for (int m = 0; m < kF32MaxTile; ++m) {
    if (m >= M) continue;
    // fc1 with the routing weight on the input: the row's weight scales its sums
    const float rs = (MODE != kModeFc2 && m < valid) ? gemm_row_scale(g, row0 + m) : 1.f;
    const float za = wave_sum_f32(accA[m]) * rs + biasA;
    float v;
    if (MODE == kModeFc2) {
      v = za;
    } else if (MODE == kModeSwiglu) {
      const float zb = wave_sum_f32(accB[m]) * rs + biasB;
      v = swiglu(za, zb, g.alpha, g.beta, g.limit);
    } else {
      v = plain_act(za, g.act);
    }
    if (lane == 0) {
      if (MODE == kModeFc2) {
        if (m < valid) static_cast<float*>(g.out)[(row0 + m) * g.ncols + col] = v;
      } else {
        if (m < valid || !g.linear)
          static_cast<float*>(g.out)[(row0 + m) * g.ncols + col] = m < valid ? v : 0.f;
      }
    }
  }
}

template <int BITS, typename ST>
static hipError_t launch_f32_t(const GemmArgs& g, int mode, int64_t max_tiles, hipStream_t s) {
  const int waves = 4;
  dim3 grid((g.ncols + waves - 1) / waves, static_cast<unsigned>(max_tiles)), block(64 * waves);
  const size_t lds = static_cast<size_t>(g.M) * g.K * sizeof(float);
  if (mode == kModeSwiglu)
    launch_gemm_kernel(gemm_f32_kernel<BITS, ST, kModeSwiglu>, grid, block, lds, s, g);
  else if (mode == kModePlainAct)
    launch_gemm_kernel(gemm_f32_kernel<BITS, ST, kModePlainAct>, grid, block, lds, s, g);
  else
    launch_gemm_kernel(gemm_f32_kernel<BITS, ST, kModeFc2>, grid, block, lds, s, g);
  return hipGetLastError();
}

hipError_t launch_gemm_f32(const GemmArgs& g, int mode, int bits, bool scale_bf16,
                           int64_t max_tiles, hipStream_t s) {
  if (max_tiles <= 0) return hipSuccess;
  if (bits == 4)
    return scale_bf16 ? launch_f32_t<4, uint16_t>(g, mode, max_tiles, s)
                      : launch_f32_t<4, float>(g, mode, max_tiles, s);
  return scale_bf16 ? launch_f32_t<8, uint16_t>(g, mode, max_tiles, s)
                    : launch_f32_t<8, float>(g, mode, max_tiles, s);
}

}  // namespace qmoe
