// Grouped dequant GEMM for bf16 activations on gfx950 MFMA (16x16x32 bf16, fp32 accumulate).
//
// ClikaRT "QMoEWoQ" page, class description: the expert weights stay quantized and each
// block is decoded inside the GEMM dot, never as a dense copy. graiphic "QMoE" page:
// stack shapes [E, N, K/pack], scales per row or per K-block, activation attributes.
//
// One workgroup = one 16-row tile of one expert x 64 output columns (four waves of 16).
// The tile's activation rows are staged in LDS, K at a time in chunks. Each lane of a
// wave owns one output column n and one quarter kq of every 32-wide K step, and decodes
// its 8 weights of the step in registers:
//   4-bit: each nibble q becomes the bfloat16 128+q by OR-ing it into the exponent
//          pattern of 128 (exact), two nibbles per 32-bit register;
//   8-bit: each byte becomes the exact bfloat16 q.
// The MFMA therefore computes sum x*(c+q) with c = 128 (4-bit) or 0 (8-bit). The zero
// point z and the offset c are removed by starting each scale block's accumulation at
// -(c+z)*sum(x over the block), and the block's scale multiplies the block's
// accumulator once. Per-row scales multiply the finished sum.
#include "common.h"
#include "launch.h"

namespace qmoe {

constexpr int kM = 16;
constexpr int kKC = kGemmChunk;
constexpr int kRowPad = 8;  // bf16 elements of padding per LDS row (keeps 16 rows on distinct banks)
constexpr int kStepsPerBatch = 8;

enum BlockMode { kPerRow = 0, kBlocks = 1, kBlocks16 = 2 };

__device__ __forceinline__ bf16x8 decode4(uint32_t w) {
  // element order of the result: [e0, e4, e1, e5, e2, e6, e3, e7] of the 8 nibbles
  const uint32_t magic = 0x43004300u, mask = 0x000F000Fu;
  u32x4 r;
  r[0] = (w & mask) | magic;
  r[1] = ((w >> 4) & mask) | magic;
  r[2] = ((w >> 8) & mask) | magic;
  r[3] = ((w >> 12) & mask) | magic;
  return __builtin_bit_cast(bf16x8, r);
}

__device__ __forceinline__ uint32_t pack_bf16_pair(float lo, float hi) {
  return static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}

__device__ __forceinline__ bf16x8 decode8(u32x2 w) {
  u32x4 r;
  r[0] = pack_bf16_pair(static_cast<float>(w[0] & 0xFF), static_cast<float>((w[0] >> 8) & 0xFF));
  r[1] = pack_bf16_pair(static_cast<float>((w[0] >> 16) & 0xFF), static_cast<float>(w[0] >> 24));
  r[2] = pack_bf16_pair(static_cast<float>(w[1] & 0xFF), static_cast<float>((w[1] >> 8) & 0xFF));
  r[3] = pack_bf16_pair(static_cast<float>((w[1] >> 16) & 0xFF), static_cast<float>(w[1] >> 24));
  return __builtin_bit_cast(bf16x8, r);
}

// Reorders 8 bf16 activations [x0..x7] to [x0, x4, x1, x5, x2, x6, x3, x7] (the 4-bit order).
__device__ __forceinline__ u32x4 order_for_nibbles(u32x4 d) {
  u32x4 o;
  o[0] = (d[0] & 0xFFFFu) | (d[2] << 16);
  o[1] = (d[0] >> 16) | (d[2] & 0xFFFF0000u);
  o[2] = (d[1] & 0xFFFFu) | (d[3] << 16);
  o[3] = (d[1] >> 16) | (d[3] & 0xFFFF0000u);
  return o;
}

__device__ __forceinline__ float bf16_lo(uint32_t d) { return __uint_as_float(d << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t d) { return __uint_as_float(d & 0xFFFF0000u); }

template <typename ST>
__device__ __forceinline__ float load_scale(const ST* p, int64_t i) {
  return load_elem(p, i);
}

template <int BITS>
struct WeightWord;
template <>
struct WeightWord<4> {
  typedef uint32_t type;  // 8 nibbles
  static __device__ __forceinline__ type load(const uint8_t* row, int k) {
    return *reinterpret_cast<const uint32_t*>(row + k / 2);
  }
  static __device__ __forceinline__ bf16x8 decode(type w) { return decode4(w); }
};
template <>
struct WeightWord<8> {
  typedef u32x2 type;  // 8 bytes
  static __device__ __forceinline__ type load(const uint8_t* row, int k) {
    return *reinterpret_cast<const u32x2*>(row + k);
  }
  static __device__ __forceinline__ bf16x8 decode(type w) { return decode8(w); }
};

template <int BITS, typename ST, int MODE, int BMODE>
__global__ __launch_bounds__(256) void gemm_bf16_m16_kernel(GemmArgs g) {
  constexpr float kCorr = BITS == 4 ? 136.0f : 128.0f;  // offset + zero point
  constexpr bool kTwo = (MODE == kModeSwiglu);
  typedef typename WeightWord<BITS>::type WT;

  __shared__ __attribute__((aligned(16))) uint16_t xs[kM][kKC + kRowPad];
  // -(c+z)*sum(x) per (scale group in the chunk, row); per-row mode keeps partial sums of 512.
  __shared__ __attribute__((aligned(16))) float corr[kKC / 16][kM];

  const int tile = blockIdx.y;
  if (tile >= *g.num_tiles) return;
  const int e = g.tile_list[2 * tile];
  const int valid = g.tile_list[2 * tile + 1];
  const int64_t row0 = static_cast<int64_t>(tile) * kM;

  const int tid = threadIdx.x;
  const int wave = tid / kWave, lane = tid % kWave;
  const int n = lane % 16, kq = lane / 16;
  const int col = blockIdx.x * 64 + wave * 16 + n;
  const bool col_ok = col < g.ncols;
  const int c = col_ok ? col : g.ncols - 1;

  // rows of the (up to two) weight streams feeding this lane's output column
  int rA = c, rB = c;
  const uint8_t* wB_base = g.w;
  const ST* sB_base = static_cast<const ST*>(g.s);
  const uint16_t* bB_base = static_cast<const uint16_t*>(g.b);
  int NB = g.N;
  if (kTwo) {
    if (g.fusion == 1) {
      rA = 2 * c;
      rB = 2 * c + 1;
    } else if (g.fusion == 2) {
      rB = g.inter + c;
    } else {
      wB_base = g.w3;
      sB_base = static_cast<const ST*>(g.s3);
      bB_base = static_cast<const uint16_t*>(g.b3);
      NB = g.inter;
    }
  }
  const int64_t row_bytes = static_cast<int64_t>(g.K) * BITS / 8;
  const int64_t gA = static_cast<int64_t>(e) * g.N + rA;
  const int64_t gB = static_cast<int64_t>(e) * NB + rB;
  const uint8_t* pA = g.w + gA * row_bytes;
  const uint8_t* pB = wB_base + gB * row_bytes;
  const ST* sA = static_cast<const ST*>(g.s) + (BMODE == kPerRow ? gA : gA * g.nb);
  const ST* sB = sB_base + (BMODE == kPerRow ? gB : gB * g.nb);

  floatx4 accA = {0.f, 0.f, 0.f, 0.f}, accB = {0.f, 0.f, 0.f, 0.f};
  float totA[4] = {0.f, 0.f, 0.f, 0.f}, totB[4] = {0.f, 0.f, 0.f, 0.f};

  const int gs = (BMODE == kPerRow) ? 512 : g.bs;  // elements per correction group
  const int glanes = gs / 8;                        // loader lanes per group (<= 64)
  const int K = g.K;

  for (int k0 = 0; k0 < K; k0 += kKC) {
    const int kc = min(kKC, K - k0);
    const int kcr = (kc + 511) & ~511;  // loader span (multiple of 512)
    __syncthreads();
    // ---- stage the tile's activation rows [k0, k0+kc) and their group sums ----
    const int g8 = kcr / 8;
    for (int f = tid; f < kM * g8; f += 256) {
      const int m = f / g8, c8 = f % g8;
      const int kk = c8 * 8;
      u32x4 d = {0u, 0u, 0u, 0u};
      if (kk < kc && m < valid) {
        int64_t src_row;
        if (MODE == kModeFc2) {
          src_row = row0 + m;
        } else {
          const int a = g.sorted_assign[row0 + m];
          src_row = a / g.topk;
        }
        d = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(g.a) + src_row * K + k0 + kk);
      }
      float ps = bf16_lo(d[0]) + bf16_hi(d[0]) + bf16_lo(d[1]) + bf16_hi(d[1]) + bf16_lo(d[2]) +
                 bf16_hi(d[2]) + bf16_lo(d[3]) + bf16_hi(d[3]);
      for (int o = 1; o < glanes; o <<= 1) ps += __shfl_xor(ps, o);
      if (c8 % glanes == 0 && kk < kcr) corr[kk / gs][m] = -kCorr * ps;
      if (BITS == 4) d = order_for_nibbles(d);
      if (kk < kKC) *reinterpret_cast<u32x4*>(&xs[m][kk]) = d;
    }
    __syncthreads();

    if (BMODE == kPerRow) {
      // this chunk's correction is applied once, before its first step
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float cs = 0.f;
        for (int p = 0; p < kcr / 512; ++p) cs += corr[p][4 * kq + i];
        accA[i] += cs;
        if (kTwo) accB[i] += cs;
      }
    }

    const int nsteps = kc / 32;
    for (int s0 = 0; s0 < nsteps; s0 += kStepsPerBatch) {
      WT wa[kStepsPerBatch], wb[kStepsPerBatch];
#pragma unroll
      for (int u = 0; u < kStepsPerBatch; ++u) {
        if (s0 + u < nsteps) {
          const int kabs = k0 + 32 * (s0 + u) + 8 * kq;
          wa[u] = WeightWord<BITS>::load(pA, kabs);
          if (kTwo) wb[u] = WeightWord<BITS>::load(pB, kabs);
        }
      }
#pragma unroll
      for (int u = 0; u < kStepsPerBatch; ++u) {
        const int s = s0 + u;
        if (s >= nsteps) break;
        const int kl = 32 * s;        // offset inside the chunk
        const int kabs = k0 + kl;     // offset inside the row
        const bf16x8 xa = *reinterpret_cast<const bf16x8*>(&xs[n][kl + 8 * kq]);
        const bf16x8 ba = WeightWord<BITS>::decode(wa[u]);
        bf16x8 bb;
        if (kTwo) bb = WeightWord<BITS>::decode(wb[u]);
        if (BMODE == kPerRow) {
          accA = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, ba, accA, 0, 0, 0);
          if (kTwo) accB = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, bb, accB, 0, 0, 0);
        } else if (BMODE == kBlocks) {
          const bool first = (kabs % g.bs) == 0;
          const bool last = ((kabs + 32) % g.bs) == 0 || (kabs + 32) >= K;
          if (first) {
            const floatx4 c0 = *reinterpret_cast<const floatx4*>(&corr[kl / g.bs][4 * kq]);
            accA = c0;
            if (kTwo) accB = c0;
          }
          accA = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, ba, accA, 0, 0, 0);
          if (kTwo) accB = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, bb, accB, 0, 0, 0);
          if (last) {
            const int gi = kabs / g.bs;
            const float sa = load_scale(sA, gi);
#pragma unroll
            for (int i = 0; i < 4; ++i) totA[i] += sa * accA[i];
            if (kTwo) {
              const float sb = load_scale(sB, gi);
#pragma unroll
              for (int i = 0; i < 4; ++i) totB[i] += sb * accB[i];
            }
          }
        } else {  // blocks of 16: the step holds two groups; lanes kq<2 hold the first
          const bf16x8 zero = {};
          const bool lo = kq < 2;
          const floatx4 c0 = *reinterpret_cast<const floatx4*>(&corr[kl / 16][4 * kq]);
          const floatx4 c1 = *reinterpret_cast<const floatx4*>(&corr[kl / 16 + 1][4 * kq]);
          const int gi = kabs / 16;
          floatx4 a0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, lo ? ba : zero, c0, 0, 0, 0);
          floatx4 a1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, lo ? zero : ba, c1, 0, 0, 0);
          const float s0a = load_scale(sA, gi), s1a = load_scale(sA, gi + 1);
#pragma unroll
          for (int i = 0; i < 4; ++i) totA[i] += s0a * a0[i] + s1a * a1[i];
          if (kTwo) {
            floatx4 b0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, lo ? bb : zero, c0, 0, 0, 0);
            floatx4 b1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, lo ? zero : bb, c1, 0, 0, 0);
            const float s0b = load_scale(sB, gi), s1b = load_scale(sB, gi + 1);
#pragma unroll
            for (int i = 0; i < 4; ++i) totB[i] += s0b * b0[i] + s1b * b1[i];
          }
        }
      }
    }
  }

  if (BMODE == kPerRow) {
    const float sa = load_scale(sA, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) totA[i] = sa * accA[i];
    if (kTwo) {
      const float sb = load_scale(sB, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) totB[i] = sb * accB[i];
    }
  }

  if (!col_ok) return;
  const float biasA = g.b ? bf16_to_f32(static_cast<const uint16_t*>(g.b)[gA]) : 0.f;
  const float biasB = (kTwo && bB_base) ? bf16_to_f32(bB_base[gB]) : 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = 4 * kq + i;
    const int64_t r = row0 + m;
    if (MODE == kModeFc2) {
      if (m < valid) static_cast<float*>(g.out)[r * g.ncols + col] = totA[i] + biasA;
    } else {
      float h = 0.f;
      if (m < valid) {
        if (MODE == kModeSwiglu)
          h = swiglu(totA[i] + biasA, totB[i] + biasB, g.alpha, g.beta, g.limit);
        else
          h = plain_act(totA[i] + biasA, g.act);
      }
      static_cast<uint16_t*>(g.out)[r * g.ncols + col] = f32_to_bf16(h);
    }
  }
}

template <int BITS, typename ST, int MODE>
static hipError_t launch_bmode(const GemmArgs& g, int64_t max_tiles, hipStream_t s) {
  dim3 grid((g.ncols + 63) / 64, static_cast<unsigned>(max_tiles)), block(256);
  if (g.bs == 0)
    gemm_bf16_m16_kernel<BITS, ST, MODE, kPerRow><<<grid, block, 0, s>>>(g);
  else if (g.bs == 16)
    gemm_bf16_m16_kernel<BITS, ST, MODE, kBlocks16><<<grid, block, 0, s>>>(g);
  else
    gemm_bf16_m16_kernel<BITS, ST, MODE, kBlocks><<<grid, block, 0, s>>>(g);
  return hipGetLastError();
}

template <int BITS, typename ST>
static hipError_t launch_mode(const GemmArgs& g, int mode, int64_t max_tiles, hipStream_t s) {
  if (mode == kModeSwiglu) return launch_bmode<BITS, ST, kModeSwiglu>(g, max_tiles, s);
  if (mode == kModePlainAct) return launch_bmode<BITS, ST, kModePlainAct>(g, max_tiles, s);
  return launch_bmode<BITS, ST, kModeFc2>(g, max_tiles, s);
}

hipError_t launch_gemm_bf16(const GemmArgs& g, int mode, int bits, bool scale_bf16,
                            int64_t max_tiles, hipStream_t s) {
  if (max_tiles <= 0) return hipSuccess;
  if (bits == 4)
    return scale_bf16 ? launch_mode<4, uint16_t>(g, mode, max_tiles, s)
                      : launch_mode<4, float>(g, mode, max_tiles, s);
  return scale_bf16 ? launch_mode<8, uint16_t>(g, mode, max_tiles, s)
                    : launch_mode<8, float>(g, mode, max_tiles, s);
}

}  // namespace qmoe
