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
constexpr int kRowPad = 8;  // bf16 elements of padding per LDS row (keeps 16 rows on distinct banks)

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

// Raw scale storage: bf16 scales stay 16-bit until they are used.
template <typename ST>
__device__ __forceinline__ float scale_value(ST v);
template <>
__device__ __forceinline__ float scale_value<uint16_t>(uint16_t v) { return bf16_to_f32(v); }
template <>
__device__ __forceinline__ float scale_value<float>(float v) { return v; }

// 4x4 transpose of 32-bit words across the four 16-lane rows of a wave: afterwards word j
// of row r holds what word r of row j held. gfx950 permlane32_swap exchanges the upper half
// of its first operand with the lower half of its second; permlane16_swap exchanges the odd
// rows of the first with the even rows of the second.
__device__ __forceinline__ void transpose_rows4(u32x4& d) {
  auto p02 = __builtin_amdgcn_permlane32_swap(d[0], d[2], false, false);
  auto p13 = __builtin_amdgcn_permlane32_swap(d[1], d[3], false, false);
  d[0] = p02[0];
  d[2] = p02[1];
  d[1] = p13[0];
  d[3] = p13[1];
  auto q01 = __builtin_amdgcn_permlane16_swap(d[0], d[1], false, false);
  auto q23 = __builtin_amdgcn_permlane16_swap(d[2], d[3], false, false);
  d[0] = q01[0];
  d[1] = q01[1];
  d[2] = q23[0];
  d[3] = q23[1];
}

// Layout of one lane's 16-byte weight load and of the MFMA steps built from it.
//   4-bit: a load holds 32 consecutive k of the lane's row; a "super-step" of 128 k is the
//          four loads of lanes kq = 0..3 and feeds four MFMAs. Without the transpose, MFMA j
//          takes word j of every lane (k slots spread over the 128); with it (scale blocks of
//          16..64), MFMA j takes the 32 consecutive k [32j, 32j+32) of the super-step.
//   8-bit: a load holds 16 consecutive k; a super-step is 64 k and feeds two MFMAs; MFMA j
//          takes bytes [8j, 8j+8) of every lane (k slots spread over the 64).
// G > 1 splits an MFMA whose k slots span G scale blocks into G MFMAs, each with the
// weights of the other blocks' lanes zeroed.
template <int BITS, typename ST, int MODE, int BS>
__global__ __launch_bounds__(256) void gemm_bf16_m16_kernel(GemmArgs g) {
  constexpr bool PERROW = BS == 0;
  // 4-bit blocks of 16..64 take the transposed layout; spans of several blocks are split
  constexpr bool XPOSE = BITS == 4 && BS > 0 && BS < 128;
  constexpr int G = BITS == 4 ? (BS == 16 ? 2 : 1) : (BS == 16 ? 4 : (BS == 32 ? 2 : 1));
  constexpr float kCorr = BITS == 4 ? 136.0f : 128.0f;  // offset + zero point
  constexpr bool kTwo = (MODE == kModeSwiglu);
  constexpr int NS = kTwo ? 2 : 1;              // weight streams per lane
  constexpr int KC = BITS == 4 ? 512 : 256;     // K per chunk (256 bytes of every row)
  constexpr int SSK = BITS == 4 ? 128 : 64;     // K per super-step
  constexpr int SPC = KC / SSK;                 // super-steps per chunk (4)
  constexpr int MPS = SSK / 32;                 // MFMAs per super-step
  constexpr int NX = KC / 128;                  // activation uint4 staged per thread
  // correction / scale group: a scale block, or the part of one inside a K chunk (the
  // block's scale then multiplies each part's accumulator)
  constexpr int GS = PERROW ? KC : (BS < KC ? BS : KC);
  constexpr int BSHIFT = BS == 16 ? 4 : BS == 32 ? 5 : BS == 64 ? 6 : BS == 128 ? 7 : BS == 256 ? 8 : 9;
  constexpr int GSHIFT = GS == 16 ? 4 : GS == 32 ? 5 : GS == 64 ? 6 : GS == 128 ? 7 : GS == 256 ? 8 : 9;
  static_assert((1 << GSHIFT) == GS, "block length must be a power of two in [16, 512]");
  constexpr int GPC = KC / GS;                    // blocks per chunk
  constexpr int TPR = 256 / (NS * 64);            // staging threads per scale row (2 or 4)
  constexpr int NSE = PERROW ? 1 : (GPC + TPR - 1) / TPR;  // scales staged per thread
  constexpr int kMaxGroups = KC / 16;

  __shared__ __attribute__((aligned(16))) uint16_t xs[kM][KC + kRowPad];
  __shared__ __attribute__((aligned(16))) float corr[kMaxGroups][kM];  // -(c+z)*sum(x) per block, row
  __shared__ float sc[PERROW ? 1 : kMaxGroups][NS * 64];                // scales per block, column

  const int tile = blockIdx.y;
  if (tile >= *g.num_tiles) return;
  const int e = g.tile_list[2 * tile];
  const int valid = g.tile_list[2 * tile + 1];
  const int64_t row0 = static_cast<int64_t>(tile) * kM;

  const int tid = threadIdx.x;
  const int wave = tid / kWave, lane = tid % kWave;
  const int n = lane % 16, kq = lane / 16;
  const int col0 = blockIdx.x * 64;
  const int col = col0 + wave * 16 + n;
  const bool col_ok = col < g.ncols;
  const int K = g.K;
  const int64_t row_bytes = static_cast<int64_t>(K) * BITS / 8;

  // stack row, weight row and scale row of column c in stream st
  auto stack_row = [&](int st, int c) -> int64_t {
    if (!kTwo) return static_cast<int64_t>(e) * g.N + c;
    if (g.fusion == 1) return static_cast<int64_t>(e) * g.N + 2 * c + st;
    if (g.fusion == 2) return static_cast<int64_t>(e) * g.N + st * g.inter + c;
    return st == 0 ? static_cast<int64_t>(e) * g.N + c : static_cast<int64_t>(e) * g.inter + c;
  };
  auto wbase = [&](int st) { return (st == 1 && kTwo && g.fusion == 0) ? g.w3 : g.w; };
  auto sbase = [&](int st) {
    return static_cast<const ST*>((st == 1 && kTwo && g.fusion == 0) ? g.s3 : g.s);
  };

  const int c = col_ok ? col : g.ncols - 1;
  const uint8_t* wrow[NS];
  int64_t grow[NS];
#pragma unroll
  for (int st = 0; st < NS; ++st) {
    grow[st] = stack_row(st, c);
    wrow[st] = wbase(st) + grow[st] * row_bytes;
  }

  constexpr int gs = GS;
  constexpr int gshift = GSHIFT;
  constexpr int glanes = GS / 8;  // loader lanes per block
  const int nchunks = (K + KC - 1) / KC;
  // scale staging: thread tid stages groups part, part + TPR, ... of scale row srow
  const int srow = tid % (NS * 64), spart = tid / (NS * 64);
  const ST* sptr = nullptr;
  if (!PERROW) {
    const int st = srow / 64;
    const int cc = min(col0 + (srow % 64), g.ncols - 1);
    sptr = sbase(st) + stack_row(st, cc) * g.nb;
  }

  // ---- staging of one chunk: activations (+ block sums) and scales ----
  u32x4 sx[NX];
  ST ss[NSE];
  auto stage_load = [&](int ci) {
    const int k0 = ci * KC;
#pragma unroll
    for (int i = 0; i < NX; ++i) {
      const int f = tid + 256 * i;
      const int m = f / (KC / 8), kk = (f % (KC / 8)) * 8;
      const bool ok = (k0 + kk < K) && (m < valid);
      int64_t src;
      if (MODE == kModeFc2) {
        src = row0 + min(m, valid - 1);
      } else {
        src = g.sorted_assign[row0 + min(m, valid - 1)] / g.topk;
      }
      const u32x4 v = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(g.a) + src * K +
                                                      min(k0 + kk, K - 8));
      sx[i] = ok ? v : u32x4{0u, 0u, 0u, 0u};
    }
    if (!PERROW) {
#pragma unroll
      for (int i = 0; i < NSE; ++i)
        ss[i] = sptr[min((k0 + (spart + TPR * i) * GS) >> BSHIFT, g.nb - 1)];
    }
  };
  auto stage_store = [&]() {
#pragma unroll
    for (int i = 0; i < NX; ++i) {
      const int f = tid + 256 * i;
      const int m = f / (KC / 8), kk = (f % (KC / 8)) * 8;
      u32x4 d = sx[i];
      float ps = bf16_lo(d[0]) + bf16_hi(d[0]) + bf16_lo(d[1]) + bf16_hi(d[1]) + bf16_lo(d[2]) +
                 bf16_hi(d[2]) + bf16_lo(d[3]) + bf16_hi(d[3]);
      for (int o = 1; o < glanes; o <<= 1) ps += __shfl_xor(ps, o);
      if ((kk & (gs - 1)) == 0) corr[kk >> gshift][m] = -kCorr * ps;
      if (BITS == 4) d = order_for_nibbles(d);
      *reinterpret_cast<u32x4*>(&xs[m][kk]) = d;
    }
    if (!PERROW) {
#pragma unroll
      for (int i = 0; i < NSE; ++i) {
        const int gi = spart + TPR * i;
        if (gi < GPC) sc[gi][srow] = scale_value<ST>(ss[i]);
      }
    }
  };

  // ---- weights of one chunk: SPC 16-byte loads per stream ----
  auto wload = [&](int ci, u32x4 (&w)[NS][SPC]) {
#pragma unroll
    for (int st = 0; st < NS; ++st)
#pragma unroll
      for (int u = 0; u < SPC; ++u) {
        const int64_t off = min<int64_t>((static_cast<int64_t>(ci) * KC + SSK * u) * BITS / 8 + 16 * kq,
                                         row_bytes - 16);
        w[st][u] = *reinterpret_cast<const u32x4*>(wrow[st] + off);
      }
  };

  floatx4 acc[NS][G];
  float tot[NS][4];
#pragma unroll
  for (int st = 0; st < NS; ++st) {
#pragma unroll
    for (int gg = 0; gg < G; ++gg) acc[st][gg] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) tot[st][i] = 0.f;
  }

  u32x4 wcur[NS][SPC];
  stage_load(0);
  wload(0, wcur);
  stage_store();
  __syncthreads();

  const int lgrp2 = kq >> 1;  // lane's block among two
  for (int ci = 0; ci < nchunks; ++ci) {
    const int cn = min(ci + 1, nchunks - 1);
    stage_load(cn);
    u32x4 wnxt[NS][SPC];
    wload(cn, wnxt);
    const int k0 = ci * KC;

    if (PERROW) {
#pragma unroll
      for (int st = 0; st < NS; ++st)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[st][0][i] += corr[0][4 * kq + i];
    }

#pragma unroll
    for (int u = 0; u < SPC; ++u) {
      const int ks = k0 + SSK * u;  // first k of the super-step
      if (ks >= K) break;
      if (XPOSE) {
#pragma unroll
        for (int st = 0; st < NS; ++st) transpose_rows4(wcur[st][u]);
      }
#pragma unroll
      for (int j = 0; j < MPS; ++j) {
        const int kj = ks + 32 * j;
        if (XPOSE && kj >= K) break;
        int xo;  // this lane's 8 activations for MFMA j, offset inside the chunk
        if (BITS == 4)
          xo = XPOSE ? (SSK * u + 32 * j + 8 * kq) : (SSK * u + 32 * kq + 8 * j);
        else
          xo = SSK * u + 16 * kq + 8 * j;
        const bf16x8 xa = *reinterpret_cast<const bf16x8*>(&xs[n][xo]);
        bf16x8 bw[NS];
#pragma unroll
        for (int st = 0; st < NS; ++st) {
          if (BITS == 4) {
            bw[st] = decode4(wcur[st][u][j]);
          } else {
            u32x2 w2 = {wcur[st][u][2 * j], wcur[st][u][2 * j + 1]};
            bw[st] = decode8(w2);
          }
        }
        if (PERROW) {
#pragma unroll
          for (int st = 0; st < NS; ++st)
            acc[st][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, bw[st], acc[st][0], 0, 0, 0);
          continue;
        }
        // span of this MFMA and where its scale blocks start and end
        int first, last, gl0;
        if (BITS == 4 && XPOSE) {
          gl0 = (kj - k0) >> gshift;
          if (G == 1) {
            first = (kj & (gs - 1)) == 0;
            last = ((kj + 32) & (gs - 1)) == 0 || kj + 32 >= K;
          } else {
            first = last = 1;  // two blocks of 16 inside the 32
          }
        } else {
          // the MFMA's k slots spread over the whole super-step [ks, ks + SSK)
          gl0 = (ks - k0) >> gshift;
          first = (j == 0) && ((ks & (gs - 1)) == 0);
          last = (j == MPS - 1) && (((ks + SSK) & (gs - 1)) == 0 || ks + SSK >= K);
        }
#pragma unroll
        for (int gg = 0; gg < G; ++gg) {
          const int gl = gl0 + gg;
          const bool mine = (G == 1) || (G == 2 ? (lgrp2 == gg) : (kq == gg));
          if (first) {
            const floatx4 c0 = *reinterpret_cast<const floatx4*>(&corr[gl][4 * kq]);
#pragma unroll
            for (int st = 0; st < NS; ++st) acc[st][gg] = c0;
          }
#pragma unroll
          for (int st = 0; st < NS; ++st) {
            const bf16x8 zero = {};
            const bf16x8 b = mine ? bw[st] : zero;
            acc[st][gg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, b, acc[st][gg], 0, 0, 0);
          }
          if (last) {
#pragma unroll
            for (int st = 0; st < NS; ++st) {
              const float sv = sc[gl][st * 64 + wave * 16 + n];
#pragma unroll
              for (int i = 0; i < 4; ++i) tot[st][i] += sv * acc[st][gg][i];
            }
          }
        }
      }
    }
    __syncthreads();
    if (ci + 1 < nchunks) stage_store();
    __syncthreads();
#pragma unroll
    for (int st = 0; st < NS; ++st)
#pragma unroll
      for (int u = 0; u < SPC; ++u) wcur[st][u] = wnxt[st][u];
  }

  if (PERROW) {
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      const float sv = scale_value<ST>(sbase(st)[grow[st]]);
#pragma unroll
      for (int i = 0; i < 4; ++i) tot[st][i] = sv * acc[st][0][i];
    }
  }

  if (!col_ok) return;
  float bias[NS];
#pragma unroll
  for (int st = 0; st < NS; ++st) {
    const uint16_t* bp = static_cast<const uint16_t*>((st == 1 && kTwo && g.fusion == 0) ? g.b3 : g.b);
    bias[st] = bp ? bf16_to_f32(bp[grow[st]]) : 0.f;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = 4 * kq + i;
    const int64_t r = row0 + m;
    if (MODE == kModeFc2) {
      if (m < valid) static_cast<float*>(g.out)[r * g.ncols + col] = tot[0][i] + bias[0];
    } else {
      float h = 0.f;
      if (m < valid) {
        if (MODE == kModeSwiglu)
          h = swiglu(tot[0][i] + bias[0], tot[NS - 1][i] + bias[NS - 1], g.alpha, g.beta, g.limit);
        else
          h = plain_act(tot[0][i] + bias[0], g.act);
      }
      static_cast<uint16_t*>(g.out)[r * g.ncols + col] = f32_to_bf16(h);
    }
  }
}

template <int BITS, typename ST, int MODE>
static hipError_t launch_bmode(const GemmArgs& g, int64_t max_tiles, hipStream_t s) {
  dim3 grid((g.ncols + 63) / 64, static_cast<unsigned>(max_tiles)), block(256);
  switch (g.bs) {
    case 0: gemm_bf16_m16_kernel<BITS, ST, MODE, 0><<<grid, block, 0, s>>>(g); break;
    case 16: gemm_bf16_m16_kernel<BITS, ST, MODE, 16><<<grid, block, 0, s>>>(g); break;
    case 32: gemm_bf16_m16_kernel<BITS, ST, MODE, 32><<<grid, block, 0, s>>>(g); break;
    case 64: gemm_bf16_m16_kernel<BITS, ST, MODE, 64><<<grid, block, 0, s>>>(g); break;
    case 128: gemm_bf16_m16_kernel<BITS, ST, MODE, 128><<<grid, block, 0, s>>>(g); break;
    case 256: gemm_bf16_m16_kernel<BITS, ST, MODE, 256><<<grid, block, 0, s>>>(g); break;
    default: gemm_bf16_m16_kernel<BITS, ST, MODE, 512><<<grid, block, 0, s>>>(g); break;
  }
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
