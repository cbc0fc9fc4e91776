// Grouped dequant GEMM for bf16 activations and prefill-sized expert groups (128-row tiles),
// bound by the bf16 MFMA rate rather than by the weight stream.
//
// ClikaRT "QMoEWoQ" page, class description: the expert weights stay quantized and each
// block is decoded inside the GEMM dot, never as a dense copy. graiphic "QMoE" page:
// stack shapes [E, N, K/pack], scales per row or per K-block, activation attributes.
//
// This kernel serves the rows layout where the LDS-direct kernels do not (8-bit blocks
// shorter than 64, or K not a whole number of K steps). Workgroup: one 128-row tile of one
// expert, four waves. Per-row scales: a 2 x 2 grid of waves of 64 rows x 4 weight-row
// slices (64 weight rows) each; block scales: 4 x 1 waves of 32 rows x 2 to 6 slices
// (prefill_nb: short blocks need more accumulators, so fewer slices). K advances one
// super-step at a time (128 k for 4-bit, 64 k for 8-bit):
//   - the tile's activations for the next super-step are loaded into registers while the
//     current one computes, then written to LDS in the nibble order of the decode, between
//     two barriers; the same pass sums them per row (per-row scales) or per scale block;
//   - each wave keeps the next super-step's weights in flight in registers and decodes its
//     16-byte loads in registers exactly as the decode-sized kernel does (4-bit: 128+q by
//     OR-ing the nibble into the exponent pattern of 128; 8-bit: exact q), so one decoded
//     weight fragment feeds one MFMA per 16-row slice of the wave's rows.
// The zero point and the +128 offset leave through the activation sums: per-row scales
// subtract (c+z) * rowsum once at the end; block scales start each block's accumulator at
// -(c+z) * blocksum.
#include "common.h"
#include "gemm_common.h"
#include "launch.h"

namespace qmoe {

constexpr int kTM = 128;     // rows per prefill tile
constexpr int kXPad = 8;     // bf16 elements of padding per LDS activation row

// 16-column weight slices per wave. Per-row scales hold 4 row slices x kNB accumulators;
// block scales hold 2 row slices x kNB x (blocks per MFMA k-slice) accumulators plus the
// scaled totals, so small blocks take fewer slices to stay within 256 VGPRs (two waves
// per SIMD).
constexpr int prefill_nb(int bits, int bs) {
  if (bs == 0) return 4;
  const int g = bits == 4 ? (bs == 16 ? 2 : 1) : (bs == 16 ? 4 : (bs == 32 ? 2 : 1));
  return g >= 4 ? 2 : (g == 2 ? 4 : 6);
}

template <int BITS, typename ST, int MODE, int BS>
__global__ __launch_bounds__(256, 2) void gemm_bf16_prefill_kernel(GemmArgs g) {
  constexpr bool PERROW = BS == 0;
  constexpr bool XPOSE = BITS == 4 && BS > 0 && BS < 128;
  constexpr int G = BITS == 4 ? (BS == 16 ? 2 : 1) : (BS == 16 ? 4 : (BS == 32 ? 2 : 1));
  constexpr float kCorr = BITS == 4 ? 136.0f : 128.0f;  // offset + zero point
  constexpr bool kTwo = (MODE == kModeSwiglu);
  constexpr int NS = kTwo ? 2 : 1;
  constexpr int kNB = prefill_nb(BITS, BS);
  constexpr int NBS = kNB / NS;                  // weight slices per stream
  constexpr int SSK = BITS == 4 ? 128 : 64;      // K per super-step
  constexpr int MPS = SSK / 32;                  // MFMA k-slices per super-step
  constexpr int WTM = PERROW ? 4 : 2;            // 16-row slices per wave
  constexpr int WM = kTM / (16 * WTM);           // waves along M
  constexpr int WN = 4 / WM;                     // waves along N
  constexpr int BCOLS = WN * NBS * 16;           // output columns per workgroup
  constexpr int NXS = kTM * SSK / 8 / 256;       // activation uint4 staged per thread
  constexpr int TPR = SSK / 8;                   // staging threads per activation row
  constexpr int GS = PERROW ? SSK : (BS < SSK ? BS : SSK);  // correction group length
  constexpr int GPS = SSK / GS;                  // correction groups per super-step
  constexpr int GLANES = GS / 8;
  constexpr int BSHIFT = BS == 16 ? 4 : BS == 32 ? 5 : BS == 64 ? 6 : BS == 128 ? 7 : BS == 256 ? 8 : 9;
  constexpr int SROWS = WN * kNB * 16;           // weight rows of the workgroup (scale rows)
  constexpr int SPT = PERROW ? 1 : (SROWS * GPS + 255) / 256;  // scales staged per thread

  __shared__ __attribute__((aligned(16))) uint16_t xs[kTM][SSK + kXPad];
  __shared__ __attribute__((aligned(16))) float corr[PERROW ? 1 : GPS][kTM];  // -(c+z) * group sums
  __shared__ float rowcorr[kTM];                                               // -(c+z) * row sums
  __shared__ float scl[PERROW ? 1 : GPS][SROWS];                               // this super-step's scales

  const int tile = blockIdx.x;
  if (tile >= gemm_tile_count(g)) return;
  const int2 tv = gemm_tile(g, tile);
  const int e = tv.x;
  const int valid = tv.y;
  const int64_t row0 = static_cast<int64_t>(tile) * kTM;

  const int tid = threadIdx.x;
  const int wave = tid / kWave, lane = tid % kWave;
  const int n = lane % 16, kq = lane / 16;
  const int wm = wave % WM, wn = wave / WM;
  const int col0 = blockIdx.y * BCOLS;
  const int K = g.K;
  const uint32_t row_bytes = static_cast<uint32_t>(K) * BITS / 8;
  const int nss = (K + SSK - 1) / SSK;

  auto local_row = [&](int st, int c) -> int {
    if (!kTwo) return c;
    if (g.fusion == 1) return 2 * c + st;
    if (g.fusion == 2) return st * g.inter + c;
    return c;
  };
  auto stream_rows = [&](int st) { return (kTwo && g.fusion == 0) ? g.inter : g.N; };
  auto stream_w = [&](int st) { return (st == 1 && kTwo && g.fusion == 0) ? g.w3 : g.w; };
  auto stream_s = [&](int st) { return (st == 1 && kTwo && g.fusion == 0) ? g.s3 : g.s; };
  auto stream_b = [&](int st) { return (st == 1 && kTwo && g.fusion == 0) ? g.b3 : g.b; };

  // weight slice b of this wave: stream b / NBS, output column group b % NBS
  rsrc_t wres[NS];
#pragma unroll
  for (int st = 0; st < NS; ++st) {
    const int nr = stream_rows(st);
    wres[st] = make_rsrc(stream_w(st) + static_cast<int64_t>(e) * nr * row_bytes,
                         static_cast<uint32_t>(nr) * row_bytes);
  }
  uint32_t woff[kNB];
  int lrow[kNB];
#pragma unroll
  for (int b = 0; b < kNB; ++b) {
    const int st = b / NBS;
    const int cl = min(col0 + wn * NBS * 16 + (b % NBS) * 16 + n, g.ncols - 1);
    lrow[b] = local_row(st, cl);
    woff[b] = static_cast<uint32_t>(lrow[b]) * row_bytes + 16 * kq;
  }
  auto wload = [&](int s, u32x4 (&w)[kNB]) {
    const uint32_t kb = static_cast<uint32_t>(s * SSK) * BITS / 8;
#pragma unroll
    for (int b = 0; b < kNB; ++b) w[b] = buf_load16(wres[b / NBS], woff[b] + kb);
  };

  // ---- activations: staging assignment (fixed rows per thread) ----
  const rsrc_t xres = make_rsrc(g.a, static_cast<uint32_t>(g.a_rows * K * 2));
  uint32_t xoff[NXS];
#pragma unroll
  for (int i = 0; i < NXS; ++i) {
    const int f = tid + 256 * i;
    const int m = f / TPR, kk = (f % TPR) * 8;
    if (m < valid) {
      const int64_t src = (MODE == kModeFc2) ? row0 + m : gemm_src_row(g, row0 + m);
      xoff[i] = static_cast<uint32_t>((src * K + kk) * 2);
    } else {
      xoff[i] = kOutOfRange;
    }
  }
  // scale staging: entry f -> (group f % GPS, workgroup weight row f / GPS)
  const ST* srow[SPT];
  int sgi[SPT];
  bool sok[SPT];
  const int nb = PERROW ? 1 : g.nb;
  if (!PERROW) {
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
      const int f = min(tid + 256 * i, SROWS * GPS - 1);
      sok[i] = tid + 256 * i < SROWS * GPS;
      const int r = f / GPS;
      sgi[i] = f % GPS;
      const int wnr = r / (kNB * 16), b = (r % (kNB * 16)) / 16, nn = r % 16;
      const int st = b / NBS;
      const int cl = min(col0 + wnr * NBS * 16 + (b % NBS) * 16 + nn, g.ncols - 1);
      const int nr = stream_rows(st);
      srow[i] = static_cast<const ST*>(stream_s(st)) + (static_cast<int64_t>(e) * nr + local_row(st, cl)) * nb;
    }
  }

  u32x4 sx[NXS];
  ST ssv[SPT];
  auto stage_load = [&](int s) {
    const int k0 = s * SSK;
#pragma unroll
    for (int i = 0; i < NXS; ++i) {
      const int kk = ((tid + 256 * i) % TPR) * 8;
      const u32x4 v = buf_load16(xres, xoff[i] + 2 * k0);
      sx[i] = (k0 + kk < K) ? v : u32x4{0u, 0u, 0u, 0u};
    }
    if (!PERROW) {
#pragma unroll
      for (int i = 0; i < SPT; ++i) ssv[i] = srow[i][min((k0 + sgi[i] * GS) >> BSHIFT, nb - 1)];
    }
  };
  float rs[NXS];  // running row sums (per-row scales), one per staged row of this thread
#pragma unroll
  for (int i = 0; i < NXS; ++i) rs[i] = 0.f;
  auto stage_store = [&]() {
#pragma unroll
    for (int i = 0; i < NXS; ++i) {
      const int f = tid + 256 * i;
      const int m = f / TPR, kk = (f % TPR) * 8;
      u32x4 d = sx[i];
      float ps = bf16_to_f32(d[0] & 0xFFFFu) + __uint_as_float(d[0] & 0xFFFF0000u) +
                 bf16_to_f32(d[1] & 0xFFFFu) + __uint_as_float(d[1] & 0xFFFF0000u) +
                 bf16_to_f32(d[2] & 0xFFFFu) + __uint_as_float(d[2] & 0xFFFF0000u) +
                 bf16_to_f32(d[3] & 0xFFFFu) + __uint_as_float(d[3] & 0xFFFF0000u);
#pragma unroll
      for (int o = 1; o < GLANES; o <<= 1) ps += __shfl_xor(ps, o);
      if (PERROW)
        rs[i] += ps;
      else if ((kk & (GS - 1)) == 0)
        corr[kk / GS][m] = -kCorr * ps;
      if (BITS == 4) d = order_for_nibbles(d);
      *reinterpret_cast<u32x4*>(&xs[m][kk]) = d;
    }
    if (!PERROW) {
#pragma unroll
      for (int i = 0; i < SPT; ++i) {
        const int f = tid + 256 * i;
        if (sok[i]) scl[sgi[i]][f / GPS] = scale_value<ST>(ssv[i]);
      }
    }
  };

  constexpr int NACC = PERROW ? 1 : G;
  floatx4 acc[WTM][kNB][NACC];
  floatx4 tot[PERROW ? 1 : WTM][PERROW ? 1 : kNB];
#pragma unroll
  for (int mt = 0; mt < WTM; ++mt)
#pragma unroll
    for (int b = 0; b < kNB; ++b) {
#pragma unroll
      for (int gg = 0; gg < NACC; ++gg) acc[mt][b][gg] = floatx4{0.f, 0.f, 0.f, 0.f};
      if (!PERROW) tot[mt][b] = floatx4{0.f, 0.f, 0.f, 0.f};
    }
  const bf16x8 zero = {};
  const int lgrp2 = kq >> 1;

  auto compute = [&](u32x4 (&w)[kNB], int s) {
    const int ks0 = s * SSK;
    if (XPOSE) {
#pragma unroll
      for (int b = 0; b < kNB; ++b) transpose_rows4(w[b]);
    }
#pragma unroll
    for (int j = 0; j < MPS; ++j) {
      const int kj = ks0 + 32 * j;
      if (XPOSE && kj >= K) break;
      int xo;
      if (BITS == 4)
        xo = XPOSE ? (32 * j + 8 * kq) : (32 * kq + 8 * j);
      else
        xo = 16 * kq + 8 * j;
      bf16x8 xa[WTM];
#pragma unroll
      for (int mt = 0; mt < WTM; ++mt)
        xa[mt] = *reinterpret_cast<const bf16x8*>(&xs[wm * WTM * 16 + mt * 16 + n][xo]);
      int first = 0, last = 0, gl0 = 0;
      if (!PERROW) {
        if (XPOSE) {
          gl0 = 32 * j / GS;
          first = G == 1 ? ((kj & (GS - 1)) == 0) : 1;
          last = G == 1 ? (((kj + 32) & (GS - 1)) == 0 || kj + 32 >= K) : 1;
        } else {
          // the MFMA's k slots spread over the whole super-step; a block longer than a
          // super-step is summed and scaled one super-step at a time (its correction
          // groups are super-step long), which the linearity of the scale allows
          gl0 = 0;
          first = j == 0 && ((ks0 & (GS - 1)) == 0);
          last = j == MPS - 1 && (((ks0 + SSK) & (GS - 1)) == 0 || ks0 + SSK >= K);
        }
      }
#pragma unroll
      for (int b = 0; b < kNB; ++b) {
        bf16x8 bw;
        if (BITS == 4) {
          bw = decode4(w[b][j]);
        } else {
          u32x2 w2 = {w[b][2 * j], w[b][2 * j + 1]};
          bw = decode8(w2);
        }
        if (PERROW) {
#pragma unroll
          for (int mt = 0; mt < WTM; ++mt)
            acc[mt][b][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[mt], bw, acc[mt][b][0], 0, 0, 0);
          continue;
        }
#pragma unroll
        for (int gg = 0; gg < G; ++gg) {
          const bool mine = (G == 1) || (G == 2 ? (lgrp2 == gg) : (kq == gg));
          const bf16x8 bm = mine ? bw : zero;
#pragma unroll
          for (int mt = 0; mt < WTM; ++mt) {
            floatx4 start = acc[mt][b][gg];
            if (first)
              start = *reinterpret_cast<const floatx4*>(&corr[gl0 + gg][wm * WTM * 16 + mt * 16 + 4 * kq]);
            acc[mt][b][gg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[mt], bm, start, 0, 0, 0);
          }
          if (last) {
            const float sv = scl[gl0 + gg][wn * kNB * 16 + b * 16 + n];
#pragma unroll
            for (int mt = 0; mt < WTM; ++mt)
#pragma unroll
              for (int i = 0; i < 4; ++i) tot[mt][b][i] += sv * acc[mt][b][gg][i];
          }
        }
      }
    }
  };

  // ---- pipeline: one super-step of activations in LDS, the next in registers ----
  u32x4 wa[kNB], wb[kNB];
  stage_load(0);
  wload(0, wa);
  stage_store();
  __syncthreads();
  for (int s = 0; s < nss; s += 2) {
    stage_load(min(s + 1, nss - 1));
    wload(min(s + 1, nss - 1), wb);
    compute(wa, s);
    __syncthreads();
    if (s + 1 < nss) stage_store();
    __syncthreads();
    stage_load(min(s + 2, nss - 1));
    wload(min(s + 2, nss - 1), wa);
    if (s + 1 < nss) compute(wb, s + 1);
    __syncthreads();
    if (s + 2 < nss) stage_store();
    __syncthreads();
  }

  // ---- epilogue ----
  if (PERROW) {
    // row corrections: the staging lanes holding a row's first 8 k write its total
#pragma unroll
    for (int i = 0; i < NXS; ++i) {
      const int f = tid + 256 * i;
      if (f % TPR == 0) rowcorr[f / TPR] = -kCorr * rs[i];
    }
    __syncthreads();
  }
  float bias[kNB];
  float svr[kNB];
#pragma unroll
  for (int b = 0; b < kNB; ++b) {
    const int st = b / NBS;
    const uint16_t* bp = static_cast<const uint16_t*>(stream_b(st));
    bias[b] = bp ? bf16_to_f32(bp[static_cast<int64_t>(e) * stream_rows(st) + lrow[b]]) : 0.f;
    svr[b] = PERROW ? scale_value<ST>(static_cast<const ST*>(stream_s(st))[static_cast<int64_t>(e) * stream_rows(st) + lrow[b]])
                    : 0.f;
  }
#pragma unroll
  for (int mt = 0; mt < WTM; ++mt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = wm * WTM * 16 + mt * 16 + 4 * kq + i;
      const int64_t r = row0 + m;
      const float rc = PERROW ? rowcorr[m] : 0.f;
      // fc1 with the routing weight on the input: the row's weight scales its sums
      const float rs = (MODE != kModeFc2 && m < valid) ? gemm_row_scale(g, r) : 1.f;
#pragma unroll
      for (int cb = 0; cb < NBS; ++cb) {
        const int col = col0 + wn * NBS * 16 + cb * 16 + n;
        if (col >= g.ncols) continue;
        float z[NS];
#pragma unroll
        for (int st = 0; st < NS; ++st) {
          const int b = st * NBS + cb;
          z[st] = (PERROW ? svr[b] * (acc[mt][b][0][i] + rc) : tot[mt][b][i]) * rs + bias[b];
        }
        if (MODE == kModeFc2) {
          if (m < valid) static_cast<float*>(g.out)[r * g.ncols + col] = z[0];
        } else {
          float h = 0.f;
          if (m < valid)
            h = (MODE == kModeSwiglu) ? swiglu(z[0], z[NS - 1], g.alpha, g.beta, g.limit)
                                      : plain_act(z[0], g.act);
          if (m < valid || !g.linear) static_cast<uint16_t*>(g.out)[r * g.ncols + col] = f32_to_bf16(h);
        }
      }
    }
  }
}

template <int BITS, typename ST, int MODE>
static hipError_t launch_prefill_mode(const GemmArgs& g, int64_t max_tiles, hipStream_t s) {
  const bool perrow = g.bs == 0;
  const int wn = perrow ? 2 : 1;
  const int bcols = wn * (prefill_nb(BITS, g.bs) / (MODE == kModeSwiglu ? 2 : 1)) * 16;
  dim3 grid(static_cast<unsigned>(max_tiles), (g.ncols + bcols - 1) / bcols), block(256);
  switch (g.bs) {
    case 0: launch_gemm_kernel(gemm_bf16_prefill_kernel<BITS, ST, MODE, 0>, grid, block, 0, s, g); break;
    case 16: launch_gemm_kernel(gemm_bf16_prefill_kernel<BITS, ST, MODE, 16>, grid, block, 0, s, g); break;
    case 32: launch_gemm_kernel(gemm_bf16_prefill_kernel<BITS, ST, MODE, 32>, grid, block, 0, s, g); break;
    case 64: launch_gemm_kernel(gemm_bf16_prefill_kernel<BITS, ST, MODE, 64>, grid, block, 0, s, g); break;
    case 128: launch_gemm_kernel(gemm_bf16_prefill_kernel<BITS, ST, MODE, 128>, grid, block, 0, s, g); break;
    case 256: launch_gemm_kernel(gemm_bf16_prefill_kernel<BITS, ST, MODE, 256>, grid, block, 0, s, g); break;
    default: launch_gemm_kernel(gemm_bf16_prefill_kernel<BITS, ST, MODE, 512>, grid, block, 0, s, g); break;
  }
  return hipGetLastError();
}

template <int BITS, typename ST>
static hipError_t launch_prefill_t(const GemmArgs& g, int mode, int64_t max_tiles, hipStream_t s) {
  if (mode == kModeSwiglu) return launch_prefill_mode<BITS, ST, kModeSwiglu>(g, max_tiles, s);
  if (mode == kModePlainAct) return launch_prefill_mode<BITS, ST, kModePlainAct>(g, max_tiles, s);
  return launch_prefill_mode<BITS, ST, kModeFc2>(g, max_tiles, s);
}

hipError_t launch_gemm_bf16_prefill(const GemmArgs& g, int mode, int bits, bool scale_bf16,
                                    int64_t max_tiles, hipStream_t s) {
  if (max_tiles <= 0) return hipSuccess;
  // per-row scales over whole K steps (any K in the tiled layout) take the kernel that
  // loads activations into LDS directly
  if (g.bs == 0 && (g.packed || g.K % (bits == 4 ? 128 : 64) == 0))
    return launch_gemm_bf16_prefill_rows(g, mode, bits, scale_bf16, max_tiles, s);
  // block scales of 16 to 128 in the tiled layout: weights scaled as they are decoded
  if (prefill_sw_supports(g))
    return launch_gemm_bf16_prefill_sw(g, mode, bits, scale_bf16, max_tiles, s);
  // other block scales likewise, except 8-bit rows-layout blocks shorter than a 64-wide
  // K step
  if (prefill_blk_supports(g, bits))
    return launch_gemm_bf16_prefill_blk(g, mode, bits, scale_bf16, max_tiles, s);
  if (bits == 4)
    return scale_bf16 ? launch_prefill_t<4, uint16_t>(g, mode, max_tiles, s)
                      : launch_prefill_t<4, float>(g, mode, max_tiles, s);
  return scale_bf16 ? launch_prefill_t<8, uint16_t>(g, mode, max_tiles, s)
                    : launch_prefill_t<8, float>(g, mode, max_tiles, s);
}

}  // namespace qmoe
