// Grouped dequant GEMM for the smallest decode batches: the weight-streaming form of the
// per-expert FFN GEMMs of the ClikaRT "QMoEWoQ" page (the codes are expanded block by block
// within the dot product, and the weights stream at their quantized size), for grids too
// small to fill the chip with 16-row tiles of several column groups each.
//
// One workgroup = one 16-row tile x one column group (16 SwiGLU outputs from a gate and
// an up stream, or 2 x 16 outputs). Its NW waves split K into NW contiguous ranges of
// tiles of the tiled weight layout (qmoe_pack_stack): every wave streams its own range,
// 16 bytes per lane per tile and stream, with the activations of its lanes read straight
// into registers (a lane holds row n's eight k of its MFMA k-group; rows past the tile's
// valid rows read zeros). There is no LDS stage and no barrier inside the K loop, so the
// waves run apart; the serial chain of a wave is 1/NW of K. The scales of the group sit
// in LDS, the ranges' partial sums meet in LDS in range order, and wave 0 stores.
//
// Arithmetic as in the 16-row tile kernel: 4-bit codes become 128 + q (8-bit: q) exactly
// in bf16, one MFMA against -(c + z) folds the offset and zero point into each scale
// group's fp32 sum, and each group's sum is scaled once (per-row scales once at the end).
#pragma once

#include <type_traits>

#include "common.h"
#include "gemm_common.h"
#include "launch.h"

namespace qmoe {

template <int BITS, typename ST, int MODE, int BS, int NW, int PD>
__global__ __launch_bounds__(NW * 64) void gemm_bf16_gemv_kernel(GemmArgs g) {
  constexpr bool PERROW = BS == 0;
  constexpr bool MX = std::is_same<ST, uint8_t>::value;  // MX FP4: scaled as converted
  static_assert(!MX || (BITS == 4 && BS == 32), "MX FP4: 4-bit, blocks of 32");
  constexpr int SSK = BITS == 4 ? 128 : 64;  // K per weight tile
  constexpr int MPS = SSK / 32;              // MFMAs per tile
  constexpr bool XPOSE = BS > 0 && BS < SSK; // several scale groups inside one tile
  constexpr int G = BS == 16 ? 2 : 1;        // scale groups inside one MFMA
  constexpr bool kTwo = MODE == kModeSwiglu;
  constexpr int NS = 2;                      // weight streams per lane
  constexpr int CW = kTwo ? 16 : 32;         // output columns of the workgroup
  constexpr int BSHIFT = BS == 16 ? 4 : BS == 32 ? 5 : BS == 64 ? 6 : BS == 128 ? 7 : BS == 256 ? 8 : 9;
  constexpr uint32_t kNegCorr = BITS == 4 ? 0xC308C308u : 0xC300C300u;
  static_assert(PD >= 1 && PD <= 4, "prefetch distance 1 to 4");

  extern __shared__ __attribute__((aligned(16))) unsigned char dyn[];  // scales, then partials

  const int tile = blockIdx.y;
  if (tile >= gemm_tile_count(g)) return;
  const int2 tv = gemm_tile(g, tile);
  const int e = tv.x;
  const int valid = min(tv.y, kM);
  const int64_t row0 = static_cast<int64_t>(tile) * kM;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
  const int n = lane % 16, kq = lane / 16;
  const int col0 = blockIdx.x * CW;
  auto col_of = [&](int st) { return col0 + (kTwo ? 0 : 16 * st) + n; };
  const int K = g.K;
  const int nss = g.kt;                                // weight tiles along K
  const int per = (nss + NW - 1) / NW;
  const int s0 = min(wave * per, nss), s1 = min(s0 + per, nss);  // this wave's K tiles

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

  // weight tile sequence of each stream (a 16-row block past the stream reads zeros)
  rsrc_t wres[NS];
  int lrow[NS];
  const int ns = (kTwo && g.fusion != 0) ? 2 : 1;
#pragma unroll
  for (int st = 0; st < NS; ++st) {
    lrow[st] = local_row(st, min(col_of(st), g.ncols - 1));  // clamped: stored only if valid
    const int si = (kTwo && g.fusion != 0) ? st : 0;
    const int rb = (col0 + (kTwo ? 0 : 16 * st)) / 16;
    const int64_t tile0 = ((static_cast<int64_t>(e) * ns + si) * g.nbk + rb) * g.kt;
    wres[st] = make_rsrc(stream_w(st) + tile0 * 1024,
                         rb < g.nbk ? static_cast<uint32_t>(g.kt) * 1024u : 0u);
  }
  // this lane's activation row (past the valid rows: out of range, zeros)
  const rsrc_t xres = make_rsrc(g.a, static_cast<uint32_t>(g.a_rows * K * 2));
  uint32_t xoff = kOutOfRange;
  if (n < valid) {
    const int64_t src = (MODE == kModeFc2) ? row0 + n : gemm_src_row(g, row0 + n);
    xoff = static_cast<uint32_t>((src * K + 8 * kq) * 2);
  }

  // ---- scales of the group's rows into LDS (one range per stream, or one for both when
  // gate and up rows interleave or the streams are adjacent column blocks) ----
  const int nb = PERROW ? 1 : g.nb;
  ST* scl = reinterpret_cast<ST*>(dyn);
  const bool one_range = !kTwo || g.fusion == 1;
  const int rowb = nb * static_cast<int>(sizeof(ST));
  if (!PERROW) {
    const int nrange = one_range ? 1 : NS;
    const int rows = one_range ? 32 : 16;
#pragma unroll
    for (int rg = 0; rg < NS; ++rg) {
      if (rg >= nrange) break;
      const int nr = stream_rows(rg);
      const rsrc_t sres = make_rsrc(static_cast<const unsigned char*>(stream_s(rg)) +
                                        static_cast<int64_t>(e) * nr * rowb,
                                    static_cast<uint32_t>(nr) * rowb);
      const int rstart = one_range ? (kTwo ? 2 * col0 : col0) : local_row(rg, col0);
      const uint32_t gstart = static_cast<uint32_t>(rstart) * rowb;
      const int granules = rows * rowb / 16;
      unsigned char* ldst = dyn + rg * rows * rowb;
      for (int it = wave; it * 64 < granules; it += NW) {
        if (it * 64 + lane < granules)
          buf_load16_lds(sres, ldst + it * 1024, gstart + 16u * (it * 64 + lane), 0);
      }
    }
  }

  // ---- register ring: PD tiles ahead ----
  struct Slot {
    u32x4 w[NS];
    u32x4 x[MPS];
  };
  auto load = [&](int ss, Slot& sl) {
    if (ss < s1) {
#pragma unroll
      for (int st = 0; st < NS; ++st) sl.w[st] = buf_load16_stream(wres[st], 16u * lane + ss * 1024u);
#pragma unroll
      for (int j = 0; j < MPS; ++j)
        sl.x[j] = buf_load16s(xres, xoff, static_cast<uint32_t>(2 * (ss * SSK + 32 * j)));
    }
  };
  Slot ring[PD + 1];
#pragma unroll
  for (int i = 0; i < PD; ++i) load(s0 + i, ring[i]);

  // the scales have landed in LDS for every wave (the only barrier before the epilogue)
  __syncthreads();
  const ST* my_scl[NS];
#pragma unroll
  for (int st = 0; st < NS; ++st)
    my_scl[st] = scl + (!kTwo ? 16 * st + n : one_range ? 2 * n + st : st * 16 + n) * nb;

  floatx4 acc[NS][G];
  float tot[NS][4];
  const floatx4 zero4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int st = 0; st < NS; ++st) {
#pragma unroll
    for (int gg = 0; gg < G; ++gg) acc[st][gg] = zero4;
#pragma unroll
    for (int i = 0; i < 4; ++i) tot[st][i] = 0.f;
  }
  const bf16x8 zero = {};
  u32x4 negc_bits = {kNegCorr, kNegCorr, kNegCorr, kNegCorr};
  asm volatile("" : "+v"(negc_bits));
  const bf16x8 negc = __builtin_bit_cast(bf16x8, negc_bits);
  const int lgrp2 = kq >> 1;

  // one weight tile: MPS MFMAs of 32 k (k-slices past K skipped), scale groups closed
  // inside the tile
  auto compute = [&](const Slot& sl, int ss) {
    const int ksu = ss * SSK;
#pragma unroll
    for (int j = 0; j < MPS; ++j) {
      const int kj = ksu + 32 * j;
      if (kj >= K) break;
      const bf16x8 xa = __builtin_bit_cast(bf16x8, sl.x[j]);
      if constexpr (MX) {
#pragma unroll
        for (int st = 0; st < NS; ++st) {
          const bf16x8 bm = decode_mx(sl.w[st][j], scale_value<ST>(my_scl[st][kj >> 5]));
          acc[st][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, bm, acc[st][0], 0, 0, 0);
        }
        continue;
      }
      bf16x8 bw[NS];
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        if (BITS == 4) {
          bw[st] = decode4(sl.w[st][j]);
        } else {
          u32x2 w2 = {sl.w[st][2 * j], sl.w[st][2 * j + 1]};
          bw[st] = decode8(w2);
        }
      }
      int first = 0, last = 0, blk0 = 0;
      if (!PERROW) {
        if (XPOSE) {
          blk0 = kj >> BSHIFT;
          first = G > 1 || (kj & (BS - 1)) == 0;
          last = G > 1 || ((kj + 32) & (BS - 1)) == 0 || kj + 32 >= K;
        } else {
          // a block of a tile or longer: summed and scaled one tile at a time
          blk0 = ksu >> BSHIFT;
          first = j == 0;
          last = j == MPS - 1 || kj + 32 >= K;
        }
      }
#pragma unroll
      for (int gg = 0; gg < G; ++gg) {
        const bool mine = (G == 1) || (lgrp2 == gg);
#pragma unroll
        for (int st = 0; st < NS; ++st) {
          const floatx4 from = first ? zero4 : acc[st][gg];
          acc[st][gg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, mine ? negc : zero, from, 0, 0, 0);
          acc[st][gg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, mine ? bw[st] : zero,
                                                                acc[st][gg], 0, 0, 0);
        }
        if (last) {
          // the 16-blocks of a 4-bit MFMA are blk0 and blk0 + 1 (the second may lie past
          // K when K is not a multiple of 32: clamped, its products are zero)
          const int blk = G > 1 ? min(blk0 + gg, nb - 1) : blk0;
#pragma unroll
          for (int st = 0; st < NS; ++st) {
            const float sv = scale_value<ST>(my_scl[st][blk]);
#pragma unroll
            for (int i = 0; i < 4; ++i) tot[st][i] += sv * acc[st][gg][i];
          }
        }
      }
    }
  };

  // PD + 1 tiles per trip so that ring slots are fixed
  for (int ss = s0; ss < s1; ss += PD + 1) {
#pragma unroll
    for (int r = 0; r <= PD; ++r) {
      load(ss + r + PD, ring[(r + PD) % (PD + 1)]);
      if (ss + r < s1) compute(ring[r], ss + r);
    }
  }

  if (MX) {
#pragma unroll
    for (int st = 0; st < NS; ++st)
#pragma unroll
      for (int i = 0; i < 4; ++i) tot[st][i] = acc[st][0][i];
  }
  if (PERROW) {
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      const float sv = scale_value<ST>(
          static_cast<const ST*>(stream_s(st))[static_cast<int64_t>(e) * stream_rows(st) + lrow[st]]);
#pragma unroll
      for (int i = 0; i < 4; ++i) tot[st][i] = sv * acc[st][0][i];
    }
  }

  // ---- the K ranges' partial sums meet in LDS, added in range order ----
  constexpr int kPart = NS * 4;
  float* red = reinterpret_cast<float*>(dyn + (PERROW ? 0 : 32 * rowb + 15) / 16 * 16);
  if (wave > 0) {
    float* my = red + (wave - 1) * kPart * 64;
#pragma unroll
    for (int st = 0; st < NS; ++st)
#pragma unroll
      for (int i = 0; i < 4; ++i) my[(st * 4 + i) * 64 + lane] = tot[st][i];
  }
  __syncthreads();
  if (wave > 0) return;
#pragma unroll
  for (int q = 1; q < NW; ++q) {
    const float* other = red + (q - 1) * kPart * 64;
#pragma unroll
    for (int st = 0; st < NS; ++st)
#pragma unroll
      for (int i = 0; i < 4; ++i) tot[st][i] += other[(st * 4 + i) * 64 + lane];
  }

  float bias[NS];
#pragma unroll
  for (int st = 0; st < NS; ++st) {
    const uint16_t* bp = static_cast<const uint16_t*>(stream_b(st));
    bias[st] = bp ? bf16_to_f32(bp[static_cast<int64_t>(e) * stream_rows(st) + lrow[st]]) : 0.f;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = 4 * kq + i;
    const int64_t r = row0 + m;
    // fc1 with the routing weight on the input: the row's weight scales its sums
    const float rs = (MODE != kModeFc2 && m < valid) ? gemm_row_scale(g, r) : 1.f;
    if (MODE == kModeSwiglu) {
      const int col = col_of(0);
      if (col >= g.ncols) continue;
      float h = 0.f;
      if (m < valid)
        h = swiglu(tot[0][i] * rs + bias[0], tot[1][i] * rs + bias[1], g.alpha, g.beta, g.limit);
      if (m < valid || !g.linear) static_cast<uint16_t*>(g.out)[r * g.ncols + col] = f32_to_bf16(h);
    } else {
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        const int col = col_of(st);
        if (col >= g.ncols) continue;
        if (MODE == kModeFc2) {
          if (m < valid) static_cast<float*>(g.out)[r * g.ncols + col] = tot[st][i] + bias[st];
        } else {
          const float h = m < valid ? plain_act(tot[st][i] * rs + bias[st], g.act) : 0.f;
          if (m < valid || !g.linear) static_cast<uint16_t*>(g.out)[r * g.ncols + col] = f32_to_bf16(h);
        }
      }
    }
  }
}

// Dynamic LDS: the group's scales (32 rows), then the partial sums of NW - 1 K ranges.
inline size_t gemm_gemv_lds(const GemmArgs& g, int scale_bytes, int nw) {
  const size_t scales = g.bs == 0 ? 0 : (32 * static_cast<size_t>(g.nb) * scale_bytes + 15) / 16 * 16;
  return scales + static_cast<size_t>(nw - 1) * 2 * 4 * 64 * 4;
}

template <int BITS, typename ST, int MODE, int NW, int PD>
static hipError_t launch_gemv(const GemmArgs& g, int64_t max_tiles, hipStream_t s) {
  constexpr int CW = MODE == kModeSwiglu ? 16 : 32;
  dim3 grid((g.ncols + CW - 1) / CW, static_cast<unsigned>(max_tiles)), block(NW * 64);
  const size_t lds = gemm_gemv_lds(g, sizeof(ST), NW);
#define QMOE_GEMV(BSV) \
  launch_gemm_kernel(gemm_bf16_gemv_kernel<BITS, ST, MODE, BSV, NW, PD>, grid, block, lds, s, g)
  if constexpr (std::is_same<ST, uint8_t>::value) {  // MX FP4: blocks of 32 only
    QMOE_GEMV(32);
  } else {
  switch (g.bs) {
    case 0: QMOE_GEMV(0); break;
    case 16: QMOE_GEMV(16); break;
    case 32: QMOE_GEMV(32); break;
    case 64: QMOE_GEMV(64); break;
    case 128: QMOE_GEMV(128); break;
    case 256: QMOE_GEMV(256); break;
    default: QMOE_GEMV(512); break;
  }
  }
#undef QMOE_GEMV
  return hipGetLastError();
}

}  // namespace qmoe
