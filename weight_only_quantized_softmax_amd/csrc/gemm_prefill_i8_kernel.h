// The int8 activation tier's dot product on the int8 matrix cores: 128-row tiles, tiled
// weight layout, 4- or 8-bit weight codes, block scales of 64 and 128.
//
// ClikaRT "QMoEWoQ" page, class description: on the int8 block tier the activation is
// quantised to int8 per block ahead of the dot product. graiphic "QMoE" page: stacks
// [E, N, K/pack], scales [E, N, K/block_size].
//
// The activations arrive as int8 codes with one power-of-two factor 2^e per row and block
// (launch_quantize_codes). The weights' codes become signed int8 (q - z) in registers: a
// byte XOR 0x80 for 8-bit codes; for 4-bit codes the nibbles go to bytes and
// (n + 0x78) ^ 0x80 turns each byte n into n - 8. v_mfma_i32_16x16x64_i8 then sums 64
// products of one row and one weight row exactly in int32, and at the end of each block
// the sum joins the fp32 total as total += float(sum) * 2^e(row, block) * s(weight row,
// block). The block sums cost three VALU per output element per block, against one FMA
// for the bf16 kernels' per-block sums, while the int8 instruction moves twice the bf16
// rate: blocks of 64 and 128 come out ahead (c5 at 4096 tokens, whole forward: 13-22%
// faster), blocks of 32 did not (16% slower), so they keep the bf16 kernels.
//
// The k a lane feeds the instruction follow the tiled weight layout: lane (n, q) holds k =
// 32j + 8q + i of its 16-row slice in word j of its 16 bytes, so for 64-k slice J it takes
// words 2J and 2J+1. The activation codes are stored with the chunks of 8 of every 64-group
// reordered (0, 4, 1, 5, 2, 6, 3, 7) so that one 16-byte granule is exactly those k.
//
// Workgroup: one 128-row tile of one expert by 128 weight rows, four waves side by side,
// each 128 rows x 2 weight-row slices of 16 (as the scaled-weight bf16 kernel). Activation
// codes reach LDS with loads that target it (double buffered, XOR-swizzled granules); the
// row factors and the weight scales of a step are loaded one step ahead into registers and
// written to a two-slot LDS ring before the step's barrier.
#pragma once

#include <type_traits>

#include "common.h"
#include "gemm_common.h"
#include "launch.h"

namespace qmoe {

namespace i8 {

constexpr int kTM = 128;   // rows per tile
constexpr int kNB = 2;     // 16-row weight slices per wave
constexpr int kMT = 8;     // 16-row MFMA tiles per wave

typedef int int4v __attribute__((ext_vector_type(4)));

// Eight 4-bit codes of one word in the tiled layout's decode order (element i in nibble
// (0, 4, 1, 5, 2, 6, 3, 7)[i]) as eight signed bytes n - 8 in k order (two words).
__device__ __forceinline__ void nibbles_to_i8(uint32_t w, uint32_t& lo8, uint32_t& hi8) {
  // low nibbles of the bytes: elements 0, 4, 1, 5; high nibbles: 2, 6, 3, 7
  const uint32_t a = ((w & 0x0F0F0F0Fu) + 0x78787878u) ^ 0x80808080u;
  const uint32_t b = (((w >> 4) & 0x0F0F0F0Fu) + 0x78787878u) ^ 0x80808080u;
  lo8 = __builtin_amdgcn_perm(b, a, 0x06040200u);  // elements 0, 1, 2, 3
  hi8 = __builtin_amdgcn_perm(b, a, 0x07050301u);  // elements 4, 5, 6, 7
}

}  // namespace i8

template <int BITS, typename ST, int MODE, int BS>
__global__ __launch_bounds__(256, 2) void gemm_i8_prefill_kernel(GemmArgs g) {
  using namespace i8;
  constexpr bool kTwo = (MODE == kModeSwiglu);
  constexpr int NS = kTwo ? 2 : 1;
  constexpr int NBS = kNB / NS;                   // slices per stream
  constexpr int SSK = BITS == 4 ? 128 : 64;       // K per step (one 1 KB tile per slice)
  constexpr int NJ = SSK / 64;                    // 64-k instructions per step
  constexpr int GPR = SSK / 16;                   // 16-byte code granules per row and step
  constexpr int NDMA = kTM * GPR / 64 / 4;        // LDS-destination loads per wave per step
  constexpr int BCOLS = 4 * NBS * 16;             // output columns per workgroup
  constexpr int STAGE = kTM * SSK;                // bytes per LDS stage
  constexpr int NBLK = BS < SSK ? SSK / BS : 1;   // blocks a step touches
  constexpr int SROWS = 4 * kNB * 16;             // weight rows of the workgroup (128)
  constexpr int SPT = (SROWS * NBLK + 255) / 256; // weight scales loaded per thread per step
  constexpr int FPT = (kTM * NBLK + 255) / 256;   // row factors loaded per thread per step
  static_assert(BS == 64 || BS == 128, "blocks of 64 and 128");

  __shared__ __attribute__((aligned(16))) int8_t xs0[STAGE];
  __shared__ __attribute__((aligned(16))) int8_t xs1[STAGE];
  __shared__ ST sring[2][SROWS * NBLK];                               // weight scales
  __shared__ __attribute__((aligned(16))) float fring[2][NBLK][kTM];  // row factors 2^e

  int tile, cblk;
  if (!xcd_item(gemm_tile_count(g), (g.ncols + BCOLS - 1) / BCOLS, tile, cblk)) return;
  const int2 tv = gemm_tile(g, tile);
  const int e = tv.x;
  const int valid = tv.y;
  const int64_t row0 = static_cast<int64_t>(tile) * kTM;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
  const int n = lane % 16, kq = lane / 16;
  const int wn = wave;
  const int col0 = cblk * BCOLS;
  const int K = g.K;
  const int nss = g.kt;
  const int nb = g.nb;

  auto local_row = [&](int st, int c) -> int {
    if (!kTwo) return c;
    if (g.fusion == 1) return 2 * c + st;
    if (g.fusion == 2) return st * g.inter + c;
    return c;
  };
  auto stream_rows = [&](int st) { return (kTwo && g.fusion == 0) ? g.inter : g.N; };
  auto stream_w = [&](int st) { return (st == 1 && kTwo && g.fusion == 0) ? g.w3 : g.w; };
  auto stream_b = [&](int st) { return (st == 1 && kTwo && g.fusion == 0) ? g.b3 : g.b; };
  auto slice_col = [&](int wnn, int b, int nn) { return col0 + wnn * NBS * 16 + (b % NBS) * 16 + nn; };

  // ---- weights: slice b's sequence of 1 KB tiles; lane l reads bytes 16 l of a step's tile
  rsrc_t wres[kNB];
#pragma unroll
  for (int b = 0; b < kNB; ++b) {
    const int st = b / NBS;
    const int ns = (kTwo && g.fusion != 0) ? 2 : 1, si = (kTwo && g.fusion != 0) ? st : 0;
    const int rb = slice_col(wn, b, 0) / 16;
    const int64_t tile0 = ((static_cast<int64_t>(e) * ns + si) * g.nbk + rb) * g.kt;
    wres[b] = make_rsrc(stream_w(st) + tile0 * 1024,
                        rb < g.nbk ? static_cast<uint32_t>(g.kt) * 1024u : 0u);
  }
  const uint32_t wlane = 16u * lane;
  auto wload = [&](int s, u32x4 (&w)[kNB]) {
#pragma unroll
    for (int b = 0; b < kNB; ++b) w[b] = buf_load16(wres[b], wlane + static_cast<uint32_t>(s) * 1024u);
  };

  // ---- weight scales: entry i of a step is weight row i / NBLK (R = wnn*32 + b*16 + nn),
  // block i % NBLK of the step
  uint32_t soff[SPT];
  int sl[SPT];
  bool sup[SPT], sok[SPT];
#pragma unroll
  for (int u = 0; u < SPT; ++u) {
    const int i = tid + 256 * u;
    sok[u] = i < SROWS * NBLK;
    const int ii = sok[u] ? i : 0;
    const int R = ii / NBLK, l = ii % NBLK;
    const int wnn = R / 32, b = (R % 32) / 16, nn = R % 16;
    const int st = b / NBS;
    const int c = min(slice_col(wnn, b, nn), g.ncols - 1);
    soff[u] = static_cast<uint32_t>((static_cast<int64_t>(e) * stream_rows(st) + local_row(st, c)) * nb);
    sl[u] = l;
    sup[u] = st == 1 && kTwo && g.fusion == 0;
  }
  const ST* const s0 = static_cast<const ST*>(g.s);
  const ST* const s1 = static_cast<const ST*>(kTwo && g.fusion == 0 ? g.s3 : g.s);

  // ---- row factors: entry i of a step is tile row i % 128, block i / 128 of the step;
  // padding rows take 0 (their codes are 0 too)
  int64_t frow[FPT];
  int fl[FPT];
  bool fok[FPT];
#pragma unroll
  for (int u = 0; u < FPT; ++u) {
    const int i = tid + 256 * u;
    fok[u] = i < kTM * NBLK;
    const int ii = fok[u] ? i : 0;
    const int r = ii % kTM;
    fl[u] = ii / kTM;
    frow[u] = -1;
    if (fok[u] && r < valid)
      frow[u] = (MODE == kModeFc2) ? row0 + r : gemm_src_row(g, row0 + r);
  }

  ST sreg[SPT];
  float freg[FPT];
  auto sload = [&](int s) {
    const int blk = BS < SSK ? s * NBLK : (s * SSK) / BS;
#pragma unroll
    for (int u = 0; u < SPT; ++u) sreg[u] = (sup[u] ? s1 : s0)[soff[u] + min(blk + sl[u], nb - 1)];
#pragma unroll
    for (int u = 0; u < FPT; ++u)
      freg[u] = frow[u] >= 0 ? g.afac[frow[u] * nb + min(blk + fl[u], nb - 1)] : 0.f;
  };
  auto sstore = [&](int slot) {
#pragma unroll
    for (int u = 0; u < SPT; ++u)
      if (sok[u]) sring[slot][tid + 256 * u] = sreg[u];
#pragma unroll
    for (int u = 0; u < FPT; ++u)
      if (fok[u]) fring[slot][fl[u]][(tid + 256 * u) % kTM] = freg[u];
  };

  // ---- activation codes: row-major stages of 128 rows x SSK bytes, granule q of row r at
  // slot q ^ key(r) (16 consecutive rows, one granule each, fall in distinct banks) ----
  auto key = [](int r) { return GPR == 8 ? ((r >> 1) & 7) : ((r >> 2) & 3); };
  const rsrc_t xres = make_rsrc(g.a, static_cast<uint32_t>(g.a_rows * K));
  uint32_t xoffs[NDMA];
#pragma unroll
  for (int t = 0; t < NDMA; ++t) {
    const int p = (wave + 4 * t) * 64 + lane;
    const int r = p / GPR, q = (p % GPR) ^ key(r);
    uint32_t off = kOutOfRange;  // padding rows land as zeros
    if (r < valid) {
      const int64_t src = (MODE == kModeFc2) ? row0 + r : gemm_src_row(g, row0 + r);
      off = static_cast<uint32_t>(src * K + 16 * q);
    }
    xoffs[t] = off;
  }
  auto xload = [&](int s, int8_t* stage) {
    const int k0 = __builtin_amdgcn_readfirstlane(s * SSK);
    // granules past K (the second half of a last 128-k step when K is an odd multiple of
    // 64) land as zeros
#pragma unroll
    for (int t = 0; t < NDMA; ++t) {
      const int p = (wave + 4 * t) * 64 + lane;
      const int q = (p % GPR) ^ key(p / GPR);
      buf_load16_lds(xres, stage + (wave + 4 * t) * 64 * 16, k0 + 16 * q < K ? xoffs[t] : kOutOfRange,
                     k0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  // A operand of 64-k slice J for row n of MFMA tile mt: granule 4J + kq
  uint32_t abase[NJ];
#pragma unroll
  for (int J = 0; J < NJ; ++J) abase[J] = static_cast<uint32_t>((n * GPR + ((4 * J + kq) ^ key(n))) * 16);

  const floatx4 zero4 = {0.f, 0.f, 0.f, 0.f};
  const int4v izero = {0, 0, 0, 0};
  floatx4 tot[kMT][kNB];
  int4v acc[kMT][kNB];
#pragma unroll
  for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
    for (int b = 0; b < kNB; ++b) {
      tot[mt][b] = zero4;
      acc[mt][b] = izero;
    }

  // joins the int32 sums of block bl (of the step, ring slot) into the totals
  auto scale_into = [&](int slot, int bl) {
    float d[kNB];
#pragma unroll
    for (int b = 0; b < kNB; ++b) d[b] = scale_value<ST>(sring[slot][(wn * 32 + b * 16 + n) * NBLK + bl]);
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt) {
      const floatx4 c = *reinterpret_cast<const floatx4*>(&fring[slot][bl][mt * 16 + 4 * kq]);
#pragma unroll
      for (int b = 0; b < kNB; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          tot[mt][b][i] = fmaf(static_cast<float>(acc[mt][b][i]) * c[i], d[b], tot[mt][b][i]);
    }
  };

  auto compute = [&](const int8_t* stage, const u32x4 (&w)[kNB], int s, int slot) {
#pragma unroll
    for (int J = 0; J < NJ; ++J) {
      const int kj = s * SSK + 64 * J;  // first k of this instruction
      if (kj >= K) break;  // past K (uniform): no block may open or close here
      // the weight operands: 16 signed bytes per slice (k order of the lane's granule)
      int4v bw[kNB];
#pragma unroll
      for (int b = 0; b < kNB; ++b) {
        if constexpr (BITS == 4) {
          uint32_t x0, x1, x2, x3;
          nibbles_to_i8(w[b][2 * J], x0, x1);
          nibbles_to_i8(w[b][2 * J + 1], x2, x3);
          bw[b] = int4v{static_cast<int>(x0), static_cast<int>(x1), static_cast<int>(x2),
                        static_cast<int>(x3)};
        } else {
          const u32x4 v = w[b] ^ u32x4{0x80808080u, 0x80808080u, 0x80808080u, 0x80808080u};
          bw[b] = __builtin_bit_cast(int4v, v);
        }
      }
      int4v xa[kMT];
#pragma unroll
      for (int mt = 0; mt < kMT; ++mt)
        xa[mt] = *reinterpret_cast<const int4v*>(stage + abase[J] + mt * 16 * GPR * 16);
      // a block opens where one starts and closes where the next starts or K ends (the last
      // block may be short)
      const bool first = (kj % BS) == 0;
      const bool last = ((kj + 64) % BS) == 0 || kj + 64 >= K;
#pragma unroll
      for (int b = 0; b < kNB; ++b)
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt)
          acc[mt][b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(xa[mt], bw[b], first ? izero : acc[mt][b],
                                                             0, 0, 0);
      if (last) scale_into(slot, BS < SSK ? (64 * J) / BS : 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- pipeline: step s reads stage s % 2, weight buffer s % 2, ring slot s % 2 ----
  static_assert(NDMA < 64, "vmcnt holds 6 bits");
  constexpr int kWaitX = (kNB & 15) | ((kNB >> 4) << 14) | (7 << 4) | (15 << 8);
  u32x4 wa[kNB], wb[kNB];
  xload(0, xs0);
  sload(0);
  wload(0, wa);
  __builtin_amdgcn_s_waitcnt(0);
  sstore(0);
  __syncthreads();
  const int npair = nss / 2;
  for (int pi = 0; pi < npair; ++pi) {
    const int s = 2 * pi;
    xload(s + 1, xs1);
    sload(s + 1);
    wload(s + 1, wb);
    compute(xs0, wa, s, 0);
    __builtin_amdgcn_s_waitcnt(kWaitX);
    sstore(1);
    __syncthreads();
    if (s + 2 < nss) {
      xload(s + 2, xs0);
      sload(s + 2);
      wload(s + 2, wa);
    }
    compute(xs1, wb, s + 1, 1);
    if (s + 2 < nss) {
      __builtin_amdgcn_s_waitcnt(kWaitX);
      sstore(0);
    }
    __syncthreads();
  }
  if (nss & 1) compute(xs0, wa, nss - 1, 0);

  // ---- epilogue: bias, activation ----
  float bias[kNB];
#pragma unroll
  for (int b = 0; b < kNB; ++b) {
    const int st = b / NBS;
    const int c = min(slice_col(wn, b, n), g.ncols - 1);
    const uint16_t* bp = static_cast<const uint16_t*>(stream_b(st));
    bias[b] = bp ? bf16_to_f32(bp[static_cast<int64_t>(e) * stream_rows(st) + local_row(st, c)]) : 0.f;
  }
#pragma unroll
  for (int mt = 0; mt < kMT; ++mt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = mt * 16 + 4 * kq + i;
      const int64_t r = row0 + m;
#pragma unroll
      for (int cb = 0; cb < NBS; ++cb) {
        const int col = slice_col(wn, cb, n);
        if (col >= g.ncols) continue;
        float z[NS];
#pragma unroll
        for (int st = 0; st < NS; ++st) z[st] = tot[mt][st * NBS + cb][i] + bias[st * NBS + cb];
        if (MODE == kModeFc2) {
          if (m < valid) static_cast<float*>(g.out)[r * g.ncols + col] = z[0];
        } else {
          float hv = 0.f;
          if (m < valid)
            hv = (MODE == kModeSwiglu) ? swiglu(z[0], z[NS - 1], g.alpha, g.beta, g.limit)
                                       : plain_act(z[0], g.act);
          if (m < valid || !g.linear) static_cast<uint16_t*>(g.out)[r * g.ncols + col] = f32_to_bf16(hv);
        }
      }
    }
  }
}

template <int BITS, typename ST, int MODE, int BS>
static hipError_t launch_i8_bs(const GemmArgs& g, int64_t max_tiles, hipStream_t s) {
  constexpr int bcols = 4 * (i8::kNB / (MODE == kModeSwiglu ? 2 : 1)) * 16;
  dim3 grid(xcd_grid((g.ncols + bcols - 1) / bcols, max_tiles)), block(256);
  launch_gemm_kernel(gemm_i8_prefill_kernel<BITS, ST, MODE, BS>, grid, block, 0, s, g);
  return hipGetLastError();
}

template <int BITS, typename ST, int MODE>
static hipError_t launch_i8_mode(const GemmArgs& g, int64_t max_tiles, hipStream_t s) {
  if (g.bs == 64) return launch_i8_bs<BITS, ST, MODE, 64>(g, max_tiles, s);
  return launch_i8_bs<BITS, ST, MODE, 128>(g, max_tiles, s);
}

template <int BITS, typename ST>
static hipError_t launch_i8_t(const GemmArgs& g, int mode, int64_t max_tiles, hipStream_t s) {
  if (mode == kModeSwiglu) return launch_i8_mode<BITS, ST, kModeSwiglu>(g, max_tiles, s);
  if (mode == kModePlainAct) return launch_i8_mode<BITS, ST, kModePlainAct>(g, max_tiles, s);
  return launch_i8_mode<BITS, ST, kModeFc2>(g, max_tiles, s);
}

}  // namespace qmoe
