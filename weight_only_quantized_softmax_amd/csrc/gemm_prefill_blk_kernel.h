// Grouped dequant GEMM, bf16 activations, 128-row tiles, one scale per output row and
// K-block: the prefill shape with block-scaled weights, bound by the bf16 MFMA rate.
//
// ClikaRT "QMoEWoQ" page, class description: the expert weights stay quantized and each
// block is decoded inside the GEMM dot. graiphic "QMoE" page: stacks [E, N, K/pack],
// scales [E, N, K/block_size] (block_size attribute).
//
// Workgroup: one 128-row tile of one expert by 128 weight rows (fused gate/up: 64 gate +
// 64 up rows = 64 output columns; otherwise 128 output columns); four waves in a 2 x 2
// grid of 64 rows x 64 weight rows each.
//   - Activations reach LDS as in the per-row kernel: buffer loads that target LDS, 16
//     bytes per lane, a double-buffered stage whose 16-byte granules are XOR-swizzled by
//     row, one barrier per K step.
//   - Each wave reads its 4 weight-row slices with one 16-byte load per slice and K step,
//     a whole step ahead, and decodes them in registers (4-bit: 128 + q by OR-ing the
//     nibble into the exponent pattern of 128; 8-bit: exact q). For 4-bit blocks shorter
//     than 128 the four lanes of a row trade words (a 4 x 4 transpose across the 16-lane
//     rows) so that each MFMA k-slice of 32 lies inside one block.
//   - The scales a K step needs (128 weight rows x its blocks) are loaded one step ahead
//     into registers and written to a two-slot LDS ring before the step's barrier.
//   - The zero point and the +128 offset leave through MFMAs of the activations against
//     the constant -(c+z). When a scale group is one k-slice (4-bit blocks of 16 or 32)
//     that product is the addend of every slice's MFMA, and the group ends with one scale
//     FMA per element; longer groups keep a per-row-slice correction accumulator that
//     joins each slice's accumulator when the group ends.
#pragma once

#include <type_traits>

#include "common.h"
#include "gemm_common.h"
#include "launch.h"

namespace qmoe {

namespace {

constexpr int kBTM = 128;  // rows per tile
constexpr int kBNB = 4;    // 16-row weight slices per wave

}  // namespace

// PK: weights in the tiled layout (qmoe_pack_stack): a slice's step is one contiguous
// 1 KB tile, already in k-slice order (word j of lane (n, q): k = 32j + 8q .. +8 of row n)
// with nibbles in decode order, so neither the cross-lane transpose nor the activation
// reorder is needed, 8-bit blocks of 16 and 32 align with k-slices, and K need not be a
// whole number of steps.
template <int BITS, typename ST, int MODE, int BS, bool PK>
__global__ __launch_bounds__(256, 2) void gemm_bf16_prefill_blk_kernel(GemmArgs g) {
  constexpr bool kTwo = (MODE == kModeSwiglu);
  constexpr int NS = kTwo ? 2 : 1;
  constexpr int NBS = kBNB / NS;                  // slices per stream
  constexpr int SSK = BITS == 4 ? 128 : 64;       // K per step
  constexpr int MPS = SSK / 32;                   // MFMA k-slices per step
  constexpr int GPR = SSK / 8;                    // 16-byte granules per activation row
  constexpr int NDMA = kBTM * GPR / 64 / 4;       // LDS-destination loads per wave per step
  constexpr int BCOLS = 2 * NBS * 16;             // output columns per workgroup
  constexpr int STAGE = kBTM * SSK;               // bf16 elements per LDS stage
  // KORD: k-slice j = k [32 j, 32 j + 32) of the step (tiled layout, or 4-bit rows with
  // blocks shorter than a step, by a cross-lane transpose)
  constexpr bool KORD = PK || (BITS == 4 && BS < 128);
  constexpr bool XPOSE = KORD && BS < SSK;        // scale groups tracked k-slice by k-slice
  constexpr bool SINGLE = XPOSE && BS <= 32;      // a scale group is one k-slice (or half)
  constexpr int G = (XPOSE && BS == 16) ? 2 : 1;  // scale groups per k-slice
  constexpr int NBLK = BS < SSK ? SSK / BS : 1;   // scale blocks a step touches
  constexpr int SROWS = kBTM;                     // weight rows of the workgroup
  constexpr int SPT = (SROWS * NBLK + 255) / 256; // scales loaded per thread per step
  // operands of the next k-slice read ahead, where the registers allow it (groups of one
  // k-slice or one step)
  constexpr bool PF = SINGLE || BS == SSK;
  constexpr uint32_t kNegCorr = BITS == 4 ? 0xC308C308u : 0xC300C300u;  // -(c+z) bf16 pair
  static_assert(PK || BITS == 4 || BS >= 64, "8-bit rows-layout blocks shorter than 64 take the other kernel");
  // MX FP4 (E8M0 scale bytes): codes scaled as they are converted, products accumulated
  // straight into the totals
  constexpr bool MX = std::is_same<ST, uint8_t>::value;
  static_assert(!MX || (BITS == 4 && BS == 32 && PK), "MX FP4: 4-bit, blocks of 32, tiled layout");

  __shared__ __attribute__((aligned(16))) uint16_t xs0[STAGE];
  __shared__ __attribute__((aligned(16))) uint16_t xs1[STAGE];
  // activation load offsets (fixed over K): in registers where they fit, else in LDS, each
  // thread reading back only what it wrote
  constexpr bool XREG = SINGLE || BITS == 8;
  __shared__ uint32_t xoffs_lds[XREG ? 1 : NDMA][256];
  uint32_t xoffs_reg[NDMA];
  auto xoff = [&](int t) -> uint32_t& { return XREG ? xoffs_reg[t] : xoffs_lds[t][threadIdx.x]; };
  __shared__ ST sring[2][SROWS * NBLK];  // scales of this step and the next

  int tile, cblk;
  if (!xcd_item(gemm_tile_count(g), (g.ncols + BCOLS - 1) / BCOLS, tile, cblk)) return;
  const int2 tv = gemm_tile(g, tile);
  const int e = tv.x;
  const int valid = tv.y;
  const int64_t row0 = static_cast<int64_t>(tile) * kBTM;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
  const int n = lane % 16, kq = lane / 16;
  const int wm = wave & 1, wn = wave >> 1;
  const int col0 = cblk * BCOLS;
  const int K = g.K;
  const uint32_t row_bytes = static_cast<uint32_t>(K) * BITS / 8;
  // rows layout: the launcher checks that K is a whole number of steps
  const int nss = PK ? g.kt : K / SSK;
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
  // column of slice b, row n of wave column wnn (clamped into the stack where it is read)
  auto slice_col = [&](int wnn, int b, int nn) { return col0 + wnn * NBS * 16 + (b % NBS) * 16 + nn; };

  // ---- weights: one descriptor per slice. Rows layout: based at the slice's first stack
  // row (rows past the stack read zeros); lane (n, kq) reads the 16 bytes at 16 kq of the
  // step's row segment. Tiled layout: the slice's sequence of 1 KB tiles (a block past the
  // stream reads zeros), lane l reading bytes 16 l of the step's tile.
  rsrc_t wres[kBNB];
  const int lstep = (kTwo && g.fusion == 1) ? 2 : 1;
#pragma unroll
  for (int b = 0; b < kBNB; ++b) {
    const int st = b / NBS;
    const int nr = stream_rows(st);
    if (PK) {
      const int ns = (kTwo && g.fusion != 0) ? 2 : 1, si = (kTwo && g.fusion != 0) ? st : 0;
      const int rb = slice_col(wn, b, 0) / 16;
      const int64_t tile0 = ((static_cast<int64_t>(e) * ns + si) * g.nbk + rb) * g.kt;
      wres[b] = make_rsrc(stream_w(st) + tile0 * 1024,
                          rb < g.nbk ? static_cast<uint32_t>(g.kt) * 1024u : 0u);
    } else {
      const int r0 = local_row(st, slice_col(wn, b, 0));
      const int64_t left = static_cast<int64_t>(max(nr - r0, 0)) * row_bytes;
      wres[b] = make_rsrc(stream_w(st) + (static_cast<int64_t>(e) * nr + r0) * row_bytes,
                          static_cast<uint32_t>(left));
    }
  }
  const uint32_t wlane = PK ? 16u * lane : static_cast<uint32_t>(lstep * n) * row_bytes + 16u * kq;
  auto wload = [&](int s, u32x4 (&w)[kBNB]) {
    const uint32_t so = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(s * SSK) * BITS / 8);
#pragma unroll
    for (int b = 0; b < kBNB; ++b)
      w[b] = PK ? buf_load16(wres[b], wlane + static_cast<uint32_t>(s) * 1024u)
                : buf_load16s(wres[b], wlane, so);
  };

  // ---- scales: entry i of a step is weight row i / NBLK of the workgroup, block
  // i % NBLK of the step; row R = wnn * 64 + b * 16 + nn. Each thread keeps a 32-bit
  // element offset and which stack it reads; the pointer is formed at each load. ----
  uint32_t soff[SPT];
  int sl[SPT];  // block of the entry inside the step
  bool sup[SPT], sok[SPT];
#pragma unroll
  for (int u = 0; u < SPT; ++u) {
    const int i = tid + 256 * u;
    sok[u] = i < SROWS * NBLK;
    const int ii = sok[u] ? i : 0;
    const int R = ii / NBLK, l = ii % NBLK;
    const int wnn = R / 64, b = (R % 64) / 16, nn = R % 16;
    const int st = b / NBS;
    const int c = min(slice_col(wnn, b, nn), g.ncols - 1);
    soff[u] = static_cast<uint32_t>((static_cast<int64_t>(e) * stream_rows(st) + local_row(st, c)) * nb);
    sl[u] = BS < SSK ? l : 0;
    sup[u] = st == 1 && kTwo && g.fusion == 0;
  }
  const ST* const s0 = static_cast<const ST*>(g.s);
  const ST* const s1 = static_cast<const ST*>(kTwo && g.fusion == 0 ? g.s3 : g.s);
  ST sreg[SPT];
  auto sload = [&](int s) {
    // first block of the step; blocks of a last, partial step that lie past K are clamped
    // to the row's last block (their activations are zero)
    const int blk = BS < SSK ? s * NBLK : (s * SSK) / BS;
#pragma unroll
    for (int u = 0; u < SPT; ++u) sreg[u] = (sup[u] ? s1 : s0)[soff[u] + min(blk + sl[u], nb - 1)];
  };
  auto sstore = [&](int slot) {
#pragma unroll
    for (int u = 0; u < SPT; ++u)
      if (sok[u]) sring[slot][tid + 256 * u] = sreg[u];
  };

  // ---- activations: row-major stages, XOR-swizzled granules ----
  auto key = [](int r) { return GPR == 16 ? (r & 15) : ((r >> 1) & 7); };
  const rsrc_t xres = make_rsrc(g.a, static_cast<uint32_t>(g.a_rows * K * 2));
  auto granule = [&](int t) {  // logical granule of load t of this lane
    const int p = (wave + 4 * t) * 64 + lane;
    return (p % GPR) ^ key(p / GPR);
  };
  // the same for every load t: 4t * 64 / GPR rows later is a multiple of the key's period
  const int gq = granule(0);
#pragma unroll
  for (int t = 0; t < NDMA; ++t) {
    const int p = (wave + 4 * t) * 64 + lane;
    const int r = p / GPR, q = granule(t);
    uint32_t off = kOutOfRange;  // padding rows land as zeros
    if (r < valid) {
      const int64_t src = (MODE == kModeFc2) ? row0 + r : gemm_src_row(g, row0 + r);
      off = static_cast<uint32_t>((src * K + 8 * q) * 2);
    }
    xoff(t) = off;
  }
  auto xload = [&](int s, uint16_t* stage) {
    const int k0 = __builtin_amdgcn_readfirstlane(s * SSK);
    if (PK && k0 + SSK > K) {
      // the last step of a K that is not a whole number of steps (tiled layout only):
      // granules past K land as zeros
#pragma unroll
      for (int t = 0; t < NDMA; ++t)
        buf_load16_lds(xres, stage + (wave + 4 * t) * 64 * 8,
                       k0 + 8 * gq < K ? xoff(t) : kOutOfRange, 2 * k0);
    } else {
#pragma unroll
      for (int t = 0; t < NDMA; ++t)
        buf_load16_lds(xres, stage + (wave + 4 * t) * 64 * 8, xoff(t), 2 * k0);
    }
    // the step-end wait counts the loads issued after these: none may move above
    __builtin_amdgcn_sched_barrier(0);
  };

  // operand reads: row r = wm*64 + mt*16 + n has key(r) = key(n). Granule of k-slice j:
  // q = 4 j + kq (transposed 4-bit), 4 kq + j (4-bit), 2 kq + j (8-bit); in every case j
  // sits in bits of q that the swizzle key leaves to an XOR, so the slot of k-slice j is
  // that of k-slice 0 with j XOR-ed in (bit 2-3 or bit 0).
  const int q0 = KORD ? kq : (BITS == 4 ? 4 : 2) * kq;
  const uint32_t abase = static_cast<uint32_t>(((wm * 64 + n) * GPR + (q0 ^ key(n))) * 16);
  auto aread = [&](const uint16_t* stage, int j, u32x4 (&xa)[4]) {
    const uint32_t aj = abase ^ static_cast<uint32_t>((KORD ? 64 : 16) * j);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
      xa[mt] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(stage) + aj +
                                               mt * 16 * GPR * 16);
  };

  const floatx4 zero4 = {0.f, 0.f, 0.f, 0.f};
  const bf16x8 zero8 = {};
  const bf16x8 negc = __builtin_bit_cast(bf16x8, u32x4{kNegCorr, kNegCorr, kNegCorr, kNegCorr});
  const int lgrp2 = kq >> 1;
  floatx4 tot[4][kBNB];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int b = 0; b < kBNB; ++b) tot[mt][b] = zero4;
  // longer scale groups: running products and the per-row-slice correction
  floatx4 acc[SINGLE ? 1 : 4][SINGLE ? 1 : kBNB];
  floatx4 cor[SINGLE ? 1 : 4];
  if (!SINGLE) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      cor[mt] = zero4;
#pragma unroll
      for (int b = 0; b < kBNB; ++b) acc[mt][b] = zero4;
    }
  }

  // The running totals are pure arithmetic, so the compiler may sink their updates past
  // later MFMAs (and hold every product until then); an empty volatile statement that
  // reads and writes a total fixes the update in program order.
  auto pin = [](floatx4& v) { asm volatile("" : "+v"(v)); };
  auto decode = [&](const u32x4& wv, int j) -> bf16x8 {
    if constexpr (BITS == 4) {
      return decode4(wv[j]);
    } else {
      const u32x2 w2 = {wv[2 * j], wv[2 * j + 1]};
      return decode8(w2);
    }
  };
  auto compute = [&](const uint16_t* stage, const u32x4 (&wl)[kBNB], int s, int slot) {
    u32x4 w[kBNB];
#pragma unroll
    for (int b = 0; b < kBNB; ++b) {
      w[b] = wl[b];
      if (KORD && !PK) transpose_rows4(w[b]);
    }
    const ST* sc = sring[slot];
    u32x4 xa[4], xn[4];
    aread(stage, 0, xa);
#pragma unroll
    for (int j = 0; j < MPS; ++j) {
      if (PF && j + 1 < MPS) aread(stage, j + 1, xn);  // next k-slice's operands, in flight
      if (!PF && j > 0) aread(stage, j, xa);
      if (BITS == 4 && !PK) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) xa[mt] = order_for_nibbles(xa[mt]);
      }
      const int kj = s * SSK + 32 * j;
      if constexpr (MX) {
        // k-slice j is block j of the step
        bf16x8 bm[kBNB];
#pragma unroll
        for (int b = 0; b < kBNB; ++b)
          bm[b] = decode_mx(w[b][j], scale_value<ST>(sc[(wn * 64 + b * 16 + n) * NBLK + j]));
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          const bf16x8 xb = __builtin_bit_cast(bf16x8, xa[mt]);
#pragma unroll
          for (int b = 0; b < kBNB; ++b)
            tot[mt][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xb, bm[b], tot[mt][b], 0, 0, 0);
        }
      } else if constexpr (SINGLE) {
#pragma unroll
        for (int gg = 0; gg < G; ++gg) {
          const bool mine = (G == 1) || (lgrp2 == gg);
          // local block of this group inside the step
          const int bl = (32 * j) / BS + gg;
          float sv[kBNB];
#pragma unroll
          for (int b = 0; b < kBNB; ++b)
            sv[b] = scale_value<ST>(sc[(wn * 64 + b * 16 + n) * NBLK + bl]);
          // software-pipelined by one product: the scaling FMAs of a product follow the
          // next product's MFMA, so they never wait on the MFMA just issued
          floatx4 aprev = zero4;
          int pprev = -1;
          auto scale_into = [&](int pidx, const floatx4& a) {
            const int pm = pidx / kBNB, pb = pidx % kBNB;
#pragma unroll
            for (int i = 0; i < 4; ++i) tot[pm][pb][i] += sv[pb] * a[i];
            pin(tot[pm][pb]);
          };
#pragma unroll
          for (int mt = 0; mt < 4; ++mt) {
            const bf16x8 xb = __builtin_bit_cast(bf16x8, xa[mt]);
            const floatx4 c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xb, mine ? negc : zero8, zero4, 0, 0, 0);
#pragma unroll
            for (int b = 0; b < kBNB; ++b) {
              const bf16x8 bw = decode(w[b], j);
              const floatx4 a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xb, mine ? bw : zero8, c, 0, 0, 0);
              if (pprev >= 0) scale_into(pprev, aprev);
              aprev = a;
              pprev = mt * kBNB + b;
            }
          }
          scale_into(pprev, aprev);
        }
      } else {
        // a group opens where a block starts and closes where the next one starts or K
        // ends (the last block may be short)
        const bool first = XPOSE ? (kj & (BS - 1)) == 0 : (j == 0 && (kj & (BS - 1)) == 0);
        // (tiled layout: k-slices past K, in the last step, end no group)
        const bool last = XPOSE ? (kj < K && (((kj + 32) & (BS - 1)) == 0 || kj + 32 >= K))
                                : (j == MPS - 1 && (((kj + 32) & (BS - 1)) == 0 || s == nss - 1));
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          const bf16x8 xb = __builtin_bit_cast(bf16x8, xa[mt]);
          cor[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xb, negc, first ? zero4 : cor[mt], 0, 0, 0);
#pragma unroll
          for (int b = 0; b < kBNB; ++b)
            acc[mt][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xb, decode(w[b], j),
                                                                 first ? zero4 : acc[mt][b], 0, 0, 0);
        }
        if (last) {
          const int bl = XPOSE ? (32 * j) / BS : 0;
#pragma unroll
          for (int b = 0; b < kBNB; ++b) {
            const float sv = scale_value<ST>(sc[(wn * 64 + b * 16 + n) * NBLK + bl]);
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
              for (int i = 0; i < 4; ++i) tot[mt][b][i] += sv * (acc[mt][b][i] + cor[mt][i]);
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) pin(tot[mt][b]);
          }
        }
      }
      if (PF && j + 1 < MPS) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) xa[mt] = xn[mt];
      }
      // one k-slice at a time: operands and decodes hoisted from later slices would spill
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- pipeline: step s reads stage s % 2, weight buffer s % 2, scale slot s % 2 ----
  static_assert(NDMA < 64, "vmcnt holds 6 bits");
  // issue order per step: activations, scales, weights; waiting down to the weight loads
  // leaves the step's activations in LDS and its scales in registers
  constexpr int kWaitX = (kBNB & 15) | ((kBNB >> 4) << 14) | (7 << 4) | (15 << 8);
  u32x4 wa[kBNB], wb[kBNB];
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
  float bias[kBNB];
#pragma unroll
  for (int b = 0; b < kBNB; ++b) {
    const int st = b / NBS;
    const int c = min(slice_col(wn, b, n), g.ncols - 1);
    const uint16_t* bp = static_cast<const uint16_t*>(stream_b(st));
    bias[b] = bp ? bf16_to_f32(bp[static_cast<int64_t>(e) * stream_rows(st) + local_row(st, c)]) : 0.f;
  }
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = wm * 64 + mt * 16 + 4 * kq + i;
      const int64_t r = row0 + m;
      // fc1 with the routing weight on the input: the row's weight scales its sums
      const float rs = (MODE != kModeFc2 && m < valid) ? gemm_row_scale(g, r) : 1.f;
#pragma unroll
      for (int cb = 0; cb < NBS; ++cb) {
        const int col = slice_col(wn, cb, n);
        if (col >= g.ncols) continue;
        float z[NS];
#pragma unroll
        for (int st = 0; st < NS; ++st) {
          const int b = st * NBS + cb;
          z[st] = tot[mt][b][i] * rs + bias[b];
        }
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

template <int BITS, typename ST, int MODE, int BS, bool PK>
static hipError_t launch_blk_bs(const GemmArgs& g, int64_t max_tiles, hipStream_t s) {
  const int bcols = 2 * (kBNB / (MODE == kModeSwiglu ? 2 : 1)) * 16;
  dim3 grid(xcd_grid((g.ncols + bcols - 1) / bcols, max_tiles)), block(256);
  launch_gemm_kernel(gemm_bf16_prefill_blk_kernel<BITS, ST, MODE, BS, PK>, grid, block, 0, s, g);
  return hipGetLastError();
}

template <int BITS, typename ST, int MODE, bool PK>
static hipError_t launch_blk_mode(const GemmArgs& g, int64_t max_tiles, hipStream_t s) {
  if constexpr (std::is_same<ST, uint8_t>::value) {  // MX FP4: blocks of 32 only
    return launch_blk_bs<BITS, ST, MODE, 32, PK>(g, max_tiles, s);
  } else {
  // 8-bit rows-layout blocks shorter than 64 are not served here (prefill_blk_supports)
  constexpr bool kShort = PK || BITS == 4;
  switch (g.bs) {
    case 16: if constexpr (kShort) return launch_blk_bs<BITS, ST, MODE, 16, PK>(g, max_tiles, s); break;
    case 32: if constexpr (kShort) return launch_blk_bs<BITS, ST, MODE, 32, PK>(g, max_tiles, s); break;
    case 64: return launch_blk_bs<BITS, ST, MODE, 64, PK>(g, max_tiles, s);
    case 128: return launch_blk_bs<BITS, ST, MODE, 128, PK>(g, max_tiles, s);
    case 256: return launch_blk_bs<BITS, ST, MODE, 256, PK>(g, max_tiles, s);
    default: return launch_blk_bs<BITS, ST, MODE, 512, PK>(g, max_tiles, s);
  }
  return hipErrorInvalidValue;
  }
}

template <int BITS, typename ST, bool PK>
static hipError_t launch_blk_t(const GemmArgs& g, int mode, int64_t max_tiles, hipStream_t s) {
  if (mode == kModeSwiglu) return launch_blk_mode<BITS, ST, kModeSwiglu, PK>(g, max_tiles, s);
  if (mode == kModePlainAct) return launch_blk_mode<BITS, ST, kModePlainAct, PK>(g, max_tiles, s);
  return launch_blk_mode<BITS, ST, kModeFc2, PK>(g, max_tiles, s);
}

template <bool PK>
static hipError_t launch_blk_layout(const GemmArgs& g, int mode, int bits, bool scale_bf16,
                                    int64_t max_tiles, hipStream_t s) {
  if (max_tiles <= 0) return hipSuccess;
  if constexpr (PK) {
    if (g.mx) return launch_blk_t<4, uint8_t, PK>(g, mode, max_tiles, s);
  }
  if (bits == 4)
    return scale_bf16 ? launch_blk_t<4, uint16_t, PK>(g, mode, max_tiles, s)
                      : launch_blk_t<4, float, PK>(g, mode, max_tiles, s);
  return scale_bf16 ? launch_blk_t<8, uint16_t, PK>(g, mode, max_tiles, s)
                    : launch_blk_t<8, float, PK>(g, mode, max_tiles, s);
}

}  // namespace qmoe
