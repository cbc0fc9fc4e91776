// Grouped dequant GEMM kernel for bf16 activations on gfx950 MFMA (16x16x32 bf16, fp32 accumulate),
// 16-row tiles: the decode and mid-size shapes, bound by streaming the quantized weights.
//
// ClikaRT "QMoEWoQ" page, class description: the expert weights stay quantized and each
// block is decoded inside the GEMM dot, never as a dense copy. graiphic "QMoE" page:
// stack shapes [E, N, K/pack], scales per row or per K-block, activation attributes.
//
// Work unit of one wave: one 16-row tile of one expert x two 16-row weight slices (gate
// and up of 16 output columns for fc1 with SwiGLU, otherwise two neighbouring groups of 16
// output columns) over a range of K. A workgroup holds four
// such waves; with split-K they share columns and divide K, and add their partial sums in
// LDS at the end. Each lane owns one output column n and one quarter kq of every 32-wide
// K step, and decodes its 8 weights of the step in registers:
//   4-bit: each nibble q becomes the bfloat16 128+q by OR-ing it into the exponent
//          pattern of 128 (exact), two nibbles per 32-bit register;
//   8-bit: each byte becomes the exact bfloat16 q.
// The MFMA therefore computes sum x*(c+q) with c = 128 (4-bit) or 0 (8-bit). The zero
// point z and the offset c leave through a second MFMA of the same activations against
// the constant -(c+z) (exact in bfloat16) into the same accumulator; a scale group's
// accumulator starts from zero and is multiplied by its block's scale once, when the
// group ends. Per-row scales multiply the finished sum.
#pragma once

#include <type_traits>

#include "common.h"
#include "gemm_common.h"
#include "gemm_gemv_kernel.h"
#include "launch.h"

namespace qmoe {

// Layout of one lane's 16-byte weight load and of the MFMA steps built from it.
//   4-bit: a load holds 32 consecutive k of the lane's row; a "super-step" of 128 k is the
//          four loads of lanes kq = 0..3 and feeds four MFMAs. Without the transpose, MFMA j
//          takes word j of every lane (k slots spread over the 128); with it (scale blocks of
//          16..64), MFMA j takes the 32 consecutive k [32j, 32j+32) of the super-step.
//   8-bit: a load holds 16 consecutive k; a super-step is 64 k and feeds two MFMAs; MFMA j
//          takes bytes [8j, 8j+8) of every lane (k slots spread over the 64).
// G > 1 splits an MFMA whose k slots span G scale blocks into G MFMAs, each with the
// weights (and the correction constant) of the other blocks' lanes zeroed.
//
// Workgroup: four waves on one 16-row tile, as CPB column groups (one wave's columns)
// times SK K-splits (CPB * SK = 4). K advances in chunks of 256 k (two 4-bit or four 8-bit
// super-steps); the split-K waves of a column group take the chunk's super-steps in turn.
// Chunk ci's activations and weights are requested two chunks ahead: the activations go
// straight into LDS (loads that target LDS, 1 KB of row segments per load, a ring of three
// 8 KB stages whose 16-byte granules are XOR-swizzled by row so that the 16 rows one MFMA
// operand reads fall in distinct banks), the weights into a three-slot register ring.
// One barrier per chunk. All scales of the workgroup's rows are copied into LDS once, at
// the start. The small stages leave room for three or four workgroups per CU, which the
// weight stream needs to keep enough loads in flight.
constexpr int kDecWaves = 4;  // waves per workgroup (eight for large tiled-layout grids)

// PK: the weights come in the tiled layout (qmoe_pack_stack): each lane's 16 bytes of a
// super-step are one contiguous 1 KB tile of its 16-row slice, already in MFMA order
// (word j of lane (n, q) holds k = 32j + 8q .. +8 of row n, nibbles in decode order).
template <int BITS, typename ST, int MODE, int BS, int SK, bool PK, int NW_, int MR, int PD>
__global__ __launch_bounds__(NW_ * 64) void gemm_bf16_tile_kernel(GemmArgs g) {
  constexpr int NW = NW_;
  // prefetch distance: chunk ci + PD is requested while chunk ci is computed, from a ring
  // of PD + 1 weight slots and LDS activation stages
  static_assert(PD >= 2 && PD <= 4, "prefetch distance 2 to 4");
  constexpr int TM = MR * kM;                   // rows of a tile: MR MFMA row blocks of 16
  constexpr bool PERROW = BS == 0;
  // MX FP4 (E8M0 scale bytes): each code is scaled as it is converted, so the MFMAs
  // accumulate the whole K with no correction term and no per-block scaling
  constexpr bool MX = std::is_same<ST, uint8_t>::value;
  static_assert(!MX || (BITS == 4 && BS == 32 && PK), "MX FP4: 4-bit, blocks of 32, tiled layout");
  constexpr int SSK0 = BITS == 4 ? 128 : 64;
  // KORD: MFMA j of a super-step takes the 32 consecutive k [32j, 32j + 32) (tiled layout,
  // or 4-bit rows with blocks shorter than a super-step, by a cross-lane transpose)
  constexpr bool KORD = PK || (BITS == 4 && BS > 0 && BS < 128);
  // scale groups no longer than a super-step, tracked MFMA by MFMA
  constexpr bool XPOSE = KORD && BS > 0 && BS < SSK0;
  constexpr int G = KORD ? (BS == 16 ? 2 : 1) : (BITS == 4 ? 1 : (BS == 16 ? 4 : (BS == 32 ? 2 : 1)));
  constexpr bool kTwo = (MODE == kModeSwiglu);
  constexpr int NS = 2;                         // weight streams (16-row slices) per lane
  constexpr int CW = kTwo ? 16 : 32;            // output columns per wave
  constexpr int KC = 256;                       // K per chunk (128 or 256 bytes of every row)
  constexpr int SSK = BITS == 4 ? 128 : 64;     // K per super-step
  constexpr int SPC = KC / SSK;                 // super-steps per chunk (2 or 4)
  static_assert(SK <= SPC, "a chunk holds at least one super-step per split");
  constexpr int SPW = SPC / SK;                 // super-steps per chunk of one wave
  constexpr int MPS = SSK / 32;                 // MFMAs per super-step
  constexpr int CPB = NW / SK;                  // column groups per workgroup
  constexpr int GPR = KC / 8;                   // 16-byte granules per chunk row (32)
  constexpr int RPL = 64 / GPR;                 // tile rows per activation load (2)
  constexpr int NDMA = TM / RPL / NW;           // activation loads per wave per chunk
  static_assert(NDMA >= 1, "every wave takes part in the activation loads");
  constexpr int STAGE = TM * KC;                // bf16 elements of one LDS stage
  constexpr int BSHIFT = BS == 16 ? 4 : BS == 32 ? 5 : BS == 64 ? 6 : BS == 128 ? 7 : BS == 256 ? 8 : 9;
  // -(c+z) as a bf16 pair: 136 = 128 + 8 (4-bit), 128 = 0 + 128 (8-bit), both exact
  constexpr uint32_t kNegCorr = BITS == 4 ? 0xC308C308u : 0xC300C300u;

  // the activation stages as separate arrays, so that the compiler can tell the stage
  // being read from the stages being filled
  __shared__ __attribute__((aligned(16))) uint16_t xs0[STAGE];
  __shared__ __attribute__((aligned(16))) uint16_t xs1[STAGE];
  __shared__ __attribute__((aligned(16))) uint16_t xs2[STAGE];
  __shared__ __attribute__((aligned(16))) uint16_t xs3[PD >= 3 ? STAGE : 8];
  __shared__ __attribute__((aligned(16))) uint16_t xs4[PD >= 4 ? STAGE : 8];
  auto stage = [&](int r) -> uint16_t* {
    return r == 0 ? xs0 : r == 1 ? xs1 : r == 2 ? xs2 : r == 3 ? xs3 : xs4;
  };
  extern __shared__ __attribute__((aligned(16))) unsigned char dyn[];  // scales

  // a grouping tile of g.M rows is covered by g.M / TM workgroup rows of TM rows each.
  // fc2 takes (workgroup row, column block) in the XCD-banded order (a 1-D grid), so that
  // the column blocks of a row run on one XCD and its L2 fetches the row's activations
  // once (2-3% on fc2 at 16- and 32-row tiles; fc1 ran about 1% slower with it and keeps
  // the 2-D grid: blockIdx.x the column block, blockIdx.y the workgroup row)
  const int nsub = g.M / TM;
  int wrow, cblk;
  if constexpr (MODE == kModeFc2) {
    if (!xcd_item(gemm_tile_count(g) * nsub, (g.ncols + CPB * CW - 1) / (CPB * CW), wrow, cblk))
      return;
  } else {
    wrow = blockIdx.y;
    cblk = blockIdx.x;
    if (wrow / nsub >= gemm_tile_count(g)) return;
  }
  const int tile = wrow / nsub, sub = wrow % nsub;
  const int2 tv = gemm_tile(g, tile);
  const int e = tv.x;
  const int valid = min(max(tv.y - sub * TM, 0), TM);
  if (MODE == kModeFc2 && valid == 0) return;  // no output rows (fc1 writes zero rows)
  const int64_t row0 = static_cast<int64_t>(tile) * g.M + sub * TM;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
  const int n = lane % 16, kq = lane / 16;
  const int ks = wave % SK, cgl = wave / SK;     // K split and column group of this wave
  const int col0 = cblk * CPB * CW;
  // output column of stream st of this lane (SwiGLU: both streams feed one column)
  auto col_of = [&](int st) { return col0 + cgl * CW + (kTwo ? 0 : 16 * st) + n; };
  const int K = g.K;
  const uint32_t row_bytes = static_cast<uint32_t>(K) * BITS / 8;
  const int nchunks = (K + KC - 1) / KC;

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

  rsrc_t wres[NS];
  uint32_t woff[NS];
  int lrow[NS];
#pragma unroll
  for (int st = 0; st < NS; ++st) {
    const int nr = stream_rows(st);
    lrow[st] = local_row(st, min(col_of(st), g.ncols - 1));  // clamped: stored only if valid
    if (PK) {
      // the slice's tile sequence: expert e, stream st, 16-row block of its first column;
      // a block past the stream reads zeros
      const int ns = (kTwo && g.fusion != 0) ? 2 : 1;
      const int si = (kTwo && g.fusion != 0) ? st : 0;
      const int rb = (col0 + cgl * CW + (kTwo ? 0 : 16 * st)) / 16;
      const int64_t tile0 = ((static_cast<int64_t>(e) * ns + si) * g.nbk + rb) * g.kt;
      wres[st] = make_rsrc(stream_w(st) + tile0 * 1024,
                           rb < g.nbk ? static_cast<uint32_t>(g.kt) * 1024u : 0u);
      woff[st] = 16u * lane;
    } else {
      wres[st] = make_rsrc(stream_w(st) + static_cast<int64_t>(e) * nr * row_bytes,
                           static_cast<uint32_t>(nr) * row_bytes);
      woff[st] = static_cast<uint32_t>(lrow[st]) * row_bytes + 16 * kq;
    }
  }
  // the weights of one wave for chunk ci: its SPW super-steps, in one burst (tiles past
  // K fall outside the tile range and read zeros)
  typedef u32x4 Slot[NS][SPW];
  auto wload = [&](int ci, Slot& w) {
#pragma unroll
    for (int v = 0; v < SPW; ++v)
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        const int ss = ci * SPC + v * SK + ks;  // super-step (tile) index along K
        const uint32_t off = PK ? static_cast<uint32_t>(ss) * 1024u
                                : static_cast<uint32_t>(ss * SSK) * BITS / 8;
        // tiled: whole 1 KB tiles, read once (nontemporal); rows layout: the other half of
        // each 128-byte line is read a chunk later and must stay cached
        w[st][v] = PK ? buf_load16_stream(wres[st], woff[st] + off) : buf_load16(wres[st], woff[st] + off);
      }
  };

  // ---- activations: load t of wave w fills stage slots [64 (w + 4t), 64 (w + 4t) + 64):
  // tile row r = (w + 4t) * RPL + lane / GPR, slot lane % GPR of the row holding logical
  // granule (slot ^ key(r)) of the row's chunk segment ----
  auto key = [](int r) { return r & 15; };
  const rsrc_t xres = make_rsrc(g.a, static_cast<uint32_t>(g.a_rows * K * 2));
  uint32_t xoff[NDMA];
  int xk[NDMA];  // first k of the lane's granule inside a chunk
#pragma unroll
  for (int t = 0; t < NDMA; ++t) {
    const int r = (wave + NW * t) * RPL + lane / GPR;
    const int q = (lane % GPR) ^ key(r);
    xk[t] = 8 * q;
    if (r < valid) {
      const int64_t src = (MODE == kModeFc2) ? row0 + r : gemm_src_row(g, row0 + r);
      xoff[t] = static_cast<uint32_t>((src * K + 8 * q) * 2);
    } else {
      xoff[t] = kOutOfRange;  // padding rows land as zeros
    }
  }
  auto xload = [&](int ci, uint16_t* stage) {
    const int k0 = __builtin_amdgcn_readfirstlane(ci * KC);
#pragma unroll
    for (int t = 0; t < NDMA; ++t) {
      // granules past K land as zeros too
      const uint32_t off = (k0 + xk[t] < K) ? xoff[t] : kOutOfRange;
      buf_load16_lds(xres, stage + (wave + NW * t) * 64 * 8, off, 2 * k0);
    }
  };

  // ---- prologue ----
  // The scale rows of the workgroup's columns are one contiguous range per stream (one
  // range in all for interleaved gate/up rows), 16-byte aligned because they start at a
  // multiple of 16 rows. They are copied into LDS first, 16 bytes per lane with loads that
  // target LDS.
  const int nb = PERROW ? 1 : g.nb;
  ST* scl = reinterpret_cast<ST*>(dyn);
  // one range for interleaved gate/up rows and for two column groups
  const bool one_range = !kTwo || g.fusion == 1;
  if (!PERROW) {
    const int rowb = nb * static_cast<int>(sizeof(ST));
    const int nrange = one_range ? 1 : NS;
    const int rows = (one_range ? 2 : 1) * CPB * 16;  // rows of one range
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
  __builtin_amdgcn_sched_barrier(0);
  Slot wr[PD + 1];
  xload(0, xs0);
  __builtin_amdgcn_sched_barrier(0);
  wload(0, wr[0]);
#pragma unroll
  for (int i = 1; i < PD; ++i) {
    if (i < nchunks) xload(i, stage(i));
    __builtin_amdgcn_sched_barrier(0);
    wload(min(i, nchunks - 1), wr[i]);
  }
  // the scales and chunk 0's activations were issued first and loads complete in order:
  // chunk 0 has landed once at most the later loads are pending (the weights of chunks
  // 0 .. PD-1 and the activations of chunks 1 .. PD-1 that exist)
  constexpr int kWgt = PD * NS * SPW;  // weight loads issued after an activation load
  static_assert(kWgt + (PD - 1) * NDMA < 64, "vmcnt holds 6 bits");
  wait_vm_sel<kWgt, NDMA, PD - 1>(min(PD - 1, nchunks - 1));
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  const ST* my_scl[NS];
#pragma unroll
  for (int st = 0; st < NS; ++st)
    my_scl[st] = scl + (!kTwo ? cgl * 32 + 16 * st + n
                        : one_range ? 2 * (cgl * 16 + n) + st : st * CPB * 16 + cgl * 16 + n) * nb;

  floatx4 acc[MR][NS][G];
  float tot[MR][NS][4];
  const floatx4 zero4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int mr = 0; mr < MR; ++mr)
#pragma unroll
    for (int gg = 0; gg < G; ++gg)
#pragma unroll
      for (int st = 0; st < NS; ++st) acc[mr][st][gg] = zero4;
#pragma unroll
  for (int mr = 0; mr < MR; ++mr)
#pragma unroll
    for (int st = 0; st < NS; ++st)
#pragma unroll
      for (int i = 0; i < 4; ++i) tot[mr][st][i] = 0.f;
  const bf16x8 zero = {};
  // the correction operand stays in its registers for the whole loop (opaque to the
  // compiler, which would otherwise rebuild it before every use)
  u32x4 negc_bits = {kNegCorr, kNegCorr, kNegCorr, kNegCorr};
  asm volatile("" : "+v"(negc_bits));
  const bf16x8 negc = __builtin_bit_cast(bf16x8, negc_bits);
  const int lgrp2 = kq >> 1;

  // Computes this wave's super-steps of chunk ci from weight slot w and LDS stage xs.
  auto compute = [&](Slot& w, const uint16_t* xs, int ci) {
    const int k0 = ci * KC;
#pragma unroll
    for (int v = 0; v < SPW; ++v) {
      const int u = v * SK + ks;    // super-step inside the chunk
      const int ksu = k0 + SSK * u; // its first k
      if (ksu >= K) break;
      u32x4 wv[NS];
#pragma unroll
      for (int st = 0; st < NS; ++st) wv[st] = w[st][v];
      if (KORD && !PK) {
#pragma unroll
        for (int st = 0; st < NS; ++st) transpose_rows4(wv[st]);
      }
#pragma unroll
      for (int j = 0; j < MPS; ++j) {
        const int kj = ksu + 32 * j;
        if (KORD && kj >= K) break;
        int q;  // logical granule of this lane's 8 activations for MFMA j, inside the chunk
        if (BITS == 4)
          q = KORD ? (16 * u + 4 * j + kq) : (16 * u + 4 * kq + j);
        else
          q = KORD ? (8 * u + 4 * j + kq) : (8 * u + 2 * kq + j);
        bf16x8 xa[MR];
#pragma unroll
        for (int mr = 0; mr < MR; ++mr) {
          u32x4 xr = *reinterpret_cast<const u32x4*>(xs + ((16 * mr + n) * GPR + (q ^ key(n))) * 8);
          if (BITS == 4 && !PK) xr = order_for_nibbles(xr);
          xa[mr] = __builtin_bit_cast(bf16x8, xr);
        }
        if constexpr (MX) {
          // this k-slice is one block: its scale byte, 32-k block (k0 >> 5) + 4u + j
          const int blk = (k0 >> 5) + u * (SSK >> 5) + j;
#pragma unroll
          for (int st = 0; st < NS; ++st) {
            const bf16x8 bm = decode_mx(wv[st][j], scale_value<ST>(my_scl[st][blk]));
#pragma unroll
            for (int mr = 0; mr < MR; ++mr)
              acc[mr][st][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[mr], bm, acc[mr][st][0], 0, 0, 0);
          }
          continue;
        }
        bf16x8 bw[NS];
#pragma unroll
        for (int st = 0; st < NS; ++st) {
          if (BITS == 4) {
            bw[st] = decode4(wv[st][j]);
          } else {
            u32x2 w2 = {wv[st][2 * j], wv[st][2 * j + 1]};
            bw[st] = decode8(w2);
          }
        }
        // where this MFMA's scale groups start and end
        int first = 0, last = 0, gl0 = 0;
        if (!PERROW) {
          if (XPOSE) {
            gl0 = kj >> BSHIFT;
            first = G > 1 || (kj & (BS - 1)) == 0;
            last = G > 1 || ((kj + 32) & (BS - 1)) == 0 || kj + 32 >= K;
          } else {
            // the super-step lies inside one block (rows layout: the MFMA's k slots spread
            // over it); a block longer than a super-step is summed and scaled one
            // super-step at a time. In k-slice order the k-slices past K are skipped, so
            // the group of a last, partial super-step ends at its last k-slice below K.
            gl0 = ksu >> BSHIFT;
            first = j == 0;
            last = j == MPS - 1 || (KORD && kj + 32 >= K);
          }
        }
#pragma unroll
        for (int gg = 0; gg < G; ++gg) {
          const bool mine = (G == 1) || (G == 2 ? (lgrp2 == gg) : (kq == gg));
          // each stream's accumulator takes the correction -(c+z) * sum x and the products;
          // a group starts from zero
#pragma unroll
          for (int mr = 0; mr < MR; ++mr) {
            if (first) {
              // a group's start: the correction depends on the activations alone, so one
              // MFMA serves every stream as the addend of its products
              const floatx4 cor =
                  __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[mr], mine ? negc : zero, zero4, 0, 0, 0);
#pragma unroll
              for (int st = 0; st < NS; ++st)
                acc[mr][st][gg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    xa[mr], mine ? bw[st] : zero, cor, 0, 0, 0);
            } else {
#pragma unroll
              for (int st = 0; st < NS; ++st) {
                acc[mr][st][gg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    xa[mr], mine ? negc : zero, acc[mr][st][gg], 0, 0, 0);
                acc[mr][st][gg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    xa[mr], mine ? bw[st] : zero, acc[mr][st][gg], 0, 0, 0);
              }
            }
          }
          if (last) {
            // the group's block: the two blocks of 16 inside one 4-bit MFMA are gl0 and
            // gl0 + 1, the blocks of an 8-bit super-step gl0 + gg; otherwise the MFMA or
            // super-step lies inside block gl0
            // (the k-slice lies below K, so a single-block group's index is below nb; in
            // k-slice order it is written as the chunk's first block plus a constant, so
            // the scale reads take immediate LDS offsets)
            int blk = XPOSE ? (k0 >> BSHIFT) + u * (SSK >> BSHIFT) + ((32 * j) >> BSHIFT) + gg
                            : gl0 + (G > 1 ? gg : 0);
            if (G > 1) blk = min(blk, nb - 1);
#pragma unroll
            for (int st = 0; st < NS; ++st) {
              const float sv = scale_value<ST>(my_scl[st][blk]);
#pragma unroll
              for (int mr = 0; mr < MR; ++mr)
#pragma unroll
                for (int i = 0; i < 4; ++i) tot[mr][st][i] += sv * acc[mr][st][gg][i];
            }
          }
        }
      }
    }
  };

  // chunk ci computes from stage / slot ci % (PD + 1) and requests chunk ci + PD into
  // the slot and stage freed one chunk earlier
  auto chunk = [&](Slot& cur, const uint16_t* xcur, Slot& ahead, uint16_t* xahead, int ci) {
    if (ci + PD < nchunks) xload(ci + PD, xahead);
    __builtin_amdgcn_sched_barrier(0);
    wload(min(ci + PD, nchunks - 1), ahead);
    compute(cur, xcur, ci);
    // chunk ci + 1's activations have landed once at most the later loads are pending:
    // the weights of chunks ci + 1 .. ci + PD and the activations of chunks
    // ci + 2 .. ci + PD that exist. A bare barrier follows: every LDS read of chunk ci has
    // returned (the MFMAs used it), and a workgroup fence would also wait for the loads
    // of the chunks ahead.
    if (ci + 1 < nchunks)
      wait_vm_sel<kWgt, NDMA, PD - 1>(min(PD - 1, nchunks - ci - 2));
    else
      __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };
  // PD + 1 chunks per trip so that ring slots and stages are fixed; a chunk past the end
  // computes nothing and only re-reads the last chunk's weights
  for (int ci = 0; ci < nchunks; ci += PD + 1) {
#pragma unroll
    for (int r = 0; r <= PD; ++r)
      chunk(wr[r], stage(r), wr[(r + PD) % (PD + 1)], stage((r + PD) % (PD + 1)), ci + r);
  }

  if (MX) {
#pragma unroll
    for (int mr = 0; mr < MR; ++mr)
#pragma unroll
      for (int st = 0; st < NS; ++st)
#pragma unroll
        for (int i = 0; i < 4; ++i) tot[mr][st][i] = acc[mr][st][0][i];
  }
  if (PERROW) {
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      const int nr = stream_rows(st);
      const float sv = scale_value<ST>(
          static_cast<const ST*>(stream_s(st))[static_cast<int64_t>(e) * nr + lrow[st]]);
#pragma unroll
      for (int mr = 0; mr < MR; ++mr)
#pragma unroll
        for (int i = 0; i < 4; ++i) tot[mr][st][i] = sv * acc[mr][st][0][i];
    }
  }

  // ---- split-K: partial sums meet in LDS (the first activation stage), in split order ----
  if (SK > 1) {
    constexpr int kPart = MR * NS * 4;  // partial sums per lane
    static_assert((SK - 1) * CPB * kPart * 64 * 4 <= STAGE * 2, "split-K partials fit one stage");
    float* red = reinterpret_cast<float*>(xs0);  // [(SK-1) * CPB][kPart][64]
    if (ks > 0) {
      float* my = red + ((ks - 1) * CPB + cgl) * kPart * 64;
#pragma unroll
      for (int mr = 0; mr < MR; ++mr)
#pragma unroll
        for (int st = 0; st < NS; ++st)
#pragma unroll
          for (int i = 0; i < 4; ++i) my[((mr * NS + st) * 4 + i) * 64 + lane] = tot[mr][st][i];
    }
    __syncthreads();
    if (ks > 0) return;
#pragma unroll
    for (int q = 1; q < SK; ++q) {
      const float* other = red + ((q - 1) * CPB + cgl) * kPart * 64;
#pragma unroll
      for (int mr = 0; mr < MR; ++mr)
#pragma unroll
        for (int st = 0; st < NS; ++st)
#pragma unroll
          for (int i = 0; i < 4; ++i) tot[mr][st][i] += other[((mr * NS + st) * 4 + i) * 64 + lane];
    }
  }

  float bias[NS];
#pragma unroll
  for (int st = 0; st < NS; ++st) {
    const uint16_t* bp = static_cast<const uint16_t*>(stream_b(st));
    bias[st] = bp ? bf16_to_f32(bp[static_cast<int64_t>(e) * stream_rows(st) + lrow[st]]) : 0.f;
  }
#pragma unroll
  for (int mr = 0; mr < MR; ++mr)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = 16 * mr + 4 * kq + i;
    const int64_t r = row0 + m;
    // fc1 with the routing weight on the input: the row's weight scales its sums
    const float rs = (MODE != kModeFc2 && m < valid) ? gemm_row_scale(g, r) : 1.f;
    if (MODE == kModeSwiglu) {
      const int col = col_of(0);
      if (col >= g.ncols) continue;
      float h = 0.f;
      if (m < valid)
        h = swiglu(tot[mr][0][i] * rs + bias[0], tot[mr][1][i] * rs + bias[1], g.alpha, g.beta,
                   g.limit);
      if (m < valid || !g.linear) static_cast<uint16_t*>(g.out)[r * g.ncols + col] = f32_to_bf16(h);
    } else {
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        const int col = col_of(st);
        if (col >= g.ncols) continue;
        if (MODE == kModeFc2) {
          if (m < valid) static_cast<float*>(g.out)[r * g.ncols + col] = tot[mr][st][i] + bias[st];
        } else {
          const float h = m < valid ? plain_act(tot[mr][st][i] * rs + bias[st], g.act) : 0.f;
          if (m < valid || !g.linear) static_cast<uint16_t*>(g.out)[r * g.ncols + col] = f32_to_bf16(h);
        }
      }
    }
  }
}

// Split-K ways from shapes only: enough wave work units to fill the chip a few times
// over, at most the super-steps of a chunk. Blocks longer than a super-step keep one split
// (their groups are summed one super-step at a time in the split's own order).
static int choose_split(const GemmArgs& g, int64_t wg_rows, int bits, int wave_cols) {
  const int ssk = bits == 4 ? 128 : 64;
  if (g.bs > ssk) return 1;
  const int64_t units = wg_rows * ((g.ncols + wave_cols - 1) / wave_cols);
  const int cap = 256 / ssk;
  int sk = 1;
  while (sk < cap && units * sk < 6144) sk *= 2;
  return sk;
}

// Dynamic LDS of the bf16 kernel: the scales of the workgroup's rows (scale_bytes each).
inline size_t gemm_bf16_lds(const GemmArgs& g, int scale_bytes, int sk, int nw = kDecWaves) {
  if (g.bs == 0) return 0;
  return static_cast<size_t>(2) * (nw / sk) * 16 * g.nb * scale_bytes;
}

template <int BITS, typename ST, int MODE, int SK, bool PK, int NW, int MR, int PD = 2>
static hipError_t launch_sk(const GemmArgs& g, int64_t max_tiles, hipStream_t s) {
  constexpr int CPB = NW / SK;
  const int wg_cols = CPB * (MODE == kModeSwiglu ? 16 : 32);
  const int cblocks = (g.ncols + wg_cols - 1) / wg_cols;
  const int64_t wg_rows = max_tiles * (g.M / (MR * kM));
  const dim3 grid = MODE == kModeFc2 ? dim3(xcd_grid(cblocks, wg_rows))
                                     : dim3(cblocks, static_cast<unsigned>(wg_rows));
  const dim3 block(NW * 64);
  const size_t lds = gemm_bf16_lds(g, sizeof(ST), SK, NW);
#define QMOE_DEC(BSV, SKV) \
  launch_gemm_kernel(gemm_bf16_tile_kernel<BITS, ST, MODE, BSV, SKV, PK, NW, MR, PD>, grid, block, lds, s, g)
  if constexpr (std::is_same<ST, uint8_t>::value) {  // MX FP4: blocks of 32 only
    QMOE_DEC(32, SK);
  } else {
  switch (g.bs) {
    case 0: QMOE_DEC(0, SK); break;
    case 16: QMOE_DEC(16, SK); break;
    case 32: QMOE_DEC(32, SK); break;
    case 64: QMOE_DEC(64, SK); break;
    case 128: QMOE_DEC(128, SK); break;
    case 256: QMOE_DEC(256, 1); break;
    default: QMOE_DEC(512, 1); break;
  }
  }
#undef QMOE_DEC
  return hipGetLastError();
}

// Eight waves per workgroup (twice the columns over the same activation stages, so more
// weight loads in flight per CU) for 4-bit tiled-layout grids that still give every CU at
// least two such workgroups, with split-K of at most 2 and the scales of two workgroups
// within the CU's LDS. (8-bit stacks run slower with eight waves.)
template <int BITS, int MODE, int MR>
static bool use_eight_waves(const GemmArgs& g, int64_t wg_rows, int sk, int scale_bytes) {
  constexpr int kCUs = 256;
  if (BITS != 4 || !g.packed || sk > 2) return false;
  const int wg_cols = (8 / sk) * (MODE == kModeSwiglu ? 16 : 32);
  const int64_t wgs = wg_rows * ((g.ncols + wg_cols - 1) / wg_cols);
  const size_t lds = gemm_bf16_lds(g, scale_bytes, sk, 8) + 3 * MR * kM * 256 * 2;
  return wgs >= 2 * kCUs && 2 * lds <= 160 * 1024;
}

// Small grids (at most two four-wave workgroups per CU, as at one to a few tokens) run the
// weight-streaming kernel instead (tiled layout): one column group per workgroup, K split
// over its waves, no LDS activation stages.
constexpr int kGemvWaves = 4;
constexpr int kGemvPD = 2;
template <int MODE>
static bool small_grid(const GemmArgs& g, int64_t wg_rows, int sk) {
  constexpr int kCUs = 256;
  const int wg_cols = (kDecWaves / sk) * (MODE == kModeSwiglu ? 16 : 32);
  return wg_rows * ((g.ncols + wg_cols - 1) / wg_cols) <= 2 * kCUs;
}

template <int BITS, typename ST, int MODE, bool PK, int MR>
static hipError_t launch_bmode_m(const GemmArgs& g, int64_t max_tiles, hipStream_t s) {
  const int64_t wg_rows = max_tiles * (g.M / (MR * kM));  // workgroup rows of the grid
  const int sk = choose_split(g, wg_rows, BITS, MODE == kModeSwiglu ? 16 : 32);
  if constexpr (PK && BITS == 4) {
    if (use_eight_waves<BITS, MODE, MR>(g, wg_rows, sk, sizeof(ST))) {
      if (sk == 1) return launch_sk<BITS, ST, MODE, 1, PK, 8, MR>(g, max_tiles, s);
      return launch_sk<BITS, ST, MODE, 2, PK, 8, MR>(g, max_tiles, s);
    }
  }
  if constexpr (PK && MR == 1) {
    if (g.M == kM && small_grid<MODE>(g, wg_rows, sk))
      return launch_gemv<BITS, ST, MODE, kGemvWaves, kGemvPD>(g, max_tiles, s);
  }
  switch (sk) {
    case 1: return launch_sk<BITS, ST, MODE, 1, PK, kDecWaves, MR>(g, max_tiles, s);
    case 2: return launch_sk<BITS, ST, MODE, 2, PK, kDecWaves, MR>(g, max_tiles, s);
    default: return launch_sk<BITS, ST, MODE, BITS == 4 ? 2 : 4, PK, kDecWaves, MR>(g, max_tiles, s);
  }
}

// Tiles of 16 rows: one MFMA row block per workgroup. Tiles of 32 rows: two row blocks
// per workgroup sharing every decoded weight, except for 4-bit fc2 with per-row scales or
// blocks of 128 and more, which ran faster as two workgroups of 16 rows each (twice the
// workgroups, with fewer registers and less LDS each).
template <int BITS, typename ST, int MODE, bool PK>
static hipError_t launch_bmode(const GemmArgs& g, int64_t max_tiles, hipStream_t s) {
  const bool halves = BITS == 4 && MODE == kModeFc2 && (g.bs == 0 || g.bs >= 128);
  if (g.M == 2 * kM && !halves) return launch_bmode_m<BITS, ST, MODE, PK, 2>(g, max_tiles, s);
  return launch_bmode_m<BITS, ST, MODE, PK, 1>(g, max_tiles, s);
}

template <int BITS, typename ST, bool PK>
static hipError_t launch_mode(const GemmArgs& g, int mode, int64_t max_tiles, hipStream_t s) {
  if (mode == kModeSwiglu) return launch_bmode<BITS, ST, kModeSwiglu, PK>(g, max_tiles, s);
  if (mode == kModePlainAct) return launch_bmode<BITS, ST, kModePlainAct, PK>(g, max_tiles, s);
  return launch_bmode<BITS, ST, kModeFc2, PK>(g, max_tiles, s);
}

// The launches of one weight layout (PK: tiled).
template <bool PK>
static hipError_t launch_gemm_bf16_layout(const GemmArgs& g, int mode, int bits, bool scale_bf16,
                                          int64_t max_tiles, hipStream_t s) {
  if (max_tiles <= 0) return hipSuccess;
  if constexpr (PK) {
    if (g.mx) return launch_mode<4, uint8_t, PK>(g, mode, max_tiles, s);
  }
  if (bits == 4)
    return scale_bf16 ? launch_mode<4, uint16_t, PK>(g, mode, max_tiles, s)
                      : launch_mode<4, float, PK>(g, mode, max_tiles, s);
  return scale_bf16 ? launch_mode<8, uint16_t, PK>(g, mode, max_tiles, s)
                    : launch_mode<8, float, PK>(g, mode, max_tiles, s);
}

}  // namespace qmoe
