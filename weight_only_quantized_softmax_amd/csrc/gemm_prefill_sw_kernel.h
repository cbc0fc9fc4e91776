// Grouped dequant GEMM, bf16 activations, 128-row tiles, block scales, tiled weight layout:
// the weights are scaled as they are decoded, once per 128-row tile, and the MFMAs sum the
// whole K with no per-output scaling.
//
// ClikaRT "QMoEWoQ" page, class description: the expert weights stay quantized and each
// block is decoded inside the GEMM dot. graiphic "QMoE" page: stacks [E, N, K/pack],
// scales [E, N, K/block_size] (block_size attribute).
//
// Each lane's 8 weights of one MFMA k-slice (32 k) lie in one scale block for blocks of 32
// and longer, and in one of the two halves for blocks of 16, so a lane multiplies its 8
// codes by a single scale: (q - z) * s is formed exactly in fp32 (a 4- or 8-bit integer
// times a bf16 or fp32 scale) with one FMA per weight. A single bf16 operand would round
// each scaled weight (relative 2^-9), which at these shapes moves the forward's output by
// about 1e-2 of its RMS on top of the output's own rounding; so the weight goes to the
// MFMAs as two bf16 operands hi + lo that sum to it exactly (split8), two MFMAs per product.
// MX FP4 codes take the hardware's scaled E2M1 conversion instead (exact in one operand).
// Compared with scaling partial sums per block, this trades one FMA per output element per
// block and the zero-point MFMAs for one extra MFMA per product and a few VALU per weight.
//
// Workgroup: one 128-row tile of one expert by 128 weight rows, four waves side by side,
// each 128 rows x 2 weight-row slices of 16, so that every weight a wave decodes feeds the
// MFMAs of all 128 rows (8 MFMAs per decoded operand). With SwiGLU the two slices of a wave
// are the gate and the up rows of its 16 output columns; otherwise two neighbouring groups
// of 16 columns.
//   - Activations: loads that target LDS, 16 bytes per lane, a double-buffered stage of
//     128 rows x one K step with its 16-byte granules XOR-swizzled by row; one barrier per
//     K step.
//   - Weights: one 16-byte load per slice and K step (one lane's share of a contiguous
//     1 KB tile), a whole step ahead.
//   - Scales: the 128 rows x the step's blocks, loaded one step ahead into registers and
//     written to a two-slot LDS ring before the step's barrier.
#pragma once

#include <type_traits>

#include "common.h"
#include "gemm_common.h"
#include "launch.h"

namespace qmoe {

namespace sw {

constexpr int kTM = 128;   // rows per tile
constexpr int kNB = 2;     // 16-row weight slices per wave
constexpr int kMT = 8;     // 16-row MFMA tiles per wave (all 128 rows)

// Eight fp32 weights (exact products (q - z) * s, in k order) as two bf16 operands whose
// sum is the weight: hi holds the upper 16 bits of each fp32 (the weight truncated to bf16)
// and lo the upper 16 bits of the remainder w - hi, which fp32 holds exactly. A 4-bit code
// times a bf16 scale has at most 12 significant bits and an 8-bit code at most 16, so the
// remainder has at most 8 and lo holds it exactly: hi + lo == w. With fp32 scales the
// remainder is truncated to 8 bits (relative error below 2^-16 of the weight).
struct Split {
  u32x4 hi, lo;
};

// hi: the upper halves of a (low 16 bits) and b (high 16 bits); lo: those of a - hi(a) and
// b - hi(b)
__device__ __forceinline__ uint2 split2(float a, float b) {
  const uint32_t ua = __float_as_uint(a), ub = __float_as_uint(b);
  const float ra = a - __uint_as_float(ua & 0xFFFF0000u);
  const float rb = b - __uint_as_float(ub & 0xFFFF0000u);
  return make_uint2(__builtin_amdgcn_perm(ub, ua, 0x07060302u),
                    __builtin_amdgcn_perm(__float_as_uint(rb), __float_as_uint(ra), 0x07060302u));
}

__device__ __forceinline__ Split split8(const float (&v)[8]) {
  Split r;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint2 h = split2(v[2 * p], v[2 * p + 1]);
    r.hi[p] = h.x;
    r.lo[p] = h.y;
  }
  return r;
}

// Eight 4-bit codes of one word in the tiled layout's decode order (element i of the k-slice
// in nibble (0, 4, 1, 5, 2, 6, 3, 7)[i]) to (q - 8) * s in k order. The low nibbles of the
// four bytes are elements 0, 4, 1, 5; the high nibbles 2, 6, 3, 7.
__device__ __forceinline__ Split decode4_scaled(uint32_t w, float s, float c) {
  const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
  const float v[8] = {fmaf(static_cast<float>(lo & 0xFF), s, c),
                      fmaf(static_cast<float>((lo >> 16) & 0xFF), s, c),
                      fmaf(static_cast<float>(hi & 0xFF), s, c),
                      fmaf(static_cast<float>((hi >> 16) & 0xFF), s, c),
                      fmaf(static_cast<float>((lo >> 8) & 0xFF), s, c),
                      fmaf(static_cast<float>(lo >> 24), s, c),
                      fmaf(static_cast<float>((hi >> 8) & 0xFF), s, c),
                      fmaf(static_cast<float>(hi >> 24), s, c)};
  return split8(v);
}

// Eight 8-bit codes (two words, element i in byte i) to (q - 128) * s.
__device__ __forceinline__ Split decode8_scaled(uint32_t w0, uint32_t w1, float s, float c) {
  const float v[8] = {fmaf(static_cast<float>(w0 & 0xFF), s, c),
                      fmaf(static_cast<float>((w0 >> 8) & 0xFF), s, c),
                      fmaf(static_cast<float>((w0 >> 16) & 0xFF), s, c),
                      fmaf(static_cast<float>(w0 >> 24), s, c),
                      fmaf(static_cast<float>(w1 & 0xFF), s, c),
                      fmaf(static_cast<float>((w1 >> 8) & 0xFF), s, c),
                      fmaf(static_cast<float>((w1 >> 16) & 0xFF), s, c),
                      fmaf(static_cast<float>(w1 >> 24), s, c)};
  return split8(v);
}

}  // namespace sw

// Blocks of 16 to 128 (MX FP4: 32), tiled layout; BITS 4 or 8.
template <int BITS, typename ST, int MODE, int BS>
__global__ __launch_bounds__(256, 2) void gemm_bf16_prefill_sw_kernel(GemmArgs g) {
  using namespace sw;
  constexpr bool kTwo = (MODE == kModeSwiglu);
  constexpr int NS = kTwo ? 2 : 1;
  constexpr int NBS = kNB / NS;                   // slices per stream
  constexpr int SSK = BITS == 4 ? 128 : 64;       // K per step (one 1 KB tile per slice)
  constexpr int MPS = SSK / 32;                   // MFMA k-slices per step
  constexpr int GPR = SSK / 8;                    // 16-byte granules per activation row
  constexpr int NDMA = kTM * GPR / 64 / 4;        // LDS-destination loads per wave per step
  constexpr int BCOLS = 4 * NBS * 16;             // output columns per workgroup
  constexpr int STAGE = kTM * SSK;                // bf16 elements per LDS stage
  constexpr int NBLK = BS < SSK ? SSK / BS : 1;   // scale blocks a step touches
  constexpr int SROWS = 4 * kNB * 16;             // weight rows of the workgroup (128)
  constexpr int SPT = (SROWS * NBLK + 255) / 256; // scales loaded per thread per step
  constexpr bool MX = std::is_same<ST, uint8_t>::value;
  static_assert(!MX || (BITS == 4 && BS == 32), "MX FP4: 4-bit, blocks of 32");
  static_assert(BS >= 16 && BS <= 128, "blocks of 16 to 128");
  // -z * s: the zero point leaves through the FMA's addend (exact in fp32)
  constexpr float kZero = BITS == 4 ? 8.0f : 128.0f;

  __shared__ __attribute__((aligned(16))) uint16_t xs0[STAGE];
  __shared__ __attribute__((aligned(16))) uint16_t xs1[STAGE];
  __shared__ ST sring[2][SROWS * NBLK];  // scales of this step and the next

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
  const int nss = g.kt;  // K steps (the tiled layout pads K to whole steps with code 0)
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
  // output column of slice b, lane row nn, for wave wnn
  auto slice_col = [&](int wnn, int b, int nn) { return col0 + wnn * NBS * 16 + (b % NBS) * 16 + nn; };

  // ---- weights: slice b's sequence of 1 KB tiles (a block past the stream reads zeros);
  // lane l reads bytes 16 l of the step's tile ----
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

  // ---- scales: entry i of a step is weight row i / NBLK of the workgroup (row
  // R = wnn * 32 + b * 16 + nn), block i % NBLK of the step ----
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
  ST sreg[SPT];
  auto sload = [&](int s) {
    // first block of the step; blocks of the last, padded step that lie past K are clamped
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
  auto granule = [&](int t) {
    const int p = (wave + 4 * t) * 64 + lane;
    return (p % GPR) ^ key(p / GPR);
  };
  const int gq = granule(0);  // the same for every load t (4t * 64 / GPR rows later)
  uint32_t xoffs[NDMA];
#pragma unroll
  for (int t = 0; t < NDMA; ++t) {
    const int p = (wave + 4 * t) * 64 + lane;
    const int r = p / GPR, q = granule(t);
    uint32_t off = kOutOfRange;  // padding rows land as zeros
    if (r < valid) {
      const int64_t src = (MODE == kModeFc2) ? row0 + r : gemm_src_row(g, row0 + r);
      off = static_cast<uint32_t>((src * K + 8 * q) * 2);
    }
    xoffs[t] = off;
  }
  auto xload = [&](int s, uint16_t* stage) {
    const int k0 = __builtin_amdgcn_readfirstlane(s * SSK);
    if (k0 + SSK > K) {
      // the last step of a K that is not a whole number of steps: granules past K land as
      // zeros
#pragma unroll
      for (int t = 0; t < NDMA; ++t)
        buf_load16_lds(xres, stage + (wave + 4 * t) * 64 * 8, k0 + 8 * gq < K ? xoffs[t] : kOutOfRange,
                       2 * k0);
    } else {
#pragma unroll
      for (int t = 0; t < NDMA; ++t) buf_load16_lds(xres, stage + (wave + 4 * t) * 64 * 8, xoffs[t], 2 * k0);
    }
    // the step-end wait counts the loads issued after these: none may move above
    __builtin_amdgcn_sched_barrier(0);
  };

  // operand reads: row r = mt*16 + n has key(r) = key(n); k-slice j's granule is
  // q = 4 j + kq, whose j bits the swizzle leaves to an XOR
  const uint32_t abase = static_cast<uint32_t>((n * GPR + (kq ^ key(n))) * 16);
  auto aread = [&](const uint16_t* stage, int j, u32x4 (&xa)[kMT]) {
    const uint32_t aj = abase ^ static_cast<uint32_t>(64 * j);
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt)
      xa[mt] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(stage) + aj +
                                               mt * 16 * GPR * 16);
  };

  const floatx4 zero4 = {0.f, 0.f, 0.f, 0.f};
  floatx4 acc[kMT][kNB];
#pragma unroll
  for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
    for (int b = 0; b < kNB; ++b) acc[mt][b] = zero4;

  // the scale of slice b for this lane's 8 weights of k-slice j (one block, see above)
  auto lane_scale = [&](const ST* sc, int b, int j) -> float {
    const ST* row = sc + (wn * 32 + b * 16 + n) * NBLK;
    if constexpr (BS == 16 && NBLK > 1) {
      return scale_value<ST>(row[2 * j + (kq >> 1)]);
    } else {
      return scale_value<ST>(row[BS < SSK ? (32 * j) / BS : 0]);
    }
  };
  auto compute = [&](const uint16_t* stage, const u32x4 (&w)[kNB], int slot) {
    const ST* sc = sring[slot];
    u32x4 xa[kMT], xn[kMT];
    aread(stage, 0, xa);
#pragma unroll
    for (int j = 0; j < MPS; ++j) {
      if (j + 1 < MPS) aread(stage, j + 1, xn);  // the next k-slice's operands, in flight
      if constexpr (MX) {
        // E2M1 codes times a power of two: exact in one bf16 operand
        bf16x8 bw[kNB];
#pragma unroll
        for (int b = 0; b < kNB; ++b) bw[b] = decode_mx(w[b][j], lane_scale(sc, b, j));
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt) {
          const bf16x8 xb = __builtin_bit_cast(bf16x8, xa[mt]);
#pragma unroll
          for (int b = 0; b < kNB; ++b)
            acc[mt][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xb, bw[b], acc[mt][b], 0, 0, 0);
        }
      } else {
        // integer codes: the scaled weight as hi + lo (exact for bf16 scales), two MFMAs
        Split bw[kNB];
#pragma unroll
        for (int b = 0; b < kNB; ++b) {
          const float sv = lane_scale(sc, b, j);
          if constexpr (BITS == 4)
            bw[b] = decode4_scaled(w[b][j], sv, -kZero * sv);
          else
            bw[b] = decode8_scaled(w[b][2 * j], w[b][2 * j + 1], sv, -kZero * sv);
        }
        // every hi product first, then every lo product: the two MFMAs into one
        // accumulator are 16 independent MFMAs apart
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
          for (int b = 0; b < kNB; ++b)
            acc[mt][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8, xa[mt]), __builtin_bit_cast(bf16x8, bw[b].hi),
                acc[mt][b], 0, 0, 0);
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
          for (int b = 0; b < kNB; ++b)
            acc[mt][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8, xa[mt]), __builtin_bit_cast(bf16x8, bw[b].lo),
                acc[mt][b], 0, 0, 0);
      }
      if (j + 1 < MPS) {
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt) xa[mt] = xn[mt];
      }
      // one k-slice at a time: decodes hoisted from later slices would hold more registers
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- pipeline: step s reads stage s % 2, weight buffer s % 2, scale slot s % 2 ----
  static_assert(NDMA < 64, "vmcnt holds 6 bits");
  // issue order per step: activations, scales, weights; waiting down to the weight loads
  // leaves the step's activations in LDS and its scales in registers
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
    compute(xs0, wa, 0);
    __builtin_amdgcn_s_waitcnt(kWaitX);
    sstore(1);
    __syncthreads();
    if (s + 2 < nss) {
      xload(s + 2, xs0);
      sload(s + 2);
      wload(s + 2, wa);
    }
    compute(xs1, wb, 1);
    if (s + 2 < nss) {
      __builtin_amdgcn_s_waitcnt(kWaitX);
      sstore(0);
    }
    __syncthreads();
  }
  if (nss & 1) compute(xs0, wa, 0);

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
          z[st] = acc[mt][b][i] * rs + bias[b];
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

template <int BITS, typename ST, int MODE, int BS>
static hipError_t launch_sw_bs(const GemmArgs& g, int64_t max_tiles, hipStream_t s) {
  constexpr int bcols = 4 * (sw::kNB / (MODE == kModeSwiglu ? 2 : 1)) * 16;
  dim3 grid(xcd_grid((g.ncols + bcols - 1) / bcols, max_tiles)), block(256);
  launch_gemm_kernel(gemm_bf16_prefill_sw_kernel<BITS, ST, MODE, BS>, grid, block, 0, s, g);
  return hipGetLastError();
}

template <int BITS, typename ST, int MODE>
static hipError_t launch_sw_mode(const GemmArgs& g, int64_t max_tiles, hipStream_t s) {
  if constexpr (std::is_same<ST, uint8_t>::value) {
    return launch_sw_bs<BITS, ST, MODE, 32>(g, max_tiles, s);
  } else {
    switch (g.bs) {
      case 16: return launch_sw_bs<BITS, ST, MODE, 16>(g, max_tiles, s);
      case 32: return launch_sw_bs<BITS, ST, MODE, 32>(g, max_tiles, s);
      case 64: return launch_sw_bs<BITS, ST, MODE, 64>(g, max_tiles, s);
      default: return launch_sw_bs<BITS, ST, MODE, 128>(g, max_tiles, s);
    }
  }
}

template <int BITS, typename ST>
static hipError_t launch_sw_t(const GemmArgs& g, int mode, int64_t max_tiles, hipStream_t s) {
  if (mode == kModeSwiglu) return launch_sw_mode<BITS, ST, kModeSwiglu>(g, max_tiles, s);
  if (mode == kModePlainAct) return launch_sw_mode<BITS, ST, kModePlainAct>(g, max_tiles, s);
  return launch_sw_mode<BITS, ST, kModeFc2>(g, max_tiles, s);
}

}  // namespace qmoe
