// Grouped dequant GEMM, 128-row tiles, 4-bit codes with bf16 block scales, tiled weight
// layout, on fp16 matrix cores: each weight is scaled as it is decoded, exactly, in one fp16
// operand, and the MFMAs sum the whole K with no per-output work per block.
//
// ClikaRT "QMoEWoQ" page, class description: the expert weights stay quantized and each
// block is decoded inside the GEMM dot. graiphic "QMoE" page: stacks [E, N, K/pack],
// scales [E, N, K/block_size] (block_size attribute), value (q - 8) * scale for 4 bits.
//
// Exactness. A 4-bit code minus its zero point, |q - 8| <= 8, has at most 3 significant
// bits and a bf16 scale 8, so (q - 8) * s has at most 11: fp16 holds it exactly once the
// scale is lifted into fp16's range. Each weight row's scales are lifted by one power of two
// 2^b (the row's largest scale into [2^12, 2^13): no product reaches 65504), and each
// activation row, already in fp16, by 2^a (f16prep.hip). Products of two fp16 are exact in
// the fp32 accumulators, so the sums equal those of the bf16 operands up to the order of the
// fp32 additions, scaled by 2^(a + b), which the epilogue divides out exactly.
//
// Decode: each nibble q goes into the fp16 pattern of 1024 (0x6400), giving 1024 + q exactly;
// one packed fp16 add of -1032 gives q - 8 and one packed fp16 multiply by the lifted scale
// gives the weight (both exact), two codes per instruction.
//
// Workgroup: one 128-row tile of one expert by 256 weight rows, four waves side by side,
// each 128 rows x 4 weight-row slices of 16 (2 gate + 2 up slices, 32 output columns, with
// SwiGLU; otherwise four neighbouring groups of 16 columns), so that every decoded weight
// feeds the MFMAs of all 128 rows and each activation fragment read from LDS feeds four
// MFMAs. Each fragment is read again for the next k-slice in place, right after its MFMAs,
// which keeps this shape within 256 registers (two waves per SIMD).
//   - Activations: loads that target LDS, 16 bytes per lane, a double-buffered stage of
//     128 rows x one K step (128 k) with its 16-byte granules XOR-swizzled by row.
//   - Weights: one 16-byte load per slice and K step (one lane's share of a contiguous 1 KB
//     tile), a whole step ahead, with the default cache policy: the tiles of one expert that
//     an XCD runs together (xcd_item's bands) read each weight tile through its L2.
//   - Scales: the 256 weight rows x the step's blocks (one row per thread), loaded a step
//     ahead into registers, lifted to fp16 when written to a two-slot LDS ring before the
//     barrier, widened to a pair when read.
//   - Rows: the tile's source-row offsets, row factors and lifts in an LDS table formed
//     once (one thread per row); the activation loads read their offsets from it.
#pragma once

#include "common.h"
#include "gemm_common.h"
#include "launch.h"

namespace qmoe {

namespace h16 {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));

constexpr int kTM = 128;   // rows per tile
constexpr int kNB = 4;     // 16-row weight slices per wave
constexpr int kMT = 8;     // 16-row MFMA tiles per wave (all 128 rows)
constexpr int kSSK = 128;  // K per step (one 1 KB tile of 4-bit codes per slice)

// Eight 4-bit codes of one tiled-layout word (decode order: the k-slice's element 2i in the
// low half of pair i, element 2i + 1 in the high half) to eight fp16 weights (q - 8) * s.
__device__ __forceinline__ half8_t decode4_h16(uint32_t w, half2_t s2) {
  const uint32_t magic = 0x64006400u, mask = 0x000F000Fu;
  const half2_t off = {static_cast<_Float16>(-1032.0f), static_cast<_Float16>(-1032.0f)};
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    half2_t v = __builtin_bit_cast(half2_t, and_or(w >> (4 * i), mask, magic));
    v = (v + off) * s2;
    r[i] = __builtin_bit_cast(uint32_t, v);
  }
  return __builtin_bit_cast(half8_t, r);
}

}  // namespace h16

template <int MODE, int BS>
__global__ __launch_bounds__(256, 2) void gemm_h16_prefill_kernel(GemmArgs g) {
  using namespace h16;
  constexpr bool kTwo = (MODE == kModeSwiglu);
  constexpr int NS = kTwo ? 2 : 1;
  constexpr int NBS = kNB / NS;                   // slices per stream
  constexpr int SSK = kSSK;
  constexpr int MPS = SSK / 32;                   // MFMA k-slices per step
  constexpr int GPR = SSK / 8;                    // 16-byte granules per activation row
  constexpr int NDMA = kTM * GPR / 64 / 4;        // LDS-destination loads per wave per step
  constexpr int BCOLS = 4 * NBS * 16;             // output columns per workgroup
  constexpr int STAGE = kTM * SSK;                // fp16 elements per LDS stage
  constexpr int NBLK = BS < SSK ? SSK / BS : 1;   // scale blocks a step touches
  constexpr int SROWS = 4 * kNB * 16;             // weight rows of the workgroup (256)
  static_assert(BS >= 16 && BS <= 128, "blocks of 16 to 128");

  __shared__ __attribute__((aligned(16))) uint16_t xs0[STAGE];
  __shared__ __attribute__((aligned(16))) uint16_t xs1[STAGE];
  __shared__ uint16_t sring[2][SROWS * NBLK];  // lifted scales (fp16), this step and next
  // the tile's rows, formed once by threads 0..127: byte offset of the row of a that feeds
  // it (kOutOfRange for padding rows), the factor on its sums (the routing weight when it
  // goes to the expert's input, else 1) and its lift (written after the main loop)
  __shared__ uint32_t rsrc[kTM];
  __shared__ float rscale[kTM];
  __shared__ int rlift[kTM];
  // the workgroup's weight rows (one per thread): bias and lift, for the epilogue
  __shared__ float wbias[SROWS];
  __shared__ int wlift[SROWS];

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
  auto stream_lift = [&](int st) { return (st == 1 && kTwo && g.fusion == 0) ? g.wlift3 : g.wlift; };
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

  // ---- scales: thread R of the workgroup owns weight row R = wnn * 16 kNB + b * 16 + nn
  // (as many rows as threads) and writes the step's NBLK blocks of it, lifted by its row's
  // power of two, to sring[slot][R * NBLK + l] ----
  static_assert(SROWS == 256, "one weight row per thread");
  uint32_t soff;
  int slift;
  float my_bias;
  const uint16_t* srow_base;
  {
    const int R = tid;
    const int wnn = R / (16 * kNB), b = (R % (16 * kNB)) / 16, nn = R % 16;
    const int st = b / NBS;
    const int c = min(slice_col(wnn, b, nn), g.ncols - 1);
    const int64_t wrow = static_cast<int64_t>(e) * stream_rows(st) + local_row(st, c);
    soff = static_cast<uint32_t>(wrow * nb);
    slift = stream_lift(st)[wrow];
    const uint16_t* bp = static_cast<const uint16_t*>(stream_b(st));
    my_bias = bp ? bf16_to_f32(bp[wrow]) : 0.f;
    srow_base = static_cast<const uint16_t*>((st == 1 && kTwo && g.fusion == 0) ? g.s3 : g.s);
  }
  uint16_t sreg[NBLK];
  auto sload = [&](int s) {
    // first block of the step; blocks of the last, padded step that lie past K are clamped
    // to the row's last block (their activations are zero)
    const int blk = BS < SSK ? s * NBLK : (s * SSK) / BS;
#pragma unroll
    for (int l = 0; l < NBLK; ++l) sreg[l] = srow_base[soff + min(blk + l, nb - 1)];
  };
  auto sstore = [&](int slot) {
#pragma unroll
    for (int l = 0; l < NBLK; ++l) {
      const _Float16 h = static_cast<_Float16>(ldexpf(bf16_to_f32(sreg[l]), slift));
      sring[slot][tid * NBLK + l] = __builtin_bit_cast(uint16_t, h);
    }
  };

  // ---- activations (fp16 rows): row-major stages, XOR-swizzled granules ----
  auto key = [](int r) { return r & 15; };
  const rsrc_t xres = make_rsrc(g.a, static_cast<uint32_t>(g.a_rows * K * 2));
  auto granule = [&](int t) {
    const int p = (wave + 4 * t) * 64 + lane;
    return (p % GPR) ^ key(p / GPR);
  };
  const int gq = granule(0);  // the same for every load t (4t * 64 / GPR rows later)
  // the first step's weights and scales depend on the expert alone: requested before the
  // row table, whose loads and division they then overlap
  u32x4 wa[kNB], wb[kNB];
  wload(0, wa);
  sload(0);
  int my_lift = 0;  // thread t < 128: the lift of row t, stored to rlift after the main loop
  if (tid < kTM) {
    const int m = tid;
    uint32_t off = kOutOfRange;  // padding rows land as zeros
    float rs = 1.f;
    if (m < valid) {
      const int64_t r = row0 + m;
      const int64_t src = (MODE == kModeFc2) ? r : gemm_src_row(g, r);
      off = static_cast<uint32_t>(src * K * 2);
      if (MODE != kModeFc2) rs = gemm_row_scale(g, r);
      my_lift = g.alift[src];
    }
    rsrc[m] = off;
    rscale[m] = rs;
  }
  wbias[tid] = my_bias;
  wlift[tid] = slift;
  __syncthreads();
  // load t of this lane: row (wave + 4t) * 64 / GPR + lane / GPR of the tile, granule gq;
  // its offset is read from the row table at each load instead of held in registers
  auto xoff = [&](int t) -> uint32_t {
    // a padding row's kOutOfRange plus the granule (and the step's scalar offset) stays
    // past every buffer, so it still reads zeros
    return rsrc[(wave + 4 * t) * (64 / GPR) + lane / GPR] + static_cast<uint32_t>(16 * gq);
  };
  auto xload = [&](int s, uint16_t* stage) {
    const int k0 = __builtin_amdgcn_readfirstlane(s * SSK);
    if (k0 + SSK > K) {
      // the last step of a K that is not a whole number of steps: granules past K land as
      // zeros
#pragma unroll
      for (int t = 0; t < NDMA; ++t)
        buf_load16_lds(xres, stage + (wave + 4 * t) * 64 * 8, k0 + 8 * gq < K ? xoff(t) : kOutOfRange,
                       2 * k0);
    } else {
#pragma unroll
      for (int t = 0; t < NDMA; ++t) buf_load16_lds(xres, stage + (wave + 4 * t) * 64 * 8, xoff(t), 2 * k0);
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

  // the lifted scale pair of slice b for this lane's 8 weights of k-slice j (one block: a
  // lane's 8 k lie in one block of 16 or longer)
  auto lane_scale = [&](const uint16_t* sc, int b, int j) -> half2_t {
    const uint16_t* row = sc + (wn * 16 * kNB + b * 16 + n) * NBLK;
    uint32_t v;
    if constexpr (BS == 16 && NBLK > 1)
      v = row[2 * j + (kq >> 1)];
    else
      v = row[BS < SSK ? (32 * j) / BS : 0];
    return __builtin_bit_cast(half2_t, v | (v << 16));
  };
  auto compute = [&](const uint16_t* stage, const u32x4 (&w)[kNB], int slot) {
    const uint16_t* sc = sring[slot];
    u32x4 xa[kMT];
    aread(stage, 0, xa);
#pragma unroll
    for (int j = 0; j < MPS; ++j) {
      half8_t bw[kNB];
#pragma unroll
      for (int b = 0; b < kNB; ++b) bw[b] = decode4_h16(w[b][j], lane_scale(sc, b, j));
      const uint32_t an = abase ^ static_cast<uint32_t>(64 * (j + 1));
#pragma unroll
      for (int mt = 0; mt < kMT; ++mt) {
        const half8_t xh = __builtin_bit_cast(half8_t, xa[mt]);
#pragma unroll
        for (int b = 0; b < kNB; ++b)
          acc[mt][b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xh, bw[b], acc[mt][b], 0, 0, 0);
        // the fragment's next k-slice, in place, while the other fragments' MFMAs run
        if (j + 1 < MPS)
          xa[mt] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(stage) + an +
                                                   mt * 16 * GPR * 16);
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
  xload(0, xs0);
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

  // ---- epilogue: the lifts divided out, bias, activation; the outputs pass through the
  // (now free) activation stages so that they leave in 16-byte row segments ----
  if (tid < kTM) rlift[tid] = my_lift;
  // every wave is past its last read of the stages, and the lifts are in place
  __syncthreads();
  float bias[kNB];
  int wl[kNB];
#pragma unroll
  for (int b = 0; b < kNB; ++b) {
    bias[b] = wbias[wn * 16 * kNB + b * 16 + n];
    wl[b] = wlift[wn * 16 * kNB + b * 16 + n];
  }
  // staging: 128 output columns per stage, rows of 256 bytes (bf16 h) or 512 bytes (fp32 y,
  // in two passes of 64 rows); the 16-byte chunk c of row r sits at slot c ^ (r mod chunks),
  // so the 16 lanes of one MFMA row and the four rows a wave writes at once fall in
  // distinct banks
  constexpr int kEl = MODE == kModeFc2 ? 4 : 2;        // bytes per output
  constexpr int kPass = MODE == kModeFc2 ? 2 : 1;
  constexpr int kRowsPass = kTM / kPass;
  constexpr int kChunkEl = 16 / kEl;                   // outputs per 16-byte chunk
  constexpr int kChunks = 128 / kChunkEl;              // chunks per staged row
  constexpr int kStages = (BCOLS + 127) / 128;
  constexpr int kRowBytes = 128 * kEl;
  static_assert(kRowsPass * kRowBytes == STAGE * 2, "a pass fills a stage");
  auto staged = [&](int rl, int c) -> char* {
    char* st = reinterpret_cast<char*>(c < 128 ? xs0 : xs1);
    const int cc = c & 127;
    return st + rl * kRowBytes + (((cc / kChunkEl) ^ (rl & (kChunks - 1))) * 16) + (cc % kChunkEl) * kEl;
  };
#pragma unroll
  for (int pass = 0; pass < kPass; ++pass) {
    if (pass > 0) __syncthreads();  // the previous pass's copies have read the stages
#pragma unroll
    for (int mt = pass * (kMT / kPass); mt < (pass + 1) * (kMT / kPass); ++mt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = mt * 16 + 4 * kq + i;
        const int rl = m - pass * kRowsPass;
        const float rs = rscale[m];
        const int al = rlift[m];
#pragma unroll
        for (int cb = 0; cb < NBS; ++cb) {
          const int cl = wn * NBS * 16 + cb * 16 + n;  // column inside the workgroup
          float z[NS];
#pragma unroll
          for (int st = 0; st < NS; ++st) {
            const int b = st * NBS + cb;
            z[st] = ldexpf(acc[mt][b][i], -(al + wl[b])) * rs + bias[b];
          }
          if (MODE == kModeFc2) {
            *reinterpret_cast<float*>(staged(rl, cl)) = z[0];
          } else {
            float hv = 0.f;
            if (m < valid)
              hv = (MODE == kModeSwiglu) ? swiglu(z[0], z[NS - 1], g.alpha, g.beta, g.limit)
                                         : plain_act(z[0], g.act);
            *reinterpret_cast<uint16_t*>(staged(rl, cl)) = f32_to_bf16(hv);
          }
        }
      }
    }
    __syncthreads();
    // copies out: chunk q of the pass is stage q / (rows * chunks), row (q / chunks) % rows,
    // chunk q % chunks; real rows only for y, every row of the tile for h (padding rows as
    // the zeros staged for them), except for the linear layer
    constexpr int kTot = kRowsPass * kChunks * kStages;
#pragma unroll
    for (int u = 0; u < (kTot + 255) / 256; ++u) {
      const int q = tid + 256 * u;
      if (q >= kTot) break;
      const int stg = q / (kRowsPass * kChunks);
      const int rl = (q / kChunks) % kRowsPass, ch = q % kChunks;
      const int m = pass * kRowsPass + rl;
      const int col = col0 + stg * 128 + ch * kChunkEl;
      if (col >= g.ncols) continue;
      if (MODE == kModeFc2 ? m >= valid : (m >= valid && g.linear)) continue;
      const char* src = reinterpret_cast<const char*>(stg == 0 ? xs0 : xs1) + rl * kRowBytes +
                        ((ch ^ (rl & (kChunks - 1))) * 16);
      const u32x4 v = *reinterpret_cast<const u32x4*>(src);
      char* dst = static_cast<char*>(g.out) + ((row0 + m) * g.ncols + col) * kEl;
      *reinterpret_cast<u32x4*>(dst) = v;
    }
  }
}

template <int MODE, int BS>
static hipError_t launch_h16_bs(const GemmArgs& g, int64_t max_tiles, hipStream_t s) {
  constexpr int bcols = 4 * (h16::kNB / (MODE == kModeSwiglu ? 2 : 1)) * 16;
  dim3 grid(xcd_grid((g.ncols + bcols - 1) / bcols, max_tiles)), block(256);
  launch_gemm_kernel(gemm_h16_prefill_kernel<MODE, BS>, grid, block, 0, s, g);
  return hipGetLastError();
}

template <int MODE>
static hipError_t launch_h16_mode(const GemmArgs& g, int64_t max_tiles, hipStream_t s) {
  switch (g.bs) {
    case 16: return launch_h16_bs<MODE, 16>(g, max_tiles, s);
    case 32: return launch_h16_bs<MODE, 32>(g, max_tiles, s);
    case 64: return launch_h16_bs<MODE, 64>(g, max_tiles, s);
    default: return launch_h16_bs<MODE, 128>(g, max_tiles, s);
  }
}

}  // namespace qmoe
