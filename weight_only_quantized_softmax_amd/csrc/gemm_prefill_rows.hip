// Grouped dequant GEMM, bf16 activations, 128-row tiles, one scale per output row: the
// prefill shape whose expert groups fill large tiles and whose cost is the bf16 MFMA rate.
//
// ClikaRT "QMoEWoQ" page, class description: the expert weights stay quantized and are
// decoded inside the GEMM dot. graiphic "QMoE" page: stacks [E, N, K/pack]; without a
// block_size every output row (a column of the transposed weight) has one scale.
//
// Workgroup: one 128-row tile of one expert, four waves, two waves per SIMD (256 registers
// a wave), the shape set by RowsShape:
//   - fc1: 1 x 4 waves, each 128 rows x 4 weight-row slices of 16 (with SwiGLU 2 gate + 2
//     up, so the workgroup covers 256 weight rows = 128 output columns), each decoded
//     weight feeding 8 MFMAs; each activation fragment is read again for the next k-slice
//     in place, right after its MFMAs, which keeps this shape within its registers;
//   - fc2: 2 x 2 waves, each 64 rows x 6 slices (192 weight rows a workgroup); in the
//     forward with 4-bit codes, where fc1 has written each row's partial sums of h (one per
//     column block) and partsum_kernel has added them up, 1 x 4 like fc1.
//   - Activations reach LDS without passing through registers: buffer loads with the LDS
//     as destination, 16 bytes per lane, 16 lanes per 256-byte row segment, two stages
//     (this K step and the next). The 16-byte granule q of row r sits at slot
//     r * G + (q ^ key(r)) of its stage, so the 16 lanes that read one MFMA operand (16
//     consecutive rows, one granule each) fall in distinct banks.
//   - Each wave reads its 8 weight-row slices with one 16-byte raw buffer load per slice
//     and K step, issued a whole step ahead into a second register buffer, and decodes
//     them in registers: 4-bit codes become 128 + q by OR-ing the nibble into the exponent
//     pattern of 128, 8-bit codes convert exactly. The 4-bit decode yields the elements of
//     a dword in the order [e0 e4 e1 e5 e2 e6 e3 e7]; the activation fragment is permuted
//     to match after its LDS read.
//   - The zero point and the +128 offset leave through the row sums of the activations:
//     acc - (c+z) * rowsum, scaled once per output row in the epilogue. In the forward
//     (XS) fc1 reads each token's row sum, formed once by launch_rowsum; otherwise the row
//     sums come from v_dot2 on the fragments the waves already read (each wave sums a
//     quarter of the rows; the quarters meet in LDS at the end).
//   - The tile's rows are formed once, by one thread per row, into an LDS table: the byte
//     offset of the row of the activations that feeds it (one division by k per row) and,
//     with the forward's row sums, its correction. The activation loads take their offsets
//     from it.
//   - fc1 (4-bit codes): the outputs pass through the freed activation stages (16-byte
//     chunks XOR-swizzled by row) and leave in 16-byte row segments; fc2's fp32 outputs and
//     8-bit codes' outputs are stored directly.
// One barrier per K step: the loads of step s+1 are issued before step s computes; the
// activation loads are waited for after it, the weight loads where they are first used
// (loads complete in issue order, so the wait counts past them).
#include <type_traits>

#include "common.h"
#include "gemm_common.h"
#include "launch.h"

namespace qmoe {

namespace {

constexpr int kRTM = 128;  // rows per tile
constexpr bool kRPF = true;  // read the next k-slice's operands ahead

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2_sum(uint32_t v, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, v),
                                         __builtin_bit_cast(bf16x2_t, 0x3F803F80u), acc, false);
}

}  // namespace

// Wave grid: WM waves along the tile's rows times 4 / WM along its columns; each wave holds
// NB 16-row weight slices against its 128 / WM rows. More rows per wave share each decoded
// weight among more MFMAs (the decode is the kernel's main VALU cost): fc1 (SwiGLU or a
// plain activation) takes 1 x 4 waves of 128 rows x 4 slices; fc2 2 x 2 waves of 64 rows
// x 6 slices, where the registers also hold the activation load offsets (measured on c3
// T=4096: fc2 1% faster so, the plain-activation linear layer 6% slower). fc2 given the
// row sums of h (XS: fc1's partial sums, in the forward) takes the 1 x 4 shape too, which
// then fits its registers (without the sums it spills inside the K loop): c3 fc2 4% faster.
template <int BITS, int MODE, bool XS = false>
struct RowsShape {
  static constexpr bool kTwo = (MODE == kModeSwiglu);
  static constexpr bool kFc2Wide = MODE == kModeFc2 && !XS;
  static constexpr int WM = kFc2Wide ? 2 : 1;
  static constexpr int NB = kFc2Wide ? 6 : 4;
  static constexpr bool XREG = WM == 2;                 // activation offsets in registers
  // explicit instruction order inside a k-slice (each MFMA followed by two VALU
  // instructions, operand reads first): measured neutral to negative, left off
  static constexpr bool SGB = false;
  static constexpr int NS = kTwo ? 2 : 1;
  static constexpr int NBS = NB / NS;                   // slices per stream
  static constexpr int SSK = BITS == 4 ? 128 : 64;      // K per step
  static constexpr int GPR = SSK / 8;                   // 16-byte granules per activation row
  static constexpr int NDMA = kRTM * GPR / 64 / 4;      // LDS-destination loads per wave per step
  static constexpr int WNC = 4 / WM;                    // waves along the columns
  static constexpr int MT = kRTM / 16 / WM;             // 16-row MFMA tiles per wave
  static constexpr int BCOLS = WNC * NBS * 16;          // output columns per workgroup
  static constexpr int STAGE = kRTM * SSK;              // bf16 elements per LDS stage
};

// One wave's share of a workgroup; WN (the wave's column position) is a template argument
// so that every choice that depends on it is made at compile time.
template <int BITS, typename ST, int MODE, int WN, bool PK, bool XS>
__device__ __forceinline__ void rows_body(const GemmArgs& g, int tile, int cblk, int wave,
                                          uint16_t* xs0, uint16_t* xs1, float* rowsum,
                                          uint32_t* rtab) {
  using S = RowsShape<BITS, MODE, XS>;
  constexpr float kCorr = BITS == 4 ? 136.0f : 128.0f;  // offset + zero point
  constexpr bool kTwo = S::kTwo;
  constexpr int NS = S::NS;
  constexpr int NBS = S::NBS;
  constexpr int SSK = S::SSK;
  constexpr int MPS = SSK / 32;                  // MFMA k-slices per step
  constexpr int GPR = S::GPR;
  constexpr int NDMA = S::NDMA;
  constexpr int BCOLS = S::BCOLS;
  constexpr int MT = S::MT;
  constexpr int kRWM = S::WM;
  constexpr int kRNB = S::NB;
  constexpr bool kRXREG = S::XREG;
  constexpr int kRSGB = S::SGB ? 1 : 0;
  constexpr int wn = WN;
  static_assert(MT == 2 * S::WNC, "each wave sums the rows of two MFMA tiles");

  const int2 tv = gemm_tile(g, tile);
  const int e = tv.x;
  const int valid = tv.y;
  const int64_t row0 = static_cast<int64_t>(tile) * kRTM;

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int n = lane % 16, kq = lane / 16;
  const int wm = wave % kRWM;
  const int col0 = cblk * BCOLS;
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

  // ---- weights: slice b of this wave is stream b / NBS, column group b % NBS. Each slice
  // has its own descriptor (scalar registers) based at the slice's first stack row, so all
  // slices share one lane offset. No clamping: rows past the stack fall outside the
  // descriptor and read zeros, and columns past ncols are never stored. Lane (n, kq) reads
  // the 16 bytes at 16 kq of the step's row segment: k = 32 kq .. +32 (4-bit) or
  // 16 kq .. +16 (8-bit), dword j (4-bit) or dword pair j (8-bit) feeding k-slice j. ----
  // Tiled layout (PK): the slice is one contiguous sequence of 1 KB tiles, one per step,
  // lane l reading bytes 16 l of each; a block past the stream reads zeros.
  rsrc_t wres[kRNB];
  const int lstep = (kTwo && g.fusion == 1) ? 2 : 1;  // stack rows between neighbouring columns
#pragma unroll
  for (int b = 0; b < kRNB; ++b) {
    const int st = b / NBS;
    const int nr = stream_rows(st);
    const int c0 = col0 + wn * NBS * 16 + (b % NBS) * 16;  // column of lane n = 0
    if (PK) {
      const int ns = (kTwo && g.fusion != 0) ? 2 : 1, si = (kTwo && g.fusion != 0) ? st : 0;
      const int rb = c0 / 16;
      const int64_t tile0 = ((static_cast<int64_t>(e) * ns + si) * g.nbk + rb) * g.kt;
      wres[b] = make_rsrc(stream_w(st) + tile0 * 1024,
                          rb < g.nbk ? static_cast<uint32_t>(g.kt) * 1024u : 0u);
    } else {
      const int r0 = local_row(st, c0);
      const int64_t left = static_cast<int64_t>(max(nr - r0, 0)) * row_bytes;
      wres[b] = make_rsrc(stream_w(st) + (static_cast<int64_t>(e) * nr + r0) * row_bytes,
                          static_cast<uint32_t>(left));
    }
  }
  // rows layout: the lane offset (range-checked) holds the row, the scalar offset the
  // step along it; tiled: the lane offset holds both (tiles past K read zeros)
  const uint32_t wlane = PK ? 16u * lane : static_cast<uint32_t>(lstep * n) * row_bytes + 16u * kq;
  auto wload = [&](int s, u32x4 (&w)[kRNB]) {
    const uint32_t so = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(s * SSK) * BITS / 8);
#pragma unroll
    for (int b = 0; b < kRNB; ++b)
      w[b] = PK ? buf_load16(wres[b], wlane + static_cast<uint32_t>(s) * 1024u)
                : buf_load16s(wres[b], wlane, so);
  };
  // stack row of this lane's column of slice b, clamped into the stack (epilogue reads)
  auto slice_row = [&](int b) {
    return local_row(b / NBS, min(col0 + wn * NBS * 16 + (b % NBS) * 16 + n, g.ncols - 1));
  };

  // ---- activations: row-major stages; load i = wave + 4 t of a step fills slots
  // 64 i .. 64 i + 63 ----
  auto key = [](int r) { return GPR == 16 ? (r & 15) : ((r >> 1) & 7); };
  const rsrc_t xres = make_rsrc(g.a, static_cast<uint32_t>(g.a_rows * K * 2));
  auto granule = [&](int t) {  // logical granule of load t of this lane
    const int p = (wave + 4 * t) * 64 + lane;
    return (p % GPR) ^ key(p / GPR);
  };
  // the same for every load t: 4t * 64 / GPR rows later is a multiple of the key's period
  const int gq = granule(0);
  // the tile's rows, formed once by threads 0..127 (one division per row): the byte offset
  // of the row of a that feeds each (kOutOfRange for padding rows: they land as zeros) and,
  // with the tokens' row sums, each row's correction (rows past the valid ones keep 0)
  if (tid < kRTM) {
    uint32_t off = kOutOfRange;
    float corr = 0.f;
    if (tid < valid) {
      const int64_t src = (MODE == kModeFc2) ? row0 + tid : gemm_src_row(g, row0 + tid);
      off = static_cast<uint32_t>(src * K * 2);
      if constexpr (XS) corr = -kCorr * g.xsum[src];
    }
    rtab[tid] = off;
    if constexpr (XS) rowsum[tid] = corr;
  }
  __syncthreads();
  // load t's offset: row (wave + 4t) * 64 / GPR + lane / GPR of the tile, granule gq; in
  // registers where they fit, else read from the row table at each load
  auto row_off = [&](int t) -> uint32_t {
    // a padding row's kOutOfRange plus the granule (and the step's scalar offset) stays
    // past every buffer, so it still reads zeros
    return rtab[((wave + 4 * t) * 64 + lane) / GPR] + 16u * static_cast<uint32_t>(gq);
  };
  uint32_t xoffs_reg[kRXREG ? NDMA : 1];
  if constexpr (kRXREG) {
#pragma unroll
    for (int t = 0; t < NDMA; ++t) xoffs_reg[t] = row_off(t);
  }
  auto xoff = [&](int t) -> uint32_t {
    if constexpr (kRXREG) return xoffs_reg[t];
    else return row_off(t);
  };
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
    // the step-end wait counts the weight loads issued after these: none may move above
    __builtin_amdgcn_sched_barrier(0);
  };

  // operand reads: row r = wm*64 + mt*16 + n has key(r) = key(n); granule q = 4 kq + j
  // (4-bit rows layout) or 2 kq + j (8-bit rows layout), j in the lowest bit(s) of q, or
  // q = 4 j + kq (tiled layout, k-slice j = k [32j, 32j + 32)), j above the bits of kq; in
  // each case the slot of k-slice j is that of k-slice 0 with j XOR-ed in; mt adds 16 rows.
  const int q0 = PK ? kq : (BITS == 4 ? 4 : 2) * kq;
  const uint32_t abase = static_cast<uint32_t>(((wm * MT * 16 + n) * GPR + (q0 ^ key(n))) * 16);
  auto aread = [&](const uint16_t* stage, int j, u32x4 (&xa)[MT]) {
    const uint32_t aj = abase ^ static_cast<uint32_t>((PK ? 64 : 16) * j);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      xa[mt] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(stage) + aj +
                                               mt * 16 * GPR * 16);
  };

  floatx4 acc[MT][kRNB];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int b = 0; b < kRNB; ++b) acc[mt][b] = floatx4{0.f, 0.f, 0.f, 0.f};
  float rs[2] = {0.f, 0.f};  // partial row sums of slices 2*wn, 2*wn+1 of this wave's rows

  auto decode = [&](const u32x4& wv, int j) -> bf16x8 {
    if constexpr (BITS == 4) {
      return decode4(wv[j]);
    } else {
      const u32x2 w2 = {wv[2 * j], wv[2 * j + 1]};
      return decode8(w2);
    }
  };
  // Eight row tiles a wave (SwiGLU): each activation fragment is read again in place, for
  // the next k-slice, right after its MFMAs have been issued, and the slice's four weights
  // are decoded before its MFMAs. The fragments of the next k-slice then need no registers
  // of their own, which keeps the wave within its 256 registers without spilling.
  auto compute_inplace = [&](const uint16_t* stage, const u32x4 (&w)[kRNB]) {
    u32x4 xa[MT];
    aread(stage, 0, xa);
#pragma unroll
    for (int j = 0; j < MPS; ++j) {
      const uint32_t an = abase ^ static_cast<uint32_t>((PK ? 64 : 16) * (j + 1));
      bf16x8 bw[kRNB];
#pragma unroll
      for (int b = 0; b < kRNB; ++b) bw[b] = decode(w[b], j);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        u32x4 xv = xa[mt];
        if (BITS == 4 && !PK) xv = order_for_nibbles(xv);
        if (!XS && (mt == 2 * wn || mt == 2 * wn + 1)) {
          // row sums of slices 2 wn, 2 wn + 1
          const int h = mt - 2 * wn;
          rs[h] = dot2_sum(xv[3], dot2_sum(xv[2], dot2_sum(xv[1], dot2_sum(xv[0], rs[h]))));
        }
#pragma unroll
        for (int b = 0; b < kRNB; ++b)
          acc[mt][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xv),
                                                               bw[b], acc[mt][b], 0, 0, 0);
        if (j + 1 < MPS)
          xa[mt] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(stage) + an +
                                                   mt * 16 * GPR * 16);
      }
    }
  };
  auto compute = [&](const uint16_t* stage, const u32x4 (&w)[kRNB]) {
    if constexpr (MT == 8) {
      compute_inplace(stage, w);
      return;
    }
    u32x4 xa[MT];
    [[maybe_unused]] u32x4 xn[MT];
    aread(stage, 0, xa);
#pragma unroll
    for (int j = 0; j < MPS; ++j) {
      if constexpr (kRPF) {
        if (j + 1 < MPS) aread(stage, j + 1, xn);  // next k-slice's operands, in flight
      } else {
        if (j > 0) aread(stage, j, xa);
      }
      if (BITS == 4 && !PK) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) xa[mt] = order_for_nibbles(xa[mt]);
      }
      // row sums of slices 2 wn, 2 wn + 1
      if constexpr (!XS) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const u32x4 v = xa[2 * wn + h];
          rs[h] = dot2_sum(v[3], dot2_sum(v[2], dot2_sum(v[1], dot2_sum(v[0], rs[h]))));
        }
      }
      bf16x8 bw = decode(w[0], j);
#pragma unroll
      for (int b = 0; b < kRNB; ++b) {
        // the next slice's decode overlaps this slice's MFMAs
        bf16x8 bn = bw;
        if (b + 1 < kRNB) bn = decode(w[b + 1], j);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          acc[mt][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xa[mt]),
                                                               bw, acc[mt][b], 0, 0, 0);
        bw = bn;
      }
      if constexpr (kRPF) {
        if (j + 1 < MPS) {
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) xa[mt] = xn[mt];
        }
      }
      if constexpr (kRSGB == 1) {
        __builtin_amdgcn_sched_group_barrier(0x100, MT, 0);  // LDS reads
#pragma unroll
        for (int i = 0; i < MT * kRNB; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
          __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);  // VALU
        }
      }
      // one k-slice at a time: operands and decodes hoisted from later slices would spill
      if (MT > 4 || kRSGB) __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- pipeline ----
  // s_waitcnt immediate: vmcnt = the weight loads issued after a step's activation loads,
  // expcnt and lgkmcnt left open
  static_assert(kRNB < 64, "vmcnt holds 6 bits");
  constexpr int kWaitX = (kRNB & 15) | ((kRNB >> 4) << 14) | (7 << 4) | (15 << 8);
  u32x4 wa[kRNB], wb[kRNB];
  xload(0, xs0);
  wload(0, wa);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  // whole pairs of steps (even steps read xs0 and wa, odd steps xs1 and wb), then an odd
  // last step
  const int npair = nss / 2;
  for (int pi = 0; pi < npair; ++pi) {
    const int s = 2 * pi;
    xload(s + 1, xs1);
    wload(s + 1, wb);
    compute(xs0, wa);
    __builtin_amdgcn_s_waitcnt(kWaitX);
    __syncthreads();
    if (s + 2 < nss) {
      xload(s + 2, xs0);
      wload(s + 2, wa);
    }
    compute(xs1, wb);
    __builtin_amdgcn_s_waitcnt(kWaitX);
    __syncthreads();
  }
  if (nss & 1) {
    compute(xs0, wa);
    __builtin_amdgcn_s_waitcnt(0);
  }

  // ---- row sums: reduce over the four k lane groups, meet in LDS ----
  if constexpr (!XS) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float v = rs[h];
      v += __shfl_xor(v, 16);
      v += __shfl_xor(v, 32);
      if (kq == 0) rowsum[wm * MT * 16 + (2 * wn + h) * 16 + n] = -kCorr * v;
    }
    __syncthreads();
  }

  // ---- epilogue: scale per output row, bias, activation; the outputs pass through the
  // (now free) activation stages so that they leave in 16-byte row segments ----
  float bias[kRNB], svr[kRNB];
#pragma unroll
  for (int b = 0; b < kRNB; ++b) {
    const int st = b / NBS;
    const int64_t idx = static_cast<int64_t>(e) * stream_rows(st) + slice_row(b);
    const uint16_t* bp = static_cast<const uint16_t*>(stream_b(st));
    bias[b] = bp ? bf16_to_f32(bp[idx]) : 0.f;
    svr[b] = scale_value<ST>(static_cast<const ST*>(stream_s(st))[idx]);
  }
  if constexpr (BITS != 4 || MODE == kModeFc2) {
    // direct stores: 8-bit codes take 64-k stages (16 KB), too small to stage the outputs;
    // fc2's fp32 rows would take two passes, which measured 2% slower on c3 than storing
    // each 4-byte value
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = wm * MT * 16 + mt * 16 + 4 * kq + i;
        const int64_t r = row0 + m;
        const float rc = rowsum[m];
        const float rs = (MODE != kModeFc2 && m < valid) ? gemm_row_scale(g, r) : 1.f;
#pragma unroll
        for (int cb = 0; cb < NBS; ++cb) {
          const int col = col0 + wn * NBS * 16 + cb * 16 + n;
          if (col >= g.ncols) continue;
          float z[NS];
#pragma unroll
          for (int st = 0; st < NS; ++st) {
            const int b = st * NBS + cb;
            z[st] = svr[b] * (acc[mt][b][i] + rc) * rs + bias[b];
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
    return;
  } else {
    // staging (fc1 and the linear layer: bf16 h): 128 output columns per stage, 128 rows of
    // 256 bytes; the 16-byte chunk c of row r sits at slot c ^ (r mod 16), so the 16 lanes of
    // one MFMA row and the four rows a wave writes at once fall in distinct banks
    constexpr int kChunks = 16;                          // 16-byte chunks per staged row
    constexpr int kStages = (BCOLS + 127) / 128;
    constexpr int kRowBytes = 256;
    static_assert(kRTM * kRowBytes == S::STAGE * 2, "the tile's rows fill a stage");
    static_assert(kStages <= 2 && kRWM == 1, "two stages, one wave row");
    auto staged = [&](int r, int c) -> uint16_t* {
      char* st = reinterpret_cast<char*>(c < 128 ? xs0 : xs1);
      const int cc = c & 127;
      return reinterpret_cast<uint16_t*>(st + r * kRowBytes + (((cc / 8) ^ (r & (kChunks - 1))) * 16) +
                                         (cc % 8) * 2);
    };
    // 16-byte stores need a 16-byte aligned output (rows are: ncols is a multiple of 32)
    const bool vec_out = (reinterpret_cast<uintptr_t>(g.out) & 15) == 0;
    // every wave is past its last read of the stages
    __syncthreads();
    // the outputs into the stages; instantiated for the SwiGLU clamp and the routing weight on
    // the input, each compiled in only where the launch has it (one uniform branch)
    const float na = swiglu_na(g.alpha);
    auto emit = [&](auto clamp_t, auto roww_t) {
      constexpr bool kClamp = decltype(clamp_t)::value, kRoww = decltype(roww_t)::value;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = mt * 16 + 4 * kq + i;
          const float rc = rowsum[m];
          // fc1 with the routing weight on the input: the row's weight scales its sums
          float rs = 1.f;
          if constexpr (kRoww) rs = m < valid ? gemm_row_scale(g, row0 + m) : 1.f;
#pragma unroll
          for (int cb = 0; cb < NBS; ++cb) {
            const int cl = wn * NBS * 16 + cb * 16 + n;  // column inside the workgroup
            float z[NS];
#pragma unroll
            for (int st = 0; st < NS; ++st) {
              const int b = st * NBS + cb;
              z[st] = kRoww ? svr[b] * (acc[mt][b][i] + rc) * rs + bias[b]
                            : fmaf(svr[b], acc[mt][b][i] + rc, bias[b]);
            }
            float hv = 0.f;
            if (m < valid)
              hv = (MODE == kModeSwiglu) ? swiglu_k<kClamp>(z[0], z[NS - 1], na, g.beta, g.limit)
                                         : plain_act(z[0], g.act);
            *staged(m, cl) = f32_to_bf16(hv);
          }
        }
      }
    };
    if constexpr (MODE == kModeSwiglu) {
      const bool clamp = g.limit < INFINITY;
      if (g.row_w) {
        if (clamp) emit(std::true_type{}, std::true_type{});
        else emit(std::false_type{}, std::true_type{});
      } else {
        if (clamp) emit(std::true_type{}, std::false_type{});
        else emit(std::false_type{}, std::false_type{});
      }
    } else {
      emit(std::false_type{}, std::true_type{});  // plain activations: one instance
    }
    __syncthreads();
    if (g.hpart) {
      // each row's sum over this workgroup's columns, of the bf16 values just staged (the
      // row sums fc2 takes its zero point's correction from): two threads a row, one per
      // half of its chunks, in every stage; padding rows sum their staged zeros
      const int m = tid / 2, half = tid % 2;
      float sum = 0.f;
#pragma unroll
      for (int stg = 0; stg < kStages; ++stg) {
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const int ch = half * 8 + c;
          const int cl = stg * 128 + ch * 8;
          if (cl >= BCOLS || col0 + cl >= g.ncols) continue;
          const u32x4 v = *reinterpret_cast<const u32x4*>(
              reinterpret_cast<const char*>(stg == 0 ? xs0 : xs1) + m * kRowBytes +
              ((ch ^ (m & (kChunks - 1))) * 16));
#pragma unroll
          for (int w = 0; w < 4; ++w)
            sum += __uint_as_float(v[w] << 16) + __uint_as_float(v[w] & 0xFFFF0000u);
        }
      }
      sum += __shfl_xor(sum, 1);
      if (half == 0) g.hpart[(row0 + m) * g.hpart_stride + cblk] = sum;
    }
    // copies out: chunk q is stage q / (128 * 16), row (q / 16) % 128, chunk q % 16; every
    // row of the tile (padding rows as the zeros staged for them), real rows only for the
    // linear layer
    constexpr int kTot = kRTM * kChunks * kStages;
#pragma unroll
    for (int u = 0; u < kTot / 256; ++u) {
      const int q = tid + 256 * u;
      const int stg = q / (kRTM * kChunks);
      const int m = (q / kChunks) % kRTM, ch = q % kChunks;
      const int cl = stg * 128 + ch * 8;
      const int col = col0 + cl;
      if (cl >= BCOLS || col >= g.ncols) continue;
      if (m >= valid && g.linear) continue;
      const char* src = reinterpret_cast<const char*>(stg == 0 ? xs0 : xs1) + m * kRowBytes +
                        ((ch ^ (m & (kChunks - 1))) * 16);
      const u32x4 v = *reinterpret_cast<const u32x4*>(src);
      uint16_t* dst = static_cast<uint16_t*>(g.out) + (row0 + m) * g.ncols + col;
      if (vec_out) {
        *reinterpret_cast<u32x4*>(dst) = v;
      } else {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          dst[2 * w] = static_cast<uint16_t>(v[w]);
          dst[2 * w + 1] = static_cast<uint16_t>(v[w] >> 16);
        }
      }
    }
  }
}

template <int BITS, typename ST, int MODE, bool PK, bool XS>
__global__ __launch_bounds__(256, 2) void gemm_bf16_prefill_rows_kernel(GemmArgs g) {
  using S = RowsShape<BITS, MODE, XS>;
  // two stages as two arrays, so that the compiler can tell the stage being read from the
  // stage being filled and does not wait for the fill before reading
  __shared__ __attribute__((aligned(16))) uint16_t xs0[S::STAGE];
  __shared__ __attribute__((aligned(16))) uint16_t xs1[S::STAGE];
  __shared__ float rowsum[kRTM];
  __shared__ uint32_t rtab[kRTM];

  int tile, cblk;
  if (!xcd_item(gemm_tile_count(g), (g.ncols + S::BCOLS - 1) / S::BCOLS, tile, cblk)) return;
  // the wave index is uniform; saying so keeps LDS bases and slice choices in scalars
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  switch (wave / S::WM) {
    case 0: rows_body<BITS, ST, MODE, 0, PK, XS>(g, tile, cblk, wave, xs0, xs1, rowsum, rtab); break;
    case 1: rows_body<BITS, ST, MODE, 1, PK, XS>(g, tile, cblk, wave, xs0, xs1, rowsum, rtab); break;
    case 2: if constexpr (S::WNC > 2) rows_body<BITS, ST, MODE, 2, PK, XS>(g, tile, cblk, wave, xs0, xs1, rowsum, rtab); break;
    default: if constexpr (S::WNC > 3) rows_body<BITS, ST, MODE, 3, PK, XS>(g, tile, cblk, wave, xs0, xs1, rowsum, rtab); break;
  }
}

template <int BITS, typename ST, int MODE>
static hipError_t launch_rows_mode(const GemmArgs& g, int64_t max_tiles, hipStream_t s) {
  const int bcols = RowsShape<BITS, MODE>::BCOLS;
  dim3 grid(xcd_grid((g.ncols + bcols - 1) / bcols, max_tiles)), block(256);
  // the forward's row sums (tiled layout): fc1 takes the tokens' sums of x, fc2 (4-bit codes)
  // those of h, formed from fc1's partial sums (only 4-bit fc1 stages its outputs and writes
  // them)
  if constexpr (MODE != kModeFc2 || BITS == 4) {
    if (g.packed && g.xsum) {
      constexpr int xbcols = RowsShape<BITS, MODE, true>::BCOLS;
      dim3 xgrid(xcd_grid((g.ncols + xbcols - 1) / xbcols, max_tiles));
      launch_gemm_kernel(gemm_bf16_prefill_rows_kernel<BITS, ST, MODE, true, true>, xgrid, block, 0, s, g);
      return hipGetLastError();
    }
  }
  if (g.packed)
    launch_gemm_kernel(gemm_bf16_prefill_rows_kernel<BITS, ST, MODE, true, false>, grid, block, 0, s, g);
  else
    launch_gemm_kernel(gemm_bf16_prefill_rows_kernel<BITS, ST, MODE, false, false>, grid, block, 0, s, g);
  return hipGetLastError();
}

template <int BITS, typename ST>
static hipError_t launch_rows_t(const GemmArgs& g, int mode, int64_t max_tiles, hipStream_t s) {
  if (mode == kModeSwiglu) return launch_rows_mode<BITS, ST, kModeSwiglu>(g, max_tiles, s);
  if (mode == kModePlainAct) return launch_rows_mode<BITS, ST, kModePlainAct>(g, max_tiles, s);
  return launch_rows_mode<BITS, ST, kModeFc2>(g, max_tiles, s);
}

int prefill_rows_fc1_cols(int mode) {
  return mode == kModeSwiglu ? RowsShape<4, kModeSwiglu, true>::BCOLS
                             : RowsShape<4, kModePlainAct, true>::BCOLS;
}

hipError_t launch_gemm_bf16_prefill_rows(const GemmArgs& g, int mode, int bits, bool scale_bf16,
                                         int64_t max_tiles, hipStream_t s) {
  if (max_tiles <= 0) return hipSuccess;
  if (bits == 4)
    return scale_bf16 ? launch_rows_t<4, uint16_t>(g, mode, max_tiles, s)
                      : launch_rows_t<4, float>(g, mode, max_tiles, s);
  return scale_bf16 ? launch_rows_t<8, uint16_t>(g, mode, max_tiles, s)
                    : launch_rows_t<8, float>(g, mode, max_tiles, s);
}

}  // namespace qmoe
