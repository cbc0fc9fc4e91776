// Helpers shared by the bf16 grouped dequant GEMM kernels: raw buffer access, nibble and
// byte decode to bfloat16, the cross-lane transpose and scale conversion.
#pragma once

#include "common.h"

namespace qmoe {

constexpr int kM = 16;  // rows of a decode tile
constexpr int kRowPad = 8;  // bf16 elements of padding per LDS row (keeps 16 rows on distinct banks)

// Raw buffer access: a descriptor (base, byte size) in scalar registers and a 32-bit byte
// offset per lane; reads at or past the size return zeros.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kBufferWord3 = 0x00020000;
constexpr uint32_t kOutOfRange = 0x80000000u;  // an offset past every buffer: reads zeros

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), kBufferWord3);
}
__device__ __forceinline__ u32x4 buf_load16(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
// A weight stream read once per launch, whole lines at a time (the tiled layout): the
// nontemporal policy (nt) lets the lines pass through the caches without displacing what
// is reused (activations, scales). A plain read of a few hundred MB runs about 8% faster
// on gfx950 with it; a stream that reads half a line now and the other half later must not
// use it (the line is gone by then).
__device__ __forceinline__ u32x4 buf_load16_stream(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2));
}
// with a wave-uniform scalar offset added to the lane offset (the range check covers the
// lane offset)
__device__ __forceinline__ u32x4 buf_load16s(rsrc_t r, uint32_t off, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, soff, 0));
}
// 16 bytes per lane from the buffer straight into LDS: lane i's bytes land at
// lds + 16 i (lds must be wave-uniform); out-of-range lanes write zeros
__device__ __forceinline__ void buf_load16_lds(rsrc_t r, void* lds, uint32_t off, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, off,
                                           soff, 0, 0);
}
__device__ __forceinline__ u32x2 buf_load8(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}
__device__ __forceinline__ uint32_t buf_load4(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
__device__ __forceinline__ uint16_t buf_load2(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint16_t, __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0));
}

// s_waitcnt with vmcnt = N, expcnt and lgkmcnt left open.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt holds 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// The same with vmcnt = BASE + i * STEP for a wave-uniform i in [0, MAXI], each count a
// compile-time immediate.
template <int BASE, int STEP, int MAXI>
__device__ __forceinline__ void wait_vm_sel(int i) {
  if constexpr (MAXI == 0) {
    wait_vm<BASE>();
  } else {
    if (i >= MAXI)
      wait_vm<BASE + MAXI * STEP>();
    else
      wait_vm_sel<BASE, STEP, MAXI - 1>(i);
  }
}

// (v & mask) | magic in one gfx950 three-input bit operation.
__device__ __forceinline__ uint32_t and_or(uint32_t v, uint32_t mask, uint32_t magic) {
  return __builtin_amdgcn_bitop3_b32(v, mask, magic, 0xEA);
}

__device__ __forceinline__ bf16x8 decode4(uint32_t w) {
  // element order of the result: [e0, e4, e1, e5, e2, e6, e3, e7] of the 8 nibbles
  const uint32_t magic = 0x43004300u, mask = 0x000F000Fu;
  u32x4 r;
  r[0] = and_or(w, mask, magic);
  r[1] = and_or(w >> 4, mask, magic);
  r[2] = and_or(w >> 8, mask, magic);
  r[3] = and_or(w >> 12, mask, magic);
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

// Reorders 8 bf16 activations [x0..x7] to [x0, x4, x1, x5, x2, x6, x3, x7] (the 4-bit
// decode order) with four byte permutes.
__device__ __forceinline__ u32x4 order_for_nibbles(u32x4 d) {
  u32x4 o;
  o[0] = __builtin_amdgcn_perm(d[2], d[0], 0x05040100u);
  o[1] = __builtin_amdgcn_perm(d[2], d[0], 0x07060302u);
  o[2] = __builtin_amdgcn_perm(d[3], d[1], 0x05040100u);
  o[3] = __builtin_amdgcn_perm(d[3], d[1], 0x07060302u);
  return o;
}


// Raw scale storage: bf16 scales stay 16-bit until they are used.
template <typename ST>
__device__ __forceinline__ float scale_value(ST v);
template <>
__device__ __forceinline__ float scale_value<uint16_t>(uint16_t v) { return bf16_to_f32(v); }
template <>
__device__ __forceinline__ float scale_value<float>(float v) { return v; }
// E8M0 (MX) scale byte e: 2^(e - 127) as the float whose exponent field is e (the MX
// conversions read only the exponent of their scale operand)
template <>
__device__ __forceinline__ float scale_value<uint8_t>(uint8_t v) {
  return __uint_as_float(static_cast<uint32_t>(v) << 23);
}

// Eight E2M1 (MX FP4) codes of a word, natural order (code i in bits [4i, 4i+4)), times a
// power-of-two scale, to eight bf16: gfx950's scaled conversion takes one byte (two
// codes, the low nibble first) per instruction; the products are exact in bf16.
__device__ __forceinline__ bf16x8 decode_mx(uint32_t w, float scale) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3);
  const u32x4 r = {__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b),
                   __builtin_bit_cast(uint32_t, c), __builtin_bit_cast(uint32_t, d)};
  return __builtin_bit_cast(bf16x8, r);
}

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

// Work order of the 128-row kernels and of the 16/32-row kernel's fc2. The hardware hands
// the workgroups of a 1-D grid to the 8 XCDs in turn (workgroup i to XCD i % 8), and each
// XCD has its own L2. Workgroup i
// takes item (i % 8) * per + i / 8 of the live items (per = ceil(live / 8)), so each XCD
// works through one contiguous run of items. Items run in bands of kBand consecutive tiles
// (one expert's tiles are consecutive): inside a band, column block by column block, the
// band's tiles in turn. The workgroups an XCD runs at once then cover a few tiles times a
// few dozen column blocks, and its L2 serves each weight block to every tile of the band
// and each activation tile to every column block. Correct for any placement; the grid
// must hold at least 8 * per workgroups (the launcher rounds columns x tiles up to a
// multiple of 8).
constexpr int kXcds = 8;
constexpr int kBand = 4;
__device__ __forceinline__ bool xcd_item(int num_tiles, int cblocks, int& tile, int& cb) {
  const int live = num_tiles * cblocks;
  const int per = (live + kXcds - 1) / kXcds;
  const int hw = blockIdx.x;
  const int k = hw / kXcds;
  const int item = (hw % kXcds) * per + k;
  if (k >= per || item >= live) return false;
  const int band = item / (kBand * cblocks);
  const int r = item - band * kBand * cblocks;
  const int bt = min(kBand, num_tiles - band * kBand);  // tiles of this band
  cb = r / bt;
  tile = band * kBand + (r - cb * bt);
  return true;
}
__host__ __device__ constexpr unsigned xcd_grid(int cblocks, int64_t max_tiles) {
  return static_cast<unsigned>((cblocks * max_tiles + kXcds - 1) / kXcds * kXcds);
}

}  // namespace qmoe
