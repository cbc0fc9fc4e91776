// Operands of the fp16 block-scale kernel (gemm_prefill_h16_kernel.h): the activation rows
// in fp16, each lifted by a power of two, and one power of two per weight row for its
// block scales.
//
// graiphic "QMoE" page: a 4-bit weight is (q - 8) * scale with one scale per output row and
// K-block (block_size attribute). |q - 8| <= 8 has at most 3 significant bits and a bf16
// scale 8, so the scaled weight has at most 11 and is exact in fp16 while its exponent
// stays in fp16's range; a bf16 activation (8 significant bits) is exact in fp16 likewise.
// Multiplying a whole row by a power of two changes no significant bit, so each row is
// lifted into fp16's range here, and the kernel divides the lifts out of its fp32 sums
// (again exact). The kernel then takes one fp16 MFMA per product and no per-block work on
// its outputs.
#include "common.h"
#include "launch.h"

namespace qmoe {

namespace {

// The exponent e that brings the magnitude whose bf16 bits (sign cleared) are m into
// [2^top, 2^(top + 1)); 0 for m = 0. A subnormal m counts as 2^-127 (it lands below 2^top,
// which keeps every bit of it).
__device__ __forceinline__ int lift_of(uint32_t m, int top) {
  if (m == 0) return 0;
  const int ef = static_cast<int>(m >> 7);
  return top - (ef == 0 ? -127 : ef - 127);
}

// Top of the lifted activations: the largest magnitude of a row lands in [2^14, 2^15), below
// fp16's largest finite 65504; every element within 2^31 of it keeps all its bits (fp16
// reaches down to 2^-24 in subnormals).
constexpr int kActTop = 14;
// Top of the lifted scales: the largest scale of a weight row lands in [2^12, 2^13); a bf16
// significand there is at most 255 * 2^5 = 8160, and 8 times that (the largest code
// magnitude) is 65280, below 65504. Scales within 2^29 of the row's largest stay exact.
constexpr int kScaleTop = 12;

// One wave per row, two passes: the largest magnitude (bf16 bits order like magnitudes once
// the sign is cleared), then every element times 2^e, rounded to nearest fp16 (exact unless
// it lies more than 2^31 below the row's largest). K % 8 == 0 and 16-byte aligned rows.
__device__ __forceinline__ void row_to_f16(const uint16_t* __restrict__ in,
                                           uint16_t* __restrict__ out,
                                           int32_t* __restrict__ lift, int64_t r, int K,
                                           int lane) {
  const uint4* src = reinterpret_cast<const uint4*>(in + r * K);
  uint4* dst = reinterpret_cast<uint4*>(out + r * K);
  const int C = K / 8;
  uint32_t m = 0;
  for (int c = lane; c < C; c += 64) {
    const uint4 v = src[c];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) m = max(m, max(w[i] & 0x7FFFu, (w[i] >> 16) & 0x7FFFu));
  }
  const int e = lift_of(wave_max_u32(m), kActTop);
  for (int c = lane; c < C; c += 64) {
    const uint4 v = src[c];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const _Float16 lo = static_cast<_Float16>(ldexpf(__uint_as_float(w[i] << 16), e));
      const _Float16 hi = static_cast<_Float16>(ldexpf(__uint_as_float(w[i] & 0xFFFF0000u), e));
      o[i] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, lo)) |
             (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, hi)) << 16);
    }
    dst[c] = make_uint4(o[0], o[1], o[2], o[3]);
  }
  if (lane == 0) lift[r] = e;
}

__global__ __launch_bounds__(256) void rows_to_f16_kernel(const uint16_t* __restrict__ in,
                                                          uint16_t* __restrict__ out,
                                                          int32_t* __restrict__ lift,
                                                          int64_t rows, int K,
                                                          const int32_t* __restrict__ num_tiles,
                                                          int tile_m) {
  const int64_t r = static_cast<int64_t>(blockIdx.x) * 4 + threadIdx.x / 64;
  // rows of tiles past the grouped GEMM's tile count hold nothing
  const int64_t used = num_tiles ? min<int64_t>(rows, int64_t(*num_tiles) * tile_m) : rows;
  if (r >= used) return;
  row_to_f16(in, out, lift, r, K, threadIdx.x % 64);
}

// Eight lanes per weight row (a wave covers eight rows): lane l of a row reads scales l,
// l + 8, ... of its nb bf16 scales; the row's largest magnitude meets over the eight lanes.
__device__ __forceinline__ void scale_lift_rows(const uint16_t* __restrict__ s,
                                                int32_t* __restrict__ lift, int64_t rows,
                                                int nb, int64_t block) {
  const int64_t r = (block * 256 + threadIdx.x) / 8;
  const int l = threadIdx.x % 8;
  uint32_t m = 0;
  if (r < rows) {
    const uint16_t* row = s + r * nb;
    for (int b = l; b < nb; b += 8) m = max(m, static_cast<uint32_t>(row[b]) & 0x7FFFu);
  }
  // lanes 8j .. 8j + 7 share a row: xor shuffles inside each group of eight
#pragma unroll
  for (int o = 1; o < 8; o <<= 1) m = max(m, static_cast<uint32_t>(__shfl_xor(static_cast<int>(m), o)));
  if (r < rows && l == 0) lift[r] = lift_of(m, kScaleTop);
}

// Everything the fp16 path needs before fc1, in one launch: the lifts of up to three
// scale stacks (fc1, fc3, fc2) and x in fp16. Workgroups [0, b0) take stack 0, the next b1
// stack 1, the next b2 stack 2, the rest four rows of x each.
struct PrepArgs {
  const uint16_t* s[3];
  int32_t* slift[3];
  int64_t srows[3];
  int nb[3];
  const uint16_t* x;
  uint16_t* x16;
  int32_t* xlift;
  int64_t T;
  int H;
};

__device__ __forceinline__ int64_t scale_blocks(int64_t rows) { return (rows * 8 + 255) / 256; }

__global__ __launch_bounds__(256) void prep_f16_kernel(PrepArgs a) {
  int64_t b = blockIdx.x;
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const int64_t nbk = a.s[i] ? scale_blocks(a.srows[i]) : 0;
    if (b < nbk) {
      scale_lift_rows(a.s[i], a.slift[i], a.srows[i], a.nb[i], b);
      return;
    }
    b -= nbk;
  }
  const int64_t r = b * 4 + threadIdx.x / 64;
  if (r < a.T) row_to_f16(a.x, a.x16, a.xlift, r, a.H, threadIdx.x % 64);
}

}  // namespace

hipError_t launch_rows_to_f16(const void* in, void* out, int32_t* lift, int64_t rows, int K,
                              const int32_t* num_tiles, int tile_m, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  if (K % 8 != 0) return hipErrorInvalidValue;
  const unsigned blocks = static_cast<unsigned>((rows + 3) / 4);
  rows_to_f16_kernel<<<blocks, 256, 0, s>>>(static_cast<const uint16_t*>(in),
                                            static_cast<uint16_t*>(out), lift, rows, K, num_tiles,
                                            tile_m);
  return hipGetLastError();
}

hipError_t launch_prep_f16(const void* const scales[3], int32_t* const lifts[3],
                           const int64_t rows[3], const int nb[3], const void* x, void* x16,
                           int32_t* xlift, int64_t T, int H, hipStream_t s) {
  if (H % 8 != 0) return hipErrorInvalidValue;
  PrepArgs a{};
  int64_t blocks = (T + 3) / 4;
  for (int i = 0; i < 3; ++i) {
    a.s[i] = static_cast<const uint16_t*>(scales[i]);
    a.slift[i] = lifts[i];
    a.srows[i] = rows[i];
    a.nb[i] = nb[i];
    if (scales[i]) blocks += (rows[i] * 8 + 255) / 256;
  }
  a.x = static_cast<const uint16_t*>(x);
  a.x16 = static_cast<uint16_t*>(x16);
  a.xlift = xlift;
  a.T = T;
  a.H = H;
  if (blocks == 0) return hipSuccess;
  prep_f16_kernel<<<static_cast<unsigned>(blocks), 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace qmoe
