// The int8 activation tier: an activation row is rounded to int8 block by block before the
// dequant GEMM (ClikaRT "QMoEWoQ" page, class description: on the int8 block tier the
// floating-point activation is quantised to int8 per block ahead of the dot product).
//
// Each block of block_size consecutive elements of a row gets the power-of-two scale 2^e,
// e the smallest exponent with max|x| <= 127 * 2^e, and the codes rint(x / 2^e) (ties to
// even), |code| <= 127. The output is code * 2^e in the activation dtype: exact in bf16 and
// fp32 (a code has at most 7 significant bits), so the GEMMs that follow take it as any
// other activation. Every step is an exact float operation, so the codes depend on no
// rounding of the hardware. in and out may be the same buffer: each element is read
// before it is written, by the thread that writes it.
#include "common.h"
#include "launch.h"

namespace qmoe {

namespace {

// The scale exponent of a block whose largest magnitude is a (a >= 0).
__device__ __forceinline__ int block_exponent(float a) {
  if (!(a > 0.f)) return 0;
  int p;
  const float m = frexpf(a, &p);  // a = m * 2^p, m in [0.5, 1)
  // 127 * 2^(p - 7) = (127 / 128) * 2^p: a fits under it when m * 128 <= 127
  return m * 128.f <= 127.f ? p - 7 : p - 6;
}

template <typename TA>
__global__ __launch_bounds__(256) void quantize_blocks_kernel(const TA* in,
                                                              TA* out, int64_t rows,
                                                              int K, int bs, int nb,
                                                              const int32_t* __restrict__ num_tiles,
                                                              int tile_m) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  // rows of tiles past the grouped GEMM's tile count hold nothing
  const int64_t used = num_tiles ? min<int64_t>(rows, int64_t(*num_tiles) * tile_m) : rows;
  if (idx >= used * nb) return;
  const int64_t r = idx / nb;
  const int b = static_cast<int>(idx % nb);
  const int k0 = b * bs, k1 = min(k0 + bs, K);
  const TA* src = in + r * K;
  TA* dst = out + r * K;
  float a = 0.f;
  for (int k = k0; k < k1; ++k) a = fmaxf(a, fabsf(load_elem(src, k)));
  const int e = block_exponent(a);
  for (int k = k0; k < k1; ++k) {
    const float code = rintf(ldexpf(load_elem(src, k), -e));
    store_elem(dst, k, ldexpf(code, e));
  }
}

// The same rounding with 16-byte accesses: each lane holds V = 16 / sizeof(TA) consecutive
// elements, the L = bs / V lanes of a block are adjacent and aligned to L within the wave,
// and they exchange their largest magnitudes with xor shuffles. Each row is laid out as
// Cp = nb * L lane slots, so a block never straddles two rows; slots past the row's C = K / V
// chunks (the ragged last block) load zeros and store nothing. Needs K % V == 0, bs % V == 0
// and 16-byte aligned rows.
template <typename TA, int L>
__global__ __launch_bounds__(256) void quantize_blocks_vec_kernel(
    const TA* in, TA* out, int64_t rows, int K, int C, int Cp,
    const int32_t* __restrict__ num_tiles, int tile_m) {
  constexpr int V = 16 / sizeof(TA);
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t used = num_tiles ? min<int64_t>(rows, int64_t(*num_tiles) * tile_m) : rows;
  const int64_t r = idx / Cp;
  const int c = static_cast<int>(idx - r * Cp);
  const bool live = r < used && c < C;
  uint4 raw = make_uint4(0, 0, 0, 0);
  if (live) raw = *reinterpret_cast<const uint4*>(in + r * K + int64_t(c) * V);
  float v[V];
  if constexpr (sizeof(TA) == 2) {
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  } else {
    v[0] = __uint_as_float(raw.x);
    v[1] = __uint_as_float(raw.y);
    v[2] = __uint_as_float(raw.z);
    v[3] = __uint_as_float(raw.w);
  }
  float a = 0.f;
#pragma unroll
  for (int i = 0; i < V; ++i) a = fmaxf(a, fabsf(v[i]));
#pragma unroll
  for (int o = L / 2; o > 0; o >>= 1) a = fmaxf(a, __shfl_xor(a, o));
  if (!live) return;
  const int e = block_exponent(a);
#pragma unroll
  for (int i = 0; i < V; ++i) v[i] = ldexpf(rintf(ldexpf(v[i], -e)), e);
  uint4 res;
  if constexpr (sizeof(TA) == 2) {
    // code * 2^e has at most 8 significant bits: the top half of the float is the bf16
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = (__float_as_uint(v[2 * i]) >> 16) | (__float_as_uint(v[2 * i + 1]) & 0xFFFF0000u);
    res = make_uint4(w[0], w[1], w[2], w[3]);
  } else {
    res = make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                     __float_as_uint(v[3]));
  }
  *reinterpret_cast<uint4*>(out + r * K + int64_t(c) * V) = res;
}

// The same rounding for bf16 rows, written as the int8 codes and a per-block factor 2^e
// for the int8 dot (the prefill kernel on v_mfma_i32_16x16x64_i8). Each lane holds 8
// consecutive elements (a chunk); the L = bs / 8 lanes of a block are adjacent. Codes go to
// codes[r][K] with the chunks of every 64 consecutive k stored in the order
// 0, 4, 1, 5, 2, 6, 3, 7, so that 16-byte granule q of a 64-group holds the k
// {8q .. 8q+7} and {32+8q .. 32+8q+7}: the k a lane of the matrix instruction takes.
// fac[r][b] = 2^e of block b. Needs K % 64 == 0 and bs in {64, 128}.
template <int L>
__global__ __launch_bounds__(256) void quantize_codes_kernel(
    const uint16_t* in, int8_t* codes, float* fac, int64_t rows, int K, int C, int Cp, int nb,
    const int32_t* __restrict__ num_tiles, int tile_m) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t used = num_tiles ? min<int64_t>(rows, int64_t(*num_tiles) * tile_m) : rows;
  const int64_t r = idx / Cp;
  const int c = static_cast<int>(idx - r * Cp);
  const bool live = r < used && c < C;
  uint4 raw = make_uint4(0, 0, 0, 0);
  if (live) raw = *reinterpret_cast<const uint4*>(in + r * K + int64_t(c) * 8);
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
  float v[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
  float a = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf(v[i]));
#pragma unroll
  for (int o = L / 2; o > 0; o >>= 1) a = fmaxf(a, __shfl_xor(a, o));
  if (!live) return;
  const int e = block_exponent(a);
  uint32_t q[2] = {0u, 0u};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int code = static_cast<int>(rintf(ldexpf(v[i], -e)));
    q[i / 4] |= (static_cast<uint32_t>(code) & 0xFFu) << (8 * (i % 4));
  }
  // chunk c of its 64-group goes to slot 2 * (c % 4) + c / 4
  const int g = c / 8, cc = c % 8;
  const int64_t pos = r * K + int64_t(g) * 64 + 16 * (cc % 4) + 8 * (cc / 4);
  *reinterpret_cast<uint2*>(codes + pos) = make_uint2(q[0], q[1]);
  if (c % L == 0) fac[r * nb + c / L] = ldexpf(1.0f, e);
}

template <typename TA>
hipError_t launch_vec(const TA* in, TA* out, int64_t rows, int K, int bs,
                      const int32_t* num_tiles, int tile_m, hipStream_t s, bool* done) {
  constexpr int V = 16 / sizeof(TA);
  *done = false;
  const bool aligned = (reinterpret_cast<uintptr_t>(in) % 16 == 0) &&
                       (reinterpret_cast<uintptr_t>(out) % 16 == 0);
  if (!aligned || K % V != 0 || bs % V != 0) return hipSuccess;
  const int L = bs / V;
  const int nb = (K + bs - 1) / bs;
  const int C = K / V, Cp = nb * L;
  const int64_t n = rows * Cp;
  const unsigned blocks = static_cast<unsigned>((n + 255) / 256);
  *done = true;
  switch (L) {
#define QMOE_QV(LL)                                                                        \
  case LL:                                                                                 \
    quantize_blocks_vec_kernel<TA, LL><<<blocks, 256, 0, s>>>(in, out, rows, K, C, Cp,     \
                                                              num_tiles, tile_m);          \
    break;
    QMOE_QV(1) QMOE_QV(2) QMOE_QV(4) QMOE_QV(8) QMOE_QV(16) QMOE_QV(32) QMOE_QV(64)
#undef QMOE_QV
    default:
      *done = false;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_codes(const void* in, int8_t* codes, float* fac, int64_t rows, int K,
                                 int bs, const int32_t* num_tiles, int tile_m, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const int L = bs / 8;
  const int nb = (K + bs - 1) / bs;
  const int C = K / 8, Cp = nb * L;
  const int64_t n = rows * Cp;
  const unsigned blocks = static_cast<unsigned>((n + 255) / 256);
  const uint16_t* x = static_cast<const uint16_t*>(in);
  switch (L) {
    case 8:
      quantize_codes_kernel<8><<<blocks, 256, 0, s>>>(x, codes, fac, rows, K, C, Cp, nb, num_tiles, tile_m);
      break;
    case 16:
      quantize_codes_kernel<16><<<blocks, 256, 0, s>>>(x, codes, fac, rows, K, C, Cp, nb, num_tiles, tile_m);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_quantize_blocks(const void* in, void* out, bool bf16, int64_t rows, int K,
                                  int bs, const int32_t* num_tiles, int tile_m, hipStream_t s) {
  const int nb = (K + bs - 1) / bs;
  const int64_t n = rows * nb;
  if (n == 0) return hipSuccess;
  bool done = false;
  const hipError_t ve =
      bf16 ? launch_vec(static_cast<const uint16_t*>(in), static_cast<uint16_t*>(out), rows, K,
                        bs, num_tiles, tile_m, s, &done)
           : launch_vec(static_cast<const float*>(in), static_cast<float*>(out), rows, K, bs,
                        num_tiles, tile_m, s, &done);
  if (done || ve != hipSuccess) return ve;
  const unsigned blocks = static_cast<unsigned>((n + 255) / 256);
  if (bf16)
    quantize_blocks_kernel<<<blocks, 256, 0, s>>>(static_cast<const uint16_t*>(in),
                                                  static_cast<uint16_t*>(out), rows, K, bs, nb,
                                                  num_tiles, tile_m);
  else
    quantize_blocks_kernel<<<blocks, 256, 0, s>>>(static_cast<const float*>(in),
                                                  static_cast<float*>(out), rows, K, bs, nb,
                                                  num_tiles, tile_m);
  return hipGetLastError();
}

}  // namespace qmoe
