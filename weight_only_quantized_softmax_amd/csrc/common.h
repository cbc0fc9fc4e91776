// Device-side helpers shared by the gfx950 kernels of the QMoE library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmoe {

constexpr int kWave = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Nearest-even conversion to bfloat16 (gfx950 converts in hardware).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 b = static_cast<__bf16>(f);
  return __builtin_bit_cast(uint16_t, b);
}

// Element loads by storage type: uint16_t holds bfloat16 bits, float is fp32.
__device__ __forceinline__ float load_elem(const uint16_t* p, int64_t i) { return bf16_to_f32(p[i]); }
__device__ __forceinline__ float load_elem(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ void store_elem(uint16_t* p, int64_t i, float v) { p[i] = f32_to_bf16(v); }
__device__ __forceinline__ void store_elem(float* p, int64_t i, float v) { p[i] = v; }

// ---- wave-wide reductions built from DPP row operations and one swizzle ----
// quad_perm [1,0,3,2] and [2,3,0,1], row_half_mirror, row_mirror combine lanes inside
// a row of 16; ds_swizzle (xor 16) combines the two rows of each half-wave; the two
// half-waves are joined through readlane, so every lane receives the result.
#define QMOE_DPP_QUAD_1032 0xB1
#define QMOE_DPP_QUAD_2301 0x4E
#define QMOE_DPP_ROW_HALF_MIRROR 0x141
#define QMOE_DPP_ROW_MIRROR 0x140
#define QMOE_SWZ_XOR16 0x401F

template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ uint32_t swz_xor16(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_ds_swizzle(static_cast<int>(v), QMOE_SWZ_XOR16));
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp<QMOE_DPP_QUAD_1032>(v));
  v = max(v, dpp<QMOE_DPP_QUAD_2301>(v));
  v = max(v, dpp<QMOE_DPP_ROW_HALF_MIRROR>(v));
  v = max(v, dpp<QMOE_DPP_ROW_MIRROR>(v));
  v = max(v, swz_xor16(v));
  uint32_t lo = __builtin_amdgcn_readlane(v, 0), hi = __builtin_amdgcn_readlane(v, 32);
  return max(lo, hi);
}

__device__ __forceinline__ float wave_sum_f32(float f) {
  uint32_t v = __float_as_uint(f);
  f += __uint_as_float(dpp<QMOE_DPP_QUAD_1032>(v));
  v = __float_as_uint(f);
  f += __uint_as_float(dpp<QMOE_DPP_QUAD_2301>(v));
  v = __float_as_uint(f);
  f += __uint_as_float(dpp<QMOE_DPP_ROW_HALF_MIRROR>(v));
  v = __float_as_uint(f);
  f += __uint_as_float(dpp<QMOE_DPP_ROW_MIRROR>(v));
  v = __float_as_uint(f);
  f += __uint_as_float(swz_xor16(v));
  v = __float_as_uint(f);
  float lo = __uint_as_float(__builtin_amdgcn_readlane(v, 0));
  float hi = __uint_as_float(__builtin_amdgcn_readlane(v, 32));
  return lo + hi;
}

// Sum over the 16 lanes of each DPP row; every lane of the row gets its row's sum.
__device__ __forceinline__ float row16_sum_f32(float f) {
  f += __uint_as_float(dpp<QMOE_DPP_QUAD_1032>(__float_as_uint(f)));
  f += __uint_as_float(dpp<QMOE_DPP_QUAD_2301>(__float_as_uint(f)));
  f += __uint_as_float(dpp<QMOE_DPP_ROW_HALF_MIRROR>(__float_as_uint(f)));
  f += __uint_as_float(dpp<QMOE_DPP_ROW_MIRROR>(__float_as_uint(f)));
  return f;
}

__device__ __forceinline__ uint64_t ballot(bool pred) { return __ballot(pred); }

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// The logistic function 1 / (1 + e^-x) with the hardware reciprocal (v_rcp_f32, about one
// ulp) instead of an IEEE division (a sequence of about nine instructions): an epilogue
// cost per output element, far below the bf16 rounding of h. It never produces NaN: e^-x
// overflows to +inf for very negative x and the reciprocal of +inf is 0.
__device__ __forceinline__ float sigmoid_fast(float x) {
  return __builtin_amdgcn_rcpf(1.0f + __expf(-x));
}

// SwiGLU of the graiphic QMoE attributes: only the gate is clamped from above,
// the up value on both sides; sigmoid written so that it never produces NaN.
__device__ __forceinline__ float swiglu(float g, float u, float alpha, float beta, float limit) {
  g = fminf(g, limit);
  u = fmaxf(-limit, fminf(u, limit));
  float sig = sigmoid_fast(alpha * g);
  return g * sig * (u + beta);
}

// The same SwiGLU for epilogues that prepare its constants once: na = -alpha * log2(e), so
// that the logistic takes one multiply and the hardware exp2 (what __expf computes, with
// alpha folded into its constant), and the clamps compiled in only when there is a limit.
template <bool CLAMP>
__device__ __forceinline__ float swiglu_k(float g, float u, float na, float beta, float limit) {
  if constexpr (CLAMP) {
    g = fminf(g, limit);
    u = fmaxf(-limit, fminf(u, limit));
  }
  const float sig = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(g * na));
  return g * sig * (u + beta);
}
__device__ __forceinline__ float swiglu_na(float alpha) { return -alpha * 1.4426950408889634f; }

// The plain activations by code: 1 identity, 2 relu, 3 silu, 4 gelu z * Phi(z) (Phi the
// standard normal CDF, through erf), 5 gelu's tanh approximation (graiphic "QMoE" page,
// activation_type; CLIKA "MoE" page, gelu_mode).
__device__ __forceinline__ float plain_act(float z, int act) {
  if (act == 2) return z > 0.f ? z : 0.f;                      // relu
  if (act == 3) return z * sigmoid_fast(z);                     // silu
  if (act == 4) return 0.5f * z * (1.0f + erff(z * 0.70710678118654752f));
  if (act == 5) {
    const float u = 0.79788456080286536f * (z + 0.044715f * z * z * z);
    return 0.5f * z * (1.0f + tanhf(u));
  }
  return z;                                                    // identity
}

}  // namespace qmoe
