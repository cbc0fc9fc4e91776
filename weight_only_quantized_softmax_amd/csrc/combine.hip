// Weighted combine of the per-assignment expert outputs.
//
// CLIKA "MoE" page: a token's output is the routing-weighted sum of its selected experts'
// outputs.
// ClikaRT "QMoEWoQ" page, forward: an optional shared_output folds into the same
// epilogue and the result takes the dtype of x.
//
// The coefficient of slot j is its routing weight, or 1 where the weight went to the expert's
// input (CLIKA "MoE" page, apply_router_weight_on_input), times the expert output scale
// (expert_output_scale).
// Each output element is produced by exactly one thread as a gather of its k rows of y,
// summed in fp32 in slot order and rounded once; no atomics, so the result is
// bit-reproducible.
#include "common.h"
#include "launch.h"

namespace qmoe {

template <typename TO, int KMAX>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y,
                                                      const int32_t* __restrict__ assign_pos,
                                                      const float* __restrict__ topk_w,
                                                      const TO* __restrict__ shared,
                                                      TO* __restrict__ out, int T, int H, int k,
                                                      CombineOpts c) {
  for (int t = blockIdx.y; t < T; t += gridDim.y) {
  const int64_t base = static_cast<int64_t>(t) * k;
  int64_t rows[KMAX];
  float w[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    rows[j] = j < k ? static_cast<int64_t>(assign_pos[base + j]) * H : 0;
    w[j] = j < k ? (c.weights ? topk_w[base + j] : 1.f) * c.scale : 0.f;
  }
  const int H4 = (H % 4 == 0) ? H / 4 : 0;  // float4 rows need H % 4 == 0
  for (int c4 = blockIdx.x * blockDim.x + threadIdx.x; c4 < H4; c4 += gridDim.x * blockDim.x) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      if (j < k) {
        const float4 v = *reinterpret_cast<const float4*>(y + rows[j] + 4 * c4);
        acc.x += w[j] * v.x;
        acc.y += w[j] * v.y;
        acc.z += w[j] * v.z;
        acc.w += w[j] * v.w;
      }
    }
    const int64_t o = static_cast<int64_t>(t) * H + 4 * c4;
    if (shared) {
      acc.x += load_elem(shared, o + 0);
      acc.y += load_elem(shared, o + 1);
      acc.z += load_elem(shared, o + 2);
      acc.w += load_elem(shared, o + 3);
    }
    store_elem(out, o + 0, acc.x);
    store_elem(out, o + 1, acc.y);
    store_elem(out, o + 2, acc.z);
    store_elem(out, o + 3, acc.w);
  }
  // columns past the last multiple of 4
  for (int c = 4 * H4 + blockIdx.x * blockDim.x + threadIdx.x; c < H; c += gridDim.x * blockDim.x) {
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
      if (j < k) acc += w[j] * y[rows[j] + c];
    const int64_t o = static_cast<int64_t>(t) * H + c;
    if (shared) acc += load_elem(shared, o);
    store_elem(out, o, acc);
  }
  }
}

template <typename TO>
static hipError_t launch_combine_t(const float* y, const int32_t* pos, const float* w,
                                   const TO* shared, TO* out, int T, int H, int k,
                                   const CombineOpts& c, hipStream_t s) {
  const int threads = 256;
  const int gx = max(1, min((H / 4 + threads - 1) / threads, 8));
  dim3 grid(gx, min(T, 65535)), block(threads);
  if (k <= 2)
    combine_kernel<TO, 2><<<grid, block, 0, s>>>(y, pos, w, shared, out, T, H, k, c);
  else if (k <= 4)
    combine_kernel<TO, 4><<<grid, block, 0, s>>>(y, pos, w, shared, out, T, H, k, c);
  else if (k <= 8)
    combine_kernel<TO, 8><<<grid, block, 0, s>>>(y, pos, w, shared, out, T, H, k, c);
  else if (k <= 16)
    combine_kernel<TO, 16><<<grid, block, 0, s>>>(y, pos, w, shared, out, T, H, k, c);
  else
    combine_kernel<TO, 32><<<grid, block, 0, s>>>(y, pos, w, shared, out, T, H, k, c);
  return hipGetLastError();
}

hipError_t launch_combine(const float* y, const int32_t* assign_pos, const float* w,
                          const void* shared, void* out, bool bf16, int T, int H, int k,
                          const CombineOpts& c, hipStream_t s) {
  if (bf16)
    return launch_combine_t(y, assign_pos, w, static_cast<const uint16_t*>(shared),
                            static_cast<uint16_t*>(out), T, H, k, c, s);
  return launch_combine_t(y, assign_pos, w, static_cast<const float*>(shared),
                          static_cast<float*>(out), T, H, k, c, s);
}

}  // namespace qmoe
