// The sum of each activation row, once per token, for the zero point's correction of the
// 128-row per-row-scale fc1 kernel; and the row sums of h for its fc2, from the partial sums
// fc1 writes per column block.
//
// graiphic "QMoE" page: a weight is (q - zero point) * scale per output row; the kernels
// decode q as 128 + q (an exact bf16) and take the offset and the zero point out of each
// output through -(128 + z) * sum_k x[k], which depends on the activation row alone. Each
// token's row x[t] is the fc1 input of its k assignments, so its sum is formed here once,
// instead of in every 128-row tile of every column block that reads the row.
#include "common.h"
#include "launch.h"

namespace qmoe {

namespace {

// One wave per row: each lane adds 8 consecutive elements per 16-byte load, stepping by
// the wave's 512 elements, then a scalar tail when K is not a multiple of 8; the lanes'
// sums meet by xor shuffles.
__global__ __launch_bounds__(256) void rowsum_kernel(const uint16_t* __restrict__ x,
                                                     float* __restrict__ out, int64_t rows,
                                                     int K) {
  const int64_t r = static_cast<int64_t>(blockIdx.x) * 4 + threadIdx.x / 64;
  const int lane = threadIdx.x % 64;
  if (r >= rows) return;
  const uint16_t* row = x + r * K;
  const int K8 = K & ~7;
  float acc = 0.f;
  const bool aligned = (reinterpret_cast<uintptr_t>(row) & 15) == 0;
  if (aligned) {
    for (int k = 8 * lane; k < K8; k += 512) {
      const uint4 v = *reinterpret_cast<const uint4*>(row + k);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i)
        acc += __uint_as_float(w[i] << 16) + __uint_as_float(w[i] & 0xFFFF0000u);
    }
    for (int k = K8 + lane; k < K; k += 64) acc += bf16_to_f32(row[k]);
  } else {
    for (int k = lane; k < K; k += 64) acc += bf16_to_f32(row[k]);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
  if (lane == 0) out[r] = acc;
}

// One wave per row: lane l adds values l, l + 64, ... of the row in order, then the lanes'
// sums meet by the fixed DPP tree of wave_sum_f32.
__global__ __launch_bounds__(256) void partsum_kernel(const float* __restrict__ parts,
                                                      float* __restrict__ out, int64_t rows, int n,
                                                      const int32_t* __restrict__ num_tiles,
                                                      int tile_m) {
  const int64_t r = static_cast<int64_t>(blockIdx.x) * 4 + threadIdx.x / 64;
  const int lane = threadIdx.x % 64;
  const int64_t used = min<int64_t>(rows, int64_t(*num_tiles) * tile_m);
  if (r >= used) return;
  const float* row = parts + r * n;
  float acc = 0.f;
  for (int j = lane; j < n; j += 64) acc += row[j];
  const float sum = wave_sum_f32(acc);
  if (lane == 0) out[r] = sum;
}

}  // namespace

hipError_t launch_partsum(const float* parts, float* out, int64_t rows, int n,
                          const int32_t* num_tiles, int tile_m, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const unsigned blocks = static_cast<unsigned>((rows + 3) / 4);
  partsum_kernel<<<blocks, 256, 0, s>>>(parts, out, rows, n, num_tiles, tile_m);
  return hipGetLastError();
}

hipError_t launch_rowsum(const void* x, float* out, int64_t rows, int K, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const unsigned blocks = static_cast<unsigned>((rows + 3) / 4);
  rowsum_kernel<<<blocks, 256, 0, s>>>(static_cast<const uint16_t*>(x), out, rows, K);
  return hipGetLastError();
}

}  // namespace qmoe
