// One-time conversion of a row-major quantized stack [E, N, K*bits/8] into the tiled
// layout that the GEMM kernels stream (tiles of 16 rows by 128 (4-bit) or 64 (8-bit)
// elements of K, 1024 bytes, one 16-byte load per lane). The layout is specified with the
// entry point in qmoe.h; the stack shapes are those of the graiphic "QMoE" page.
//
// One thread per 16-byte lane chunk of a tile: it gathers the chunk's elements from the
// rows of the source stack (bytes read one at a time: a rows-layout K need not keep
// 32-bit alignment) and writes the chunk with one 16-byte store.
#include "common.h"
#include "launch.h"

namespace qmoe {

namespace {

__device__ __forceinline__ uint32_t code_at(const uint8_t* row, int64_t k, int K, int bits) {
  if (k >= K) return 0u;
  if (bits == 8) return row[k];
  const uint32_t b = row[k >> 1];
  return (k & 1) ? (b >> 4) : (b & 15u);
}

}  // namespace

__global__ __launch_bounds__(256) void pack_stack_kernel(const uint8_t* __restrict__ src,
                                                         uint8_t* __restrict__ dst, PackArgs a) {
  const int64_t chunk = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t nchunks = static_cast<int64_t>(a.E) * a.S * a.NB * a.KT * 64;
  if (chunk >= nchunks) return;
  const int l = static_cast<int>(chunk % 64);
  int64_t tile = chunk / 64;
  const int t = static_cast<int>(tile % a.KT);
  tile /= a.KT;
  const int b = static_cast<int>(tile % a.NB);
  tile /= a.NB;
  const int s = static_cast<int>(tile % a.S);
  const int e = static_cast<int>(tile / a.S);
  const int n = l % 16, q = l / 16;
  const int r = 16 * b + n;  // row of the stream
  const int ssk = a.bits == 4 ? 128 : 64;
  const int64_t row_bytes = static_cast<int64_t>(a.K) * a.bits / 8;
  uint32_t out[4] = {0u, 0u, 0u, 0u};
  if (r < a.rows) {
    // stack row of stream row r: interleaved gate/up (2r + s), concatenated (s*rows + r)
    const int64_t srow = a.fusion == 1 ? 2 * r + s : (a.fusion == 2 ? static_cast<int64_t>(s) * a.rows + r : r);
    const uint8_t* row = src + (static_cast<int64_t>(e) * a.N + srow) * row_bytes;
    for (int j = 0; j < ssk / 32; ++j) {
      const int64_t k0 = static_cast<int64_t>(t) * ssk + 32 * j + 8 * q;
      if (a.bits == 4) {
        // element i goes to nibble (0, 4, 1, 5, 2, 6, 3, 7)[i] of word j (MX FP4: nibble i)
        uint32_t w = 0u;
        for (int i = 0; i < 8; ++i) {
          const int p = a.natural ? i : (i >> 1) + ((i & 1) << 2);
          w |= code_at(row, k0 + i, a.K, 4) << (4 * p);
        }
        out[j] = w;
      } else {
        // bytes 8j + i, i < 8: words 2j and 2j + 1
        uint32_t lo = 0u, hi = 0u;
        for (int i = 0; i < 4; ++i) {
          lo |= code_at(row, k0 + i, a.K, 8) << (8 * i);
          hi |= code_at(row, k0 + 4 + i, a.K, 8) << (8 * i);
        }
        out[2 * j] = lo;
        out[2 * j + 1] = hi;
      }
    }
  }
  const u32x4 v = {out[0], out[1], out[2], out[3]};
  *reinterpret_cast<u32x4*>(dst + chunk * 16) = v;
}

hipError_t launch_pack_stack(const uint8_t* src, uint8_t* dst, const PackArgs& a, hipStream_t s) {
  const int64_t nchunks = static_cast<int64_t>(a.E) * a.S * a.NB * a.KT * 64;
  if (nchunks == 0) return hipSuccess;
  const int64_t blocks = (nchunks + 255) / 256;
  pack_stack_kernel<<<static_cast<unsigned>(blocks), 256, 0, s>>>(src, dst, a);
  return hipGetLastError();
}

}  // namespace qmoe
