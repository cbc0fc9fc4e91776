// Grouping of token-expert assignments by expert into padded row tiles.
//
// The per-expert work lists behind the per-expert kernels of the ClikaRT "QMoEWoQ"
// page: assignment a = t*k + j goes to expert topk_ids[a]; every expert's rows are
// consecutive, in ascending a, and padded to a multiple of the tile height M.
//
// Determinism without order-dependent atomics: counting uses atomics (a count does
// not depend on arrival order); ranks come from wave ballots -- the lanes holding
// the same expert id are found by matching the id bit by bit over ceil(log2 E)
// ballots, and a lane's rank is the number of matching lanes below it -- plus
// per-wave counts in LDS summed in wave order, and per-block bases summed in block
// order. The result is a pure function of topk_ids.
#include "common.h"
#include "launch.h"
#include "route.h"

namespace qmoe {

constexpr int kPermThreads = 1024;
constexpr int kPermWaves = kPermThreads / kWave;
static_assert(kPermWaves <= kWave, "the wave totals are scanned by one wave");

// Exclusive scan of one int per thread over the block; also returns the total.
__device__ int block_exclusive_scan(int v, int* tmp /* kPermWaves + 1 */, int* total) {
  const int tid = threadIdx.x, lane = tid % kWave, w = tid / kWave;
  int inc = v;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    int o = __shfl_up(inc, d);
    if (lane >= d) inc += o;
  }
  if (lane == kWave - 1) tmp[w] = inc;
  __syncthreads();
  if (w == 0) {
    // the waves' totals, scanned by the first wave's lanes (kPermWaves <= 64)
    const int c = lane < kPermWaves ? tmp[lane] : 0;
    int cin = c;
#pragma unroll
    for (int d = 1; d < kPermWaves; d <<= 1) {
      const int o = __shfl_up(cin, d);
      if (lane >= d) cin += o;
    }
    if (lane < kPermWaves) tmp[lane] = cin - c;
    if (lane == kPermWaves - 1) tmp[kPermWaves] = cin;
  }
  __syncthreads();
  const int excl = tmp[w] + inc - v;
  *total = tmp[kPermWaves];
  __syncthreads();
  return excl;
}

// Counts of assignments [a0, a1) per expert into cnt (LDS, zeroed by the caller).
__device__ void block_histogram(const int32_t* __restrict__ ids, int64_t a0, int64_t a1, int* cnt) {
  for (int64_t a = a0 + threadIdx.x; a < a1; a += blockDim.x) atomicAdd(&cnt[ids[a]], 1);
}

// Writes the stable positions of assignments [a0, a1): run[e] (LDS) holds the next free
// row of expert e and is advanced past the chunk's rows. wc is LDS [kPermWaves][E].
__device__ void block_rank_scatter(const int32_t* __restrict__ ids, int64_t a0, int64_t a1, int E,
                                   int ebits, int* run, int* wc, int32_t* __restrict__ sorted_assign,
                                   int32_t* __restrict__ assign_pos) {
  const int tid = threadIdx.x, lane = tid % kWave, w = tid / kWave;
  for (int64_t base = a0; base < a1; base += kPermThreads) {
    const int64_t a = base + tid;
    const bool valid = a < a1;
    const int e = valid ? ids[a] : 0;
    for (int i = tid; i < kPermWaves * E; i += kPermThreads) wc[i] = 0;
    __syncthreads();
    uint64_t same = ballot(valid);
    for (int b = 0; b < ebits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t ones = ballot(bit);
      same &= bit ? ones : ~ones;
    }
    const int rank = __popcll(same & ((1ull << lane) - 1ull));
    if (valid && rank == 0) wc[w * E + e] = __popcll(same);
    __syncthreads();
    // per expert: its first row for each wave (run[e] plus the counts of the waves
    // before), in place over wc, and run[e] advanced past the chunk
    for (int ee = tid; ee < E; ee += kPermThreads) {
      int r = run[ee];
      for (int w2 = 0; w2 < kPermWaves; ++w2) {
        const int c = wc[w2 * E + ee];
        wc[w2 * E + ee] = r;
        r += c;
      }
      run[ee] = r;
    }
    __syncthreads();
    if (valid) {
      const int pos = wc[w * E + e] + rank;
      sorted_assign[pos] = static_cast<int32_t>(a);
      assign_pos[a] = pos;
    }
    __syncthreads();
  }
}

// From per-expert counts: padded offsets, counts, tiles, padding markers and the tile count.
// Expert e is handled by thread e (E <= kPermThreads). off_lds receives the offsets.
__device__ void block_layout(const int* cnt, int E, int M, int* scan_tmp, int* off_lds,
                             int32_t* __restrict__ counts, int32_t* __restrict__ padded_offsets,
                             int32_t* __restrict__ sorted_assign, int32_t* __restrict__ tile_list,
                             int32_t* __restrict__ num_tiles) {
  const int e = threadIdx.x;
  const int c = e < E ? cnt[e] : 0;
  const int ntile = (c + M - 1) / M;
  int total = 0;
  const int excl = block_exclusive_scan(ntile * M, scan_tmp, &total);
  if (e < E) {
    off_lds[e] = excl;
    counts[e] = c;
    padded_offsets[e + 1] = excl + ntile * M;
    if (e == 0) padded_offsets[0] = 0;
    const int t0 = excl / M;
    for (int i = 0; i < ntile; ++i) {
      tile_list[2 * (t0 + i)] = e;
      tile_list[2 * (t0 + i) + 1] = min(M, c - i * M);
    }
    for (int r = excl + c; r < excl + ntile * M; ++r) sorted_assign[r] = -1;
  }
  if (threadIdx.x == 0) *num_tiles = total / M;
  __syncthreads();
}

// Whole grouping in one block (small assignment counts).
__global__ __launch_bounds__(kPermThreads) void permute_fused_kernel(
    const int32_t* __restrict__ ids, int64_t A, int E, int ebits, int M,
    int32_t* __restrict__ counts, int32_t* __restrict__ padded_offsets,
    int32_t* __restrict__ sorted_assign, int32_t* __restrict__ assign_pos,
    int32_t* __restrict__ tile_list, int32_t* __restrict__ num_tiles) {
  extern __shared__ int lds[];
  int* cnt = lds;                 // [E]
  int* run = cnt + E;             // [E]
  int* scan_tmp = run + E;        // [kPermWaves + 1]
  int* wc = scan_tmp + kPermWaves + 1;  // [kPermWaves][E]
  for (int i = threadIdx.x; i < E; i += kPermThreads) cnt[i] = 0;
  __syncthreads();
  block_histogram(ids, 0, A, cnt);
  __syncthreads();
  block_layout(cnt, E, M, scan_tmp, run, counts, padded_offsets, sorted_assign, tile_list,
               num_tiles);
  block_rank_scatter(ids, 0, A, E, ebits, run, wc, sorted_assign, assign_pos);
}

// Routing and grouping of a small batch in one block: each 16-lane row (or each wave, for
// more than 256 experts or k > 16) of the block routes one token (route.h) into LDS, the
// routed ids reach every wave through the barrier, and the block then groups them as
// permute_fused_kernel does (the ids never go to memory: nothing after the grouping reads
// them). One launch in place of two where the batch fits one pass.
template <typename TA, int G, int V>
__global__ __launch_bounds__(kPermThreads) void route_permute_kernel(
    const TA* __restrict__ logits, int T, int E, int k, int normalize, RouteOpts o, int ebits,
    int M, float* __restrict__ topk_w, int32_t* __restrict__ counts,
    int32_t* __restrict__ padded_offsets, int32_t* __restrict__ sorted_assign,
    int32_t* __restrict__ assign_pos, int32_t* __restrict__ tile_list,
    int32_t* __restrict__ num_tiles) {
  extern __shared__ int lds[];
  int* cnt = lds;                 // [E]
  int* run = cnt + E;             // [E]
  int* scan_tmp = run + E;        // [kPermWaves + 1]
  int* wc = scan_tmp + kPermWaves + 1;  // [kPermWaves][E]
  int* ids = wc + kPermWaves * E;       // [T * k]
  const int t = threadIdx.x / G;  // one token per group of G lanes
  if (t < T) route_token<TA, G, V>(logits, t, E, k, normalize, o, ids, topk_w);
  for (int i = threadIdx.x; i < E; i += kPermThreads) cnt[i] = 0;
  __syncthreads();  // the ids each group wrote are visible to the whole block
  const int64_t A = static_cast<int64_t>(T) * k;
  block_histogram(ids, 0, A, cnt);
  __syncthreads();
  block_layout(cnt, E, M, scan_tmp, run, counts, padded_offsets, sorted_assign, tile_list,
               num_tiles);
  block_rank_scatter(ids, 0, A, E, ebits, run, wc, sorted_assign, assign_pos);
}

// Multi-block grouping, step 1: per-block counts blk[b][e].
__global__ __launch_bounds__(kPermThreads) void permute_hist_kernel(const int32_t* __restrict__ ids,
                                                                    int64_t A, int E, int chunk,
                                                                    int32_t* __restrict__ blk) {
  extern __shared__ int cnt[];
  for (int i = threadIdx.x; i < E; i += kPermThreads) cnt[i] = 0;
  __syncthreads();
  const int64_t a0 = static_cast<int64_t>(blockIdx.x) * chunk;
  const int64_t a1 = min(A, a0 + chunk);
  block_histogram(ids, a0, a1, cnt);
  __syncthreads();
  for (int i = threadIdx.x; i < E; i += kPermThreads) blk[static_cast<int64_t>(blockIdx.x) * E + i] = cnt[i];
}

// Step 2 (one block): totals, layout, and blk[b][e] turned into each block's first row.
__global__ __launch_bounds__(kPermThreads) void permute_layout_kernel(
    int nblk, int E, int M, int32_t* __restrict__ blk, int32_t* __restrict__ counts,
    int32_t* __restrict__ padded_offsets, int32_t* __restrict__ sorted_assign,
    int32_t* __restrict__ tile_list, int32_t* __restrict__ num_tiles) {
  extern __shared__ int lds[];
  int* cnt = lds;            // [E]
  int* off = cnt + E;        // [E]
  int* scan_tmp = off + E;   // [kPermWaves + 1]
  const int e = threadIdx.x;
  if (e < E) {
    int run = 0;
    for (int b = 0; b < nblk; ++b) {
      const int c = blk[static_cast<int64_t>(b) * E + e];
      blk[static_cast<int64_t>(b) * E + e] = run;
      run += c;
    }
    cnt[e] = run;
  }
  __syncthreads();
  block_layout(cnt, E, M, scan_tmp, off, counts, padded_offsets, sorted_assign, tile_list,
               num_tiles);
  if (e < E)
    for (int b = 0; b < nblk; ++b) blk[static_cast<int64_t>(b) * E + e] += off[e];
}

// Step 3: stable scatter of each block's assignments from its first rows.
__global__ __launch_bounds__(kPermThreads) void permute_scatter_kernel(
    const int32_t* __restrict__ ids, int64_t A, int E, int ebits, int chunk,
    const int32_t* __restrict__ blk, int32_t* __restrict__ sorted_assign,
    int32_t* __restrict__ assign_pos) {
  extern __shared__ int lds[];
  int* run = lds;      // [E]
  int* wc = run + E;   // [kPermWaves][E]
  for (int i = threadIdx.x; i < E; i += kPermThreads)
    run[i] = blk[static_cast<int64_t>(blockIdx.x) * E + i];
  __syncthreads();
  const int64_t a0 = static_cast<int64_t>(blockIdx.x) * chunk;
  const int64_t a1 = min(A, a0 + chunk);
  block_rank_scatter(ids, a0, a1, E, ebits, run, wc, sorted_assign, assign_pos);
}

static int bits_for(int E) {
  int b = 0;
  while ((1 << b) < E) ++b;
  return b;
}

size_t permute_scratch_bytes(int64_t A, int E) {
  if (A <= kPermFusedMax) return 0;
  const int64_t nblk = (A + kPermChunk - 1) / kPermChunk;
  return static_cast<size_t>(nblk) * E * sizeof(int32_t);
}

bool route_permute_fits(int64_t T, int64_t A, int64_t E, int64_t k) {
  const int G = route_by_rows(static_cast<int>(E), static_cast<int>(k)) ? 16 : kWave;
  return A <= kPermFusedMax && T <= kPermThreads / G;
}

template <typename TA, int G, int V>
static void launch_rp(const TA* logits, int T, int E, int k, int normalize, const RouteOpts& o,
                      int M,
                      float* w, int32_t* counts, int32_t* padded_offsets, int32_t* sorted_assign,
                      int32_t* assign_pos, int32_t* tile_list, int32_t* num_tiles, hipStream_t s) {
  const size_t lds =
      (2 * E + kPermWaves + 1 + kPermWaves * E + static_cast<size_t>(T) * k) * sizeof(int);
  route_permute_kernel<TA, G, V><<<1, kPermThreads, lds, s>>>(
      logits, T, E, k, normalize, o, bits_for(E), M, w, counts, padded_offsets,
      sorted_assign, assign_pos, tile_list, num_tiles);
}

template <typename TA, int G>
static void launch_rp_g(const TA* logits, int T, int E, int k, int normalize, const RouteOpts& o,
                        int M,
                        float* w, int32_t* counts, int32_t* padded_offsets, int32_t* sorted_assign,
                        int32_t* assign_pos, int32_t* tile_list, int32_t* num_tiles, hipStream_t s) {
  const int V = (E + G - 1) / G;
#define QMOE_RP(VV) launch_rp<TA, G, VV>(logits, T, E, k, normalize, o, M, w, counts, \
                                         padded_offsets, sorted_assign, assign_pos, tile_list, \
                                         num_tiles, s)
  if (V <= 1) QMOE_RP(1);
  else if (V <= 2) QMOE_RP(2);
  else if (V <= 4) QMOE_RP(4);
  else if (V <= 8) QMOE_RP(8);
  else QMOE_RP(16);
#undef QMOE_RP
}

template <typename TA>
static void launch_rp_t(const TA* logits, int T, int E, int k, int normalize, const RouteOpts& o,
                        int M,
                        float* w, int32_t* counts, int32_t* padded_offsets, int32_t* sorted_assign,
                        int32_t* assign_pos, int32_t* tile_list, int32_t* num_tiles, hipStream_t s) {
  if (route_by_rows(E, k))
    launch_rp_g<TA, 16>(logits, T, E, k, normalize, o, M, w, counts, padded_offsets,
                        sorted_assign, assign_pos, tile_list, num_tiles, s);
  else
    launch_rp_g<TA, kWave>(logits, T, E, k, normalize, o, M, w, counts, padded_offsets,
                           sorted_assign, assign_pos, tile_list, num_tiles, s);
}

hipError_t launch_route_permute(const void* logits, bool bf16, int T, int E, int k, int normalize,
                                const RouteOpts& o, int M, float* w, int32_t* counts,
                                int32_t* padded_offsets, int32_t* sorted_assign,
                                int32_t* assign_pos, int32_t* tile_list, int32_t* num_tiles,
                                hipStream_t s) {
  if (bf16)
    launch_rp_t(static_cast<const uint16_t*>(logits), T, E, k, normalize, o, M, w, counts,
                padded_offsets, sorted_assign, assign_pos, tile_list, num_tiles, s);
  else
    launch_rp_t(static_cast<const float*>(logits), T, E, k, normalize, o, M, w, counts,
                padded_offsets, sorted_assign, assign_pos, tile_list, num_tiles, s);
  return hipGetLastError();
}

hipError_t launch_permute(const int32_t* ids, int64_t A, int E, int M, int32_t* counts,
                          int32_t* padded_offsets, int32_t* sorted_assign, int32_t* assign_pos,
                          int32_t* tile_list, int32_t* num_tiles, void* scratch, hipStream_t s) {
  const int ebits = bits_for(E);
  if (A <= kPermFusedMax) {
    const size_t lds = (2 * E + kPermWaves + 1 + kPermWaves * E) * sizeof(int);
    permute_fused_kernel<<<1, kPermThreads, lds, s>>>(ids, A, E, ebits, M, counts, padded_offsets,
                                                      sorted_assign, assign_pos, tile_list,
                                                      num_tiles);
    return hipGetLastError();
  }
  const int nblk = static_cast<int>((A + kPermChunk - 1) / kPermChunk);
  int32_t* blk = static_cast<int32_t*>(scratch);
  permute_hist_kernel<<<nblk, kPermThreads, E * sizeof(int), s>>>(ids, A, E, kPermChunk, blk);
  permute_layout_kernel<<<1, kPermThreads, (2 * E + kPermWaves + 1) * sizeof(int), s>>>(
      nblk, E, M, blk, counts, padded_offsets, sorted_assign, tile_list, num_tiles);
  permute_scatter_kernel<<<nblk, kPermThreads, (E + kPermWaves * E) * sizeof(int), s>>>(
      ids, A, E, ebits, kPermChunk, blk, sorted_assign, assign_pos);
  return hipGetLastError();
}

}  // namespace qmoe
