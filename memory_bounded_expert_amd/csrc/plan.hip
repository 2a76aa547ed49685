// Chunk planner on the device: for every chunk of the eq. (1) schedule
// ("Bounded-streaming operators" summary, Methodology 1, eq. (1) and
// "Strided chunk membership"), the expert-contiguous permutation of the
// chunk's routed pairs ("Permute" of "Training Trillion-Parameter MoE ...",
// section 3.3).
//
// Rows of one expert are ordered by token position.  The order is built from
// per-block 64-bit membership masks (one bit per token of a 64-token block),
// so every count and rank is a popcount: no step depends on the order in
// which atomics land, and the result is a pure function of the routing.
//
//   plan_count    grid (nblk, K), one wave: masks -> block counts, ranks
//   plan_scan     grid K: per-expert prefix over blocks, exclusive scan over
//                 experts -> offsets, block bases, GEMM tile list
//   plan_scatter  grid over N*k pairs: perm and pos
#include "device_common.hpp"
#include "moe_internal.h"

namespace moe {
namespace {

__global__ __launch_bounds__(kPlanBlock) void plan_count_kernel(
    const int32_t* __restrict__ idx, int64_t N, int K, int k, int E, int64_t nblk,
    int32_t* __restrict__ blk_counts, int32_t* __restrict__ rank) {
  extern __shared__ unsigned long long mask[];  // [E]
  const int lane = threadIdx.x;
  const int64_t b = blockIdx.x;
  const int i = blockIdx.y;
  for (int e = lane; e < E; e += kPlanBlock) mask[e] = 0ull;
  __syncthreads();
  const int64_t n_i = (N - i + K - 1) / K;
  const int64_t j = b * kPlanBlock + lane;
  const bool valid = j < n_i;
  const int64_t t = i + j * K;
  if (valid) {
    for (int s = 0; s < k; ++s) {
      const int e = idx[t * k + s];
      if ((unsigned)e < (unsigned)E) atomicOr(&mask[e], 1ull << lane);
    }
  }
  __syncthreads();
  int32_t* cnt = blk_counts + ((int64_t)i * nblk + b) * E;
  for (int e = lane; e < E; e += kPlanBlock) cnt[e] = __popcll(mask[e]);
  if (valid) {
    const unsigned long long below = (1ull << lane) - 1ull;
    for (int s = 0; s < k; ++s) {
      const int e = idx[t * k + s];
      rank[t * k + s] = ((unsigned)e < (unsigned)E) ? __popcll(mask[e] & below) : 0;
    }
  }
}

constexpr int kMaxE = 1024;

// Inclusive Hillis-Steele scan of one int per thread over the work-group.
__device__ int block_inclusive_scan(int v, int* buf) {
  const int tid = threadIdx.x;
  buf[tid] = v;
  __syncthreads();
  for (int off = 1; off < kThreads; off <<= 1) {
    const int add = tid >= off ? buf[tid - off] : 0;
    __syncthreads();
    buf[tid] += add;
    __syncthreads();
  }
  const int r = buf[tid];
  __syncthreads();
  return r;
}

// tiles: every segment in row_tile-row tiles.  With small_tiles set, the
// same segments are also listed split: a segment of 1..kRowTile rows gets one
// kRowTile-row tile in small_tiles (at most E per chunk), a longer one its
// row_tile-row tiles in long_tiles.
__global__ __launch_bounds__(kThreads) void plan_scan_kernel(int32_t* __restrict__ blk, int E,
                                                             int64_t nblk,
                                                             int32_t* __restrict__ offsets,
                                                             int2* __restrict__ tiles,
                                                             int32_t* __restrict__ tile_count,
                                                             int64_t max_tiles, int row_tile,
                                                             int2* __restrict__ small_tiles,
                                                             int32_t* __restrict__ small_count,
                                                             int2* __restrict__ long_tiles,
                                                             int32_t* __restrict__ long_count) {
  __shared__ int tot[kMaxE];
  __shared__ int eoff[kMaxE];
  __shared__ int buf[kThreads];
  const int i = blockIdx.x;
  const int tid = threadIdx.x;
  int32_t* base = blk + (int64_t)i * nblk * E;
  // per-expert exclusive prefix over the chunk's blocks, in place; the counts
  // are read eight blocks ahead of the writes so the reads overlap
  constexpr int kAhead = 8;
  for (int e = tid; e < E; e += kThreads) {
    int run = 0;
    for (int64_t b0 = 0; b0 < nblk; b0 += kAhead) {
      int c[kAhead];
#pragma unroll
      for (int u = 0; u < kAhead; ++u) c[u] = b0 + u < nblk ? base[(b0 + u) * E + e] : 0;
#pragma unroll
      for (int u = 0; u < kAhead; ++u) {
        if (b0 + u < nblk) base[(b0 + u) * E + e] = run;
        run += c[u];
      }
    }
    tot[e] = run;
  }
  __syncthreads();
  // exclusive scan over experts; each thread owns a contiguous run of experts
  const int seg = (E + kThreads - 1) / kThreads;
  const int e0 = tid * seg;
  const int e1 = min(E, e0 + seg);
  const bool split = small_tiles != nullptr;
  auto is_small = [&](int m) { return split && m > 0 && m <= kRowTile; };
  int rows = 0, ntile = 0, nsmall = 0, nlong = 0;
  for (int e = e0; e < e1; ++e) {
    rows += tot[e];
    const int nt = (tot[e] + row_tile - 1) / row_tile;
    ntile += nt;
    if (is_small(tot[e]))
      ++nsmall;
    else
      nlong += nt;
  }
  int row_run = block_inclusive_scan(rows, buf) - rows;
  int tile_run = block_inclusive_scan(ntile, buf) - ntile;
  int small_run = block_inclusive_scan(nsmall, buf) - nsmall;
  int long_run = block_inclusive_scan(nlong, buf) - nlong;
  int32_t* off = offsets + (int64_t)i * (E + 1);
  int2* tl = tiles + (int64_t)i * max_tiles;
  int2* ll = split ? long_tiles + (int64_t)i * max_tiles : nullptr;
  for (int e = e0; e < e1; ++e) {
    off[e] = row_run;
    eoff[e] = row_run;
    const int nt = (tot[e] + row_tile - 1) / row_tile;
    for (int q = 0; q < nt; ++q) tl[tile_run + q] = make_int2(e, row_run + q * row_tile);
    tile_run += nt;
    if (is_small(tot[e])) {
      small_tiles[(int64_t)i * E + small_run++] = make_int2(e, row_run);
    } else if (split) {
      for (int q = 0; q < nt; ++q) ll[long_run + q] = make_int2(e, row_run + q * row_tile);
      long_run += nt;
    }
    row_run += tot[e];
  }
  if (tid == kThreads - 1) {
    off[E] = row_run;
    tile_count[i] = tile_run;
    if (split) {
      small_count[i] = small_run;
      long_count[i] = long_run;
    }
  }
  __syncthreads();
  for (int e = tid; e < E; e += kThreads) {
    const int o = eoff[e];
    for (int64_t b0 = 0; b0 < nblk; b0 += kAhead) {
      int c[kAhead];
#pragma unroll
      for (int u = 0; u < kAhead; ++u) c[u] = b0 + u < nblk ? base[(b0 + u) * E + e] : 0;
#pragma unroll
      for (int u = 0; u < kAhead; ++u)
        if (b0 + u < nblk) base[(b0 + u) * E + e] = c[u] + o;
    }
  }
}

__global__ __launch_bounds__(kThreads) void plan_scatter_kernel(
    const int32_t* __restrict__ idx, int64_t N, int K, int k, int E, int64_t nblk,
    const int32_t* __restrict__ base, const int32_t* __restrict__ rank, int32_t* __restrict__ perm,
    int32_t* __restrict__ pos, const float* __restrict__ gates, float* __restrict__ row_gates) {
  const int64_t p = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (p >= N * k) return;
  const int64_t t = p / k;
  const int64_t i = t % K;
  const int64_t j = t / K;
  const int64_t b = j / kPlanBlock;
  const int e = idx[p];
  if ((unsigned)e >= (unsigned)E) {
    pos[p] = 0;
    return;
  }
  const int r = base[(i * nblk + b) * E + e] + rank[p];
  pos[p] = r;
  const int64_t q = N / K, rem = N % K;
  const int64_t pb = (int64_t)k * (i * q + (i < rem ? i : rem));
  perm[pb + r] = (int32_t)p;
  if (row_gates) row_gates[pb + r] = gates[p];
}

}  // namespace

hipError_t launch_plan(const int32_t* idx, int64_t N, int K, int k, int E, const PlanBuffers& b,
                       hipStream_t st, const float* gates, int* launches) {
  if (b.row_gates && !gates) return hipErrorInvalidValue;
  if (N == 0) return hipSuccess;
  plan_count_kernel<<<dim3((unsigned)b.nblk, (unsigned)K), kPlanBlock,
                      (size_t)E * sizeof(unsigned long long), st>>>(idx, N, K, k, E, b.nblk,
                                                                    b.blk, b.rank);
  plan_scan_kernel<<<K, kThreads, 0, st>>>(b.blk, E, b.nblk, b.offsets, b.tiles, b.tile_count,
                                           b.max_tiles, b.row_tile, b.small_tiles,
                                           b.small_count, b.long_tiles, b.long_count);
  const int64_t pairs = N * k;
  plan_scatter_kernel<<<(unsigned)ceil_div(pairs, kThreads), kThreads, 0, st>>>(
      idx, N, K, k, E, b.nblk, b.blk, b.rank, b.perm, b.pos, gates, b.row_gates);
  if (launches) *launches += 3;
  return hipGetLastError();
}

}  // namespace moe
