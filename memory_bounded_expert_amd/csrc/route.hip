// Router top-k and gates: one wave64 per token.
//
// Each token selects its top-k experts ("Memory-Efficient Expert Routing for
// Distributed MoE Training", section 2.1).  Slot s holds the s-th expert in
// the order (logit descending, expert index ascending); IEEE comparison, so
// -0.0 and +0.0 tie and the lower index wins; a NaN logit ranks as -inf.  The
// gates are the softmax of the logits restricted to the selected experts,
// which equals the softmax over all E experts restricted and renormalised
// ("896 routed experts, 16 activated": "Training Trillion-Parameter MoE ...",
// section 1, is the widest shape served).
#include "device_common.hpp"
#include "moe_internal.h"

#include <climits>

namespace moe {
namespace {

struct Cand {
  float v;
  int i;  // INT_MAX: no candidate
};

// A NaN logit is read as -inf, so that the comparisons below form one total
// order (logit descending, index ascending) on any input: every token then
// gets k distinct experts, each slot written once.
__device__ __forceinline__ float rank_key(float x) { return __builtin_isnan(x) ? -INFINITY : x; }

// (v, i) beats (w, j) when v > w, or v and w do not compare greater either
// way (equal, or +0/-0) and i < j.
__device__ __forceinline__ bool beats(float v, int i, float w, int j) {
  if (i == INT_MAX) return false;
  if (j == INT_MAX) return true;
  if (v > w) return true;
  if (w > v) return false;
  return i < j;
}

// parts != nullptr: the logits are the sum of the router's S K-slice
// partials (s ascending) plus bias, and are written to `logits` first.
template <int VPL>
__global__ __launch_bounds__(kThreads) void topk_gates_kernel(float* __restrict__ logits,
                                                              int64_t N, int E, int k,
                                                              int32_t* __restrict__ idx,
                                                              float* __restrict__ gates,
                                                              const float* __restrict__ parts,
                                                              int S,
                                                              const float* __restrict__ bias) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (t >= N) return;  // whole wave leaves together
  float* row = logits + t * E;
  float v[VPL];
  uint32_t avail = 0;
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    const int e = lane + 64 * j;
    v[j] = 0.f;
    if (e < E) {
      if (parts) {
        float acc = parts[t * E + e];
        for (int s = 1; s < S; ++s) acc += parts[((int64_t)s * N + t) * E + e];
        v[j] = acc + (bias ? bias[e] : 0.f);
        row[e] = v[j];
      } else {
        v[j] = row[e];
      }
      v[j] = rank_key(v[j]);
      avail |= 1u << j;
    }
  }
  float my_v = 0.f;
  int my_i = 0;
  for (int s = 0; s < k; ++s) {
    float bv = 0.f;
    int bi = INT_MAX;
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      // j ascending visits this lane's experts in ascending order, so a
      // strict comparison keeps the lower index on ties
      if ((avail >> j) & 1u) {
        if (bi == INT_MAX || v[j] > bv) {
          bv = v[j];
          bi = lane + 64 * j;
        }
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off, 64);
      const int oi = __shfl_xor(bi, off, 64);
      if (beats(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if (lane == (bi & 63)) avail &= ~(1u << (bi >> 6));
    if (lane == s) {
      my_v = bv;
      my_i = bi;
    }
  }
  const float top = __shfl(my_v, 0, 64);
  float ex = lane < k ? expf(my_v - top) : 0.f;
  float sum = ex;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off, 64);
  if (lane < k) {
    idx[t * k + lane] = my_i;
    gates[t * k + lane] = ex / sum;
  }
}

// E <= 64: lane e holds expert e's logit and computes its rank directly --
// the number of experts that beat it under the same order (logit descending,
// index ascending, IEEE comparison) -- from the wave's 64 logits staged in
// LDS.  Lanes with rank < k own slot `rank`.  The gate denominator is a wave
// sum over the selected lanes.
__global__ __launch_bounds__(kThreads) void topk_rank_kernel(float* __restrict__ logits, int64_t N,
                                                             int E, int k,
                                                             int32_t* __restrict__ idx,
                                                             float* __restrict__ gates,
                                                             const float* __restrict__ parts,
                                                             int S,
                                                             const float* __restrict__ bias) {
  __shared__ float sv[kThreads / 64][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t t = (int64_t)blockIdx.x * (kThreads / 64) + w;
  if (t >= N) return;  // whole wave leaves together; no block barrier below
  float* row = logits + t * E;
  const bool valid = lane < E;
  float v = -INFINITY;
  if (valid) {
    if (parts) {
      float acc = parts[t * E + lane];
      for (int s = 1; s < S; ++s) acc += parts[((int64_t)s * N + t) * E + lane];
      v = acc + (bias ? bias[lane] : 0.f);
      row[lane] = v;
    } else {
      v = row[lane];
    }
    v = rank_key(v);
  }
  sv[w][lane] = v;
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_s_waitcnt(0xC07F);  // this wave's LDS writes done (lgkmcnt 0)
  int rank = 0;
  float top = -INFINITY;
#pragma unroll
  for (int j4 = 0; j4 < 16; ++j4) {
    const float4 q = *reinterpret_cast<const float4*>(&sv[w][4 * j4]);
    const float o[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int j = 4 * j4 + m;
      if (j < E) {
        top = fmaxf(top, o[m]);
        rank += (o[m] > v || (!(v > o[m]) && j < lane)) ? 1 : 0;
      }
    }
  }
  const bool sel = valid && rank < k;
  float ex = sel ? expf(v - top) : 0.f;
  float sum = ex;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off, 64);
  if (sel) {
    idx[t * k + rank] = lane;
    gates[t * k + rank] = ex / sum;
  }
}

}  // namespace

hipError_t launch_topk(const float* logits_in, int64_t N, int E, int k, int32_t* idx, float* gates,
                       hipStream_t st, const float* parts, int S, const float* bias) {
  if (N == 0) return hipSuccess;
  // written only when summing partials
  float* logits = const_cast<float*>(logits_in);
  const int per_block = kThreads / 64;
  const dim3 grid((unsigned)((N + per_block - 1) / per_block));
  const int vpl = (E + 63) / 64;
  if (vpl <= 1) {
    topk_rank_kernel<<<grid, kThreads, 0, st>>>(logits, N, E, k, idx, gates, parts, S, bias);
    return hipGetLastError();
  }
  if (vpl <= 2)
    topk_gates_kernel<2><<<grid, kThreads, 0, st>>>(logits, N, E, k, idx, gates, parts, S, bias);
  else if (vpl <= 4)
    topk_gates_kernel<4><<<grid, kThreads, 0, st>>>(logits, N, E, k, idx, gates, parts, S, bias);
  else if (vpl <= 8)
    topk_gates_kernel<8><<<grid, kThreads, 0, st>>>(logits, N, E, k, idx, gates, parts, S, bias);
  else
    topk_gates_kernel<16><<<grid, kThreads, 0, st>>>(logits, N, E, k, idx, gates, parts, S, bias);
  return hipGetLastError();
}

}  // namespace moe
