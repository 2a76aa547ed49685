// C ABI of the vocabulary projection with cross-entropy over vocabulary
// strips, and its small kernels.
//
// Follows the "Bounded-streaming operators" summary, Methodology 2
// (Ring-DTP): the batch meets the vocabulary projection one strip at a time,
// each strip's partial normalisers are folded into a running per-token state
// (running max m, normaliser z, target logit) with the online-softmax
// recurrence of eq. (3), and nothing strip-sized outlives its strip (eq. (2)
// with one rank: the strip is a vocabulary interval of v_chunk entries).  The
// loss equals the unchunked cross-entropy ("Training Trillion-Parameter MoE
// Large Language Models", section 3.5, vocabulary-axis chunking).
//
// Forward, per strip: one GEMM whose epilogue reduces every 128-column slice
// of its logit tile to a per-row (max, sum of exp) pair (the logits never
// leave the chip), then one fold launch that applies eq. (3) to the strip's
// pairs in vocabulary order.  Backward, per strip: the same GEMM recomputes
// the logits and stores the strip's logit gradient (bf16), then dX's fp32
// running sum takes G W_s in one accumulation chain and dW_s = G^T X.
#include <cmath>

#include "cce.h"
#include "device_common.hpp"
#include "moe_internal.h"

#define MOE_API extern "C" __attribute__((visibility("default")))

namespace moe {
namespace {

constexpr uint32_t kCceMagic = 0x43434531u;  // "CCE1"
constexpr int kCceThreads = 256;

struct CceLayout {
  size_t pmax = 0, psum = 0, m = 0, z = 0, ytgt = 0;  // forward
  size_t g = 0, dx = 0, dl = 0;                       // backward
  size_t total = 0;
};

// Columns of the strip buffers: the widest strip rounded up to whole
// 256-column logit tiles (v_chunk itself unless the vocabulary is narrower).
int strip_cols(int64_t V, int v_chunk) {
  return (int)std::min<int64_t>(v_chunk, ceil_div(V, 256) * 256);
}

CceLayout cce_layout(int64_t N, int H, int cols, bool backward) {
  CceLayout L;
  size_t cur = 0;
  auto take = [&](size_t bytes) {
    const size_t o = cur;
    cur = (cur + bytes + 255) & ~(size_t)255;
    return o;
  };
  const size_t n = (size_t)N;
  if (!backward) {
    const size_t nsl = (size_t)cols / kCceSlice;
    L.pmax = take(nsl * n * 4);
    L.psum = take(nsl * n * 4);
    L.m = take(n * 4);
    L.z = take(n * 4);
    L.ytgt = take(n * 4);
  } else {
    L.g = take(n * (size_t)cols * 2);
    L.dx = take(n * (size_t)H * 4);
    L.dl = take(n * 4);
  }
  L.total = cur;
  return L;
}

// Eq. (3) over the strip's slice pairs, in vocabulary order, continuing the
// running state of the earlier strips (first: start from the empty state;
// last: finish with lse = m + log z and the loss).  An empty slice (every
// column past the vocabulary end) has max -inf and is skipped.
// One thread per token, 64-token blocks (a batch of a few thousand tokens
// still spreads over the CUs); the slice pairs are loaded kFoldBatch at a time
// ahead of the sequential fold so their latency overlaps.
constexpr int kFoldThreads = 64;
constexpr int kFoldBatch = 8;
__global__ __launch_bounds__(kFoldThreads) void cce_fold_kernel(
    const float* __restrict__ pmax, const float* __restrict__ psum, int nslices, int64_t N,
    float* __restrict__ m, float* __restrict__ z, int first, int last,
    const float* __restrict__ ytgt, const int32_t* __restrict__ targets, int64_t V,
    float* __restrict__ loss, float* __restrict__ lse) {
  const int64_t t = (int64_t)blockIdx.x * kFoldThreads + threadIdx.x;
  if (t >= N) return;
  float mm = first ? -INFINITY : m[t];
  float zz = first ? 0.f : z[t];
  for (int s0 = 0; s0 < nslices; s0 += kFoldBatch) {
    float a[kFoldBatch], b[kFoldBatch];
#pragma unroll
    for (int u = 0; u < kFoldBatch; ++u) {
      const bool in = s0 + u < nslices;
      a[u] = in ? pmax[(int64_t)(s0 + u) * N + t] : -INFINITY;
      b[u] = in ? psum[(int64_t)(s0 + u) * N + t] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < kFoldBatch; ++u) {
      if (a[u] == -INFINITY) continue;  // empty slice (or past the strip's last)
      if (a[u] > mm) {
        zz = zz * expf(mm - a[u]) + b[u];  // m' = a: the old normaliser is rescaled
        mm = a[u];
      } else {
        zz = zz + b[u] * expf(a[u] - mm);  // m' = m: the slice's sum is rescaled
      }
    }
  }
  if (last) {
    const float l = mm + logf(zz);
    lse[t] = l;
    const int tg = targets[t];
    loss[t] = (tg >= 0 && (int64_t)tg < V) ? l - ytgt[t] : 0.f;
  } else {
    m[t] = mm;
    z[t] = zz;
  }
}

// Upstream gradient with ignored tokens (target outside [0, V)) zeroed.
__global__ __launch_bounds__(kCceThreads) void cce_prep_kernel(
    const float* __restrict__ dloss, const int32_t* __restrict__ targets, int64_t N, int64_t V,
    float* __restrict__ dl) {
  const int64_t t = (int64_t)blockIdx.x * kCceThreads + threadIdx.x;
  if (t >= N) return;
  const int tg = targets[t];
  dl[t] = (tg >= 0 && (int64_t)tg < V) ? dloss[t] : 0.f;
}

// dX = bf16(running fp32 sum), round to nearest even; 4 values per thread.
__global__ __launch_bounds__(kCceThreads) void cce_round_kernel(const float* __restrict__ src,
                                                             bf16_t* __restrict__ dst, int64_t n4) {
  const int64_t i = (int64_t)blockIdx.x * kCceThreads + threadIdx.x;
  if (i >= n4) return;
  const f32x4_t v = reinterpret_cast<const f32x4_t*>(src)[i];
  ushort4 o;
  o.x = f2bf(v[0]);
  o.y = f2bf(v[1]);
  o.z = f2bf(v[2]);
  o.w = f2bf(v[3]);
  reinterpret_cast<ushort4*>(dst)[i] = o;
}

unsigned blocks(int64_t n) { return (unsigned)ceil_div(n, kCceThreads); }

bool plan_ok(const cce_plan_t* p) { return p != nullptr && p->magic == kCceMagic; }

}  // namespace
}  // namespace moe

using namespace moe;

#define CCE_CHECK(call)                        \
  do {                                         \
    if ((call) != hipSuccess) return MOE_EHIP; \
  } while (0)

MOE_API int cce_plan(int64_t N, int32_t H, int64_t V, int32_t v_chunk, int32_t dtype,
                     cce_plan_t* out) {
  if (!out || N < 0 || V < 1 || H < 1 || v_chunk < 1) return MOE_EINVAL;
  if (dtype != MOE_F32 && dtype != MOE_BF16) return MOE_EINVAL;
  if (dtype != MOE_BF16 || H % 128 != 0 || v_chunk % 256 != 0) return MOE_EUNSUPPORTED;
  const int64_t lim = (int64_t)1 << 30;
  if (N * (int64_t)H >= lim || N * (int64_t)v_chunk >= lim || (int64_t)v_chunk * H >= lim)
    return MOE_EUNSUPPORTED;
  cce_plan_t p{};
  p.magic = kCceMagic;
  p.dtype = dtype;
  p.N = N;
  p.V = V;
  p.H = H;
  p.v_chunk = v_chunk;
  p.S = N == 0 ? 0 : (int32_t)ceil_div(V, v_chunk);
  p.strip_bound_bytes = N * std::min<int64_t>(v_chunk, V) * 2;
  p.unchunked_logit_bytes = N * V * 4;
  const int cols = strip_cols(V, v_chunk);
  p.fwd_workspace_bytes = N == 0 ? 0 : (int64_t)cce_layout(N, H, cols, false).total;
  p.bwd_workspace_bytes = N == 0 ? 0 : (int64_t)cce_layout(N, H, cols, true).total;
  *out = p;
  return MOE_OK;
}

MOE_API int cce_forward(const cce_plan_t* plan, const void* X, const void* W,
                        const int32_t* targets, float* loss, float* lse, void* workspace,
                        size_t workspace_bytes, void* stream) {
  if (!plan_ok(plan)) return MOE_EINVAL;
  const cce_plan_t& P = *plan;
  if (P.N == 0) return MOE_OK;
  if (!X || !W || !targets || !loss || !lse || !workspace) return MOE_EINVAL;
  if ((uintptr_t)workspace % 256) return MOE_EINVAL;
  if (workspace_bytes < (size_t)P.fwd_workspace_bytes) return MOE_EWORKSPACE;
  const CceLayout L = cce_layout(P.N, P.H, strip_cols(P.V, P.v_chunk), false);
  hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)workspace;
  float* pmax = (float*)(ws + L.pmax);
  float* psum = (float*)(ws + L.psum);
  float* m = (float*)(ws + L.m);
  float* z = (float*)(ws + L.z);
  float* ytgt = (float*)(ws + L.ytgt);
  (void)hipGetLastError();
  for (int s = 0; s < P.S; ++s) {
    const int64_t v0 = (int64_t)s * P.v_chunk;
    const int w = (int)std::min<int64_t>(P.v_chunk, P.V - v0);
    const bf16_t* Ws = (const bf16_t*)W + v0 * P.H;
    CCE_CHECK(gemm_cce_logits(false, X, Ws, P.N, P.H, w, v0, targets, pmax, psum, ytgt, nullptr,
                              nullptr, nullptr, 0, st));
    // slices the GEMM wrote: whole 256-column tiles, two slices each
    const int nsl = (int)ceil_div(w, 256) * (256 / kCceSlice);
    cce_fold_kernel<<<(unsigned)ceil_div(P.N, kFoldThreads), kFoldThreads, 0, st>>>(
        pmax, psum, nsl, P.N, m, z, s == 0, s == P.S - 1, ytgt, targets, P.V, loss, lse);
    CCE_CHECK(hipGetLastError());
  }
  return MOE_OK;
}

MOE_API int cce_backward(const cce_plan_t* plan, const void* X, const void* W,
                         const int32_t* targets, const float* lse, const float* dloss, void* dX,
                         float* dW, void* workspace, size_t workspace_bytes, void* stream) {
  if (!plan_ok(plan)) return MOE_EINVAL;
  const cce_plan_t& P = *plan;
  if (!dW) return MOE_EINVAL;
  if (P.N > 0 && (!X || !W || !targets || !lse || !dloss || !dX || !workspace)) return MOE_EINVAL;
  if (P.N > 0 && (uintptr_t)workspace % 256) return MOE_EINVAL;
  if (workspace_bytes < (size_t)P.bwd_workspace_bytes) return MOE_EWORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  (void)hipGetLastError();
  if (P.N == 0) {  // no tokens: dW = 0
    CCE_CHECK(launch_fill_zero(dW, (size_t)P.V * P.H * sizeof(float), st));
    return MOE_OK;
  }
  const int cols = strip_cols(P.V, P.v_chunk);
  const CceLayout L = cce_layout(P.N, P.H, cols, true);
  char* ws = (char*)workspace;
  bf16_t* G = (bf16_t*)(ws + L.g);
  float* dx = (float*)(ws + L.dx);
  float* dl = (float*)(ws + L.dl);
  cce_prep_kernel<<<blocks(P.N), kCceThreads, 0, st>>>(dloss, targets, P.N, P.V, dl);
  CCE_CHECK(hipGetLastError());
  for (int s = 0; s < P.S; ++s) {
    const int64_t v0 = (int64_t)s * P.v_chunk;
    const int w = (int)std::min<int64_t>(P.v_chunk, P.V - v0);
    const bf16_t* Ws = (const bf16_t*)W + v0 * P.H;
    CCE_CHECK(gemm_cce_logits(true, X, Ws, P.N, P.H, w, v0, targets, nullptr, nullptr, nullptr,
                              lse, dl, G, cols, st));
    CCE_CHECK(gemm_cce_dx(G, cols, Ws, P.N, P.H, w, dx, s == 0, st));
    CCE_CHECK(gemm_cce_dw(G, cols, X, P.N, P.H, w, dW + v0 * P.H, st));
  }
  const int64_t n4 = P.N * P.H / 4;
  cce_round_kernel<<<blocks(n4), kCceThreads, 0, st>>>(dx, (bf16_t*)dX, n4);
  CCE_CHECK(hipGetLastError());
  return MOE_OK;
}

MOE_API int cce_debug_stage(const cce_plan_t* plan, int32_t stage, int32_t strip, const void* X,
                            const void* W, const int32_t* targets, float* loss, float* lse,
                            const float* dloss, void* dX, float* dW, void* workspace,
                            size_t workspace_bytes, void* stream) {
  (void)dloss;
  (void)dX;
  if (!plan_ok(plan)) return MOE_EINVAL;
  const cce_plan_t& P = *plan;
  if (stage < CCE_STAGE_LOGITS || stage > CCE_STAGE_DW || strip < 0 || strip >= P.S)
    return MOE_EINVAL;
  if (!X || !W || !targets || !lse || !workspace || (uintptr_t)workspace % 256) return MOE_EINVAL;
  const bool bwd = stage >= CCE_STAGE_GRAD;
  if (workspace_bytes < (size_t)(bwd ? P.bwd_workspace_bytes : P.fwd_workspace_bytes))
    return MOE_EWORKSPACE;
  if (stage == CCE_STAGE_FOLD && !loss) return MOE_EINVAL;
  if (stage == CCE_STAGE_DW && !dW) return MOE_EINVAL;
  const int cols = strip_cols(P.V, P.v_chunk);
  const CceLayout L = cce_layout(P.N, P.H, cols, bwd);
  hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)workspace;
  const int64_t v0 = (int64_t)strip * P.v_chunk;
  const int w = (int)std::min<int64_t>(P.v_chunk, P.V - v0);
  const bf16_t* Ws = (const bf16_t*)W + v0 * P.H;
  (void)hipGetLastError();
  switch (stage) {
    case CCE_STAGE_LOGITS:
      CCE_CHECK(gemm_cce_logits(false, X, Ws, P.N, P.H, w, v0, targets, (float*)(ws + L.pmax),
                                (float*)(ws + L.psum), (float*)(ws + L.ytgt), nullptr, nullptr,
                                nullptr, 0, st));
      break;
    case CCE_STAGE_FOLD: {
      const int nsl = (int)ceil_div(w, 256) * (256 / kCceSlice);
      cce_fold_kernel<<<(unsigned)ceil_div(P.N, kFoldThreads), kFoldThreads, 0, st>>>(
          (float*)(ws + L.pmax), (float*)(ws + L.psum), nsl, P.N, (float*)(ws + L.m),
          (float*)(ws + L.z), strip == 0, strip == P.S - 1, (float*)(ws + L.ytgt), targets, P.V,
          loss, lse);
      CCE_CHECK(hipGetLastError());
      break;
    }
    case CCE_STAGE_GRAD:
      CCE_CHECK(gemm_cce_logits(true, X, Ws, P.N, P.H, w, v0, targets, nullptr, nullptr, nullptr,
                                lse, (float*)(ws + L.dl), ws + L.g, cols, st));
      break;
    case CCE_STAGE_DX:
      CCE_CHECK(gemm_cce_dx(ws + L.g, cols, Ws, P.N, P.H, w, (float*)(ws + L.dx), strip == 0, st));
      break;
    default:
      CCE_CHECK(gemm_cce_dw(ws + L.g, cols, X, P.N, P.H, w, dW + v0 * P.H, st));
      break;
  }
  return MOE_OK;
}
