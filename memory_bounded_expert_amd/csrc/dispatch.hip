// Data movement around the grouped GEMMs: gather (permute), combine
// (unpermute: the sum of a token's gate-scaled expert rows), and the backward
// pass's elementwise and combine steps
// ("Training Trillion-Parameter MoE ...", section 3.3: Permute, Grouped GEMM,
// Unpermute; "Memory-Efficient Expert Routing ...", section 2.1: outputs are
// returned and recombined).
//
// Every kernel moves rows in 16-byte chunks with consecutive threads on
// consecutive chunks of a row, so each wave reads and writes whole 128-byte
// segments.  No kernel here uses atomics: sums run in a fixed order.
#include "device_common.hpp"
#include "moe_internal.h"

namespace moe {
namespace {

inline unsigned grid_for(int64_t work, int64_t per_block) {
  int64_t g = ceil_div(work, per_block);
  if (g > 65535 * 8) g = 65535 * 8;
  return (unsigned)(g < 1 ? 1 : g);
}

// dst[pos[t, s]] = src[t] for the tokens t = i + j K of chunk i and their k
// slots: each token's row is read once and written to its k rows of the
// chunk's expert-contiguous buffer (every row of the buffer holds exactly one
// pair).  Slots whose expert index is out of range (a corrupt routing input)
// have no row and are skipped.
template <typename T>
__global__ __launch_bounds__(kThreads) void gather_kernel(const T* __restrict__ src,
                                                          T* __restrict__ dst,
                                                          const int32_t* __restrict__ idx,
                                                          const int32_t* __restrict__ pos,
                                                          int E, int K, int i, int64_t n_i,
                                                          int64_t R, int k, int H) {
  const int cpr = H * (int)sizeof(T) / 16;
  const int64_t total = n_i * cpr;
  for (int64_t q = (int64_t)blockIdx.x * kThreads + threadIdx.x; q < total;
       q += (int64_t)gridDim.x * kThreads) {
    const int64_t j = q / cpr;
    const int c = (int)(q - j * cpr);
    const int64_t t = i + j * (int64_t)K;
    const u32x4_t v = reinterpret_cast<const u32x4_t*>(src + t * H)[c];
    for (int s = 0; s < k; ++s) {
      const int e = idx[t * k + s];
      const int64_t r = pos[t * k + s];
      if ((unsigned)e < (unsigned)E && (uint64_t)r < (uint64_t)R)
        reinterpret_cast<u32x4_t*>(dst + r * H)[c] = v;
    }
  }
}

// Y[t] = sum_{s<k} O[pos[t,s]] for the tokens of chunk i, the rows already
// scaled by their gates in the down projection's epilogue; fp32 sum in slot
// order, one rounding at the store.
template <typename T>
__global__ __launch_bounds__(kThreads) void combine_kernel(const T* __restrict__ O,
                                                           const int32_t* __restrict__ pos,
                                                           T* __restrict__ Y, int K, int i,
                                                           int64_t n_i, int k, int H) {
  constexpr int EPC = Elem<T>::kPer16B;
  const int cpr = H / EPC;
  const int64_t total = n_i * cpr;
  for (int64_t q = (int64_t)blockIdx.x * kThreads + threadIdx.x; q < total;
       q += (int64_t)gridDim.x * kThreads) {
    const int64_t j = q / cpr;
    const int c = (int)(q - j * cpr);
    const int64_t t = i + j * (int64_t)K;
    float acc[EPC];
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[e] = 0.f;
    // slots in batches of SB: all of a batch's row loads are issued before
    // any is consumed; the sum still runs in slot order
    constexpr int SB = 8;
    for (int s0 = 0; s0 < k; s0 += SB) {
      u32x4_t raw[SB];
#pragma unroll
      for (int u = 0; u < SB; ++u) {
        if (s0 + u < k) {
          const int64_t r = pos[t * k + s0 + u];
          raw[u] = reinterpret_cast<const u32x4_t*>(O + r * H)[c];
        }
      }
#pragma unroll
      for (int u = 0; u < SB; ++u) {
        if (s0 + u < k) {
          float v[EPC];
          unpack16(raw[u], v, T());
#pragma unroll
          for (int e = 0; e < EPC; ++e) acc[e] += v[e];
        }
      }
    }
    reinterpret_cast<u32x4_t*>(Y + t * H)[c] = pack16(acc, T());
  }
}

__global__ __launch_bounds__(kThreads) void fill_zero_kernel(u32x4_t* __restrict__ p, int64_t n16) {
  for (int64_t q = (int64_t)blockIdx.x * kThreads + threadIdx.x; q < n16;
       q += (int64_t)gridDim.x * kThreads)
    p[q] = u32x4_t{0u, 0u, 0u, 0u};
}

__global__ __launch_bounds__(kThreads) void fill_zero_tail_kernel(uint8_t* __restrict__ p,
                                                                  int64_t n) {
  const int64_t q = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (q < n) p[q] = 0;
}

// dst[c][r] = src[r][c] through a 32x32 LDS tile.
template <typename T>
__global__ __launch_bounds__(kThreads) void transpose_kernel(const T* __restrict__ src,
                                                             T* __restrict__ dst, int rows,
                                                             int cols) {
  __shared__ T tile[32][33];
  const int r0 = blockIdx.y * 32, c0 = blockIdx.x * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 32 x 8
  for (int y = ty; y < 32; y += 8) {
    const int r = r0 + y, c = c0 + tx;
    if (r < rows && c < cols) tile[y][tx] = src[(int64_t)r * cols + c];
  }
  __syncthreads();
  for (int y = ty; y < 32; y += 8) {
    const int c = c0 + y, r = r0 + tx;
    if (r < rows && c < cols) dst[(int64_t)c * rows + r] = tile[tx][y];
  }
}

// Per permuted row r (pair p = perm[r], gate g):
//   dgate_p = sum_f dh[r,f] h[r,f]                (dh = dY W_down^T, unscaled)
//   da = g dh u sigma(a) (1 + a (1 - sigma(a))),  du = g dh silu(a),  hg = g h
// da, du and hg overwrite a, u and h in place.  One work-group per row; the
// dgate sum is a fixed tree over the work-group.
template <typename T>
__global__ __launch_bounds__(kThreads) void swiglu_bwd_kernel(
    const float* __restrict__ dh, T* __restrict__ a_da, T* __restrict__ u_du,
    T* __restrict__ h_hg, const int32_t* __restrict__ perm, const float* __restrict__ gates,
    float* __restrict__ dgates, int64_t R, int F, int64_t Nk) {
  constexpr int EPC = Elem<T>::kPer16B;
  __shared__ float red[kThreads];
  const int cpr = F / EPC;
  for (int64_t r = blockIdx.x; r < R; r += gridDim.x) {
    int32_t p = perm[r];
    const bool ok = (uint64_t)p < (uint64_t)Nk;  // false only on a corrupt plan
    if (!ok) p = 0;
    const float g = gates[p];
    float part = 0.f;
    for (int c = threadIdx.x; c < cpr; c += kThreads) {
      const int64_t base = r * F + (int64_t)c * EPC;
      float av[EPC], uv[EPC], hv[EPC], dv[EPC];
      unpack16(*reinterpret_cast<const u32x4_t*>(a_da + base), av, T());
      unpack16(*reinterpret_cast<const u32x4_t*>(u_du + base), uv, T());
      unpack16(*reinterpret_cast<const u32x4_t*>(h_hg + base), hv, T());
#pragma unroll
      for (int q = 0; q < EPC; q += 4) {
        const float4 d4 = *reinterpret_cast<const float4*>(dh + base + q);
        dv[q] = d4.x; dv[q + 1] = d4.y; dv[q + 2] = d4.z; dv[q + 3] = d4.w;
      }
      float da[EPC], du[EPC], hg[EPC];
#pragma unroll
      for (int q = 0; q < EPC; ++q) {
        part = fmaf(dv[q], hv[q], part);
        const float sa = 1.f / (1.f + expf(-av[q]));
        const float d = g * dv[q];
        da[q] = d * uv[q] * sa * (1.f + av[q] * (1.f - sa));
        du[q] = d * av[q] * sa;
        hg[q] = g * hv[q];
      }
      *reinterpret_cast<u32x4_t*>(a_da + base) = pack16(da, T());
      *reinterpret_cast<u32x4_t*>(u_du + base) = pack16(du, T());
      *reinterpret_cast<u32x4_t*>(h_hg + base) = pack16(hg, T());
    }
    red[threadIdx.x] = part;
    __syncthreads();
    for (int off = kThreads / 2; off > 0; off >>= 1) {
      if ((int)threadIdx.x < off) red[threadIdx.x] += red[threadIdx.x + off];
      __syncthreads();
    }
    if (threadIdx.x == 0 && ok) dgates[p] = red[0];
    __syncthreads();
  }
}

// For the tokens of chunk i:
//   dl_s = g_s (dg_s - sum_s' g_s' dg_s'),  dlogits[t] = dl at the selected
//   experts and 0 elsewhere,
//   dX[t] = sum_s dXp[pos[t,s]] + sum_s dl_s W_r^T[S_t[s]]  (fp32, slot order,
//   one rounding).
// With dgp set, slot s's dgate is first summed over the nparts shares
// dgp[nt][pos[t,s]] (nt ascending) and stored to dgates.
template <typename T>
__global__ __launch_bounds__(kThreads) void combine_bwd_kernel(
    const T* __restrict__ dXp, const T* __restrict__ WrT, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ pos, const float* __restrict__ gates,
    float* __restrict__ dgates, T* __restrict__ dX, float* __restrict__ dlogits, int K,
    int i, int64_t n_i, int k, int E, int H, const float* __restrict__ dgp, int nparts,
    int64_t prow) {
  constexpr int EPC = Elem<T>::kPer16B;
  __shared__ float dl[64];
  __shared__ float dgs[64];
  __shared__ float gs[64];
  __shared__ int ex[64];
  __shared__ int64_t rows[64];
  const int cpr = H / EPC;
  for (int64_t j = blockIdx.x; j < n_i; j += gridDim.x) {
    const int64_t t = i + j * (int64_t)K;
    if ((int)threadIdx.x < k) {
      // slot s's loads in parallel; thread 0 then works from LDS only
      const int s = threadIdx.x;
      const int64_t r = pos[t * k + s];
      float v;
      if (dgp) {
        v = 0.f;
        for (int nt = 0; nt < nparts; ++nt) v += dgp[nt * prow + r];
        dgates[t * k + s] = v;
      } else {
        v = dgates[t * k + s];
      }
      dgs[s] = v;
      gs[s] = gates[t * k + s];
      const int e = idx[t * k + s];
      ex[s] = ((unsigned)e < (unsigned)E) ? e : 0;
      rows[s] = r;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      float sdot = 0.f;
      for (int s = 0; s < k; ++s) sdot = fmaf(gs[s], dgs[s], sdot);
      for (int s = 0; s < k; ++s) dl[s] = gs[s] * (dgs[s] - sdot);
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += kThreads) {
      float v = 0.f;
      for (int s = 0; s < k; ++s)
        if (ex[s] == e) v = dl[s];
      dlogits[t * E + e] = v;
    }
    for (int c = threadIdx.x; c < cpr; c += kThreads) {
      float acc[EPC];
#pragma unroll
      for (int q = 0; q < EPC; ++q) acc[q] = 0.f;
      for (int s = 0; s < k; ++s) {
        float v[EPC];
        unpack16(reinterpret_cast<const u32x4_t*>(dXp + rows[s] * H)[c], v, T());
#pragma unroll
        for (int q = 0; q < EPC; ++q) acc[q] += v[q];
      }
      for (int s = 0; s < k; ++s) {
        float w[EPC];
        unpack16(reinterpret_cast<const u32x4_t*>(WrT + (int64_t)ex[s] * H)[c], w, T());
#pragma unroll
        for (int q = 0; q < EPC; ++q) acc[q] = fmaf(dl[s], w[q], acc[q]);
      }
      reinterpret_cast<u32x4_t*>(dX + t * H)[c] = pack16(acc, T());
    }
    __syncthreads();
  }
}

template <typename T, int COLS>
__global__ __launch_bounds__(kThreads) void dwr_kernel(const T* __restrict__ X,
                                                       const int32_t* __restrict__ perm,
                                                       const int32_t* __restrict__ offsets,
                                                       const float* __restrict__ dlogits,
                                                       float* __restrict__ dWr, int k, int E,
                                                       int H, int64_t N) {
  // dW_r[:, e] += sum over the chunk's rows r of expert e of
  // X[t(r), :] * dlogits[t(r), e], t(r) = perm[r] / k (the token's row of X
  // itself: each token is read by its k experts' work-groups, from cache
  // after the first); rows of other experts would add
  // dlogits[t, e] = 0 exactly, so they are skipped.  One work-group per
  // (COLS-wide column block of H, expert).  The expert's segment goes in
  // blocks of kThreads rows: the block's tokens and dlogits are staged in LDS
  // first (one load each per thread), then CPB threads cover a row's COLS
  // values with 16-byte loads, RG row groups taking every RG-th row
  // (ascending per thread) with UNR rows' loads in flight.  The groups'
  // partial sums are added in group order at the end, so the result does not
  // depend on timing.
  constexpr int EPC = Elem<T>::kPer16B;
  constexpr int CPB = COLS / EPC;
  static_assert(COLS % EPC == 0 && kThreads % CPB == 0 && COLS <= kThreads, "column block");
  constexpr int RG = kThreads / CPB;
  constexpr int UNR = 16;
  __shared__ float part[RG][COLS + 1];
  __shared__ int64_t tok[kThreads];
  __shared__ float dl[kThreads];
  const int e = blockIdx.y;
  const int cb = blockIdx.x;
  const int cg = threadIdx.x % CPB, rg = threadIdx.x / CPB;
  const int r0 = offsets[e], r1 = offsets[e + 1];
  if (r1 <= r0) return;
  const int64_t col = (int64_t)cb * COLS + cg * EPC;
  float acc[EPC];
#pragma unroll
  for (int q = 0; q < EPC; ++q) acc[q] = 0.f;
  for (int b0 = r0; b0 < r1; b0 += kThreads) {
    const int nb = min(kThreads, r1 - b0);
    __syncthreads();  // the previous block's rows are consumed
    if ((int)threadIdx.x < nb) {
      const int64_t t = perm[b0 + threadIdx.x] / k;
      const bool ok = (uint64_t)t < (uint64_t)N;  // t >= N only on a corrupt plan
      tok[threadIdx.x] = ok ? t : 0;
      dl[threadIdx.x] = ok ? dlogits[t * E + e] : 0.f;
    }
    __syncthreads();
    int j = rg;
    for (; j + (UNR - 1) * RG < nb; j += UNR * RG) {
      u32x4_t v[UNR];
#pragma unroll
      for (int u = 0; u < UNR; ++u) v[u] = *reinterpret_cast<const u32x4_t*>(X + tok[j + u * RG] * H + col);
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        float x[EPC];
        unpack16(v[u], x, T());
        const float d = dl[j + u * RG];
#pragma unroll
        for (int q = 0; q < EPC; ++q) acc[q] = fmaf(d, x[q], acc[q]);
      }
    }
    for (; j < nb; j += RG) {
      float x[EPC];
      unpack16(*reinterpret_cast<const u32x4_t*>(X + tok[j] * H + col), x, T());
      const float d = dl[j];
#pragma unroll
      for (int q = 0; q < EPC; ++q) acc[q] = fmaf(d, x[q], acc[q]);
    }
  }
#pragma unroll
  for (int q = 0; q < EPC; ++q) part[rg][cg * EPC + q] = acc[q];
  __syncthreads();
  if (threadIdx.x < COLS) {
    float s = 0.f;
    for (int g = 0; g < RG; ++g) s += part[g][threadIdx.x];
    dWr[((int64_t)cb * COLS + threadIdx.x) * E + e] += s;
  }
}

}  // namespace

hipError_t launch_gather(int dtype, const void* src, void* dst, const int32_t* idx,
                         const int32_t* pos, int E, int K, int i, int64_t n_i, int k, int H,
                         hipStream_t st) {
  if (n_i == 0) return hipSuccess;
  const int64_t chunks = n_i * H * elem_bytes(dtype) / 16;
  const unsigned grid = grid_for(chunks, kThreads);
  const int64_t R = n_i * k;
  if (dtype == MOE_BF16)
    gather_kernel<bf16_t><<<grid, kThreads, 0, st>>>((const bf16_t*)src, (bf16_t*)dst, idx, pos, E,
                                                     K, i, n_i, R, k, H);
  else
    gather_kernel<float><<<grid, kThreads, 0, st>>>((const float*)src, (float*)dst, idx, pos, E, K,
                                                    i, n_i, R, k, H);
  return hipGetLastError();
}

hipError_t launch_combine(int dtype, const void* O, const int32_t* pos, void* Y, int64_t N, int K,
                          int i, int64_t n_i, int k, int H, hipStream_t st) {
  (void)N;
  if (n_i == 0) return hipSuccess;
  const int64_t chunks = n_i * H * elem_bytes(dtype) / 16;
  const unsigned grid = grid_for(chunks, kThreads);
  if (dtype == MOE_BF16)
    combine_kernel<bf16_t><<<grid, kThreads, 0, st>>>((const bf16_t*)O, pos, (bf16_t*)Y, K, i, n_i,
                                                      k, H);
  else
    combine_kernel<float><<<grid, kThreads, 0, st>>>((const float*)O, pos, (float*)Y, K, i,
                                                     n_i, k, H);
  return hipGetLastError();
}

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t st) {
  if (bytes == 0) return hipSuccess;
  const int64_t n16 = (int64_t)(bytes / 16);
  if (n16 > 0)
    fill_zero_kernel<<<grid_for(n16, kThreads * 4), kThreads, 0, st>>>((u32x4_t*)p, n16);
  const int64_t tail = (int64_t)(bytes - (size_t)n16 * 16);
  if (tail > 0) fill_zero_tail_kernel<<<1, kThreads, 0, st>>>((uint8_t*)p + n16 * 16, tail);
  return hipGetLastError();
}

hipError_t launch_transpose(int dtype, const void* src, void* dst, int rows, int cols,
                            hipStream_t st) {
  const dim3 grid((unsigned)ceil_div(cols, 32), (unsigned)ceil_div(rows, 32));
  if (dtype == MOE_BF16)
    transpose_kernel<bf16_t><<<grid, kThreads, 0, st>>>((const bf16_t*)src, (bf16_t*)dst, rows,
                                                        cols);
  else
    transpose_kernel<float><<<grid, kThreads, 0, st>>>((const float*)src, (float*)dst, rows, cols);
  return hipGetLastError();
}

hipError_t launch_swiglu_bwd(int dtype, const float* dh, void* a_da, void* u_du, void* h_hg,
                             const int32_t* perm, const float* gates, float* dgates, int64_t R,
                             int F, int64_t Nk, hipStream_t st) {
  if (R == 0) return hipSuccess;
  const unsigned grid = grid_for(R, 1);
  if (dtype == MOE_BF16)
    swiglu_bwd_kernel<bf16_t><<<grid, kThreads, 0, st>>>(dh, (bf16_t*)a_da, (bf16_t*)u_du,
                                                         (bf16_t*)h_hg, perm, gates, dgates, R, F,
                                                         Nk);
  else
    swiglu_bwd_kernel<float><<<grid, kThreads, 0, st>>>(dh, (float*)a_da, (float*)u_du,
                                                        (float*)h_hg, perm, gates, dgates, R, F,
                                                        Nk);
  return hipGetLastError();
}

hipError_t launch_combine_bwd(int dtype, const void* dXp, const void* WrT, const int32_t* idx,
                              const int32_t* pos, const float* gates, float* dgates,
                              void* dX, float* dlogits, int64_t N, int K, int i, int64_t n_i,
                              int k, int E, int H, hipStream_t st, const float* dgp, int nparts,
                              int64_t prow) {
  (void)N;
  if (n_i == 0) return hipSuccess;
  const unsigned grid = grid_for(n_i, 1);
  if (dtype == MOE_BF16)
    combine_bwd_kernel<bf16_t><<<grid, kThreads, 0, st>>>(
        (const bf16_t*)dXp, (const bf16_t*)WrT, idx, pos, gates, dgates, (bf16_t*)dX, dlogits, K,
        i, n_i, k, E, H, dgp, nparts, prow);
  else
    combine_bwd_kernel<float><<<grid, kThreads, 0, st>>>((const float*)dXp, (const float*)WrT, idx,
                                                         pos, gates, dgates, (float*)dX, dlogits, K,
                                                         i, n_i, k, E, H, dgp, nparts, prow);
  return hipGetLastError();
}

hipError_t launch_dwr(int dtype, const void* X, const int32_t* perm, const int32_t* offsets,
                      const float* dlogits, float* dWr, int k, int E, int H, int64_t N,
                      hipStream_t st) {
  // column blocks of 256, 128 or 64 (the widest dividing H; H is a
  // multiple of 64, checked when the plan is made; fp32 at most 128)
  const int cols = (dtype == MOE_BF16 && H % 256 == 0) ? 256 : (H % 128 == 0 ? 128 : 64);
  if (H % 64 != 0) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(H / cols), (unsigned)E);
  if (dtype == MOE_BF16) {
    const bf16_t* x = (const bf16_t*)X;
    if (cols == 256) dwr_kernel<bf16_t, 256><<<grid, kThreads, 0, st>>>(x, perm, offsets, dlogits, dWr, k, E, H, N);
    else if (cols == 128) dwr_kernel<bf16_t, 128><<<grid, kThreads, 0, st>>>(x, perm, offsets, dlogits, dWr, k, E, H, N);
    else dwr_kernel<bf16_t, 64><<<grid, kThreads, 0, st>>>(x, perm, offsets, dlogits, dWr, k, E, H, N);
  } else {
    const float* x = (const float*)X;
    if (cols == 128) dwr_kernel<float, 128><<<grid, kThreads, 0, st>>>(x, perm, offsets, dlogits, dWr, k, E, H, N);
    else dwr_kernel<float, 64><<<grid, kThreads, 0, st>>>(x, perm, offsets, dlogits, dWr, k, E, H, N);
  }
  return hipGetLastError();
}

}  // namespace moe
