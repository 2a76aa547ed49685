// Grouped GEMM on gfx950 MFMA ("Grouped GEMM organizes computation by
// expert-aggregated batches": "Training Trillion-Parameter MoE ...",
// section 3.3).
//
// One kernel template serves every contraction of the layer:
//   Mode::Rows    C[rows of expert e] = A[rows] . B[e]   (row-grouped: the
//                 permuted buffer's expert segments; M-tiles come from the
//                 planner's per-chunk tile list, so no host sync is needed)
//   Mode::Dense   one plain GEMM (router logits)
//   Mode::Expert  C[e] += A_e^T . B_e over the rows of expert e (weight
//                 gradients; the reduction runs over the chunk's rows)
//
// Work-group: 256 threads = 4 waves in a 2 x 2 grid over a BM x BN tile
// (BN per operand group; DUAL carries two B operands side by side, e.g.
// gate and up, sharing the A tile).  Each wave owns a (BM/2) x (BN/2) block of
// 16 x 16 accumulators per group.
//
// LDS holds both operands "K-contiguous": every LDS row is one M (or N)
// index with 128 bytes of K (8 chunks of 16 bytes: 64 bf16 or 32 fp32).
// Chunk c of row r sits at slot c ^ (r & 7), which makes the MFMA operand
// reads (16 rows x one chunk per quarter-wave) and all the tile writes free of
// bank conflicts.  Operands stored K-contiguous in memory are copied 16 bytes
// at a time; operands stored M/N-contiguous are loaded as 8 x 8 (bf16) or
// 4 x 4 (fp32) blocks and transposed in registers on the way into LDS.
// Two LDS stages: the global loads of K-tile t+1 are in flight while the
// MFMAs consume tile t; one barrier per K-tile.
//
// MFMA: v_mfma_f32_16x16x32_bf16 for bf16 (fp32 accumulation), and for fp32
// four v_mfma_f32_16x16x4_f32 per 16-byte chunk.  Every output element is
// reduced in the same K order whatever the tile's M extent or position, so a
// row's result does not depend on which other rows share its tile -- the
// property that makes chunked and unchunked runs bitwise equal.
#pragma once

#include "device_common.hpp"
#include "moe_internal.h"

namespace moe {
namespace gemm {

enum class Mode { Rows, Dense, Expert };
enum class Epi { Store, SwiGLU, SwiGLUSave, F32, BiasF32, AccF32 };

struct Params {
  const void* A;
  const void* A2;  // second K segment (KCAT)
  int64_t lda;
  const void* B;
  const void* B2;  // second operand group (DUAL) or second K segment (KCAT)
  int64_t ldb;
  int64_t b_estride;  // elements between experts' B (Rows mode)
  void* C;
  void* C2;
  void* C3;
  int64_t ldc;
  int64_t c_estride;  // elements between experts' C (Expert mode)
  int M, N, K, Kseg;
  const int2* tiles;
  const int32_t* tile_count;
  const int32_t* offsets;
  const float* bias;
};

__device__ __forceinline__ int swz(int row, int c) { return c ^ (row & 7); }

template <typename T> struct Mfma;
template <> struct Mfma<bf16_t> {
  __device__ static __forceinline__ void run(const u32x4_t& a, const u32x4_t& b, f32x4_t& acc) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), acc, 0, 0, 0);
  }
};
template <> struct Mfma<float> {
  // lane group G = lane/16 holds k = 4*(chunk) + j in element j; MFMA j sums
  // k-slot G over the four groups, four MFMAs cover the 16 k of a step.
  __device__ static __forceinline__ void run(const u32x4_t& a, const u32x4_t& b, f32x4_t& acc) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
  }
};

__device__ __forceinline__ uint32_t word(const u32x4_t& v, int i) { return v[i]; }

// in[r] = 16 bytes of row r (contiguous index c); out[c] = 16 bytes of
// column c (index r contiguous).
__device__ __forceinline__ void transpose_block(const u32x4_t* in, u32x4_t* out, bf16_t) {
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t lo = word(in[2 * j], c >> 1);
      const uint32_t hi = word(in[2 * j + 1], c >> 1);
      w[j] = (c & 1) ? ((lo >> 16) | (hi & 0xFFFF0000u)) : ((lo & 0xFFFFu) | (hi << 16));
    }
    out[c] = u32x4_t{w[0], w[1], w[2], w[3]};
  }
}
__device__ __forceinline__ void transpose_block(const u32x4_t* in, u32x4_t* out, float) {
#pragma unroll
  for (int c = 0; c < 4; ++c)
    out[c] = u32x4_t{word(in[0], c), word(in[1], c), word(in[2], c), word(in[3], c)};
}

template <typename T, Mode MODE, int BM, int BN, bool DUAL, bool A_K, bool B_K, bool KCAT, Epi EPI>
__global__ __launch_bounds__(kThreads) void gemm_kernel(const Params p) {
  constexpr int EPC = Elem<T>::kPer16B;
  constexpr int BK = 8 * EPC;
  constexpr int NB = DUAL ? 2 : 1;
  constexpr int NCOL = BN * NB;
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int FM = WM / 16, FN = WN / 16;
  constexpr int A_BLK = 8 * BM / EPC;    // transposing loads: EPC x EPC blocks
  constexpr int B_BLK = 8 * NCOL / EPC;
  constexpr int A_UNITS = A_K ? (BM * 8) / kThreads : (A_BLK + kThreads - 1) / kThreads;
  constexpr int B_UNITS = B_K ? (NCOL * 8) / kThreads : (B_BLK + kThreads - 1) / kThreads;
  constexpr int A_REGS = A_K ? A_UNITS : A_UNITS * EPC;
  constexpr int B_REGS = B_K ? B_UNITS : B_UNITS * EPC;
  static_assert(FM >= 1 && FN >= 1, "tile too small for 2x2 waves of 16x16");
  static_assert(!A_K || (BM * 8) % kThreads == 0, "A tile / threads");
  static_assert(!B_K || (NCOL * 8) % kThreads == 0, "B tile / threads");
  static_assert(!(DUAL && KCAT), "DUAL and KCAT are exclusive");

  __shared__ u32x4_t As[2][BM * 8];
  __shared__ u32x4_t Bs[2][NCOL * 8];

  const int tid = threadIdx.x;
  int e = 0, m0 = 0, row_end = 0;
  const int n0 = blockIdx.y * BN;
  int64_t k_begin = 0;
  int k_len = p.K;
  if constexpr (MODE == Mode::Rows) {
    if ((int)blockIdx.x >= *p.tile_count) return;
    const int2 tl = p.tiles[blockIdx.x];
    e = tl.x;
    m0 = tl.y;
    row_end = p.offsets[e + 1];
  } else if constexpr (MODE == Mode::Dense) {
    m0 = blockIdx.x * BM;
    row_end = p.M;
  } else {
    e = blockIdx.z;
    k_begin = p.offsets[e];
    k_len = p.offsets[e + 1] - (int)k_begin;
    if (k_len <= 0) return;
    m0 = blockIdx.x * BM;
    row_end = p.M;
  }
  const T* Ap = static_cast<const T*>(p.A);
  const T* A2p = static_cast<const T*>(p.A2);
  const int64_t boff = (MODE == Mode::Rows) ? (int64_t)e * p.b_estride : 0;
  const T* Bp = static_cast<const T*>(p.B) + boff;
  const T* B2p = (DUAL || KCAT) ? static_cast<const T*>(p.B2) + boff : nullptr;
  const int nk = (k_len + BK - 1) / BK;
  const u32x4_t zero = u32x4_t{0u, 0u, 0u, 0u};

  u32x4_t ra[A_REGS];
  u32x4_t rb[B_REGS];
  f32x4_t acc[NB][FM][FN];
#pragma unroll
  for (int g = 0; g < NB; ++g)
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[g][i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  auto load = [&](int kt) __attribute__((always_inline)) {
    const int k0 = kt * BK;
    // ---- A
    if constexpr (A_K) {
      const T* src = Ap;
      int kk = k0;
      if constexpr (KCAT) {
        if (k0 >= p.Kseg) {
          src = A2p;
          kk = k0 - p.Kseg;
        }
      }
#pragma unroll
      for (int u = 0; u < A_UNITS; ++u) {
        const int lin = tid + u * kThreads;
        const int m = lin >> 3, c = lin & 7;
        const int row = m0 + m;
        ra[u] = row < row_end
                    ? *reinterpret_cast<const u32x4_t*>(src + (int64_t)row * p.lda + kk + c * EPC)
                    : zero;
      }
    } else {
#pragma unroll
      for (int u = 0; u < A_UNITS; ++u) {
        const int blk = tid + u * kThreads;
        const int kb = blk & 7, mb = blk >> 3;
#pragma unroll
        for (int q = 0; q < EPC; ++q) {
          const int kr = k0 + kb * EPC + q;
          ra[u * EPC + q] =
              (blk < A_BLK && kr < k_len)
                  ? *reinterpret_cast<const u32x4_t*>(Ap + (k_begin + kr) * p.lda + m0 + mb * EPC)
                  : zero;
        }
      }
    }
    // ---- B
    if constexpr (B_K) {
      const T* s1 = Bp;
      int kk = k0;
      if constexpr (KCAT) {
        if (k0 >= p.Kseg) {
          s1 = B2p;
          kk = k0 - p.Kseg;
        }
      }
#pragma unroll
      for (int u = 0; u < B_UNITS; ++u) {
        const int lin = tid + u * kThreads;
        const int n = lin >> 3, c = lin & 7;
        const int g = n / BN;
        const int nin = n - g * BN;
        const T* src = (DUAL && g) ? B2p : s1;
        rb[u] = *reinterpret_cast<const u32x4_t*>(src + (int64_t)(n0 + nin) * p.ldb + kk + c * EPC);
      }
    } else {
#pragma unroll
      for (int u = 0; u < B_UNITS; ++u) {
        const int blk = tid + u * kThreads;
        const int kb = blk & 7, nb = blk >> 3;
        const int ncol = nb * EPC;
        const int g = ncol / BN;
        const int nin = ncol - g * BN;
        const T* src = (DUAL && g) ? B2p : Bp;
        const int gc = n0 + nin;
        const bool colok = blk < B_BLK && (MODE != Mode::Dense || gc < p.N);
#pragma unroll
        for (int q = 0; q < EPC; ++q) {
          const int kr = k0 + kb * EPC + q;
          const bool ok = colok && (MODE != Mode::Expert || kr < k_len);
          rb[u * EPC + q] =
              ok ? *reinterpret_cast<const u32x4_t*>(src + (k_begin + kr) * p.ldb + gc) : zero;
        }
      }
    }
  };

  auto store = [&](int buf) __attribute__((always_inline)) {
    if constexpr (A_K) {
#pragma unroll
      for (int u = 0; u < A_UNITS; ++u) {
        const int lin = tid + u * kThreads;
        const int m = lin >> 3, c = lin & 7;
        As[buf][m * 8 + swz(m, c)] = ra[u];
      }
    } else {
#pragma unroll
      for (int u = 0; u < A_UNITS; ++u) {
        const int blk = tid + u * kThreads;
        if (blk < A_BLK) {
          const int kb = blk & 7, mb = blk >> 3;
          u32x4_t t[EPC];
          transpose_block(&ra[u * EPC], t, T());
#pragma unroll
          for (int cc = 0; cc < EPC; ++cc) {
            const int m = mb * EPC + cc;
            As[buf][m * 8 + swz(m, kb)] = t[cc];
          }
        }
      }
    }
    if constexpr (B_K) {
#pragma unroll
      for (int u = 0; u < B_UNITS; ++u) {
        const int lin = tid + u * kThreads;
        const int n = lin >> 3, c = lin & 7;
        Bs[buf][n * 8 + swz(n, c)] = rb[u];
      }
    } else {
#pragma unroll
      for (int u = 0; u < B_UNITS; ++u) {
        const int blk = tid + u * kThreads;
        if (blk < B_BLK) {
          const int kb = blk & 7, nb = blk >> 3;
          u32x4_t t[EPC];
          transpose_block(&rb[u * EPC], t, T());
#pragma unroll
          for (int cc = 0; cc < EPC; ++cc) {
            const int n = nb * EPC + cc;
            Bs[buf][n * 8 + swz(n, kb)] = t[cc];
          }
        }
      }
    }
  };

  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;

  auto compute = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int c = ks * 4 + (lane >> 4);
      u32x4_t af[FM];
      u32x4_t bv[NB][FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int r = wm * WM + i * 16 + (lane & 15);
        af[i] = As[buf][r * 8 + swz(r, c)];
      }
#pragma unroll
      for (int g = 0; g < NB; ++g)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int n = g * BN + wn * WN + j * 16 + (lane & 15);
          bv[g][j] = Bs[buf][n * 8 + swz(n, c)];
        }
#pragma unroll
      for (int g = 0; g < NB; ++g)
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j) Mfma<T>::run(af[i], bv[g][j], acc[g][i][j]);
    }
  };

  load(0);
  store(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) load(kt + 1);
    compute(cur);
    if (kt + 1 < nk) store(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue: lane holds column (lane & 15), rows 4*(lane>>4) + 0..3 of
  // each 16 x 16 accumulator.
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int grow = m0 + wm * WM + i * 16 + 4 * (lane >> 4) + q;
        const int gcol = n0 + wn * WN + j * 16 + (lane & 15);
        if (grow >= row_end) continue;
        const int64_t o = (int64_t)grow * p.ldc + gcol;
        const float v0 = acc[0][i][j][q];
        if constexpr (EPI == Epi::Store) {
          static_cast<T*>(p.C)[o] = Elem<T>::from_f(v0);
        } else if constexpr (EPI == Epi::SwiGLU || EPI == Epi::SwiGLUSave) {
          const float v1 = acc[NB - 1][i][j][q];
          const float hv = v0 / (1.f + expf(-v0)) * v1;
          static_cast<T*>(p.C)[o] = Elem<T>::from_f(hv);
          if constexpr (EPI == Epi::SwiGLUSave) {
            static_cast<T*>(p.C2)[o] = Elem<T>::from_f(v0);
            static_cast<T*>(p.C3)[o] = Elem<T>::from_f(v1);
          }
        } else if constexpr (EPI == Epi::F32) {
          static_cast<float*>(p.C)[o] = v0;
        } else if constexpr (EPI == Epi::BiasF32) {
          if (gcol < p.N) static_cast<float*>(p.C)[o] = v0 + (p.bias ? p.bias[gcol] : 0.f);
        } else {  // AccF32
          float* C = static_cast<float*>(p.C) + (int64_t)e * p.c_estride;
          C[o] += v0;
          if constexpr (DUAL) {
            float* C2 = static_cast<float*>(p.C2) + (int64_t)e * p.c_estride;
            C2[o] += acc[1][i][j][q];
          }
        }
      }
}

template <typename T, Mode MODE, int BM, int BN, bool DUAL, bool A_K, bool B_K, bool KCAT, Epi EPI>
hipError_t launch(const Params& p, dim3 grid, hipStream_t st) {
  gemm_kernel<T, MODE, BM, BN, DUAL, A_K, B_K, KCAT, EPI><<<grid, kThreads, 0, st>>>(p);
  return hipGetLastError();
}

inline int pick_bn(int n, bool allow256) {
  if (allow256 && n % 256 == 0) return 256;
  if (n % 128 == 0) return 128;
  return 64;
}

}  // namespace gemm
}  // namespace moe
