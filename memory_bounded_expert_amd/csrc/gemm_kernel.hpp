// Grouped GEMM on gfx950 MFMA ("Grouped GEMM organizes computation by
// expert-aggregated batches": "Training Trillion-Parameter MoE ...",
// section 3.3): the definitions shared by both GEMM kernels (modes,
// epilogues, parameters, buffer resources, MFMA wrappers) and the
// register-staged kernel that runs the fp32 configuration.  bf16 products
// run the LDS-pipeline kernel of gemm_lds.hpp.
//
// The kernel templates serve every contraction of the layer:
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
// Two LDS stages fed from one (STAGES = 1) or two register stages: the
// global loads of the next K-tile(s) are in flight while the MFMAs consume
// the current one; one barrier per K-tile.  Operand loads are buffer loads
// from per-tile resources, so ragged edges read zeros without branches.
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

// ExpertIdx / ExpertIdxB: Expert with the K-rows of the M-contiguous A, or
// of the N-contiguous B, read through a row index (Params::k_rows; LDS
// pipeline only).
enum class Mode { Rows, Dense, Expert, ExpertIdx, ExpertIdxB };
// CEStats and CEGrad are the vocabulary-strip cross-entropy epilogues (LDS
// pipeline, Dense mode only).
// SwiGLUBwd is the SwiGLU backward fused into dY W_down^T (LDS pipeline,
// Rows mode only).
enum class Epi { Store, SwiGLU, SwiGLUSave, F32, BiasF32, AccF32, CEStats, CEGrad, SwiGLUBwd };

struct Params {
  const void* A;
  const void* A2;  // second K segment (KCAT)
  int64_t lda;
  const void* B;
  const void* B2;  // second operand group (DUAL) or second K segment (KCAT)
  int64_t ldb;
  int64_t b_estride;  // elements between experts' B (Rows mode)
  int64_t a_kt;  // > 0: A K-tile-major, element (r, k) at (k / 32) a_kt + 32 r + k % 32
  int64_t c_kt;  // > 0: C likewise, element (r, n) at (n / 32) c_kt + 32 r + n % 32
  void* C;
  void* C2;
  void* C3;
  int64_t ldc;
  int64_t c_estride;  // elements between experts' C (Expert mode)
  int M, N, K, Kseg;
  int ntiles;  // Rows mode: N-tiles per M-tile (N / BN)
  int tile_group;  // Expert mode: M-tiles per dispatch group (0 or 1: N-tile fastest)
  const int2* tiles;
  const int32_t* tile_count;
  const int32_t* offsets;  // Rows: expert row offsets; Expert: segment rows (or null: one of K)
  const float* bias;
  // Rows mode, LDS pipeline only: when set, row r of A is row
  // a_rows[r] / a_row_div of the matrix at A (a_src_rows rows): the permuted
  // input is read straight from X through the chunk's permutation.
  const int32_t* a_rows;
  int a_row_div;
  int64_t a_src_rows;
  // Epi::AccF32, LDS pipeline only: store the tile (C = tile) instead of
  // accumulating; experts with no rows then store zeros.
  int acc_init;
  // Epi::AccF32, LDS pipeline only (ignored with acc_init): load C into the
  // accumulators before the K loop and store the result, so that C + A B is
  // one fp32 accumulation chain continuing C's own.
  int acc_chain;
  // Epi::CEStats / Epi::CEGrad: the N columns of the tile grid are vocabulary
  // entries ce_col0 + n; ce_targets[row] is the row's target entry.
  const int32_t* ce_targets;
  int64_t ce_col0;
  float* ce_pmax;          // CEStats: [slice][M] max of a 1-wave column slice
  float* ce_psum;          // CEStats: [slice][M] sum of exp(logit - that max)
  float* ce_ytgt;          // CEStats: [M] the target's logit (its slice writes it)
  const float* ce_lse;     // CEGrad: [M] log-normaliser
  const float* ce_dl;      // CEGrad: [M] upstream gradient, 0 for ignored rows
  // Epi::SwiGLUBwd: C = h (then g h), C2 = a (then da), C3 = u (then du),
  // row r's pair sw_perm[r] (< sw_nk) and its gate; sw_dgp[n-tile][row]
  // (row stride sw_rows) receives the tile's share of sum_f dh' h.
  const int32_t* sw_perm;
  const float* sw_gates;
  float* sw_dgp;
  int64_t sw_rows;
  int64_t sw_nk;
  // Mode::ExpertIdx (ExpertIdxB): K-row r of expert e's segment (row
  // offsets[e] + r of the chunk) is row floor(k_rows[offsets[e] + r] / d) of
  // the k_src_rows-row matrix at A (B), instead of row offsets[e] + r.
  // k_row_mul = ceil(2^32 / d) for d >= 2 (0 for d = 1), so that
  // floor(n / d) = mulhi(n, k_row_mul), exact for n * d < 2^32; the source's
  // bytes must stay below 2^31.
  const int32_t* k_rows;
  uint32_t k_row_mul;
  int64_t k_src_rows;
  // Epi::Store in Mode::Rows: row r (of the chunk) is multiplied by
  // row_scale[r] in fp32 before its one rounding (nullptr: unscaled).  The
  // down projection passes its rows' gates.
  const float* row_scale;
};

__device__ __forceinline__ int swz(int row, int c) { return c ^ (row & 7); }

// Buffer resource over [base, base + bytes): a load whose offset lies past
// `bytes` returns zeros, so ragged tiles need no branches.  Word 3 is the
// gfx9 raw-buffer format (32-bit data, no swizzle).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int n = (int)(bytes < 0 ? 0 : (bytes > 0x7FFFFFF0 ? 0x7FFFFFF0 : bytes));
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}
constexpr uint32_t kOob = 0x7FFFFFF0u;  // an offset no resource covers
// A pointer that is the same in every lane of the wave, moved to scalar
// registers (the compiler cannot always prove the uniformity itself).
template <typename P>
__device__ __forceinline__ P* wave_uniform(P* ptr) {
  const uint64_t v = reinterpret_cast<uint64_t>(ptr);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<P*>(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ u32x4_t bload(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}

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

// Work-group ids are handed out round-robin over the 8 XCDs (id mod 8), each
// with its own L2.  Renumbers id L of a grid of `total` work-groups so that
// every XCD runs one contiguous range of the new ids (a bijection on
// [0, total)).
constexpr int kCus = 256;  // compute units (MI355X: 8 XCDs of 32)

__device__ __forceinline__ int xcd_contiguous(int L, int total) {
  const int xcd = L & 7, slot = L >> 3;
  const int q = total >> 3, r = total & 7;
  return xcd < r ? xcd * (q + 1) + slot : r * (q + 1) + (xcd - r) * q + slot;
}

// The (expert, rows, N-tile) tile that renumbered id lid of a row-grouped
// grid computes.  An expert's M-tiles are consecutive in the tile list and
// start at offsets[e] + i * bm, so its ids are the range [first * ntiles,
// (first + me) * ntiles); inside that range they run N-tile major, M-tile
// minor.  The me work-groups that read one slice of the expert's weights
// then have adjacent ids, so they run at the same time on one XCD and share
// the slice in its L2, and the ntiles work-groups that read one M-tile's
// rows lie within me * ntiles ids of each other.
struct RowsTile {
  int e, m0, nt, row_end;
};
__device__ __forceinline__ RowsTile rows_tile(const int2* tiles, const int32_t* offsets, int lid,
                                              int ntiles, int bm) {
  const int mtg = lid / ntiles;
  const int2 tl = tiles[mtg];
  const int seg0 = offsets[tl.x], seg1 = offsets[tl.x + 1];
  const int me = (seg1 - seg0 + bm - 1) / bm;
  const int local = lid - (mtg - (tl.y - seg0) / bm) * ntiles;
  const int nt = local / me;
  return RowsTile{tl.x, seg0 + (local - nt * me) * bm, nt, seg1};
}

// Weight-gradient grids are (M-tiles, N-tiles, experts).  The tiles of one
// expert all read that expert's activation rows, so they go to one XCD (the
// renumbered ids run expert by expert) and the rows are fetched into one L2
// instead of eight.  Inside an expert the ids run N-tile fastest, or, with
// group > 1, in groups of `group` M-tiles (the last may be short) with the
// M-tile fastest inside a group: then the work-groups an XCD runs together
// form a group x (their number / group) block of tiles that shares its
// A and B K-tiles through L2 -- what a long K (many rows) needs.
struct ExpertTile {
  int e, mt, nt;
};
__device__ __forceinline__ ExpertTile expert_tile(int group) {
  const int gx = gridDim.x, gy = gridDim.y, per = gx * gy;
  const int L = blockIdx.x + gx * (blockIdx.y + gy * blockIdx.z);
  const int lid = xcd_contiguous(L, per * gridDim.z);
  ExpertTile t;
  t.e = lid / per;
  const int rem = lid - t.e * per;
  if (group > 1) {
    const int span = group * gy;
    const int grp = rem / span;
    const int gsz = min(group, gx - grp * group);
    const int r = rem - grp * span;
    t.nt = r / gsz;
    t.mt = grp * group + (r - t.nt * gsz);
  } else {
    t.mt = rem / gy;
    t.nt = rem - t.mt * gy;
  }
  return t;
}

template <typename T, Mode MODE, int BM, int BN, bool DUAL, bool A_K, bool B_K, bool KCAT, Epi EPI,
          int STAGES = 1>
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
  // a B operand group must cover whole waves of loading threads
  static_assert(!DUAL || (B_K ? (BN * 8) % 64 == 0 : (BN * 8 / EPC) % 64 == 0),
                "operand group not wave-aligned");

  __shared__ u32x4_t As[2][BM * 8];
  __shared__ u32x4_t Bs[2][NCOL * 8];

  const int tid = threadIdx.x;
  int e = 0, m0 = 0, row_end = 0;
  int n0 = blockIdx.y * BN;
  int64_t k_begin = 0;
  int k_len = p.K;
  if constexpr (MODE == Mode::Rows) {
    // 1-D grid over (M-tile, N-tile) pairs, sized for the worst case; the
    // chunk's real M-tile count is on the device.  Hardware hands out
    // work-group ids round-robin over the 8 XCDs (each with its own L2), so
    // the ids are renumbered to give every XCD a contiguous run of tiles in
    // (M-tile, N-tile) order: the work-groups an XCD runs together then share
    // their A rows (same M-tile) and their expert's weights (neighbouring
    // M-tiles) through that XCD's L2.
    const int total = *p.tile_count * p.ntiles;
    const int L = blockIdx.x;
    if (L >= total) return;
    const int lid = xcd_contiguous(L, total);
    const int mt = lid / p.ntiles;
    n0 = (lid - mt * p.ntiles) * BN;
    const int2 tl = p.tiles[mt];
    e = tl.x;
    m0 = tl.y;
    row_end = p.offsets[e + 1];
  } else if constexpr (MODE == Mode::Dense) {
    m0 = blockIdx.x * BM;
    row_end = p.M;
  } else {
    const ExpertTile t = expert_tile(p.tile_group);
    e = t.e;
    k_begin = p.offsets[e];
    k_len = p.offsets[e + 1] - (int)k_begin;
    if (k_len <= 0) return;
    m0 = t.mt * BM;
    n0 = t.nt * BN;
    row_end = p.M;
  }
  // The tile descriptor is the same for the whole work-group; make that
  // visible so addresses and buffer resources stay in scalar registers.
  e = __builtin_amdgcn_readfirstlane(e);
  m0 = __builtin_amdgcn_readfirstlane(m0);
  n0 = __builtin_amdgcn_readfirstlane(n0);
  row_end = __builtin_amdgcn_readfirstlane(row_end);
  k_len = __builtin_amdgcn_readfirstlane(k_len);
  k_begin = (int64_t)__builtin_amdgcn_readfirstlane((int)k_begin);
  const T* Ap = static_cast<const T*>(p.A);
  const T* A2p = static_cast<const T*>(p.A2);
  const int64_t boff = (MODE == Mode::Rows) ? (int64_t)e * p.b_estride : 0;
  const T* Bp = static_cast<const T*>(p.B) + boff;
  const T* B2p = (DUAL || KCAT) ? static_cast<const T*>(p.B2) + boff : nullptr;
  const int nk = (k_len + BK - 1) / BK;
  constexpr int64_t TS = sizeof(T);
  // Per-tile resources: every offset below is relative to the tile's first
  // row / column and stays far below 2^31.
  rsrc_t rA, rA2, rB, rB2;
  if constexpr (A_K) {
    const int64_t rows = (int64_t)min(row_end - m0, BM);
    rA = make_rsrc(Ap + (int64_t)m0 * p.lda, rows * p.lda * TS);
    rA2 = make_rsrc(KCAT ? A2p + (int64_t)m0 * p.lda : Ap, KCAT ? rows * p.lda * TS : 0);
  } else {
    rA = make_rsrc(Ap + k_begin * p.lda + m0, (int64_t)k_len * p.lda * TS);
    rA2 = rA;
  }
  if constexpr (B_K) {
    rB = make_rsrc(Bp + (int64_t)n0 * p.ldb, (int64_t)BN * p.ldb * TS);
    rB2 = make_rsrc(B2p ? B2p + (int64_t)n0 * p.ldb : Bp, B2p ? (int64_t)BN * p.ldb * TS : 0);
  } else if constexpr (MODE == Mode::Expert) {
    rB = make_rsrc(Bp + k_begin * p.ldb + n0, (int64_t)k_len * p.ldb * TS);
    rB2 = make_rsrc(B2p ? B2p + k_begin * p.ldb + n0 : Bp, B2p ? (int64_t)k_len * p.ldb * TS : 0);
  } else {
    rB = make_rsrc(Bp + n0, (int64_t)p.K * p.ldb * TS);
    rB2 = make_rsrc(B2p ? B2p + n0 : Bp, B2p ? (int64_t)p.K * p.ldb * TS : 0);
  }
  // N-major B of a DUAL tile: per-group base and size, for resources built
  // from a wave-uniform pointer inside the load loop
  const T* bt0 = (MODE == Mode::Expert) ? Bp + k_begin * p.ldb + n0 : Bp + n0;
  const T* bt1 = B2p ? ((MODE == Mode::Expert) ? B2p + k_begin * p.ldb + n0 : B2p + n0) : bt0;
  const int64_t bbytes = (MODE == Mode::Expert ? (int64_t)k_len : (int64_t)p.K) * p.ldb * TS;

  u32x4_t ra0[A_REGS], rb0[B_REGS];
  u32x4_t ra1[STAGES > 1 ? A_REGS : 1], rb1[STAGES > 1 ? B_REGS : 1];
  f32x4_t acc[NB][FM][FN];
#pragma unroll
  for (int g = 0; g < NB; ++g)
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[g][i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  auto load = [&](int kt, auto& ra, auto& rb) __attribute__((always_inline)) {
    const int k0 = kt * BK;
    // ---- A
    if constexpr (A_K) {
      bool second = false;
      int kk = k0;
      if constexpr (KCAT) {
        second = k0 >= p.Kseg;
        kk = second ? k0 - p.Kseg : k0;
      }
#pragma unroll
      for (int u = 0; u < A_UNITS; ++u) {
        const int lin = tid + u * kThreads;
        const int m = lin >> 3, c = lin & 7;
        const uint32_t off = (uint32_t)((m * p.lda + kk + c * EPC) * TS);
        ra[u] = bload(second ? rA2 : rA, off);  // rows past the segment read zero
      }
    } else {
#pragma unroll
      for (int u = 0; u < A_UNITS; ++u) {
        const int blk = tid + u * kThreads;
        const int kb = blk & 7, mb = blk >> 3;
#pragma unroll
        for (int q = 0; q < EPC; ++q) {
          const int kr = k0 + kb * EPC + q;
          uint32_t off = (uint32_t)((kr * p.lda + mb * EPC) * TS);
          if constexpr (A_BLK % kThreads != 0) off = blk < A_BLK ? off : kOob;
          ra[u * EPC + q] = bload(rA, off);  // rows past k_len read zero
        }
      }
    }
    // ---- B
    if constexpr (B_K) {
      bool second = false;
      int kk = k0;
      if constexpr (KCAT) {
        second = k0 >= p.Kseg;
        kk = second ? k0 - p.Kseg : k0;
      }
#pragma unroll
      for (int u = 0; u < B_UNITS; ++u) {
        const int lin = tid + u * kThreads;
        const int n = lin >> 3, c = lin & 7;
        const int g = DUAL ? n / BN : 0;
        const int nin = n - g * BN;
        const uint32_t off = (uint32_t)((nin * p.ldb + kk + c * EPC) * TS);
        rb[u] = bload(((DUAL && g) || second) ? rB2 : rB, off);
      }
    } else {
#pragma unroll
      for (int u = 0; u < B_UNITS; ++u) {
        const int blk = tid + u * kThreads;
        const int kb = blk & 7, nb = blk >> 3;
        const int ncol = nb * EPC;
        // each operand group spans whole waves (static_assert above), so the
        // group, and with it the resource, is wave-uniform
        const int g = DUAL ? ncol / BN : 0;
        const int nin = ncol - g * BN;
        rsrc_t r = rB;
        if constexpr (DUAL) r = make_rsrc(wave_uniform(g ? bt1 : bt0), bbytes);
        bool colok = true;
        if constexpr (B_BLK % kThreads != 0) colok = blk < B_BLK;
        if constexpr (MODE == Mode::Dense) colok = colok && n0 + nin < p.N;
#pragma unroll
        for (int q = 0; q < EPC; ++q) {
          const int kr = k0 + kb * EPC + q;
          const uint32_t off = colok ? (uint32_t)((kr * p.ldb + nin) * TS) : kOob;
          rb[u * EPC + q] = bload(r, off);
        }
      }
    }
  };

  auto store = [&](int buf, const auto& ra, const auto& rb) __attribute__((always_inline)) {
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
        if (A_BLK % kThreads == 0 || blk < A_BLK) {
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
        if (B_BLK % kThreads == 0 || blk < B_BLK) {
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

  if constexpr (STAGES == 1) {
    // two LDS stages fed from one register stage: the loads of tile t+1 are
    // in flight while the MFMAs consume tile t
    load(0, ra0, rb0);
    store(0, ra0, rb0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const int cur = kt & 1;
      if (kt + 1 < nk) load(kt + 1, ra0, rb0);
      compute(cur);
      if (kt + 1 < nk) store(cur ^ 1, ra0, rb0);
      __syncthreads();
    }
  } else {
    // two LDS stages fed from two register stages (tiles t+1 and t+2 in
    // flight), unrolled by two so each register set is named statically;
    // prefetches past the last tile reload it (clamped) instead of branching
    const int last = nk - 1;
    load(0, ra0, rb0);
    load(min(1, last), ra1, rb1);
    store(0, ra0, rb0);
    __syncthreads();
    for (int kt = 0; kt < nk; kt += 2) {
      load(min(kt + 2, last), ra0, rb0);
      compute(0);
      store(1, ra1, rb1);
      __syncthreads();
      if (kt + 1 >= nk) break;
      load(min(kt + 3, last), ra1, rb1);
      compute(1);
      store(0, ra0, rb0);
      __syncthreads();
    }
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
          float gv = 1.f;
          if constexpr (MODE == Mode::Rows) {
            if (p.row_scale) gv = p.row_scale[grow];
          }
          static_cast<T*>(p.C)[o] = Elem<T>::from_f(v0 * gv);
        } else if constexpr (EPI == Epi::SwiGLU || EPI == Epi::SwiGLUSave) {
          const float v1 = acc[NB - 1][i][j][q];
          // silu with the hardware exp and reciprocal (about 1 ulp each)
          const float hv = __fdividef(v0, 1.f + __expf(-v0)) * v1;
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
