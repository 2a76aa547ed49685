// Order-invariant expert weight gradients (opt-in plan flag MOE_PLAN_EXACT_DW).
//
// The pages require the chunked computation to reach exactly the unchunked
// values and gradients, only in another order ("Bounded-streaming operators"
// summary, Design Requirements).  The expert weight gradients sum over
// tokens, and strided chunks reorder that sum; an fp32 sum then differs in
// its last bits.  Here every summand is made exact and the sum is taken in
// integers, so no order can change it:
//
//  * Each operand column gets a power-of-two quantum from its largest
//    magnitude over the whole batch: X and dY per column h (one pass over
//    the batch), da, du and g h per expert and column f (a first pass over
//    the chunks that runs the recompute and the dh GEMM only).  A column
//    whose largest magnitude m satisfies m < 2^e maps x to the integer
//    v = rint(x 2^(14-e)), |v| <= 2^14 -- a function of the value and the
//    whole batch, not of the chunking.
//  * v = 256 hi + lo with lo in [-128, 127] and hi in [-64, 64] (two int8
//    digits), so an operand product is 2^16 hi hi' + 2^8 (hi lo' + lo hi') +
//    lo lo': three exact int32 sums per output element (v_mfma_i32_16x16x64_i8;
//    at most 2^14 per term and at most 65,536 rows per expert and chunk keep
//    every partial below 2^31), combined into an exact int64 and added into
//    a 64-bit accumulator per weight element chunk by chunk.
//  * After the last chunk each accumulator becomes fp32 with one rounding:
//    dW = acc 2^((eA - 14) + (eB - 14)).
//
// The GEMM reads both operands K-contiguous: per chunk, the digit planes of
// the expert rows are written transposed ([column][row]), each expert's
// segment padded to a multiple of 64 rows with zero digits.
#include "device_common.hpp"
#include "gemm_lds.hpp"  // make_srd, lds_load16, lds_barrier, wait_vmcnt, kswz, expert_tile
#include "moe_internal.h"

namespace moe {
namespace {

using gemm::i32x4_t;

typedef int i32x4v_t __attribute__((ext_vector_type(4)));

constexpr int kQBits = 14;  // |v| <= 2^14

// e with m < 2^e for the non-negative float with bit pattern mbits (the
// biased exponent minus 126 for a normal number; subnormals and zero take
// the smallest normal's).
__device__ __forceinline__ int col_exp(uint32_t mbits) {
  const int be = (int)((mbits >> 23) & 0xFF);
  return (be == 0 ? 1 : be) - 126;
}

__device__ __forceinline__ void to_digits(float x, int e, int& hi, int& lo) {
  const int v = (int)rintf(ldexpf(x, kQBits - e));
  lo = ((v + 128) & 255) - 128;
  hi = (v - lo) >> 8;
}

// |x| of the 8 bf16 in a 16-byte chunk, as fp32 bit patterns (which order
// like the magnitudes), max-merged into m.
__device__ __forceinline__ void max_abs8(const u32x4_t& v, uint32_t* m) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m[2 * i] = max(m[2 * i], (w[i] & 0x7FFFu) << 16);
    m[2 * i + 1] = max(m[2 * i + 1], (w[i] >> 16 & 0x7FFFu) << 16);
  }
}

// ---- column maxima over a whole [N][C] bf16 matrix (X, dY)
constexpr int kColRows = 256;  // rows per work-group

__global__ __launch_bounds__(kThreads) void colmax_kernel(const bf16_t* __restrict__ src, int64_t N,
                                                          int C, uint32_t* __restrict__ out) {
  __shared__ uint32_t sm[4][64 * 8];
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  const int c0 = (blockIdx.x * 64 + tx) * 8;
  const int64_t r0 = (int64_t)blockIdx.y * kColRows;
  const int64_t r1 = min(N, r0 + kColRows);
  uint32_t m[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (c0 < C)
    for (int64_t r = r0 + ty; r < r1; r += 4)
      max_abs8(*reinterpret_cast<const u32x4_t*>(src + r * C + c0), m);
#pragma unroll
  for (int j = 0; j < 8; ++j) sm[ty][tx * 8 + j] = m[j];
  __syncthreads();
  if (ty == 0 && c0 < C) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t v = max(max(sm[0][tx * 8 + j], sm[1][tx * 8 + j]),
                             max(sm[2][tx * 8 + j], sm[3][tx * 8 + j]));
      if (v) atomicMax(out + c0 + j, v);
    }
  }
}

// ---- per expert column maxima over a chunk's rows of da, du and g h ([R][C]
// bf16 each, expert segments offsets[e] .. offsets[e+1])
constexpr int kSegRows = 64;

__global__ __launch_bounds__(kThreads) void colmax_rows_kernel(
    const bf16_t* __restrict__ a, const bf16_t* __restrict__ u, const bf16_t* __restrict__ h,
    const int32_t* __restrict__ offsets, int E, int C, uint32_t* __restrict__ amax,
    uint32_t* __restrict__ umax, uint32_t* __restrict__ hmax) {
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  const int c0 = (blockIdx.x * 64 + tx) * 8;
  const int R = offsets[E];
  const int r0 = blockIdx.y * kSegRows;
  if (c0 >= C || r0 >= R) return;
  const int r1 = min(R, r0 + kSegRows);
  int r = r0 + ty;
  if (r >= r1) return;
  // expert of row r: the last e with offsets[e] <= r
  int lo = 0, hi = E - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (offsets[mid] <= r) lo = mid; else hi = mid - 1;
  }
  int e = lo;
  uint32_t ma[8] = {0, 0, 0, 0, 0, 0, 0, 0}, mu[8] = {0, 0, 0, 0, 0, 0, 0, 0},
           mh[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  auto flush = [&]() {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (ma[j]) atomicMax(amax + (int64_t)e * C + c0 + j, ma[j]);
      if (mu[j]) atomicMax(umax + (int64_t)e * C + c0 + j, mu[j]);
      if (mh[j]) atomicMax(hmax + (int64_t)e * C + c0 + j, mh[j]);
      ma[j] = mu[j] = mh[j] = 0;
    }
  };
  for (; r < r1; r += 4) {
    while (r >= offsets[e + 1]) {  // rows ascend, so experts only move forward
      flush();
      ++e;
    }
    const int64_t o = (int64_t)r * C + c0;
    max_abs8(*reinterpret_cast<const u32x4_t*>(a + o), ma);
    max_abs8(*reinterpret_cast<const u32x4_t*>(u + o), mu);
    max_abs8(*reinterpret_cast<const u32x4_t*>(h + o), mh);
  }
  flush();
}

// ---- padded segment starts of a chunk: offpad[e] = sum over e' < e of
// count_e' rounded up to 64 (E <= 1024, one work-group)
__global__ __launch_bounds__(1024) void pad_offsets_kernel(const int32_t* __restrict__ offsets,
                                                          int E, int32_t* __restrict__ offpad) {
  __shared__ int32_t s[1024];
  const int t = threadIdx.x;
  const int cnt = t < E ? offsets[t + 1] - offsets[t] : 0;
  s[t] = (cnt + 63) & ~63;
  __syncthreads();
  for (int d = 1; d < 1024; d <<= 1) {
    const int v = t >= d ? s[t - d] : 0;
    __syncthreads();
    s[t] += v;
    __syncthreads();
  }
  if (t < E) offpad[t + 1] = s[t];
  if (t == 0) offpad[0] = 0;
}

// ---- digit planes of one chunk, transposed and padded (see the header)
constexpr int kDigitMats = 5;

struct DigitSrc {
  const bf16_t* src;      // rows of ld elements
  int64_t ld;
  int C;                  // columns
  const int32_t* rows;    // chunk row -> source row (rows[r] / row_div), or nullptr
  int row_div;
  const uint32_t* cmax;   // column maxima: [C], or [E][C] when per_expert
  int per_expert;
  int8_t* hi;             // [C][ldk]
  int8_t* lo;
};
struct DigitArgs {
  DigitSrc s[kDigitMats];
  const int32_t* offsets;  // [E+1] chunk segments
  const int32_t* offpad;   // [E+1] padded segment starts
  int E;
  int64_t ldk;
};

constexpr int kDigitColBlocks = 4;  // 64-column blocks per work-group
__global__ __launch_bounds__(kThreads) void digitize_kernel(const DigitArgs a) {
  __shared__ int8_t shi[64][64 + 16];
  __shared__ int8_t slo[64][64 + 16];
  __shared__ int se;
  const DigitSrc& s = a.s[blockIdx.z];
  const int rp0 = blockIdx.x * 64;
  const int cb0 = blockIdx.y * kDigitColBlocks * 64;
  if (cb0 >= s.C || rp0 >= a.offpad[a.E]) return;  // (uniform over the work-group)
  const int t = threadIdx.x;
  if (t == 0) {
    // the expert whose padded segment holds rp0: the last e with offpad[e] <= rp0
    int lo = 0, hi = a.E - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a.offpad[mid] <= rp0) lo = mid; else hi = mid - 1;
    }
    se = lo;
  }
  __syncthreads();
  const int e = se;
  const int rel0 = rp0 - a.offpad[e];
  const int cnt = a.offsets[e + 1] - a.offsets[e];
  const int rbase = a.offsets[e];
  const int cc = t & 7;  // this thread's 8 columns of a block: c0 + cc*8 .. +8
  // this thread's two source rows (64-row block, two passes of 32), the same
  // for every column block
  int64_t srow[2];
  bool have[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int r = (t + q * kThreads) >> 3;  // 0..63
    const int rel = rel0 + r;
    have[q] = rel < cnt;
    const int row = rbase + (have[q] ? rel : 0);
    srow[q] = s.rows ? (int64_t)(s.rows[row] / s.row_div) : (int64_t)row;
  }
  for (int b = 0; b < kDigitColBlocks; ++b) {
    const int c0 = cb0 + b * 64;
    if (c0 >= s.C) break;  // (uniform)
    // both rows' loads first, then their digits
    u32x4_t raw[2];
#pragma unroll
    for (int q = 0; q < 2; ++q)
      raw[q] = have[q] ? *reinterpret_cast<const u32x4_t*>(s.src + srow[q] * s.ld + c0 + cc * 8)
                       : u32x4_t{0u, 0u, 0u, 0u};
    int ex[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      ex[j] = col_exp(s.cmax[(s.per_expert ? (int64_t)e * s.C : 0) + c0 + cc * 8 + j]);
    if (b > 0) __syncthreads();  // the previous block's planes have left LDS
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int r = (t + q * kThreads) >> 3;
      float v[8];
      unpack16(raw[q], v, bf16_t());
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        int dh, dl;
        to_digits(v[j], ex[j], dh, dl);
        shi[cc * 8 + j][r] = (int8_t)dh;
        slo[cc * 8 + j][r] = (int8_t)dl;
      }
    }
    __syncthreads();
    const int c = t >> 2, part = t & 3;
    const int64_t o = (int64_t)(c0 + c) * a.ldk + rp0 + part * 16;
    *reinterpret_cast<u32x4_t*>(s.hi + o) = *reinterpret_cast<const u32x4_t*>(&shi[c][part * 16]);
    *reinterpret_cast<u32x4_t*>(s.lo + o) = *reinterpret_cast<const u32x4_t*>(&slo[c][part * 16]);
  }
}

// ---- the exact weight-gradient product: acc64[e][m][n] (+)= sum over the
// chunk's rows k of expert e of vA[m][k] vB[n][k], from the digit planes
struct ExactParams {
  const int8_t* a_hi;
  const int8_t* a_lo;  // [M][ldk]
  const int8_t* b_hi;
  const int8_t* b_lo;  // [N][ldk]
  int64_t ldk;
  const int32_t* offsets;
  const int32_t* offpad;
  uint32_t* c_lo;  // [E][M][N] low words
  int32_t* c_hi;   // [E][M][N] high words
  int M, N;
  int init;        // store instead of accumulate (the first chunk)
};

constexpr int kXBM = 128, kXBN = 64, kXBK = 64;  // tile; K-tile in bytes (int8 values)
constexpr int kXNS = 3;                           // LDS stages
constexpr int kXStage = (2 * kXBM + 2 * kXBN) * kXBK;
constexpr int kXPT = 6;                           // loads per thread per K-tile
static_assert(4 * 64 * 36 * 8 <= kXNS * kXStage, "epilogue staging must fit the stages");

__global__ __launch_bounds__(kThreads, 2) void exact_wgrad_kernel(const ExactParams p) {
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  const gemm::ExpertTile tl = gemm::expert_tile(1);
  const int e = __builtin_amdgcn_readfirstlane(tl.e);
  const int m0 = __builtin_amdgcn_readfirstlane(tl.mt * kXBM);
  const int n0 = __builtin_amdgcn_readfirstlane(tl.nt * kXBN);
  const int k_len = __builtin_amdgcn_readfirstlane(p.offsets[e + 1] - p.offsets[e]);
  const int kofs = __builtin_amdgcn_readfirstlane(p.offpad[e]);
  if (k_len <= 0 && !p.init) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;  // 2 x 2 waves of 64 x 32
  const int l16 = lane & 15, lg = lane >> 4;
  const int nk = (k_len + kXBK - 1) / kXBK;
  const int last = nk - 1;

  const i32x4_t rAh = gemm::make_srd(p.a_hi + (int64_t)m0 * p.ldk + kofs, (int64_t)kXBM * p.ldk);
  const i32x4_t rAl = gemm::make_srd(p.a_lo + (int64_t)m0 * p.ldk + kofs, (int64_t)kXBM * p.ldk);
  const i32x4_t rBh = gemm::make_srd(p.b_hi + (int64_t)n0 * p.ldk + kofs, (int64_t)kXBN * p.ldk);
  const i32x4_t rBl = gemm::make_srd(p.b_lo + (int64_t)n0 * p.ldk + kofs, (int64_t)kXBN * p.ldk);
  const uint32_t ldk = (uint32_t)p.ldk;

  // K-tile kt into stage s: each wave loads 16-row pieces 2w, 2w+1 of each A
  // plane and piece w of each B plane (lane L of a piece: row L/4, 16-byte
  // chunk L%4, swizzled as the fragment reads expect)
  auto issue = [&](int kt, int s) __attribute__((always_inline)) {
    unsigned char* st = smem + s * kXStage;
    const int pos = lane & 3;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int ins = 2 * wave + u;
      const int row = ins * 16 + (lane >> 2);
      const uint32_t off = (uint32_t)row * ldk + (uint32_t)(kt * kXBK + ((pos ^ gemm::kswz<4>(row)) << 4));
      gemm::lds_load16(rAh, st + ins * 1024, off);
      gemm::lds_load16(rAl, st + kXBM * kXBK + ins * 1024, off);
    }
    {
      const int row = wave * 16 + (lane >> 2);
      const uint32_t off = (uint32_t)row * ldk + (uint32_t)(kt * kXBK + ((pos ^ gemm::kswz<4>(row)) << 4));
      gemm::lds_load16(rBh, st + 2 * kXBM * kXBK + wave * 1024, off);
      gemm::lds_load16(rBl, st + 2 * kXBM * kXBK + kXBN * kXBK + wave * 1024, off);
    }
  };

  i32x4v_t acc[3][4][2];
#pragma unroll
  for (int c = 0; c < 3; ++c)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[c][i][j] = i32x4v_t{0, 0, 0, 0};

  if (nk > 0) {
#pragma unroll
    for (int s = 0; s < kXNS - 1; ++s) issue(min(s, last), s);
    for (int kt = 0; kt < nk; ++kt) {
      gemm::wait_vmcnt<(kXNS - 2) * kXPT>();  // tile kt has landed (this thread's loads)
      gemm::lds_barrier();                   // ... everyone's; tile kt-1's stage is free
      issue(min(kt + kXNS - 1, last), (kt + kXNS - 1) % kXNS);
      const unsigned char* st = smem + (kt % kXNS) * kXStage;
      u32x4_t ah[4], al[4], bh[2], bl[2];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = wm * 64 + i * 16 + l16;
        const int o = row * kXBK + ((lg ^ gemm::kswz<4>(row)) << 4);
        ah[i] = *reinterpret_cast<const u32x4_t*>(st + o);
        al[i] = *reinterpret_cast<const u32x4_t*>(st + kXBM * kXBK + o);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int row = wn * 32 + j * 16 + l16;
        const int o = row * kXBK + ((lg ^ gemm::kswz<4>(row)) << 4);
        bh[j] = *reinterpret_cast<const u32x4_t*>(st + 2 * kXBM * kXBK + o);
        bl[j] = *reinterpret_cast<const u32x4_t*>(st + 2 * kXBM * kXBK + kXBN * kXBK + o);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const i32x4v_t a_h = __builtin_bit_cast(i32x4v_t, ah[i]);
          const i32x4v_t a_l = __builtin_bit_cast(i32x4v_t, al[i]);
          const i32x4v_t b_h = __builtin_bit_cast(i32x4v_t, bh[j]);
          const i32x4v_t b_l = __builtin_bit_cast(i32x4v_t, bl[j]);
          acc[0][i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a_h, b_h, acc[0][i][j], 0, 0, 0);
          acc[1][i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a_h, b_l, acc[1][i][j], 0, 0, 0);
          acc[1][i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a_l, b_h, acc[1][i][j], 0, 0, 0);
          acc[2][i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a_l, b_l, acc[2][i][j], 0, 0, 0);
        }
    }
    gemm::wait_vmcnt<0>();
  }

  // exact partial 2^16 hh + 2^8 (hl + lh) + ll (lane: rows 4 lg + q of
  // fragment row i, column l16), parked in this wave's share of the freed
  // stages (64 rows of 32 values, rows padded to 36 so the four row groups
  // of a write land in distinct banks), then added into the 64-bit
  // accumulator four columns at a time: 16-byte, row-contiguous accesses to
  // the low and high words, all of a lane's old values requested first
  // (non-temporal: each accumulator word is read and written once per
  // launch, and the digit planes that other tiles read stay in L2)
  constexpr int kLd = 36;
  gemm::lds_barrier();  // every wave is done with the operand stages
  int64_t* stg = reinterpret_cast<int64_t*>(smem + wave * (64 * kLd * 8));
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        stg[(i * 16 + 4 * lg + q) * kLd + j * 16 + l16] =
            ((int64_t)acc[0][i][j][q] << 16) + ((int64_t)acc[1][i][j][q] << 8) +
            (int64_t)acc[2][i][j][q];
  gemm::wave_lds_sync();
  constexpr int kIt = 64 * 32 / 4 / 64;  // 4-column pieces per lane
  int64_t base[kIt];
  u32x4_t olo[kIt], ohi[kIt];
#pragma unroll
  for (int it = 0; it < kIt; ++it) {
    const int item = lane + 64 * it, r = item >> 3, c4 = (item & 7) * 4;
    base[it] = ((int64_t)e * p.M + m0 + wm * 64 + r) * p.N + n0 + wn * 32 + c4;
    if (!p.init) {
      olo[it] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p.c_lo + base[it]));
      ohi[it] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p.c_hi + base[it]));
    }
  }
#pragma unroll
  for (int it = 0; it < kIt; ++it) {
    const int item = lane + 64 * it, r = item >> 3, c4 = (item & 7) * 4;
    u32x4_t lo, hi;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      int64_t v = stg[r * kLd + c4 + c];
      if (!p.init) v += (int64_t)(((uint64_t)ohi[it][c] << 32) | olo[it][c]);
      lo[c] = (uint32_t)(uint64_t)v;
      hi[c] = (uint32_t)(uint64_t)(v >> 32);
    }
    __builtin_nontemporal_store(lo, reinterpret_cast<u32x4_t*>(p.c_lo + base[it]));
    __builtin_nontemporal_store(hi, reinterpret_cast<u32x4_t*>(p.c_hi + base[it]));
  }
}

// ---- accumulators to fp32 in place: dW = acc 2^((eA - 14) + (eB - 14)),
// one rounding (the low words live in dW itself)
__global__ __launch_bounds__(kThreads) void exact_finalize_kernel(
    float* __restrict__ dw, const int32_t* __restrict__ c_hi, const uint32_t* __restrict__ amax,
    int a_per_expert, const uint32_t* __restrict__ bmax, int b_per_expert, int E, int M, int N) {
  const int64_t total = (int64_t)E * M * N;
  const int64_t i0 = ((int64_t)blockIdx.x * kThreads + threadIdx.x) * 4;
  if (i0 >= total) return;
  const int64_t mn = (int64_t)M * N;
  const int e = (int)(i0 / mn);
  const int64_t rem = i0 - (int64_t)e * mn;
  const int m = (int)(rem / N), n = (int)(rem - (int64_t)m * N);  // 4 columns n .. n+3 (N % 4 == 0)
  const int ea = col_exp(amax[(a_per_expert ? (int64_t)e * M : 0) + m]);
  uint32_t* lo = reinterpret_cast<uint32_t*>(dw);
  const u32x4_t l = *reinterpret_cast<const u32x4_t*>(lo + i0);
  const u32x4_t h = *reinterpret_cast<const u32x4_t*>(c_hi + i0);
  float out[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int eb = col_exp(bmax[(b_per_expert ? (int64_t)e * N : 0) + n + j]);
    const int64_t acc = (int64_t)(((uint64_t)h[j] << 32) | l[j]);
    out[j] = (float)ldexp((double)acc, (ea - kQBits) + (eb - kQBits));
  }
  *reinterpret_cast<f32x4_t*>(dw + i0) = f32x4_t{out[0], out[1], out[2], out[3]};
}

}  // namespace

hipError_t launch_colmax(const void* src, int64_t N, int C, uint32_t* out, hipStream_t st) {
  if (N == 0) return hipSuccess;
  const dim3 grid((unsigned)ceil_div(C, 512), (unsigned)ceil_div(N, kColRows));
  colmax_kernel<<<grid, kThreads, 0, st>>>(static_cast<const bf16_t*>(src), N, C, out);
  return hipGetLastError();
}

hipError_t launch_colmax_rows(const void* a, const void* u, const void* h, const int32_t* offsets,
                              int E, int C, int64_t max_rows, uint32_t* amax, uint32_t* umax,
                              uint32_t* hmax, hipStream_t st) {
  if (max_rows == 0) return hipSuccess;
  const dim3 grid((unsigned)ceil_div(C, 512), (unsigned)ceil_div(max_rows, kSegRows));
  colmax_rows_kernel<<<grid, kThreads, 0, st>>>(
      static_cast<const bf16_t*>(a), static_cast<const bf16_t*>(u),
      static_cast<const bf16_t*>(h), offsets, E, C, amax, umax, hmax);
  return hipGetLastError();
}

hipError_t launch_digitize(const ExactChunk& x, hipStream_t st, int* launches) {
  pad_offsets_kernel<<<1, 1024, 0, st>>>(x.offsets, x.E, x.offpad);
  if (hipError_t err = hipGetLastError(); err != hipSuccess) return err;
  if (launches) ++*launches;
  DigitArgs a{};
  const DigitPlanesSrc* in[kDigitMats] = {&x.X, &x.dY, &x.da, &x.du, &x.hg};
  int cmax_cols = 0;
  for (int z = 0; z < kDigitMats; ++z) {
    const DigitPlanesSrc& d = *in[z];
    a.s[z] = DigitSrc{static_cast<const bf16_t*>(d.src), d.ld, d.C, d.rows, d.row_div, d.cmax,
                      d.per_expert, d.hi, d.lo};
    cmax_cols = d.C > cmax_cols ? d.C : cmax_cols;
  }
  a.offsets = x.offsets;
  a.offpad = x.offpad;
  a.E = x.E;
  a.ldk = x.ldk;
  const dim3 grid((unsigned)(x.ldk / 64), (unsigned)ceil_div(cmax_cols, 64 * kDigitColBlocks),
                  kDigitMats);
  digitize_kernel<<<grid, kThreads, 0, st>>>(a);
  if (hipError_t err = hipGetLastError(); err != hipSuccess) return err;
  if (launches) ++*launches;
  return hipSuccess;
}

hipError_t launch_exact_wgrad(const int8_t* a_hi, const int8_t* a_lo, const int8_t* b_hi,
                              const int8_t* b_lo, int64_t ldk, const int32_t* offsets,
                              const int32_t* offpad, uint32_t* c_lo, int32_t* c_hi, int E, int M,
                              int N, bool init, hipStream_t st) {
  if (M % kXBM || N % kXBN) return hipErrorInvalidValue;
  static bool attr = false;
  if (hipError_t err = gemm::set_lds_attr(exact_wgrad_kernel, kXNS * kXStage, attr);
      err != hipSuccess)
    return err;
  ExactParams p{a_hi, a_lo, b_hi, b_lo, ldk, offsets, offpad, c_lo, c_hi, M, N, init ? 1 : 0};
  const dim3 grid((unsigned)(M / kXBM), (unsigned)(N / kXBN), (unsigned)E);
  exact_wgrad_kernel<<<grid, kThreads, kXNS * kXStage, st>>>(p);
  return hipGetLastError();
}

hipError_t launch_exact_finalize(float* dw, const int32_t* c_hi, const uint32_t* amax,
                                 bool a_per_expert, const uint32_t* bmax, bool b_per_expert, int E,
                                 int M, int N, hipStream_t st) {
  const int64_t total = (int64_t)E * M * N;
  if (total == 0) return hipSuccess;
  exact_finalize_kernel<<<(unsigned)ceil_div(total / 4, kThreads), kThreads, 0, st>>>(
      dw, c_hi, amax, a_per_expert, bmax, b_per_expert, E, M, N);
  return hipGetLastError();
}

}  // namespace moe
