// bf16 grouped GEMM on gfx950 with an LDS-only operand pipeline.
//
// Same contraction modes as gemm_kernel.hpp (Rows: expert segments of a
// chunk, M-tiles from the planner's device-side list; Dense: router, optionally
// split over K; Expert: weight gradients), v_mfma_f32_16x16x32_bf16 with fp32
// accumulation on a WGM x WGN grid of waves (Shape below), and the same K
// order for every output element -- so a row's result does not depend on
// which rows share its tile.  How operands reach the MFMAs:
//
//  * Every operand tile goes from HBM straight into LDS with buffer loads
//    that write LDS (16 bytes per lane; lane L of a wave lands at base +
//    16 L).  No staging registers, so 3 to 6 LDS stages fit and NS-1 K-tiles
//    are in flight per work-group while the MFMAs consume the current one.
//    Loads past a tile's valid rows (buffer resource bounds) write zeros.
//    The bf16 forward's gate/up product can take its A rows straight from X
//    through the chunk's permutation (Params::a_rows).
//  * K-contiguous operands (activation rows; weights in the transposed
//    products) are stored as rows of BK/8 chunks of 16 bytes with a
//    row-dependent XOR swizzle of the chunk index, read with ds_read_b128.
//  * M/N-contiguous operands (weights in the forward products; activations
//    in the weight gradients) stay M/N-contiguous in LDS and are read with
//    ds_read_b64_tr_b16: in each 16-lane group, lanes 4j..4j+3 address row j
//    and lane i receives column i of rows 0..3, so two reads give a lane the
//    8 consecutive k of one column that the MFMA operand needs.  Chunk c of
//    row k sits at c ^ sw(k); sw makes the 32 lanes of each half-wave hit 64
//    distinct banks.
//
// The global-side permutation that realises each swizzle is applied in the
// per-lane load offsets, so the LDS writes of a wave stay one contiguous KiB.
#pragma once

#include <type_traits>

#include "device_common.hpp"
#include "gemm_kernel.hpp"  // Mode, Epi, Params, make_rsrc, wave_uniform
#include "moe_internal.h"

namespace moe {
namespace gemm {

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t* lds_s16x4_p;
typedef __attribute__((address_space(3))) void* lds_void_p;

constexpr int kLdsBytes = 160 * 1024;

// swizzle of a row of RC 16-byte chunks read with the transposing loads
template <int RC>
__device__ __forceinline__ int trswz(int k) {
  if constexpr (RC >= 16) return 2 * ((k & 3) | (((k >> 3) & 1) << 2));
  else return 2 * (((k >> 1) & 1) | (((k >> 3) & 1) << 1));
}

// Buffer resource as four scalar dwords, for the inline-asm loads below.
typedef int i32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4_t make_srd(const void* base, int64_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const int n = (int)(bytes < 0 ? 0 : (bytes > 0x7FFFFFF0 ? 0x7FFFFFF0 : bytes));
  i32x4_t r;
  r.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r.y = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32) & 0xFFFF);  // stride 0
  r.z = __builtin_amdgcn_readfirstlane(n);
  r.w = 0x00020000;
  return r;
}

// 16 bytes per lane from a buffer straight into LDS at lds + 16 * lane.
// Written as inline asm on purpose: the compiler cannot tell that the LDS
// reads of the stage being computed do not alias the stages being filled, and
// would otherwise drain every load (vmcnt(0)) before each LDS read.  The
// pipeline does its own vmcnt accounting; no compiler-visible vector memory
// operation is outstanding while these are in flight.
__device__ __forceinline__ void lds_load16(const i32x4_t& srd, void* lds, uint32_t voff) {
  const uint32_t m0v =
      __builtin_amdgcn_readfirstlane((uint32_t)reinterpret_cast<uintptr_t>((lds_void_p)lds));
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(m0v), "v"(voff), "s"(srd)
               : "memory", "m0");
}

// The same with the LDS destination as a 32-bit LDS address (no conversion
// of a generic pointer per load)
__device__ __forceinline__ void lds_load16_at(const i32x4_t& srd, uint32_t lds_addr, uint32_t voff) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_addr);
  // (a resource chosen by a wave-uniform condition: kept in scalar registers)
  i32x4_t r;
  r.x = __builtin_amdgcn_readfirstlane(srd.x);
  r.y = __builtin_amdgcn_readfirstlane(srd.y);
  r.z = __builtin_amdgcn_readfirstlane(srd.z);
  r.w = __builtin_amdgcn_readfirstlane(srd.w);
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(m0v), "v"(voff), "s"(r)
               : "memory", "m0");
}

// 4 bytes per lane from a buffer straight into LDS at lds + 4 * lane (every
// lane writes, lanes past the resource write zeros)
__device__ __forceinline__ void lds_load4(const i32x4_t& srd, void* lds, uint32_t voff) {
  const uint32_t m0v =
      __builtin_amdgcn_readfirstlane((uint32_t)reinterpret_cast<uintptr_t>((lds_void_p)lds));
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :
               : "s"(m0v), "v"(voff), "s"(srd)
               : "memory", "m0");
}

// Work-group barrier for the LDS pipeline: waits for this wave's LDS reads
// only (outstanding global->LDS loads stay in flight across it).  The wait is
// the builtin, not inline asm, so that the compiler's own wait-count tracking
// knows every earlier LDS read has completed and inserts no further waits
// for those registers.  The immediate is the gfx9 s_waitcnt encoding with
// vmcnt and expcnt at their maxima (no wait) and lgkmcnt = 0.
__device__ __forceinline__ void lds_barrier() {
  constexpr int kWaitLgkm0 = 0xC07F;  // vmcnt 63, expcnt 7, lgkmcnt 0
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  __builtin_amdgcn_s_barrier();
}

// Orders one wave's LDS writes before its later LDS reads of other lanes'
// data (and those reads before later writes): the DS unit executes a wave's
// instructions in order, so waiting for this wave's own LDS operations
// (lgkmcnt 0) and keeping the compiler from moving memory operations across
// is enough; no work-group barrier.
__device__ __forceinline__ void wave_lds_sync() {
  constexpr int kWaitLgkm0 = 0xC07F;  // vmcnt 63, expcnt 7, lgkmcnt 0
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Rows per slice of a wave's WM x WN accumulator block in the weight-gradient
// read-modify-write: the largest power-of-two share of WM (at least one
// fragment row) whose padded rows fit the wave's LDS share and that gives each
// lane at most 8 vectors of 16 bytes, so two slices' old values fit in
// registers beside the accumulators.
template <int WM, int LD, int VW, int PWB>
constexpr int acc_slice_rows() {
  int sr = WM;
  while (sr > 16 && (sr * LD * 4 > PWB || sr * VW > 8 * 64)) sr /= 2;
  return sr;
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Work-group shape: BM x BN output tile (BN per operand group), WGM x WGN
// waves each owning a (BM/WGM) x (BN/WGN) block, K-tiles of BK, and the number
// of work-groups meant to share a CU (its LDS is split between them).
template <int BM_, int BN_, int WGM_, int WGN_, int BK_, int WG_PER_CU_>
struct Shape {
  static constexpr int BM = BM_, BN = BN_, WGM = WGM_, WGN = WGN_, BK = BK_;
  static constexpr int WG_PER_CU = WG_PER_CU_;
};

// KIDX: room for the row-indexed K slots (at most 6 stages of 256 bytes per
// wave) comes off the stages' budget
template <class S, bool DUAL, bool KIDX = false>
struct LdsCfg {
  static constexpr int BM = S::BM, BN = S::BN, BK = S::BK;
  static constexpr int NB = DUAL ? 2 : 1;
  static constexpr int NCOL = BN * NB;
  static constexpr int CK = BK / 8;  // 16-byte chunks per K-contiguous LDS row
  static constexpr int A_BYTES = BM * BK * 2;
  static constexpr int B_BYTES = NCOL * BK * 2;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int BUDGET = kLdsBytes / S::WG_PER_CU - (KIDX ? S::WGM * S::WGN * 6 * 256 : 0);
  static constexpr int NS_FIT = (BUDGET / STAGE) > 6 ? 6 : (BUDGET / STAGE);
  // an even stage count keeps the unrolled main loop at NS steps (the two
  // fragment register sets alternate); odd counts above 3 drop one stage
  static constexpr int NS = (NS_FIT % 2 == 1 && NS_FIT > 3) ? NS_FIT - 1 : NS_FIT;
  static constexpr int WAVES = S::WGM * S::WGN;
  static constexpr int THREADS = 64 * WAVES;
  // wave-instructions (1 KiB each) per tile, and per wave
  static constexpr int A_INSTR = A_BYTES / 1024;
  static constexpr int B_INSTR = B_BYTES / 1024;
  static constexpr int A_PW = A_INSTR / WAVES;
  static constexpr int B_PW = B_INSTR / WAVES;
  static constexpr int PER_TILE = A_PW + B_PW;  // loads per thread per K-tile
  static_assert(BK == 32 || BK == 64, "BK");
  static_assert(A_INSTR % WAVES == 0 && B_INSTR % WAVES == 0, "tile must split over the waves");
  static_assert(NS >= 3, "need at least three LDS stages");
};

// How an AccF32 kernel moves C: each wave carries its WM x WN block of C
// through a private share of the (then idle) operand stages, SR rows at a
// time, so that global memory sees 16-byte, row-contiguous accesses instead
// of the fragments' 4-byte scatter.  Rows are padded by 4 floats so the four
// row groups of a fragment land in distinct banks.
template <class S, class C>
struct AccGeom {
  static constexpr int WM = S::BM / S::WGM, WN = S::BN / S::WGN;
  static constexpr int LD = WN + 4;                        // padded row, floats
  static constexpr int VW = WN / 4;                        // 16-byte vectors per row
  static constexpr int PWB = C::NS * C::STAGE / C::WAVES;  // LDS bytes per wave
  static constexpr int SR = acc_slice_rows<WM, LD, VW, PWB>();
  static constexpr int NSL = WM / SR;                      // slices per operand group
  static constexpr int NSUB = C::NB * NSL;
  static constexpr int PER = SR * VW / 64;                 // vectors per lane per slice
  static constexpr int FS = SR / 16;                       // fragment rows per slice
  static_assert(SR % 16 == 0 && WM % SR == 0, "slices of whole fragment rows");
  static_assert(SR * LD * 4 <= PWB, "accumulator slice must fit the wave's LDS share");
  static_assert((SR * VW) % 64 == 0 && PER <= 8, "slice must split over the lanes");
};

// swizzle of a K-contiguous row of CK chunks (conflict-free ds_read_b128 of
// 16 rows x one chunk)
template <int CK>
__device__ __forceinline__ int kswz(int r) {
  if constexpr (CK == 8) return r & 7;
  else return (r >> 2) & 3;
}

// Row-indexed K (Mode::ExpertIdx, ExpertIdxB): K-rows per wave per K-tile (a
// wave's loads of an M-contiguous A or one N-contiguous B tile cover BK /
// WAVES consecutive rows), and the
// slots' place and size in LDS (past the stages; per wave, one 256-byte slot
// per stage, since a dword load into LDS writes all 64 lanes).
constexpr bool mode_kidx(Mode m) { return m == Mode::ExpertIdx || m == Mode::ExpertIdxB; }
template <int BK, int WAVES>
constexpr int kidx_rows() {
  static_assert(BK % WAVES == 0 && BK / WAVES <= 64, "index rows per wave");
  return BK / WAVES;
}
template <class C>
constexpr int kidx_offset() { return C::NS * C::STAGE; }
template <Mode MODE, class S, bool DUAL>
constexpr int lds_bytes() {
  using C = LdsCfg<S, DUAL, mode_kidx(MODE)>;
  constexpr int b = C::NS * C::STAGE + (mode_kidx(MODE) ? C::WAVES * C::NS * 256 : 0);
  static_assert(b <= kLdsBytes / S::WG_PER_CU, "LDS over the work-group's share");
  return b;
}

// The work-group's whole product.  bid is the work-group's index in a Rows
// grid (in a pair launch, its index in its own list's grid); the other modes
// read blockIdx themselves.
template <Mode MODE, class S, bool DUAL, bool A_K, bool B_K, bool KCAT, Epi EPI>
__device__ __forceinline__ void gemm_lds_body(const Params& p, int bid) {
  using C = LdsCfg<S, DUAL, mode_kidx(MODE)>;
  using T = bf16_t;
  constexpr int BM = S::BM, BN = S::BN, BK = S::BK, NB = C::NB, NS = C::NS, CK = C::CK;
  constexpr int WM = BM / S::WGM, WN = BN / S::WGN;
  constexpr int FM = WM / 16, FN = WN / 16;
  constexpr int KS = BK / 32;  // MFMA k-steps per K-tile
  constexpr int RCA = BM / 8;  // chunks per LDS row of an M-contiguous A tile
  constexpr int RCB = BN / 8;  // chunks per LDS row of an N-contiguous B group
  static_assert(FM >= 1 && FN >= 1, "wave tile too small");
  static_assert(!(DUAL && KCAT), "DUAL and KCAT are exclusive");
  static_assert(!(DUAL && B_K), "DUAL needs an N-contiguous B");
  static_assert(A_K || RCA >= 8, "M-contiguous A needs BM >= 64");
  constexpr bool KIDX_A = MODE == Mode::ExpertIdx, KIDX_B = MODE == Mode::ExpertIdxB;
  constexpr bool KIDX = KIDX_A || KIDX_B;
  constexpr bool EXPERT = MODE == Mode::Expert || KIDX;
  static_assert(!KIDX_A || (!A_K && !KCAT), "row-indexed K needs an M-contiguous A");
  static_assert(!KIDX_B || (!B_K && !DUAL && !KCAT), "row-indexed K needs one N-contiguous B");
  // loads per thread per K-tile (an indexed product adds its index block)
  constexpr int PT = C::PER_TILE + (KIDX ? 1 : 0);
  static_assert(B_K || RCB >= 8, "N-contiguous B needs BN >= 64");

  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];

  const int tid = threadIdx.x;
  // wave index in a scalar register: LDS destinations (M0) and operand-group
  // resources derive from it
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int e = 0, m0 = 0, row_end = 0;
  int n0 = blockIdx.y * BN;
  int64_t k_begin = 0;
  int k_len = p.K;
  if constexpr (MODE == Mode::Rows) {
    // XCD-aware renumbering of the 1-D grid (xcd_contiguous), then the
    // expert-local N-major order of rows_tile
    const int total = *p.tile_count * p.ntiles;
    if (bid >= total) return;
    const RowsTile t = rows_tile(p.tiles, p.offsets, xcd_contiguous(bid, total), p.ntiles, BM);
    e = t.e;
    m0 = t.m0;
    n0 = t.nt * BN;
    row_end = t.row_end;
  } else if constexpr (MODE == Mode::Dense) {
    // blockIdx.z: K slice of a split product (slice z covers
    // [z * Kseg, (z + 1) * Kseg) and writes the z-th partial output)
    m0 = blockIdx.x * BM;
    row_end = p.M;
    if (gridDim.z > 1) k_len = p.Kseg;
  } else {
    const ExpertTile t = expert_tile(p.tile_group);
    e = t.e;
    // segment e's rows; without offsets, one segment of K rows
    k_begin = p.offsets ? p.offsets[e] : 0;
    k_len = p.offsets ? p.offsets[e + 1] - (int)k_begin : p.K;
    if (k_len <= 0 && !p.acc_init) return;  // nothing to add
    m0 = t.mt * BM;
    n0 = t.nt * BN;
    row_end = p.M;
  }
  e = __builtin_amdgcn_readfirstlane(e);
  m0 = __builtin_amdgcn_readfirstlane(m0);
  n0 = __builtin_amdgcn_readfirstlane(n0);
  row_end = __builtin_amdgcn_readfirstlane(row_end);
  k_len = __builtin_amdgcn_readfirstlane(k_len);
  k_begin = (int64_t)__builtin_amdgcn_readfirstlane((int)k_begin);

  const int64_t kslice = (MODE == Mode::Dense && gridDim.z > 1) ? (int64_t)blockIdx.z * p.Kseg : 0;
  const T* Ap = static_cast<const T*>(p.A) + kslice;
  const T* A2p = static_cast<const T*>(p.A2);
  const int64_t boff = (MODE == Mode::Rows) ? (int64_t)e * p.b_estride : kslice * p.ldb;
  const T* Bp = static_cast<const T*>(p.B) + boff;
  const T* B2p = (DUAL || KCAT) ? static_cast<const T*>(p.B2) + boff : Bp;
  const int nk = (k_len + BK - 1) / BK;
  constexpr int64_t TS = 2;

  // ---- per-tile buffer resources (offsets below are tile-relative)
  i32x4_t rA, rA2, rB, rB2;
  // Row-indexed A (Rows mode): byte offset of the source row of each of this
  // lane's A-load rows, or kOob past the segment end.
  constexpr int RPIK = 64 / CK;  // K-contiguous rows per load instruction
  uint32_t arow[C::A_PW];
  const bool gathered = MODE == Mode::Rows && A_K && !KCAT && p.a_rows != nullptr;
  if constexpr (A_K) {
    const int64_t rows = (int64_t)min(row_end - m0, BM);
    if (gathered) {
      rA = make_srd(Ap, p.a_src_rows * p.lda * TS);
#pragma unroll
      for (int u = 0; u < C::A_PW; ++u) {
        const int row = (wave * C::A_PW + u) * RPIK + lane / CK;
        arow[u] = kOob;
        if (row < rows) {
          const int src = p.a_rows[m0 + row] / p.a_row_div;
          if ((uint64_t)src < (uint64_t)p.a_src_rows) arow[u] = (uint32_t)((int64_t)src * p.lda * TS);
        }
      }
    } else if (p.a_kt) {
      // K-tile-major A (BK = 32: one block per K-tile): the tile's rows of a
      // block are 64-byte rows; rows past the tile are masked (the resource
      // runs on through the other rows and blocks)
      rA = make_srd(Ap + (int64_t)m0 * 32, ((int64_t)p.K / 32 * p.a_kt - (int64_t)m0 * 32) * TS);
#pragma unroll
      for (int u = 0; u < C::A_PW; ++u) {
        const int row = (wave * C::A_PW + u) * RPIK + lane / CK;
        arow[u] = row < rows ? (uint32_t)(row * 32 * TS) : kOob;
      }
    } else {
      rA = make_srd(Ap + (int64_t)m0 * p.lda, rows * p.lda * TS);
#pragma unroll
      for (int u = 0; u < C::A_PW; ++u) {
        const int row = (wave * C::A_PW + u) * RPIK + lane / CK;
        arow[u] = (uint32_t)(row * p.lda * TS);
      }
    }
    rA2 = KCAT ? make_srd(A2p + (int64_t)m0 * p.lda, rows * p.lda * TS) : rA;
  } else if constexpr (KIDX_A) {
    // the whole source matrix from column m0: row offsets come per K-row
    rA = make_srd(Ap + m0, (p.k_src_rows * p.lda - m0) * TS);
    rA2 = rA;
  } else {
    rA = make_srd(Ap + k_begin * p.lda + m0, (int64_t)k_len * p.lda * TS);
    rA2 = rA;
  }
  if constexpr (B_K) {
    // (Dense: B rows past N -- the ragged end of a vocabulary strip -- read as zeros)
    const int64_t brows = MODE == Mode::Dense ? (int64_t)max(0, min(BN, p.N - n0)) : (int64_t)BN;
    rB = make_srd(Bp + (int64_t)n0 * p.ldb, brows * p.ldb * TS);
    rB2 = KCAT ? make_srd(B2p + (int64_t)n0 * p.ldb, (int64_t)BN * p.ldb * TS) : rB;
  } else {
    const int64_t rows = EXPERT ? (int64_t)k_len : (int64_t)p.K;
    const int64_t kb = EXPERT ? k_begin : 0;
    if constexpr (KIDX_B) {
      // the whole source matrix from column n0: row offsets come per K-row
      rB = make_srd(Bp + n0, (p.k_src_rows * p.ldb - n0) * TS);
    } else {
      rB = make_srd(Bp + kb * p.ldb + n0, (MODE == Mode::Dense ? (int64_t)k_len : rows) * p.ldb * TS);
    }
    rB2 = DUAL ? make_srd(B2p + kb * p.ldb + n0, rows * p.ldb * TS) : rB;
  }


  // ---- row-indexed K (Mode::ExpertIdx: A; ExpertIdxB: B).  A wave's loads
  // of that operand's K-tile cover KW consecutive K-rows.  Each wave keeps
  // the k_rows entries of its own rows in private LDS slots past the stages,
  // one 256-byte slot per stage: the slot of stage s holds the entries of
  // the tile that stage s receives next.  issue() reads its rows' entries
  // from the slot, then refills the slot with those of the tile the stage
  // receives NS tiles later, as one more load of the same K-tile: the
  // pipeline's waits then also cover the entries (only the wave that loaded
  // a slot reads it).
  constexpr int KW = kidx_rows<BK, C::WAVES>();
  i32x4_t rI{};
  uint32_t ibase = 0;  // this lane's first entry in slot 0 (LDS address)
  // entry n -> byte offset of its source row (kOob past the source), in
  // 32-bit arithmetic: the source's bytes stay below 2^31
  const uint32_t krow_bytes = (uint32_t)((KIDX_A ? p.lda : p.ldb) * TS);
  const uint32_t ksrc_rows = (uint32_t)p.k_src_rows;
  auto src_offset = [&](uint32_t n) __attribute__((always_inline)) -> uint32_t {
    const uint32_t src = p.k_row_mul ? __umulhi(n, p.k_row_mul) : n;
    return src < ksrc_rows ? src * krow_bytes : kOob;
  };
  if constexpr (KIDX) {
    rI = make_srd(p.k_rows + k_begin, (int64_t)k_len * 4);
    ibase = (uint32_t)reinterpret_cast<uintptr_t>((lds_void_p)smem) + kidx_offset<C>() +
            (uint32_t)(wave * NS * 256 + (lane / (KIDX_A ? RCA : RCB)) * 4);
  }
  auto load_idx = [&](int kt, int s) __attribute__((always_inline)) {
    const int r = kt * BK + wave * KW + lane;
    const uint32_t off = (lane < KW && r < k_len) ? (uint32_t)r * 4u : kOob;
    lds_load4(rI, smem + kidx_offset<C>() + (wave * NS + s) * 256, off);
  };

  // ---- per-lane parts of the load offsets (bytes; 32-bit, every resource
  // spans less than 2^31 bytes), computed once: issue() adds the K-tile's
  // wave-uniform part, so a K-step's loads cost one add each.  An offset of
  // kOob (rows past the segment end, B columns past N) stays past every
  // resource after the add.  The LDS destinations are 32-bit LDS addresses.
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane((uint32_t)reinterpret_cast<uintptr_t>((lds_void_p)smem));
  uint32_t aoff[C::A_PW], boff_l[C::B_PW];
  const uint32_t a_rowb = (uint32_t)(p.lda * TS), b_rowb = (uint32_t)(p.ldb * TS);  // row pitches
  // bytes from one 32-wide K block of a K-contiguous A to the next
  const uint32_t a_ktb = p.a_kt ? (uint32_t)(p.a_kt * TS) : (uint32_t)(32 * TS);
#pragma unroll
  for (int u = 0; u < C::A_PW; ++u) {
    const int ins = wave * C::A_PW + u;
    if constexpr (A_K) {
      const int row = ins * RPIK + lane / CK;
      const int c = (lane % CK) ^ kswz<CK>(row);
      aoff[u] = arow[u] == kOob ? kOob : arow[u] + (uint32_t)(c * 8 * TS);
    } else if constexpr (!KIDX_A) {
      constexpr int RPI = 64 / RCA;
      const int k = ins * RPI + lane / RCA;
      const int c = (lane % RCA) ^ trswz<RCA>(k);
      aoff[u] = (uint32_t)k * a_rowb + (uint32_t)(c * 8 * TS);
    } else {
      aoff[u] = 0;
    }
  }
#pragma unroll
  for (int u = 0; u < C::B_PW; ++u) {
    const int ins = wave * C::B_PW + u;
    if constexpr (B_K) {
      const int row = ins * RPIK + lane / CK;
      const int c = (lane % CK) ^ kswz<CK>(row);
      boff_l[u] = (uint32_t)row * b_rowb + (uint32_t)(c * 8 * TS);
    } else if constexpr (!KIDX_B) {
      constexpr int PER_G = BK * RCB / 64;
      constexpr int RPI = 64 / RCB;
      const int gi = ins % PER_G;
      const int k = gi * RPI + lane / RCB;
      const int c = (lane % RCB) ^ trswz<RCB>(k);
      bool ok = true;
      if constexpr (MODE == Mode::Dense) ok = n0 + c * 8 < p.N;
      boff_l[u] = ok ? (uint32_t)k * b_rowb + (uint32_t)(c * 8 * TS) : kOob;
    } else {
      boff_l[u] = 0;
    }
  }

  // ---- issue the loads of K-tile kt into LDS stage s (an indexed product
  // then loads the k_rows entries of tile kn into the stage's slot)
  auto issue = [&](int kt, int s, int kn) __attribute__((always_inline)) {
    const int k0 = kt * BK;
    bool second = false;  // K segment of a KCAT product (uniform)
    int kk = k0;
    if constexpr (KCAT) {
      second = k0 >= p.Kseg;
      kk = second ? k0 - p.Kseg : k0;
    }
    // A
#pragma unroll
    for (int u = 0; u < C::A_PW; ++u) {
      const int ins = wave * C::A_PW + u;
      const uint32_t dst = lds0 + (uint32_t)(s * C::STAGE + ins * 1024);
      if constexpr (A_K) {
        lds_load16_at(second ? rA2 : rA, dst, aoff[u] + (uint32_t)(kk >> 5) * a_ktb);
      } else {
        constexpr int RPI = 64 / RCA;
        const int k = ins * RPI + lane / RCA;
        const int kr = k0 + k;
        uint32_t off;
        if constexpr (KIDX_A) {
          // row k of the tile is entry u * RPI + lane / RCA of this wave's slot
          const int c = (lane % RCA) ^ trswz<RCA>(k);
          const uint32_t n = *reinterpret_cast<const __attribute__((address_space(3))) uint32_t*>(
              (uintptr_t)(ibase + (uint32_t)(s * 256 + u * RPI * 4)));
          const uint32_t ro = src_offset(n);
          off = (kr < k_len && ro != kOob) ? ro + (uint32_t)(c * 8 * TS) : kOob;
        } else {
          off = kr < k_len ? aoff[u] + (uint32_t)k0 * a_rowb : kOob;
        }
        lds_load16_at(rA, dst, off);
      }
    }
    // B
#pragma unroll
    for (int u = 0; u < C::B_PW; ++u) {
      const int ins = wave * C::B_PW + u;
      const uint32_t dst = lds0 + (uint32_t)(s * C::STAGE + C::A_BYTES + ins * 1024);
      if constexpr (B_K) {
        lds_load16_at(second ? rB2 : rB, dst, boff_l[u] + (uint32_t)kk * (uint32_t)TS);
      } else {
        // group g holds instructions [g * PER_G, (g + 1) * PER_G): wave-uniform
        constexpr int PER_G = BK * RCB / 64;
        constexpr int RPI = 64 / RCB;
        const int g = ins / PER_G;
        uint32_t off;
        if constexpr (KIDX_B) {
          // row k of the tile is entry u * RPI + lane / RCB of this wave's
          // slot (one group: ins = wave * B_PW + u)
          const int k = (ins - g * PER_G) * RPI + lane / RCB;
          const int c = (lane % RCB) ^ trswz<RCB>(k);
          const uint32_t n = *reinterpret_cast<const __attribute__((address_space(3))) uint32_t*>(
              (uintptr_t)(ibase + (uint32_t)(s * 256 + u * RPI * 4)));
          const uint32_t ro = src_offset(n);
          off = (k0 + k < k_len && ro != kOob) ? ro + (uint32_t)(c * 8 * TS) : kOob;
        } else if constexpr (EXPERT) {
          const int k = (ins - g * PER_G) * RPI + lane / RCB;
          off = k0 + k < k_len ? boff_l[u] + (uint32_t)k0 * b_rowb : kOob;
        } else {
          off = boff_l[u] + (uint32_t)k0 * b_rowb;
        }
        lds_load16_at((DUAL && g) ? rB2 : rB, dst, off);
      }
    }
    if constexpr (KIDX) load_idx(kn, s);
  };

  // waves wave and wave + 4 share a SIMD; with wm = wave / WGN they cover
  // different row slices, so a tile whose last slices are empty (the ragged
  // end of an expert segment) leaves each SIMD with less MFMA work
  const int wm = wave / S::WGN, wn = wave % S::WGN;
  f32x4_t acc[NB][FM][FN];
#pragma unroll
  for (int g = 0; g < NB; ++g)
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[g][i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int l16 = lane & 15, lg = lane >> 4;  // column/row within a fragment, k-group
  if constexpr (EPI == Epi::AccF32) {
    if (p.acc_chain && !p.acc_init) {
      // C into the accumulators (rows past row_end as zeros), through this
      // wave's LDS share, before the pipeline takes the stages over
      using AG = AccGeom<S, C>;
      float* stg = reinterpret_cast<float*>(smem + wave * AG::PWB);
      const int rw0 = m0 + wm * WM, cw0 = n0 + wn * WN;
#pragma unroll
      for (int s = 0; s < AG::NSUB; ++s) {
        const int g = s / AG::NSL, sl = s - g * AG::NSL;
        const float* Cg = static_cast<const float*>(g == 0 ? p.C : p.C2) + (int64_t)e * p.c_estride;
        f32x4_t v[AG::PER];
#pragma unroll
        for (int u = 0; u < AG::PER; ++u) {
          const int idx = lane + u * 64, r = idx / AG::VW, c4 = idx - r * AG::VW;
          const int row = rw0 + sl * AG::SR + r;
          v[u] = row < row_end ? *reinterpret_cast<const f32x4_t*>(Cg + (int64_t)row * p.ldc + cw0 + c4 * 4)
                               : f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
        wave_lds_sync();  // the previous slice's fragment reads are done
#pragma unroll
        for (int u = 0; u < AG::PER; ++u) {
          const int idx = lane + u * 64, r = idx / AG::VW, c4 = idx - r * AG::VW;
          *reinterpret_cast<f32x4_t*>(stg + r * AG::LD + c4 * 4) = v[u];
        }
        wave_lds_sync();
#pragma unroll
        for (int i = 0; i < AG::FS; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q)
              acc[g][sl * AG::FS + i][j][q] = stg[(i * 16 + 4 * lg + q) * AG::LD + j * 16 + l16];
      }
      lds_barrier();  // every wave is done with its share before the stages refill
    }
  }

  // ---- MFMA operand reads.  Every fragment address is a lane-dependent base
  // plus a compile-time constant (stage, k-step, half, group and fragment
  // offsets), because each swizzle depends only on the lane:
  //  * b128 reads of a K-contiguous tile: row r = w0 + f * 16 + l16 and chunk
  //    c = ks * 4 + lg, with the swizzle a function of l16 alone, so one base
  //    per k-step and + f * 16 rows per fragment;
  //  * transposing reads of an M/N-contiguous tile: row k = ks * 32 + lg * 8 +
  //    trj (+ 4 for the high half), whose swizzle bits (k & 3 and bit 3) come
  //    from trj and lg alone, so one base per fragment column and + ks * 32 /
  //    + 4 rows for k-step and half.
  // The bases are re-laundered every K-step so that the compiler does not
  // hoist one address register per (stage, fragment) out of the loop.
  const int trj = l16 >> 2, trq = l16 & 3;    // transposing read: row j, segment q
  constexpr int NBA = A_K ? KS : FM;
  constexpr int NBB = B_K ? KS : FN;
  uint32_t baseA[NBA], baseB[NBB];
  {
    const uint32_t smem0 = (uint32_t)reinterpret_cast<uintptr_t>((lds_void_p)smem);
    auto tr_base = [&](int rc_bytes, int col) -> uint32_t {
      const int k = lg * 8 + trj;
      const int sw = (rc_bytes >> 4) >= 16 ? trswz<16>(k) : trswz<8>(k);
      return (uint32_t)(k * rc_bytes + ((((col >> 3)) ^ sw) << 4) + (((col >> 2) & 1) << 3));
    };
#pragma unroll
    for (int b = 0; b < NBA; ++b) {
      if constexpr (A_K) {
        const int r = wm * WM + l16;
        baseA[b] = smem0 + (uint32_t)(r * (CK * 16) + (((b * 4 + lg) ^ kswz<CK>(r)) << 4));
      } else {
        baseA[b] = smem0 + tr_base(RCA * 16, wm * WM + b * 16 + trq * 4);
      }
    }
#pragma unroll
    for (int b = 0; b < NBB; ++b) {
      if constexpr (B_K) {
        const int n = wn * WN + l16;
        baseB[b] = smem0 + C::A_BYTES + (uint32_t)(n * (CK * 16) + (((b * 4 + lg) ^ kswz<CK>(n)) << 4));
      } else {
        baseB[b] = smem0 + C::A_BYTES + tr_base(RCB * 16, wn * WN + b * 16 + trq * 4);
      }
    }
  }
  auto launder = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int b = 0; b < NBA; ++b) asm volatile("" : "+v"(baseA[b]));
#pragma unroll
    for (int b = 0; b < NBB; ++b) asm volatile("" : "+v"(baseB[b]));
    if constexpr (KIDX) asm volatile("" : "+v"(ibase));
  };
  auto ld128 = [](uint32_t addr) __attribute__((always_inline)) -> u32x4_t {
    return *reinterpret_cast<const __attribute__((address_space(3))) u32x4_t*>((uintptr_t)addr);
  };
  auto ldtr = [](uint32_t lo_addr, uint32_t hi_off) __attribute__((always_inline)) -> u32x4_t {
    const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_p)(uintptr_t)lo_addr);
    const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_p)(uintptr_t)(lo_addr + hi_off));
    return __builtin_bit_cast(u32x4_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  // operand fragments of one K-tile: two register sets, so that the next
  // tile's fragments are read while the MFMAs consume the current ones
  u32x4_t fa[2][KS][FM];
  u32x4_t fb[2][KS][NB][FN];
  auto read_frags = [&](int s, int set) __attribute__((always_inline)) {
    const uint32_t so = (uint32_t)(s * C::STAGE);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        if constexpr (A_K)
          fa[set][ks][i] = ld128(baseA[ks] + so + (uint32_t)(i * 16 * CK * 16));
        else
          fa[set][ks][i] = ldtr(baseA[i] + so + (uint32_t)(ks * 32 * RCA * 16), 4 * RCA * 16);
      }
#pragma unroll
      for (int g = 0; g < NB; ++g)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          if constexpr (B_K)
            fb[set][ks][g][j] = ld128(baseB[ks] + so + (uint32_t)(j * 16 * CK * 16));
          else
            fb[set][ks][g][j] = ldtr(baseB[j] + so + (uint32_t)(g * BK * RCB * 16 + ks * 32 * RCB * 16),
                                     4 * RCB * 16);
        }
    }
  };
  auto mfmas = [&](int set) __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int g = 0; g < NB; ++g)
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j) Mfma<bf16_t>::run(fa[set][ks][i], fb[set][ks][g][j], acc[g][i][j]);
  };

  // Row scales of a scaled store, one per lane (the wave's row slice is at
  // most 64 rows): requested before the pipeline's first loads, so they
  // have landed long before the epilogue reads them
  float row_scale_lane = 1.f;
  if constexpr (MODE == Mode::Rows && EPI == Epi::Store) {
    static_assert(WM <= 64, "one row scale per lane");
    const int row = m0 + wm * WM + lane;
    if (p.row_scale && lane < WM && row < row_end) row_scale_lane = p.row_scale[row];
  }
  // The SwiGLU backward's row gates (two dependent loads: the row's pair,
  // then its gate), likewise requested before the pipeline: the epilogue's
  // thread t handles rows slab*SR + t/G8 + it*(THREADS/G8) of the tile, so
  // a wave's threads touch BM/WAVES distinct rows; lane q of the wave holds
  // the gate of the wave's q-th row (order: slab, iteration, row within the
  // wave's group).
  float sw_gate_lane = 0.f;
  if constexpr (MODE == Mode::Rows && EPI == Epi::SwiGLUBwd) {
    constexpr int G8 = BN / 8, RPW = 64 / G8, RSTEP = C::THREADS / G8;
    static_assert(64 % G8 == 0 && C::THREADS % G8 == 0 && BM / C::WAVES <= 64, "gate table");
    constexpr int SLAB_FIT = (NS * C::STAGE) / (WM * (BN + 4) * 4);
    constexpr int SLAB = SLAB_FIT >= S::WGM ? S::WGM : (SLAB_FIT >= 2 && S::WGM % 2 == 0 ? 2 : 1);
    constexpr int SR = SLAB * WM, ITEMS = SR * G8 / C::THREADS;
    if (lane < BM / C::WAVES) {
      const int j = lane % RPW, it = (lane / RPW) % ITEMS, sl = lane / (RPW * ITEMS);
      const int row = m0 + sl * SR + wave * RPW + j + it * RSTEP;
      if (row < row_end) {
        const int32_t pr = p.sw_perm[row];
        if ((uint64_t)pr < (uint64_t)p.sw_nk) sw_gate_lane = p.sw_gates[pr];
      }
    }
  }

  // ---- pipeline.  NS stages; tile t goes to stage t % NS.  The prologue
  // fills every stage and reads tile 0's fragments.  Iteration kt then
  //   waits until tile kt+1 has landed (this thread's loads, then everyone's,
  //     via the barrier -- which also orders every wave's reads of tile kt's
  //     stage before it is refilled),
  //   refills that stage with tile kt+NS,
  //   reads tile kt+1's fragments while the MFMAs run on tile kt's.
  // Tiles past the last are issued as copies of the last one (clamped index)
  // so that every iteration waits on the same count; the extra fragment read
  // of the final iteration hits such a copy and is not used.  The loop is
  // unrolled so that every stage index and register set is a compile-time
  // constant.
  constexpr int U = (NS % 2 == 0) ? NS : 2 * NS;
  if (nk > 0) {  // (an expert with no rows in store mode skips to the epilogue)
  const int last = nk - 1;
  if constexpr (KIDX) {
    // the first NS tiles' entries, landed before the prologue reads them
#pragma unroll
    for (int s = 0; s < NS; ++s) load_idx(min(s, last), s);
    wait_vmcnt<0>();
  }
#pragma unroll
  for (int s = 0; s < NS; ++s) issue(min(s, last), s, min(s + NS, last));
  // a wave whose rows all lie past the segment end only helps with the loads
  const bool active = m0 + wm * WM < row_end;
  wait_vmcnt<(NS - 1) * PT>();
  lds_barrier();
  if (active) read_frags(0, 0);
  for (int kt0 = 0; kt0 < nk; kt0 += U) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kt = kt0 + u;
      if (kt >= nk) break;
      wait_vmcnt<(NS - 2) * PT>();
      lds_barrier();
      launder();
      issue(min(kt + NS, last), u % NS, min(kt + 2 * NS, last));
      if (active) {
        read_frags((u + 1) % NS, (u + 1) & 1);
        mfmas(u & 1);
        // Issue order: one MFMA, then one fragment read, pair by pair, then
        // whatever is left.  Spreading the LDS reads evenly over the MFMA
        // phase keeps the LDS command queue from filling (a full queue
        // stalls the wave's in-order issue, MFMAs included).
        constexpr int NRD = KS * (A_K ? FM : 2 * FM) + KS * NB * FN * (B_K ? 1 : 2);
        constexpr int NMF = KS * NB * FM * FN;
        constexpr int PAIRS = NRD < NMF ? NRD : NMF;
#pragma unroll
        for (int q = 0; q < PAIRS; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
        }
        if constexpr (NMF > PAIRS) __builtin_amdgcn_sched_group_barrier(0x008, NMF - PAIRS, 0);
        if constexpr (NRD > PAIRS) __builtin_amdgcn_sched_group_barrier(0x100, NRD - PAIRS, 0);
      }
    }
  }
  wait_vmcnt<0>();
  }

  if constexpr (EPI == Epi::AccF32) {
    // C += tile (fp32 read-modify-write), or C = tile with acc_init or
    // acc_chain (the accumulators then already hold the whole sum).  Each
    // wave moves its own block through its LDS share (AccGeom); the old
    // values of slices s+1 .. s+PD are in flight while slice s is added and
    // stored (the fragment registers are free by then), so the reads'
    // latency overlaps PD slices' work.  Each element
    // is old + new in one fp32 add.  The operand stages are free once every
    // wave's last fragment reads are done (the barrier); after it each wave
    // touches only its own share.  Rows past row_end are neither read nor
    // written.  C is read and written once per launch, so its accesses are
    // marked non-temporal: they then do not evict the operand rows that the
    // expert's other tiles read from L2.
    using AG = AccGeom<S, C>;
    float* stg = reinterpret_cast<float*>(smem + wave * AG::PWB);
    const int rw0 = m0 + wm * WM, cw0 = n0 + wn * WN;  // this wave's block
    auto grow = [&](int s, int u) __attribute__((always_inline)) {
      const int sl = s - (s / AG::NSL) * AG::NSL;
      return rw0 + sl * AG::SR + (lane + u * 64) / AG::VW;
    };
    auto gptr = [&](int s, int u) __attribute__((always_inline)) {
      const int g = s / AG::NSL;
      const int idx = lane + u * 64, r = idx / AG::VW, c4 = idx - r * AG::VW;
      float* Cg = static_cast<float*>(g == 0 ? p.C : p.C2) + (int64_t)e * p.c_estride;
      return reinterpret_cast<f32x4_t*>(Cg + (int64_t)grow(s, u) * p.ldc + cw0 + c4 * 4);
    };
    const bool accumulate = !p.acc_init && !p.acc_chain;
    constexpr int PD = 3;  // slices of old values requested ahead
    f32x4_t old[PD + 1][AG::PER];
    if (accumulate) {
#pragma unroll
      for (int s0 = 0; s0 < PD && s0 < AG::NSUB; ++s0)
#pragma unroll
        for (int u = 0; u < AG::PER; ++u)
          if (grow(s0, u) < row_end) old[s0][u] = __builtin_nontemporal_load(gptr(s0, u));
    }
    lds_barrier();  // every wave's last fragment reads are done
#pragma unroll
    for (int s = 0; s < AG::NSUB; ++s) {
      const int g = s / AG::NSL, sl = s - g * AG::NSL;
#pragma unroll
      for (int i = 0; i < AG::FS; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            stg[(i * 16 + 4 * lg + q) * AG::LD + j * 16 + l16] = acc[g][sl * AG::FS + i][j][q];
      wave_lds_sync();
      if (accumulate && s + PD < AG::NSUB) {
#pragma unroll
        for (int u = 0; u < AG::PER; ++u)
          if (grow(s + PD, u) < row_end) old[(s + PD) % (PD + 1)][u] = __builtin_nontemporal_load(gptr(s + PD, u));
      }
#pragma unroll
      for (int u = 0; u < AG::PER; ++u) {
        const int idx = lane + u * 64, r = idx / AG::VW, c4 = idx - r * AG::VW;
        const f32x4_t add = *reinterpret_cast<const f32x4_t*>(stg + r * AG::LD + c4 * 4);
        if (grow(s, u) < row_end) __builtin_nontemporal_store(accumulate ? old[s % (PD + 1)][u] + add : add, gptr(s, u));
      }
      wave_lds_sync();  // this slice's reads are done before the next slice's writes
    }
    return;
  }

  if constexpr (EPI == Epi::CEStats) {
    // Vocabulary-strip cross-entropy, forward: the tile's logits stay on
    // chip.  Per row, each wave reduces its WN-column slice (columns past N,
    // the ragged end of the strip, excluded) to the slice's max m and
    // sum of exp(logit - m): first over the lane's own columns in column
    // order, then over the 16 lanes of the row group by xor butterflies
    // (commutative pairwise steps, so every lane ends with the same bits).
    // Slice s of the strip covers columns [s WN, (s + 1) WN), the same
    // vocabulary columns whatever the strip width.  The lane holding the
    // row's target column also writes that logit.
    const int col0 = n0 + wn * WN;
    const int slice = col0 / WN;
    const int64_t M = p.M;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int row = m0 + wm * WM + i * 16 + 4 * lg + q;
        float mx = -INFINITY;
#pragma unroll
        for (int j = 0; j < FN; ++j)
          if (col0 + j * 16 + l16 < p.N) mx = fmaxf(mx, acc[0][i][j][q]);
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
        float sm = 0.f;
#pragma unroll
        for (int j = 0; j < FN; ++j)
          if (col0 + j * 16 + l16 < p.N) sm += __expf(acc[0][i][j][q] - mx);
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) sm += __shfl_xor(sm, o);
        if (row < row_end) {
          if (l16 == 0) {
            p.ce_pmax[slice * M + row] = mx;
            p.ce_psum[slice * M + row] = sm;
          }
          const int64_t rel = (int64_t)p.ce_targets[row] - p.ce_col0 - col0;
          if (rel >= 0 && rel < WN && (int)(rel & 15) == l16) {
            float v = 0.f;
#pragma unroll
            for (int j = 0; j < FN; ++j)
              if ((int)(rel >> 4) == j) v = acc[0][i][j][q];
            p.ce_ytgt[row] = v;
          }
        }
      }
    return;
  }

  if constexpr (MODE == Mode::Rows && EPI == Epi::SwiGLUBwd) {
    // SwiGLU backward fused into dh' = dYp W_down^T, which is never stored.
    // Per row r (pair p = sw_perm[r], gate g) and column f, with s =
    // sigmoid(a): da = g dh' u s (1 + a (1 - s)), du = g dh' a s, hg = g h,
    // written over a, u and h; and the tile's share of dgate_p = sum_f dh' h,
    // written to sw_dgp[n-tile][r] (the tiles are added in order later).
    // dh' goes through the free operand stages slab by slab (as the staged
    // stores), so each thread takes 8 consecutive columns of one row: 16-byte
    // accesses to a, u and h, and the row's share is a lane-order sum then an
    // xor butterfly over the G8 threads of the row (consecutive lanes).
    constexpr int LD = BN + 4;  // padded row, floats
    constexpr int G8 = BN / 8;  // 8-column groups per row
    constexpr int SLAB_FIT = (NS * C::STAGE) / (WM * LD * 4);
    constexpr int SLAB = SLAB_FIT >= S::WGM ? S::WGM : (SLAB_FIT >= 2 && S::WGM % 2 == 0 ? 2 : 1);
    constexpr int SR = SLAB * WM;
    static_assert(SR * LD * 4 <= NS * C::STAGE, "staging must fit the LDS stages");
    static_assert(S::WGM % SLAB == 0, "slabs of whole wave row slices");
    static_assert(64 % G8 == 0 && (SR * G8) % C::THREADS == 0,
                  "a row's threads share one wave; every thread runs the same iterations");
    float* stg = reinterpret_cast<float*>(smem);
    T* Ch = static_cast<T*>(p.C);
    T* Ca = static_cast<T*>(p.C2);
    T* Cu = static_cast<T*>(p.C3);
    float* dgp = p.sw_dgp + (int64_t)(n0 / BN) * p.sw_rows;
    // thread t: 8 columns c of rows t/G8 + it*RSTEP of each slab; all of a
    // slab's a, u, h pieces are requested before the first is used, and the
    // gates come from the table loaded before the pipeline
    constexpr int RPW = 64 / G8, RSTEP = C::THREADS / G8, ITEMS = SR * G8 / C::THREADS;
    const int c = tid % G8, rt = tid / G8;
#pragma unroll
    for (int sl = 0; sl < S::WGM / SLAB; ++sl) {
      lds_barrier();  // previous users of the LDS are done
      if (wm / SLAB == sl) {
        const int r0 = (wm - sl * SLAB) * WM;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q)
              stg[(r0 + i * 16 + 4 * lg + q) * LD + wn * WN + j * 16 + l16] = acc[0][i][j][q];
      }
      const int row0 = m0 + sl * SR;
      u32x4_t va[ITEMS], vu[ITEMS], vh[ITEMS];
#pragma unroll
      for (int it = 0; it < ITEMS; ++it) {
        const int grow = row0 + rt + it * RSTEP;
        if (grow < row_end) {
          const int64_t o = (int64_t)grow * p.ldc + n0 + c * 8;
          va[it] = *reinterpret_cast<const u32x4_t*>(Ca + o);
          vu[it] = *reinterpret_cast<const u32x4_t*>(Cu + o);
          vh[it] = *reinterpret_cast<const u32x4_t*>(Ch + o);
        }
      }
      lds_barrier();
      // results overwrite the loaded pieces in registers; every store of
      // the slab goes out after the last computation, so no store waits on
      // another piece's loads
      float parts[ITEMS];
#pragma unroll
      for (int it = 0; it < ITEMS; ++it) {
        const int r = rt + it * RSTEP;
        const bool ok = row0 + r < row_end;
        // this row's gate: table entry (sl, it, row within the wave's group)
        const float g = __shfl(sw_gate_lane, (sl * ITEMS + it) * RPW + (rt % RPW), 64);
        float part = 0.f;
        if (ok) {
          float dv[8], av[8], uv[8], hv[8];
          const f32x4_t d0 = *reinterpret_cast<const f32x4_t*>(stg + r * LD + c * 8);
          const f32x4_t d1 = *reinterpret_cast<const f32x4_t*>(stg + r * LD + c * 8 + 4);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            dv[q] = d0[q];
            dv[q + 4] = d1[q];
          }
          unpack16(va[it], av, T());
          unpack16(vu[it], uv, T());
          unpack16(vh[it], hv, T());
          float da[8], du[8], hg[8];
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            part = fmaf(dv[q], hv[q], part);
            const float sa = logistic(av[q]);
            const float d = g * dv[q];
            da[q] = d * uv[q] * sa * (1.f + av[q] * (1.f - sa));
            du[q] = d * av[q] * sa;
            hg[q] = g * hv[q];
          }
          va[it] = pack16(da, T());
          vu[it] = pack16(du, T());
          vh[it] = pack16(hg, T());
        } else {
          // (never stored; defined on every path so that the stores below
          // do not wait on the loads that target these registers)
          va[it] = vu[it] = vh[it] = u32x4_t{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int m = 1; m < G8; m <<= 1) part += __shfl_xor(part, m);
        parts[it] = part;
      }
#pragma unroll
      for (int it = 0; it < ITEMS; ++it) {
        const int grow = row0 + rt + it * RSTEP;
        if (grow < row_end) {
          const int64_t o = (int64_t)grow * p.ldc + n0 + c * 8;
          *reinterpret_cast<u32x4_t*>(Ca + o) = va[it];
          *reinterpret_cast<u32x4_t*>(Cu + o) = vu[it];
          *reinterpret_cast<u32x4_t*>(Ch + o) = vh[it];
          if (c == 0) dgp[grow] = parts[it];
        }
      }
    }
    return;
  }

  if constexpr ((MODE == Mode::Rows && (EPI == Epi::Store || EPI == Epi::SwiGLU ||
                                       EPI == Epi::SwiGLUSave || EPI == Epi::F32)) ||
                (MODE == Mode::Dense && EPI == Epi::CEGrad)) {
    // Row-grouped outputs go out through LDS: each wave parks its fragment
    // values (computed exactly as below) in the free operand stages, slab by
    // slab of wave row slices, and the work-group then writes the slab with
    // 16-byte, row-contiguous stores, skipping rows past the segment end.
    // Rows are padded by 16 bytes (fragment row groups land in distinct
    // banks; 16-byte reads stay aligned).
    auto stage_store = [&](auto* Cbase, auto value) __attribute__((always_inline)) {
      using OT = typename std::remove_pointer<decltype(Cbase)>::type;
      constexpr int ES = (int)sizeof(OT);
      constexpr int LD = BN + 16 / ES;       // padded row, elements
      constexpr int VE = 16 / ES;            // elements per 16-byte vector
      constexpr int V = BN / VE;             // vectors per tile row
      constexpr int SLAB_FIT = (NS * C::STAGE) / (WM * LD * ES);
      constexpr int SLAB = SLAB_FIT >= S::WGM ? S::WGM : (SLAB_FIT >= 2 && S::WGM % 2 == 0 ? 2 : 1);
      constexpr int SR = SLAB * WM;
      static_assert(SR * LD * ES <= NS * C::STAGE, "output staging must fit the LDS stages");
      static_assert(S::WGM % SLAB == 0, "slabs of whole wave row slices");
      OT* stg = reinterpret_cast<OT*>(smem);
#pragma unroll
      for (int sl = 0; sl < S::WGM / SLAB; ++sl) {
        lds_barrier();  // previous users of the LDS are done
        if (wm / SLAB == sl) {
          const int r0 = (wm - sl * SLAB) * WM;
#pragma unroll
          for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
              for (int q = 0; q < 4; ++q)
                stg[(r0 + i * 16 + 4 * lg + q) * LD + wn * WN + j * 16 + l16] = value(i, j, q);
        }
        lds_barrier();
        const int row0 = m0 + sl * SR;
        for (int idx = tid; idx < SR * V; idx += C::THREADS) {
          const int r = idx / V, c = idx - r * V;
          if (row0 + r >= row_end) break;  // rows ascend with idx
          const int col = n0 + c * VE;
          OT* dst = p.c_kt ? Cbase + (int64_t)(col >> 5) * p.c_kt + (int64_t)(row0 + r) * 32 + (col & 31)
                           : Cbase + (int64_t)(row0 + r) * p.ldc + col;
          *reinterpret_cast<u32x4_t*>(dst) = *reinterpret_cast<const u32x4_t*>(stg + r * LD + c * VE);
        }
      }
    };
    if constexpr (EPI == Epi::Store) {
      // each row times its scale (the down projection's gates; 1 without
      // row_scale, which leaves the value unchanged), then rounded once.
      // Lane l loaded the scale of the wave's row l before the pipeline.
      float rg[FM][4];
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) rg[i][q] = __shfl(row_scale_lane, i * 16 + 4 * lg + q, 64);
      stage_store(static_cast<T*>(p.C), [&](int i, int j, int q) { return f2bf(acc[0][i][j][q] * rg[i][q]); });
    } else if constexpr (EPI == Epi::CEGrad) {
      // Vocabulary-strip cross-entropy, backward: the strip's logit gradient
      // dl_row (exp(logit - lse_row) - [column == target_row]), bf16;
      // columns past N (the ragged end of the strip) and rows with dl = 0
      // (ignored tokens) store zeros.
      float rlse[FM][4], rdl[FM][4];
      int64_t rtc[FM][4];  // target column relative to this wave's first column
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int row = min(m0 + wm * WM + i * 16 + 4 * lg + q, row_end - 1);
          rlse[i][q] = p.ce_lse[row];
          rdl[i][q] = p.ce_dl[row];
          rtc[i][q] = (int64_t)p.ce_targets[row] - p.ce_col0 - (n0 + wn * WN);
        }
      stage_store(static_cast<T*>(p.C), [&](int i, int j, int q) {
        const int c = j * 16 + l16;
        const float pr = __expf(acc[0][i][j][q] - rlse[i][q]);
        const float gv = rdl[i][q] * (pr - (rtc[i][q] == c ? 1.f : 0.f));
        return f2bf(n0 + wn * WN + c < p.N ? gv : 0.f);
      });
    } else if constexpr (EPI == Epi::F32) {
      stage_store(static_cast<float*>(p.C), [&](int i, int j, int q) { return acc[0][i][j][q]; });
    } else {
      stage_store(static_cast<T*>(p.C), [&](int i, int j, int q) {
        const float v0 = acc[0][i][j][q], v1 = acc[NB - 1][i][j][q];
        return f2bf(swiglu_h(v0, v1));
      });
      if constexpr (EPI == Epi::SwiGLUSave) {
        stage_store(static_cast<T*>(p.C2), [&](int i, int j, int q) { return f2bf(acc[0][i][j][q]); });
        stage_store(static_cast<T*>(p.C3), [&](int i, int j, int q) { return f2bf(acc[NB - 1][i][j][q]); });
      }
    }
    return;
  }

  // ---- epilogue (as gemm_kernel.hpp)
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int grow = m0 + wm * WM + i * 16 + 4 * lg + q;
        const int gcol = n0 + wn * WN + j * 16 + l16;
        if (grow >= row_end) continue;
        const int64_t o = (int64_t)grow * p.ldc + gcol;
        const float v0 = acc[0][i][j][q];
        if constexpr (EPI == Epi::Store) {
          static_cast<T*>(p.C)[o] = f2bf(v0);
        } else if constexpr (EPI == Epi::SwiGLU || EPI == Epi::SwiGLUSave) {
          const float v1 = acc[NB - 1][i][j][q];
          const float hv = swiglu_h(v0, v1);
          static_cast<T*>(p.C)[o] = f2bf(hv);
          if constexpr (EPI == Epi::SwiGLUSave) {
            static_cast<T*>(p.C2)[o] = f2bf(v0);
            static_cast<T*>(p.C3)[o] = f2bf(v1);
          }
        } else if constexpr (EPI == Epi::F32) {
          if constexpr (MODE == Mode::Dense) {  // partial of a split product
            if (gcol < p.N) static_cast<float*>(p.C)[(int64_t)blockIdx.z * p.c_estride + o] = v0;
          } else {
            static_cast<float*>(p.C)[o] = v0;
          }
        } else if constexpr (EPI == Epi::BiasF32) {
          if (gcol < p.N) static_cast<float*>(p.C)[o] = v0 + (p.bias ? p.bias[gcol] : 0.f);
        }
      }
}

template <Mode MODE, class S, bool DUAL, bool A_K, bool B_K, bool KCAT, Epi EPI>
__global__ __launch_bounds__(64 * S::WGM * S::WGN)
__attribute__((amdgpu_waves_per_eu(S::WG_PER_CU * S::WGM * S::WGN / 4))) void gemm_lds_kernel(const Params p) {
  gemm_lds_body<MODE, S, DUAL, A_K, B_K, KCAT, EPI>(p, (int)blockIdx.x);
}

// One row-grouped product's template configuration, for the pair kernel.
template <class S_, bool DUAL_, bool A_K_, bool B_K_, bool KCAT_, Epi EPI_>
struct RowsGemm {
  using S = S_;
  using C = LdsCfg<S_, DUAL_>;
  __device__ static __forceinline__ void run(const Params& p, int bid) {
    gemm_lds_body<Mode::Rows, S_, DUAL_, A_K_, B_K_, KCAT_, EPI_>(p, bid);
  }
};

// Two row-grouped products in one launch (the two tile lists of a split
// chunk plan).  Each list renumbers its own ids, so both spread over all
// XCDs (renumbering the combined range instead measured slower: one list's
// slower tiles then crowd some XCDs), and on every XCD the two lists' tiles
// are interleaved in proportion to their counts, except that the XCD's last
// round holds second-list tiles only.  The lists differ in what bounds them
// under skewed routing (long segments: many rows per weight slice, MFMA
// work; short ones: a whole weight slice for few rows, HBM traffic), so
// running them side by side overlaps the two rather than taking them one
// after the other; the shorter 128-row tiles last keep the launch's tail
// short (interleaving to the end measured 6% slower on balanced routing).
// With ALT, a launch whose two lists come to fewer than split_min
// work-groups runs G1 over pu instead (the chunk's unsplit tile list, as a
// single-product launch would), where G2's larger tiles would leave too few
// rounds.
template <class G1, class G2, bool ALT = false>
__global__ __launch_bounds__(64 * G1::C::WAVES)
__attribute__((amdgpu_waves_per_eu(G1::S::WG_PER_CU * G1::C::WAVES / 4))) void gemm_lds_pair_kernel(
    const Params p1, const Params p2, const Params pu, int split_min) {
  static_assert(G1::C::WAVES == G2::C::WAVES && G1::S::WG_PER_CU == G2::S::WG_PER_CU,
                "paired products need the same work-group shape");
  const int b = (int)blockIdx.x;
  const int t1 = __builtin_amdgcn_readfirstlane(*p1.tile_count * p1.ntiles);
  const int t2 = __builtin_amdgcn_readfirstlane(*p2.tile_count * p2.ntiles);
  bool whole = false;
  if constexpr (ALT) whole = t1 + t2 < split_min;
  int L = b;
  bool first = whole;
  if (!whole) {
    // ids with b % 8 == x reach XCD x in the order j = b / 8; that XCD holds
    // c1 ids of the first list (those L < t1 with L % 8 == x) and c2 of the second
    const int x = b & 7, j = b >> 3;
    const int c1 = t1 > x ? (t1 - x + 7) >> 3 : 0;
    const int c2 = t2 > x ? (t2 - x + 7) >> 3 : 0;
    if (j >= c1 + c2) return;
    // the XCD's last round (one work-group per CU) takes second-list tiles
    // only; before it, ci ids interleave all c1 first-list tiles with the
    // other second-list ones
    const int R = min(c2, kCus / 8);
    const int ci = c1 + c2 - R;
    L = x + 8 * (c2 - R + (j - ci));
    if (j < ci) {
      // first-list tiles among this XCD's first j ids: ceil(j c1 / ci)
      const int j1 = (int)(((int64_t)j * c1 + ci - 1) / ci);
      const int j1n = (int)(((int64_t)(j + 1) * c1 + ci - 1) / ci);
      first = j1n > j1;
      L = first ? x + 8 * j1 : x + 8 * (j - j1);
    }
  }
  if (first)
    G1::run(ALT && whole ? pu : p1, L);
  else
    G2::run(p2, L);
}

template <class KERN>
hipError_t set_lds_attr(KERN kern, int lds, bool& done) {
  if (done) return hipSuccess;  // per instantiation; benign race (idempotent)
  hipError_t err = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (err == hipSuccess) done = true;
  return err;
}

template <Mode MODE, class S, bool DUAL, bool A_K, bool B_K, bool KCAT, Epi EPI>
hipError_t launch_lds(const Params& p, dim3 grid, hipStream_t st) {
  using C = LdsCfg<S, DUAL, mode_kidx(MODE)>;
  auto kern = gemm_lds_kernel<MODE, S, DUAL, A_K, B_K, KCAT, EPI>;
  constexpr int lds = lds_bytes<MODE, S, DUAL>();
  static bool attr_set = false;
  if (hipError_t err = set_lds_attr(kern, lds, attr_set); err != hipSuccess) return err;
  kern<<<grid, C::THREADS, lds, st>>>(p);
  return hipGetLastError();
}

// G1 over a 1-D Rows grid of n1 work-groups and G2 over n2, as one kernel
// (with pu, as gemm_lds_pair_kernel's ALT: n1 must then cover pu's grid).
template <class G1, class G2, bool ALT = false>
hipError_t launch_lds_pair(const Params& p1, int n1, const Params& p2, int n2, hipStream_t st,
                           const Params* pu = nullptr, int split_min = 0) {
  if (ALT != (pu != nullptr)) return hipErrorInvalidValue;
  auto kern = gemm_lds_pair_kernel<G1, G2, ALT>;
  constexpr int l1 = G1::C::NS * G1::C::STAGE, l2 = G2::C::NS * G2::C::STAGE;
  constexpr int lds = l1 > l2 ? l1 : l2;
  static bool attr_set = false;
  if (hipError_t err = set_lds_attr(kern, lds, attr_set); err != hipSuccess) return err;
  // n1, n2: each list's largest possible number of work-groups; every XCD
  // then gets at least as many ids as its tiles of both lists (the kernel
  // reads the actual counts)
  const int n1p = (n1 + 7) & ~7;
  kern<<<dim3((unsigned)(n1p + n2)), G1::C::THREADS, lds, st>>>(p1, p2, pu ? *pu : p1, split_min);
  return hipGetLastError();
}

}  // namespace gemm
}  // namespace moe
