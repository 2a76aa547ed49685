// The backward's per-chunk recompute and dh products in one kernel (bf16,
// 256-row tiles of a chunk's expert segments, 128 columns of F per tile).
//
// The SwiGLU expert of the "Memory-bounded expert" page is recomputed in the
// backward from the chunk's inputs (Methodology 1, nested gradient
// checkpointing), then differentiated:
//   a = Xp W_gate[e], u = Xp W_up[e], h = silu(a) u          (phase 1)
//   dh' = dYp W_down[e]^T                                    (phase 2)
//   s = sigmoid(a), da = g dh' u s (1 + a (1 - s)), du = g dh' a s, hg = g h
// and, per row and tile, the share sum_f dh' h of dgate.  Run as two
// products, the first stores a, u and h (bf16) and the second reads them
// back after its K loop; here each work-group keeps its tile's a, u and h in
// registers (rounded to bf16, as the stored copies are) between the two K
// loops, so they never reach HBM: per 65,536-token chunk that is 3 x 67 MB
// written and read again.
//
// Both K loops are the direct-to-LDS pipeline of gemm_lds_body (same stage
// layouts, swizzles, fragment reads, MFMA shape and K order), so a, u, h and
// dh' -- hence da, du and hg -- are bitwise those of the two-product path,
// and the per-128-column dgate shares are summed in that path's order, so
// chunkings whose chunks take different tile shapes still agree bitwise.
#pragma once

#include "gemm_lds.hpp"

namespace moe {
namespace gemm {

struct FusedBwdParams {
  const void* X;   // phase 1 A: [a_src_rows][lda] (gathered) or the chunk's rows
  const void* dY;  // phase 2 A: the same row mapping as X
  int64_t lda;     // H
  const int32_t* a_rows;  // row r of the chunk is row a_rows[r] / a_row_div (null: row r)
  int a_row_div;
  int64_t a_src_rows;
  const void* Wg;  // [E][H][F]
  const void* Wu;  // [E][H][F]
  const void* Wd;  // [E][F][H]
  int H, F;
  void* h_hg;  // [rows][F]: receives g h
  void* a_da;  // [rows][F]: receives da
  void* u_du;  // [rows][F]: receives du
  const int2* tiles;
  const int32_t* tile_count;
  const int32_t* offsets;
  int ntiles;  // F / 128
  const int32_t* perm;  // row r's pair (its gate is gates[perm[r]] when perm[r] < nk)
  const float* gates;
  int64_t nk;
  float* dgp;  // [ntiles][dgp_rows]: the tile's share of sum_f dh' h per row
  int64_t dgp_rows;
};

using FusedBwdShape = Shape<256, 128, 4, 2, 32, 1>;

template <class S>
__global__ __launch_bounds__(64 * S::WGM * S::WGN)
__attribute__((amdgpu_waves_per_eu(S::WGM * S::WGN / 4))) void fused_bwd_kernel(const FusedBwdParams p) {
  using C = LdsCfg<S, true>;  // phase 1's stages (DUAL); phase 2 uses a part of each
  using T = bf16_t;
  constexpr int BM = S::BM, BN = S::BN, BK = S::BK, NS = C::NS, CK = C::CK;
  constexpr int WM = BM / S::WGM, WN = BN / S::WGN;
  constexpr int FM = WM / 16, FN = WN / 16, KS = BK / 32;
  constexpr int RCB = BN / 8;
  constexpr int RPIK = 64 / CK;
  constexpr int64_t TS = 2;
  constexpr int A_PW = C::A_PW;
  constexpr int B1_PW = C::B_PW;                        // N-contiguous W_gate | W_up
  constexpr int B2_PW = (BN * BK * 2 / 1024) / C::WAVES;  // K-contiguous W_down rows
  constexpr int PT1 = A_PW + B1_PW, PT2 = A_PW + B2_PW;
  // phase 2's stages are packed (A and the W_down rows only), which leaves
  // room past them for the tile's h, row-major bf16 [BM][BN]
  constexpr int STAGE2 = C::A_BYTES + BN * BK * 2;
  constexpr int H_OFF = NS * STAGE2;
  constexpr int H_BYTES = BM * BN * 2;
  static_assert(H_OFF + H_BYTES <= kLdsBytes, "h must fit past phase 2's stages");
  constexpr int U = NS;
  static_assert(NS % 2 == 0, "an even stage count");
  static_assert(B2_PW >= 1 && (BN * BK * 2 / 1024) % C::WAVES == 0, "W_down tile must split over the waves");
  static_assert(WM == 64, "one gate per lane");

  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / S::WGN, wn = wave % S::WGN;
  const int l16 = lane & 15, lg = lane >> 4;

  const int total = *p.tile_count * p.ntiles;
  const int bid = (int)blockIdx.x;
  if (bid >= total) return;
  const RowsTile t = rows_tile(p.tiles, p.offsets, xcd_contiguous(bid, total), p.ntiles, BM);
  const int e = __builtin_amdgcn_readfirstlane(t.e);
  const int m0 = __builtin_amdgcn_readfirstlane(t.m0);
  const int n0 = __builtin_amdgcn_readfirstlane(t.nt * BN);
  const int row_end = __builtin_amdgcn_readfirstlane(t.row_end);
  const int64_t rows = (int64_t)min(row_end - m0, BM);

  // A rows: this lane's source-row byte offsets (the same for X and dY)
  uint32_t arow[A_PW];
  i32x4_t rX, rD;
  const bool gathered = p.a_rows != nullptr;
  if (gathered) {
    rX = make_srd(p.X, p.a_src_rows * p.lda * TS);
    rD = make_srd(p.dY, p.a_src_rows * p.lda * TS);
#pragma unroll
    for (int u = 0; u < A_PW; ++u) {
      const int row = (wave * A_PW + u) * RPIK + lane / CK;
      arow[u] = kOob;
      if (row < rows) {
        const int src = p.a_rows[m0 + row] / p.a_row_div;
        if ((uint64_t)src < (uint64_t)p.a_src_rows) arow[u] = (uint32_t)((int64_t)src * p.lda * TS);
      }
    }
  } else {
    rX = make_srd(static_cast<const T*>(p.X) + (int64_t)m0 * p.lda, rows * p.lda * TS);
    rD = make_srd(static_cast<const T*>(p.dY) + (int64_t)m0 * p.lda, rows * p.lda * TS);
#pragma unroll
    for (int u = 0; u < A_PW; ++u) {
      const int row = (wave * A_PW + u) * RPIK + lane / CK;
      arow[u] = (uint32_t)(row * p.lda * TS);
    }
  }
  const int64_t wstride = (int64_t)p.H * p.F;
  const i32x4_t rG = make_srd(static_cast<const T*>(p.Wg) + e * wstride + n0, (int64_t)p.H * p.F * TS);
  const i32x4_t rU = make_srd(static_cast<const T*>(p.Wu) + e * wstride + n0, (int64_t)p.H * p.F * TS);
  const i32x4_t rW = make_srd(static_cast<const T*>(p.Wd) + e * wstride + (int64_t)n0 * p.H,
                              (int64_t)BN * p.H * TS);

  // this lane's row gate (row wm * WM + lane of the tile), requested before
  // the pipelines so that it has landed by the epilogue
  float gate_lane = 0.f;
  {
    const int row = m0 + wm * WM + lane;
    if (row < row_end) {
      const int32_t pr = p.perm[row];
      if ((uint64_t)pr < (uint64_t)p.nk) gate_lane = p.gates[pr];
    }
  }

  // This lane's load offsets inside a K-tile, 32-bit (a K-tile adds k0 * 2 to
  // the A and W_down offsets, k0 * F * 2 to the W_gate / W_up ones): A rows
  // (kOob past the segment: such loads read zeros), W_gate | W_up rows k of
  // the tile, W_down rows n of the tile; with each operand's chunk swizzle.
  uint32_t aoff[A_PW], b1off[B1_PW], b2off[B2_PW];
#pragma unroll
  for (int u = 0; u < A_PW; ++u) {
    const int row = (wave * A_PW + u) * RPIK + lane / CK;
    const int c = (lane % CK) ^ kswz<CK>(row);
    aoff[u] = arow[u] == kOob ? kOob : arow[u] + (uint32_t)(c * 8 * TS);
  }
#pragma unroll
  for (int u = 0; u < B1_PW; ++u) {
    constexpr int PER_G = BK * RCB / 64;
    constexpr int RPI = 64 / RCB;
    const int ins = wave * B1_PW + u;
    const int k = (ins % PER_G) * RPI + lane / RCB;
    const int c = (lane % RCB) ^ trswz<RCB>(k);
    b1off[u] = (uint32_t)((k * p.F + c * 8) * (int)TS);
  }
#pragma unroll
  for (int u = 0; u < B2_PW; ++u) {
    const int row = (wave * B2_PW + u) * RPIK + lane / CK;
    const int c = (lane % CK) ^ kswz<CK>(row);
    b2off[u] = (uint32_t)((row * p.H + c * 8) * (int)TS);
  }
  auto stage_a = [&](int s) -> unsigned char* { return smem + s * C::STAGE; };
  auto stage_b = [&](int s) -> unsigned char* { return smem + s * C::STAGE + C::A_BYTES; };
  auto stage_a2 = [&](int s) -> unsigned char* { return smem + s * STAGE2; };
  auto stage_b2 = [&](int s) -> unsigned char* { return smem + s * STAGE2 + C::A_BYTES; };
  // phase 1: K-tile kt of X rows, W_gate and W_up (N-contiguous groups)
  auto issue1 = [&](int kt, int s) __attribute__((always_inline)) {
    const uint32_t ka = (uint32_t)(kt * BK * (int)TS), kb = (uint32_t)(kt * BK * p.F * (int)TS);
#pragma unroll
    for (int u = 0; u < A_PW; ++u)
      lds_load16(rX, stage_a(s) + (wave * A_PW + u) * 1024, aoff[u] + ka);
#pragma unroll
    for (int u = 0; u < B1_PW; ++u) {
      constexpr int PER_G = BK * RCB / 64;
      const int ins = wave * B1_PW + u;
      lds_load16(ins / PER_G ? rU : rG, stage_b(s) + ins * 1024, b1off[u] + kb);
    }
  };
  // phase 2: K-tile kt of dY rows and of W_down's rows n0.. (K-contiguous)
  auto issue2 = [&](int kt, int s) __attribute__((always_inline)) {
    const uint32_t ka = (uint32_t)(kt * BK * (int)TS);
#pragma unroll
    for (int u = 0; u < A_PW; ++u)
      lds_load16(rD, stage_a2(s) + (wave * A_PW + u) * 1024, aoff[u] + ka);
#pragma unroll
    for (int u = 0; u < B2_PW; ++u)
      lds_load16(rW, stage_b2(s) + (wave * B2_PW + u) * 1024, b2off[u] + ka);
  };

  // fragment addresses (those of gemm_lds_body for K-contiguous A, N- and
  // K-contiguous B)
  const int trj = l16 >> 2, trq = l16 & 3;
  const uint32_t smem0 = (uint32_t)reinterpret_cast<uintptr_t>((lds_void_p)smem);
  uint32_t baseA[KS], baseB1[FN], baseB2[KS];
  {
#pragma unroll
    for (int b = 0; b < KS; ++b) {
      const int r = wm * WM + l16;
      baseA[b] = smem0 + (uint32_t)(r * (CK * 16) + (((b * 4 + lg) ^ kswz<CK>(r)) << 4));
    }
#pragma unroll
    for (int b = 0; b < FN; ++b) {
      const int k = lg * 8 + trj;
      const int col = wn * WN + b * 16 + trq * 4;
      const int sw = RCB >= 16 ? trswz<16>(k) : trswz<8>(k);
      baseB1[b] = smem0 + C::A_BYTES +
                  (uint32_t)(k * (RCB * 16) + (((col >> 3) ^ sw) << 4) + (((col >> 2) & 1) << 3));
    }
  }
  // re-laundered every step, so that the compiler keeps one register per
  // base and offset instead of hoisting one per stage or K-tile
  auto launder1 = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int b = 0; b < KS; ++b) asm volatile("" : "+v"(baseA[b]));
#pragma unroll
    for (int b = 0; b < FN; ++b) asm volatile("" : "+v"(baseB1[b]));
#pragma unroll
    for (int u = 0; u < A_PW; ++u) asm volatile("" : "+v"(aoff[u]));
#pragma unroll
    for (int u = 0; u < B1_PW; ++u) asm volatile("" : "+v"(b1off[u]));
  };
  auto launder2 = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int b = 0; b < KS; ++b) asm volatile("" : "+v"(baseA[b]));
#pragma unroll
    for (int b = 0; b < KS; ++b) asm volatile("" : "+v"(baseB2[b]));
#pragma unroll
    for (int u = 0; u < A_PW; ++u) asm volatile("" : "+v"(aoff[u]));
#pragma unroll
    for (int u = 0; u < B2_PW; ++u) asm volatile("" : "+v"(b2off[u]));
  };
  auto ld128 = [](uint32_t addr) __attribute__((always_inline)) -> u32x4_t {
    return *reinterpret_cast<const __attribute__((address_space(3))) u32x4_t*>((uintptr_t)addr);
  };
  auto ldtr = [](uint32_t lo_addr, uint32_t hi_off) __attribute__((always_inline)) -> u32x4_t {
    const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_p)(uintptr_t)lo_addr);
    const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_p)(uintptr_t)(lo_addr + hi_off));
    return __builtin_bit_cast(u32x4_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  // K = H in both products, a multiple of BK * NS (the launch checks it): the
  // unrolled steps need no exit in the middle, which would keep older
  // accumulator values alive and spill
  const bool active = m0 + wm * WM < row_end;
  const int nk = p.H / BK;
  const int last = nk - 1;

  // ---- phase 1: a and u
  uint32_t pa[FM][FN][2], pu[FM][FN][2], ph[FM][FN][2];  // bf16 pairs (rows 4 lg + 0..3)
  T* hrow = reinterpret_cast<T*>(smem + H_OFF);  // h, row-major [BM][BN]
  {
    f32x4_t acc[2][FM][FN];
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[g][i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    u32x4_t fa[2][KS][FM];
    u32x4_t fb[2][KS][2][FN];
    auto read_frags = [&](int s, int set) __attribute__((always_inline)) {
      const uint32_t so = (uint32_t)(s * C::STAGE);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
        for (int i = 0; i < FM; ++i) fa[set][ks][i] = ld128(baseA[ks] + so + (uint32_t)(i * 16 * CK * 16));
#pragma unroll
        for (int g = 0; g < 2; ++g)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            fb[set][ks][g][j] = ldtr(baseB1[j] + so + (uint32_t)(g * BK * RCB * 16 + ks * 32 * RCB * 16),
                                     4 * RCB * 16);
      }
    };
#pragma unroll
    for (int s = 0; s < NS; ++s) issue1(min(s, last), s);
    wait_vmcnt<(NS - 1) * PT1>();
    lds_barrier();
    if (active) read_frags(0, 0);
    for (int kt0 = 0; kt0 < nk; kt0 += U) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int kt = kt0 + u;
        wait_vmcnt<(NS - 2) * PT1>();
        lds_barrier();
        launder1();
        issue1(min(kt + NS, last), u % NS);
        if (active) {
          read_frags((u + 1) % NS, (u + 1) & 1);
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int g = 0; g < 2; ++g)
#pragma unroll
              for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                  Mfma<bf16_t>::run(fa[u & 1][ks][i], fb[u & 1][ks][g][j], acc[g][i][j]);
          constexpr int NRD = KS * FM + KS * 2 * FN * 2;
          constexpr int NMF = KS * 2 * FM * FN;
          constexpr int PAIRS = NRD < NMF ? NRD : NMF;
#pragma unroll
          for (int q = 0; q < PAIRS; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          }
          if constexpr (NMF > PAIRS) __builtin_amdgcn_sched_group_barrier(0x008, NMF - PAIRS, 0);
          if constexpr (NRD > PAIRS) __builtin_amdgcn_sched_group_barrier(0x100, NRD - PAIRS, 0);
        }
      }
    }
    wait_vmcnt<0>();
    // a, u and h = silu(a) u, each rounded once to bf16 (h from the fp32
    // accumulators, as the forward's SwiGLU epilogue computes it)
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        bf16_t va[4], vu[4], vh[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float v0 = acc[0][i][j][q], v1 = acc[1][i][j][q];
          va[q] = f2bf(v0);
          vu[q] = f2bf(v1);
          vh[q] = f2bf(swiglu_h(v0, v1));
        }
        pa[i][j][0] = (uint32_t)va[0] | ((uint32_t)va[1] << 16);
        pa[i][j][1] = (uint32_t)va[2] | ((uint32_t)va[3] << 16);
        pu[i][j][0] = (uint32_t)vu[0] | ((uint32_t)vu[1] << 16);
        pu[i][j][1] = (uint32_t)vu[2] | ((uint32_t)vu[3] << 16);
        ph[i][j][0] = (uint32_t)vh[0] | ((uint32_t)vh[1] << 16);
        ph[i][j][1] = (uint32_t)vh[2] | ((uint32_t)vh[3] << 16);
      }
  }
  lds_barrier();  // every wave's phase-1 fragment reads are done before the stages refill
  // h waits in LDS (past phase 2's stages) until the epilogue
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t x = ph[i][j][q >> 1];
        hrow[(wm * WM + i * 16 + 4 * lg + q) * BN + wn * WN + j * 16 + l16] =
            (bf16_t)((q & 1) ? (x >> 16) : (x & 0xFFFF));
      }

  // ---- phase 2: dh'.  Its lane-derived addresses come from a laundered
  // copy of the thread id, so that nothing of them is computed early and kept
  // live through phase 1.
  {
    int t2 = tid;
    asm volatile("" : "+v"(t2));
    const int x16 = t2 & 15, xg = (t2 & 63) >> 4;
#pragma unroll
    for (int b = 0; b < KS; ++b) {
      const int n = wn * WN + x16;
      baseB2[b] = smem0 + C::A_BYTES + (uint32_t)(n * (CK * 16) + (((b * 4 + xg) ^ kswz<CK>(n)) << 4));
    }
  }
  f32x4_t acc2[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc2[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  {
    u32x4_t fa[2][KS][FM];
    u32x4_t fb[2][KS][FN];
    auto read_frags = [&](int s, int set) __attribute__((always_inline)) {
      const uint32_t so = (uint32_t)(s * STAGE2);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
        for (int i = 0; i < FM; ++i) fa[set][ks][i] = ld128(baseA[ks] + so + (uint32_t)(i * 16 * CK * 16));
#pragma unroll
        for (int j = 0; j < FN; ++j) fb[set][ks][j] = ld128(baseB2[ks] + so + (uint32_t)(j * 16 * CK * 16));
      }
    };
#pragma unroll
    for (int s = 0; s < NS; ++s) issue2(min(s, last), s);
    wait_vmcnt<(NS - 1) * PT2>();
    lds_barrier();
    if (active) read_frags(0, 0);
    for (int kt0 = 0; kt0 < nk; kt0 += U) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int kt = kt0 + u;
        wait_vmcnt<(NS - 2) * PT2>();
        lds_barrier();
        launder2();
        issue2(min(kt + NS, last), u % NS);
        if (active) {
          read_frags((u + 1) % NS, (u + 1) & 1);
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
              for (int j = 0; j < FN; ++j) Mfma<bf16_t>::run(fa[u & 1][ks][i], fb[u & 1][ks][j], acc2[i][j]);
          constexpr int NRD = KS * FM + KS * FN;
          constexpr int NMF = KS * FM * FN;
          constexpr int PAIRS = NRD < NMF ? NRD : NMF;
#pragma unroll
          for (int q = 0; q < PAIRS; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          }
          if constexpr (NMF > PAIRS) __builtin_amdgcn_sched_group_barrier(0x008, NMF - PAIRS, 0);
          if constexpr (NRD > PAIRS) __builtin_amdgcn_sched_group_barrier(0x100, NRD - PAIRS, 0);
        }
      }
    }
    wait_vmcnt<0>();
  }
  lds_barrier();  // the stages are free: the epilogue stages through them

  // ---- epilogue.  Element (i, j, q) of this lane: tile row wm*WM + i*16 +
  // 4*eg + q, column wn*WN + j*16 + e16 (from a laundered thread id, as above).
  int te = tid;
  asm volatile("" : "+v"(te));
  const int e16 = te & 15, eg = (te & 63) >> 4;
  auto unpk = [](const uint32_t (&w)[2], int q) __attribute__((always_inline)) -> float {
    const uint32_t x = w[q >> 1];
    return bf2f((bf16_t)((q & 1) ? (x >> 16) : (x & 0xFFFF)));
  };
  float* gtab = reinterpret_cast<float*>(smem);  // [BM] row gates
  float* dvs = gtab + BM;                        // [SR][LDV] a slab of dh', fp32
  constexpr int LDV = BN + 4;
  constexpr int SR = WM;                         // one wave row slice per slab
  static_assert((BM + SR * LDV) * 4 <= H_OFF, "gate table and dh' slab end before h");
  if (wn == 0) gtab[wm * WM + (te & 63)] = gate_lane;

  // Per row: g h (16-byte stores), and the tile's share of dgate_p =
  // sum_f dh' h in the SwiGLU-backward epilogue's order for 128 columns: each
  // thread sums 8 consecutive columns in order (fmaf), then an xor butterfly
  // over the row's 16 threads.  dh' goes through LDS one wave row slice at a
  // time; h is read from its LDS copy.
  constexpr int G8 = BN / 8;  // 16 threads per row
  constexpr int RSTEP = C::THREADS / G8;
  static_assert(G8 == 16 && SR % RSTEP == 0, "row layout");
  T* Chg = static_cast<T*>(p.h_hg);
#pragma unroll
  for (int sl = 0; sl < S::WGM; ++sl) {
    lds_barrier();  // the previous slab's readers are done (and the gate table written)
    if (wm == sl) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            dvs[(i * 16 + 4 * eg + q) * LDV + wn * WN + j * 16 + e16] = acc2[i][j][q];
    }
    lds_barrier();
    const int c = te % G8;
#pragma unroll
    for (int it = 0; it < SR / RSTEP; ++it) {
      const int r = te / G8 + it * RSTEP;  // row within the slab
      const int tr = sl * SR + r;          // row within the tile
      const f32x4_t d0 = *reinterpret_cast<const f32x4_t*>(dvs + r * LDV + c * 8);
      const f32x4_t d1 = *reinterpret_cast<const f32x4_t*>(dvs + r * LDV + c * 8 + 4);
      const u32x4_t hw = *reinterpret_cast<const u32x4_t*>(hrow + tr * BN + c * 8);
      float hv[8];
      unpack16(hw, hv, T());
      const float g = gtab[tr];
      float part = 0.f, hg[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        part = fmaf(q < 4 ? d0[q] : d1[q - 4], hv[q], part);
        hg[q] = g * hv[q];
      }
#pragma unroll
      for (int m = 1; m < G8; m <<= 1) part += __shfl_xor(part, m);
      if (m0 + tr < row_end) {
        *reinterpret_cast<u32x4_t*>(Chg + (int64_t)(m0 + tr) * p.F + n0 + c * 8) = pack16(hg, T());
        if (c == 0) p.dgp[(int64_t)(n0 / BN) * p.dgp_rows + m0 + tr] = part;
      }
    }
  }

  // da and du, each staged through LDS as bf16 rows (padded by 16 bytes) and
  // written with 16-byte row-contiguous stores
  constexpr int LD = BN + 8;
  constexpr int V = BN / 8;
  T* stg = reinterpret_cast<T*>(smem + BM * 4);  // past the gate table
  static_assert(BM * 4 + BM * LD * 2 <= H_OFF, "output staging ends before h");
  float rg[FM][4];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) rg[i][q] = __shfl(gate_lane, i * 16 + 4 * eg + q, 64);
#pragma unroll
  for (int o = 0; o < 2; ++o) {
    lds_barrier();  // the previous users of the staging area are done
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float av = unpk(pa[i][j], q), uv = unpk(pu[i][j], q);
          const float sa = logistic(av);
          const float d = rg[i][q] * acc2[i][j][q];
          const float v = o == 0 ? d * uv * sa * (1.f + av * (1.f - sa)) : d * av * sa;
          stg[(wm * WM + i * 16 + 4 * eg + q) * LD + wn * WN + j * 16 + e16] = f2bf(v);
        }
    lds_barrier();
    T* Cout = static_cast<T*>(o == 0 ? p.a_da : p.u_du);
    for (int idx = te; idx < BM * V; idx += C::THREADS) {
      const int r = idx / V, c = idx - r * V;
      if (m0 + r >= row_end) break;  // rows ascend with idx
      *reinterpret_cast<u32x4_t*>(Cout + (int64_t)(m0 + r) * p.F + n0 + c * 8) =
          *reinterpret_cast<const u32x4_t*>(stg + r * LD + c * 8);
    }
  }
}

template <class S>
hipError_t launch_fused_bwd(const FusedBwdParams& p, dim3 grid, hipStream_t st) {
  using C = LdsCfg<S, true>;
  if (p.H % (S::BK * C::NS) != 0 || p.F % S::BN != 0) return hipErrorInvalidValue;
  auto kern = fused_bwd_kernel<S>;
  constexpr int lds = kLdsBytes;
  static bool attr_set = false;
  if (hipError_t err = set_lds_attr(kern, lds, attr_set); err != hipSuccess) return err;
  kern<<<grid, C::THREADS, lds, st>>>(p);
  return hipGetLastError();
}

}  // namespace gemm
}  // namespace moe
