// Backward contractions: dY W_down^T, [da du] [W_gate W_up]^T, and the
// per-expert weight gradients accumulated chunk by chunk.
#include "gemm_fused_bwd.hpp"
#include "gemm_kernel.hpp"
#include "gemm_lds.hpp"

namespace moe {
using namespace gemm;

namespace {
// 256-row tiles: 4 x 2 waves of 64 x (BN/2)
template <int BN>
using Big = Shape<256, BN, 4, 2, 32, 1>;

hipError_t dh_bf16(const Params& p, dim3 grid, int bn, int rt, hipStream_t st) {
  if (rt == kRowTileLarge) {
    if (bn == 256) return launch_lds<Mode::Rows, Big<256>, false, true, true, false, Epi::F32>(p, grid, st);
    if (bn == 128) return launch_lds<Mode::Rows, Big<128>, false, true, true, false, Epi::F32>(p, grid, st);
    return hipErrorInvalidValue;
  }
  if (bn == 256) return launch_lds<Mode::Rows, Shape<128, 256, 2, 4, 64, 1>, false, true, true, false, Epi::F32>(p, grid, st);
  if (bn == 128) return launch_lds<Mode::Rows, Shape<128, 128, 2, 4, 64, 1>, false, true, true, false, Epi::F32>(p, grid, st);
  return launch_lds<Mode::Rows, Shape<128, 64, 2, 4, 64, 1>, false, true, true, false, Epi::F32>(p, grid, st);
}

hipError_t dh_swiglu_bf16(const Params& p, dim3 grid, int bn, int rt, hipStream_t st) {
  constexpr Epi E = Epi::SwiGLUBwd;
  if (rt == kRowTileLarge) {
    if (bn == 256) return launch_lds<Mode::Rows, Big<256>, false, true, true, false, E>(p, grid, st);
    if (bn == 128) return launch_lds<Mode::Rows, Big<128>, false, true, true, false, E>(p, grid, st);
    return hipErrorInvalidValue;
  }
  if (bn == 256) return launch_lds<Mode::Rows, Shape<128, 256, 2, 4, 64, 1>, false, true, true, false, E>(p, grid, st);
  if (bn == 128) return launch_lds<Mode::Rows, Shape<128, 128, 2, 4, 64, 1>, false, true, true, false, E>(p, grid, st);
  return launch_lds<Mode::Rows, Shape<128, 64, 2, 4, 64, 1>, false, true, true, false, E>(p, grid, st);
}

hipError_t dx_bf16(const Params& p, dim3 grid, int bn, int rt, hipStream_t st) {
  if (rt == kRowTileLarge) {
    if (bn == 256) return launch_lds<Mode::Rows, Big<256>, false, true, true, true, Epi::Store>(p, grid, st);
    if (bn == 128) return launch_lds<Mode::Rows, Big<128>, false, true, true, true, Epi::Store>(p, grid, st);
    return hipErrorInvalidValue;
  }
  if (bn == 256) return launch_lds<Mode::Rows, Shape<128, 256, 2, 4, 64, 1>, false, true, true, true, Epi::Store>(p, grid, st);
  if (bn == 128) return launch_lds<Mode::Rows, Shape<128, 128, 2, 4, 64, 1>, false, true, true, true, Epi::Store>(p, grid, st);
  return launch_lds<Mode::Rows, Shape<128, 64, 2, 4, 64, 1>, false, true, true, true, Epi::Store>(p, grid, st);
}

template <int BM, Mode MODE>
hipError_t wgu_bf16(const Params& p, dim3 grid, int bn, hipStream_t st) {
  if (bn == 128) return launch_lds<MODE, Shape<BM, 128, 2, 2, 32, 2>, true, false, false, false, Epi::AccF32>(p, grid, st);
  return launch_lds<MODE, Shape<BM, 64, 2, 4, 64, 1>, true, false, false, false, Epi::AccF32>(p, grid, st);
}

template <int BM, Mode MODE>
hipError_t wd_bf16(const Params& p, dim3 grid, int bn, hipStream_t st) {
  if (bn == 256) return launch_lds<MODE, Shape<BM, 256, 2, 2, 32, 2>, false, false, false, false, Epi::AccF32>(p, grid, st);
  if (bn == 128) return launch_lds<MODE, Shape<BM, 128, 2, 4, 64, 1>, false, false, false, false, Epi::AccF32>(p, grid, st);
  return launch_lds<MODE, Shape<BM, 64, 2, 4, 64, 1>, false, false, false, false, Epi::AccF32>(p, grid, st);
}

// K-rows read through rows[r] / k of a x_rows-row source: the division as
// a multiply-shift, exact while every rows[r] * k < 2^32 (rows[r] < x_rows k)
bool set_k_rows(Params& p, const int32_t* rows, int k, int64_t x_rows) {
  if (k < 1 || x_rows < 1 || !indexed_rows_ok(x_rows, k)) return false;
  p.k_rows = rows;
  p.k_row_mul = k == 1 ? 0u : (uint32_t)(((1ull << 32) + (uint64_t)k - 1) / (uint64_t)k);
  p.k_src_rows = x_rows;
  return true;
}

template <typename T>
hipError_t dh_t(const Params& p, dim3 grid, int bn, hipStream_t st) {
  if (bn == 256) return launch<T, Mode::Rows, 128, 256, false, true, true, false, Epi::F32>(p, grid, st);
  if (bn == 128) return launch<T, Mode::Rows, 128, 128, false, true, true, false, Epi::F32>(p, grid, st);
  return launch<T, Mode::Rows, 128, 64, false, true, true, false, Epi::F32>(p, grid, st);
}

template <typename T>
hipError_t dx_t(const Params& p, dim3 grid, int bn, hipStream_t st) {
  if (bn == 256) return launch<T, Mode::Rows, 128, 256, false, true, true, true, Epi::Store>(p, grid, st);
  if (bn == 128) return launch<T, Mode::Rows, 128, 128, false, true, true, true, Epi::Store>(p, grid, st);
  return launch<T, Mode::Rows, 128, 64, false, true, true, true, Epi::Store>(p, grid, st);
}

template <typename T, int BM>
hipError_t wgu_t(const Params& p, dim3 grid, int bn, hipStream_t st) {
  if (bn == 128) return launch<T, Mode::Expert, BM, 128, true, false, false, false, Epi::AccF32>(p, grid, st);
  return launch<T, Mode::Expert, BM, 64, true, false, false, false, Epi::AccF32>(p, grid, st);
}

template <typename T, int BM>
hipError_t wd_t(const Params& p, dim3 grid, int bn, hipStream_t st) {
  if (bn == 256) return launch<T, Mode::Expert, BM, 256, false, false, false, false, Epi::AccF32>(p, grid, st);
  if (bn == 128) return launch<T, Mode::Expert, BM, 128, false, false, false, false, Epi::AccF32>(p, grid, st);
  return launch<T, Mode::Expert, BM, 64, false, false, false, false, Epi::AccF32>(p, grid, st);
}
}  // namespace

hipError_t gemm_dh(int dtype, const RowsGeom& g, const void* dYp, const void* Wd, float* dh, int H,
                   int F, hipStream_t st) {
  if (g.grid_m == 0) return hipSuccess;
  Params p{};
  p.A = dYp; p.lda = H;
  p.B = Wd; p.ldb = H; p.b_estride = (int64_t)F * H;  // row f of W_down[e] holds K = H
  p.C = dh; p.ldc = F;
  p.N = F; p.K = H;
  p.tiles = g.tiles; p.tile_count = g.tile_count; p.offsets = g.offsets;
  const int bn = g.row_tile == kRowTileLarge ? (F % 256 == 0 ? 256 : 128) : pick_bn(F, true);
  p.ntiles = F / bn;
  const dim3 grid((unsigned)(g.grid_m * p.ntiles));
  return dtype == MOE_BF16 ? dh_bf16(p, grid, bn, g.row_tile, st) : dh_t<float>(p, grid, bn, st);
}

// The dgate shares are per 128 columns of F (64 when F is not a multiple of
// 128), whatever the row tiles, so that chunkings whose chunks take different
// tile shapes (or the fused recompute + dh kernel) sum them alike.
int dh_ntiles(const RowsGeom& g, int F) {
  (void)g;
  return F / (F % kFusedDhTile == 0 ? kFusedDhTile : 64);
}

hipError_t gemm_dh_swiglu(const RowsGeom& g, const void* dYp, const void* Wd, void* a_da,
                          void* u_du, void* h_hg, const int32_t* perm, const float* gates,
                          float* dgp, int64_t rows, int64_t Nk, int H, int F, hipStream_t st,
                          int k, int64_t x_rows) {
  if (g.grid_m == 0) return hipSuccess;
  Params p{};
  p.A = dYp; p.lda = H;
  if (x_rows > 0) {  // row r of the chunk is row perm[r] / k of dY
    if (k < 1) return hipErrorInvalidValue;
    p.a_rows = perm; p.a_row_div = k; p.a_src_rows = x_rows;
  }
  p.B = Wd; p.ldb = H; p.b_estride = (int64_t)F * H;  // row f of W_down[e] holds K = H
  p.C = h_hg; p.C2 = a_da; p.C3 = u_du; p.ldc = F;
  p.N = F; p.K = H;
  p.tiles = g.tiles; p.tile_count = g.tile_count; p.offsets = g.offsets;
  p.sw_perm = perm; p.sw_gates = gates; p.sw_dgp = dgp; p.sw_rows = rows; p.sw_nk = Nk;
  p.ntiles = dh_ntiles(g, F);
  const int bn = F / p.ntiles;
  const dim3 grid((unsigned)(g.grid_m * p.ntiles));
  return dh_swiglu_bf16(p, grid, bn, g.row_tile, st);
}

hipError_t gemm_recompute_dh(const RowsGeom& g, const void* Xp, const void* dYp, const void* Wg,
                             const void* Wu, const void* Wd, void* a_da, void* u_du, void* h_hg,
                             const int32_t* perm, const float* gates, float* dgp, int64_t rows,
                             int64_t Nk, int H, int F, hipStream_t st, int k, int64_t x_rows) {
  if (g.grid_m == 0) return hipSuccess;
  if (g.row_tile != kRowTileLarge || F % kFusedDhTile != 0 || H % 128 != 0) return hipErrorInvalidValue;
  static_assert(FusedBwdShape::BN == kFusedDhTile && FusedBwdShape::BM == kRowTileLarge, "tile");
  FusedBwdParams p{};
  p.X = Xp; p.dY = dYp; p.lda = H;
  if (x_rows > 0) {  // row r of the chunk is row perm[r] / k of X and of dY
    if (k < 1) return hipErrorInvalidValue;
    p.a_rows = perm; p.a_row_div = k; p.a_src_rows = x_rows;
  }
  p.Wg = Wg; p.Wu = Wu; p.Wd = Wd;
  p.H = H; p.F = F;
  p.h_hg = h_hg; p.a_da = a_da; p.u_du = u_du;
  p.tiles = g.tiles; p.tile_count = g.tile_count; p.offsets = g.offsets;
  p.ntiles = F / kFusedDhTile;
  p.perm = perm; p.gates = gates; p.nk = Nk;
  p.dgp = dgp; p.dgp_rows = rows;
  const dim3 grid((unsigned)(g.grid_m * p.ntiles));
  return launch_fused_bwd<FusedBwdShape>(p, grid, st);
}

hipError_t gemm_dx(int dtype, const RowsGeom& g, const void* da, const void* du, const void* Wg,
                   const void* Wu, void* dXp, int H, int F, hipStream_t st) {
  if (g.grid_m == 0) return hipSuccess;
  Params p{};
  p.A = da; p.A2 = du; p.lda = F;
  p.B = Wg; p.B2 = Wu; p.ldb = F; p.b_estride = (int64_t)H * F;  // row h of W_gate[e] holds K = F
  p.C = dXp; p.ldc = H;
  p.N = H; p.K = 2 * F; p.Kseg = F;
  p.tiles = g.tiles; p.tile_count = g.tile_count; p.offsets = g.offsets;
  const int bn = g.row_tile == kRowTileLarge ? (H % 256 == 0 ? 256 : 128) : pick_bn(H, true);
  p.ntiles = H / bn;
  const dim3 grid((unsigned)(g.grid_m * p.ntiles));
  return dtype == MOE_BF16 ? dx_bf16(p, grid, bn, g.row_tile, st) : dx_t<float>(p, grid, bn, st);
}

hipError_t gemm_wgrad_gu(int dtype, const int32_t* offsets, const void* Xp, const void* da,
                         const void* du, float* dWg, float* dWu, int E, int H, int F,
                         hipStream_t st, bool init, const int32_t* rows, int k, int64_t x_rows) {
  if (init && dtype != MOE_BF16) return hipErrorInvalidValue;
  Params p{};
  p.acc_init = init ? 1 : 0;
  p.A = Xp; p.lda = H;
  if (rows && (dtype != MOE_BF16 || !set_k_rows(p, rows, k, x_rows))) return hipErrorInvalidValue;
  p.B = da; p.B2 = du; p.ldb = F;
  p.C = dWg; p.C2 = dWu; p.ldc = F; p.c_estride = (int64_t)H * F;
  p.M = H; p.N = F;
  p.offsets = offsets;
  const int bm = H % 128 == 0 ? 128 : 64;
  const int bn = F % 128 == 0 ? 128 : 64;
  const dim3 grid((unsigned)(H / bm), (unsigned)(F / bn), (unsigned)E);
  if (rows)
    return bm == 128 ? wgu_bf16<128, Mode::ExpertIdx>(p, grid, bn, st)
                     : wgu_bf16<64, Mode::ExpertIdx>(p, grid, bn, st);
  if (dtype == MOE_BF16)
    return bm == 128 ? wgu_bf16<128, Mode::Expert>(p, grid, bn, st)
                     : wgu_bf16<64, Mode::Expert>(p, grid, bn, st);
  return bm == 128 ? wgu_t<float, 128>(p, grid, bn, st) : wgu_t<float, 64>(p, grid, bn, st);
}

hipError_t gemm_wgrad_d(int dtype, const int32_t* offsets, const void* hg, const void* dYp,
                        float* dWd, int E, int H, int F, hipStream_t st, bool init,
                        const int32_t* rows, int k, int64_t x_rows) {
  if (init && dtype != MOE_BF16) return hipErrorInvalidValue;
  Params p{};
  if (rows && (dtype != MOE_BF16 || !set_k_rows(p, rows, k, x_rows))) return hipErrorInvalidValue;
  p.acc_init = init ? 1 : 0;
  p.A = hg; p.lda = F;
  p.B = dYp; p.ldb = H;
  p.C = dWd; p.ldc = H; p.c_estride = (int64_t)F * H;
  p.M = F; p.N = H;
  p.offsets = offsets;
  const int bm = F % 128 == 0 ? 128 : 64;
  const int bn = pick_bn(H, true);
  const dim3 grid((unsigned)(F / bm), (unsigned)(H / bn), (unsigned)E);
  if (dtype == MOE_BF16)
    return rows ? (bm == 128 ? wd_bf16<128, Mode::ExpertIdxB>(p, grid, bn, st)
                             : wd_bf16<64, Mode::ExpertIdxB>(p, grid, bn, st))
                : (bm == 128 ? wd_bf16<128, Mode::Expert>(p, grid, bn, st)
                             : wd_bf16<64, Mode::Expert>(p, grid, bn, st));
  return bm == 128 ? wd_t<float, 128>(p, grid, bn, st) : wd_t<float, 64>(p, grid, bn, st);
}

}  // namespace moe
