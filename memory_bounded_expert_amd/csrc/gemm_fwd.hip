// Forward contractions: router logits, expert up-projection with the fused
// SwiGLU epilogue, expert down-projection.
#include "gemm_kernel.hpp"
#include "gemm_lds.hpp"

namespace moe {
using namespace gemm;

namespace {
// 256-row tiles: 4 x 2 waves of 64 x (BN/2) per operand group
template <int BN>
using Big = Shape<256, BN, 4, 2, 32, 1>;

hipError_t up_swiglu_bf16(const Params& p, dim3 grid, int bn, bool save, int rt, hipStream_t st) {
  if (rt == kRowTileLarge) {
    if (bn == 128)
      return save ? launch_lds<Mode::Rows, Big<128>, true, true, false, false, Epi::SwiGLUSave>(p, grid, st)
                  : launch_lds<Mode::Rows, Big<128>, true, true, false, false, Epi::SwiGLU>(p, grid, st);
    return hipErrorInvalidValue;
  }
  if (bn == 256) return launch_lds<Mode::Rows, Shape<128, 256, 2, 4, 32, 1>, true, true, false, false, Epi::SwiGLU>(p, grid, st);
  if (bn == 128) {
    return save ? launch_lds<Mode::Rows, Shape<128, 128, 2, 4, 64, 1>, true, true, false, false, Epi::SwiGLUSave>(p, grid, st)
                : launch_lds<Mode::Rows, Shape<128, 128, 2, 4, 64, 1>, true, true, false, false, Epi::SwiGLU>(p, grid, st);
  }
  return save ? launch_lds<Mode::Rows, Shape<128, 64, 2, 4, 64, 1>, true, true, false, false, Epi::SwiGLUSave>(p, grid, st)
              : launch_lds<Mode::Rows, Shape<128, 64, 2, 4, 64, 1>, true, true, false, false, Epi::SwiGLU>(p, grid, st);
}

hipError_t down_bf16(const Params& p, dim3 grid, int bn, int rt, hipStream_t st) {
  if (rt == kRowTileLarge) {
    if (bn == 256) return launch_lds<Mode::Rows, Big<256>, false, true, false, false, Epi::Store>(p, grid, st);
    if (bn == 128) return launch_lds<Mode::Rows, Big<128>, false, true, false, false, Epi::Store>(p, grid, st);
    return hipErrorInvalidValue;
  }
  if (bn == 512) return launch_lds<Mode::Rows, Shape<128, 512, 2, 4, 32, 1>, false, true, false, false, Epi::Store>(p, grid, st);
  if (bn == 256) return launch_lds<Mode::Rows, Shape<128, 256, 2, 4, 64, 1>, false, true, false, false, Epi::Store>(p, grid, st);
  if (bn == 128) return launch_lds<Mode::Rows, Shape<128, 128, 2, 4, 64, 1>, false, true, false, false, Epi::Store>(p, grid, st);
  return launch_lds<Mode::Rows, Shape<128, 64, 2, 4, 64, 1>, false, true, false, false, Epi::Store>(p, grid, st);
}

// Split plans: the 256-row tiles and the short segments' 128-row tiles of one
// product in one launch.
template <class G1>
hipError_t up_pair(const Params& pb, int nb, const Params& ps, int ns, int bns, hipStream_t st) {
  if (bns == 256)
    return launch_lds_pair<G1, RowsGemm<Shape<128, 256, 2, 4, 32, 1>, true, true, false, false, Epi::SwiGLU>>(pb, nb, ps, ns, st);
  if (bns == 128)
    return launch_lds_pair<G1, RowsGemm<Shape<128, 128, 2, 4, 64, 1>, true, true, false, false, Epi::SwiGLU>>(pb, nb, ps, ns, st);
  return hipErrorInvalidValue;
}

template <typename T>
hipError_t up_swiglu_t(const Params& p, dim3 grid, int bn, bool save, hipStream_t st) {
  if (bn == 128) {
    return save ? launch<T, Mode::Rows, 128, 128, true, true, false, false, Epi::SwiGLUSave>(p, grid, st)
                : launch<T, Mode::Rows, 128, 128, true, true, false, false, Epi::SwiGLU>(p, grid, st);
  }
  return save ? launch<T, Mode::Rows, 128, 64, true, true, false, false, Epi::SwiGLUSave>(p, grid, st)
              : launch<T, Mode::Rows, 128, 64, true, true, false, false, Epi::SwiGLU>(p, grid, st);
}

template <typename T>
hipError_t down_t(const Params& p, dim3 grid, int bn, hipStream_t st) {
  if (bn == 256) return launch<T, Mode::Rows, 128, 256, false, true, false, false, Epi::Store>(p, grid, st);
  if (bn == 128) return launch<T, Mode::Rows, 128, 128, false, true, false, false, Epi::Store>(p, grid, st);
  return launch<T, Mode::Rows, 128, 64, false, true, false, false, Epi::Store>(p, grid, st);
}
}  // namespace

hipError_t gemm_up_swiglu(int dtype, const RowsGeom& g, const void* Xp, const void* Wg,
                          const void* Wu, void* h, void* a, void* u, int H, int F, hipStream_t st,
                          const int32_t* rows, int k, int64_t x_rows, const RowsGeom* gs) {
  if (g.grid_m == 0) return hipSuccess;
  Params p{};
  p.A = Xp; p.lda = H;
  if (rows) {
    if (dtype != MOE_BF16) return hipErrorInvalidValue;
    p.a_rows = rows; p.a_row_div = k; p.a_src_rows = x_rows;
  }
  p.B = Wg; p.B2 = Wu; p.ldb = F; p.b_estride = (int64_t)H * F;
  p.C = h; p.C2 = a; p.C3 = u; p.ldc = F;
  p.N = F; p.K = H;
  p.tiles = g.tiles; p.tile_count = g.tile_count; p.offsets = g.offsets;
  const bool save = a != nullptr;
  const bool big = g.row_tile == kRowTileLarge;
  if (g.kt_rows > 0) {
    // the forward's K-tile-major h (written here, read by the down projection)
    if (dtype != MOE_BF16 || save || !big || F % 32) return hipErrorInvalidValue;
    p.c_kt = g.kt_rows * 32;
  }
  const int bn = (dtype == MOE_BF16 && !save && !big && F % 256 == 0) ? 256 : (F % 128 == 0 ? 128 : 64);
  p.ntiles = F / bn;
  const dim3 grid((unsigned)(g.grid_m * p.ntiles));
  if (gs && dtype == MOE_BF16 && big && !save && bn == 128) {
    Params ps = p;
    ps.tiles = gs->tiles; ps.tile_count = gs->tile_count;
    const int bns = F % 256 == 0 ? 256 : 128;
    ps.ntiles = F / bns;
    return up_pair<RowsGemm<Big<128>, true, true, false, false, Epi::SwiGLU>>(
        p, (int)grid.x, ps, (int)(gs->grid_m * ps.ntiles), bns, st);
  }
  if (gs) return hipErrorInvalidValue;
  return dtype == MOE_BF16 ? up_swiglu_bf16(p, grid, bn, save, g.row_tile, st)
                           : up_swiglu_t<float>(p, grid, bn, save, st);
}

hipError_t gemm_down(int dtype, const RowsGeom& g, const void* h, const void* Wd, void* O, int H,
                     int F, hipStream_t st, const float* row_gates, const RowsGeom* gl,
                     const RowsGeom* gs) {
  if (g.grid_m == 0) return hipSuccess;
  Params p{};
  p.A = h; p.lda = F;
  p.B = Wd; p.ldb = H; p.b_estride = (int64_t)F * H;
  p.C = O; p.ldc = H;
  p.row_scale = row_gates;
  p.N = H; p.K = F;
  p.tiles = g.tiles; p.tile_count = g.tile_count; p.offsets = g.offsets;
  if (g.kt_rows > 0) {
    // h K-tile-major: read by the 256-row shapes, whose K-tiles are 32 wide
    if (dtype != MOE_BF16 || g.row_tile != kRowTileLarge || F % 32) return hipErrorInvalidValue;
    p.a_kt = g.kt_rows * 32;
  }
  const int bn = g.row_tile == kRowTileLarge ? (H % 256 == 0 ? 256 : 128)
                 : (dtype == MOE_BF16 && H % 512 == 0) ? 512 : pick_bn(H, true);
  p.ntiles = H / bn;
  if (gl && gs && dtype == MOE_BF16 && g.row_tile == kRowTileLarge && H % 512 == 0) {
    // the long segments' 256-row tiles and the short ones' 128 x 512 tiles
    // (K-tiles 32 wide, as the K-tile-major h needs) in one launch
    // (128 rows: twice the weight bytes in flight per stage for a segment
    // of few rows).  Below four rounds of work-groups the larger tiles cost
    // more in the launch's tail than that gains, and the launch runs g's
    // unsplit list in 256-row tiles instead.
    Params pl = p, ps = p;
    pl.tiles = gl->tiles; pl.tile_count = gl->tile_count;
    ps.tiles = gs->tiles; ps.tile_count = gs->tile_count;
    ps.ntiles = H / 512;
    // the first grid also covers g's (the unsplit list's ids start at 0)
    return launch_lds_pair<RowsGemm<Big<256>, false, true, false, false, Epi::Store>,
                           RowsGemm<Shape<128, 512, 2, 4, 32, 1>, false, true, false, false, Epi::Store>,
                           true>(pl, (int)(std::max(gl->grid_m, g.grid_m) * pl.ntiles), ps,
                                 (int)(gs->grid_m * ps.ntiles), st, &p, 4 * kCus);
  }
  const dim3 grid((unsigned)(g.grid_m * p.ntiles));
  return dtype == MOE_BF16 ? down_bf16(p, grid, bn, g.row_tile, st) : down_t<float>(p, grid, bn, st);
}

hipError_t gemm_router(int dtype, const void* X, const void* Wr, const float* bias, float* logits,
                       int64_t N, int H, int E, hipStream_t st, float* parts, int S) {
  if (N == 0) return hipSuccess;
  Params p{};
  p.A = X; p.lda = H;
  p.B = Wr; p.ldb = E;
  p.C = logits; p.ldc = E;
  p.M = (int)N; p.N = E; p.K = H;
  p.bias = bias;
  if (S > 1) {
    if (dtype != MOE_BF16 || !parts || H % (64 * S) != 0) return hipErrorInvalidValue;
    p.C = parts; p.c_estride = N * E; p.Kseg = H / S; p.bias = nullptr;
    const dim3 grid((unsigned)ceil_div(N, 128), (unsigned)ceil_div(E, 64), (unsigned)S);
    return launch_lds<Mode::Dense, Shape<128, 64, 2, 4, 64, 1>, false, true, false, false, Epi::F32>(p, grid, st);
  }
  const dim3 grid((unsigned)ceil_div(N, 128), (unsigned)ceil_div(E, 64));
  return dtype == MOE_BF16
             ? launch_lds<Mode::Dense, Shape<128, 64, 2, 4, 64, 1>, false, true, false, false, Epi::BiasF32>(p, grid, st)
             : launch<float, Mode::Dense, 128, 64, false, true, false, false, Epi::BiasF32>(p, grid, st);
}

}  // namespace moe
