// Contractions of the vocabulary-strip cross-entropy (bf16, LDS pipeline):
// the strip's logits X W_s^T with the statistics or gradient epilogue, the
// running sum dX += G W_s, and the strip's weight gradient dW_s = G^T X.
#include "gemm_kernel.hpp"
#include "gemm_lds.hpp"

namespace moe {
using namespace gemm;

namespace {
// 256 x 256 tiles of 4 x 2 waves; each wave's 64 x 128 block is one
// 128-column vocabulary slice of the statistics.
using Logit = Shape<256, 256, 4, 2, 32, 1>;
static_assert(Logit::BN / Logit::WGN == kCceSlice, "statistics slice = one wave's columns");
}  // namespace

hipError_t gemm_cce_logits(bool grad, const void* X, const void* Ws, int64_t N, int H, int w,
                           int64_t col0, const int32_t* targets, float* pmax, float* psum,
                           float* ytgt, const float* lse, const float* dl, void* G, int ldg,
                           hipStream_t st) {
  if (N == 0 || w == 0) return hipSuccess;
  Params p{};
  p.A = X; p.lda = H;
  p.B = Ws; p.ldb = H;
  p.M = (int)N; p.N = w; p.K = H;
  p.ce_targets = targets; p.ce_col0 = col0;
  const dim3 grid((unsigned)ceil_div(N, Logit::BM), (unsigned)ceil_div(w, Logit::BN));
  if (!grad) {
    p.ce_pmax = pmax; p.ce_psum = psum; p.ce_ytgt = ytgt;
    return launch_lds<Mode::Dense, Logit, false, true, true, false, Epi::CEStats>(p, grid, st);
  }
  p.ce_lse = lse; p.ce_dl = dl;
  p.C = G; p.ldc = ldg;
  return launch_lds<Mode::Dense, Logit, false, true, true, false, Epi::CEGrad>(p, grid, st);
}

hipError_t gemm_cce_dx(const void* G, int ldg, const void* Ws, int64_t N, int H, int w,
                       float* dx, bool first, hipStream_t st) {
  if (N == 0) return hipSuccess;
  Params p{};
  p.A = G; p.lda = ldg;
  p.B = Ws; p.ldb = H;
  p.C = dx; p.ldc = H;
  p.M = (int)N; p.N = H; p.K = w;
  p.acc_init = first ? 1 : 0;
  p.acc_chain = 1;
  const int bn = H % 256 == 0 ? 256 : 128;
  const dim3 grid((unsigned)ceil_div(N, 256), (unsigned)(H / bn));
  if (bn == 256)
    return launch_lds<Mode::Dense, Shape<256, 256, 4, 2, 32, 1>, false, true, false, false, Epi::AccF32>(p, grid, st);
  return launch_lds<Mode::Dense, Shape<256, 128, 4, 2, 32, 1>, false, true, false, false, Epi::AccF32>(p, grid, st);
}

hipError_t gemm_cce_dw(const void* G, int ldg, const void* X, int64_t N, int H, int w, float* dws,
                       hipStream_t st) {
  if (w == 0) return hipSuccess;
  Params p{};
  p.A = G; p.lda = ldg;
  p.B = X; p.ldb = H;
  p.C = dws; p.ldc = H; p.c_estride = 0;
  p.M = w; p.N = H; p.K = (int)N;  // one segment: rows [0, N) of G and X (no offsets)
  p.acc_init = 1;
  // K = N rows is long: 8 x 8 blocks of tiles run together and share their
  // K-tiles through L2 (the N-tile-fastest order re-reads all of X per M-tile)
  p.tile_group = kCceDwGroup;
  const int bn = H % 256 == 0 ? 256 : 128;
  const dim3 grid((unsigned)ceil_div(w, 128), (unsigned)(H / bn), 1u);
  if (bn == 256)
    return launch_lds<Mode::Expert, Shape<128, 256, 2, 2, 32, 2>, false, false, false, false, Epi::AccF32>(p, grid, st);
  return launch_lds<Mode::Expert, Shape<128, 128, 2, 4, 64, 1>, false, false, false, false, Epi::AccF32>(p, grid, st);
}

}  // namespace moe
