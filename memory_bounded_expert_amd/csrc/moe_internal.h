// Internal interfaces of libmoebound: chunk geometry, workspace layout and
// the kernel launchers.  Host code only; nothing here is exported.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moebound.h"

namespace moe {

// Rows of one M-tile of the row-grouped GEMMs; the planner emits its tile
// lists in this granularity.  Each M-tile streams its expert's whole weight
// slice, so an expert segment just over one tile costs two weight passes.
// bf16 chunks whose experts average at least kLargeTileMinRows rows use
// kRowTileLarge: under balanced routing segments cluster around the mean, and
// at a mean of about 128 rows half of them would spill into a second, almost
// empty 128-row tile.  (Under skewed routing the mean says little; the plan
// has no routing data to tell.)  Everything else uses kRowTile.
constexpr int kRowTile = 128;
constexpr int kRowTileLarge = 256;
constexpr int kLargeTileMinRows = 96;
// Tokens per planner block: one wave, one 64-bit membership mask per expert.
constexpr int kPlanBlock = 64;
constexpr uint32_t kPlanMagic = 0x4d4f4542u;  // "MOEB"

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Chunk i of K over N tokens (strided membership: tokens i, i+K, ...).
struct ChunkGeom {
  int64_t n;          // tokens in the chunk, ceil((N - i) / K)
  int64_t pair_base;  // k * (tokens in chunks 0..i-1)
};
inline ChunkGeom chunk_geom(int64_t N, int64_t K, int64_t k, int64_t i) {
  const int64_t q = N / K, rem = N % K;
  ChunkGeom g;
  g.n = q + (i < rem ? 1 : 0);
  g.pair_base = k * (i * q + (i < rem ? i : rem));
  return g;
}

inline int elem_bytes(int dtype) { return dtype == MOE_BF16 ? 2 : 4; }

// K slices of the bf16 router product: enough that the (N/128) x (E/64)
// output tiles times the slices fill the chip, each slice a whole number of
// 64-wide K-tiles and at least 256 deep.
inline int router_splits(const moe_plan_t& p) {
  if (p.dtype != MOE_BF16 || p.N == 0) return 1;
  const int64_t tiles = ceil_div(p.N, 128) * ceil_div(p.E, 64);
  int s = 1;
  while (s < 8 && tiles * s < 512 && p.H % (128 * s) == 0 && p.H / (2 * s) >= 256) s *= 2;
  return s;
}

// The bf16 forward reads each chunk's permuted input rows straight from X
// inside the gate/up GEMM (no gather kernel, no permuted-input buffer) when X
// fits one buffer resource's 32-bit offsets.
inline bool fused_gather(const moe_plan_t& p) {
  return p.dtype == MOE_BF16 && (int64_t)p.N * p.H * 2 <= 0x7FFFFFF0LL;
}

// A row index n of a pair (token n / k) divided by a multiply-shift stays
// exact while n * k < 2^32 for every n < x_rows * k.
inline bool indexed_rows_ok(int64_t x_rows, int k) {
  return x_rows >= 0 && k >= 1 && (uint64_t)x_rows * (uint64_t)k * (uint64_t)k < (1ull << 32);
}

// The bf16 backward also reads the permuted inputs from X (the recompute's
// gate/up GEMM and the gate/up weight gradient), so it keeps no Xp either,
// and the permuted output gradients from dY (the dh GEMM and the down weight
// gradient), so no gather runs.
inline bool fused_gather_bwd(const moe_plan_t& p) {
  return fused_gather(p) && indexed_rows_ok(p.N, p.k);
}

// Order-invariant weight gradients (MOE_PLAN_EXACT_DW): padded rows of a
// chunk's digit planes (each expert segment rounded up to 64 rows).
inline int64_t exact_ldk(const moe_plan_t& p) {
  return ((int64_t)p.k * p.c_eff + 64 * (int64_t)p.E + 63) / 64 * 64;
}
inline bool exact_dw_ok(const moe_plan_t& p) {
  return p.dtype == MOE_BF16 && p.H % 128 == 0 && p.F % 128 == 0 && p.c_eff <= 65536 &&
         (p.N == 0 || fused_gather_bwd(p)) &&
         (int64_t)(p.H > p.F ? p.H : p.F) * exact_ldk(p) < ((int64_t)1 << 31);
}

// Upper bound on the row-grouped GEMM's M-tiles of T rows for a chunk of R
// pairs: sum_e ceil(M_e / T) <= R / T + (number of non-empty experts).
inline int64_t max_row_tiles(int64_t R, int E, int T) {
  return R / T + (R < E ? R : E);
}
// Row tile for a plan: the large tile when the average expert segment of a
// full chunk (k c_eff rows over E experts) has at least kLargeTileMinRows rows.
inline int row_tile_for(const moe_plan_t& p) {
  return (p.dtype == MOE_BF16 && p.H % 128 == 0 && p.F % 128 == 0 &&
          (int64_t)p.k * p.c_eff >= (int64_t)kLargeTileMinRows * p.E)
             ? kRowTileLarge
             : kRowTile;
}

// The bf16 forward with kRowTileLarge tiles also lists its segments split: a
// segment of at most kRowTile rows gets one kRowTile-row tile (a 256-row tile
// over it leaves half its waves and loads idle), the others keep their
// 256-row tiles (two 128-row tiles would stream their weights twice).  The
// gate/up product runs the split lists as one launch; the down projection
// stays on the one list of 256-row tiles, which measured faster for it.
inline bool split_tiles(const moe_plan_t& p) {
  return p.dtype == MOE_BF16 && row_tile_for(p) == kRowTileLarge;
}

// The bf16 backward with kRowTileLarge tiles runs a chunk's recompute and
// dh products as one kernel (a, u, h stay in registers; 128-column tiles of F).
inline bool fused_recompute_dh(const moe_plan_t& p) {
  return p.dtype == MOE_BF16 && row_tile_for(p) == kRowTileLarge;
}

// Byte offsets of the workspace regions (each 256-byte aligned).
struct Layout {
  size_t logits = 0;      // [N][E] f32, forward only, when the caller passes none
  size_t rparts = 0;      // [S][N][E] f32 router partials (split router product)
  size_t rank = 0;        // [N*k] i32  rank of a pair inside its planner block
  size_t blk = 0;         // [K][nblk][E] i32 block counts, then block bases
  size_t offsets = 0;     // [K][E+1] i32
  size_t tiles = 0;       // [K][max_tiles] int2 (expert, first row)
  size_t tile_count = 0;  // [K] i32
  size_t small_tiles = 0; // [K][E] int2 forward with split tiles: short segments' tiles
  size_t small_count = 0; // [K] i32
  size_t long_tiles = 0;  // [K][max_tiles] int2 forward with split tiles: the other segments'
  size_t long_count = 0;  // [K] i32
  size_t perm = 0;        // [N*k] i32
  size_t pos = 0;         // [N*k] i32
  size_t row_gates = 0;   // [N*k] f32 forward: gates in permuted-row order
  size_t xp = 0;          // [k c_eff][H]  permuted inputs (dispatch buffer 1)
  size_t o = 0;           // [k c_eff][H]  expert outputs / (dY rows, then) dXp (buffer 2)
  size_t h = 0;           // [k c_eff][F]  h (forward); h, then g*h (backward)
  size_t a = 0;           // [k c_eff][F]  backward: a, then da
  size_t u = 0;           // [k c_eff][F]  backward: u, then du
  size_t dh = 0;          // [k c_eff][F] f32 backward, fp32: dY W_down^T
  size_t dgp = 0;         // [F/64][k c_eff] f32 backward, bf16: dgate shares per N-tile
  size_t wrt = 0;         // [E][H] backward: W_r transposed
  size_t dgates = 0;      // [N*k] f32 backward, when the caller passes none
  // backward with MOE_PLAN_EXACT_DW (exact_dw.hip):
  size_t cmax = 0;        // u32 column maxima: X [H], dY [H], da, du, g h [E][F] each
  size_t offpad = 0;      // [E+1] i32 padded segment starts of the current chunk
  size_t planes = 0;      // int8 digit planes [C][ldk]: X, dY (C = H), da, du, g h (C = F), hi and lo
  size_t acc_hi = 0;      // [3][E][H][F] i32 high words of the dW_gate, dW_up, dW_down accumulators
  int64_t ldk = 0;        // padded rows per digit plane
  size_t total = 0;
  int64_t nblk = 0;
  int64_t max_tiles = 0;
  int row_tile = kRowTile;
  bool split = false;     // small_tiles / small_count present
};

// ---- order-invariant weight gradients (exact_dw.hip)
// Column maxima of |x| as fp32 bit patterns (atomicMax into zeroed arrays):
// over all N rows of a bf16 [N][C] matrix ...
hipError_t launch_colmax(const void* src, int64_t N, int C, uint32_t* out, hipStream_t st);
// ... and per expert over a chunk's expert-sorted rows of three bf16 [R][C]
// buffers (segments offsets[e] .. offsets[e+1], at most max_rows rows).
hipError_t launch_colmax_rows(const void* a, const void* u, const void* h, const int32_t* offsets,
                              int E, int C, int64_t max_rows, uint32_t* amax, uint32_t* umax,
                              uint32_t* hmax, hipStream_t st);
// One matrix whose chunk rows become digit planes: row r of the chunk is
// source row rows[r] / row_div (or r itself without rows) of src.
struct DigitPlanesSrc {
  const void* src;
  int64_t ld;
  int C;
  const int32_t* rows;
  int row_div;
  const uint32_t* cmax;  // [C], or [E][C] with per_expert
  int per_expert;
  int8_t* hi;            // [C][ldk]
  int8_t* lo;
};
struct ExactChunk {
  DigitPlanesSrc X, dY, da, du, hg;
  const int32_t* offsets;  // the chunk's [E+1] segments
  int32_t* offpad;         // [E+1] written: padded segment starts
  int E;
  int64_t ldk;
};
// The chunk's padded segment starts, then the digit planes of all five
// (two kernels, added to *launches).
hipError_t launch_digitize(const ExactChunk& x, hipStream_t st, int* launches);
// acc64[e][m][n] (init: =, else +=) sum over expert e's chunk rows of
// vA[m][k] vB[n][k], from digit planes; the 64-bit accumulator is split into
// c_lo (low words) and c_hi.  M % 128 == 0, N % 64 == 0.
hipError_t launch_exact_wgrad(const int8_t* a_hi, const int8_t* a_lo, const int8_t* b_hi,
                              const int8_t* b_lo, int64_t ldk, const int32_t* offsets,
                              const int32_t* offpad, uint32_t* c_lo, int32_t* c_hi, int E, int M,
                              int N, bool init, hipStream_t st);
// dw[e][m][n] = acc64 * 2^((eA_m - 14) + (eB_n - 14)), rounded once to fp32,
// in place over the low words in dw.
hipError_t launch_exact_finalize(float* dw, const int32_t* c_hi, const uint32_t* amax,
                                 bool a_per_expert, const uint32_t* bmax, bool b_per_expert, int E,
                                 int M, int N, hipStream_t st);

enum class Pass { Forward, Backward, Debug };
Layout make_layout(const moe_plan_t& p, Pass pass, bool need_logits, bool need_dgates);

// The forward call's argument checks (plan and required pointers; MOE_OK or
// the status to return) and its launch sequence on a workspace of at least
// make_layout(P, Pass::Forward, logits == nullptr, false).total bytes.
int check_forward_args(const moe_plan_t* plan, const void* X, const void* W_r,
                       const void* W_gate, const void* W_up, const void* W_down, const void* Y,
                       const int32_t* topk_idx, const float* gates);
int forward_impl(const moe_plan_t& P, const void* X, const void* W_r, const float* router_bias,
                 const void* W_gate, const void* W_up, const void* W_down, void* Y,
                 int32_t* topk_idx, float* gates, float* logits, void* workspace,
                 hipStream_t st, moe_stats_t* stats);

// ---- launchers (all asynchronous on `st`; return the first enqueue error)
// With parts != nullptr the logits are first summed from the router's S
// partials (s ascending), plus bias, and written to logits.
hipError_t launch_topk(const float* logits, int64_t N, int E, int k, int32_t* idx, float* gates,
                       hipStream_t st, const float* parts = nullptr, int S = 1,
                       const float* bias = nullptr);

struct PlanBuffers {
  int32_t* rank;
  int32_t* blk;
  int32_t* offsets;
  int2* tiles;
  int32_t* tile_count;
  int32_t* perm;
  int32_t* pos;
  float* row_gates;      // [N*k] gate of each permuted row (forward), or nullptr
  int64_t nblk;
  int64_t max_tiles;
  int row_tile;
  int2* small_tiles;     // nullptr: one tile list (split_tiles)
  int32_t* small_count;
  int2* long_tiles;
  int32_t* long_count;
};
// Plans every chunk at once: counts, scans and scatters the whole batch's
// routed pairs (O(N k) int32, nothing H-wide) in 3 launches, added to
// *launches when it is given.
// With b.row_gates set, also writes each permuted row's gate (gates [N*k]).
hipError_t launch_plan(const int32_t* idx, int64_t N, int K, int k, int E, const PlanBuffers& b,
                       hipStream_t st, const float* gates = nullptr, int* launches = nullptr);

// Data movement (dtype-dispatched: 0 f32, 1 bf16).
// Permute (gather) of chunk i: dst[pos[t, s]] = src[t] for each token t of the
// chunk and slot s with a valid expert idx[t, s] (each token row read once).
hipError_t launch_gather(int dtype, const void* src, void* dst, const int32_t* idx,
                         const int32_t* pos, int E, int K, int i, int64_t n_i, int k, int H,
                         hipStream_t st);
// Y[t] = sum_s O[pos[t, s]] over the k gate-scaled expert rows of each token
// of chunk i.
hipError_t launch_combine(int dtype, const void* O, const int32_t* pos, void* Y, int64_t N, int K,
                          int i, int64_t n_i, int k, int H, hipStream_t st);
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t st);
hipError_t launch_transpose(int dtype, const void* src, void* dst, int rows, int cols,
                            hipStream_t st);
hipError_t launch_swiglu_bwd(int dtype, const float* dh, void* a_da, void* u_du, void* h_hg,
                             const int32_t* perm_chunk, const float* gates, float* dgates,
                             int64_t R, int F, int64_t Nk, hipStream_t st);
// With dgp != nullptr the slots' dgates are first summed from the dh GEMM's
// per-N-tile shares (dgp [nparts][prow], tiles in order) and written to dgates.
hipError_t launch_combine_bwd(int dtype, const void* dXp, const void* WrT, const int32_t* idx,
                              const int32_t* pos, const float* gates, float* dgates,
                              void* dX, float* dlogits, int64_t N, int K, int i, int64_t n_i,
                              int k, int E, int H, hipStream_t st, const float* dgp = nullptr,
                              int nparts = 0, int64_t prow = 0);
// dW_r += X^T dlogits over chunk i's pairs (row r of the chunk's buffer is token
// perm_chunk[r] / k of X), summed per expert in row order.
hipError_t launch_dwr(int dtype, const void* X, const int32_t* perm_chunk, const int32_t* offsets,
                      const float* dlogits, float* dWr, int k, int E, int H, int64_t N,
                      hipStream_t st);

// GEMMs (tile schemes: gemm_lds.hpp for bf16, gemm_kernel.hpp for fp32).
struct RowsGeom {
  const int2* tiles;
  const int32_t* tile_count;
  const int32_t* offsets;
  int64_t grid_m;  // upper bound on the chunk's M-tiles
  int row_tile;    // rows per M-tile (kRowTile or kRowTileLarge)
  // > 0: the forward's h is stored K-tile-major -- 32-column blocks, each
  // holding all kt_rows rows of those 32 columns (64 bytes per row) -- so
  // that the down projection's A loads read whole 16 KiB blocks
  int64_t kt_rows = 0;
};
// The rows of the forward's K-tile-major h (bf16 chunks on 256-row tiles,
// whose gate/up epilogue and down projection take it so), else 0.
inline int64_t h_kt_rows(const moe_plan_t& p) {
  return (p.dtype == MOE_BF16 && row_tile_for(p) == kRowTileLarge) ? (int64_t)p.k * p.c_eff : 0;
}
// h = silu(Xp W_gate[e]) * (Xp W_up[e]) per expert segment; save_au also
// stores a and u.  With rows != nullptr (bf16 only), Xp is not a buffer:
// row r is row rows[r] / k of X (x_rows rows), read straight from X.
// With gs (a split plan's short-segment list, bf16 forward only), g (then
// the split plan's long-segment list) in 256-row tiles and gs in 128-row
// tiles run as one launch.
hipError_t gemm_up_swiglu(int dtype, const RowsGeom& g, const void* Xp, const void* Wg,
                          const void* Wu, void* h, void* a, void* u, int H, int F, hipStream_t st,
                          const int32_t* rows = nullptr, int k = 1, int64_t x_rows = 0,
                          const RowsGeom* gs = nullptr);
// O[r] = row_gates[r] (h[r] W_down[e]): each chunk row scaled by its pair's
// gate before the one rounding (row_gates as the planner lays them out).
// With gl and gs (a split plan's two lists; bf16, 256-row tiles, H a
// multiple of 512), gl's 256-row tiles and gs's 128-row tiles run as one
// launch; otherwise g's tiles.
hipError_t gemm_down(int dtype, const RowsGeom& g, const void* h, const void* Wd, void* O, int H,
                     int F, hipStream_t st, const float* row_gates,
                     const RowsGeom* gl = nullptr, const RowsGeom* gs = nullptr);
// dh = dYp W_down[e]^T (fp32 out)
hipError_t gemm_dh(int dtype, const RowsGeom& g, const void* dYp, const void* Wd, float* dh, int H,
                   int F, hipStream_t st);
// bf16: dh' = dYp W_down[e]^T with the SwiGLU backward in the epilogue (as
// launch_swiglu_bwd, dh' never stored): da, du, g h over a, u, h; the per
// N-tile shares of dgate into dgp [dh_ntiles][rows] (N-tiles of 128 columns,
// 64 when F is not a multiple of 128).
int dh_ntiles(const RowsGeom& g, int F);
// With x_rows > 0, dYp is not a buffer: row r of the chunk is row perm[r] / k
// of the x_rows-row dY, read straight from it.
hipError_t gemm_dh_swiglu(const RowsGeom& g, const void* dYp, const void* Wd, void* a_da,
                          void* u_du, void* h_hg, const int32_t* perm, const float* gates,
                          float* dgp, int64_t rows, int64_t Nk, int H, int F, hipStream_t st,
                          int k = 1, int64_t x_rows = 0);
// bf16, kRowTileLarge geometry: a = Xp W_gate[e], u = Xp W_up[e], h =
// silu(a) u (kept in registers, rounded to bf16), then dh' = dYp W_down[e]^T
// and the SwiGLU backward as gemm_dh_swiglu's, in one kernel: da, du and g h
// into a_da, u_du, h_hg, and the per 128-column tile shares of dgate into
// dgp [F / 128][rows].  With x_rows > 0 row r of the chunk is row perm[r] / k
// of X and dY (x_rows rows each); otherwise Xp and dYp are the chunk's rows.
hipError_t gemm_recompute_dh(const RowsGeom& g, const void* Xp, const void* dYp, const void* Wg,
                             const void* Wu, const void* Wd, void* a_da, void* u_du, void* h_hg,
                             const int32_t* perm, const float* gates, float* dgp, int64_t rows,
                             int64_t Nk, int H, int F, hipStream_t st, int k, int64_t x_rows);
constexpr int kFusedDhTile = 128;  // columns of F per tile of gemm_recompute_dh
// dXp = da W_gate[e]^T + du W_up[e]^T
hipError_t gemm_dx(int dtype, const RowsGeom& g, const void* da, const void* du, const void* Wg,
                   const void* Wu, void* dXp, int H, int F, hipStream_t st);
// dW_gate[e] += Xp_e^T da_e, dW_up[e] += Xp_e^T du_e; with init (bf16 only)
// the products are stored instead (dW = ..., zeros for experts with no rows).
// With rows != nullptr (bf16 only), Xp is X (x_rows rows): row r of the
// chunk is row rows[r] / k of X (indexed_rows_ok must hold).
hipError_t gemm_wgrad_gu(int dtype, const int32_t* offsets, const void* Xp, const void* da,
                         const void* du, float* dWg, float* dWu, int E, int H, int F,
                         hipStream_t st, bool init = false, const int32_t* rows = nullptr,
                         int k = 1, int64_t x_rows = 0);
// dW_down[e] += hg_e^T dYp_e (init as gemm_wgrad_gu).  With rows != nullptr
// (bf16 only), dYp is dY (x_rows rows): row r of the chunk is row rows[r] / k
// of dY (indexed_rows_ok must hold).
hipError_t gemm_wgrad_d(int dtype, const int32_t* offsets, const void* hg, const void* dYp,
                        float* dWd, int E, int H, int F, hipStream_t st, bool init = false,
                        const int32_t* rows = nullptr, int k = 1, int64_t x_rows = 0);
// logits = X W_r (+ bias), fp32 out.  With S > 1 (bf16 only) the product is
// split over K: parts[s] = X[:, s H/S : (s+1) H/S] W_r[s H/S : (s+1) H/S, :]
// for s < S ([S][N][E] fp32, no bias), and launch_topk adds them up.
hipError_t gemm_router(int dtype, const void* X, const void* Wr, const float* bias, float* logits,
                       int64_t N, int H, int E, hipStream_t st, float* parts = nullptr,
                       int S = 1);

// ---- vocabulary-strip cross-entropy (cce.hip, gemm_cce.hip)
// Columns per statistics slice: one wave's columns of the logits tile.
constexpr int kCceSlice = 128;
// M-tiles per dispatch group of the weight-gradient product (expert_tile).
constexpr int kCceDwGroup = 8;
// Logits of one strip, X [N][H] times Ws [w][H]^T.  grad = false: per-row
// slice statistics into pmax/psum [slice][N] and the target logit into ytgt.
// grad = true: the strip's logit gradient into G [N][ldg] bf16 (lse, dl [N]).
hipError_t gemm_cce_logits(bool grad, const void* X, const void* Ws, int64_t N, int H, int w,
                           int64_t col0, const int32_t* targets, float* pmax, float* psum,
                           float* ytgt, const float* lse, const float* dl, void* G, int ldg,
                           hipStream_t st);
// dx [N][H] fp32 = (first ? 0 : dx) + G[:, :w] Ws, one accumulation chain.
hipError_t gemm_cce_dx(const void* G, int ldg, const void* Ws, int64_t N, int H, int w,
                       float* dx, bool first, hipStream_t st);
// dws [w][H] fp32 = G[:, :w]^T X.
hipError_t gemm_cce_dw(const void* G, int ldg, const void* X, int64_t N, int H, int w, float* dws,
                       hipStream_t st);

}  // namespace moe
