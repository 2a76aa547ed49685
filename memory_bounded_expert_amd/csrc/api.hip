// C ABI of libmoebound: argument checks, the eq. (1) chunk plan, workspace
// carving and the per-chunk launch sequence.
//
// The chunk schedule follows the "Bounded-streaming operators" summary,
// Methodology 1 (PipelinedLLEP): eq. (1) gives K and c_eff, chunk i holds the
// strided token positions i, i+K, ..., and the dispatch buffers are sized by
// k * c_eff rows, never by N ("Memory bound", read with E_p = 1 and c_eff).
// The backward pass recomputes each chunk's expert intermediates from X and
// reuses the same buffers for the next chunk ("Nested gradient
// checkpointing"; hop-local recomputation in "Memory-Efficient Expert Routing
// for Distributed MoE Training", section 3.3).
//
// The library allocates nothing and never synchronises: every buffer comes
// from the caller's workspace and every kernel goes on the caller's stream.
#include <algorithm>
#include <cstring>

#include "moe_internal.h"

#define MOE_API extern "C" __attribute__((visibility("default")))

namespace moe {

Layout make_layout(const moe_plan_t& p, Pass pass, bool need_logits, bool need_dgates) {
  Layout L;
  size_t cur = 0;
  auto take = [&](size_t bytes) {
    const size_t o = cur;
    cur = (cur + bytes + 255) & ~(size_t)255;
    return o;
  };
  const size_t N = (size_t)p.N, k = (size_t)p.k, E = (size_t)p.E, H = (size_t)p.H,
               F = (size_t)p.F, K = (size_t)p.K, ce = (size_t)p.c_eff;
  const size_t b = (size_t)elem_bytes(p.dtype);
  if (N == 0) return L;
  L.nblk = ceil_div((int64_t)ce, kPlanBlock);
  L.row_tile = row_tile_for(p);
  L.max_tiles = max_row_tiles((int64_t)(k * ce), (int)E, L.row_tile);
  if (pass == Pass::Forward && need_logits) L.logits = take(N * E * 4);
  if (pass == Pass::Forward && router_splits(p) > 1) L.rparts = take((size_t)router_splits(p) * N * E * 4);
  L.rank = take(N * k * 4);
  L.blk = take(K * (size_t)L.nblk * E * 4);
  L.offsets = take(K * (E + 1) * 4);
  L.tiles = take(K * (size_t)L.max_tiles * 8);
  L.tile_count = take(K * 4);
  if (pass == Pass::Forward && split_tiles(p)) {
    L.split = true;
    L.small_tiles = take(K * E * 8);
    L.small_count = take(K * 4);
    L.long_tiles = take(K * (size_t)L.max_tiles * 8);
    L.long_count = take(K * 4);
  }
  if (pass != Pass::Debug) {
    L.perm = take(N * k * 4);
    L.pos = take(N * k * 4);
    if (pass == Pass::Forward) L.row_gates = take(N * k * 4);
    const size_t rows = k * ce;
    // the bf16 passes read their permuted inputs straight from X
    if (pass == Pass::Backward ? !fused_gather_bwd(p) : !fused_gather(p))
      L.xp = take(rows * H * b);
    L.o = take(rows * H * b);
    L.h = take(rows * F * b);
    if (pass == Pass::Backward) {
      L.a = take(rows * F * b);
      L.u = take(rows * F * b);
      // fp32: dY W_down^T for the separate SwiGLU backward; bf16: the dh
      // GEMM's per-N-tile dgate shares (at most F/64 tiles)
      if (p.dtype == MOE_BF16)
        L.dgp = take(((size_t)F / 64) * rows * 4);
      else
        L.dh = take(rows * F * 4);
      L.wrt = take(E * H * b);
      if (need_dgates) L.dgates = take(N * k * 4);
      if (p.flags & MOE_PLAN_EXACT_DW) {
        L.ldk = exact_ldk(p);
        L.cmax = take((2 * H + 3 * E * F) * 4);
        L.offpad = take((E + 1) * 4);
        L.planes = take(2 * (2 * H + 3 * F) * (size_t)L.ldk);
        L.acc_hi = take(3 * E * H * F * 4);
      }
    }
  }
  L.total = cur;
  return L;
}

namespace {

bool plan_ok(const moe_plan_t* p) { return p != nullptr && p->magic == kPlanMagic; }

PlanBuffers plan_buffers(char* ws, const Layout& L, int32_t* offsets, int32_t* perm,
                         int32_t* pos) {
  PlanBuffers b;
  b.rank = (int32_t*)(ws + L.rank);
  b.blk = (int32_t*)(ws + L.blk);
  b.offsets = offsets ? offsets : (int32_t*)(ws + L.offsets);
  b.tiles = (int2*)(ws + L.tiles);
  b.tile_count = (int32_t*)(ws + L.tile_count);
  b.perm = perm ? perm : (int32_t*)(ws + L.perm);
  b.pos = pos ? pos : (int32_t*)(ws + L.pos);
  b.row_gates = L.row_gates ? (float*)(ws + L.row_gates) : nullptr;
  b.nblk = L.nblk;
  b.max_tiles = L.max_tiles;
  b.row_tile = L.row_tile;
  b.small_tiles = L.split ? (int2*)(ws + L.small_tiles) : nullptr;
  b.small_count = L.split ? (int32_t*)(ws + L.small_count) : nullptr;
  b.long_tiles = L.split ? (int2*)(ws + L.long_tiles) : nullptr;
  b.long_count = L.split ? (int32_t*)(ws + L.long_count) : nullptr;
  return b;
}

RowsGeom rows_geom(const PlanBuffers& b, const moe_plan_t& P, int i, int64_t R) {
  RowsGeom g;
  g.tiles = b.tiles + (int64_t)i * b.max_tiles;
  g.tile_count = b.tile_count + i;
  g.offsets = b.offsets + (int64_t)i * (P.E + 1);
  g.grid_m = max_row_tiles(R, P.E, b.row_tile);
  g.row_tile = b.row_tile;
  return g;
}

// Whether a split plan's down projection runs over its two lists: only
// where experts average fewer than two 256-row tiles per chunk (with more,
// segments of at most 128 rows are rare, and the two-list launch measured
// about 2% slower than the one-list kernel on the same tiles).
bool split_down(bool split, int64_t R, const moe_plan_t& P) {
  return split && R < 2 * (int64_t)kRowTileLarge * P.E;
}

// The long segments' list of a split plan (row_tile-row tiles).
RowsGeom long_geom(const PlanBuffers& b, const moe_plan_t& P, int i, int64_t R) {
  RowsGeom g = rows_geom(b, P, i, R);
  g.tiles = b.long_tiles + (int64_t)i * b.max_tiles;
  g.tile_count = b.long_count + i;
  return g;
}

// The short segments' list of a split plan (one kRowTile-row tile each).
RowsGeom small_geom(const PlanBuffers& b, const moe_plan_t& P, int i, int64_t R) {
  RowsGeom g;
  g.tiles = b.small_tiles + (int64_t)i * P.E;
  g.tile_count = b.small_count + i;
  g.offsets = b.offsets + (int64_t)i * (P.E + 1);
  g.grid_m = std::min<int64_t>(R, P.E);
  g.row_tile = kRowTile;
  return g;
}

void fill_stats(moe_stats_t* s, const moe_plan_t& P, int launches, size_t ws, size_t inter,
                int hbufs = 2) {
  if (!s) return;
  std::memset(s, 0, sizeof(*s));
  s->K = P.K;
  s->launches = launches;
  s->c_eff = P.c_eff;
  s->max_pairs_per_chunk = (int64_t)P.k * P.c_eff;  // chunk 0 holds c_eff tokens
  s->dispatch_bytes = hbufs * (int64_t)P.k * P.c_eff * P.H * elem_bytes(P.dtype);
  s->dispatch_bound_bytes = P.dispatch_bound_bytes;
  s->intermediate_bytes = (int64_t)inter;
  s->workspace_bytes = (int64_t)ws;
}

}  // namespace
}  // namespace moe

using namespace moe;

#define MOE_CHECK(call)                        \
  do {                                         \
    if ((call) != hipSuccess) return MOE_EHIP; \
    ++launches;                                \
  } while (0)

MOE_API const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument";
    case MOE_EUNSUPPORTED: return "unsupported shape or dtype";
    case MOE_EWORKSPACE: return "workspace too small";
    case MOE_EHIP: return "HIP runtime error at enqueue";
    default: return "unknown status";
  }
}

MOE_API int moe_plan_chunks(int64_t N, int32_t H, int32_t F, int32_t E, int32_t k, int32_t c,
                            int32_t K_max, int32_t dtype, moe_plan_t* out) {
  if (!out || N < 0 || c < 1 || K_max < 1 || k < 1 || H < 1 || F < 1 || E < 1 || k > E)
    return MOE_EINVAL;
  if (dtype != MOE_F32 && dtype != MOE_BF16) return MOE_EINVAL;
  const int epc = dtype == MOE_BF16 ? 8 : 4;
  if (H % 64 || F % 64 || E % epc || E > 1024 || k > 64) return MOE_EUNSUPPORTED;
  if (N * (int64_t)k >= ((int64_t)1 << 31)) return MOE_EUNSUPPORTED;
  moe_plan_t p;
  std::memset(&p, 0, sizeof(p));
  p.magic = kPlanMagic;
  p.dtype = dtype;
  p.N = N;
  p.H = H;
  p.F = F;
  p.E = E;
  p.k = k;
  p.c = c;
  p.K_max = K_max;
  if (N > 0) {
    const int64_t K = std::min<int64_t>(ceil_div(N, c), K_max);  // eq. (1)
    if (K > 65535) return MOE_EUNSUPPORTED;
    p.K = (int32_t)K;
    p.c_eff = ceil_div(N, K);  // eq. (1)
  }
  p.max_pairs_per_chunk = (int64_t)k * p.c_eff;
  p.dispatch_bound_bytes = 2 * (int64_t)k * p.c_eff * H * elem_bytes(dtype);
  p.fwd_workspace_bytes = (int64_t)make_layout(p, Pass::Forward, true, false).total;
  p.bwd_workspace_bytes = (int64_t)make_layout(p, Pass::Backward, false, true).total;
  p.debug_workspace_bytes = (int64_t)make_layout(p, Pass::Debug, false, false).total;
  *out = p;
  return MOE_OK;
}

namespace moe {

int check_forward_args(const moe_plan_t* plan, const void* X, const void* W_r,
                       const void* W_gate, const void* W_up, const void* W_down, const void* Y,
                       const int32_t* topk_idx, const float* gates) {
  if (!plan_ok(plan)) return MOE_EINVAL;
  if (plan->N == 0) return MOE_OK;
  if (!X || !W_r || !W_gate || !W_up || !W_down || !Y || !topk_idx || !gates) return MOE_EINVAL;
  return MOE_OK;
}

int forward_impl(const moe_plan_t& P, const void* X, const void* W_r, const float* router_bias,
                 const void* W_gate, const void* W_up, const void* W_down, void* Y,
                 int32_t* topk_idx, float* gates, float* logits, void* workspace,
                 hipStream_t st, moe_stats_t* stats) {
  if (P.N == 0) {
    fill_stats(stats, P, 0, 0, 0);
    return MOE_OK;
  }
  const Layout L = make_layout(P, Pass::Forward, logits == nullptr, false);
  char* ws = (char*)workspace;
  float* lg = logits ? logits : (float*)(ws + L.logits);
  int launches = 0;
  (void)hipGetLastError();

  const int rs = router_splits(P);
  float* rparts = rs > 1 ? (float*)(ws + L.rparts) : nullptr;
  MOE_CHECK(gemm_router(P.dtype, X, W_r, router_bias, lg, P.N, P.H, P.E, st, rparts, rs));
  MOE_CHECK(launch_topk(lg, P.N, P.E, P.k, topk_idx, gates, st, rparts, rs, router_bias));
  const PlanBuffers pb = plan_buffers(ws, L, nullptr, nullptr, nullptr);
  if (launch_plan(topk_idx, P.N, P.K, P.k, P.E, pb, st, gates, &launches) != hipSuccess)
    return MOE_EHIP;
  const bool fused = fused_gather(P);
  void* xp = ws + L.xp;
  void* o = ws + L.o;
  void* h = ws + L.h;
  for (int i = 0; i < P.K; ++i) {
    const ChunkGeom g = chunk_geom(P.N, P.K, P.k, i);
    const int64_t R = (int64_t)P.k * g.n;
    RowsGeom rg = rows_geom(pb, P, i, R);
    rg.kt_rows = h_kt_rows(P);
    const int32_t* perm_i = pb.perm + g.pair_base;
    // a split plan runs the gate/up product over its two split lists (the
    // short segments' 128-row tiles and the rest) as one launch
    const bool split = pb.small_tiles != nullptr;
    RowsGeom rgl = split ? long_geom(pb, P, i, R) : rg;
    RowsGeom rgs = split ? small_geom(pb, P, i, R) : rg;
    rgl.kt_rows = rgs.kt_rows = rg.kt_rows;
    const RowsGeom* gs = split ? &rgs : nullptr;
    if (fused) {
      MOE_CHECK(gemm_up_swiglu(P.dtype, rgl, X, W_gate, W_up, h, nullptr, nullptr, P.H, P.F, st,
                               perm_i, P.k, P.N, gs));
    } else {
      MOE_CHECK(launch_gather(P.dtype, X, xp, topk_idx, pb.pos, P.E, P.K, i, g.n, P.k, P.H, st));
      MOE_CHECK(gemm_up_swiglu(P.dtype, rgl, xp, W_gate, W_up, h, nullptr, nullptr, P.H, P.F, st,
                               nullptr, 1, 0, gs));
    }
    // the gates scale the expert rows in the down projection's epilogue; the
    // combine then sums each token's k rows
    MOE_CHECK(gemm_down(P.dtype, rg, h, W_down, o, P.H, P.F, st, pb.row_gates + g.pair_base,
                        split_down(split, R, P) ? &rgl : nullptr, gs));
    MOE_CHECK(launch_combine(P.dtype, o, pb.pos, Y, P.N, P.K, i, g.n, P.k, P.H, st));
  }
  fill_stats(stats, P, launches, L.total,
             (size_t)P.k * P.c_eff * P.F * elem_bytes(P.dtype), fused ? 1 : 2);
  return MOE_OK;
}

}  // namespace moe

MOE_API int moe_plan_set_flags(moe_plan_t* plan, int32_t flags) {
  if (!plan_ok(plan) || (flags & ~MOE_PLAN_EXACT_DW)) return MOE_EINVAL;
  if ((flags & MOE_PLAN_EXACT_DW) && !exact_dw_ok(*plan)) return MOE_EUNSUPPORTED;
  plan->flags = flags;
  plan->bwd_workspace_bytes = (int64_t)make_layout(*plan, Pass::Backward, false, true).total;
  return MOE_OK;
}

MOE_API int moe_bounded_forward(const moe_plan_t* plan, const void* X, const void* W_r,
                                const float* router_bias, const void* W_gate, const void* W_up,
                                const void* W_down, void* Y, int32_t* topk_idx, float* gates,
                                float* logits, void* workspace, size_t workspace_bytes,
                                void* stream, moe_stats_t* stats) {
  if (int s = check_forward_args(plan, X, W_r, W_gate, W_up, W_down, Y, topk_idx, gates))
    return s;
  const moe_plan_t& P = *plan;
  if (P.N > 0) {
    if (!workspace) return MOE_EINVAL;
    if ((uintptr_t)workspace % 256) return MOE_EINVAL;
    if (workspace_bytes < (size_t)P.fwd_workspace_bytes) return MOE_EWORKSPACE;
  }
  return forward_impl(P, X, W_r, router_bias, W_gate, W_up, W_down, Y, topk_idx, gates, logits,
                      workspace, (hipStream_t)stream, stats);
}

namespace moe {
namespace {

// Everything one backward call's kernels read and write, resolved once.
struct BwdCall {
  const moe_plan_t* P;
  Layout L;
  PlanBuffers pb;
  hipStream_t st;
  const void *X, *W_r, *W_gate, *W_up, *W_down, *dY;
  const int32_t* topk_idx;
  const float* gates;
  void* dX;
  float *dW_gate, *dW_up, *dW_down, *dlogits, *dg, *dW_r;
  void *wrt, *xp, *o, *h, *a, *u;
  float *dh, *dgp;
  bool fused;         // bf16: permuted rows of X and dY read through perm
  bool fused_swiglu;  // bf16: SwiGLU backward in the dh GEMM's epilogue
  bool fused_rdh;     // bf16, 256-row tiles: recompute inside the dh kernel
  bool wg_init;       // bf16: chunk 0 stores dW instead of accumulating
  bool exact;         // MOE_PLAN_EXACT_DW: order-invariant weight gradients
  uint32_t *xmax, *dymax, *amax, *umax, *hmax;  // exact: column maxima
  int32_t* offpad;
  int8_t* plane[10];  // exact: hi/lo digit planes of X, dY, da, du, g h
  int32_t* acc_hi[3]; // exact: high words of the dW_gate, dW_up, dW_down accumulators
};

// Backward stages that only the order-invariant weight gradients run (after
// the public enum moe_bwd_stage's).
enum {
  kBStageExactZero = 100,  // zero the column maxima
  kBStageColmaxXY,         // column maxima of X and dY over the batch
  kBStageColmaxRows,       // per chunk: column maxima of da, du, g h per expert
  kBStageFinalize          // accumulators to fp32 dW
};

BwdCall bwd_call(const moe_plan_t& P, const void* X, const void* W_r, const void* W_gate,
                 const void* W_up, const void* W_down, const void* dY, const int32_t* topk_idx,
                 const float* gates, void* dX, float* dW_gate, float* dW_up, float* dW_down,
                 float* dlogits, float* dgates, float* dW_r, void* workspace, hipStream_t st) {
  BwdCall c;
  c.P = &P;
  c.L = make_layout(P, Pass::Backward, false, dgates == nullptr);
  char* ws = (char*)workspace;
  c.pb = plan_buffers(ws, c.L, nullptr, nullptr, nullptr);
  c.st = st;
  c.X = X; c.W_r = W_r; c.W_gate = W_gate; c.W_up = W_up; c.W_down = W_down; c.dY = dY;
  c.topk_idx = topk_idx; c.gates = gates; c.dX = dX;
  c.dW_gate = dW_gate; c.dW_up = dW_up; c.dW_down = dW_down; c.dlogits = dlogits;
  c.dg = dgates ? dgates : (float*)(ws + c.L.dgates);
  c.dW_r = dW_r;
  c.wrt = ws + c.L.wrt;
  c.xp = ws + c.L.xp;
  c.o = ws + c.L.o;  // dXp (fp32 and the gathering path: the dY rows first)
  c.h = ws + c.L.h;  // h, then g h
  c.a = ws + c.L.a;  // a, then da
  c.u = ws + c.L.u;  // u, then du
  c.dh = (float*)(ws + c.L.dh);
  c.dgp = (float*)(ws + c.L.dgp);
  c.fused_swiglu = P.dtype == MOE_BF16;
  c.fused_rdh = fused_recompute_dh(P);
  c.fused = fused_gather_bwd(P);
  c.wg_init = P.dtype == MOE_BF16 && P.N > 0;
  c.exact = (P.flags & MOE_PLAN_EXACT_DW) != 0;
  if (c.exact) {
    const int64_t H = P.H, F = P.F, E = P.E, ldk = c.L.ldk;
    uint32_t* cm = (uint32_t*)(ws + c.L.cmax);
    c.xmax = cm;
    c.dymax = cm + H;
    c.amax = cm + 2 * H;
    c.umax = c.amax + E * F;
    c.hmax = c.umax + E * F;
    c.offpad = (int32_t*)(ws + c.L.offpad);
    int8_t* pl = (int8_t*)(ws + c.L.planes);
    const int64_t cols[5] = {H, H, F, F, F};
    for (int z = 0; z < 5; ++z) {
      c.plane[2 * z] = pl;
      c.plane[2 * z + 1] = pl + cols[z] * ldk;
      pl += 2 * cols[z] * ldk;
    }
    int32_t* ah = (int32_t*)(ws + c.L.acc_hi);
    for (int w = 0; w < 3; ++w) c.acc_hi[w] = ah + (int64_t)w * E * H * F;
  }
  return c;
}

// Runs backward stage `stage` (enum moe_bwd_stage); the per-chunk stages act
// on chunk i.  Adds the kernels it enqueues to *launches.
hipError_t bwd_stage(const BwdCall& c, int stage, int i, int* launches) {
  const moe_plan_t& P = *c.P;
  const hipStream_t st = c.st;
  hipError_t err = hipSuccess;
  auto run = [&](hipError_t e) {
    if (err == hipSuccess) {
      err = e;
      if (e == hipSuccess) ++*launches;
    }
  };
  if (stage == MOE_BSTAGE_ZERO) {
    // bf16: chunk 0's weight-gradient products store dW (zeros for experts
    // without rows) and later chunks accumulate; fp32 accumulates from zero
    const size_t wbytes = (size_t)P.E * P.H * P.F * sizeof(float);
    if (!c.wg_init) {
      run(launch_fill_zero(c.dW_gate, wbytes, st));
      run(launch_fill_zero(c.dW_up, wbytes, st));
      run(launch_fill_zero(c.dW_down, wbytes, st));
    }
    if (c.dW_r) run(launch_fill_zero(c.dW_r, (size_t)P.H * P.E * sizeof(float), st));
    return err;
  }
  if (stage == MOE_BSTAGE_TRANSPOSE) {
    run(launch_transpose(P.dtype, c.W_r, c.wrt, P.H, P.E, st));
    return err;
  }
  if (stage == kBStageExactZero) {
    run(launch_fill_zero(c.xmax, (2 * (size_t)P.H + 3 * (size_t)P.E * P.F) * 4, st));
    return err;
  }
  if (stage == kBStageColmaxXY) {
    run(launch_colmax(c.X, P.N, P.H, c.xmax, st));
    run(launch_colmax(c.dY, P.N, P.H, c.dymax, st));
    return err;
  }
  if (stage == kBStageFinalize) {
    // dW_gate, dW_up: A = X (per column h), B = da, du (per expert and f);
    // dW_down: A = g h (per expert and f), B = dY (per column h)
    run(launch_exact_finalize(c.dW_gate, c.acc_hi[0], c.xmax, false, c.amax, true, P.E, P.H,
                              P.F, st));
    run(launch_exact_finalize(c.dW_up, c.acc_hi[1], c.xmax, false, c.umax, true, P.E, P.H, P.F,
                              st));
    run(launch_exact_finalize(c.dW_down, c.acc_hi[2], c.hmax, true, c.dymax, false, P.E, P.F,
                              P.H, st));
    return err;
  }
  if (stage == MOE_BSTAGE_PLAN) return launch_plan(c.topk_idx, P.N, P.K, P.k, P.E, c.pb, st, nullptr, launches);

  const ChunkGeom g = chunk_geom(P.N, P.K, P.k, i);
  const int64_t R = (int64_t)P.k * g.n;
  const RowsGeom rg = rows_geom(c.pb, P, i, R);
  const int32_t* perm_i = c.pb.perm + g.pair_base;
  const bool first = c.wg_init && i == 0;
  if (c.exact && (stage == MOE_BSTAGE_WGRAD_DOWN || stage == MOE_BSTAGE_WGRAD_GATE_UP)) {
    // order-invariant weight gradients: WGRAD_DOWN writes the chunk's digit
    // planes and runs the down product, WGRAD_GATE_UP the other two
    const int64_t ldk = c.L.ldk;
    uint32_t* lo_g = reinterpret_cast<uint32_t*>(c.dW_gate);
    uint32_t* lo_u = reinterpret_cast<uint32_t*>(c.dW_up);
    uint32_t* lo_d = reinterpret_cast<uint32_t*>(c.dW_down);
    const bool init = i == 0;
    if (stage == MOE_BSTAGE_WGRAD_DOWN) {
      ExactChunk x;
      x.X = DigitPlanesSrc{c.X, P.H, P.H, perm_i, P.k, c.xmax, 0, c.plane[0], c.plane[1]};
      x.dY = DigitPlanesSrc{c.dY, P.H, P.H, perm_i, P.k, c.dymax, 0, c.plane[2], c.plane[3]};
      x.da = DigitPlanesSrc{c.a, P.F, P.F, nullptr, 1, c.amax, 1, c.plane[4], c.plane[5]};
      x.du = DigitPlanesSrc{c.u, P.F, P.F, nullptr, 1, c.umax, 1, c.plane[6], c.plane[7]};
      x.hg = DigitPlanesSrc{c.h, P.F, P.F, nullptr, 1, c.hmax, 1, c.plane[8], c.plane[9]};
      x.offsets = rg.offsets;
      x.offpad = c.offpad;
      x.E = P.E;
      x.ldk = ldk;
      if (launch_digitize(x, st, launches) != hipSuccess) return hipErrorLaunchFailure;
      run(launch_exact_wgrad(c.plane[8], c.plane[9], c.plane[2], c.plane[3], ldk, rg.offsets,
                             c.offpad, lo_d, c.acc_hi[2], P.E, P.F, P.H, init, st));
    } else {
      run(launch_exact_wgrad(c.plane[0], c.plane[1], c.plane[4], c.plane[5], ldk, rg.offsets,
                             c.offpad, lo_g, c.acc_hi[0], P.E, P.H, P.F, init, st));
      run(launch_exact_wgrad(c.plane[0], c.plane[1], c.plane[6], c.plane[7], ldk, rg.offsets,
                             c.offpad, lo_u, c.acc_hi[1], P.E, P.H, P.F, init, st));
    }
    return err;
  }
  if (stage == kBStageColmaxRows) {
    run(launch_colmax_rows(c.a, c.u, c.h, rg.offsets, P.E, P.F, (int64_t)P.k * P.c_eff, c.amax,
                           c.umax, c.hmax, st));
    return err;
  }
  switch (stage) {
    case MOE_BSTAGE_RECOMPUTE:  // this chunk's expert intermediates a, u, h
      if (c.fused_rdh) {
        // computed inside the dh stage's kernel; only the X rows' gather
        // (when they are not read through perm) happens here
        if (!c.fused)
          run(launch_gather(P.dtype, c.X, c.xp, c.topk_idx, c.pb.pos, P.E, P.K, i, g.n, P.k, P.H,
                            st));
      } else if (c.fused) {
        run(gemm_up_swiglu(P.dtype, rg, c.X, c.W_gate, c.W_up, c.h, c.a, c.u, P.H, P.F, st,
                           perm_i, P.k, P.N));
      } else {
        run(launch_gather(P.dtype, c.X, c.xp, c.topk_idx, c.pb.pos, P.E, P.K, i, g.n, P.k, P.H,
                          st));
        run(gemm_up_swiglu(P.dtype, rg, c.xp, c.W_gate, c.W_up, c.h, c.a, c.u, P.H, P.F, st));
      }
      break;
    case MOE_BSTAGE_DH:  // dh' = dYp W_down^T and the SwiGLU backward
      // (bf16 reads the dY rows through perm; the gathered copy's buffer
      // then only receives dXp)
      if (!c.fused)
        run(launch_gather(P.dtype, c.dY, c.o, c.topk_idx, c.pb.pos, P.E, P.K, i, g.n, P.k, P.H,
                          st));
      if (c.fused_rdh) {
        run(gemm_recompute_dh(rg, c.fused ? c.X : c.xp, c.fused ? c.dY : c.o, c.W_gate, c.W_up,
                              c.W_down, c.a, c.u, c.h, perm_i, c.gates, c.dgp,
                              (int64_t)P.k * P.c_eff, P.N * P.k, P.H, P.F, st, P.k,
                              c.fused ? P.N : 0));
      } else if (c.fused_swiglu) {
        run(gemm_dh_swiglu(rg, c.fused ? c.dY : c.o, c.W_down, c.a, c.u, c.h, perm_i, c.gates,
                           c.dgp, (int64_t)P.k * P.c_eff, P.N * P.k, P.H, P.F, st, P.k,
                           c.fused ? P.N : 0));
      } else {
        run(gemm_dh(P.dtype, rg, c.o, c.W_down, c.dh, P.H, P.F, st));
        run(launch_swiglu_bwd(P.dtype, c.dh, c.a, c.u, c.h, perm_i, c.gates, c.dg, R, P.F,
                              P.N * P.k, st));
      }
      break;
    case MOE_BSTAGE_WGRAD_DOWN:
      run(gemm_wgrad_d(P.dtype, rg.offsets, c.h, c.fused ? c.dY : c.o, c.dW_down, P.E, P.H,
                       P.F, st, first, c.fused ? perm_i : nullptr, P.k, P.N));
      break;
    case MOE_BSTAGE_WGRAD_GATE_UP:
      run(gemm_wgrad_gu(P.dtype, rg.offsets, c.fused ? c.X : c.xp, c.a, c.u, c.dW_gate,
                        c.dW_up, P.E, P.H, P.F, st, first, c.fused ? perm_i : nullptr, P.k,
                        P.N));
      break;
    case MOE_BSTAGE_DX:
      run(gemm_dx(P.dtype, rg, c.a, c.u, c.W_gate, c.W_up, c.o, P.H, P.F, st));
      break;
    case MOE_BSTAGE_COMBINE_BWD:
      run(launch_combine_bwd(P.dtype, c.o, c.wrt, c.topk_idx, c.pb.pos, c.gates, c.dg, c.dX,
                             c.dlogits, P.N, P.K, i, g.n, P.k, P.E, P.H, st,
                             c.fused_swiglu ? c.dgp : nullptr,
                             c.fused_swiglu ? dh_ntiles(rg, P.F) : 0, (int64_t)P.k * P.c_eff));
      break;
    case MOE_BSTAGE_DWR:
      if (c.dW_r)
        run(launch_dwr(P.dtype, c.X, perm_i, rg.offsets, c.dlogits, c.dW_r, P.k, P.E, P.H, P.N,
                       st));
      break;
    default:
      return hipErrorInvalidValue;
  }
  return err;
}

}  // namespace
}  // namespace moe

MOE_API int moe_bounded_backward(const moe_plan_t* plan, const void* X, const void* W_r,
                                 const void* W_gate, const void* W_up, const void* W_down,
                                 const void* dY, const int32_t* topk_idx, const float* gates,
                                 void* dX, float* dW_gate, float* dW_up, float* dW_down,
                                 float* dlogits, float* dgates, float* dW_r, void* workspace,
                                 size_t workspace_bytes, void* stream, moe_stats_t* stats) {
  if (!plan_ok(plan)) return MOE_EINVAL;
  const moe_plan_t& P = *plan;
  if (!dW_gate || !dW_up || !dW_down) return MOE_EINVAL;
  if (P.N > 0 && (!X || !W_r || !W_gate || !W_up || !W_down || !dY || !topk_idx || !gates ||
                  !dX || !dlogits || !workspace))
    return MOE_EINVAL;
  if (P.N > 0 && (uintptr_t)workspace % 256) return MOE_EINVAL;
  if (workspace_bytes < (size_t)P.bwd_workspace_bytes) return MOE_EWORKSPACE;
  int launches = 0;
  (void)hipGetLastError();
  const BwdCall c = bwd_call(P, X, W_r, W_gate, W_up, W_down, dY, topk_idx, gates, dX, dW_gate,
                             dW_up, dW_down, dlogits, dgates, dW_r, workspace,
                             (hipStream_t)stream);
  if (bwd_stage(c, MOE_BSTAGE_ZERO, 0, &launches) != hipSuccess) return MOE_EHIP;
  if (P.N == 0) {
    fill_stats(stats, P, launches, 0, 0);
    return MOE_OK;
  }
  for (int s = MOE_BSTAGE_TRANSPOSE; s <= MOE_BSTAGE_PLAN; ++s)
    if (bwd_stage(c, s, 0, &launches) != hipSuccess) return MOE_EHIP;
  if (c.exact) {
    // first pass: the column maxima that fix every operand's grid (whole
    // batch, so the same for every chunking)
    for (int s : {(int)kBStageExactZero, (int)kBStageColmaxXY})
      if (bwd_stage(c, s, 0, &launches) != hipSuccess) return MOE_EHIP;
    for (int i = 0; i < P.K; ++i)
      for (int s : {(int)MOE_BSTAGE_RECOMPUTE, (int)MOE_BSTAGE_DH, (int)kBStageColmaxRows})
        if (bwd_stage(c, s, i, &launches) != hipSuccess) return MOE_EHIP;
  }
  for (int i = 0; i < P.K; ++i)
    for (int s = MOE_BSTAGE_RECOMPUTE; s <= MOE_BSTAGE_DWR; ++s)
      if (bwd_stage(c, s, i, &launches) != hipSuccess) return MOE_EHIP;
  if (c.exact && bwd_stage(c, kBStageFinalize, 0, &launches) != hipSuccess) return MOE_EHIP;
  fill_stats(stats, P, launches, c.L.total,
             (size_t)P.k * P.c_eff * P.F * (3 * elem_bytes(P.dtype) + (c.fused_swiglu ? 0 : 4)),
             c.fused ? 1 : 2);
  return MOE_OK;
}

MOE_API int moe_debug_stage_bwd(const moe_plan_t* plan, int32_t stage, int32_t chunk,
                                const void* X, const void* W_r, const void* W_gate,
                                const void* W_up, const void* W_down, const void* dY,
                                const int32_t* topk_idx, const float* gates, void* dX,
                                float* dW_gate, float* dW_up, float* dW_down, float* dlogits,
                                float* dgates, float* dW_r, void* workspace,
                                size_t workspace_bytes, void* stream) {
  if (!plan_ok(plan)) return MOE_EINVAL;
  const moe_plan_t& P = *plan;
  if (P.N == 0 || stage < MOE_BSTAGE_ZERO || stage > MOE_BSTAGE_DWR) return MOE_EINVAL;
  if (P.flags & MOE_PLAN_EXACT_DW) return MOE_EUNSUPPORTED;
  if (stage >= MOE_BSTAGE_RECOMPUTE && (chunk < 0 || chunk >= P.K)) return MOE_EINVAL;
  if (!X || !W_r || !W_gate || !W_up || !W_down || !dY || !topk_idx || !gates || !dX ||
      !dW_gate || !dW_up || !dW_down || !dlogits || !workspace)
    return MOE_EINVAL;
  if ((uintptr_t)workspace % 256) return MOE_EINVAL;
  if (workspace_bytes < (size_t)P.bwd_workspace_bytes) return MOE_EWORKSPACE;
  int launches = 0;
  (void)hipGetLastError();
  const BwdCall c = bwd_call(P, X, W_r, W_gate, W_up, W_down, dY, topk_idx, gates, dX, dW_gate,
                             dW_up, dW_down, dlogits, dgates, dW_r, workspace,
                             (hipStream_t)stream);
  return bwd_stage(c, stage, chunk, &launches) == hipSuccess ? MOE_OK : MOE_EHIP;
}

MOE_API int moe_debug_topk(const float* logits, int64_t N, int32_t E, int32_t k,
                           int32_t* topk_idx, float* gates, void* stream) {
  if (N < 0 || k < 1 || E < 1 || k > E) return MOE_EINVAL;
  if (E > 1024 || k > 64) return MOE_EUNSUPPORTED;
  if (N == 0) return MOE_OK;
  if (!logits || !topk_idx || !gates) return MOE_EINVAL;
  (void)hipGetLastError();
  return launch_topk(logits, N, E, k, topk_idx, gates, (hipStream_t)stream) == hipSuccess
             ? MOE_OK
             : MOE_EHIP;
}

MOE_API int moe_debug_plan(const moe_plan_t* plan, const int32_t* topk_idx, int32_t* offsets,
                           int32_t* perm, int32_t* pos, void* workspace, size_t workspace_bytes,
                           void* stream) {
  if (!plan_ok(plan)) return MOE_EINVAL;
  const moe_plan_t& P = *plan;
  if (P.N == 0) return MOE_OK;
  if (!topk_idx || !offsets || !perm || !pos || !workspace) return MOE_EINVAL;
  if ((uintptr_t)workspace % 256) return MOE_EINVAL;
  if (workspace_bytes < (size_t)P.debug_workspace_bytes) return MOE_EWORKSPACE;
  const Layout L = make_layout(P, Pass::Debug, false, false);
  (void)hipGetLastError();
  const PlanBuffers pb = plan_buffers((char*)workspace, L, offsets, perm, pos);
  return launch_plan(topk_idx, P.N, P.K, P.k, P.E, pb, (hipStream_t)stream) == hipSuccess
             ? MOE_OK
             : MOE_EHIP;
}

MOE_API int moe_debug_stage(const moe_plan_t* plan, int32_t stage, int32_t chunk, const void* X,
                            const void* W_r, const float* router_bias, const void* W_gate,
                            const void* W_up, const void* W_down, void* Y, int32_t* topk_idx,
                            float* gates, void* workspace, size_t workspace_bytes, void* stream) {
  if (!plan_ok(plan)) return MOE_EINVAL;
  const moe_plan_t& P = *plan;
  if (P.N == 0 || stage < MOE_STAGE_ROUTER || stage > MOE_STAGE_COMBINE) return MOE_EINVAL;
  if (stage >= MOE_STAGE_GATHER && (chunk < 0 || chunk >= P.K)) return MOE_EINVAL;
  if (!X || !W_r || !W_gate || !W_up || !W_down || !Y || !topk_idx || !gates || !workspace)
    return MOE_EINVAL;
  if ((uintptr_t)workspace % 256) return MOE_EINVAL;
  if (workspace_bytes < (size_t)P.fwd_workspace_bytes) return MOE_EWORKSPACE;
  const bool fused = fused_gather(P);
  if (stage == MOE_STAGE_GATHER && fused) return MOE_EUNSUPPORTED;  // no gather kernel
  const Layout L = make_layout(P, Pass::Forward, true, false);
  hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)workspace;
  float* lg = (float*)(ws + L.logits);
  const int rs = router_splits(P);
  float* rparts = rs > 1 ? (float*)(ws + L.rparts) : nullptr;
  const PlanBuffers pb = plan_buffers(ws, L, nullptr, nullptr, nullptr);
  (void)hipGetLastError();
  hipError_t err = hipSuccess;
  if (stage == MOE_STAGE_ROUTER) {
    err = gemm_router(P.dtype, X, W_r, router_bias, lg, P.N, P.H, P.E, st, rparts, rs);
  } else if (stage == MOE_STAGE_TOPK) {
    err = launch_topk(lg, P.N, P.E, P.k, topk_idx, gates, st, rparts, rs, router_bias);
  } else if (stage == MOE_STAGE_PLAN) {
    err = launch_plan(topk_idx, P.N, P.K, P.k, P.E, pb, st, gates);
  } else {
    const ChunkGeom g = chunk_geom(P.N, P.K, P.k, chunk);
    const int64_t R = (int64_t)P.k * g.n;
    RowsGeom rg = rows_geom(pb, P, chunk, R);
    rg.kt_rows = h_kt_rows(P);
    const int32_t* perm_i = pb.perm + g.pair_base;
    void* xp = ws + L.xp;
    void* o = ws + L.o;
    void* h = ws + L.h;
    const bool split = pb.small_tiles != nullptr;  // the lists the forward call uses
    RowsGeom rgl = split ? long_geom(pb, P, chunk, R) : rg;
    RowsGeom rgs = split ? small_geom(pb, P, chunk, R) : rg;
    rgl.kt_rows = rgs.kt_rows = rg.kt_rows;
    const RowsGeom* gs = split ? &rgs : nullptr;
    switch (stage) {
      case MOE_STAGE_GATHER:
        err = launch_gather(P.dtype, X, xp, topk_idx, pb.pos, P.E, P.K, chunk, g.n, P.k, P.H, st);
        break;
      case MOE_STAGE_GEMM_UP:
        err = fused ? gemm_up_swiglu(P.dtype, rgl, X, W_gate, W_up, h, nullptr, nullptr, P.H,
                                     P.F, st, perm_i, P.k, P.N, gs)
                    : gemm_up_swiglu(P.dtype, rgl, xp, W_gate, W_up, h, nullptr, nullptr, P.H,
                                     P.F, st, nullptr, 1, 0, gs);
        break;
      case MOE_STAGE_GEMM_DOWN:
        err = gemm_down(P.dtype, rg, h, W_down, o, P.H, P.F, st, pb.row_gates + g.pair_base,
                        split_down(split, R, P) ? &rgl : nullptr, gs);
        break;
      default:
        err = launch_combine(P.dtype, o, pb.pos, Y, P.N, P.K, chunk, g.n, P.k, P.H, st);
    }
  }
  return err == hipSuccess ? MOE_OK : MOE_EHIP;
}
