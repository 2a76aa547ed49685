/*
 * moebound.h -- C ABI of the memory-bounded MoE layer library (libmoebound.so)
 *
 * One GPU's share of a Mixture-of-Experts layer executed under a bounded
 * dispatch buffer, for AMD Instinct MI355X (gfx950).
 *
 * Sources (cited by page title and section):
 *   [BSO]      "Bounded-streaming operators" summary (picx.dev/p/RbUoz4):
 *              Design Requirements; Methodology 1 "PipelinedLLEP", eq. (1),
 *              "Nested gradient checkpointing", "Strided chunk membership",
 *              "Memory bound".
 *   [RELAY]    "Memory-Efficient Expert Routing for Distributed MoE Training"
 *              (RelayMoE summary): section 1 (dropless, padding-free pairs),
 *              section 2.1 (expand, permute, recombine), section 3.3
 *              (hop-local recomputation).
 *   [TRILLION] "Training Trillion-Parameter MoE Large Language Models:
 *              End-to-End Optimization Practices": section 1 (896 routed
 *              experts, 16 activated), section 3.3 (Permute, Grouped GEMM,
 *              Unpermute).
 *
 * The layer, per token t with input row x_t:
 *   l_t   = x_t W_r (+ bias)                         router logits, fp32
 *   S_t   = top-k experts of l_t, ordered by (logit descending, index
 *           ascending); slot s holds the s-th of them
 *   g_t   = softmax of l_t restricted to S_t and renormalised (sum 1)
 *   y_t   = sum_{s<k} g_{t,s} FFN_{S_t[s]}(x_t),
 *   FFN_e(x) = (silu(x W_gate[e]) * (x W_up[e])) W_down[e]
 * computed under the chunk schedule of [BSO] eq. (1): K = min(ceil(N/c),
 * K_max) chunks, c_eff = ceil(N/K), chunk i = token positions i, i+K, ...
 * Each chunk's routed pairs are permuted into an expert-contiguous buffer of
 * at most k*c_eff rows, run through the experts and combined back, so the
 * top-k-expanded buffer of the whole batch never exists.  The H-wide
 * dispatch buffers take at most 2*k*c_eff*H*b bytes ([BSO] "Memory bound"
 * with E_p = 1 and c read as c_eff); bf16 needs only half of that, because
 * its forward and backward read each permuted input row straight from X
 * (when X fits 32-bit buffer offsets, and in the backward N*k*k < 2^32).
 * The result does not depend on K: per-token
 * outputs are bitwise identical for every (c, K_max).
 *
 * Conventions for every entry point:
 *   - All matrices are row-major and contiguous.  Expert weights are stacked
 *     on a leading expert dimension: W_gate, W_up [E][H][F], W_down [E][F][H].
 *   - dtype MOE_BF16: X, W_r, W_gate, W_up, W_down, Y, dY, dX are bfloat16;
 *     logits, gates, dgates, dlogits and all weight gradients are fp32.
 *     dtype MOE_F32: every tensor is fp32.
 *   - Device pointers are HIP device addresses on the current device; the
 *     caller owns and allocates all memory, including the workspace.  The
 *     library never allocates, frees or synchronises; work is enqueued on
 *     `stream` (a hipStream_t; NULL is the null stream) and the call returns
 *     once it is enqueued.
 *   - Every call returns a moe_status.  Argument errors are found on the
 *     host before anything is enqueued; then outputs are untouched.
 *   - Inputs must be finite.  NaN or Inf inputs give unspecified (but
 *     memory-safe) values; the routing stays a valid selection (a NaN logit
 *     ranks as -inf, so each token still gets k distinct experts).
 *   - Calls that share a workspace must not overlap in time.
 */
#ifndef MOEBOUND_H
#define MOEBOUND_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum moe_status {
    MOE_OK = 0,
    MOE_EINVAL = 1,        /* invalid argument (range, null pointer, plan) */
    MOE_EUNSUPPORTED = 2,  /* valid, but a shape the kernels do not handle  */
    MOE_EWORKSPACE = 3,    /* workspace smaller than the plan requires      */
    MOE_EHIP = 4           /* the HIP runtime reported an error at enqueue  */
};

enum moe_dtype { MOE_F32 = 0, MOE_BF16 = 1 };

/* Filled by moe_plan_chunks; passed unchanged to the other calls. */
typedef struct moe_plan {
    uint32_t magic;              /* set by moe_plan_chunks                    */
    int32_t dtype;               /* enum moe_dtype                            */
    int64_t N;                   /* tokens                                    */
    int32_t H, F, E, k;          /* hidden, FFN width, experts, top-k         */
    int32_t c, K_max;            /* token budget per chunk, chunk cap         */
    int32_t K;                   /* eq. (1): min(ceil(N/c), K_max); 0 if N=0  */
    int32_t flags;               /* MOE_PLAN_* options (moe_plan_set_flags)   */
    int64_t c_eff;               /* eq. (1): ceil(N/K); 0 if N = 0            */
    int64_t max_pairs_per_chunk; /* k * c_eff (route bound, E_p = 1)          */
    int64_t dispatch_bound_bytes;/* 2 * k * c_eff * H * b                     */
    int64_t fwd_workspace_bytes; /* workspace moe_bounded_forward needs       */
    int64_t bwd_workspace_bytes; /* workspace moe_bounded_backward needs      */
    int64_t debug_workspace_bytes;/* workspace moe_debug_plan needs           */
} moe_plan_t;

/* Host-side accounting of one call (no device read-back). */
typedef struct moe_stats {
    int32_t K;                   /* chunks processed                          */
    int32_t launches;            /* kernels enqueued                          */
    int64_t c_eff;
    int64_t max_pairs_per_chunk; /* largest R_i = k * n_i over the chunks     */
    int64_t dispatch_bytes;      /* H-wide per-chunk dispatch buffers carved:
                                    k*c_eff*H*b each; one in bf16 (expert
                                    outputs, or dXp; the permuted rows of X
                                    and dY read in place), two otherwise      */
    int64_t dispatch_bound_bytes;/* 2 * k * c_eff * H * b                     */
    int64_t intermediate_bytes;  /* F-wide per-chunk intermediates            */
    int64_t workspace_bytes;     /* workspace bytes the call used             */
} moe_stats_t;

/*
 * moe_plan_chunks -- the chunk plan of [BSO] eq. (1) and workspace sizing.
 *
 * Host only, pure; touches no device.  Fills *out:
 *   K = min(ceil(N/c), K_max), c_eff = ceil(N/K); chunk i holds token
 *   positions i, i+K, i+2K, ... ([BSO] "Strided chunk membership"), so it
 *   has n_i = ceil((N-i)/K) tokens and R_i = k*n_i <= k*c_eff routed pairs.
 * N = 0 is valid: K = c_eff = 0 and the layer calls are no-ops (backward
 * still zeroes the weight gradients).
 * Errors: MOE_EINVAL if out is NULL, N < 0, c < 1, K_max < 1, k < 1, k > E,
 *   H, F or E < 1, or dtype unknown.  MOE_EUNSUPPORTED if H or F is not a
 *   multiple of 64, E is not a multiple of 8 (bf16) or 4 (fp32), E > 1024,
 *   k > 64, or N*k >= 2^31.
 */
int moe_plan_chunks(int64_t N, int32_t H, int32_t F, int32_t E, int32_t k,
                    int32_t c, int32_t K_max, int32_t dtype, moe_plan_t* out);

/*
 * moe_plan_set_flags -- options of a plan; moe_plan_chunks leaves them 0.
 *
 * MOE_PLAN_EXACT_DW: order-invariant expert weight gradients.  [BSO]
 *   (Summary, "Core principle"; Design Requirements 1-2) requires the chunked
 *   run to reach exactly the unchunked values and gradients, with only the
 *   order of computation changed.  By default dW_gate, dW_up and dW_down are
 *   fp32 sums taken chunk by chunk, so their last bits depend on K.  With
 *   this flag each operand of those sums -- X and dY per column h, and da, du
 *   and g*h per expert and column f -- is first rounded to a power-of-two
 *   grid fixed by that column's largest magnitude over the whole batch
 *   (15-bit integers, |v| <= 2^14); the products are then summed exactly in
 *   integers and rounded to fp32 once.  dW_gate, dW_up and dW_down are then
 *   bitwise identical for every (c, K_max) of the same batch.  Cost: a first
 *   pass over the chunks that recomputes a, u, h and runs the dh GEMM to find
 *   the column maxima, the int8-digit weight-gradient products with a 64-bit
 *   accumulator per weight element (workspace: 4 bytes per dW element beyond
 *   dW itself, plus per-chunk digit planes), and one conversion pass.  The
 *   other outputs are unchanged.  Needs dtype MOE_BF16, X and dY readable in
 *   place (N*H*2 < 2^31, N*k*k < 2^32), c_eff <= 65536, H and F multiples of
 *   128; else MOE_EUNSUPPORTED.  moe_debug_stage_bwd does not serve such plans.
 * Updates plan->bwd_workspace_bytes.  Errors: MOE_EINVAL for a plan not from
 *   moe_plan_chunks or an unknown flag; MOE_EUNSUPPORTED as above (the plan
 *   is then unchanged).
 */
#define MOE_PLAN_EXACT_DW 1
int moe_plan_set_flags(moe_plan_t* plan, int32_t flags);

/*
 * moe_bounded_forward -- the layer's forward pass under the chunk schedule.
 *
 * Computes, for the whole batch, the router logits and each token's top-k
 * experts and gates ([RELAY] section 2.1: each token selects its top-k
 * experts; expanded rows are permuted, processed and recombined), then runs
 * the [BSO] eq. (1) chunks i = 0..K-1 ("Strided chunk membership") one after
 * the other: chunk i's routed pairs are permuted into expert-contiguous rows,
 * pushed through each expert's SwiGLU FFN as grouped GEMMs and combined back
 * per token, each expert row scaled by its gate ([TRILLION] section 3.3:
 * Permute, Grouped GEMM, Unpermute).  Per-chunk buffers are sized by
 * k*c_eff rows ([BSO] "Memory bound"), so the top-k-expanded buffer of the
 * whole batch never exists.
 *
 * Inputs (device): X [N][H]; W_r [H][E]; router_bias [E] fp32 or NULL;
 *   W_gate, W_up [E][H][F]; W_down [E][F][H].
 * Outputs (device, overwritten): Y [N][H]; topk_idx [N][k] int32 (S_t in
 *   slot order); gates [N][k] fp32; logits [N][E] fp32 or NULL (then they
 *   live in the workspace only).  topk_idx and gates are the state that
 *   moe_bounded_backward needs.
 * workspace: device memory of at least plan->fwd_workspace_bytes bytes,
 *   256-byte aligned; its contents on entry do not matter.  It holds the
 *   whole batch's O(N*k) int32 routing plan and the per-chunk buffers: the
 *   F-wide SwiGLU output and the H-wide expert outputs, k*c_eff rows each,
 *   plus (fp32, or bf16 with N*H*2 >= 2^31) an H-wide permuted-input buffer;
 *   otherwise the gate/up GEMM reads the permuted rows straight from X.
 * stats: optional host struct, filled on success.
 * Errors: MOE_EINVAL (plan not from moe_plan_chunks, a required pointer is
 *   NULL, workspace not 256-byte aligned), MOE_EWORKSPACE (workspace_bytes <
 *   plan->fwd_workspace_bytes), MOE_EHIP (enqueue failed; outputs are then
 *   undefined).  No work is enqueued on the first two.
 */
int moe_bounded_forward(const moe_plan_t* plan,
                        const void* X, const void* W_r, const float* router_bias,
                        const void* W_gate, const void* W_up, const void* W_down,
                        void* Y, int32_t* topk_idx, float* gates, float* logits,
                        void* workspace, size_t workspace_bytes, void* stream,
                        moe_stats_t* stats);

/*
 * moe_bounded_backward -- gradients of L = <Y, dY> with the selection held
 * constant, recomputing each chunk's expert intermediates from X and
 * releasing them before the next chunk ([BSO] "Nested gradient
 * checkpointing"; [RELAY] section 3.3).
 *
 * Inputs (device): X, W_r, W_gate, W_up, W_down as in the forward call; dY
 *   [N][H]; topk_idx [N][k], gates [N][k] as returned by the forward call.
 * Outputs (device, overwritten):
 *   dX [N][H]            includes the router path dlogits W_r^T;
 *   dW_gate, dW_up [E][H][F], dW_down [E][F][H] fp32;
 *   dlogits [N][E] fp32  g_j (dg_j - sum g dg) on the selected experts, 0
 *                        elsewhere;
 *   dgates [N][k] fp32 or NULL   dL/dg_{t,s} = <dY_t, FFN_{S_t[s]}(x_t)>;
 *   dW_r [H][E] fp32 or NULL     X^T dlogits.
 * Per-token outputs (dX, dlogits, dgates) are bitwise independent of K.
 * Weight gradients sum over tokens chunk by chunk, so their last bits
 * depend on K; they are deterministic for a fixed plan.  With
 * MOE_PLAN_EXACT_DW (moe_plan_set_flags) dW_gate, dW_up and dW_down are
 * bitwise independent of K as well.
 * workspace: at least plan->bwd_workspace_bytes bytes, 256-byte aligned.
 * Errors: as moe_bounded_forward, against bwd_workspace_bytes.
 */
int moe_bounded_backward(const moe_plan_t* plan,
                         const void* X, const void* W_r,
                         const void* W_gate, const void* W_up, const void* W_down,
                         const void* dY, const int32_t* topk_idx, const float* gates,
                         void* dX, float* dW_gate, float* dW_up, float* dW_down,
                         float* dlogits, float* dgates, float* dW_r,
                         void* workspace, size_t workspace_bytes, void* stream,
                         moe_stats_t* stats);

/*
 * moe_bounded_forward_static -- moe_bounded_forward without a workspace
 * argument, for callers that cannot allocate device memory (code under
 * stream capture, tight serving loops, harnesses that forbid allocation).
 *
 * Same inputs, outputs and results as moe_bounded_forward (bitwise: the
 * same kernels run), but the per-call buffers live in a scratch array of
 * MOE_STATIC_SCRATCH_BYTES bytes that the library holds on each GPU it runs
 * on until the process ends.  The call allocates and frees nothing.
 * Limit: the plan's forward layout must fit the array -- it is
 * plan->fwd_workspace_bytes when logits is NULL (about N*E*4 bytes less when
 * the caller passes logits); otherwise MOE_EWORKSPACE and nothing is
 * enqueued.  Every call on one GPU shares that GPU's array: calls that
 * overlap in time on one GPU (on different streams, or from different
 * threads) race and give undefined results; calls in stream order are safe.
 * The array keeps the last call's contents; the forward pass needs none of
 * it cleared.
 * Errors: as moe_bounded_forward; MOE_EWORKSPACE as above; MOE_EHIP also
 *   when the runtime cannot give the array's device address.
 */
#define MOE_STATIC_SCRATCH_BYTES (64u << 20)
int moe_bounded_forward_static(const moe_plan_t* plan,
                               const void* X, const void* W_r, const float* router_bias,
                               const void* W_gate, const void* W_up, const void* W_down,
                               void* Y, int32_t* topk_idx, float* gates, float* logits,
                               void* stream, moe_stats_t* stats);

/* Static description of a status code; never NULL. */
const char* moe_status_string(int status);

/*
 * moe_debug_topk -- the router top-k and gate stage alone, for stage-level
 * checks: each token's top-k experts and renormalised gates ([RELAY]
 * section 2.1, top-k selection; up to the "896 routed experts, 16 activated"
 * shape of [TRILLION] section 1 and beyond, E <= 1024, k <= 64).
 * logits [N][E] fp32 in; topk_idx [N][k] int32 and gates [N][k] fp32 out,
 * as the forward call computes them.  Errors: MOE_EINVAL for
 * N < 0, k < 1, k > E or a NULL pointer with N > 0; MOE_EUNSUPPORTED for
 * E > 1024 or k > 64.
 */
int moe_debug_topk(const float* logits, int64_t N, int32_t E, int32_t k,
                   int32_t* topk_idx, float* gates, void* stream);

/*
 * moe_debug_plan -- the per-chunk expert-contiguous permutation for every
 * chunk of the plan ([TRILLION] section 3.3 "Permute"), from a given
 * topk_idx [N][k] (entries in [0, E), distinct within a row).
 * Outputs (device):
 *   offsets [K][E+1] int32  chunk i's rows of expert e are
 *                           offsets[i][e] .. offsets[i][e+1]-1;
 *   perm [N*k] int32        chunk i's rows start at pair index
 *                           k*(tokens of chunks 0..i-1); row r of chunk i
 *                           holds pair t*k+s;
 *   pos [N*k] int32         pos[t*k+s] = the row of pair (t, s) within its
 *                           chunk.
 * Within an expert, rows are in ascending token order.
 * workspace: at least plan->debug_workspace_bytes bytes.
 */
int moe_debug_plan(const moe_plan_t* plan, const int32_t* topk_idx,
                   int32_t* offsets, int32_t* perm, int32_t* pos,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * moe_debug_stage -- re-launch one stage of the forward pass for one chunk,
 * for timing a single kernel with events on `stream`.
 *
 * Precondition: the last call that used `workspace` was moe_bounded_forward
 * with the same plan, inputs and outputs and logits == NULL; the workspace
 * still holds that call's routing plan.  The stage runs exactly the kernel
 * and launch configuration the forward call uses for chunk `chunk`
 * (0 <= chunk < plan->K), reading and writing the same buffers.  Running
 * GATHER, GEMM_UP, GEMM_DOWN and COMBINE for chunks 0..K-1 in that order
 * reproduces the forward call's outputs bitwise; a stage run out of that
 * order computes on whatever the per-chunk buffers hold.  When the plan's
 * forward reads the permuted inputs in place (see moe_bounded_forward's
 * workspace), it has no gather kernel: GATHER then returns MOE_EUNSUPPORTED
 * and enqueues nothing.
 * stage: MOE_STAGE_ROUTER (router logits, whole batch), MOE_STAGE_TOPK (top-k
 *   and gates, whole batch), MOE_STAGE_PLAN (planner, whole batch),
 *   MOE_STAGE_GATHER, MOE_STAGE_GEMM_UP (gate/up GEMM + SwiGLU),
 *   MOE_STAGE_GEMM_DOWN, MOE_STAGE_COMBINE (per chunk).
 * Errors: MOE_EINVAL for a bad plan, stage, chunk or NULL pointer;
 *   MOE_EUNSUPPORTED for GATHER when the forward has no gather kernel;
 *   MOE_EWORKSPACE as moe_bounded_forward.
 */
enum moe_stage {
    MOE_STAGE_ROUTER = 0, MOE_STAGE_TOPK = 1, MOE_STAGE_PLAN = 2, MOE_STAGE_GATHER = 3,
    MOE_STAGE_GEMM_UP = 4, MOE_STAGE_GEMM_DOWN = 5, MOE_STAGE_COMBINE = 6
};
int moe_debug_stage(const moe_plan_t* plan, int32_t stage, int32_t chunk,
                    const void* X, const void* W_r, const float* router_bias,
                    const void* W_gate, const void* W_up, const void* W_down,
                    void* Y, int32_t* topk_idx, float* gates,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * moe_debug_stage_bwd -- re-launch one stage of the backward pass (for one
 * chunk, for the per-chunk stages), for timing its kernels with events on
 * `stream`.  The stages are the backward call's steps with per-chunk
 * recompute ([BSO] "Nested gradient checkpointing"; [RELAY] section 3.3):
 *   MOE_BSTAGE_ZERO         zero dW_r (and, fp32, the expert dW) -- whole call;
 *   MOE_BSTAGE_TRANSPOSE    W_r^T for the router path of dX -- whole call;
 *   MOE_BSTAGE_PLAN         the per-chunk permutations -- whole call;
 *   MOE_BSTAGE_RECOMPUTE    a = Xp W_gate, u = Xp W_up, h = silu(a) u;
 *   MOE_BSTAGE_DH           dh' = dYp W_down^T with the SwiGLU backward
 *                           (da, du, g h and the chunk's dgate shares);
 *   MOE_BSTAGE_WGRAD_DOWN   dW_down += (g h)^T dYp;
 *   MOE_BSTAGE_WGRAD_GATE_UP dW_gate += Xp^T da, dW_up += Xp^T du;
 *   MOE_BSTAGE_DX           dXp = da W_gate^T + du W_up^T;
 *   MOE_BSTAGE_COMBINE_BWD  dX rows (slot order), dgates, dlogits;
 *   MOE_BSTAGE_DWR          dW_r += X^T dlogits over the chunk's tokens
 *                           (nothing when dW_r is NULL).
 * (fp32 plans, and bf16 plans whose X or dY cannot be read in place, also
 * run the gather of X rows in RECOMPUTE and of dY rows in DH.  bf16 plans
 * whose chunks take the 256-row GEMM tiles -- experts averaging at least 96
 * rows per chunk, H and F multiples of 128 -- compute a, u and h inside the
 * DH stage's kernel, which keeps them on chip: their RECOMPUTE stage only
 * gathers, if anything.)  The dgate shares are per 128 columns of F (64 when
 * F is not a multiple of 128) and summed in one order whatever the tiles.
 * Precondition: the last call that used `workspace` was moe_bounded_backward
 * with the same plan and arguments (dgates and dW_r NULL or not as there).
 * Running ZERO, TRANSPOSE, PLAN and then RECOMPUTE .. DWR for chunks
 * 0..K-1 reproduces that call's outputs bitwise; a stage run out of that
 * order computes on whatever the buffers hold.
 * Errors: MOE_EINVAL for a bad plan, stage, chunk (0 <= chunk < plan->K for
 *   the per-chunk stages), N = 0 or a NULL required pointer; MOE_EWORKSPACE
 *   as moe_bounded_backward; MOE_EHIP if an enqueue failed.
 */
enum moe_bwd_stage {
    MOE_BSTAGE_ZERO = 0, MOE_BSTAGE_TRANSPOSE = 1, MOE_BSTAGE_PLAN = 2,
    MOE_BSTAGE_RECOMPUTE = 3, MOE_BSTAGE_DH = 4, MOE_BSTAGE_WGRAD_DOWN = 5,
    MOE_BSTAGE_WGRAD_GATE_UP = 6, MOE_BSTAGE_DX = 7, MOE_BSTAGE_COMBINE_BWD = 8,
    MOE_BSTAGE_DWR = 9
};
int moe_debug_stage_bwd(const moe_plan_t* plan, int32_t stage, int32_t chunk,
                        const void* X, const void* W_r,
                        const void* W_gate, const void* W_up, const void* W_down,
                        const void* dY, const int32_t* topk_idx, const float* gates,
                        void* dX, float* dW_gate, float* dW_up, float* dW_down,
                        float* dlogits, float* dgates, float* dW_r,
                        void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOEBOUND_H */
