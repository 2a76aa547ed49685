/*
 * cce.h -- C ABI of the vocabulary projection with cross-entropy computed
 * over vocabulary strips (part of libmoebound.so), for AMD Instinct MI355X
 * (gfx950).
 *
 * Sources (cited by page title and section):
 *   [BSO]      "Bounded-streaming operators" summary (picx.dev/p/RbUoz4):
 *              Methodology 2 "Ring-DTP": a token batch meets the vocabulary
 *              projection one strip of vocabulary columns at a time; each
 *              strip's partial normaliser is folded into a running per-token
 *              state (running max, normaliser, target logit) and the strip is
 *              released; eq. (2) (logit memory of one strip) and eq. (3)
 *              (the online-softmax recurrence).  On one GPU there is a single
 *              rank and the strips are vocabulary intervals.
 *   [TRILLION] "Training Trillion-Parameter MoE Large Language Models:
 *              End-to-End Optimization Practices", section 3.5 "Large
 *              Vocabulary Loss" (vocabulary-axis chunked cross-entropy, equal
 *              to the unchunked loss; loss and gradients formed per strip).
 *
 * The operator, per token t with hidden row x_t and target index tg_t:
 *   y_t    = x_t W^T                      logits over the vocabulary, fp32
 *   lse_t  = log sum_v exp(y_tv)
 *   loss_t = lse_t - y_{t, tg_t}          (0 for an ignored token)
 * and, for an upstream gradient dloss_t (1/N for a mean over tokens),
 *   dy_tv  = dloss_t (exp(y_tv - lse_t) - [v == tg_t])   (0 if ignored)
 *   dX     = dy W,   dW = dy^T X.
 * The vocabulary is processed in S = ceil(V / v_chunk) strips of v_chunk
 * columns (the last may be short).  The forward pass never stores logits:
 * each GEMM tile folds its logits into per-row partial (max, sum of exp)
 * pairs, and the strip's pairs are folded into the running state by eq. (3)
 * in vocabulary order.  The backward pass recomputes each strip's logits,
 * forms the strip's logit gradient (N x v_chunk bf16, the only strip-sized
 * buffer: plan.strip_bound_bytes) and consumes it in the dX and dW
 * products before the next strip.
 *
 * Every output is bitwise independent of v_chunk: the partial pairs cover
 * fixed 128-column slices of the vocabulary and are folded in one sequence
 * whatever the strip width; dX accumulates strip after strip in one
 * continuous fp32 chain (each strip's product starts from the running sum);
 * dW rows of one vocabulary entry are formed inside one strip.
 *
 * Conventions: as moebound.h (row-major contiguous device tensors, caller-
 * owned memory and workspace, no allocation or synchronisation, work
 * enqueued on `stream`, enum moe_status returns, host-side argument checks
 * before anything is enqueued, finite inputs).
 *   X [N][H] and W [V][H] (one row per vocabulary entry) are bfloat16;
 *   targets [N] int32; loss, lse, dloss [N] fp32; dX [N][H] bfloat16;
 *   dW [V][H] fp32.
 *   A target outside [0, V) marks an ignored token: loss 0, lse still
 *   computed, no gradient from it.
 */
#ifndef CCE_H
#define CCE_H

#include <stddef.h>
#include <stdint.h>

#include "moebound.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Filled by cce_plan; passed unchanged to the other calls. */
typedef struct cce_plan {
    uint32_t magic;               /* set by cce_plan                          */
    int32_t dtype;                /* enum moe_dtype (MOE_BF16)                */
    int64_t N;                    /* tokens                                   */
    int64_t V;                    /* vocabulary entries                       */
    int32_t H;                    /* hidden width                             */
    int32_t v_chunk;              /* strip width                              */
    int32_t S;                    /* strips, ceil(V / v_chunk); 0 if N = 0    */
    int32_t reserved0;
    int64_t strip_bound_bytes;    /* N * min(v_chunk, V) * 2: one logit-
                                     gradient strip (bf16)                   */
    int64_t unchunked_logit_bytes;/* N * V * 4: the fp32 logits of the whole
                                     vocabulary, never formed                */
    int64_t fwd_workspace_bytes;  /* workspace cce_forward needs              */
    int64_t bwd_workspace_bytes;  /* workspace cce_backward needs             */
} cce_plan_t;

/*
 * cce_plan -- strip plan and workspace sizing.  Host only, pure.
 * N = 0 is valid (S = 0; the calls are no-ops, except that cce_backward
 * still zeroes dW).
 * Errors: MOE_EINVAL if out is NULL, N < 0, V < 1, H < 1, v_chunk < 1 or
 *   dtype unknown.  MOE_EUNSUPPORTED if dtype is not MOE_BF16, H is not a
 *   multiple of 128, v_chunk is not a multiple of 256, or N*H, N*v_chunk or
 *   v_chunk*H reach 2^30 (32-bit buffer offsets; W itself may be larger, it
 *   is addressed one strip at a time).
 */
int cce_plan(int64_t N, int32_t H, int64_t V, int32_t v_chunk, int32_t dtype,
             cce_plan_t* out);

/*
 * cce_forward -- per-token loss and log-normaliser.
 * Inputs (device): X [N][H] bf16, W [V][H] bf16, targets [N] int32.
 * Outputs (device, overwritten): loss [N] fp32, lse [N] fp32 (the state
 *   cce_backward needs).
 * workspace: at least plan->fwd_workspace_bytes bytes, 256-byte aligned;
 *   contents on entry do not matter.  It holds one strip's partial (max,
 *   sum of exp) pairs, N * cols / 128 of each, and the running state; cols =
 *   min(v_chunk, V rounded up to a multiple of 256).
 * Errors: MOE_EINVAL (plan not from cce_plan, a required pointer NULL with
 *   N > 0, workspace not 256-byte aligned), MOE_EWORKSPACE (too small),
 *   MOE_EHIP (enqueue failed).  Nothing is enqueued on the first two.
 */
int cce_forward(const cce_plan_t* plan, const void* X, const void* W,
                const int32_t* targets, float* loss, float* lse,
                void* workspace, size_t workspace_bytes, void* stream);

/*
 * cce_backward -- gradients of sum_t dloss_t loss_t.
 * Inputs (device): X, W, targets as in cce_forward; lse [N] fp32 as
 *   returned by cce_forward; dloss [N] fp32.
 * Outputs (device, overwritten): dX [N][H] bf16 (rounded once from the fp32
 *   sum over the vocabulary), dW [V][H] fp32.
 * workspace: at least plan->bwd_workspace_bytes bytes, 256-byte aligned: the
 *   strip's logit gradient (N x cols bf16, cols as in cce_forward) and dX's
 *   fp32 running sum.
 * Errors: as cce_forward, against bwd_workspace_bytes.
 */
int cce_backward(const cce_plan_t* plan, const void* X, const void* W,
                 const int32_t* targets, const float* lse, const float* dloss,
                 void* dX, float* dW, void* workspace, size_t workspace_bytes,
                 void* stream);

/*
 * cce_debug_stage -- re-launch one kernel of one strip, for timing a single
 * kernel with events on `stream`.
 *
 * Precondition: the last call that used `workspace` was cce_forward (stages
 * LOGITS, FOLD) or cce_backward (stages GRAD, DX, DW) with the same plan and
 * arguments; the stage runs exactly the kernel and launch configuration that
 * call uses for strip `strip` (0 <= strip < plan->S), on the same buffers.
 * Outputs are whatever those buffers then hold (DX adds onto dX's running
 * sum again); the next cce_forward / cce_backward call recomputes them.
 * stage: CCE_STAGE_LOGITS (logits GEMM with the slice statistics), FOLD
 *   (eq. (3) over the strip's slices), GRAD (logits GEMM with the logit
 *   gradient), DX (dX running sum += G W_s), DW (dW_s = G^T X).
 * Errors: MOE_EINVAL for a bad plan, stage, strip or NULL pointer;
 *   MOE_EWORKSPACE as the call the stage belongs to.
 */
enum cce_stage {
    CCE_STAGE_LOGITS = 0, CCE_STAGE_FOLD = 1, CCE_STAGE_GRAD = 2, CCE_STAGE_DX = 3,
    CCE_STAGE_DW = 4
};
int cce_debug_stage(const cce_plan_t* plan, int32_t stage, int32_t strip,
                    const void* X, const void* W, const int32_t* targets,
                    float* loss, float* lse, const float* dloss, void* dX, float* dW,
                    void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* CCE_H */
