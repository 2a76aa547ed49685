"""Plain, slow, fp64 CPU oracle for the vocabulary projection with cross-entropy,
computed over vocabulary strips (test infrastructure only).

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use it.  The HIP library never calls
it, and it shares no code, tables or constants with the HIP library.

Pages followed (cited by title and section):

[BSO]      "Bounded-streaming operators" summary (picx.dev/p/RbUoz4):
           Methodology 2 "Ring-DTP" -- a batch meets the vocabulary projection
           one strip of columns at a time, each strip's partial normaliser is
           folded into a running per-token state (running max, normaliser,
           target logit) and the strip is released; eq. (2) (logit memory of
           one strip) and eq. (3) (the online-softmax recurrence).  With one
           GPU there is one rank, and the strips are vocabulary intervals.
[TRILLION] "Training Trillion-Parameter MoE Large Language Models: End-to-End
           Optimization Practices", section 3.5 "Large Vocabulary Loss":
           vocabulary-axis chunked cross-entropy, numerically equivalent to
           the unchunked loss, with loss and gradients formed strip by strip.

The method reaches the unchunked cross-entropy exactly (up to rounding
order), so ``ce_forward`` / ``ce_backward`` are that plain definition; the
strip recurrence is a separate function (``ce_fold_strips``), checked against
the definition.

Readings taken where the pages are silent or garbled:
  * W is stored vocabulary-major, [V, H] (one row per vocabulary entry);
    logits are X W^T;
  * the statistics are per token: eq. (3) keeps one running max and
    normaliser per token and rescales the normaliser when the max grows (the
    extracted two-pass sketch of [TRILLION] 3.5 keeps a single max and adds
    unscaled sums, which does not give a softmax; eq. (3) is taken);
  * a target outside [0, V) marks an ignored token: loss 0, no gradient;
  * the loss is returned per token; a mean over tokens is the caller's
    upstream gradient dloss = 1/N;
  * gradients: dlogits[t, v] = dloss[t] (softmax(logits_t)[v] - [v == target_t]),
    dX = dlogits W, dW = dlogits^T X.

Parity pins: ``tests/test_oracle_ce.py`` checks every function against closed
forms (uniform logits, two classes, huge equal logits), brute force with
exactly rounded sums on tiny inputs, torch's fp64 cross-entropy and its
autograd (library routines), central finite differences and the zero-sum of
each token's logit gradient.  No function is parity-unpinned.
"""

from __future__ import annotations

from typing import List, Tuple

import numpy as np

f64 = np.float64


def ce_strips(V: int, v_chunk: int) -> List[Tuple[int, int]]:
    """Vocabulary strips [v0, v1) of width v_chunk (the last may be short), in
    vocabulary order ([BSO] Methodology 2: each strip is met once; [TRILLION]
    3.5: vocabulary chunks)."""
    if V < 1 or v_chunk < 1:
        raise ValueError("V and v_chunk must be positive")
    return [(v0, min(v0 + v_chunk, V)) for v0 in range(0, V, v_chunk)]


def strip_bound_bytes(N: int, v_chunk: int, V: int, b: int) -> int:
    """Bytes of one logit (or logit-gradient) strip, N x min(v_chunk, V) values
    of b bytes: the per-strip logit memory of [BSO] eq. (2) with the vocabulary
    interval of one strip in place of V / P."""
    return N * min(v_chunk, V) * b


def ce_logits(X: np.ndarray, W: np.ndarray) -> np.ndarray:
    """logits = X W^T, fp64 ([BSO] Methodology 2: the strip Y = X W_r)."""
    return np.asarray(X, f64) @ np.asarray(W, f64).T


def _valid(targets: np.ndarray, V: int) -> np.ndarray:
    t = np.asarray(targets, np.int64)
    return (t >= 0) & (t < V)


def ce_forward(X: np.ndarray, W: np.ndarray, targets: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Plain cross-entropy: lse_t = log sum_v exp(y_tv) (with the row max
    subtracted first), loss_t = lse_t - y_{t, target_t}; ignored tokens have
    loss 0.  Returns (loss [N], lse [N])."""
    y = ce_logits(X, W)
    V = y.shape[1]
    m = y.max(axis=1)
    lse = m + np.log(np.exp(y - m[:, None]).sum(axis=1))
    ok = _valid(targets, V)
    t = np.where(ok, np.asarray(targets, np.int64), 0)
    loss = np.where(ok, lse - y[np.arange(y.shape[0]), t], 0.0)
    return loss, lse


def ce_fold_strips(X: np.ndarray, W: np.ndarray, targets: np.ndarray, v_chunk: int):
    """The strip schedule of [BSO] Methodology 2 with eq. (3): for each strip
    in vocabulary order form only that strip's logits, fold them into the
    running per-token state (m, z, y_target) with
        m' = max(m, max_v y_v),   z' = exp(m - m') z + sum_v exp(y_v - m'),
    take the target logit when the target falls in the strip, and drop the
    strip.  Returns (loss, lse, m, z, y_target)."""
    X = np.asarray(X, f64)
    W = np.asarray(W, f64)
    N, V = X.shape[0], W.shape[0]
    m = np.full(N, -np.inf)
    z = np.zeros(N)
    yt = np.zeros(N)
    tg = np.asarray(targets, np.int64)
    for v0, v1 in ce_strips(V, v_chunk):
        y = X @ W[v0:v1].T                      # the strip, N x (v1 - v0)
        m_new = np.maximum(m, y.max(axis=1))
        scale = np.where(np.isfinite(m), np.exp(m - m_new), 0.0)
        z = scale * z + np.exp(y - m_new[:, None]).sum(axis=1)
        m = m_new
        inside = (tg >= v0) & (tg < v1)
        rows = np.nonzero(inside)[0]
        yt[rows] = y[rows, tg[rows] - v0]
    lse = m + np.log(z)
    loss = np.where(_valid(tg, V), lse - yt, 0.0)
    return loss, lse, m, z, yt


def ce_dlogits(X: np.ndarray, W: np.ndarray, targets: np.ndarray, lse: np.ndarray,
               dloss: np.ndarray) -> np.ndarray:
    """dlogits[t, v] = dloss_t (exp(y_tv - lse_t) - [v == target_t]); rows of
    ignored tokens are zero."""
    y = ce_logits(X, W)
    N, V = y.shape
    g = np.exp(y - np.asarray(lse, f64)[:, None])
    ok = _valid(targets, V)
    t = np.asarray(targets, np.int64)
    rows = np.nonzero(ok)[0]
    g[rows, t[rows]] -= 1.0
    g *= np.asarray(dloss, f64)[:, None]
    g[~ok] = 0.0
    return g


def ce_backward(X: np.ndarray, W: np.ndarray, targets: np.ndarray, lse: np.ndarray,
                dloss: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Gradients of sum_t dloss_t loss_t: dX = dlogits W [N, H],
    dW = dlogits^T X [V, H]."""
    g = ce_dlogits(X, W, targets, lse, dloss)
    return g @ np.asarray(W, f64), g.T @ np.asarray(X, f64)


def ce_forward_tokens(X_rows: np.ndarray, W: np.ndarray, targets_rows: np.ndarray):
    """ce_forward for a subset of tokens (each token's loss depends on its own
    row only): used for sampled checks of large batches."""
    return ce_forward(X_rows, W, targets_rows)


def ce_backward_tokens(X_rows: np.ndarray, W: np.ndarray, targets_rows: np.ndarray,
                       dloss_rows: np.ndarray) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """dX rows and the dW contribution of a subset of tokens.  When dloss is
    zero for every other token this dW is the whole weight gradient.
    Returns (dX_rows, dW, lse_rows)."""
    _, lse = ce_forward(X_rows, W, targets_rows)
    dX, dW = ce_backward(X_rows, W, targets_rows, lse, dloss_rows)
    return dX, dW, lse


def ce_backward_tokens_rows(X_rows: np.ndarray, W: np.ndarray, targets_rows: np.ndarray,
                            dloss_rows: np.ndarray, vocab_rows: np.ndarray):
    """As ce_backward_tokens, but the weight gradient only for the vocabulary
    entries vocab_rows: dW[v] = sum_t dlogits[t, v] x_t, where dlogits[t, v] =
    dloss_t (exp(y_tv - lse_t) - [v == target_t]) and lse_t runs over the whole
    vocabulary.  Returns (dX_rows, dW[vocab_rows], lse_rows)."""
    _, lse = ce_forward(X_rows, W, targets_rows)
    Xf = np.asarray(X_rows, f64)
    dX = ce_dlogits(X_rows, W, targets_rows, lse, dloss_rows) @ np.asarray(W, f64)
    vr = np.asarray(vocab_rows, np.int64)
    y = Xf @ np.asarray(W, f64)[vr].T                 # logits of the chosen entries
    g = np.exp(y - lse[:, None])
    tg = np.asarray(targets_rows, np.int64)
    g -= (tg[:, None] == vr[None, :])
    g *= np.asarray(dloss_rows, f64)[:, None]
    g[~_valid(tg, W.shape[0])] = 0.0
    return dX, g.T @ Xf, lse
