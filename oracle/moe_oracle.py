"""Plain, slow, fp64 CPU oracle for one GPU's share of a memory-bounded MoE layer.

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use it.  The HIP library never calls
it, and it shares no code, tables or constants with the HIP library.

Pages followed (cited by title and section):

[BSO]     "Bounded-streaming operators" summary (picx.dev/p/RbUoz4):
          "Design Requirements" (exact values and gradients; only the order of
          computation changes), Methodology 1 "PipelinedLLEP" eq. (1) (chunk
          count, effective chunk size, route bound), "Strided chunk
          membership", "Memory bound" (2 E_p k c H b).
[RELAY]   "Memory-Efficient Expert Routing for Distributed MoE Training"
          (RelayMoE summary, paperlayer.ai 2610.07333v1): section 2.1 (each
          token selects its top-k experts; tokens are expanded and permuted,
          outputs returned and recombined), section 1 (dropless, padding-free
          processing of routed token-expert pairs), section 3.3 (hop-local
          recomputation in backward).
[TRILLION] "Training Trillion-Parameter MoE Large Language Models: End-to-End
          Optimization Practices": section 1 (896 routed experts, 16 active),
          section 3.3 (Permute, Grouped GEMM over expert-aggregated batches,
          Unpermute).

The pages define the chunk schedule and require that it leaves values and
gradients unchanged.  This oracle therefore computes the plain *unchunked*
layer; the chunk plan and the per-chunk permutation are separate functions,
checked against their own definitions.

Readings taken where the pages are silent (each is listed with the design
notes of the repository):
  * top-k order: logit descending, ties to the lower expert index; IEEE
    comparison, so -0.0 and +0.0 tie; a NaN logit ranks as -inf;
  * selection is made on the logits, gates are the softmax over all experts
    restricted to the selected ones and renormalised to sum to one;
  * the expert FFN is SwiGLU: (silu(x W_gate) * (x W_up)) W_down, no biases;
  * the slot order of a token's k experts is their rank in the top-k order;
  * the route bound and buffer bound use c_eff (the chunk size eq. (1) yields)
    and E_p = 1 (one GPU owns every expert);
  * within one expert, a chunk's rows are ordered by token position
    (a stable counting sort of the chunk's pairs taken in (token, slot) order);
  * backward treats the selection as constant.

Parity pins: every function here is pinned by ``tests/test_oracle_*.py``
against closed forms, the page's worked instance of eq. (1), brute force on
tiny inputs, library routines (torch fp64 autograd, scipy softmax) and finite
differences.  No function is parity-unpinned.
"""

from __future__ import annotations

from typing import Callable, Optional, Tuple

import numpy as np

f64 = np.float64


# ----------------------------------------------------------------------------
# Chunk plan: [BSO] Methodology 1, eq. (1) and "Strided chunk membership"
# ----------------------------------------------------------------------------

def plan_chunks(N: int, c: int, K_max: int) -> Tuple[int, int]:
    """Eq. (1): K = min(ceil(N / c), K_max) and c_eff = ceil(N / K).

    An empty batch (N == 0) has nothing to split and yields (0, 0)."""
    if N < 0 or c < 1 or K_max < 1:
        raise ValueError("need N >= 0, c >= 1, K_max >= 1")
    if N == 0:
        return 0, 0
    K = min(-(-N // c), K_max)  # exact integer ceilings
    c_eff = -(-N // K)
    return K, c_eff


def chunk_tokens(N: int, K: int, i: int) -> np.ndarray:
    """Chunk i holds token positions i, i+K, i+2K, ... (strided membership)."""
    return np.arange(i, N, K, dtype=np.int64)


def chunk_sizes(N: int, K: int) -> np.ndarray:
    """Number of tokens in each of the K chunks (counted by enumeration)."""
    return np.array([len(chunk_tokens(N, K, i)) for i in range(K)], dtype=np.int64)


def pair_base(N: int, K: int, k: int, i: int) -> int:
    """Index of chunk i's first routed pair when the chunks' pairs are laid
    out one chunk after another: k times the tokens of chunks 0..i-1."""
    return int(k * sum(len(chunk_tokens(N, K, j)) for j in range(i)))


def dispatch_bound_bytes(k: int, c_eff: int, H: int, b: int, E_p: int = 1) -> int:
    """[BSO] "Memory bound": dispatch buffers take at most 2 E_p k c H b bytes
    (read with c = c_eff and E_p = 1)."""
    return 2 * E_p * k * c_eff * H * b


# ----------------------------------------------------------------------------
# Routing: [RELAY] section 2.1 (each token selects its top-k experts)
# ----------------------------------------------------------------------------

def router_logits(X: np.ndarray, Wr: np.ndarray, bias: Optional[np.ndarray] = None) -> np.ndarray:
    """l = X W_r (+ bias), in fp64 on the exact input values."""
    l = np.asarray(X, f64) @ np.asarray(Wr, f64)
    if bias is not None:
        l = l + np.asarray(bias, f64)[None, :]
    return l


def topk_select(logits: np.ndarray, k: int) -> np.ndarray:
    """The k experts with the largest logits, slot s = rank s in the order
    (logit descending, expert index ascending).  A NaN logit is read as -inf
    (so it ties with -inf and the index decides), which keeps the order total
    on any input.  Returns int64 [N, k]."""
    l = np.asarray(logits)
    l = np.where(np.isnan(l), -np.inf, l)
    N, E = l.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    experts = np.broadcast_to(np.arange(E), (N, E))
    # lexsort: last key is primary.  -l sorts descending; -0.0 == +0.0 compare
    # equal, so they tie and the expert index decides.
    order = np.lexsort((experts, -l), axis=-1)
    return order[:, :k].astype(np.int64)


def gates_from_logits(logits: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """Softmax over all E experts (max-subtracted), restricted to the selected
    experts and renormalised to sum to one."""
    l = np.asarray(logits, f64)
    m = l.max(axis=1, keepdims=True)
    p = np.exp(l - m)
    p = p / p.sum(axis=1, keepdims=True)
    ps = np.take_along_axis(p, np.asarray(idx), axis=1)
    return ps / ps.sum(axis=1, keepdims=True)


def route(logits: np.ndarray, k: int) -> Tuple[np.ndarray, np.ndarray]:
    idx = topk_select(logits, k)
    return idx, gates_from_logits(logits, idx)


# ----------------------------------------------------------------------------
# Per-chunk permutation: [TRILLION] section 3.3 (Permute / Unpermute around
# a grouped GEMM over expert-aggregated batches)
# ----------------------------------------------------------------------------

def permute_chunk(idx: np.ndarray, E: int, K: int, i: int):
    """Expert-contiguous layout of chunk i's routed pairs.

    The chunk's pairs, taken in (token ascending, slot ascending) order, are
    stably sorted by expert.  Returns
      offsets [E+1] : exclusive prefix sum of the per-expert pair counts,
      perm_t, perm_s [R_i] : token and slot of each permuted row,
      pos [n_i, k] : permuted row of pair (j-th token of the chunk, slot s).
    """
    idx = np.asarray(idx)
    N, k = idx.shape
    toks = chunk_tokens(N, K, i)
    n = len(toks)
    pair_t = np.repeat(toks, k)
    pair_s = np.tile(np.arange(k, dtype=np.int64), n)
    pair_e = idx[toks].reshape(-1)
    order = np.argsort(pair_e, kind="stable")
    counts = np.bincount(pair_e, minlength=E)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    pos = np.empty(n * k, dtype=np.int64)
    pos[order] = np.arange(n * k, dtype=np.int64)
    return offsets, pair_t[order], pair_s[order], pos.reshape(n, k)


# ----------------------------------------------------------------------------
# Expert FFN (SwiGLU) and the layer
# ----------------------------------------------------------------------------

def silu(z: np.ndarray) -> np.ndarray:
    """silu(z) = z / (1 + e^-z); written so that no intermediate overflows."""
    z = np.asarray(z, f64)
    out = np.empty_like(z)
    pos = z >= 0
    out[pos] = z[pos] / (1.0 + np.exp(-z[pos]))
    ez = np.exp(z[~pos])
    out[~pos] = z[~pos] * ez / (1.0 + ez)
    return out


def sigmoid(z: np.ndarray) -> np.ndarray:
    z = np.asarray(z, f64)
    out = np.empty_like(z)
    pos = z >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-z[pos]))
    ez = np.exp(z[~pos])
    out[~pos] = ez / (1.0 + ez)
    return out


def expert_ffn(x: np.ndarray, Wg: np.ndarray, Wu: np.ndarray, Wd: np.ndarray) -> np.ndarray:
    """FFN_e(x) = (silu(x W_gate) * (x W_up)) W_down for the rows of x."""
    x = np.asarray(x, f64)
    a = x @ np.asarray(Wg, f64)
    u = x @ np.asarray(Wu, f64)
    return (silu(a) * u) @ np.asarray(Wd, f64)


def _experts_accessor(Wg, Wu, Wd) -> Callable[[int], Tuple[np.ndarray, np.ndarray, np.ndarray]]:
    if callable(Wg):
        return Wg
    return lambda e: (np.asarray(Wg[e], f64), np.asarray(Wu[e], f64), np.asarray(Wd[e], f64))


def moe_forward(X, Wr, bias, Wg, Wu, Wd, k: int, idx: Optional[np.ndarray] = None):
    """Unchunked layer: y_t = sum_s g_{t,s} FFN_{S_t[s]}(x_t).

    ``Wg`` may be a callable e -> (W_gate[e], W_up[e], W_down[e]) (then Wu, Wd
    are ignored).  ``idx`` (optional) fixes the selection, e.g. to evaluate the
    expert math under another implementation's routing; the gates are then
    the renormalised softmax of this oracle's fp64 logits at those experts.
    Returns (Y, idx, gates, logits)."""
    X = np.asarray(X, f64)
    logits = router_logits(X, Wr, bias)
    if idx is None:
        idx = topk_select(logits, k)
    idx = np.asarray(idx, np.int64)
    g = gates_from_logits(logits, idx)
    experts = _experts_accessor(Wg, Wu, Wd)
    N, H = X.shape
    E = logits.shape[1]
    Y = np.zeros((N, H), f64)
    for e in range(E):
        rows_t, rows_s = np.nonzero(idx == e)
        if len(rows_t) == 0:
            continue
        wg, wu, wd = experts(e)
        o = expert_ffn(X[rows_t], wg, wu, wd)
        # a token selects an expert at most once, so rows_t has no repeats
        Y[rows_t] += g[rows_t, rows_s][:, None] * o
    return Y, idx, g, logits


def forward_tokens(x_rows, idx_rows, gate_rows, experts: Callable[[int], Tuple]) -> np.ndarray:
    """y for a few tokens, one at a time, given their selection and gates
    (used for sampled checks at sizes where the full oracle is too slow)."""
    x_rows = np.asarray(x_rows, f64)
    out = np.zeros_like(x_rows)
    for r in range(x_rows.shape[0]):
        for s in range(idx_rows.shape[1]):
            wg, wu, wd = experts(int(idx_rows[r, s]))
            out[r] += float(gate_rows[r, s]) * expert_ffn(x_rows[r:r + 1], wg, wu, wd)[0]
    return out


def expert_grads(x, dy, g, wg, wu, wd):
    """Gradients carried by the rows routed to one expert (rows of x, their
    upstream rows dy and gates g), with L = <Y, dY>:
      o = (silu(a) * u) W_d,  a = x W_g,  u = x W_u
      dL/dg      = <dy, o>
      dh         = g dy W_d^T
      da         = dh * u * sigma(a) (1 + a (1 - sigma(a))),   du = dh * silu(a)
      dW_d      += h^T (g dy),  dW_g += x^T da,  dW_u += x^T du
      dx        += da W_g^T + du W_u^T
    Returns (dx_rows, dWg, dWu, dWd, dgate_rows)."""
    x = np.asarray(x, f64)
    dy = np.asarray(dy, f64)
    g = np.asarray(g, f64)[:, None]
    wg, wu, wd = (np.asarray(w, f64) for w in (wg, wu, wd))
    a = x @ wg
    u = x @ wu
    sa = sigmoid(a)
    h = a * sa * u
    o = h @ wd
    dgate = np.sum(dy * o, axis=1)
    dh = g * (dy @ wd.T)
    dWd = h.T @ (g * dy)
    da = dh * u * sa * (1.0 + a * (1.0 - sa))
    du = dh * a * sa
    return da @ wg.T + du @ wu.T, x.T @ da, x.T @ du, dWd, dgate


def router_grads(gates, dgates, idx, E: int) -> np.ndarray:
    """dlogits for gates g_j = exp(l_j) / sum_{S_t} exp(l) (the full softmax's
    normaliser cancels in the renormalisation):
      dl_j = g_j (dg_j - sum_j' g_j' dg_j') on the selected experts, 0 elsewhere."""
    gates = np.asarray(gates, f64)
    dgates = np.asarray(dgates, f64)
    dsel = gates * (dgates - np.sum(gates * dgates, axis=1, keepdims=True))
    dl = np.zeros((gates.shape[0], E), f64)
    np.put_along_axis(dl, np.asarray(idx, np.int64), dsel, axis=1)
    return dl


def moe_backward(X, Wr, Wg, Wu, Wd, dY, idx, gates):
    """Gradients of L = <Y, dY> with the selection held constant: the expert
    part of every routed pair (expert_grads), then the router part
    (router_grads), dx_t += dl_t W_r^T and dW_r = X^T dl.
    Returns dict with dX, dWg, dWu, dWd, dlogits, dgates, dWr."""
    X = np.asarray(X, f64)
    dY = np.asarray(dY, f64)
    Wr = np.asarray(Wr, f64)
    idx = np.asarray(idx, np.int64)
    gates = np.asarray(gates, f64)
    N, H = X.shape
    E = Wr.shape[1]
    k = idx.shape[1]
    experts = _experts_accessor(Wg, Wu, Wd)
    F = experts(0)[0].shape[1]
    dX = np.zeros((N, H), f64)
    dWg = np.zeros((E, H, F), f64)
    dWu = np.zeros((E, H, F), f64)
    dWd = np.zeros((E, F, H), f64)
    dgates = np.zeros((N, k), f64)
    for e in range(E):
        rows_t, rows_s = np.nonzero(idx == e)
        if len(rows_t) == 0:
            continue
        dx, dWg[e], dWu[e], dWd[e], dg = expert_grads(
            X[rows_t], dY[rows_t], gates[rows_t, rows_s], *experts(e))
        dgates[rows_t, rows_s] = dg
        dX[rows_t] += dx
    dlogits = router_grads(gates, dgates, idx, E)
    dX += dlogits @ Wr.T
    dWr = X.T @ dlogits
    return dict(dX=dX, dWg=dWg, dWu=dWu, dWd=dWd, dlogits=dlogits, dgates=dgates, dWr=dWr)


def backward_tokens(x_rows, dy_rows, idx_rows, gate_rows, experts: Callable[[int], Tuple], Wr):
    """dX, dgates and dlogits of a few tokens, one at a time (sampled checks
    at sizes where the full oracle is too slow).  Returns (dX, dgates, dlogits)."""
    x_rows = np.asarray(x_rows, f64)
    dy_rows = np.asarray(dy_rows, f64)
    Wr = np.asarray(Wr, f64)
    n, k = idx_rows.shape
    E = Wr.shape[1]
    dX = np.zeros_like(x_rows)
    dg = np.zeros((n, k), f64)
    for r in range(n):
        for s in range(k):
            dx, _, _, _, d = expert_grads(x_rows[r:r + 1], dy_rows[r:r + 1],
                                          np.asarray(gate_rows[r:r + 1, s]), *experts(int(idx_rows[r, s])))
            dX[r] += dx[0]
            dg[r, s] = d[0]
    dl = router_grads(gate_rows, dg, idx_rows, E)
    dX += dl @ Wr.T
    return dX, dg, dl


# ----------------------------------------------------------------------------
# Rounding bound that decides which routing flips between fp32 and fp64 logits are allowed
# ----------------------------------------------------------------------------

# unit roundoff of binary32 (24-bit significand, round to nearest): 2^-24
FP32_UNIT_ROUNDOFF = 2.0 ** -24


def logit_error_bound(X, Wr, bias=None) -> np.ndarray:
    """Per-token bound tau_t = 2 gamma_H max_e sum_h |x_th w_he| (+ one rounding
    of the bias add), gamma_H = H u / (1 - H u), u = 2^-24: the classical bound
    on the error of an fp32 sum of H exact products, doubled because a flip
    needs two logits to move.  A top-k that differs from the fp64 one is
    acceptable only where the fp64 gap between the k-th and (k+1)-th logit is
    at most tau_t."""
    X = np.asarray(X, f64)
    Wr = np.asarray(Wr, f64)
    H = X.shape[1]
    u = FP32_UNIT_ROUNDOFF
    gam = H * u / (1 - H * u)
    mag = np.abs(X) @ np.abs(Wr)
    l = X @ Wr
    if bias is not None:
        mag = mag + np.abs(np.asarray(bias, f64))[None, :]
        l = l + np.asarray(bias, f64)[None, :]
    per = gam * mag + u * np.abs(l)
    return 2.0 * per.max(axis=1)
