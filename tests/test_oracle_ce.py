"""Pins for the vocabulary-strip cross-entropy oracle: closed forms, brute
force with exactly rounded sums, torch's fp64 cross-entropy and autograd,
central finite differences, and the strip recurrence against the plain
definition."""

import math

import numpy as np
import pytest
import torch

import oracle

IGNORE = -100


def problem(seed, N=9, H=5, V=13, ignore=(2,)):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((N, H))
    W = rng.standard_normal((V, H)) * 0.7
    t = rng.integers(0, V, N)
    for i in ignore:
        t[i] = IGNORE
    dloss = rng.standard_normal(N)
    return X, W, t, dloss


def brute_loss(X, W, t):
    """-log softmax by explicit loops, sums rounded once (math.fsum)."""
    N, V = X.shape[0], W.shape[0]
    out = []
    for i in range(N):
        y = [math.fsum(X[i, h] * W[v, h] for h in range(X.shape[1])) for v in range(V)]
        if not 0 <= t[i] < V:
            out.append(0.0)
            continue
        m = max(y)
        lse = m + math.log(math.fsum(math.exp(a - m) for a in y))
        out.append(lse - y[t[i]])
    return np.array(out)


def test_strips_cover_vocabulary_once():
    for V in (1, 7, 64, 1000, 1001):
        for c in (1, 3, 64, 999, 5000):
            s = oracle.ce_strips(V, c)
            assert s[0][0] == 0 and s[-1][1] == V
            assert all(a[1] == b[0] for a, b in zip(s, s[1:]))
            assert all(0 < v1 - v0 <= c for v0, v1 in s)
            assert len(s) == -(-V // c)
    with pytest.raises(ValueError):
        oracle.ce_strips(0, 4)


def test_strip_bound_bytes():
    assert oracle.strip_bound_bytes(8192, 8192, 200_000, 2) == 8192 * 8192 * 2
    assert oracle.strip_bound_bytes(10, 64, 40, 4) == 10 * 40 * 4


def test_uniform_logits_closed_form():
    # W = 0: every logit is 0, so lse = log V and the loss is log V
    X, _, t, dloss = problem(0)
    V = 13
    W = np.zeros((V, X.shape[1]))
    loss, lse = oracle.ce_forward(X, W, t)
    assert np.allclose(lse, math.log(V), rtol=0, atol=1e-15)
    ok = t >= 0
    assert np.allclose(loss[ok], math.log(V), rtol=0, atol=1e-15)
    assert np.all(loss[~ok] == 0)
    g = oracle.ce_dlogits(X, W, t, lse, dloss)
    want = np.tile(1.0 / V, (len(t), V))
    want[np.arange(len(t))[ok], t[ok]] -= 1.0
    want *= dloss[:, None]
    want[~ok] = 0
    assert np.allclose(g, want, rtol=0, atol=1e-15)


def test_two_classes_closed_form():
    # V = 2: loss = log(1 + exp(y_other - y_target)) (softplus of the margin)
    rng = np.random.default_rng(1)
    X = rng.standard_normal((6, 3))
    W = rng.standard_normal((2, 3))
    t = np.array([0, 1, 1, 0, 1, 0])
    loss, _ = oracle.ce_forward(X, W, t)
    y = X @ W.T
    margin = y[np.arange(6), 1 - t] - y[np.arange(6), t]
    assert np.allclose(loss, np.log1p(np.exp(margin)), rtol=1e-14, atol=0)


def test_large_equal_logits_do_not_overflow():
    # every logit 1000: lse = 1000 + log V exactly, loss = log V
    X = np.full((2, 1), 10.0)
    W = np.full((4, 1), 100.0)
    loss, lse = oracle.ce_forward(X, W, np.array([3, 0]))
    assert np.allclose(lse, 1000.0 + math.log(4), rtol=1e-15)
    assert np.allclose(loss, math.log(4), rtol=1e-12)
    l2, s2, *_ = oracle.ce_fold_strips(X, W, np.array([3, 0]), 3)
    assert np.allclose(s2, 1000.0 + math.log(4), rtol=1e-15)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_forward_brute_force(seed):
    X, W, t, _ = problem(seed)
    loss, _ = oracle.ce_forward(X, W, t)
    assert np.allclose(loss, brute_loss(X, W, t), rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("seed", [3, 4])
def test_forward_and_grads_vs_torch(seed):
    X, W, t, dloss = problem(seed, N=17, H=8, V=29, ignore=(0, 5))
    x = torch.tensor(X, requires_grad=True)
    w = torch.tensor(W, requires_grad=True)
    tt = torch.tensor(t)
    ref = torch.nn.functional.cross_entropy(x @ w.T, tt, reduction="none", ignore_index=IGNORE)
    (ref * torch.tensor(dloss)).sum().backward()
    loss, lse = oracle.ce_forward(X, W, t)
    assert np.allclose(loss, ref.detach().numpy(), rtol=1e-13, atol=1e-14)
    assert np.allclose(lse, torch.logsumexp(x @ w.T, dim=1).detach().numpy(), rtol=1e-14)
    dX, dW = oracle.ce_backward(X, W, t, lse, dloss)
    assert np.allclose(dX, x.grad.numpy(), rtol=1e-12, atol=1e-14)
    assert np.allclose(dW, w.grad.numpy(), rtol=1e-12, atol=1e-14)


def test_grads_finite_differences():
    X, W, t, dloss = problem(5, N=5, H=4, V=7, ignore=(1,))
    f = lambda X_, W_: float(np.dot(oracle.ce_forward(X_, W_, t)[0], dloss))
    _, lse = oracle.ce_forward(X, W, t)
    dX, dW = oracle.ce_backward(X, W, t, lse, dloss)
    eps = 1e-6
    for A, G in ((X, dX), (W, dW)):
        num = np.zeros_like(A)
        for idx in np.ndindex(*A.shape):
            old = A[idx]
            A[idx] = old + eps
            up = f(X, W)
            A[idx] = old - eps
            dn = f(X, W)
            A[idx] = old
            num[idx] = (up - dn) / (2 * eps)
        assert np.allclose(G, num, rtol=1e-6, atol=1e-8)


def test_dlogits_rows_sum_to_zero_and_ignored_rows_vanish():
    X, W, t, dloss = problem(6, N=12, H=6, V=31, ignore=(3, 7))
    _, lse = oracle.ce_forward(X, W, t)
    g = oracle.ce_dlogits(X, W, t, lse, dloss)
    assert np.allclose(g.sum(axis=1), 0.0, atol=1e-14)
    assert np.all(g[[3, 7]] == 0)
    # softmax rows: g / dloss + onehot is a probability vector
    ok = t >= 0
    p = g[ok] / dloss[ok, None]
    p[np.arange(ok.sum()), t[ok]] += 1.0
    assert np.all(p > 0) and np.allclose(p.sum(axis=1), 1.0, atol=1e-14)


@pytest.mark.parametrize("v_chunk", [1, 4, 13, 50, 1000])
def test_fold_strips_equals_definition(v_chunk):
    # eq. (3) strip by strip gives the plain loss (up to rounding order)
    X, W, t, _ = problem(7, N=10, H=6, V=50, ignore=(4,))
    W = W * 3.0  # spread the logits so the running max moves between strips
    loss, lse = oracle.ce_forward(X, W, t)
    l2, s2, m, z, yt = oracle.ce_fold_strips(X, W, t, v_chunk)
    assert np.allclose(s2, lse, rtol=1e-14, atol=1e-14)
    assert np.allclose(l2, loss, rtol=1e-12, atol=1e-13)
    y = X @ W.T
    # (the strips' products round like the whole product up to BLAS blocking)
    assert np.allclose(m, y.max(axis=1), rtol=1e-14, atol=0)
    assert np.allclose(z, np.exp(y - m[:, None]).sum(axis=1), rtol=1e-13)
    ok = t >= 0
    assert np.allclose(yt[ok], y[np.arange(len(t))[ok], t[ok]], rtol=1e-14, atol=1e-15)


def test_token_subsets_match_whole_batch():
    X, W, t, dloss = problem(8, N=14, H=5, V=23, ignore=(2,))
    loss, lse = oracle.ce_forward(X, W, t)
    rows = np.array([1, 2, 9, 13])
    d_sparse = np.zeros_like(dloss)
    d_sparse[rows] = dloss[rows]
    dX_all, dW_all = oracle.ce_backward(X, W, t, lse, d_sparse)
    dXr, dWr, lser = oracle.ce_backward_tokens(X[rows], W, t[rows], dloss[rows])
    assert np.allclose(lser, lse[rows], rtol=1e-15)
    assert np.allclose(dXr, dX_all[rows], rtol=1e-13, atol=1e-15)
    assert np.allclose(dWr, dW_all, rtol=1e-13, atol=1e-15)
    lr, _ = oracle.ce_forward_tokens(X[rows], W, t[rows])
    assert np.allclose(lr, loss[rows], rtol=1e-15)


def test_vocab_row_subset_matches_full_weight_gradient():
    X, W, t, dloss = problem(9, N=8, H=5, V=37, ignore=(6,))
    rows = np.array([0, 5, 36, int(t[0]), int(t[3])])
    dXf, dWf, lsef = oracle.ce_backward_tokens(X, W, t, dloss)
    dXr, dWr, lser = oracle.ce_backward_tokens_rows(X, W, t, dloss, rows)
    assert np.array_equal(lser, lsef) and np.array_equal(dXr, dXf)
    assert np.allclose(dWr, dWf[rows], rtol=1e-13, atol=1e-15)
