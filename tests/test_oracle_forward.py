"""Pins for the oracle's forward pass: brute-force dense evaluation, closed
forms, special cases and chunked == unchunked."""

import math

import numpy as np
import pytest
import torch

import oracle


def dense_bruteforce(X, Wr, bias, Wg, Wu, Wd, k):
    """Pure-Python loops, every expert evaluated for every token, with a dense
    gate vector that is zero off the top-k set."""
    N, H = len(X), len(X[0])
    E, F = len(Wg), len(Wg[0][0])
    Y = [[0.0] * H for _ in range(N)]
    for t in range(N):
        l = [sum(X[t][h] * Wr[h][e] for h in range(H)) + (bias[e] if bias is not None else 0.0)
             for e in range(E)]
        sel = sorted(range(E), key=lambda e: (-l[e], e))[:k]
        z = sum(math.exp(l[e] - l[sel[0]]) for e in sel)
        G = [math.exp(l[e] - l[sel[0]]) / z if e in sel else 0.0 for e in range(E)]
        for e in range(E):
            a = [sum(X[t][h] * Wg[e][h][f] for h in range(H)) for f in range(F)]
            u = [sum(X[t][h] * Wu[e][h][f] for h in range(H)) for f in range(F)]
            hh = [a[f] / (1 + math.exp(-a[f])) * u[f] for f in range(F)]
            for o in range(H):
                Y[t][o] += G[e] * sum(hh[f] * Wd[e][f][o] for f in range(F))
    return np.array(Y)


def tiny_problem(seed, N=7, H=4, E=5, F=6, bias=True):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((N, H))
    Wr = rng.standard_normal((H, E))
    b = rng.standard_normal(E) if bias else None
    Wg = rng.standard_normal((E, H, F)) * 0.7
    Wu = rng.standard_normal((E, H, F)) * 0.7
    Wd = rng.standard_normal((E, F, H)) * 0.7
    return X, Wr, b, Wg, Wu, Wd


@pytest.mark.parametrize("seed,k", [(0, 1), (1, 2), (2, 3), (3, 5)])
def test_dense_bruteforce(seed, k):
    X, Wr, b, Wg, Wu, Wd = tiny_problem(seed)
    Y, idx, g, l = oracle.moe_forward(X, Wr, b, Wg, Wu, Wd, k)
    Yb = dense_bruteforce(X.tolist(), Wr.tolist(), None if b is None else b.tolist(),
                          Wg.tolist(), Wu.tolist(), Wd.tolist(), k)
    np.testing.assert_allclose(Y, Yb, rtol=1e-12, atol=1e-12)


def test_scalar_closed_form():
    # E = k = 1, H = F = 1: y = silu(x wg) (x wu) wd
    X = np.array([[2.0]])
    Y, idx, g, _ = oracle.moe_forward(X, np.array([[1.0]]), None, np.array([[[0.5]]]),
                                      np.array([[[3.0]]]), np.array([[[-1.0]]]), 1)
    assert idx.tolist() == [[0]] and g.tolist() == [[1.0]]
    expect = -(1.0 / (1.0 + math.exp(-1.0))) * 6.0
    assert abs(Y[0, 0] - expect) < 1e-15


def test_single_expert_is_textbook_swiglu():
    rng = np.random.default_rng(3)
    X = rng.standard_normal((9, 16))
    Wg, Wu, Wd = (rng.standard_normal((1, 16, 24)), rng.standard_normal((1, 16, 24)),
                  rng.standard_normal((1, 24, 16)))
    Y, _, _, _ = oracle.moe_forward(X, rng.standard_normal((16, 1)), None, Wg, Wu, Wd, 1)
    x = torch.from_numpy(X)
    ref = (torch.nn.functional.silu(x @ torch.from_numpy(Wg[0])) * (x @ torch.from_numpy(Wu[0]))) \
        @ torch.from_numpy(Wd[0])
    np.testing.assert_allclose(Y, ref.numpy(), rtol=1e-12, atol=1e-12)


def test_special_cases():
    X, Wr, b, Wg, Wu, Wd = tiny_problem(4, bias=False)
    # identical experts: the gates sum to one, so y = FFN(x)
    Wg2, Wu2, Wd2 = (np.repeat(W[:1], 5, 0) for W in (Wg, Wu, Wd))
    Y, _, _, _ = oracle.moe_forward(X, Wr, None, Wg2, Wu2, Wd2, 3)
    np.testing.assert_allclose(Y, oracle.expert_ffn(X, Wg[0], Wu[0], Wd[0]), rtol=1e-12, atol=1e-13)
    # X = 0 and no bias: all logits tie, the first k experts are chosen, Y = 0
    Y, idx, g, _ = oracle.moe_forward(np.zeros_like(X), Wr, None, Wg, Wu, Wd, 3)
    assert np.all(Y == 0) and idx.tolist() == [[0, 1, 2]] * len(X)
    np.testing.assert_allclose(g, 1 / 3, rtol=1e-15)
    # W_down = 0: Y = 0
    Y, _, _, _ = oracle.moe_forward(X, Wr, None, Wg, Wu, np.zeros_like(Wd), 2)
    assert np.all(Y == 0)


def test_forward_tokens_matches_layer():
    X, Wr, b, Wg, Wu, Wd = tiny_problem(5)
    Y, idx, g, _ = oracle.moe_forward(X, Wr, b, Wg, Wu, Wd, 2)
    experts = lambda e: (Wg[e], Wu[e], Wd[e])
    Yt = oracle.forward_tokens(X[[1, 4]], idx[[1, 4]], g[[1, 4]], experts)
    np.testing.assert_allclose(Yt, Y[[1, 4]], rtol=1e-13)


@pytest.mark.parametrize("N,c,K_max,k", [(37, 8, 4, 2), (37, 100, 4, 3), (50, 3, 7, 5)])
def test_chunked_schedule_reaches_unchunked_result(N, c, K_max, k):
    """The chunk schedule (plan, strided chunks, permute, per-expert FFN,
    gate-weighted combine) reaches the unchunked layer's result."""
    X, Wr, b, Wg, Wu, Wd = tiny_problem(6, N=N)
    Y, idx, g, _ = oracle.moe_forward(X, Wr, b, Wg, Wu, Wd, k)
    K, _ = oracle.plan_chunks(N, c, K_max)
    Yc = np.zeros_like(Y)
    for i in range(K):
        off, pt, ps, pos = oracle.permute_chunk(idx, 5, K, i)
        O = np.zeros((len(pt), X.shape[1]))
        for e in range(5):
            r0, r1 = off[e], off[e + 1]
            if r1 > r0:
                O[r0:r1] = oracle.expert_ffn(X[pt[r0:r1]], Wg[e], Wu[e], Wd[e])
        for j, t in enumerate(oracle.chunk_tokens(N, K, i)):
            for s in range(k):
                Yc[t] += g[t, s] * O[pos[j, s]]
    np.testing.assert_allclose(Yc, Y, rtol=1e-12, atol=1e-14)
