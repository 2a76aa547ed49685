"""Pins for the oracle's backward pass: torch fp64 autograd of an independent
dense formulation, central finite differences, and the router-gradient
invariants."""

import numpy as np
import pytest
import torch

import oracle


def problem(seed, N=11, H=6, E=5, F=7, k=3):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((N, H))
    Wr = rng.standard_normal((H, E))
    Wg = rng.standard_normal((E, H, F)) * 0.6
    Wu = rng.standard_normal((E, H, F)) * 0.6
    Wd = rng.standard_normal((E, F, H)) * 0.6
    dY = rng.standard_normal((N, H))
    return X, Wr, Wg, Wu, Wd, dY, k


def torch_dense_grads(X, Wr, Wg, Wu, Wd, dY, idx):
    """Dense formulation in torch fp64: every expert for every token, a dense
    gate matrix built with a mask, autograd for the gradients."""
    t = lambda a: torch.tensor(a, dtype=torch.float64, requires_grad=True)
    x, wr, wg, wu, wd = t(X), t(Wr), t(Wg), t(Wu), t(Wd)
    logits = x @ wr
    logits.retain_grad()
    N, E = logits.shape
    mask = torch.zeros(N, E, dtype=torch.float64)
    mask.scatter_(1, torch.from_numpy(idx), 1.0)
    p = torch.softmax(logits, dim=1) * mask
    G = p / p.sum(1, keepdim=True)
    y = torch.zeros_like(x)
    for e in range(E):
        h = torch.nn.functional.silu(x @ wg[e]) * (x @ wu[e])
        y = y + G[:, e:e + 1] * (h @ wd[e])
    (y * torch.from_numpy(dY)).sum().backward()
    return dict(dX=x.grad.numpy(), dWr=wr.grad.numpy(), dWg=wg.grad.numpy(),
                dWu=wu.grad.numpy(), dWd=wd.grad.numpy(), dlogits=logits.grad.numpy())


@pytest.mark.parametrize("seed,k", [(0, 1), (1, 2), (2, 3), (3, 5)])
def test_against_torch_autograd(seed, k):
    X, Wr, Wg, Wu, Wd, dY, _ = problem(seed, k=k)
    _, idx, g, _ = oracle.moe_forward(X, Wr, None, Wg, Wu, Wd, k)
    got = oracle.moe_backward(X, Wr, Wg, Wu, Wd, dY, idx, g)
    ref = torch_dense_grads(X, Wr, Wg, Wu, Wd, dY, idx)
    for name in ("dX", "dWr", "dWg", "dWu", "dWd", "dlogits"):
        np.testing.assert_allclose(got[name], ref[name], rtol=1e-10, atol=1e-12, err_msg=name)


def loss(X, Wr, Wg, Wu, Wd, dY, idx, k):
    Y, _, _, _ = oracle.moe_forward(X, Wr, None, Wg, Wu, Wd, k, idx=idx)
    return float(np.sum(Y * dY))


def test_central_finite_differences():
    X, Wr, Wg, Wu, Wd, dY, k = problem(11)
    _, idx, g, l = oracle.moe_forward(X, Wr, None, Wg, Wu, Wd, k)
    grads = oracle.moe_backward(X, Wr, Wg, Wu, Wd, dY, idx, g)
    eps = 1e-6
    rng = np.random.default_rng(0)
    arrays = dict(X=X, Wr=Wr, Wg=Wg, Wu=Wu, Wd=Wd)
    gname = dict(X="dX", Wr="dWr", Wg="dWg", Wu="dWu", Wd="dWd")
    for name, A in arrays.items():
        for _ in range(6):
            pos = tuple(int(rng.integers(0, s)) for s in A.shape)
            keep = A[pos]
            A[pos] = keep + eps
            lp = loss(X, Wr, Wg, Wu, Wd, dY, idx, k)
            A[pos] = keep - eps
            lm = loss(X, Wr, Wg, Wu, Wd, dY, idx, k)
            A[pos] = keep
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - grads[gname[name]][pos]) <= 1e-6 * max(1.0, abs(fd)), (name, pos)


def test_dgates_match_finite_differences_of_the_gates():
    """dL/dg_s = <dY_t, FFN_{S_t[s]}(x_t)>: perturb one gate directly."""
    X, Wr, Wg, Wu, Wd, dY, k = problem(12)
    _, idx, g, _ = oracle.moe_forward(X, Wr, None, Wg, Wu, Wd, k)
    grads = oracle.moe_backward(X, Wr, Wg, Wu, Wd, dY, idx, g)
    t, s = 4, 1
    o = oracle.expert_ffn(X[t:t + 1], Wg[idx[t, s]], Wu[idx[t, s]], Wd[idx[t, s]])[0]
    assert abs(grads["dgates"][t, s] - float(o @ dY[t])) < 1e-12


def test_router_gradient_invariants():
    X, Wr, Wg, Wu, Wd, dY, k = problem(13, N=40, E=9, k=4)
    _, idx, g, _ = oracle.moe_forward(X, Wr, None, Wg, Wu, Wd, k)
    d = oracle.moe_backward(X, Wr, Wg, Wu, Wd, dY, idx, g)
    off = np.ones_like(d["dlogits"], dtype=bool)
    np.put_along_axis(off, idx, False, axis=1)
    assert np.all(d["dlogits"][off] == 0.0)
    np.testing.assert_allclose(d["dlogits"].sum(1), 0.0, atol=1e-12)
    # k = 1: the single gate is constant 1, so no gradient reaches the router
    _, idx1, g1, _ = oracle.moe_forward(X, Wr, None, Wg, Wu, Wd, 1)
    d1 = oracle.moe_backward(X, Wr, Wg, Wu, Wd, dY, idx1, g1)
    assert np.all(d1["dlogits"] == 0.0) and np.all(d1["dWr"] == 0.0)


def test_backward_tokens_and_expert_grads_match_layer():
    X, Wr, Wg, Wu, Wd, dY, k = problem(14, N=20, E=6, k=3)
    _, idx, g, _ = oracle.moe_forward(X, Wr, None, Wg, Wu, Wd, k)
    d = oracle.moe_backward(X, Wr, Wg, Wu, Wd, dY, idx, g)
    rows = [0, 7, 19]
    experts = lambda e: (Wg[e], Wu[e], Wd[e])
    dx, dg, dl = oracle.backward_tokens(X[rows], dY[rows], idx[rows], g[rows], experts, Wr)
    np.testing.assert_allclose(dx, d["dX"][rows], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dg, d["dgates"][rows], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dl, d["dlogits"][rows], rtol=1e-12, atol=1e-13)
    e = int(idx[7, 1])
    rt, rs = np.nonzero(idx == e)
    _, dWg, dWu, dWd, _ = oracle.expert_grads(X[rt], dY[rt], g[rt, rs], *experts(e))
    np.testing.assert_allclose(dWg, d["dWg"][e], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dWd, d["dWd"][e], rtol=1e-12, atol=1e-13)
