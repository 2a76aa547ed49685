"""Pins for the oracle's routing: top-k selection order and renormalised gates."""

import numpy as np
import pytest
import scipy.special

import oracle


def brute_topk_row(l, k):
    return sorted(range(len(l)), key=lambda e: (-float(l[e]), e))[:k]


def test_topk_brute_force_with_ties():
    rng = np.random.default_rng(5)
    for _ in range(200):
        N, E = rng.integers(1, 6), rng.integers(1, 12)
        k = int(rng.integers(1, E + 1))
        l = rng.integers(-3, 3, size=(N, E)).astype(np.float64)  # many ties
        idx = oracle.topk_select(l, k)
        for t in range(N):
            assert list(idx[t]) == brute_topk_row(l[t], k)


def test_topk_defining_property():
    rng = np.random.default_rng(6)
    l = rng.standard_normal((50, 17))
    l[:, 3] = l[:, 9]  # exact ties between two experts
    k = 5
    idx = oracle.topk_select(l, k)
    for t in range(l.shape[0]):
        sel = list(idx[t])
        rest = [e for e in range(17) if e not in sel]
        for e in sel:
            for f in rest:
                assert l[t, e] > l[t, f] or (l[t, e] == l[t, f] and e < f)
        for s in range(k - 1):
            a, b = sel[s], sel[s + 1]
            assert l[t, a] > l[t, b] or (l[t, a] == l[t, b] and a < b)


def test_topk_special_cases():
    E, k = 8, 3
    assert oracle.topk_select(np.zeros((2, E)), k).tolist() == [[0, 1, 2]] * 2
    assert oracle.topk_select(np.full((1, E), 1.5), E).tolist() == [list(range(E))]
    # duplicated router columns: the lower expert index comes first
    X = np.random.default_rng(0).standard_normal((4, 6))
    Wr = np.random.default_rng(1).standard_normal((6, 5))
    Wr[:, 4] = Wr[:, 1]
    l = oracle.router_logits(X, Wr)
    idx = oracle.topk_select(l, 5)
    for t in range(4):
        r = list(idx[t])
        assert r.index(1) + 1 == r.index(4)
    # signed zeros tie
    assert oracle.topk_select(np.array([[-0.0, 0.0]]), 1).tolist() == [[0]]
    assert oracle.topk_select(np.array([[0.0, -0.0]]), 1).tolist() == [[0]]
    with pytest.raises(ValueError):
        oracle.topk_select(np.zeros((1, 3)), 4)


def test_gates_closed_forms():
    rng = np.random.default_rng(7)
    l = rng.standard_normal((40, 9)) * 3
    # k = 1: the gate is exactly one
    _, g1 = oracle.route(l, 1)
    assert np.all(g1 == 1.0)
    # k = 2: g0 = sigmoid(l0 - l1)
    idx, g2 = oracle.route(l, 2)
    l0 = np.take_along_axis(l, idx[:, :1], 1)[:, 0]
    l1 = np.take_along_axis(l, idx[:, 1:2], 1)[:, 0]
    np.testing.assert_allclose(g2[:, 0], 1 / (1 + np.exp(l1 - l0)), rtol=1e-13)
    np.testing.assert_allclose(g2[:, 1], 1 / (1 + np.exp(l0 - l1)), rtol=1e-13)
    # k = E: the full softmax (library routine), in the top-k order
    idx, gE = oracle.route(l, 9)
    sm = scipy.special.softmax(l, axis=1)
    np.testing.assert_allclose(gE, np.take_along_axis(sm, idx, 1), rtol=1e-12)


def test_gates_invariants():
    rng = np.random.default_rng(8)
    l = rng.standard_normal((64, 896)) * 2
    idx, g = oracle.route(l, 16)
    np.testing.assert_allclose(g.sum(1), 1.0, rtol=0, atol=1e-14)
    assert np.all(np.diff(g, axis=1) <= 1e-15)  # non-increasing in the slot
    # shift invariance of the softmax
    _, gs = oracle.route(l + 123.0, 16)
    np.testing.assert_allclose(gs, g, rtol=1e-11)
    # an unselected logit that stays unselected does not move the gates
    l2 = l.copy()
    t = 3
    sel = set(idx[t].tolist())
    f = next(e for e in range(896) if e not in sel)
    l2[t, f] = l[t, f] - 5.0
    _, g2 = oracle.route(l2, 16)
    np.testing.assert_allclose(g2[t], g[t], rtol=1e-13)
    # the gates equal a softmax over the selected logits alone
    sel_l = np.take_along_axis(l, idx, 1)
    np.testing.assert_allclose(g, scipy.special.softmax(sel_l, axis=1), rtol=1e-12)


def test_logit_error_bound_covers_fp32_sums():
    rng = np.random.default_rng(9)
    H, E = 512, 16
    X = rng.standard_normal((32, H)).astype(np.float32)
    Wr = (rng.standard_normal((H, E)) * 0.02).astype(np.float32)
    l64 = oracle.router_logits(X, Wr)
    # fp32 recursive summation, the worst ordering for the classical bound
    acc = np.zeros((32, E), np.float32)
    for h in range(H):
        acc = (acc + np.float32(1) * (X[:, h:h + 1] * Wr[h:h + 1, :]).astype(np.float32)).astype(np.float32)
    tau = oracle.logit_error_bound(X, Wr)
    assert np.all(np.abs(acc - l64).max(1) <= tau / 2)
