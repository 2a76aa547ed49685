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


def test_topk_nan_reads_as_minus_inf():
    """NaN logits: brute force over a pure-Python order in which NaN is the
    same key as -inf (ties broken by index); every row gets k distinct
    experts."""
    rng = np.random.default_rng(15)
    key = lambda v: float("-inf") if v != v else float(v)
    for _ in range(200):
        N, E = rng.integers(1, 6), rng.integers(1, 12)
        k = int(rng.integers(1, E + 1))
        l = rng.integers(-2, 2, size=(N, E)).astype(np.float64)
        l[rng.random((N, E)) < 0.3] = np.nan
        l[rng.random((N, E)) < 0.1] = -np.inf
        idx = oracle.topk_select(l, k)
        for t in range(N):
            assert list(idx[t]) == sorted(range(E), key=lambda e: (-key(l[t, e]), e))[:k]
            assert len(set(idx[t].tolist())) == k


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


def _tight_case():
    """Two exact products whose fp32 sum rounds by exactly one unit roundoff:
    1 + 2^-24 is the midpoint between 1 and the next binary32 number, and
    round-to-nearest-even returns 1.  Returns (X, Wr, fp32 error)."""
    X = np.array([[1.0, 2.0 ** -24]], np.float32)
    Wr = np.array([[1.0], [1.0]], np.float32)
    s32 = np.float32(X[0, 0] * Wr[0, 0]) + np.float32(X[0, 1] * Wr[1, 0])
    err = abs(float(s32) - (1.0 + 2.0 ** -24))
    return X, Wr, err


def test_logit_error_bound_closed_form():
    """Pinned from above by the classical bound's value on a 2-term sum.
    With X = [[1, 1]] and W_r = [[1], [1]]: sum |x w| = 2, l = 2, so
    tau = 2 (gamma_2 * 2 + u * 2), gamma_n = n u / (1 - n u), where u is the
    binary32 unit roundoff, taken here from numpy's float32 epsilon (eps / 2)
    rather than from the oracle."""
    u = float(np.finfo(np.float32).eps) / 2
    g2 = 2 * u / (1 - 2 * u)
    tau = oracle.logit_error_bound(np.array([[1.0, 1.0]]), np.array([[1.0], [1.0]]))
    assert tau.shape == (1,)
    assert tau[0] == 2 * (g2 * 2 + u * 2)
    # with a bias of 0.5: sum |x w| + |b| = 2.5, l = 2.5
    tb = oracle.logit_error_bound(np.array([[1.0, 1.0]]), np.array([[1.0], [1.0]]),
                                  np.array([0.5]))
    np.testing.assert_allclose(tb[0], 2 * (g2 * 2.5 + u * 2.5), rtol=1e-15, atol=0)


def test_logit_error_bound_is_nearly_attained():
    """Pinned from above by a real rounding error: a 2-term fp32 sum whose
    error is exactly u (a round-half-to-even tie) reaches a third of tau/2
    (gamma_2 (1 + u) + u (1 + u) ~ 3u).  A bound built on u = 2^-23, or
    doubled, would sit at a sixth of it and fail."""
    X, Wr, err = _tight_case()
    assert err == 2.0 ** -24
    half = oracle.logit_error_bound(X, Wr)[0] / 2
    assert err <= half
    assert err / half >= 0.3333


def test_logit_error_bound_planted_wrong_roundoff_is_caught(monkeypatch):
    """A planted mistake in the oracle (unit roundoff 2^-23 instead of 2^-24)
    makes the bound too loose; the near-attainment check above catches it."""
    from oracle import moe_oracle

    X, Wr, err = _tight_case()
    monkeypatch.setattr(moe_oracle, "FP32_UNIT_ROUNDOFF", 2.0 ** -23)
    half = moe_oracle.logit_error_bound(X, Wr)[0] / 2
    assert err / half < 0.3333
