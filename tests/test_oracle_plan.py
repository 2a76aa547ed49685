"""Pins for the oracle's chunk plan (eq. (1) of the bounded-streaming operators
page, Methodology 1 "PipelinedLLEP", and its strided chunk membership)."""

import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def brute_plan(N, c, K_max):
    """Eq. (1) by search: the fewest chunks of at most c tokens that cover N,
    capped at K_max, then the smallest chunk size that covers N with K chunks."""
    if N == 0:
        return 0, 0
    K0 = 1
    while K0 * c < N:
        K0 += 1
    K = min(K0, K_max)
    ce = 1
    while K * ce < N:
        ce += 1
    return K, ce


def test_page_worked_instance():
    g = json.load(open(os.path.join(GOLDEN, "plan_page_instance.json")))
    for K_max in (g["K"], g["K"] + 1, 16, 1000):
        K, ce = oracle.plan_chunks(g["N"], g["c"], K_max)
        assert K == g["K"]
        assert ce == g["c_eff_expected"]
    lo, hi = g["N_range_giving_K10"]
    for N in (lo, lo + 1, (lo + hi) // 2, hi):
        assert oracle.plan_chunks(N, g["c"], 64)[0] == g["K"]
    assert oracle.plan_chunks(lo - 1, g["c"], 64)[0] == g["K"] - 1
    assert oracle.plan_chunks(hi + 1, g["c"], 64)[0] == g["K"] + 1


def test_exhaustive_small_against_search():
    for N in range(0, 121):
        for c in range(1, N + 3):
            for K_max in range(1, 21):
                assert oracle.plan_chunks(N, c, K_max) == brute_plan(N, c, K_max), (N, c, K_max)


def test_invalid_arguments():
    for args in ((-1, 4, 2), (10, 0, 2), (10, 4, 0)):
        with pytest.raises(ValueError):
            oracle.plan_chunks(*args)


@pytest.mark.parametrize("N,c,K_max", [(1, 1, 1), (7, 3, 8), (256, 64, 8), (300, 7, 20),
                                       (4096, 1024, 8), (16384, 2048, 16), (8192, 1024, 8),
                                       (65536, 4096, 16), (1000, 1, 3), (1001, 1000, 1)])
def test_membership_invariants(N, c, K_max):
    K, ce = oracle.plan_chunks(N, c, K_max)
    sizes = oracle.chunk_sizes(N, K)
    assert sizes.sum() == N
    assert sizes.max() == ce
    assert sizes.max() - sizes.min() <= 1
    assert 1 <= K <= N
    # closed form of the strided chunk size
    assert all(sizes[i] == -(-(N - i) // K) for i in range(K))
    # every token is in exactly one chunk, chunk i holds t = i mod K
    seen = np.zeros(N, dtype=np.int64)
    for i in range(K):
        t = oracle.chunk_tokens(N, K, i)
        assert np.all(t % K == i)
        seen[t] += 1
    assert np.all(seen == 1)
    # route bound (E_p = 1): pairs per chunk <= k c_eff, for any k
    for k in (1, 2, 8, 16):
        assert (k * sizes).max() <= k * ce
    # when K_max does not bind, c_eff never exceeds the budget c
    if K == -(-N // c):
        assert ce <= c
    # pair bases are the running sum of k n_i
    for k in (1, 3):
        run = 0
        for i in range(K):
            assert oracle.pair_base(N, K, k, i) == run
            run += k * sizes[i]


@pytest.mark.parametrize("k,c_eff,H,b,expect", [
    (2, 64, 64, 4, 64 * 1024),            # tiny fp32: 64 KiB
    (8, 1024, 2048, 2, 64 * 2**20),       # balanced bf16: 64 MiB
    (8, 2048, 4096, 2, 256 * 2**20),      # zipf bf16: 256 MiB
    (16, 1024, 2048, 2, 128 * 2**20),     # 896 experts: 128 MiB
    (8, 4096, 2048, 2, 256 * 2**20),      # train bf16: 256 MiB
])
def test_dispatch_bound(k, c_eff, H, b, expect):
    assert oracle.dispatch_bound_bytes(k, c_eff, H, b) == expect
