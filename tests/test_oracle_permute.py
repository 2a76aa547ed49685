"""Pins for the oracle's per-chunk permutation (expert-contiguous layout of a
chunk's routed pairs)."""

import numpy as np
import pytest

import oracle


def random_idx(rng, N, E, k):
    return np.stack([rng.permutation(E)[:k] for _ in range(N)]).astype(np.int64)


def test_hand_example():
    # N=5 tokens, K=2 chunks, top-2 of 3 experts.  Chunk 0 = tokens 0, 2, 4.
    idx = np.array([[2, 0], [1, 2], [0, 1], [2, 1], [0, 2]])
    off, pt, ps, pos = oracle.permute_chunk(idx, 3, 2, 0)
    # pairs in (token, slot) order: (0,0)e2 (0,1)e0 (2,0)e0 (2,1)e1 (4,0)e0 (4,1)e2
    # grouped by expert, token ascending: e0 -> (0,1)(2,0)(4,0); e1 -> (2,1); e2 -> (0,0)(4,1)
    assert off.tolist() == [0, 3, 4, 6]
    assert pt.tolist() == [0, 2, 4, 2, 0, 4]
    assert ps.tolist() == [1, 0, 0, 1, 0, 1]
    assert pos.tolist() == [[4, 0], [1, 3], [2, 5]]
    # chunk 1 = tokens 1, 3: (1,0)e1 (1,1)e2 (3,0)e2 (3,1)e1
    off, pt, ps, pos = oracle.permute_chunk(idx, 3, 2, 1)
    assert off.tolist() == [0, 0, 2, 4]
    assert pt.tolist() == [1, 3, 1, 3]
    assert ps.tolist() == [0, 1, 1, 0]
    assert pos.tolist() == [[0, 2], [3, 1]]


@pytest.mark.parametrize("N,E,k,c,K_max", [(256, 8, 2, 64, 8), (300, 13, 4, 7, 20),
                                           (97, 5, 5, 10, 3), (64, 896, 16, 16, 8), (1, 4, 2, 1, 1)])
def test_invariants(N, E, k, c, K_max):
    rng = np.random.default_rng(N + E)
    idx = random_idx(rng, N, E, k)
    K, ce = oracle.plan_chunks(N, c, K_max)
    seen = np.zeros((N, k), np.int64)
    for i in range(K):
        off, pt, ps, pos = oracle.permute_chunk(idx, E, K, i)
        toks = oracle.chunk_tokens(N, K, i)
        R = len(toks) * k
        assert len(pt) == R <= k * ce
        # offsets: exclusive prefix sum of the per-expert counts, counted by hand
        counts = [0] * E
        for t in toks:
            for s in range(k):
                counts[idx[t, s]] += 1
        run = [0]
        for e in range(E):
            run.append(run[-1] + counts[e])
        assert off.tolist() == run
        # each segment holds exactly expert e's pairs, token ascending
        for e in range(E):
            seg_t, seg_s = pt[off[e]:off[e + 1]], ps[off[e]:off[e + 1]]
            assert np.all(idx[seg_t, seg_s] == e)
            assert np.all(np.diff(seg_t) > 0)
        # pos is the inverse of (perm_t, perm_s)
        for j, t in enumerate(toks):
            for s in range(k):
                r = pos[j, s]
                assert pt[r] == t and ps[r] == s
        seen[pt, ps] += 1
    # every routed pair is processed exactly once over all chunks
    assert np.all(seen == 1)
