"""Stage-level parity on the GPU, bit-exact: the router top-k (and its gates)
and the per-chunk permutation against the fp64 oracle."""

import numpy as np
import pytest
import torch

import oracle
from gpu_common import DEV, B, needs_gpu, require_lib, say

pytestmark = [pytest.mark.gpu, needs_gpu]


@pytest.mark.parametrize("N,E,k", [(1000, 8, 1), (1000, 8, 2), (777, 64, 8), (513, 128, 8),
                                   (300, 896, 16), (129, 1024, 64), (64, 64, 64), (5, 40, 3)])
def test_topk_random(N, E, k):
    require_lib()
    say(f"topk N={N} E={E} k={k}")
    rng = np.random.default_rng(N * 31 + E)
    lg = rng.standard_normal((N, E)).astype(np.float32)
    idx, g = B.moe_debug_topk(torch.from_numpy(lg).to(DEV), k)
    idx, g = idx.cpu().numpy(), g.cpu().numpy()
    ref = oracle.topk_select(lg.astype(np.float64), k)
    assert np.array_equal(idx, ref)
    np.testing.assert_allclose(g, oracle.gates_from_logits(lg.astype(np.float64), ref), rtol=0,
                               atol=2e-6)
    np.testing.assert_allclose(g.sum(1), 1.0, atol=1e-5)


def test_topk_forced_ties():
    require_lib()
    rng = np.random.default_rng(3)
    cases = []
    cases.append(rng.integers(-2, 3, size=(500, 64)).astype(np.float32))      # many ties
    cases.append(np.zeros((8, 896), np.float32))                                 # all equal
    z = np.zeros((16, 8), np.float32)
    z[:, ::2] = -0.0                                                              # +0 / -0 ties
    cases.append(z)
    d = rng.standard_normal((64, 128)).astype(np.float32)
    d[:, 100] = d[:, 7]                                                           # duplicated expert
    d[:, 64] = d[:, 3]                                                            # across lanes
    cases.append(d)
    for lg in cases:
        for k in (1, 2, 7, min(16, lg.shape[1])):
            idx, g = B.moe_debug_topk(torch.from_numpy(lg).to(DEV), k)
            ref = oracle.topk_select(lg.astype(np.float64), k)
            assert np.array_equal(idx.cpu().numpy(), ref), (lg.shape, k)
    idx, g = B.moe_debug_topk(torch.from_numpy(cases[0]).to(DEV), 1)
    assert np.all(g.cpu().numpy() == 1.0)  # k = 1: the gate is exactly one


@pytest.mark.parametrize("E", [40, 64, 896])
def test_topk_nan_logits(E):
    """NaN logits rank as -inf (both top-k kernels: E <= 64 and above): the
    selection is bit-exact against the oracle and every slot holds a distinct
    expert; rows whose selected logits are finite keep finite gates."""
    require_lib()
    rng = np.random.default_rng(E)
    N = 300
    lg = rng.standard_normal((N, E)).astype(np.float32)
    lg[rng.random((N, E)) < 0.2] = np.nan
    lg[:4] = np.nan                  # rows of NaN only
    lg[4:8, ::3] = -np.inf           # NaN and -inf together
    for k in (1, 5, 16):
        say(f"topk NaN E={E} k={k}")
        idx, g = B.moe_debug_topk(torch.from_numpy(lg).to(DEV), k)
        idx, g = idx.cpu().numpy(), g.cpu().numpy()
        assert np.array_equal(idx, oracle.topk_select(lg.astype(np.float64), k))
        assert all(len(set(r.tolist())) == k for r in idx)
        fin = np.all(np.isfinite(np.take_along_axis(lg, idx, 1)), axis=1)
        assert np.all(np.isfinite(g[fin]))


@pytest.mark.parametrize("N,E,k,c,K_max", [
    (256, 8, 2, 64, 8),          # tiny workload's plan (K = 4)
    (4096, 64, 8, 1024, 8),      # balanced shape
    (8192, 896, 16, 1024, 8),    # 896 experts
    (1000, 16, 3, 97, 7),        # ragged chunks (1000 = 7*142 + 6)
    (5000, 64, 8, 5000, 1),      # one chunk spanning many planner blocks
    (70, 8, 8, 9, 100),          # k = E, K = 8
    (1, 8, 2, 4, 4),             # one token
])
def test_plan_bit_exact(N, E, k, c, K_max):
    require_lib()
    say(f"plan N={N} E={E} k={k} c={c} K_max={K_max}")
    rng = np.random.default_rng(N + E)
    if E >= 64:  # skewed routing: low experts hot
        w = 1.0 / np.arange(1, E + 1)
        idx = np.stack([rng.choice(E, size=k, replace=False, p=w / w.sum()) for _ in range(N)])
    else:
        idx = np.stack([rng.permutation(E)[:k] for _ in range(N)])
    idx = idx.astype(np.int32)
    H = 64
    plan = B.moe_plan_chunks(N, H, H, E, k, c, K_max, B.MOE_BF16)
    offs, perm, pos = B.moe_debug_plan(plan, torch.from_numpy(idx).to(DEV))
    offs, perm, pos = offs.cpu().numpy(), perm.cpu().numpy(), pos.cpu().numpy()
    K, ce = oracle.plan_chunks(N, c, K_max)
    assert plan.K == K
    for i in range(K):
        o, pt, ps, ps_pos = oracle.permute_chunk(idx, E, K, i)
        base = oracle.pair_base(N, K, k, i)
        R = len(pt)
        assert R <= k * ce
        assert np.array_equal(offs[i], o), i
        assert np.array_equal(perm[base:base + R], pt * k + ps), i
        toks = oracle.chunk_tokens(N, K, i)
        got_pos = pos.reshape(N, k)[toks]
        assert np.array_equal(got_pos, ps_pos), i


@pytest.mark.parametrize("name,n,c", [("tiny_f32", 256, 64), ("train_bf16", 777, 49)])
def test_backward_stages_replay_the_call(name, n, c):
    """moe_debug_stage_bwd: the whole-call stages and then every per-chunk
    stage of chunks 0..K-1, in the backward call's order, rewrite the call's
    outputs (first overwritten with garbage) bitwise."""
    import datagen
    from gpu_common import DevInputs, plan_for

    require_lib()
    wl = datagen.WORKLOADS[name]
    inp = datagen.Inputs(wl.with_(N=n), dy=True)
    d = DevInputs(inp)
    plan = plan_for(wl, N=n, c=c)
    say(f"backward stages {name} N={n} K={plan.K}")
    _, idx, g, _, _ = B.moe_bounded_forward(plan, d.X, d.Wr, d.bias, d.Wg, d.Wu, d.Wd)
    ws = B.workspace(plan, "bwd", DEV)
    out = B.moe_bounded_backward(plan, d.X, d.Wr, d.Wg, d.Wu, d.Wd, d.dY, idx, g, ws=ws)
    out.pop("stats")
    torch.cuda.synchronize()
    ref = {k_: v.clone() for k_, v in out.items()}
    for v in out.values():
        v.view(torch.uint8).fill_(0x7F)
    for s in ("zero", "transpose", "plan"):
        B.moe_debug_stage_bwd(plan, s, 0, d.X, d.Wr, d.Wg, d.Wu, d.Wd, d.dY, idx, g, out, ws)
    for i in range(plan.K):
        for s in ("recompute", "dh", "wgrad_down", "wgrad_gate_up", "dx", "combine_bwd", "dwr"):
            B.moe_debug_stage_bwd(plan, s, i, d.X, d.Wr, d.Wg, d.Wu, d.Wd, d.dY, idx, g, out, ws)
    torch.cuda.synchronize()
    for k_, v in out.items():
        assert torch.equal(v.view(torch.uint8), ref[k_].view(torch.uint8)), k_
