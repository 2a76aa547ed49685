"""Whole-layer parity on the GPU for the method's degenerate and edge cases,
through the C ABI, against the full fp64 oracle (forward and backward):

  * k = E (every expert selected; the gates are the full softmax) with a
    ragged last chunk;
  * a single token (one chunk of one row per selected expert), fp32;
  * 64 experts with 20 tokens of top-2: most experts have no rows in a chunk;
  * k = 1 (every gate exactly 1; the backward's row-indexed loads then take
    a pair index as its token, with no division);
  * one token per chunk (c = 1, K = N);
  * K_max binding: c = 10 asks for 100 chunks, K_max = 3 gives c_eff = 334
    (with F = 256 also: chunked and unchunked runs on different tile shapes
    and backward kernels);
  * every token routed to the same two experts (a Zipf(12) router bias over
    8 experts with top-2): two full segments per chunk, six empty experts;
  * the largest k: k = E = 64, every token in every expert;
  * the largest E: 1024 experts with top-64 (most experts hold a few rows
    of a chunk, many none);
  * fp32 with k = E = 4;
  * N = 0: both entry points succeed and enqueue nothing but the weight
    gradients' zero fill.

Each case also checks chunked == unchunked (K_max = 1) bitwise for the
per-token outputs and run-to-run determinism (run_workload does both).  The
H = 64 cases run the weight gradients in 64-row tiles, so the row-indexed
products are exercised in their 64- and 128-row shapes."""

import numpy as np
import pytest
import torch

import datagen
from gpu_common import DEV, B, needs_gpu, require_lib, say
from test_gpu_layer import run_workload

pytestmark = [pytest.mark.gpu, needs_gpu]

BF = datagen.WORKLOADS["train_bf16"]   # x ~ N(0, 1), weights ~ N(0, 0.02), backward
F32 = datagen.WORKLOADS["tiny_f32"]    # everything ~ N(0, 0.02), fp32, backward

CASES = {
    # k = E = 8: K = 4 chunks of 10, 9, 9, 9 tokens
    "k_eq_E_bf16": BF.with_(name="k_eq_E_bf16", N=37, H=64, E=8, k=8, F=128, c=10, K_max=8),
    # one token, top-2 of 8 experts, fp32
    "one_token_f32": F32.with_(name="one_token_f32", N=1, H=64, E=8, k=2, F=64, c=4, K_max=4),
    # 20 tokens over 64 experts: at most 10 non-empty experts per chunk
    "sparse_experts_bf16": BF.with_(name="sparse_experts_bf16", N=20, H=128, E=64, k=2, F=64,
                                    c=6, K_max=8),
    # k = 1
    "top1_bf16": BF.with_(name="top1_bf16", N=50, H=64, E=8, k=1, F=64, c=16, K_max=4),
    # c = 1: nine chunks of one token
    "one_token_per_chunk_bf16": BF.with_(name="one_token_per_chunk_bf16", N=9, H=64, E=8, k=2,
                                         F=64, c=1, K_max=16),
    # K_max binds: K = 3 chunks of 334, 333, 333 tokens
    "kmax_binds_bf16": BF.with_(name="kmax_binds_bf16", N=1000, H=128, E=16, k=4, F=128, c=10,
                                K_max=3),
    # the same with F = 256: the K = 3 chunks (83 rows per expert) take the
    # 128-row tiles and the two-kernel backward, the unchunked run (250 rows
    # per expert) the 256-row tiles and the fused recompute + dh kernel; the
    # dgate shares must still be summed alike
    "mixed_tiles_bf16": BF.with_(name="mixed_tiles_bf16", N=1000, H=128, E=16, k=4, F=256, c=10,
                                 K_max=3),
    # all routing on two experts: segments of a whole chunk, the rest empty
    "two_hot_experts_bf16": BF.with_(name="two_hot_experts_bf16", N=600, H=128, E=8, k=2, F=128,
                                     c=300, K_max=4, zipf_s=12.0),
    # k = E = 64
    "k64_bf16": BF.with_(name="k64_bf16", N=10, H=64, E=64, k=64, F=64, c=4, K_max=4),
    # E = 1024 (the largest the ABI takes), top-64: 2 chunks of 100 tokens
    "max_experts_bf16": BF.with_(name="max_experts_bf16", N=200, H=64, E=1024, k=64, F=64, c=100,
                                 K_max=4),
    # fp32, k = E = 4
    "k_eq_E_f32": F32.with_(name="k_eq_E_f32", N=30, H=64, E=4, k=4, F=64, c=8, K_max=8),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_edge_case(name):
    wl = CASES[name]
    say(f"[{name}] N={wl.N} H={wl.H} E={wl.E} k={wl.k} F={wl.F} c={wl.c} K_max={wl.K_max}")
    run_workload(name, full=False, wl=wl, reduced=(wl.N, wl.c))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_zero_tokens(dtype):
    require_lib()
    H, F, E, k = 64, 64, 8, 2
    plan = B.moe_plan_chunks(0, H, F, E, k, 16, 4, B.MOE_BF16 if dtype == "bf16" else B.MOE_F32)
    assert plan.K == 0 and plan.fwd_workspace_bytes == 0
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    r = lambda *s: torch.randn(*s, device=DEV).to(dt)
    X, Wr, Wg, Wu, Wd = r(0, H), r(H, E), r(E, H, F), r(E, H, F), r(E, F, H)
    Y, idx, g, lg, st = B.moe_bounded_forward(plan, X, Wr, None, Wg, Wu, Wd)
    torch.cuda.synchronize()
    assert Y.shape == (0, H) and idx.shape == (0, k) and st["K"] == 0
    # the weight gradients are overwritten with zeros, everything else is empty
    dWg = torch.full((E, H, F), 7.0, device=DEV)
    out = B.moe_bounded_backward(plan, X, Wr, Wg, Wu, Wd, r(0, H), idx, g, dW_gate=dWg)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out["dW_gate"]) == 0
    assert torch.count_nonzero(out["dW_up"]) == 0 and torch.count_nonzero(out["dW_down"]) == 0
    assert torch.count_nonzero(out["dW_r"]) == 0
    assert out["dX"].shape == (0, H)
