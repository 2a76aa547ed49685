"""The layer's calls under HIP graph capture, through the C ABI.

No entry point synchronises, allocates, copies through the host or clears
memory with a memset, so a call enqueued on a capturing stream records only
its kernels.  Each test captures a call with its outputs and workspace
allocated beforehand, then replays the graph several times, with eager work
between the replays (the outputs overwritten by fill kernels) and a
synchronisation after each, and checks every replay against the eager call
bitwise.  New inputs copied into the captured input buffers must then give
what an eager call on them gives: the graph reads its inputs at replay time.

Cases: the bf16 forward and backward of a ragged 16-chunk batch (777 tokens,
H 2048, 64 experts, top-8), the fp32 configuration (register-staged GEMMs),
and the vocabulary-strip cross-entropy forward and backward (300 tokens,
V 3000 in strips of 1024)."""

import numpy as np
import pytest
import torch

import datagen
from gpu_common import DEV, B, DevInputs, needs_gpu, plan_for, require_lib, say, to_dev

pytestmark = [pytest.mark.gpu, needs_gpu]

REPLAYS = 3


def capture(fn):
    # warm-up on a side stream (default priority), then capture on torch's
    # capture stream, which is the current stream inside the context
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def bits(t):
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16)
    if t.dtype == torch.float32:
        return t.view(torch.int32)
    return t


def replay_and_check(name, g, outs, refs):
    for r in range(REPLAYS):
        for t in outs.values():
            t.fill_(7)  # eager work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, t in outs.items():
            assert torch.equal(bits(t), bits(refs[k])), f"{name}: replay {r}: {k} differs"
    say(f"[{name}] {REPLAYS} replays bitwise equal to the eager call")


MOE_CASES = {
    "train_bf16": dict(N=777, c=49),
    "tiny_f32": dict(N=256, c=64),
}


@pytest.mark.parametrize("name", sorted(MOE_CASES))
def test_moe_forward_backward_graph(name):
    require_lib()
    wl = datagen.WORKLOADS[name]
    cs = MOE_CASES[name]
    inp = datagen.Inputs(wl, N=cs["N"], dy=True)
    d = DevInputs(inp)
    plan = plan_for(wl, N=cs["N"], c=cs["c"])
    dt = d.X.dtype
    N, H, F, E, k = plan.N, plan.H, plan.F, plan.E, plan.k
    say(f"[{name}] N={N} K={plan.K} c_eff={plan.c_eff}")
    f32 = torch.float32
    fo = {"Y": torch.empty((N, H), dtype=dt, device=DEV),
          "idx": torch.empty((N, k), dtype=torch.int32, device=DEV),
          "gates": torch.empty((N, k), dtype=f32, device=DEV),
          "logits": torch.empty((N, E), dtype=f32, device=DEV)}
    wsf = B.workspace(plan, "fwd", DEV)

    def fwd():
        B.moe_bounded_forward(plan, d.X, d.Wr, d.bias, d.Wg, d.Wu, d.Wd, Y=fo["Y"],
                              topk_idx=fo["idx"], gates=fo["gates"], logits=fo["logits"], ws=wsf)

    fwd()
    torch.cuda.synchronize()
    fref = {kk: t.clone() for kk, t in fo.items()}
    gf = capture(fwd)
    replay_and_check(f"{name} forward", gf, fo, fref)

    # the backward reads the forward's routing: fixed copies of it
    idx, gates = fref["idx"].clone(), fref["gates"].clone()
    bo = {"dX": torch.empty((N, H), dtype=dt, device=DEV),
          "dW_gate": torch.empty((E, H, F), dtype=f32, device=DEV),
          "dW_up": torch.empty((E, H, F), dtype=f32, device=DEV),
          "dW_down": torch.empty((E, F, H), dtype=f32, device=DEV),
          "dlogits": torch.empty((N, E), dtype=f32, device=DEV),
          "dgates": torch.empty((N, k), dtype=f32, device=DEV),
          "dW_r": torch.empty((H, E), dtype=f32, device=DEV)}
    wsb = B.workspace(plan, "bwd", DEV)

    def bwd():
        B.moe_bounded_backward(plan, d.X, d.Wr, d.Wg, d.Wu, d.Wd, d.dY, idx, gates, ws=wsb, **bo)

    bwd()
    torch.cuda.synchronize()
    bref = {kk: t.clone() for kk, t in bo.items()}
    gb = capture(bwd)
    replay_and_check(f"{name} backward", gb, bo, bref)

    # new inputs into the captured buffers: the replay follows them
    inp2 = datagen.Inputs(wl.with_(seed=wl.seed + 1), N=N, dy=True)
    d.X.copy_(to_dev(inp2.X, wl))
    d.dY.copy_(to_dev(inp2.dY, wl))
    torch.cuda.synchronize()
    gf.replay()
    torch.cuda.synchronize()
    got = {kk: t.clone() for kk, t in fo.items()}
    Y2, idx2, g2, lg2, _ = B.moe_bounded_forward(plan, d.X, d.Wr, d.bias, d.Wg, d.Wu, d.Wd)
    torch.cuda.synchronize()
    assert not torch.equal(bits(got["Y"]), bits(fref["Y"]))
    for kk, t in (("Y", Y2), ("idx", idx2), ("gates", g2), ("logits", lg2)):
        assert torch.equal(bits(got[kk]), bits(t)), f"{name}: forward replay on new X: {kk}"
    gb.replay()
    torch.cuda.synchronize()
    out2 = B.moe_bounded_backward(plan, d.X, d.Wr, d.Wg, d.Wu, d.Wd, d.dY, idx, gates)
    torch.cuda.synchronize()
    for kk in bo:
        assert torch.equal(bits(bo[kk]), bits(out2[kk])), f"{name}: backward replay on new inputs: {kk}"
    say(f"[{name}] replays on new inputs equal eager calls on them")


def test_cce_graph():
    require_lib()
    wl = datagen.CE_WORKLOADS["vocab_small_bf16"].with_(name="graph", N=300, H=256, V=3000,
                                                        v_chunk=1024)
    inp = datagen.CeInputs(wl)
    bf = lambda a: torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.bfloat16)
    X, W = bf(inp.X), bf(inp.W)
    t = torch.from_numpy(np.ascontiguousarray(inp.targets)).to(DEV)
    dloss = torch.from_numpy(inp.dloss).to(DEV)
    plan = B.cce_plan(wl.N, wl.H, wl.V, wl.v_chunk)
    wsf, wsb = B.workspace(plan, "fwd", DEV), B.workspace(plan, "bwd", DEV)
    o = {"loss": torch.empty(wl.N, device=DEV), "lse": torch.empty(wl.N, device=DEV),
         "dX": torch.empty((wl.N, wl.H), dtype=torch.bfloat16, device=DEV),
         "dW": torch.empty((wl.V, wl.H), device=DEV)}

    def both():
        B.cce_forward(plan, X, W, t, loss=o["loss"], lse=o["lse"], ws=wsf)
        B.cce_backward(plan, X, W, t, o["lse"], dloss, dX=o["dX"], dW=o["dW"], ws=wsb)

    both()
    torch.cuda.synchronize()
    ref = {kk: v.clone() for kk, v in o.items()}
    g = capture(both)
    replay_and_check("cce", g, o, ref)
