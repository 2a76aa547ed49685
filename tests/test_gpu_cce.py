"""Vocabulary-strip cross-entropy on the GPU, through the C ABI, against the
fp64 oracle:

  * a small ragged case (777 tokens, V = 20,000 in strips of 4096, 5% of the
    targets ignored) against the whole oracle, forward and backward, with the
    mean-loss upstream gradient and with a random one;
  * bitwise independence of every output from the strip width (strips of 256,
    4096 and one strip covering the vocabulary) and run-to-run determinism;
  * edge cases: one token, a vocabulary narrower than one tile, a last strip
    one column wide, targets on strip boundaries, every token ignored, no
    tokens;
  * the full-size case (8192 tokens, H 7168, V 200,000, strips of 8192) on
    sampled tokens and vocabulary rows, in the launch configuration the
    benchmark times, and its strip-width invariance against strips of 65,536;
  * the per-kernel debug stages, re-launched in pipeline order, reproduce
    the calls' outputs bitwise.

Tolerances: every output within 1e-2 of max|oracle| (the bf16 bound of the
layer's contract).  The loss and log-normaliser are also held to 1e-3: the
logits are fp32 sums of exact bf16 products, and fp32 summation error over H
terms stays far below that for these inputs."""

import numpy as np
import pytest
import torch

import datagen
import oracle
from gpu_common import DEV, B, BF16_TOL, dev_to_f64, needs_gpu, rel_err, require_lib, say

pytestmark = [pytest.mark.gpu, needs_gpu]

LOSS_TOL = 1e-3
SMALL = datagen.CE_WORKLOADS["vocab_small_bf16"]
FULL = datagen.CE_WORKLOADS["vocab_bf16"]


def bf16_dev(a):
    return torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.bfloat16)


class CeDev:
    def __init__(self, inp: datagen.CeInputs, targets=None):
        self.inp = inp
        self.X = bf16_dev(inp.X)
        self.W = bf16_dev(inp.W)
        self.targets_np = inp.targets if targets is None else np.asarray(targets, np.int32)
        self.t = torch.from_numpy(np.ascontiguousarray(self.targets_np)).to(DEV)
        self.dloss = torch.from_numpy(inp.dloss).to(DEV)


def run(d: CeDev, vc: int, dloss=None):
    inp = d.inp
    plan = B.cce_plan(inp.N, inp.wl.H, inp.wl.V, vc)
    loss, lse = B.cce_forward(plan, d.X, d.W, d.t)
    dX, dW = B.cce_backward(plan, d.X, d.W, d.t, lse, d.dloss if dloss is None else dloss)
    torch.cuda.synchronize()
    return dict(loss=loss, lse=lse, dX=dX, dW=dW)


def bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def same_bits(a, b):
    return all(torch.equal(bits(a[k]), bits(b[k])) for k in ("loss", "lse", "dX", "dW"))


def check_against_oracle(name, d: CeDev, out, dloss_np):
    inp = d.inp
    X64, W64 = inp.to_f64(inp.X), inp.to_f64(inp.W)
    loss, lse = oracle.ce_forward(X64, W64, d.targets_np)
    dX, dW = oracle.ce_backward(X64, W64, d.targets_np, lse, dloss_np)
    errs = {"loss": rel_err(dev_to_f64(out["loss"]), loss),
            "lse": rel_err(dev_to_f64(out["lse"]), lse),
            "dX": rel_err(dev_to_f64(out["dX"]), dX),
            "dW": rel_err(dev_to_f64(out["dW"]), dW)}
    say(f"[{name}] max|gpu-oracle|/max|oracle|: " + ", ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    assert errs["loss"] <= LOSS_TOL and errs["lse"] <= LOSS_TOL
    assert all(v <= BF16_TOL for v in errs.values()), errs
    ign = np.nonzero((d.targets_np < 0) | (d.targets_np >= inp.wl.V))[0]
    if len(ign):
        assert torch.count_nonzero(out["loss"][torch.from_numpy(ign).to(DEV)]) == 0
        assert torch.count_nonzero(out["dX"][torch.from_numpy(ign).to(DEV)].float()) == 0


def test_small_against_oracle_and_strip_invariance():
    require_lib()
    inp = datagen.CeInputs(SMALL)
    d = CeDev(inp)
    say(f"[small] N={inp.N} H={SMALL.H} V={SMALL.V} v_chunk={SMALL.v_chunk}, "
        f"{int((inp.targets < 0).sum())} ignored")
    out = run(d, SMALL.v_chunk)
    check_against_oracle("small", d, out, inp.dloss.astype(np.float64))
    # strip width: 256-wide strips, and one strip over the whole vocabulary
    for vc in (256, -(-SMALL.V // 256) * 256):
        other = run(d, vc)
        assert same_bits(out, other), f"v_chunk {vc} differs"
        say(f"[small] v_chunk {vc}: bitwise identical")
    assert same_bits(out, run(d, SMALL.v_chunk)), "not deterministic"
    # a random upstream gradient (signs and magnitudes per token)
    g = np.random.default_rng(5).standard_normal(inp.N).astype(np.float32)
    out2 = run(d, SMALL.v_chunk, dloss=torch.from_numpy(g).to(DEV))
    check_against_oracle("small, random dloss", d, out2, g.astype(np.float64))


EDGE = {
    # one token, a vocabulary narrower than one 256-column tile
    "one_token": dict(N=1, H=128, V=100, v_chunk=256),
    # 300 tokens (a ragged row tile); V = 257 leaves a last strip one column wide
    "one_column_strip": dict(N=300, H=256, V=257, v_chunk=256),
    # several strips, targets placed on strip and tile boundaries
    "boundaries": dict(N=64, H=384, V=3000, v_chunk=512),
}


@pytest.mark.parametrize("name", sorted(EDGE))
def test_edge_case(name):
    require_lib()
    wl = SMALL.with_(name=name, ignore_frac=0.0, **EDGE[name])
    inp = datagen.CeInputs(wl)
    t = inp.targets.copy()
    V, vc = wl.V, wl.v_chunk
    special = [0, V - 1, min(vc - 1, V - 1), min(vc, V - 1), min(255, V - 1), min(256, V - 1)]
    t[:min(len(special), wl.N)] = special[:wl.N]
    d = CeDev(inp, targets=t)
    say(f"[{name}] N={wl.N} H={wl.H} V={V} v_chunk={vc} targets[:6]={t[:6].tolist()}")
    out = run(d, vc)
    check_against_oracle(name, d, out, inp.dloss.astype(np.float64))
    one = run(d, -(-V // 256) * 256)
    assert same_bits(out, one), "strip width changed the result"


def test_every_token_ignored():
    require_lib()
    wl = SMALL.with_(name="all_ignored", N=40, H=128, V=600, v_chunk=256, ignore_frac=0.0)
    inp = datagen.CeInputs(wl)
    d = CeDev(inp, targets=np.full(wl.N, -100, np.int32))
    out = run(d, wl.v_chunk)
    assert torch.count_nonzero(out["loss"]) == 0
    assert torch.count_nonzero(out["dX"].float()) == 0 and torch.count_nonzero(out["dW"]) == 0
    _, lse = oracle.ce_forward(inp.to_f64(inp.X), inp.to_f64(inp.W), d.targets_np)
    assert rel_err(dev_to_f64(out["lse"]), lse) <= LOSS_TOL


def test_zero_tokens():
    require_lib()
    plan = B.cce_plan(0, 128, 1000, 256)
    X = torch.empty((0, 128), dtype=torch.bfloat16, device=DEV)
    W = torch.randn(1000, 128, device=DEV).to(torch.bfloat16)
    t = torch.empty(0, dtype=torch.int32, device=DEV)
    loss, lse = B.cce_forward(plan, X, W, t)
    dW = torch.full((1000, 128), 7.0, device=DEV)
    dX, dW = B.cce_backward(plan, X, W, t, lse, torch.empty(0, device=DEV), dW=dW)
    torch.cuda.synchronize()
    assert loss.numel() == 0 and dX.shape == (0, 128)
    assert torch.count_nonzero(dW) == 0


@pytest.fixture(scope="module")
def full_inputs():
    say(f"[full] drawing inputs N={FULL.N} H={FULL.H} V={FULL.V}")
    return datagen.CeInputs(FULL, progress=say)


def test_full_size_sampled(full_inputs):
    require_lib()
    inp = full_inputs
    d = CeDev(inp)
    rng = np.random.default_rng(11)
    toks = np.sort(rng.choice(FULL.N, 16, replace=False))
    # upstream gradient only on the sampled tokens: dW is then exactly their
    # contribution, which the oracle forms from their own rows
    g = np.zeros(FULL.N, np.float32)
    g[toks] = rng.standard_normal(len(toks)).astype(np.float32)
    gd = torch.from_numpy(g).to(DEV)
    out = run(d, FULL.v_chunk, dloss=gd)
    say("[full] GPU done; oracle on sampled tokens")
    W64 = inp.to_f64(inp.W)
    X64 = inp.to_f64(inp.X[toks])
    t_s = inp.targets[toks]
    loss, lse = oracle.ce_forward_tokens(X64, W64, t_s)
    idx = torch.from_numpy(toks).to(DEV)
    e_loss = rel_err(dev_to_f64(out["loss"][idx]), loss)
    e_lse = rel_err(dev_to_f64(out["lse"][idx]), lse)
    vrows = np.unique(np.concatenate([t_s[t_s >= 0], rng.choice(FULL.V, 200, replace=False),
                                      [0, FULL.V - 1]]))
    dXr, dWr, _ = oracle.ce_backward_tokens_rows(X64, W64, t_s, g[toks].astype(np.float64), vrows)
    e_dx = rel_err(dev_to_f64(out["dX"][idx]), dXr)
    e_dw = rel_err(dev_to_f64(out["dW"][torch.from_numpy(vrows).to(DEV)]), dWr)
    say(f"[full] sampled rel err: loss {e_loss:.2e} lse {e_lse:.2e} dX {e_dx:.2e} dW {e_dw:.2e}")
    assert e_loss <= LOSS_TOL and e_lse <= LOSS_TOL and e_dx <= BF16_TOL and e_dw <= BF16_TOL
    rest = torch.ones(FULL.N, dtype=torch.bool, device=DEV)
    rest[idx] = False
    assert torch.count_nonzero(out["dX"][rest].float()) == 0
    del W64
    # the same batch in strips of 65,536: bitwise identical
    other = run(d, 65536, dloss=gd)
    assert same_bits(out, other), "strip width changed the full-size result"
    say("[full] strips of 65,536: bitwise identical")


def test_debug_stages_replay_the_calls():
    # re-launching every strip's kernels in pipeline order through
    # cce_debug_stage reproduces the calls' outputs bitwise (the benchmark's
    # per-kernel timings rely on it)
    require_lib()
    wl = SMALL.with_(name="stages", N=300, H=256, V=3000, v_chunk=1024)
    inp = datagen.CeInputs(wl)
    d = CeDev(inp)
    plan = B.cce_plan(wl.N, wl.H, wl.V, wl.v_chunk)
    wsf, wsb = B.workspace(plan, "fwd", DEV), B.workspace(plan, "bwd", DEV)
    loss, lse = B.cce_forward(plan, d.X, d.W, d.t, ws=wsf)
    dX, dW = B.cce_backward(plan, d.X, d.W, d.t, lse, d.dloss, ws=wsb)
    torch.cuda.synchronize()
    loss0, lse0, dW0 = loss.clone(), lse.clone(), dW.clone()
    loss.zero_(); lse.zero_(); dW.zero_()
    for s in range(plan.S):
        for st in ("logits", "fold"):
            B.cce_debug_stage(plan, st, s, d.X, d.W, d.t, loss, lse, d.dloss, dX, dW, wsf)
    for s in range(plan.S):
        for st in ("grad", "dx", "dw"):
            B.cce_debug_stage(plan, st, s, d.X, d.W, d.t, loss, lse, d.dloss, dX, dW, wsb)
    torch.cuda.synchronize()
    assert torch.equal(loss, loss0) and torch.equal(lse, lse0) and torch.equal(dW, dW0)
