"""End-to-end parity of the HIP layer against the fp64 oracle, through the C ABI.

For each workload:
  * a reduced batch (ragged strided chunks, several GEMM tiles) against the
    full unchunked oracle: routing bit-exact on the GPU's logits, outputs to
    max|gpu - oracle| / max|oracle| <= 1e-2 (bf16) or 1e-5 (fp32);
  * the full batch in the launch configuration the benchmark times: routing
    for every token, outputs on sampled tokens (and, for backward, the weight
    gradients of sampled experts) evaluated one by one by the oracle;
  * chunked == unchunked: the same call with K_max = 1 gives bitwise equal
    per-token outputs; two runs give bitwise equal results;
  * the dispatch buffers stay within 2 k c_eff H b (half of it when the bf16
    forward reads its permuted rows from X inside the GEMM).

Beyond the named workloads: grouped expert tiles, the split tile lists of
short segments, and a batch whose X is too large for the in-GEMM gather, so
the forward gathers into its own buffer.
"""

import numpy as np
import pytest
import torch

import datagen
import oracle
from gpu_common import (BF16_TOL, DEV, F32_TOL, DevInputs, backward, check_routing, dev_to_f64,
                        forward, needs_gpu, plan_for, rel_err, require_lib, say)

pytestmark = [pytest.mark.gpu, needs_gpu]

# reduced batch: (N, c) keeping the workload's K and a ragged last chunk
REDUCED = {
    "tiny_f32": (256, 64),
    "balanced_bf16": (1003, 251),
    "zipf_bf16": (301, 38),
    "many_experts_bf16": (515, 65),
    "train_bf16": (777, 49),
}


def _oracle_fwd(inp, X64, idx):
    Y, _, g, _ = oracle.moe_forward(X64, inp.f64("Wr"), inp.bias, inp.expert_f64, None, None,
                                    inp.wl.k, idx=idx)
    return Y, g


def _sub(d, n):
    sub = DevInputs.__new__(DevInputs)
    sub.__dict__.update(d.__dict__)
    sub.X = d.X[:n].contiguous()
    sub.dY = None if d.dY is None else d.dY[:n].contiguous()
    return sub


def _sample_tokens(N, n=40, seed=0):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, 1, N - 1], rng.choice(N, n, replace=False)]))


DW_ROWS_MAX = 70000


def run_workload(name, full=True, wl=None, reduced=None):
    require_lib()
    wl = datagen.WORKLOADS[name] if wl is None else wl
    tol = F32_TOL if wl.dtype == "f32" else BF16_TOL
    b = 4 if wl.dtype == "f32" else 2
    say(f"[{name}] generating inputs")
    inp = datagen.Inputs(wl, progress=say)
    d = DevInputs(inp)

    # ---- reduced batch against the full oracle
    n, c = REDUCED[name] if reduced is None else reduced
    ds = _sub(d, n)
    plan = plan_for(wl, N=n, c=c)
    say(f"[{name}] reduced forward N={n} K={plan.K} c_eff={plan.c_eff}")
    Y, idx, g, lg, st = forward(ds, plan)
    idx_np = idx.cpu().numpy()
    rows = np.arange(n)
    check_routing(inp, lg.cpu().numpy(), idx_np, g.cpu().numpy(), rows=rows)
    X64 = inp.to_f64(inp.X[:n])
    Yref, gref = _oracle_fwd(inp, X64, idx_np)
    err = rel_err(dev_to_f64(Y), Yref)
    say(f"[{name}] reduced Y rel err {err:.3e}")
    assert err <= tol
    assert st["dispatch_bytes"] <= oracle.dispatch_bound_bytes(wl.k, plan.c_eff, wl.H, b)
    # chunked == unchunked, bitwise
    p1 = plan_for(wl, N=n, c=c, K_max=1)
    Y1, idx1, g1, lg1, _ = forward(ds, p1)
    assert torch.equal(lg, lg1) and torch.equal(idx, idx1) and torch.equal(g, g1)
    assert torch.equal(Y.view(torch.int16) if Y.dtype == torch.bfloat16 else Y,
                       Y1.view(torch.int16) if Y1.dtype == torch.bfloat16 else Y1)

    if wl.backward:
        say(f"[{name}] reduced backward")
        out = backward(ds, plan, idx, g)
        ref = oracle.moe_backward(X64, inp.f64("Wr"), inp.expert_f64, None, None,
                                  inp.to_f64(inp.dY[:n]), idx_np, g.cpu().numpy().astype(np.float64))
        for key, rk in (("dX", "dX"), ("dW_gate", "dWg"), ("dW_up", "dWu"), ("dW_down", "dWd"),
                        ("dlogits", "dlogits"), ("dgates", "dgates"), ("dW_r", "dWr")):
            e_ = rel_err(dev_to_f64(out[key]), ref[rk])
            say(f"[{name}]   {key} rel err {e_:.3e}")
            assert e_ <= tol, key
        out1 = backward(ds, p1, idx, g)
        for key in ("dX", "dlogits", "dgates"):
            assert torch.equal(out[key].view(torch.int16) if out[key].dtype == torch.bfloat16
                               else out[key],
                               out1[key].view(torch.int16) if out1[key].dtype == torch.bfloat16
                               else out1[key]), key
        for key in ("dW_gate", "dW_up", "dW_down"):
            dk = rel_err(dev_to_f64(out[key]), dev_to_f64(out1[key]))
            say(f"[{name}]   {key} chunked vs unchunked {dk:.2e}")
            assert dk <= 1e-5
        again = backward(ds, plan, idx, g)
        for key in ("dX", "dW_gate", "dW_up", "dW_down", "dlogits", "dgates", "dW_r"):
            assert torch.equal(again[key], out[key]), key
        del out, out1, again

    if not full or n == wl.N:
        return
    # ---- full batch, sampled tokens
    plan = plan_for(wl)
    say(f"[{name}] full forward N={wl.N} K={plan.K} c_eff={plan.c_eff}")
    Y, idx, g, lg, st = forward(d, plan)
    idx_np = idx.cpu().numpy()
    flips = check_routing(inp, lg.cpu().numpy(), idx_np, g.cpu().numpy())
    say(f"[{name}] routing ok, {flips} tokens flipped within the fp32 bound")
    toks = _sample_tokens(wl.N)
    X64 = inp.to_f64(inp.X[toks])
    l64 = oracle.router_logits(X64, inp.f64("Wr"), inp.bias)
    gt = oracle.gates_from_logits(l64, idx_np[toks])
    Yt = oracle.forward_tokens(X64, idx_np[toks], gt, inp.expert_f64)
    err = rel_err(dev_to_f64(Y[torch.from_numpy(toks).to(DEV)]), Yt)
    say(f"[{name}] full Y rel err on {len(toks)} sampled tokens {err:.3e}")
    assert err <= tol
    # the bf16 forward reads its permuted inputs straight from X (when X fits
    # one buffer resource's 32-bit offsets): one H-wide buffer (the expert
    # outputs) instead of the bound's two
    bound = oracle.dispatch_bound_bytes(wl.k, plan.c_eff, wl.H, b)
    in_place = wl.dtype == "bf16" and wl.N * wl.H * 2 <= 0x7FFFFFF0
    assert st["dispatch_bytes"] == (bound // 2 if in_place else bound)
    Y2, idx2, g2, lg2, _ = forward(d, plan)
    assert torch.equal(Y, Y2) and torch.equal(idx, idx2) and torch.equal(lg, lg2)
    del Y2, idx2, g2, lg2
    p1 = plan_for(wl, K_max=1)
    say(f"[{name}] full forward unchunked")
    Y1, idx1, g1, lg1, st1 = forward(d, p1)
    assert torch.equal(idx, idx1) and torch.equal(g, g1)
    assert torch.equal(Y.view(torch.int16), Y1.view(torch.int16))
    say(f"[{name}] dispatch bytes {st['dispatch_bytes']} (unchunked {st1['dispatch_bytes']})")
    del Y1, idx1, g1, lg1
    torch.cuda.empty_cache()

    if wl.backward:
        say(f"[{name}] full backward")
        out = backward(d, plan, idx, g)
        dYt = inp.to_f64(inp.dY[toks])
        dXt, dgt, dlt = oracle.backward_tokens(X64, dYt, idx_np[toks],
                                               g.cpu().numpy()[toks].astype(np.float64),
                                               inp.expert_f64, inp.f64("Wr"))
        tsel = torch.from_numpy(toks).to(DEV)
        for key, ref in (("dX", dXt), ("dgates", dgt), ("dlogits", dlt)):
            e_ = rel_err(dev_to_f64(out[key][tsel]), ref)
            say(f"[{name}]   sampled {key} rel err {e_:.3e}")
            assert e_ <= tol, key
        gnp = g.cpu().numpy().astype(np.float64)
        counts = np.bincount(idx_np.reshape(-1), minlength=wl.E)
        # the most-routed expert with at most DW_ROWS_MAX rows (the fp64
        # oracle's weight gradients over them take seconds), the least-routed
        # one, and one more
        hot = int(np.argmax(np.where(counts <= DW_ROWS_MAX, counts, -1)))
        for e in sorted({hot, int(np.argmin(counts)), 7 % wl.E}):
            rt, rs = np.nonzero(idx_np == e)
            _, dWg, dWu, dWd, _ = oracle.expert_grads(inp.to_f64(inp.X[rt]), inp.to_f64(inp.dY[rt]),
                                                      gnp[rt, rs], *inp.expert_f64(e))
            for key, ref in (("dW_gate", dWg), ("dW_up", dWu), ("dW_down", dWd)):
                e_ = rel_err(dev_to_f64(out[key][e]), ref)
                say(f"[{name}]   expert {e} ({counts[e]} rows) {key} rel err {e_:.3e}")
                assert e_ <= tol, (key, e)
        p1 = plan_for(wl, K_max=1)
        say(f"[{name}] full backward unchunked")
        out1 = backward(d, p1, idx, g)
        for key in ("dX", "dlogits", "dgates"):
            a, b_ = out[key], out1[key]
            if a.dtype == torch.bfloat16:
                a, b_ = a.view(torch.int16), b_.view(torch.int16)
            assert torch.equal(a, b_), key
        # weight gradients sum over tokens chunk by chunk: their last bits
        # depend on K, but every expert's (not only the sampled ones') must
        # agree with the unchunked run to fp32 rounding.  Two orders of an
        # fp32 sum of n terms differ by about u sqrt(n) of its scale (the
        # random-walk growth of rounding errors); n is the largest expert's
        # row count, and the bound is never below 1e-5
        order_tol = max(1e-5, 2 * 2.0 ** -24 * np.sqrt(counts.max()))
        for key in ("dW_gate", "dW_up", "dW_down", "dW_r"):
            dk = rel_err(dev_to_f64(out[key]), dev_to_f64(out1[key]))
            say(f"[{name}]   {key} chunked vs unchunked {dk:.2e} (bound {order_tol:.2e})")
            assert dk <= order_tol, key
        del out1
        # dW_r = X^T dlogits over the whole batch, against fp64 on the GPU's
        # dlogits (checked above on the sampled tokens): within the oracle
        # tolerance, and elementwise within the rigorous bound of an fp32
        # sum of N rounded products, gamma_{N+1} (|X|^T |dlogits|)
        dl = out["dlogits"].cpu().numpy().astype(np.float64)
        Xf = inp.f64("X")
        dwr_ref = Xf.T @ dl
        mag = np.abs(Xf).T @ np.abs(dl)
        del Xf
        e_ = rel_err(dev_to_f64(out["dW_r"]), dwr_ref)
        say(f"[{name}]   full dW_r rel err vs fp64 X^T dlogits {e_:.3e}")
        assert e_ <= tol
        u = 2.0 ** -24
        gam = (wl.N + 1) * u / (1 - (wl.N + 1) * u)
        assert np.all(np.abs(dev_to_f64(out["dW_r"]) - dwr_ref) <= gam * mag), "dW_r rounding bound"


def test_tiny_f32():
    run_workload("tiny_f32")


def test_balanced_bf16():
    run_workload("balanced_bf16")


def test_many_experts_bf16():
    run_workload("many_experts_bf16")


def test_zipf_bf16():
    run_workload("zipf_bf16")


def test_train_bf16():
    run_workload("train_bf16")


# Chunks whose experts average 96 rows or more take the 256-row GEMM tiles
# (bf16, H and F multiples of 128).  This small case lands there: K = 3 chunks
# of c_eff = 534 tokens, about 267 rows per expert per chunk, so each expert
# has one full 256-row tile and a ragged one whose upper row slices are empty.
LARGE_TILE = datagen.WORKLOADS["train_bf16"].with_(
    name="large_tile_bf16", N=1600, H=256, E=8, k=4, F=384, c=560, K_max=16)


def test_large_row_tile_bf16():
    wl = LARGE_TILE
    plan = plan_for(wl)
    assert plan.K == 3 and plan.c_eff == 534
    assert wl.k * plan.c_eff >= 96 * wl.E and wl.H % 128 == 0 and wl.F % 128 == 0
    run_workload(wl.name, full=False, wl=wl, reduced=(wl.N, wl.c))


# Experts spanning several full 256-row tiles: K = 2 chunks of 1024 tokens
# give about 512 rows per expert per chunk (two or three M-tiles each), and
# the unchunked comparison run about 1024 (four or five).
GROUPED = datagen.WORKLOADS["train_bf16"].with_(
    name="grouped_tiles_bf16", N=2048, H=256, E=8, k=4, F=384, c=1024, K_max=16)


def test_grouped_row_tiles_bf16():
    wl = GROUPED
    plan = plan_for(wl)
    assert plan.K == 2 and plan.c_eff == 1024
    run_workload(wl.name, full=False, wl=wl, reduced=(wl.N, wl.c))


# Chunks averaging ~125 rows per expert take 256-row tiles, and the forward's
# gate/up GEMM then runs the chunk's segments as two lists in one launch:
# segments of at most 128 rows in 128-row tiles, longer ones in 256-row tiles.
# K = 2 chunks of 1000 tokens over 16 experts, top-2: segments straddle 128
# rows, so both lists are populated; the unchunked comparison run (about 250
# rows per expert) is split too, with other segments in each list.
SPLIT_TILES = datagen.WORKLOADS["train_bf16"].with_(
    name="split_tiles_bf16", N=2000, H=256, E=16, k=2, F=256, c=1000, K_max=16)


def test_split_tile_lists_bf16():
    wl = SPLIT_TILES
    plan = plan_for(wl)
    assert plan.K == 2 and plan.c_eff == 1000
    assert wl.k * plan.c_eff >= 96 * wl.E  # 256-row tiles, hence the split lists
    run_workload(wl.name, full=False, wl=wl, reduced=(wl.N, wl.c))


# The down projection of a split plan with H a multiple of 512, whose experts
# average fewer than 512 rows per chunk, runs the short segments in 128 x 512
# tiles beside the long ones' 256-row tiles in one launch when the two lists
# come to 1,024 work-groups or more (the long list's M-tiles times H/256 plus
# the short segments times H/512), and the unsplit 256-row list below that.
# Zipf-routed, H = 4096, top-4 over 64 experts: K = 2 chunks of 3000 tokens
# (F = 256) take the two lists, K = 2 chunks of 2000 tokens (F = 128) the
# unsplit list; both unchunked comparison runs take the two lists.
SPLIT_DOWN = datagen.WORKLOADS["zipf_bf16"].with_(
    name="split_down_bf16", N=6000, H=4096, E=64, k=4, F=256, c=3000, K_max=16)
SPLIT_DOWN_FEW = datagen.WORKLOADS["zipf_bf16"].with_(
    name="split_down_few_bf16", N=4000, H=4096, E=64, k=4, F=128, c=2000, K_max=16)


def _down_work_groups(wl, K):
    """Per chunk, the split down launch's work-groups under the fp64 routing."""
    inp = datagen.Inputs(wl, experts=False)
    idx = oracle.topk_select(inp.to_f64(inp.X) @ inp.f64("Wr") + inp.bias, wl.k)
    out = []
    for i in range(K):
        cnt = np.bincount(idx[i::K].reshape(-1), minlength=wl.E)
        long_tiles = sum(-(-int(c) // 256) for c in cnt if c > 128)
        short = int(np.count_nonzero((cnt > 0) & (cnt <= 128)))
        assert long_tiles > 0 and short > 0
        out.append(long_tiles * (wl.H // 256) + short * (wl.H // 512))
    return out


@pytest.mark.parametrize("wl,split", [(SPLIT_DOWN, True), (SPLIT_DOWN_FEW, False)],
                         ids=["two_lists", "unsplit"])
def test_split_down_projection_bf16(wl, split):
    plan = plan_for(wl)
    assert plan.K == 2 and wl.H % 512 == 0
    assert 96 * wl.E <= wl.k * plan.c_eff < 512 * wl.E
    wgs = _down_work_groups(wl, plan.K)
    say(f"[{wl.name}] split down work-groups per chunk {wgs}")
    # clear of the 1,024 threshold, so that routing flips within the fp32
    # bound cannot move a chunk across it
    assert all((w >= 1100) if split else (w <= 980) for w in wgs)
    run_workload(wl.name, full=False, wl=wl, reduced=(wl.N, wl.c))


# X of 2^31 bytes or more does not fit one buffer resource, so the bf16
# forward gathers the permuted rows into their buffer (two H-wide buffers, the
# whole bound) instead of reading them from X inside the GEMM, and the
# backward gathers the X and dY rows (the recompute, the dh GEMM and the
# weight gradients then read the buffers, not X and dY through perm).
# 524,800 tokens of H = 2048 (X = 2.15 GB), 128 experts under Zipf(1.2)
# routing, top-2, in K = 8 chunks of 65,600 tokens: 256-row tiles with the
# split lists (the coldest experts keep segments of at most 128 rows).
UNFUSED = datagen.WORKLOADS["zipf_bf16"].with_(
    name="unfused_gather_bf16", N=524800, H=2048, E=128, k=2, F=128, c=65600, K_max=8,
    backward=True)


def test_unfused_gather_bf16():
    wl = UNFUSED
    plan = plan_for(wl)
    assert plan.K == 8 and plan.c_eff == 65600
    assert wl.N * wl.H * 2 > 0x7FFFFFF0 and wl.k * plan.c_eff >= 96 * wl.E
    run_workload(wl.name, full=True, wl=wl, reduced=(2000, 500))
