"""Order-invariant expert weight gradients (plan flag MOE_PLAN_EXACT_DW) on the
GPU, through the C ABI.

The pages require the chunked run to reach exactly the unchunked values and
gradients ("Bounded-streaming operators" summary: Summary, "Core principle";
Design Requirements 1-2).  With the flag, dW_gate, dW_up and dW_down must be
bitwise identical for K = 16, 7 and 1 on the same batch, and within the bf16
tolerance of the fp64 oracle; the other outputs are those of the default
backward, bitwise.
"""

import numpy as np
import pytest
import torch

import datagen
import oracle
from gpu_common import (BF16_TOL, B, DevInputs, dev_to_f64, needs_gpu, plan_for, rel_err,
                        require_lib, say)

pytestmark = [pytest.mark.gpu, needs_gpu]

DW = ("dW_gate", "dW_up", "dW_down")


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


def _run(wl, n, plans):
    """Forward once (routing), then the default and the order-invariant
    backward for each (c, K_max); returns the routing, the outputs and the
    oracle's gradients."""
    inp = datagen.Inputs(wl, N=n, dy=True, progress=say)
    d = DevInputs(inp)
    base = plan_for(wl, N=n, c=plans[0][0], K_max=plans[0][1])
    _, idx, g, _, _ = B.moe_bounded_forward(base, d.X, d.Wr, d.bias, d.Wg, d.Wu, d.Wd)
    outs = []
    for c, kmax in plans:
        p = plan_for(wl, N=n, c=c, K_max=kmax)
        ref = B.moe_bounded_backward(p, d.X, d.Wr, d.Wg, d.Wu, d.Wd, d.dY, idx, g)
        B.moe_plan_set_flags(p, B.MOE_PLAN_EXACT_DW)
        say(f"[{wl.name}] exact dW backward N={n} K={p.K} c_eff={p.c_eff}")
        ex = B.moe_bounded_backward(p, d.X, d.Wr, d.Wg, d.Wu, d.Wd, d.dY, idx, g)
        torch.cuda.synchronize()
        outs.append((p.K, ref, ex))
    idx_np = idx.cpu().numpy()
    orc = oracle.moe_backward(inp.f64("X"), inp.f64("Wr"), inp.expert_f64, None, None,
                              inp.f64("dY"), idx_np, g.cpu().numpy().astype(np.float64))
    return idx_np, outs, orc


def _check(wl, n, plans):
    require_lib()
    idx_np, outs, orc = _run(wl, n, plans)
    K0, ref0, ex0 = outs[0]
    for K, ref, ex in outs:
        # the other outputs are the default backward's, bitwise
        for key in ("dX", "dlogits", "dgates", "dW_r"):
            assert torch.equal(_bits(ex[key]), _bits(ref[key])), (K, key)
        for key, rk in zip(DW, ("dWg", "dWu", "dWd")):
            # order-invariant: bitwise the same for every chunking
            assert torch.equal(ex[key], ex0[key]), (K, K0, key)
            e_ = rel_err(dev_to_f64(ex[key]), orc[rk])
            d_ = rel_err(dev_to_f64(ex[key]), dev_to_f64(ref[key]))
            say(f"[{wl.name}]   K={K} {key}: rel err vs oracle {e_:.2e}, vs the default "
                f"(fp32-sum) path {d_:.2e}")
            assert e_ <= BF16_TOL, (K, key)
    # experts without rows have exactly zero weight gradients
    counts = np.bincount(idx_np.reshape(-1), minlength=wl.E)
    for e in np.nonzero(counts == 0)[0]:
        for key in DW:
            assert not torch.any(ex0[key][int(e)]), (int(e), key)
    return counts


def test_exact_dw_reduced_training_shape():
    """The 65,536-token training layer's shape (H 2048, 64 experts, top-8,
    F 1024) on 2000 tokens: c = 125 gives K = 16, K_max = 7 gives K = 7,
    K_max = 1 the unchunked run."""
    wl = datagen.WORKLOADS["train_bf16"]
    _check(wl, 2000, [(125, 16), (125, 7), (125, 1)])


def test_exact_dw_skewed_with_empty_experts():
    """Zipf-skewed routing over 16 experts, top-2, 300 tokens: hot experts
    span several 64-row segments, some experts get no rows in some chunks (or
    at all); K = 8, 3 and 1."""
    wl = datagen.WORKLOADS["zipf_bf16"].with_(name="zipf_small_bf16", N=300, H=256, E=16, k=2,
                                              F=256, c=38, K_max=16, zipf_s=2.0)
    counts = _check(wl, 300, [(38, 16), (38, 3), (38, 1)])
    say(f"[zipf_small_bf16] rows per expert {counts.tolist()}")
