"""Shared helpers of the GPU parity tests: device copies of the seeded inputs,
calls through the C ABI, and the comparisons against the fp64 oracle."""

from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import datagen
import oracle
from memory_bounded_expert_amd import binding as B

HAVE_GPU = torch.cuda.is_available()
DEV = torch.device("cuda:0") if HAVE_GPU else None

BF16_TOL = 1e-2
F32_TOL = 1e-5


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def require_lib():
    B.lib()  # raises if the HIP library is missing: no fallback exists


def dtype_of(wl):
    return B.MOE_BF16 if wl.dtype == "bf16" else B.MOE_F32


def to_dev(a, wl):
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def dev_to_f64(t):
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


class DevInputs:
    def __init__(self, inp: datagen.Inputs):
        wl = inp.wl
        self.inp = inp
        self.X = to_dev(inp.X, wl)
        self.Wr = to_dev(inp.Wr, wl)
        self.bias = None if inp.bias is None else torch.from_numpy(inp.bias).to(DEV)
        self.Wg = to_dev(inp.Wg, wl)
        self.Wu = to_dev(inp.Wu, wl)
        self.Wd = to_dev(inp.Wd, wl)
        self.dY = to_dev(inp.dY, wl)


def plan_for(wl, N=None, c=None, K_max=None):
    return B.moe_plan_chunks(wl.N if N is None else N, wl.H, wl.F, wl.E, wl.k,
                             wl.c if c is None else c, wl.K_max if K_max is None else K_max,
                             dtype_of(wl))


def forward(d: DevInputs, plan):
    Y, idx, g, lg, st = B.moe_bounded_forward(plan, d.X, d.Wr, d.bias, d.Wg, d.Wu, d.Wd)
    torch.cuda.synchronize()
    return Y, idx, g, lg, st


def backward(d: DevInputs, plan, idx, gates):
    out = B.moe_bounded_backward(plan, d.X, d.Wr, d.Wg, d.Wu, d.Wd, d.dY, idx, gates)
    torch.cuda.synchronize()
    return out


def rel_err(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(got - ref)) / (den if den > 0 else 1.0))


def check_routing(inp, lg_gpu, idx_gpu, g_gpu, rows=None):
    """Routing contract: the GPU's top-k equals the oracle's top-k of the GPU's
    own fp32 logits bit for bit; gates match to fp32 rounding; logits match
    the fp64 oracle to the fp32 summation bound; and any flip against the
    oracle's own fp64 routing sits inside that bound.  Returns #flips."""
    X = inp.f64("X") if rows is None else inp.to_f64(inp.X[rows])
    Wr = inp.f64("Wr")
    l64 = oracle.router_logits(X, Wr, inp.bias)
    lg = lg_gpu.astype(np.float64)
    tau = oracle.logit_error_bound(X, Wr, inp.bias)
    assert np.all(np.abs(lg - l64).max(1) <= tau / 2), "router logits outside the fp32 bound"
    k = idx_gpu.shape[1]
    ref_idx = oracle.topk_select(lg, k)
    assert np.array_equal(idx_gpu.astype(np.int64), ref_idx), "top-k differs from oracle on GPU logits"
    ref_g = oracle.gates_from_logits(lg, ref_idx)
    assert np.max(np.abs(g_gpu - ref_g)) <= 2e-6, "gates"
    own = oracle.topk_select(l64, k)
    diff = np.nonzero(np.any(own != ref_idx, axis=1))[0]
    for t in diff:
        for j in np.nonzero(own[t] != ref_idx[t])[0]:
            gap = abs(l64[t, own[t, j]] - l64[t, ref_idx[t, j]])
            assert gap <= tau[t], f"flip at token {t} slot {j}: gap {gap} > tau {tau[t]}"
    return len(diff)


needs_gpu = pytest.mark.skipif(not HAVE_GPU, reason="needs a GPU")
