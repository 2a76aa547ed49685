"""The static-scratch forward (moe_bounded_forward_static, for callers that
cannot allocate) against the workspace forward, through the C ABI: the same
kernels run, so every output must be bitwise equal.  Two calls in a row on
the shared scratch array, the second with a smaller batch (the array then
holds the first call's contents), and a third back at the first size."""

import numpy as np
import pytest
import torch

import datagen
from gpu_common import B, DEV, DevInputs, needs_gpu, plan_for, require_lib, say

pytestmark = [pytest.mark.gpu, needs_gpu]


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


def _check(d, plan, label):
    say(f"no-alloc forward {label}: N={plan.N} K={plan.K}")
    ref = B.moe_bounded_forward(plan, d.X, d.Wr, d.bias, d.Wg, d.Wu, d.Wd)
    got = B.moe_bounded_forward_static(plan, d.X, d.Wr, d.bias, d.Wg, d.Wu, d.Wd)
    torch.cuda.synchronize()
    for name, a, b in zip(("Y", "topk_idx", "gates", "logits"), got[:4], ref[:4]):
        assert torch.equal(_bits(a), _bits(b)), (label, name)
    assert got[4]["launches"] == ref[4]["launches"]
    # logits left to the scratch array: the routing and output are unchanged
    got2 = B.moe_bounded_forward_static(plan, d.X, d.Wr, d.bias, d.Wg, d.Wu, d.Wd,
                                        want_logits=False)
    torch.cuda.synchronize()
    for name, a, b in zip(("Y", "topk_idx", "gates"), got2[:3], ref[:3]):
        assert torch.equal(_bits(a), _bits(b)), (label, "no logits", name)


def _sub(d, n):
    s = DevInputs.__new__(DevInputs)
    s.__dict__.update(d.__dict__)
    s.X = d.X[:n].contiguous()
    return s


@pytest.mark.parametrize("name,sizes", [
    ("balanced_bf16", [(4096, 1024), (1003, 251), (4096, 1024)]),
    ("tiny_f32", [(256, 64), (77, 20)]),
])
def test_static_forward_matches_workspace_forward(name, sizes):
    require_lib()
    wl = datagen.WORKLOADS[name]
    inp = datagen.Inputs(wl, N=max(n for n, _ in sizes), progress=say)
    d = DevInputs(inp)
    for n, c in sizes:
        plan = plan_for(wl, N=n, c=c)
        assert plan.fwd_workspace_bytes <= 64 << 20
        _check(_sub(d, n), plan, f"{name} N={n}")


def test_static_forward_rejects_a_plan_over_the_scratch_size():
    require_lib()
    wl = datagen.WORKLOADS["train_bf16"]
    plan = plan_for(wl)
    assert plan.fwd_workspace_bytes > 64 << 20
    x = torch.empty(1, device=DEV)  # never read: the call returns before any launch
    with pytest.raises(B.MoeError) as err:
        B.lib()  # loaded
        st = B.MoeStats()
        status = B.lib().moe_bounded_forward_static(
            B.ctypes.byref(plan), *[B._vp(x.data_ptr())] * 10, None, B.ctypes.byref(st))
        B._check(status, "moe_bounded_forward_static")
    assert err.value.status == B.MOE_EWORKSPACE
