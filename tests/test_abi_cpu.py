"""The C ABI on the host, without a GPU: the library loads and exports every
function the header declares, the structs match the C layout, the chunk plan
matches the oracle's eq. (1), and argument errors come back before anything
is enqueued."""

import ctypes
import os
import subprocess
import tempfile

import numpy as np
import pytest

import oracle
from memory_bounded_expert_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(not os.path.exists(B.LIB_PATH),
                                reason="libmoebound.so not built (run __graft_entry__.build())")


def test_exports_every_declared_function():
    names = B.declared_functions()
    assert set(names) == {"moe_plan_chunks", "moe_plan_set_flags", "moe_bounded_forward",
                          "moe_bounded_forward_static",
                          "moe_bounded_backward",
                          "moe_status_string", "moe_debug_topk", "moe_debug_plan",
                          "moe_debug_stage", "moe_debug_stage_bwd", "cce_plan", "cce_forward",
                          "cce_backward",
                          "cce_debug_stage"}
    L = B.lib()
    for n in names:
        assert hasattr(L, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    assert set(names) <= exported


def test_struct_layout_matches_c():
    src = r"""
#include <stdio.h>
#include <stddef.h>
#include "moebound.h"
#include "cce.h"
#define O(s, f) printf("%s.%s %zu\n", #s, #f, offsetof(s, f));
int main(void) {
  printf("plan %zu\nstats %zu\ncce %zu\n", sizeof(moe_plan_t), sizeof(moe_stats_t),
         sizeof(cce_plan_t));
  O(moe_plan_t, N) O(moe_plan_t, K) O(moe_plan_t, flags) O(moe_plan_t, c_eff)
  O(moe_plan_t, debug_workspace_bytes)
  O(moe_stats_t, c_eff) O(moe_stats_t, workspace_bytes)
  O(cce_plan_t, V) O(cce_plan_t, H) O(cce_plan_t, S) O(cce_plan_t, strip_bound_bytes)
  O(cce_plan_t, bwd_workspace_bytes)
  return 0;
}
"""
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "t.c")
        open(c, "w").write(src)
        exe = os.path.join(d, "t")
        subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                        c, "-o", exe], check=True)
        lines = dict(l.rsplit(" ", 1) for l in subprocess.run([exe], capture_output=True,
                                                              text=True).stdout.splitlines())
    assert int(lines["plan"]) == ctypes.sizeof(B.MoePlan)
    assert int(lines["stats"]) == ctypes.sizeof(B.MoeStats)
    for f in ("N", "K", "flags", "c_eff", "debug_workspace_bytes"):
        assert int(lines[f"moe_plan_t.{f}"]) == getattr(B.MoePlan, f).offset
    for f in ("c_eff", "workspace_bytes"):
        assert int(lines[f"moe_stats_t.{f}"]) == getattr(B.MoeStats, f).offset
    assert int(lines["cce"]) == ctypes.sizeof(B.CcePlan)
    for f in ("V", "H", "S", "strip_bound_bytes", "bwd_workspace_bytes"):
        assert int(lines[f"cce_plan_t.{f}"]) == getattr(B.CcePlan, f).offset


def test_plan_matches_oracle_exhaustively():
    for N in range(0, 200):
        for c in range(1, N + 3, max(1, N // 15)):
            for K_max in (1, 2, 3, 5, 8, 13, 20):
                p = B.moe_plan_chunks(N, 64, 64, 8, 2, c, K_max, B.MOE_F32)
                K, ce = oracle.plan_chunks(N, c, K_max)
                assert (p.K, p.c_eff) == (K, ce), (N, c, K_max)
                assert p.max_pairs_per_chunk == 2 * ce
                assert p.dispatch_bound_bytes == oracle.dispatch_bound_bytes(2, ce, 64, 4)


def test_plan_page_instance_and_workloads():
    p = B.moe_plan_chunks(65536, 7168, 2048, 64, 8, 6554, 10, B.MOE_BF16)
    assert (p.K, p.c_eff) == (10, 6554)
    expect = {  # (N, c, K_max) -> (K, c_eff)
        (256, 64, 8): (4, 64), (4096, 1024, 8): (4, 1024), (16384, 2048, 16): (8, 2048),
        (8192, 1024, 8): (8, 1024), (65536, 4096, 16): (16, 4096),
    }
    for (N, c, K_max), kc in expect.items():
        assert oracle.plan_chunks(N, c, K_max) == kc
        q = B.moe_plan_chunks(N, 2048, 1024, 64, 8, c, K_max, B.MOE_BF16)
        assert (q.K, q.c_eff) == kc


def test_workspace_bounded_by_chunk_not_batch():
    # the H-wide per-chunk buffers scale with c_eff, not N
    a = B.moe_plan_chunks(65536, 2048, 1024, 64, 8, 4096, 16, B.MOE_BF16)
    b = B.moe_plan_chunks(65536, 2048, 1024, 64, 8, 4096, 1, B.MOE_BF16)
    assert a.dispatch_bound_bytes * 16 == b.dispatch_bound_bytes
    assert a.fwd_workspace_bytes < b.fwd_workspace_bytes / 6
    assert a.bwd_workspace_bytes < b.bwd_workspace_bytes / 6
    assert a.dispatch_bound_bytes == 2 * 8 * 4096 * 2048 * 2


@pytest.mark.parametrize("args,status", [
    ((-1, 64, 64, 8, 2, 4, 4, 0), B.MOE_EINVAL),     # N < 0
    ((10, 64, 64, 8, 2, 0, 4, 0), B.MOE_EINVAL),     # c = 0
    ((10, 64, 64, 8, 2, 4, 0, 0), B.MOE_EINVAL),     # K_max = 0
    ((10, 64, 64, 8, 0, 4, 4, 0), B.MOE_EINVAL),     # k = 0
    ((10, 64, 64, 8, 9, 4, 4, 0), B.MOE_EINVAL),     # k > E
    ((10, 64, 64, 8, 2, 4, 4, 7), B.MOE_EINVAL),     # dtype
    ((10, 0, 64, 8, 2, 4, 4, 0), B.MOE_EINVAL),      # H = 0
    ((10, 96, 64, 8, 2, 4, 4, 0), B.MOE_EUNSUPPORTED),   # H % 64
    ((10, 64, 96, 8, 2, 4, 4, 0), B.MOE_EUNSUPPORTED),   # F % 64
    ((10, 64, 64, 12, 2, 4, 4, 1), B.MOE_EUNSUPPORTED),  # E % 8 for bf16
    ((10, 64, 64, 2048, 2, 4, 4, 0), B.MOE_EUNSUPPORTED),  # E > 1024
    ((10, 64, 64, 128, 65, 4, 4, 0), B.MOE_EUNSUPPORTED),  # k > 64
    ((2**28, 64, 64, 16, 8, 4, 4, 0), B.MOE_EUNSUPPORTED),  # N k >= 2^31
])
def test_plan_errors(args, status):
    plan = B.MoePlan()
    assert B.lib().moe_plan_chunks(*args, ctypes.byref(plan)) == status


def test_empty_batch_is_noop():
    p = B.moe_plan_chunks(0, 64, 64, 8, 2, 4, 4, B.MOE_F32)
    assert (p.K, p.c_eff, p.fwd_workspace_bytes, p.dispatch_bound_bytes) == (0, 0, 0, 0)
    st = B.MoeStats()
    assert B.lib().moe_bounded_forward(ctypes.byref(p), *([None] * 10), None, 0, None,
                                       ctypes.byref(st)) == B.MOE_OK
    assert st.K == 0 and st.launches == 0


def test_forward_argument_errors_before_any_launch():
    L = B.lib()
    p = B.moe_plan_chunks(256, 64, 128, 8, 2, 64, 8, B.MOE_F32)
    fake = ctypes.c_void_p(0x100000)  # never dereferenced: every check below fails first
    ptrs = [fake] * 10
    # a plan that did not come from moe_plan_chunks
    bad = B.MoePlan()
    assert L.moe_bounded_forward(ctypes.byref(bad), *ptrs, fake, 1 << 30, None, None) == B.MOE_EINVAL
    # a required pointer missing
    miss = list(ptrs)
    miss[0] = None
    assert L.moe_bounded_forward(ctypes.byref(p), *miss, fake, 1 << 30, None, None) == B.MOE_EINVAL
    # misaligned workspace
    assert L.moe_bounded_forward(ctypes.byref(p), *ptrs, ctypes.c_void_p(0x100010), 1 << 30, None,
                                 None) == B.MOE_EINVAL
    # workspace one byte short
    assert L.moe_bounded_forward(ctypes.byref(p), *ptrs, fake, p.fwd_workspace_bytes - 1, None,
                                 None) == B.MOE_EWORKSPACE
    bptrs = [fake] * 15
    assert L.moe_bounded_backward(ctypes.byref(p), *bptrs, fake, p.bwd_workspace_bytes - 1, None,
                                  None) == B.MOE_EWORKSPACE
    assert L.moe_debug_plan(ctypes.byref(p), fake, fake, fake, fake, fake,
                            p.debug_workspace_bytes - 1, None) == B.MOE_EWORKSPACE
    assert L.moe_debug_stage(ctypes.byref(p), 4, 0, *ptrs[:9], fake, p.fwd_workspace_bytes - 1,
                             None) == B.MOE_EWORKSPACE
    assert L.moe_debug_stage(ctypes.byref(p), 9, 0, *ptrs[:9], fake, 1 << 30, None) == B.MOE_EINVAL
    assert L.moe_debug_stage(ctypes.byref(p), 4, p.K, *ptrs[:9], fake, 1 << 30, None) == B.MOE_EINVAL
    assert L.moe_debug_topk(fake, 4, 8, 9, fake, fake, None) == B.MOE_EINVAL
    assert L.moe_debug_topk(fake, 4, 2048, 9, fake, fake, None) == B.MOE_EUNSUPPORTED
    sb = [fake] * 15
    assert L.moe_debug_stage_bwd(ctypes.byref(p), 5, 0, *sb, fake, p.bwd_workspace_bytes - 1,
                                 None) == B.MOE_EWORKSPACE
    assert L.moe_debug_stage_bwd(ctypes.byref(p), 10, 0, *sb, fake, 1 << 30, None) == B.MOE_EINVAL
    assert L.moe_debug_stage_bwd(ctypes.byref(p), 5, p.K, *sb, fake, 1 << 30, None) == B.MOE_EINVAL
    assert L.moe_debug_stage_bwd(ctypes.byref(bad), 5, 0, *sb, fake, 1 << 30, None) == B.MOE_EINVAL
    sm = list(sb)
    sm[5] = None  # dY
    assert L.moe_debug_stage_bwd(ctypes.byref(p), 5, 0, *sm, fake, 1 << 30, None) == B.MOE_EINVAL



def test_bf16_forward_reads_permuted_inputs_in_place():
    """The bf16 forward's gate/up GEMM reads each permuted input row straight
    from X: its workspace holds one H-wide per-chunk buffer (the expert
    outputs) and the debug GATHER stage reports that no gather kernel exists,
    before any launch.  The bf16 backward reads them from X as well (the
    recompute and the gate/up weight gradient): one H-wide buffer (dY rows,
    then dXp) besides its three F-wide ones."""
    L = B.lib()
    N, H, F, E, k, c, K_max = 4096, 2048, 1408, 64, 8, 1024, 8
    p = B.moe_plan_chunks(N, H, F, E, k, c, K_max, B.MOE_BF16)
    rows = k * p.c_eff
    hbuf, fbuf = rows * H * 2, rows * F * 2
    assert hbuf + fbuf <= p.fwd_workspace_bytes < 2 * hbuf + fbuf
    assert hbuf + 3 * fbuf <= p.bwd_workspace_bytes < 2 * hbuf + 3 * fbuf
    fake = ctypes.c_void_p(0x100000)  # never dereferenced
    assert L.moe_debug_stage(ctypes.byref(p), 3, 0, *([fake] * 9), fake, p.fwd_workspace_bytes,
                             None) == B.MOE_EUNSUPPORTED
    # fp32 keeps the explicit gather and both buffers
    q = B.moe_plan_chunks(256, 64, 128, 8, 2, 64, 8, B.MOE_F32)
    assert q.fwd_workspace_bytes >= 2 * 2 * q.c_eff * 64 * 4
    assert q.bwd_workspace_bytes >= 2 * 2 * q.c_eff * 64 * 4


def test_bf16_backward_reads_in_place_within_the_division_guard():
    """The bf16 backward reads its permuted rows of X and dY through perm and
    divides each pair index by k with a multiply-shift, exact while N k^2 <
    2^32.  One token more than that bound and the backward keeps the
    gathered permuted-input buffer (k c_eff H b bytes more workspace);
    everything else in the layout changes by a few pair-indexed words."""
    H, F, E, k, c = 64, 64, 64, 64, 1024
    n_max = (1 << 32) // (k * k)  # first N with N k^2 >= 2^32
    K_max = n_max // c
    a = B.moe_plan_chunks(n_max - 1, H, F, E, k, c, K_max, B.MOE_BF16)
    b = B.moe_plan_chunks(n_max, H, F, E, k, c, K_max, B.MOE_BF16)
    assert a.c_eff == b.c_eff == c
    hbuf = k * c * H * 2
    assert hbuf <= b.bwd_workspace_bytes - a.bwd_workspace_bytes <= hbuf + 8 * 256
    # the forward's in-place read has no such guard
    assert abs(b.fwd_workspace_bytes - a.fwd_workspace_bytes) <= 8 * 256


@pytest.mark.parametrize("k", list(range(1, 65)))
def test_pair_index_division_by_multiply_shift(k):
    """floor(n / k) = mulhi(n, ceil(2^32 / k)) for every pair index n < x_rows
    k when x_rows k^2 < 2^32 (k = 1 passes n through): the identity the
    row-indexed GEMM loads use, checked at the guard's largest x_rows, on
    both sides of every multiple of k near the top and at random indices."""
    m = 0 if k == 1 else -(-(1 << 32) // k)
    x_rows = ((1 << 32) - 1) // (k * k)
    top = x_rows * k
    rng = np.random.default_rng(k)
    ns = set(range(max(0, top - 4 * k - 3), top))
    ns.update(int(v) for v in rng.integers(0, top, 2000))
    for q in range(1, 200):
        for d in (-1, 0, 1):
            ns.add(min(top - 1, max(0, q * k + d)))
    for n in ns:
        got = n if m == 0 else (n * m) >> 32
        assert got == n // k, (k, n)


def test_status_strings():
    for s in range(0, 6):
        assert isinstance(B.status_string(s), str) and B.status_string(s)


# ---- vocabulary-strip cross-entropy: plan and argument checks (host only)


def test_cce_plan_strips_and_bounds():
    for N, H, V, vc in ((8192, 7168, 200_000, 8192), (777, 512, 20_000, 4096), (1, 128, 1, 256),
                        (5, 256, 300, 256), (3, 128, 1000, 1024)):
        p = B.cce_plan(N, H, V, vc)
        assert p.S == len(oracle.ce_strips(V, vc))
        assert p.strip_bound_bytes == oracle.strip_bound_bytes(N, vc, V, 2)
        assert p.unchunked_logit_bytes == N * V * 4
        # forward workspace: one strip's slice statistics and the running
        # state, O(N v_chunk / 128); backward: the bf16 strip and dX's fp32 sum
        # (strip buffers are whole 256-column tiles wide)
        cols = min(vc, -(-V // 256) * 256)
        assert p.fwd_workspace_bytes <= 8 * N * cols // 128 + 3 * 4 * N + 5 * 256
        assert p.bwd_workspace_bytes <= 2 * N * cols + 4 * N * H + 4 * N + 4 * 256
        assert 2 * N * cols - p.strip_bound_bytes < 2 * N * 256
    assert B.cce_plan(0, 128, 10, 256).S == 0


@pytest.mark.parametrize("args,status", [
    ((-1, 128, 10, 256, 1), B.MOE_EINVAL),
    ((4, 0, 10, 256, 1), B.MOE_EINVAL),
    ((4, 128, 0, 256, 1), B.MOE_EINVAL),
    ((4, 128, 10, 0, 1), B.MOE_EINVAL),
    ((4, 128, 10, 256, 7), B.MOE_EINVAL),
    ((4, 128, 10, 256, 0), B.MOE_EUNSUPPORTED),     # fp32
    ((4, 192, 10, 256, 1), B.MOE_EUNSUPPORTED),     # H % 128
    ((4, 128, 10, 384, 1), B.MOE_EUNSUPPORTED),     # v_chunk % 256
    ((2**21, 512, 10, 256, 1), B.MOE_EUNSUPPORTED),  # N H >= 2^30
    ((8, 128, 10, 2**23, 1), B.MOE_EUNSUPPORTED),   # v_chunk H >= 2^30
])
def test_cce_plan_errors(args, status):
    plan = B.CcePlan()
    assert B.lib().cce_plan(*args, ctypes.byref(plan)) == status


def test_cce_argument_errors_before_any_launch():
    L = B.lib()
    p = B.cce_plan(300, 256, 5000, 1024)
    fake = ctypes.c_void_p(0x100000)  # never dereferenced: every check below fails first
    bad = B.CcePlan()
    assert L.cce_forward(ctypes.byref(bad), *[fake] * 5, fake, 1 << 30, None) == B.MOE_EINVAL
    assert L.cce_forward(ctypes.byref(p), None, *[fake] * 4, fake, 1 << 30, None) == B.MOE_EINVAL
    assert L.cce_forward(ctypes.byref(p), *[fake] * 5, ctypes.c_void_p(0x100010), 1 << 30,
                         None) == B.MOE_EINVAL
    assert L.cce_forward(ctypes.byref(p), *[fake] * 5, fake, p.fwd_workspace_bytes - 1,
                         None) == B.MOE_EWORKSPACE
    assert L.cce_backward(ctypes.byref(p), *[fake] * 7, fake, p.bwd_workspace_bytes - 1,
                          None) == B.MOE_EWORKSPACE
    assert L.cce_backward(ctypes.byref(p), *[fake] * 6, None, fake, 1 << 30, None) == B.MOE_EINVAL
    assert L.cce_debug_stage(ctypes.byref(p), 5, 0, *[fake] * 8, fake, 1 << 30, None) == B.MOE_EINVAL
    assert L.cce_debug_stage(ctypes.byref(p), 0, p.S, *[fake] * 8, fake, 1 << 30, None) == B.MOE_EINVAL
    assert L.cce_debug_stage(ctypes.byref(p), 3, 0, *[fake] * 8, fake, p.bwd_workspace_bytes - 1,
                             None) == B.MOE_EWORKSPACE
    # no tokens: forward is a no-op; backward still needs dW (it zeroes it)
    p0 = B.cce_plan(0, 256, 5000, 1024)
    assert L.cce_forward(ctypes.byref(p0), *[None] * 5, None, 0, None) == B.MOE_OK
    assert L.cce_backward(ctypes.byref(p0), *[None] * 7, None, 0, None) == B.MOE_EINVAL


def test_binding_argument_counts_match_the_headers():
    """Every declared function's parameter count equals the number of
    argument types the ctypes binding gives it (a miscount would pass
    pointers in the wrong positions)."""
    import re

    L = B.lib()
    for h in B.HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        for m in re.finditer(r"\b((?:moe|cce)_[a-z_]+)\s*\(([^;{]*?)\)\s*;", text, flags=re.S):
            name, params = m.group(1), m.group(2).strip()
            n = 0 if params in ("", "void") else params.count(",") + 1
            assert len(getattr(L, name).argtypes) == n, (name, n)


def test_static_forward_errors_before_any_launch():
    """The static-scratch forward rejects a plan whose forward layout exceeds
    MOE_STATIC_SCRATCH_BYTES, and bad arguments, on the host before it asks
    for the scratch array's address or enqueues anything."""
    import re

    L = B.lib()
    text = open(os.path.join(B.INCLUDE, "moebound.h")).read()
    m = re.search(r"#define MOE_STATIC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    cap = int(m.group(1)) << int(m.group(2))
    assert cap == 64 << 20
    fake = ctypes.c_void_p(0x100000)  # never dereferenced
    ptrs = [fake] * 10
    big = B.moe_plan_chunks(65536, 2048, 1024, 64, 8, 4096, 16, B.MOE_BF16)
    assert big.fwd_workspace_bytes > cap
    assert L.moe_bounded_forward_static(ctypes.byref(big), *ptrs, None, None) == B.MOE_EWORKSPACE
    bad = B.MoePlan()
    assert L.moe_bounded_forward_static(ctypes.byref(bad), *ptrs, None, None) == B.MOE_EINVAL
    p = B.moe_plan_chunks(4096, 2048, 1408, 64, 8, 1024, 8, B.MOE_BF16)
    assert p.fwd_workspace_bytes <= cap  # the balanced 4096-token forward fits
    miss = list(ptrs)
    miss[3] = None  # W_gate
    assert L.moe_bounded_forward_static(ctypes.byref(p), *miss, None, None) == B.MOE_EINVAL


def test_plan_set_flags():
    """MOE_PLAN_EXACT_DW: accepted for bf16 plans whose X and dY are read in
    place and c_eff <= 65536 (the backward workspace grows by the column
    maxima, the digit planes and the high words of the accumulators);
    refused otherwise, leaving the plan unchanged."""
    N, H, F, E, k = 65536, 2048, 1024, 64, 8
    p = B.moe_plan_chunks(N, H, F, E, k, 4096, 16, B.MOE_BF16)
    base = p.bwd_workspace_bytes
    B.moe_plan_set_flags(p, B.MOE_PLAN_EXACT_DW)
    assert p.flags == B.MOE_PLAN_EXACT_DW
    ldk = -(-(k * p.c_eff + 64 * E) // 64) * 64
    extra = p.bwd_workspace_bytes - base
    need = (2 * H + 3 * E * F) * 4 + (E + 1) * 4 + 2 * (2 * H + 3 * F) * ldk + 3 * E * H * F * 4
    assert need <= extra <= need + 4 * 256
    B.moe_plan_set_flags(p, 0)
    assert p.flags == 0 and p.bwd_workspace_bytes == base
    # refusals: unknown flag, fp32, c_eff above 65536, a plan not from moe_plan_chunks
    with pytest.raises(B.MoeError) as e1:
        B.moe_plan_set_flags(p, 2)
    assert e1.value.status == B.MOE_EINVAL
    f32 = B.moe_plan_chunks(256, 64, 128, 8, 2, 64, 8, B.MOE_F32)
    with pytest.raises(B.MoeError) as e2:
        B.moe_plan_set_flags(f32, B.MOE_PLAN_EXACT_DW)
    assert e2.value.status == B.MOE_EUNSUPPORTED and f32.flags == 0
    wide = B.moe_plan_chunks(70000, 256, 256, 8, 2, 70000, 1, B.MOE_BF16)
    with pytest.raises(B.MoeError) as e3:
        B.moe_plan_set_flags(wide, B.MOE_PLAN_EXACT_DW)
    assert e3.value.status == B.MOE_EUNSUPPORTED
    with pytest.raises(B.MoeError) as e4:
        B.moe_plan_set_flags(B.MoePlan(), B.MOE_PLAN_EXACT_DW)
    assert e4.value.status == B.MOE_EINVAL
    # the backward's debug stages do not serve such plans
    B.moe_plan_set_flags(p, B.MOE_PLAN_EXACT_DW)
    fake = ctypes.c_void_p(0x100000)
    assert B.lib().moe_debug_stage_bwd(ctypes.byref(p), 5, 0, *[fake] * 15, fake, 1 << 40,
                                       None) == B.MOE_EUNSUPPORTED
