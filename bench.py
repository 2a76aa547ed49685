#!/usr/bin/env python3
"""Benchmark of the memory-bounded MoE layer on one MI355X.

One step = one pass of the layer's whole hot path over one batch of synthetic
inputs that are resident in HBM before the timed region starts.  For a
forward+backward workload (the default, `train_bf16`) that is the forward --
router GEMM, top-k and gates, chunk plan, and per chunk the gate/up grouped
GEMM with SwiGLU (the permute folded into its operand loads), the down grouped
GEMM with the gate scaling, the combine -- followed by the backward with
per-chunk recompute (dX, dW_gate/up/down, dlogits, dgates, dW_r).  Forward-only
workloads time the forward alone.

Default workload: 65,536 tokens, H=2048, 64 experts, top-8, F=1024 SwiGLU,
c=4096, K_max=16 (K = 16 chunks), bf16 with fp32 accumulation, upstream
gradient dY ~ N(0, 1).  Prints one JSON line on stdout (everything else goes
to stderr):
  value = routed token-expert pairs per second (N*k / time per step),
  roofline = the forward gate/up grouped GEMM against its roof (bf16 MFMA
             when its arithmetic intensity is above the ridge, else HBM), from
             HIP events around re-launches of that kernel on the layer's stream,
  grouped_gemm = MFMA utilisation of the forward grouped GEMMs,
  cpu_baseline = the fp64 oracle (forward, and backward for a forward+backward
             workload) on a bounded token sample of the same workload.

--workload vocab_bf16 (or vocab_small_bf16) benchmarks the vocabulary
projection with cross-entropy over vocabulary strips instead: one step = the
forward (per-token loss and log-normaliser) and backward (dX, dW) of 8192
tokens over H=7168, V=200,000 in strips of 8192 entries; value = tokens/s.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
FP32_PEAK_TFLOPS = 157.3


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or "unknown"."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# Sources that decide what the forward GEMM kernels do and how they are
# launched; a traffic record taken with other sources is not used.
GEMM_SOURCES = ("gemm_lds.hpp", "gemm_kernel.hpp", "gemm_fwd.hip", "device_common.hpp",
                "moe_internal.h", "plan.hip", "api.hip")


def gemm_sources_sha256():
    import hashlib
    h = hashlib.sha256()
    for name in GEMM_SOURCES:
        with open(os.path.join(ROOT, "memory_bounded_expert_amd", "csrc", name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def measured_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` from the rocprofv3 FETCH_SIZE and
    WRITE_SIZE passes summarised under profiles/ (each scaled by what the same
    counter reads for a plain device copy of known size), or None when no
    summary covers the current GEMM sources."""
    d = os.path.join(ROOT, "profiles")
    if not os.path.isdir(d):
        return None
    sha = gemm_sources_sha256()
    for name in sorted(os.listdir(d)):
        if not name.endswith(".md"):
            continue
        with open(os.path.join(d, name)) as f:
            for line in f:
                if not line.startswith("traffic-record: "):
                    continue
                r = json.loads(line[len("traffic-record: "):])
                if r["workload"] == workload and r["kernel"] == kernel and r["sources_sha256"] == sha:
                    return int(1024 * (r["fetch_kib_per_dispatch"] * r["fetch_scale"] +
                                       r["write_kib_per_dispatch"] * r["write_scale"]))
    return None


def stage_work(stage, wl, b, n_i, R_i, E_i):
    """Algorithmic (bytes, flops) of one launch of a stage on a chunk with n_i
    tokens, R_i routed pairs and E_i non-empty experts."""
    H, F = wl.H, wl.F
    if stage == "gemm_up":
        return (2 * E_i * H * F * b + R_i * H * b + R_i * F * b), 4.0 * R_i * H * F
    if stage == "gemm_down":  # (plus each row's pair index and gate)
        return (E_i * F * H * b + R_i * F * b + R_i * H * b + R_i * 8), 2.0 * R_i * H * F
    if stage == "gather":  # read each token once, write its k rows
        return (n_i + R_i) * H * b, 0.0
    if stage == "combine":  # read the k gate-scaled rows and their positions, write the token
        return (R_i + n_i) * H * b + R_i * 4, 1.0 * R_i * H
    raise KeyError(stage)


def fused_recompute_dh(wl, c_eff):
    """Whether the library runs a chunk's recompute inside its dh kernel: bf16
    with the 256-row tiles (experts averaging at least 96 rows per chunk, H and
    F multiples of 128)."""
    return (wl.dtype == "bf16" and wl.H % 128 == 0 and wl.F % 128 == 0
            and wl.k * c_eff >= 96 * wl.E)


def bwd_stage_work(stage, wl, b, n_i, R_i, E_i, first, fused=False):
    """Algorithmic (bytes, flops) of one launch of a per-chunk backward stage
    on a chunk with n_i tokens, R_i routed pairs and E_i non-empty experts
    (first: chunk 0, whose weight-gradient products store dW instead of
    reading and writing it; fused: the recompute runs inside the dh stage,
    whose a, u and h then never leave the kernel)."""
    H, F, E = wl.H, wl.F, wl.E
    shares = (F // 128 if F % 128 == 0 else F // 64) * R_i * 4  # dgate shares
    if stage == "recompute":  # weights, X rows; a, u, h out
        if fused:
            return 0, 0.0
        return 2 * E_i * H * F * b + R_i * H * b + 3 * R_i * F * b, 4.0 * R_i * H * F
    if stage == "dh":  # W_down, dY rows, a/u/h in, da/du/gh out, gates and dgate shares
        if fused:  # + W_gate, W_up and X rows; a, u, h stay on chip
            return (3 * E_i * F * H * b + 2 * R_i * H * b + 3 * R_i * F * b + R_i * 8
                    + shares), 6.0 * R_i * H * F
        return (E_i * F * H * b + R_i * H * b + 6 * R_i * F * b + R_i * 8 + shares,
                2.0 * R_i * H * F)
    if stage == "wgrad_down":  # g h, dY rows in; fp32 dW_down read + written (chunk 0: written)
        dw = E * F * H * 4 if first else 2 * E_i * F * H * 4
        return R_i * F * b + R_i * H * b + R_i * 4 + dw, 2.0 * R_i * H * F
    if stage == "wgrad_gate_up":  # X rows, da, du in; fp32 dW_gate, dW_up read + written
        dw = 2 * E * H * F * 4 if first else 4 * E_i * H * F * 4
        return R_i * H * b + 2 * R_i * F * b + R_i * 4 + dw, 4.0 * R_i * H * F
    if stage == "dx":  # da, du, W_gate, W_up in; dXp out
        return 2 * R_i * F * b + 2 * E_i * H * F * b + R_i * H * b, 4.0 * R_i * H * F
    if stage == "combine_bwd":  # dXp rows in, dX and dlogits rows out, router path
        return (R_i + n_i) * H * b + n_i * E * 4 + E * H * b + R_i * 12, 2.0 * n_i * wl.k * H
    if stage == "dwr":  # X rows and dlogits of the chunk's tokens; dW_r read + written
        return n_i * H * b + n_i * E * 4 + R_i * 4 + 2 * H * E * 4, 2.0 * R_i * H
    raise KeyError(stage)


def roof_of(byts, flops, us, peak_tf):
    """The stage's roof (bf16 MFMA when its intensity is above the ridge, else
    HBM) and its achieved fraction of it."""
    if flops and flops / byts * 1e-3 * HBM_PEAK_GBS > peak_tf:
        tf = flops / us / 1e6
        return {"bound": "mfma", "achieved": round(tf, 1), "peak": peak_tf, "unit": "TFLOP/s",
                "frac": round(tf / peak_tf, 4)}
    gbs = byts / us / 1e3
    return {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4)}


def cce_stage_work(stage, N, H, w):
    """Algorithmic (bytes, flops) of one launch of a vocabulary-strip
    cross-entropy stage on a strip of w vocabulary entries (bf16 X, W and
    logit gradient; fp32 statistics, dX running sum and dW)."""
    gemm = 2.0 * N * H * w
    x, ws, g = N * H * 2, w * H * 2, N * w * 2
    if stage == "logits":  # X, the strip of W, slice statistics out
        return x + ws + N * (w // 128) * 8 + N * 4, gemm
    if stage == "fold":  # slice statistics in, running state
        return N * (w // 128) * 8 + N * 16, 0.0
    if stage == "grad":  # X, the strip of W, logit gradient out
        return x + ws + g + N * 12, gemm
    if stage == "dx":  # logit gradient, the strip of W, dX running sum read and written
        return g + ws + N * H * 8, gemm
    if stage == "dw":  # logit gradient, X, the strip's dW rows out
        return g + x + w * H * 4, gemm
    raise KeyError(stage)


def cce_main(args, datagen, np, torch, B):
    """One step = forward + backward of the vocabulary projection with
    cross-entropy over vocabulary strips, on one batch of N tokens."""
    dev = torch.device("cuda:0")
    wl = datagen.CE_WORKLOADS[args.workload]
    log(f"generating {wl.name} inputs")
    inp = datagen.CeInputs(wl)
    bf = lambda a: torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
    X, W = bf(inp.X), bf(inp.W)
    t = torch.from_numpy(inp.targets).to(dev)
    dloss = torch.from_numpy(inp.dloss).to(dev)
    N, H, V, vc = wl.N, wl.H, wl.V, wl.v_chunk
    plan = B.cce_plan(N, H, V, vc)
    stream = torch.cuda.current_stream(dev)
    loss = torch.empty(N, dtype=torch.float32, device=dev)
    lse = torch.empty_like(loss)
    dX = torch.empty((N, H), dtype=torch.bfloat16, device=dev)
    dW = torch.empty((V, H), dtype=torch.float32, device=dev)
    # a plain 256 MiB device copy, outside the timed region: the reference for
    # scaling the HBM byte counters of a profiled run
    hbm_copy = calibration_copy(torch, dev)
    torch.cuda.synchronize()
    mem0 = torch.cuda.memory_allocated(dev)
    torch.cuda.reset_peak_memory_stats(dev)
    wsf = B.workspace(plan, "fwd", dev)
    wsb = B.workspace(plan, "bwd", dev)
    log(f"plan: S={plan.S} strips of {vc}, workspace fwd {plan.fwd_workspace_bytes} B, "
        f"bwd {plan.bwd_workspace_bytes} B")

    def fwd():
        B.cce_forward(plan, X, W, t, loss=loss, lse=lse, ws=wsf, stream=stream)

    def bwd():
        B.cce_backward(plan, X, W, t, lse, dloss, dX=dX, dW=dW, ws=wsb, stream=stream)

    ev = lambda: torch.cuda.Event(enable_timing=True)

    def timed(fn, k):
        e0, e1 = ev(), ev()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(k):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / k

    for _ in range(args.warmup):
        fwd()
        bwd()
    w0 = time.perf_counter()
    ms = timed(lambda: (fwd(), bwd()), args.steps)
    wall = (time.perf_counter() - w0) / args.steps * 1e3
    peak_extra = torch.cuda.max_memory_allocated(dev) - mem0
    ms_f = timed(fwd, args.steps)
    log(f"forward+backward: {ms:.3f} ms/step ({N / (ms / 1e3):.4g} tokens/s); forward {ms_f:.3f} ms")

    # per-kernel: re-launch each stage of each strip in pipeline order
    lead = GpuLead(torch, stream)
    fwd()
    torch.cuda.synchronize()
    stages = {}
    strips = [min(vc, V - s * vc) for s in range(plan.S)]
    for group, names in (("fwd", ("logits", "fold")), ("bwd", ("grad", "dx", "dw"))):
        if group == "bwd":
            bwd()
        marks = {n: [] for n in names}
        for _ in range(args.stage_reps):
            lead(2.0)  # the strips' long GEMMs keep the queue ahead after the first
            for si in range(plan.S):
                for n in names:
                    e0, e1 = ev(), ev()
                    e0.record(stream)
                    B.cce_debug_stage(plan, n, si, X, W, t, loss, lse, dloss, dX, dW,
                                      wsf if group == "fwd" else wsb, stream=stream)
                    e1.record(stream)
                    marks[n].append((e0, e1))
        torch.cuda.synchronize()
        for n in names:
            us = float(np.mean([a.elapsed_time(b_) for a, b_ in marks[n]])) * 1e3
            byts = float(np.mean([cce_stage_work(n, N, H, w)[0] for w in strips]))
            flops = float(np.mean([cce_stage_work(n, N, H, w)[1] for w in strips]))
            rec = {"us_per_launch": round(us, 2), "launches_per_step": plan.S,
                   "GB_per_s": round(byts / us / 1e3, 1), "alg_bytes_per_launch": int(byts)}
            if flops:
                rec["TFLOP_per_s"] = round(flops / us / 1e6, 1)
                rec["mfma_frac"] = round(flops / us / 1e6 / BF16_PEAK_TFLOPS, 4)
                rec["alg_flops_per_launch"] = int(flops)
            stages[n] = rec
            log(f"  {n:7s} {rec}")
    # the timed outputs are reproduced by a fresh forward + backward
    fwd()
    bwd()
    torch.cuda.synchronize()
    dom = max(stages, key=lambda n: stages[n]["us_per_launch"])
    d = stages[dom]
    roof = {"bound": "mfma", "achieved": d["TFLOP_per_s"], "peak": BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": round(d["TFLOP_per_s"] / BF16_PEAK_TFLOPS, 4),
            "traffic": measured_traffic(wl.name, dom), "kernel": dom}
    gemm_flops = 8.0 * N * H * V
    out = {
        "metric": "tokens/s (forward+backward) of the vocabulary projection with cross-entropy "
                  "at bounded strip memory",
        "value": round(N / (ms / 1e3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded normals, bf16-rounded; uniform targets)",
        "config": {"workload": wl.name, "N": N, "H": H, "V": V, "v_chunk": vc, "S": plan.S,
                   "parallelism": "single GPU"},
        "forward_ms": round(ms_f, 4),
        "gemm_TFLOP_per_s": round(gemm_flops / (ms / 1e3) / 1e12, 1),
        "roofline": roof,
        "hbm_copy": hbm_copy,
        "memory": {"strip_bound_bytes": plan.strip_bound_bytes,
                   "unchunked_logit_bytes": plan.unchunked_logit_bytes,
                   "fwd_workspace_bytes": plan.fwd_workspace_bytes,
                   "bwd_workspace_bytes": plan.bwd_workspace_bytes,
                   "peak_alloc_during_steps": int(peak_extra)},
        "stages": stages,
        "wall_ms_per_step": round(wall, 4),
    }
    if not args.no_cpu_baseline:
        import oracle
        from threadpoolctl import threadpool_info

        n_s = min(args.cpu_tokens, 1536, N)
        log(f"cpu baseline: fp64 oracle forward + backward of {n_s} tokens")
        W64 = inp.to_f64(inp.W)
        X64 = inp.to_f64(inp.X[:n_s])
        c0 = time.perf_counter()
        oracle.ce_forward_tokens(X64, W64, inp.targets[:n_s])
        oracle.ce_backward_tokens(X64, W64, inp.targets[:n_s], inp.dloss[:n_s].astype(np.float64))
        cpu_s = time.perf_counter() - c0
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
        out["cpu_baseline"] = {"value": round(n_s / cpu_s, 2), "unit": "tokens/s",
                               "cores": threads, "kind": "oracle",
                               "sample": f"first {n_s} of {N} tokens over the whole vocabulary: "
                                         f"loss, dX and dW, {cpu_s:.1f} s",
                               "host_cpus": len(os.sched_getaffinity(0)),
                               "cpu_model": cpu_model()}
        log(f"cpu baseline: {cpu_s:.2f} s, {threads} BLAS threads")
    print(json.dumps(out), flush=True)


class GpuLead:
    """A device-side spin queued ahead of a sequence of timed launches, so that
    the host enqueues the whole sequence while the GPU is still busy: without
    it the host's per-call latency (the Python binding, the event records)
    becomes idle GPU time inside the event pairs of short launches.  The spin
    is torch's cycle-count sleep kernel, calibrated once against events."""

    def __init__(self, torch, stream):
        self.torch, self.stream = torch, stream
        self.cycles_per_ms = None
        if hasattr(torch.cuda, "_sleep"):
            n = 2_000_000
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            with torch.cuda.stream(stream):
                e0.record(stream)
                torch.cuda._sleep(n)
                e1.record(stream)
            torch.cuda.synchronize()
            self.cycles_per_ms = n / max(e0.elapsed_time(e1), 1e-3)

    def __call__(self, ms):
        if self.cycles_per_ms is None:
            return
        with self.torch.cuda.stream(self.stream):
            self.torch.cuda._sleep(int(ms * self.cycles_per_ms))


def calibration_copy(torch, dev):
    """A 256 MiB device-to-device copy (read 256 MiB, write 256 MiB).  The
    first one is the reference for scaling a profiled run's HBM byte
    counters; five more are timed for the rate a plain copy reaches on this
    machine (context for the HBM roofline, whose peak stays the published
    8 TB/s)."""
    src = torch.empty(64 << 20, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    gbs = 5 * 2 * src.numel() * 4 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    log(f"plain 256 MiB copy: {gbs:.0f} GB/s (read + write)")
    return {"GB_per_s": round(gbs, 1), "bytes_per_copy": 2 * (256 << 20)}


def graph_replay(torch, args, call, outs, units):
    """The same step captured once into a HIP graph (torch.cuda.CUDAGraph; the
    call enqueues on the current stream, which is the capture stream inside
    the context) and replayed: W untimed replays, then K timed ones between
    events on the replaying stream.  The step's kernels then start without
    host launch gaps; the work is unchanged (checked: the replay's outputs
    equal the eager step's bitwise)."""
    ref = [t.clone() for t in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for _ in range(max(1, args.warmup)):
        g.replay()
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(args.steps):
        g.replay()
    e1.record(st)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    bit = lambda t: t.view(torch.int16) if t.dtype == torch.bfloat16 else t
    same = all(torch.equal(bit(a), bit(b_)) for a, b_ in zip(outs, ref))
    assert same, "graph replay differs from the eager step"
    del g
    log(f"graph replay: {ms:.3f} ms/step ({units / (ms / 1e3):.4g} per s)")
    return {"ms_per_step": round(ms, 4), "per_s": round(units / (ms / 1e3), 1)}


def blas_yardstick(torch, wl, plan, stages, backward=False):
    """torch.bmm (the vendor BLAS) on one chunk's expert products with every
    expert given the same number of rows, stored contiguously: E x [m, H] x
    [H, 2F] for gate and up side by side, E x [m, F] x [F, H] for the down
    projection, m = k c_eff / E rounded down to a multiple of 16.  No gather,
    no SwiGLU, no ragged segments: a plain-GEMM reference point for the
    grouped GEMMs' times on the same shapes."""
    dev = torch.device("cuda:0")
    E, H, F = wl.E, wl.H, wl.F
    m = max(16, (wl.k * plan.c_eff // E) // 16 * 16)
    g = torch.Generator(device=dev).manual_seed(7)
    bf = torch.bfloat16
    A = torch.randn(E, m, H, device=dev, dtype=bf, generator=g)
    Wgu = torch.randn(E, H, 2 * F, device=dev, dtype=bf, generator=g)
    Hh = torch.randn(E, m, F, device=dev, dtype=bf, generator=g)
    Wd = torch.randn(E, F, H, device=dev, dtype=bf, generator=g)
    res = {"rows_per_expert": m}
    def time_us(fn, reps=20):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps

    for name, fn, flops in (("gemm_up", lambda: torch.bmm(A, Wgu), 4.0 * E * m * H * F),
                            ("gemm_down", lambda: torch.bmm(Hh, Wd), 2.0 * E * m * H * F)):
        us = time_us(fn)
        ours = stages[name]
        res[name] = {"bmm_us": round(us, 2), "bmm_TFLOP_per_s": round(flops / us / 1e6, 1),
                     "grouped_us": ours["us_per_launch"],
                     "grouped_TFLOP_per_s": ours.get("TFLOP_per_s")}
        log(f"  yardstick {name}: torch.bmm {us:.1f} us ({flops / us / 1e6:.0f} TFLOP/s) on "
            f"{E} x [{m} rows]; grouped GEMM {ours['us_per_launch']} us")
    del A, Wgu, Hh, Wd
    if backward:
        # the weight-gradient shapes (K = the m rows of an expert), bf16
        # outputs: the library has no fp32 read-modify-write of dW, which the
        # layer's weight-gradient GEMMs also do (4x these output bytes)
        XT = torch.randn(E, H, m, device=dev, dtype=bf, generator=g)
        D = torch.randn(E, m, 2 * F, device=dev, dtype=bf, generator=g)
        HT = torch.randn(E, F, m, device=dev, dtype=bf, generator=g)
        DY = torch.randn(E, m, H, device=dev, dtype=bf, generator=g)
        o1 = torch.empty(E, H, 2 * F, device=dev, dtype=bf)
        o2 = torch.empty(E, F, H, device=dev, dtype=bf)
        for name, fn, flops in (("wgrad_gate_up", lambda: torch.bmm(XT, D, out=o1), 4.0 * E * m * H * F),
                                ("wgrad_down", lambda: torch.bmm(HT, DY, out=o2), 2.0 * E * m * H * F)):
            us = time_us(fn)
            res[name] = {"bmm_us": round(us, 2), "bmm_TFLOP_per_s": round(flops / us / 1e6, 1)}
            log(f"  yardstick {name}: torch.bmm {us:.1f} us ({flops / us / 1e6:.0f} TFLOP/s), bf16 out")
        del XT, D, HT, DY, o1, o2
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="train_bf16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=4096,
                    help="tokens of the batch the oracle runs for the CPU baseline "
                         "(forward+backward workloads: at most 2048)")
    ap.add_argument("--stage-reps", type=int, default=5)
    ap.add_argument("--backward", action="store_true",
                    help="forward-only workloads: also time forward+backward steps (reported "
                         "under forward_backward); a forward+backward workload always does")
    ap.add_argument("--exact-dw", action="store_true",
                    help="also time the backward with order-invariant weight gradients "
                         "(plan flag MOE_PLAN_EXACT_DW; reported under forward_backward.exact_dw)")
    ap.add_argument("--blas-yardstick", action="store_true",
                    help="also time the vendor library's batched GEMM (torch.bmm) on one chunk's "
                         "expert products with equal, contiguous row groups (reported under "
                         "blas_yardstick; context for the grouped GEMMs, not part of the step)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this layer runs on one GPU; multi-GPU runs are not part of this "
              "build (the expert-parallel sharding is described in the design notes)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import datagen
    from memory_bounded_expert_amd import binding as B

    if not torch.cuda.is_available():
        log("bench.py: no GPU visible")
        sys.exit(1)
    if args.workload in datagen.CE_WORKLOADS:
        return cce_main(args, datagen, np, torch, B)
    dev = torch.device("cuda:0")
    wl = datagen.WORKLOADS[args.workload]
    bf = wl.dtype == "bf16"
    b = 2 if bf else 4
    # a forward+backward workload's step is the whole hot path: forward, then
    # backward with per-chunk recompute
    train = wl.backward
    want_bwd = train or args.backward
    log(f"generating {wl.name} inputs")
    inp = datagen.Inputs(wl, dy=want_bwd)

    def up(a):
        if a is None:
            return None
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    X, Wr, Wg, Wu, Wd = (up(a) for a in (inp.X, inp.Wr, inp.Wg, inp.Wu, inp.Wd))
    bias = None if inp.bias is None else torch.from_numpy(inp.bias).to(dev)
    plan = B.moe_plan_chunks(wl.N, wl.H, wl.F, wl.E, wl.k, wl.c, wl.K_max,
                             B.MOE_BF16 if bf else B.MOE_F32)
    N, k, K = wl.N, wl.k, plan.K
    dt = torch.bfloat16 if bf else torch.float32
    Y = torch.empty((N, wl.H), dtype=dt, device=dev)
    idx = torch.empty((N, k), dtype=torch.int32, device=dev)
    gates = torch.empty((N, k), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        return B.moe_bounded_forward(plan, X, Wr, bias, Wg, Wu, Wd, Y=Y, topk_idx=idx, gates=gates,
                                     logits=None, want_logits=False, ws=ws, stream=stream)

    # a plain 256 MiB device copy, outside the timed region: the reference
    # for scaling the HBM byte counters of a profiled run (read 256 MiB,
    # write 256 MiB)
    hbm_copy = calibration_copy(torch, dev)
    # device memory the layer adds on top of its inputs and outputs: the
    # workspace (routing plan + the bounded per-chunk buffers)
    mem0 = torch.cuda.memory_allocated(dev)
    torch.cuda.reset_peak_memory_stats(dev)
    ws = B.workspace(plan, "fwd", dev)
    log(f"plan: K={K} c_eff={plan.c_eff} workspace={plan.fwd_workspace_bytes} B")
    for _ in range(args.warmup):
        stats = step()[4]
    torch.cuda.synchronize()
    t_ev0 = torch.cuda.Event(enable_timing=True)
    t_ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    t_ev0.record(stream)
    for _ in range(args.steps):
        stats = step()[4]
    t_ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms = t_ev0.elapsed_time(t_ev1) / args.steps
    peak_extra = torch.cuda.max_memory_allocated(dev) - mem0
    pairs = N * k
    value = pairs / (ms / 1e3)
    graph = graph_replay(torch, args, lambda: B.moe_bounded_forward(
        plan, X, Wr, bias, Wg, Wu, Wd, Y=Y, topk_idx=idx, gates=gates, logits=None,
        want_logits=False, ws=ws), [Y, idx, gates], pairs)
    log(f"forward: {ms:.3f} ms/step (wall {wall / args.steps * 1e3:.3f} ms/step), "
        f"{value:.4g} pairs/s")

    # ---- per-stage timing: re-launch each stage on the same stream with events
    lead = GpuLead(torch, stream)
    idx_np = idx.cpu().numpy()
    chunks = []
    for i in range(K):
        toks = np.arange(i, N, K)
        chunks.append((len(toks), len(toks) * k, len(np.unique(idx_np[toks]))))
    # whole-batch stages: events around repeated launches
    stages = {}
    ev = lambda: torch.cuda.Event(enable_timing=True)
    for stage in ("router", "topk", "plan"):
        e0, e1 = ev(), ev()
        lead(1.0 + 0.1 * args.stage_reps)
        e0.record(stream)
        for _ in range(args.stage_reps):
            B.moe_debug_stage(plan, stage, 0, X, Wr, bias, Wg, Wu, Wd, Y, idx, gates, ws,
                              stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        stages[stage] = {"us_per_launch": round(e0.elapsed_time(e1) * 1e3 / args.stage_reps, 2),
                         "launches_per_step": 1}
    # per-chunk stages: replay the chunk loop in order (so every launch sees
    # the same buffers as in the forward call), one event pair per launch
    per_chunk = ["gather", "gemm_up", "gemm_down", "combine"]
    try:  # the bf16 forward reads its permuted inputs inside the gate/up GEMM
        B.moe_debug_stage(plan, "gather", 0, X, Wr, bias, Wg, Wu, Wd, Y, idx, gates, ws,
                          stream=stream)
    except B.MoeError as err_:
        if err_.status != B.MOE_EUNSUPPORTED:
            raise
        per_chunk.remove("gather")
        log("  (no gather kernel: the gate/up GEMM reads the permuted rows from X)")
    marks = {s_: [] for s_ in per_chunk}
    for _ in range(args.stage_reps):
        lead(1.0 + 0.15 * K * len(per_chunk))
        for i in range(K):
            for stage in per_chunk:
                e0, e1 = ev(), ev()
                e0.record(stream)
                B.moe_debug_stage(plan, stage, i, X, Wr, bias, Wg, Wu, Wd, Y, idx, gates, ws,
                                  stream=stream)
                e1.record(stream)
                marks[stage].append((e0, e1))
    torch.cuda.synchronize()
    for stage in per_chunk:
        us = float(np.mean([a.elapsed_time(b_) for a, b_ in marks[stage]])) * 1e3
        rec = {"us_per_launch": round(us, 2), "launches_per_step": K}
        byts = float(np.mean([stage_work(stage, wl, b, *c)[0] for c in chunks]))
        flops = float(np.mean([stage_work(stage, wl, b, *c)[1] for c in chunks]))
        rec["GB_per_s"] = round(byts / us / 1e3, 1)
        rec["hbm_frac"] = round(byts / us / 1e3 / HBM_PEAK_GBS, 4)
        rec["alg_bytes_per_launch"] = int(byts)
        if stage.startswith("gemm"):
            tf = flops / us / 1e6
            peak = BF16_PEAK_TFLOPS if bf else FP32_PEAK_TFLOPS
            rec["TFLOP_per_s"] = round(tf, 1)
            rec["mfma_frac"] = round(tf / peak, 4)
            rec["alg_flops_per_launch"] = int(flops)
            rec["intensity_flop_per_B"] = round(flops / byts, 1)
        stages[stage] = rec
    for stage, rec in stages.items():
        log(f"  {stage:10s} {rec}")
    # the forward call's outputs are unchanged by the re-launches
    Yc = Y.clone()
    step()
    torch.cuda.synchronize()
    assert torch.equal(Yc.view(torch.int16) if bf else Yc, Y.view(torch.int16) if bf else Y)

    dom = max(stages, key=lambda s: stages[s]["us_per_launch"] * stages[s]["launches_per_step"])
    d = stages[dom]
    peak_tf = BF16_PEAK_TFLOPS if bf else FP32_PEAK_TFLOPS
    if "alg_flops_per_launch" in d and d["intensity_flop_per_B"] * 1e-3 * HBM_PEAK_GBS > peak_tf:
        roof = {"bound": "mfma", "achieved": d["TFLOP_per_s"], "peak": peak_tf, "unit": "TFLOP/s",
                "frac": round(d["TFLOP_per_s"] / peak_tf, 4)}
    else:
        roof = {"bound": "hbm", "achieved": d["GB_per_s"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(d["GB_per_s"] / HBM_PEAK_GBS, 4)}
    roof["traffic"] = measured_traffic(wl.name, dom)
    roof["kernel"] = dom
    gemm_flops = sum(np.mean([stage_work(s, wl, b, *c)[1] for c in chunks]) * K
                     for s in ("gemm_up", "gemm_down"))
    gemm_us = sum(stages[s]["us_per_launch"] * K for s in ("gemm_up", "gemm_down"))

    yard = (blas_yardstick(torch, wl, plan, stages, args.backward)
            if args.blas_yardstick and bf else None)

    fb = None
    if want_bwd:
        # one step = forward (routing saved) + backward with per-chunk recompute:
        # dX, dW_gate/up/down (fp32), dlogits, dgates and dW_r
        dY = up(inp.dY)
        wsb = B.workspace(plan, "bwd", dev)
        f32 = torch.float32
        grads = dict(dX=torch.empty((N, wl.H), dtype=dt, device=dev),
                 dW_gate=torch.empty((wl.E, wl.H, wl.F), dtype=f32, device=dev),
                 dW_up=torch.empty((wl.E, wl.H, wl.F), dtype=f32, device=dev),
                 dW_down=torch.empty((wl.E, wl.F, wl.H), dtype=f32, device=dev),
                 dlogits=torch.empty((N, wl.E), dtype=f32, device=dev),
                 dgates=torch.empty((N, k), dtype=f32, device=dev),
                 dW_r=torch.empty((wl.H, wl.E), dtype=f32, device=dev))

        def bstep():
            return B.moe_bounded_backward(plan, X, Wr, Wg, Wu, Wd, dY, idx, gates, ws=wsb,
                                          stream=stream, **grads)

        def fbstep():
            step()
            bstep()

        for _ in range(args.warmup):
            fbstep()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        w0 = time.perf_counter()
        e0.record(stream)
        for _ in range(args.steps):
            fbstep()
        e1.record(stream)
        torch.cuda.synchronize()
        wall_fb = time.perf_counter() - w0
        ms_fb = e0.elapsed_time(e1) / args.steps
        e0.record(stream)
        for _ in range(args.steps):
            bstep()
        e1.record(stream)
        torch.cuda.synchronize()
        ms_b = e0.elapsed_time(e1) / args.steps
        # backward GEMM flops: 12 H F per pair, plus the 4 H F per pair recompute
        bflops = 16.0 * pairs * wl.H * wl.F
        fb = {"ms_per_step": round(ms_fb, 4), "pairs_per_s": round(pairs / (ms_fb / 1e3), 1),
              "wall_ms_per_step": round(wall_fb / args.steps * 1e3, 4),
              "backward_ms": round(ms_b, 4),
              "backward_gemm_TFLOP_per_s": round(bflops / (ms_b / 1e3) / 1e12, 1),
              "workspace_bytes": plan.bwd_workspace_bytes}
        log(f"forward+backward: {ms_fb:.3f} ms/step, {fb['pairs_per_s']:.4g} pairs/s; "
            f"backward {ms_b:.3f} ms ({fb['backward_gemm_TFLOP_per_s']} TFLOP/s over its GEMM flops)")

        # per-kernel: re-launch each backward stage of each chunk in the
        # backward call's order, one event pair per launch
        bnames = ["recompute", "dh", "wgrad_down", "wgrad_gate_up", "dx", "combine_bwd", "dwr"]
        bstep()
        torch.cuda.synchronize()
        bmarks = {n_: [] for n_ in bnames}
        for _ in range(args.stage_reps):
            lead(2.0 + 0.3 * K * len(bnames))
            for s_ in ("zero", "transpose", "plan"):
                B.moe_debug_stage_bwd(plan, s_, 0, X, Wr, Wg, Wu, Wd, dY, idx, gates, grads, wsb,
                                      stream=stream)
            for i in range(K):
                for n_ in bnames:
                    e0, e1 = ev(), ev()
                    e0.record(stream)
                    B.moe_debug_stage_bwd(plan, n_, i, X, Wr, Wg, Wu, Wd, dY, idx, gates, grads,
                                          wsb, stream=stream)
                    e1.record(stream)
                    bmarks[n_].append((e0, e1))
        torch.cuda.synchronize()
        bst = {}
        peak_b = BF16_PEAK_TFLOPS if bf else FP32_PEAK_TFLOPS
        for n_ in bnames:
            us = float(np.mean([a.elapsed_time(b_) for a, b_ in bmarks[n_]])) * 1e3
            fz = fused_recompute_dh(wl, plan.c_eff)
            work = [bwd_stage_work(n_, wl, b, *c_, first=(ci == 0), fused=fz)
                    for ci, c_ in enumerate(chunks)]
            byts = float(np.mean([w_[0] for w_ in work]))
            flops = float(np.mean([w_[1] for w_ in work]))
            rec = {"us_per_launch": round(us, 2), "launches_per_step": K}
            if byts > 0:
                rec.update({"alg_bytes_per_launch": int(byts), "GB_per_s": round(byts / us / 1e3, 1),
                            "alg_flops_per_launch": int(flops),
                            "TFLOP_per_s": round(flops / us / 1e6, 1),
                            "roof": roof_of(byts, flops, us, peak_b)})
            else:  # (no kernel of its own: done inside the dh stage)
                rec["note"] = "done inside the dh stage's kernel"
            bst[n_] = rec
            log(f"  {n_:13s} {rec}")
        fb["stages"] = bst
        # the re-launches reproduce the backward call's outputs bitwise
        ref_g = {k_: v_.clone() for k_, v_ in grads.items()}
        bstep()
        torch.cuda.synchronize()
        for k_, v_ in grads.items():
            same = torch.equal(v_.view(torch.int16) if v_.dtype == torch.bfloat16 else v_,
                               ref_g[k_].view(torch.int16) if v_.dtype == torch.bfloat16
                               else ref_g[k_])
            assert same, f"backward stage re-launches changed {k_}"
        del ref_g

        if args.exact_dw and bf:
            # the opt-in order-invariant weight gradients: the same step with
            # the plan flag (a first pass over the chunks finds the column
            # maxima; int8-digit products into 64-bit accumulators)
            pe = B.moe_plan_chunks(wl.N, wl.H, wl.F, wl.E, wl.k, wl.c, wl.K_max, plan.dtype)
            B.moe_plan_set_flags(pe, B.MOE_PLAN_EXACT_DW)
            wse = B.workspace(pe, "bwd", dev)
            gx = {k_: torch.empty_like(v_) for k_, v_ in grads.items()}

            def xstep():
                return B.moe_bounded_backward(pe, X, Wr, Wg, Wu, Wd, dY, idx, gates, ws=wse,
                                              stream=stream, **gx)

            for _ in range(max(1, args.warmup)):
                xstep()
            torch.cuda.synchronize()
            e0.record(stream)
            for _ in range(args.steps):
                xstep()
            e1.record(stream)
            torch.cuda.synchronize()
            ms_x = e0.elapsed_time(e1) / args.steps
            for k_ in ("dX", "dlogits", "dgates", "dW_r"):  # unchanged by the flag
                a_, b2 = gx[k_], grads[k_]
                if a_.dtype == torch.bfloat16:
                    a_, b2 = a_.view(torch.int16), b2.view(torch.int16)
                assert torch.equal(a_, b2), f"exact-dW backward changed {k_}"
            fb["exact_dw"] = {"backward_ms": round(ms_x, 4),
                              "vs_default_backward": round(ms_x / ms_b, 3),
                              "workspace_bytes": pe.bwd_workspace_bytes}
            log(f"exact-dW backward: {ms_x:.3f} ms ({ms_x / ms_b:.2f}x the default), workspace "
                f"{pe.bwd_workspace_bytes} B")
            del wse, gx

    p1 = B.moe_plan_chunks(wl.N, wl.H, wl.F, wl.E, wl.k, wl.c, 1, plan.dtype)
    step_ms = fb["ms_per_step"] if train else ms
    step_wall = fb["wall_ms_per_step"] if train else wall / args.steps * 1e3
    out = {
        "metric": "routed token-expert pairs/s + grouped-GEMM MFMA util at bounded dispatch buffer",
        "value": round(pairs / (step_ms / 1e3), 1),
        "unit": "pairs/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if bf else "f32",
        "data": "synthetic (seeded normals, bf16-rounded; random-init expert weights)",
        "config": {"workload": wl.name, "N": N, "H": wl.H, "E": wl.E, "top_k": k, "F": wl.F,
                   "c": wl.c, "K_max": wl.K_max, "K": K, "c_eff": plan.c_eff,
                   "step": "forward+backward" if train else "forward",
                   "parallelism": "single GPU"},
        "forward": {"ms_per_step": round(ms, 4), "pairs_per_s": round(value, 1)},
        "forward_backward": fb,
        "graph_replay": graph,
        "hbm_copy": hbm_copy,
        "blas_yardstick": yard,
        "roofline": roof,
        "grouped_gemm": {"TFLOP_per_s": round(gemm_flops / gemm_us / 1e6, 1),
                         "mfma_frac": round(gemm_flops / gemm_us / 1e6 / peak_tf, 4),
                         "gate_up_mfma_frac": stages["gemm_up"].get("mfma_frac"),
                         "down_mfma_frac": stages["gemm_down"].get("mfma_frac"),
                         "target_mfma_frac": 0.6},
        "dispatch": {"buffer_bytes": stats["dispatch_bytes"],
                     "bound_bytes": plan.dispatch_bound_bytes,
                     "unchunked_buffer_bytes": p1.dispatch_bound_bytes,
                     "workspace_bytes": plan.fwd_workspace_bytes,
                     "unchunked_workspace_bytes": p1.fwd_workspace_bytes,
                     "peak_alloc_during_steps": int(peak_extra)},
        "stages": stages,
        "wall_ms_per_step": round(step_wall, 4),
    }

    if not args.no_cpu_baseline:
        import oracle
        from threadpoolctl import threadpool_info

        n_s = min(args.cpu_tokens, 2048 if train else N, N)
        what = "forward + backward" if train else "forward"
        log(f"cpu baseline: fp64 oracle {what} on the first {n_s} tokens")
        X64 = inp.to_f64(inp.X[:n_s])
        dY64 = inp.to_f64(inp.dY[:n_s]) if train else None
        Wr64 = inp.f64("Wr")
        # repeat the whole sample until about 10 s of CPU work (at most 8 times)
        reps, c0 = 0, time.perf_counter()
        while reps < 8 and (reps == 0 or time.perf_counter() - c0 < 10.0):
            _, idx_s, g_s, _ = oracle.moe_forward(X64, Wr64, inp.bias, inp.expert_f64, None,
                                                  None, k)
            if train:
                oracle.moe_backward(X64, Wr64, inp.expert_f64, None, None, dY64, idx_s, g_s)
            reps += 1
        cpu_s = time.perf_counter() - c0
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
        out["cpu_baseline"] = {
            "value": round(reps * n_s * k / cpu_s, 1), "unit": "pairs/s",
            "cores": threads, "kind": "oracle",
            "sample": f"first {n_s} of {N} tokens, full {what} incl. routing and fp64 upcast "
                      f"of the weights, {reps} runs in {cpu_s:.1f} s",
            "host_cpus": len(os.sched_getaffinity(0)), "cpu_model": cpu_model()}
        log(f"cpu baseline: {reps} runs, {cpu_s:.2f} s, {threads} BLAS threads on "
            f"{len(os.sched_getaffinity(0))} host CPUs ({cpu_model()})")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
