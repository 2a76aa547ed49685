"""Seeded synthetic inputs for the memory-bounded MoE layer.

This module is shared by the fp64 oracle's tests, the GPU parity tests and the
benchmark.  It holds no arithmetic of the layer itself: it draws normals,
rounds them to bfloat16 and builds the router bias.  Nothing here routes,
permutes, multiplies or combines.

Streams.  Every tensor draws from its own PCG64 stream seeded with
``SeedSequence([seed, tensor_id])``; expert weights use one stream per expert,
``SeedSequence([seed, tensor_id, e])``, so a single expert's weights can be
regenerated without drawing the whole stack (the oracle's sampled checks at
full size rely on this).

Rounding.  bf16 inputs are fp32 normals rounded to bfloat16 with
round-to-nearest-even; both sides then see the same exact values (the oracle
upcasts the bf16 values to fp64 exactly).

Workloads.  The five named workloads carry the shapes, value scales and
routing skew of the memory-bounded MoE layer's measurements: a tiny fp32 case
the oracle runs in well under a second, a balanced 64-expert case, a
Zipf(1.2)-skewed 128-expert case, an 896-expert top-16 case (the
"896 routed experts, 16 activated" shape of the trillion-parameter MoE article,
section 1) and a 65,536-token forward+backward case.  No dataset is involved.
"""

from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np

# tensor ids (one PCG64 stream each)
TID_X = 1
TID_WR = 2
TID_BIAS = 3
TID_WG = 4
TID_WU = 5
TID_WD = 6
TID_DY = 7


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    N: int
    H: int
    E: int
    k: int
    F: int
    c: int
    K_max: int
    dtype: str  # "f32" or "bf16"
    x_std: float
    w_std: float
    zipf_s: Optional[float] = None  # router bias ~ Zipf(s) over experts
    backward: bool = False
    seed: int = 0

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS: Dict[str, Workload] = {
    # tiny fp32 forward (and backward) parity case
    "tiny_f32": Workload("tiny_f32", N=256, H=64, E=8, k=2, F=128, c=64, K_max=8,
                         dtype="f32", x_std=0.02, w_std=0.02, backward=True),
    # balanced routing, 64 experts, top-8
    "balanced_bf16": Workload("balanced_bf16", N=4096, H=2048, E=64, k=8, F=1408,
                              c=1024, K_max=8, dtype="bf16", x_std=1.0, w_std=0.02),
    # Zipf(1.2) skewed router bias over 128 experts
    "zipf_bf16": Workload("zipf_bf16", N=16384, H=4096, E=128, k=8, F=1536, c=2048,
                          K_max=16, dtype="bf16", x_std=1.0, w_std=0.02, zipf_s=1.2),
    # many small experts: 896 experts, top-16
    "many_experts_bf16": Workload("many_experts_bf16", N=8192, H=2048, E=896, k=16,
                                  F=512, c=1024, K_max=8, dtype="bf16", x_std=1.0,
                                  w_std=0.02),
    # forward + backward with per-chunk recompute
    "train_bf16": Workload("train_bf16", N=65536, H=2048, E=64, k=8, F=1024, c=4096,
                           K_max=16, dtype="bf16", x_std=1.0, w_std=0.02,
                           backward=True),
}


def rng(seed: int, *ids: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, *ids])))


def normal_f32(shape, std: float, seed: int, *ids: int) -> np.ndarray:
    x = rng(seed, *ids).standard_normal(shape, dtype=np.float32)
    x *= np.float32(std)
    return x


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bfloat16 (round to nearest, ties to even); returns uint16 bits.

    Inputs are finite normals, so the NaN path is never needed; it is kept
    quiet-NaN preserving for completeness."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    nan = (u & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    r = r.astype(np.uint16)
    if nan.any():
        r[nan] = ((u[nan] >> np.uint32(16)) | np.uint32(0x40)).astype(np.uint16)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def zipf_bias(E: int, s: float, seed: int) -> np.ndarray:
    """Router bias drawn so that expert popularity follows Zipf(s).

    Expert e gets popularity rank pi(e)+1 (pi a seeded permutation) and bias
    ln w_r with w_r = r^-s / sum_r r^-s.  Returned as fp32."""
    r = np.arange(1, E + 1, dtype=np.float64)
    w = r ** (-s)
    w /= w.sum()
    pi = rng(seed, TID_BIAS).permutation(E)
    return np.log(w[pi]).astype(np.float32)


class Inputs:
    """Host copies of one workload's inputs, in storage form.

    For bf16 workloads the storage arrays are uint16 bit patterns; for f32
    they are float32.  ``f64(name)`` gives exact fp64 values for the oracle.
    Expert weights are [E, H, F] (gate, up) and [E, F, H] (down), row-major.
    """

    def __init__(self, wl: Workload, experts: bool = True, dy: Optional[bool] = None,
                 N: Optional[int] = None, progress=None):
        self.wl = wl
        self.N = wl.N if N is None else N
        s = wl.seed
        bf = wl.dtype == "bf16"
        conv = f32_to_bf16_bits if bf else (lambda a: a)
        self.X = conv(normal_f32((self.N, wl.H), wl.x_std, s, TID_X))
        self.Wr = conv(normal_f32((wl.H, wl.E), wl.w_std, s, TID_WR))
        self.bias = zipf_bias(wl.E, wl.zipf_s, s) if wl.zipf_s is not None else None
        want_dy = wl.backward if dy is None else dy
        self.dY = conv(normal_f32((self.N, wl.H), 1.0, s, TID_DY)) if want_dy else None
        self.Wg = self.Wu = self.Wd = None
        if experts:
            st = np.uint16 if bf else np.float32
            self.Wg = np.empty((wl.E, wl.H, wl.F), st)
            self.Wu = np.empty((wl.E, wl.H, wl.F), st)
            self.Wd = np.empty((wl.E, wl.F, wl.H), st)
            for e in range(wl.E):
                g, u, d = self.expert_storage(e)
                self.Wg[e], self.Wu[e], self.Wd[e] = g, u, d
                if progress is not None and (e + 1) % 16 == 0:
                    progress(f"{wl.name}: experts {e + 1}/{wl.E} drawn")

    def expert_storage(self, e: int):
        wl = self.wl
        conv = f32_to_bf16_bits if wl.dtype == "bf16" else (lambda a: a)
        g = conv(normal_f32((wl.H, wl.F), wl.w_std, wl.seed, TID_WG, e))
        u = conv(normal_f32((wl.H, wl.F), wl.w_std, wl.seed, TID_WU, e))
        d = conv(normal_f32((wl.F, wl.H), wl.w_std, wl.seed, TID_WD, e))
        return g, u, d

    def to_f64(self, a: np.ndarray) -> np.ndarray:
        if a is None:
            return None
        if a.dtype == np.uint16:
            return bf16_bits_to_f32(a).astype(np.float64)
        return a.astype(np.float64)

    def f64(self, name: str) -> np.ndarray:
        return self.to_f64(getattr(self, name))

    def expert_f64(self, e: int):
        """fp64 (W_gate[e], W_up[e], W_down[e]), from the stored stack if present."""
        if self.Wg is not None:
            return self.to_f64(self.Wg[e]), self.to_f64(self.Wu[e]), self.to_f64(self.Wd[e])
        return tuple(self.to_f64(a) for a in self.expert_storage(e))


# ---------------------------------------------------------------------------
# Vocabulary projection with cross-entropy, computed over vocabulary strips.
# Tensor ids of its own streams; W is drawn in blocks of CE_W_BLOCK rows, one
# stream per block, so any block can be regenerated alone.

TID_CE_X = 11
TID_CE_W = 12
TID_CE_T = 13
TID_CE_IGN = 14
CE_W_BLOCK = 4096


@dataclasses.dataclass(frozen=True)
class CeWorkload:
    name: str
    N: int        # tokens
    H: int        # hidden width
    V: int        # vocabulary
    v_chunk: int  # vocabulary strip width
    dtype: str    # "bf16"
    x_std: float
    w_std: float
    ignore_frac: float = 0.0  # fraction of tokens whose target is ignored (-100)
    seed: int = 0

    def with_(self, **kw) -> "CeWorkload":
        return dataclasses.replace(self, **kw)


CE_WORKLOADS: Dict[str, CeWorkload] = {
    # the vocabulary-projection shape of the bounded-streaming measurements
    # (H 7168, V 200,000) on one GPU, 8192 tokens, strips of 8192 entries
    "vocab_bf16": CeWorkload("vocab_bf16", N=8192, H=7168, V=200_000, v_chunk=8192,
                             dtype="bf16", x_std=1.0, w_std=0.02),
    # small case the oracle runs whole: ragged last strip and ragged tiles
    "vocab_small_bf16": CeWorkload("vocab_small_bf16", N=777, H=512, V=20_000, v_chunk=4096,
                                   dtype="bf16", x_std=1.0, w_std=0.05, ignore_frac=0.05),
}


class CeInputs:
    """Host copies of one CE workload's inputs: X [N, H] and W [V, H] as bf16
    bit patterns (uint16), targets [N] int32 uniform over the vocabulary (a
    seeded fraction set to -100, the ignored marker), dloss [N] fp32 = 1/N
    (the upstream gradient of the mean loss)."""

    def __init__(self, wl: CeWorkload, N: Optional[int] = None, progress=None):
        self.wl = wl
        self.N = wl.N if N is None else N
        s = wl.seed
        self.X = f32_to_bf16_bits(normal_f32((self.N, wl.H), wl.x_std, s, TID_CE_X))
        self.W = np.empty((wl.V, wl.H), np.uint16)
        for b0 in range(0, wl.V, CE_W_BLOCK):
            self.W[b0:b0 + CE_W_BLOCK] = self.w_block(b0 // CE_W_BLOCK)
            if progress is not None and (b0 // CE_W_BLOCK) % 16 == 15:
                progress(f"{wl.name}: W rows {b0 + CE_W_BLOCK}/{wl.V} drawn")
        t = rng(s, TID_CE_T).integers(0, wl.V, self.N, dtype=np.int64)
        if wl.ignore_frac > 0:
            ign = rng(s, TID_CE_IGN).random(self.N) < wl.ignore_frac
            t[ign] = -100
        self.targets = t.astype(np.int32)
        self.dloss = np.full(self.N, 1.0 / max(self.N, 1), np.float32)

    def w_block(self, blk: int) -> np.ndarray:
        wl = self.wl
        rows = min(CE_W_BLOCK, wl.V - blk * CE_W_BLOCK)
        return f32_to_bf16_bits(normal_f32((rows, wl.H), wl.w_std, wl.seed, TID_CE_W, blk))

    @staticmethod
    def to_f64(a: np.ndarray) -> np.ndarray:
        return bf16_bits_to_f32(a).astype(np.float64)
