"""The seeded input generator: bf16 rounding and reproducibility."""

import numpy as np
import torch

import datagen


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * s for s in (1e-3, 1, 1e3)])
    # exact ties: low 16 bits 0x8000, both parities of bit 16
    ties = (np.arange(64, dtype=np.uint32) << 16 | 0x3F808000).view(np.float32)
    x = np.concatenate([x, ties, -ties])
    ours = datagen.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = datagen.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_inputs_reproducible_and_per_expert():
    wl = datagen.WORKLOADS["tiny_f32"]
    a, b = datagen.Inputs(wl), datagen.Inputs(wl)
    for n in ("X", "Wr", "Wg", "Wu", "Wd", "dY"):
        assert np.array_equal(getattr(a, n), getattr(b, n))
    lazy = datagen.Inputs(wl, experts=False)
    for e in (0, 5):
        for w, ref in zip(lazy.expert_f64(e), a.expert_f64(e)):
            assert np.array_equal(w, ref)
    assert abs(a.X.std() - 0.02) < 0.002


def test_zipf_bias_shape():
    b = datagen.zipf_bias(128, 1.2, 0)
    w = np.exp(b.astype(np.float64))
    assert abs(w.sum() - 1) < 1e-6
    r = np.sort(w)[::-1]
    assert abs(r[0] / r[1] - 2 ** 1.2) < 1e-4
