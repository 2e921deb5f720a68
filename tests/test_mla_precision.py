"""Precision design of the MLA attention kernel, checked on the CPU.

The kernel runs PV on bf16 MFMA. Rounding each softmax weight p to bf16
(8 significant bits) before PV, while the denominator sums the fp32 weights,
leaves each weighted sum off by up to 2^-9 relative per weight; splitting p
into a hi and a lo bf16 part (two MFMAs) leaves about 2^-17. This test
emulates both on the MLA workload's shapes (selection over the shared
latent cache; ai4snews digest, Perspective) at several seeds, against the
exact weighted sum, and requires the split to stay far inside the 2e-3
output tolerance. No GPU code runs here."""
import math
from dataclasses import replace

import numpy as np
import pytest

from token_level_sparse_amd import synth

TOL = 2e-3


def _bf16(x):
    return synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(np.asarray(x, np.float64))).astype(np.float64)


def _weighted_errors(seed, heads=16, n=2048):
    cfg = replace(synth.MLA_DSV3, B=1, T=4096, k=n, seed=seed)
    inp = synth.make_mla(cfg)
    rng = np.random.default_rng(seed)
    rows = np.sort(rng.choice(cfg.T, n, replace=False))
    C = synth.bf16_bits_to_f32(inp.latent[0][rows]).astype(np.float64)      # [n, 576]
    qn = synth.bf16_bits_to_f32(inp.q_nope[0]).astype(np.float64)
    qr = synth.bf16_bits_to_f32(inp.q_rope[0]).astype(np.float64)
    Wk = synth.bf16_bits_to_f32(inp.W_uk).astype(np.float64)
    L = cfg.d_latent
    scale = 1.0 / math.sqrt(cfg.d_nope + cfg.d_rope)
    worst = {"exact_vs_hi": 0.0, "exact_vs_hilo": 0.0}
    for h in range(heads):
        qa = np.concatenate([Wk[h].T @ qn[h], qr[h]])                        # absorbed query [576]
        logits = scale * (C @ qa)
        p = np.exp(logits - logits.max()).astype(np.float32).astype(np.float64)   # fp32 weights
        den = p.sum()
        exact = (p @ C[:, :L]) / den
        hi = _bf16(p)
        lo = _bf16(p - hi)
        for name, pw in (("exact_vs_hi", hi), ("exact_vs_hilo", hi + lo)):
            got = (pw @ C[:, :L]) / den
            err = np.abs(got - exact) / np.maximum(1.0, np.abs(exact))
            worst[name] = max(worst[name], float(err.max()))
    return worst


@pytest.mark.parametrize("seed", [1, 5, 13])
def test_pv_weight_split_bounds_rounding(seed):
    w = _weighted_errors(seed)
    assert w["exact_vs_hilo"] <= TOL / 20, w        # the kernel's form: far inside the tolerance
    assert w["exact_vs_hilo"] <= w["exact_vs_hi"] / 16, w
