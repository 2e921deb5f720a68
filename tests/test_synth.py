"""The seeded generator: determinism, batch-prefix property, distribution
moments, sink scaling, page-table structure."""
from dataclasses import replace

import numpy as np

from token_level_sparse_amd import synth


def test_deterministic_and_prefix():
    cfg = replace(synth.BATCHED_128K, B=2, T=512)
    a = synth.make_gqa(cfg)
    b = synth.make_gqa(cfg)
    for x, y in [(a.q, b.q), (a.K, b.K), (a.V, b.V), (a.P, b.P)]:
        np.testing.assert_array_equal(x, y)
    big = synth.make_gqa(replace(cfg, B=3))
    np.testing.assert_array_equal(big.K[:2], a.K)
    np.testing.assert_array_equal(big.q[:2], a.q)
    k, v = synth.unit_kv(a, 1, 5)
    np.testing.assert_array_equal(k, a.K[1, 5])
    np.testing.assert_array_equal(v, a.V[1, 5])


def test_moments_and_sinks():
    cfg = replace(synth.LLAMA8B_32K, T=8192)
    k = synth.bf16_bits_to_f32(synth.gen_keys_unit(cfg, 0, 3, cfg.T)).astype(np.float64)
    body = k[synth.SINKS:]
    assert abs(body.mean()) < 0.02
    # per coordinate: |A row|^2 (about 1 on average) + noise 0.09
    assert 0.85 < body.var() < 1.35
    nosink = synth.bf16_bits_to_f32(synth.gen_keys_unit(replace(cfg, sinks=False), 0, 3, cfg.T))
    np.testing.assert_array_equal(k[:synth.SINKS], synth.SINK_SCALE * nosink[:synth.SINKS])
    np.testing.assert_array_equal(k[synth.SINKS:], nosink[synth.SINKS:])
    v = synth.bf16_bits_to_f32(synth.gen_values_unit(cfg, 0, 3, cfg.T))
    assert abs(v.mean()) < 0.01 and abs(v.var() - 1) < 0.02


def test_projection_orthonormal():
    P = synth.gen_projection(3, 8, 128, 32)
    for j in range(8):
        np.testing.assert_allclose(P[j].T.astype(np.float64) @ P[j], np.eye(32), atol=1e-6)


def test_paged_lengths_and_table():
    cfg = replace(synth.PAGED_QWEN14B, T=4096, len_lo=2000, len_hi=4096)
    inp = synth.make_gqa(cfg)
    assert np.all((inp.seq_lens >= 2000) & (inp.seq_lens <= 4096))
    for b in range(cfg.B):
        n = (int(inp.seq_lens[b]) + 15) // 16
        assert np.all(inp.page_table[b, :n] >= 0) and np.all(inp.page_table[b, n:] == -1)
    assert inp.num_pages == sum((int(t) + 15) // 16 for t in inp.seq_lens)
