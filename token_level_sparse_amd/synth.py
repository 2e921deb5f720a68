"""Seeded synthetic inputs for the JSSA decode path.

This module is shared by the GPU path's callers (tests, bench) and by the
CPU oracle's callers. It holds no arithmetic of the method itself: it only
draws random tensors, rounds them to the storage type and lays them out
(contiguous or paged). Projection, scoring, selection and attention live in
the HIP library and, independently, in the oracle.

The pages run JSSA on real models and long-context suites (LongBench, RULER,
reasoning sets); none of that is available here, so these generators stand in
for them with the models' layer shapes and a low-rank-plus-noise key/query
structure (JSSA abstract on weekinpapers, "Abstract": long-context decode over
a GQA KV cache; the digest on ai4snews, "Perspective": the model roster).

Random streams: one numpy PCG64 stream per (seed, tensor id, index...), so a
batch of 4 is a prefix of a batch of 16 and units can be drawn in parallel.
Tensor ids: 0 key basis A, 1 keys, 2 queries, 3 values, 4 projection P,
5 lengths and page tables, 6 MLA weights and queries, 7 calibration query
samples.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace

import numpy as np

T_A, T_KEYS, T_Q, T_V, T_P, T_LEN, T_MLA, T_CALQ = range(8)
LATENT_RANK = 24          # rank of the key/query basis A
NOISE = 0.3               # isotropic noise added to keys and queries
SINKS = 4                 # positions 0..3 carry keys scaled by SINK_SCALE
SINK_SCALE = 4.0
PAGE = 16                 # tokens per page in the paged layout


def stream(seed: int, tensor_id: int, *idx: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tensor_id, *idx])))


def f32_to_bf16_bits(x) -> np.ndarray:
    """fp64/fp32 -> fp32 -> bf16 bit pattern, round-to-nearest-even on the
    fp32 bits (storage conversion of generated data only)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


# --------------------------------------------------------------------------
# GQA workloads
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class GqaConfig:
    name: str
    B: int
    Hq: int
    Hkv: int
    d: int
    T: int            # max_seq: cache capacity per sequence
    r: int
    k: int
    seed: int
    paged: bool = False
    len_lo: int = 0   # ragged lengths drawn uniform in [len_lo, len_hi]; 0 = all T
    len_hi: int = 0
    sinks: bool = True
    ks: tuple = field(default=())
    # key model: "lowrank" (i.i.d. tokens) or "clustered" (segments of
    # cluster_len tokens share a latent centre; within a segment the latent
    # moves by cluster_noise and the isotropic noise is cluster_noise too)
    key_model: str = "lowrank"
    cluster_len: int = 512
    cluster_noise: float = 0.05

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv


# The five workloads (tiny; LLaMA-3.1-8B layer at 32K; 128K batched;
# Qwen3-14B paged ragged; DeepSeek-V3-shaped MLA below).
TINY = GqaConfig("tiny_gqa_4k", B=1, Hq=8, Hkv=2, d=128, T=4096, r=32, k=256, seed=1)
LLAMA8B_32K = GqaConfig("llama3.1-8b_layer_32k", B=1, Hq=32, Hkv=8, d=128, T=32768, r=32, k=256, seed=2)
BATCHED_128K = GqaConfig("gqa_128k_b16", B=16, Hq=32, Hkv=8, d=128, T=131072, r=32, k=256, seed=3)
PAGED_QWEN14B = GqaConfig("qwen3-14b_paged_ragged", B=8, Hq=40, Hkv=8, d=128, T=131072, r=48, k=256,
                          seed=4, paged=True, len_lo=65536, len_hi=131072, ks=(256, 1024, 2048))


@dataclass
class GqaInputs:
    cfg: GqaConfig
    q: np.ndarray            # [B,Hq,d] bf16 bits
    P: np.ndarray            # [Hkv,d,r] float32
    seq_lens: np.ndarray     # [B] int32
    K: np.ndarray            # contiguous [B,Hkv,T,d] bf16 bits, or pool [Npg,Hkv,16,d]
    V: np.ndarray
    page_table: np.ndarray | None = None   # [B,max_pages] int32 (-1 past the sequence)
    num_pages: int = 0


def key_basis(cfg: GqaConfig, j: int) -> np.ndarray:
    return stream(cfg.seed, T_A, j).standard_normal((cfg.d, LATENT_RANK)) / math.sqrt(LATENT_RANK)


def gen_keys_unit(cfg: GqaConfig, b: int, j: int, n: int, basis: np.ndarray | None = None) -> np.ndarray:
    """Keys of sequence b, KV head j, positions 0..n-1, as bf16 bits [n,d]."""
    A = key_basis(cfg, j) if basis is None else basis
    g = stream(cfg.seed, T_KEYS, b, j)
    if cfg.key_model == "clustered":
        # a stand-in for the locality of real caches (neighbouring tokens of
        # one passage are alike): the latent is piecewise constant over
        # segments, plus small per-token movement and noise
        nseg = (n + cfg.cluster_len - 1) // cfg.cluster_len
        centres = g.standard_normal((nseg, LATENT_RANK))
        z = np.repeat(centres, cfg.cluster_len, axis=0)[:n]
        z += cfg.cluster_noise * g.standard_normal((n, LATENT_RANK))
        x = z @ A.T
        x += cfg.cluster_noise * g.standard_normal((n, cfg.d))
        if cfg.sinks:
            x[:SINKS] *= SINK_SCALE
        return f32_to_bf16_bits(x)
    z = g.standard_normal((n, LATENT_RANK))
    eps = g.standard_normal((n, cfg.d))
    x = z @ A.T
    x += NOISE * eps
    if cfg.sinks:
        x[:SINKS] *= SINK_SCALE
    return f32_to_bf16_bits(x)


def gen_values_unit(cfg: GqaConfig, b: int, j: int, n: int) -> np.ndarray:
    return f32_to_bf16_bits(stream(cfg.seed, T_V, b, j).standard_normal((n, cfg.d)))


def gen_queries(cfg: GqaConfig) -> np.ndarray:
    q = np.empty((cfg.B, cfg.Hq, cfg.d), np.uint16)
    bases = [key_basis(cfg, j) for j in range(cfg.Hkv)]
    for b in range(cfg.B):
        for h in range(cfg.Hq):
            g = stream(cfg.seed, T_Q, b, h)
            w = g.standard_normal(LATENT_RANK)
            eps = g.standard_normal(cfg.d)
            q[b, h] = f32_to_bf16_bits(bases[h // cfg.G] @ w + NOISE * eps)
    return q


def gen_calib_queries(cfg: GqaConfig, n: int) -> np.ndarray:
    """n decode-query samples [n, Hq, d] (bf16 bits) drawn like gen_queries
    (basis of the head's KV group times a fresh latent, plus noise), from a
    stream of their own: the sample set a subspace is calibrated on."""
    q = np.empty((n, cfg.Hq, cfg.d), np.uint16)
    for h in range(cfg.Hq):
        g = stream(cfg.seed, T_CALQ, h)
        w = g.standard_normal((n, LATENT_RANK))
        eps = g.standard_normal((n, cfg.d))
        q[:, h] = f32_to_bf16_bits(w @ key_basis(cfg, h // cfg.G).T + NOISE * eps)
    return q


def gen_projection(seed: int, n_heads: int, d: int, r: int) -> np.ndarray:
    """Per-head orthonormal d x r basis (QR of a Gaussian, columns sign-fixed
    by sign(diag R)); a stand-in for the calibrated subspace, whose
    calibration is outside the decode path."""
    P = np.empty((n_heads, d, r), np.float32)
    for j in range(n_heads):
        M = stream(seed, T_P, j).standard_normal((d, r))
        Q, R = np.linalg.qr(M)
        s = np.sign(np.diag(R))
        s[s == 0] = 1.0
        P[j] = (Q * s).astype(np.float32)
    return P


def gen_seq_lens(cfg: GqaConfig) -> np.ndarray:
    if cfg.len_lo <= 0:
        return np.full(cfg.B, cfg.T, np.int32)
    g = stream(cfg.seed, T_LEN)
    return g.integers(cfg.len_lo, cfg.len_hi, size=cfg.B, endpoint=True).astype(np.int32)


def gen_page_table(cfg: GqaConfig, seq_lens: np.ndarray):
    """Pages of PAGE tokens get physical ids from a seeded permutation; table
    slots past a sequence's last page hold -1."""
    max_pages = (cfg.T + PAGE - 1) // PAGE
    npages = [(int(t) + PAGE - 1) // PAGE for t in seq_lens]
    total = int(sum(npages))
    g = stream(cfg.seed, T_LEN, 1)
    perm = g.permutation(total).astype(np.int32)
    table = np.full((cfg.B, max_pages), -1, np.int32)
    off = 0
    for b, n in enumerate(npages):
        table[b, :n] = perm[off:off + n]
        off += n
    return table, total


def _fill_units(cfg: GqaConfig, seq_lens, fn):
    units = [(b, j) for b in range(cfg.B) for j in range(cfg.Hkv)]
    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(lambda u: fn(*u, int(seq_lens[u[0]])), units))


def make_gqa(cfg: GqaConfig) -> GqaInputs:
    """All inputs of one decode step of one layer."""
    seq_lens = gen_seq_lens(cfg)
    q = gen_queries(cfg)
    P = gen_projection(cfg.seed, cfg.Hkv, cfg.d, cfg.r)
    bases = [key_basis(cfg, j) for j in range(cfg.Hkv)]
    if not cfg.paged:
        K = np.zeros((cfg.B, cfg.Hkv, cfg.T, cfg.d), np.uint16)
        V = np.zeros_like(K)

        def fill(b, j, n):
            K[b, j, :n] = gen_keys_unit(cfg, b, j, n, bases[j])
            V[b, j, :n] = gen_values_unit(cfg, b, j, n)
        _fill_units(cfg, seq_lens, fill)
        return GqaInputs(cfg, q, P, seq_lens, K, V)
    table, total = gen_page_table(cfg, seq_lens)
    K = np.zeros((total, cfg.Hkv, PAGE, cfg.d), np.uint16)
    V = np.zeros_like(K)

    def fill_paged(b, j, n):
        kk = gen_keys_unit(cfg, b, j, n, bases[j])
        vv = gen_values_unit(cfg, b, j, n)
        t = np.arange(n)
        pages = table[b, t // PAGE]
        K[pages, j, t % PAGE] = kk
        V[pages, j, t % PAGE] = vv
    _fill_units(cfg, seq_lens, fill_paged)
    return GqaInputs(cfg, q, P, seq_lens, K, V, table, total)


def unit_kv(inp: GqaInputs, b: int, j: int):
    """Logical (unpaged) K and V rows of one (sequence, KV head), regenerated
    from the seed: [T_b,d] bf16 bits each."""
    n = int(inp.seq_lens[b])
    return gen_keys_unit(inp.cfg, b, j, n), gen_values_unit(inp.cfg, b, j, n)


def with_batch(cfg: GqaConfig, B: int) -> GqaConfig:
    return replace(cfg, B=B)


# --------------------------------------------------------------------------
# MLA workload (DeepSeek-V3-shaped shared latent cache)
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class MlaConfig:
    name: str
    B: int
    H: int
    d_latent: int
    d_rope: int
    d_nope: int
    d_v: int
    r: int
    T: int
    k: int
    seed: int
    sinks: bool = True

    @property
    def d_c(self) -> int:
        return self.d_latent + self.d_rope


MLA_DSV3 = MlaConfig("deepseek-v3_mla_128k", B=4, H=128, d_latent=512, d_rope=64, d_nope=128, d_v=128,
                     r=64, T=131072, k=2048, seed=5)


@dataclass
class MlaInputs:
    cfg: MlaConfig
    q_nope: np.ndarray   # [B,H,d_nope] bf16 bits
    q_rope: np.ndarray   # [B,H,d_rope] bf16 bits
    W_uk: np.ndarray     # [H,d_nope,d_latent] bf16 bits
    W_uv: np.ndarray     # [H,d_v,d_latent] bf16 bits
    P: np.ndarray        # [d_c,r] float32
    latent: np.ndarray   # [B,T,d_c] bf16 bits
    seq_lens: np.ndarray


def gen_latent_unit(cfg: MlaConfig, b: int, n: int) -> np.ndarray:
    A = stream(cfg.seed, T_A, 0).standard_normal((cfg.d_c, LATENT_RANK)) / math.sqrt(LATENT_RANK)
    g = stream(cfg.seed, T_KEYS, b, 0)
    x = g.standard_normal((n, LATENT_RANK)) @ A.T
    x += NOISE * g.standard_normal((n, cfg.d_c))
    if cfg.sinks:
        x[:SINKS] *= SINK_SCALE
    return f32_to_bf16_bits(x)


def make_mla(cfg: MlaConfig) -> MlaInputs:
    g = stream(cfg.seed, T_MLA)
    q_nope = f32_to_bf16_bits(g.standard_normal((cfg.B, cfg.H, cfg.d_nope)))
    q_rope = f32_to_bf16_bits(g.standard_normal((cfg.B, cfg.H, cfg.d_rope)))
    W_uk = f32_to_bf16_bits(g.standard_normal((cfg.H, cfg.d_nope, cfg.d_latent)) / math.sqrt(cfg.d_nope))
    W_uv = f32_to_bf16_bits(g.standard_normal((cfg.H, cfg.d_v, cfg.d_latent)) / math.sqrt(cfg.d_latent))
    P = gen_projection(cfg.seed, 1, cfg.d_c, cfg.r)[0]
    seq_lens = np.full(cfg.B, cfg.T, np.int32)
    latent = np.zeros((cfg.B, cfg.T, cfg.d_c), np.uint16)

    def fill(b):
        latent[b] = gen_latent_unit(cfg, b, cfg.T)
    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(fill, range(cfg.B)))
    return MlaInputs(cfg, q_nope, q_rope, W_uk, W_uv, P, latent, seq_lens)
