"""Device-side plumbing around the C ABI: upload seeded inputs, allocate the
buffers each stage writes, and chain the entry points of one decode step.

PyTorch is used for device memory and streams only; every step of the path
runs in the HIP library. The chains follow the JSSA decode step (score ->
top-k -> indexed attention -> combine), the dense full-KV baseline
(dense -> combine) and the gather ablation (score -> top-k -> gather ->
dense over the gathered rows -> combine).
"""
from __future__ import annotations

import math

import numpy as np
import torch

from . import jssa
from .synth import GqaInputs, MlaInputs, PAGE


def to_device(a: np.ndarray, device="cuda") -> torch.Tensor:
    """Upload a numpy array; bf16 bit patterns (uint16) become int16 tensors."""
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


class GqaCache:
    """One layer's cache and inputs on the GPU (contiguous or paged)."""

    def __init__(self, inp: GqaInputs, device="cuda"):
        cfg = inp.cfg
        self.cfg = cfg
        self.B, self.Hq, self.Hkv, self.d, self.T, self.r = cfg.B, cfg.Hq, cfg.Hkv, cfg.d, cfg.T, cfg.r
        self.q = to_device(inp.q, device)
        self.P = to_device(inp.P, device)
        self.K = to_device(inp.K, device)
        self.V = to_device(inp.V, device)
        self.seq_lens = to_device(inp.seq_lens.astype(np.int32), device)
        self.paged = inp.page_table is not None
        if self.paged:
            self.page_table = to_device(inp.page_table.astype(np.int32), device)
            self.num_pages = inp.num_pages
            self.Kp = torch.zeros((inp.num_pages, cfg.Hkv, PAGE, cfg.r), dtype=torch.int16, device=device)
            self.desc = jssa.gqa_desc(cfg.B, cfg.Hq, cfg.Hkv, cfg.r, cfg.T, cfg.d, PAGE, inp.num_pages,
                                      inp.page_table.shape[1], self.page_table, self.seq_lens)
        else:
            self.page_table = None
            self.num_pages = 0
            self.Kp = torch.zeros((cfg.B, cfg.Hkv, cfg.T, cfg.r), dtype=torch.int16, device=device)
            self.desc = jssa.gqa_desc(cfg.B, cfg.Hq, cfg.Hkv, cfg.r, cfg.T, cfg.d, 0, 0, 0, None,
                                      self.seq_lens)
        self.scale = 1.0 / math.sqrt(cfg.d)

    def project(self, stream=None):
        jssa.jssa_project_keys(self.desc, self.K, self.P, self.Kp, stream)


def default_splits(k: int, units: int = 1, blocks: int = 256, attend_fused: bool = True) -> int:
    """Splits of the selected set. Up to 512 selected tokens with the final
    selection and the attention sharing a kernel (attend_fused): one.
    Otherwise the power of two (up to 64) that brings the attention launch
    closest to one block per compute unit from below (`units` = B * Hkv
    (sequence, KV head) pairs, one block per pair and split), keeping at
    least 128 rows per split beyond 512 selected tokens and 64 up to it.
    Measured: paged Qwen at k = 2048 (64 pairs) 22.7 us of attention at 4
    splits, 32.5 us at 8; 128K B = 4 at k = 2048 (32 pairs) best at 8."""
    if k <= 512 and attend_fused:
        return 1
    rows = 128 if k > 512 else 64
    s = 1
    while s < 64 and 2 * s * units <= blocks and 2 * s <= k // rows:
        s *= 2
    return max(s, 2) if k > 512 else s


class SparseStep:
    """score -> top-k -> gather-free indexed split-K attention -> combine.

    fused=True runs score and top-k as one pass (jssa_score_topk, which does
    not write the fp32 score row); fused=False runs jssa_score then jssa_topk.
    Both give the same indices. With S = 1 the single partial is already the
    normalised output and its log-sum-exp (the combine of one split is the
    identity), so out/lse are views of the partial buffers and no combine is
    launched."""

    def __init__(self, c: GqaCache, k: int, S: int | None = None, fused: bool = False,
                 keep_scores: bool = True):
        dev = c.q.device
        S = default_splits(k, c.B * c.Hkv, attend_fused=fused) if S is None else S
        self.c, self.k, self.S, self.fused = c, k, S, fused
        self.scores = torch.empty((c.B, c.Hkv, c.T), dtype=torch.float32, device=dev) \
            if (keep_scores or not fused) else None
        nbytes = jssa.jssa_topk_workspace_size(c.B, c.Hkv, c.T, k)
        nf = jssa.jssa_score_topk_workspace_size(c.desc, k)
        self.ws = torch.empty(max(nbytes, nf, 16), dtype=torch.uint8, device=dev)
        self.idx = torch.empty((c.B, c.Hkv, k), dtype=torch.int32, device=dev)
        self.part_o = torch.empty((c.B, c.Hq, S, c.d), dtype=torch.float32, device=dev)
        self.part_lse = torch.empty((c.B, c.Hq, S), dtype=torch.float32, device=dev)
        if S == 1:
            self.out = self.part_o.view(c.B, c.Hq, c.d)
            self.lse = self.part_lse.view(c.B, c.Hq)
        else:
            self.out = torch.empty((c.B, c.Hq, c.d), dtype=torch.float32, device=dev)
            self.lse = torch.empty((c.B, c.Hq), dtype=torch.float32, device=dev)

    def score(self, stream=None):
        c = self.c
        jssa.jssa_score(c.desc, c.q, c.P, c.Kp, self.scores, stream)

    def topk(self, stream=None):
        c = self.c
        jssa.jssa_topk(c.B, c.Hkv, c.T, c.seq_lens, self.scores, self.k, self.idx, self.ws, None, stream)

    def attend(self, stream=None):
        c = self.c
        jssa.jssa_indexed_decode(c.desc, c.q, c.K, c.V, self.idx, self.k, self.S, c.scale, self.part_o,
                                 self.part_lse, stream)

    def combine(self, stream=None):
        c = self.c
        if self.S > 1:
            jssa.jssa_combine(c.B, c.Hq, self.S, c.d, self.part_o, self.part_lse, self.out, 0, self.lse, stream)

    def score_topk(self, stream=None):
        c = self.c
        jssa.jssa_score_topk(c.desc, c.q, c.P, c.Kp, self.k, self.scores, self.idx, self.ws, None, stream)

    def score_chunks(self, stream=None):
        c = self.c
        jssa.jssa_score_topk_chunks(c.desc, c.q, c.P, c.Kp, self.k, self.scores, self.ws, None, stream)

    def select_final(self, stream=None):
        jssa.jssa_score_topk_final(self.c.desc, self.k, self.ws, self.idx, None, stream)

    def final_attend(self, stream=None):
        """Final selection and one-split attention in one call (S == 1)."""
        c = self.c
        jssa.jssa_score_topk_final_attend(c.desc, self.k, self.ws, c.q, c.K, c.V, c.scale, self.idx, self.out,
                                          self.lse, None, stream)

    def stages(self):
        """The launches of one step, in order. Fused with one split: the
        chunk pass, then final selection + attention; fused with S splits:
        the chunk pass, the final selection, the split attention and the
        combine; unfused: jssa_score, jssa_topk, attention (+ combine)."""
        if self.fused and self.S == 1:
            return [self.score_chunks, self.final_attend]
        head = [self.score_chunks, self.select_final] if self.fused else [self.score, self.topk]
        return head + [self.attend] + ([self.combine] if self.S > 1 else [])

    def run(self, stream=None):
        for f in self.stages():
            f(stream)

    def capture(self):
        """Record one step's launches into a HIP graph (replayed by replay()).
        The entry points allocate, synchronise and memset nothing, so the
        whole step is capturable; it reads the current contents of q, the
        caches and seq_lens at every replay."""
        self.run()                                   # warm: first launches outside the capture
        torch.cuda.synchronize()
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            self.run()
        return self.graph

    def replay(self):
        self.graph.replay()


class DenseStep:
    """Full-KV split-K attention -> combine."""

    def __init__(self, c: GqaCache, S: int = 64):
        dev = c.q.device
        self.c, self.S = c, S
        self.part_o = torch.empty((c.B, c.Hq, S, c.d), dtype=torch.float32, device=dev)
        self.part_lse = torch.empty((c.B, c.Hq, S), dtype=torch.float32, device=dev)
        self.out = torch.empty((c.B, c.Hq, c.d), dtype=torch.float32, device=dev)
        self.lse = torch.empty((c.B, c.Hq), dtype=torch.float32, device=dev)

    def attend(self, stream=None):
        c = self.c
        jssa.jssa_dense_decode(c.desc, c.q, c.K, c.V, self.S, c.scale, self.part_o, self.part_lse, stream)

    def combine(self, stream=None):
        c = self.c
        jssa.jssa_combine(c.B, c.Hq, self.S, c.d, self.part_o, self.part_lse, self.out, 0, self.lse, stream)

    def run(self, stream=None):
        self.attend(stream)
        self.combine(stream)


class GatherStep:
    """Gather ablation: score -> top-k -> copy the selected rows into a
    contiguous [B,Hkv,k,d] buffer -> dense attention over it -> combine."""

    def __init__(self, sparse: SparseStep, S: int | None = None):
        c = sparse.c
        dev = c.q.device
        self.sp, self.c = sparse, c
        self.S = S or sparse.S
        k = sparse.k
        self.Kg = torch.empty((c.B, c.Hkv, k, c.d), dtype=torch.int16, device=dev)
        self.Vg = torch.empty_like(self.Kg)
        self.lens = torch.empty(c.B, dtype=torch.int32, device=dev)
        self.gdesc = jssa.gqa_desc(c.B, c.Hq, c.Hkv, c.r, k, c.d, 0, 0, 0, None, self.lens)
        self.part_o = torch.empty((c.B, c.Hq, self.S, c.d), dtype=torch.float32, device=dev)
        self.part_lse = torch.empty((c.B, c.Hq, self.S), dtype=torch.float32, device=dev)
        self.out = torch.empty((c.B, c.Hq, c.d), dtype=torch.float32, device=dev)
        self.lse = torch.empty((c.B, c.Hq), dtype=torch.float32, device=dev)

    def gather(self, stream=None):
        c = self.c
        jssa.jssa_gather_kv(c.desc, c.K, c.V, self.sp.idx, self.sp.k, self.Kg, self.Vg, self.lens, stream)

    def attend(self, stream=None):
        c = self.c
        jssa.jssa_dense_decode(self.gdesc, c.q, self.Kg, self.Vg, self.S, c.scale, self.part_o,
                               self.part_lse, stream)

    def combine(self, stream=None):
        c = self.c
        jssa.jssa_combine(c.B, c.Hq, self.S, c.d, self.part_o, self.part_lse, self.out, 0, self.lse, stream)

    def run(self, stream=None):
        self.sp.score(stream)
        self.sp.topk(stream)
        self.gather(stream)
        self.attend(stream)
        self.combine(stream)


class MlaStep:
    """MLA: absorb -> score + top-k (one set per sequence) -> indexed MFMA
    attention over the latent rows -> combine + value up-projection."""

    def __init__(self, inp: MlaInputs, S: int = 16, device="cuda"):
        cfg = inp.cfg
        self.cfg, self.S, self.k = cfg, S, cfg.k
        self.q_nope = to_device(inp.q_nope, device)
        self.q_rope = to_device(inp.q_rope, device)
        self.W_uk = to_device(inp.W_uk, device)
        self.W_uv = to_device(inp.W_uv, device)
        self.P = to_device(inp.P, device)
        self.latent = to_device(inp.latent, device)
        self.seq_lens = to_device(inp.seq_lens.astype(np.int32), device)
        self.desc = jssa.mla_desc(cfg.B, cfg.H, cfg.r, cfg.T, cfg.d_latent, cfg.d_rope, cfg.d_nope, cfg.d_v,
                                  self.seq_lens)
        self.scale = 1.0 / math.sqrt(cfg.d_nope + cfg.d_rope)
        B, H = cfg.B, cfg.H
        self.Kp = torch.zeros((B, cfg.T, cfg.r), dtype=torch.int16, device=device)
        self.q_abs = torch.empty((B, H, cfg.d_c), dtype=torch.float32, device=device)
        self.U = torch.empty((H, cfg.d_nope, cfg.r), dtype=torch.float32, device=device)   # W_uk[h] . P_lat
        self.q_sel = torch.empty((B, 64, cfg.r), dtype=torch.float32, device=device)   # the query in 64 parts
        self.scores = torch.empty((B, cfg.T), dtype=torch.float32, device=device)
        nbytes = max(jssa.jssa_topk_workspace_size(B, 1, cfg.T, cfg.k),
                     jssa.jssa_mla_score_topk_workspace_size(self.desc, cfg.k))
        self.ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=device)
        self.idx = torch.empty((B, cfg.k), dtype=torch.int32, device=device)
        self.part_o = torch.empty((B, H, S, cfg.d_latent), dtype=torch.float32, device=device)
        self.part_lse = torch.empty((B, H, S), dtype=torch.float32, device=device)
        self.o_lat = torch.empty((B, H, cfg.d_latent), dtype=torch.float32, device=device)
        self.lse = torch.empty((B, H), dtype=torch.float32, device=device)
        self.out = torch.empty((B, H, cfg.d_v), dtype=torch.float32, device=device)

    def project(self, stream=None):
        """Set-up: the projected latent cache and the folded selection weights."""
        jssa.jssa_mla_project_latent(self.desc, self.latent, self.P, self.Kp, stream)
        jssa.jssa_mla_fold_selection(self.desc, self.W_uk, self.P, self.U, stream)

    def run(self, stream=None):
        cfg = self.cfg
        jssa.jssa_mla_absorb_q(self.desc, self.q_nope, self.q_rope, self.W_uk, self.P, self.U, self.q_abs,
                               self.q_sel, stream)
        jssa.jssa_mla_score_topk(self.desc, self.q_sel, self.Kp, self.k, self.scores, self.idx, self.ws, None,
                                 stream)
        jssa.jssa_mla_indexed_decode(self.desc, self.q_abs, self.latent, self.idx, self.k, self.S,
                                     self.scale, self.part_o, self.part_lse, stream)
        jssa.jssa_mla_combine_up_v(self.desc, self.S, self.part_o, self.part_lse, self.W_uv, self.out, self.lse,
                                   stream)


# ---------------------------------------------------------------------------
# Subspace calibration (offline): second moments on the GPU, the spectral
# step on the host, both in the library.
# ---------------------------------------------------------------------------
def calib_key_moments(c: GqaCache, stream=None) -> torch.Tensor:
    """S_k per KV head [Hkv, d, d] fp32 over every valid token of the cache."""
    ws = torch.empty(jssa.jssa_calib_workspace_size(c.desc), dtype=torch.uint8, device=c.K.device)
    out = torch.empty((c.Hkv, c.d, c.d), dtype=torch.float32, device=c.K.device)
    jssa.jssa_calib_key_moments(c.desc, c.K, out, ws, stream=stream)
    return out


def calib_query_moments(q_samples: torch.Tensor, Hkv: int, stream=None) -> torch.Tensor:
    """S_q per KV head [Hkv, d, d] fp32 from decode-query samples [N, Hq, d]."""
    N, Hq, d = q_samples.shape
    out = torch.empty((Hkv, d, d), dtype=torch.float32, device=q_samples.device)
    ws = torch.empty(jssa.jssa_calib_query_workspace_size(Hkv), dtype=torch.uint8, device=q_samples.device)
    jssa.jssa_calib_query_moments(N, Hq, Hkv, q_samples, out, ws, stream=stream)
    return out


def calibrate(c: GqaCache, q_samples: torch.Tensor, r: int):
    """Calibrated projection P [Hkv, d, r] (fp32, on the cache's device) and
    the kept eigenvalues [Hkv, r] of each head's marginal operator."""
    Sk = calib_key_moments(c).cpu().numpy()
    Sq = calib_query_moments(q_samples, c.Hkv).cpu().numpy()
    Ps, ws = [], []
    for j in range(c.Hkv):
        P, w = jssa.jssa_calib_projection(Sq[j], Sk[j], r)
        Ps.append(P)
        ws.append(w)
    return torch.from_numpy(np.stack(Ps)).to(c.K.device), np.stack(ws)


# ---------------------------------------------------------------------------
# Top-delta step: the fused chunk pass, then the final selection with the
# top-delta filter and the attention over the kept tokens.
# ---------------------------------------------------------------------------
class TopDeltaStep:
    def __init__(self, cache: GqaCache, k_max: int, delta: float, n_sink: int = 4, n_local: int = 64):
        c = cache
        self.c, self.k_max = c, k_max
        self.rule = jssa.topdelta_rule(delta, n_sink, n_local)
        dev = c.K.device
        self.ws = torch.empty(jssa.jssa_score_topdelta_workspace_size(c.desc, k_max), dtype=torch.uint8, device=dev)
        self.idx = torch.empty((c.B, c.Hkv, k_max), dtype=torch.int32, device=dev)
        self.counts = torch.empty((c.B, c.Hkv), dtype=torch.int32, device=dev)
        self.out = torch.empty((c.B, c.Hq, c.d), dtype=torch.float32, device=dev)
        self.lse = torch.empty((c.B, c.Hq), dtype=torch.float32, device=dev)

    def select(self, stream=None):
        c = self.c
        jssa.jssa_score_topdelta(c.desc, c.q, c.P, c.Kp, self.k_max, self.rule, c.scale, self.idx, self.counts,
                                 self.ws, stream=stream)

    def run(self, stream=None):
        c = self.c
        jssa.jssa_score_topdelta_attend(c.desc, c.q, c.P, c.Kp, c.K, c.V, self.k_max, self.rule, c.scale, self.idx,
                                        self.counts, self.out, self.lse, self.ws, stream=stream)


# ---------------------------------------------------------------------------
# Screened step: tile bounds (kept with the cache), screening against a seed
# set, the chunk pass over the kept tiles, then the usual final selection.
# ---------------------------------------------------------------------------
class ScreenedStep:
    def __init__(self, cache: GqaCache, k: int, seeds: torch.Tensor):
        c = cache
        self.c, self.k = c, k
        dev = c.K.device
        self.seeds = seeds.contiguous()
        self.n_seed = int(seeds.shape[-1]) if seeds is not None else 0
        self.bounds = torch.empty(jssa.jssa_tile_bounds_size(c.desc) // 2, dtype=torch.int16, device=dev)
        self.ws = torch.empty(jssa.jssa_score_topk_screened_workspace_size(c.desc, k), dtype=torch.uint8,
                              device=dev)
        self.idx = torch.empty((c.B, c.Hkv, k), dtype=torch.int32, device=dev)
        self.kept_tiles = torch.empty((c.B, c.Hkv), dtype=torch.int32, device=dev)
        self.out = torch.empty((c.B, c.Hq, c.d), dtype=torch.float32, device=dev)
        self.lse = torch.empty((c.B, c.Hq), dtype=torch.float32, device=dev)

    def build_bounds(self, stream=None):
        jssa.jssa_build_tile_bounds(self.c.desc, self.c.Kp, self.bounds, stream)

    def update_bounds(self, pos, n_new, stream=None):
        """After an append of n_new tokens at pos (device int32 [B]) and the
        matching seq_lens update: rebuild only the tiles holding them."""
        jssa.jssa_update_tile_bounds(self.c.desc, self.c.Kp, pos, n_new, self.bounds, stream)

    def chunks(self, stream=None):
        c = self.c
        jssa.jssa_score_topk_screened_chunks(c.desc, c.q, c.P, c.Kp, self.bounds, self.seeds, self.n_seed, self.k,
                                             self.kept_tiles, self.ws, stream=stream)

    def final(self, stream=None):
        jssa.jssa_score_topk_final(self.c.desc, self.k, self.ws, self.idx, stream=stream)

    def final_attend(self, stream=None):
        c = self.c
        jssa.jssa_score_topk_final_attend(c.desc, self.k, self.ws, c.q, c.K, c.V, c.scale, self.idx, self.out,
                                          self.lse, stream=stream)
