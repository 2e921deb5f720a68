"""Helpers of the GPU parity tests: oracle per (sequence, KV head) unit and
the comparison rules.

Parity rules (spec tolerances of the decode path):
* indices: per unit the GPU list holds min(k, T_b) distinct tokens in
  [0, T_b), strictly ascending, then -1 padding; every token in the symmetric
  difference with the oracle's set has an oracle score within 1e-4 (relative)
  of the oracle's k-th score;
* attention outputs (fp32) and lse: |gpu - oracle| <= 2e-3 * max(1, |oracle|)
  element by element, the oracle run on the GPU's own index set.
"""
from __future__ import annotations

import math

import numpy as np

from oracle import jssa_oracle as O
from token_level_sparse_amd import synth

IDX_REL = 1e-4
OUT_TOL = 2e-3


def unit_rows(inp: synth.GqaInputs, b: int, j: int):
    """Logical K and V rows [T_b, d] of one unit, read out of the host arrays.
    Positions without a page (reading R7) hold no row; they come back as
    zero rows and are marked absent by unit_valid."""
    n = int(inp.seq_lens[b])
    t = np.arange(n)
    if inp.page_table is None:
        return inp.K[b, j, :n], inp.V[b, j, :n]
    ok = unit_valid(inp, b)
    K = np.zeros((n, inp.K.shape[-1]), inp.K.dtype)
    V = np.zeros((n, inp.V.shape[-1]), inp.V.dtype)
    K[ok] = O.paged_rows(inp.K, inp.page_table[b], j, t[ok])
    V[ok] = O.paged_rows(inp.V, inp.page_table[b], j, t[ok])
    return K, V


def oracle_unit(inp: synth.GqaInputs, b: int, j: int, rows=None):
    """(K, V, Kp, s, hs) of one unit; absent positions score -inf (R3, R7)."""
    cfg = inp.cfg
    K, V = unit_rows(inp, b, j) if rows is None else rows
    hs = list(O.group_heads(j, cfg.G))
    Kp = O.project_keys(K, inp.P[j])
    s = O.subspace_scores(inp.q[b, hs], inp.P[j], Kp)
    if rows is None:
        s = np.where(unit_valid(inp, b), s, -np.inf)
    return K, V, Kp, s, hs


def check_indices(gpu_idx: np.ndarray, s: np.ndarray, k: int) -> int:
    """Returns the number of tolerated swaps; asserts the rule. s holds the
    oracle scores of positions [0, T_b), -inf for absent positions."""
    Tb = s.shape[0]
    n = min(k, int(np.sum(s > -np.inf)))
    g = gpu_idx[:n].astype(np.int64)
    assert np.all(gpu_idx[n:] == -1), "padding past min(k, existing tokens) must be -1"
    if n == 0:
        return 0
    assert np.all(g >= 0) and np.all(g < Tb), "indices outside [0, T_b)"
    assert np.all(np.diff(g) > 0), "indices must be strictly ascending"
    assert np.all(s[g] > -np.inf), "an absent token was selected"
    o = O.select_topk(s, k)[:n]
    diff = np.setxor1d(g, o)
    if diff.size:
        sk = O.kth_score(s, k)
        assert np.isfinite(sk), f"sets differ while the k-th score is {sk}"
        bad = diff[np.abs(s[diff] - sk) > IDX_REL * abs(sk)]
        assert bad.size == 0, f"swapped tokens {bad[:8]} outside the tie band (s_k={sk})"
    return int(diff.size // 2)


def check_close(got, ref, tol=OUT_TOL, what="output"):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    both_inf = np.isneginf(got) & np.isneginf(ref)
    g, r = np.where(both_inf, 0, got), np.where(both_inf, 0, ref)
    err = np.abs(g - r)
    lim = tol * np.maximum(1.0, np.abs(r))
    assert np.all(np.isfinite(g)), f"{what}: non-finite values"
    assert np.all(err <= lim), f"{what}: max abs err {err.max():.3g} (limit {tol} rel/abs)"
    return float(err.max()) if err.size else 0.0


def check_attention(inp, b, j, hs, K, V, sel, out, lse, scale):
    o_ref, lse_ref = O.attend(inp.q[b, hs], K[sel], V[sel], scale)
    e1 = check_close(out[b, hs], o_ref, what=f"out b={b} j={j}")
    e2 = check_close(lse[b, hs], lse_ref, what=f"lse b={b} j={j}")
    return max(e1, e2)


def scale_of(cfg) -> float:
    return 1.0 / math.sqrt(cfg.d)


def unit_valid(inp: synth.GqaInputs, b: int) -> np.ndarray:
    """Tokens of sequence b that have a valid page (all of them when contiguous)."""
    n = int(inp.seq_lens[b])
    if inp.page_table is None:
        return np.ones(n, bool)
    pg = inp.page_table[b][np.arange(n) // 16]
    return (pg >= 0) & (pg < inp.num_pages)


def check_topdelta(gpu_idx, gpu_cnt, s, valid, k_max, delta, n_sink, n_local, scale, G) -> int:
    """Top-delta parity (reading R13): the GPU lists gpu_cnt distinct valid
    tokens ascending, then -1; its set equals the oracle's except for tokens
    whose oracle score lies within IDX_REL (relative) of the threshold or of
    the last kept score (both sides decide on fp32 scores computed in
    different orders). Returns the number of such tokens."""
    o_idx, o_cnt = O.select_topdelta(s, k_max, delta, n_sink, n_local, scale, G, valid)
    g = np.asarray(gpu_idx[:gpu_cnt], np.int64)
    assert np.all(gpu_idx[gpu_cnt:] == -1), "padding past the count must be -1"
    assert np.all(np.diff(g) > 0), "indices must be strictly ascending"
    if gpu_cnt:
        assert g[0] >= 0 and g[-1] < s.shape[0] and np.all(valid[g]), "kept tokens must be valid"
    diff = np.setxor1d(g, o_idx[:o_cnt])
    if diff.size == 0:
        assert gpu_cnt == o_cnt
        return 0
    thr = O.topdelta_threshold(s, delta, n_sink, n_local, scale, G, valid)
    s32 = s.astype(np.float32).astype(np.float64)
    kept = o_idx[:o_cnt]
    s_last = s32[kept].min() if o_cnt else -np.inf
    m = thr + delta * G / scale
    band_thr = IDX_REL * max(abs(m), abs(thr), 1e-30)
    ok = (np.abs(s[diff] - thr) <= band_thr) | (np.abs(s[diff] - s_last) <= IDX_REL * max(abs(s_last), 1e-30))
    assert np.all(ok), f"tokens {diff[~ok][:8]} differ outside the tie bands (thr={thr}, last={s_last})"
    assert abs(gpu_cnt - o_cnt) <= diff.size
    return int(diff.size)
