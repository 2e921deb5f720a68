"""GPU parity: every stage of the HIP path against the fp64 oracle on the
same seeded inputs, called through the C ABI."""
from __future__ import annotations

import math
from dataclasses import replace

import numpy as np
import pytest
import torch

from oracle import jssa_oracle as O
from token_level_sparse_amd import synth
from tests import gpu_util as U

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def J():
    from token_level_sparse_amd import jssa  # fails loudly when the library is missing
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return jssa


@pytest.fixture(scope="module")
def PL():
    from token_level_sparse_amd import pipeline
    return pipeline


def _np(t: torch.Tensor) -> np.ndarray:
    a = t.detach().cpu().numpy()
    return a.view(np.uint16) if a.dtype == np.int16 else a


# Ragged shapes: T not a multiple of any tile, lengths that leave part-filled
# chunks, an empty sequence, a sequence shorter than k.
RAGGED = replace(synth.LLAMA8B_32K, name="ragged", B=4, T=5000, len_lo=1, len_hi=5000, seed=77)


def ragged_inputs(cfg=RAGGED, lens=(5000, 0, 131, 3333)):
    inp = synth.make_gqa(replace(cfg, len_lo=0))
    lens = np.array(lens, np.int32)
    inp.seq_lens = lens
    return inp


# ---------------------------------------------------------------------------
# projected keys (append / project)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("r", [16, 32, 48, 64, 128])
def test_project_keys_bit_exact(J, PL, r):
    cfg = replace(synth.TINY, r=r, T=1000, B=2, seed=10 + r)
    inp = synth.make_gqa(cfg)
    c = PL.GqaCache(inp)
    c.project()
    torch.cuda.synchronize()
    Kp = _np(c.Kp)
    for b in range(cfg.B):
        for j in range(cfg.Hkv):
            np.testing.assert_array_equal(Kp[b, j], O.project_keys(inp.K[b, j], inp.P[j]))


def test_project_keys_paged_and_ragged(J, PL):
    cfg = replace(synth.PAGED_QWEN14B, B=3, T=3000, len_lo=1000, len_hi=3000, seed=21)
    inp = synth.make_gqa(cfg)
    c = PL.GqaCache(inp)
    c.project()
    torch.cuda.synchronize()
    Kp = _np(c.Kp)
    for b in range(cfg.B):
        for j in range(cfg.Hkv):
            K, _ = U.unit_rows(inp, b, j)
            got = O.paged_rows(Kp, inp.page_table[b], j, np.arange(K.shape[0]))
            np.testing.assert_array_equal(got, O.project_keys(K, inp.P[j]))


@pytest.mark.parametrize("paged", [False, True])
def test_append_kv(J, PL, paged):
    cfg = replace(synth.PAGED_QWEN14B if paged else synth.TINY, B=2, T=512, len_lo=0, r=32, seed=31)
    if paged:
        cfg = replace(cfg, len_lo=512, len_hi=512)
    inp = synth.make_gqa(cfg)
    c = PL.GqaCache(inp)
    n_new = 5
    rng = np.random.default_rng(3)
    k_new = synth.f32_to_bf16_bits(rng.standard_normal((cfg.B, cfg.Hkv, n_new, cfg.d)))
    v_new = synth.f32_to_bf16_bits(rng.standard_normal((cfg.B, cfg.Hkv, n_new, cfg.d)))
    pos = np.array([100, 509], np.int32)          # second sequence runs past max_seq: 3 slots skipped
    J.jssa_append_kv(c.desc, c.K, c.V, c.Kp, PL.to_device(k_new), PL.to_device(v_new), c.P,
                     PL.to_device(pos), n_new)
    torch.cuda.synchronize()
    K, V, Kp = _np(c.K), _np(c.V), _np(c.Kp)
    for b in range(cfg.B):
        for j in range(cfg.Hkv):
            for i in range(n_new):
                t = int(pos[b]) + i
                if t >= cfg.T:
                    continue
                if paged:
                    pg = inp.page_table[b, t // 16]
                    kr, vr, kpr = K[pg, j, t % 16], V[pg, j, t % 16], Kp[pg, j, t % 16]
                else:
                    kr, vr, kpr = K[b, j, t], V[b, j, t], Kp[b, j, t]
                np.testing.assert_array_equal(kr, k_new[b, j, i])
                np.testing.assert_array_equal(vr, v_new[b, j, i])
                np.testing.assert_array_equal(kpr, O.project_keys(k_new[b, j, i][None], inp.P[j])[0])
    # untouched rows stay untouched
    if not paged:
        np.testing.assert_array_equal(K[0, :, :100], inp.K[0, :, :100])


# ---------------------------------------------------------------------------
# scores
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("r", [16, 32, 48, 64, 128])
def test_score_parity(J, PL, r):
    inp = ragged_inputs(replace(RAGGED, r=r, seed=40 + r))
    c = PL.GqaCache(inp)
    c.project()
    st = PL.SparseStep(c, k=64)
    st.score()
    torch.cuda.synchronize()
    S = _np(st.scores)
    for b in range(inp.cfg.B):
        Tb = int(inp.seq_lens[b])
        for j in range(inp.cfg.Hkv):
            K, V, Kp, s, hs = U.oracle_unit(inp, b, j)
            qp = O.project_query(inp.q[b, hs], inp.P[j])
            bound = 1e-5 * (np.abs(O.bf16_to_f64(Kp) * qp).sum(1) + 1e-30)
            assert np.all(np.abs(S[b, j, :Tb] - s) <= bound), (b, j)
            assert np.all(np.isneginf(S[b, j, Tb:]))


# ---------------------------------------------------------------------------
# top-k on host-made scores (identical fp32 input on both sides: bit-exact)
# ---------------------------------------------------------------------------
def _topk_case(J, B, H, T, k, lens, scores):
    dev = "cuda"
    sc = torch.from_numpy(scores).to(dev)
    sl = torch.from_numpy(np.asarray(lens, np.int32)).to(dev)
    n = J.jssa_topk_workspace_size(B, H, T, k)
    ws = torch.empty(max(n, 16), dtype=torch.uint8, device=dev)
    idx = torch.empty((B, H, k), dtype=torch.int32, device=dev)
    J.jssa_topk(B, H, T, sl, sc, k, idx, ws)
    torch.cuda.synchronize()
    got = idx.cpu().numpy()
    for b in range(B):
        for h in range(H):
            Tb = int(lens[b])
            np.testing.assert_array_equal(got[b, h], O.select_topk(scores[b, h, :Tb].astype(np.float64), k),
                                          err_msg=f"b={b} h={h} T_b={Tb} k={k}")
    return got


@pytest.mark.parametrize("T,k", [(4096, 256), (32768, 256), (50000, 1), (20000, 1024), (70000, 2048),
                                 (40000, 4096), (3000, 3000), (1500, 700), (100, 7),
                                 # rows whose length is not a multiple of 4 (scalar score loads), one
                                 # token past a chunk, exactly one chunk; few rows with a budget whose
                                 # 8192-token lists would need merging take 32768-token chunks
                                 # (70000 and 40000 above, and 32769: odd, one past a wide chunk)
                                 (9999, 300), (8193, 256), (8192, 256), (17, 5), (32769, 2048)])
def test_topk_bit_exact(J, T, k):
    rng = np.random.default_rng(T + k)
    B, H = 3, 2
    s = rng.standard_normal((B, H, T)).astype(np.float32)
    s[0, 1] = np.round(s[0, 1] * 4) / 4                   # heavy exact ties
    s[1, 0, : T // 2] = 1.0                               # a long plateau at the top
    s[1, 0, T // 2:] = rng.standard_normal(T - T // 2).astype(np.float32) * 0.1
    s[2, 1, ::3] = -0.0
    s[2, 1, 1::3] = 0.0
    lens = [T, max(1, T // 3), min(T, max(1, k // 2))]
    _topk_case(J, B, H, T, k, lens, s)


@pytest.mark.parametrize("T,k", [(4096, 256), (40000, 256), (70000, 2048)])
def test_topk_small_tied_bin(J, T, k):
    """A few tokens tie exactly at the k-th score, with some of them taken:
    the bin holding the k-th key is small, so the final pass ranks it within
    one wave, and the tied tokens taken must be the lowest-indexed ones."""
    rng = np.random.default_rng(T + 7 * k)
    B, H = 2, 2
    s = rng.standard_normal((B, H, T)).astype(np.float32)
    for b in range(B):
        for h in range(H):
            order = np.argsort(-s[b, h], kind="stable")
            lo = k - 3 if (b + h) % 2 == 0 else k - 1          # 3 of 5, or 1 of 5 tied tokens taken
            s[b, h, order[lo:lo + 5]] = s[b, h, order[k - 1]]
    _topk_case(J, B, H, T, k, [T, T - 5], s)


def test_topk_long_row_multi_round(J):
    """A row long enough that the chunk lists need more than one merge."""
    rng = np.random.default_rng(5)
    T, k = 600000, 4096
    s = rng.standard_normal((1, 1, T)).astype(np.float32)
    _topk_case(J, 1, 1, T, k, [T], s)


def test_topk_absent_tokens(J):
    """-inf marks a position without a token: never selected, so a row with
    fewer than k existing tokens lists exactly those, then -1 (reading R3)."""
    rng = np.random.default_rng(41)
    B, H, T, k = 2, 2, 20000, 300
    s = rng.standard_normal((B, H, T)).astype(np.float32)
    s[0, 0, rng.random(T) < 0.3] = -np.inf              # scattered absent positions
    s[0, 1, :] = -np.inf
    s[0, 1, [5, 9000, 17000]] = [1.0, -2.0, 0.5]          # three tokens exist
    s[1, 0, 8192:16384] = -np.inf                        # one whole chunk absent
    s[1, 1, :] = -np.inf                                 # nothing exists
    got = _topk_case(J, B, H, T, k, [T, T], s)
    np.testing.assert_array_equal(got[0, 1, :4], [5, 9000, 17000, -1])
    assert np.all(got[1, 1] == -1)


def test_topk_empty_and_all_equal(J):
    T, k = 9000, 300
    s = np.zeros((2, 1, T), np.float32)
    s[1, 0] = 2.5
    got = _topk_case(J, 2, 1, T, k, [0, T], s)
    assert np.all(got[0] == -1)
    np.testing.assert_array_equal(got[1, 0], np.arange(k))


# ---------------------------------------------------------------------------
# whole sparse step, dense, gather ablation, combine
# ---------------------------------------------------------------------------
def _sparse_and_check(J, PL, inp, k, S, units=None, fused=False):
    c = PL.GqaCache(inp)
    c.project()
    st = PL.SparseStep(c, k=k, S=S, fused=fused)
    st.run()
    torch.cuda.synchronize()
    idx, out, lse = _np(st.idx), _np(st.out), _np(st.lse)
    cfg = inp.cfg
    swaps = 0
    for b in range(cfg.B):
        for j in range(cfg.Hkv):
            if units is not None and (b, j) not in units:
                continue
            K, V, Kp, s, hs = U.oracle_unit(inp, b, j)
            swaps += U.check_indices(idx[b, j], s, k)
            sel = idx[b, j][idx[b, j] >= 0]
            U.check_attention(inp, b, j, hs, K, V, sel, out, lse, c.scale)
    return c, st, swaps


@pytest.mark.parametrize("cfg,k,S", [(synth.TINY, 256, 8), (synth.LLAMA8B_32K, 256, 8),
                                     (synth.LLAMA8B_32K, 256, 1), (synth.LLAMA8B_32K, 1, 4),
                                     # several 32-row batches per wave (the next batch's tokens
                                     # load while this one is multiplied), a partial last one
                                     (synth.LLAMA8B_32K, 1024, 1), (synth.TINY, 1000, 2),
                                     # splits past the list's end (k = 3 over 8 splits)
                                     (synth.TINY, 3, 8),
                                     # 2- and 4-wave attention blocks (33..64 and 65..128 rows
                                     # per split), one with a partial batch
                                     (synth.TINY, 64, 1), (synth.TINY, 128, 1), (synth.LLAMA8B_32K, 100, 1)])
def test_sparse_step_parity(J, PL, cfg, k, S):
    _sparse_and_check(J, PL, synth.make_gqa(cfg), k, S)


def test_sparse_step_ragged(J, PL):
    _sparse_and_check(J, PL, ragged_inputs(), 256, 8)


@pytest.mark.parametrize("cfg,k,S", [(synth.TINY, 256, 1), (synth.LLAMA8B_32K, 256, 1), (RAGGED, 300, 2)])
def test_sparse_step_fused(J, PL, cfg, k, S):
    inp = ragged_inputs() if cfg is RAGGED else synth.make_gqa(cfg)
    _sparse_and_check(J, PL, inp, k, S, fused=True)


FULL16K = replace(synth.LLAMA8B_32K, B=1, T=16384, seed=84)


@pytest.mark.parametrize("case", ["ragged32", "r48_paged_k2048", "r128_k4096", "tiny_k1", "r16_T100",
                                  "full_k64", "full_k256_ties", "full_all_equal", "full_k257",
                                  "paged_full_invalid", "clustered_full_k256",
                                  "lists_k2048", "lists_paged_ragged_k2048", "lists_clustered_k2048",
                                  "lists_all_equal_k2048"])
def test_score_topk_fused_equals_split(J, PL, case):
    """The fused score + top-k pass returns exactly the indices (and, when
    asked, the scores) of jssa_score followed by jssa_topk. The full_* and
    paged_full_* cases fill every 8192-token chunk, which takes the fused
    kernel's top-two bound path for k <= 256 (ties, all-equal scores, -inf
    tokens behind invalid pages), its fallback to the histogram select on
    clustered keys, and the general path for k = 257. The lists_* cases
    (8 chunks, k = 2048) take the chunk-list path: lists of 1024 per chunk,
    one final pass over their union, where the lists hold each row's top k
    (low-rank keys, contiguous and paged with ragged lengths) and where some
    row needs the selection from its scores (clustered keys, all scores
    equal)."""
    edit = None
    if case.startswith("lists_"):
        T64 = replace(synth.LLAMA8B_32K, B=1, T=65536, seed=87)
        k = 2048
        if case == "lists_k2048":
            inp = synth.make_gqa(T64)
        elif case == "lists_paged_ragged_k2048":
            inp = synth.make_gqa(replace(synth.PAGED_QWEN14B, B=2, T=65536, len_lo=30000, len_hi=65536, seed=88))
        elif case == "lists_clustered_k2048":
            inp = synth.make_gqa(replace(T64, key_model="clustered", cluster_len=4096, seed=89))
        else:
            inp = synth.make_gqa(T64)
            edit = lambda c: c.Kp.zero_()
    elif case.startswith("full_"):
        inp = synth.make_gqa(FULL16K)
        k = {"full_k64": 64, "full_k256_ties": 256, "full_all_equal": 200, "full_k257": 257}[case]
        if case == "full_k256_ties":      # 37 distinct projected keys per (b, j): long runs of equal scores
            edit = lambda c: c.Kp.copy_(c.Kp[:, :, torch.arange(c.Kp.shape[2], device=c.Kp.device) % 37])
        elif case == "full_all_equal":
            edit = lambda c: c.Kp.zero_()
    elif case == "clustered_full_k256":       # neighbouring tokens alike: the top-two bound falls back
        inp, k = synth.make_gqa(replace(FULL16K, key_model="clustered", cluster_len=256, seed=86)), 256
    elif case == "paged_full_invalid":
        inp = synth.make_gqa(replace(synth.PAGED_QWEN14B, B=2, T=16384, len_lo=16384, len_hi=16384, seed=85))
        k = 256
        table = inp.page_table.copy()
        table[0, 7] = -1
        table[0, 600] = -1
        table[1, 1000] = inp.num_pages + 3

        def edit(c):
            c.page_table.copy_(torch.from_numpy(table).cuda())
    elif case == "ragged32":
        inp, k = ragged_inputs(), 256
    elif case == "r48_paged_k2048":
        inp, k = synth.make_gqa(replace(synth.PAGED_QWEN14B, B=2, T=40000, len_lo=20000, len_hi=40000, seed=81)), 2048
    elif case == "r128_k4096":
        inp, k = synth.make_gqa(replace(synth.TINY, r=128, T=20000, B=2, seed=82)), 4096
    elif case == "tiny_k1":
        inp, k = synth.make_gqa(synth.TINY), 1
    else:
        inp, k = synth.make_gqa(replace(synth.TINY, r=16, T=100, seed=83)), 60
    c = PL.GqaCache(inp)
    c.project()
    if edit is not None:
        edit(c)
        torch.cuda.synchronize()
    a = PL.SparseStep(c, k=k, fused=False)
    a.score()
    a.topk()
    b = PL.SparseStep(c, k=k, fused=True, keep_scores=True)
    b.score_topk()
    nb = PL.SparseStep(c, k=k, fused=True, keep_scores=False)
    nb.score_topk()
    # the two halves of the fused call, issued separately
    h = PL.SparseStep(c, k=k, fused=True, keep_scores=True)
    h.score_chunks()
    h.select_final()
    torch.cuda.synchronize()
    np.testing.assert_array_equal(_np(b.idx), _np(a.idx))
    np.testing.assert_array_equal(_np(nb.idx), _np(a.idx))
    np.testing.assert_array_equal(_np(h.idx), _np(a.idx))
    np.testing.assert_array_equal(_np(b.scores), _np(a.scores))
    np.testing.assert_array_equal(_np(h.scores), _np(a.scores))
    # the tie-heavy and full-chunk cases also against the oracle's own
    # selection, computed from its own (identically edited) projected keys
    if case in ("full_k256_ties", "full_all_equal", "paged_full_invalid", "clustered_full_k256", "full_k64",
                "lists_clustered_k2048", "lists_all_equal_k2048"):
        if case == "paged_full_invalid":
            inp.page_table = table
        idx = _np(a.idx)
        for bb in range(inp.cfg.B):
            for j in range(inp.cfg.Hkv):
                K, V, Kp, s_, hs = U.oracle_unit(inp, bb, j)
                if case == "full_k256_ties":
                    Kp = Kp[np.arange(Kp.shape[0]) % 37]
                elif case in ("full_all_equal", "lists_all_equal_k2048"):
                    Kp = np.zeros_like(Kp)
                if case in ("full_k256_ties", "full_all_equal", "lists_all_equal_k2048"):
                    s_ = O.subspace_scores(inp.q[bb, hs], inp.P[j], Kp)
                U.check_indices(idx[bb, j], s_, k)
                if case in ("full_all_equal", "lists_all_equal_k2048"):   # all scores tie: the k lowest indices
                    np.testing.assert_array_equal(idx[bb, j], np.arange(k))


@pytest.mark.parametrize("case", ["no_seq_lens", "b65_ragged", "b64_ragged"])
def test_chunk_pass_launch_orders(J, PL, case):
    """The chunk pass maps launch positions to (sequence, KV head, chunk)
    two ways: with per-sequence lengths and up to 64 sequences the real
    chunks come first (packed), otherwise each row's chunks are rotated.
    Both must give the indices (and scores) of jssa_score + jssa_topk."""
    if case == "no_seq_lens":
        inp = synth.make_gqa(replace(synth.TINY, B=2, T=20000, seed=91))
    else:
        B = 65 if case == "b65_ragged" else 64
        inp = synth.make_gqa(replace(synth.TINY, B=B, Hq=4, Hkv=1, T=17000, len_lo=1, len_hi=17000, seed=92))
    c = PL.GqaCache(inp)
    c.project()
    if case == "no_seq_lens":                       # every row full: the lengths may be left out
        assert np.all(inp.seq_lens == c.T)
        c.desc = J.gqa_desc(c.B, c.Hq, c.Hkv, c.r, c.T, c.d, 0, 0, 0, None, None)
    k = 256
    a = PL.SparseStep(c, k=k, fused=False)
    a.score()
    a.topk()
    b = PL.SparseStep(c, k=k, fused=True, keep_scores=True)
    b.score_topk()
    nb = PL.SparseStep(c, k=k, fused=True, keep_scores=False)
    nb.score_topk()
    torch.cuda.synchronize()
    np.testing.assert_array_equal(_np(b.idx), _np(a.idx))
    np.testing.assert_array_equal(_np(nb.idx), _np(a.idx))
    np.testing.assert_array_equal(_np(b.scores), _np(a.scores))
    # and against the oracle on a few rows
    for bb in sorted({0, c.B // 2, c.B - 1}):
        for j in range(c.Hkv):
            _, _, _, s, _ = U.oracle_unit(inp, bb, j)
            U.check_indices(_np(nb.idx)[bb, j], s, k)


@pytest.mark.parametrize("case", ["llama_k256", "ragged_k100", "qwen_paged_k256_G5", "tiny_k512", "G8_k300", "k1024_split"])
def test_final_attend_matches_separate(J, PL, case):
    """jssa_score_topk_final_attend writes the indices of the separate final
    selection and, within float rounding, the one-split attention of
    jssa_indexed_decode on them; outputs also checked against the oracle."""
    if case == "llama_k256":
        inp, k = synth.make_gqa(replace(synth.LLAMA8B_32K, B=2, T=20000, seed=95)), 256
    elif case == "ragged_k100":
        inp, k = ragged_inputs(), 100
    elif case == "qwen_paged_k256_G5":
        inp, k = synth.make_gqa(replace(synth.PAGED_QWEN14B, B=2, T=20000, len_lo=9000, len_hi=20000, seed=96)), 256
    elif case == "tiny_k512":
        inp, k = synth.make_gqa(synth.TINY), 512
    elif case == "G8_k300":
        inp, k = synth.make_gqa(replace(synth.TINY, Hq=16, Hkv=2, seed=97)), 300
    else:                                                 # falls back to separate launches inside the call
        inp, k = synth.make_gqa(replace(synth.LLAMA8B_32K, B=1, T=30000, seed=98)), 1024
    c = PL.GqaCache(inp)
    c.project()
    a = PL.SparseStep(c, k=k, S=1, fused=True, keep_scores=False)
    a.score_chunks()
    a.select_final()
    a.attend()
    f = PL.SparseStep(c, k=k, S=1, fused=True, keep_scores=False)
    f.score_chunks()
    f.final_attend()
    torch.cuda.synchronize()
    np.testing.assert_array_equal(_np(f.idx), _np(a.idx))
    U.check_close(_np(f.out), _np(a.out), tol=1e-5, what="fused vs separate out")
    U.check_close(_np(f.lse), _np(a.lse), tol=1e-5, what="fused vs separate lse")
    cfg = inp.cfg
    idx, out, lse = _np(f.idx), _np(f.out), _np(f.lse)
    for b in range(cfg.B):
        for j in range(cfg.Hkv):
            K, V, Kp, s, hs = U.oracle_unit(inp, b, j)
            U.check_indices(idx[b, j], s, k)
            sel = idx[b, j][idx[b, j] >= 0]
            U.check_attention(inp, b, j, hs, K, V, sel, out, lse, c.scale)


@pytest.mark.parametrize("k", [256, 1024, 2048])
def test_sparse_step_paged_qwen(J, PL, k):
    cfg = replace(synth.PAGED_QWEN14B, B=3, T=20000, len_lo=9000, len_hi=20000, seed=50 + k)
    _sparse_and_check(J, PL, synth.make_gqa(cfg), k, 8)


def test_sparse_k_equals_T_is_dense(J, PL):
    cfg = replace(synth.TINY, T=2048, B=2)
    inp = synth.make_gqa(cfg)
    c, st, _ = _sparse_and_check(J, PL, inp, cfg.T, 16)
    np.testing.assert_array_equal(_np(st.idx), np.broadcast_to(np.arange(cfg.T), st.idx.shape))
    dn = PL.DenseStep(c, S=16)
    dn.run()
    torch.cuda.synchronize()
    U.check_close(_np(dn.out), _np(st.out), tol=1e-5, what="k=T sparse vs dense")


@pytest.mark.parametrize("cfg,S", [(synth.TINY, 7), (synth.LLAMA8B_32K, 64), (RAGGED, 16)])
def test_dense_parity(J, PL, cfg, S):
    inp = ragged_inputs() if cfg is RAGGED else synth.make_gqa(cfg)
    c = PL.GqaCache(inp)
    dn = PL.DenseStep(c, S=S)
    dn.run()
    torch.cuda.synchronize()
    out, lse = _np(dn.out), _np(dn.lse)
    for b in range(inp.cfg.B):
        for j in range(inp.cfg.Hkv):
            K, V = U.unit_rows(inp, b, j)
            hs = list(O.group_heads(j, inp.cfg.G))
            o_ref, lse_ref = O.dense_unit(inp.q[b, hs], K, V, c.scale)
            U.check_close(out[b, hs], o_ref, what=f"dense b={b} j={j}")
            U.check_close(lse[b, hs], lse_ref, what=f"dense lse b={b} j={j}")


def test_dense_paged(J, PL):
    cfg = replace(synth.PAGED_QWEN14B, B=2, T=6000, len_lo=3000, len_hi=6000, seed=61)
    inp = synth.make_gqa(cfg)
    c = PL.GqaCache(inp)
    dn = PL.DenseStep(c, S=32)
    dn.run()
    torch.cuda.synchronize()
    out = _np(dn.out)
    for b in range(cfg.B):
        for j in range(cfg.Hkv):
            K, V = U.unit_rows(inp, b, j)
            hs = list(O.group_heads(j, cfg.G))
            U.check_close(out[b, hs], O.dense_unit(inp.q[b, hs], K, V, c.scale)[0], what="dense paged")


def test_gather_ablation(J, PL):
    inp = ragged_inputs()
    c = PL.GqaCache(inp)
    c.project()
    st = PL.SparseStep(c, k=256, S=8)
    st.run()
    ga = PL.GatherStep(st, S=4)
    ga.run()
    torch.cuda.synchronize()
    idx, Kg, Vg, lens = _np(st.idx), _np(ga.Kg), _np(ga.Vg), _np(ga.lens)
    for b in range(inp.cfg.B):
        assert lens[b] == min(256, int(inp.seq_lens[b]))
        for j in range(inp.cfg.Hkv):
            K, V = U.unit_rows(inp, b, j)
            sel = idx[b, j]
            ok = sel >= 0
            np.testing.assert_array_equal(Kg[b, j][ok], K[sel[ok]])
            np.testing.assert_array_equal(Vg[b, j][ok], V[sel[ok]])
            assert np.all(Kg[b, j][~ok] == 0)
            hs = list(O.group_heads(j, inp.cfg.G))
            U.check_attention(inp, b, j, hs, K, V, sel[ok], _np(ga.out), _np(ga.lse), c.scale)


@pytest.mark.parametrize("S,dv", [(1, 128), (8, 128), (64, 128), (5, 512)])
def test_combine_parity(J, S, dv):
    rng = np.random.default_rng(S * 7 + dv)
    B, H = 3, 5
    po = rng.standard_normal((B, H, S, dv)).astype(np.float32)
    pl = (rng.standard_normal((B, H, S)) * 3).astype(np.float32)
    pl[0, 0, :] = -np.inf                        # an all-empty row
    if S > 1:
        pl[1, 2, 0] = -np.inf                    # one empty split
    out = torch.empty((B, H, dv), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, H), dtype=torch.float32, device="cuda")
    J.jssa_combine(B, H, S, dv, torch.from_numpy(po).cuda(), torch.from_numpy(pl).cuda(), out, 0, lse)
    outb = torch.empty((B, H, dv), dtype=torch.int16, device="cuda")
    J.jssa_combine(B, H, S, dv, torch.from_numpy(po).cuda(), torch.from_numpy(pl).cuda(), outb, 1, None)
    torch.cuda.synchronize()
    o, l = out.cpu().numpy(), lse.cpu().numpy()
    for b in range(B):
        for h in range(H):
            ro, rl = O.combine(po[b, h], pl[b, h])
            U.check_close(o[b, h], ro, tol=1e-5, what="combine")
            U.check_close(l[b, h], rl, tol=1e-5, what="combine lse")
    ob = synth.bf16_bits_to_f32(outb.cpu().numpy().view(np.uint16))
    np.testing.assert_array_equal(ob, synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(o)))


def test_graph_replay_matches_eager(J, PL):
    """The fused step captured in a HIP graph gives the eager result on every
    replay, with eager work and synchronisation between replays and the
    outputs cleared before each one."""
    inp = synth.make_gqa(replace(synth.LLAMA8B_32K, B=2, T=20000, seed=91))
    c = PL.GqaCache(inp)
    c.project()
    st = PL.SparseStep(c, k=256, S=2, fused=True, keep_scores=False)
    st.run()
    torch.cuda.synchronize()
    ref_idx, ref_out, ref_lse = st.idx.clone(), st.out.clone(), st.lse.clone()
    st.capture()
    junk = torch.randn(1 << 20, device="cuda")
    for rep in range(4):
        st.idx.fill_(-7)
        st.out.fill_(float("nan"))
        st.lse.fill_(float("nan"))
        junk.mul_(1.0001).add_(0.5)                 # unrelated eager work between replays
        torch.cuda.synchronize()
        st.replay()
        torch.cuda.synchronize()
        assert torch.equal(st.idx, ref_idx), rep
        assert torch.equal(st.out, ref_out), rep
        assert torch.equal(st.lse, ref_lse), rep


def test_deterministic_repeat(J, PL):
    inp = synth.make_gqa(synth.LLAMA8B_32K)
    c = PL.GqaCache(inp)
    c.project()
    st = PL.SparseStep(c, k=256, S=8)
    st.run()
    torch.cuda.synchronize()
    a = (_np(st.idx).copy(), _np(st.out).copy(), _np(st.scores).copy())
    st.run()
    torch.cuda.synchronize()
    np.testing.assert_array_equal(_np(st.idx), a[0])
    np.testing.assert_array_equal(_np(st.out), a[1])
    np.testing.assert_array_equal(_np(st.scores), a[2])


def test_invalid_page_entries_are_absent(J, PL):
    """A page-table entry outside [0, num_pages) inside T_b hides its 16
    tokens: never scored above -inf, never selected, never attended."""
    cfg = replace(synth.PAGED_QWEN14B, B=2, T=2048, len_lo=2048, len_hi=2048, seed=71)
    inp = synth.make_gqa(cfg)
    c = PL.GqaCache(inp)
    c.project()
    table = inp.page_table.copy()
    table[0, 3] = -1
    table[1, 10] = inp.num_pages + 5
    c.page_table.copy_(torch.from_numpy(table).cuda())
    st = PL.SparseStep(c, k=256, S=8)
    st.run()
    torch.cuda.synchronize()
    S_ = _np(st.scores)
    assert np.all(np.isneginf(S_[0, :, 48:64])) and np.all(np.isneginf(S_[1, :, 160:176]))
    idx = _np(st.idx)
    assert not np.any((idx[0] >= 48) & (idx[0] < 64))
    assert not np.any((idx[1] >= 160) & (idx[1] < 176))
    assert np.all(np.isfinite(_np(st.out)))


@pytest.mark.parametrize("fused,S", [(True, 1), (True, 4), (False, 1), (False, 4)])
def test_paged_fewer_existing_tokens_than_k(J, PL, fused, S):
    """Positions behind invalid page-table entries hold no token (reading
    R7). Sequence 0 keeps only three pages (48 tokens < k): its selection is
    exactly those tokens, then -1, and the attention runs over them alone;
    sequence 1 loses every other page; sequence 2 is whole. Compared with the
    oracle's selection on the fused and the split paths."""
    cfg = replace(synth.PAGED_QWEN14B, B=3, T=4096, len_lo=3000, len_hi=4096, seed=73)
    inp = synth.make_gqa(cfg)
    table = inp.page_table
    n0 = (int(inp.seq_lens[0]) + 15) // 16
    keep0 = {2, 5, n0 - 1}
    for p in range(n0):
        if p not in keep0:
            table[0, p] = -1 if p % 2 else inp.num_pages + p
    n1 = (int(inp.seq_lens[1]) + 15) // 16
    table[1, 1:n1:2] = -7
    k = 256
    c, st, _ = _sparse_and_check(J, PL, inp, k, S, fused=fused)
    idx = _np(st.idx)
    exist0 = np.nonzero(U.unit_valid(inp, 0))[0]
    assert exist0.size < k
    for j in range(cfg.Hkv):
        np.testing.assert_array_equal(idx[0, j, :exist0.size], exist0)
        assert np.all(idx[0, j, exist0.size:] == -1)
        assert np.all(U.unit_valid(inp, 1)[idx[1, j]])


# ---------------------------------------------------------------------------
# top-delta selection (reading R13)
# ---------------------------------------------------------------------------
TD_CASES = {
    "tiny_d0.5": (lambda: synth.make_gqa(synth.TINY), 256, 0.5, 4, 64),
    "tiny_d2_capped": (lambda: synth.make_gqa(synth.TINY), 256, 2.0, 4, 64),
    "tiny_d3": (lambda: synth.make_gqa(synth.TINY), 256, 3.0, 4, 64),
    "tiny_no_special": (lambda: synth.make_gqa(synth.TINY), 256, 0.5, 0, 0),
    "ragged_d2": (lambda: ragged_inputs(), 300, 2.0, 4, 64),
    "llama_d1_k1024": (lambda: synth.make_gqa(synth.LLAMA8B_32K), 1024, 1.0, 4, 64),
    "llama_d2_k4096_merge": (lambda: synth.make_gqa(synth.LLAMA8B_32K), 4096, 2.0, 4, 64),
    "paged_hidden_sinks": (None, 512, 2.0, 4, 64),
}


def _td_inputs(case):
    make = TD_CASES[case][0]
    if make is not None:
        return make()
    inp = synth.make_gqa(replace(synth.PAGED_QWEN14B, B=2, T=20000, len_lo=8000, len_hi=20000, seed=93))
    inp.page_table[0, 0] = -1                       # sequence 0: its sink tokens have no page
    last = (int(inp.seq_lens[1]) - 1) // 16
    inp.page_table[1, last - 1] = -1                # sequence 1: part of its local window has no page
    return inp


@pytest.mark.parametrize("case", list(TD_CASES))
def test_topdelta_parity(J, PL, case):
    _, k_max, delta, ns, nl = TD_CASES[case]
    inp = _td_inputs(case)
    c = PL.GqaCache(inp)
    c.project()
    st = PL.TopDeltaStep(c, k_max, delta, ns, nl)
    st.select()
    torch.cuda.synchronize()
    idx, cnt = _np(st.idx), _np(st.counts)
    cfg = inp.cfg
    for b in range(cfg.B):
        valid = U.unit_valid(inp, b)
        for j in range(cfg.Hkv):
            _, _, _, s, _ = U.oracle_unit(inp, b, j)
            U.check_topdelta(idx[b, j], int(cnt[b, j]), s, valid, k_max, delta, ns, nl, c.scale, cfg.G)


def test_topdelta_infinite_delta_is_topk(J, PL):
    inp = synth.make_gqa(synth.LLAMA8B_32K)
    c = PL.GqaCache(inp)
    c.project()
    st = PL.TopDeltaStep(c, 256, float("inf"))
    st.select()
    ref = PL.SparseStep(c, k=256, fused=True)
    ref.score_topk()
    torch.cuda.synchronize()
    np.testing.assert_array_equal(_np(st.idx), _np(ref.idx))
    assert np.all(_np(st.counts) == 256)


@pytest.mark.parametrize("case", ["tiny_d2_capped", "llama_d1_k1024", "paged_hidden_sinks"])
def test_topdelta_attend(J, PL, case):
    """Selection + attention (fused with the final selection when k_max <=
    512, else followed by the indexed kernel): the indices equal the
    selection-only call's, outputs match the oracle on the GPU's kept set."""
    _, k_max, delta, ns, nl = TD_CASES[case]
    inp = _td_inputs(case)
    c = PL.GqaCache(inp)
    c.project()
    sel = PL.TopDeltaStep(c, k_max, delta, ns, nl)
    sel.select()
    st = PL.TopDeltaStep(c, k_max, delta, ns, nl)
    st.run()
    torch.cuda.synchronize()
    np.testing.assert_array_equal(_np(st.idx), _np(sel.idx))
    np.testing.assert_array_equal(_np(st.counts), _np(sel.counts))
    idx, cnt, out, lse = _np(st.idx), _np(st.counts), _np(st.out), _np(st.lse)
    cfg = inp.cfg
    for b in range(cfg.B):
        for j in range(cfg.Hkv):
            K, V, _, _, hs = U.oracle_unit(inp, b, j)
            U.check_attention(inp, b, j, hs, K, V, idx[b, j][:cnt[b, j]], out, lse, c.scale)


# ---------------------------------------------------------------------------
# lossless tile screening (reading R14)
# ---------------------------------------------------------------------------
def _prev_step_seeds(PL, c, inp, k, noise=0.1, rs=7):
    """The previous decode step's selection: the top-k under a nearby query."""
    rng = np.random.default_rng(rs)
    q_prev = synth.f32_to_bf16_bits(O.bf16_to_f64(inp.q) + noise * rng.standard_normal(inp.q.shape))
    q_keep = c.q
    c.q = torch.from_numpy(q_prev.view(np.int16)).cuda()
    st = PL.SparseStep(c, k=k, fused=True)
    st.score_topk()
    torch.cuda.synchronize()
    c.q = q_keep
    return st.idx.clone()


def _screen_inputs(case):
    if case == "tiny":
        return synth.make_gqa(synth.TINY), 256
    if case == "llama_random_seeds":
        return synth.make_gqa(synth.LLAMA8B_32K), 256
    if case == "clustered_32k":
        return synth.make_gqa(replace(synth.LLAMA8B_32K, key_model="clustered", seed=95)), 256
    if case == "clustered_paged_invalid":
        inp = synth.make_gqa(replace(synth.PAGED_QWEN14B, B=2, T=20000, len_lo=9000, len_hi=20000, seed=96,
                                     key_model="clustered"))
        inp.page_table[0, 5] = -1
        inp.page_table[1, 40] = -1
        return inp, 512
    if case == "ragged_dup_seeds":
        return ragged_inputs(), 100
    if case == "clustered_long":                              # tiles past the preloaded iterations
        return synth.make_gqa(replace(synth.TINY, B=1, T=140000, key_model="clustered", seed=96)), 128
    if case.startswith("clustered_r"):                        # ranks 16, 64, 128: other kernel shapes
        r = int(case[len("clustered_r"):])
        return synth.make_gqa(replace(synth.TINY, B=2, T=20000, r=r, key_model="clustered", seed=98 + r)), 128
    return synth.make_gqa(synth.TINY), 64                     # no_seeds


@pytest.mark.parametrize("case", ["tiny", "llama_random_seeds", "clustered_32k", "clustered_paged_invalid",
                                  "ragged_dup_seeds", "no_seeds", "clustered_long", "clustered_r16",
                                  "clustered_r64", "clustered_r128"])
def test_screened_topk_lossless(J, PL, case):
    inp, k = _screen_inputs(case)
    cfg = inp.cfg
    c = PL.GqaCache(inp)
    c.project()
    if case == "llama_random_seeds":
        seeds = torch.randint(0, cfg.T, (cfg.B, cfg.Hkv, 3 * k), dtype=torch.int32, device="cuda")
    elif case == "ragged_dup_seeds":
        prev = _prev_step_seeds(PL, c, inp, k)
        seeds = torch.cat([prev, prev[:, :, :40], torch.full_like(prev[:, :, :8], 10 ** 6)], dim=2).contiguous()
    elif case == "no_seeds":
        seeds = torch.zeros((cfg.B, cfg.Hkv, 0), dtype=torch.int32, device="cuda")
    else:
        seeds = _prev_step_seeds(PL, c, inp, k)
    sc = PL.ScreenedStep(c, k, seeds)
    sc.build_bounds()
    sc.chunks()
    sc.final()
    plain = PL.SparseStep(c, k=k, fused=True)
    plain.score_topk()
    torch.cuda.synchronize()
    np.testing.assert_array_equal(_np(sc.idx), _np(plain.idx))          # the selection is unchanged
    # bounds: exact bf16 min / max per tile
    nt = (cfg.T + 63) // 64
    ntg = (nt + 63) // 64                                     # groups of 64 tiles, vector-major inside
    bd = _np(sc.bounds).reshape(cfg.B, cfg.Hkv, ntg, 2, cfg.r // 8, 64, 8).transpose(0, 1, 2, 5, 3, 4, 6)
    bd = bd.reshape(cfg.B, cfg.Hkv, ntg * 64, 2, cfg.r)
    bdf = O.bf16_to_f64(bd)
    # keep bits written after the jssa_score_topk workspace
    base = J.jssa_score_topk_workspace_size(c.desc, k)
    off = (base + 255) // 256 * 256
    nwords = 2 * ((nt + 63) // 64)
    kw = _np(sc.ws)[off:off + cfg.B * cfg.Hkv * nwords * 4].view(np.uint32).reshape(cfg.B, cfg.Hkv, nwords)
    kept_gpu = _np(sc.kept_tiles)
    sd = _np(seeds)
    dropped, total = 0, 0
    for b in range(cfg.B):
        valid = U.unit_valid(inp, b)
        Tb = int(inp.seq_lens[b])
        ntb = (Tb + 63) // 64
        for j in range(cfg.Hkv):
            K, _, Kp, s, hs = U.oracle_unit(inp, b, j)
            lo, hi = O.tile_bounds(Kp, valid)
            np.testing.assert_array_equal(bdf[b, j, :ntb, 0], lo)
            np.testing.assert_array_equal(bdf[b, j, :ntb, 1], hi)
            qp = O.project_query(inp.q[b, hs], inp.P[j])
            _, keep_o = O.screened_topk(np.where(valid, s, -np.inf), qp, Kp, sd[b, j], k, valid)
            bits = np.unpackbits(kw[b, j].view(np.uint8), bitorder="little")[:ntb].astype(bool)
            assert np.all(bits[keep_o]), "a tile the oracle keeps was dropped"
            assert kept_gpu[b, j] == bits.sum()
            dropped += ntb - bits.sum()
            total += ntb
    if case.startswith("clustered"):
        assert dropped / total > 0.3, f"clustered keys: only {dropped}/{total} tiles dropped"
    if case == "no_seeds":
        assert dropped == 0


@pytest.mark.parametrize("case", ["one_token", "span_and_clip", "paged_r48"])
def test_update_tile_bounds_equals_rebuild(J, PL, case):
    """After an append (and the matching seq_lens update), rebuilding only
    the tiles that hold the new tokens gives the bounds of a full rebuild."""
    if case == "paged_r48":
        cfg = replace(synth.PAGED_QWEN14B, B=2, T=1024, len_lo=600, len_hi=900, seed=41)
    else:
        cfg = replace(synth.TINY, B=3, T=4096, len_lo=1000, len_hi=3000, seed=42)
    inp = synth.make_gqa(cfg)
    if case == "span_and_clip":
        inp.seq_lens = np.array([2000, cfg.T - 30, 1500], np.int32)
    c = PL.GqaCache(inp)
    c.project()
    sc = PL.ScreenedStep(c, 64, torch.zeros((cfg.B, cfg.Hkv, 0), dtype=torch.int32, device="cuda"))
    sc.bounds.zero_()
    sc.build_bounds()
    lens = inp.seq_lens.astype(np.int64)
    if case == "one_token":
        n_new, pos = 1, lens.copy()
    elif case == "span_and_clip":   # overwrite from a 64-aligned start, append past max_seq, a negative start
        n_new, pos = 100, np.array([640, cfg.T - 30, -3])
    else:
        n_new, pos = 7, lens.copy()
    rng = np.random.default_rng(5)
    k_new = synth.f32_to_bf16_bits(rng.standard_normal((cfg.B, cfg.Hkv, n_new, cfg.d)))
    v_new = synth.f32_to_bf16_bits(rng.standard_normal((cfg.B, cfg.Hkv, n_new, cfg.d)))
    pos_d = PL.to_device(pos.astype(np.int32))
    before = sc.bounds.clone()
    J.jssa_append_kv(c.desc, c.K, c.V, c.Kp, PL.to_device(k_new), PL.to_device(v_new), c.P, pos_d, n_new)
    new_lens = np.maximum(lens, np.minimum(pos + n_new, cfg.T)).astype(np.int32)
    c.seq_lens.copy_(PL.to_device(new_lens))
    sc.update_bounds(pos_d, n_new)
    full = torch.zeros_like(sc.bounds)
    J.jssa_build_tile_bounds(c.desc, c.Kp, full)
    torch.cuda.synchronize()
    assert torch.equal(sc.bounds, full)
    assert not torch.equal(before, full)                      # the append did change some tiles


def test_screened_final_attend_identical(J, PL):
    inp = synth.make_gqa(replace(synth.LLAMA8B_32K, key_model="clustered", seed=97))
    c = PL.GqaCache(inp)
    c.project()
    seeds = _prev_step_seeds(PL, c, inp, 256)
    sc = PL.ScreenedStep(c, 256, seeds)
    sc.build_bounds()
    sc.chunks()
    sc.final_attend()
    plain = PL.SparseStep(c, k=256, S=1, fused=True)
    plain.run()
    torch.cuda.synchronize()
    np.testing.assert_array_equal(_np(sc.idx), _np(plain.idx))
    np.testing.assert_array_equal(_np(sc.out), _np(plain.out))
    np.testing.assert_array_equal(_np(sc.lse), _np(plain.lse))


# ---------------------------------------------------------------------------
# subspace calibration: second moments (GPU), spectral step (host library),
# oracle top-k recall of the calibrated subspace
# ---------------------------------------------------------------------------
def _valid_key_rows(inp, j):
    """Every valid token's key row of KV head j (all sequences), skipping
    tokens behind page-table entries outside [0, num_pages)."""
    out = []
    for b in range(inp.cfg.B):
        n = int(inp.seq_lens[b])
        if inp.page_table is None:
            out.append(inp.K[b, j, :n])
            continue
        t = np.arange(n)
        pg = inp.page_table[b][t // 16]
        t = t[(pg >= 0) & (pg < inp.num_pages)]
        out.append(O.paged_rows(inp.K, inp.page_table[b], j, t))
    return np.concatenate(out, axis=0) if out else np.zeros((0, 128), np.uint16)


def _moment_limit(S_ref, n_chain):
    """Worst-case fp32 summation error of a mean of products x_a x_b over a
    chain of n_chain roundings: n_chain * 2^-24 * mean|x_a x_b|, and
    mean|x_a x_b| <= sqrt(S_aa S_bb) (Cauchy-Schwarz)."""
    dg = np.sqrt(np.abs(np.diag(S_ref)))
    return 1.01 * (n_chain + 2) * 2.0 ** -24 * np.outer(dg, dg) + 1e-30


@pytest.mark.parametrize("case", ["tiny", "ragged", "paged_invalid", "llama32k"])
def test_calib_key_moments(J, PL, case):
    if case == "tiny":
        inp = synth.make_gqa(synth.TINY)
    elif case == "ragged":
        inp = ragged_inputs()
    elif case == "paged_invalid":
        inp = synth.make_gqa(replace(synth.PAGED_QWEN14B, B=3, T=20000, len_lo=1, len_hi=20000, seed=91))
        inp.page_table[0, 2] = -1
        inp.page_table[1, 0] = inp.num_pages + 7
    else:
        inp = synth.make_gqa(synth.LLAMA8B_32K)
    c = PL.GqaCache(inp)
    got = _np(PL.calib_key_moments(c))
    again = _np(PL.calib_key_moments(c))
    np.testing.assert_array_equal(got, again)              # fixed-order sums: same bits
    cfg = inp.cfg
    npb = max(1, 512 // cfg.Hkv)
    units = cfg.B * ((cfg.T + 8191) // 8192)
    n_chain = 32 * ((units + npb - 1) // npb) * 64 + npb * 4    # MFMA adds per wave + partial slots
    for j in range(cfg.Hkv):
        ref = O.key_second_moment(_valid_key_rows(inp, j))
        err = np.abs(got[j] - ref)
        assert np.all(err <= _moment_limit(ref, n_chain)), f"head {j}: max err {err.max():.3g}"
        np.testing.assert_array_equal(got[j], got[j].T)


def test_calib_query_moments(J, PL):
    cfg = synth.LLAMA8B_32K
    qs = synth.gen_calib_queries(cfg, 1000)                # 1000: a partial last batch of 64
    got = _np(PL.calib_query_moments(torch.from_numpy(qs.view(np.int16)).cuda(), cfg.Hkv))
    for j in range(cfg.Hkv):
        ref = O.query_second_moment(qs, j, cfg.G)
        err = np.abs(got[j] - ref)
        assert np.all(err <= _moment_limit(ref, 1000 + cfg.G)), f"head {j}: max err {err.max():.3g}"


def test_calib_end_to_end_recall(J, PL):
    """Calibrate on the GPU, check the basis against the oracle through the
    bound it minimises, then select with it: the indices obey the parity
    rule for that basis, and they recover far more of the exact (full-width)
    top-k than the random orthonormal basis does."""
    cfg, k, r = synth.LLAMA8B_32K, 256, 32
    inp = synth.make_gqa(cfg)
    qs = synth.gen_calib_queries(cfg, 2048)
    c = PL.GqaCache(inp)
    P_cal, ev = PL.calibrate(c, torch.from_numpy(qs.view(np.int16)).cuda(), r)
    Pn = _np(P_cal).astype(np.float64)
    for j in range(cfg.Hkv):
        Sk = O.key_second_moment(inp.K[0, j])
        Sq = O.query_second_moment(qs, j, cfg.G)
        Po, wo = O.calibrate_projection(Sq, Sk, r)
        np.testing.assert_allclose(Pn[j].T @ Pn[j], np.eye(r), atol=2e-6)
        assert O.marginal_bound(Pn[j], Sq, Sk) <= O.marginal_bound(Po, Sq, Sk) * (1 + 1e-4)
        np.testing.assert_allclose(ev[j], wo, rtol=2e-4)
        # the well-separated signal subspace (rank 24 in the synthetic keys) is the same one
        P24 = Pn[j][:, :24]
        np.testing.assert_allclose(P24 @ P24.T, Po[:, :24] @ Po[:, :24].T, atol=2e-3)
    # selection with the calibrated basis (fp32 P as stored)
    c.P = P_cal.contiguous()
    c.project()
    cal = PL.SparseStep(c, k=k, fused=True)
    cal.score_topk()
    # exact top-k: full-width scores, i.e. rank 128 with P = I on K itself
    eye = torch.eye(128, dtype=torch.float32, device="cuda").repeat(cfg.Hkv, 1, 1).contiguous()
    d_exact = J.gqa_desc(cfg.B, cfg.Hq, cfg.Hkv, 128, cfg.T, seq_lens=c.seq_lens)
    idx_exact = torch.empty((cfg.B, cfg.Hkv, k), dtype=torch.int32, device="cuda")
    ws = torch.empty(J.jssa_score_topk_workspace_size(d_exact, k), dtype=torch.uint8, device="cuda")
    J.jssa_score_topk(d_exact, c.q, eye, c.K, k, None, idx_exact, ws)
    rnd_c = PL.GqaCache(inp)
    rnd_c.project()
    rnd = PL.SparseStep(rnd_c, k=k, fused=True)
    rnd.score_topk()
    torch.cuda.synchronize()
    gi, ge, gr = _np(cal.idx), _np(idx_exact), _np(rnd.idx)
    rec_cal, rec_rnd = [], []
    for j in range(cfg.Hkv):
        hs = list(O.group_heads(j, cfg.G))
        K = inp.K[0, j]
        U.check_indices(gi[0, j], O.subspace_scores(inp.q[0, hs], Pn[j], O.project_keys(K, Pn[j])), k)
        U.check_indices(ge[0, j], O.subspace_scores(inp.q[0, hs], np.eye(128), K), k)
        rec_cal.append(O.topk_recall(gi[0, j], ge[0, j]))
        rec_rnd.append(O.topk_recall(gr[0, j], ge[0, j]))
    assert np.mean(rec_cal) >= 0.85, rec_cal
    assert np.mean(rec_cal) >= np.mean(rec_rnd) + 0.4, (rec_cal, rec_rnd)


# ---------------------------------------------------------------------------
# MLA
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("seed,B,T,k,S", [(5, 2, 6000, 512, 4), (1, 4, 4096, 2048, 16), (2, 4, 4096, 2048, 16),
                                          (3, 4, 4096, 2048, 8), (7, 4, 4096, 2048, 16), (11, 4, 4096, 2048, 16),
                                          (13, 4, 4096, 2048, 16),
                                          # ragged splits and steps: k / S not a multiple of 16, a split
                                          # smaller than a step, one slot, and the chunk-bound selection
                                          # with a partial last chunk
                                          (17, 2, 3000, 100, 3), (19, 1, 2048, 1, 1), (23, 3, 5000, 333, 7)])
def test_mla_parity(J, PL, seed, B, T, k, S):
    _mla_parity(PL, replace(synth.MLA_DSV3, B=B, T=T, k=k, seed=seed), S)


@pytest.mark.parametrize("H,B", [(48, 3), (192, 3), (128, 9)])
def test_mla_parity_head_counts(J, PL, H, B):
    """Head and sequence counts beside the workload's: with 48 heads, 16 of
    the 64 selection query classes hold no head (their parts are 0); with
    192, each class holds 3 heads, so its second chunk of 2 is partial; 9
    sequences take the query blocks through a second pass (sequences go 4
    at a time through a selection block, 8 through an absorb block)."""
    _mla_parity(PL, replace(synth.MLA_DSV3, B=B, H=H, T=3000 if B < 8 else 1500, k=300, seed=29 + H + B), 4)


def _mla_parity(PL, cfg, S):
    inp = synth.make_mla(cfg)
    st = PL.MlaStep(inp, S=S)
    st.project()
    torch.cuda.synchronize()
    Kp = _np(st.Kp)
    for b in range(cfg.B):
        np.testing.assert_array_equal(Kp[b], O.project_keys(inp.latent[b], inp.P))
    # folded selection weights U[h] = W_uk[h] . P_lat: fp64 sums rounded once
    # to fp32, so within 2^-24 relative of the fp64 product (plus fp64 noise)
    P64 = inp.P.astype(np.float64)
    W64 = O.bf16_to_f64(inp.W_uk)
    Uref = W64 @ P64[:512]
    mag = np.abs(W64) @ np.abs(P64[:512])
    Ug = _np(st.U).astype(np.float64)
    assert np.all(np.abs(Ug - Uref) <= 2.0 ** -24 * np.abs(Uref) + 1e-12 * mag), np.abs(Ug - Uref).max()
    st.run()
    torch.cuda.synchronize()
    qsel = _np(st.q_sel)
    for b in range(cfg.B):
        qa = O.mla_absorbed_query(inp.q_nope[b], inp.q_rope[b], inp.W_uk)
        U.check_close(_np(st.q_abs)[b], qa, tol=1e-4, what="absorbed query")
        # part g of the selection query: the heads h = g, g + 64, ... each
        # contribute P^T qa_h = (W_uk[h] P_lat)^T q_nope_h + P_rope^T q_rope_h;
        # the parts add up to P^T sum_h qa
        qbar = qa.sum(0)
        parts = np.stack([sum((P64.T @ qa[h] for h in range(g, cfg.H, 64)), np.zeros(cfg.r)) for g in range(64)])
        U.check_close(qsel[b], parts, tol=1e-4, what="selection query parts")
        U.check_close(qsel[b].astype(np.float64).sum(0), P64.T @ qbar, tol=1e-4, what="selection query")
    idx, out, lse = _np(st.idx), _np(st.out), _np(st.lse)
    for b in range(cfg.B):
        s = O.mla_scores(inp.q_nope[b], inp.q_rope[b], inp.W_uk, inp.P, O.project_keys(inp.latent[b], inp.P))
        U.check_indices(idx[b], s, cfg.k)
        sel = idx[b][idx[b] >= 0]
        o, _, l = O.mla_attend_explicit(inp.q_nope[b], inp.q_rope[b], inp.W_uk, inp.W_uv, inp.latent[b][sel],
                                        st.scale)
        U.check_close(out[b], o, what=f"mla out b={b}")
        U.check_close(lse[b], l, what=f"mla lse b={b}")


_MLA_TOPK_CASES = [
    # name, B, max_seq, k, lengths (None: all max_seq), kind
    ("full_128k", 4, 131072, 2048, None, "random"),
    ("ragged", 4, 131072, 2048, [131072, 100003, 5000, 1], "random"),
    ("unaligned_rows", 3, 70001, 1000, [70001, 69999, 40000], "random"),
    ("clustered", 2, 65536, 1024, None, "clustered"),
    ("all_tied", 2, 32768, 512, None, "tied"),
    ("small_k", 2, 131072, 64, None, "random"),
    ("k_4096", 1, 131072, 4096, None, "random"),
    ("no_bound_path", 2, 4096, 2048, None, "random"),
]


@pytest.mark.parametrize("case", _MLA_TOPK_CASES, ids=[c[0] for c in _MLA_TOPK_CASES])
def test_mla_score_topk_matches_separate_passes(J, case):
    """jssa_mla_score_topk (score stream with per-chunk lists, one final
    pass over their union with the on-device check and the per-row
    selection from scores when a chunk held more of the top k than its list)
    against jssa_mla_score + jssa_topk on the same inputs: identical scores
    and identical indices, and the indices equal the oracle's selection on
    those scores. Covers the list path where the lists suffice (full 128K,
    unaligned rows, k = 64 and 4096), rows they do not suffice for (a short
    ragged row with k near its length, 600 clustered top tokens in two
    chunks, every score tied) and the plain path (too few chunks for
    lists)."""
    name, B, T, k, lens, kind = case
    r, H = 64, 128
    rng = np.random.default_rng(sum(map(ord, name)))
    # the query in 64 parts (as jssa_mla_absorb_q writes it); qsel is their
    # sum, for building keys near it
    qshare = (rng.standard_normal((B, 64, r)) / 8.0).astype(np.float32)
    qsel = qshare.astype(np.float64).sum(1)
    if kind == "tied":
        kp = np.zeros((B, T, r), np.float32)            # every score 0: the lowest indices win
    else:
        kp = rng.standard_normal((B, T, r)).astype(np.float32)
        if kind == "clustered":                         # 600 near-identical top tokens in two chunks
            kp[:, 3000:3600] = 4.0 * qsel[:, None, :] + 0.01 * rng.standard_normal((B, 600, r))
    kp_bits = synth.f32_to_bf16_bits(kp).view(np.int16)
    lens_np = np.full(B, T, np.int32) if lens is None else np.asarray(lens, np.int32)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    q_t, kp_t, sl = dev(qshare), dev(kp_bits), dev(lens_np)
    desc = J.mla_desc(B, H, r, T, seq_lens=sl)
    s1 = torch.empty((B, T), dtype=torch.float32, device="cuda")
    s2 = torch.empty_like(s1)
    i1 = torch.empty((B, k), dtype=torch.int32, device="cuda")
    i2 = torch.empty_like(i1)
    ws1 = torch.empty(max(J.jssa_mla_score_topk_workspace_size(desc, k), 16), dtype=torch.uint8, device="cuda")
    ws2 = torch.empty(max(J.jssa_topk_workspace_size(B, 1, T, k), 16), dtype=torch.uint8, device="cuda")
    print(f"[case] mla score_topk {name} B={B} T={T} k={k}", flush=True)
    J.jssa_mla_score_topk(desc, q_t, kp_t, k, s1, i1, ws1)
    J.jssa_mla_score(desc, q_t, kp_t, s2)
    J.jssa_topk(B, 1, T, sl, s2, k, i2, ws2)
    torch.cuda.synchronize()
    sc1, sc2 = _np(s1), _np(s2)
    np.testing.assert_array_equal(sc1.view(np.uint32), sc2.view(np.uint32))
    np.testing.assert_array_equal(_np(i1), _np(i2))
    for b in range(B):
        n = int(lens_np[b])
        np.testing.assert_array_equal(_np(i1)[b], O.select_topk(sc1[b, :n].astype(np.float64), k))


@pytest.mark.parametrize("S", [1, 5, 16, 64])
@pytest.mark.parametrize("B,H", [(3, 32), (5, 16)])
def test_mla_combine_up_matches_two_calls(J, S, B, H):
    """jssa_mla_combine_up_v against jssa_combine + jssa_mla_up_v on random
    partials (some splits empty: lse -inf) and random W_uv: same lse and
    output up to fp32 summation order; sequence counts that leave the last
    pass of 4 partial (3, 5)."""
    rng = np.random.default_rng(100 + S + 7 * B)
    po = rng.standard_normal((B, H, S, 512)).astype(np.float32)
    pl = (3.0 * rng.standard_normal((B, H, S))).astype(np.float32)
    pl[0, 0, :] = -np.inf                                 # a row with no weight at all
    if S > 1:
        pl[1, :, ::2] = -np.inf                           # rows with empty splits
    wuv = synth.f32_to_bf16_bits(rng.standard_normal((H, 128, 512)) / np.sqrt(512)).view(np.int16)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    po_t, pl_t, w_t = dev(po), dev(pl), dev(wuv)
    desc = J.mla_desc(B, H, 64, 1024)
    out1 = torch.empty((B, H, 128), dtype=torch.float32, device="cuda")
    lse1 = torch.empty((B, H), dtype=torch.float32, device="cuda")
    olat = torch.empty((B, H, 512), dtype=torch.float32, device="cuda")
    out2 = torch.empty_like(out1)
    lse2 = torch.empty_like(lse1)
    print(f"[case] mla combine_up S={S}", flush=True)
    J.jssa_mla_combine_up_v(desc, S, po_t, pl_t, w_t, out1, lse1)
    J.jssa_combine(B, H, S, 512, po_t, pl_t, olat, 0, lse2)
    J.jssa_mla_up_v(desc, olat, w_t, out2)
    torch.cuda.synchronize()
    np.testing.assert_allclose(_np(lse1), _np(lse2), rtol=1e-6, atol=1e-6)
    np.testing.assert_allclose(_np(out1), _np(out2), rtol=1e-5, atol=1e-6)
    assert np.all(_np(out1)[0, 0] == 0.0) and _np(lse1)[0, 0] == -np.inf


# ---------------------------------------------------------------------------
# full size: the 128K x B=16 workload in the launch configuration the
# benchmark times; sampled units against the oracle, properties everywhere
# ---------------------------------------------------------------------------
def test_full_size_128k_b16_sampled(J, PL):
    """The 128K x B=16 workload in the launch configuration the benchmark
    times (fused chunk pass, then final selection + attention at one split),
    checked on all 128 (sequence, KV head) units against the oracle
    (indices, outputs, log-sum-exps, sampled projected-key rows) and
    everywhere for the properties that hold at any size; the separate entry
    points must give the same indices."""
    cfg = synth.BATCHED_128K
    inp = synth.make_gqa(cfg)
    c = PL.GqaCache(inp)
    c.project()
    st = PL.SparseStep(c, k=cfg.k, fused=True, keep_scores=False)
    assert [f.__name__ for f in st.stages()] == ["score_chunks", "final_attend"]
    st.run()
    sep = PL.SparseStep(c, k=cfg.k, fused=False)
    sep.run()
    torch.cuda.synchronize()
    np.testing.assert_array_equal(_np(st.idx), _np(sep.idx))
    idx, out, lse = _np(st.idx), _np(st.out), _np(st.lse)
    assert np.all(np.diff(idx, axis=-1) > 0) and idx.min() >= 0 and idx.max() < cfg.T
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    rng = np.random.default_rng(0)
    rows = rng.choice(cfg.T, 2048, replace=False)
    kp_rows = _np(c.Kp[:, :, torch.from_numpy(rows).cuda()])

    def unit(bj):
        b, j = bj
        K, V, Kp, s, hs = U.oracle_unit(inp, b, j)
        np.testing.assert_array_equal(kp_rows[b, j], Kp[rows])
        swaps = U.check_indices(idx[b, j], s, cfg.k)
        U.check_attention(inp, b, j, hs, K, V, idx[b, j], out, lse, c.scale)
        return swaps
    # every (sequence, KV head) unit of the step against the oracle
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(8) as ex:
        list(ex.map(unit, [(b, j) for b in range(cfg.B) for j in range(cfg.Hkv)]))


def test_full_size_128k_b16_extensions_sampled(J, PL):
    """The 128K x B=16 workload through the scope's extension rows, in the
    configurations the benchmark times: top-delta selection + attention
    (delta 2, k_max 256), screening with the previous step's selection as
    seeds, and the calibration moments; checked on sampled units (and one
    KV head over all sequences) against the oracle."""
    cfg = synth.BATCHED_128K
    inp = synth.make_gqa(cfg)
    c = PL.GqaCache(inp)
    c.project()
    k = cfg.k
    units = [(0, 0), (5, 3), (11, 6), (15, 7)]
    # top-delta + attention
    td = PL.TopDeltaStep(c, k, 2.0, 4, 64)
    td.run()
    torch.cuda.synchronize()
    idx, cnt, out, lse = _np(td.idx), _np(td.counts), _np(td.out), _np(td.lse)
    assert np.all(np.isfinite(out[cnt.repeat(cfg.G, axis=1) > 0]))
    oracle_units = {}
    for b, j in units:
        K, V, Kp, s, hs = U.oracle_unit(inp, b, j)
        oracle_units[(b, j)] = (K, V, Kp, s, hs)
        valid = np.ones(s.shape[0], bool)
        U.check_topdelta(idx[b, j], int(cnt[b, j]), s, valid, k, 2.0, 4, 64, c.scale, cfg.G)
        U.check_attention(inp, b, j, hs, K, V, idx[b, j][:cnt[b, j]], out, lse, c.scale)
    # screening with the previous step's selection as seeds
    seeds = _prev_step_seeds(PL, c, inp, k)
    sc = PL.ScreenedStep(c, k, seeds)
    sc.build_bounds()
    sc.chunks()
    sc.final()
    plain = PL.SparseStep(c, k=k, fused=True)
    plain.score_topk()
    torch.cuda.synchronize()
    np.testing.assert_array_equal(_np(sc.idx), _np(plain.idx))
    sd = _np(seeds)
    base = J.jssa_score_topk_workspace_size(c.desc, k)
    off = (base + 255) // 256 * 256
    nt = cfg.T // 64
    kw = _np(sc.ws)[off:off + cfg.B * cfg.Hkv * (nt // 32) * 4].view(np.uint32).reshape(cfg.B, cfg.Hkv, nt // 32)
    for b, j in units:
        K, V, Kp, s, hs = oracle_units[(b, j)]
        qp = O.project_query(inp.q[b, hs], inp.P[j])
        _, keep_o = O.screened_topk(s, qp, Kp, sd[b, j], k)
        bits = np.unpackbits(kw[b, j].view(np.uint8), bitorder="little")[:nt].astype(bool)
        assert np.all(bits[keep_o])
    # calibration moments: one KV head over all 16 sequences, and the queries
    Sk = _np(PL.calib_key_moments(c))
    ref = O.key_second_moment(inp.K[:, 2].reshape(-1, cfg.d))
    npb = 512 // cfg.Hkv
    n_chain = 32 * ((cfg.B * (cfg.T // 8192) + npb - 1) // npb) * 64 + npb * 4
    assert np.all(np.abs(Sk[2] - ref) <= _moment_limit(ref, n_chain))
    qs = synth.gen_calib_queries(cfg, 4096)
    Sq = _np(PL.calib_query_moments(torch.from_numpy(qs.view(np.int16)).cuda(), cfg.Hkv))
    for j in (0, 7):
        refq = O.query_second_moment(qs, j, cfg.G)
        assert np.all(np.abs(Sq[j] - refq) <= _moment_limit(refq, 4096 + cfg.G))


def test_full_size_qwen_paged_k2048_sampled(J, PL):
    """Paged, ragged Qwen3-14B-shaped workload at full size with the largest
    budget of its sweep, in the benchmark's launch configuration (chunk pass,
    merge levels + final selection, four-split attention, combine)."""
    cfg = replace(synth.PAGED_QWEN14B, k=2048)
    inp = synth.make_gqa(cfg)
    c = PL.GqaCache(inp)
    c.project()
    st = PL.SparseStep(c, k=cfg.k, fused=True, keep_scores=False)
    assert st.S == 4
    st.run()
    torch.cuda.synchronize()
    idx, out, lse = _np(st.idx), _np(st.out), _np(st.lse)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    for b, j in [(0, 0), (5, 3), (7, 7)]:
        n = min(cfg.k, int(inp.seq_lens[b]))
        assert np.all(np.diff(idx[b, j, :n]) > 0) and np.all(idx[b, j, n:] == -1)
        K, V, Kp, s, hs = U.oracle_unit(inp, b, j)
        U.check_indices(idx[b, j], s, cfg.k)
        U.check_attention(inp, b, j, hs, K, V, idx[b, j][:n], out, lse, c.scale)


def test_full_size_mla_sampled(J, PL):
    """DeepSeek-V3-shaped MLA workload at full size (B=4, T=128K, k=2048) in
    the benchmark's launch configuration (16 splits), two sequences checked
    against the explicit (non-absorbed) oracle on the GPU's selected set."""
    cfg = synth.MLA_DSV3
    inp = synth.make_mla(cfg)
    st = PL.MlaStep(inp)
    assert st.S == 16
    st.project()
    st.run()
    torch.cuda.synchronize()
    idx, out, lse = _np(st.idx), _np(st.out), _np(st.lse)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    for b in (0, 3):
        assert np.all(np.diff(idx[b]) > 0)
        Kp = O.project_keys(inp.latent[b], inp.P)
        rows = np.random.default_rng(b).choice(cfg.T, 1024, replace=False)
        np.testing.assert_array_equal(_np(st.Kp[b, torch.from_numpy(rows).cuda()]), Kp[rows])
        s = O.mla_scores(inp.q_nope[b], inp.q_rope[b], inp.W_uk, inp.P, Kp)
        U.check_indices(idx[b], s, cfg.k)
        o, _, l = O.mla_attend_explicit(inp.q_nope[b], inp.q_rope[b], inp.W_uk, inp.W_uv, inp.latent[b][idx[b]],
                                        st.scale)
        U.check_close(out[b], o, what=f"mla out b={b}")
        U.check_close(lse[b], l, what=f"mla lse b={b}")
