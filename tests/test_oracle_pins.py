"""Pins of the CPU oracle against facts that do not come from the oracle:
hand-derived fixtures, closed forms, library routines and brute force.

Each test names the operation it pins; the operations are those of the JSSA
decode step (JSSA abstract on weekinpapers, Abstract; digest on ai4snews,
Synopsis and Interpretation)."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import jssa_oracle as O
from token_level_sparse_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _num(expr: str) -> float:
    expr = expr.replace("^", "**")
    return float(eval(expr, {"__builtins__": {}}, {"e": math.e, "ln": math.log}))


def bf16(x):
    return synth.f32_to_bf16_bits(np.asarray(x, np.float64))


# ---------------------------------------------------------------------------
# bf16 rounding (projected key storage)
# ---------------------------------------------------------------------------
def _exact_nearest_bf16(x: float) -> int:
    """Brute force: among bf16 patterns next to the truncated pattern, pick
    the nearest in exact rational arithmetic; ties go to the even pattern."""
    if x == 0.0:
        return 0x8000 if math.copysign(1.0, x) < 0 else 0
    base = int(np.float32(x).view(np.uint32) >> 16)
    best = None
    xf = Fraction(x)
    for cand in range(max(base - 2, 0) if x > 0 else base - 2, base + 3):
        if cand < 0 or cand > 0xFFFF:
            continue
        v = np.uint32(cand << 16).view(np.float32)
        if not np.isfinite(v):
            continue
        if (v < 0) != (x < 0) and v != 0:
            continue
        dist = abs(Fraction(float(v)) - xf)
        key = (dist, cand & 1)
        if best is None or key < best[0]:
            best = (key, cand)
    return best[1]


def test_bf16_golden_values():
    g = _golden("bf16_rounding.json")
    for c in g["cases"]:
        x = _num(c["x"]) if "^" in c["x"] else float(c["x"])
        got = int(O.round_to_bf16(np.array([x]))[0])
        assert got == int(c["bits"], 16), (c, hex(got))


def test_bf16_matches_torch_on_fp32_inputs():
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 2**32, size=20000, dtype=np.uint64).astype(np.uint32)
    x32 = bits.view(np.float32)
    x32 = x32[np.isfinite(x32) & (np.abs(x32) < 3.3e38)]
    ref = torch.from_numpy(x32.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = O.round_to_bf16(x32.astype(np.float64))
    np.testing.assert_array_equal(got, ref)


def test_bf16_exact_nearest_on_fp64_inputs():
    rng = np.random.default_rng(8)
    xs = np.concatenate([rng.standard_normal(1500) * 10.0 ** rng.integers(-30, 30, 1500),
                         1.0 + (2 * rng.integers(0, 128, 200) + 1) * 2.0 ** -8,   # exact halfway points
                         rng.standard_normal(200) * 2.0 ** -128])                  # subnormal range
    got = O.round_to_bf16(xs)
    for x, g in zip(xs, got):
        assert int(g) == _exact_nearest_bf16(float(x)), (x, hex(int(g)))


# ---------------------------------------------------------------------------
# Projected key cache
# ---------------------------------------------------------------------------
def test_projection_identity_is_bitwise_copy():
    rng = np.random.default_rng(1)
    K = bf16(rng.standard_normal((64, 128)))
    np.testing.assert_array_equal(O.project_keys(K, np.eye(128, dtype=np.float32)), K)


def test_projection_signed_permutation_is_exact():
    rng = np.random.default_rng(2)
    K = bf16(rng.standard_normal((32, 128)))
    perm = rng.permutation(128)[:32]
    sign = rng.choice([-1.0, 1.0], 32)
    P = np.zeros((128, 32), np.float32)
    P[perm, np.arange(32)] = sign
    expect = bf16(synth.bf16_bits_to_f32(K)[:, perm] * sign)
    np.testing.assert_array_equal(O.project_keys(K, P), expect)


def test_projection_exact_rational_tiny():
    rng = np.random.default_rng(3)
    T, d, r = 5, 16, 4
    K = bf16(rng.standard_normal((T, d)))
    P = rng.standard_normal((d, r)).astype(np.float32)
    Kf = synth.bf16_bits_to_f32(K)
    got = O.project_keys(K, P)
    for t in range(T):
        for c in range(r):
            exact = sum(Fraction(float(Kf[t, i])) * Fraction(float(P[i, c])) for i in range(d))
            assert int(got[t, c]) == _exact_nearest_bf16(float(exact)), (t, c)


# ---------------------------------------------------------------------------
# Subspace scores
# ---------------------------------------------------------------------------
def test_score_golden_group_sum():
    g = _golden("score_group_sum.json")
    q = bf16(g["q"])
    K = bf16(g["K"])
    s = O.subspace_scores(q, np.eye(4, dtype=np.float32), K)
    np.testing.assert_array_equal(s, np.array(g["scores"]))


def test_score_identity_projection_equals_exact_qk():
    """r = d, P = I: the subspace score is the exact group-summed q.k,
    computed here with torch fp64 from the raw operands."""
    rng = np.random.default_rng(4)
    G, T, d = 4, 300, 128
    q = bf16(rng.standard_normal((G, d)))
    K = bf16(rng.standard_normal((T, d)))
    s = O.subspace_scores(q, np.eye(d, dtype=np.float32), O.project_keys(K, np.eye(d, dtype=np.float32)))
    qt = torch.from_numpy(synth.bf16_bits_to_f32(q).astype(np.float64))
    Kt = torch.from_numpy(synth.bf16_bits_to_f32(K).astype(np.float64))
    ref = (Kt @ qt.T).sum(dim=1).numpy()
    np.testing.assert_allclose(s, ref, rtol=1e-12, atol=1e-12)


def test_score_linearity_per_head_form():
    rng = np.random.default_rng(5)
    G, T, d, r = 5, 200, 128, 48
    q = bf16(rng.standard_normal((G, d)))
    P = synth.gen_projection(11, 1, d, r)[0]
    Kp = bf16(rng.standard_normal((T, r)))
    s = O.subspace_scores(q, P, Kp)
    Kpf = synth.bf16_bits_to_f32(Kp).astype(np.float64)
    per_head = sum(Kpf @ (P.astype(np.float64).T @ synth.bf16_bits_to_f32(q[h]).astype(np.float64))
                   for h in range(G))
    np.testing.assert_allclose(s, per_head, rtol=1e-12, atol=1e-12 * np.abs(per_head).max())


def test_score_exact_rational_tiny():
    rng = np.random.default_rng(6)
    G, T, d, r = 3, 12, 16, 8
    q = bf16(rng.standard_normal((G, d)))
    P = rng.standard_normal((d, r)).astype(np.float32)
    Kp = bf16(rng.standard_normal((T, r)))
    s = O.subspace_scores(q, P, Kp)
    qf = synth.bf16_bits_to_f32(q)
    Kpf = synth.bf16_bits_to_f32(Kp)
    qbar = [sum(Fraction(float(qf[h, i])) for h in range(G)) for i in range(d)]
    qp = [sum(Fraction(float(P[i, c])) * qbar[i] for i in range(d)) for c in range(r)]
    for t in range(T):
        exact = sum(qp[c] * Fraction(float(Kpf[t, c])) for c in range(r))
        assert abs(s[t] - float(exact)) <= 1e-13 * max(1.0, abs(float(exact)))


# ---------------------------------------------------------------------------
# Top-k selection
# ---------------------------------------------------------------------------
def test_topk_golden_ties():
    g = _golden("topk_ties.json")
    s = np.array(g["scores"])
    for c in g["cases"]:
        np.testing.assert_array_equal(O.select_topk(s, c["k"]), c["idx"])


@pytest.mark.parametrize("seed", range(20))
def test_topk_brute_force_small(seed):
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(1, 65))
    s = rng.integers(-4, 5, n).astype(np.float64) * 0.5     # many exact ties
    if seed % 2:
        s = rng.standard_normal(n)
    k = int(rng.integers(1, 70))
    ref = sorted(sorted(range(n), key=lambda t: (-s[t], t))[:k])
    got = O.select_topk(s, k)
    assert list(got[:len(ref)]) == ref
    assert all(x == -1 for x in got[len(ref):])


def test_topk_special_cases():
    rng = np.random.default_rng(9)
    s = rng.standard_normal(1000)
    np.testing.assert_array_equal(O.select_topk(s, 1000), np.arange(1000))
    assert O.select_topk(s, 1)[0] == np.argmax(s.astype(np.float32))
    eq = np.full(50, 2.0)
    np.testing.assert_array_equal(O.select_topk(eq, 7), np.arange(7))
    # scores equal in fp32 (the decision precision) tie on index
    a = 1.0
    b = 1.0 + 2.0 ** -40
    np.testing.assert_array_equal(O.select_topk(np.array([a, b]), 1), [0])


def _val(x: str) -> float:
    try:
        return float(x)
    except ValueError:
        return _num(x)


def test_kth_score_and_absent_tokens_golden():
    """The k-th score (the anchor of the index tie band) and the selection
    with absent (-inf) tokens against hand-derived values; it distinguishes
    -0.0 from +0.0 by sign, so the returned token is pinned, not only its
    magnitude."""
    g = _golden("kth_score_hand.json")
    s = np.array([_val(x) for x in g["scores"]])
    for c in g["cases"]:
        want = _val(c["kth"])
        got = O.kth_score(s, c["k"])
        assert got == want and math.copysign(1.0, got) == math.copysign(1.0, want), (c, got)
        np.testing.assert_array_equal(O.select_topk(s, c["k"]), c["idx"])
    f = g["fp32_tie"]
    s2 = np.array([_val(x) for x in f["scores"]])
    assert s2[1] != s2[0]                              # distinct in fp64, equal in fp32
    assert O.kth_score(s2, f["k"]) == _val(f["kth"])
    np.testing.assert_array_equal(O.select_topk(s2, f["k"]), f["idx"])
    e = g["none_exist"]
    s3 = np.array([_val(x) for x in e["scores"]])
    np.testing.assert_array_equal(O.select_topk(s3, e["k"]), e["idx"])
    with pytest.raises(ValueError):
        O.kth_score(s3, e["k"])


@pytest.mark.parametrize("seed", range(8))
def test_kth_score_brute_force_small(seed):
    """k-th score against a plain Python sort of (score, index) pairs on
    small rows with many exact ties, absent tokens and signed zeros."""
    rng = np.random.default_rng(300 + seed)
    n = int(rng.integers(1, 40))
    s = rng.integers(-3, 4, n).astype(np.float64) * 0.25
    s[rng.random(n) < 0.2] = -np.inf
    s[s == 0] = np.where(rng.random(int((s == 0).sum())) < 0.5, -0.0, 0.0)
    alive = [t for t in range(n) if s[t] != -np.inf]
    ranked = sorted(alive, key=lambda t: (-(s[t] + 0.0), t))
    for k in range(1, n + 3):
        if not ranked:
            with pytest.raises(ValueError):
                O.kth_score(s, k)
            continue
        assert O.kth_score(s, k) == s[ranked[min(k, len(ranked)) - 1]]
        sel = sorted(ranked[:k])
        assert list(O.select_topk(s, k)) == sel + [-1] * (k - len(sel))


@pytest.mark.parametrize("seed", range(6))
def test_fp32_decision_differs_from_exact_only_within_one_ulp(seed):
    """Reading R3 decides on fp32-rounded scores. Rounding to nearest is
    monotone, so against a selection decided on the exact (fp64) scores the
    two sets may differ only among tokens within one fp32 ulp (2^-23
    relative) of the k-th score. Built with many exact scores that differ by
    less than an fp32 ulp."""
    rng = np.random.default_rng(500 + seed)
    m = 1000
    n, k = 3 * m, 3 * int(rng.integers(20, 200)) + 1   # the boundary splits one triple
    base = np.abs(rng.standard_normal(m)) + 0.1
    # three exact scores per value, all one fp32 value; the lowest index
    # holds the smallest, so the two rules keep different members
    s = np.concatenate([base * (1 - 2.0 ** -35), base, base * (1 + 2.0 ** -30)])
    exact = sorted(range(n), key=lambda t: (-s[t], t))[:k]
    got = O.select_topk(s, k)
    diff = np.setxor1d(got, exact)
    sk = O.kth_score(s, k)
    assert np.all(np.abs(s[diff] - sk) <= 2.0 ** -23 * abs(sk)), diff
    assert diff.size > 0                               # the test does reach the coarsening


# ---------------------------------------------------------------------------
# Attention over the selected set, combine
# ---------------------------------------------------------------------------
def test_attention_golden():
    g = _golden("attention_two_tokens.json")
    q, K, V = bf16(g["q"]), bf16(g["K"]), bf16(g["V"])
    for c in g["cases"]:
        sel = c["sel"]
        o, lse = O.attend(q, K[sel], V[sel], 1.0)
        np.testing.assert_allclose(o[0], [_num(x) for x in c["o"]], rtol=1e-14, atol=1e-15)
        assert abs(lse[0] - _num(c["lse"])) < 1e-14


def test_dense_matches_torch_sdpa():
    """Dense attention of a whole GQA layer = torch's fp64 scaled-dot-product
    attention with KV heads repeated over their query groups."""
    rng = np.random.default_rng(10)
    Hq, Hkv, T, d = 8, 2, 77, 128
    G = Hq // Hkv
    q = bf16(rng.standard_normal((Hq, d)))
    K = bf16(rng.standard_normal((Hkv, T, d)))
    V = bf16(rng.standard_normal((Hkv, T, d)))
    out = np.zeros((Hq, d))
    for j in range(Hkv):
        hs = list(O.group_heads(j, G))
        out[hs] = O.dense_unit(q[hs], K[j], V[j], 1 / math.sqrt(d))[0]
    f = lambda a: torch.from_numpy(synth.bf16_bits_to_f32(a).astype(np.float64))
    ref = torch.nn.functional.scaled_dot_product_attention(
        f(q)[:, None, :], f(K).repeat_interleave(G, 0), f(V).repeat_interleave(G, 0))[:, 0, :]
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-12, atol=1e-12)


def test_sparse_with_k_equal_T_is_dense():
    cfg = synth.TINY
    inp = synth.make_gqa(cfg)
    j = 1
    hs = list(O.group_heads(j, cfg.G))
    K, V = inp.K[0, j], inp.V[0, j]
    Kp = O.project_keys(K, inp.P[j])
    _, idx, o, lse = O.sparse_unit(inp.q[0, hs], inp.P[j], Kp, K, V, cfg.T, 1 / math.sqrt(cfg.d))
    od, lsed = O.dense_unit(inp.q[0, hs], K, V, 1 / math.sqrt(cfg.d))
    np.testing.assert_array_equal(idx, np.arange(cfg.T))
    np.testing.assert_array_equal(o, od)
    np.testing.assert_array_equal(lse, lsed)


def test_attention_k1_and_convexity():
    rng = np.random.default_rng(11)
    q = bf16(rng.standard_normal((4, 128)))
    K = bf16(rng.standard_normal((40, 128)))
    V = bf16(rng.standard_normal((40, 128)))
    o, lse = O.attend(q, K[[17]], V[[17]], 0.1)
    np.testing.assert_array_equal(o, np.broadcast_to(synth.bf16_bits_to_f32(V[17]), o.shape))
    sel = [1, 5, 9, 30]
    o, lse = O.attend(q, K[sel], V[sel], 0.1)
    Vf = synth.bf16_bits_to_f32(V[sel])
    assert np.all(o <= Vf.max(0) + 1e-12) and np.all(o >= Vf.min(0) - 1e-12)
    logits = 0.1 * synth.bf16_bits_to_f32(q).astype(np.float64) @ synth.bf16_bits_to_f32(K[sel]).T
    np.testing.assert_allclose(np.exp(logits - lse[:, None]).sum(1), 1.0, rtol=1e-13)


@pytest.mark.parametrize("splits", [1, 2, 3, 7, 64])
def test_combine_split_invariance(splits):
    rng = np.random.default_rng(12 + splits)
    q = bf16(rng.standard_normal((1, 128)))
    K = bf16(rng.standard_normal((256, 128)) * 2)
    V = bf16(rng.standard_normal((256, 128)))
    o_all, lse_all = O.attend(q, K, V, 1 / math.sqrt(128))
    cuts = np.sort(rng.choice(np.arange(1, 256), splits - 1, replace=False)) if splits > 1 else []
    parts = np.split(np.arange(256), cuts)
    po, pl = zip(*[O.attend(q, K[p], V[p], 1 / math.sqrt(128)) for p in parts])
    o, lse = O.combine(np.stack([x[0] for x in po]), np.array([x[0] for x in pl]))
    np.testing.assert_allclose(o, o_all[0], rtol=1e-12, atol=1e-13)
    assert abs(lse - lse_all[0]) < 1e-12
    # an empty split contributes nothing
    o2, lse2 = O.combine(np.vstack([np.stack([x[0] for x in po]), np.full((1, 128), 5.0)]),
                         np.append([x[0] for x in pl], -np.inf))
    np.testing.assert_allclose(o2, o, rtol=1e-15)


# ---------------------------------------------------------------------------
# Per-head independence
# ---------------------------------------------------------------------------
def test_per_head_selection_independence():
    cfg = synth.TINY
    inp = synth.make_gqa(cfg)
    Kp = [O.project_keys(inp.K[0, j], inp.P[j]) for j in range(cfg.Hkv)]
    sel = []
    for j in range(cfg.Hkv):
        hs = list(O.group_heads(j, cfg.G))
        sel.append(O.select_topk(O.subspace_scores(inp.q[0, hs], inp.P[j], Kp[j]), cfg.k))
    # perturb KV head 1's keys and queries: head 0's set is bit-unchanged
    q2 = inp.q.copy()
    q2[0, cfg.G:] = bf16(np.random.default_rng(0).standard_normal((cfg.G, cfg.d)))
    Kp1 = Kp[1][::-1].copy()
    s0 = O.subspace_scores(q2[0, :cfg.G], inp.P[0], Kp[0])
    np.testing.assert_array_equal(O.select_topk(s0, cfg.k), sel[0])
    s1 = O.subspace_scores(q2[0, cfg.G:], inp.P[1], Kp1)
    assert not np.array_equal(O.select_topk(s1, cfg.k), sel[1])
    # the two heads pick distinct sets
    assert not np.array_equal(sel[0], sel[1])


# ---------------------------------------------------------------------------
# Paged addressing
# ---------------------------------------------------------------------------
def test_paged_matches_contiguous():
    from dataclasses import replace
    cfg = replace(synth.PAGED_QWEN14B, B=2, T=2048, len_lo=1000, len_hi=2048)
    paged = synth.make_gqa(cfg)
    flat = synth.make_gqa(replace(cfg, paged=False))
    np.testing.assert_array_equal(paged.seq_lens, flat.seq_lens)
    table = paged.page_table
    used = table[table >= 0]
    assert sorted(used.tolist()) == list(range(paged.num_pages))          # a permutation
    for b in range(cfg.B):
        n = int(paged.seq_lens[b])
        for j in range(cfg.Hkv):
            t = np.arange(n)
            np.testing.assert_array_equal(O.logical_rows(paged.K, b, j, t, table), flat.K[b, j, :n])
            np.testing.assert_array_equal(O.logical_rows(paged.V, b, j, t, table), flat.V[b, j, :n])
    # identity table over an unpermuted pool reads the same rows
    ident = np.arange(cfg.T // 16, dtype=np.int32)[None].repeat(cfg.B, 0)
    pool = flat.K.reshape(cfg.B, cfg.Hkv, cfg.T // 16, 16, cfg.d).transpose(0, 2, 1, 3, 4)
    pool = pool.reshape(cfg.B * cfg.T // 16, cfg.Hkv, 16, cfg.d)
    for b in range(cfg.B):
        t = np.arange(int(flat.seq_lens[b]))
        np.testing.assert_array_equal(O.logical_rows(pool, b, 3, t, ident + b * (cfg.T // 16)), flat.K[b, 3, t])


def test_paged_rows_reject_positions_without_a_page():
    """Reading R7: a table entry outside [0, pages) holds no token; reading a
    row there is an error, and page_valid marks exactly those positions."""
    pool = np.arange(3 * 1 * 16 * 2, dtype=np.uint16).reshape(3, 1, 16, 2)
    table = np.array([2, -1, 0, 3], np.int32)                   # pages 2, none, 0, none
    t = np.arange(64)
    np.testing.assert_array_equal(O.page_valid(table, t, 3), (t < 16) | ((t >= 32) & (t < 48)))
    np.testing.assert_array_equal(O.paged_rows(pool, table, 0, [0, 17 + 16, 15]),
                                  pool[[2, 0, 2], 0, [0, 1, 15]])
    for bad in ([16], [63], [5, 20]):
        with pytest.raises(ValueError):
            O.paged_rows(pool, table, 0, bad)


# ---------------------------------------------------------------------------
# MLA
# ---------------------------------------------------------------------------
def _tiny_mla(seed=21, H=4, L=32, R=8, dn=16, dv=8, n=40):
    rng = np.random.default_rng(seed)
    return (bf16(rng.standard_normal((H, dn))), bf16(rng.standard_normal((H, R))),
            bf16(rng.standard_normal((H, dn, L)) / 4), bf16(rng.standard_normal((H, dv, L)) / 4),
            bf16(rng.standard_normal((n, L + R))))


def test_mla_absorbed_equals_explicit():
    qn, qr, Wk, Wv, C = _tiny_mla()
    scale = 1 / math.sqrt(24)
    o, o_lat, lse = O.mla_attend_explicit(qn, qr, Wk, Wv, C, scale)
    qa = O.mla_absorbed_query(qn, qr, Wk)                       # [H, L+R]
    Cf = synth.bf16_bits_to_f32(C).astype(np.float64)
    logits = scale * qa @ Cf.T
    p = np.exp(logits - logits.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    o_abs = np.einsum("hvc,hc->hv", synth.bf16_bits_to_f32(Wv).astype(np.float64), p @ Cf[:, :32])
    np.testing.assert_allclose(o, o_abs, rtol=1e-12, atol=1e-12)


def test_mla_brute_force_loops():
    qn, qr, Wk, Wv, C = _tiny_mla(H=2, L=8, R=4, dn=4, dv=3, n=6)
    f = lambda a: synth.bf16_bits_to_f32(a).astype(np.float64)
    qn_, qr_, Wk_, Wv_, C_ = map(f, (qn, qr, Wk, Wv, C))
    o, _, lse = O.mla_attend_explicit(qn, qr, Wk, Wv, C, 0.5)
    for h in range(2):
        logits = []
        for t in range(6):
            kn = [sum(Wk_[h, a, c] * C_[t, c] for c in range(8)) for a in range(4)]
            logits.append(0.5 * (sum(qn_[h, a] * kn[a] for a in range(4)) +
                                 sum(qr_[h, c] * C_[t, 8 + c] for c in range(4))))
        m = max(logits)
        w = [math.exp(x - m) for x in logits]
        Z = sum(w)
        olat = [sum(w[t] * C_[t, c] for t in range(6)) / Z for c in range(8)]
        for v in range(3):
            assert abs(o[h, v] - sum(Wv_[h, v, c] * olat[c] for c in range(8))) < 1e-12
        assert abs(lse[h] - (m + math.log(Z))) < 1e-12


def test_mla_sparse_with_k_equal_T_is_dense():
    """With k = T the selection keeps every latent row, so sparse MLA equals
    dense MLA over the whole latent cache (the k = T fact of the decode step
    on the shared-latent path)."""
    qn, qr, Wk, Wv, C = _tiny_mla(n=37)
    P = synth.gen_projection(7, 1, 40, 8)[0]
    s = O.mla_scores(qn, qr, Wk, P, O.project_keys(C, P))
    idx = O.select_topk(s, C.shape[0])
    np.testing.assert_array_equal(idx, np.arange(C.shape[0]))
    dense = O.mla_attend_explicit(qn, qr, Wk, Wv, C, 0.3)
    sparse = O.mla_attend_explicit(qn, qr, Wk, Wv, C[idx], 0.3)
    for a, b in zip(dense, sparse):
        np.testing.assert_array_equal(a, b)
    # and with k < T the output differs (the pin is not vacuous)
    part = O.mla_attend_explicit(qn, qr, Wk, Wv, C[O.select_topk(s, 5)], 0.3)
    assert not np.allclose(part[0], dense[0])


def test_mla_score_is_summed_per_head_projection():
    qn, qr, Wk, Wv, C = _tiny_mla()
    rng = np.random.default_rng(3)
    P = synth.gen_projection(3, 1, 40, 8)[0]
    Kp = O.project_keys(C, P)
    s = O.mla_scores(qn, qr, Wk, P, Kp)
    qa = O.mla_absorbed_query(qn, qr, Wk)
    Kpf = synth.bf16_bits_to_f32(Kp).astype(np.float64)
    ref = sum(Kpf @ (P.astype(np.float64).T @ qa[h]) for h in range(qa.shape[0]))
    np.testing.assert_allclose(s, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


# ---------------------------------------------------------------------------
# subspace calibration (JSSA abstract on weekinpapers, Abstract: a shared
# query-key subspace from a marginal bound on the score-preservation error
# with a closed-form spectral solution; the reading is spelled out in the
# oracle's header, R12)
# ---------------------------------------------------------------------------
def _orthonormal(rng, d, r):
    q, _ = np.linalg.qr(rng.standard_normal((d, r)))
    return q


def test_calib_second_moments_brute_force():
    """Second moments against explicit Python loops over rows and heads."""
    rng = np.random.default_rng(11)
    K = bf16(rng.standard_normal((5, 4)))
    Kf = [[O.bf16_to_f64(K[t, i]) for i in range(4)] for t in range(5)]
    want = [[sum(float(Kf[t][a]) * float(Kf[t][b]) for t in range(5)) / 5 for b in range(4)] for a in range(4)]
    np.testing.assert_allclose(O.key_second_moment(K), want, rtol=1e-15, atol=1e-15)
    q = bf16(rng.standard_normal((3, 6, 4)))          # N=3 samples, Hq=6, G=3 -> 2 KV heads
    for j in range(2):
        qb = [[sum(float(O.bf16_to_f64(q[n, h, i])) for h in range(3 * j, 3 * j + 3)) for i in range(4)]
              for n in range(3)]
        want = [[sum(qb[n][a] * qb[n][b] for n in range(3)) / 3 for b in range(4)] for a in range(4)]
        np.testing.assert_allclose(O.query_second_moment(q, j, 3), want, rtol=1e-14, atol=1e-14)


def test_calib_diagonal_closed_form():
    """Diagonal moments: the calibrated basis is the coordinate axes with the
    largest a_i/sum(a) + b_i/sum(b), in that order, each +1."""
    a = np.array([4.0, 1.0, 9.0, 0.5, 2.0, 3.5])
    b = np.array([0.1, 6.0, 0.2, 0.3, 5.0, 0.4])
    w = a / a.sum() + b / b.sum()
    P, ev = O.calibrate_projection(np.diag(a), np.diag(b), 3)
    want_axes = list(np.argsort(-w)[:3])
    for c, ax in enumerate(want_axes):
        e = np.zeros(6)
        e[ax] = 1.0
        np.testing.assert_allclose(P[:, c], e, atol=1e-12)
        assert ev[c] == pytest.approx(w[ax], rel=1e-12)


def test_calib_bound_holds_and_is_met_by_rank_r_data():
    """The mean |score error| never exceeds the marginal bound (a theorem for
    sample moments too); on data inside an r-dim subspace the calibrated basis
    preserves every score exactly while a random one does not."""
    rng = np.random.default_rng(12)
    d, r = 16, 4
    qb = rng.standard_normal((200, d)) * np.linspace(0.2, 2.0, d)
    K = rng.standard_normal((300, d)) @ rng.standard_normal((d, d)) / 4
    Sq, Sk = qb.T @ qb / 200, K.T @ K / 300
    Pc, _ = O.calibrate_projection(Sq, Sk, r)
    for P in [Pc] + [_orthonormal(rng, d, r) for _ in range(5)]:
        assert O.preservation_error(P, qb, K) <= O.marginal_bound(P, Sq, Sk) * (1 + 1e-12)
    B = _orthonormal(rng, d, r)                            # the data's subspace
    qb = rng.standard_normal((50, r)) @ B.T
    K = rng.standard_normal((80, r)) @ B.T
    Sq, Sk = qb.T @ qb / 50, K.T @ K / 80
    Pc, _ = O.calibrate_projection(Sq, Sk, r)
    assert O.preservation_error(Pc, qb, K) < 1e-12
    assert abs(O.marginal_bound(Pc, Sq, Sk)) < 1e-12
    assert O.preservation_error(_orthonormal(rng, d, r), qb, K) > 1e-2


def test_calib_minimises_bound_brute_force():
    """d = 3, r = 1: a dense search over unit vectors on the half sphere finds
    no basis with a smaller marginal bound than the calibrated one, and the
    best grid point lies next to it."""
    rng = np.random.default_rng(13)
    A = rng.standard_normal((3, 3))
    Bm = rng.standard_normal((3, 3))
    Sq, Sk = A @ A.T, Bm @ Bm.T * 3
    Pc, _ = O.calibrate_projection(Sq, Sk, 1)
    best, arg = np.inf, None
    for th in np.linspace(0, np.pi / 2, 181):
        for ph in np.linspace(0, 2 * np.pi, 721):
            v = np.array([[np.sin(th) * np.cos(ph)], [np.sin(th) * np.sin(ph)], [np.cos(th)]])
            val = O.marginal_bound(v, Sq, Sk)
            if val < best:
                best, arg = val, v
    assert O.marginal_bound(Pc, Sq, Sk) <= best + 1e-12
    assert abs(float(arg[:, 0] @ Pc[:, 0])) > 0.999


def test_calib_invariances():
    """Scaling either moment leaves the basis unchanged (trace-normalised
    operator); the basis is orthonormal and sign-fixed."""
    rng = np.random.default_rng(14)
    A = rng.standard_normal((8, 8))
    Bm = rng.standard_normal((8, 3))
    Sq, Sk = A @ A.T, Bm @ Bm.T + 0.1 * np.eye(8)
    P1, _ = O.calibrate_projection(Sq, Sk, 3)
    P2, _ = O.calibrate_projection(7.0 * Sq, 0.01 * Sk, 3)
    np.testing.assert_allclose(P1, P2, atol=1e-10)
    np.testing.assert_allclose(P1.T @ P1, np.eye(3), atol=1e-12)
    for c in range(3):
        i = int(np.argmax(np.abs(P1[:, c])))
        assert P1[i, c] > 0


def test_topk_recall_hand_values():
    assert O.topk_recall([1, 2, 3, -1], [2, 3, 4, 5]) == 0.5
    assert O.topk_recall([7, 8], [8, 7]) == 1.0
    assert O.topk_recall([-1, -1], [-1, -1]) == 1.0


# ---------------------------------------------------------------------------
# top-delta selection (Faster Than Flash review on evolve.pub, Summary and
# FAQ: the top-delta rule with a sink/local pseudo-max; reading R13 in the
# oracle's header)
# ---------------------------------------------------------------------------
def test_topdelta_golden_hand():
    g = _golden("topdelta_hand.json")
    s, valid = np.array(g["scores"]), np.array(g["valid"], bool)
    for c in g["cases"]:
        idx, cnt = O.select_topdelta(s, c["k_max"], c["delta"], c["n_sink"], c["n_local"], g["scale"], g["G"], valid)
        np.testing.assert_array_equal(idx, c["idx"])
        assert cnt == c["count"]


def test_topdelta_infinite_delta_is_topk():
    rng = np.random.default_rng(31)
    for _ in range(10):
        n = int(rng.integers(1, 300))
        s = rng.integers(-5, 6, n) * 0.25 if rng.random() < 0.5 else rng.standard_normal(n)
        k = int(rng.integers(1, 400))
        idx, cnt = O.select_topdelta(s, k, np.inf, 4, 16, 0.1, 4)
        np.testing.assert_array_equal(idx, O.select_topk(s, k))
        assert cnt == min(k, n)


def test_topdelta_failsafe_and_monotone():
    """The pseudo-max never exceeds the true max, so the kept set (uncapped)
    contains every token within delta of the true max; a larger delta keeps
    a superset."""
    rng = np.random.default_rng(32)
    for _ in range(20):
        n = int(rng.integers(8, 500))
        s = rng.standard_normal(n) * 3
        G, scale = int(rng.integers(1, 9)), float(rng.uniform(0.05, 1.0))
        d1, d2 = sorted(rng.uniform(0, 10, 2))
        i1, c1 = O.select_topdelta(s, n, d1, 4, 32, scale, G)
        i2, c2 = O.select_topdelta(s, n, d2, 4, 32, scale, G)
        k1, k2 = set(i1[:c1]), set(i2[:c2])
        assert k1 <= k2
        s32 = s.astype(np.float32).astype(np.float64)
        true_set = set(np.nonzero(s32 >= s32.max() - d1 * G / scale)[0])
        assert true_set <= k1


@pytest.mark.parametrize("seed", range(12))
def test_topdelta_brute_force_small(seed):
    rng = np.random.default_rng(200 + seed)
    n = int(rng.integers(0, 40))
    s = rng.integers(-3, 4, n) * 0.5
    valid = rng.random(n) < 0.8
    ns, nl = int(rng.integers(0, 5)), int(rng.integers(0, 9))
    delta, G, scale, k = float(rng.choice([0.0, 0.3, 1.0, 5.0])), 2, 0.5, int(rng.integers(1, 45))
    m = None
    for t in range(n):
        if valid[t] and (t < ns or t >= n - nl):
            m = s[t] if m is None else max(m, s[t])
    kept = [t for t in range(n) if valid[t] and (m is None or s[t] >= m - delta * G / scale)]
    kept = sorted(sorted(kept, key=lambda t: (-s[t], t))[:k])
    idx, cnt = O.select_topdelta(s, k, delta, ns, nl, scale, G, valid)
    assert cnt == len(kept)
    np.testing.assert_array_equal(idx, kept + [-1] * (k - len(kept)))


# ---------------------------------------------------------------------------
# lossless screening (DoSA article on cctest.ai, How the method works: seed
# threshold, upper-bound certificate, unchanged top-k; reading R14 in the
# oracle's header)
# ---------------------------------------------------------------------------
def _clustered_keys(rng, n, r, seg=256, noise=0.1):
    """Keys in segments of `seg` tokens around their own random centre (a
    topic per segment): tiles inside a segment are narrow boxes."""
    c = rng.standard_normal(((n + seg - 1) // seg, r))
    return bf16(np.repeat(c, seg, axis=0)[:n] + noise * rng.standard_normal((n, r)))


def test_screen_hand_values():
    """Two-token tile [[1, -2], [3, 0]], qp = [2, -1]: lo = [1, -2], hi = [3, 0],
    ub = max(2, 6) + max(2, 0) = 8 >= the scores 4 and 6. A third, invalid
    row does not widen the box."""
    Kp = bf16([[1, -2], [3, 0], [100, 100]])
    lo, hi = O.tile_bounds(Kp, valid=[1, 1, 0], tile=3)
    np.testing.assert_array_equal(lo, [[1, -2]])
    np.testing.assert_array_equal(hi, [[3, 0]])
    assert O.tile_upper_bounds([2.0, -1.0], lo, hi)[0] == 8.0
    lo, hi = O.tile_bounds(bf16([[2, 5]] * 4), tile=4)          # identical rows: the bound is attained
    assert O.tile_upper_bounds([1.5, -0.5], lo, hi)[0] == 1.5 * 2 - 0.5 * 5


def test_screen_seed_closed_form():
    """tau is the k-th largest score over the distinct valid seeds: scores
    s_t = t, seeds {990, 5, 700, 990, -1, 5000, 800}, k = 3 -> {990, 800,
    700, 5} ranked, tau = 700; with token 800 invalid, tau = 5; fewer than k
    valid seeds -> -inf."""
    s = np.arange(1000.0)
    seeds = [990, 5, 700, 990, -1, 5000, 800]
    assert O.seed_threshold(s, seeds, 3) == 700.0
    v = np.ones(1000, bool)
    v[800] = False
    assert O.seed_threshold(s, seeds, 3, v) == 5.0
    assert O.seed_threshold(s, seeds, 5) == -np.inf


@pytest.mark.parametrize("seed", range(6))
def test_screen_bounds_sound_and_lossless(seed):
    """Every tile bound covers its tokens' scores, tau never exceeds the
    k-th score, and the screened selection equals the plain one, whatever
    the seeds. With the previous step's selection as seeds (a nearby query)
    and clustered keys, most tiles are skipped."""
    rng = np.random.default_rng(300 + seed)
    n, r = int(rng.integers(600, 6000)), 16
    Kp = _clustered_keys(rng, n, r) if seed % 2 else bf16(rng.standard_normal((n, r)))
    qp = rng.standard_normal(r) * 3
    valid = rng.random(n) < 0.97
    Kf = O.bf16_to_f64(Kp)
    s = np.where(valid, Kf @ qp, -np.inf)
    k = int(rng.integers(1, 80))
    lo, hi = O.tile_bounds(Kp, valid)
    ub = O.tile_upper_bounds(qp, lo, hi)
    for i in range(ub.shape[0]):
        seg = s[i * 64:(i + 1) * 64]
        if np.isfinite(seg.max()):
            assert ub[i] >= seg.max() - 1e-9 * (1 + abs(seg.max()))
    qprev = qp + 0.3 * rng.standard_normal(r)                  # the previous step's query
    seeds = O.select_topk(np.where(valid, Kf @ qprev, -np.inf), k)
    seeds_rand = rng.integers(0, n, 3 * k)
    s32 = s.astype(np.float32).astype(np.float64)
    for sd in (seeds, seeds_rand):
        tau = O.seed_threshold(s, sd, k, valid)
        assert tau <= np.sort(s32)[::-1][k - 1]
        got, keep = O.screened_topk(s, qp, Kp, sd, k, valid)
        np.testing.assert_array_equal(got, O.select_topk(s, k))
    if seed % 2:
        _, keep = O.screened_topk(s, qp, Kp, seeds, k, valid)
        assert keep.mean() < 0.7, f"clustered keys: {keep.mean():.2f} of tiles kept"
