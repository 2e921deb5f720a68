"""CPU oracle for the JSSA sparse decode step: plain, slow, fp64.

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check of the entry
module and the CPU-baseline leg of the benchmark may import this module. The
HIP library never calls it and shares no code with it; the only thing both
sides share is the seeded input generator (token_level_sparse_amd.synth),
which holds none of the method's arithmetic.

Each function computes one step of the method directly from its definition,
in float64, with numpy primitives (matmul, exp, sort) as the only building
blocks. Sources (page title, section):

* [JSSA-A]  "Joint Subspace Sparse Attention for Efficient Long-Context
            Decoding" (weekinpapers, arXiv 2610.19026v1), Abstract.
* [JSSA-S]  ai4snews digest "JSSA makes token-level sparse decoding
            gather-free ...", Synopsis.
* [JSSA-I]  same digest, Interpretation (scoring space, gather-free reads).
* [JSSA-P]  same digest, Perspective (GQA / hybrid / MLA coverage).
* [DOSA]    "DoSA Makes Sparse Attention Selection Conditional Without
            Approximation" (cctest.ai), How the method works (seed threshold,
            upper-bound certificate, exact top-k preserved).
* [FFD]     "Faster Than Flash: Exploiting Attention Sparsity for Efficient
            Long-Context Decoding" (evolve.pub review), Summary, Key claims
            and FAQ (the top-delta rule, the sink/local pseudo-max and its
            fail-safe property).

Readings where the pages are silent:

R1 group aggregation: a KV head's score is the raw sum over its GQA group of
   the query heads' subspace scores (by linearity: the projected group-summed
   query dotted with the projected key).
R2 the projected key cache stores bf16(K_j P_j), rounded to nearest-even
   from the exact (fp64) product.
R3 selection: among the tokens that exist, the first min(k, n) of the
   total order (score descending, token index ascending), returned ascending
   by index and padded with -1; n counts the existing tokens. A token past
   T_b or behind an invalid page has the score -inf and does not exist: it
   is never selected. Scores are compared after rounding to fp32 (-0.0 ranks
   equal to +0.0, ties go to the lower index). The pages fix no precision
   for the selection, and the GPU ranks fp32 scores; a comparison that turns
   floats into an integer result is taken here in that precision. Rounding
   to nearest is monotone, so it never reverses two exact scores; it only
   merges exact scores that round to one fp32 value into a tie. The result
   therefore differs from a selection on exact scores only among tokens
   within one fp32 ulp (2^-23 relative) of the k-th score, far inside the
   1e-4 tie band of the index comparison, and on fp32 score rows (the
   top-k entry point's input) it is the exact selection.
R4 attention over a selected set: softmax(scale * q K_S^T) V_S per query
   head, base e, with log-sum-exp lse = m + ln(sum exp(l - m)); an empty set
   gives o = 0, lse = -inf.
R5 split partials merge by weights exp(lse_s) (log-sum-exp combine).
R6 query head h reads KV head floor(h / G).
R7 paged layout: token t of sequence b lives in page table[b][t // 16], slot
   t % 16, of a pool laid out [pages, Hkv, 16, width]. A table entry outside
   [0, pages) holds no token: its 16 positions do not exist (score -inf).
R8 MLA: keys are [W_uk[h] c[:512]; c[512:]], values c[:512], output
   W_uv[h] (sum_t p_t c_t[:512]); the selection score projects the summed
   absorbed query [W_uk[h]^T q_nope; q_rope] and the latent row through one
   rank-r basis; one selected set per sequence.
(R9 to R11 fix the GPU side's precision and output type only.)
R13 top-delta selection ([FFD], the top-delta rule and its fail-safe
   pseudo-max, applied per token and per KV head instead of per block): the
   approximate logit of token t is the group-mean subspace logit
   l_t = scale * s_t / G. The pseudo-max m~ is the largest s_t over the
   first n_sink and the last n_local positions of the sequence (valid tokens
   only); a token is kept when scale * s_t / G >= scale * m~ / G - delta,
   i.e. s_t >= m~ - delta * G / scale. The kept set is capped at k_max
   tokens by the order of R3 and listed like R3's, with its size. No valid
   special token (or T_b = 0): nothing is filtered. Decisions are taken on
   scores rounded to fp32, the threshold in fp64.
R14 lossless screening ([DOSA]: a seed set gives a lower bound on the
   winning threshold; candidates whose upper bound falls below it are
   dropped before exact scoring, and the top-k is unchanged). Applied to the
   one r-dim dot product s_t = qp . Kp_t: a tile of 64 consecutive tokens
   has the box bound ub = sum_c max(qp_c lo_c, qp_c hi_c), lo and hi the
   per-dimension minimum and maximum of its valid projected keys, so
   ub >= s_t for each of its tokens. The seed set is a caller-given list of
   token indices per (sequence, KV head) (in decoding, e.g. the previous
   step's selection); tau is the k-th largest fp32 score over its distinct
   valid entries (-inf with fewer than k). A tile with ub < tau holds no
   token of the top-k (each of its scores is below tau <= the k-th score)
   and is skipped.
R12 subspace calibration ([JSSA-A]: the subspace minimises a token-score
   preservation error, which is bounded by a marginal objective with a
   closed-form spectral solution; the formulas are not on the pages). The
   error of one (query, key) pair is e = qbar^T k - qbar^T P P^T k =
   qbar^T Q k with Q = I - P P^T, qbar the group-summed query. Since Q is a
   projector, |e| = |(Q qbar)^T (Q k)| <= |Q qbar| |Q k| <= (lam |Q qbar|^2 +
   |Q k|^2 / lam) / 2 for any lam > 0 (Cauchy-Schwarz, then AM-GM), so
   E|e| <= tr(Q (lam S_q + S_k / lam)) / 2 with S_q = E[qbar qbar^T] and
   S_k = E[k k^T]: a bound that depends on the two marginal second moments
   only and is linear in Q. Over orthonormal P [d,r] it is smallest when P
   spans the top-r eigenvectors of M = lam S_q + S_k / lam (Ky Fan). lam =
   sqrt(tr S_k / tr S_q) makes the two terms equal at P = 0; up to a
   positive factor M is then S_q / tr S_q + S_k / tr S_k. Columns are
   ordered by descending eigenvalue, each signed so that its entry of
   largest magnitude (first such index on a tie) is positive.
"""
from __future__ import annotations

import numpy as np

PAGE = 16


# ---------------------------------------------------------------------------
# bf16 helpers (storage type of q, K, V, Kp)
# ---------------------------------------------------------------------------
def bf16_to_f64(bits) -> np.ndarray:
    """Widen bf16 bit patterns exactly: a bf16 is the top half of an fp32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def round_to_bf16(x) -> np.ndarray:
    """Round float64 values to bf16 (8 significant bits), nearest-even, and
    return the bit patterns. Written from the definition: scale the value so
    its quantum becomes 1, round to the nearest integer (ties to even), scale
    back. The quantum of a bf16 normal in [2^(e-1), 2^e) is 2^(e-8); bf16
    subnormals share the fixed quantum 2^-133."""
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    quantum_exp = np.maximum(e - 8, -133)
    rounded = np.ldexp(np.rint(np.ldexp(x, -quantum_exp)), quantum_exp)
    with np.errstate(over="ignore"):          # beyond the bf16 range -> inf
        r32 = rounded.astype(np.float32)
    return (r32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


# ---------------------------------------------------------------------------
# Step 1 (append / build): the projected key cache  [JSSA-S], [JSSA-A]
# Scoring happens in a low-dimensional subspace shared by queries and keys;
# keys are kept projected so that scoring reads r values per token (R2).
# ---------------------------------------------------------------------------
def project_keys(K_bits, P) -> np.ndarray:
    """Kp = bf16(K P) for rows K [n,d] (bf16 bits) and basis P [d,r]."""
    return round_to_bf16(bf16_to_f64(K_bits) @ np.asarray(P, np.float64))


# ---------------------------------------------------------------------------
# Step 2: subspace scores per KV head  [JSSA-S], [JSSA-I], [JSSA-A]
# ---------------------------------------------------------------------------
def group_heads(j: int, G: int) -> range:
    """Query heads served by KV head j (R6)."""
    return range(j * G, (j + 1) * G)


def project_query(q_group_bits, P_j) -> np.ndarray:
    """qp = P_j^T sum_h q_h over the group's query heads (R1)."""
    qbar = bf16_to_f64(q_group_bits).sum(axis=0)
    return np.asarray(P_j, np.float64).T @ qbar


def subspace_scores(q_group_bits, P_j, Kp_bits) -> np.ndarray:
    """s_t = qp . Kp_t for every row of Kp [n,r]; fp64."""
    return bf16_to_f64(Kp_bits) @ project_query(q_group_bits, P_j)


# ---------------------------------------------------------------------------
# Step 3: distinct top-k token set per KV head  [JSSA-S], [JSSA-A]
# ---------------------------------------------------------------------------
def selection_order(scores) -> np.ndarray:
    """The existing tokens (score > -inf) in the order of R3: fp32-rounded
    score descending, then token index ascending."""
    s32 = np.asarray(scores, np.float64).astype(np.float32).astype(np.float64)
    t = np.nonzero(s32 > -np.inf)[0]
    return t[np.lexsort((t, -s32[t]))]


def select_topk(scores, k: int) -> np.ndarray:
    """Indices of the first min(k, n) existing tokens in the order (score
    desc, index asc), sorted ascending and padded with -1 to length k (R3)."""
    keep = np.sort(selection_order(scores)[:k])
    out = np.full(k, -1, np.int64)
    out[:keep.shape[0]] = keep
    return out


def kth_score(scores, k: int) -> float:
    """The (fp64) score of the last token the selection keeps: the min(k, n)-th
    existing token of R3's order. No token kept: ValueError."""
    order = selection_order(scores)
    if order.shape[0] == 0 or k < 1:
        raise ValueError("the selection keeps no token")
    return float(np.asarray(scores, np.float64)[order[min(k, order.shape[0]) - 1]])


# ---------------------------------------------------------------------------
# Step 4: attention over the selected rows  [JSSA-I], [JSSA-A]
# Selected rows are used where they lie in the cache; the arithmetic is that
# of ordinary softmax attention restricted to the selected set (R4).
# ---------------------------------------------------------------------------
def attend(q_bits, K_rows_bits, V_rows_bits, scale: float):
    """o [G,d], lse [G] for query rows q [G,d] over key/value rows [n,d]."""
    q = bf16_to_f64(q_bits)
    G = q.shape[0]
    V_rows_bits = np.asarray(V_rows_bits)
    n = V_rows_bits.shape[0]
    if n == 0:
        return np.zeros((G, V_rows_bits.shape[1])), np.full(G, -np.inf)
    Kr = bf16_to_f64(K_rows_bits)
    Vr = bf16_to_f64(V_rows_bits)
    logits = scale * (q @ Kr.T)
    m = logits.max(axis=1)
    w = np.exp(logits - m[:, None])
    l = w.sum(axis=1)
    return (w @ Vr) / l[:, None], m + np.log(l)


def combine(part_o, part_lse):
    """Merge split partials o_s [S,d], lse_s [S] into (o [d], lse) (R5)."""
    part_o = np.asarray(part_o, np.float64)
    part_lse = np.asarray(part_lse, np.float64)
    m = part_lse.max()
    if m == -np.inf:
        return np.zeros(part_o.shape[-1]), -np.inf
    w = np.exp(part_lse - m)
    return (w[:, None] * part_o).sum(axis=0) / w.sum(), m + np.log(w.sum())


# ---------------------------------------------------------------------------
# Paged addressing (R7)
# ---------------------------------------------------------------------------
def page_valid(table_row, t, num_pages: int) -> np.ndarray:
    """Whether logical positions t have a page (R7)."""
    pg = np.asarray(table_row, np.int64)[np.asarray(t, np.int64) // PAGE]
    return (pg >= 0) & (pg < num_pages)


def paged_rows(pool, table_row, j: int, t) -> np.ndarray:
    """Rows of KV head j at logical positions t from a pool [pages,Hkv,16,w].
    Every position must have a page (ValueError otherwise: such a position
    holds no row, R7)."""
    t = np.asarray(t, np.int64)
    pool = np.asarray(pool)
    pg = np.asarray(table_row, np.int64)[t // PAGE]
    if np.any((pg < 0) | (pg >= pool.shape[0])):
        raise ValueError("a position without a page holds no row")
    return pool[pg, j, t % PAGE]


def logical_rows(cache, b: int, j: int, t, page_table=None) -> np.ndarray:
    if page_table is None:
        return np.asarray(cache)[b, j, np.asarray(t, np.int64)]
    return paged_rows(cache, page_table[b], j, t)


# ---------------------------------------------------------------------------
# Whole step on one (sequence, KV head) unit
# ---------------------------------------------------------------------------
def sparse_unit(q_group_bits, P_j, Kp_bits, K_bits, V_bits, k: int, scale: float):
    """Score -> select -> attend for one (b, j) whose cache rows are given
    logically ([T_b, .]). Returns (scores fp64, idx, o [G,d], lse [G])."""
    s = subspace_scores(q_group_bits, P_j, Kp_bits)
    idx = select_topk(s, k)
    sel = idx[idx >= 0]
    o, lse = attend(q_group_bits, np.asarray(K_bits)[sel], np.asarray(V_bits)[sel], scale)
    return s, idx, o, lse


def dense_unit(q_group_bits, K_bits, V_bits, scale: float):
    """Full-KV attention for one (b, j): every cached row t < T_b."""
    return attend(q_group_bits, K_bits, V_bits, scale)


# ---------------------------------------------------------------------------
# MLA shared latent cache  [JSSA-P] (R8)
# ---------------------------------------------------------------------------
def mla_absorbed_query(q_nope_bits, q_rope_bits, W_uk_bits) -> np.ndarray:
    """qa_h = [W_uk[h]^T q_nope_h ; q_rope_h] for every head: [H, d_c]."""
    qn = bf16_to_f64(q_nope_bits)            # [H, d_nope]
    W = bf16_to_f64(W_uk_bits)               # [H, d_nope, d_latent]
    q_lat = np.einsum("hi,hic->hc", qn, W)
    return np.concatenate([q_lat, bf16_to_f64(q_rope_bits)], axis=1)


def mla_scores(q_nope_bits, q_rope_bits, W_uk_bits, P, Kp_lat_bits) -> np.ndarray:
    """s_t = (P^T sum_h qa_h) . Kp_lat_t; one score per latent row."""
    qbar = mla_absorbed_query(q_nope_bits, q_rope_bits, W_uk_bits).sum(axis=0)
    return bf16_to_f64(Kp_lat_bits) @ (np.asarray(P, np.float64).T @ qbar)


def mla_attend_explicit(q_nope_bits, q_rope_bits, W_uk_bits, W_uv_bits, C_rows_bits, scale: float):
    """Explicit (non-absorbed) MLA attention over latent rows C [n, d_c]:
    per head, keys k_t = [W_uk[h] c_t[:L]; c_t[L:]], values v_t = c_t[:L],
    output W_uv[h] (sum_t p_t v_t). Returns (o [H, d_v], o_lat [H, L], lse [H])."""
    qn = bf16_to_f64(q_nope_bits)
    qr = bf16_to_f64(q_rope_bits)
    Wk = bf16_to_f64(W_uk_bits)
    Wv = bf16_to_f64(W_uv_bits)
    C = bf16_to_f64(C_rows_bits)
    H, L = Wk.shape[0], Wk.shape[2]
    n = C.shape[0]
    o = np.zeros((H, Wv.shape[1]))
    o_lat = np.zeros((H, L))
    lse = np.full(H, -np.inf)
    if n == 0:
        return o, o_lat, lse
    c_lat, c_rope = C[:, :L], C[:, L:]
    for h in range(H):
        k_nope = c_lat @ Wk[h].T                       # [n, d_nope]
        logits = scale * (k_nope @ qn[h] + c_rope @ qr[h])
        m = logits.max()
        w = np.exp(logits - m)
        o_lat[h] = (w @ c_lat) / w.sum()
        o[h] = Wv[h] @ o_lat[h]
        lse[h] = m + np.log(w.sum())
    return o, o_lat, lse


# ---------------------------------------------------------------------------
# Subspace calibration (R12)  [JSSA-A]; [JSSA-I] (queries and keys kept
# together; recall of the exact top-k measures the ranking); [JSSA-P]
# (bounding the marginal objective bounds the error of the exact scores)
# ---------------------------------------------------------------------------
def key_second_moment(K_rows_bits) -> np.ndarray:
    """S_k = mean over the rows k of K [n, d] of k k^T (fp64); zeros if n = 0."""
    K = bf16_to_f64(K_rows_bits).reshape(-1, np.asarray(K_rows_bits).shape[-1])
    if K.shape[0] == 0:
        return np.zeros((K.shape[1], K.shape[1]))
    return K.T @ K / K.shape[0]


def query_second_moment(q_samples_bits, j: int, G: int) -> np.ndarray:
    """S_q = mean over samples n of qbar_n qbar_n^T, qbar_n = sum of the query
    heads of KV head j's group in sample n (q [N, Hq, d], bf16 bits)."""
    q = bf16_to_f64(q_samples_bits)[:, group_heads(j, G), :].sum(axis=1)   # [N, d]
    if q.shape[0] == 0:
        return np.zeros((q.shape[1], q.shape[1]))
    return q.T @ q / q.shape[0]


def marginal_operator(S_q, S_k) -> np.ndarray:
    """M = S_q / tr S_q + S_k / tr S_k (R12); a zero-trace term is left out."""
    M = np.zeros_like(np.asarray(S_q, np.float64))
    for S in (S_q, S_k):
        t = float(np.trace(S))
        if t > 0:
            M = M + np.asarray(S, np.float64) / t
    return M


def sign_fix(V) -> np.ndarray:
    """Sign each column so that its entry of largest magnitude is positive."""
    V = np.array(V, np.float64)
    for c in range(V.shape[1]):
        i = int(np.argmax(np.abs(V[:, c])))
        if V[i, c] < 0:
            V[:, c] = -V[:, c]
    return V


def calibrate_projection(S_q, S_k, r: int):
    """P [d, r]: the top-r eigenvectors of the marginal operator (R12), columns
    by descending eigenvalue, sign-fixed; also returns the r eigenvalues."""
    M = marginal_operator(S_q, S_k)
    w, V = np.linalg.eigh(M)                   # ascending
    order = np.argsort(-w, kind="stable")[:r]
    return sign_fix(V[:, order]), w[order]


def marginal_bound(P, S_q, S_k) -> float:
    """tr(Q (lam S_q + S_k / lam)) / 2 with Q = I - P P^T and lam =
    sqrt(tr S_k / tr S_q): the upper bound on the mean |e| (R12)."""
    P = np.asarray(P, np.float64)
    Q = np.eye(P.shape[0]) - P @ P.T
    lam = np.sqrt(np.trace(S_k) / np.trace(S_q))
    return float(np.trace(Q @ (lam * np.asarray(S_q) + np.asarray(S_k) / lam)) / 2)


def preservation_error(P, qbar, K) -> float:
    """Mean over all (query, key) pairs of |qbar^T k - qbar^T P P^T k| for
    queries qbar [Nq, d] and keys K [Nk, d] given as float arrays."""
    P = np.asarray(P, np.float64)
    qbar = np.asarray(qbar, np.float64)
    K = np.asarray(K, np.float64)
    exact = qbar @ K.T
    approx = (qbar @ P) @ (K @ P).T
    return float(np.abs(exact - approx).mean())


def topk_recall(selected, reference) -> float:
    """|selected & reference| / |reference| over the valid (>= 0) entries."""
    a = set(int(x) for x in np.asarray(selected).ravel() if x >= 0)
    b = set(int(x) for x in np.asarray(reference).ravel() if x >= 0)
    return len(a & b) / len(b) if b else 1.0


# ---------------------------------------------------------------------------
# Top-delta selection (R13)  [FFD]
# ---------------------------------------------------------------------------
def topdelta_threshold(scores, delta: float, n_sink: int, n_local: int, scale: float, G: int,
                       valid=None) -> float:
    """s_thr = m~ - delta * G / scale, m~ the largest fp32-rounded score over
    the first n_sink and last n_local positions that are valid; -inf when
    there is none."""
    s32 = np.asarray(scores, np.float64).astype(np.float32).astype(np.float64)
    n = s32.shape[0]
    t = np.arange(n)
    ok = np.ones(n, bool) if valid is None else np.asarray(valid, bool)
    special = ok & ((t < n_sink) | (t >= n - n_local))
    if not special.any():
        return -np.inf
    return float(s32[special].max()) - delta * G / scale


def select_topdelta(scores, k_max: int, delta: float, n_sink: int, n_local: int, scale: float, G: int,
                    valid=None):
    """(indices [k_max] ascending, -1 padded; count): the valid tokens with
    fp32 score >= the top-delta threshold, at most k_max of them, chosen in
    the order (score desc, index asc) (R13, R3)."""
    s32 = np.asarray(scores, np.float64).astype(np.float32).astype(np.float64)
    n = s32.shape[0]
    ok = np.ones(n, bool) if valid is None else np.asarray(valid, bool)
    thr = topdelta_threshold(scores, delta, n_sink, n_local, scale, G, ok)
    cand = np.nonzero(ok & (s32 >= thr))[0]
    order = cand[np.lexsort((cand, -s32[cand]))]
    keep = np.sort(order[:k_max])
    out = np.full(k_max, -1, np.int64)
    out[:keep.shape[0]] = keep
    return out, int(keep.shape[0])


# ---------------------------------------------------------------------------
# Lossless screening (R14)  [DOSA]
# ---------------------------------------------------------------------------
SCREEN_TILE = 64


def tile_bounds(Kp_bits, valid=None, tile: int = SCREEN_TILE):
    """Per tile of `tile` consecutive tokens: (lo, hi) [ntiles, r], the
    per-dimension min and max of the tile's valid projected keys (fp64);
    a tile without a valid token gets lo = +inf, hi = -inf."""
    Kp = bf16_to_f64(Kp_bits)
    n, r = Kp.shape
    ok = np.ones(n, bool) if valid is None else np.asarray(valid, bool)
    nt = (n + tile - 1) // tile
    lo = np.full((nt, r), np.inf)
    hi = np.full((nt, r), -np.inf)
    for i in range(nt):
        rows = Kp[i * tile:(i + 1) * tile][ok[i * tile:(i + 1) * tile]]
        if rows.shape[0]:
            lo[i] = rows.min(axis=0)
            hi[i] = rows.max(axis=0)
    return lo, hi


def tile_upper_bounds(qp, lo, hi) -> np.ndarray:
    """ub per tile = sum_c max(qp_c lo_c, qp_c hi_c) (-inf for empty tiles)."""
    qp = np.asarray(qp, np.float64)
    empty = ~np.isfinite(lo).all(axis=1)
    l = np.where(np.isfinite(lo), lo, 0.0)
    h = np.where(np.isfinite(hi), hi, 0.0)
    ub = np.maximum(l * qp, h * qp).sum(axis=1)
    return np.where(empty, -np.inf, ub)


def seed_threshold(scores, seeds, k: int, valid=None) -> float:
    """tau: the k-th largest fp32-rounded score over the distinct valid
    tokens listed in `seeds` (entries outside [0, T_b) ignored); -inf when
    there are fewer than k."""
    s32 = np.asarray(scores, np.float64).astype(np.float32).astype(np.float64)
    n = s32.shape[0]
    sd = np.unique(np.asarray(seeds, np.int64).ravel())
    sd = sd[(sd >= 0) & (sd < n)]
    if valid is not None:
        sd = sd[np.asarray(valid, bool)[sd]]
    if sd.shape[0] < k:
        return -np.inf
    return float(np.sort(s32[sd])[::-1][k - 1])


def screened_topk(scores, qp, Kp_bits, seeds, k: int, valid=None):
    """(R3's selection restricted to the tokens of the tiles that survive
    screening, the keep flag per tile)."""
    lo, hi = tile_bounds(Kp_bits, valid)
    keep_tile = tile_upper_bounds(qp, lo, hi) >= seed_threshold(scores, seeds, k, valid)
    n = np.asarray(scores).shape[0]
    ok = np.ones(n, bool) if valid is None else np.asarray(valid, bool)
    alive = ok & np.repeat(keep_tile, SCREEN_TILE)[:n]
    s = np.where(alive, np.asarray(scores, np.float64), -np.inf)
    cand = np.nonzero(alive)[0]
    s32 = s.astype(np.float32).astype(np.float64)
    order = cand[np.lexsort((cand, -s32[cand]))]
    keepi = np.sort(order[:k])
    out = np.full(k, -1, np.int64)
    out[:keepi.shape[0]] = keepi
    return out, keep_tile
