"""Each plausible mistake planted in the oracle (on the CPU) must make at
least one pin fail: this shows the pins constrain every step."""
import numpy as np
import pytest

from oracle import jssa_oracle as O
import tests.test_oracle_pins as pins


def _truncate_bf16(x):
    x = np.asarray(x, np.float64).astype(np.float32)
    return (x.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _mean_query(q_group_bits, P_j):
    return np.asarray(P_j, np.float64).T @ O.bf16_to_f64(q_group_bits).mean(axis=0)


def _first_head_query(q_group_bits, P_j):
    return np.asarray(P_j, np.float64).T @ O.bf16_to_f64(q_group_bits)[0]


def _topk_highest_index_ties(scores, k):
    s = np.asarray(scores, np.float64).astype(np.float32).astype(np.float64)
    n = s.shape[0]
    order = np.lexsort((-np.arange(n), -s))
    out = np.full(k, -1, np.int64)
    keep = np.sort(order[:min(k, n)])
    out[:keep.shape[0]] = keep
    return out


def _topk_score_order(scores, k):
    s = np.asarray(scores, np.float64).astype(np.float32).astype(np.float64)
    order = np.lexsort((np.arange(s.shape[0]), -s))[:min(k, s.shape[0])]
    out = np.full(k, -1, np.int64)
    out[:order.shape[0]] = order
    return out


def _attend_unscaled(q_bits, K_rows_bits, V_rows_bits, scale):
    return _orig_attend(q_bits, K_rows_bits, V_rows_bits, 1.0)


def _attend_no_max(q_bits, K_rows_bits, V_rows_bits, scale):
    o, lse = _orig_attend(q_bits, K_rows_bits, V_rows_bits, scale)
    return o, lse - np.log(np.asarray(K_rows_bits).shape[0])


def _combine_wrong_sign(part_o, part_lse):
    part_lse = np.asarray(part_lse, np.float64)
    w = np.exp(-(part_lse - part_lse.max()))
    return (w[:, None] * np.asarray(part_o)).sum(0) / w.sum(), part_lse.max() + np.log(w.sum())


def _group_strided(j, G):
    return range(j, j + 2 * G, 2)


def _paged_swapped(pool, table_row, j, t):
    t = np.asarray(t, np.int64)
    return np.asarray(pool)[np.asarray(table_row)[t % 16], j, t // 16 % 16]


def _mla_no_rope(qn, qr, Wk, Wv, C, scale):
    return _orig_mla(qn, np.zeros_like(qr), Wk, Wv, C, scale)


def _marginal_unnormalised(S_q, S_k):
    return np.asarray(S_q, np.float64) + np.asarray(S_k, np.float64)


def _calib_bottom(S_q, S_k, r):
    w, V = np.linalg.eigh(_orig_marginal(S_q, S_k))
    return O.sign_fix(V[:, :r]), w[:r]


def _query_moment_mean_heads(q_samples_bits, j, G):
    return _orig_qmoment(q_samples_bits, j, G) / (G * G)


def _key_moment_sum(K_rows_bits):
    K = np.asarray(K_rows_bits)
    return _orig_kmoment(K) * K.reshape(-1, K.shape[-1]).shape[0]


def _bound_lam_inverted(P, S_q, S_k):
    P = np.asarray(P, np.float64)
    Q = np.eye(P.shape[0]) - P @ P.T
    lam = np.sqrt(np.trace(S_q) / np.trace(S_k))
    return float(np.trace(Q @ (lam * np.asarray(S_q) + np.asarray(S_k) / lam)) / 2)


def _topdelta_global_max(scores, k_max, delta, n_sink, n_local, scale, G, valid=None):
    n = len(scores)
    return _orig_topdelta(scores, k_max, delta, n, 0, scale, G, valid)


def _topdelta_no_group(scores, k_max, delta, n_sink, n_local, scale, G, valid=None):
    return _orig_topdelta(scores, k_max, delta, n_sink, n_local, scale, 1, valid)


def _strict_impl(scores, k_max, delta, n_sink, n_local, scale, G, valid=None):
    s32 = np.asarray(scores, np.float64).astype(np.float32).astype(np.float64)
    n = s32.shape[0]
    ok = np.ones(n, bool) if valid is None else np.asarray(valid, bool)
    thr = O.topdelta_threshold(scores, delta, n_sink, n_local, scale, G, ok)
    cand = np.nonzero(ok & (s32 > thr))[0]
    order = cand[np.lexsort((cand, -s32[cand]))]
    keep = np.sort(order[:k_max])
    out = np.full(k_max, -1, np.int64)
    out[:keep.shape[0]] = keep
    return out, int(keep.shape[0])


def _threshold_local_off_by_one(scores, delta, n_sink, n_local, scale, G, valid=None):
    return _orig_threshold(scores, delta, n_sink, max(0, n_local - 1), scale, G, valid)


def _ub_min(qp, lo, hi):
    qp = np.asarray(qp, np.float64)
    l = np.where(np.isfinite(lo), lo, 0.0)
    h = np.where(np.isfinite(hi), hi, 0.0)
    return np.minimum(l * qp, h * qp).sum(axis=1)


def _seed_with_duplicates(scores, seeds, k, valid=None):
    s32 = np.asarray(scores, np.float64).astype(np.float32).astype(np.float64)
    sd = np.asarray(seeds, np.int64).ravel()
    sd = sd[(sd >= 0) & (sd < s32.shape[0])]
    if valid is not None:
        sd = sd[np.asarray(valid, bool)[sd]]
    return -np.inf if sd.shape[0] < k else float(np.sort(s32[sd])[::-1][k - 1])


def _tile_bounds_all_rows(Kp_bits, valid=None, tile=64):
    return _orig_tile_bounds(Kp_bits, None, tile)


def _seed_threshold_kplus1(scores, seeds, k, valid=None):
    return _orig_seed_threshold(scores, seeds, k + 1, valid)


def _kth_off_by_one(scores, k):
    order = O.selection_order(scores)
    return float(np.asarray(scores, np.float64)[order[min(k, order.shape[0] - 1)]])


def _order_with_absent(scores):
    s32 = np.asarray(scores, np.float64).astype(np.float32).astype(np.float64)
    t = np.arange(s32.shape[0])
    return t[np.lexsort((t, -s32))]


def _order_fp64(scores):
    s = np.asarray(scores, np.float64)
    t = np.nonzero(s > -np.inf)[0]
    return t[np.lexsort((t, -s[t]))]


def _paged_rows_unchecked(pool, table_row, j, t):
    t = np.asarray(t, np.int64)
    return np.asarray(pool)[np.asarray(table_row)[t // 16], j, t % 16]


_orig_tile_bounds = O.tile_bounds
_orig_seed_threshold = O.seed_threshold
_orig_topdelta = O.select_topdelta
_orig_threshold = O.topdelta_threshold
_orig_attend = O.attend
_orig_mla = O.mla_attend_explicit
_orig_marginal = O.marginal_operator
_orig_qmoment = O.query_second_moment
_orig_kmoment = O.key_second_moment

MUTATIONS = [
    ("round_to_bf16", _truncate_bf16, [pins.test_bf16_golden_values]),
    ("project_query", _mean_query, [pins.test_score_golden_group_sum]),
    ("project_query", _first_head_query, [pins.test_score_golden_group_sum]),
    ("select_topk", _topk_highest_index_ties, [pins.test_topk_golden_ties]),
    ("select_topk", _topk_score_order, [pins.test_topk_golden_ties]),
    ("attend", _attend_unscaled, [pins.test_dense_matches_torch_sdpa]),
    ("attend", _attend_no_max, [pins.test_attention_golden]),
    ("combine", _combine_wrong_sign, [lambda: pins.test_combine_split_invariance(3)]),
    ("group_heads", _group_strided, [pins.test_dense_matches_torch_sdpa]),
    ("paged_rows", _paged_swapped, [pins.test_paged_matches_contiguous]),
    ("mla_attend_explicit", _mla_no_rope, [pins.test_mla_brute_force_loops]),
    ("marginal_operator", _marginal_unnormalised, [pins.test_calib_invariances, pins.test_calib_diagonal_closed_form]),
    ("calibrate_projection", _calib_bottom, [pins.test_calib_diagonal_closed_form]),
    ("query_second_moment", _query_moment_mean_heads, [pins.test_calib_second_moments_brute_force]),
    ("key_second_moment", _key_moment_sum, [pins.test_calib_second_moments_brute_force]),
    ("marginal_bound", _bound_lam_inverted, [pins.test_calib_minimises_bound_brute_force]),
    ("select_topdelta", _topdelta_global_max, [pins.test_topdelta_golden_hand]),
    ("select_topdelta", _topdelta_no_group, [pins.test_topdelta_golden_hand]),
    ("select_topdelta", _strict_impl, [pins.test_topdelta_golden_hand]),
    ("topdelta_threshold", _threshold_local_off_by_one, [pins.test_topdelta_golden_hand]),
    ("tile_upper_bounds", _ub_min, [lambda: pins.test_screen_bounds_sound_and_lossless(1)]),
    ("seed_threshold", _seed_with_duplicates, [pins.test_screen_seed_closed_form]),
    ("tile_bounds", _tile_bounds_all_rows, [pins.test_screen_hand_values]),
    ("seed_threshold", _seed_threshold_kplus1, [pins.test_screen_seed_closed_form]),
    ("kth_score", _kth_off_by_one, [pins.test_kth_score_and_absent_tokens_golden]),
    ("selection_order", _order_with_absent, [pins.test_kth_score_and_absent_tokens_golden]),
    ("selection_order", _order_fp64, [pins.test_kth_score_and_absent_tokens_golden]),
    ("paged_rows", _paged_rows_unchecked, [pins.test_paged_rows_reject_positions_without_a_page]),
]


@pytest.mark.parametrize("name,fn,checks", MUTATIONS, ids=[f"{m[0]}:{m[1].__name__}" for m in MUTATIONS])
def test_planted_mistake_is_caught(monkeypatch, name, fn, checks):
    monkeypatch.setattr(O, name, fn)
    caught = 0
    for check in checks:
        try:
            check()
        except (AssertionError, ValueError, IndexError, pytest.fail.Exception):
            caught += 1
    assert caught >= 1, f"mutation {name}/{fn.__name__} passed every pin"
