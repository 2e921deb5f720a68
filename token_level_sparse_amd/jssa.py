"""ctypes binding of libjssa.so (argument marshalling only).

Every function has the name and argument order of the C entry point declared
in include/jssa.h. Tensor arguments are torch tensors on the GPU (their
data_ptr is passed; bf16 data may be any 2-byte dtype), or None for optional
pointers. `stream` defaults to torch's current stream on the current device.
A nonzero status raises JssaError carrying the library's message.

Importing this module loads the library and fails loudly when it has not
been built: there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# JSSA_LIBRARY names another build of the same library (the host-sanitizer
# build of the test suite); by default the in-tree libjssa.so
LIB_PATH = os.environ.get("JSSA_LIBRARY") or os.path.join(_HERE, "libjssa.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python -m token_level_sparse_amd.build`")
_lib = ctypes.CDLL(LIB_PATH)

OK, ERR_NULL, ERR_SHAPE, ERR_UNSUPPORTED, ERR_ALIGN, ERR_WORKSPACE, ERR_HIP, ERR_NUMERIC = range(8)

ENTRY_POINTS = (
    "jssa_append_kv", "jssa_project_keys", "jssa_score", "jssa_topk_workspace_size", "jssa_topk",
    "jssa_score_topk_workspace_size", "jssa_score_topk", "jssa_score_topk_noalloc", "jssa_score_topk_chunks",
    "jssa_score_topk_final",
    "jssa_score_topk_final_attend",
    "jssa_indexed_decode", "jssa_combine", "jssa_dense_decode", "jssa_gather_kv",
    "jssa_mla_project_latent", "jssa_mla_fold_selection", "jssa_mla_absorb_q", "jssa_mla_score", "jssa_mla_score_topk_workspace_size",
    "jssa_mla_score_topk", "jssa_mla_indexed_decode", "jssa_mla_combine_up_v",
    "jssa_mla_up_v", "jssa_score_topdelta_workspace_size", "jssa_score_topdelta", "jssa_score_topdelta_attend",
    "jssa_tile_bounds_size", "jssa_build_tile_bounds", "jssa_update_tile_bounds",
    "jssa_score_topk_screened_workspace_size",
    "jssa_score_topk_screened_chunks", "jssa_calib_workspace_size", "jssa_calib_query_workspace_size", "jssa_calib_key_moments", "jssa_calib_query_moments",
    "jssa_calib_projection", "jssa_status_string", "jssa_last_error", "jssa_version",
)


class JssaError(RuntimeError):
    def __init__(self, status: int, fn: str, msg: str):
        super().__init__(f"{fn} -> {status}: {msg}")
        self.status = status


class GqaDesc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
                ("d", ctypes.c_int32), ("r", ctypes.c_int32), ("max_seq", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("num_pages", ctypes.c_int32),
                ("max_pages_per_seq", ctypes.c_int32), ("page_table", ctypes.c_void_p),
                ("seq_lens", ctypes.c_void_p)]


class MlaDesc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("d_latent", ctypes.c_int32),
                ("d_rope", ctypes.c_int32), ("d_nope", ctypes.c_int32), ("d_v", ctypes.c_int32),
                ("r", ctypes.c_int32), ("max_seq", ctypes.c_int32), ("seq_lens", ctypes.c_void_p)]


class TopDeltaRule(ctypes.Structure):
    _fields_ = [("delta", ctypes.c_float), ("n_sink", ctypes.c_int32), ("n_local", ctypes.c_int32)]


_vp, _i32, _f32, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
_P = ctypes.POINTER
_SIGS = {
    "jssa_append_kv": [_P(GqaDesc), _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp],
    "jssa_project_keys": [_P(GqaDesc), _vp, _vp, _vp, _vp],
    "jssa_score": [_P(GqaDesc), _vp, _vp, _vp, _vp, _vp],
    "jssa_topk_workspace_size": [_i32, _i32, _i32, _i32, _P(_sz)],
    "jssa_topk": [_i32, _i32, _i32, _vp, _vp, _i32, _vp, _vp, _sz, _vp],
    "jssa_score_topk_workspace_size": [_P(GqaDesc), _i32, _P(_sz)],
    "jssa_score_topk": [_P(GqaDesc), _vp, _vp, _vp, _i32, _vp, _vp, _vp, _sz, _vp],
    "jssa_score_topk_noalloc": [_P(GqaDesc), _vp, _vp, _vp, _i32, _vp, _vp, _vp],
    "jssa_score_topk_chunks": [_P(GqaDesc), _vp, _vp, _vp, _i32, _vp, _vp, _sz, _vp],
    "jssa_score_topk_final": [_P(GqaDesc), _i32, _vp, _sz, _vp, _vp],
    "jssa_score_topk_final_attend": [_P(GqaDesc), _i32, _vp, _sz, _vp, _vp, _vp, _f32, _vp, _vp, _vp, _vp],
    "jssa_indexed_decode": [_P(GqaDesc), _vp, _vp, _vp, _vp, _i32, _i32, _f32, _vp, _vp, _vp],
    "jssa_combine": [_i32, _i32, _i32, _i32, _vp, _vp, _vp, _i32, _vp, _vp],
    "jssa_dense_decode": [_P(GqaDesc), _vp, _vp, _vp, _i32, _f32, _vp, _vp, _vp],
    "jssa_gather_kv": [_P(GqaDesc), _vp, _vp, _vp, _i32, _vp, _vp, _vp, _vp],
    "jssa_mla_project_latent": [_P(MlaDesc), _vp, _vp, _vp, _vp],
    "jssa_mla_fold_selection": [_P(MlaDesc), _vp, _vp, _vp, _vp],
    "jssa_mla_absorb_q": [_P(MlaDesc), _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp],
    "jssa_mla_score": [_P(MlaDesc), _vp, _vp, _vp, _vp],
    "jssa_mla_score_topk_workspace_size": [_P(MlaDesc), _i32, _P(_sz)],
    "jssa_mla_score_topk": [_P(MlaDesc), _vp, _vp, _i32, _vp, _vp, _vp, _sz, _vp],
    "jssa_mla_indexed_decode": [_P(MlaDesc), _vp, _vp, _vp, _i32, _i32, _f32, _vp, _vp, _vp],
    "jssa_mla_up_v": [_P(MlaDesc), _vp, _vp, _vp, _vp],
    "jssa_mla_combine_up_v": [_P(MlaDesc), _i32, _vp, _vp, _vp, _vp, _vp, _vp],
    "jssa_score_topdelta_workspace_size": [_P(GqaDesc), _i32, _P(_sz)],
    "jssa_score_topdelta": [_P(GqaDesc), _vp, _vp, _vp, _i32, _P(TopDeltaRule), _f32, _vp, _vp, _vp, _sz, _vp],
    "jssa_score_topdelta_attend": [_P(GqaDesc), _vp, _vp, _vp, _vp, _vp, _i32, _P(TopDeltaRule), _f32, _vp, _vp,
                                   _vp, _vp, _vp, _sz, _vp],
    "jssa_tile_bounds_size": [_P(GqaDesc), _P(_sz)],
    "jssa_build_tile_bounds": [_P(GqaDesc), _vp, _vp, _vp],
    "jssa_update_tile_bounds": [_P(GqaDesc), _vp, _vp, _i32, _vp, _vp],
    "jssa_score_topk_screened_workspace_size": [_P(GqaDesc), _i32, _P(_sz)],
    "jssa_score_topk_screened_chunks": [_P(GqaDesc), _vp, _vp, _vp, _vp, _vp, _i32, _i32, _vp, _vp, _sz, _vp],
    "jssa_calib_workspace_size": [_P(GqaDesc), _P(_sz)],
    "jssa_calib_key_moments": [_P(GqaDesc), _vp, _vp, _vp, _sz, _vp],
    "jssa_calib_query_workspace_size": [_i32, _P(_sz)],
    "jssa_calib_query_moments": [_i32, _i32, _i32, _vp, _vp, _vp, _sz, _vp],
    "jssa_calib_projection": [_i32, _i32, _vp, _vp, _vp, _vp],
}
for _name, _args in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.argtypes = _args
    _f.restype = ctypes.c_int32
_lib.jssa_status_string.argtypes = [ctypes.c_int32]
_lib.jssa_status_string.restype = ctypes.c_char_p
_lib.jssa_last_error.argtypes = []
_lib.jssa_last_error.restype = ctypes.c_char_p
_lib.jssa_version.argtypes = []
_lib.jssa_version.restype = ctypes.c_int32


def _p(t):
    """Device pointer of a tensor (None -> NULL). Non-tensors (ints) pass
    through as raw addresses, which lets tests probe the host-side checks."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_contiguous():
        raise ValueError("tensor arguments must be contiguous")
    return t.data_ptr()


def _s(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def _check(rc: int, fn: str):
    if rc != OK:
        raise JssaError(rc, fn, _lib.jssa_last_error().decode())


def gqa_desc(B, Hq, Hkv, r, max_seq, d=128, page_size=0, num_pages=0, max_pages_per_seq=0,
             page_table=None, seq_lens=None) -> GqaDesc:
    return GqaDesc(B, Hq, Hkv, d, r, max_seq, page_size, num_pages, max_pages_per_seq,
                   _p(page_table), _p(seq_lens))


def mla_desc(B, H, r, max_seq, d_latent=512, d_rope=64, d_nope=128, d_v=128, seq_lens=None) -> MlaDesc:
    return MlaDesc(B, H, d_latent, d_rope, d_nope, d_v, r, max_seq, _p(seq_lens))


def jssa_version() -> int:
    return _lib.jssa_version()


def jssa_status_string(status: int) -> str:
    return _lib.jssa_status_string(status).decode()


def jssa_last_error() -> str:
    return _lib.jssa_last_error().decode()


def jssa_append_kv(desc, K, V, Kp, k_new, v_new, P, pos, n_new, stream=None):
    _check(_lib.jssa_append_kv(ctypes.byref(desc), _p(K), _p(V), _p(Kp), _p(k_new), _p(v_new),
                               _p(P), _p(pos), n_new, _s(stream)), "jssa_append_kv")


def jssa_project_keys(desc, K, P, Kp, stream=None):
    _check(_lib.jssa_project_keys(ctypes.byref(desc), _p(K), _p(P), _p(Kp), _s(stream)),
           "jssa_project_keys")


def jssa_score(desc, q, P, Kp, scores, stream=None):
    _check(_lib.jssa_score(ctypes.byref(desc), _p(q), _p(P), _p(Kp), _p(scores), _s(stream)),
           "jssa_score")


def jssa_topk_workspace_size(B, H, max_seq, k) -> int:
    n = _sz(0)
    _check(_lib.jssa_topk_workspace_size(B, H, max_seq, k, ctypes.byref(n)), "jssa_topk_workspace_size")
    return n.value


def jssa_topk(B, H, max_seq, seq_lens, scores, k, idx, ws, ws_bytes=None, stream=None):
    if ws_bytes is None:
        ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(_lib.jssa_topk(B, H, max_seq, _p(seq_lens), _p(scores), k, _p(idx), _p(ws), ws_bytes,
                          _s(stream)), "jssa_topk")


def jssa_score_topk_workspace_size(desc, k) -> int:
    n = _sz(0)
    _check(_lib.jssa_score_topk_workspace_size(ctypes.byref(desc), k, ctypes.byref(n)),
           "jssa_score_topk_workspace_size")
    return n.value


def jssa_score_topk(desc, q, P, Kp, k, scores, idx, ws, ws_bytes=None, stream=None):
    if ws_bytes is None:
        ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(_lib.jssa_score_topk(ctypes.byref(desc), _p(q), _p(P), _p(Kp), k, _p(scores), _p(idx), _p(ws),
                                ws_bytes, _s(stream)), "jssa_score_topk")


def jssa_score_topk_noalloc(desc, q, P, Kp, k, scores, idx, stream=None):
    _check(_lib.jssa_score_topk_noalloc(ctypes.byref(desc), _p(q), _p(P), _p(Kp), k, _p(scores), _p(idx),
                                        _s(stream)), "jssa_score_topk_noalloc")


def jssa_score_topk_chunks(desc, q, P, Kp, k, scores, ws, ws_bytes=None, stream=None):
    if ws_bytes is None:
        ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(_lib.jssa_score_topk_chunks(ctypes.byref(desc), _p(q), _p(P), _p(Kp), k, _p(scores), _p(ws), ws_bytes,
                                       _s(stream)), "jssa_score_topk_chunks")


def jssa_score_topk_final(desc, k, ws, idx, ws_bytes=None, stream=None):
    if ws_bytes is None:
        ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(_lib.jssa_score_topk_final(ctypes.byref(desc), k, _p(ws), ws_bytes, _p(idx), _s(stream)),
           "jssa_score_topk_final")


def jssa_score_topk_final_attend(desc, k, ws, q, K, V, scale, idx, out, lse, ws_bytes=None, stream=None):
    if ws_bytes is None:
        ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(_lib.jssa_score_topk_final_attend(ctypes.byref(desc), k, _p(ws), ws_bytes, _p(q), _p(K), _p(V), scale,
                                             _p(idx), _p(out), _p(lse), _s(stream)), "jssa_score_topk_final_attend")


def jssa_indexed_decode(desc, q, K, V, idx, k, S, scale, part_o, part_lse, stream=None):
    _check(_lib.jssa_indexed_decode(ctypes.byref(desc), _p(q), _p(K), _p(V), _p(idx), k, S, scale,
                                    _p(part_o), _p(part_lse), _s(stream)), "jssa_indexed_decode")


def jssa_combine(B, H, S, dv, part_o, part_lse, out, out_bf16=0, lse=None, stream=None):
    _check(_lib.jssa_combine(B, H, S, dv, _p(part_o), _p(part_lse), _p(out), out_bf16, _p(lse),
                             _s(stream)), "jssa_combine")


def jssa_dense_decode(desc, q, K, V, S, scale, part_o, part_lse, stream=None):
    _check(_lib.jssa_dense_decode(ctypes.byref(desc), _p(q), _p(K), _p(V), S, scale, _p(part_o),
                                  _p(part_lse), _s(stream)), "jssa_dense_decode")


def jssa_gather_kv(desc, K, V, idx, k, Kg, Vg, lens_out, stream=None):
    _check(_lib.jssa_gather_kv(ctypes.byref(desc), _p(K), _p(V), _p(idx), k, _p(Kg), _p(Vg),
                               _p(lens_out), _s(stream)), "jssa_gather_kv")


def jssa_mla_project_latent(desc, latent, P, Kp_lat, stream=None):
    _check(_lib.jssa_mla_project_latent(ctypes.byref(desc), _p(latent), _p(P), _p(Kp_lat), _s(stream)),
           "jssa_mla_project_latent")


def jssa_mla_fold_selection(desc, W_uk, P, U, stream=None):
    _check(_lib.jssa_mla_fold_selection(ctypes.byref(desc), _p(W_uk), _p(P), _p(U), _s(stream)),
           "jssa_mla_fold_selection")


def jssa_mla_absorb_q(desc, q_nope, q_rope, W_uk, P, U, q_abs, q_sel, stream=None):
    _check(_lib.jssa_mla_absorb_q(ctypes.byref(desc), _p(q_nope), _p(q_rope), _p(W_uk), _p(P), _p(U), _p(q_abs),
                                  _p(q_sel), _s(stream)), "jssa_mla_absorb_q")


def jssa_mla_score(desc, q_sel, Kp_lat, scores, stream=None):
    _check(_lib.jssa_mla_score(ctypes.byref(desc), _p(q_sel), _p(Kp_lat), _p(scores), _s(stream)),
           "jssa_mla_score")


def jssa_mla_score_topk_workspace_size(desc, k) -> int:
    n = _sz(0)
    _check(_lib.jssa_mla_score_topk_workspace_size(ctypes.byref(desc), k, ctypes.byref(n)),
           "jssa_mla_score_topk_workspace_size")
    return n.value


def jssa_mla_score_topk(desc, q_sel, Kp_lat, k, scores, idx, ws, ws_bytes=None, stream=None):
    if ws_bytes is None:
        ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(_lib.jssa_mla_score_topk(ctypes.byref(desc), _p(q_sel), _p(Kp_lat), k, _p(scores), _p(idx), _p(ws),
                                    ws_bytes, _s(stream)), "jssa_mla_score_topk")


def jssa_mla_indexed_decode(desc, q_abs, latent, idx, k, S, scale, part_o, part_lse, stream=None):
    _check(_lib.jssa_mla_indexed_decode(ctypes.byref(desc), _p(q_abs), _p(latent), _p(idx), k, S, scale,
                                        _p(part_o), _p(part_lse), _s(stream)), "jssa_mla_indexed_decode")


def jssa_mla_up_v(desc, o_lat, W_uv, out, stream=None):
    _check(_lib.jssa_mla_up_v(ctypes.byref(desc), _p(o_lat), _p(W_uv), _p(out), _s(stream)),
           "jssa_mla_up_v")


def jssa_mla_combine_up_v(desc, S, part_o, part_lse, W_uv, out, lse=None, stream=None):
    _check(_lib.jssa_mla_combine_up_v(ctypes.byref(desc), S, _p(part_o), _p(part_lse), _p(W_uv), _p(out), _p(lse),
                                      _s(stream)), "jssa_mla_combine_up_v")


def jssa_calib_workspace_size(desc) -> int:
    n = _sz(0)
    _check(_lib.jssa_calib_workspace_size(ctypes.byref(desc), ctypes.byref(n)), "jssa_calib_workspace_size")
    return n.value


def jssa_calib_key_moments(desc, K, moments, ws, ws_bytes=None, stream=None):
    if ws_bytes is None:
        ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(_lib.jssa_calib_key_moments(ctypes.byref(desc), _p(K), _p(moments), _p(ws), ws_bytes, _s(stream)),
           "jssa_calib_key_moments")


def jssa_calib_query_workspace_size(Hkv) -> int:
    n = _sz(0)
    _check(_lib.jssa_calib_query_workspace_size(Hkv, ctypes.byref(n)), "jssa_calib_query_workspace_size")
    return n.value


def jssa_calib_query_moments(N, Hq, Hkv, q, moments, ws, ws_bytes=None, stream=None):
    if ws_bytes is None:
        ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(_lib.jssa_calib_query_moments(N, Hq, Hkv, _p(q), _p(moments), _p(ws), ws_bytes, _s(stream)),
           "jssa_calib_query_moments")


def jssa_calib_projection(S_q, S_k, r: int):
    """Host call: S_q, S_k numpy [d, d] (converted to fp32). Returns (P [d, r]
    fp32, eigenvalues [r] fp64)."""
    import numpy as np
    S_q = np.ascontiguousarray(S_q, dtype=np.float32)
    S_k = np.ascontiguousarray(S_k, dtype=np.float32)
    d = S_q.shape[0]
    if S_q.shape != (d, d) or S_k.shape != (d, d):
        raise ValueError("S_q and S_k must be square and of one size")
    P = np.empty((d, r), np.float32)
    w = np.empty(r, np.float64)
    _check(_lib.jssa_calib_projection(d, r, S_q.ctypes.data, S_k.ctypes.data, P.ctypes.data, w.ctypes.data),
           "jssa_calib_projection")
    return P, w


def topdelta_rule(delta: float, n_sink: int = 4, n_local: int = 64) -> TopDeltaRule:
    return TopDeltaRule(delta, n_sink, n_local)


def jssa_score_topdelta_workspace_size(desc, k_max) -> int:
    n = _sz(0)
    _check(_lib.jssa_score_topdelta_workspace_size(ctypes.byref(desc), k_max, ctypes.byref(n)),
           "jssa_score_topdelta_workspace_size")
    return n.value


def jssa_score_topdelta(desc, q, P, Kp, k_max, rule, scale, idx, counts, ws, ws_bytes=None, stream=None):
    if ws_bytes is None:
        ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(_lib.jssa_score_topdelta(ctypes.byref(desc), _p(q), _p(P), _p(Kp), k_max,
                                    None if rule is None else ctypes.byref(rule), scale, _p(idx), _p(counts),
                                    _p(ws), ws_bytes, _s(stream)), "jssa_score_topdelta")


def jssa_score_topdelta_attend(desc, q, P, Kp, K, V, k_max, rule, scale, idx, counts, out, lse, ws,
                               ws_bytes=None, stream=None):
    if ws_bytes is None:
        ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(_lib.jssa_score_topdelta_attend(ctypes.byref(desc), _p(q), _p(P), _p(Kp), _p(K), _p(V), k_max,
                                           None if rule is None else ctypes.byref(rule), scale, _p(idx),
                                           _p(counts), _p(out), _p(lse), _p(ws), ws_bytes, _s(stream)),
           "jssa_score_topdelta_attend")


def jssa_tile_bounds_size(desc) -> int:
    n = _sz(0)
    _check(_lib.jssa_tile_bounds_size(ctypes.byref(desc), ctypes.byref(n)), "jssa_tile_bounds_size")
    return n.value


def jssa_build_tile_bounds(desc, Kp, bounds, stream=None):
    _check(_lib.jssa_build_tile_bounds(ctypes.byref(desc), _p(Kp), _p(bounds), _s(stream)), "jssa_build_tile_bounds")


def jssa_update_tile_bounds(desc, Kp, pos, n_new, bounds, stream=None):
    _check(_lib.jssa_update_tile_bounds(ctypes.byref(desc), _p(Kp), _p(pos), n_new, _p(bounds), _s(stream)),
           "jssa_update_tile_bounds")


def jssa_score_topk_screened_workspace_size(desc, k) -> int:
    n = _sz(0)
    _check(_lib.jssa_score_topk_screened_workspace_size(ctypes.byref(desc), k, ctypes.byref(n)),
           "jssa_score_topk_screened_workspace_size")
    return n.value


def jssa_score_topk_screened_chunks(desc, q, P, Kp, bounds, seeds, n_seed, k, kept_tiles, ws, ws_bytes=None,
                                    stream=None):
    if ws_bytes is None:
        ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(_lib.jssa_score_topk_screened_chunks(ctypes.byref(desc), _p(q), _p(P), _p(Kp), _p(bounds), _p(seeds),
                                                n_seed, k, _p(kept_tiles), _p(ws), ws_bytes, _s(stream)),
           "jssa_score_topk_screened_chunks")
