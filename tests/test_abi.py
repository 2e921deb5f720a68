"""The C-ABI library: it loads, exports every entry point include/jssa.h
declares, and rejects bad arguments on the host before any HIP call (so these
tests run without a GPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "jssa.h")
LIB = os.path.join(ROOT, "token_level_sparse_amd", "libjssa.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libjssa.so not built")


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(jssa_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    lib = ctypes.CDLL(LIB)
    names = declared_symbols()
    assert len(names) >= 17
    for n in names:
        assert hasattr(lib, n), n
    from token_level_sparse_amd import jssa
    assert set(jssa.ENTRY_POINTS) == set(names)


@pytest.fixture(scope="module")
def J():
    from token_level_sparse_amd import jssa
    return jssa


A = 1 << 20          # a 16-byte aligned fake address: never dereferenced
MIS = A + 4


def _status(fn, *args):
    from token_level_sparse_amd import jssa
    with pytest.raises(jssa.JssaError) as e:
        fn(*args)
    return e.value.status


def test_version_and_strings(J):
    assert J.jssa_version() >= 100
    assert J.jssa_status_string(J.ERR_WORKSPACE) == "workspace too small"


def test_desc_validation(J):
    ok = J.gqa_desc(2, 32, 8, 32, 4096)
    bad_d = J.gqa_desc(2, 32, 8, 32, 4096, d=64)
    bad_r = J.gqa_desc(2, 32, 8, 40, 4096)
    bad_g = J.gqa_desc(2, 30, 8, 32, 4096)
    big_g = J.gqa_desc(1, 64, 2, 32, 4096)
    bad_page = J.gqa_desc(2, 32, 8, 32, 4096, page_size=8)
    paged_null = J.gqa_desc(2, 32, 8, 32, 4096, page_size=16, num_pages=10, max_pages_per_seq=256)
    paged_short = J.gqa_desc(2, 32, 8, 32, 4096, page_size=16, num_pages=10, max_pages_per_seq=100,
                             page_table=A)
    f = J.jssa_score
    assert _status(f, bad_d, A, A, A, A) == J.ERR_UNSUPPORTED
    assert _status(f, bad_r, A, A, A, A) == J.ERR_UNSUPPORTED
    assert _status(f, bad_g, A, A, A, A) == J.ERR_SHAPE
    assert _status(f, big_g, A, A, A, A) == J.ERR_UNSUPPORTED
    assert _status(f, bad_page, A, A, A, A) == J.ERR_UNSUPPORTED
    assert _status(f, paged_null, A, A, A, A) == J.ERR_NULL
    assert _status(f, paged_short, A, A, A, A) == J.ERR_SHAPE
    assert _status(f, ok, None, A, A, A) == J.ERR_NULL
    assert _status(f, ok, A, A, MIS, A) == J.ERR_ALIGN
    assert "Kp" in J.jssa_last_error()
    assert _status(J.jssa_dense_decode, ok, A, A, A, 0, 1.0, A, A) == J.ERR_SHAPE
    assert _status(J.jssa_dense_decode, ok, A, A, A, 300, 1.0, A, A) == J.ERR_SHAPE
    assert _status(J.jssa_indexed_decode, ok, A, A, A, A, 0, 8, 1.0, A, A) == J.ERR_SHAPE
    assert _status(J.jssa_indexed_decode, ok, A, A, A, A, 5000, 8, 1.0, A, A) == J.ERR_SHAPE
    assert _status(J.jssa_indexed_decode, ok, A, A, A, A, 256, 65, 1.0, A, A) == J.ERR_SHAPE
    assert _status(J.jssa_append_kv, ok, A, A, A, A, A, A, A, 0) == J.ERR_SHAPE
    assert _status(J.jssa_gather_kv, ok, A, A, A, 256, A, MIS, None) == J.ERR_ALIGN


def test_topk_workspace(J):
    n = J.jssa_topk_workspace_size(16, 8, 131072, 256)
    assert n > 16 * 8 * 256 * 8           # at least one candidate list per row
    assert J.jssa_topk_workspace_size(1, 1, 1000, 10) > 0
    assert _status(J.jssa_topk_workspace_size, 1, 1, 100, 101) == J.ERR_SHAPE
    assert _status(J.jssa_topk_workspace_size, 1, 1, 10000, 4097) == J.ERR_SHAPE
    assert _status(J.jssa_topk, 16, 8, 131072, None, A, 256, A, A, n - 1) == J.ERR_WORKSPACE
    assert _status(J.jssa_topk, 16, 8, 131072, None, None, 256, A, A, n) == J.ERR_NULL
    for T, k in [(1 << 24, 4096), (1 << 24, 1), (262144, 4096), (131072, 2048)]:
        assert J.jssa_topk_workspace_size(4, 2, T, k) > 0


def test_workspace_is_bounded_by_the_budget(J):
    """Each 8192-token chunk keeps at most max(2k, k + 64) candidates, so the
    workspace grows with the budget, not with the chunk length: at 128K x
    B = 16 x Hkv = 8 with k = 256 it stays under 64 MB (16 segments of 512
    key/index slots per row, plus one 16-byte summary per segment)."""
    d = J.gqa_desc(16, 32, 8, 32, 131072)
    n = J.jssa_score_topk_workspace_size(d, 256)
    rows, nseg = 16 * 8, 16
    assert n <= 64 << 20
    assert n >= rows * nseg * (512 * 8 + 16)
    assert J.jssa_topk_workspace_size(16, 8, 131072, 256) <= 64 << 20
    # and it grows with k (two candidate slots per budget unit per chunk)
    assert J.jssa_score_topk_workspace_size(d, 1024) > 3 * n


def test_combine_and_mla_validation(J):
    assert _status(J.jssa_combine, 1, 1, 0, 128, A, A, A) == J.ERR_SHAPE
    assert _status(J.jssa_combine, 1, 1, 4, 130, A, A, A) == J.ERR_UNSUPPORTED
    assert _status(J.jssa_combine, 1, 1, 4, 128, A, A, A, 0, A + 2) == J.ERR_ALIGN
    m_ok = J.mla_desc(4, 128, 64, 131072)
    m_badh = J.mla_desc(4, 100, 64, 131072)
    m_badr = J.mla_desc(4, 128, 48, 131072)
    assert _status(J.jssa_mla_score, m_badh, A, A, A) == J.ERR_UNSUPPORTED
    assert _status(J.jssa_mla_score, m_badr, A, A, A) == J.ERR_UNSUPPORTED
    assert _status(J.jssa_mla_absorb_q, m_ok, A, A, A, None, A, A, A) == J.ERR_NULL
    assert _status(J.jssa_mla_absorb_q, m_ok, A, A, A, A, None, A, A) == J.ERR_NULL   # no folded weights
    assert _status(J.jssa_mla_fold_selection, m_ok, A, None, A) == J.ERR_NULL
    assert _status(J.jssa_mla_fold_selection, m_badr, A, A, A) == J.ERR_UNSUPPORTED
    assert _status(J.jssa_mla_indexed_decode, m_ok, A, A, A, 2048, 0, 0.1, A, A) == J.ERR_SHAPE
    assert _status(J.jssa_mla_up_v, m_ok, A, None, A) == J.ERR_NULL


def test_calib_validation(J):
    ok = J.gqa_desc(2, 32, 8, 32, 4096)
    need = J.jssa_calib_workspace_size(ok)
    assert need > 0
    assert _status(J.jssa_calib_key_moments, ok, A, A, A, need - 1) == J.ERR_WORKSPACE
    assert _status(J.jssa_calib_key_moments, ok, None, A, A, need) == J.ERR_NULL
    assert _status(J.jssa_calib_key_moments, ok, A, MIS, A, need) == J.ERR_ALIGN
    qneed = J.jssa_calib_query_workspace_size(8)
    assert _status(J.jssa_calib_query_moments, 0, 32, 8, A, A, A, qneed) == J.ERR_SHAPE
    assert _status(J.jssa_calib_query_moments, 16, 30, 8, A, A, A, qneed) == J.ERR_SHAPE
    assert _status(J.jssa_calib_query_moments, 16, 32, 8, A, A, A, qneed - 1) == J.ERR_WORKSPACE
    import numpy as np
    with pytest.raises(J.JssaError) as e:
        J.jssa_calib_projection(np.eye(8), np.eye(8), 9)
    assert e.value.status == J.ERR_SHAPE
    with pytest.raises(J.JssaError) as e:
        J.jssa_calib_projection(np.zeros((8, 8)), np.zeros((8, 8)), 2)
    assert e.value.status == J.ERR_SHAPE
    assert J.jssa_status_string(J.ERR_NUMERIC) == "numerical routine did not converge"


def test_calib_projection_host_matches_oracle(J):
    """The library's host spectral step (cyclic Jacobi) against the oracle's
    (numpy eigh of the same marginal operator): eigenvalues, the spanned
    subspace, orthonormality, and the closed-form diagonal case."""
    import numpy as np
    from oracle import jssa_oracle as O
    rng = np.random.default_rng(21)
    for d, r, rank_k in ((128, 32, 24), (128, 16, 128), (40, 8, 5)):
        A_ = rng.standard_normal((d, d)) / np.sqrt(d)
        B_ = rng.standard_normal((d, rank_k))
        Sq = (A_ @ A_.T).astype(np.float32)
        Sk = (B_ @ B_.T / rank_k + 0.09 * np.eye(d)).astype(np.float32)
        P, w = J.jssa_calib_projection(Sq, Sk, r)
        Po, wo = O.calibrate_projection(Sq.astype(np.float64), Sk.astype(np.float64), r)
        np.testing.assert_allclose(w, wo, rtol=1e-10, atol=1e-14)
        np.testing.assert_allclose(P.astype(np.float64).T @ P, np.eye(r), atol=2e-6)
        np.testing.assert_allclose(P @ P.T, Po @ Po.T, atol=2e-5)
    a = np.array([4.0, 1.0, 9.0, 0.5, 2.0, 3.5], np.float32)
    b = np.array([0.1, 6.0, 0.2, 0.3, 5.0, 0.4], np.float32)
    P, _ = J.jssa_calib_projection(np.diag(a), np.diag(b), 3)
    wgt = a / a.sum() + b / b.sum()
    for c, ax in enumerate(np.argsort(-wgt)[:3]):
        e = np.zeros(6, np.float32)
        e[ax] = 1.0
        np.testing.assert_allclose(P[:, c], e, atol=1e-7)
