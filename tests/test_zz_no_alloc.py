"""The no-allocation variant of the score + top-k entry point
(jssa_score_topk_noalloc, candidate lists in the library's static scratch)
against jssa_score_topk with a caller workspace, through the C ABI: two calls
in a row, the second with a smaller input, each bit-identical (indices and
scores) to the allocating entry point; and a shape beyond the scratch limit
is refused without a launch."""
from dataclasses import replace

import numpy as np
import pytest
import torch

from token_level_sparse_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def J():
    from token_level_sparse_amd import jssa
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return jssa


def _both(J, PL, cfg, k):
    inp = synth.make_gqa(cfg)
    c = PL.GqaCache(inp)
    c.project()
    scores_a = torch.empty((cfg.B, cfg.Hkv, cfg.T), dtype=torch.float32, device="cuda")
    idx_a = torch.empty((cfg.B, cfg.Hkv, k), dtype=torch.int32, device="cuda")
    ws = torch.empty(J.jssa_score_topk_workspace_size(c.desc, k), dtype=torch.uint8, device="cuda")
    J.jssa_score_topk(c.desc, c.q, c.P, c.Kp, k, scores_a, idx_a, ws)
    scores_b = torch.full_like(scores_a, 7.0)
    idx_b = torch.full_like(idx_a, -7)
    J.jssa_score_topk_noalloc(c.desc, c.q, c.P, c.Kp, k, scores_b, idx_b)
    torch.cuda.synchronize()
    assert torch.equal(idx_a, idx_b)
    assert torch.equal(scores_a, scores_b)
    return idx_b


def test_noalloc_matches_workspace_entry_point_twice(J):
    from token_level_sparse_amd import pipeline as PL
    big = replace(synth.LLAMA8B_32K, B=4, T=40000, len_lo=20000, len_hi=40000, seed=91)
    small = replace(synth.TINY, seed=92)
    i1 = _both(J, PL, big, 256)
    i2 = _both(J, PL, small, 100)          # smaller, and the scratch keeps the first call's contents
    assert i1.shape != i2.shape


def test_noalloc_rejects_shapes_beyond_the_scratch(J):
    d = J.gqa_desc(64, 256, 32, 32, 1 << 20)
    need = J.jssa_score_topk_workspace_size(d, 4096)
    assert need > 16 << 20
    A = 1 << 12
    with pytest.raises(J.JssaError) as e:
        J.jssa_score_topk_noalloc(d, A, A, A, 4096, None, A)
    assert e.value.status == J.ERR_WORKSPACE and "static scratch" in str(e.value)
