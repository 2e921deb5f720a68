"""Host-side launch policy of the Python layer (no GPU): the split count of
the indexed attention."""
import pytest

from token_level_sparse_amd.pipeline import default_splits


@pytest.mark.parametrize("k", [1, 100, 256, 512])
def test_one_split_up_to_512(k):
    # the final selection and the attention share a kernel
    assert default_splits(k, units=1) == 1
    assert default_splits(k, units=512) == 1


@pytest.mark.parametrize("k,units,want", [
    (256, 128, 2),     # 128K, B = 16, attention launched on its own: 256 blocks
    (256, 64, 4),
    (512, 16, 8),
    (64, 128, 1),      # 64 rows cannot be split further
    (100, 512, 1),     # the pairs alone fill the CUs
])
def test_unfused_attention_up_to_512_fills_the_cus(k, units, want):
    s = default_splits(k, units, attend_fused=False)
    assert s == want
    assert s == 1 or (s * units <= 256 and k // s >= 64)


@pytest.mark.parametrize("k,units,want", [
    (2048, 64, 4),     # paged Qwen: 8 sequences x 8 KV heads
    (1024, 64, 4),
    (2048, 32, 8),     # 128K, B = 4
    (2048, 128, 2),    # 128K, B = 16: two splits already fill the CUs
    (4096, 1, 32),     # one row: capped by 128 rows per split
    (513, 1, 4),
])
def test_fills_the_cus_once(k, units, want):
    assert default_splits(k, units) == want


@pytest.mark.parametrize("k", [513, 1000, 2048, 4096])
@pytest.mark.parametrize("units", [1, 3, 16, 64, 100, 256, 1000])
def test_split_rules(k, units):
    s = default_splits(k, units)
    assert s >= 2 and s & (s - 1) == 0 and s <= 64          # a power of two from 2 to 64
    assert s == 2 or k // s >= 128                          # at least 128 rows per split beyond 2
    assert s == 2 or s * units <= 256                       # never more than one block per CU beyond 2
    # the next power of two would overfill the CUs, thin the splits or pass 64
    assert 2 * s * units > 256 or 2 * s > k // 128 or s == 64
