"""The layout's split size: the longest power-of-two split of at most 8192
tokens that leaves at least 1536 full work items (batch x KV heads x
floor(longest cached context / T)) and whose items, tails included (KV heads
x sum of ceil((capacity - 1) / T)), fit the 3072 wavefronts the matrix-core
split kernel keeps resident; failing that, the smallest T whose items fit
one round, or 8192 when none does. Layouts only (all pages in HBM); no
kernel runs."""
import numpy as np
import pytest

import decode_attention_zero_amd as dkv
from tests.conftest import gpu_available

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X")]


@pytest.mark.parametrize("batch,cached,want", [
    (32, 57344, 8192),     # 32 x 8 x 7 = 1792 full items (a threshold of 2048 gave 4096: 3584 items)
    (192, 8192, 8192),     # exactly 1536 full items
    (192, 8191, 4096),     # one token short of a full 8192 split: 1536 items of 4096
    (8, 32768, 1024),      # 1024 items at 2048 tokens are too few: 2048 of 1024
    (138, 12288, 8192),    # 4096 would give 3312 full items, past one round; 8192: 2208 items
    (192, 24575, 8192),    # 4608 items at 8192 (3 per sequence and KV head): the fewest rounds
])
def test_split_size_rule(monkeypatch, batch, cached, want):
    monkeypatch.delenv("DKV_SPLIT_TOKENS", raising=False)
    shape = dkv.Shape.of(512, 8, 8, 64, 1)                     # 8 KV heads, 32 KiB pages
    cap = np.full(batch, cached + 1, np.int32)                # the fresh token's slot
    pool = dkv.kv_alloc_hbm(shape, batch * (-(-(cached + 1) // 16)))
    try:
        layout = dkv.kv_layout_create(shape, cap, np.full(batch, 1 << 30, np.int32), None, pool)
        try:
            assert layout.split_tokens == want
        finally:
            layout.free()
    finally:
        pool.free()


def test_decode_headroom_is_not_counted(monkeypatch):
    """Capacity past the cached tokens adds a short tail split that does not
    count as an item: batch 64 x 16384 tokens keeps 4096-token splits (2048
    items) with 64 or 1000 tokens of headroom."""
    monkeypatch.delenv("DKV_SPLIT_TOKENS", raising=False)
    shape = dkv.Shape.of(512, 8, 8, 64, 1)
    for headroom in (1, 64, 1000):
        cap = np.full(64, 16384 + headroom, np.int32)
        pool = dkv.kv_alloc_hbm(shape, 64 * (-(-(16384 + headroom) // 16)))
        try:
            layout = dkv.kv_layout_create(shape, cap, np.full(64, 1 << 30, np.int32), None, pool)
            try:
                assert layout.split_tokens == 4096, headroom
            finally:
                layout.free()
        finally:
            pool.free()
