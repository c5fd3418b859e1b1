"""The bench's CPU/GPU split comparator lays its CPU-side pages out itself;
this checks that layout against the library's own element offsets
(kv_page_offset), on the CPU."""
import numpy as np

import bench
import decode_attention_zero_amd as dkv


def test_kv_pages_match_the_library_layout():
    Hkv, d, L = 8, 128, 37                       # three pages, the last partial
    shape = dkv.Shape.of(4096, 32, Hkv, d, 1)
    rng = np.random.default_rng(7)
    K = rng.integers(0, 1 << 16, (L, Hkv, d), dtype=np.uint16)
    V = rng.integers(0, 1 << 16, (L, Hkv, d), dtype=np.uint16)
    pages = bench.kv_pages(K, V, dkv.PAGE_TOKENS)
    assert pages.shape[0] == 3 and pages[0].nbytes == dkv.kv_page_bytes(shape)
    for t in range(L):
        p, tt = divmod(t, dkv.PAGE_TOKENS)
        flat = pages[p].reshape(-1)
        for g in range(Hkv):
            for c, src in ((0, K), (1, V)):
                for i in (0, 1, 63, 127):
                    assert flat[dkv.kv_page_offset(shape, tt, g, c, i) // 2] == src[t, g, i], (t, g, c, i)
    assert not pages[2].reshape(Hkv, 2, dkv.PAGE_TOKENS, d)[:, :, L - 32:].any()   # padding is zero
