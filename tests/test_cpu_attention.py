"""The host-CPU attention comparator on plain host pages (no GPU): element
by element against the fp64 oracle on seeded K/V, queries and fresh tokens.

Pages are built here in the page layout the header defines (per page:
[KV head][K|V][16 tokens][head_dim] bf16), with NaN bit patterns in every
slot past the cached tokens, at ragged lengths that cross the comparator's
1024-token work items, for head_dim 64 and 128 and groups of 1 to 8. The
thread count must not change a bit."""
import numpy as np
import pytest

import decode_attention_zero_amd as dkv
import synth
from tests import harness as H

PAGE = 16
TIGHT_REL_L2 = 1e-5
MAX_ABS = 1e-4
SEED = 0xC0A7


def build_pages(K, V, L, n_kv_heads, head_dim):
    """Pages of one sequence holding tokens [0, L) of K, V ([L][Hkv][d] bf16 bits)."""
    pages = []
    for p in range((L + PAGE - 1) // PAGE):
        page = np.full((n_kv_heads, 2, PAGE, head_dim), 0x7FC0, np.uint16)
        t0, t1 = p * PAGE, min(L, (p + 1) * PAGE)
        page[:, 0, :t1 - t0, :] = K[t0:t1].transpose(1, 0, 2)
        page[:, 1, :t1 - t0, :] = V[t0:t1].transpose(1, 0, 2)
        pages.append(page)
    return pages


@pytest.mark.parametrize("head_dim,group", [(64, 1), (64, 2), (64, 4), (64, 8), (128, 4), (128, 8)])
def test_cpu_attention_pages_match_oracle(oracle, head_dim, group):
    Hkv, Hq, d = 2, 2 * group, head_dim
    shape = dkv.Shape.of(512, Hq, Hkv, d, 1)
    ctx = np.array([0, 1, 15, 16, 17, 1023, 1024, 1025, 2100], np.int32)
    B = len(ctx)
    tag = head_dim * 16 + group
    Ks = [synth.normal_bf16(SEED, 1, tag * 64 + b, int(L) * Hkv * d, 1.0).reshape(int(L), Hkv, d) for b, L in
          enumerate(ctx)]
    Vs = [synth.normal_bf16(SEED, 2, tag * 64 + b, int(L) * Hkv * d, 1.0).reshape(int(L), Hkv, d) for b, L in
          enumerate(ctx)]
    q = np.stack([synth.normal_f64(SEED, 3, tag * 64 + b, Hq * d) for b in range(B)]).astype(np.float32)
    q = q.reshape(B, Hq, d)
    kn = np.stack([synth.normal_bf16(SEED, 4, tag * 64 + b, Hkv * d, 1.0) for b in range(B)]).reshape(B, Hkv, d)
    vn = np.stack([synth.normal_bf16(SEED, 5, tag * 64 + b, Hkv * d, 1.0) for b in range(B)]).reshape(B, Hkv, d)
    pages = [build_pages(Ks[b], Vs[b], int(ctx[b]), Hkv, d) for b in range(B)]

    out, used = dkv.cpu_attention_pages(shape, pages, q, kn, vn, ctx, 3)
    assert used == 3
    ref = np.zeros((B, Hq, d))
    for b in range(B):
        for h in range(Hq):
            g = oracle.kv_head_of(h, Hq, Hkv)
            ref[b, h] = oracle.attention_head(q[b, h].astype(np.float64), Ks[b][:, g, :], Vs[b][:, g, :],
                                              H.bf16_to_f64(kn[b, g]), H.bf16_to_f64(vn[b, g]))
    assert np.all(np.isfinite(out))
    assert H.rel_l2(out, ref) <= TIGHT_REL_L2
    assert np.abs(out - ref).max() <= MAX_ABS
    out1, _ = dkv.cpu_attention_pages(shape, pages, q, kn, vn, ctx, 1)
    assert np.array_equal(out1.view(np.uint32), out.view(np.uint32))


def test_cpu_attention_pages_rejects_bad_input():
    shape = dkv.Shape.of(512, 4, 2, 64, 1)
    page = np.zeros((2, 2, PAGE, 64), np.uint16)
    q = np.zeros((1, 4, 64), np.float32)
    kv = np.zeros((1, 2, 64), np.uint16)
    with pytest.raises(dkv.DkvError):                  # 17 tokens need two pages
        dkv.cpu_attention_pages(shape, [[page]], q, kv, kv, np.array([17], np.int32), 1)
    with pytest.raises(dkv.DkvError):                  # thread count
        dkv.cpu_attention_pages(shape, [[page]], q, kv, kv, np.array([5], np.int32), 0)
    with pytest.raises(dkv.DkvError):                  # head_dim 96 is not supported
        dkv.cpu_attention_pages(dkv.Shape.of(512, 4, 2, 96, 1), [[np.zeros((2, 2, PAGE, 96), np.uint16)]],
                                np.zeros((1, 4, 96), np.float32), np.zeros((1, 2, 96), np.uint16),
                                np.zeros((1, 2, 96), np.uint16), np.array([5], np.int32), 1)
