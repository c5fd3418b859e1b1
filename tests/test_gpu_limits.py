"""The decode step at the largest batch a layout takes, and one sequence
longer than 2 GiB of KV.

A layout holds at most 65535 sequences: the step's item list packs the
sequence index into 16 bits, and the fresh-token kernel's bookkeeping for the
list reads every earlier sequence's split count. At that batch, with short
ragged contexts (0 to 40 tokens, so most sequences end inside their first or
second page), sampled sequences -- the first and the last included -- match
the oracle head by head, every output is finite, the written-back slots
hold the fresh K/V within one bf16 ulp, and the all-HBM and all-host
placements give identical bits.
"""
import numpy as np
import pytest

from synth import configs
from tests import harness as H
from tests.conftest import gpu_available
from tests.test_gpu_parity import FP32_SLACK, MAX_ABS, REL_L2, bits

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X")]

MAX_BATCH = 65535


def test_batch_at_the_layout_maximum(oracle):
    wl = configs.TINY.replace(batch=MAX_BATCH)
    rng = np.random.default_rng(65535)
    ctx = rng.choice([0, 1, 2, 15, 16, 17, 33, 40], size=MAX_BATCH).astype(np.int32)
    sample = sorted({0, 1, 2, MAX_BATCH - 2, MAX_BATCH - 1, *rng.choice(MAX_BATCH, 61, replace=False).tolist()})
    H.log("batch %d, %d cached tokens, sampled sequences %s" % (MAX_BATCH, int(ctx.sum()), sample[:8]))
    outs = []
    for tail in (1 << 20, 0):          # every page in HBM, then every page on the host
        s = H.Setup(wl, ctx_lens=ctx, hbm_tail=tail)
        try:
            outs.append(bits(s.run()))
            if len(outs) == 1:
                slots = {b: H.dkv.kv_read(s.layout, 0, b, int(ctx[b]), 1) for b in sample}
        finally:
            s.free()
    assert np.array_equal(outs[0], outs[1])
    got_all = H.bf16_to_f64(outs[0])
    assert np.all(np.isfinite(got_all))

    d, Hq, Hkv = wl.head_dim, wl.n_q_heads, wl.n_kv_heads
    got = np.stack([got_all[b] for b in sample])
    ref = np.zeros_like(got)
    x, W = wl.x(0), wl.W(0)
    for i, b in enumerate(sample):
        y = oracle.qkv_projection(x[b], W)
        for h in range(Hq):
            o, y = H.oracle_head(oracle, wl, 0, b, h, int(ctx[b]), y)
            ref[i, h * d:(h + 1) * d] = o
        for slot, want in ((slots[b][0][0], y[Hq * d:(Hq + Hkv) * d]), (slots[b][1][0], y[(Hq + Hkv) * d:])):
            have = H.bf16_to_f64(slot.reshape(-1))
            ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(want), 1e-30))) - 7) + FP32_SLACK
            assert np.all(np.abs(have - want) <= ulp), b
    assert np.abs(got - ref).max() <= MAX_ABS
    assert H.rel_l2(got, ref) <= REL_L2


def test_one_sequence_past_two_gib(oracle):
    """One sequence of 600,017 cached tokens at the 8B shape: 2.3 GiB of KV,
    so page addresses and offsets pass 2^31 bytes inside one pool. Sampled
    query heads (each KV head's first and last) match the oracle, the last
    cached tokens read back as appended, the fresh slot holds k_new / v_new
    within one bf16 ulp, and the all-host and all-HBM placements give
    identical bits (outputs and written-back slot)."""
    wl = configs.LLAMA8B_HOST.replace(batch=1)
    L = 600_017
    ctx = np.array([L], np.int32)
    outs, slots = [], []
    for tail in (0, 1 << 30):
        s = H.Setup(wl, ctx_lens=ctx, hbm_tail=tail)
        try:
            assert s.kv_bytes_read() > (1 << 31)
            outs.append(bits(s.run()))
            H.log("one sequence of %d tokens, %s: split %d tokens"
                  % (L, "host" if tail == 0 else "HBM", s.layout.split_tokens))
            # the last cached tokens read back as appended, and the fresh slot
            k_end, v_end = H.dkv.kv_read(s.layout, 0, 0, L - 3, 3)
            assert np.array_equal(k_end, wl.kv("k", 0, 0, L - 3, L))
            assert np.array_equal(v_end, wl.kv("v", 0, 0, L - 3, L))
            slots.append(H.dkv.kv_read(s.layout, 0, 0, L, 1))
        finally:
            s.free()
    assert np.array_equal(outs[0], outs[1])
    assert all(np.array_equal(a, b) for a, b in zip(slots[0], slots[1]))
    got = H.bf16_to_f64(outs[0][0])
    assert np.all(np.isfinite(got))
    d, G = wl.head_dim, wl.group
    heads = sorted({g * G for g in range(wl.n_kv_heads)} | {g * G + G - 1 for g in range(wl.n_kv_heads)})
    y = oracle.qkv_projection(wl.x(0)[0], wl.W(0))
    Hq, Hkv = wl.n_q_heads, wl.n_kv_heads
    for slot, want in ((slots[0][0][0], y[Hq * d:(Hq + Hkv) * d]), (slots[0][1][0], y[(Hq + Hkv) * d:])):
        have = H.bf16_to_f64(slot.reshape(-1))
        ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(want), 1e-30))) - 7) + FP32_SLACK
        assert np.all(np.abs(have - want) <= ulp)
    ref = np.zeros((len(heads), d))
    for i, h in enumerate(heads):
        ref[i], y = H.oracle_head(oracle, wl, 0, 0, h, L, y)
    sel = np.stack([got[h * d:(h + 1) * d] for h in heads])
    assert np.abs(sel - ref).max() <= MAX_ABS
    assert H.rel_l2(sel, ref) <= REL_L2
