"""One GPU's share of a sharded decode step gives the same bits as the whole
batch on one GPU.

The two ways of splitting a step over GPUs that need no communication before
the output -- by sequence (each GPU holds some of the sequences) and by KV
head (each GPU holds some KV heads, their query heads and the matching W_qkv
rows, as in tensor parallelism) -- leave every output element's arithmetic
unchanged, provided the split size and the projection's form are the same on
every GPU. By default both follow the batch, so a sharded deployment fixes
them; here the DKV_SPLIT_TOKENS and DKV_PROJ_* knobs do. Each test runs the
share on its own layout and compares it bit for bit with the matching slice
of the whole batch's output, with host and HBM pages mixed.
"""
import numpy as np
import pytest

from synth import configs
from tests import harness as H

pytestmark = pytest.mark.gpu

FIXED = {"DKV_SPLIT_TOKENS": "256", "DKV_PROJ_MFMA_MIN_BATCH": "1", "DKV_PROJ_SPLITK_MIN_BATCH": "1"}


def _bits(t):
    return t.cpu().numpy().view(np.uint32)


@pytest.fixture
def fixed_knobs(monkeypatch):
    for k, v in FIXED.items():
        monkeypatch.setenv(k, v)


@pytest.mark.parametrize("first", [1, 2, 3])
def test_sequence_share_matches_full_batch(fixed_knobs, first):
    """The first `first` sequences on a layout of their own: their inputs are
    the whole batch's first sequences element for element (the generator's
    streams are per sequence), and so must their fp32 outputs be."""
    parent = configs.LLAMA70B_LONG.replace(batch=6, n_layers=1)
    ctx = np.array([700, 47, 1000, 0, 256, 3000], np.int32)
    tail = np.array([0, 16, 1 << 20, 0, 100, 500], np.int32)
    whole = H.Setup(parent, ctx_lens=ctx, hbm_tail=tail)
    try:
        ref = _bits(whole.run(f32=True))
    finally:
        whole.free()
    share = H.Setup(configs.SHARE_70B_BY_SEQUENCE.replace(batch=first, n_layers=1), ctx_lens=ctx[:first],
                    hbm_tail=tail[:first])
    try:
        assert share.layout.split_tokens == 256
        got = _bits(share.run(f32=True))
    finally:
        share.free()
    assert np.array_equal(got, ref[:first])


@pytest.mark.parametrize("g0,kh", [(0, 1), (3, 1), (6, 2)])
def test_kv_head_share_matches_full_batch(fixed_knobs, g0, kh):
    """KV heads g0 .. g0+kh-1 on a layout of their own: the share's W_qkv is
    the whole W's rows of those heads' query heads, K head and V head (in
    [Q | K | V] order), its pages hold those heads' K/V, and its output must
    be the whole output's columns of those query heads, bit for bit."""
    parent = configs.LLAMA8B_HOST.replace(batch=3, n_layers=1)
    d, Hq, Hkv, G = parent.head_dim, parent.n_q_heads, parent.n_kv_heads, parent.group
    ctx = np.array([700, 1000, 33], np.int32)
    tail = np.array([0, 300, 1 << 20], np.int32)
    whole = H.Setup(parent, ctx_lens=ctx, hbm_tail=tail)
    try:
        ref = _bits(whole.run(f32=True))
    finally:
        whole.free()

    sub = parent.replace(name=parent.name + "-kvheads", n_q_heads=kh * G, n_kv_heads=kh)
    W = parent.W(0)
    rows = np.concatenate([np.arange(g0 * G * d, (g0 + kh) * G * d),
                           Hq * d + np.arange(g0 * d, (g0 + kh) * d),
                           (Hq + Hkv) * d + np.arange(g0 * d, (g0 + kh) * d)])
    W_sub = np.ascontiguousarray(W[rows])

    def heads_only(layer, b, t0, t1):
        return (np.ascontiguousarray(parent.kv("k", layer, b, t0, t1)[:, g0:g0 + kh]),
                np.ascontiguousarray(parent.kv("v", layer, b, t0, t1)[:, g0:g0 + kh]))

    share = H.Setup(sub, ctx_lens=ctx, hbm_tail=tail, kv_writer=heads_only)
    try:
        import torch
        share.W[0] = torch.from_numpy(W_sub.view(np.int16)).cuda().view(torch.bfloat16)
        assert share.layout.split_tokens == 256
        got = _bits(share.run(f32=True))
    finally:
        share.free()
    assert np.array_equal(got, ref[:, g0 * G * d:(g0 + kh) * G * d])
