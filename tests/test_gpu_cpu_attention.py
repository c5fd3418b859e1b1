"""The host-CPU attention comparator (dkv_cpu_attention) against the oracle.

The comparator reads a layout's host pages in place on the CPU and attends
with fp32 arithmetic, so it is checked like the GPU path: element by element
against the fp64 oracle on the same seeded K/V, queries and fresh token, at
ragged lengths (empty cache, a partial page, several 1024-token work items)
and at group sizes 1, 4 and 8. A layout with HBM pages among the cached
tokens is refused. Needs a GPU only because pools are pinned with HIP."""
import numpy as np
import pytest

import synth
from synth import configs
from tests import harness as H
from tests.conftest import gpu_available

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X")]

TIGHT_REL_L2 = 1e-5
MAX_ABS = 1e-4

CASES = [
    (configs.TINY, [1, 1024, 0]),
    (configs.LLAMA8B_HOST, [0, 17, 2077]),
    (configs.LLAMA70B_LONG.replace(n_layers=1), [33, 3000]),
]


def step_inputs(wl, B):
    d, Hq, Hkv = wl.head_dim, wl.n_q_heads, wl.n_kv_heads
    q = np.stack([synth.normal_f64(wl.seed, 40, b, Hq * d) for b in range(B)]).astype(np.float32)
    kn = np.stack([synth.normal_bf16(wl.seed, 41, b, Hkv * d, 1.0) for b in range(B)])
    vn = np.stack([synth.normal_bf16(wl.seed, 42, b, Hkv * d, 1.0) for b in range(B)])
    return q.reshape(B, Hq, d), kn.reshape(B, Hkv, d), vn.reshape(B, Hkv, d)


@pytest.mark.parametrize("wl,ctx", CASES, ids=[c[0].name for c in CASES])
def test_cpu_attention_matches_oracle(oracle, wl, ctx):
    import decode_attention_zero_amd as dkv
    ctx = np.asarray(ctx, np.int32)
    B = len(ctx)
    s = H.Setup(wl, ctx_lens=ctx, hbm_tail=0, layers=[0])
    try:
        q, kn, vn = step_inputs(wl, B)
        out, used = dkv.cpu_attention(s.layout, 0, q, kn, vn, ctx, 4)
        assert used == 4
        K, V = H.logical_kv(wl, 0, ctx)
        d, Hq, Hkv = wl.head_dim, wl.n_q_heads, wl.n_kv_heads
        ref = np.zeros((B, Hq, d))
        for b in range(B):
            L = int(ctx[b])
            for h in range(Hq):
                g = oracle.kv_head_of(h, Hq, Hkv)
                ref[b, h] = oracle.attention_head(q[b, h].astype(np.float64), K[b, :L, g, :], V[b, :L, g, :],
                                                  H.bf16_to_f64(kn[b, g]), H.bf16_to_f64(vn[b, g]))
        rel = H.rel_l2(out, ref)
        H.log("cpu attention %s ctx %s: rel-L2 %.2e" % (wl.name, list(ctx), rel))
        assert np.all(np.isfinite(out))
        assert rel <= TIGHT_REL_L2
        assert np.abs(out - ref).max() <= MAX_ABS
        # Thread count does not change the arithmetic of any item or the merge order.
        out1, _ = dkv.cpu_attention(s.layout, 0, q, kn, vn, ctx, 1)
        assert np.array_equal(out1.view(np.uint32), out.view(np.uint32))
    finally:
        s.free()


def test_cpu_attention_refuses_hbm_pages():
    import decode_attention_zero_amd as dkv
    wl = configs.TINY
    ctx = np.asarray([40], np.int32)
    s = H.Setup(wl, ctx_lens=ctx, hbm_tail=16, layers=[0])
    try:
        q, kn, vn = step_inputs(wl, 1)
        with pytest.raises(dkv.DkvError, match="HBM"):
            dkv.cpu_attention(s.layout, 0, q, kn, vn, ctx, 2)
        with pytest.raises(dkv.DkvError):
            dkv.cpu_attention(s.layout, 0, q, kn, vn, np.asarray([41], np.int32), 2)   # past capacity
    finally:
        s.free()


def test_cpu_stream_read_sums_words():
    import decode_attention_zero_amd as dkv
    buf = dkv.HostBuffer(1 << 20)
    try:
        words = buf.view(np.uint64, (1 << 17,))
        words[:] = np.arange(1 << 17, dtype=np.uint64)
        assert dkv.cpu_stream_read(buf.host_ptr, 1 << 20, 3) == int(words.sum())
    finally:
        buf.free()
