"""The five workloads at their full sizes, in the launch configuration the
benchmark times (capacity = ctx + 1, the layout's own split size, the
workload's placement), against the fp64 oracle over the WHOLE attn_out of a
layer: every sequence and query head of configs 1-4, and of layer 0 of the
eight layers of config 5 (its other layers on sampled (sequence, head) pairs,
the oracle drawing only the sampled KV head's rows).

Gates on each whole output: max-abs 2e-2 and rel-L2 5e-3 (bf16 attn_out
against the oracle's fp64 definition), plus the tight rel-L2 1e-4 of
decode_step_f32 against the oracle fed the same bf16-rounded fresh K/V. The
fresh K/V written back to slot ctx_lens[b] of every sequence must be within
one bf16 ulp (plus fp32-accumulation slack) of the oracle's fp64 projection.

Each sequence's KV is drawn from the generator once: its chunks go to
kv_append, and the whole of it to the oracle (one decode_step call per
sequence, threaded over its query heads inside the oracle, and one
attention_head call per head on host threads for the tight reference)."""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

from synth import configs
from tests import harness as H
from tests.conftest import gpu_available

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X")]

MAX_ABS = 2e-2
REL_L2 = 5e-3
TIGHT_REL_L2 = 1e-4
# fp32 accumulation error of a 4096/8192-term projection row: ~1e-5 absolute at most
# for these inputs; a misplaced slot or row would be off by ~|y| ~ 1.
FP32_SLACK = 1e-4
SAMPLES_PER_OTHER_LAYER = 2
HOST_THREADS = 16


class WholeLayerKV:
    """kv_writer for H.Setup that draws each sequence of `layer` once, whole,
    hands out its chunks and keeps it for the oracle (other layers are drawn
    chunk by chunk)."""

    def __init__(self, wl, layer):
        self.wl, self.layer = wl, layer
        self.K, self.V = {}, {}

    def __call__(self, layer, b, t0, t1):
        wl = self.wl
        if layer != self.layer:
            return wl.kv("k", layer, b, t0, t1), wl.kv("v", layer, b, t0, t1)
        if b not in self.K:
            L = int(wl.ctx_lens()[b])
            self.K[b] = wl.kv("k", layer, b, 0, L)
            self.V[b] = wl.kv("v", layer, b, 0, L)
        return self.K[b][t0:t1], self.V[b][t0:t1]

    def rows(self, b, L):
        d, Hkv = self.wl.head_dim, self.wl.n_kv_heads
        if L == 0:
            empty = np.zeros((0, Hkv, d), np.uint16)
            return empty, empty
        return self.K[b], self.V[b]


def whole_layer_reference(orc, wl, layer, ctx, kv, pool):
    """Oracle attn_out [B][Hq*d] (fp64 definition), the same with the fresh
    K/V rounded to bf16 (for the tight gate), and each sequence's fp64
    projection rows of the fresh K and V."""
    d, Hq, Hkv, G = wl.head_dim, wl.n_q_heads, wl.n_kv_heads, wl.group
    B = len(ctx)
    x, W = wl.x(layer)[:B], wl.W(layer)
    ref = np.empty((B, Hq * d))
    tight = np.empty_like(ref)
    fresh = []
    for b in range(B):
        L = int(ctx[b])
        K, V = kv.rows(b, L)
        r = orc.decode_step(x[b:b + 1], W, ctx[b:b + 1], K[None], V[None], Hq, Hkv, d, threads=HOST_THREADS)
        ref[b] = r["attn_out"][0]
        kn = H.bf16_to_f64(orc.f64_to_bf16(r["k_new"][0]))
        vn = H.bf16_to_f64(orc.f64_to_bf16(r["v_new"][0]))
        q = r["q"][0]
        jobs = []
        for g in range(Hkv):
            Kg = np.ascontiguousarray(K[:, g, :])
            Vg = np.ascontiguousarray(V[:, g, :])
            for h in range(g * G, (g + 1) * G):
                jobs.append((h, pool.submit(orc.attention_head, q[h], Kg, Vg, kn[g], vn[g])))
        for h, job in jobs:
            tight[b, h * d:(h + 1) * d] = job.result()
        fresh.append((r["k_new"][0], r["v_new"][0]))
    return ref, tight, fresh


def sample_pairs(wl, layer, n):
    rng = np.random.default_rng(1000 + layer)
    pairs = {(0, 0), (wl.batch - 1, wl.n_q_heads - 1)}
    while len(pairs) < min(n, wl.batch * wl.n_q_heads):
        pairs.add((int(rng.integers(wl.batch)), int(rng.integers(wl.n_q_heads))))
    return sorted(pairs)


def check_slots(s, li, b, k_ref, v_ref):
    k_slot, v_slot = H.dkv.kv_read(s.layout, li, b, int(s.ctx[b]), 1)
    for slot, yref in ((k_slot[0], k_ref), (v_slot[0], v_ref)):
        g = H.bf16_to_f64(slot.reshape(-1))
        yref = np.asarray(yref).reshape(-1)
        ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(yref), 1e-30))) - 7) + FP32_SLACK
        assert np.all(np.abs(g - yref) <= ulp), (li, b)


def gates(got, ref, got32, tight, what, head_dim=None):
    err = np.abs(got - ref)
    rel = H.rel_l2(got, ref)
    rel32 = H.rel_l2(got32, tight)
    where = ""
    if head_dim:
        worst = np.unravel_index(int(np.argmax(err)), err.shape)
        where = " (largest error: sequence %d, query head %d)" % (worst[0], worst[1] // head_dim)
    H.log("%s: max-abs %.3e rel-L2 %.3e tight rel-L2 %.3e over %d outputs%s"
          % (what, err.max(), rel, rel32, got.size, where))
    assert np.all(np.isfinite(got)) and np.all(np.isfinite(got32)), what
    assert err.max() <= MAX_ABS and rel <= REL_L2, (what, err.max(), rel)
    assert rel32 <= TIGHT_REL_L2, (what, rel32)


@pytest.mark.parametrize("wl", configs.ALL, ids=[w.name for w in configs.ALL])
def test_full_size_workload(oracle, wl):
    import torch
    H.log("full-size %s: setting up" % wl.name)
    kv = WholeLayerKV(wl, layer=0)
    s = H.Setup(wl, kv_writer=kv, verbose=True)
    pool = ThreadPoolExecutor(HOST_THREADS)
    try:
        d, Hq, Hkv = wl.head_dim, wl.n_q_heads, wl.n_kv_heads
        # Layer 0, whole.
        out = H.bf16_to_f64(s.run(0).view(torch.int16).cpu().numpy().view(np.uint16))
        out32 = s.run(0, f32=True).cpu().numpy().astype(np.float64)
        ref, tight, fresh = whole_layer_reference(oracle, wl, 0, s.ctx, kv, pool)
        gates(out, ref, out32, tight, "%s layer 0, whole attn_out" % wl.name, head_dim=d)
        for b in range(s.batch):
            check_slots(s, 0, b, *fresh[b])
        H.log("layer 0: write-back of all %d sequences within 1 ulp" % s.batch)
        kv.K.clear()
        kv.V.clear()
        # Other layers (config 5): sampled (sequence, query head) pairs.
        got, refs, got32, refs32 = [], [], [], []
        for li in range(1, len(s.layers)):
            layer = s.layers[li]
            o = H.bf16_to_f64(s.run(li).view(torch.int16).cpu().numpy().view(np.uint16))
            o32 = s.run(li, f32=True).cpu().numpy().astype(np.float64)
            ys = {}
            for b, h in sample_pairs(wl, layer, SAMPLES_PER_OTHER_LAYER):
                L = int(s.ctx[b])
                r, ys[b] = H.oracle_head(oracle, wl, layer, b, h, L, y=ys.get(b))
                rt, _ = H.oracle_head(oracle, wl, layer, b, h, L, y=ys[b], round_fresh=True)
                got.append(o[b, h * d:(h + 1) * d])
                refs.append(r)
                got32.append(o32[b, h * d:(h + 1) * d])
                refs32.append(rt)
            for b, y in ys.items():
                check_slots(s, li, b, y[Hq * d:(Hq + Hkv) * d], y[(Hq + Hkv) * d:])
        if got:
            gates(np.concatenate(got)[None], np.concatenate(refs)[None], np.concatenate(got32)[None],
                  np.concatenate(refs32)[None], "%s layers 1-%d, %d sampled heads"
                  % (wl.name, len(s.layers) - 1, len(got)))
        s.layout.check_status()
    finally:
        pool.shutdown()
        s.free()
