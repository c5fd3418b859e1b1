"""Seeded random sweep of the decode step against the fp64 oracle.

Each case draws a shape (head_dim 64/128, group 1/2/4/8, 1-8 KV heads, hidden
512-2048), a batch with ragged context lengths (uniform, plus the page and
split edges 0, 1, 15, 16, 17, T-1, T, T+1), spare capacity, a per-sequence
HBM window, and the launch knobs the layout reads at creation (split length T,
split kernel variant, looping wavefront count, projection thresholds and
split-k range count). It
checks, through the C ABI:
  * fp32 output against the oracle fed the bf16-rounded fresh K/V:
    rel-L2 <= 1e-4;
  * bf16 output against the oracle: max-abs 2e-2, rel-L2 5e-3;
  * the written-back slot of every sequence within one bf16 ulp of the
    oracle's fresh K/V, and the cached tokens before it unchanged;
  * identical fp32 bits with every page on the host and with every page in
    HBM, on a different wavefront count (the split length fixes the bits,
    placement and launch shape must not).
Cases are printed before they run so a failure names its draw."""
import numpy as np
import pytest

from synth import configs
from tests import harness as H
from tests.conftest import gpu_available
from tests.test_gpu_parity import FP32_SLACK, MAX_ABS, REL_L2, TIGHT_REL_L2, bits, tight_reference

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X")]

N_CASES = 128
KNOBS = ("DKV_SPLIT_TOKENS", "DKV_SPLIT_KERNEL", "DKV_SPLIT_WAVES", "DKV_PROJ_MFMA_MIN_BATCH",
         "DKV_LDS_RING", "DKV_PROJ_SPLITK_MIN_BATCH", "DKV_PROJ_RANGES")


def draw(i):
    rng = np.random.default_rng(0x5EED + 7919 * i)
    d = int(rng.choice([64, 128]))
    G = int(rng.choice([1, 2, 4, 4, 8, 8]))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    hidden = int(rng.choice([512, 1024, 1536, 2048]))
    B = int(rng.integers(1, 13)) if rng.random() < 0.8 else int(rng.integers(16, 25))
    T = int(rng.choice([16, 32, 64, 144, 256, 512, 1024]))
    edges = [0, 1, 15, 16, 17, T - 1, T, T + 1, 2 * T + 1]
    ctx = [int(rng.choice(edges)) if rng.random() < 0.4 else int(rng.integers(0, 2500)) for _ in range(B)]
    slack = [int(rng.choice([0, 0, 15, 16, 100])) for _ in range(B)]
    cap = [c + 1 + s for c, s in zip(ctx, slack)]
    tail = [int(rng.choice([0, 0, 1, 16, 17, 100, 1 << 20])) if rng.random() < 0.8 else int(rng.integers(0, cc + 1))
            for cc in cap]
    variants = ["regs", "lds"] + (["mfma"] if G >= 4 else []) + (["ldsmfma"] if G >= 4 and d == 128 else [])
    env = {"DKV_SPLIT_TOKENS": str(T),
           "DKV_SPLIT_KERNEL": str(rng.choice(variants + [None])),
           "DKV_SPLIT_WAVES": str(rng.choice(["", "0", "3", "64", "256"])),
           "DKV_PROJ_MFMA_MIN_BATCH": str(rng.choice(["", "1", "8", "1000"])),
           "DKV_LDS_RING": str(rng.choice(["", "2", "3", "4"])),
           "DKV_PROJ_SPLITK_MIN_BATCH": str(rng.choice(["", "", "1", "16"])),
           "DKV_PROJ_RANGES": str(rng.choice(["", "", "1", "2", "4", "8"]))}
    env = {k: v for k, v in env.items() if v not in ("", "None")}
    wl = configs.TINY.replace(name="sweep-%d" % i, seed=0x5EED0000 + i, batch=B, hidden=hidden,
                              n_q_heads=G * Hkv, n_kv_heads=Hkv, head_dim=d)
    return wl, np.array(ctx, np.int32), np.array(cap, np.int32), np.array(tail, np.int32), env


def set_env(monkeypatch, env):
    for k in KNOBS:
        monkeypatch.delenv(k, raising=False)
    for k, v in env.items():
        monkeypatch.setenv(k, v)


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_case(oracle, monkeypatch, i):
    wl, ctx, cap, tail, env = draw(i)
    H.log("case %d: d %d Hq %d Hkv %d hidden %d batch %d ctx %s cap %s tail %s env %s"
          % (i, wl.head_dim, wl.n_q_heads, wl.n_kv_heads, wl.hidden, wl.batch, ctx.tolist(), cap.tolist(),
             tail.tolist(), env))
    set_env(monkeypatch, env)
    s = H.Setup(wl, ctx_lens=ctx, hbm_tail=tail, capacity=cap)
    try:
        assert s.layout.split_tokens == int(env["DKV_SPLIT_TOKENS"])
        if "DKV_SPLIT_KERNEL" in env:
            assert s.layout.split_kernel == env["DKV_SPLIT_KERNEL"]
        out32 = s.run(f32=True).cpu().numpy()
        out = bits(s.run())
        waves = s.layout.split_waves
        d, Hq, Hkv = wl.head_dim, wl.n_q_heads, wl.n_kv_heads
        slots = [H.dkv.kv_read(s.layout, 0, b, int(ctx[b]), 1) for b in range(wl.batch)]
        prev = [H.dkv.kv_read(s.layout, 0, b, 0, int(ctx[b]))[0] if ctx[b] else None for b in range(wl.batch)]
    finally:
        s.free()

    assert np.all(np.isfinite(out32))
    rel = H.rel_l2(out32.astype(np.float64), tight_reference(oracle, wl, 0, ctx))
    assert rel <= TIGHT_REL_L2, rel
    ref = H.oracle_full(oracle, wl, 0, ctx)["attn_out"]
    got = H.bf16_to_f64(out)
    assert np.abs(got - ref).max() <= MAX_ABS and H.rel_l2(got, ref) <= REL_L2
    for b in range(wl.batch):
        y = oracle.qkv_projection(wl.x(0)[b], wl.W(0))
        for slot, want in ((slots[b][0][0], y[Hq * d:(Hq + Hkv) * d]), (slots[b][1][0], y[(Hq + Hkv) * d:])):
            have = H.bf16_to_f64(slot.reshape(-1))
            ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(want), 1e-30))) - 7) + FP32_SLACK
            assert np.all(np.abs(have - want) <= ulp), b
        if ctx[b]:
            assert np.array_equal(prev[b], wl.kv("k", 0, b, 0, int(ctx[b]))), b

    # The same split length on other placements and another wavefront count.
    for other_tail, other_waves in ((0, "0" if waves else "5"), (1 << 20, "2")):
        set_env(monkeypatch, dict(env, DKV_SPLIT_WAVES=other_waves))
        s = H.Setup(wl, ctx_lens=ctx, hbm_tail=other_tail, capacity=cap)
        try:
            again = s.run(f32=True).cpu().numpy()
        finally:
            s.free()
        assert np.array_equal(again.view(np.uint32), out32.view(np.uint32)), (other_tail, other_waves)


N_LARGE = 6


def draw_large(i):
    """Llama-sized rows (hidden 4096 or 8192, head_dim 128, group 4 or 8) at
    batches of 8 to 300 with short contexts, so that every projection form
    (split-k with 8 to 2 ranges, the tiled kernel from 192 sequences) meets
    the attention path; KV and the oracle's projection stay small enough for
    the CPU (hidden 8192 up to batch 130)."""
    rng = np.random.default_rng(0x1A76E + 104729 * i)
    hidden = int(rng.choice([4096, 8192]))
    G = int(rng.choice([4, 8]))
    Hkv = int(rng.choice([2, 8]))
    B = int(rng.choice([8, 40, 64, 130] + ([200, 300] if hidden == 4096 else [])))
    T = int(rng.choice([16, 64, 256]))
    ctx = [int(rng.integers(0, 300)) for _ in range(B)]
    cap = [c + 1 + int(rng.choice([0, 16])) for c in ctx]
    tail = [int(rng.choice([0, 1 << 20, 32])) for _ in range(B)]
    env = {"DKV_SPLIT_TOKENS": str(T)}
    if rng.random() < 0.3:
        env["DKV_PROJ_RANGES"] = str(rng.choice(["1", "2", "4"]))
    # W's scale as in the workloads of that width (0.02 at 4096, 0.015 at
    # 8192), which keeps the projection's outputs, and so the bf16 rounding of
    # the fresh values, within the absolute gate's range.
    base = configs.LLAMA8B_HOST if hidden == 4096 else configs.LLAMA70B_LONG
    wl = base.replace(name="sweep-large-%d" % i, seed=0x1A760000 + i, batch=B, hidden=hidden,
                      n_q_heads=G * Hkv, n_kv_heads=Hkv, n_layers=1)
    return wl, np.array(ctx, np.int32), np.array(cap, np.int32), np.array(tail, np.int32), env


@pytest.mark.parametrize("i", range(N_LARGE))
def test_random_large_case(oracle, monkeypatch, i):
    wl, ctx, cap, tail, env = draw_large(i)
    H.log("large case %d: Hq %d Hkv %d hidden %d batch %d T %s env %s"
          % (i, wl.n_q_heads, wl.n_kv_heads, wl.hidden, wl.batch, env["DKV_SPLIT_TOKENS"], env))
    set_env(monkeypatch, env)
    s = H.Setup(wl, ctx_lens=ctx, hbm_tail=tail, capacity=cap)
    try:
        out32 = s.run(f32=True).cpu().numpy()
        out = bits(s.run())
    finally:
        s.free()
    assert np.all(np.isfinite(out32))
    rel = H.rel_l2(out32.astype(np.float64), tight_reference(oracle, wl, 0, ctx))
    assert rel <= TIGHT_REL_L2, rel
    ref = H.oracle_full(oracle, wl, 0, ctx)["attn_out"]
    got = H.bf16_to_f64(out)
    assert np.abs(got - ref).max() <= MAX_ABS and H.rel_l2(got, ref) <= REL_L2
    s = H.Setup(wl, ctx_lens=ctx, hbm_tail=0, capacity=cap)
    try:
        again = s.run(f32=True).cpu().numpy()
    finally:
        s.free()
    assert np.array_equal(again.view(np.uint32), out32.view(np.uint32))
