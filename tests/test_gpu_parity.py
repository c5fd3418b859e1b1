"""GPU path vs the fp64 oracle, through the C ABI.

Gates (stated for bf16 inputs with fp32 accumulation): max-abs error 2e-2 and
relative L2 error 5e-3 on attn_out. Because one dropped or duplicated token
at long context moves rel-L2 by only ~1/sqrt(L), these tests also use
  * a tight gate: decode_step_f32 (no output rounding) against the oracle fed
    the same bf16-rounded fresh K/V the path writes back: rel-L2 <= 1e-4;
  * planted keys that dominate the softmax at split, page and placement edges;
  * bit-identity across placements and across repeated runs.
"""
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


def bits(t):
    import torch
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def f32(t):
    return t.cpu().numpy().astype(np.float64)


def assert_gates(got, ref, what):
    err = np.abs(got - ref)
    rel = H.rel_l2(got, ref)
    H.log("%s: max-abs %.3e rel-L2 %.3e" % (what, err.max(), rel))
    assert np.all(np.isfinite(got)), what
    assert err.max() <= MAX_ABS, (what, err.max())
    assert rel <= REL_L2, (what, rel)


def tight_reference(orc, wl, layer, ctx, heads=None, kv_writer=None, x=None, W=None):
    """Oracle outputs [B][Hq*d] with the fresh K/V rounded to bf16 as the path does."""
    x = wl.x(layer)[:len(ctx)] if x is None else x
    W = wl.W(layer) if W is None else W
    d, Hq, Hkv = wl.head_dim, wl.n_q_heads, wl.n_kv_heads
    out = np.full((len(ctx), Hq * d), np.nan)
    for b in range(len(ctx)):
        y = orc.qkv_projection(x[b], W)
        L = int(ctx[b])
        if kv_writer is not None:
            Kall, Vall = kv_writer(layer, b, 0, L) if L else (np.zeros((0, Hkv, d), np.uint16),) * 2
        for h in (range(Hq) if heads is None else heads):
            g = orc.kv_head_of(h, Hq, Hkv)
            q = y[h * d:(h + 1) * d]
            kn = H.bf16_to_f64(orc.f64_to_bf16(y[Hq * d + g * d:Hq * d + (g + 1) * d]))
            vn = H.bf16_to_f64(orc.f64_to_bf16(y[(Hq + Hkv) * d + g * d:(Hq + Hkv) * d + (g + 1) * d]))
            if kv_writer is not None:
                K, V = Kall[:, g, :], Vall[:, g, :]
            else:
                K = wl.kv_head("k", layer, b, g, 0, L)
                V = wl.kv_head("v", layer, b, g, 0, L)
            out[b, h * d:(h + 1) * d] = orc.attention_head(q, K, V, kn, vn)
    return out


def check_tight(got32, ref, what, mask=None):
    if mask is not None:
        got32, ref = got32[mask], ref[mask]
    rel = H.rel_l2(got32, ref)
    H.log("%s: tight rel-L2 %.3e" % (what, rel))
    assert rel <= TIGHT_REL_L2, (what, rel)


# --------------------------------------------------------------------------- workloads
def test_tiny_workload(oracle):
    wl = configs.TINY
    s = H.Setup(wl)
    try:
        out = s.run()
        ref = H.oracle_full(oracle, wl, 0, s.ctx)["attn_out"]
        assert_gates(H.bf16_to_f64(bits(out)), ref, wl.name)
        out32 = s.run(f32=True)
        check_tight(f32(out32), tight_reference(oracle, wl, 0, s.ctx), wl.name)
    finally:
        s.free()


@pytest.mark.parametrize("ctx", [[0, 1, 17, 1000], [33, 512, 513, 2049],
                                 [(37 * i) % 700 for i in range(40)]],
                         ids=["b4-short", "b4-mid", "b40-mfma-projection"])
def test_llama8b_shape_ragged(oracle, ctx):
    wl = configs.LLAMA8B_HOST.replace(batch=len(ctx))
    s = H.Setup(wl, ctx_lens=ctx, hbm_tail=0)
    try:
        out = s.run()
        ref = H.oracle_full(oracle, wl, 0, s.ctx)["attn_out"]
        assert_gates(H.bf16_to_f64(bits(out)), ref, "llama8b ragged %s" % ctx)
        check_tight(f32(s.run(f32=True)), tight_reference(oracle, wl, 0, s.ctx), "llama8b ragged")
    finally:
        s.free()


def test_llama70b_shape_group8(oracle):
    wl = configs.LLAMA70B_LONG.replace(batch=2, n_layers=2)
    ctx = [300, 47]
    s = H.Setup(wl, ctx_lens=ctx, hbm_tail=0)
    try:
        for li in range(2):
            out = s.run(li)
            ref = H.oracle_full(oracle, wl, li, s.ctx)["attn_out"]
            assert_gates(H.bf16_to_f64(bits(out)), ref, "llama70b layer %d" % li)
            check_tight(f32(s.run(li, f32=True)), tight_reference(oracle, wl, li, s.ctx),
                        "llama70b layer %d" % li)
    finally:
        s.free()


@pytest.mark.parametrize("wl_name", ["tiny-h512-b1-ctx1024", "llama3-8b-b8-ctx32768-host",
                                     "llama3-70b-b16-ctx131072-8layers-host"], ids=["g1", "g4", "g8"])
def test_stale_slots_do_not_leak(oracle, wl_name):
    """Slots past ctx_lens[b] in a sequence's last pages may hold any bits
    (here NaN in K and V): the masked tokens must contribute nothing."""
    ctx = [5, 16, 33, 700]
    wl = configs.BY_NAME[wl_name].replace(batch=len(ctx), n_layers=1)
    cap = [c + 40 for c in ctx]
    s = H.Setup(wl, ctx_lens=ctx, capacity=cap, hbm_tail=[0, 1 << 20, 24, 0])
    try:
        for b, (L, C) in enumerate(zip(ctx, cap)):
            nan = np.full((C - L, wl.n_kv_heads, wl.head_dim), 0x7FC0, np.uint16)
            H.dkv.kv_append(s.layout, 0, b, L, nan, nan)
        got = f32(s.run(f32=True))
        assert np.all(np.isfinite(got))
        check_tight(got, tight_reference(oracle, wl, 0, s.ctx), "%s stale NaN slots" % wl_name)
    finally:
        s.free()


@pytest.mark.parametrize("split", [16, 64, 1024])
def test_split_and_page_edges(oracle, monkeypatch, split):
    monkeypatch.setenv("DKV_SPLIT_TOKENS", str(split))
    T = split
    ctx = sorted({0, 1, 15, 16, 17, T - 1, T, T + 1, 2 * T - 1, 2 * T, 2 * T + 1, 3 * T + 5})
    wl = configs.LLAMA8B_HOST.replace(batch=len(ctx))
    s = H.Setup(wl, ctx_lens=ctx, hbm_tail=0)
    try:
        assert s.layout.split_tokens == T
        ref = tight_reference(oracle, wl, 0, s.ctx)
        check_tight(f32(s.run(f32=True)), ref, "split %d edges" % T)
        assert_gates(H.bf16_to_f64(bits(s.run())), ref, "split %d edges (bf16)" % T)
    finally:
        s.free()


# --------------------------------------------------------------------------- exactness
PROJ_KNOBS = ("DKV_PROJ_MFMA_MIN_BATCH", "DKV_PROJ_SPLITK_MIN_BATCH", "DKV_PROJ_RANGES")


@pytest.mark.parametrize("shape_name,batch,knobs", [
    ("llama8b", 1, {}), ("llama8b", 3, {}), ("llama8b", 6, {}), ("llama70b", 3, {}),
    ("llama8b", 12, {"DKV_PROJ_MFMA_MIN_BATCH": "64"}),
    ("llama8b", 3, {"DKV_PROJ_MFMA_MIN_BATCH": "1", "DKV_PROJ_SPLITK_MIN_BATCH": "1"}),
    ("llama8b", 3, {"DKV_PROJ_MFMA_MIN_BATCH": "1"}),
    ("llama8b", 1, {"DKV_PROJ_MFMA_MIN_BATCH": "1"}), ("llama8b", 8, {}),
    ("llama8b", 8, {"DKV_PROJ_SPLITK_MIN_BATCH": "16"}), ("llama8b", 16, {}),
    ("llama8b", 17, {}), ("llama8b", 32, {}), ("llama8b", 40, {}), ("llama8b", 64, {}),
    ("llama8b", 70, {}), ("llama8b", 130, {}), ("llama8b", 300, {}), ("llama8b", 384, {}), ("llama8b", 520, {}),
    ("llama8b", 520, {"DKV_PROJ_RANGES": "4"}), ("tiny", 2600, {}), ("llama8b", 12, {"DKV_PROJ_RANGES": "1"}), ("llama8b", 24, {"DKV_PROJ_RANGES": "2"}),
    ("llama8b", 48, {"DKV_PROJ_RANGES": "4"}), ("llama70b", 16, {}), ("llama70b", 33, {}),
    ("llama70b", 8, {"DKV_PROJ_SPLITK_MIN_BATCH": "16"})])
def test_projection_integer_exact(oracle, monkeypatch, shape_name, batch, knobs):
    """Small-integer x and W make every product and fp32 sum exact, so the
    written-back K/V must equal the oracle's fp64 values rounded to bf16, bit
    for bit; with an empty history attn_out is exactly bf16(v_new). Batches
    below 8 take the VALU projection by default (tiles of 4 and 8 sequences;
    16 with DKV_PROJ_MFMA_MIN_BATCH=64), and the streamed one-tile MFMA kernel
    with DKV_PROJ_MFMA_MIN_BATCH=1 (as do batches 8 to 15 with
    DKV_PROJ_SPLITK_MIN_BATCH=16); from 8 (or, forced, from 1) the split-k
    MFMA kernel stages x in tiles of 16, 32 or 64 sequences (3, 17, 40: a
    partly filled tile; 70, 130: two and three 64-sequence tiles) and writes
    one slab per range of the hidden dimension (8 by default up to one
    64-sequence tile, then 4 and 2 as the tiles grow; 1, 2 and 4 forced),
    which the fresh-token kernel adds; from 192 (when its workgroups fill
    half the CUs: 300, 384, 520, and the tiny shape at 2600) the tiled MFMA
    kernel (256-sequence tiles, the last partly filled at 300, 520 and 2600;
    W tiles dealt to the XCDs at hidden 4096, in plain order for the tiny
    shape's 12 W tiles; two ranges at 300 and 384, one at 520, four
    forced)."""
    import synth
    for k in PROJ_KNOBS:
        monkeypatch.delenv(k, raising=False)
    for k, v in knobs.items():
        monkeypatch.setenv(k, v)
    base = {"llama8b": configs.LLAMA8B_HOST, "llama70b": configs.LLAMA70B_LONG, "tiny": configs.TINY}[shape_name]
    wl = base.replace(batch=batch, n_layers=1)
    ctx = np.array([[0, 5, 16][b % 3] for b in range(batch)], np.int32)
    xi = synth.int_bf16(99, 20, 0, wl.batch * wl.hidden, -4, 4).reshape(wl.batch, wl.hidden)
    Wi = synth.int_bf16(99, 21, 0, wl.n_qkv * wl.hidden, -4, 4).reshape(wl.n_qkv, wl.hidden)
    s = H.Setup(wl, ctx_lens=ctx, hbm_tail=0)
    try:
        import torch
        s.x[0] = torch.from_numpy(xi.view(np.int16)).cuda().view(torch.bfloat16)
        s.W[0] = torch.from_numpy(Wi.view(np.int16)).cuda().view(torch.bfloat16)
        out = bits(s.run())
        d, Hq, Hkv = wl.head_dim, wl.n_q_heads, wl.n_kv_heads
        for b in range(wl.batch):
            y = oracle.qkv_projection(xi[b], Wi)
            kn = oracle.f64_to_bf16(y[Hq * d:(Hq + Hkv) * d]).reshape(Hkv, d)
            vn = oracle.f64_to_bf16(y[(Hq + Hkv) * d:]).reshape(Hkv, d)
            k_slot, v_slot = H.dkv.kv_read(s.layout, 0, b, int(ctx[b]), 1)
            assert np.array_equal(k_slot[0], kn), b
            assert np.array_equal(v_slot[0], vn), b
        # empty history: the output is the fresh value, exactly
        y = oracle.qkv_projection(xi[0], Wi)
        for h in range(Hq):
            g = oracle.kv_head_of(h, Hq, Hkv)
            vn = oracle.f64_to_bf16(y[(Hq + Hkv) * d + g * d:(Hq + Hkv) * d + (g + 1) * d])
            assert np.array_equal(out[0, h * d:(h + 1) * d], vn), h
    finally:
        s.free()


@pytest.mark.parametrize("shape_name,batch,knobs,kernel", [
    ("llama8b", 1, {}, "gemv"), ("llama8b", 7, {}, "gemv"), ("llama8b", 8, {}, "splitk"),
    ("llama8b", 64, {}, "splitk"), ("llama8b", 256, {}, "splitk"), ("llama8b", 257, {}, "tiled"),
    ("llama8b", 384, {}, "tiled"), ("llama70b", 191, {}, "splitk"), ("llama70b", 192, {}, "tiled"),
    ("tiny", 1100, {}, "splitk"), ("tiny", 2600, {}, "tiled"),
    ("llama8b", 12, {"DKV_PROJ_SPLITK_MIN_BATCH": "16"}, "stream"),
    ("llama8b", 3, {"DKV_PROJ_MFMA_MIN_BATCH": "1"}, "stream"),
    ("llama8b", 12, {"DKV_PROJ_MFMA_MIN_BATCH": "64"}, "gemv")])
def test_projection_kernel_choice(monkeypatch, shape_name, batch, knobs, kernel):
    """The projection form a layout reports (and its steps run): the GEMV
    below 8 sequences, the split-k kernel from 8, the tiled kernel from 192
    sequences once its workgroups fill half the CUs (at hidden 4096, 48 W
    tiles, from 257: one 256-sequence tile and two ranges give 96; at hidden
    8192, 80 W tiles x 2 ranges from 192; the tiny shape's 12 W tiles from
    2600), and the thresholds' overrides."""
    for k in PROJ_KNOBS:
        monkeypatch.delenv(k, raising=False)
    for k, v in knobs.items():
        monkeypatch.setenv(k, v)
    base = {"llama8b": configs.LLAMA8B_HOST, "llama70b": configs.LLAMA70B_LONG, "tiny": configs.TINY}[shape_name]
    wl = base.replace(batch=batch, n_layers=1)
    shape = H.dkv.Shape.of(wl.hidden, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, 1)
    pool = H.dkv.kv_alloc_hbm(shape, batch)
    try:
        layout = H.dkv.kv_layout_create(shape, np.full(batch, 2, np.int32), np.full(batch, 1 << 30, np.int32),
                                        None, pool)
        assert layout.projection_kernel == "qkv_proj_%s_kernel" % kernel
        layout.free()
    finally:
        pool.free()


def test_write_back_within_one_ulp(oracle):
    wl = configs.LLAMA8B_HOST.replace(batch=2)
    ctx = np.array([40, 7], np.int32)
    s = H.Setup(wl, ctx_lens=ctx, hbm_tail=0)
    try:
        s.run()
        d, Hq, Hkv = wl.head_dim, wl.n_q_heads, wl.n_kv_heads
        for b in range(2):
            y = oracle.qkv_projection(wl.x(0)[b], wl.W(0))
            k_slot, v_slot = H.dkv.kv_read(s.layout, 0, b, int(ctx[b]), 1)
            for slot, ref in ((k_slot[0], y[Hq * d:(Hq + Hkv) * d]), (v_slot[0], y[(Hq + Hkv) * d:])):
                got = H.bf16_to_f64(slot.reshape(-1))
                ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 1e-30))) - 7) + FP32_SLACK
                assert np.all(np.abs(got - ref) <= ulp), b
            # the cached tokens before the slot are untouched
            k_prev, _ = H.dkv.kv_read(s.layout, 0, b, 0, int(ctx[b]))
            assert np.array_equal(k_prev, wl.kv("k", 0, b, 0, int(ctx[b])))
    finally:
        s.free()


# --------------------------------------------------------------------------- structure
def _planted_writer(wl, oracle, plant):
    """K/V source that plants, at each (b, t) in `plant`, keys aligned with the
    oracle's query of every head of group 0 (so the token dominates them)."""
    d, Hq, Hkv = wl.head_dim, wl.n_q_heads, wl.n_kv_heads
    G = Hq // Hkv
    qs = {}

    def writer(layer, b, t0, t1):
        k = wl.kv("k", layer, b, t0, t1)
        v = wl.kv("v", layer, b, t0, t1)
        if b not in qs:
            y = oracle.qkv_projection(wl.x(layer)[b], wl.W(layer))
            qg = y[:G * d].reshape(G, d).sum(axis=0)
            qs[b] = qg / np.linalg.norm(qg)
        for (pb, pt) in plant:
            if pb == b and t0 <= pt < t1:
                k[pt - t0, 0, :] = oracle.f64_to_bf16(qs[b] * 24.0)
        return k, v
    return writer


def test_planted_tokens_at_edges(oracle, monkeypatch):
    monkeypatch.setenv("DKV_SPLIT_TOKENS", "64")
    ctx = [200, 200, 200, 131]
    wl = configs.LLAMA8B_HOST.replace(batch=4)
    # split edges (63/64), page edges (15/16), the host/HBM boundary of sequence 2,
    # the first and last cached tokens
    plant = [(0, 63), (1, 64), (0, 15), (1, 16), (2, 111), (2, 112), (3, 0), (3, 130)]
    writer = _planted_writer(wl, oracle, plant)
    tails = np.array([0, 0, 81, 0], np.int32)      # seq 2: 201 slots, pages 7.. (token 112..) HBM
    s = H.Setup(wl, ctx_lens=ctx, hbm_tail=tails, kv_writer=writer)
    try:
        assert s.layout.page_tier(2, 7) == 1 and s.layout.page_tier(2, 6) == 0
        ref = tight_reference(oracle, wl, 0, s.ctx, kv_writer=writer)
        got = f32(s.run(f32=True))
        check_tight(got, ref, "planted")
        G = wl.group
        d = wl.head_dim
        # the planted key dominates: group-0 heads are close to V of the planted token
        for b in range(4):
            rel = H.rel_l2(got[b, :G * d], ref[b, :G * d])
            assert rel < TIGHT_REL_L2, (b, rel)
    finally:
        s.free()


def test_placement_bit_identity(oracle):
    """The same KV placed all-host, all-HBM and split must give identical bits."""
    wl = configs.LLAMA8B_HOST.replace(batch=3)
    ctx = np.array([700, 1030, 64], np.int32)
    outs, outs32, slots = [], [], []
    for tail in (0, 10 ** 6, 300):
        s = H.Setup(wl, ctx_lens=ctx, hbm_tail=tail)
        try:
            outs.append(bits(s.run()))
            outs32.append(s.run(f32=True).cpu().numpy())
            slots.append([H.dkv.kv_read(s.layout, 0, b, int(ctx[b]), 1) for b in range(3)])
        finally:
            s.free()
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])
    assert np.array_equal(outs32[0].view(np.uint32), outs32[1].view(np.uint32))
    assert np.array_equal(outs32[0].view(np.uint32), outs32[2].view(np.uint32))
    for b in range(3):
        for i in (1, 2):
            assert np.array_equal(slots[0][b][0], slots[i][b][0])
            assert np.array_equal(slots[0][b][1], slots[i][b][1])
    ref = H.oracle_full(oracle, wl, 0, ctx)["attn_out"]
    assert_gates(H.bf16_to_f64(outs[0]), ref, "placements")


@pytest.mark.parametrize("head_dim", [128, 64])
def test_kv_append_from_device_buffers(head_dim):
    """kv_append from device tensors (one scatter kernel) writes the pages a
    host-array append would: a run that starts off a page boundary and
    crosses from host pages into HBM pages reads back exactly, and after the
    original rows are written back the same way the decode step gives the
    bits it gave before. One host and one device buffer are refused."""
    import torch
    wl = configs.LLAMA8B_HOST.replace(batch=3) if head_dim == 128 else \
        configs.TINY.replace(batch=3, n_kv_heads=4)
    ctx = np.array([0, 37, 700], np.int32)
    s = H.Setup(wl, ctx_lens=ctx, hbm_tail=300)          # sequence 2: slots from 400 on are HBM
    try:
        assert s.layout.page_tier(2, 24) == 0 and s.layout.page_tier(2, 25) == 1
        before = bits(s.run())
        t0, t1 = 389, 431
        rng = np.random.default_rng(11)
        shp = (t1 - t0, wl.n_kv_heads, wl.head_dim)
        k_new = rng.integers(0, 1 << 16, shp, dtype=np.uint16) & 0x7F7F      # finite bf16 patterns
        v_new = rng.integers(0, 1 << 16, shp, dtype=np.uint16) & 0x7F7F
        dev = lambda a: torch.from_numpy(a.view(np.int16)).cuda()
        H.dkv.kv_append(s.layout, 0, 2, t0, dev(k_new), dev(v_new))
        k_back, v_back = H.dkv.kv_read(s.layout, 0, 2, t0, t1 - t0)
        assert np.array_equal(k_back, k_new) and np.array_equal(v_back, v_new)
        k_old, v_old = wl.kv("k", 0, 2, t0, t1), wl.kv("v", 0, 2, t0, t1)
        k_dev, v_host = dev(k_old), np.ascontiguousarray(v_old)
        with pytest.raises(H.dkv.DkvError):          # the C ABI refuses one device and one host buffer
            H.dkv._check(H.dkv.lib().kv_append(s.layout.handle, 0, 2, t0, t1 - t0, k_dev.data_ptr(),
                                                 v_host.ctypes.data, None))
        H.dkv.kv_append(s.layout, 0, 2, t0, dev(k_old), dev(v_old))
        torch.cuda.synchronize()
        assert np.array_equal(bits(s.run()), before)
    finally:
        s.free()


@pytest.mark.parametrize("head_dim,n_q_heads,n_kv_heads", [
    (64, 8, 4), (64, 16, 4), (64, 32, 4), (128, 8, 4), (128, 2, 2), (128, 8, 1)],
    ids=["d64-g2", "d64-g4", "d64-g8", "d128-g2", "d128-g1", "d128-g8-one-kv-head"])
def test_every_head_dim_and_group(oracle, head_dim, n_q_heads, n_kv_heads):
    """Every supported (head_dim, group) pair that the workloads do not use,
    and one KV head (the shape of a by-KV-head share of 8 heads): the
    oracle's gates with host and HBM pages mixed, identical bits across
    placements, and the naive per-query-head comparator identical to the
    grouped kernel."""
    wl = configs.TINY.replace(batch=4, hidden=1024, n_q_heads=n_q_heads, n_kv_heads=n_kv_heads,
                              head_dim=head_dim)
    ctx = np.array([0, 17, 300, 1100], np.int32)
    outs32 = []
    for tail in ([0, 40, 1 << 20, 200], 0, 1 << 20):
        s = H.Setup(wl, ctx_lens=ctx, hbm_tail=tail)
        try:
            outs32.append(s.run(f32=True).cpu().numpy())
            if len(outs32) == 1:
                check_tight(outs32[0].astype(np.float64), tight_reference(oracle, wl, 0, ctx),
                            "d%d g%d" % (head_dim, wl.group))
                assert_gates(H.bf16_to_f64(bits(s.run())), H.oracle_full(oracle, wl, 0, ctx)["attn_out"],
                             "d%d g%d" % (head_dim, wl.group))
                default = s.layout.split_kernel
                assert default == ("mfma" if wl.group >= 4 else "regs")
                s.layout.split_kernel = "naive"
                assert np.array_equal(s.run(f32=True).cpu().numpy().view(np.uint32), outs32[0].view(np.uint32))
                s.layout.split_kernel = default
        finally:
            s.free()
    for o in outs32[1:]:
        assert np.array_equal(o.view(np.uint32), outs32[0].view(np.uint32))


def test_repeat_runs_are_bitwise_identical():
    wl = configs.LLAMA8B_HOST.replace(batch=2)
    s = H.Setup(wl, ctx_lens=[3000, 1111], hbm_tail=[0, 500])
    try:
        first = bits(s.run())
        for _ in range(3):
            assert np.array_equal(bits(s.run()), first)
    finally:
        s.free()


def test_layouts_on_concurrent_streams():
    """Two layouts (group 4 with host pages, group 8 all in HBM) stepped on two
    streams at once, several steps interleaved: each keeps its own page
    tables and scratch, so every output equals the same layout's output on
    one stream, bit for bit."""
    import torch
    s4 = H.Setup(configs.LLAMA8B_HOST.replace(batch=3), ctx_lens=[700, 1030, 64], hbm_tail=0)
    s8 = H.Setup(configs.LLAMA70B_LONG.replace(batch=2, n_layers=1), ctx_lens=[2000, 333], hbm_tail=1 << 20)
    try:
        want4 = s4.run(f32=True).cpu().numpy().view(np.uint32)
        want8 = s8.run(f32=True).cpu().numpy().view(np.uint32)
        a, b = torch.cuda.Stream(), torch.cuda.Stream()
        outs4 = [torch.empty_like(torch.from_numpy(want4.view(np.float32))).cuda() for _ in range(3)]
        outs8 = [torch.empty_like(torch.from_numpy(want8.view(np.float32))).cuda() for _ in range(3)]
        torch.cuda.synchronize()
        for i in range(3):
            H.dkv.decode_step_f32(s4.layout, 0, s4.x[0], s4.W[0], s4.ctx_dev, outs4[i], a)
            H.dkv.decode_step_f32(s8.layout, 0, s8.x[0], s8.W[0], s8.ctx_dev, outs8[i], b)
        torch.cuda.synchronize()
        for i in range(3):
            assert np.array_equal(outs4[i].cpu().numpy().view(np.uint32), want4), i
            assert np.array_equal(outs8[i].cpu().numpy().view(np.uint32), want8), i
        s4.layout.check_status()
        s8.layout.check_status()
    finally:
        s4.free()
        s8.free()


def test_out_of_range_context_is_flagged():
    import torch
    wl = configs.LLAMA8B_HOST.replace(batch=2)
    s = H.Setup(wl, ctx_lens=[40, 40], hbm_tail=0)
    try:
        before = H.dkv.kv_read(s.layout, 0, 1, 0, 41)
        s.ctx_dev = torch.tensor([40, 41], dtype=torch.int32, device="cuda")   # 41 == capacity
        out = s.run(f32=True).cpu().numpy()
        with pytest.raises(H.dkv.DkvError) as ei:
            s.layout.check_status()
        assert ei.value.status == -3
        assert np.all(np.isnan(out[1])) and np.all(np.isfinite(out[0]))
        after = H.dkv.kv_read(s.layout, 0, 1, 0, 41)
        assert np.array_equal(before[0], after[0]) and np.array_equal(before[1], after[1])
        s.layout.check_status()          # the flag was cleared
        s.ctx_dev = torch.tensor([40, -1], dtype=torch.int32, device="cuda")
        out = s.run(f32=True).cpu().numpy()
        assert np.all(np.isnan(out[1]))
        with pytest.raises(H.dkv.DkvError):
            s.layout.check_status()
    finally:
        s.free()


# --------------------------------------------------------------------------- kernel variants
@pytest.mark.parametrize("wl_name,ctx", [
    ("tiny-h512-b1-ctx1024", [1024]),
    ("llama3-8b-b8-ctx32768-host", [0, 1, 17, 700, 2049]),
    ("llama3-70b-b16-ctx131072-8layers-host", [300, 47, 1025]),
], ids=["g1-d64", "g4-d128", "g8-d128"])
def test_split_kernel_variants_bit_identical(oracle, monkeypatch, wl_name, ctx):
    """The register-double-buffer and the LDS producer/consumer split kernels
    (VALU arithmetic) and, from groups of 4, the matrix-core kernel meet the
    oracle's gates with host and HBM pages mixed. Up to groups of 4 the two
    VALU kernels compute every head in the same order (identical bits); at
    group 8 the register kernel splits each page's tokens over two
    wavefronts, which changes the order of the fp32 sums. The layout's
    default is the matrix-core kernel from groups of 4; the LDS ring with a
    matrix-core consumer gives its bits exactly."""
    wl = configs.BY_NAME[wl_name].replace(batch=len(ctx), n_layers=1)
    variants = ("regs", "lds", "mfma", "ldsmfma") if wl.group >= 4 else ("regs", "lds")
    monkeypatch.delenv("DKV_SPLIT_KERNEL", raising=False)
    s = H.Setup(wl, ctx_lens=ctx[:1], hbm_tail=0)
    try:
        assert s.layout.split_kernel == ("mfma" if wl.group >= 4 else "regs")
    finally:
        s.free()
    outs, outs32 = {}, {}
    for variant in variants:
        monkeypatch.setenv("DKV_SPLIT_KERNEL", variant)
        s = H.Setup(wl, ctx_lens=ctx, hbm_tail=[0, 40, 1 << 20, 16, 0][:len(ctx)])
        try:
            assert s.layout.split_kernel == variant
            outs[variant] = bits(s.run())
            outs32[variant] = s.run(f32=True).cpu().numpy()
        finally:
            s.free()
    if wl.group < 8:
        assert np.array_equal(outs["regs"], outs["lds"])
        assert np.array_equal(outs32["regs"].view(np.uint32), outs32["lds"].view(np.uint32))
    if wl.group >= 4:
        assert np.array_equal(outs["mfma"], outs["ldsmfma"])
        assert np.array_equal(outs32["mfma"].view(np.uint32), outs32["ldsmfma"].view(np.uint32))
    ref = H.oracle_full(oracle, wl, 0, np.asarray(ctx, np.int32))["attn_out"]
    tight = tight_reference(oracle, wl, 0, np.asarray(ctx, np.int32))
    for variant in variants:
        assert_gates(H.bf16_to_f64(outs[variant]), ref, "%s %s" % (wl_name, variant))
        check_tight(outs32[variant].astype(np.float64), tight, "%s %s" % (wl_name, variant))


def test_lds_split_kernel_split_edges(oracle, monkeypatch):
    """Ring wrap-around and partial last pages: splits of 1..9 pages."""
    monkeypatch.setenv("DKV_SPLIT_KERNEL", "lds")
    monkeypatch.setenv("DKV_SPLIT_TOKENS", "144")
    ctx = [1, 15, 16, 17, 63, 64, 65, 143, 144, 145, 300]
    wl = configs.LLAMA8B_HOST.replace(batch=len(ctx))
    s = H.Setup(wl, ctx_lens=ctx, hbm_tail=0)
    try:
        assert s.layout.split_kernel == "lds" and s.layout.split_tokens == 144
        check_tight(f32(s.run(f32=True)), tight_reference(oracle, wl, 0, s.ctx), "lds split 144 edges")
    finally:
        s.free()


@pytest.mark.parametrize("wl_name", ["llama3-8b-b8-ctx32768-host", "llama3-70b-b16-ctx131072-8layers-host"],
                         ids=["g4", "g8"])
def test_lds_ring_depths_and_poison(oracle, monkeypatch, wl_name):
    """Race detector of the LDS producer/consumer handoff: ring depths 2, 3
    and 4, each with every freed slot filled with NaN before its refill
    (DKV_POISON=1), give the same bits as the unpoisoned 4-slot ring (and, at
    group 4, as the register kernel); a consumer reading a slot before its
    loads landed would show up as NaN."""
    wl = configs.BY_NAME[wl_name].replace(batch=4, n_layers=1)
    ctx = [1, 300, 1030, 2100]
    tail = [0, 40, 1 << 20, 300]

    def run(env):
        for k in ("DKV_SPLIT_KERNEL", "DKV_LDS_RING", "DKV_POISON"):
            monkeypatch.delenv(k, raising=False)
        for k, v in env.items():
            monkeypatch.setenv(k, v)
        s = H.Setup(wl, ctx_lens=ctx, hbm_tail=tail)
        try:
            return s.run(f32=True).cpu().numpy().view(np.uint32)
        finally:
            s.free()

    base = run({"DKV_SPLIT_KERNEL": "lds"})
    assert np.all(np.isfinite(base.view(np.float32)))
    for ring in ("2", "3", "4"):
        got = run({"DKV_SPLIT_KERNEL": "lds", "DKV_LDS_RING": ring, "DKV_POISON": "1"})
        assert np.array_equal(got, base), ring
    if wl.group <= 4:
        assert np.array_equal(run({"DKV_SPLIT_KERNEL": "regs"}), base)
    check_tight(base.view(np.float32).astype(np.float64), tight_reference(oracle, wl, 0, np.asarray(ctx, np.int32)),
                "lds ring %s" % wl_name)


@pytest.mark.parametrize("wl_name", ["llama3-8b-b8-ctx32768-host", "llama3-70b-b16-ctx131072-8layers-host"],
                         ids=["g4", "g8"])
def test_lds_mfma_ring_depths_poison_and_edges(oracle, monkeypatch, wl_name):
    """The LDS ring with a matrix-core consumer: ring depths 2, 3 and 4 with
    every freed slot filled with NaN before its refill (DKV_POISON=1), over
    splits of 144 tokens (9 pages: ring wrap-around) with partial first,
    middle and last pages and host and HBM pages mixed, give the bits of the
    matrix-core register kernel; a consumer reading a slot before its DMA
    landed, or a wrong swizzle, would show."""
    wl = configs.BY_NAME[wl_name].replace(n_layers=1)
    ctx = [1, 15, 16, 17, 145, 300, 1030]
    wl = wl.replace(batch=len(ctx))
    tail = [0, 1 << 20, 0, 16, 40, 300, 500]

    def run(env):
        for k in ("DKV_SPLIT_KERNEL", "DKV_LDS_RING", "DKV_POISON", "DKV_SPLIT_TOKENS"):
            monkeypatch.delenv(k, raising=False)
        monkeypatch.setenv("DKV_SPLIT_TOKENS", "144")
        for k, v in env.items():
            monkeypatch.setenv(k, v)
        s = H.Setup(wl, ctx_lens=ctx, hbm_tail=tail)
        try:
            assert s.layout.split_kernel == env["DKV_SPLIT_KERNEL"]
            return s.run(f32=True).cpu().numpy().view(np.uint32)
        finally:
            s.free()

    base = run({"DKV_SPLIT_KERNEL": "mfma"})
    assert np.all(np.isfinite(base.view(np.float32)))
    for ring in ("2", "3", "4"):
        got = run({"DKV_SPLIT_KERNEL": "ldsmfma", "DKV_LDS_RING": ring, "DKV_POISON": "1"})
        assert np.array_equal(got, base), ring
    check_tight(base.view(np.float32).astype(np.float64), tight_reference(oracle, wl, 0, np.asarray(ctx, np.int32)),
                "lds-mfma ring %s" % wl_name)


# --------------------------------------------------------------------------- comparators
@pytest.mark.parametrize("wl_name", ["llama3-8b-b8-ctx32768-host", "llama3-70b-b16-ctx131072-8layers-host"],
                         ids=["g4", "g8"])
def test_comparators_are_bit_identical(oracle, wl_name):
    """The naive zero-copy comparator (one work item per query head) and the
    staging comparator (copy-engine copy of the host pool into an HBM pool,
    then the step on the HBM copy) compute the same bits as the method."""
    wl = configs.BY_NAME[wl_name].replace(batch=3, n_layers=1)
    ctx = [700, 1030, 64]
    host = H.Setup(wl, ctx_lens=ctx, hbm_tail=0)
    zeros = lambda layer, b, t0, t1: (np.zeros((t1 - t0, wl.n_kv_heads, wl.head_dim), np.uint16),) * 2
    staged = H.Setup(wl, ctx_lens=ctx, hbm_tail=1 << 20, kv_writer=zeros)
    try:
        want = bits(host.run())
        want32 = host.run(f32=True).cpu().numpy().view(np.uint32)
        default = host.layout.split_kernel
        assert default == "mfma"
        host.layout.split_kernel = "naive"
        assert host.layout.split_kernel == "naive"
        assert np.array_equal(bits(host.run()), want)
        assert np.array_equal(host.run(f32=True).cpu().numpy().view(np.uint32), want32)
        host.layout.split_kernel = default
        assert staged.n_host_pages == 0 and staged.n_hbm_pages == host.n_host_pages
        assert not np.array_equal(bits(staged.run()), want)      # zeros before staging
        H.dkv.kv_pool_copy(staged.hbm_pool, host.host_pool, host.host_pool.info()[1])
        assert np.array_equal(bits(staged.run()), want)
        ref = H.oracle_full(oracle, wl, 0, np.asarray(ctx, np.int32))["attn_out"]
        assert_gates(H.bf16_to_f64(want), ref, "comparators")
    finally:
        host.free()
        staged.free()


def test_wave_count_does_not_change_bits(monkeypatch):
    """The register split kernel on one wavefront per item or on a few looping
    wavefronts (the default when host pages exist) gives the same bits."""
    wl = configs.LLAMA8B_HOST.replace(batch=3)
    ctx = [700, 1030, 64]
    outs = {}
    for waves in ("0", "7", None):
        if waves is None:
            monkeypatch.delenv("DKV_SPLIT_WAVES", raising=False)
        else:
            monkeypatch.setenv("DKV_SPLIT_WAVES", waves)
        s = H.Setup(wl, ctx_lens=ctx, hbm_tail=[0, 300, 0])
        try:
            assert s.layout.split_waves == (256 if waves is None else int(waves))
            outs[waves] = s.run(f32=True).cpu().numpy().view(np.uint32)
        finally:
            s.free()
    assert np.array_equal(outs["0"], outs["7"]) and np.array_equal(outs["0"], outs[None])
    monkeypatch.delenv("DKV_SPLIT_WAVES", raising=False)
    s = H.Setup(wl, ctx_lens=ctx, hbm_tail=1 << 20)
    try:
        assert s.layout.split_waves == 0          # all-HBM: one wavefront per item
    finally:
        s.free()
    s = H.Setup(wl, ctx_lens=[700, 1030, 10], hbm_tail=[1 << 20, 1 << 20, 0])
    try:
        assert s.n_host_pages == 1 and s.n_hbm_pages == 109
        assert s.layout.split_waves == 0          # 1 host page in 110: HBM decides the step
    finally:
        s.free()


# --------------------------------------------------------------------------- work-item list
ITEM_FORMS = [("regs", "0"), ("regs", "5"), ("lds", "0"), ("mfma", "0"), ("mfma", "5"), ("ldsmfma", "0")]


def test_item_list_edges(oracle, monkeypatch):
    """The split kernels take their (sequence, split) work items from a list
    the fresh-token kernel builds from ctx_lens each step, on a grid sized by
    the capacities. Sequences of capacity 1 (no split at all) and of empty
    context, contexts that shrink from one step to the next (the list is
    rebuilt), and an out-of-range sequence in the middle of the batch (it
    lists no item, the others keep theirs) give the oracle's outputs on every
    split kernel form, one wavefront per item or a few looping wavefronts,
    with identical bits across the forms of one arithmetic."""
    import torch
    monkeypatch.setenv("DKV_SPLIT_TOKENS", "64")
    wl = configs.LLAMA8B_HOST.replace(batch=7)
    cap = [1, 300, 65, 1000, 1, 2000, 130]
    # Contexts never grow from one step to the next, so the fresh K/V a step
    # writes back (slot ctx_lens[b]) is never read by a later one.
    steps = [[0, 299, 64, 999, 0, 1999, 129],
             [0, 17, 64, 64, 0, 1499, 1],
             [0, 300, 0, 5, 0, 7, 1]]            # sequence 1: ctx == capacity, out of range
    tails = [0, 1 << 20, 0, 500, 0, 1 << 20, 40]
    outs = {}
    for variant, waves in ITEM_FORMS:
        monkeypatch.setenv("DKV_SPLIT_KERNEL", variant)
        monkeypatch.setenv("DKV_SPLIT_WAVES", waves)
        s = H.Setup(wl, ctx_lens=steps[0], capacity=cap, hbm_tail=tails)
        try:
            assert s.layout.split_kernel == variant and s.layout.split_tokens == 64
            assert s.layout.split_waves == int(waves)
            got = []
            for i, ctx in enumerate(steps):
                s.ctx_dev = torch.tensor(ctx, dtype=torch.int32, device="cuda")
                got.append(s.run(f32=True).cpu().numpy())
                if i < 2:
                    s.layout.check_status()
                else:
                    with pytest.raises(H.dkv.DkvError):
                        s.layout.check_status()
            outs[(variant, waves)] = got
        finally:
            s.free()
    for i, ctx in enumerate(steps):
        c = np.asarray(ctx, np.int32)
        ok = c < np.asarray(cap)
        ref = tight_reference(oracle, wl, 0, np.where(ok, c, 0))
        for form, got in outs.items():
            assert np.all(np.isnan(got[i][~ok])), (form, i)
            check_tight(got[i].astype(np.float64), ref, "item list %s step %d" % (form, i), mask=ok)
        for a, b in (("regs", "lds"), ("mfma", "ldsmfma")):
            same = [f for f in outs if f[0] in (a, b)]
            for f in same[1:]:
                assert np.array_equal(outs[same[0]][i][ok].view(np.uint32), outs[f][i][ok].view(np.uint32)), (f, i)
