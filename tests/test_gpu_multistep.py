"""Multi-step decode through the C ABI: decode_step followed by kv_advance,
step after step, eagerly and replayed from one captured HIP graph, on a
layout whose HBM part is a sliding window of the most recent pages.

Inputs are chosen so that every fresh K/V value is computed exactly: x holds
small integers and W_qkv small multiples of 1/16 or 1/64, so the projection
is exact in fp32 and fp64 and both sides round the same value to bf16. The oracle then
rebuilds each step's context itself (the seeded initial cache plus the K/V
it projected for the earlier steps) and never sees a GPU output.

Checked: every step's attn_out against the oracle (bf16 gates and the tight
fp32 gate); graph replays bit-identical to the eager run; after the run, the
written-back slots (host pages demoted by the window and HBM pages still in
it) equal the oracle's bf16 K/V bit for bit, the seeded cache is untouched,
and each page sits in the tier the window puts it in."""
import dataclasses

import numpy as np
import pytest

import synth
from synth import configs
from tests import harness as H
from tests.conftest import gpu_available

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X")]

MAX_ABS = 2e-2
REL_L2 = 5e-3
TIGHT_REL_L2 = 1e-4


@dataclasses.dataclass(frozen=True)
class Case:
    wl: configs.Workload
    ctx0: tuple
    steps: int
    window: int            # HBM window tokens
    w_div: float           # W_qkv = integers in [-2, 2] / w_div


TINY = Case(configs.TINY.replace(batch=3), (5, 30, 47), 40, 32, 16.0)
# Group of 8 query heads (two wavefronts per split item) and hidden 8192.
G8 = Case(configs.LLAMA70B_LONG.replace(batch=2, n_layers=1), (7, 40), 20, 32, 64.0)
# Batch 16: the projection runs on the matrix cores.
MFMA16 = Case(configs.LLAMA8B_HOST.replace(batch=16),
              tuple(int(v) for v in (np.arange(16) * 37) % 61), 18, 16, 64.0)


def bf16_bits(values: np.ndarray) -> np.ndarray:
    """Exact bf16 bit patterns of values that bf16 represents exactly."""
    f = np.asarray(values, np.float32)
    bits = (f.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(H.bf16_to_f64(bits), f.astype(np.float64))
    return bits


def step_inputs(c: Case):
    """x_t: integers in [-2, 2]; W_qkv: integers in [-2, 2] / w_div (bf16 bits)."""
    wl = c.wl
    xs = [synth.int_bf16(7, 30, t, wl.batch * wl.hidden, -2, 2).reshape(wl.batch, wl.hidden)
          for t in range(c.steps)]
    Wk = H.bf16_to_f64(synth.int_bf16(7, 31, 0, wl.n_qkv * wl.hidden, -2, 2)).reshape(wl.n_qkv, wl.hidden)
    return xs, bf16_bits(Wk / c.w_div)


def wl_kv(c: Case, which, b):
    return c.wl.kv(which, 0, b, 0, int(c.ctx0[b]))


def oracle_run(orc, c: Case, xs, W):
    """Per step: the oracle's [B][Hq*d] output and each sequence's fresh bf16 K/V."""
    wl = c.wl
    d, Hq, Hkv = wl.head_dim, wl.n_q_heads, wl.n_kv_heads
    Kc = [[wl_kv(c, "k", b)] for b in range(wl.batch)]
    Vc = [[wl_kv(c, "v", b)] for b in range(wl.batch)]
    outs, fresh = [], []
    for t in range(c.steps):
        out = np.zeros((wl.batch, Hq * d))
        fk = []
        for b in range(wl.batch):
            y = orc.qkv_projection(xs[t][b], W)
            kn = orc.f64_to_bf16(y[Hq * d:(Hq + Hkv) * d]).reshape(Hkv, d)
            vn = orc.f64_to_bf16(y[(Hq + Hkv) * d:]).reshape(Hkv, d)
            K = np.concatenate(Kc[b])
            V = np.concatenate(Vc[b])
            for h in range(Hq):
                g = orc.kv_head_of(h, Hq, Hkv)
                out[b, h * d:(h + 1) * d] = orc.attention_head(
                    y[h * d:(h + 1) * d], K[:, g, :], V[:, g, :], H.bf16_to_f64(kn[g]), H.bf16_to_f64(vn[g]))
            Kc[b].append(kn[None])
            Vc[b].append(vn[None])
            fk.append((kn, vn))
        outs.append(out)
        fresh.append(fk)
    return outs, fresh


def make_layout(c: Case, windowed: bool):
    import torch
    import decode_attention_zero_amd as dkv
    wl = c.wl
    ctx0 = np.asarray(c.ctx0, np.int32)
    shape = dkv.Shape.of(wl.hidden, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, 1)
    cap = ctx0 + c.steps + 1
    pages = [int(dkv.kv_placement(int(v), 0)[0]) for v in cap]
    host = dkv.kv_alloc_host(shape, sum(pages))
    hbm = None
    if windowed:
        hbm = dkv.kv_alloc_hbm(shape, sum(min(p, -(-c.window // 16)) for p in pages))
        layout = dkv.kv_layout_create_windowed(shape, cap, c.window, ctx0, host, hbm)
    else:
        layout = dkv.kv_layout_create(shape, cap, None, host, None)
    for b in range(wl.batch):
        if c.ctx0[b]:
            dkv.kv_append(layout, 0, b, 0, wl_kv(c, "k", b), wl_kv(c, "v", b))
    ctx = torch.from_numpy(ctx0.copy()).cuda()
    return dkv, layout, host, hbm, ctx


def free_all(layout, host, hbm):
    import torch
    torch.cuda.synchronize()
    layout.free()
    host.free()
    if hbm:
        hbm.free()


def run_eager(c: Case, windowed, xs, W):
    import torch
    dkv, layout, host, hbm, ctx = make_layout(c, windowed)
    Wd = torch.from_numpy(W.view(np.int16)).cuda().view(torch.bfloat16)
    outs = []
    try:
        for t in range(c.steps):
            x = torch.from_numpy(xs[t].view(np.int16)).cuda().view(torch.bfloat16)
            out = dkv.decode_step_f32(layout, 0, x, Wd, ctx)
            dkv.kv_advance(layout, ctx)
            outs.append(out.cpu().numpy())
        assert np.array_equal(ctx.cpu().numpy(), np.asarray(c.ctx0) + c.steps)
        layout.check_status()
        return outs, dkv, layout, host, hbm
    except Exception:
        free_all(layout, host, hbm)
        raise


def check_against_oracle(orc, c: Case, windowed):
    xs, W = step_inputs(c)
    ref, fresh = oracle_run(orc, c, xs, W)
    outs, dkv, layout, host, hbm = run_eager(c, windowed, xs, W)
    try:
        worst = 0.0
        for t in range(c.steps):
            got = outs[t].astype(np.float64)
            rel = H.rel_l2(got, ref[t])
            worst = max(worst, rel)
            assert np.all(np.isfinite(got)), t
            assert rel <= TIGHT_REL_L2, (t, rel)
            assert np.abs(got - ref[t]).max() <= MAX_ABS, t
        H.log("multistep %s %s: %d steps, worst tight rel-L2 %.3e" % (
            c.wl.name, "window" if windowed else "static", c.steps, worst))
        Wp = -(-c.window // 16)
        for b in range(c.wl.batch):
            L0 = int(c.ctx0[b])
            k_all, v_all = dkv.kv_read(layout, 0, b, 0, L0 + c.steps)
            assert np.array_equal(k_all[:L0], wl_kv(c, "k", b)), b
            assert np.array_equal(v_all[:L0], wl_kv(c, "v", b)), b
            for t in range(c.steps):
                assert np.array_equal(k_all[L0 + t], fresh[t][b][0]), (b, t)
                assert np.array_equal(v_all[L0 + t], fresh[t][b][1]), (b, t)
            if windowed:
                P = (L0 + c.steps) // 16
                for p in range((L0 + c.steps + 1 + 15) // 16):
                    want = 1 if P - Wp < p <= P else 0
                    assert layout.page_tier(b, p) == want, (b, p, P)
    finally:
        free_all(layout, host, hbm)


@pytest.mark.parametrize("windowed", [True, False], ids=["window", "static-host"])
def test_multistep_eager_against_oracle(oracle, windowed):
    check_against_oracle(oracle, TINY, windowed)


@pytest.mark.parametrize("case", [G8, MFMA16], ids=["group8-hidden8192", "batch16-mfma-projection"])
def test_multistep_window_other_shapes(oracle, case):
    check_against_oracle(oracle, case, True)


@pytest.mark.parametrize("case,waves", [(TINY, 0), (TINY, 256), (MFMA16, 0), (MFMA16, 256)],
                         ids=["tiny-per-item", "tiny-looping", "batch16-per-item", "batch16-looping"])
def test_multistep_graph_replay_matches_eager(oracle, monkeypatch, case, waves):
    """One captured graph (decode_step + kv_advance) replayed for every step,
    with the next step's x copied in and a synchronisation between replays;
    every replay equals the eager run bit for bit. The split kernel runs as
    one wavefront per item or as looping wavefronts that take items from the
    layout's shared counter; the step's projection kernel (at batch 16 its
    partial-sum kernel) zeroes that counter, so each replay starts the queue
    afresh. The eager outputs are the same bits under either form."""
    import torch
    c = case
    wl = c.wl
    xs, W = step_inputs(c)
    monkeypatch.setenv("DKV_SPLIT_WAVES", "0")
    plain, dkv, layout, host, hbm = run_eager(c, True, xs, W)
    free_all(layout, host, hbm)
    monkeypatch.setenv("DKV_SPLIT_WAVES", str(waves))
    eager, dkv, layout, host, hbm = run_eager(c, True, xs, W)
    assert layout.split_waves == waves
    free_all(layout, host, hbm)
    for t in range(c.steps):
        assert np.array_equal(eager[t].view(np.uint32), plain[t].view(np.uint32)), t
    dkv, layout, host, hbm, ctx = make_layout(c, True)
    try:
        assert layout.split_waves == waves
        Wd = torch.from_numpy(W.view(np.int16)).cuda().view(torch.bfloat16)
        x_buf = torch.empty((wl.batch, wl.hidden), dtype=torch.bfloat16, device="cuda")
        out = torch.empty((wl.batch, wl.n_q_heads * wl.head_dim), dtype=torch.float32, device="cuda")
        g = torch.cuda.CUDAGraph()
        stream = torch.cuda.Stream()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=stream):
            dkv.decode_step_f32(layout, 0, x_buf, Wd, ctx, out)
            dkv.kv_advance(layout, ctx)
        torch.cuda.synchronize()
        assert np.array_equal(ctx.cpu().numpy(), np.asarray(c.ctx0))    # capture ran nothing
        for t in range(c.steps):
            x_buf.copy_(torch.from_numpy(xs[t].view(np.int16)).cuda().view(torch.bfloat16))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert np.array_equal(out.cpu().numpy().view(np.uint32), eager[t].view(np.uint32)), t
        assert np.array_equal(ctx.cpu().numpy(), np.asarray(c.ctx0) + c.steps)
        layout.check_status()
    finally:
        free_all(layout, host, hbm)


def test_advance_stops_at_capacity():
    import torch
    import decode_attention_zero_amd as dkv
    wl = TINY.wl
    shape = dkv.Shape.of(wl.hidden, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, 1)
    cap = np.array([4, 40], np.int32)
    host = dkv.kv_alloc_host(shape, 1 + 3)
    layout = dkv.kv_layout_create(shape, cap, None, host, None)
    try:
        ctx = torch.tensor([2, 5], dtype=torch.int32, device="cuda")
        dkv.kv_advance(layout, ctx)                     # 3 < 4: fine
        torch.cuda.synchronize()
        layout.check_status()
        dkv.kv_advance(layout, ctx)                     # 4 would leave no slot: stays, flagged
        torch.cuda.synchronize()
        assert ctx.cpu().tolist() == [3, 7]
        with pytest.raises(dkv.DkvError):
            layout.check_status()
    finally:
        torch.cuda.synchronize()
        layout.free()
        host.free()
