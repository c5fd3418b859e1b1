"""Sets a workload up on the GPU through the C ABI and computes the oracle's
answer for it. Used by the GPU tests; the oracle side only ever sees the
generator's inputs, never anything the GPU produced."""
from __future__ import annotations

import sys
import time

import numpy as np

import decode_attention_zero_amd as dkv
from synth.configs import PAGE_TOKENS, Workload

APPEND_CHUNK = 8192


def log(msg: str) -> None:
    print("[harness %s] %s" % (time.strftime("%H:%M:%S"), msg), flush=True)
    sys.stdout.flush()


def bf16_to_f64(bits) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def rel_l2(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.linalg.norm(got - ref) / np.linalg.norm(ref))


class Setup:
    """A workload resident on the GPU: pools, layout, KV pages, x, W, ctx_lens."""

    def __init__(self, wl: Workload, ctx_lens=None, hbm_tail=None, layers=None,
                 capacity=None, kv_writer=None, host_flags=dkv.HOST_COHERENT, verbose=False):
        import torch
        self.wl = wl
        self.layers = list(range(wl.n_layers)) if layers is None else list(layers)
        self.ctx = np.asarray(wl.ctx_lens() if ctx_lens is None else ctx_lens, dtype=np.int32)
        self.batch = len(self.ctx)
        self.capacity = (self.ctx + 1).astype(np.int32) if capacity is None else \
            np.asarray(capacity, dtype=np.int32)
        if hbm_tail is None:
            hbm_tail = wl.hbm_tail(self.ctx)
        elif np.isscalar(hbm_tail):
            hbm_tail = np.full(self.batch, hbm_tail, dtype=np.int32)
        self.hbm_tail = np.asarray(hbm_tail, dtype=np.int32)
        self.shape = dkv.Shape.of(wl.hidden, wl.n_q_heads, wl.n_kv_heads, wl.head_dim,
                                  len(self.layers))
        n_host = n_hbm = 0
        for b in range(self.batch):
            n, first = dkv.kv_placement(int(self.capacity[b]), int(self.hbm_tail[b]))
            n_host += first
            n_hbm += n - first
        n_host *= len(self.layers)
        n_hbm *= len(self.layers)
        self.host_pool = dkv.kv_alloc_host(self.shape, n_host, host_flags) if n_host else None
        self.hbm_pool = dkv.kv_alloc_hbm(self.shape, n_hbm) if n_hbm else None
        self.layout = dkv.kv_layout_create(self.shape, self.capacity, self.hbm_tail,
                                           self.host_pool, self.hbm_pool)
        self.n_host_pages, self.n_hbm_pages = n_host, n_hbm
        dev = torch.device("cuda", 0)
        self.x = []
        self.W = []
        for li, layer in enumerate(self.layers):
            x = wl.x(layer)[:self.batch]
            self.x.append(torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16))
            self.W.append(torch.from_numpy(wl.W(layer).view(np.int16)).to(dev).view(torch.bfloat16))
            for b in range(self.batch):
                L = int(self.ctx[b])
                for t0 in range(0, L, APPEND_CHUNK):
                    t1 = min(L, t0 + APPEND_CHUNK)
                    if kv_writer is not None:
                        k, v = kv_writer(layer, b, t0, t1)
                    else:
                        k = wl.kv("k", layer, b, t0, t1)
                        v = wl.kv("v", layer, b, t0, t1)
                    dkv.kv_append(self.layout, li, b, t0, k, v)
            if verbose:
                log("layer %d resident (%d sequences)" % (layer, self.batch))
        self.ctx_dev = torch.from_numpy(self.ctx.copy()).to(dev)
        self.kv_writer = kv_writer

    def run(self, li: int = 0, f32: bool = False, out=None):
        fn = dkv.decode_step_f32 if f32 else dkv.decode_step
        return fn(self.layout, li, self.x[li], self.W[li], self.ctx_dev, out)

    def host_kv_bytes(self) -> int:
        return self.n_host_pages * dkv.kv_page_bytes(self.shape)

    def kv_bytes_read(self) -> int:
        """Algorithmic KV bytes one step of one layer reads (cached tokens only)."""
        return int(self.ctx.astype(np.int64).sum()) * self.wl.kv_bytes_per_token

    def free(self):
        import torch
        torch.cuda.synchronize()
        self.layout.free()
        if self.host_pool:
            self.host_pool.free()
        if self.hbm_pool:
            self.hbm_pool.free()


# ------------------------------------------------------------------------------- oracle side
def logical_kv(wl: Workload, layer: int, ctx: np.ndarray, kv_writer=None):
    """[B][Lmax][Hkv][d] K and V in logical order (small workloads only)."""
    B = len(ctx)
    Lmax = int(ctx.max()) if B else 0
    K = np.zeros((B, max(Lmax, 1), wl.n_kv_heads, wl.head_dim), np.uint16)
    V = np.zeros_like(K)
    for b in range(B):
        L = int(ctx[b])
        if L:
            if kv_writer is not None:
                K[b, :L], V[b, :L] = kv_writer(layer, b, 0, L)
            else:
                K[b, :L] = wl.kv("k", layer, b, 0, L)
                V[b, :L] = wl.kv("v", layer, b, 0, L)
    return K, V


def oracle_full(orc, wl: Workload, layer: int, ctx: np.ndarray, x=None, W=None, kv_writer=None):
    x = wl.x(layer)[:len(ctx)] if x is None else x
    W = wl.W(layer) if W is None else W
    K, V = logical_kv(wl, layer, ctx, kv_writer)
    return orc.decode_step(x, W, ctx, K, V, wl.n_q_heads, wl.n_kv_heads, wl.head_dim)


def oracle_head(orc, wl: Workload, layer: int, b: int, h: int, L: int, y=None,
                round_fresh: bool = False):
    """Oracle output of one (sequence, query head), drawing only that KV head's
    rows from the generator. Returns (out [d], y) where y is the fp64 projection
    of sequence b (reusable across heads)."""
    if y is None:
        y = orc.qkv_projection(wl.x(layer)[b], wl.W(layer))
    d, Hq, Hkv = wl.head_dim, wl.n_q_heads, wl.n_kv_heads
    g = orc.kv_head_of(h, Hq, Hkv)
    q = y[h * d:(h + 1) * d]
    kn = y[Hq * d + g * d: Hq * d + (g + 1) * d]
    vn = y[(Hq + Hkv) * d + g * d: (Hq + Hkv) * d + (g + 1) * d]
    if round_fresh:
        kn = bf16_to_f64(orc.f64_to_bf16(kn))
        vn = bf16_to_f64(orc.f64_to_bf16(vn))
    K = wl.kv_head("k", layer, b, g, 0, L)
    V = wl.kv_head("v", layer, b, g, 0, L)
    return orc.attention_head(q, K, V, kn, vn), y
