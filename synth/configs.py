"""The five decode-step workloads as input recipes (shapes, distributions,
placement, seeds). No decode arithmetic lives here.

Shapes follow the workload list the project is measured on: a tiny plumbing
case, a Llama-3-8B-shaped layer (hidden 4096, 32 query / 8 KV heads,
head_dim 128) at three batch/context/placement mixes, and a Llama-3-70B-shaped
stack of 8 layers (hidden 8192, 64 / 8 heads). Values: W ~ N(0, sigma_w^2),
hidden states and cached K/V ~ N(0, 1), all rounded to bf16.

Element streams (see ``synth.c``): x and W use stream = layer; the K and V
caches use stream = layer * 65536 + sequence, indexed in logical order
((t * Hkv + g) * d + i); ctx_lens use tensor 5, stream 0.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass

import numpy as np

import synth

PAGE_TOKENS = 16


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    batch: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    n_layers: int
    ctx: int                  # cached tokens per sequence (when ctx_range is None)
    w_sigma: float
    ctx_range: tuple | None = None      # (lo, hi) inclusive: L_b ~ U{lo..hi}
    hbm_tail_tokens: int = 0            # last tokens (incl. the new slot) placed in HBM
    hbm_fraction: float | None = None   # alternative: fraction of the L_b+1 tokens in HBM
    x_sigma: float = 1.0
    kv_sigma: float = 1.0

    # ---- derived sizes ---------------------------------------------------
    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def n_qkv(self) -> int:
        return (self.n_q_heads + 2 * self.n_kv_heads) * self.head_dim

    @property
    def kv_bytes_per_token(self) -> int:
        return self.n_kv_heads * 2 * self.head_dim * 2

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    # ---- inputs ------------------------------------------------------------
    def ctx_lens(self) -> np.ndarray:
        if self.ctx_range is None:
            return np.full(self.batch, self.ctx, dtype=np.int32)
        lo, hi = self.ctx_range
        return synth.uniform_i32(self.seed, synth.TENSOR_CTX, 0, self.batch, lo, hi)

    def hbm_tail(self, ctx_lens: np.ndarray) -> np.ndarray:
        """Tokens (counted from the end of the L_b + 1 slots) that sit in HBM."""
        if self.hbm_fraction is not None:
            total = ctx_lens.astype(np.int64) + 1
            host = np.floor(ctx_lens.astype(np.float64) * (1.0 - self.hbm_fraction)).astype(np.int64)
            return (total - host).astype(np.int32)
        return np.full(len(ctx_lens), self.hbm_tail_tokens, dtype=np.int32)

    def x(self, layer: int = 0) -> np.ndarray:
        n = self.batch * self.hidden
        return synth.normal_bf16(self.seed, synth.TENSOR_X, layer, n, self.x_sigma).reshape(
            self.batch, self.hidden)

    def W(self, layer: int = 0) -> np.ndarray:
        n = self.n_qkv * self.hidden
        return synth.normal_bf16(self.seed, synth.TENSOR_W, layer, n, self.w_sigma).reshape(
            self.n_qkv, self.hidden)

    def kv_stream(self, layer: int, seq: int) -> int:
        return layer * 65536 + seq

    def kv(self, which: str, layer: int, seq: int, t0: int, t1: int,
           out: np.ndarray | None = None) -> np.ndarray:
        """Cached K or V rows [t1 - t0][Hkv][d] of one sequence (bf16 bits)."""
        tensor = synth.TENSOR_K if which == "k" else synth.TENSOR_V
        row = self.n_kv_heads * self.head_dim
        n = (t1 - t0) * row
        flat = None if out is None else out.reshape(-1)
        flat = synth.normal_bf16(self.seed, tensor, self.kv_stream(layer, seq), n,
                                 self.kv_sigma, offset=t0 * row, out=flat)
        return flat.reshape(t1 - t0, self.n_kv_heads, self.head_dim)

    def kv_head(self, which: str, layer: int, seq: int, g: int, t0: int, t1: int) -> np.ndarray:
        """One KV head's rows [t1 - t0][d] of one sequence (bf16 bits)."""
        tensor = synth.TENSOR_K if which == "k" else synth.TENSOR_V
        row = self.n_kv_heads * self.head_dim
        return synth.normal_bf16_rows(self.seed, tensor, self.kv_stream(layer, seq),
                                      t0 * row + g * self.head_dim, t1 - t0, self.head_dim,
                                      row, self.kv_sigma)


def _seed(i: int) -> int:
    return 0xD1EC7000 + i


# 1: tiny plumbing case (100 % host)
TINY = Workload("tiny-h512-b1-ctx1024", _seed(1), batch=1, hidden=512, n_q_heads=8,
                n_kv_heads=8, head_dim=64, n_layers=1, ctx=1024, w_sigma=0.02)
# 2: Llama-3-8B layer, batch 8 at 32768, pure zero-copy (100 % host)
LLAMA8B_HOST = Workload("llama3-8b-b8-ctx32768-host", _seed(2), batch=8, hidden=4096,
                        n_q_heads=32, n_kv_heads=8, head_dim=128, n_layers=1, ctx=32768,
                        w_sigma=0.02)
# 3: Llama-3-8B layer, batch 32, L_b ~ U{8192..131072}, last 4096 tokens in HBM
LLAMA8B_HYBRID = Workload("llama3-8b-b32-ctxU8k-128k-hbm4096", _seed(3), batch=32,
                          hidden=4096, n_q_heads=32, n_kv_heads=8, head_dim=128,
                          n_layers=1, ctx=0, ctx_range=(8192, 131072), w_sigma=0.02,
                          hbm_tail_tokens=4096)
# 4: Llama-3-8B layer, batch 64 at 16384, 50 % HBM / 50 % host
LLAMA8B_DENSE = Workload("llama3-8b-b64-ctx16384-half-hbm", _seed(4), batch=64, hidden=4096,
                         n_q_heads=32, n_kv_heads=8, head_dim=128, n_layers=1, ctx=16384,
                         w_sigma=0.02, hbm_fraction=0.5)
# 5: Llama-3-70B layers, batch 16 at 131072, 8 layers, 100 % host
LLAMA70B_LONG = Workload("llama3-70b-b16-ctx131072-8layers-host", _seed(5), batch=16,
                         hidden=8192, n_q_heads=64, n_kv_heads=8, head_dim=128, n_layers=8,
                         ctx=131072, w_sigma=0.015)

ALL = [TINY, LLAMA8B_HOST, LLAMA8B_HYBRID, LLAMA8B_DENSE, LLAMA70B_LONG]

# One GPU's share of a workload when 8 GPUs split it (each share runs alone
# on one GPU here). By sequence, a GPU holds B/8 of the sequences; these
# shares keep their parent's seed, so their inputs are the parent's first
# sequences, element for element. By KV head, a GPU holds Hkv/8 KV heads
# with their query heads and the matching W rows (drawn from the same
# distribution as the parent's W, not sliced from it).
SHARE_70B_BY_SEQUENCE = LLAMA70B_LONG.replace(name="llama3-70b-b2-ctx131072-8layers-host", batch=2)
SHARE_70B_BY_KV_HEAD = LLAMA70B_LONG.replace(name="llama3-70b-b16-ctx131072-8layers-host-1kvhead",
                                             n_q_heads=8, n_kv_heads=1)
SHARE_8B_BY_SEQUENCE = LLAMA8B_HOST.replace(name="llama3-8b-b1-ctx32768-host", batch=1)
SHARES = [SHARE_70B_BY_SEQUENCE, SHARE_70B_BY_KV_HEAD, SHARE_8B_BY_SEQUENCE]

BY_NAME = {w.name: w for w in ALL + SHARES}
