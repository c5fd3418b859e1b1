"""fp64 CPU oracle for one zero-copy decode step -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. The GPU path neither imports nor calls
it, and it uses nothing of the GPU path.

The arithmetic lives in ``oracle.c`` (plain C, fp64, one loop per definition;
see its header for the definition and the passages it follows). This module
only marshals numpy arrays into it. ``Oracle(path)`` loads another build of
the same source (the mutation tests use that).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "oracle.c")
LIBRARY = os.path.join(_HERE, "liboracle.so")

DEFAULT_THREADS = min(16, os.cpu_count() or 1)


def compile_library(src: str = SOURCE, out: str = LIBRARY) -> str:
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall",
                           "-o", tmp, src, "-lm"])
    os.replace(tmp, out)
    return out


def build(force: bool = False) -> str:
    if force or not os.path.exists(LIBRARY) or os.path.getmtime(LIBRARY) < os.path.getmtime(SOURCE):
        compile_library()
    return LIBRARY


def _p(a: np.ndarray) -> int:
    if not a.flags["C_CONTIGUOUS"]:
        raise ValueError("oracle inputs must be C-contiguous")
    return a.ctypes.data


class Oracle:
    def __init__(self, path: str | None = None):
        self.path = path or build()
        L = self.lib = ctypes.CDLL(self.path)
        i64, p, d = ctypes.c_int64, ctypes.c_void_p, ctypes.c_double
        L.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_to_f64.restype = d
        L.oracle_f64_to_bf16.argtypes = [d]
        L.oracle_f64_to_bf16.restype = ctypes.c_uint16
        L.oracle_qkv_projection.argtypes = [p, p, i64, i64, p]
        L.oracle_qkv_projection.restype = None
        L.oracle_softmax_scale.argtypes = [i64]
        L.oracle_softmax_scale.restype = d
        L.oracle_attention_head.argtypes = [p, i64, p, p, i64, i64, p, p, p]
        L.oracle_attention_head.restype = ctypes.c_int
        L.oracle_attention_partial.argtypes = [p, i64, p, p, i64, i64, p, p, i64, i64, p, p, p]
        L.oracle_attention_partial.restype = None
        L.oracle_merge_partials.argtypes = [i64, i64, p, p, p, p]
        L.oracle_merge_partials.restype = None
        L.oracle_kv_head_of.argtypes = [i64, i64, i64]
        L.oracle_kv_head_of.restype = i64
        L.oracle_decode_step.argtypes = [i64, i64, i64, i64, i64, p, p, p, p, p, i64,
                                         p, p, p, p, ctypes.c_int]
        L.oracle_decode_step.restype = ctypes.c_int
        L.oracle_gemm_nt_entries.argtypes = [p, p, i64, p, p, i64, p]
        L.oracle_gemm_nt_entries.restype = None

    # -- scalars ---------------------------------------------------------------
    def bf16_to_f64(self, bits) -> np.ndarray:
        b = np.asarray(bits, dtype=np.uint16)
        return np.array([self.lib.oracle_bf16_to_f64(int(v)) for v in b.reshape(-1)],
                        dtype=np.float64).reshape(b.shape)

    def f64_to_bf16(self, x) -> np.ndarray:
        a = np.asarray(x, dtype=np.float64)
        return np.array([self.lib.oracle_f64_to_bf16(float(v)) for v in a.reshape(-1)],
                        dtype=np.uint16).reshape(a.shape)

    def softmax_scale(self, d: int) -> float:
        return self.lib.oracle_softmax_scale(d)

    def kv_head_of(self, h: int, n_q_heads: int, n_kv_heads: int) -> int:
        return self.lib.oracle_kv_head_of(h, n_q_heads, n_kv_heads)

    # -- pieces ------------------------------------------------------------------
    def qkv_projection(self, x: np.ndarray, W: np.ndarray) -> np.ndarray:
        """y = W x for one hidden state x [hidden] (bf16 bits), W [N][hidden]."""
        x = np.ascontiguousarray(x, dtype=np.uint16)
        W = np.ascontiguousarray(W, dtype=np.uint16)
        n_out, hidden = W.shape
        assert x.shape == (hidden,)
        y = np.empty(n_out, dtype=np.float64)
        self.lib.oracle_qkv_projection(_p(x), _p(W), hidden, n_out, _p(y))
        return y

    @staticmethod
    def _cache(K, V, d):
        K = np.ascontiguousarray(K, dtype=np.uint16).reshape(-1, d)
        V = np.ascontiguousarray(V, dtype=np.uint16).reshape(-1, d)
        if K.shape[0] == 0:
            K = np.zeros((1, d), np.uint16)
            V = np.zeros((1, d), np.uint16)
        return K, V

    def attention_head(self, q, K, V, k_new, v_new) -> np.ndarray:
        """Softmax attention of q [d] over cache rows K, V [L][d] (bf16 bits)
        followed by the fresh token (k_new, v_new fp64 [d])."""
        q = np.ascontiguousarray(q, dtype=np.float64)
        d = q.shape[0]
        L = int(np.asarray(K).size // d)
        Kc, Vc = self._cache(K, V, d)
        kn = np.ascontiguousarray(k_new, dtype=np.float64)
        vn = np.ascontiguousarray(v_new, dtype=np.float64)
        out = np.empty(d, dtype=np.float64)
        if self.lib.oracle_attention_head(_p(q), d, _p(Kc), _p(Vc), d, L, _p(kn), _p(vn), _p(out)) != 0:
            raise MemoryError("oracle_attention_head: no memory for %d scores" % (L + 1))
        return out

    def attention_partial(self, q, K, V, k_new, v_new, t0: int, t1: int):
        q = np.ascontiguousarray(q, dtype=np.float64)
        d = q.shape[0]
        L = int(np.asarray(K).size // d)
        Kc, Vc = self._cache(K, V, d)
        kn = np.ascontiguousarray(k_new, dtype=np.float64)
        vn = np.ascontiguousarray(v_new, dtype=np.float64)
        m = ctypes.c_double()
        l = ctypes.c_double()
        o = np.empty(d, dtype=np.float64)
        self.lib.oracle_attention_partial(_p(q), d, _p(Kc), _p(Vc), d, L, _p(kn), _p(vn),
                                          t0, t1, ctypes.addressof(m), ctypes.addressof(l), _p(o))
        return m.value, l.value, o

    def merge_partials(self, m, l, o) -> np.ndarray:
        m = np.ascontiguousarray(m, dtype=np.float64)
        l = np.ascontiguousarray(l, dtype=np.float64)
        o = np.ascontiguousarray(o, dtype=np.float64)
        n, d = o.shape
        out = np.empty(d, dtype=np.float64)
        self.lib.oracle_merge_partials(n, d, _p(m), _p(l), _p(o), _p(out))
        return out

    # -- whole step ----------------------------------------------------------------
    def decode_step(self, x, W, ctx_lens, K, V, n_q_heads: int, n_kv_heads: int,
                    head_dim: int, threads: int = DEFAULT_THREADS) -> dict:
        """x [B][hidden], W [N][hidden], K/V [B][Lmax][Hkv][d] (bf16 bits),
        ctx_lens [B]. Returns fp64 attn_out [B][Hq*d], k_new/v_new [B][Hkv][d],
        q [B][Hq][d]."""
        x = np.ascontiguousarray(x, dtype=np.uint16)
        W = np.ascontiguousarray(W, dtype=np.uint16)
        ctx = np.ascontiguousarray(ctx_lens, dtype=np.int32)
        K = np.ascontiguousarray(K, dtype=np.uint16)
        V = np.ascontiguousarray(V, dtype=np.uint16)
        B, hidden = x.shape
        Lmax = K.shape[1]
        if Lmax == 0:
            K = np.zeros((B, 1, n_kv_heads, head_dim), np.uint16)
            V = K
        attn = np.empty((B, n_q_heads * head_dim), dtype=np.float64)
        kn = np.empty((B, n_kv_heads, head_dim), dtype=np.float64)
        vn = np.empty((B, n_kv_heads, head_dim), dtype=np.float64)
        q = np.empty((B, n_q_heads, head_dim), dtype=np.float64)
        rc = self.lib.oracle_decode_step(B, hidden, n_q_heads, n_kv_heads, head_dim,
                                         _p(x), _p(W), _p(ctx), _p(K), _p(V), max(Lmax, 1),
                                         _p(attn), _p(kn), _p(vn), _p(q), threads)
        if rc != 0:
            raise ValueError("oracle_decode_step rejected its arguments or ran out of memory")
        return {"attn_out": attn, "k_new": kn, "v_new": vn, "q": q}

    # -- host-operand GEMM (C = A x B^T) ------------------------------------------
    def gemm_nt_entries(self, A, B, rows, cols) -> np.ndarray:
        """C[rows[e]][cols[e]] of C = A x B^T in fp64 (A [M][K], B [N][K] bf16 bits)."""
        A = np.ascontiguousarray(A, dtype=np.uint16)
        B = np.ascontiguousarray(B, dtype=np.uint16)
        assert A.ndim == 2 and B.ndim == 2 and A.shape[1] == B.shape[1]
        r = np.ascontiguousarray(rows, dtype=np.int64)
        c = np.ascontiguousarray(cols, dtype=np.int64)
        assert r.shape == c.shape
        assert r.size == 0 or (0 <= r.min() and r.max() < A.shape[0]
                               and 0 <= c.min() and c.max() < B.shape[0])
        out = np.empty(r.shape, dtype=np.float64)
        self.lib.oracle_gemm_nt_entries(_p(A), _p(B), A.shape[1], _p(r), _p(c), r.size, _p(out))
        return out

    def gemm_nt(self, A, B) -> np.ndarray:
        """Full C = A x B^T in fp64 (small shapes)."""
        M, N = np.asarray(A).shape[0], np.asarray(B).shape[0]
        rows, cols = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
        return self.gemm_nt_entries(A, B, rows.reshape(-1), cols.reshape(-1)).reshape(M, N)


_default: Oracle | None = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default

