"""Seeded synthetic inputs for the decode-step workloads.

A module of its own: it holds no part of the decode computation, only the
counter-based generator (Philox4x32-10 + Box-Muller, see ``synth.c``) and the
workload recipes in :mod:`synth.configs`. Both the oracle's tests and the GPU
path's tests and benchmark draw their inputs from here.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB = os.path.join(_HERE, "libsynth.so")

TENSOR_X = 1
TENSOR_W = 2
TENSOR_K = 3
TENSOR_V = 4
TENSOR_CTX = 5

DEFAULT_THREADS = min(16, os.cpu_count() or 1)


def build(force: bool = False) -> str:
    """Compile ``libsynth.so`` with gcc (OpenMP) next to its source."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        _lib = ctypes.CDLL(build())
        u64, u32, i64, i32 = ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int64, ctypes.c_int32
        p = ctypes.c_void_p
        _lib.synth_philox4x32_10.argtypes = [p, p, p]
        _lib.synth_normal_bf16.argtypes = [u64, u32, u32, u64, u64, ctypes.c_double, p, ctypes.c_int]
        _lib.synth_normal_bf16_rows.argtypes = [u64, u32, u32, u64, u64, u64, u64,
                                                ctypes.c_double, p, u64, ctypes.c_int]
        _lib.synth_normal_f64.argtypes = [u64, u32, u32, u64, u64, p]
        _lib.synth_uniform_i32.argtypes = [u64, u32, u32, u64, u64, i64, i64, p]
        _lib.synth_int_bf16.argtypes = [u64, u32, u32, u64, u64, i32, i32, p, ctypes.c_int]
        for f in ("synth_philox4x32_10", "synth_normal_bf16", "synth_normal_bf16_rows",
                  "synth_normal_f64", "synth_uniform_i32", "synth_int_bf16"):
            getattr(_lib, f).restype = None
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def philox4x32_10(ctr, key) -> np.ndarray:
    c = np.ascontiguousarray(ctr, dtype=np.uint32)
    k = np.ascontiguousarray(key, dtype=np.uint32)
    out = np.zeros(4, dtype=np.uint32)
    lib().synth_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def normal_bf16(seed: int, tensor: int, stream: int, n: int, sigma: float,
                offset: int = 0, out: np.ndarray | None = None,
                threads: int = DEFAULT_THREADS) -> np.ndarray:
    """bf16 bit patterns (uint16) of sigma * N(0, 1), elements offset..offset+n-1."""
    if out is None:
        out = np.empty(n, dtype=np.uint16)
    assert out.dtype == np.uint16 and out.size == n
    lib().synth_normal_bf16(seed, tensor, stream, offset, n, sigma, _ptr(out), threads)
    return out


def normal_bf16_rows(seed: int, tensor: int, stream: int, offset: int, n_rows: int,
                     row_len: int, src_stride: int, sigma: float,
                     threads: int = DEFAULT_THREADS) -> np.ndarray:
    """[n_rows][row_len] slice of a logical tensor whose rows are src_stride apart."""
    out = np.empty((n_rows, row_len), dtype=np.uint16)
    lib().synth_normal_bf16_rows(seed, tensor, stream, offset, n_rows, row_len, src_stride,
                                 sigma, _ptr(out), row_len, threads)
    return out


def normal_f64(seed: int, tensor: int, stream: int, n: int, offset: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.float64)
    lib().synth_normal_f64(seed, tensor, stream, offset, n, _ptr(out))
    return out


def uniform_i32(seed: int, tensor: int, stream: int, n: int, lo: int, hi: int,
                offset: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.int32)
    lib().synth_uniform_i32(seed, tensor, stream, offset, n, lo, hi, _ptr(out))
    return out


def int_bf16(seed: int, tensor: int, stream: int, n: int, lo: int, hi: int,
             offset: int = 0, threads: int = DEFAULT_THREADS) -> np.ndarray:
    out = np.empty(n, dtype=np.uint16)
    lib().synth_int_bf16(seed, tensor, stream, offset, n, lo, hi, _ptr(out), threads)
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact decode of bf16 bit patterns (for inspecting generated inputs)."""
    return (bits.astype(np.uint32) << 16).view(np.float32)
