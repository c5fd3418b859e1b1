"""Zero-copy decode attention for MI355X (gfx950): Python binding.

A thin ctypes layer over the C ABI in ``include/dkv.h`` (``libdkv.so``, built
in-tree by :func:`build`). Functions keep the C names; device buffers are
passed as torch tensors (only their addresses and the current HIP stream are
used), host buffers as numpy arrays. Every step of the decode path runs in the
library's HIP kernels; there is no fallback -- without the built library the
functions raise.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from ._build import LIBRARY, build_library

__all__ = [
    "DkvError", "Shape", "Pool", "Layout", "build", "lib", "kv_page_bytes", "kv_page_offset",
    "kv_placement", "kv_alloc_host", "kv_alloc_hbm", "kv_layout_create", "kv_append", "kv_read",
    "decode_step", "decode_step_f32", "probe_stream_read", "probe_stream_read_cycled", "probe_page_read",
    "PAGE_TOKENS",
]

PAGE_TOKENS = 16
HOST_COHERENT = 0
HOST_NONCOHERENT = 1

_STATUS = {0: "DKV_OK", -1: "DKV_E_INVALID_ARG", -2: "DKV_E_OUT_OF_MEMORY", -3: "DKV_E_CAPACITY",
           -4: "DKV_E_HIP", -5: "DKV_E_UNSUPPORTED"}


class DkvError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("%s: %s" % (_STATUS.get(status, str(status)), message))
        self.status = status


class Shape(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("n_layers", ctypes.c_int32), ("page_tokens", ctypes.c_int32)]

    @classmethod
    def of(cls, hidden, n_q_heads, n_kv_heads, head_dim, n_layers=1):
        return cls(hidden, n_q_heads, n_kv_heads, head_dim, n_layers, PAGE_TOKENS)


_lib = None


def build() -> str:
    """Compiles the HIP library for gfx950 (always) and returns its path."""
    global _lib
    _lib = None
    return build_library()


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIBRARY):
            raise RuntimeError("libdkv.so is not built; run __graft_entry__.build() "
                               "(decode_attention_zero_amd.build()) first")
        L = ctypes.CDLL(LIBRARY)
        P, I32, I64, U32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32
        SP = ctypes.POINTER(Shape)
        sig = {
            "dkv_last_error": ([], ctypes.c_char_p),
            "kv_page_bytes": ([SP], I64),
            "kv_page_offset": ([SP, I32, I32, I32, I32], I64),
            "kv_placement": ([I32, I32, P, P], I32),
            "kv_alloc_host": ([SP, I64, U32, P], I32),
            "kv_alloc_hbm": ([SP, I64, P], I32),
            "kv_pool_free_pages": ([P, P], I32),
            "kv_pool_info": ([P, P, P, P], I32),
            "kv_pool_free": ([P], I32),
            "kv_layout_create": ([SP, I32, P, P, P, P, P], I32),
            "kv_layout_create_windowed": ([SP, I32, P, P, P, P, P, P], I32),
            "kv_advance": ([P, P, P], I32),
            "kv_layout_free": ([P], I32),
            "kv_layout_page_tier": ([P, I32, I32, P], I32),
            "kv_layout_split_tokens": ([P], I32),
            "kv_layout_split_kernel": ([P], I32),
            "kv_layout_set_split_kernel": ([P, I32], I32),
            "kv_layout_split_waves": ([P], I32),
            "kv_layout_projection_kernel": ([P], I32),
            "kv_layout_check_status": ([P], I32),
            "kv_append": ([P, I32, I32, I32, I32, P, P, P], I32),
            "kv_read": ([P, I32, I32, I32, I32, P, P], I32),
            "decode_step": ([P, I32, P, P, P, P, P], I32),
            "decode_step_f32": ([P, I32, P, P, P, P, P], I32),
            "decode_step_noalloc": ([P, I32, P, P, P, P, P], I32),
            "decode_step_noalloc_scratch_bytes": ([], ctypes.c_size_t),
            "dkv_probe_stream_read": ([P, ctypes.c_uint64, I32, I32, I32, P], I32),
            "dkv_probe_stream_read_cycled": ([P, ctypes.c_uint64, I32, I32, I32, I32, P], I32),
            "dkv_probe_page_read": ([P, ctypes.c_uint64, I32, I32, I32, I32, I32, P], I32),
            "kv_pool_copy": ([P, P, I64, P], I32),
            "dkv_host_buffer_alloc": ([ctypes.c_uint64, U32, P, P], I32),
            "dkv_host_buffer_free": ([P], I32),
            "dkv_copy": ([P, P, ctypes.c_uint64, P], I32),
            "dkv_gemm_bf16_nt": ([P, P, P, I32, I32, I32, I32, P], I32),
            "dkv_gemm_bf16_nt_bstationary": ([P, P, P, I32, I32, I32, P, ctypes.c_uint64, P], I32),
            "dkv_gemm_bstationary_workspace_bytes": ([I32, I32, I32], ctypes.c_uint64),
            "kv_layout_timing_enable": ([P, I32, I32], I32),
            "kv_layout_timing_read": ([P, P, P, P, P, P], I32),
            "dkv_cpu_attention": ([P, I32, P, P, P, P, P, I32, P], I32),
            "dkv_cpu_stream_read": ([P, ctypes.c_uint64, I32, P], I32),
            "dkv_cpu_attention_pages": ([P, I32, SP, I32, P, P, P, P, P, I32, P], I32),
        }
        for name, (args, res) in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


EXPORTED = ["dkv_last_error", "kv_page_bytes", "kv_page_offset", "kv_placement", "kv_alloc_host",
            "kv_alloc_hbm", "kv_pool_free_pages", "kv_pool_info", "kv_pool_free",
            "kv_layout_create", "kv_layout_create_windowed", "kv_advance", "kv_layout_free", "kv_layout_page_tier", "kv_layout_split_tokens",
            "kv_layout_split_kernel", "kv_layout_set_split_kernel", "kv_layout_split_waves", "kv_layout_projection_kernel", "kv_layout_check_status", "kv_append", "kv_read", "decode_step", "decode_step_f32",
            "decode_step_noalloc", "decode_step_noalloc_scratch_bytes", "dkv_probe_stream_read", "dkv_probe_stream_read_cycled", "dkv_probe_page_read", "kv_pool_copy", "dkv_host_buffer_alloc", "dkv_host_buffer_free",
            "dkv_copy", "dkv_gemm_bf16_nt", "dkv_gemm_bf16_nt_bstationary", "dkv_gemm_bstationary_workspace_bytes",
            "kv_layout_timing_enable", "kv_layout_timing_read",
            "dkv_cpu_attention", "dkv_cpu_stream_read", "dkv_cpu_attention_pages"]


PROJECTION_KERNELS = {0: "qkv_proj_gemv_kernel", 1: "qkv_proj_stream_kernel", 2: "qkv_proj_splitk_kernel",
                      3: "qkv_proj_tiled_kernel"}


def _check(status: int) -> None:
    if status != 0:
        raise DkvError(status, lib().dkv_last_error().decode(errors="replace"))


def _np_ptr(a: np.ndarray) -> int:
    if not a.flags["C_CONTIGUOUS"]:
        raise ValueError("host buffers must be C-contiguous")
    return a.ctypes.data


def _stream_ptr(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream or None
    if isinstance(stream, int):
        return stream or None
    return stream.cuda_stream or None


# ----------------------------------------------------------------------------- pure host
def kv_page_bytes(shape: Shape) -> int:
    return lib().kv_page_bytes(ctypes.byref(shape))


def kv_page_offset(shape: Shape, token_in_page: int, kv_head: int, kv_select: int, dim: int) -> int:
    return lib().kv_page_offset(ctypes.byref(shape), token_in_page, kv_head, kv_select, dim)


def kv_placement(capacity_tokens: int, hbm_tail_tokens: int) -> tuple[int, int]:
    n = ctypes.c_int32()
    f = ctypes.c_int32()
    _check(lib().kv_placement(capacity_tokens, hbm_tail_tokens, ctypes.byref(n), ctypes.byref(f)))
    return n.value, f.value


# ----------------------------------------------------------------------------- pools, layouts
class Pool:
    def __init__(self, handle: int, shape: Shape, tier: int):
        self.handle = handle
        self.shape = shape
        self.tier = tier

    def free_pages(self) -> int:
        n = ctypes.c_int64()
        _check(lib().kv_pool_free_pages(self.handle, ctypes.byref(n)))
        return n.value

    def info(self) -> tuple[int, int, int]:
        base = ctypes.c_void_p()
        nbytes = ctypes.c_int64()
        tier = ctypes.c_int32()
        _check(lib().kv_pool_info(self.handle, ctypes.byref(base), ctypes.byref(nbytes),
                                  ctypes.byref(tier)))
        return base.value or 0, nbytes.value, tier.value

    def free(self) -> None:
        if self.handle:
            _check(lib().kv_pool_free(self.handle))
            self.handle = None


def kv_pool_copy(dst: Pool, src: Pool, nbytes: int, stream=None) -> None:
    """Staging comparator: copy-engine copy of src's first nbytes into dst."""
    _check(lib().kv_pool_copy(dst.handle, src.handle, nbytes, _stream_ptr(stream)))


def kv_alloc_host(shape: Shape, n_pages: int, flags: int = HOST_COHERENT) -> Pool:
    h = ctypes.c_void_p()
    _check(lib().kv_alloc_host(ctypes.byref(shape), n_pages, flags, ctypes.byref(h)))
    return Pool(h.value, shape, 0)


def kv_alloc_hbm(shape: Shape, n_pages: int) -> Pool:
    h = ctypes.c_void_p()
    _check(lib().kv_alloc_hbm(ctypes.byref(shape), n_pages, ctypes.byref(h)))
    return Pool(h.value, shape, 1)


class Layout:
    def __init__(self, handle: int, shape: Shape, batch: int, capacity: np.ndarray):
        self.handle = handle
        self.shape = shape
        self.batch = batch
        self.capacity = capacity

    @property
    def split_tokens(self) -> int:
        return lib().kv_layout_split_tokens(self.handle)

    @property
    def split_kernel(self) -> str:
        """'regs' (register double buffer, VALU), 'lds' (producer/consumer LDS
        ring, VALU), 'mfma' (register double buffer, matrix cores), 'ldsmfma'
        (LDS ring, matrix-core consumer) or 'naive' (comparator: one work item
        per query head)."""
        return {0: "regs", 1: "lds", 2: "naive", 3: "mfma", 4: "ldsmfma"}[lib().kv_layout_split_kernel(self.handle)]

    @property
    def split_waves(self) -> int:
        """Wavefronts of the register split kernel (0: one per work item)."""
        return lib().kv_layout_split_waves(self.handle)

    @property
    def projection_kernel(self) -> str:
        """The QKV projection kernel this layout's steps run."""
        return PROJECTION_KERNELS[lib().kv_layout_projection_kernel(self.handle)]

    @split_kernel.setter
    def split_kernel(self, name: str) -> None:
        _check(lib().kv_layout_set_split_kernel(self.handle, {"regs": 0, "lds": 1, "naive": 2, "mfma": 3,
                                                              "ldsmfma": 4}[name]))

    def page_tier(self, seq: int, page: int) -> int:
        t = ctypes.c_int32()
        _check(lib().kv_layout_page_tier(self.handle, seq, page, ctypes.byref(t)))
        return t.value

    def check_status(self) -> None:
        _check(lib().kv_layout_check_status(self.handle))

    def timing_enable(self, enable: bool = True, max_steps: int = 1024, split_only: bool = False) -> None:
        mode = 0 if not enable else (2 if split_only else 1)
        _check(lib().kv_layout_timing_enable(self.handle, mode, max_steps))

    def timing_read(self) -> dict:
        """Summed per-kernel milliseconds and the step count since the last read."""
        p, f, s, c = ctypes.c_double(), ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
        n = ctypes.c_int32()
        _check(lib().kv_layout_timing_read(self.handle, ctypes.byref(p), ctypes.byref(f), ctypes.byref(s),
                                           ctypes.byref(c), ctypes.byref(n)))
        return {"projection": p.value, "fresh": f.value, "split": s.value, "combine": c.value,
                "steps": n.value}

    def free(self) -> None:
        if self.handle:
            _check(lib().kv_layout_free(self.handle))
            self.handle = None


def kv_layout_create(shape: Shape, capacity_tokens, hbm_tail_tokens=None,
                     host_pool: Pool | None = None, hbm_pool: Pool | None = None) -> Layout:
    cap = np.ascontiguousarray(capacity_tokens, dtype=np.int32)
    tail = None if hbm_tail_tokens is None else np.ascontiguousarray(hbm_tail_tokens, dtype=np.int32)
    if tail is not None and tail.shape != cap.shape:
        raise ValueError("hbm_tail_tokens must have one entry per sequence")
    h = ctypes.c_void_p()
    _check(lib().kv_layout_create(ctypes.byref(shape), len(cap), _np_ptr(cap),
                                  None if tail is None else _np_ptr(tail),
                                  host_pool.handle if host_pool else None,
                                  hbm_pool.handle if hbm_pool else None, ctypes.byref(h)))
    return Layout(h.value, shape, len(cap), cap)


def kv_layout_create_windowed(shape: Shape, capacity_tokens, window_tokens, ctx_lens,
                              host_pool: Pool, hbm_pool: Pool) -> Layout:
    """Layout whose HBM part is a window of the most recent pages, slid by kv_advance."""
    cap = np.ascontiguousarray(capacity_tokens, dtype=np.int32)
    win = np.ascontiguousarray(np.broadcast_to(np.asarray(window_tokens, dtype=np.int32), cap.shape))
    ctx = np.ascontiguousarray(ctx_lens, dtype=np.int32)
    if ctx.shape != cap.shape:
        raise ValueError("ctx_lens must have one entry per sequence")
    h = ctypes.c_void_p()
    _check(lib().kv_layout_create_windowed(ctypes.byref(shape), len(cap), _np_ptr(cap), _np_ptr(win),
                                           _np_ptr(ctx), host_pool.handle, hbm_pool.handle,
                                           ctypes.byref(h)))
    return Layout(h.value, shape, len(cap), cap)


def kv_advance(layout: Layout, ctx_lens, stream=None) -> None:
    """ctx_lens[b] += 1 on the device (int32 device tensor, in place), sliding a
    windowed layout's HBM window; enqueued on `stream` (default: current)."""
    import torch
    if ctx_lens.dtype != torch.int32 or tuple(ctx_lens.shape) != (layout.batch,):
        raise ValueError("ctx_lens must be an int32 [batch] device tensor")
    _check(lib().kv_advance(layout.handle, _dev_ptr(ctx_lens, "ctx_lens"), _stream_ptr(stream)))


def kv_append(layout: Layout, layer: int, seq: int, start_token: int, k, v, stream=0) -> None:
    """k, v: [n][Hkv][d] bf16 in logical order -- host uint16 numpy arrays (bf16
    bits), or contiguous bf16/int16 device tensors (scattered into the pages by
    a kernel on `stream`, default: the null stream)."""
    s = layout.shape
    if hasattr(k, "is_cuda") or hasattr(v, "is_cuda"):
        import torch
        for t, name in ((k, "k"), (v, "v")):
            if not (hasattr(t, "is_cuda") and t.is_cuda) or t.dtype not in (torch.bfloat16, torch.int16):
                raise ValueError("%s must be a bf16 (or int16) device tensor like the other" % name)
        n = k.shape[0]
        if tuple(k.shape) != (n, s.n_kv_heads, s.head_dim) or tuple(v.shape) != tuple(k.shape):
            raise ValueError("k and v must be [n][n_kv_heads][head_dim]")
        _check(lib().kv_append(layout.handle, layer, seq, start_token, n, _dev_ptr(k, "k"), _dev_ptr(v, "v"),
                               _stream_ptr(stream) if stream else None))
        return
    k = np.ascontiguousarray(k, dtype=np.uint16)
    v = np.ascontiguousarray(v, dtype=np.uint16)
    n = k.shape[0] if k.ndim > 0 else 0
    if k.shape != (n, s.n_kv_heads, s.head_dim) or v.shape != k.shape:
        raise ValueError("k and v must be [n][n_kv_heads][head_dim]")
    _check(lib().kv_append(layout.handle, layer, seq, start_token, n, _np_ptr(k), _np_ptr(v),
                           _stream_ptr(stream) if stream else None))


def kv_read(layout: Layout, layer: int, seq: int, start_token: int, n_tokens: int):
    s = layout.shape
    k = np.empty((n_tokens, s.n_kv_heads, s.head_dim), dtype=np.uint16)
    v = np.empty_like(k)
    _check(lib().kv_read(layout.handle, layer, seq, start_token, n_tokens, _np_ptr(k), _np_ptr(v)))
    return k, v


# ----------------------------------------------------------------------------- decode step
def _dev_ptr(t, name: str) -> int:
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t.data_ptr()


def _step(fn, layout, layer, q_in, W_qkv, ctx_lens, attn_out, stream):
    import torch
    for t, name, dt in ((q_in, "q_in", torch.bfloat16), (W_qkv, "W_qkv", torch.bfloat16),
                        (ctx_lens, "ctx_lens", torch.int32)):
        if t.dtype != dt:
            raise ValueError("%s must be %s" % (name, dt))
    s = layout.shape
    n_qkv = (s.n_q_heads + 2 * s.n_kv_heads) * s.head_dim
    if tuple(q_in.shape) != (layout.batch, s.hidden):
        raise ValueError("q_in must be [batch][hidden]")
    if tuple(W_qkv.shape) != (n_qkv, s.hidden):
        raise ValueError("W_qkv must be [(Hq + 2 Hkv) d][hidden]")
    if tuple(ctx_lens.shape) != (layout.batch,):
        raise ValueError("ctx_lens must be [batch]")
    if tuple(attn_out.shape) != (layout.batch, s.n_q_heads * s.head_dim):
        raise ValueError("attn_out must be [batch][Hq d]")
    _check(fn(layout.handle, layer, _dev_ptr(q_in, "q_in"), _dev_ptr(W_qkv, "W_qkv"),
              _dev_ptr(ctx_lens, "ctx_lens"), _dev_ptr(attn_out, "attn_out"), _stream_ptr(stream)))
    return attn_out


def decode_step(layout: Layout, layer: int, q_in, W_qkv, ctx_lens, attn_out=None, stream=None):
    """One decode step of `layer`; returns attn_out [batch][Hq*d] bf16 (device)."""
    import torch
    if attn_out is None:
        s = layout.shape
        attn_out = torch.empty((layout.batch, s.n_q_heads * s.head_dim), dtype=torch.bfloat16,
                               device=q_in.device)
    if attn_out.dtype != torch.bfloat16:
        raise ValueError("attn_out must be bfloat16")
    return _step(lib().decode_step, layout, layer, q_in, W_qkv, ctx_lens, attn_out, stream)


def decode_step_f32(layout: Layout, layer: int, q_in, W_qkv, ctx_lens, attn_out=None,
                    stream=None):
    """decode_step with an fp32 attn_out (no output rounding)."""
    import torch
    if attn_out is None:
        s = layout.shape
        attn_out = torch.empty((layout.batch, s.n_q_heads * s.head_dim), dtype=torch.float32,
                               device=q_in.device)
    if attn_out.dtype != torch.float32:
        raise ValueError("attn_out must be float32")
    return _step(lib().decode_step_f32, layout, layer, q_in, W_qkv, ctx_lens, attn_out, stream)


def decode_step_noalloc(layout: Layout, layer: int, q_in, W_qkv, ctx_lens, attn_out, stream=None):
    """decode_step on the library's static device scratch (no allocation in the
    call); attn_out [batch][Hq*d] bf16 must be given."""
    import torch
    if attn_out is None or attn_out.dtype != torch.bfloat16:
        raise ValueError("attn_out must be a bfloat16 device tensor")
    return _step(lib().decode_step_noalloc, layout, layer, q_in, W_qkv, ctx_lens, attn_out, stream)


def decode_step_noalloc_scratch_bytes() -> int:
    return int(lib().decode_step_noalloc_scratch_bytes())


def probe_stream_read(device_ptr: int, nbytes: int, grid: int = 256, unroll: int = 2,
                      reps: int = 3) -> float:
    """Median milliseconds of a kernel streaming-read of nbytes at device_ptr."""
    ms = ctypes.c_float()
    _check(lib().dkv_probe_stream_read(device_ptr, nbytes, grid, unroll, reps, ctypes.byref(ms)))
    return ms.value


def probe_stream_read_cycled(device_ptr: int, nbytes: int, n_regions: int, grid: int = 256,
                             unroll: int = 2, reps: int = 3) -> float:
    """Median milliseconds of a cold streaming-read of nbytes: timed run r
    reads the r mod n_regions-th of n_regions consecutive regions."""
    ms = ctypes.c_float()
    _check(lib().dkv_probe_stream_read_cycled(device_ptr, nbytes, n_regions, grid, unroll, reps,
                                              ctypes.byref(ms)))
    return ms.value


def probe_page_read(device_ptr: int, nbytes: int, page_bytes: int, runs: int, waves: int,
                    skew: bool = False, reps: int = 3) -> float:
    """Median milliseconds of a read of nbytes in the split kernel's access
    pattern (waves wavefronts, each streaming one run of every page of its
    item), with no arithmetic."""
    ms = ctypes.c_float()
    _check(lib().dkv_probe_page_read(device_ptr, nbytes, page_bytes, runs, waves, int(skew), reps,
                                     ctypes.byref(ms)))
    return ms.value


# ----------------------------------------------------------------------------- host-operand GEMM
class HostBuffer:
    """Pinned, mapped host memory: `array` is a numpy view of it, `device_ptr`
    the address kernels use."""

    def __init__(self, nbytes: int, flags: int = HOST_COHERENT):
        h, d = ctypes.c_void_p(), ctypes.c_void_p()
        _check(lib().dkv_host_buffer_alloc(nbytes, flags, ctypes.byref(h), ctypes.byref(d)))
        self.host_ptr, self.device_ptr, self.nbytes = h.value, d.value, nbytes
        self.array = np.ctypeslib.as_array((ctypes.c_uint8 * nbytes).from_address(self.host_ptr))

    def view(self, dtype, shape) -> np.ndarray:
        return self.array.view(dtype)[:int(np.prod(shape))].reshape(shape)

    def free(self) -> None:
        if self.host_ptr:
            self.array = None
            _check(lib().dkv_host_buffer_free(self.host_ptr))
            self.host_ptr = None


def copy(dst_ptr: int, src_ptr: int, nbytes: int, stream=None) -> None:
    """Copy-engine copy between device-known addresses (the swap-in of staging)."""
    _check(lib().dkv_copy(dst_ptr, src_ptr, nbytes, _stream_ptr(stream)))


def gemm_bstationary_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(lib().dkv_gemm_bstationary_workspace_bytes(M, N, K))


def gemm_bf16_nt_bstationary(A, B_ptr: int, C, M: int, N: int, K: int, workspace, stream=None):
    """C [M][N] fp32 = A [M][K] bf16 x B^T (B [N][K] bf16 at B_ptr, HBM or host),
    B-stationary: each B tile fetched once; `workspace` a device tensor of at
    least gemm_bstationary_workspace_bytes(M, N, K) bytes."""
    import torch
    if A.dtype != torch.bfloat16 or tuple(A.shape) != (M, K):
        raise ValueError("A must be a bf16 [M][K] device tensor")
    if C.dtype != torch.float32 or tuple(C.shape) != (M, N):
        raise ValueError("C must be an fp32 [M][N] device tensor")
    nbytes = workspace.numel() * workspace.element_size()
    _check(lib().dkv_gemm_bf16_nt_bstationary(_dev_ptr(A, "A"), B_ptr, _dev_ptr(C, "C"), M, N, K,
                                              _dev_ptr(workspace, "workspace"), nbytes, _stream_ptr(stream)))
    return C


def gemm_bf16_nt(A, B_ptr: int, C, M: int, N: int, K: int, cpu_aware: bool, stream=None):
    """C [M][N] fp32 (device tensor) = A [M][K] bf16 (device tensor) x B^T, with B
    [N][K] bf16 at device address B_ptr (HBM or a mapped host buffer)."""
    import torch
    if A.dtype != torch.bfloat16 or tuple(A.shape) != (M, K):
        raise ValueError("A must be a bf16 [M][K] device tensor")
    if C.dtype != torch.float32 or tuple(C.shape) != (M, N):
        raise ValueError("C must be an fp32 [M][N] device tensor")
    _check(lib().dkv_gemm_bf16_nt(_dev_ptr(A, "A"), B_ptr, _dev_ptr(C, "C"), M, N, K,
                                  1 if cpu_aware else 0, _stream_ptr(stream)))
    return C



# ----------------------------------------------------------------------------- attention on the host CPU
def cpu_attention(layout: "Layout", layer: int, q: np.ndarray, k_new: np.ndarray, v_new: np.ndarray,
                  ctx_lens: np.ndarray, n_threads: int) -> tuple[np.ndarray, int]:
    """Comparator: one step's attention computed by n_threads host threads over
    the layout's host pages (q [B][Hq][d] fp32, k_new/v_new [B][Hkv][d] bf16
    bits, ctx_lens [B] int32, all numpy). Returns (out [B][Hq][d] fp32, threads used)."""
    s = layout.shape
    B = layout.batch
    q = np.ascontiguousarray(q, np.float32)
    k_new = np.ascontiguousarray(k_new, np.uint16)
    v_new = np.ascontiguousarray(v_new, np.uint16)
    ctx = np.ascontiguousarray(ctx_lens, np.int32)
    if q.shape != (B, s.n_q_heads, s.head_dim) or k_new.shape != (B, s.n_kv_heads, s.head_dim) \
            or v_new.shape != k_new.shape or ctx.shape != (B,):
        raise ValueError("cpu_attention: shapes must be q [B][Hq][d], k_new/v_new [B][Hkv][d], ctx_lens [B]")
    out = np.empty_like(q)
    used = ctypes.c_int32()
    _check(lib().dkv_cpu_attention(layout.handle, layer, _np_ptr(q), _np_ptr(k_new), _np_ptr(v_new),
                                   _np_ptr(ctx), _np_ptr(out), n_threads, ctypes.byref(used)))
    return out, used.value


def cpu_attention_pages(shape: Shape, pages: list, q: np.ndarray, k_new: np.ndarray, v_new: np.ndarray,
                        ctx_lens: np.ndarray, n_threads: int) -> tuple[np.ndarray, int]:
    """The host-CPU attention on plain host pages, no GPU: pages[b] is a list
    of C-contiguous uint16 numpy arrays of kv_page_bytes(shape) bytes each
    (sequence b's pages in order). Returns (out [B][Hq][d] fp32, threads used)."""
    B = len(pages)
    max_pages = max(1, max(len(p) for p in pages))
    table = (ctypes.c_void_p * (B * max_pages))()
    for b, row in enumerate(pages):
        for i, page in enumerate(row):
            if page.nbytes != kv_page_bytes(shape):
                raise ValueError("page of the wrong size")
            table[b * max_pages + i] = _np_ptr(page)
    q = np.ascontiguousarray(q, np.float32)
    k_new = np.ascontiguousarray(k_new, np.uint16)
    v_new = np.ascontiguousarray(v_new, np.uint16)
    ctx = np.ascontiguousarray(ctx_lens, np.int32)
    if q.shape != (B, shape.n_q_heads, shape.head_dim) or k_new.shape != (B, shape.n_kv_heads, shape.head_dim) \
            or v_new.shape != k_new.shape or ctx.shape != (B,):
        raise ValueError("cpu_attention_pages: shapes must be q [B][Hq][d], k_new/v_new [B][Hkv][d], ctx_lens [B]")
    out = np.empty_like(q)
    used = ctypes.c_int32()
    _check(lib().dkv_cpu_attention_pages(table, max_pages, ctypes.byref(shape), B, _np_ptr(q), _np_ptr(k_new),
                                         _np_ptr(v_new), _np_ptr(ctx), _np_ptr(out), n_threads,
                                         ctypes.byref(used)))
    return out, used.value


def cpu_stream_read(host_ptr: int, nbytes: int, n_threads: int) -> int:
    """Reads nbytes of host memory on n_threads threads; returns the 64-bit word sum."""
    total = ctypes.c_uint64()
    _check(lib().dkv_cpu_stream_read(host_ptr, nbytes, n_threads, ctypes.byref(total)))
    return total.value
