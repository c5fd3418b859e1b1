"""Error paths of the C ABI that need a device: every one returns a status
and a message before anything is enqueued, and leaves the library usable.

Covered: double free of pools and layouts, calls (the accessors included) on
a freed layout or pool, a pool freed while a layout still holds its pages,
null and misaligned pointers handed to decode_step, an HBM pool larger than
HBM, unsupported shapes and bad capacities at layout creation, more splits
per sequence than a launch grid holds. (A host pool
larger than host memory is not exercised: pinning is not guaranteed to fail
before it has touched memory.)"""
import ctypes

import numpy as np
import pytest

import decode_attention_zero_amd as dkv
from tests.conftest import gpu_available

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X")]

E_INVALID_ARG, E_OUT_OF_MEMORY, E_UNSUPPORTED = -1, -2, -5


def small_layout():
    shape = dkv.Shape.of(512, 8, 4, 64, 1)
    host = dkv.kv_alloc_host(shape, 4)
    layout = dkv.kv_layout_create(shape, np.array([20, 30], np.int32), None, host, None)
    return shape, host, layout


def test_double_free_and_use_after_free_are_refused():
    L = dkv.lib()
    shape, host, layout = small_layout()
    h_layout, h_pool = layout.handle, host.handle
    assert L.kv_pool_free(h_pool) == E_INVALID_ARG          # a layout still holds its pages
    assert "still use" in L.dkv_last_error().decode()
    layout.free()
    assert L.kv_layout_free(h_layout) == E_INVALID_ARG      # freed twice
    assert L.kv_layout_check_status(h_layout) == E_INVALID_ARG
    assert L.kv_layout_split_tokens(h_layout) == 0 and L.kv_layout_split_kernel(h_layout) == -1
    assert L.kv_layout_split_waves(h_layout) == -1 and L.kv_layout_projection_kernel(h_layout) == -1
    assert L.kv_layout_set_split_kernel(h_layout, 0) == E_INVALID_ARG
    tier = ctypes.c_int32(-7)
    assert L.kv_layout_page_tier(h_layout, 0, 0, ctypes.byref(tier)) == E_INVALID_ARG and tier.value == -7
    assert L.kv_layout_timing_enable(h_layout, 1, 4) == E_INVALID_ARG
    assert L.kv_layout_timing_read(h_layout, None, None, None, None, None) == E_INVALID_ARG
    ctx = np.zeros(2, np.int32)
    assert L.kv_advance(h_layout, ctx.ctypes.data, None) == E_INVALID_ARG
    k = np.zeros((1, 4, 64), np.uint16)
    assert L.kv_append(h_layout, 0, 0, 0, 1, k.ctypes.data, k.ctypes.data, None) == E_INVALID_ARG
    host.free()
    assert L.kv_pool_free(h_pool) == E_INVALID_ARG          # freed twice
    n = ctypes.c_int64()
    assert L.kv_pool_free_pages(h_pool, ctypes.byref(n)) == E_INVALID_ARG
    out = ctypes.c_void_p()
    assert L.kv_layout_create(ctypes.byref(shape), 1, np.array([4], np.int32).ctypes.data, None, h_pool, None,
                              ctypes.byref(out)) == E_INVALID_ARG
    assert L.kv_pool_free(None) == 0 and L.kv_layout_free(None) == 0
    # the library still works
    shape, host, layout = small_layout()
    layout.free()
    host.free()


def test_decode_step_rejects_null_and_misaligned_pointers():
    import torch
    L = dkv.lib()
    shape, host, layout = small_layout()
    try:
        dev = torch.device("cuda", 0)
        x = torch.zeros((2, 512 + 8), dtype=torch.bfloat16, device=dev)
        W = torch.zeros((8 * 64 + 2 * 4 * 64, 512), dtype=torch.bfloat16, device=dev)
        ctx = torch.tensor([3, 5], dtype=torch.int32, device=dev)
        raw = torch.zeros(64, dtype=torch.uint8, device=dev)
        out = torch.empty((2, 8 * 64), dtype=torch.bfloat16, device=dev)
        step = L.decode_step
        ok = (layout.handle, 0, x.data_ptr(), W.data_ptr(), ctx.data_ptr(), out.data_ptr(), None)
        for i in (2, 3, 4, 5):
            args = list(ok)
            args[i] = None
            assert step(*args) == E_INVALID_ARG, i
        bad = [list(ok) for _ in range(3)]
        bad[0][2] = x.data_ptr() + 2                       # q_in off 16-byte alignment
        bad[1][4] = raw.data_ptr() + 1                     # ctx_lens off 4-byte alignment
        bad[2][5] = out.data_ptr() + 1                     # attn_out off 2-byte alignment
        for args in bad:
            assert step(*args) == E_INVALID_ARG
            assert "align" in L.dkv_last_error().decode()
        assert step(*ok) == 0                              # the valid call still runs
        torch.cuda.synchronize()
        layout.check_status()
    finally:
        layout.free()
        host.free()


def test_hbm_pool_larger_than_hbm_is_out_of_memory():
    L = dkv.lib()
    shape = dkv.Shape.of(4096, 32, 8, 128, 1)            # 64 KiB pages
    out = ctypes.c_void_p()
    assert L.kv_alloc_hbm(ctypes.byref(shape), 1 << 24, ctypes.byref(out)) == E_OUT_OF_MEMORY   # 1 TiB
    assert out.value is None
    pool = dkv.kv_alloc_hbm(shape, 2)                     # and a normal allocation still works
    pool.free()


def test_layout_creation_errors():
    L = dkv.lib()
    shape = dkv.Shape.of(512, 8, 4, 64, 1)
    host = dkv.kv_alloc_host(shape, 2)
    try:
        out = ctypes.c_void_p()
        cap = np.array([40], np.int32)                    # 3 pages, the pool has 2
        assert L.kv_layout_create(ctypes.byref(shape), 1, cap.ctypes.data, None, host.handle, None,
                                  ctypes.byref(out)) != 0
        assert out.value is None and host.free_pages() == 2
        cap0 = np.array([0], np.int32)
        assert L.kv_layout_create(ctypes.byref(shape), 1, cap0.ctypes.data, None, host.handle, None,
                                  ctypes.byref(out)) == E_INVALID_ARG
        odd = dkv.Shape.of(512, 12, 4, 64, 1)             # group of 3
        assert L.kv_layout_create(ctypes.byref(odd), 1, np.array([4], np.int32).ctypes.data, None, None,
                                  None, ctypes.byref(out)) == E_UNSUPPORTED
    finally:
        host.free()


def test_too_many_splits_per_sequence_is_unsupported(monkeypatch):
    """Splits of a sequence are a launch-grid dimension (at most 65535): a
    layout whose capacity needs more (here 16-token splits of 1,048,592
    tokens, 65,537 splits) is refused at creation, its pages given back; one
    split fewer is accepted."""
    L = dkv.lib()
    monkeypatch.setenv("DKV_SPLIT_TOKENS", "16")
    shape = dkv.Shape.of(512, 8, 8, 64, 1)                # 32 KiB pages
    n_pages = 65537 + 1                                   # cached tokens / 16, plus the fresh slot's page
    pool = dkv.kv_alloc_hbm(shape, n_pages)
    try:
        out = ctypes.c_void_p()
        cap = np.array([65537 * 16 + 1], np.int32)
        assert L.kv_layout_create(ctypes.byref(shape), 1, cap.ctypes.data, cap.ctypes.data, None, pool.handle,
                                  ctypes.byref(out)) == E_UNSUPPORTED
        assert "65535" in L.dkv_last_error().decode()
        assert out.value is None and pool.free_pages() == n_pages
        ok = dkv.kv_layout_create(shape, np.array([65535 * 16 + 1], np.int32), np.array([1 << 30], np.int32),
                                  None, pool)
        assert ok.split_tokens == 16
        ok.free()
    finally:
        pool.free()


def test_plan_log(monkeypatch, capfd):
    """DKV_LOG=1 prints the layout's launch plan on stderr; nothing else changes."""
    monkeypatch.setenv("DKV_LOG", "1")
    shape = dkv.Shape.of(4096, 32, 8, 128, 1)
    host = dkv.kv_alloc_host(shape, 8)
    try:
        layout = dkv.kv_layout_create(shape, np.array([40, 50], np.int32), None, host, None)
        layout.free()
    finally:
        host.free()
    err = capfd.readouterr().err
    assert "[dkv] layout: batch 2" in err and "split kernel mfma" in err, err


def test_timing_modes():
    """kv_layout_timing_enable: mode 1 times every kernel of a step, mode 2
    only the split kernel (the others read 0 ms), any other mode is refused
    and leaves timing off; the step's output is the same in every mode."""
    import torch
    L = dkv.lib()
    shape = dkv.Shape.of(512, 8, 4, 64, 1)
    host = dkv.kv_alloc_host(shape, 8)
    try:
        layout = dkv.kv_layout_create(shape, np.array([60, 30], np.int32), None, host, None)
        k = np.full((40, 4, 64), 0x3F80, np.uint16)
        dkv.kv_append(layout, 0, 0, 0, k, k)
        x = torch.ones((2, 512), dtype=torch.bfloat16, device="cuda")
        W = torch.full(((8 + 8) * 64, 512), 0.01, dtype=torch.bfloat16, device="cuda")
        ctx = torch.tensor([40, 0], dtype=torch.int32, device="cuda")
        ref = dkv.decode_step(layout, 0, x, W, ctx).cpu()
        for split_only in (False, True):
            layout.timing_enable(True, 3, split_only=split_only)
            for _ in range(3):
                assert torch.equal(dkv.decode_step(layout, 0, x, W, ctx).cpu(), ref)
            t = layout.timing_read()
            assert t["steps"] == 3 and t["split"] > 0
            others = [t["projection"], t["fresh"], t["combine"]]
            assert all(v == 0 for v in others) if split_only else all(v > 0 for v in others), t
            layout.timing_enable(False)
        assert L.kv_layout_timing_enable(layout.handle, 3, 4) == E_INVALID_ARG
        assert L.kv_layout_timing_enable(layout.handle, -1, 4) == E_INVALID_ARG
        dkv.decode_step(layout, 0, x, W, ctx)
        assert layout.timing_read()["steps"] == 0
        layout.free()
    finally:
        host.free()
