"""The C-ABI library on the CPU: it loads, exports every function its headers
declare, and its pure host functions (page layout, placement policy) behave
as documented. No GPU calls."""
import glob
import os
import re
import subprocess

import numpy as np
import pytest

import decode_attention_zero_amd as dkv
from tests.conftest import ROOT

DECL = re.compile(r"^(?:const\s+)?[A-Za-z_]\w*\s*\*?\s*([A-Za-z_]\w*)\s*\(", re.M)


def declared_functions():
    names = []
    for h in sorted(glob.glob(os.path.join(ROOT, "include", "*.h"))):
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        for m in DECL.finditer(text):
            line = text[m.start():text.find("\n", m.start())]
            if line.startswith(("typedef", "#", "extern")):
                continue
            names.append(m.group(1))
    return names


def test_headers_declare_the_boundary():
    names = declared_functions()
    for must in ("kv_alloc_host", "kv_alloc_hbm", "kv_append", "decode_step", "kv_layout_create",
                 "kv_read", "dkv_last_error", "kv_placement", "kv_page_offset"):
        assert must in names
    assert sorted(names) == sorted(set(names))


def test_library_exports_every_declared_symbol():
    lib = dkv.lib()
    out = subprocess.run(["nm", "-D", "--defined-only", dkv.LIBRARY], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)
    assert sorted(dkv.EXPORTED) == sorted(declared_functions())


def test_page_layout_is_head_major_and_aligned():
    s = dkv.Shape.of(4096, 32, 8, 128)
    assert dkv.kv_page_bytes(s) == 8 * 2 * 16 * 128 * 2 == 65536
    # run of (page, head g): K rows then V rows, 8 KiB contiguous, 128-B aligned
    for g in range(8):
        base = dkv.kv_page_offset(s, 0, g, 0, 0)
        assert base == g * 8192 and base % 128 == 0
        assert dkv.kv_page_offset(s, 15, g, 0, 127) == base + 4096 - 2
        assert dkv.kv_page_offset(s, 0, g, 1, 0) == base + 4096
        assert dkv.kv_page_offset(s, 15, g, 1, 127) == base + 8192 - 2
    offs = {dkv.kv_page_offset(s, t, g, c, i) for t in range(16) for g in range(8)
            for c in range(2) for i in range(0, 128, 8)}
    assert len(offs) == 16 * 8 * 2 * 16
    assert dkv.kv_page_offset(s, 16, 0, 0, 0) == -1
    assert dkv.kv_page_offset(s, 0, 8, 0, 0) == -1
    assert dkv.kv_page_offset(s, 0, 0, 2, 0) == -1
    assert dkv.kv_page_offset(s, 0, 0, 0, 128) == -1
    t = dkv.Shape.of(512, 8, 8, 64)
    assert dkv.kv_page_bytes(t) == 32768
    assert dkv.kv_page_offset(t, 3, 2, 1, 5) == ((2 * 2 + 1) * 16 + 3) * 128 + 10


def contiguous_runs(offsets, elem=2):
    """Number of maximal runs of consecutive elements among byte offsets."""
    offs = sorted(offsets)
    return 1 + sum(1 for a, b in zip(offs, offs[1:]) if b != a + elem)


def test_fragments_per_head_against_token_major(golden):
    """Beluga's count on the KV Offload wiki: a 16-token GQA block with 8 KV
    heads is 128 separate fragments when stored token-major. Gathering each
    head's K rows of one block from a token-major array [t][g][d] yields that
    count; the library's head-major page yields one contiguous run per
    (page, head)."""
    fact = golden["fragments_16_token_gqa_block"]
    T, Hkv, d = fact["tokens"], fact["kv_heads"], 128
    token_major = sum(contiguous_runs([((t * Hkv + g) * d + i) * 2 for t in range(T) for i in range(d)])
                      for g in range(Hkv))
    assert token_major == fact["fragments"]
    s = dkv.Shape.of(5120, 40, Hkv, d)
    head_major = sum(contiguous_runs([dkv.kv_page_offset(s, t, g, 0, i) for t in range(T) for i in range(d)])
                     for g in range(Hkv))
    assert head_major == Hkv
    # K then V of one head: still one run (8 KiB at d = 128)
    both = [dkv.kv_page_offset(s, t, 3, c, i) for c in range(2) for t in range(T) for i in range(d)]
    assert contiguous_runs(both) == 1 and max(both) - min(both) == 2 * T * d * 2 - 2


def test_placement_policy():
    assert dkv.kv_placement(16385, 0) == (1025, 1025)
    assert dkv.kv_placement(16385, 8193) == (1025, 512)        # 50 %: first 8192 tokens host
    assert dkv.kv_placement(100001, 4096) == (6251, 6251 - 256)
    assert dkv.kv_placement(1, 0) == (1, 1)
    assert dkv.kv_placement(1, 5) == (1, 0)
    assert dkv.kv_placement(33, 10 ** 6) == (3, 0)
    assert dkv.kv_placement(32, 16) == (2, 1)
    assert dkv.kv_placement(32, 17) == (2, 0)
    with pytest.raises(dkv.DkvError) as e:
        dkv.kv_placement(0, 0)
    assert e.value.status == -1
    with pytest.raises(dkv.DkvError):
        dkv.kv_placement(10, -1)


def test_invalid_shapes_are_rejected_without_a_gpu():
    bad = dkv.Shape(4096, 30, 8, 128, 1, 16)          # 30 % 8 != 0
    assert dkv.kv_page_bytes(bad) == 0
    with pytest.raises(dkv.DkvError) as e:
        dkv.kv_alloc_host(bad, 4)
    assert e.value.status == -1
    with pytest.raises(dkv.DkvError):
        dkv.kv_alloc_hbm(dkv.Shape(4096, 32, 8, 128, 1, 32), 4)   # page_tokens must be 16


def test_swap_buffer_fact_is_two_byte_elements(golden):
    """Fig. 2(a)'s 200 MB buffer for a 10240 x 10240 operand means 2-byte
    elements (bf16/fp16), the element size of this library's KV pages."""
    f = golden["swap_buffer_bytes"]
    assert f["matrix_dim"] ** 2 * f["bytes_per_element"] == 200 * 2 ** 20


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """Without the built HIP library every entry point raises; nothing falls
    back to another implementation."""
    import torch
    monkeypatch.setattr(dkv, "LIBRARY", str(tmp_path / "libdkv.so"))
    monkeypatch.setattr(dkv, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        dkv.lib()
    with pytest.raises(RuntimeError, match="not built"):
        dkv.kv_page_bytes(dkv.Shape.of(4096, 32, 8, 128, 1))
    x = torch.zeros((1, 512), dtype=torch.bfloat16)
    with pytest.raises(RuntimeError, match="not built"):
        dkv.decode_step(dkv.Layout(1, dkv.Shape.of(512, 8, 8, 64, 1), 1, np.array([2], np.int32)), 0, x,
                        torch.zeros((1536, 512), dtype=torch.bfloat16), torch.zeros(1, dtype=torch.int32),
                        torch.zeros((1, 512), dtype=torch.bfloat16))
