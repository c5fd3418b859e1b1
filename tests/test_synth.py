"""The seeded input generator: Philox4x32-10 known answers, determinism,
slicing consistency and distribution sanity of the workload recipes."""
import numpy as np
import pytest

import synth
from synth import configs


# Known-answer vectors of Philox4x32-10 from the Random123 distribution
# (Salmon et al., SC'11): (counter, key) -> output.
PHILOX_KAT = [
    ((0, 0, 0, 0), (0, 0), (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
    ((0xFFFFFFFF,) * 4, (0xFFFFFFFF, 0xFFFFFFFF), (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)),
    ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0),
     (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1)),
]


@pytest.mark.parametrize("ctr,key,expect", PHILOX_KAT)
def test_philox_known_answers(ctr, key, expect):
    assert tuple(int(v) for v in synth.philox4x32_10(ctr, key)) == expect


def test_normal_is_deterministic_and_offset_consistent():
    a = synth.normal_bf16(7, synth.TENSOR_K, 3, 1000, 1.0)
    b = synth.normal_bf16(7, synth.TENSOR_K, 3, 1000, 1.0, threads=1)
    assert np.array_equal(a, b)
    c = synth.normal_bf16(7, synth.TENSOR_K, 3, 600, 1.0, offset=400)
    assert np.array_equal(a[400:], c)
    d = synth.normal_bf16(7, synth.TENSOR_V, 3, 1000, 1.0)
    assert not np.array_equal(a, d)


def test_normal_distribution_sanity():
    z = synth.normal_f64(11, 1, 0, 400000)
    assert abs(z.mean()) < 0.01
    assert abs(z.std() - 1.0) < 0.01
    assert abs(np.mean(z ** 3)) < 0.02
    assert abs(np.mean(z ** 4) - 3.0) < 0.05
    bits = synth.normal_bf16(11, 1, 0, 1000, 0.02)
    vals = synth.bf16_bits_to_f32(bits)
    assert 0.015 < vals.std() < 0.025


def test_uniform_ints_cover_range():
    v = synth.uniform_i32(5, synth.TENSOR_CTX, 0, 20000, 8192, 131072)
    assert v.min() >= 8192 and v.max() <= 131072
    assert v.min() < 8192 + 200 and v.max() > 131072 - 200
    ib = synth.int_bf16(5, 9, 0, 5000, -16, 16)
    vals = synth.bf16_bits_to_f32(ib)
    assert np.array_equal(vals, np.round(vals)) and vals.min() == -16 and vals.max() == 16


def test_kv_head_slice_matches_full_rows():
    w = configs.LLAMA8B_HOST.replace(ctx=64)
    full = w.kv("k", 0, 3, 10, 40)
    for g in (0, 5, 7):
        sl = w.kv_head("k", 0, 3, g, 10, 40)
        assert np.array_equal(full[:, g, :], sl)
    v = w.kv("v", 0, 3, 10, 40)
    assert not np.array_equal(full, v)


def test_workload_shapes():
    w = configs.LLAMA8B_HOST
    assert (w.group, w.n_qkv, w.kv_bytes_per_token) == (4, 6144, 4096)
    assert configs.TINY.n_qkv == 1536 and configs.TINY.kv_bytes_per_token == 2048
    assert configs.LLAMA70B_LONG.n_qkv == 10240
    lens = configs.LLAMA8B_HYBRID.ctx_lens()
    assert lens.shape == (32,) and lens.min() >= 8192 and lens.max() <= 131072
    assert np.array_equal(lens, configs.LLAMA8B_HYBRID.ctx_lens())
    d = configs.LLAMA8B_DENSE
    tail = d.hbm_tail(d.ctx_lens())
    assert np.all(tail == 8193)          # first 8192 tokens host, the rest + new slot HBM


def test_bf16_values_are_rne_of_the_fp64_normals(oracle):
    """The generator's bulk bf16 path equals the oracle's independent fp64 ->
    bf16 round-to-nearest-even of the generator's fp64 normals."""
    for sigma, off in ((1.0, 0), (0.02, 12345), (0.015, 7)):
        z = synth.normal_f64(3, synth.TENSOR_W, 2, 3001, offset=off)
        bits = synth.normal_bf16(3, synth.TENSOR_W, 2, 3001, sigma, offset=off)
        assert np.array_equal(bits, oracle.f64_to_bf16(sigma * z))
    rows = synth.normal_bf16_rows(3, synth.TENSOR_K, 9, 6, 5, 7, 13, 1.0)
    for r in range(5):
        assert np.array_equal(rows[r], synth.normal_bf16(3, synth.TENSOR_K, 9, 7, 1.0,
                                                        offset=6 + 13 * r))
