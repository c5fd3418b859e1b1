"""Host-operand GEMM (C = A x B^T, bf16 in, fp32 out) through the C ABI,
against the fp64 oracle.

Tolerance: every entry is one fp32 sum of K exact bf16 products, in some
order, so |C - C_exact| <= gamma_K * sum_k |a_k b_k| with gamma_K =
K u / (1 - K u), u = 2^-24 (the standard forward bound for floating-point
summation, any order). Small-integer operands make every product and partial
sum exact, so there the comparison is bit for bit. All variants (B in HBM or
in pinned host memory, row-major or CPU-aware tile order) must give
identical bits."""
import numpy as np
import pytest

import synth
from tests import harness as H
from tests.conftest import gpu_available

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X")]

U = 2.0 ** -24


def bound(A, B, K):
    a = np.abs(H.bf16_to_f64(A))
    b = np.abs(H.bf16_to_f64(B))
    g = K * U / (1 - K * U)
    return g * (a @ b.T)


def run_variants(dkv, A, B, M, N, K):
    """C for every (placement of B, tile order); host buffer freed on return."""
    import torch
    Ad = torch.from_numpy(A.view(np.int16)).cuda().view(torch.bfloat16)
    Bd = torch.from_numpy(B.view(np.int16)).cuda().view(torch.bfloat16)
    hb = dkv.HostBuffer(B.nbytes)
    try:
        hb.view(np.uint16, B.shape)[...] = B
        outs = {}
        for where, ptr in (("hbm", Bd.data_ptr()), ("host", hb.device_ptr)):
            for order in ((False, True) if (N // 128) % 8 == 0 else (False,)):
                C = torch.empty((M, N), dtype=torch.float32, device="cuda")
                dkv.gemm_bf16_nt(Ad, ptr, C, M, N, K, order)
                torch.cuda.synchronize()
                outs[(where, order)] = C.cpu().numpy()
        return outs
    finally:
        torch.cuda.synchronize()
        hb.free()


@pytest.mark.parametrize("M,N,K", [(128, 128, 64), (256, 1024, 192), (384, 2048, 1024)])
def test_gemm_against_oracle_and_variants_identical(oracle, M, N, K):
    import decode_attention_zero_amd as dkv
    A = synth.normal_bf16(11, 50, M, M * K, 1.0).reshape(M, K)
    B = synth.normal_bf16(11, 51, N, N * K, 1.0).reshape(N, K)
    outs = run_variants(dkv, A, B, M, N, K)
    first = next(iter(outs.values()))
    for key, C in outs.items():
        assert np.array_equal(C.view(np.uint32), first.view(np.uint32)), key
    ref = oracle.gemm_nt(A, B)
    err = np.abs(first.astype(np.float64) - ref)
    bnd = bound(A, B, K)
    H.log("gemm %dx%dx%d: max err %.3e, max err / bound %.3f" % (M, N, K, err.max(), (err / bnd).max()))
    assert np.all(err <= bnd)


def test_gemm_integer_exact(oracle):
    import decode_attention_zero_amd as dkv
    M, N, K = 256, 1024, 320
    A = synth.int_bf16(12, 52, 0, M * K, -6, 6).reshape(M, K)
    B = synth.int_bf16(12, 53, 0, N * K, -6, 6).reshape(N, K)
    outs = run_variants(dkv, A, B, M, N, K)
    ref = oracle.gemm_nt(A, B)
    for key, C in outs.items():
        assert np.array_equal(C.astype(np.float64), ref), key


def test_gemm_rejects_bad_shapes():
    import torch
    import decode_attention_zero_amd as dkv
    A = torch.zeros((128, 64), dtype=torch.bfloat16, device="cuda")
    C = torch.zeros((128, 256), dtype=torch.float32, device="cuda")
    B = torch.zeros((256, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(dkv.DkvError):      # N / 128 = 2: no CPU-aware order
        dkv.gemm_bf16_nt(A, B.data_ptr(), C, 128, 256, 64, True)
    with pytest.raises(dkv.DkvError):      # K not a multiple of 64
        dkv.gemm_bf16_nt(A[:, :32].contiguous(), B.data_ptr(), C, 128, 256, 32, False)


def run_bstationary(dkv, A, B, M, N, K):
    """C of the B-stationary form with B in HBM and in pinned host memory."""
    import torch
    Ad = torch.from_numpy(A.view(np.int16)).cuda().view(torch.bfloat16)
    Bd = torch.from_numpy(B.view(np.int16)).cuda().view(torch.bfloat16)
    ws = torch.empty(dkv.gemm_bstationary_workspace_bytes(M, N, K) // 4, dtype=torch.float32, device="cuda")
    hb = dkv.HostBuffer(B.nbytes)
    try:
        hb.view(np.uint16, B.shape)[...] = B
        outs = {}
        for where, ptr in (("hbm", Bd.data_ptr()), ("host", hb.device_ptr)):
            C = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
            dkv.gemm_bf16_nt_bstationary(Ad, ptr, C, M, N, K, ws)
            torch.cuda.synchronize()
            outs[where] = C.cpu().numpy()
        return outs
    finally:
        torch.cuda.synchronize()
        hb.free()


@pytest.mark.parametrize("M,N,K", [(64, 128, 512), (256, 384, 1536), (320, 1024, 2048)])
def test_gemm_bstationary_against_oracle(oracle, M, N, K):
    """The B-stationary form (each 128 x 512 tile of B fetched once, partial
    sums per k tile added in k order): one fp32 sum per k tile plus the
    adds of the tiles, so within the same gamma_K bound of the fp64 oracle
    (its partial sums are themselves sums of |a b| terms); B in HBM and on
    the host give identical bits."""
    import decode_attention_zero_amd as dkv
    A = synth.normal_bf16(13, 54, M, M * K, 1.0).reshape(M, K)
    B = synth.normal_bf16(13, 55, N, N * K, 1.0).reshape(N, K)
    outs = run_bstationary(dkv, A, B, M, N, K)
    assert np.array_equal(outs["hbm"].view(np.uint32), outs["host"].view(np.uint32))
    ref = oracle.gemm_nt(A, B)
    err = np.abs(outs["host"].astype(np.float64) - ref)
    bnd = bound(A, B, K)
    H.log("gemm b-stationary %dx%dx%d: max err %.3e, max err / bound %.3f" % (M, N, K, err.max(), (err / bnd).max()))
    assert np.all(np.isfinite(outs["host"])) and np.all(err <= bnd)


def test_gemm_bstationary_integer_exact(oracle):
    """Small-integer operands: every partial and every add is exact, so the
    B-stationary form gives the oracle's values bit for bit."""
    import decode_attention_zero_amd as dkv
    M, N, K = 192, 256, 1024
    A = synth.int_bf16(14, 56, 0, M * K, -6, 6).reshape(M, K)
    B = synth.int_bf16(14, 57, 0, N * K, -6, 6).reshape(N, K)
    outs = run_bstationary(dkv, A, B, M, N, K)
    ref = oracle.gemm_nt(A, B)
    for key, C in outs.items():
        assert np.array_equal(C.astype(np.float64), ref), key


def test_gemm_bstationary_rejects_bad_arguments():
    import torch
    import decode_attention_zero_amd as dkv
    A = torch.zeros((64, 512), dtype=torch.bfloat16, device="cuda")
    B = torch.zeros((128, 512), dtype=torch.bfloat16, device="cuda")
    C = torch.full((64, 128), 7.0, dtype=torch.float32, device="cuda")
    need = dkv.gemm_bstationary_workspace_bytes(64, 128, 512)
    assert need == 64 * 128 * 4
    small = torch.zeros(need // 4 - 1, dtype=torch.float32, device="cuda")
    with pytest.raises(dkv.DkvError) as e:
        dkv.gemm_bf16_nt_bstationary(A, B.data_ptr(), C, 64, 128, 512, small)
    assert e.value.status == -3
    ws = torch.zeros(need // 4, dtype=torch.float32, device="cuda")
    with pytest.raises(dkv.DkvError):      # K not a multiple of 512
        dkv.gemm_bf16_nt_bstationary(A[:, :256].contiguous(), B.data_ptr(), C, 64, 128, 256, ws)
    torch.cuda.synchronize()
    assert bool((C == 7.0).all())          # nothing was enqueued
