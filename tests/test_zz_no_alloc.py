"""decode_step_noalloc -- the decode step on the library's static device
scratch, for callers that cannot allocate device memory -- against
decode_step on the same layouts, through the C ABI.

Two calls in a row on the static scratch (the second on a smaller layout,
so it runs over what the first left there) must give the same bits as
decode_step, and so meet every gate decode_step's own tests hold it to; a
layout whose step needs more scratch than the static array is refused
before anything is enqueued."""
import numpy as np
import pytest

from synth import configs
from tests import harness as H
from tests.conftest import gpu_available

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X")]


def _bits(t):
    import torch
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def test_noalloc_matches_decode_step_on_two_calls_in_a_row(oracle):
    import torch
    rng = np.random.default_rng(7)
    # Batch 64 (split-k projection, 8 ranges of the hidden dimension), ragged
    # contexts, half of each sequence in HBM; then batch 3 (GEMV projection),
    # all host pages, a much smaller scratch.
    big = H.Setup(configs.LLAMA8B_DENSE, ctx_lens=rng.integers(0, 3000, 64).astype(np.int32))
    small = H.Setup(configs.LLAMA8B_HOST.replace(batch=3), ctx_lens=[0, 17, 1500], hbm_tail=0)
    try:
        limit = H.dkv.decode_step_noalloc_scratch_bytes()
        H.log("static scratch %d bytes" % limit)
        refs = [s.run() for s in (big, small)]
        torch.cuda.synchronize()
        outs = [torch.full_like(r, float("nan")) for r in refs]
        for s, out in zip((big, small), outs):
            H.dkv.decode_step_noalloc(s.layout, 0, s.x[0], s.W[0], s.ctx_dev, out)
        torch.cuda.synchronize()
        for s, ref, out, name in zip((big, small), refs, outs, ("batch 64", "batch 3")):
            s.layout.check_status()
            assert np.array_equal(_bits(out), _bits(ref)), name
            H.log("%s: decode_step_noalloc bit-identical to decode_step" % name)
        # And the small layout's step once more from a fresh state against the
        # oracle, so the shared comparison is anchored to the definition.
        got = H.bf16_to_f64(_bits(outs[1]))
        ref = H.oracle_full(oracle, small.wl, 0, small.ctx)["attn_out"]
        assert np.abs(got - ref).max() <= 2e-2 and H.rel_l2(got, ref) <= 5e-3
    finally:
        big.free()
        small.free()


def test_noalloc_refuses_a_layout_beyond_the_static_scratch():
    import torch
    wl = configs.LLAMA8B_HOST.replace(batch=256)
    # 256 sequences at hidden 4096: 8 projection slabs of 256 x 6144 fp32
    # alone take 50 MB, more than the 32 MiB array.
    s = H.Setup(wl, ctx_lens=np.full(256, 16, np.int32), hbm_tail=0)
    try:
        out = torch.full((256, wl.n_q_heads * wl.head_dim), float("nan"), dtype=torch.bfloat16, device="cuda")
        with pytest.raises(H.dkv.DkvError) as err:
            H.dkv.decode_step_noalloc(s.layout, 0, s.x[0], s.W[0], s.ctx_dev, out)
        assert err.value.status == -3 and "scratch" in str(err.value)
        torch.cuda.synchronize()
        assert torch.isnan(out.float()).all()           # nothing was enqueued
    finally:
        s.free()
