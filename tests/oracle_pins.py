"""Pins of the fp64 oracle to facts that do not come from the oracle itself.

Each ``pin_*`` takes an :class:`oracle.Oracle` and raises AssertionError when
the oracle disagrees with the fact. ``test_oracle_pins.py`` runs them on the
real oracle (all must pass) and on mutated copies of its source (each mutant
must fail at least one). The facts:

* library routines: numpy's fp64 matmul for the projection, torch's fp64
  ``scaled_dot_product_attention`` (grouped heads, one query) for attention;
* a second implementation: attention in plain Python loops with math.exp
  and math.fsum on tiny shapes;
* closed forms: a one-token context returns its V exactly; equal scores return
  the mean of V; adding a constant to every score changes nothing; the output
  is affine in V; a dominant planted key returns its V; hand-derived softmax
  weights (e^i / sum e^j) for keys with scores 0, 1, 2, 3;
* invariants: merging per-range softmax states over any partition equals the
  unsplit result; permuting cached (K, V) rows jointly changes nothing;
* bf16 round-to-nearest-even facts (ties to even, no double rounding).
"""
from __future__ import annotations

import math

import numpy as np

RNG_SEED = 20261202


def _bf16_bits(x: np.ndarray) -> np.ndarray:
    """bf16 bits of values that are exactly representable (checked)."""
    f = np.asarray(x, dtype=np.float32)
    bits = (f.view(np.uint32) >> 16).astype(np.uint16)
    back = (bits.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(back, f), "value not exactly representable in bf16"
    return bits


def _decode(bits) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _rand_bf16(rng, shape, scale=1.0):
    f = (rng.standard_normal(shape) * scale).astype(np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)   # truncation: any bf16 value will do


def _rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


# --------------------------------------------------------------------------- bf16
def pin_bf16_decode(o):
    cases = {0x3F80: 1.0, 0xC000: -2.0, 0x0001: 2.0 ** -133, 0x0000: 0.0, 0x3E80: 0.25,
             0x4780: 65536.0, 0x3F81: 1.0 + 2.0 ** -7}
    for bits, val in cases.items():
        assert o.bf16_to_f64(np.array([bits]))[0] == val, hex(bits)


def pin_bf16_round_to_nearest_even(o):
    one = 1.0
    cases = [
        (one, 0x3F80),
        (one + 2.0 ** -8, 0x3F80),                 # tie -> even (down)
        (one + 3 * 2.0 ** -8, 0x3F82),             # tie -> even (up)
        (one + 2.0 ** -8 + 2.0 ** -30, 0x3F81),    # just above the tie: up (fp32 would round first)
        (one + 2.0 ** -8 - 2.0 ** -40, 0x3F80),    # just below the tie
        (-one - 2.0 ** -8, 0xBF80),
        (3.0, 0x4040),
        (-0.0, 0x8000),
        (2.0 ** -133, 0x0001),                     # smallest subnormal
        (1.5 * 2.0 ** -133, 0x0002),               # subnormal tie -> even
    ]
    for x, bits in cases:
        got = int(o.f64_to_bf16(np.array([x]))[0])
        assert got == bits, (x, hex(got), hex(bits))
    # agreement with torch's fp32 -> bf16 RNE on fp32-representable values
    import torch
    rng = np.random.default_rng(RNG_SEED)
    f = rng.standard_normal(2000).astype(np.float32) * np.float32(3.0)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = o.f64_to_bf16(f.astype(np.float64))
    assert np.array_equal(got, ref)


# ---------------------------------------------------------------------- projection
def pin_projection_matches_numpy(o):
    rng = np.random.default_rng(RNG_SEED + 1)
    hidden, n_out = 96, 40
    x = _rand_bf16(rng, hidden)
    W = _rand_bf16(rng, (n_out, hidden), 0.05)
    y = o.qkv_projection(x, W)
    ref = _decode(W) @ _decode(x)
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-14)


def pin_projection_integer_exact(o):
    rng = np.random.default_rng(RNG_SEED + 2)
    hidden, n_out = 64, 24
    xi = rng.integers(-16, 17, hidden)
    Wi = rng.integers(-16, 17, (n_out, hidden))
    y = o.qkv_projection(_bf16_bits(xi), _bf16_bits(Wi))
    assert np.array_equal(y, (Wi @ xi).astype(np.float64))


# ----------------------------------------------------------------------- attention
def _sdpa_ref(q, K, V, k_new, v_new, n_q_heads, n_kv_heads):
    """torch fp64 SDPA for one decode query per head. q [Hq][d], K/V [L][Hkv][d] (f64)."""
    import torch
    import torch.nn.functional as F
    d = q.shape[-1]
    Kf = np.concatenate([K, k_new[None]], axis=0)       # [L+1][Hkv][d]
    Vf = np.concatenate([V, v_new[None]], axis=0)
    qt = torch.from_numpy(np.ascontiguousarray(q[None, :, None, :]))
    kt = torch.from_numpy(np.ascontiguousarray(Kf.transpose(1, 0, 2)[None]))
    vt = torch.from_numpy(np.ascontiguousarray(Vf.transpose(1, 0, 2)[None]))
    out = F.scaled_dot_product_attention(qt, kt, vt, enable_gqa=(n_q_heads != n_kv_heads))
    return out[0, :, 0, :].numpy()                       # [Hq][d]


def pin_attention_matches_torch_sdpa(o):
    rng = np.random.default_rng(RNG_SEED + 3)
    for L, d in [(0, 8), (1, 8), (5, 16), (37, 32), (130, 64)]:
        q = rng.standard_normal(d) * 0.7
        K = _rand_bf16(rng, (L, d))
        V = _rand_bf16(rng, (L, d))
        kn = rng.standard_normal(d)
        vn = rng.standard_normal(d)
        got = o.attention_head(q, K, V, kn, vn)
        ref = _sdpa_ref(q[None], _decode(K)[:, None, :], _decode(V)[:, None, :], kn[None],
                        vn[None], 1, 1)[0]
        assert _rel(got, ref) < 1e-12, (L, d, _rel(got, ref))


def pin_attention_brute_force_fsum(o):
    """A second, independent fp64 implementation on tiny shapes: plain Python
    loops, math.exp and math.fsum (exactly rounded sums), softmax written out
    with its max subtracted."""
    rng = np.random.default_rng(RNG_SEED + 13)
    for L, d in [(1, 3), (4, 5), (9, 8)]:
        q = [float(v) for v in rng.standard_normal(d)]
        K = _rand_bf16(rng, (L, d))
        V = _rand_bf16(rng, (L, d))
        kn = [float(v) for v in rng.standard_normal(d)]
        vn = [float(v) for v in rng.standard_normal(d)]
        keys = [[float(x) for x in row] for row in _decode(K)] + [kn]
        vals = [[float(x) for x in row] for row in _decode(V)] + [vn]
        scale = 1.0 / math.sqrt(d)
        scores = [math.fsum(q[i] * k[i] for i in range(d)) * scale for k in keys]
        top = max(scores)
        w = [math.exp(sc - top) for sc in scores]
        total = math.fsum(w)
        ref = [math.fsum(w[j] * vals[j][i] for j in range(L + 1)) / total for i in range(d)]
        got = o.attention_head(np.array(q), K, V, np.array(kn), np.array(vn))
        assert _rel(got, ref) < 1e-13, (L, d, _rel(got, ref))


def pin_one_token_context_returns_v(o):
    rng = np.random.default_rng(RNG_SEED + 4)
    d = 64
    q = rng.standard_normal(d) * 5.0
    kn = rng.standard_normal(d)
    vn = rng.standard_normal(d)
    out = o.attention_head(q, np.zeros((0, d), np.uint16), np.zeros((0, d), np.uint16), kn, vn)
    assert np.array_equal(out, vn)


def pin_equal_scores_give_mean(o):
    rng = np.random.default_rng(RNG_SEED + 5)
    d, L = 16, 23
    K = _rand_bf16(rng, (L, d))
    V = _rand_bf16(rng, (L, d))
    kn = rng.standard_normal(d)
    vn = rng.standard_normal(d)
    out = o.attention_head(np.zeros(d), K, V, kn, vn)            # q = 0: every score is 0
    Vf = np.concatenate([_decode(V), vn[None]], axis=0)
    mean = np.array([math.fsum(Vf[:, i]) / (L + 1) for i in range(d)])
    assert np.allclose(out, mean, rtol=1e-13, atol=1e-15)
    # identical keys (all equal to the fresh key) also give equal scores
    Ki = _bf16_bits(np.tile(_decode(K[0]), (L, 1)))
    out2 = o.attention_head(rng.standard_normal(d), Ki, V, _decode(K[0]), vn)
    assert np.allclose(out2, mean, rtol=1e-12, atol=1e-14)


def pin_hand_worked_softmax_weights(o):
    # d = 16, scale 1/4; q = 4 e0; keys j e0 (j = 0..3, the last one fresh) -> scores j.
    # With one-hot values V_j = e_j the output is e^j / (1 + e + e^2 + e^3).
    d = 16
    q = np.zeros(d)
    q[0] = 4.0
    K = np.zeros((3, d))
    V = np.zeros((3, d))
    for j in range(3):
        K[j, 0] = j
        V[j, j] = 1.0
    kn = np.zeros(d)
    kn[0] = 3.0
    vn = np.zeros(d)
    vn[3] = 1.0
    out = o.attention_head(q, _bf16_bits(K), _bf16_bits(V), kn, vn)
    s = 1 + math.e + math.e ** 2 + math.e ** 3
    expect = np.zeros(d)
    expect[:4] = [1 / s, math.e / s, math.e ** 2 / s, math.e ** 3 / s]
    assert np.allclose(out, expect, rtol=1e-14, atol=1e-16)


def pin_shift_invariance(o):
    # Adding delta to the e0 component of every key adds (q0 * delta / sqrt(d)) to
    # every score. Integer-valued keys keep K + delta exact in bf16.
    rng = np.random.default_rng(RNG_SEED + 6)
    d, L = 8, 40
    Ki = rng.integers(-8, 9, (L, d)).astype(np.float64)
    V = _rand_bf16(rng, (L, d))
    q = rng.standard_normal(d)
    q[0] = 600.0       # scores reach ~1700, so the softmax must subtract its max
    kn = rng.integers(-8, 9, d).astype(np.float64)
    vn = rng.standard_normal(d)
    base = o.attention_head(q, _bf16_bits(Ki), V, kn, vn)
    assert np.all(np.isfinite(base))
    K2 = Ki.copy()
    K2[:, 0] += 4.0
    kn2 = kn.copy()
    kn2[0] += 4.0
    shifted = o.attention_head(q, _bf16_bits(K2), V, kn2, vn)   # every score + ~849
    assert np.all(np.isfinite(shifted))
    assert np.allclose(shifted, base, rtol=1e-12, atol=1e-14)


def pin_affine_in_v(o):
    rng = np.random.default_rng(RNG_SEED + 7)
    d, L = 16, 31
    K = _rand_bf16(rng, (L, d))
    Vi = rng.integers(-20, 21, (L, d)).astype(np.float64)
    q = rng.standard_normal(d)
    kn = rng.standard_normal(d)
    vn = rng.standard_normal(d)
    base = o.attention_head(q, K, _bf16_bits(Vi), kn, vn)
    alpha, beta = 2.0, 3.0
    out = o.attention_head(q, K, _bf16_bits(alpha * Vi + beta), kn, alpha * vn + beta)
    assert np.allclose(out, alpha * base + beta, rtol=1e-13, atol=1e-13)


def pin_planted_token(o):
    rng = np.random.default_rng(RNG_SEED + 8)
    d, L = 32, 50
    q = np.zeros(d)
    q[0] = 8.0
    for pos in [0, 1, 17, L - 1, L]:                 # L = the fresh token
        K = rng.integers(-1, 2, (L, d)).astype(np.float64)
        K[:, 0] = 0.0
        kn = np.zeros(d)
        V = _rand_bf16(rng, (L, d))
        vn = rng.standard_normal(d)
        if pos < L:
            K[pos, 0] = 64.0                          # score 64*8/sqrt(32) ~ 90.5 vs 0
            target = _decode(V[pos])
        else:
            kn[0] = 64.0
            target = vn
        out = o.attention_head(q, _bf16_bits(K), V, kn, vn)
        # every other weight is e^-90.5 ~ 5e-40
        assert np.max(np.abs(out - target)) < 1e-30, pos


def pin_split_merge_equals_unsplit(o):
    rng = np.random.default_rng(RNG_SEED + 9)
    d, L = 16, 97
    K = _rand_bf16(rng, (L, d))
    V = _rand_bf16(rng, (L, d))
    q = rng.standard_normal(d) * 2.0
    kn = rng.standard_normal(d)
    vn = rng.standard_normal(d)
    ref = o.attention_head(q, K, V, kn, vn)
    for trial in range(6):
        n_cut = int(rng.integers(0, 8))
        cuts = sorted(set(int(c) for c in rng.integers(1, L + 1, n_cut)))
        edges = [0] + cuts + [L + 1]
        ms, ls, os_ = [], [], []
        for t0, t1 in zip(edges[:-1], edges[1:]):
            m, l, ov = o.attention_partial(q, K, V, kn, vn, t0, t1)
            ms.append(m)
            ls.append(l)
            os_.append(ov)
        merged = o.merge_partials(ms, ls, np.array(os_))
        assert _rel(merged, ref) < 1e-13, (trial, edges)
    # the partial state of a single key is (s, 1, V)
    m, l, ov = o.attention_partial(q, K, V, kn, vn, L, L + 1)
    assert l == 1.0 and np.array_equal(ov, vn)
    assert abs(m - float(np.dot(q, kn)) / math.sqrt(d)) < 1e-12


def pin_permutation_invariance(o):
    rng = np.random.default_rng(RNG_SEED + 10)
    d, L = 16, 45
    K = _rand_bf16(rng, (L, d))
    V = _rand_bf16(rng, (L, d))
    q = rng.standard_normal(d)
    kn = rng.standard_normal(d)
    vn = rng.standard_normal(d)
    ref = o.attention_head(q, K, V, kn, vn)
    perm = rng.permutation(L)
    out = o.attention_head(q, K[perm], V[perm], kn, vn)
    assert _rel(out, ref) < 1e-13
    # swapping the fresh token with cached row 0 (values exact in bf16) changes nothing
    kn_b = _decode(K[0])
    vn_b = _decode(V[0])
    K2 = K.copy()
    V2 = V.copy()
    Kn_bits = _bf16_bits(_decode(K[5]))
    K2[0] = Kn_bits
    V2[0] = V[5]
    ref2 = o.attention_head(q, K2, V2, kn_b, vn_b)
    K3 = K2.copy()
    V3 = V2.copy()
    K3[0] = K[0]
    V3[0] = V[0]
    out3 = o.attention_head(q, K3, V3, _decode(K[5]), _decode(V[5]))
    assert _rel(out3, ref2) < 1e-13


def pin_decode_step_matches_libraries(o):
    """Whole step on a tiny GQA shape vs numpy projection + torch SDPA."""
    rng = np.random.default_rng(RNG_SEED + 11)
    B, hidden, Hq, Hkv, d = 3, 48, 6, 2, 8
    n_out = (Hq + 2 * Hkv) * d
    Lmax = 20
    x = _rand_bf16(rng, (B, hidden))
    W = _rand_bf16(rng, (n_out, hidden), 0.2)
    ctx = np.array([0, 7, 20], dtype=np.int32)
    K = _rand_bf16(rng, (B, Lmax, Hkv, d))
    V = _rand_bf16(rng, (B, Lmax, Hkv, d))
    res = o.decode_step(x, W, ctx, K, V, Hq, Hkv, d, threads=2)
    for b in range(B):
        y = _decode(W) @ _decode(x[b])
        q = y[:Hq * d].reshape(Hq, d)
        kn = y[Hq * d:(Hq + Hkv) * d].reshape(Hkv, d)
        vn = y[(Hq + Hkv) * d:].reshape(Hkv, d)
        L = int(ctx[b])
        ref = _sdpa_ref(q, _decode(K[b, :L]), _decode(V[b, :L]), kn, vn, Hq, Hkv)
        assert _rel(res["attn_out"][b], ref.reshape(-1)) < 1e-12, b
        assert np.allclose(res["k_new"][b], kn, rtol=1e-13, atol=1e-15)
        assert np.allclose(res["v_new"][b], vn, rtol=1e-13, atol=1e-15)
        assert np.allclose(res["q"][b], q, rtol=1e-13, atol=1e-15)


def pin_gqa_grouping(o):
    assert [o.kv_head_of(h, 32, 8) for h in range(8)] == [0, 0, 0, 0, 1, 1, 1, 1]
    assert o.kv_head_of(31, 32, 8) == 7
    assert [o.kv_head_of(h, 8, 8) for h in range(8)] == list(range(8))
    assert o.kv_head_of(63, 64, 8) == 7 and o.kv_head_of(8, 64, 8) == 1


def pin_gemm_brute_force(o):
    """C = A x B^T, element by element in plain Python with math.fsum, on a
    shape where rows, columns and k all differ (a transposed operand or a
    swapped index changes the answer)."""
    rng = np.random.default_rng(RNG_SEED + 40)
    M, N, K = 3, 5, 7
    A = _rand_bf16(rng, (M, K))
    B = _rand_bf16(rng, (N, K))
    a, b = _decode(A), _decode(B)
    C = o.gemm_nt(A, B)
    for i in range(M):
        for j in range(N):
            ref = math.fsum(float(a[i, k]) * float(b[j, k]) for k in range(K))
            assert abs(C[i, j] - ref) <= 1e-12 * (1.0 + abs(ref)), (i, j)


def pin_gemm_matches_numpy_and_is_exact_on_integers(o):
    """Sampled entries equal numpy's fp64 matmul (library routine); with
    small-integer operands every entry is an exact integer."""
    rng = np.random.default_rng(RNG_SEED + 41)
    M, N, K = 40, 24, 96
    A = _rand_bf16(rng, (M, K))
    B = _rand_bf16(rng, (N, K), 0.3)
    ref = _decode(A) @ _decode(B).T
    rows = rng.integers(0, M, 50)
    cols = rng.integers(0, N, 50)
    got = o.gemm_nt_entries(A, B, rows, cols)
    assert np.allclose(got, ref[rows, cols], rtol=1e-12, atol=1e-12)
    ai = rng.integers(-5, 6, (M, K))
    bi = rng.integers(-5, 6, (N, K))
    Ci = o.gemm_nt(_bf16_bits(ai), _bf16_bits(bi))
    assert np.array_equal(Ci, (ai @ bi.T).astype(np.float64))


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
