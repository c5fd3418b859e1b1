"""The oracle against its pins, and mutated copies of the oracle against the
same pins (every mutant must be caught by at least one)."""
import os
import subprocess

import numpy as np
import pytest

import oracle as oracle_pkg
from tests import oracle_pins



@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin, oracle):
    pin(oracle)


# Plausible mistakes, each a textual edit of oracle.c: (name, original, mutated).
MUTANTS = [
    ("scale_1_over_d", "return 1.0 / sqrt((double)d);", "return 1.0 / (double)d;"),
    ("fresh_token_dropped", "const int64_t n = L + 1;", "const int64_t n = L;"),
    ("gqa_interleaved", "return h / (n_q_heads / n_kv_heads);", "return h % n_kv_heads;"),
    ("projection_transposed",
     "acc += oracle_bf16_to_f64(w[k]) * oracle_bf16_to_f64(x[k]);",
     "acc += oracle_bf16_to_f64(W[k * n_out + n]) * oracle_bf16_to_f64(x[k]);"),
    ("no_max_subtraction", "s[j] = exp(s[j] - m);", "s[j] = exp(s[j]);"),
    ("cache_row_off_by_one",
     "return j < L ? oracle_bf16_to_f64(K[j * tok_stride + i]) : k_new[i];",
     "return j < L ? oracle_bf16_to_f64(K[(j + 1 < L ? j + 1 : j) * tok_stride + i]) : k_new[i];"),
    ("score_sign", "acc += q[i] * key_elem(K, tok_stride, L, k_new, j, i);",
     "acc -= q[i] * key_elem(K, tok_stride, L, k_new, j, i);"),
    ("values_read_from_keys",
     "double v = j < L ? oracle_bf16_to_f64(V[j * tok_stride + i]) : v_new[i];",
     "double v = j < L ? oracle_bf16_to_f64(K[j * tok_stride + i]) : v_new[i];"),
    ("merge_ignores_max", "denom += exp(m[s] - M) * l[s];", "denom += l[s];"),
    ("partial_counts_keys", "l += p;", "l += 1.0;"),
    ("fresh_key_from_group0", "const double *kn = yb + n_q_heads * d + g * d;",
     "const double *kn = yb + n_q_heads * d;"),
    ("fresh_value_is_key", "const double *vn = yb + (n_q_heads + n_kv_heads) * d + g * d;",
     "const double *vn = yb + n_q_heads * d + g * d;"),
    ("cache_head_ignored", "const uint16_t *Kb = K + (b * Lmax) * tok_stride + g * d;",
     "const uint16_t *Kb = K + (b * Lmax) * tok_stride;"),
    ("bf16_ties_away", "double r = nearbyint(ldexp(x, -qexp));",
     "double r = round(ldexp(x, -qexp));"),
    ("bf16_double_rounding", "double r = nearbyint(ldexp(x, -qexp));",
     "double r = nearbyint(ldexp((double)(float)x, -qexp));"),
    ("bf16_decode_shift", "uint32_t u = (uint32_t)h << 16;", "uint32_t u = (uint32_t)h << 15;"),
    ("merge_unweighted_output", "acc += exp(m[s] - M) * o[s * d + i];", "acc += o[s * d + i];"),
    ("gemm_operand_transposed", "const uint16_t *b = B + cols[e] * K;", "const uint16_t *b = B + cols[e];"),
    ("gemm_k_range_short", "for (int64_t k = 0; k < K; ++k)\n            acc += oracle_bf16_to_f64(a[k])",
     "for (int64_t k = 1; k < K; ++k)\n            acc += oracle_bf16_to_f64(a[k])"),
]


def test_mutant_table_is_distinct():
    names = [m[0] for m in MUTANTS]
    assert len(names) == len(set(names))


@pytest.mark.parametrize("name,orig,mut", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, orig, mut, tmp_path):
    src = open(oracle_pkg.SOURCE).read()
    n = src.count(orig)
    assert n >= 1, "mutation site vanished from oracle.c: %s" % orig
    path = tmp_path / ("oracle_%s.c" % name)
    path.write_text(src.replace(orig, mut))
    so = str(tmp_path / ("liboracle_%s.so" % name))
    oracle_pkg.compile_library(str(path), so)
    mutant = oracle_pkg.Oracle(so)
    failed = []
    with np.errstate(all="ignore"):
        for pin in oracle_pins.ALL_PINS:
            try:
                pin(mutant)
            except (AssertionError, ValueError, FloatingPointError):
                failed.append(pin.__name__)
    assert failed, "no pin catches mutant %s" % name
