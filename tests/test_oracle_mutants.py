"""Plant plausible mistakes in the oracle's C source and check that the pins in
``test_oracle.py`` catch every one of them (runs on the CPU only).

Each mutant is a textual edit of ``oracle/gemm_oracle.c`` compiled into a temporary
directory; the pins run against it in a child process (a mutant that reads out of bounds
may crash, which also counts as caught).
"""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# (name, [(old, new), ...]); every "old" must occur in the source.
MUTANTS = [
    ("drop_first_k_term", [("for (int64_t k = 0; k < K; ++k)", "for (int64_t k = 1; k < K; ++k)")]),
    ("drop_last_k_term", [("for (int64_t k = 0; k < K; ++k)", "for (int64_t k = 0; k + 1 < K; ++k)")]),
    ("transposed_B", [("Bd[k * N + j]", "Bd[j * K + k]"), ("B[k * N + j]", "B[j * K + k]")]),
    ("transposed_A", [("Ad[i * K + k]", "Ad[k * M + i]"),
                      ("A[i * K + k]", "A[k * (N + 0) + i]")]),
    ("bias_by_row", [("oracle_f16_to_f64(bias[j])", "oracle_f16_to_f64(bias[i % N])")]),
    ("gelu_erfc_sign", [("erfc(-x / sqrt(2.0))", "erfc(x / sqrt(2.0))")]),
    ("gelu_tanh_form", [("0.5 * x * (1.0 + erf(x / sqrt(2.0)))",
                         "0.5 * x * (1.0 + tanh(0.7978845608028654 * (x + 0.044715 * x * x * x)))")]),
    ("gelu_missing", [("if (epi == 2) v = oracle_gelu(v);", "if (epi == 3) v = oracle_gelu(v);")]),
    ("bias_missing", [("double v = s + bias_j;", "double v = s + 0.0 * bias_j;")]),
    ("gelu_before_bias", [("double v = s + bias_j;\n    if (epi == 2) v = oracle_gelu(v);",
                           "double v = s;\n    if (epi == 2) v = oracle_gelu(v);\n    v += bias_j;")]),
    ("ties_away_from_zero", [("return (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;", "return fl + 1.0;")]),
    ("truncate_not_round", [("if (d > 0.5) return fl + 1.0;", "if (d > 1.5) return fl + 1.0;")]),
    ("decode_exponent_bias", [("e - 25", "e - 24")]),
    ("decode_subnormal_scale", [("ldexp((double)f, -24)", "ldexp((double)f, -25)")]),
    ("decode_drops_sign", [("return sign ? -v : v;", "return v;")]),
    ("overflow_unhandled", [("if (a >= 65520.0)", "if (a >= 1.0e300)")]),
    ("subnormal_encode_flush", [("double n = round_half_even(ldexp(a, 24));", "double n = 0.0;")]),
    ("fp32_accumulation", [("double s = 0.0;", "float s = 0.0f;"),
                           ("for (int64_t j = 0; j < N; ++j) acc[j] += a * Bd[k * N + j];",
                            "for (int64_t j = 0; j < N; ++j) acc[j] = (float)(acc[j] + a * Bd[k * N + j]);")]),
    ("softmax_no_max_shift", [("s += exp(oracle_f16_to_f64(xr[j]) - m);", "s += exp(oracle_f16_to_f64(xr[j]) - 0.0 * m);")]),
    ("softmax_skips_first", [("for (int64_t j = 0; j < N; ++j) s += exp(", "for (int64_t j = 1; j < N; ++j) s += exp(")]),
    ("softmax_wrong_axis", [("const uint16_t *xr = x + i * N;", "const uint16_t *xr = x + (i * N) % (N > 1 ? N : 1);")]),
    ("vector_add_subtracts", [("oracle_f16_to_f64(a[i]) + oracle_f16_to_f64(b[i])",
                               "oracle_f16_to_f64(a[i]) - oracle_f16_to_f64(b[i])")]),
    ("vector_add_drops_b", [("oracle_f16_to_f64(a[i]) + oracle_f16_to_f64(b[i])",
                             "oracle_f16_to_f64(a[i]) + 0.0 * oracle_f16_to_f64(b[i])")]),
    ("attn_causal_strict", [("return (causal && i + 1 < Sk) ? i + 1 : Sk;",
                             "return (causal && i < Sk) ? i : Sk;")]),
    ("attn_causal_ignored", [("return (causal && i + 1 < Sk) ? i + 1 : Sk;", "return Sk;")]),
    ("attn_no_scale", [("sbuf[j] = scale * dot;", "sbuf[j] = dot;")]),
    ("attn_transposed_k", [("oracle_f16_to_f64(kb[j * D + d])", "oracle_f16_to_f64(kb[d * nkeys + j])")]),
    ("attn_transposed_v", [("oracle_f16_to_f64(vb[j * D + d])", "oracle_f16_to_f64(vb[d * nkeys + j])")]),
    ("attn_not_normalised", [("oi[d] = oracle_f64_to_f16(acc / l);", "oi[d] = oracle_f64_to_f16(acc);")]),
    ("attn_lse_no_log", [("*lse_i = m + log(l);", "*lse_i = m + l;")]),
    ("attn_no_max_shift", [("sbuf[j] = exp(sbuf[j] - m);", "sbuf[j] = exp(sbuf[j]);")]),
    ("attn_kv_of_pair_zero", [("k + b * Sk * D, v + b * Sk * D, scale,\n                              allowed_keys",
                               "k, v, scale,\n                              allowed_keys")]),
    ("vector_add_float_sum", [("oracle_f16_to_f64(a[i]) + oracle_f16_to_f64(b[i])",
                               "(double)(float)(oracle_f16_to_f64(a[i]) + oracle_f16_to_f64(b[i]) * 1.0000001)")]),
]


def test_every_mutation_applies():
    src = open(oracle.SOURCE).read()
    for name, edits in MUTANTS:
        for old, _ in edits:
            assert old in src, (name, old)


@pytest.mark.parametrize("name,edits", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(tmp_path, name, edits):
    src = open(oracle.SOURCE).read()
    for old, new in edits:
        src = src.replace(old, new)
    csrc = tmp_path / "mutant.c"
    csrc.write_text(src)
    lib = tmp_path / "libmutant.so"
    subprocess.run(oracle.compile_command(str(csrc), str(lib)), check=True,
                   stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL)
    env = dict(os.environ, ORACLE_LIB=str(lib), OMP_NUM_THREADS="4")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle.py")],
                       cwd=ROOT, env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                       timeout=600)
    assert r.returncode != 0, "mutant %s survived every pin:\n%s" % (name, r.stdout.decode()[-2000:])
