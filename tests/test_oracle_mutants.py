"""The oracle's pins catch plausible mistakes.

Each case copies oracle.c, plants one mistake in the copy (a dropped term, a wrong
sign, offset or index, a transposed operand, a broken IEEE decode), builds it with
gcc on the CPU and checks that at least one pin of tests/oracle_pins.py fails on
it.  The real oracle is never modified.
"""
import os

import pytest

from oracle import build as oracle_build
from oracle.oracle import Oracle
from tests import oracle_pins

MUTANTS = {
    "zero_point_7": ("(double)(code - 8)", "(double)(code - 7)"),
    "sign_flip": ("(double)(code - 8)", "(double)(8 - code)"),
    "scale_transposed": ("group * N + n", "n * (K / group_size) + group"),
    "group_modulo": ("int64_t group = k / group_size;", "int64_t group = k % (K / group_size);"),
    "fwd_k_reversed": ("element(x, act_dtype, m * K + k)", "element(x, act_dtype, m * K + (K - 1 - k))"),
    "bwd_n_reversed": ("element(d_out, act_dtype, m * N + n)", "element(d_out, act_dtype, m * N + (N - 1 - n))"),
    "fwd_first_term_dropped": ("for (int64_t k = 0; k < K; ++k) {", "for (int64_t k = 1; k < K; ++k) {"),
    "bwd_first_term_dropped": ("for (int64_t n = 0; n < N; ++n) {", "for (int64_t n = 1; n < N; ++n) {"),
    "fwd_norm_signed": ("norm += fabs(a) * fabs(w);", "norm += a * w;"),
    "bwd_norm_signed": ("norm += fabs(g) * fabs(w);", "norm += fabs(g) * w;"),
    "f16_exponent_bias": ("exponent - 25", "exponent - 24"),
    "f16_subnormal": ("ldexp((double)fraction, -24)", "ldexp((double)fraction, -25)"),
    "bf16_hidden_bit": ("(fraction | 0x80)", "(fraction | 0x100)"),
    "f32_exponent_bias": ("exponent - 150", "exponent - 149"),
    "threads_reorder": ("int64_t m = o / N, n = o % N;", "int64_t m = o % M, n = o / M;"),
    "embedding_ids_reversed": ("int64_t n = ids[t];", "int64_t n = ids[T - 1 - t];"),
    "embedding_out_of_range_one": (": 0.0;", ": 1.0;"),
    "embedding_k_reversed": ("group_size, n, k)\n", "group_size, n, K - 1 - k)\n"),
    "dq8ca_scale_256": ("(hi - lo) / 255.0f", "(hi - lo) / 256.0f"),
    "dq8ca_zero_point_sign": ("int z = -128 - (int)rintf(lo * inv);", "int z = -128 + (int)rintf(lo * inv);"),
    "dq8ca_truncate": ("int t = (int)rintf(v * inv) + z;", "int t = (int)(v * inv) + z;"),
    "dq8ca_clamp_126": ("if (t > 127) t = 127;", "if (t > 126) t = 126;"),
    "dq8ca_range_without_zero": ("float lo = 0.0f, hi = 0.0f;", "float lo = 1e30f, hi = -1e30f;"),
    "dq8ca_linear_without_zp": ("(double)((int)q[m * K + k] - (int)zp[m])", "(double)((int)q[m * K + k])"),
    "dq8ca_linear_first_row_scale": ("const double sm = (double)scale[m];", "const double sm = (double)scale[0];"),
    "lora_fwd_alpha_dropped": ("y[row * N + col] += alpha * acc * (double)B[col * rank + j];",
                               "y[row * N + col] += acc * (double)B[col * rank + j];"),
    "lora_fwd_B_transposed": ("y[row * N + col] += alpha * acc * (double)B[col * rank + j];",
                              "y[row * N + col] += alpha * acc * (double)B[j * N + col];"),
    "lora_bwd_dx_sign": ("dx[row * K + c] += alpha * u * (double)A[j * K + c];",
                         "dx[row * K + c] -= alpha * u * (double)A[j * K + c];"),
    "lora_bwd_dA_from_t": ("dA[j * K + c] += alpha * u * a;", "dA[j * K + c] += alpha * tx * a;"),
    "lora_bwd_dB_from_u": ("dB[col * rank + j] += alpha * g * tx;", "dB[col * rank + j] += alpha * g * u;"),
    "adamw_no_bias_correction": ("param -= lr * (m1 / bias1) / (sqrt(v1 / bias2) + eps);",
                                 "param -= lr * m1 / (sqrt(v1) + eps);"),
    "adamw_coupled_decay": ("        const double grad = (double)g[i];\n        param -= lr * weight_decay * param;",
                            "        const double grad = (double)g[i] + weight_decay * param;"),
    "adamw_eps_inside_sqrt": ("(sqrt(v1 / bias2) + eps)", "sqrt(v1 / bias2 + eps)"),
    "adamw_beta2_in_first_moment": ("const double m1 = beta1 * (double)m[i] + (1.0 - beta1) * grad;",
                                    "const double m1 = beta1 * (double)m[i] + (1.0 - beta2) * grad;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(oracle_build.SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not unique"
    mutant_src = tmp_path / "oracle_mutant.c"
    mutant_src.write_text(src.replace(old, new))
    lib = oracle_build.build(src=str(mutant_src), out=str(tmp_path / f"liboracle_{name}.so"))
    o = Oracle(lib)
    failed = []
    for pin in oracle_pins.PINS:
        try:
            pin(o)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"no pin caught mutant {name}"
