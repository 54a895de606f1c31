"""Planted mistakes in the oracle must fail a pin (CPU only).

Each mutant is a one-line textual change to a copy of ``oracle/w4a16_oracle.c``
(a dropped term, a wrong sign, index or shift, a transposed operand), built
with gcc into a temporary library. The pins of ``tests/test_oracle.py`` run
against it; at least one must fail. The real oracle is never modified.
"""

from __future__ import annotations

import os
import subprocess

import pytest
import torch

import tests.test_oracle as pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "w4a16_oracle.c")

# (name, original text, planted text). Each original must occur exactly once.
MUTANTS = [
    ("unpack_reversed_nibbles", "codes[n * K + k] = (uint8_t)((w >> (4 * (k % 8)))",
     "codes[n * K + k] = (uint8_t)((w >> (4 * (7 - k % 8)))"),
    ("unpack_wrong_word", "uint32_t w = words[n * K8 + k / 8];", "uint32_t w = words[n * K8 + k % K8];"),
    ("pack_reversed", "w |= ((uint32_t)(codes[n * K + 8 * j + i] & 0xFu)) << (4 * i);",
     "w |= ((uint32_t)(codes[n * K + 8 * j + i] & 0xFu)) << (4 * (7 - i));"),
    ("zeros_unpack_row_order", "zeros[n * Kg + g] = (uint8_t)((zp_words[(n / 8) * Kg + g] >> (4 * (n % 8)))",
     "zeros[n * Kg + g] = (uint8_t)((zp_words[(n / 8) * Kg + g] >> (4 * (7 - n % 8)))"),
    ("zero_of_row_order", "return (int)((zp_words[(n / 8) * Kg + g] >> (4 * (n % 8))) & 0xFu);",
     "return (int)((zp_words[(n / 8) * Kg + g] >> (4 * (7 - n % 8))) & 0xFu);"),
    ("zero_of_transposed", "return (int)((zp_words[(n / 8) * Kg + g]", "return (int)((zp_words[(g % (n / 8 + 1)) * Kg + g]"),
    ("symmetric_zero_7", "if (qtype == W4O_UINT4B8) return 8;", "if (qtype == W4O_UINT4B8) return 7;"),
    ("symmetric_uses_zero_points", "if (qtype == W4O_UINT4B8) return 8;", "if (qtype == W4O_UINT4B8 && zp_words == NULL) return 8;"),
    ("missing_zero_is_8", "if (zp_words == NULL) return 0;", "if (zp_words == NULL) return 8;"),
    ("dequant_sign", "out[k] = (double)(q - z) * scales[n * Kg + g];", "out[k] = (double)(z - q) * scales[n * Kg + g];"),
    ("dequant_drop_zero", "out[k] = (double)(q - z) * scales[n * Kg + g];", "out[k] = (double)(q) * scales[n * Kg + g];"),
    ("group_modulo", "int64_t g = k / Ge;", "int64_t g = k % Kg;"),
    ("scale_transposed", "out[k] = (double)(q - z) * scales[n * Kg + g];",
     "out[k] = (double)(q - z) * scales[(g * (n + 1)) % Kg + n * Kg];"),
    ("gemm_drops_last_k", "for (int64_t k = 0; k < K; ++k) acc += a[k] * wrow[k];",
     "for (int64_t k = 0; k < K - 1; ++k) acc += a[k] * wrow[k];"),
    ("gemm_wrong_a_row", "const double *a = A + m * lda;", "const double *a = A + (M - 1 - m) * lda;"),
    ("gemm_output_transposed", "C[m * N + n] = acc;", "C[n * M + m] = acc;"),
    ("gemm_bias_dropped", "if (bias != NULL) acc += bias[n];", "if (bias != NULL) acc += 0.0;"),
    ("gemm_bias_wrong_index", "if (bias != NULL) acc += bias[n];", "if (bias != NULL) acc += bias[m % N];"),
    ("encode_nibble_order", "<< (4 * (i / 2) + 16 * (i % 2));", "<< (4 * i);"),
    ("encode_lane_rows", "const int64_t n = 16 * nt + l % 16;", "const int64_t n = 16 * nt + (l / 4) % 16;"),
    ("encode_subblock", "const int64_t k0 = 128 * kt + 32 * s + 8 * (l / 16);",
     "const int64_t k0 = 128 * kt + 32 * (l / 16) + 8 * s;"),
    ("encode_scale_order", "const int64_t off = S0 + ((nt * Kg + g) * 16 + r) * 2;",
     "const int64_t off = S0 + ((nt * 16 + r) * Kg + g) * 2;"),
]

# Pins to run (function, kwargs). Parametrised pins are listed per case.
PIN_CALLS = [
    (pins.test_gptq_hand_words, {}),
    (pins.test_gptq_little_endian_byte_view, {}),
    (pins.test_zero_point_hand_words, {}),
    (pins.test_zero_point_byte_view, {}),
    (pins.test_dequant_symmetric_closed_form, {"G": 32}),
    (pins.test_dequant_symmetric_closed_form, {"G": -1}),
    (pins.test_dequant_asymmetric_closed_form, {"G": 32}),
    (pins.test_dequant_asymmetric_closed_form, {"G": -1}),
    (pins.test_dequant_symmetric_ignores_zero_points, {}),
    (pins.test_gemm_zero_weights_give_bias, {"qtype": pins.UINT4}),
    (pins.test_gemm_uniform_codes_unit_scales, {"cval": 1}),
    (pins.test_gemm_unit_codes_group_scales, {}),
    (pins.test_gemm_identity_activations, {}),
    (pins.test_gemm_exact_rational, dict(M=2, N=16, K=128, G=128, qtype=pins.UINT4, with_bias=True)),
    (pins.test_device_encoder_hand_words, {}),
    (pins.test_device_encoder_inverse, {}),
]


def _run_pins(oracle_mod):
    failed = []
    for fn, kw in PIN_CALLS:
        try:
            fn(oracle_mod, **kw)
        except AssertionError:
            failed.append(fn.__name__)
    return failed


@pytest.mark.parametrize("name,orig,planted", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(oracle_mod, tmp_path, name, orig, planted):
    src = open(SRC).read()
    assert src.count(orig) == 1, f"mutant {name}: anchor text not found exactly once"
    mut_c = tmp_path / "mutant.c"
    mut_c.write_text(src.replace(orig, planted))
    lib = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-std=c99", "-O1", "-fopenmp", "-fPIC", "-shared", "-o", str(lib), str(mut_c)], check=True)
    torch.manual_seed(0)
    with oracle_mod._use_library(str(lib)):
        failed = _run_pins(oracle_mod)
    assert failed, f"mutant {name} passed every pin"


def test_unmutated_oracle_passes_the_same_pins(oracle_mod):
    assert _run_pins(oracle_mod) == []
