"""Planted mistakes in the oracle must fail a pin (CPU only).

Each mutant is a one-line textual change to a copy of ``oracle/w4a16_oracle.c``
(a dropped term, a wrong sign, index or shift, a transposed operand), built
with gcc into a temporary library. The pins of ``tests/test_oracle.py`` run
against it; at least one must fail. The numpy readers of the other checkpoint
orientations get the same treatment from a mutated copy of
``oracle/__init__.py`` loaded as a separate module. The real oracle is never
modified.
"""

from __future__ import annotations

import os
import subprocess
import types

import pytest
import torch

import tests.test_oracle as pins

ORACLE_DIR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle")
SRC = os.path.join(ORACLE_DIR, "w4a16_oracle.c")
PY_SRC = os.path.join(ORACLE_DIR, "__init__.py")

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
    ("encode_scale_order", "const int64_t off = S0 + ((nt * Kgp + g) * 16 + r) * 2;",
     "const int64_t off = S0 + ((nt * 16 + r) * Kgp + g) * 2;"),
    ("encode_scales_unpadded_stride", "const int64_t off = S0 + ((nt * Kgp + g) * 16 + r) * 2;",
     "const int64_t off = S0 + ((nt * Kg + g) * 16 + r) * 2;"),
    ("layout_k_rounded_to_64", "return (K + 127) / 128 * 128;", "return (K + 63) / 64 * 64;"),
    ("layout_n_rounded_to_8", "return (N + 15) / 16 * 16;", "return (N + 7) / 8 * 8;"),
    ("encode_scales_of_padding_rows", "for (int r = 0; r < 16 && 16 * nt + r < N; ++r) {",
     "for (int r = 0; r < 16 && 16 * nt + r < N - 1; ++r) {"),
    ("layout_groups_unpadded", "return K / Ge == 1 ? 1 : padded_k(K) / Ge;", "return K / Ge;"),
    ("encode_zeros_unpadded_stride", "out[Z0 + (nt * Kgp + g) * 16 + r]", "out[Z0 + (nt * Kg + g) * 16 + r]"),
    ("a8_truncates", "const float t = rintf((float)A[m * K + k] / s);", "const float t = truncf((float)A[m * K + k] / s);"),
    ("a8_scale_128", "const float s = amax / 127.0f;", "const float s = amax / 128.0f;"),
    ("w4a8_zero_7", "isum += (int64_t)q[m * K + k] * (code - 8);", "isum += (int64_t)q[m * K + k] * (code - 7);"),
    ("w4a8_no_row_scale", "acc *= (double)xs[m];", "acc *= 1.0;"),
    ("w4a8_group_scale_index", "acc += scales[n * Kg + g] * (double)isum;", "acc += scales[n * Kg] * (double)isum;"),
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
    (pins.test_device_size_hand_values, {}),
    (pins.test_device_encoder_padded_k_hand_words, {}),
    (pins.test_device_encoder_padded_groups_hand_values, {}),
    (pins.test_device_encoder_padded_inverse, {}),
    (pins.test_device_encoder_padded_n_hand_words, {}),
    (pins.test_device_encoder_padded_n_inverse, {}),
    (pins.test_quant_a8_hand_values, {}),
    (pins.test_quant_a8_properties, {}),
    (pins.test_gemm_w4a8_exact_rational, {"G": 32, "with_bias": True}),
    (pins.test_gemm_w4a8_zero_weights_give_bias, {}),
    (pins.test_gemm_w4a8_matches_dequantised_product, {}),
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
    subprocess.run(["gcc", "-std=c99", "-O1", "-fopenmp", "-fPIC", "-shared", "-o", str(lib), str(mut_c), "-lm"], check=True)
    torch.manual_seed(0)
    with oracle_mod._use_library(str(lib)):
        failed = _run_pins(oracle_mod)
    assert failed, f"mutant {name} passed every pin"


def test_unmutated_oracle_passes_the_same_pins(oracle_mod):
    assert _run_pins(oracle_mod) == []


# Mutants of the numpy orientation readers in oracle/__init__.py.
PY_MUTANTS = [
    ("int4_reversed_nibbles", "shifts = np.arange(8, dtype=np.uint32) * 4", "shifts = (7 - np.arange(8, dtype=np.uint32)) * 4"),
    ("int4_interleave", "v = v.reshape(w.shape[0], w.shape[1] * 8)",
     "v = np.swapaxes(v, -1, -2).reshape(w.shape[0], w.shape[1] * 8)"),
    ("weight_no_transpose", "return np.ascontiguousarray(codes.T) if output_dim != 0 else codes", "return codes"),
    ("weight_packed_dim_ignored", "codes = unpack_int4(weight, packed_dim)", "codes = unpack_int4(weight, 1 - output_dim)"),
    ("zeros_no_transpose", "        zw = np.ascontiguousarray(zw.T)\n    return unpack_int4(zw, 0)",
     "        pass\n    return unpack_int4(zw, 0)"),
    ("zeros_wrong_dim", "return unpack_int4(zw, 0)", "return np.ascontiguousarray(unpack_int4(zw, 1).T)"),
    ("scales_no_transpose", "return (s.t() if output_dim != 0 else s).contiguous()", "return s.contiguous()"),
]

PY_PIN_CALLS = [(pins.test_layout_hand_words, {"idx": i}) for i in range(6)] + [
    (pins.test_layout_canonical_matches_c_unpack, {}),
    (pins.test_layout_zero_points_match_c_unpack, {}),
    (pins.test_layout_scales_orientation, {}),
]


def _mutated_module(src: str):
    mod = types.ModuleType("oracle_mutant")
    mod.__file__ = PY_SRC  # so it finds (and shares) the built C library
    exec(compile(src, PY_SRC, "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name,orig,planted", PY_MUTANTS, ids=[m[0] for m in PY_MUTANTS])
def test_planted_reader_mistake_is_caught(oracle_mod, name, orig, planted):
    src = open(PY_SRC).read()
    assert src.count(orig) == 1, f"mutant {name}: anchor text not found exactly once"
    mod = _mutated_module(src.replace(orig, planted))
    failed = []
    for fn, kw in PY_PIN_CALLS:
        try:
            fn(mod, **kw)
        except (AssertionError, ValueError):
            failed.append(fn.__name__)
    assert failed, f"mutant {name} passed every pin"


def test_unmutated_readers_pass_the_same_pins(oracle_mod):
    mod = _mutated_module(open(PY_SRC).read())
    for fn, kw in PY_PIN_CALLS:
        fn(mod, **kw)
