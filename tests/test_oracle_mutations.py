"""The oracle's pins must catch plausible mistakes.

Each case plants one mistake in a copy of the oracle's C source (on the CPU,
in a temporary directory), builds it, and runs the pin tests against that
build: at least one pin has to fail.  This shows the pins constrain every
step of the oracle: decode, sum of squares, mean, eps, weight, table index,
partner index, sign, rounding.
"""
import os

import numpy as np
import pytest

import oracle
import tests.test_oracle_pins as pins

MUTATIONS = {
    "drop_last_square": ("sum_sq += v[d] * v[d];", "if (d + 1 < D) sum_sq += v[d] * v[d];"),
    "sum_not_mean": ("sum_sq / (double)D", "sum_sq"),
    "eps_outside_root": ("1.0 / sqrt(ms + eps64)", "1.0 / sqrt(ms) + eps64"),
    "gamma_reversed": ("(double)gamma[d]", "(double)gamma[D - 1 - d]"),
    "first_sign": ("oh[a] = nrm[a] * ca - nrm[b] * sa;", "oh[a] = nrm[a] * ca + nrm[b] * sa;"),
    "both_signs": ("oh[a] = nrm[a] * ca - nrm[b] * sa;\n                oh[b] = nrm[b] * cb + nrm[a] * sb;",
                   "oh[a] = nrm[a] * ca + nrm[b] * sa;\n                oh[b] = nrm[b] * cb - nrm[a] * sb;"),
    "cos_of_first_for_both": ("cb = table_value(cos, cos_dtype, row * D + b)",
                              "cb = table_value(cos, cos_dtype, row * D + a)"),
    "sin_of_second_for_both": ("sa = table_value(sin, cos_dtype, row * D + a)",
                               "sa = table_value(sin, cos_dtype, row * D + b)"),
    "cos_sin_swapped": ("ca = table_value(cos,", "ca = table_value(sin,"),
    "per_head_row_transposed": ("t * heads + h;", "t + h * heads;"),
    "rotate_half_partner": ("b = i + half;", "b = D - 1 - i;"),
    "fp16_subnormal_scale": ("ldexp((double)m / 1024.0, -14)", "ldexp((double)m / 1024.0, -15)"),
    "bf16_bias": ("1.0 + (double)m / 128.0, e - 127", "1.0 + (double)m / 128.0, e - 126"),
    "round_ties_away": ("rint(a / q)", "round(a / q)"),
    "gamma_after_rope_missing": ("nrm[d] = v[d] * r * (double)gamma[d];", "nrm[d] = v[d] * r;"),
}

PIN_TESTS = [
    (pins.test_decode_bf16_exhaustive, {}),
    (pins.test_decode_fp16_exhaustive, {}),
    (pins.test_round_fp16_matches_numpy, {}),
    (pins.test_round_bf16_properties, {}),
    (pins.test_norm_matches_torch_rms_norm, {"x_dtype": "fp16", "head_dim": 64}),
    (pins.test_interleaved_is_complex_multiply, {}),
    (pins.test_rotate_half_textbook_form, {}),
    (pins.test_rms_closed_form, {}),
    (pins.test_styles_agree_under_permutation, {}),
    (pins.test_pair_norm_identity, {"style": "interleaved"}),
    (pins.test_brute_force_fused_qkv, {"style": "rotate_half", "cos_layout": "per_head",
                                       "x_dtype": "bf16", "cos_dtype": "fp32", "head_dim": 64}),
]


def _caught(variant) -> list:
    caught = []
    for fn, kw in PIN_TESTS:
        try:
            with np.errstate(all="ignore"):
                fn(variant, **kw)
        except AssertionError:
            caught.append(fn.__name__)
    return caught


def test_unmutated_source_passes_every_pin():
    assert _caught(oracle.default()) == []


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(tmp_path, name):
    old, new = MUTATIONS[name]
    with open(oracle.SRC) as f:
        src = f.read()
    assert src.count(old) >= 1, "mutation anchor not found: " + name
    mutated = src.replace(old, new, 1)
    path = os.path.join(tmp_path, "mut.c")
    with open(path, "w") as f:
        f.write(mutated)
    lib = oracle.compile_source(path, os.path.join(tmp_path, "libmut.so"))
    caught = _caught(oracle.Oracle(lib))
    assert caught, "no pin catches mutation " + name


# ----------------------------------------------------------------------------- adaptive layer norm

import tests.test_oracle_adaln_pins as adaln_pins  # noqa: E402

ADALN_MUTATIONS = {
    "adaln_unbiased_variance": ("const double var = sum_dev / (double)C;",
                                "const double var = sum_dev / (double)(C - 1);"),
    "adaln_eps_outside_root": ("1.0 / sqrt(var + eps64)", "1.0 / sqrt(var) + eps64"),
    "adaln_scale_without_one": ("(1.0 + mod_value(scale", "(mod_value(scale"),
    "adaln_batch_modulo": ("const int64_t b = r / rows_per_batch;",
                           "const int64_t b = r % rows_per_batch;"),
    "adaln_shift_read_from_scale": ("+ mod_value(shift, mod_dtype, b * C + c);",
                                    "+ mod_value(scale, mod_dtype, b * C + c);"),
    "adaln_mean_not_subtracted": ("const double n = (decode16(xr[c], x_dtype) - mean) * inv;",
                                  "const double n = decode16(xr[c], x_dtype) * inv;"),
    "adaln_fp16_mod_decoded_as_bf16": ("return decode16(((const uint16_t*)table)[index], dtype);",
                                       "return decode16(((const uint16_t*)table)[index], QKR_O_BF16);"),
    "adaln_drop_last_in_mean": ("for (int64_t c = 0; c < C; ++c)\n            sum += ",
                                "for (int64_t c = 0; c + 1 < C; ++c)\n            sum += "),
}

ADALN_PIN_TESTS = [
    (adaln_pins.test_zero_modulation_is_torch_layer_norm, {"x_dtype": "bf16", "hidden": 64}),
    (adaln_pins.test_scale_minus_one_gives_shift_exactly, {}),
    (adaln_pins.test_constant_row_gives_shift_exactly, {}),
    (adaln_pins.test_output_moments, {}),
    (adaln_pins.test_affine_invariance, {}),
    (adaln_pins.test_brute_force, {"x_dtype": "bf16", "mod_dtype": "fp16", "hidden": 24}),
]


def _caught_adaln(variant) -> list:
    caught = []
    for fn, kw in ADALN_PIN_TESTS:
        try:
            with np.errstate(all="ignore"):
                fn(variant, **kw)
        except AssertionError:
            caught.append(fn.__name__)
    return caught


def test_unmutated_source_passes_every_adaln_pin():
    assert _caught_adaln(oracle.default()) == []


@pytest.mark.parametrize("name", sorted(ADALN_MUTATIONS))
def test_adaln_mutation_is_caught(tmp_path, name):
    old, new = ADALN_MUTATIONS[name]
    with open(oracle.SRC) as f:
        src = f.read()
    assert src.count(old) >= 1, "mutation anchor not found: " + name
    path = os.path.join(tmp_path, "mut.c")
    with open(path, "w") as f:
        f.write(src.replace(old, new, 1))
    lib = oracle.compile_source(path, os.path.join(tmp_path, "libmut.so"))
    assert _caught_adaln(oracle.Oracle(lib)), "no pin catches mutation " + name


# ----------------------------------------------------------------------------- group norm + SiLU

import tests.test_oracle_gn_pins as gn_pins  # noqa: E402

GN_MUTATIONS = {
    "gn_unbiased_variance": ("sqrt(sum_dev / (double)gsize + eps64)",
                             "sqrt(sum_dev / (double)(gsize - 1) + eps64)"),
    "gn_eps_outside_root": ("sqrt(sum_dev / (double)gsize + eps64)",
                            "sqrt(sum_dev / (double)gsize) + eps64"),
    "gn_channel_shifted": ("const int64_t c = c0 + e / spatial;",
                           "const int64_t c = c0 + (e / spatial + 1) % cg;"),
    "gn_group_rotated": ("const int64_t c0 = (q % groups) * cg;",
                         "const int64_t c0 = ((q + 1) % groups) * cg;"),
    "gn_silu_sign": ("oq[e] = y / (1.0 + exp(-y));", "oq[e] = y / (1.0 + exp(y));"),
    "gn_no_beta": ("+ mod_value(beta, param_dtype, c);", "+ 0.0;"),
    "gn_gamma_read_from_beta": ("* inv * mod_value(gamma, param_dtype, c)",
                                "* inv * mod_value(beta, param_dtype, c)"),
    "gn_mean_drops_last": ("for (int64_t e = 0; e < gsize; ++e)\n            sum += ",
                           "for (int64_t e = 0; e + 1 < gsize; ++e)\n            sum += "),
}

GN_PIN_TESTS = [
    (gn_pins.test_matches_torch_group_norm_silu, {"groups": 4, "x_dtype": "bf16",
                                                   "param_dtype": "fp32"}),
    (gn_pins.test_instance_norm_special_case, {}),
    (gn_pins.test_zero_gamma_and_constant_groups_give_silu_of_beta, {}),
    (gn_pins.test_silu_odd_part_identity, {}),
    (gn_pins.test_brute_force, {"x_dtype": "fp16", "param_dtype": "fp16"}),
]


def _caught_gn(variant) -> list:
    caught = []
    for fn, kw in GN_PIN_TESTS:
        try:
            with np.errstate(all="ignore"):
                fn(variant, **kw)
        except AssertionError:
            caught.append(fn.__name__)
    return caught


def test_unmutated_source_passes_every_gn_pin():
    assert _caught_gn(oracle.default()) == []


@pytest.mark.parametrize("name", sorted(GN_MUTATIONS))
def test_gn_mutation_is_caught(tmp_path, name):
    old, new = GN_MUTATIONS[name]
    with open(oracle.SRC) as f:
        src = f.read()
    assert src.count(old) >= 1, "mutation anchor not found: " + name
    path = os.path.join(tmp_path, "mut.c")
    with open(path, "w") as f:
        f.write(src.replace(old, new, 1))
    lib = oracle.compile_source(path, os.path.join(tmp_path, "libmut.so"))
    assert _caught_gn(oracle.Oracle(lib)), "no pin catches mutation " + name
