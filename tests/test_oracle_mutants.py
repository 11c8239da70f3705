"""Sensitivity of the oracle's pins: plausible mistakes planted in copies of
the oracle's C source (CPU only) must each fail at least one pin."""
import os
import subprocess

import pytest

import oracle
import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "pda_oracle.c")

MUTANTS = {
    "gqa_map_modulo": ("const int32_t g = h / G;", "const int32_t g = h % num_kv_heads;"),
    "last_page_full": ("if (i == cnt - 1)", "if (0)"),
    "last_valid_short": ("for (int32_t j = 0; j < valid; ++j)",
                         "for (int32_t j = 0; j < valid - 1; ++j)"),
    "scale_inverted": ("score[t] = acc * scale;", "score[t] = acc / scale;"),
    "no_max_shift": ("double w = exp(score[t] - M);", "double w = exp(score[t]);"),
    "sign_flip": ("double w = exp(score[t] - M);", "double w = exp(M - score[t]);"),
    "strides_swapped": ("(int64_t)j * tok + (int64_t)g * kvh", "(int64_t)j * kvh + (int64_t)g * tok"),
    "v_from_k": ("pool + v_base + rows[t]", "pool + k_base + rows[t]"),
    "dot_skips_d0": ("for (int32_t d = 0; d < head_dim; ++d) acc +=",
                     "for (int32_t d = 1; d < head_dim; ++d) acc +="),
    "no_normalise": ("L > 0.0 ? op[d] / L : 0.0", "L > 0.0 ? op[d] : 0.0"),
    "first_tile_only": ("for (int32_t t = 0; t < n_tiles; ++t)", "for (int32_t t = 0; t < 1; ++t)"),
    "mask_ignored": ("mask[(int64_t)s * mask_stride + pos] != 0", "1"),
    "mask_inverted": ("mask[(int64_t)s * mask_stride + pos] != 0", "mask[(int64_t)s * mask_stride + pos] == 0"),
    "mask_position_per_page": ("                ++pos;\n", ""),
    "q_head_swapped": ("q + ((int64_t)s * num_q_heads + h) * head_dim",
                       "q + ((int64_t)s * num_q_heads + (num_q_heads - 1 - h)) * head_dim"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_fails_a_pin(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    path = tmp_path / f"{name}.c"
    path.write_text(src.replace(old, new))
    so = tmp_path / f"lib{name}.so"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", str(so), str(path),
                    "-lm"], check=True)
    lib = oracle.load_library(str(so))

    def attend(**kw):
        return oracle.attend(**kw, lib=lib)

    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(attend)
        except (AssertionError, ValueError, FloatingPointError):
            failed.append(pin.__name__)
    try:
        oracle_pins.pin_tiled_merge(attend, oracle.merge)
    except (AssertionError, ValueError):
        failed.append("pin_tiled_merge")
    assert failed, f"mutant {name} passed every pin"
