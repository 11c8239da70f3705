"""Sensitivity of the oracle's pins: plausible mistakes planted in copies of
the oracle's C source (CPU only) must each fail at least one pin."""
import os
import subprocess

import pytest

import oracle
import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "pda_oracle.c")

MUTANTS = {
    "gqa_map_modulo": ("(sh % num_q_heads);\n            const int32_t g = h / G;",
                       "(sh % num_q_heads);\n            const int32_t g = h % num_kv_heads;"),
    "prefill_gqa_modulo": ("(si % q_len);\n            const int32_t g = h / G;",
                           "(si % q_len);\n            const int32_t g = h % num_kv_heads;"),
    "last_page_full": ("if (i == cnt - 1)", "if (0)"),
    "last_valid_short": ("for (int32_t j = 0; j < valid; ++j)",
                         "for (int32_t j = 0; j < valid - 1; ++j)"),
    "scale_inverted": ("score[t] = acc * scale;", "score[t] = acc / scale;"),
    "no_max_shift": ("double w = exp(score[t] - M);", "double w = exp(score[t]);"),
    "sign_flip": ("double w = exp(score[t] - M);", "double w = exp(M - score[t]);"),
    "strides_swapped": ("(int64_t)j * tok + (int64_t)g * kvh", "(int64_t)j * kvh + (int64_t)g * tok"),
    "v_from_k": ("vpool + rows[t]", "kpool + rows[t]"),
    "dot_skips_d0": ("for (int32_t d = 0; d < head_dim; ++d) acc +=",
                     "for (int32_t d = 1; d < head_dim; ++d) acc +="),
    "no_normalise": ("L > 0.0 ? op[d] / L : 0.0", "L > 0.0 ? op[d] : 0.0"),
    "first_tile_only": ("capacity);\n        const int32_t *list", "capacity);\n        if (t > 0) break;\n        const int32_t *list"),
    "mask_ignored": ("mask_row[pos] != 0", "1"),
    "mask_inverted": ("mask_row[pos] != 0", "mask_row[pos] == 0"),
    "mask_position_per_page": ("                ++pos;\n", ""),
    "q_head_swapped": ("q + ((int64_t)s * num_q_heads + h) * head_dim",
                       "q + ((int64_t)s * num_q_heads + (num_q_heads - 1 - h)) * head_dim"),
    "prefill_causal_strict": ("causal ? P - q_len + i :", "causal ? P - q_len + i - 1 :"),
    "prefill_top_left": ("causal ? P - q_len + i :", "causal ? (int64_t)i :"),
    "prefill_causal_ignored": ("causal ? P - q_len + i : INT64_MAX", "INT64_MAX"),
    "prefill_q_layout": ("q + (si * num_q_heads + h) * head_dim",
                         "q + (((int64_t)s * num_q_heads + h) * q_len + i) * head_dim"),
    "prefill_mask_query_shared": ("(int64_t)i * mask_q_stride", "(int64_t)0 * mask_q_stride"),
    "prefill_mask_seq_shared": ("mask + (int64_t)s * mask_seq_stride", "mask + (int64_t)0 * mask_seq_stride"),
    "rope_sin_sign": ("out[row + 2 * j] = re * cj - im * sj;", "out[row + 2 * j] = re * cj + im * sj;"),
    "rope_half_split": ("re = bf16_to_f64(x[row + 2 * j]), im = bf16_to_f64(x[row + 2 * j + 1]);",
                        "re = bf16_to_f64(x[row + j]), im = bf16_to_f64(x[row + j + half]);"),
    "rope_cos_sin_swapped": ("cj = (double)c[j], sj = (double)sn[j];", "cj = (double)sn[j], sj = (double)c[j];"),
    "rope_position_ignored": ("clamp_i32(positions[t], 0, max_positions - 1)",
                              "clamp_i32((int32_t)(t % max_positions), 0, max_positions - 1)"),
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

    def prefill(**kw):
        return oracle.prefill(**kw, lib=lib)

    def rope(*a, **kw):
        return oracle.rope(*a, **kw, lib=lib)

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
    for pin in oracle_pins.PREFILL_PINS:
        try:
            pin(prefill, attend)
        except (AssertionError, ValueError, FloatingPointError):
            failed.append(pin.__name__)
    for pin in oracle_pins.ROPE_PINS:
        try:
            pin(rope)
        except (AssertionError, ValueError, FloatingPointError):
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"
