"""Plant plausible mistakes in a copy of the oracle and check that the pins catch each one.

Each mutant is a textual edit of ``oracle/attn_oracle.c`` compiled into a temporary
library; the pin functions of ``test_oracle.py`` are then run against it and at least
one of them must fail.  This is evidence that the pins constrain every part of the
oracle (grouping, scale, max shift, normalisation, lengths, operands, merge, mask, codec).
"""
import importlib.util
import os

import pytest

import test_oracle as pins

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "attn_oracle.c")

MUTANTS = {
    "interleaved_groups": ("int kh = h / G;", "int kh = h % KH;"),
    "no_max_shift": ("double w = exp(s[j] - m);", "double w = exp(s[j]);"),
    "no_scale": ("return scale * acc;", "return acc;"),
    "no_normalise": ("dst[d] /= l;", "dst[d] /= 1.0;"),
    "length_off_by_one": ("0, seqlens[b], Hsz", "0, seqlens[b] - (seqlens[b] > 1), Hsz"),
    "values_from_keys": ("const uint16_t *vrow = vbase + (j0 + j) * Hsz;",
                         "const uint16_t *vrow = kbase + (j0 + j) * Hsz;"),
    "merge_sign": ("double f = exp(m[i] - M);", "double f = exp(M - m[i]);"),
    "merge_drops_l_weight": ("Lsum += l[i] * f;", "Lsum += l[i];"),
    "mask_excludes_diagonal": ("0, i + 1, Hsz", "0, i + (i == 0), Hsz"),
    "codec_shift": ("((uint32_t)bits) << 16", "((uint32_t)bits) << 15"),
    "transposed_q_index": ("attend_rows(q + bh * Hsz", "attend_rows(q + (bh % Hq) * Hsz"),
    "fp8_fnuz_bias": ("v = ldexp(1.0 + (double)m / 8.0, e - 7);", "v = ldexp(1.0 + (double)m / 8.0, e - 8);"),
    "fp8_no_subnormals": ("v = ldexp((double)m / 8.0, -6);", "v = 0.0;"),
    "fp8_sign_lost": ("return sign ? -v : v;", "return v;"),
    "fp8_v_scale_dropped": ("dst[d] += w * (v_scale * oracle_fp8_e4m3_to_f64(vb[j * Hsz + d]));",
                            "dst[d] += w * oracle_fp8_e4m3_to_f64(vb[j * Hsz + d]);"),
    "fp8_k_scale_dropped": ("(k_scale * oracle_fp8_e4m3_to_f64(kb[j * Hsz + d]))", "oracle_fp8_e4m3_to_f64(kb[j * Hsz + d])"),
    "multi_mask_off_by_one": ("int64_t last = (int64_t)seqlens[b] - gamma + t;", "int64_t last = (int64_t)seqlens[b] - gamma + t - 1;"),
    "multi_mask_top_left": ("int64_t last = (int64_t)seqlens[b] - gamma + t;", "int64_t last = t;"),
    "prefill_wrong_kv_head": ("const uint16_t *kb = k + ((int64_t)b * KH + kh) * ISL * Hsz;",
                              "const uint16_t *kb = k + ((int64_t)b * KH + (h % KH)) * ISL * Hsz;"),
}

PIN_CALLS = [
    (pins.test_bf16_codec_known_patterns, {}),
    (pins.test_single_key_returns_its_value, {}),
    (pins.test_two_keys_logistic_closed_form, {"k0": 2.0, "expect_w0": 1 / (1 + 2.718281828459045 ** -1.0)}),
    (pins.test_zero_query_gives_mean_of_values, {}),
    (pins.test_constant_values_return_the_constant, {}),
    (pins.test_identity_values_expose_weights_that_sum_to_one, {}),
    (pins.test_planted_huge_score_selects_its_value, {}),
    (pins.test_arbitrary_splits_merge_to_full_result, {"seed": 0}),
    (pins.test_gqa_equals_mha_with_contiguously_repeated_kv, {}),
    (pins.test_decode_matches_torch_sdpa_fp64, {"Hq": 8, "KH": 2, "Hsz": 64}),
    (pins.test_prefill_matches_torch_sdpa_causal_fp64, {}),
    (pins.test_prefill_row0_is_v0_and_rows_match_decode, {}),
    (pins.test_fp8_e4m3_known_codes, {}),
    (pins.test_fp8_e4m3_all_codes_match_torch, {}),
    (pins.test_fp8_decode_equals_bf16_decode_of_the_same_values, {"k_scale": 0.5, "v_scale": 4.0}),
    (pins.test_fp8_decode_closed_forms, {}),
    (pins.test_multi_gamma1_is_decode, {}),
    (pins.test_multi_equals_last_rows_of_causal_prefill, {"gamma": 4}),
    (pins.test_multi_first_draft_sees_the_prefix_only, {}),
]


def _mutant_module(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation anchor for {name} not found"
    msrc = tmp_path / f"attn_oracle_{name}.c"
    msrc.write_text(src.replace(old, new))
    spec = importlib.util.spec_from_file_location(f"oracle_mutant_{name}",
                                                  os.path.join(ROOT, "oracle", "__init__.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    mod._SRC = str(msrc)
    mod._LIB_PATH = str(tmp_path / f"liboracle_{name}.so")
    mod._lib = None
    mod.build()
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_mutant(tmp_path, name):
    old, new = MUTANTS[name]
    mod = _mutant_module(tmp_path, name, old, new)
    caught = []
    for fn, kw in PIN_CALLS:
        try:
            fn(mod, **kw)
        except (AssertionError, ValueError, FloatingPointError):
            caught.append(fn.__name__)
    assert caught, f"no pin caught mutant {name}"


def test_unmutated_copy_passes_all_pins(tmp_path):
    mod = _mutant_module(tmp_path, "identity", "#include <math.h>", "#include <math.h>")
    for fn, kw in PIN_CALLS:
        fn(mod, **kw)
