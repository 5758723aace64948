"""The oracle's pins must catch plausible mistakes.

Each case plants one mistake in a copy of oracle.c (a dropped term, a wrong
sign, index or offset, a transposed operand), builds it on the CPU, binds it
in place of the real oracle and runs the pin tests: at least one must fail.
"""
import ctypes
import os
import subprocess

import pytest

import oracle
from tests import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTANTS = {
    "top_left_causal": ("int64_t n = kv_len - qo_len + i + 1;", "int64_t n = i + 1;"),
    "causal_off_by_one": ("int64_t n = kv_len - qo_len + i + 1;", "int64_t n = kv_len - qo_len + i;"),
    "scale_dropped": ("s[j] = sm_scale * dot;", "s[j] = dot;"),
    "lse_without_max": ("*lse_out = m + log(l);", "*lse_out = log(l);"),
    "exp_sign_flipped": ("s[j] = exp(s[j] - m);", "s[j] = exp(m - s[j]);"),
    "v_head_stride_dropped": ("int64_t voff = ((ks + j) * num_heads + h) * dvo;",
                              "int64_t voff = ((ks + j) * num_heads) * dvo;"),
    "k_sequence_offset_dropped": ("int64_t koff = ((ks + j) * num_heads + h) * dqk;",
                                  "int64_t koff = ((j) * num_heads + h) * dqk;"),
    "owner_search_strict": ("if ((int64_t)indptr[mid] <= t) lo = mid;",
                            "if ((int64_t)indptr[mid] < t) lo = mid;"),
    "merge_weights_swapped": ("double wa = exp(a - out_lse), wb = exp(b - out_lse);",
                              "double wa = exp(b - out_lse), wb = exp(a - out_lse);"),
    "merge_lse_without_max": ("double out_lse = mx + log(ea + eb);",
                              "double out_lse = log(ea + eb);"),
    "decompress_w_transposed": (
        "load_elem(w_uk, dtype, (int64_t)c * num_heads * dnope + (int64_t)h * dnope + d)",
        "load_elem(w_uk, dtype, (int64_t)d * num_heads * dnope + (int64_t)h * dnope + c)"),
    "absorbed_value_from_the_wrong_dims": ("int64_t latent_at = (ks + j) * dqk;",
                                           "int64_t latent_at = (ks + j) * dqk + (dqk - dvo);"),
    "absorbed_row_stride": ("int64_t row_at = (ks + j) * dqk;", "int64_t row_at = (ks + j) * dvo;"),
    "absorbed_head_stride_dropped": ("int64_t q_at = ((int64_t)t * num_heads + h) * dqk;",
                                     "int64_t q_at = ((int64_t)t * num_heads) * dqk;"),
    "decompress_rope_not_copied": ("k_row[dnope + d] = load_elem(k_rope, dtype, t * drope + d);",
                                   "k_row[dnope + d] = 0.0;"),
}

PIN_TESTS = [
    lambda: [pins.test_golden_prefill(c) for c in pins._golden()["prefill"]],
    lambda: [pins.test_golden_merge(c) for c in pins._golden()["merge"]],
    lambda: pins.test_single_visible_key_returns_that_value_row(pins.torch.float32),
    pins.test_equal_scores_average_the_visible_values,
    lambda: pins.test_brute_force_library_softmax(True, ([5, 0, 12, 3], [9, 4, 12, 1])),
    pins.test_per_head_data_is_not_mixed,
    pins.test_split_merge_equals_union,
    pins.test_batch_equals_sequences_alone,
    pins.test_chunked_prefill_equals_one_bottom_right_causal_call,
    pins.test_decompress_one_hot_latent_picks_weight_rows,
    pins.test_decompress_matches_float64_matmul,
    pins.test_absorbed_single_visible_key_returns_that_latent_row,
    pins.test_absorbed_equal_scores_average_the_latent_rows,
    lambda: pins.test_absorbed_brute_force_library_softmax(True),
]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path, monkeypatch):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    path = tmp_path / "mutant.c"
    path.write_text(src.replace(old, new))
    lib_path = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-fopenmp", str(path),
                    "-o", str(lib_path), "-lm"], check=True)
    monkeypatch.setattr(oracle, "_lib", oracle.bind(ctypes.CDLL(str(lib_path))))
    caught = 0
    for t in PIN_TESTS:
        try:
            t()
        except AssertionError:
            caught += 1
    assert caught > 0, f"no pin caught the planted mistake {name}"
