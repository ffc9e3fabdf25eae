"""Planted mistakes in a copy of the oracle must each fail at least one pin.

The oracle source is copied to a temporary directory, one plausible slip is
written into the copy, the copy is compiled with gcc, and the pin suite of
tests/test_oracle_pins.py is run against it.  A mutant that every pin lets
through would mean the pins do not pin that part of the oracle.  Every mutant
stays in bounds (no out-of-range reads), so a mutant cannot crash the run.
"""
import os
import shutil
import subprocess

import pytest

import oracle
from tests import test_oracle_pins as pins

MUTANTS = {
    "head_map_modulo": ("long g = h / rep;", "long g = h % H_kv;"),
    "causal_off_by_one": ("long last = i + (n_k - n_q);", "long last = i + (n_k - n_q) - 1;"),
    "causal_top_left": ("long last = i + (n_k - n_q);", "long last = i;"),
    "dropped_scale": ("s[j] = scale * acc;", "s[j] = acc;"),
    "lse_without_max": ("*lse_out = m + log(z);", "*lse_out = log(z);"),
    "lse_log2": ("*lse_out = m + log(z);", "*lse_out = m + log2(z);"),
    "no_normalisation": ("for (j = first; j < n_visible; ++j) s[j] /= z;", ""),
    "exp_sign_flipped": ("s[j] = exp(s[j] - m);", "s[j] = exp(m - s[j]);"),
    "values_reversed": ("size_t row = kv_off + (size_t)j * (size_t)d;",
                        "size_t row = kv_off + (size_t)(n_visible - 1 - j) * (size_t)d;"),
    "max_is_first_score": ("if (s[j] > m) m = s[j];", "if (s[j] > m) m = m;"),
    "decode_reads_padding": ("kv_off, len, first, len, d, scale, s,", "kv_off, N_max, first, N_max, d, scale, s,"),
    "window_off_by_one": ("long f = i + (n_k - n_q) - w + 1;", "long f = i + (n_k - n_q) - w;"),
    "window_top_left": ("long f = i + (n_k - n_q) - w + 1;", "long f = i - w + 1;"),
    "window_ignored": ("if (w <= 0) return 0;", "return 0;"),
    "decode_window_off_by_one": ("long first = window > 0 && len > window ? len - window : 0;",
                                 "long first = window > 0 && len > window ? len - window + 1 : 0;"),
    "decode_window_ignored": ("long first = window > 0 && len > window ? len - window : 0;", "long first = 0;"),
    "empty_row_lse_zero": ("*lse_out = -INFINITY;", "*lse_out = 0.0;"),
}


def _pin_suite():
    """A fixed selection of the pins, each called with concrete arguments."""
    P = pins
    calls = []
    for causal in (False, True):
        for nq, nk in ((7, 7), (5, 9), (9, 5)):
            calls.append(lambda c=causal, a=nq, b=nk: P.test_probability_rows_sum_to_one(c, a, b))
            calls.append(lambda c=causal, a=nq, b=nk: P.test_zero_query_closed_form(c, a, b))
        for h, hk in ((8, 2), (6, 3), (4, 1)):
            calls.append(lambda c=causal, a=h, b=hk: P.test_gqa_equals_repeated_mha(a, b, c))
        calls.append(lambda c=causal: P.test_linear_in_v_and_shift_invariant(c))
        for shape in ((2, 4, 2, 33, 33, 16), (1, 8, 1, 17, 40, 8), (2, 6, 3, 40, 17, 12)):
            calls.append(lambda c=causal, s=shape: P.test_matches_torch_cpu_fp64(s, c))
        for shape in ((1, 2, 1, 3, 3, 2), (2, 4, 2, 2, 4, 3), (1, 3, 1, 4, 2, 2)):
            calls.append(lambda c=causal, s=shape: P.test_brute_force_tiny(s, c))
    calls += [P.test_causal_row_zero_and_single_key, P.test_one_dominant_key_at_extreme_scale, P.test_rows_with_no_visible_key,
              P.test_joint_key_value_permutation, P.test_scale_is_applied_to_scores,
              P.test_matches_torch_sdpa, P.test_decode_equals_single_query_prefill_and_split_merge,
              P.test_window_matches_pages_example, P.test_brute_force_tiny_window, P.test_decode_window]
    for nq, nk, w in ((9, 9, 3), (4, 11, 5), (11, 4, 2), (6, 6, 1)):
        calls.append(lambda a=nq, b=nk, c=w: P.test_window_zero_query_closed_form(a, b, c))
    return calls


def _build_mutant(tmp_path, name, old, new):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "attn_oracle.c")).read()
    assert old in src, f"mutant {name}: pattern not found in the oracle source"
    mutated = src.replace(old, new)
    d = tmp_path / name
    d.mkdir()
    c = d / "attn_oracle.c"
    c.write_text(mutated)
    so = d / "libmutant.so"
    subprocess.check_call(["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", str(c), "-o", str(so), "-lm"])
    return str(so)


def test_unmutated_oracle_passes_suite():
    for call in _pin_suite():
        call()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path, monkeypatch):
    old, new = MUTANTS[name]
    lib = oracle.load_library(_build_mutant(tmp_path, name, old, new))
    monkeypatch.setattr(oracle, "_lib", lib)
    caught = 0
    for call in _pin_suite():
        try:
            call()
        except (AssertionError, ValueError):
            caught += 1
    assert caught > 0, f"no pin catches mutant {name}"
    shutil.rmtree(tmp_path / name, ignore_errors=True)
