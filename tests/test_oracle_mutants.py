"""Planted mistakes in a copy of the oracle must each fail some pin.

Each mutant edits the oracle's source text on the CPU (the oracle module on
disk is untouched), then the pin tests of ``test_oracle_pins`` are re-run
against the mutant.  A mutant that no pin catches fails this test.
"""

import os
import types

import pytest

import tests.test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "specverify_oracle.py")

MUTANTS = {
    "ratio_transposed": ("ratio = P[x] / Q[x]", "ratio = Q[x] / P[x]"),
    "residual_sign": ("diff = P - Q", "diff = Q - P"),
    "accept_not_strict": ("if u[b, k] < alphas[k]:", "if u[b, k] <= alphas[k]:"),
    "cdf_not_strict": ("hit = t < C", "hit = t <= C"),
    "bonus_from_last_row": ("y, margin = icdf(P[nb], uf)", "y, margin = icdf(P[-1] if False else P[0], uf)"),
    "draft_row_shift": ("processed_distribution(widen_row(draft[b, k], dtype)",
                        "processed_distribution(widen_row(draft[b, (k + 1) % draft.shape[1]], dtype)"),
    "temperature_multiplies": ("np.exp((z[kept] - m) / temperature)", "np.exp((z[kept] - m) * temperature)"),
    "topk_off_by_one": ("np.partition(z, V - k)[V - k]", "np.partition(z, V - k - 1)[V - k - 1]"),
    "residual_from_next_row": ("r = residual(P[stop], Q[stop])", "r = residual(P[stop + 1], Q[stop])"),
    "scan_does_not_stop": ("            stop, path = k, PATH_REJECT\n            break",
                           "            stop, path = k, PATH_REJECT"),
    "eos_ignored": ("            if x == eos_id:", "            if x == eos_id and False:"),
    "beta_uses_max": ("return np.minimum(P, Q).sum()", "return np.maximum(P, Q).sum()"),
    "topp_margin_one_sided": ("            margin = min(margin, top_p - c[M - 1])",
                              "            margin = min(margin, margin)"),
    "topp_margin_unnormalised": ("        margin = c[M] - top_p\n", "        margin = running[M] - top_p\n"),
    "topp_margin_overflags": ("        margin = c[M] - top_p\n", "        margin = (c[M] - top_p) * 1e-9\n"),
    "topp_flag_window_narrow": ("        if min(topp_rows) < TOPP_FLAG_ABS:",
                                "        if min(topp_rows) < TOPP_FLAG_ABS * 1e-3:"),
    "topp_flag_pos_next": ("            flag_kind, flag_pos = FLAG_TOPP, k\n",
                           "            flag_kind, flag_pos = FLAG_TOPP, k + 1\n"),
    "bonus_topp_flag_ignored": ('res["topp_margin_rows"][b, nb] < TOPP_FLAG_ABS:',
                                'res["topp_margin_rows"][b, nb] < 0.0:'),
    "topp_flag_past_stop": ("    last_decided = min(stop, nb - 1)", "    last_decided = nb - 1"),
    "topp_margin_row_mixup": ('res["topp_margin_rows"][b, K + 1 + k] = info["topp_margin"]',
                              'res["topp_margin_rows"][b, k] = info["topp_margin"]'),
    "beta_rows_swapped": ("zd = widen_row(draft[b, k], dtype)\n            if not",
                          "zd = widen_row(draft[b, (k + 1) % draft.shape[1]], dtype)\n            if not"),
}

CHECKS = [
    "test_worked_example_exact_fractions",
    "test_worked_example_replay",
    "test_worked_example_bonus_and_strict_cdf",
    "test_sample_semantics_exact",
    "test_two_token_closed_form",
    "test_topk_brute_force_with_ties",
    "test_exhaustive_round_law_positionwise",
    "test_exhaustive_round_law_ragged_bonus_row",
    "test_strict_accept_never_takes_a_zero_probability_token",
    "test_eos_truncation_invariant",
    "test_acceptance_rate_worked_example",
    "test_acceptance_rates_equal_expected_acceptance_per_position",
    "test_topp_margin_exact_decimal",
    "test_topp_flag_marks_the_cut_inside_its_window",
    "test_topp_flag_on_the_bonus_row_and_not_past_the_stop",
]


def _mutant_module(old, new):
    with open(SRC, encoding="utf-8") as f:
        text = f.read()
    assert text.count(old) == 1, old
    mod = types.ModuleType("oracle_mutant")
    exec(compile(text.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


def _run_check(name):
    fn = getattr(pins, name)
    if name == "test_worked_example_replay":
        fn("f64", 1e-12)
    elif name == "test_acceptance_rates_equal_expected_acceptance_per_position":
        fn(0, 1.0)
    else:
        fn()


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_mutant_is_caught(mutant, monkeypatch):
    old, new = MUTANTS[mutant]
    monkeypatch.setattr(pins, "O", _mutant_module(old, new))
    caught = []
    for name in CHECKS:
        try:
            _run_check(name)
        except Exception:          # an assertion, or a crash the mutant causes
            caught.append(name)
    assert caught, f"no pin catches mutant {mutant}"


def test_unmutated_copy_passes_every_check(monkeypatch):
    monkeypatch.setattr(pins, "O", _mutant_module("import numpy as np", "import numpy as np"))
    for name in CHECKS:
        _run_check(name)
