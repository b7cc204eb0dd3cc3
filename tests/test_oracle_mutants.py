"""Planted mistakes: each mutant of the oracle's C source must fail at least one pin.

The mutants are built on the CPU into a temporary directory from text edits of
oracle/sattn_oracle.c; the oracle itself is never modified.  This shows that
the pins in oracle_pins.py constrain every part of the definition (scale,
window bounds, GQA mapping, both sink semantics, normalisation, lse, gather,
merge weights).
"""
import os

import pytest

import oracle
from oracle_pins import ALL_PINS

MUTANTS = {
    "scale_dropped": ("logit[j] = scale * dot", "logit[j] = dot"),
    "exp_base2": ("double e = exp(logit[j] - m);", "double e = exp2(logit[j] - m);"),
    "gqa_modulo": ("const int g = h / G;", "const int g = h % Hkv;"),
    "window_left_off_by_one": ("0 : i - window_left;", "0 : i - window_left + 1;"),
    "window_right_off_by_one": ("L - 1 : i + window_right;", "L - 1 : i + window_right + 1;"),
    "global_position": ("const int64_t i = t - a;", "const int64_t i = t;"),
    "key0_on_first_window_key": ("(sink_mode == SINK_KEY0 && j == 0)", "(sink_mode == SINK_KEY0 && j == lo)"),
    "key0_sink_in_log2_units": ("(sink_mode == SINK_KEY0 && j == 0) ? (double)sinks[h]",
                                "(sink_mode == SINK_KEY0 && j == 0) ? (double)sinks[h] * 1.4426950408889634"),
    "value_reads_key": ("vr[n] = v + ", "vr[n] = k + "),
    "null_sink_not_in_denominator": ("if (null_sink) den += exp(sink - m);", ""),
    "lse_without_max": ("*lse = m + log(den);", "*lse = log(den);"),
    "indexed_key0_by_list_slot": ("(sink_mode == SINK_KEY0 && x == 0)", "(sink_mode == SINK_KEY0 && j == 0)"),
    "indexed_duplicates_accepted": ("dup |= sorted[j] == sorted[j - 1];", "(void)0;"),
    "merge_sink_dropped": ("if (null_sink) W += exp((double)sinks[h] - M);", ""),
    "merge_weight_inverted": ("double w = exp((double)part_lse[c * rows * H + rh] - M);",
                              "double w = exp(M - (double)part_lse[c * rows * H + rh]);"),
}


def _failures(lib):
    failed = []
    for pin in ALL_PINS:
        try:
            pin(lib)
        except (AssertionError, ValueError):
            failed.append(pin.__name__)
    return failed


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    with open(oracle.SRC) as f:
        src = f.read()
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    mutated = tmp_path / "mutant.c"
    mutated.write_text(src.replace(old, new))
    so = oracle.build(str(mutated), str(tmp_path / "libmutant.so"))
    lib = oracle.load(so)
    failed = _failures(lib)
    assert failed, f"mutant {name} passed every pin"


def test_unmutated_passes_all(tmp_path):
    so = oracle.build(oracle.SRC, str(tmp_path / "libclean.so"))
    assert _failures(oracle.load(so)) == []
