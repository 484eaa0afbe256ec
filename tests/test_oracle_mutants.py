"""Planted mistakes in the oracle must each fail at least one pin.

Every mutant is a copy of oracle/oracle.c with one plausible slip (a dropped
term, a wrong sign, index or operand), built with gcc into a temporary
library and run against the pin battery.  This shows the pins constrain
every part of the oracle, not only that the oracle passes them.
"""
import os
import subprocess

import pytest

import oracle
from oracle_pins import PINS

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "oracle.c")

MUTANTS = {
    "head_map_interleaved": ("const int g = h / M;", "const int g = h % J->Hkv;"),
    "scale_dropped": ("s[t] = J->scale * acc;", "s[t] = acc;"),
    "max_added_not_subtracted": ("s[t] = exp(s[t] - mx);", "s[t] = exp(s[t] + mx);"),
    "no_normalisation": ("for (int t = 0; t < n; ++t) s[t] /= z;", ";"),
    "keys_as_values": ("o[j] += p * widen(J->v,", "o[j] += p * widen(J->k,"),
    "one_token_too_many": ("const int n = J->lengths[b];", "const int n = J->lengths[b] < J->T_cap ? J->lengths[b] + 1 : J->lengths[b];"),
    "query_of_kv_head": ("((size_t)b * J->Hq + h) * (size_t)D", "((size_t)b * J->Hq + g) * (size_t)D"),
    "kv_head_ignored": ("((size_t)b * J->Hkv + g) * (size_t)J->T_cap", "((size_t)b * J->Hkv) * (size_t)J->T_cap"),
    "keys_transposed": ("widen(J->k, J->dtype, kvoff + (size_t)t * D + j)", "widen(J->k, J->dtype, kvoff + (size_t)j * J->T_cap + t)"),
    "values_transposed": ("widen(J->v, J->dtype, kvoff + (size_t)t * D + j)", "widen(J->v, J->dtype, kvoff + (size_t)j * J->T_cap + t)"),
    "bf16_widen_shift": ("<< 16;", "<< 15;"),
    "natural_exp_swapped_for_base2": ("s[t] = exp(s[t] - mx);", "s[t] = exp2(s[t] - mx);"),
    "last_token_dropped": ("for (int t = 0; t < n; ++t) {\n        const double p", "for (int t = 0; t + 1 < n; ++t) {\n        const double p"),
    "max_over_first_token_only": ("if (s[t] > mx) mx = s[t];", "if (0) mx = s[t];"),
}


def _passes_all(lib):
    failed = []
    for pin in PINS:
        try:
            pin(lib)
        except (AssertionError, ValueError, FloatingPointError):
            failed.append(pin.__name__)
    return failed


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique/absent"
    path = tmp_path / f"oracle_{name}.c"
    path.write_text(src.replace(old, new))
    lib_path = str(tmp_path / f"liboracle_{name}.so")
    oracle.build(str(path), lib_path)
    failed = _passes_all(oracle.load(lib_path))
    assert failed, f"mutant {name} passed every pin"


def test_unmutated_oracle_passes(tmp_path):
    lib_path = str(tmp_path / "liboracle_clean.so")
    oracle.build(SRC, lib_path)
    assert _passes_all(oracle.load(lib_path)) == []
