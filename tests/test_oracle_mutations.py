"""Planted mistakes in copies of the oracle must each fail at least one pin.

Every mutation below is a plausible slip in a hand-written attention loop nest (a dropped
term, a wrong index, a wrong operand, a missing normalisation).  Each altered copy of
oracle/attn_oracle.c is compiled on the CPU into a temporary library and run through the
pins of tests/oracle_pins.py; the test passes only if some pin rejects it.
"""
import os

import pytest

import oracle
from tests import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "attn_oracle.c")

MUTATIONS = {
    "no_running_max": ("if (s[j - first] > m) m = s[j - first];", "(void)m;"),
    "no_max_subtraction": ("const double p = exp(s[j - first] - m);", "const double p = exp(s[j - first]);"),
    "gqa_modulo_map": ("const int64_t g = h / (Hq / Hkv);", "const int64_t g = h % Hkv;"),
    "strict_causal": ("const int64_t last = causal ? i : n - 1;", "const int64_t last = causal ? i - 1 : n - 1;"),
    "lse_without_max": ("*lse = m + log(l);", "*lse = log(l);"),
    "dropped_alpha": ("s[j - first] = alpha * dot;", "s[j - first] = dot;"),
    "k_as_value": ("const double* vrow = v + ((start + j) * Hkv + g) * d;",
                   "const double* vrow = k + ((start + j) * Hkv + g) * d;"),
    "no_normalisation": ("for (int64_t c = 0; c < d; ++c) o_row[c] /= l;", ""),
    "dropped_last_key": ("for (int64_t j = first; j <= last; ++j) {\n    const double p",
                         "for (int64_t j = first; j < last; ++j) {\n    const double p"),
    "query_from_key_head": ("const double* qrow = q + (t * Hq + h) * d;",
                            "const double* qrow = q + (t * Hq + g) * d;"),
    "sequence_end_ignored": ("const int64_t n = cu[b + 1] - start;", "const int64_t n = cu[nseq] - start;"),
    "window_off_by_one": ("const int64_t lo = i - window + 1;", "const int64_t lo = i - window;"),
    "sequence_search_takes_first_of_equal_offsets": (
        "    if (cu[mid] <= t) lo = mid; else hi = mid - 1;\n  }\n  return lo;",
        "    if (cu[mid] <= t) lo = mid; else hi = mid - 1;\n  }\n  while (lo > 0 && cu[lo - 1] == cu[lo]) --lo;\n  return lo;"),
    "window_ignored": ("const int64_t first = (window > 0 && lo > 0) ? lo : 0;", "const int64_t first = 0;"),
    "window_from_sequence_start": ("const int64_t first = (window > 0 && lo > 0) ? lo : 0;",
                                   "const int64_t first = (window > 0 && lo > 0) ? lo - (int64_t)(start > 0) : 0;"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, tmp_path):
    old, new = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    mutated = tmp_path / "mutated.c"
    mutated.write_text(src.replace(old, new))
    so = oracle.compile_source(str(mutated), str(tmp_path / "libmutated.so"))
    lib = oracle.OracleLib(so)
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(lib)
        except (AssertionError, ValueError, IndexError):
            failed.append(pin.__name__)
    assert failed, f"no pin caught the planted mistake {name}"
