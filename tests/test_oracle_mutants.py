"""The oracle's pins must catch plausible mistakes.

Each mutant below plants one typical slip in a copy of the oracle source (a
wrong head map, an off-by-one window, a dropped scale or normalisation, a
transposed operand, a wrong layout ...), compiles it with gcc on the CPU and
runs the pin suite against it.  At least one pin has to fail for every mutant;
a mutant that survives means the pins leave that part of the oracle unchecked.
"""
import ctypes
import os
import subprocess

import pytest

import oracle
from tests import test_oracle_next as next_pins
from tests import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "gqa_oracle.c")

MUTANTS = {
    "tiled_head_map": ("return h / (hq / hkv);", "return h % hkv;"),
    "window_off_by_one": ("int64_t back = w - 1;", "int64_t back = w;"),
    "scale_dropped": ("scratch[j - lo] = scale * dot;", "scratch[j - lo] = dot;"),
    "no_max_subtraction": ("scratch[i] = exp(scratch[i] - m);", "scratch[i] = exp(scratch[i]);"),
    "value_from_key_lane": ("z[c] += p * vrow[j * (int64_t)d + c];",
                            "z[c] += p * krow[j * (int64_t)d + c];"),
    "feature_index_reversed": ("dot += q[c] * krow[j * (int64_t)d + c];",
                               "dot += q[c] * krow[j * (int64_t)d + (d - 1 - c)];"),
    "no_normalisation": ("scratch[i] /= sum;", "scratch[i] /= 1.0;"),
    "padding_not_zeroed": ("if (t >= nb) {", "if (t > nb) {"),
    "decode_misses_newest_key": ("int64_t t = nb - 1;", "int64_t t = (nb > 1) ? nb - 2 : 0;"),
    "causal_bound_exclusive": ("lo, t, d,\n", "lo, t - (t > lo), d,\n"),
    "batch_offset_ignored": ("const double *krow = k + ((int64_t)b * hkv + g) * C * d;\n"
                             "            const double *vrow = v + ((int64_t)b * hkv + g) * C * d;\n"
                             "            for (int t = 0;",
                             "const double *krow = k + ((int64_t)g) * C * d;\n"
                             "            const double *vrow = v + ((int64_t)g) * C * d;\n"
                             "            for (int t = 0;"),
    "output_layout_transposed": ("double *z = out + (((int64_t)b * T + t) * hq + h) * d;",
                                 "double *z = out + (((int64_t)b * hq + h) * T + t) * d;"),
}

PINS = [
    ("test_worked_example_printed_rows", True),
    ("test_worked_example_derived_rows", True),
    ("test_worked_example_head_map", True),
    ("test_head_map_table", False),
    ("test_window_start_table", False),
    ("test_prefill_matches_brute_force_exhaustive", False),
    ("test_decode_matches_brute_force_exhaustive", False),
    ("test_zero_scores_give_mean_of_permitted_values", False),
    ("test_single_permitted_key_returns_its_value_exactly", False),
    ("test_two_keys_closed_form", False),
    ("test_dominant_score_is_one_hot_and_finite", False),
    ("test_padded_rows_are_zero", False),
    ("test_decode_equals_prefill_last_row", False),
    ("test_decode_query_sees_all_previous_keys", False),
]


def _build_mutant(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    path = tmp_path / f"{name}.c"
    path.write_text(src.replace(old, new))
    lib = tmp_path / f"lib{name}.so"
    cmd = list(oracle.GCC_CMD)
    cmd[cmd.index("-o") + 1] = str(lib)
    cmd[cmd.index(oracle._SRC)] = str(path)
    subprocess.run(cmd, check=True)
    return str(lib)


# Mistakes in the functions for queries against a cached prefix, packed
# segments, the candidate commit and the rolling cache.  (Only mutants that
# keep every access in bounds: a mutant runs inside the test process.)
MUTANTS_NEXT = {
    # the pages' own cache mask bug: queries aligned to the top left
    "prefix_top_left_alignment": ("int64_t p = (int64_t)sb - tb + i;", "int64_t p = i;"),
    "prefix_segment_ignored": ("int64_t seg = segs ? segs[(int64_t)b * Tq + i] : 0;",
                               "int64_t seg = 0;"),
    "prefix_window_drops_segment": ("oracle_window_start(p, seg, window)",
                                    "oracle_window_start(p, 0, window)"),
    "ring_slot_shifted": ("int64_t slot = ring ? j % C : j;",
                          "int64_t slot = ring ? (j + 1) % C : j;"),
    "candidate_one_cell_late": ("int64_t slot = ring ? (int64_t)(nb - 1) % C : nb - 1;",
                                "int64_t slot = ring ? (int64_t)nb % C : (nb < C ? nb : nb - 1);"),
    "candidate_value_not_committed": ("memcpy(v + dst, vnew + src, sizeof(double) * d);", ""),
}

PINS_NEXT = [
    ("test_prefix_full_prompt_equals_prefill", False),
    ("test_prefix_one_token_equals_decode", False),
    ("test_prefix_printed_last_row", True),
    ("test_prefix_matches_dense_tril_mask", False),
    ("test_prefix_matches_brute_force", False),
    ("test_packed_segments_stated_cells", True),
    ("test_packing_equals_separate_sequences", False),
    ("test_candidate_commit_is_exact_and_local", False),
    ("test_candidate_is_seen_by_its_own_query", False),
    ("test_ring_equals_linear_window", False),
    ("test_ring_streaming_appends", False),
]

ORACLE_FUNCTIONS = ("oracle_kv_head_for_query", "oracle_window_start", "oracle_kv_cache_bytes",
                    "oracle_prefill", "oracle_decode", "oracle_expanded",
                    "oracle_attend_prefix", "oracle_decode_cache")


def _run_pins(name, old, new, module, pin_list, tmp_path, golden_dir, monkeypatch):
    path = _build_mutant(tmp_path, name, old, new)
    real = oracle.lib()
    mutant = ctypes.CDLL(path)
    for fn in ORACLE_FUNCTIONS:
        getattr(mutant, fn).argtypes = getattr(real, fn).argtypes
        getattr(mutant, fn).restype = getattr(real, fn).restype
    monkeypatch.setattr(oracle, "_lib", mutant)
    failed = []
    for pin, wants_golden in pin_list:
        f = getattr(module, pin)
        try:
            f(golden_dir) if wants_golden else f()
        except (AssertionError, oracle.OracleError):
            failed.append(pin)
    assert failed, f"mutant {name} survived every pin"


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path, golden_dir, monkeypatch):
    old, new = MUTANTS[name]
    _run_pins(name, old, new, pins, PINS, tmp_path, golden_dir, monkeypatch)


@pytest.mark.parametrize("name", sorted(MUTANTS_NEXT))
def test_next_pins_catch_mutant(name, tmp_path, golden_dir, monkeypatch):
    old, new = MUTANTS_NEXT[name]
    _run_pins(name, old, new, next_pins, PINS_NEXT, tmp_path, golden_dir, monkeypatch)
