"""Mutation check of the oracle pins: plant one plausible mistake at a time in
a COPY of the oracle's C source (never in the oracle itself), build it, run the
pin battery against it in a child process, and require that some pin fails.

A mutant that survives means the pins have a blind spot.  Mutants are chosen
so that none reads or writes out of bounds.
"""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# (name, text in csa_oracle.c, replacement)
MUTANTS = [
    ("prev_rows_shifted", "rows[K] = own - r + i;", "rows[K] = own - r + i + (i + 1 < r);"),
    ("prev_half_uses_second_half", "colbase[K] = 0;", "colbase[K] = (coff - 1) * d;"),
    ("own_half_uses_first_half", "rows[K] = own + i;\n        colbase[K] = (coff - 1) * d;",
     "rows[K] = own + i;\n        colbase[K] = 0;"),
    ("first_block_mask_too_wide", "if (coff == 2 && b >= 1) {", "if (coff == 2 && b >= 2) {"),
    ("ape_position_reversed", "colbase[K] = (coff - 1) * d;\n        pos[K] = i;",
     "colbase[K] = (coff - 1) * d;\n        pos[K] = r - 1 - i;"),
    ("ape_dropped_f32", "+ ape[(int64_t)pos[k] * W + col];\n        v[k] = oracle_f32_from_bf16",
     "+ 0.0f * ape[(int64_t)pos[k] * W + col];\n        v[k] = oracle_f32_from_bf16"),
    ("ape_dropped_f64", "x[k] = score[rows[k] * W + col] + ape[(int64_t)pos[k] * W + col];",
     "x[k] = score[rows[k] * W + col];"),
    ("sum_skips_an_entry", "for (int k = 1; k < K; ++k) Z = Z + e[k];",
     "for (int k = 2; k < K; ++k) Z = Z + e[k];"),
    ("sum_stops_at_64_entries", "for (int k = 1; k < K; ++k) Z = Z + e[k];",
     "for (int k = 1; k < K && k < 64; ++k) Z = Z + e[k];"),
    ("acc_skips_first_entry", "for (int k = 0; k < K; ++k) acc = fmaf(e[k], v[k], acc);",
     "for (int k = 1; k < K; ++k) acc = fmaf(e[k], v[k], acc);"),
    ("acc_stops_at_64_entries", "for (int k = 0; k < K; ++k) acc = fmaf(e[k], v[k], acc);",
     "for (int k = 0; k < K && k < 64; ++k) acc = fmaf(e[k], v[k], acc);"),
    ("wrong_normaliser", "float R = 1.0f / Z;", "float R = 1.0f / (Z + e[0]);"),
    ("f64_unnormalised", "p[k] = p[k] / Z;", "p[k] = p[k] / (Z + 1.0);"),
    ("bwd_sign_f32", "float dsk = a * (v[k] - o);", "float dsk = a * (o - v[k]);"),
    ("bwd_sign_f64", "double dsk = a * (v[k] - o);", "double dsk = a * (o - v[k]);"),
    ("dkv_missing_dout", "dkv[slot] = oracle_bf16_from_f32(a);", "dkv[slot] = oracle_bf16_from_f32(e[k] * R);"),
    ("dape_position_reversed", "dape[(int64_t)pos[k] * W + col] += (double)ds",
     "dape[(int64_t)(r - 1 - pos[k]) * W + col] += (double)ds"),
    ("dape_f64_dropped_window_term", "dape[(int64_t)pos[k] * W + col] += dsk;",
     "dape[(int64_t)pos[k] * W + col] += (k ? dsk : 0.0);"),
    ("no_zero_fill", "memset(dkv, 0, sizeof(uint16_t) * (size_t)(T_cap * W));", ""),
    ("ln2_lo_sign", "LN2_LO = -0x1.05c610p-29f;", "LN2_LO = 0x1.05c610p-29f;"),
    ("taylor_digit", "0x1.111112p-7f", "0x1.111111p-7f"),
    ("taylor_dropped_term", "0x1.6c16c2p-10f, 0x1.a01a02p-13f};", "0x1.6c16c2p-10f, 0.0f};"),
    ("taylor_degree_six", "float q = EXP_C[7];\n    for (int n = 6;", "float q = EXP_C[6];\n    for (int n = 5;"),
    ("exp_clamp_too_high", "static const float EXP_Y_MIN = -104.0f;", "static const float EXP_Y_MIN = -40.0f;"),
    ("bf16_ties_away", "u += 0x7FFFu + ((u >> 16) & 1u);", "u += 0x8000u;"),
    ("bf16_truncate", "u += 0x7FFFu + ((u >> 16) & 1u);", ""),
    ("total_comp_ceil", "total += L / r;", "total += (L + r - 1) / r;"),
    ("max_not_subtracted", "e[k] = oracle_exp_f32(x[k] - m);", "e[k] = oracle_exp_f32(x[k] - m + 1.0f);"),
]

BATTERY = r"""
import sys
sys.path.insert(0, {root!r})
import oracle
oracle._LIB = {lib!r}
oracle._lib = None
from _pytest.outcomes import Skipped
from tests import test_oracle_pins as T
cases = [T.CASES[i] for i in (0, 2, 5, 9, 13, 17, 21, len(T.CASES) - 1)]
checks = [
    ("constants", T.test_exp_constants_are_their_exact_definitions, [()]),
    ("exp_special", T.test_exp_special_values, [()]),
    ("bf16", T.test_bf16_rounding_is_nearest_even, [()]),
    ("count", T.test_output_count_matches_block_count, [(c,) for c in cases]),
    ("tiny_count", T.test_tiny_workload_row_count, [()]),
    ("brute_f64", T.test_f64_oracle_matches_slot_side_brute_force, [(c,) for c in cases]),
    ("one_hot", T.test_one_hot_window_reproduces_kv_bitwise, [(c,) for c in cases]),
    ("uniform", T.test_uniform_scores_give_the_window_mean, [(c,) for c in cases]),
    ("zero_set", T.test_zero_set_is_the_never_consumed_set, [(c,) for c in cases]),
    ("f32_vs_f64", T.test_f32_oracle_within_bf16_rounding_of_f64, [(c,) for c in cases]),
    ("autograd", T.test_f64_oracle_matches_torch_autograd, [(c,) for c in cases[:4]]),
    ("exp_domain", T.test_exp_accuracy_over_domain, [()]),
]
for name, fn, arglists in checks:
    for args in arglists:
        try:
            fn(*args)
        except Skipped:
            pass
        except Exception as e:
            print("CAUGHT", name, type(e).__name__)
            sys.exit(3)
print("SURVIVED")
sys.exit(0)
"""


def _build_mutant(src: str, old: str, new: str, out_path: str):
    assert src.count(old) >= 1, old
    mutated = src.replace(old, new, 1)
    c_path = out_path[:-3] + ".c"
    with open(c_path, "w") as f:
        f.write(mutated)
    subprocess.check_call(["gcc", *oracle.CFLAGS, "-o", out_path, c_path, "-lm"])


def test_mutants_are_unique_edits():
    src = open(os.path.join(ROOT, "oracle", "csa_oracle.c")).read()
    for name, old, _ in MUTANTS:
        assert src.count(old) >= 1, name


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(name, old, new):
    src = open(os.path.join(ROOT, "oracle", "csa_oracle.c")).read()
    with tempfile.TemporaryDirectory() as tmp:
        lib = os.path.join(tmp, f"mut_{name}.so")
        _build_mutant(src, old, new, lib)
        code = BATTERY.format(root=ROOT, lib=lib)
        res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=600,
                             env={**os.environ, "OMP_NUM_THREADS": "4"})
    assert res.returncode == 3 and "CAUGHT" in res.stdout, (name, res.stdout[-500:], res.stderr[-2000:])
