"""The pins must catch plausible mistakes in the oracle (CPU only).

Each mutant is oracle.c with one deliberate slip (a dropped term, a flipped sign, a wrong
index or bound).  It is compiled into a temporary library, swapped in for the real oracle,
and the pin tests are run against it: at least one must fail.  The real oracle source is
never modified.
"""
from __future__ import annotations

import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import oracle
import test_oracle_kmean as kmn
import test_oracle_pins as pins
import test_oracle_pipeline as pipe
import test_oracle_vscale as vsc
from helpers import small

MUTANTS = {
    "centering_sign": ("float c = fabsf(v - m);", "float c = fabsf(v + m);"),
    "floor_dropped": ("out[(b * H + hh) * slots + j] = fmaxf(ORA_FLOOR, amax);",
                      "out[(b * H + hh) * slots + j] = amax;"),
    "used_fix_dropped": ("if (u < S && g == partial_live && hi > u) hi = u;", ""),
    "minmax_includes_padding": ("        if (hi > u) hi = u;\n", "\n"),
    "derive_min_side_sign": ("c = fmaxf(c, fmaxf(mx - m, m - mn));",
                             "c = fmaxf(c, fmaxf(mx - m, mn - m));"),
    "derive_min_side_dropped": ("c = fmaxf(c, fmaxf(mx - m, m - mn));",
                                "c = fmaxf(c, mx - m);"),
    "derive_toucher_off_by_one": ("lo < ORA_GROUP * g + ORA_GROUP && ORA_GROUP * g < hi",
                                  "lo <= ORA_GROUP * g + ORA_GROUP && ORA_GROUP * g <= hi"),
    "derive_boundary_index_swapped": ("int er = (g == first_group(r, L)) ? 0 : 1;",
                                      "int er = (g == first_group(r, L)) ? 1 : 0;"),
    "scale_divisor": ("q_amax[(b * H + hh) * slots + sl] / 127.0f",
                      "q_amax[(b * H + hh) * slots + sl] / 128.0f"),
    "clamp_bound": ("if (q < -127.0f) q = -127.0f;", "if (q < -128.0f) q = -128.0f;"),
    "round_half_away": ("float q = rintf(x / scale);", "float q = roundf(x / scale);"),
    "shard_grid_slot": ("int64_t sl = (rank * L + l) / ORA_GROUP - g0;",
                        "int64_t sl = l / ORA_GROUP;"),
    "pack_head_index": ("int64_t dst = ((b * L + l) * h + j) * D + d;",
                        "int64_t dst = ((b * h + j) * L + l) * D + d;"),
    "e4m3_truncates": ("float n = rintf(ldexpf(a, 3 - E));",
                       "float n = floorf(ldexpf(a, 3 - E));"),
    "e4m3_saturates_to_nan": ("if (a >= 448.0f) return sign | 0x7E;",
                              "if (a >= 448.0f) return sign | 0x7F;"),
    "e4m3_subnormal_step": ("float n = rintf(ldexpf(a, 9));", "float n = rintf(ldexpf(a, 8));"),
    "fp16_subnormal_exponent": ("mag = ldexpf((float)m, -24);", "mag = ldexpf((float)m, -25);"),
    "unpack_scale_source": ("int64_t s = ORA_GROUP * g / L;",
                            "int64_t s = (ORA_GROUP * g + ORA_GROUP - 1) / L;"),
    "unpack_v_tail": ("uint8_t vb = 0;", "uint8_t vb = 1;"),
    "unpack_v_transpose": ("v8[((b * D + d) * h + j) * spad + t] = vb;",
                           "v8[((b * h + j) * D + d) * spad + t] = vb;"),
    "slots_formula": ("(L + ORA_GROUP - 1) / ORA_GROUP + 1", "(L + ORA_GROUP - 1) / ORA_GROUP"),
    "v_scale_multiplies": ("vf = vf / v_scale[(b * H + hh) * D + d];",
                           "vf = vf * v_scale[(b * H + hh) * D + d];"),
    "v_scale_local_head": ("vf = vf / v_scale[(b * H + hh) * D + d];",
                           "vf = vf / v_scale[(b * H + j) * D + d];"),
    "v_scale_ignored": ("if (v_scale) vf = vf / v_scale[(b * H + hh) * D + d];", ""),
    "minmax_keeps_negative_zero": ("if (v == 0.0f) v = 0.0f;", ""),
    "kmean_divides_by_rows": ("float m = (float)(sum / (double)u);",
                              "float m = (float)(sum / (double)S);"),
    "kmean_sums_padding": ("for (int64_t t = 0; t < u; t++) {", "for (int64_t t = 0; t < S; t++) {"),
    "kmean_rank_major_rows": ("int64_t r = t / L, l = t % L;", "int64_t r = t % P, l = t / P;"),
    "kmean_binary32_sum": ("double sum = 0.0;", "float sum = 0.0f;"),
    "kmean_binary32_divide": ("float m = (float)(sum / (double)u);",
                              "float m = (float)sum / (float)u;"),
    "bf16_truncates": ("return (uint16_t)((u + 0x7FFFu + lsb) >> 16);",
                       "return (uint16_t)(u >> 16);"),
    "bf16_ties_away": ("return (uint16_t)((u + 0x7FFFu + lsb) >> 16);",
                       "return (uint16_t)((u + 0x8000u) >> 16);"),
    "unpack_source_rank_interleaved": ("const uint8_t* chunk = recv + (t / L) * cb;",
                                       "const uint8_t* chunk = recv + (t % P) * cb;"),
    "unpack_k_from_q_section": ("k8[((b * S + t) * h + j) * D + d] = (int8_t)chunk[sec + src];",
                                "k8[((b * S + t) * h + j) * D + d] = (int8_t)chunk[src];"),
    "unpack_scale_width_floor": ("int64_t W = (ns + ORA_GROUP - 1) / ORA_GROUP;",
                                 "int64_t W = ns / ORA_GROUP + (ns < ORA_GROUP);"),
    "unpack_k_scale_section": ("memcpy(&kv, chunk + 3 * sec + ssec + 4 * ((b * h + j) * slots + sl), 4);",
                               "memcpy(&kv, chunk + 3 * sec + 4 * ((b * h + j) * slots + sl), 4);"),
    "unpack_scale_slot_shift": ("int64_t sl = g - first_group(s, L);",
                                "int64_t sl = g - first_group(s, L) + (s > 0);"),
    "pack_k_scale_from_q": ("ks[(b * h + j) * slots + sl] = k_amax[(b * H + hh) * slots + sl] / 127.0f;",
                            "ks[(b * h + j) * slots + sl] = q_amax[(b * H + hh) * slots + sl] / 127.0f;"),
    "derive_mean_dropped": ("                        float m = mean ? elem(mean, (b * H + hh) * D + d, dtype) : 0.0f;\n                        float mn = gathered",
                            "                        float m = 0.0f;\n                        float mn = gathered"),
    "derive_last_toucher_only": ("best = fmaxf(best, c);", "best = c;"),
    "quant_reciprocal_multiply": ("float q = rintf(x / scale);", "float q = rintf(x * (1.0f / scale));"),
    "pack_mean_local_head": ("float kc = elem(k, src, dtype) - elem(mean, (b * H + hh) * D + d, dtype);",
                             "float kc = elem(k, src, dtype) - elem(mean, (b * H + j) * D + d, dtype);"),
}


def battery(first_failure_only: bool = False):
    """A quick subset of the pin tests.  Returns the names of those that failed (only the
    first one when first_failure_only: enough to know a mutant is caught)."""
    failed = []
    checks = [
        ("e4m3_table", lambda: pins.test_e4m3_ocp_table(None)),
        ("quant_ties", lambda: pins.test_quant_i8_ties_go_to_even(None)),
        ("decode_fp16", lambda: pins.test_input_decoding_matches_library(None, torch.float16)),
        ("worked_example", lambda: pipe.test_hand_worked_example(None)),
        ("padding_only", lambda: pipe.test_padding_only_slice_contributes_floor(None)),
        ("signed_zero_minmax",
         lambda: pipe.test_boundary_minmax_signed_zeros(None, torch.bfloat16)),
        ("only_partial_live", lambda: pipe.test_only_partial_live_group_changes(None, 195)),
        ("v_scale_hand", lambda: vsc.test_hand_worked_values(None)),
        ("v_scale_definition", lambda: vsc.test_v_scale_matches_definition(None, vsc.CASES[0])),
        ("k_mean_recipe", lambda: kmn.test_k_mean_against_exact_sum(None, (4, 2, 33, 4, 64),
                                                                    torch.bfloat16)),
        ("k_mean_recipe_fp16", lambda: kmn.test_k_mean_against_exact_sum(None, (2, 1, 100, 2, 64),
                                                                         torch.float16)),
        ("k_mean_wide_range",
         lambda: kmn.test_k_mean_wide_range_against_exact_sum(None, torch.bfloat16)),
        ("k_mean_workload", lambda: kmn.test_k_mean_matches_workload_recipe(None)),
        ("dtype_rounding_bf16",
         lambda: kmn.test_dtype_rounding_matches_library(None, torch.bfloat16)),
    ]
    for w in [small(B=2, P=4, L=100, H=8, D=64, used=301, scale_sequence=301, seed=1),
              small(P=2, L=65, H=4, D=128, dtype=torch.float16, used=100, seed=2),
              small(P=6, L=31, H=6, D=64, used=150, seed=3),
              small(P=8, L=200, H=8, D=64, seed=4),
              small(P=4, L=128, H=4, D=64, used=400, seed=5)]:
        checks.append((f"definition_{w.name}", lambda w=w: pipe.test_pipeline_matches_definition(
            None, w)))
    # the slowest check last: a caught mutant usually stops before it
    checks.append(("e4m3_exhaustive_bf16",
                   lambda: pins.test_e4m3_exhaustive_vs_brute_force_and_torch(None, torch.bfloat16)))
    for name, fn in checks:
        try:
            fn()
        except (AssertionError, ValueError, RuntimeError, IndexError):
            failed.append(name)
            if first_failure_only:
                break
    return failed


@pytest.fixture(scope="module")
def source():
    return open(oracle.SRC_PATH).read()


def test_real_oracle_passes_battery(olib):
    assert battery() == []


def _run_battery_with(lib_path: str) -> int:
    """Child process entry: swap in the library at lib_path, run the battery.  Exit 0 when
    a pin failed (mutant caught), 3 when every pin passed."""
    oracle._lib = oracle.lib(lib_path)
    failed = battery(first_failure_only=True)
    print("failed pins:", failed)
    return 0 if failed else 3


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(olib, source, tmp_path, name):
    old, new = MUTANTS[name]
    assert source.count(old) >= 1, f"mutation site for {name} not found"
    src = tmp_path / "mutant.c"
    src.write_text(source.replace(old, new, 1))
    so = oracle.build(out=str(tmp_path / "libmutant.so"), src=str(src))
    # a mutant may write out of bounds: run it in a child process; a crash also counts as
    # caught, since the pin run could not complete
    here = os.path.dirname(os.path.abspath(__file__))
    code = ("import sys; sys.path[:0] = [%r, %r]; import test_oracle_mutants as m; "
            "sys.exit(m._run_battery_with(%r))" % (here, os.path.dirname(here), so))
    proc = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                          timeout=600)
    assert proc.returncode != 3, f"mutant {name} passed every pin"
    assert proc.returncode == 0 or proc.returncode < 0, proc.stderr[-2000:]
