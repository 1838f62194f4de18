"""The pins must catch plausible mistakes in the oracle.

Each case plants one mistake in a copy of oracle/adq_oracle.c (a dropped
term, a misplaced epsilon, a wrong sign, constant, index, rounding mode,
packing order or validity rule), builds it on the CPU, routes the oracle
wrapper to it and runs the pin checks of test_oracle_pins.py until one
fails.  A mutant that passes every pin would mean the pins cannot tell it
from the formulas; the test fails in that case.
"""
import os
import subprocess

import pytest

import oracle
import test_oracle_lora_pins as lora_pins
import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle",
                   "adq_oracle.c")

MUTANTS = [
    ("beta dropped", "double b = beta ? oracle_storage_value(beta[j], dtype) : 0.0;",
     "double b = 0.0;"),
    ("epsilon outside the root", "sqrt(ss / (double)n + eps)", "sqrt(ss / (double)n) + eps"),
    ("sum instead of mean", "sqrt(ss / (double)n + eps)", "sqrt(ss + eps)"),
    ("x1 - x2", "v += oracle_storage_value(x2[off + j], dtype)",
     "v -= oracle_storage_value(x2[off + j], dtype)"),
    ("wrong divisor for the scale", "(float)(m / Q)", "(float)(m / (Q + 1.0))"),
    ("round half away from zero", "double c = nearbyint(v);", "double c = round(v);"),
    ("smooth scale ignored", "y[j] * oracle_storage_value(smooth[k][j], dtype) : y[j]",
     "y[j] : y[j]"),
    ("smooth scales swapped", "const uint16_t* smooth[2] = {smooth1, smooth2};",
     "const uint16_t* smooth[2] = {smooth2, smooth1};"),
    ("signed instead of absolute maximum", "if (fabs(in) > m) m = fabs(in);",
     "if (in > m) m = in;"),
    ("nibbles swapped", "(uint8_t)(lo | (hi << 4))", "(uint8_t)(hi | (lo << 4))"),
    ("smooth2 without smooth1 accepted", "if (has_s2 && !has_s1) return 0;", ""),
    ("mask[0] rule dropped", "if (has_s1 && !mask[0]) return 0;", ""),
    ("gamma indexed backwards", "oracle_storage_value(gamma[j], dtype)",
     "oracle_storage_value(gamma[n - 1 - j], dtype)"),
    ("xOut truncated", "double q = nearbyint(m / quantum);", "double q = floor(m / quantum);"),
    ("no clamp of the scale to float", "const float sc = (float)(m / Q);",
     "const double sc = m / Q;"),
    # AddLora
    ("lora: layer of weightA ignored", "const uint16_t* a = wa + ((g * l + layer) * h1) * rank;",
     "const uint16_t* a = wa + ((g * l + 0) * h1) * rank;"),
    ("lora: layer of weightB ignored", "wb + ((g * l + layer) * rank) * h2",
     "wb + ((g * l + 0) * rank) * h2"),
    ("lora: weightA read transposed", "oracle_storage_value(a[k * rank + r], dtype)",
     "oracle_storage_value(a[(k * rank + r) % h1 * rank + (k * rank + r) / h1], dtype)"),
    ("lora: weightB row and column swapped", "oracle_storage_value(bm[r * h2 + j], dtype)",
     "oracle_storage_value(bm[(r * h2 + j) % rank * h2 + (r * h2 + j) / rank], dtype)"),
    ("lora: y not accumulated", "double v = oracle_storage_value(yr[y_offset + j], dtype);",
     "double v = 0.0;"),
    ("lora: scale not applied", "v += z2 * s;", "v += z2;"),
    ("lora: scale kept in double", "const double s = (double)(float)scale;",
     "const double s = scale;"),
    ("lora: last adapter treated as none", "const int valid = g >= 0 && g < w;",
     "const int valid = g >= 0 && g < w - 1;"),
    ("lora: shrink skipped", "z = oracle_storage_value(xr[r], dtype);",
     "z = oracle_storage_value(xr[rank - 1 - r], dtype);"),
    # the consumer GEMM
    ("gemm: bias dropped", "(bias ? (double)bias[ni[t]] : 0.0)", "0.0"),
    ("gemm: activation scale ignored", "(double)a_scale[mi[t]]", "1.0"),
    ("gemm: first column's weight scale everywhere", "(double)w_scale[ni[t]]",
     "(double)w_scale[0]"),
    ("gemm: weights read back to front", "(int64_t)ar[j] * (int64_t)wr[j]",
     "(int64_t)ar[j] * (int64_t)wr[k - 1 - j]"),
    ("gemm: activations off by one", "(int64_t)ar[j] * (int64_t)wr[j]",
     "(int64_t)ar[(j + 1) % k] * (int64_t)wr[j]"),
    ("gemm: sum truncated to 16 bits", "if (sums) sums[t] = s;", "s = (int16_t)s; if (sums) sums[t] = s;"),
]


def _battery():
    checks = [("mask table", pins.test_mask_truth_table)]
    checks += [(f"worked row {c['name']}", lambda c=c: pins.test_worked_rows(c))
               for c in pins._CASES]
    checks += [
        ("closed forms", pins.test_closed_form_constant_and_one_hot_rows),
        ("int4 packing", pins.test_pack_int4_nibble_order),
        ("rms_norm vs torch", pins.test_rmsnorm_step_matches_torch_rms_norm),
        ("xOut bf16", lambda: pins.test_xout_is_correctly_rounded_sum("bf16")),
        ("xOut fp16", lambda: pins.test_xout_is_correctly_rounded_sum("fp16")),
    ]
    checks += [(f"brute force {s}", lambda s=s: pins.test_brute_force_tiny_rows(s))
               for s in range(6)]
    checks += [
        ("lora worked", lora_pins.test_lora_worked_example),
        ("lora worked without weightA", lora_pins.test_lora_worked_example_without_weight_a),
        ("lora closed form", lora_pins.test_lora_identity_expand_closed_form),
        ("lora copies", lora_pins.test_lora_columns_outside_slice_and_unassigned_rows_are_copied),
    ]
    checks += [(f"lora numpy {dt} {a}", lambda dt=dt, a=a: lora_pins.test_lora_matches_numpy_products(dt, a))
               for dt, a in (("bf16", True), ("fp16", True), ("bf16", False))]
    checks += [
        ("gemm worked", pins.test_gemm_worked_example),
        ("gemm numpy", pins.test_gemm_sums_match_numpy_integer_matmul),
        ("gemm closed form", pins.test_gemm_scaled_identity_closed_form),
    ]
    return checks


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(name, old, new, tmp_path):
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old}"
    mutant = tmp_path / "mutant.c"
    mutant.write_text(src.replace(old, new))
    lib = tmp_path / "libmutant.so"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", str(mutant), "-o",
                           str(lib), "-lm"])
    caught = None
    with oracle.use_library(str(lib)):
        for label, check in _battery():
            try:
                check()
            except Exception:  # an assertion, or a rejected call
                caught = label
                break
    assert caught is not None, f"no pin catches the mutant '{name}'"
