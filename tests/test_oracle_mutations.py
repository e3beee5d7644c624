"""Strength of the oracle's pins: plant plausible mistakes in copies of
oracle/ep_oracle.c (each rebuilt on its own) and require the pin tests to
reject every one.  The mistakes are planted in the oracle, on the CPU; the
unmodified oracle must pass the same battery."""
import os
import subprocess

import pytest

import oracle
from oracle import build as obuild
from tests import test_oracle_dedup as tdd
from tests import test_oracle_dispatch_combine as tdc
from tests import test_oracle_layout as tlay
from tests import test_oracle_numerics as tnum

# (name, text in ep_oracle.c, replacement) -- each text must occur exactly once
MUTANTS = [
    ("e4m3 ties away from zero (normal range)", "double m = nearbyint(ldexp(a, 3 - E));",
     "double m = round(ldexp(a, 3 - E));"),
    ("e4m3 ties away from zero (subnormal range)", "double m = nearbyint(ldexp(a, 9));",
     "double m = round(ldexp(a, 9));"),
    ("e4m3 subnormal threshold off by a binade", "if (a < ldexp(1.0, -6)) {",
     "if (a < ldexp(1.0, -7)) {"),
    ("e4m3 saturates only from 480 (464..480 become NaN)", "if (a >= 448.0)", "if (a >= 480.0)"),
    ("e4m3 sign dropped on zero", "return (uint8_t)(sign | (uint8_t)m);         /* m = 8 is 0x08 = 2^-6 */",
     "return (uint8_t)((m == 0.0 ? 0 : sign) | (uint8_t)m);"),
    ("bf16 ties rounded up", "if (discarded > 0x8000u || (discarded == 0x8000u && (hi & 1u)))",
     "if (discarded >= 0x8000u)"),
    ("bf16 truncation", "        hi = (uint16_t)(hi + 1u);", "        hi = hi;"),
    ("bad id does not set status", "if (e >= E) { st |= 1u; continue; }\n        expert_count[e] += 1;",
     "if (e >= E) { continue; }\n        expert_count[e] += 1;"),
    ("partition offset one expert late", "part_offset[p] = expert_offset[p * L];",
     "part_offset[p] = expert_offset[p * L + (p * L + 1 <= E ? 1 : 0)];"),
    ("slots filled from the back of each expert", "int32_t r = cursor[e]++;",
     "int32_t r = expert_offset[e] + expert_offset[e + 1] - 1 - cursor[e]++;"),
    ("src_pair tail not cleared", "for (int64_t r = N; r < npairs; ++r) src_pair[r] = -1;",
     "for (int64_t r = N; r < npairs; ++r) src_pair[r] = 0;"),
    ("scale amax/447", "float scale = amax / 448.0f;", "float scale = amax / 447.0f;"),
    ("amax without abs", "amax = fmaxf(amax, fabsf(oracle_bf16_to_f32(xb[j])));",
     "amax = fmaxf(amax, oracle_bf16_to_f32(xb[j]));"),
    ("reciprocal multiply instead of division",
     "oracle_e4m3fn_encode(oracle_bf16_to_f32(xb[j]) / scale);",
     "oracle_e4m3fn_encode(oracle_bf16_to_f32(xb[j]) * (1.0f / scale));"),
    ("combine in reverse k order", "            for (int k = 0; k < K; ++k) {\n                int32_t r = row_of_pair[(int64_t)t * K + k];\n                if (r < 0) continue;\n                acc = fmaf",
     "            for (int k = K - 1; k >= 0; --k) {\n                int32_t r = row_of_pair[(int64_t)t * K + k];\n                if (r < 0) continue;\n                acc = fmaf"),
    ("combine multiply then add",
     "acc = fmaf(w[(int64_t)t * K + k], oracle_bf16_to_f32(y[(int64_t)r * H + c]), acc);\n            }\n            out[",
     "acc = w[(int64_t)t * K + k] * oracle_bf16_to_f32(y[(int64_t)r * H + c]) + acc;\n            }\n            out["),
    ("combine uses weight k=0 for every k",
     "acc = fmaf(w[(int64_t)t * K + k], oracle_bf16_to_f32(y[(int64_t)r * H + c]), acc);\n            }\n            out[",
     "acc = fmaf(w[(int64_t)t * K], oracle_bf16_to_f32(y[(int64_t)r * H + c]), acc);\n            }\n            out["),
    ("dedup mask records k+1", "kmask[(int64_t)t * P + e / L] |= 1u << k;",
     "kmask[(int64_t)t * P + e / L] |= 1u << ((k + 1) % K);"),
    ("dedup rows token-descending", "        for (int t = 0; t < T; ++t) {\n            int64_t i = (int64_t)t * P + p;",
     "        for (int t = T - 1; t >= 0; --t) {\n            int64_t i = (int64_t)t * P + p;"),
    ("dedup level 2 sums in reverse partition order", "            for (int p = 0; p < P; ++p) {\n                int32_t r = tp_row[(int64_t)t * P + p];",
     "            for (int p = P - 1; p >= 0; --p) {\n                int32_t r = tp_row[(int64_t)t * P + p];"),
    ("dedup level 1 multiply then add",
     "                    acc = fmaf(w[(int64_t)t * K + k], oracle_bf16_to_f32(y[(int64_t)r * H + c]), acc);\n                }\n                partial",
     "                    acc = w[(int64_t)t * K + k] * oracle_bf16_to_f32(y[(int64_t)r * H + c]) + acc;\n                }\n                partial"),
    ("dedup level 1 keeps masked entries",
     "                    if (r < 0) continue;\n                    acc = fmaf(w[(int64_t)t * K + k]",
     "                    if (r < 0) r = 0;\n                    acc = fmaf(w[(int64_t)t * K + k]"),
]

BATTERY = [
    tnum.test_golden_points_oracle_and_table,
    tnum.test_round_trip_all_finite_codes,
    tnum.test_negative_mirror_and_random_patterns,
    tnum.test_bf16_rne_hand_values,
    tnum.test_bf16_rne_against_torch_random_patterns,
    tlay.test_hand_worked_example,
    tlay.test_brute_force_random_small_cases,
    lambda: tlay.test_invariants_on_workloads("tiny_4x1024"),
    lambda: tlay.test_invariants_on_workloads("masked_16384x4096_bf16"),
    tlay.test_all_masked_and_empty,
    tdc.test_hand_worked_block,
    lambda: tdc.test_fp8_dispatch_against_fp64_route("tiny_4x1024"),
    lambda: tdc.test_fp8_dispatch_against_fp64_route("ll_128x7168"),
    lambda: tdc.test_combine_bit_exact_at_full_size("ll_128x7168"),
    tdc.test_dequantisation_bound_and_zero_block,
    tdc.test_combine_exact_rational_small,
    tdc.test_identity_experts_return_dequantised_input,
    tdc.test_k1_unit_weight_returns_y_and_bf16_identity,
    tdd.test_hand_worked_example,
    tdd.test_brute_force_random_small_cases,
    lambda: tdd.test_two_level_combine_exact("ll_128x7168"),
    tdd.test_single_partition_tokens_equal_plain_combine,
    tdd.test_reduce_order_hand_worked,
    tdd.test_partial_with_every_entry_is_the_plain_combine,
]


def run_battery(stop_at_first=True):
    failed = 0
    for fn in BATTERY:
        try:
            fn()
        except Exception:
            failed += 1
            if stop_at_first:
                break
    return failed


def build_variant(src_text, out):
    c = out + ".c"
    open(c, "w").write(src_text)
    subprocess.run(["gcc", *obuild.CFLAGS, c, "-o", out, "-lm"], check=True, capture_output=True)
    return out


@pytest.fixture(scope="module")
def source():
    return open(obuild.SRC).read()


@pytest.mark.slow
def test_unmodified_oracle_passes_battery(source, tmp_path):
    oracle.use_library(build_variant(source, str(tmp_path / "orig.so")))
    try:
        assert run_battery(stop_at_first=False) == 0
    finally:
        oracle.use_library(None)


@pytest.mark.slow
@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(source, tmp_path, name, old, new):
    assert source.count(old) == 1, "mutation target not unique: " + name
    path = build_variant(source.replace(old, new), str(tmp_path / "mutant.so"))
    oracle.use_library(path)
    try:
        assert run_battery() > 0, "no pin caught: " + name
    finally:
        oracle.use_library(None)
