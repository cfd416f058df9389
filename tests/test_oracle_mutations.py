"""The pins catch plausible mistakes in the oracle (CPU only).

Each case copies the oracle, the pin tests and the input generators into a
temporary directory, plants one mistake in the copy of the oracle's C source
(a wrong tie rule, scale divisor, source-position encoding, summation order,
padding, nibble order, ...), and runs the pin that should notice it.  The case
passes only if that pin fails on the mutated copy, so every pin named here is
shown to constrain the part of the oracle it claims to.  The repository's own
oracle is never modified.
"""

import os
import re
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# (name, text in oracle/mep_oracle.c, replacement, pin that must fail)
MUTATIONS = [
    ("e4m3_ties_to_odd",
     "else if (a == mid && (c & 1)) c = c - 1; /* tie: keep the even code */",
     "else if (a == mid && !(c & 1)) c = c - 1; /* tie: keep the even code */",
     "test_e4m3_encode_at_every_boundary"),
    ("e4m3_saturates_one_code_low",
     "while (c < 0x7E && oracle_e4m3_decode((uint8_t)c) < a) c++;",
     "while (c < 0x7D && oracle_e4m3_decode((uint8_t)c) < a) c++;",
     "test_e4m3_saturates_and_keeps_sign"),
    ("e4m3_subnormal_exponent",
     "if (e == 0) v = ldexp((double)m / 8.0, -6);",
     "if (e == 0) v = ldexp((double)m / 8.0, -7);",
     "test_e4m3_decode_table"),
    ("bf16_truncates", "if (a == vlo) pick = lo;", "if (1) pick = lo;",
     "test_bf16_rne_matches_torch"),
    ("scale_divisor_480", "float s = amax / 448.0f;", "float s = amax / 480.0f;",
     "test_dispatch_fp8_scales_and_codes"),
    ("amax_signed", "float v = fabsf(oracle_bf16_to_f32(x[b * 128 + i]));",
     "float v = oracle_bf16_to_f32(x[b * 128 + i]);", "test_quant_row_edge_blocks"),
    ("zero_block_loses_sign", "if (s == 0.0f) q[b * 128 + i] = signbit(xf) ? 0x80 : 0x00;",
     "if (s == 0.0f) q[b * 128 + i] = 0x00;", "test_quant_row_edge_blocks"),
    ("plan_duplicate_not_flagged", "if (e[jj] == e[j]) status |= ORACLE_ST_DUP_EXPERT;",
     "if (0) status |= ORACLE_ST_DUP_EXPERT;", "test_plan_status_bits"),
    ("plan_bad_index_not_flagged", "status |= ORACLE_ST_BAD_INDEX;", "(void)0;",
     "test_plan_status_bits"),
    ("src_token_pos_multiplier", "src_rank * (R * cap) + t; /* R4 */",
     "src_rank * cap + t; /* R4 */", "test_plan_hand_worked_example"),
    ("dispatch_weights_of_other_token",
     "memcpy(recv_w + row * k, w + (int64_t)t * k, sizeof(float) * (size_t)k);",
     "memcpy(recv_w + row * k, w + (int64_t)(T - 1 - t) * k, sizeof(float) * (size_t)k);",
     "test_dispatch_bf16_rows_are_copies"),
    ("carry_scales_dropped", "if (sd > 0) memcpy(s_tmp, xs + (int64_t)t * sd,",
     "if (0) memcpy(s_tmp, xs + (int64_t)t * sd,", "test_carry_copies_bytes_and_scale_rows"),
    ("combine_unfused",
     "acc = fmaf(w[(int64_t)t * k + j], oracle_bf16_to_f32(y[row * H + h]), acc);",
     "acc = acc + w[(int64_t)t * k + j] * oracle_bf16_to_f32(y[row * H + h]);",
     "test_combine_is_fused_chain_in_top_k_order"),
    ("combine_reversed_order",
     "for (int32_t j = 0; j < k; j++) {\n        int32_t s = slot[",
     "for (int32_t j = k - 1; j >= 0; j--) {\n        int32_t s = slot[",
     "test_combine_is_fused_chain_in_top_k_order"),
    ("combine_weight_of_other_position",
     "acc = fmaf(w[(int64_t)t * k + j], oracle_bf16_to_f32(y[row * H + h]), acc);",
     "acc = fmaf(w[(int64_t)t * k + (k - 1 - j)], oracle_bf16_to_f32(y[row * H + h]), acc);",
     "test_combine_top1_unit_weight_and_one_hot"),
    ("expert_major_no_padding",
     "em_offsets[e + 1] = em_offsets[e] + ((n + 127) / 128) * 128;",
     "em_offsets[e + 1] = em_offsets[e] + n;", "test_expert_major_overflow_status"),
    ("expert_major_descending_slots", "for (int32_t s = 0; s < recv_counts[r]; s++) {",
     "for (int32_t s = recv_counts[r] - 1; s >= 0; s--) {", "test_standard_moe_by_brute_force"),
    ("expert_major_local_src_pos", "em_src_pos[dst] = pos;",
     "em_src_pos[dst] = pos - src_rank * (R * cap);", "test_expert_major_layout"),
    ("combine_em_reversed_order",
     "for (int32_t j = 0; j < k; j++) {\n        int32_t row = tok_em_row[",
     "for (int32_t j = k - 1; j >= 0; j--) {\n        int32_t row = tok_em_row[",
     "test_expert_major_combine_is_fused_chain_in_top_k_order"),
    ("e2m1_ties_to_odd", "(c & 1)) c = c - 1;\n  }", "!(c & 1)) c = c - 1;\n  }",
     "test_e2m1_encode_matches_brute_force"),
    ("mx_exponent_off_by_one", "se = ex - 1 - 2;", "se = ex - 2;",
     "test_mx4_exact_blocks_round_trip"),
    ("mx_nibble_order", "q[(b * 32 + i) / 2] = (uint8_t)(c0 | (c1 << 4));",
     "q[(b * 32 + i) / 2] = (uint8_t)(c1 | (c0 << 4));", "test_mx4_exact_blocks_round_trip"),
    ("convert_all_ranks", "if (e / epr != r) continue; /* the expert lives on another rank */",
     "(void)0; /* the expert lives on another rank */", "test_convert_combine_hand_worked_example"),
    ("convert_unweighted",
     "acc = fmaf(recv_w[row * k + j], oracle_bf16_to_f32(y_em[em_of_j[j] * H + h]), acc);",
     "acc = fmaf(1.0f, oracle_bf16_to_f32(y_em[em_of_j[j] * H + h]), acc);",
     "test_convert_combine_hand_worked_example"),
    ("convert_unfused",
     "acc = fmaf(recv_w[row * k + j], oracle_bf16_to_f32(y_em[em_of_j[j] * H + h]), acc);",
     "acc = acc + recv_w[row * k + j] * oracle_bf16_to_f32(y_em[em_of_j[j] * H + h]);",
     "test_convert_combine_input_is_fused_chain_per_rank"),
    ("convert_reversed_order",
     "for (int32_t j = 0; j < k; j++) {\n          if (em_of_j[j] < 0) continue;",
     "for (int32_t j = k - 1; j >= 0; j--) {\n          if (em_of_j[j] < 0) continue;",
     "test_convert_combine_input_is_fused_chain_per_rank"),
    ("convert_repeated_expert_twice", "if (!first) continue; /* a repeated expert has one row */",
     "(void)first; /* a repeated expert has one row */",
     "test_convert_then_rank_sum_equals_expert_major_combine_on_exact_data"),
    ("convert_rank_local_source", "if (em_src_pos[i] == pos) { em_of_j[j] = i; break; }",
     "if (em_src_pos[i] == pos % cap) { em_of_j[j] = i; break; }",
     "test_convert_combine_hand_worked_example"),
    ("rank_sum_every_position", "if (first) row_of_j[j] = (int64_t)r * cap + s;",
     "row_of_j[j] = (int64_t)r * cap + s;", "test_convert_combine_hand_worked_example"),
    ("rank_sum_reversed_order",
     "for (int32_t j = 0; j < k; j++) {\n        if (row_of_j[j] < 0) continue;",
     "for (int32_t j = k - 1; j >= 0; j--) {\n        if (row_of_j[j] < 0) continue;",
     "test_combine_rank_sum_adds_rank_rows_in_first_position_order"),
]


def _mutated_copy(base, name, old, new):
    src = open(os.path.join(ROOT, "oracle", "mep_oracle.c")).read()
    assert src.count(old) == 1, f"{name}: the text to mutate occurs {src.count(old)} times"
    d = os.path.join(base, name)
    os.makedirs(os.path.join(d, "oracle"))
    os.makedirs(os.path.join(d, "tests"))
    for f in ("__init__.py", "oracle.py"):
        shutil.copy(os.path.join(ROOT, "oracle", f), os.path.join(d, "oracle", f))
    with open(os.path.join(d, "oracle", "mep_oracle.c"), "w") as f:
        f.write(src.replace(old, new))
    for f in ("conftest.py", "test_oracle_pins.py"):
        shutil.copy(os.path.join(ROOT, "tests", f), os.path.join(d, "tests", f))
    shutil.copytree(os.path.join(ROOT, "tests", "golden"), os.path.join(d, "tests", "golden"))
    shutil.copytree(os.path.join(ROOT, "synthetic"), os.path.join(d, "synthetic"),
                    ignore=shutil.ignore_patterns("__pycache__"))
    return d


def _run_pin(d, pin):
    r = subprocess.run([sys.executable, "-m", "pytest", f"tests/test_oracle_pins.py::{pin}",
                        "-q", "-p", "no:cacheprovider"], cwd=d, capture_output=True, text=True,
                       timeout=600, env={**os.environ, "OMP_NUM_THREADS": "1"})
    return r.returncode, r.stdout + r.stderr


def test_every_planted_mistake_fails_its_pin(tmp_path):
    names = [m[0] for m in MUTATIONS]
    assert len(set(names)) == len(names)
    dirs = [_mutated_copy(str(tmp_path), n, old, new) for n, old, new, _ in MUTATIONS]
    with ThreadPoolExecutor(max_workers=min(6, os.cpu_count() or 1)) as ex:
        results = list(ex.map(_run_pin, dirs, [m[3] for m in MUTATIONS]))
    missed = []
    for (name, _, _, pin), (rc, out) in zip(MUTATIONS, results):
        summary = out.strip().splitlines()[-1] if out.strip() else ""
        # a pin failure (exit status 1 with failed tests), not a build or collection error
        if not (rc == 1 and re.search(r"\b\d+ failed\b", summary) and "error" not in summary):
            missed.append(f"{name} -> {pin}: rc={rc}: {summary}")
    assert not missed, "mutations the pins did not catch:\n" + "\n".join(missed)

