"""The oracle's pins must catch plausible mistakes: each case below plants
one mistake in a copy of oracle.c (a dropped term, a wrong index or bound, a
transposed operand, a wrong constant), builds it into its own library, points
the oracle at it and runs the pins that cover that function.  At least one
of them has to fail.  The mutants only change arithmetic or indices inside
the arrays' bounds, so a mutant cannot write out of bounds."""
import ctypes  # noqa: F401  (the oracle loads through ctypes)
import os
import subprocess

import pytest

import oracle
import test_oracle_pins as pins

C = pins.CASES

MUTANTS = [
    ("bf16 rounding: tie-to-even term dropped",
     "uint32_t r = u + 0x7FFFu + lsb;", "uint32_t r = u + 0x7FFFu;",
     [pins.test_bf16_rne_matches_torch_on_random_and_ties]),
    ("e4m3: saturates to the NaN code",
     "return sign | 0x7E;                 /* satfinite: +-448            */",
     "return sign | 0x7F;",
     [pins.test_e4m3fn_hand_values, pins.test_e4m3fn_matches_brute_force_nearest, pins.test_quant_block_hand_values]),
    ("e4m3: truncates instead of rounding",
     "double n = nearbyint(a / quantum);", "double n = floor(a / quantum);",
     [pins.test_e4m3fn_hand_values, pins.test_e4m3fn_matches_brute_force_nearest, pins.test_quant_block_hand_values]),
    ("e4m3: subnormal range boundary off by one binade",
     "    if (lead < -6)\n        lead = -6;", "    if (lead < -7)\n        lead = -7;",
     [pins.test_e4m3fn_hand_values, pins.test_e4m3fn_matches_brute_force_nearest]),
    ("e4m3 decode: subnormal quantum 2^-10",
     "v = ldexp((double)m, -9);", "v = ldexp((double)m, -10);",
     [pins.test_e4m3fn_decode_roundtrip_and_bound]),
    ("quantisation: inverse scale transposed",
     "float inv = 448.0f / a;", "float inv = a / 448.0f;",
     [lambda: pins.test_quant_block_properties("normal"), pins.test_quant_block_special_cases, pins.test_quant_block_hand_values]),
    ("quantisation: scale inverted",
     "float s = a / 448.0f;", "float s = 448.0f / a;",
     [lambda: pins.test_quant_block_properties("normal"), pins.test_quant_block_special_cases, pins.test_quant_block_hand_values]),
    ("layout: repeated ids not rejected",
     "} else if (e >= E || seen[e]) {", "} else if (e >= E) {",
     [lambda: pins.test_layout_and_slots_against_independent_definitions(C[3], "dirty")]),
    ("layout: partition index e % P",
     "is_token_in_partition[(size_t)t * P + e / epp] = 1;",
     "is_token_in_partition[(size_t)t * P + e % P] = 1;",
     [lambda: pins.test_layout_and_slots_against_independent_definitions(C[4], "clean")]),
    ("layout: invalid ids not counted",
     "                ok = 0;                               /* invalid         */\n                ninv++;",
     "                ok = 0;                               /* invalid         */",
     [lambda: pins.test_layout_and_slots_against_independent_definitions(C[3], "dirty")]),
    ("offsets: running term dropped",
     "off[e + 1] = off[e] + num_tokens_per_expert[e];", "off[e + 1] = num_tokens_per_expert[e];",
     [lambda: pins.test_layout_and_slots_against_independent_definitions(C[2], "clean")]),
    ("aligned offsets: rounded down",
     "off[e + 1] = off[e] + ((c + A - 1) / A) * A;", "off[e + 1] = off[e] + (c / A) * A;",
     [lambda: pins.test_aligned_offsets_closed_form(64), pins.test_layout_worked_example]),
    ("slots: wrong source token",
     "src_token[s] = t;", "src_token[s] = t > 0 ? t - 1 : 0;",
     [lambda: pins.test_layout_and_slots_against_independent_definitions(C[2], "clean")]),
    ("slots: capacity bound off by one",
     "if (s < capacity) {", "if (s < capacity - 1) {",
     [pins.test_dispatch_capacity_drops_rows]),
    ("static slots: row off by one",
     "slot[i] = (int32_t)e * cap + r;", "slot[i] = (int32_t)e * cap + r + (r + 1 < cap);",
     [lambda: pins.test_static_slots_against_stable_sort(128, 256, 8, 16, "clean"), pins.test_layout_worked_example]),
    ("FP8 input: scales of the previous token",
     "memcpy(scales + (size_t)r * nb, xs + (size_t)t * nb, sizeof(float) * (size_t)nb);",
     "memcpy(scales + (size_t)r * nb, xs + (size_t)(t > 0 ? t - 1 : 0) * nb, sizeof(float) * (size_t)nb);",
     [pins.test_fp8_input_dispatch_copies_codes_and_scales]),
    ("FP8 input: codes of the mirrored token",
     "memcpy(recv + (size_t)r * H, xq + (size_t)t * H, (size_t)H);",
     "memcpy(recv + (size_t)r * H, xq + (size_t)(T - 1 - t) * H, (size_t)H);",
     [pins.test_fp8_input_dispatch_copies_codes_and_scales]),
    ("dispatch: only the first block's scale copied",
     "memcpy(scales + (size_t)r * nb, s, sizeof(float) * (size_t)nb);",
     "memcpy(scales + (size_t)r * nb, s, sizeof(float));",
     [lambda: pins.test_dispatch_rows_are_the_source_rows(True)]),
    ("combine: accumulation dropped",
     "acc = fmaf(w[(size_t)t * K + k], oracle_bf16_to_f32(y[(size_t)r * H + j]), acc);",
     "acc = fmaf(w[(size_t)t * K + k], oracle_bf16_to_f32(y[(size_t)r * H + j]), 0.0f);",
     [pins.test_combine_pow2_weights_exact, pins.test_combine_within_one_ulp_of_exact_sum]),
    ("combine: weight index transposed",
     "acc = fmaf(w[(size_t)t * K + k], oracle_bf16_to_f32(y[(size_t)r * H + j]), acc);",
     "acc = fmaf(w[(size_t)k * T + t], oracle_bf16_to_f32(y[(size_t)r * H + j]), acc);",
     [pins.test_combine_pow2_weights_exact, pins.test_combine_within_one_ulp_of_exact_sum]),
    ("FP8 combine: scale of the wrong block",
     "scales[(size_t)r * nb + j / 128]", "scales[(size_t)r * nb + j % nb]",
     [pins.test_combine_fp8_single_pair_matches_torch_dequant, pins.test_layout_worked_example]),
    ("dispatch backward: running sum dropped",
     "acc = acc + oracle_bf16_to_f32(grad_recv[(size_t)r * H + j]);",
     "acc = oracle_bf16_to_f32(grad_recv[(size_t)r * H + j]);",
     [lambda: pins.test_dispatch_backward_is_the_adjoint_of_dispatch(33, 8, 3, 2, 16), pins.test_layout_worked_example]),
    ("combine backward: weight dropped from grad_y",
     "grad_y[(size_t)r * H + j] = oracle_bf16_rne(wk * oracle_bf16_to_f32(g[j]));",
     "grad_y[(size_t)r * H + j] = oracle_bf16_rne(oracle_bf16_to_f32(g[j]));",
     [lambda: pins.test_combine_backward_grad_y_is_the_adjoint_of_combine(40, 8, 3, 2, 16), pins.test_layout_worked_example]),
    ("combine backward: grad_w from the weight instead of y",
     "(double)oracle_bf16_to_f32(y[(size_t)r * H + j]);",
     "(double)wk;",
     [pins.test_combine_backward_grad_w_matches_finite_differences, pins.test_layout_worked_example]),
    ("dispatch backward: k loop reversed",
     "            for (int k = 0; k < K; ++k) {\n                int32_t r = slot[(size_t)t * K + k];\n"
     "                if (r < 0)\n                    continue;\n                acc = acc + oracle_bf16_to_f32(grad_recv",
     "            for (int k = K - 1; k >= 0; --k) {\n                int32_t r = slot[(size_t)t * K + k];\n"
     "                if (r < 0)\n                    continue;\n                acc = acc + oracle_bf16_to_f32(grad_recv",
     [pins.test_dispatch_backward_exact_fp32_chain_in_k_order]),
    ("FP8 combine: k loop reversed",
     "            for (int k = 0; k < K; ++k) {\n                int32_t r = slot[(size_t)t * K + k];\n"
     "                if (r < 0)\n                    continue;\n                float v = oracle_e4m3fn_to_f32",
     "            for (int k = K - 1; k >= 0; --k) {\n                int32_t r = slot[(size_t)t * K + k];\n"
     "                if (r < 0)\n                    continue;\n                float v = oracle_e4m3fn_to_f32",
     [lambda: pins.test_combine_fp8_exact_fp32_chain_in_k_order(False),
      lambda: pins.test_combine_fp8_exact_fp32_chain_in_k_order(True)]),
    ("FP8 combine: multiply and add rounded separately",
     "acc = fmaf(wk, v, acc);", "acc = acc + wk * v;",
     [lambda: pins.test_combine_fp8_exact_fp32_chain_in_k_order(True)]),
    ("combine backward: grad_w accumulated in fp32",
     "double dot = 0.0;", "float dot = 0.0f;",
     [pins.test_combine_backward_grad_w_is_the_exact_dot_rounded_once,
      pins.test_combine_backward_grad_w_wide_range_within_double_bound]),
    ("rank routing: destinations in descending order",
     "        for (int p = 0; p < P; ++p)\n            if (hit[p])",
     "        for (int p = P - 1; p >= 0; --p)\n            if (hit[p])",
     [lambda: pins.test_rank_routing_against_brute_force(50, 16, 4, 4, "clean"), pins.test_ep_worked_example]),
    ("pack metadata: local id not offset by the partition's first expert",
     "local_idx[(size_t)r * K + k] = local ? e - p * epp : -1;",
     "local_idx[(size_t)r * K + k] = local ? e - p : -1;",
     [lambda: pins.test_pack_metadata_against_brute_force(50, 16, 4, 4, "clean"), pins.test_ep_worked_example]),
    ("pack metadata: weights of experts elsewhere not zeroed",
     "local_w[(size_t)r * K + k] = local ? topk_weights[(size_t)t * K + k] : 0.0f;",
     "local_w[(size_t)r * K + k] = topk_weights[(size_t)t * K + k];",
     [lambda: pins.test_pack_metadata_against_brute_force(50, 16, 4, 4, "clean"), pins.test_ep_worked_example]),
    ("pack metadata: repeated ids taken as local",
     "int local = ok[k] && e / epp == p;",
     "int local = e >= 0 && e < E && e / epp == p;",
     [lambda: pins.test_pack_metadata_against_brute_force(200, 64, 6, 8, "dirty"), pins.test_ep_worked_example]),
]


@pytest.mark.parametrize("name,orig,new,checks", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_the_mutant(name, orig, new, checks, tmp_path, monkeypatch):
    src = open(oracle._SRC).read()
    assert src.count(orig) == 1, f"mutation site not unique: {orig!r}"
    mutated = tmp_path / "oracle.c"
    mutated.write_text(src.replace(orig, new))
    (tmp_path / "oracle.h").write_text(open(os.path.join(os.path.dirname(oracle._SRC), "oracle.h")).read())
    so = tmp_path / "liboracle_mutant.so"
    subprocess.run(["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
                    "-shared", "-o", str(so), str(mutated), "-lm"], check=True)
    monkeypatch.setattr(oracle, "LIB_PATH", str(so))
    monkeypatch.setattr(oracle, "_lib", None)
    caught = []
    for check in checks:
        try:
            check()
        except AssertionError:
            caught.append(getattr(check, "__name__", "check"))
    assert caught, f"no pin caught the mutant: {name}"
