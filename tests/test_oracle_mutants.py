"""The pins are sensitive: plausible mistakes planted in copies of the oracle (compiled
here, on the CPU) must each make at least one pin fail."""
import os
import subprocess
import tempfile

import numpy as np
import pytest

import oracle
from tests import test_oracle_pins as P

# (name, original text, mutated text) applied to oracle.c
MUTANTS = [
    ("remap_multiplier", "return t + l * E;", "return t + l * S;"),
    ("remap_sentinel_dropped", "if (t < 0) return t;", "if (t < 0) return -1;"),
    ("remap_slot_range", "l < 0 || l >= S", "l < 0 || l > S"),
    ("align_unstable", "for (int64_t p = 0; p < numel; ++p) {\n            int32_t b = key[p];",
     "for (int64_t p = numel - 1; p >= 0; --p) {\n            int32_t b = key[p];"),
    ("align_overpad", "total += (count[b] + BM - 1) / BM * BM;",
     "total += (count[b] / BM + 1) * BM;"),
    ("align_sentinel_tag", "(b == V) ? -1 : (int32_t)b", "(int32_t)b"),
    ("align_pad_value", "sorted_ids[i] = (int32_t)numel;", "sorted_ids[i] = -1;"),
    ("shrink_drops_last_k", "for (int32_t k = 0; k < K; ++k)\n                    acc += load_elem(A",
     "for (int32_t k = 0; k < K - 1; ++k)\n                    acc += load_elem(A"),
    ("shrink_transposed_A", "load_elem(A, arow + k, dtype)",
     "load_elem(A, (int64_t)e * R * K + (int64_t)k * R + i, dtype)"),
    ("shrink_row_of_pair", "(p / row_div) * ld_x;\n            for (int32_t i = 0",
     "(p % row_div) * ld_x;\n            for (int32_t i = 0"),
    ("expand_slice", "const int32_t g = n / width;\n                const int64_t brow = ((int64_t)e",
     "const int32_t g = 0;\n                const int64_t brow = ((int64_t)e"),
    ("expand_scale_slot", "(double)scale[e / E]", "(double)scale[0]"),
    ("expand_truncates", "nearbyint(ldexp(a, -q))", "trunc(ldexp(a, -q))"),
    ("expand_sign", "acc += load_elem(B, brow + jj, dtype) * s[",
     "acc -= load_elem(B, brow + jj, dtype) * s["),
    ("rank_reads_past_end", "for (int32_t jj = 0; jj < rl; ++jj)",
     "for (int32_t jj = 0; jj <= rl && jj < r; ++jj)"),
    ("rank_zero_as_full", "return v < 0 ? 0 : (v > r ? r : v);",
     "return v <= 0 ? r : (v > r ? r : v);"),
    ("rank_shrink_ignored", "if (i % r >= rl) {", "if (0) {"),
    ("combine_reads_sentinel_rows", "if (t < 0 || t >= E) continue;  /* no local expert: no row */",
     "if (t >= E) continue;"),
    ("combine_weight_of_token", "(double)topk_weights[p] * load_elem(rows",
     "(double)topk_weights[m] * load_elem(rows"),
    ("combine_truncates", "((float *)y)[o] = (float)v;", "((float *)y)[o] = (float)(v * (1.0 - 1e-6));"),
    ("fused_scale_dropped", "row += (double)scale[l] * d;", "row += d;"),
    ("fused_weight_dropped", "acc += (double)topk_weights[p] * row;", "acc += row;"),
    ("fused_rank_ignored", "for (int32_t j = 0; j < rl; ++j) d +=",
     "for (int32_t j = 0; j < R; ++j) d +="),
    ("gemm_slot_ignored", "v = virtual_id(t, l, E, S);\n            rl",
     "v = t;\n            rl"),
    ("gemm_scale_dropped", "acc += (double)scale[l] * d;", "acc += d;"),
    ("gemm_row_of_pair", "const int64_t xrow = (p / row_div) * ld_x;\n        int32_t v = -1",
     "const int64_t xrow = (p % row_div) * ld_x;\n        int32_t v = -1"),
    ("gemm_rank_ignored", "rl = v >= 0 ? slot_rank(slot_ranks, l, r) : 0;",
     "rl = v >= 0 ? r : 0;"),
    ("fused_no_adapter_drops_base",
     "double row = load_elem(base, p * ld_base + n, dtype);\n"
     "                const int32_t v = virtual_id(t, lora_ids[m], E, S);",
     "const int32_t v = virtual_id(t, lora_ids[m], E, S);\n"
     "                if (v < 0) continue;\n"
     "                double row = load_elem(base, p * ld_base + n, dtype);"),
]


def _battery(lib):
    """Run every oracle pin against `lib`; return the names of the pins that failed."""
    failed = []
    cases = [
        ("bf16_literals", lambda: [P.test_bf16_literal_cases(lib, v, b) for v, b in [
            (1.0 + 2.0 ** -8, 0x3F80), (1.0 + 3 * 2.0 ** -8, 0x3F82), (2.0 ** -134, 0)]]),
        ("bf16_torch", lambda: P.test_bf16_matches_torch_on_float32_values(lib)),
        ("remap_cases", lambda: P.test_remap_worked_cases(lib)),
        ("remap_invariants", lambda: P.test_remap_invariants(lib)),
        ("align_bruteforce", lambda: P.test_align_matches_stable_argsort_bruteforce(lib)),
        ("align_inline", lambda: P.test_align_inline_remap_equals_remap_then_align(lib)),
        ("align_sentinel", lambda: P.test_align_sentinel_only_and_empty(lib)),
        ("identity_f32", lambda: P.test_delta_equals_per_pair_identity(lib, P.configs.C0)),
        ("identity_bf16", lambda: P.test_delta_equals_per_pair_identity(lib, P.SMALL_BF16)),
        ("gemm_chain", lambda: P.test_one_bucket_is_a_plain_gemm_chain(lib)),
        ("linearity", lambda: P.test_linearity_in_scale_and_zero_A(lib)),
        ("ranked_f32", lambda: P.test_ranked_delta_equals_full_rank_on_zeroed_weights(
            lib, P.RANKED[0])),
        ("ranked_bf16", lambda: P.test_ranked_delta_equals_full_rank_on_zeroed_weights(
            lib, P.RANKED[1])),
        ("combine_matvec", lambda: [P.test_combine_is_a_batched_matvec(lib, d)
                                    for d in ("f32", "bf16")]),
        ("combine_local", lambda: [P.test_combine_reads_only_local_pairs(lib, d)
                                   for d in ("f32", "bf16")]),
        ("fused_k1", lambda: [P.test_fused_combine_one_unit_slot_equals_expand(lib, c)
                              for c in P.FUSED]),
        ("fused_rows", lambda: [P.test_fused_combine_equals_combine_of_expanded_rows(lib, c)
                                for c in P.FUSED]),
        ("fused_base", lambda: [P.test_fused_combine_without_adapters_is_the_base_combine(
            lib, c) for c in P.FUSED]),
        ("fused_ranked", lambda: P.test_fused_combine_ranked_equals_full_rank_on_zeroed_weights(
            lib)),
        ("gemm_matvec", lambda: [P.test_base_gemm_is_a_per_pair_matvec(lib, c)
                                 for c in P.GEMM[:2]]),
        ("gemm_fused", lambda: [P.test_fused_gemm_reduces_to_its_parts(lib, c) for c in P.GEMM]),
    ]
    for name, fn in cases:
        try:
            fn()
        except (AssertionError, ValueError):
            failed.append(name)
    return failed


@pytest.fixture(scope="module")
def mutant_dir():
    with tempfile.TemporaryDirectory() as d:
        yield d


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(mutant_dir, name, old, new):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "oracle.c")).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not unique"
    path_c = os.path.join(mutant_dir, f"{name}.c")
    path_so = os.path.join(mutant_dir, f"{name}.so")
    open(path_c, "w").write(src.replace(old, new))
    subprocess.run(["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-fopenmp", "-o", path_so,
                    path_c, "-lm"], check=True)
    saved_lib, saved_path = oracle._lib, oracle._LIB
    try:
        oracle._lib, oracle._LIB = None, path_so
        failed = _battery(oracle)
    finally:
        oracle._lib, oracle._LIB = saved_lib, saved_path
    assert failed, f"mutant {name} passed every pin"


def test_unmutated_oracle_passes_battery():
    oracle.build()
    assert _battery(oracle) == []
