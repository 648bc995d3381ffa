"""The algorithmic byte model behind the roofline's `achieved` (bench.py), pinned on the CPU:
the weight bytes per touched virtual expert against the per-expert sizes written out from
the layer shapes (a 30B-A3B-shaped layer at rank 32: gate_up A 64 x 2048 and B 1536 x 32,
down A 32 x 768 and B 2048 x 32, bf16), the split of a stage into its two launches, and
the terms that scale with pairs, tokens and touched experts."""
import pytest

import bench
from virtual_expert_routed_amd import configs


def stats(P=160, D=147, T=23, blocks=148):
    return {"P": P, "D": D, "T": T, "valid_blocks": blocks}


def weight_bytes_per_expert(cfg):
    # the stage bytes at one touched expert minus those at none
    one = sum(bench.stage_bytes(cfg, st, stats(P=0, D=1, T=0, blocks=0)) for st in cfg.stages)
    none = sum(bench.stage_bytes(cfg, st, stats(P=0, D=0, T=0, blocks=0)) for st in cfg.stages)
    return one - none


@pytest.mark.parametrize("cfg,expected", [
    (configs.C1, (64 * 2048 + 1536 * 32 + 32 * 768 + 2048 * 32) * 2),   # 540,672
    (configs.C2, 540672),
    (configs.C3, 540672),
    (configs.C4, (128 * 4096 + 3072 * 64 + 64 * 1536 + 4096 * 64) * 2),  # 2,162,688
    (configs.C0, (8 * 64 + 32 * 8) * 4),                                 # fp32, one stage
])
def test_weight_bytes_per_touched_expert(cfg, expected):
    assert weight_bytes_per_expert(cfg) == expected


@pytest.mark.parametrize("cfg", [configs.C0, configs.C1, configs.C4], ids=lambda c: c.name)
def test_stage_is_its_two_launches_without_s_and_one_copy_of_the_routing(cfg):
    s = stats()
    for st in cfg.stages:
        routing = 4 * (s["P"] + s["valid_blocks"])
        both = bench.shrink_bytes(cfg, st, s) + bench.expand_bytes(cfg, st, s)
        assert bench.stage_bytes(cfg, st, s) == both - 8 * s["P"] * st.R - routing


def test_terms_scale_with_pairs_tokens_and_experts():
    cfg = configs.C1
    gu, down = cfg.stages
    base = stats()
    # gate_up reads token rows: one more token adds one x row of K bf16
    assert (bench.stage_bytes(cfg, gu, stats(T=24)) - bench.stage_bytes(cfg, gu, base)
            == gu.K * 2)
    # down reads pair rows: one more pair adds its h row, its out row read and written, and
    # its routing entry
    assert (bench.stage_bytes(cfg, down, stats(P=161)) - bench.stage_bytes(cfg, down, base)
            == down.K * 2 + 2 * down.N * 2 + 4)
    # the whole C1 layer at about 159 pairs over 146 touched experts (the estimate made for
    # this workload from its generator): about 81.5 MB
    est = stats(P=159, D=146, T=23, blocks=147)
    total = sum(bench.stage_bytes(cfg, st, est) for st in cfg.stages)
    assert 81.0e6 < total < 82.0e6


def test_code_hash_ignores_comments_and_layout_only():
    # the counter summaries stay valid across a rewording, and only then
    base = "int f(int a) {\n  return a + 1;  // one more\n}\n/* note */\n"
    reworded = "int f(int a) {   // the successor\n  return a + 1;\n}\n/* other\n note */"
    changed = "int f(int a) {\n  return a + 2;  // one more\n}\n/* note */\n"
    assert bench.code_sha256([base]) == bench.code_sha256([reworded])
    assert bench.code_sha256([base]) != bench.code_sha256([changed])
    assert bench.code_sha256([base, base]) != bench.code_sha256([base])


def test_counter_summaries_name_their_kernel_and_code():
    # every committed counter summary carries the lines bench reads back
    import glob
    import os
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    files = glob.glob(os.path.join(root, "profiles", "pmc_traffic_*.md"))
    assert files
    for f in files:
        text = open(f).read()
        for key in ("kernel: ", "kernel_source_sha256: ", "traffic_bytes_per_launch: "):
            assert key in text, (f, key)
