"""The reference geometry's launch grids that the pages print (tests/golden/reference_grid.txt)
pin bench.py's calculator, which reports the same grids for these configurations as context."""
import os

import bench
from tests import conftest
from virtual_expert_routed_amd import configs

GOLDEN = os.path.join(conftest.ROOT, "tests", "golden", "reference_grid.txt")


def rows():
    for line in open(GOLDEN):
        line = line.split("#")[0].strip()
        if line:
            grid_m, n, block_n, ctas = (int(x) for x in line.split()[:4])
            yield grid_m, n, block_n, ctas


def test_golden_grids_reproduce():
    got = list(rows())
    assert len(got) == 4
    for grid_m, n, block_n, ctas in got:
        assert bench.reference_ctas(grid_m, n, block_n) == ctas


def test_grid_ratio_equals_n_ratio():
    # the page's observation: 153984 / 6416 = 6144 / 256 = 24
    assert bench.reference_ctas(1604, 6144) // bench.reference_ctas(1604, 256) == 6144 // 256


def test_reference_grid_m_vs_real_block_bound():
    # the worst-case buffer has a block per bucket; the real-pairs bound has at most numel
    from virtual_expert_routed_amd import binding as mb
    for cfg in (configs.C1, configs.C2):
        ref = bench.reference_grid_m(cfg)
        ours = mb.mol_align_max_blocks(cfg.numel, cfg.V, cfg.block_m)
        assert ours <= ref
    assert bench.reference_grid_m(configs.C1) == 1012
    assert mb.mol_align_max_blocks(configs.C1.numel, configs.C1.V, configs.C1.block_m) == 184


def test_n2_config_has_the_pages_decode_shape():
    # MindLab PR 24 page: down expand N = 6144 and gate/up expands N = 256 at r = 32 and
    # BLOCK_M = 64, ~1.1 k routed pairs, and a worst-case buffer of 1604 blocks
    c = configs.N2
    gate_up, down = c.stages
    assert (down.N, down.r, c.block_m) == (6144, 32, 64)
    assert gate_up.N // gate_up.slices == 256 and gate_up.r == 32
    assert 1000 <= c.numel - c.sentinel_count <= 1200
    grid_m = bench.reference_grid_m(c)
    assert abs(grid_m - 1604) <= 0.01 * 1604
    assert abs(bench.reference_ctas(grid_m, 6144) - 153984) <= 0.01 * 153984
    assert abs(bench.reference_ctas(grid_m, 256) - 6416) <= 0.01 * 6416
