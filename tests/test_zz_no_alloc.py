"""mol_lora_delta_noalloc (s in the library's own per-GPU scratch, nothing allocated) against
mol_lora_delta (s in a caller's workspace) through the C ABI: the same kernels, so the
outputs must be bit-identical. Two calls in a row share the scratch, the second with a
smaller input, so a result that leaned on the previous call's s would show; the largest
case fills the scratch exactly (numel * R = MOL_DELTA_SCRATCH_FLOATS) and takes the MFMA
kernels."""
import numpy as np
import pytest
import torch

from virtual_expert_routed_amd import binding as mb
from virtual_expert_routed_amd import configs, inputs
from virtual_expert_routed_amd.layer import DeviceLayer

pytestmark = pytest.mark.gpu

# 2048 tokens x top-8 = 16384 pairs, gate_up R = 2 * 128 = 256: 4,194,304 floats of s
AT_LIMIT = configs.scaled(configs.C1, name="noalloc_at_limit", M=2048, hidden=64, E=8, S=2,
                          rank=128, stages=configs._two_stage(64, 64, 128),
                          sentinel_count=300, nolora_count=100)


def _delta_both_ways(dl, si):
    c = dl.cfg
    st = c.stages[si]
    start = dl.out[si].clone()
    dl.delta(si)
    want = dl.out[si].clone()
    dl.out[si].copy_(start)
    mb.mol_lora_delta_noalloc(dl.xin[si], dl.row_div[si], dl.A[si], st.slices, dl.B[si],
                              dl.scale, c.E, *dl.routing(), c.numel, c.V, c.block_m,
                              dl.out[si], slot_ranks=dl.slot_ranks)
    torch.cuda.synchronize()
    return want, dl.out[si]


@pytest.mark.parametrize("first,second", [(configs.C2, configs.C1), (AT_LIMIT, configs.C0)],
                         ids=["c2_then_c1", "limit_then_c0"])
def test_noalloc_delta_matches_workspace_delta(first, second):
    assert first.numel * max(s.R for s in first.stages) > \
        second.numel * max(s.R for s in second.stages)
    for cfg in (first, second):
        print(f"[noalloc] {cfg.name}", flush=True)
        base = [inputs.base_out(cfg, si, seed=1) for si in range(len(cfg.stages))]
        dl = DeviceLayer(inputs.generate(cfg, seed=1), outs=base)
        dl.align()
        for si in range(len(cfg.stages)):
            want, got = _delta_both_ways(dl, si)
            assert torch.equal(got, want), f"{cfg.name} stage {si}"
        del dl
    assert AT_LIMIT.numel * AT_LIMIT.stages[0].R == mb.MOL_DELTA_SCRATCH_FLOATS


def test_noalloc_rejects_beyond_its_scratch():
    cfg = configs.scaled(AT_LIMIT, name="noalloc_over", M=2049)
    dl = DeviceLayer(inputs.generate(cfg, seed=2))
    dl.align()
    st = cfg.stages[0]
    with pytest.raises(mb.MolError) as e:
        mb.mol_lora_delta_noalloc(dl.xin[0], dl.row_div[0], dl.A[0], st.slices, dl.B[0],
                                  dl.scale, cfg.E, *dl.routing(), cfg.numel, cfg.V,
                                  cfg.block_m, dl.out[0])
    assert e.value.status == mb.MOL_E_LIMIT
    torch.cuda.synchronize()
