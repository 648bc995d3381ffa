"""Guard bands around every buffer the library writes: each output (routing buffers, s, out,
the delta workspace, the combine's y) is a view into a larger allocation whose bands before
and after hold a fixed pattern. After every call the bands must be unchanged, and the
results must still match the oracle, on shapes whose sizes are not multiples of 4, 8 or
64, on the MFMA path and on the three-kernel align path."""
import numpy as np
import pytest
import torch

import oracle
from tests import pins
from virtual_expert_routed_amd import binding as mb
from virtual_expert_routed_amd import configs, inputs
from virtual_expert_routed_amd.layer import to_device

pytestmark = pytest.mark.gpu

BAND = 4096  # bytes on each side (a multiple of 16 keeps every view 16-byte aligned)
PATTERN = 0x5A


class Guarded:
    """A view of `n` elements of `dtype` with BAND bytes of PATTERN before and after."""

    def __init__(self, n, dtype, dev):
        esz = torch.empty((), dtype=dtype).element_size()
        self.raw = torch.full((2 * BAND + max(1, n) * esz,), PATTERN, dtype=torch.uint8,
                              device=dev)
        self.view = self.raw[BAND:BAND + max(1, n) * esz].view(dtype)[:n]

    def intact(self):
        raw = self.raw.cpu().numpy()
        return bool(np.all(raw[:BAND] == PATTERN) and np.all(raw[-BAND:] == PATTERN))


def _edge(**kw):
    base = dict(name="bounds", dtype="bf16", M=37, hidden=136, E=8, topk=3, S=3, rank=16,
                stages=configs._two_stage(136, 40, 16), sentinel_count=9, nolora_count=4,
                block_m=16)
    base.update(kw)
    return configs.scaled(configs.C1, **base)


CASES = [
    configs.C0,
    configs.C1,
    _edge(name="ragged_111"),
    _edge(name="bm48_ragged", M=199, block_m=48),
    _edge(name="f32_ragged", dtype="f32", M=23, rank=4, E=5, S=2,
          stages=configs._two_stage(136, 40, 4)),
    _edge(name="mfma_4096", M=1024, topk=4, E=8, S=2, hidden=256,
          stages=configs._two_stage(256, 128, 32), rank=32, sentinel_count=10,
          nolora_count=10, block_m=64),
    _edge(name="large_align", M=4099, topk=2, E=64, S=4, hidden=64,
          stages=configs._two_stage(64, 64, 8), rank=8, block_m=16),
]


def _f64(a, cfg):
    return pins.bf16_bits_to_f64(a) if cfg.dtype == "bf16" else np.asarray(a, np.float64)


def _host(t, cfg):
    if cfg.dtype == "bf16":
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


@pytest.mark.parametrize("cfg", CASES, ids=[c.name for c in CASES])
def test_no_write_outside_any_output(cfg):
    print(f"[bounds] {cfg.name}", flush=True)
    dev = torch.device("cuda")
    bf16 = cfg.dtype == "bf16"
    odt = torch.bfloat16 if bf16 else torch.float32
    inp = inputs.generate(cfg, seed=2)
    w = inputs.topk_weights(cfg, 2)
    (srt, eid, npp), s_ref, out_ref = oracle.run_layer(inp)
    numel, V, BM = cfg.numel, cfg.V, cfg.block_m
    mbk = mb.mol_align_max_blocks(numel, V, BM)
    guards = {}

    def guard(name, n, dtype):
        guards[name] = Guarded(n, dtype, dev)
        return guards[name].view

    topk = torch.from_numpy(inp.topk_ids).to(dev)
    lora = torch.from_numpy(inp.lora_ids).to(dev)
    scale = torch.from_numpy(inp.scale).to(dev)
    sorted_ids = guard("sorted_ids", mbk * BM, torch.int32)
    expert_ids = guard("expert_ids", mbk, torch.int32)
    npp_t = guard("num_post_padded", 1, torch.int32)
    wsb = mb.mol_align_workspace_bytes(numel, V, BM)
    align_ws = guard("align_workspace", wsb, torch.uint8) if wsb else None
    mb.mol_align_block_size(topk, lora, cfg.E, cfg.S, BM, sorted_ids, expert_ids, npp_t,
                            align_ws)
    torch.cuda.synchronize()
    n_gpu = int(npp_t.item())
    assert n_gpu == npp
    assert np.array_equal(sorted_ids[:npp].cpu().numpy(), srt)
    assert np.array_equal(expert_ids[: npp // BM].cpu().numpy(), eid)
    routing = (sorted_ids, expert_ids, npp_t)

    for si, (st, sin) in enumerate(zip(cfg.stages, inp.stages)):
        A = to_device(sin.A, dev, bf16)
        B = to_device(sin.B, dev, bf16)
        xin = to_device(sin.xin, dev, bf16)
        s = guard(f"s{si}", numel * st.R, torch.float32).view(numel, st.R)
        mb.mol_lora_shrink(xin, sin.row_div, A, *routing, numel, V, BM, s=s, slices=st.slices,
                           num_experts=cfg.E)
        out = guard(f"out{si}", numel * st.N, odt).view(numel, st.N)
        out.zero_()
        mb.mol_lora_expand(s, st.slices, B, scale, cfg.E, *routing, numel, V, BM, out)
        out2 = guard(f"out_delta{si}", numel * st.N, odt).view(numel, st.N)
        out2.zero_()
        ws = guard(f"delta_workspace{si}",
                   max(256, mb.mol_delta_workspace_bytes(numel, st.R, V, BM)), torch.uint8)
        mb.mol_lora_delta(xin, sin.row_div, A, st.slices, B, scale, cfg.E, *routing, numel, V,
                          BM, out2, ws)
        torch.cuda.synchronize()
        ref = _f64(out_ref[si], cfg)
        for got in (out, out2):
            g = _f64(_host(got, cfg), cfg)
            assert np.max(np.abs(g - ref)) <= 1e-2 * np.max(np.abs(ref)) + 1e-3, st.name
        if st.slices == 1 and si == len(cfg.stages) - 1:  # the down stage: its combine
            wt = torch.from_numpy(w).to(dev)
            y = guard("y_combine", cfg.M * st.N, odt).view(cfg.M, st.N)
            mb.mol_moe_combine(out, topk, wt, cfg.E, y=y)
            y2 = guard("y_fused", cfg.M * st.N, odt).view(cfg.M, st.N)
            base = torch.zeros_like(out)
            mb.mol_lora_expand_combine(s, B, scale, topk, lora, wt, cfg.E, cfg.S, base, y=y2)
            torch.cuda.synchronize()
            yr = _f64(oracle.lora_expand_combine(
                np.nan_to_num(s_ref[si]), sin.B, inp.scale, inp.topk_ids, inp.lora_ids, w,
                cfg.E, cfg.S, np.zeros((numel, st.N), dtype=sin.B.dtype)), cfg)
            for got in (y, y2):
                g = _f64(_host(got, cfg), cfg)
                assert np.max(np.abs(g - yr)) <= 1e-2 * np.max(np.abs(yr)) + 1e-3
    bad = [name for name, gd in guards.items() if not gd.intact()]
    assert not bad, f"{cfg.name}: writes outside {bad}"
