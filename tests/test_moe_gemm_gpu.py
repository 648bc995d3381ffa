"""GPU parity of the base MoE grouped GEMM (mol_moe_gemm), alone and with the LoRA delta
fused into its epilogue, through the C ABI against the CPU oracle on the same seeded inputs.
Each case checks, per stage:

* the base GEMM alone, within max|err| <= 1e-2 max|ref| + 1e-3;
* the fused form on zero base weights, which is the LoRA delta alone, to the same bound;
* the fused form with the base weights, to the same bound;
* rows of pairs without a local expert are left bit for bit as they were.
"""
import numpy as np
import pytest
import torch

import oracle
from tests import pins
from virtual_expert_routed_amd import binding as mb
from virtual_expert_routed_amd import configs, inputs
from virtual_expert_routed_amd.layer import to_device

pytestmark = pytest.mark.gpu

REL, ABS = 1e-2, 1e-3


def _edge(**kw):
    base = dict(name="gemm_edge", dtype="bf16", M=37, hidden=136, E=8, topk=3, S=3, rank=16,
                stages=configs._two_stage(136, 40, 16), sentinel_count=9, nolora_count=4,
                block_m=16)
    base.update(kw)
    return configs.scaled(configs.C1, **base)


CASES = [
    configs.C0,
    configs.C1,
    configs.C2,
    configs.N2,  # the pages' decode shape: K = 6144 on the gate_up stage, N = 6144 on the down
    _edge(name="ragged"),
    _edge(name="ranked", slot_ranks=(16, 5, 0)),
    _edge(name="many_per_expert", M=200, E=4, topk=2, S=2, block_m=64),
    _edge(name="f32", dtype="f32", M=23, rank=4, E=5, S=2, stages=configs._two_stage(136, 40, 4)),
    # the largest ranks the boundary accepts (256 bytes of one B row slice) at contraction
    # lengths short enough that a column's lanes hold fewer rank vectors than the slice has:
    # each lane must sum more than one vector of the rank (bf16 K = 256, r = 128; fp32 K =
    # 128, r = 64), at full rank and with ranks that end inside a vector
    _edge(name="rank128_bf16_k256", M=23, hidden=256, E=4, topk=2, S=2, rank=128,
          stages=configs._two_stage(256, 256, 128)),
    _edge(name="rank128_bf16_k256_ranked", M=23, hidden=256, E=4, topk=2, S=3, rank=128,
          stages=configs._two_stage(256, 256, 128), slot_ranks=(128, 71, 0)),
    _edge(name="rank64_f32_k128", dtype="f32", M=19, hidden=128, E=4, topk=2, S=2, rank=64,
          stages=configs._two_stage(128, 128, 64)),
    _edge(name="rank64_f32_k128_ranked", dtype="f32", M=19, hidden=128, E=4, topk=2, S=2,
          rank=64, stages=configs._two_stage(128, 128, 64), slot_ranks=(37, 64)),
]


def _f64(a, cfg):
    return pins.bf16_bits_to_f64(a) if cfg.dtype == "bf16" else np.asarray(a, np.float64)


def _host(t, cfg):
    if cfg.dtype == "bf16":
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def _tol(gpu, ref, what, mask):
    g, r = gpu[mask], ref[mask]
    if r.size == 0:
        return
    assert np.all(np.isfinite(g)), what
    err = float(np.max(np.abs(g - r)))
    bound = REL * float(np.max(np.abs(r))) + ABS
    assert err <= bound, f"{what}: max err {err:.3g} > {bound:.3g}"


@pytest.mark.parametrize("cfg", CASES, ids=[c.name for c in CASES])
def test_base_gemm_and_fused_delta(cfg):
    print(f"[moe_gemm] {cfg.name}", flush=True)
    dev = torch.device("cuda")
    bf16 = cfg.dtype == "bf16"
    inp = inputs.generate(cfg, seed=4)
    inp.scale[:] = np.linspace(0.5, 2.0, cfg.S, dtype=np.float32)
    numel, BM = cfg.numel, cfg.block_m
    t = inp.topk_ids.reshape(-1)
    local = (t >= 0) & (t < cfg.E)
    topk = torch.from_numpy(inp.topk_ids).to(dev)
    lora = torch.from_numpy(inp.lora_ids).to(dev)
    scale = torch.from_numpy(inp.scale).to(dev)
    ranks = None if inp.slot_ranks is None else torch.from_numpy(inp.slot_ranks).to(dev)
    # routing by virtual expert for the LoRA shrink, by base expert for the base GEMM
    vrt = mb.mol_align_block_size(topk, lora, cfg.E, cfg.S, BM)
    brt = mb.mol_align_block_size(topk, None, cfg.E, 1, BM)
    srt, eid, npp = oracle.align_block_size(inp.topk_ids, inp.lora_ids, cfg.E, cfg.S, BM)
    for si, (st, sin) in enumerate(zip(cfg.stages, inp.stages)):
        W = inputs.base_weights(cfg, si, seed=4)
        start = inputs.base_out(cfg, si, seed=4)
        s_ref = np.nan_to_num(oracle.lora_shrink(sin.xin, sin.row_div, sin.A, srt, eid, npp,
                                                 numel, BM, slices=st.slices,
                                                 slot_ranks=inp.slot_ranks, E=cfg.E))
        fkw = dict(s=s_ref, slices=st.slices, B=sin.B, scale=inp.scale, lora_ids=inp.lora_ids,
                   S=cfg.S, slot_ranks=inp.slot_ranks)
        ref_base = oracle.moe_gemm(sin.xin, sin.row_div, W, inp.topk_ids, cfg.E, start.copy())
        ref_fused = oracle.moe_gemm(sin.xin, sin.row_div, W, inp.topk_ids, cfg.E, start.copy(),
                                    **fkw)
        ref_delta = oracle.moe_gemm(sin.xin, sin.row_div, np.zeros_like(W), inp.topk_ids,
                                    cfg.E, start.copy(), **fkw)
        Wd = to_device(W, dev, bf16)
        Wz = torch.zeros_like(Wd)
        A = to_device(sin.A, dev, bf16)
        B = to_device(sin.B, dev, bf16)
        xin = to_device(sin.xin, dev, bf16)
        s = mb.mol_lora_shrink(xin, sin.row_div, A, *vrt, numel, cfg.V, BM, slices=st.slices,
                               slot_ranks=ranks, num_experts=cfg.E)
        lkw = dict(s=s, slices=st.slices, B=B, slot_scale=scale, lora_ids=lora, topk=cfg.topk,
                   num_slots=cfg.S, slot_ranks=ranks)
        results = {}
        for name, Wt, kw in (("base", Wd, {}), ("delta", Wz, lkw), ("fused", Wd, lkw)):
            out = to_device(start, dev, bf16)
            mb.mol_moe_gemm(xin, sin.row_div, Wt, *brt, numel, BM, out, **kw)
            torch.cuda.synchronize()
            results[name] = _host(out, cfg)
        for name, ref in (("base", ref_base), ("delta", ref_delta), ("fused", ref_fused)):
            got = results[name]
            _tol(_f64(got, cfg), _f64(ref, cfg), f"{cfg.name} stage {si} {name}", local)
            assert np.array_equal(got[~local], start[~local]), f"{name}: untouched rows"


def test_fused_gemm_repeats_bit_identically():
    cfg = configs.C1
    dev = torch.device("cuda")
    inp = inputs.generate(cfg, seed=5)
    topk = torch.from_numpy(inp.topk_ids).to(dev)
    lora = torch.from_numpy(inp.lora_ids).to(dev)
    scale = torch.from_numpy(inp.scale).to(dev)
    vrt = mb.mol_align_block_size(topk, lora, cfg.E, cfg.S, cfg.block_m)
    brt = mb.mol_align_block_size(topk, None, cfg.E, 1, cfg.block_m)
    st, sin = cfg.stages[0], inp.stages[0]
    xin = to_device(sin.xin, dev, True)
    s = mb.mol_lora_shrink(xin, sin.row_div, to_device(sin.A, dev, True), *vrt, cfg.numel, cfg.V,
                           cfg.block_m, slices=st.slices, num_experts=cfg.E)
    W = to_device(inputs.base_weights(cfg, 0, seed=5), dev, True)
    B = to_device(sin.B, dev, True)
    outs = []
    for _ in range(2):
        out = torch.zeros((cfg.numel, st.N), dtype=torch.bfloat16, device=dev)
        mb.mol_moe_gemm(xin, sin.row_div, W, *brt, cfg.numel, cfg.block_m, out, s=s,
                        slices=st.slices, B=B, slot_scale=scale, lora_ids=lora, topk=cfg.topk,
                        num_slots=cfg.S)
        outs.append(out)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])


def test_base_gemm_replays_in_a_hip_graph():
    """The routing, the LoRA shrink and the fused base GEMM of a stage captured in one
    hipGraph: every replay equals the eager result."""
    cfg = _edge(name="graph", M=29)
    dev = torch.device("cuda")
    inp = inputs.generate(cfg, seed=8)
    st, sin = cfg.stages[0], inp.stages[0]
    topk = torch.from_numpy(inp.topk_ids).to(dev)
    lora = torch.from_numpy(inp.lora_ids).to(dev)
    scale = torch.from_numpy(inp.scale).to(dev)
    nb = mb.mol_align_max_blocks(cfg.numel, cfg.V, cfg.block_m)
    nbb = mb.mol_align_max_blocks(cfg.numel, cfg.E, cfg.block_m)
    vrt = (torch.empty(nb * cfg.block_m, dtype=torch.int32, device=dev),
           torch.empty(nb, dtype=torch.int32, device=dev),
           torch.empty(1, dtype=torch.int32, device=dev))
    brt = (torch.empty(nbb * cfg.block_m, dtype=torch.int32, device=dev),
           torch.empty(nbb, dtype=torch.int32, device=dev),
           torch.empty(1, dtype=torch.int32, device=dev))
    xin = to_device(sin.xin, dev, True)
    A = to_device(sin.A, dev, True)
    B = to_device(sin.B, dev, True)
    W = to_device(inputs.base_weights(cfg, 0, seed=8), dev, True)
    s = torch.empty((cfg.numel, st.R), dtype=torch.float32, device=dev)
    out = torch.zeros((cfg.numel, st.N), dtype=torch.bfloat16, device=dev)

    def body():
        mb.mol_align_block_size(topk, lora, cfg.E, cfg.S, cfg.block_m, *vrt)
        mb.mol_align_block_size(topk, None, cfg.E, 1, cfg.block_m, *brt)
        mb.mol_lora_shrink(xin, sin.row_div, A, *vrt, cfg.numel, cfg.V, cfg.block_m, s=s,
                           slices=st.slices, num_experts=cfg.E)
        mb.mol_moe_gemm(xin, sin.row_div, W, *brt, cfg.numel, cfg.block_m, out, s=s,
                        slices=st.slices, B=B, slot_scale=scale, lora_ids=lora, topk=cfg.topk,
                        num_slots=cfg.S)

    out.fill_(3.0)  # rows of pairs without a local expert keep what they held
    body()
    torch.cuda.synchronize()
    eager = out.clone()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            body()
    torch.cuda.current_stream().wait_stream(stream)
    for rep in range(3):
        out.fill_(3.0)
        s.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep}"
