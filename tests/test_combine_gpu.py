"""GPU parity of the combine after the down projection, through the C ABI, against the
CPU oracle on the same seeded inputs:

* mol_moe_combine on generated rows: within half a unit in the last place of the exact
  weighted sum, within one unit of the oracle's rounding, and never reading the rows of
  pairs that have no local expert (they hold NaN here);
* mol_lora_expand_combine (the down expand fused with the combine) and the unfused chain
  mol_lora_expand -> mol_moe_combine: from zero base rows within the path's tolerance
  max|err| <= 1e-2 max|ref| + 1e-3; from nonzero base rows within that plus one unit of
  the result (and, for the chain, one unit of each rounded pair row, weighted); the fused
  call leaves the base rows untouched.
"""
import numpy as np
import pytest
import torch

import oracle
from tests import pins, shared
from virtual_expert_routed_amd import binding as mb
from virtual_expert_routed_amd import configs, inputs
from virtual_expert_routed_amd.layer import DeviceLayer, to_device

pytestmark = pytest.mark.gpu

REL, ABS = 1e-2, 1e-3


def _edge(**kw):
    base = dict(name="cedge", dtype="bf16", M=37, hidden=128, E=8, topk=3, S=3, rank=16,
                stages=configs._two_stage(128, 40, 16), sentinel_count=9, nolora_count=4,
                block_m=16)
    base.update(kw)
    return configs.scaled(configs.C1, **base)


CASES = [
    configs.C0,
    configs.C1,
    configs.C2,
    configs.N2,  # the pages' decode shape: the down rows are 6144 wide
    _edge(name="topk1", topk=1, sentinel_count=5),
    _edge(name="ranked", slot_ranks=(16, 5, 0)),
    _edge(name="all_nolora", M=20, nolora_count=20),
    _edge(name="all_sentinel", M=6, topk=2, sentinel_count=12, nolora_count=0),
    _edge(name="ragged_n_r8", hidden=136, stages=configs._two_stage(136, 24, 8), rank=8),
    _edge(name="r128", stages=configs._two_stage(128, 72, 128), rank=128, M=9),
    _edge(name="topk_13", M=11, topk=13, E=16, sentinel_count=7),
    _edge(name="f32_r4", dtype="f32", M=19, rank=4, E=5, S=2,
          stages=configs._two_stage(128, 40, 4)),
]
IDS = [c.name for c in CASES]


def _f64(a, cfg):
    return pins.bf16_bits_to_f64(a) if cfg.dtype == "bf16" else np.asarray(a, np.float64)


def _host(t, cfg):
    if cfg.dtype == "bf16":
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def _local(cfg, topk_ids):
    return ((topk_ids >= 0) & (topk_ids < cfg.E)).reshape(-1)


@pytest.mark.parametrize("cfg", CASES, ids=IDS)
def test_combine_matches_oracle_and_skips_missing_rows(cfg):
    print(f"[combine] {cfg.name}", flush=True)
    inp = inputs.generate(cfg, seed=3, tensors=False)
    si = len(cfg.stages) - 1
    rows = inputs.base_out(cfg, si, seed=3)
    off = ~_local(cfg, inp.topk_ids)
    rows[off] = np.uint16(0x7FC0) if cfg.dtype == "bf16" else np.float32(np.nan)
    w = inputs.topk_weights(cfg, 3)
    ref = _f64(oracle.moe_combine(rows, inp.topk_ids, w, cfg.E), cfg)
    exact = np.matmul(w.astype(np.float64)[:, None, :],
                      np.where(off[:, None], 0.0, _f64(rows, cfg)).reshape(cfg.M, cfg.topk, -1))[:, 0]
    dev = torch.device("cuda")
    y = mb.mol_moe_combine(to_device(rows, dev, cfg.dtype == "bf16"),
                           torch.from_numpy(inp.topk_ids).to(dev), torch.from_numpy(w).to(dev),
                           cfg.E)
    got = _f64(_host(y, cfg), cfg)
    assert np.all(np.isfinite(got))
    # within half a unit in the last place of the exact sum; and at most one unit from the
    # oracle's own rounding of its double sum (an fp32 sum can round the other way near a
    # tie; adjacent bf16 values are up to 2^-7 apart relative to the smaller)
    half = 2.0 ** -8 if cfg.dtype == "bf16" else 2.0 ** -23
    assert np.all(np.abs(got - exact) <= half * np.abs(exact) + 1e-6)
    assert np.all(np.abs(got - ref) <= 4 * half * np.abs(ref) + 1e-6)


def _down(cfg, seed, base_rows, device=True):
    """Oracle result (and the device layer) for the down stage of one layer."""
    inp = inputs.generate(cfg, seed=seed)
    si = len(cfg.stages) - 1
    st, sin = cfg.stages[si], inp.stages[si]
    srt, eid, npp = oracle.align_block_size(inp.topk_ids, inp.lora_ids, cfg.E, cfg.S,
                                            cfg.block_m)
    s = oracle.lora_shrink(sin.xin, sin.row_div, sin.A, srt, eid, npp, cfg.numel, cfg.block_m,
                           slot_ranks=inp.slot_ranks, E=cfg.E)
    w = inputs.topk_weights(cfg, seed)
    ref = oracle.lora_expand_combine(np.nan_to_num(s), sin.B, inp.scale, inp.topk_ids,
                                     inp.lora_ids, w, cfg.E, cfg.S, base_rows,
                                     slot_ranks=inp.slot_ranks)
    if not device:
        return inp, None, _f64(ref, cfg)
    outs = [np.zeros((cfg.numel, x.N), dtype=sin.B.dtype) for x in cfg.stages]
    outs[si] = base_rows.copy()
    dl = DeviceLayer(inp, outs=outs, topk_weights=w)
    return inp, dl, _f64(ref, cfg)


@pytest.mark.parametrize("cfg", CASES, ids=IDS)
def test_fused_and_chained_from_zero_base(cfg):
    print(f"[expand_combine zero base] {cfg.name}", flush=True)
    si = len(cfg.stages) - 1
    zero = np.zeros((cfg.numel, cfg.stages[si].N),
                    dtype=np.uint16 if cfg.dtype == "bf16" else np.float32)
    inp, dl, ref = _down(cfg, 5, zero)
    dl.align()
    dl.shrink(si)
    base = dl.out[si].clone()
    fused = _f64(_host(dl.expand_combine(), cfg), cfg)
    assert torch.equal(dl.out[si], base)  # the fused call never writes the rows
    _check_tol(fused, ref, f"{cfg.name} fused")
    dl.expand(si)
    chained = _f64(_host(dl.combine(), cfg), cfg)
    _check_tol(chained, ref, f"{cfg.name} expand then combine")


@pytest.mark.parametrize("cfg", [configs.C1, CASES[IDS.index("ranked")], CASES[-1]],
                         ids=["c1", "ranked", "f32"])
def test_fused_and_chained_from_nonzero_base(cfg):
    print(f"[expand_combine base] {cfg.name}", flush=True)
    si = len(cfg.stages) - 1
    base_rows = inputs.base_out(cfg, si, seed=6)
    zero = np.zeros_like(base_rows)
    _, _, ref0 = _down(cfg, 6, zero, device=False)
    inp, dl, ref = _down(cfg, 6, base_rows)
    dl.align()
    dl.shrink(si)
    ulp = 2.0 ** -7 if cfg.dtype == "bf16" else 2.0 ** -22  # one unit, relative
    bound = REL * np.max(np.abs(ref0)) + ABS + ulp * np.abs(ref)
    # the chained path also rounds every pair row (base + delta) before the weighted sum:
    # one more unit of each row, weighted
    w = dl.topk_weights.cpu().numpy().astype(np.float64)
    local = _local(cfg, inp.topk_ids).reshape(cfg.M, cfg.topk, 1)
    rows_mag = (np.abs(_f64(base_rows, cfg)) + np.max(np.abs(ref0))).reshape(cfg.M, cfg.topk, -1)
    chain_extra = ulp * np.matmul(w[:, None, :], rows_mag * local)[:, 0]
    for what, fn in (("fused", dl.expand_combine), ("chained", None)):
        if fn is None:
            dl.expand(si)
            y = dl.combine()
        else:
            y = fn()
        got = _f64(_host(y, cfg), cfg)
        assert np.all(np.isfinite(got)), what
        b = bound + (chain_extra if fn is None else 0.0)
        assert np.all(np.abs(got - ref) <= b), f"{cfg.name} {what}"


FULL = [configs.C3, configs.C4]


@pytest.mark.parametrize("cfg", FULL, ids=[c.name for c in FULL])
def test_combine_full_size(cfg):
    """mol_moe_combine over every token of a full-size prefill layer: within one unit of the
    oracle everywhere, within half a unit of the exact weighted sum on a seeded sample of
    tokens, and never reading the rows of pairs without a local expert (NaN here)."""
    print(f"[combine full size] {cfg.name}", flush=True)
    inp = inputs.generate(cfg, seed=0, tensors=False)
    si = len(cfg.stages) - 1
    rows = inputs.base_out(cfg, si, seed=3)
    off = ~_local(cfg, inp.topk_ids)
    rows[off] = np.uint16(0x7FC0)
    w = inputs.topk_weights(cfg, 3)
    ref = _f64(oracle.moe_combine(rows, inp.topk_ids, w, cfg.E), cfg)
    dev = torch.device("cuda")
    y = mb.mol_moe_combine(to_device(rows, dev, True), torch.from_numpy(inp.topk_ids).to(dev),
                           torch.from_numpy(w).to(dev), cfg.E)
    got = _f64(_host(y, cfg), cfg)
    del y
    assert np.all(np.isfinite(got))
    half = 2.0 ** -8
    assert np.all(np.abs(got - ref) <= 4 * half * np.abs(ref) + 1e-6)
    tok = np.sort(np.random.default_rng(1).choice(cfg.M, size=512, replace=False))
    r3 = rows.reshape(cfg.M, cfg.topk, -1)[tok]
    o3 = off.reshape(cfg.M, cfg.topk)[tok]
    exact = np.matmul(w[tok].astype(np.float64)[:, None, :],
                      np.where(o3[:, :, None], 0.0, _f64(r3, cfg)))[:, 0]
    assert np.all(np.abs(got[tok] - exact) <= half * np.abs(exact) + 1e-6)


@pytest.mark.parametrize("cfg", FULL, ids=[c.name for c in FULL])
def test_fused_and_chained_full_size_sampled(cfg):
    """The down expand fused with the combine, and the unfused chain, on a full-size prefill
    layer from zero base rows: the whole layer runs on the GPU, and a seeded sample of 256
    tokens is compared with the oracle, which computes each token from its own pairs only."""
    print(f"[expand_combine full size] {cfg.name}", flush=True)
    inp = shared.generate(cfg, 0)
    si = len(cfg.stages) - 1
    st, sin = cfg.stages[si], inp.stages[si]
    w = inputs.topk_weights(cfg, 0)
    tok = np.sort(np.random.default_rng(2).choice(cfg.M, size=256, replace=False))
    pairs = (tok[:, None] * cfg.topk + np.arange(cfg.topk)[None, :]).reshape(-1)
    mask = np.zeros(cfg.numel, np.uint8)
    mask[pairs] = 1
    srt, eid, npp = oracle.align_block_size(inp.topk_ids, inp.lora_ids, cfg.E, cfg.S,
                                            cfg.block_m)
    s_ref = oracle.lora_shrink(sin.xin, sin.row_div, sin.A, srt, eid, npp, cfg.numel,
                               cfg.block_m, pair_mask=mask, slot_ranks=inp.slot_ranks, E=cfg.E)
    zero = np.zeros((tok.size * cfg.topk, st.N), dtype=np.uint16)
    ref = _f64(oracle.lora_expand_combine(np.nan_to_num(s_ref[pairs]), sin.B, inp.scale,
                                          inp.topk_ids[tok], inp.lora_ids[tok], w[tok], cfg.E,
                                          cfg.S, zero, slot_ranks=inp.slot_ranks), cfg)
    dl = DeviceLayer(inp, topk_weights=w)
    dl.align()
    dl.shrink(si)
    fused = _f64(_host(dl.expand_combine(), cfg), cfg)[tok]
    _check_tol(fused, ref, f"{cfg.name} fused (sampled tokens)")
    assert not torch.any(dl.out[si]), "the fused call never writes the pair rows"
    dl.expand(si)
    chained = _f64(_host(dl.combine(), cfg), cfg)[tok]
    _check_tol(chained, ref, f"{cfg.name} expand then combine (sampled tokens)")
    del dl
    torch.cuda.synchronize()


def _check_tol(gpu, ref, what):
    assert gpu.shape == ref.shape, what
    assert np.all(np.isfinite(gpu)), what
    err = float(np.max(np.abs(gpu - ref))) if ref.size else 0.0
    bound = REL * float(np.max(np.abs(ref))) + ABS if ref.size else 0.0
    assert err <= bound, f"{what}: max err {err:.3g} > {bound:.3g}"


def test_combine_empty_batch():
    dev = torch.device("cuda")
    ids = torch.zeros((0, 4), dtype=torch.int32, device=dev)
    w = torch.zeros((0, 4), dtype=torch.float32, device=dev)
    rows = torch.zeros((0, 64), dtype=torch.bfloat16, device=dev)
    y = mb.mol_moe_combine(rows, ids, w, 8)
    assert y.shape == (0, 64)
    torch.cuda.synchronize()


def test_combine_calls_replay_in_a_hip_graph():
    """The layer, then the combine and the fused down expand + combine, captured in one
    hipGraph: every replay (with eager work and syncs between) equals the eager result."""
    cfg = configs.C1
    inp = inputs.generate(cfg, seed=7)
    w = inputs.topk_weights(cfg, 7)
    dl = DeviceLayer(inp, topk_weights=w)
    y_fused = torch.empty_like(dl.y)

    def body():
        dl.run()
        dl.combine()
        mb.mol_lora_expand_combine(dl.s[-1], dl.B[-1], dl.scale, dl.topk_ids, dl.lora_ids,
                                   dl.topk_weights, cfg.E, cfg.S, dl.out[-1], y=y_fused)

    for o in dl.out:
        o.zero_()
    body()
    torch.cuda.synchronize()
    eager = [t.clone() for t in (*dl.out, dl.y, y_fused)]
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            body()
    torch.cuda.current_stream().wait_stream(stream)
    for rep in range(3):
        for o in dl.out:
            o.zero_()
        dl.y.fill_(7.0)
        y_fused.fill_(7.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip((*dl.out, dl.y, y_fused), eager):
            assert torch.equal(a, b), f"replay {rep}"
