"""GPU parity: the HIP path through the C ABI against the CPU oracle on the same seeded
inputs. Routing (remap, align) must match bit for bit; deltas must satisfy, per output
tensor over the rows that receive a delta,
    max |gpu - ref| <= 1e-2 * max |ref| + 1e-3.
The small configs are compared everywhere; the two prefill configs at full size are
compared on the whole routing and on a seeded sample of pairs that the oracle computes
one by one."""
import numpy as np
import pytest
import torch

import oracle
from tests import pins, shared
from virtual_expert_routed_amd import binding as mb
from virtual_expert_routed_amd import configs, inputs
from virtual_expert_routed_amd.layer import DeviceLayer

pytestmark = pytest.mark.gpu

REL, ABS = 1e-2, 1e-3


def within_tol(gpu, ref, what):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, what
    if ref.size == 0:
        return
    err = np.max(np.abs(gpu - ref))
    bound = REL * np.max(np.abs(ref)) + ABS
    assert np.all(np.isfinite(gpu)), what
    assert err <= bound, f"{what}: max err {err:.3g} > {bound:.3g}"


def as_f64(a, cfg):
    return pins.bf16_bits_to_f64(a) if cfg.dtype == "bf16" else np.asarray(a, np.float64)


def sample_mask(cfg, routing, n=768, seed=0, hot=16):
    """Pairs the oracle computes one by one at full size: a seeded sample of n pairs; one
    pair, at a seeded position, of every block that holds real pairs (so every block of the
    routing is compared); every pair of the first and the last block of each of the `hot`
    fullest buckets (so every hot virtual expert's full tile and its ragged tail are
    compared whole); and every pair of the last block."""
    srt, eid, npp = routing
    rng = np.random.default_rng(seed)
    mask = np.zeros(cfg.numel, np.uint8)
    mask[rng.choice(cfg.numel, size=min(n, cfg.numel), replace=False)] = 1
    blocks = srt.reshape(-1, cfg.block_m)
    fill = (blocks < cfg.numel).sum(1)
    nz = np.nonzero(fill)[0]
    pick = np.minimum((rng.random(nz.size) * fill[nz]).astype(np.int64), fill[nz] - 1)
    mask[blocks[nz, pick]] = 1
    whole = [len(blocks) - 1]
    valid = eid >= 0
    if valid.any():
        per_bucket = np.bincount(eid[valid], weights=fill[valid], minlength=cfg.V)
        for b in np.argsort(-per_bucket, kind="stable")[:hot]:
            if per_bucket[b] == 0:
                break
            idx = np.nonzero(eid == b)[0]
            whole += [int(idx[0]), int(idx[-1])]
    for b in whole:
        rows = blocks[b][blocks[b] < cfg.numel]
        mask[rows] = 1
    return mask


class Case:
    def __init__(self, cfg, seed=0, sampled=False):
        oracle.build()
        self.cfg = cfg
        self.inp = shared.generate(cfg, seed)
        self.routing = oracle.align_block_size(self.inp.topk_ids, self.inp.lora_ids, cfg.E,
                                               cfg.S, cfg.block_m)
        self.mask = sample_mask(cfg, self.routing) if sampled else None
        srt, eid, npp = self.routing
        self.s, self.out = [], []
        for st, sin in zip(cfg.stages, self.inp.stages):
            s = oracle.lora_shrink(sin.xin, sin.row_div, sin.A, srt, eid, npp, cfg.numel,
                                   cfg.block_m, pair_mask=self.mask, slices=st.slices,
                                   slot_ranks=self.inp.slot_ranks, E=cfg.E)
            out = np.zeros((cfg.numel, st.N), dtype=sin.B.dtype)
            oracle.lora_expand(s, st.slices, sin.B, self.inp.scale, cfg.E, srt, eid, npp,
                               cfg.numel, cfg.block_m, out, pair_mask=self.mask,
                               slot_ranks=self.inp.slot_ranks)
            self.s.append(s)
            self.out.append(out)
        vids = oracle.virtual_topk(self.inp.topk_ids, self.inp.lora_ids, cfg.E, cfg.S)
        valid = ((vids >= 0) & (vids < cfg.V)).reshape(-1)
        self.rows = valid if self.mask is None else (valid & self.mask.astype(bool))
        self.no_delta = ~valid


_cache = {}


def get_case(cfg):
    if cfg.name not in _cache:
        big = cfg.numel > 4096
        if big:  # keep one big case in host memory at a time
            for k in [k for k, c in _cache.items() if c.cfg.numel > 4096]:
                del _cache[k]
        _cache[cfg.name] = Case(cfg, sampled=big)
    return _cache[cfg.name]


ALL = [configs.C0, configs.C1, configs.C2, configs.C3, configs.C4, configs.N2]
IDS = [c.name for c in ALL]


def announce(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("cfg", ALL, ids=IDS)
def test_remap_and_align_bit_exact(cfg):
    announce(f"[routing] {cfg.name}")
    case = get_case(cfg)
    dl = DeviceLayer(case.inp)
    vids = dl.remap().cpu().numpy()
    assert np.array_equal(vids, oracle.virtual_topk(case.inp.topk_ids, case.inp.lora_ids,
                                                    cfg.E, cfg.S))
    dl.align()
    srt, eid, npp = dl.routing_host()
    assert npp == case.routing[2]
    assert np.array_equal(srt, case.routing[0])
    assert np.array_equal(eid, case.routing[1])
    # the same routing from precomputed virtual ids (no inline remap)
    vt = torch.from_numpy(vids).cuda()
    s2, e2, n2 = mb.mol_align_block_size(vt, None, cfg.V, 1, cfg.block_m)
    n2 = int(n2.item())
    assert n2 == npp
    assert np.array_equal(s2[:n2].cpu().numpy(), srt)
    assert np.array_equal(e2[: n2 // cfg.block_m].cpu().numpy(), eid)
    torch.cuda.synchronize()


PLAN_MARK = -7  # what the tests fill a plan buffer with before the align


def check_plan(cfg, plan_t, routing):
    """The align's work plan on the device equals its rebuild from the oracle's routing;
    for a batch that gets no plan the align leaves the buffer (filled with PLAN_MARK)
    untouched."""
    srt, eid, npp = routing
    written, runs = pins.expected_plan(cfg.numel, cfg.V, cfg.block_m, srt, eid, npp)
    plan = plan_t.cpu().numpy()
    if not written:
        assert np.all(plan == PLAN_MARK), f"{cfg.name}: plan written for a batch without one"
        return
    assert tuple(plan[:8]) == (len(runs), 0, 0, 0, 0, 0, 0, 0), cfg.name
    d = plan[8:8 + 4 * len(runs)].reshape(-1, 4)
    if runs:
        assert np.array_equal(d[:, :3], np.array(runs, dtype=np.int64)), f"{cfg.name}: runs"


@pytest.mark.parametrize("cfg", ALL, ids=IDS)
def test_align_work_plan(cfg):
    announce(f"[plan] {cfg.name}")
    case = get_case(cfg)
    dl = DeviceLayer(case.inp)
    dl.plan.fill_(PLAN_MARK)
    dl.align()
    check_plan(cfg, dl.plan, case.routing)
    torch.cuda.synchronize()


@pytest.mark.parametrize("cfg", ALL, ids=IDS)
def test_shrink_expand_and_fused_delta_parity(cfg):
    announce(f"[delta] {cfg.name}")
    case = get_case(cfg)
    dl = DeviceLayer(case.inp)
    dl.align()
    rows = case.rows
    for si, st in enumerate(cfg.stages):
        s = dl.shrink(si).cpu().numpy()
        within_tol(s[rows], case.s[si][rows], f"{cfg.name}/{st.name}/s")
        out_u = dl.expand(si)
        got = dl.out_host(si)
        within_tol(as_f64(got[rows], cfg), as_f64(case.out[si][rows], cfg),
                   f"{cfg.name}/{st.name}/out")
        assert np.all(got[case.no_delta] == 0), "rows without a delta were written"
        del got
        # one call for the stage: bit-identical to shrink + expand
        unfused = out_u.clone()
        dl.out[si].zero_()
        dl.delta(si)
        assert torch.equal(dl.out[si], unfused), "mol_lora_delta differs from shrink+expand"
    torch.cuda.synchronize()


@pytest.mark.parametrize("cfg", [configs.C0, configs.C1, configs.C2], ids=IDS[:3])
def test_repeat_runs_are_bit_identical(cfg):
    case = get_case(cfg)
    dl = DeviceLayer(case.inp)
    first = [o.clone() for o in dl.run()]
    for o in dl.out:
        o.zero_()
    second = dl.run()
    for a, b in zip(first, second):
        assert torch.equal(a, b)


def _nonzero_base_case(cfg):
    return get_case(cfg) if cfg.name in IDS else Case(cfg)


def _nonzero_base_cfgs():
    by = {c.name: c for c in EDGE}
    return [configs.C0, configs.C1, by["mfma_blocks"], by["ranked_mfma"], by["mfma_r64_zipf"],
            configs.C4]


def test_delta_adds_into_nonzero_output(cfg):
    """The delta added into nonzero output rows (out read, added to and rounded once), on
    the VALU kernels (C0, C1) and on the MFMA expand's read-add-round of old values (the
    MFMA edge shapes and the full-size C4 layer, sampled as in the parity test)."""
    announce(f"[nonzero base] {cfg.name}")
    case = _nonzero_base_case(cfg)
    base = [inputs.base_out(cfg, si, seed=5) for si in range(len(cfg.stages))]
    dl = DeviceLayer(case.inp, outs=base)
    dl.run()
    srt, eid, npp = case.routing
    for si, st in enumerate(cfg.stages):
        sin = case.inp.stages[si]
        ref = base[si].copy()
        oracle.lora_expand(case.s[si], st.slices, sin.B, case.inp.scale, cfg.E, srt, eid, npp,
                           cfg.numel, cfg.block_m, ref, pair_mask=case.mask,
                           slot_ranks=case.inp.slot_ranks)
        got = dl.out_host(si)
        assert np.array_equal(got[case.no_delta], base[si][case.no_delta])
        b64 = as_f64(base[si][case.rows], cfg)
        g64, r64 = as_f64(got[case.rows], cfg), as_f64(ref[case.rows], cfg)
        del got, ref
        d_ref = r64 - b64
        ulp = np.abs(b64) * 2.0 ** -7 if cfg.dtype == "bf16" else np.abs(b64) * 2.0 ** -23
        bound = REL * np.max(np.abs(d_ref)) + ABS + ulp
        assert np.all(np.abs(g64 - r64) <= bound), f"{cfg.name}/{st.name}"
    del dl
    torch.cuda.synchronize()


def _edge_cfg(**kw):
    base = dict(name="edge", dtype="bf16", M=37, hidden=128, E=8, topk=3, S=3, rank=16,
                block_m=16, stages=configs._two_stage(128, 48, 16), expert_dist="uniform",
                sentinel_count=5, nolora_count=4, lora_dist="uniform", w_sigma=0.05)
    base.update(kw)
    return configs.LayerConfig(**base)


EDGE = [
    _edge_cfg(name="ragged_bm16"),
    _edge_cfg(name="bm1", block_m=1),
    _edge_cfg(name="bm_max", block_m=1024, M=300),
    _edge_cfg(name="bm48_not_pow2", block_m=48, M=200),
    _edge_cfg(name="single_token", M=1, topk=2, sentinel_count=0, nolora_count=0),
    _edge_cfg(name="all_nolora", M=20, nolora_count=20),
    _edge_cfg(name="all_sentinel", M=6, topk=2, sentinel_count=12, nolora_count=0),
    _edge_cfg(name="f32_slices", dtype="f32", M=19, rank=4, E=5, S=2),
    _edge_cfg(name="large_path_ragged", M=4099, topk=2, E=64, S=4, hidden=64,
              stages=configs._two_stage(64, 32, 8), rank=8, block_m=32, sentinel_count=70,
              nolora_count=300, expert_dist="zipf"),
    _edge_cfg(name="ceiling_small", M=40, topk=2, E=8191, S=1, hidden=64, rank=8,
              stages=configs._two_stage(64, 32, 8), nolora_count=0, block_m=8),
    _edge_cfg(name="ceiling_large", M=3000, topk=4, E=4095, S=2, hidden=64, rank=8,
              stages=configs._two_stage(64, 32, 8), nolora_count=0, block_m=8,
              sentinel_count=100),
    # from 4096 pairs (8 per bucket on average) on, blocks of >= 4 real pairs take the bf16
    # MFMA kernels and the rest the VALU kernels: full blocks, ragged last blocks and small
    # buckets side by side
    _edge_cfg(name="mfma_blocks", M=1024, topk=4, E=8, S=2, hidden=256, rank=32,
              stages=configs._two_stage(256, 128, 32), block_m=64, sentinel_count=40,
              nolora_count=30),
    _edge_cfg(name="mfma_r64_zipf", M=2048, topk=2, E=16, S=2, hidden=256, rank=64,
              stages=configs._two_stage(256, 192, 64), block_m=64, sentinel_count=20,
              nolora_count=50, expert_dist="zipf"),
    _edge_cfg(name="mfma_bm128", M=1024, topk=4, E=8, S=2, hidden=128, rank=32,
              stages=configs._two_stage(128, 64, 32), block_m=128, sentinel_count=10,
              nolora_count=10),
    _edge_cfg(name="mfma_bm48_not_pow2", M=1024, topk=4, E=8, S=2, hidden=256, rank=32,
              stages=configs._two_stage(256, 128, 32), block_m=48, sentinel_count=10,
              nolora_count=10),
    # per-slot ranks: the weights past a slot's rank hold NaN, rank 5 and 20 end inside a
    # 16-byte weight vector, rank 0 adds nothing (VALU bf16 and fp32, and MFMA)
    _edge_cfg(name="ranked_bf16", slot_ranks=(16, 5, 0)),
    _edge_cfg(name="ranked_f32", dtype="f32", M=19, rank=4, E=5, S=2, slot_ranks=(3, 0)),
    _edge_cfg(name="ranked_mfma", M=1024, topk=4, E=8, S=2, hidden=256, rank=32,
              stages=configs._two_stage(256, 128, 32), block_m=64, sentinel_count=10,
              nolora_count=10, slot_ranks=(20, 32)),
    # k tails past the staged chunk, and an expand slice width (136) that is not a
    # multiple of 64, which keeps the expand on the VALU kernel
    _edge_cfg(name="mfma_ragged_k", M=1024, topk=4, E=8, S=2, hidden=264, rank=32,
              stages=configs._two_stage(264, 136, 32), block_m=64, sentinel_count=10,
              nolora_count=10),
]


test_delta_adds_into_nonzero_output = pytest.mark.parametrize(
    "cfg", _nonzero_base_cfgs(), ids=[c.name for c in _nonzero_base_cfgs()])(
    test_delta_adds_into_nonzero_output)


@pytest.mark.parametrize("cfg", EDGE, ids=[c.name for c in EDGE])
def test_edge_cases(cfg):
    announce(f"[edge] {cfg.name}")
    case = Case(cfg)
    dl = DeviceLayer(case.inp)
    dl.plan.fill_(PLAN_MARK)
    dl.align()
    srt, eid, npp = dl.routing_host()
    assert npp == case.routing[2]
    assert np.array_equal(srt, case.routing[0]) and np.array_equal(eid, case.routing[1])
    assert npp // cfg.block_m <= dl.max_blocks
    check_plan(cfg, dl.plan, case.routing)
    blockwise = DeviceLayer(case.inp, use_plan=False)  # the same calls without the plan
    blockwise.align()
    for si, st in enumerate(cfg.stages):
        dl.delta(si)
        blockwise.delta(si)
        got = as_f64(dl.out_host(si), cfg)
        within_tol(as_f64(blockwise.out_host(si), cfg)[case.rows],
                   as_f64(case.out[si], cfg)[case.rows], f"{cfg.name}/{st.name} (no plan)")
        within_tol(got[case.rows], as_f64(case.out[si], cfg)[case.rows],
                   f"{cfg.name}/{st.name}")
        assert np.all(got[case.no_delta] == 0)
        if cfg.slot_ranks is not None:
            s = dl.delta_ws[si][:cfg.numel * st.R * 4].view(torch.float32).view(cfg.numel, st.R)
            s = s.cpu().numpy()
            within_tol(s[case.rows], case.s[si][case.rows], f"{cfg.name}/{st.name}/s")
            assert np.all(np.isfinite(s[case.rows]))
    torch.cuda.synchronize()


# Batch sizes at the align kernels' selection bounds (one wave per workgroup up to 256
# pairs; 16-wave workgroups up to 4096; three kernels above), each with small and large
# virtual expert counts, out-of-range ids and no-adapter tokens. The bucket counts V + 1
# (8, 1025, 3001, 4097, 8191) cover each number of buckets a thread owns in the small align
# (1, 2, 4, 8, 8), whose counter rows are padded to a multiple of it (1025 -> 1026,
# 3001 -> 3004, 4097 -> 4104, 8191 -> 8192; 8 needs none).
ALIGN_BOUNDS = [(M, k, E, S, bm) for (M, k) in ((1, 1), (63, 1), (16, 4), (65, 1), (32, 4),
                                                (255, 1), (32, 8), (257, 1), (1024, 4),
                                                (4097, 1))
                for (E, S, bm) in ((7, 1, 16), (128, 8, 64), (1000, 3, 16), (1024, 4, 32),
                                   (4095, 2, 48))]


@pytest.mark.parametrize("M,k,E,S,bm", ALIGN_BOUNDS)
def test_align_sizes_at_kernel_bounds(M, k, E, S, bm):
    announce(f"[align bounds] M={M} topk={k} E={E} S={S} BM={bm}")
    rng = np.random.default_rng(M * 7 + k * 131 + E + S + bm)
    ids = rng.integers(-2, E + 2, size=(M, k)).astype(np.int32)
    lora = rng.integers(-1, S + 1, size=M).astype(np.int32)
    srt, eid, npp = oracle.align_block_size(ids, lora, E, S, bm)
    plan = mb.new_plan(M * k, E * S, bm, "cuda").fill_(PLAN_MARK)
    s2, e2, n2 = mb.mol_align_block_size(torch.from_numpy(ids).cuda(),
                                         torch.from_numpy(lora).cuda(), E, S, bm, plan=plan)
    n2 = int(n2.item())
    assert n2 == npp
    assert np.array_equal(s2[:n2].cpu().numpy(), srt)
    assert np.array_equal(e2[: n2 // bm].cpu().numpy(), eid)
    cfg = configs.scaled(configs.C1, name="bounds", M=M, topk=k, E=E, S=S, block_m=bm)
    check_plan(cfg, plan, (srt, eid, npp))


def test_empty_batch():
    cfg = _edge_cfg(name="empty", M=0, sentinel_count=0, nolora_count=0)
    inp = inputs.generate(cfg, 0)
    dl = DeviceLayer(inp)
    dl.npp.fill_(-7)
    dl.align()
    assert int(dl.npp.item()) == 0
    for si in range(len(cfg.stages)):
        dl.delta(si)
        dl.shrink(si)
        dl.expand(si)
    torch.cuda.synchronize()


@pytest.mark.parametrize("cfg", [configs.C1, configs.C2], ids=IDS[1:3])
def test_delta_never_reads_stale_s(cfg):
    """Poison the workspace's s rows with NaN and feed two different activations through
    the same workspace: a read of s before it is written would show up as NaN or as the
    previous call's values."""
    case = get_case(cfg)
    dl = DeviceLayer(case.inp)
    dl.align()
    for si, st in enumerate(cfg.stages):
        s_bytes = cfg.numel * st.R * 4
        for flip in (1.0, -0.5):
            dl.delta_ws[si][:s_bytes].view(torch.float32).fill_(float("nan"))
            if flip != 1.0:
                dl.xin[si].mul_(flip)
            dl.out[si].zero_()
            dl.shrink(si)
            dl.expand(si)
            ref = dl.out[si].clone()
            dl.out[si].zero_()
            dl.delta(si)
            torch.cuda.synchronize()
            assert torch.equal(dl.out[si], ref), f"{cfg.name} stage {si} flip {flip}"
            assert not torch.isnan(dl.out[si].float()).any()


def test_hip_graph_replays_match_eager():
    cfg = configs.C1
    case = get_case(cfg)
    dl = DeviceLayer(case.inp)
    dl.run()
    eager = [o.clone() for o in dl.out]
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        for o in dl.out:
            o.zero_()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=stream):
            dl.run()
    torch.cuda.current_stream().wait_stream(stream)
    for rep in range(4):
        for o in dl.out:
            o.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(dl.out, eager):
            assert torch.equal(a, b), f"replay {rep}"
