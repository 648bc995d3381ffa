"""Pins for the CPU oracle: it is checked against things other than itself.

* remap      - hand-worked cases of the pages' rule and its invariants: negative ids
               come back bit-for-bit (any negative value), a valid pair decodes back to
               (expert, slot), every other pair is -1 (virtual-experts remap snippet in
               the sglang PR 24171 summary; the -1 "no adapter" contract of MindLab
               sglang PR 24).
* align      - numpy's stable argsort + per-bucket padding on many random tiny cases,
               plus the structural invariants of a padded counting sort.
* shrink/expand - the per-pair identity delta = scale * B_e (A_e x) with numpy matmuls,
               the one-bucket special case that is a plain GEMM chain (X A^T) B^T,
               linearity in scale, zero A, and token permutation.
* bf16 rounding - literal IEEE cases, torch's float32 -> bfloat16 conversion, and an
               integer round-half-even on the binary64 bit pattern.
"""
import itertools

import copy

import numpy as np
import pytest
import torch

from tests import pins
from virtual_expert_routed_amd import configs, inputs


# ----------------------------------------------------------------------------- bf16


@pytest.mark.parametrize("value,bits", [
    (1.0, 0x3F80),
    (-2.5, 0xC020),
    (1.0 + 2.0 ** -8, 0x3F80),            # tie -> even (down)
    (1.0 + 3 * 2.0 ** -8, 0x3F82),        # tie -> even (up)
    (1.0 + 2.0 ** -8 + 2.0 ** -40, 0x3F81),  # just above the tie -> up
    (2.0 ** -126, 0x0080),                # smallest normal
    (2.0 ** -133, 0x0001),                # smallest subnormal
    (2.0 ** -134, 0x0000),                # tie between 0 and 2^-133 -> even (0)
    (3 * 2.0 ** -134, 0x0002),            # tie between 1 and 2 quanta -> even (2)
    (255 * 2.0 ** 120, 0x7F7F),           # largest finite
    (255.5 * 2.0 ** 120, 0x7F80),         # tie towards 256*2^120 -> overflow
    (float("inf"), 0x7F80),
    (-0.0, 0x8000),
])
def test_bf16_literal_cases(oracle_lib, value, bits):
    assert int(oracle_lib.bf16_from_double(np.array([value]))[0]) == bits


def test_bf16_nan(oracle_lib):
    b = int(oracle_lib.bf16_from_double(np.array([np.nan]))[0])
    assert (b & 0x7F80) == 0x7F80 and (b & 0x7F) != 0


def test_bf16_matches_torch_on_float32_values(oracle_lib):
    rng = np.random.default_rng(1)
    f = np.concatenate([
        rng.standard_normal(200000).astype(np.float32),
        (rng.standard_normal(20000) * 1e-38).astype(np.float32),   # subnormal range
        (rng.standard_normal(20000) * 1e37).astype(np.float32),
    ])
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle_lib.bf16_from_double(f.astype(np.float64))
    assert np.array_equal(got, ref)


def test_bf16_matches_integer_rne_on_doubles(oracle_lib):
    rng = np.random.default_rng(2)
    d = rng.standard_normal(300000) * np.exp(rng.uniform(-20, 20, 300000))
    # exact ties and near-ties in double (not representable as float32)
    base = pins.bf16_bits_to_f64(rng.integers(0x0100, 0x7F00, 1000, dtype=np.uint16))
    d = np.concatenate([d, base * (1 + 2.0 ** -8), base * (1 + 2.0 ** -8 + 2.0 ** -50),
                        base * (1 + 2.0 ** -8 - 2.0 ** -50)])
    assert np.array_equal(oracle_lib.bf16_from_double(d), pins.bf16_rne_bits(d))


# ---------------------------------------------------------------------------- remap


def test_remap_worked_cases(oracle_lib):
    E, S = 4, 3
    topk = np.array([[0, 3], [2, -1], [1, -7], [4, 0], [3, 1], [-2147483648, 2]], np.int32)
    lora = np.array([0, 2, -1, 1, 3, 1], np.int32)
    want = np.array([[0, 3], [10, -1], [-1, -7], [-1, 4], [-1, -1], [-2147483648, 6]],
                    np.int32)
    assert np.array_equal(oracle_lib.virtual_topk(topk, lora, E, S), want)


def test_remap_invariants(oracle_lib):
    rng = np.random.default_rng(3)
    M, k, E, S = 400, 6, 16, 5
    topk = rng.integers(-40, E + 6, size=(M, k), dtype=np.int32)
    topk[0, 0] = np.iinfo(np.int32).min
    lora = rng.integers(-2, S + 2, size=M, dtype=np.int32)
    v = oracle_lib.virtual_topk(topk, lora, E, S)
    l = np.repeat(lora, k).reshape(M, k)
    neg = topk < 0
    assert np.array_equal(v[neg], topk[neg])                      # sentinels untouched
    ok = (~neg) & (topk < E) & (l >= 0) & (l < S)
    assert np.all((v[ok] >= 0) & (v[ok] < E * S))
    assert np.array_equal(v[ok] % E, topk[ok]) and np.array_equal(v[ok] // E, l[ok])
    assert np.all(v[(~neg) & (~ok)] == -1)


# ---------------------------------------------------------------------------- align


def _check_align_invariants(srt, eid, npp, key, V, BM):
    numel = key.size
    assert npp % BM == 0 and npp == srt.size and eid.size == npp // BM
    counts = np.bincount(key, minlength=V + 1)
    assert npp == int(np.sum(-(-counts // BM) * BM))
    real = srt[srt < numel]
    assert np.array_equal(np.sort(real), np.arange(numel))        # each pair exactly once
    assert np.all(srt[srt >= numel] == numel)                     # padding value
    blocks = srt.reshape(-1, BM) if npp else srt.reshape(0, BM)
    last = -2
    seen_sentinel = False
    for b, row in enumerate(blocks):
        members = row[row < numel]
        assert members.size > 0                                   # no empty blocks
        kk = np.unique(key[members])
        assert kk.size == 1
        want = -1 if kk[0] == V else kk[0]
        assert eid[b] == want
        if eid[b] == -1:
            seen_sentinel = True
        else:
            assert not seen_sentinel and eid[b] >= last           # sentinel blocks last
            last = eid[b]
        assert np.all(np.diff(members) > 0)                       # stable inside a block
    nz = min(numel, V + 1)
    assert npp // BM <= -(-(numel + nz * (BM - 1)) // BM)


def test_align_matches_stable_argsort_bruteforce(oracle_lib):
    rng = np.random.default_rng(4)
    cases = 0
    for numel, V, BM in itertools.product(range(0, 13), range(1, 7), (1, 2, 4)):
        for _ in range(4):
            ids = rng.integers(-3, V + 3, size=(numel, 1), dtype=np.int32)
            got = oracle_lib.align_block_size(ids, None, V, 1, BM)
            want = pins.align_by_argsort(ids, None, V, 1, BM)
            assert np.array_equal(got[0], want[0]) and np.array_equal(got[1], want[1])
            assert got[2] == want[2]
            key = pins.keys_of(ids, None, V, 1)
            _check_align_invariants(got[0], got[1], got[2], key, V, BM)
            cases += 1
    assert cases == 13 * 6 * 3 * 4


def test_align_inline_remap_equals_remap_then_align(oracle_lib):
    rng = np.random.default_rng(5)
    for _ in range(50):
        M, k = int(rng.integers(0, 40)), int(rng.integers(1, 5))
        E, S, BM = int(rng.integers(1, 9)), int(rng.integers(1, 5)), int(rng.integers(1, 9))
        topk = rng.integers(-2, E + 2, size=(M, k), dtype=np.int32)
        lora = rng.integers(-1, S + 1, size=M, dtype=np.int32)
        a = oracle_lib.align_block_size(topk, lora, E, S, BM)
        v = oracle_lib.virtual_topk(topk, lora, E, S)
        b = oracle_lib.align_block_size(v, None, E * S, 1, BM)
        c = pins.align_by_argsort(topk, lora, E, S, BM)
        for x, y, z in zip(a[:2], b[:2], c[:2]):
            assert np.array_equal(x, y) and np.array_equal(x, z)
        assert a[2] == b[2] == c[2]


@pytest.mark.parametrize("cfg", [configs.C0, configs.C1, configs.C2])
def test_align_invariants_on_configs(oracle_lib, cfg):
    inp = inputs.generate(cfg, seed=0, tensors=False)
    srt, eid, npp = oracle_lib.align_block_size(inp.topk_ids, inp.lora_ids, cfg.E, cfg.S,
                                                cfg.block_m)
    key = pins.keys_of(inp.topk_ids, inp.lora_ids, cfg.E, cfg.S)
    _check_align_invariants(srt, eid, npp, key, cfg.V, cfg.block_m)
    want = pins.align_by_argsort(inp.topk_ids, inp.lora_ids, cfg.E, cfg.S, cfg.block_m)
    assert np.array_equal(srt, want[0]) and np.array_equal(eid, want[1])


def test_align_sentinel_only_and_empty(oracle_lib):
    srt, eid, npp = oracle_lib.align_block_size(np.full((5, 2), -1, np.int32), None, 4, 1, 4)
    assert npp == 12 and list(eid) == [-1, -1, -1]
    assert list(srt[:10]) == list(range(10)) and list(srt[10:]) == [10, 10]
    srt, eid, npp = oracle_lib.align_block_size(np.zeros((0, 3), np.int32), None, 4, 1, 4)
    assert npp == 0 and srt.size == 0 and eid.size == 0


# ----------------------------------------------------------------------- shrink/expand


def _run_stage(oracle_lib, inp, si, out=None, pair_mask=None):
    cfg = inp.cfg
    st, sin = cfg.stages[si], inp.stages[si]
    srt, eid, npp = oracle_lib.align_block_size(inp.topk_ids, inp.lora_ids, cfg.E, cfg.S,
                                                cfg.block_m)
    s = oracle_lib.lora_shrink(sin.xin, sin.row_div, sin.A, srt, eid, npp, cfg.numel,
                               cfg.block_m, pair_mask=pair_mask)
    if out is None:
        out = np.zeros((cfg.numel, st.N), dtype=sin.B.dtype)
    oracle_lib.lora_expand(s, st.slices, sin.B, inp.scale, cfg.E, srt, eid, npp, cfg.numel,
                           cfg.block_m, out, pair_mask=pair_mask)
    return s, out


def _small(cfg, **kw):
    return configs.scaled(cfg, **kw)


SMALL_BF16 = _small(configs.C1, name="c1_small", M=9, topk=3, hidden=96, E=6, S=3, rank=8,
                    stages=configs._two_stage(96, 40, 8), sentinel_count=4, nolora_count=2)


@pytest.mark.parametrize("cfg", [configs.C0, SMALL_BF16])
def test_delta_equals_per_pair_identity(oracle_lib, cfg):
    inp = inputs.generate(cfg, seed=0)
    vids = oracle_lib.virtual_topk(inp.topk_ids, inp.lora_ids, cfg.E, cfg.S)
    for si, st in enumerate(cfg.stages):
        sin = inp.stages[si]
        s, out = _run_stage(oracle_lib, inp, si)
        s_ref, d_ref = pins.delta_per_pair(cfg.E, cfg.S, cfg.topk, vids, st, sin.xin,
                                           sin.row_div, sin.A, sin.B, inp.scale)
        has = ~np.isnan(s_ref[:, 0])
        assert np.array_equal(has, ~np.isnan(s[:, 0]))
        np.testing.assert_allclose(s[has], s_ref[has], rtol=1e-12, atol=1e-12)
        if cfg.dtype == "f32":
            want = d_ref.astype(np.float32)
            np.testing.assert_allclose(out, want, rtol=1e-6, atol=1e-7)
        else:
            want = pins.bf16_rne_bits(d_ref)
            # the oracle rounds its own double sum; sums differ only in the last bits of
            # a double, so the rounded bf16 may differ only where d_ref sits on a tie
            assert np.mean(out == want) > 0.9999
            assert np.all(np.abs(pins.bf16_bits_to_f64(out) - d_ref)
                          <= np.abs(d_ref) * 2.0 ** -8 + 1e-30)
        assert np.all(out[~has] == 0)                             # no delta, untouched


def test_one_bucket_is_a_plain_gemm_chain(oracle_lib):
    # S = 1, E = 1, no sentinels: every pair lands on virtual expert 0, so the shrink
    # is X A_0^T and the expand is (X A_0^T) B_0^T, a plain GEMM chain.
    cfg = _small(configs.C0, name="one_bucket", M=37, hidden=48, E=1, topk=1, S=1, rank=6,
                 block_m=8, stages=(configs.Stage("lora", K=48, R=6, N=20, slices=1,
                                                  input="x"),),
                 sentinel_count=0, lora_dist="uniform", scale=0.75)
    inp = inputs.generate(cfg, seed=7)
    s, out = _run_stage(oracle_lib, inp, 0)
    X = inp.x.astype(np.float64)
    A = inp.stages[0].A[0].astype(np.float64)
    B = inp.stages[0].B[0].astype(np.float64)
    np.testing.assert_allclose(s, X @ A.T, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(out, (0.75 * (X @ A.T) @ B.T).astype(np.float32),
                               rtol=1e-6, atol=1e-7)


def test_linearity_in_scale_and_zero_A(oracle_lib):
    cfg = _small(configs.C0, name="lin", M=16, sentinel_count=3)
    inp = inputs.generate(cfg, seed=11)
    _, out1 = _run_stage(oracle_lib, inp, 0)
    inp.scale[:] = [2.0, -0.5]
    _, out2 = _run_stage(oracle_lib, inp, 0)
    vids = oracle_lib.virtual_topk(inp.topk_ids, inp.lora_ids, cfg.E, cfg.S).reshape(-1)
    for p, v in enumerate(vids):
        if 0 <= v < cfg.V:
            f = 2.0 if v // cfg.E == 0 else -0.5
            np.testing.assert_allclose(out2[p], f * out1[p], rtol=1e-6, atol=1e-7)
    inp.stages[0].A[:] = 0
    base = inputs.base_out(cfg, 0, seed=11)
    _, out3 = _run_stage(oracle_lib, inp, 0, out=base.copy())
    assert np.array_equal(out3, base)


RANKED = [
    _small(configs.C0, name="ranked_f32", slot_ranks=(5, 0)),
    _small(SMALL_BF16, name="ranked_bf16", slot_ranks=(8, 3, 0)),
]


def _zeroed_past_rank(inp):
    """The same layer with every weight past its slot's rank set to 0 and no rank table."""
    z = copy.deepcopy(inp)
    for sin in z.stages:
        for w in (sin.A, sin.B):
            bad = np.isnan(pins.bf16_bits_to_f64(w) if w.dtype == np.uint16 else w)
            w[bad] = 0
    z.slot_ranks = None
    return z


@pytest.mark.parametrize("cfg", RANKED, ids=[c.name for c in RANKED])
def test_ranked_delta_equals_full_rank_on_zeroed_weights(oracle_lib, cfg):
    # An adapter of rank rl is the full-rank path on weights that are zero past rl; the
    # ranked inputs hold NaN there, so reading one element too many shows up. Rank 0 adds
    # nothing: its rows keep the starting values bit for bit.
    inp = inputs.generate(cfg, seed=4)
    assert any(np.isnan(pins.bf16_bits_to_f64(st.A) if st.A.dtype == np.uint16 else st.A).any()
               for st in inp.stages)
    base = [inputs.base_out(cfg, si, seed=4) for si in range(len(cfg.stages))]
    (srt, eid, npp), s_r, o_r = oracle_lib.run_layer(inp, outs=[b.copy() for b in base])
    _, s_z, o_z = oracle_lib.run_layer(_zeroed_past_rank(inp), outs=[b.copy() for b in base])
    vids = oracle_lib.virtual_topk(inp.topk_ids, inp.lora_ids, cfg.E, cfg.S).reshape(-1)
    real = (vids >= 0) & (vids < cfg.V)
    zero_rank = real & (np.asarray(cfg.slot_ranks)[np.where(real, vids, 0) // cfg.E] == 0)
    for si in range(len(cfg.stages)):
        assert np.array_equal(s_r[si][real], s_z[si][real])
        assert not np.isnan(s_r[si][real]).any()
        assert np.array_equal(o_r[si], o_z[si])
        assert np.array_equal(o_r[si][zero_rank | ~real], base[si][zero_rank | ~real])
    assert zero_rank.any()


def test_full_ranks_equal_no_rank_table(oracle_lib):
    cfg = _small(SMALL_BF16, name="full_ranks", slot_ranks=(8, 8, 8))
    inp = inputs.generate(cfg, seed=2)
    _, s1, o1 = oracle_lib.run_layer(inp)
    inp.slot_ranks = None
    _, s2, o2 = oracle_lib.run_layer(inp)
    for a, b in zip(s1 + o1, s2 + o2):
        assert np.array_equal(np.nan_to_num(a, nan=7.0), np.nan_to_num(b, nan=7.0))


def test_token_permutation_permutes_rows(oracle_lib):
    cfg = SMALL_BF16
    inp = inputs.generate(cfg, seed=3)
    _, out = _run_stage(oracle_lib, inp, 0)
    perm = np.random.default_rng(0).permutation(cfg.M)
    inp.topk_ids = inp.topk_ids[perm].copy()
    inp.lora_ids = inp.lora_ids[perm].copy()
    inp.stages[0].xin = inp.x[perm].copy()
    _, outp = _run_stage(oracle_lib, inp, 0)
    pair_perm = (perm[:, None] * cfg.topk + np.arange(cfg.topk)[None, :]).reshape(-1)
    assert np.array_equal(outp, out[pair_perm])


def test_pair_mask_restricts_to_sampled_pairs(oracle_lib):
    inp = inputs.generate(SMALL_BF16, seed=0)
    s_full, o_full = _run_stage(oracle_lib, inp, 1)
    mask = np.zeros(SMALL_BF16.numel, np.uint8)
    mask[::3] = 1
    s_m, o_m = _run_stage(oracle_lib, inp, 1, pair_mask=mask)
    sel = mask.astype(bool)
    assert np.array_equal(o_m[sel], o_full[sel]) and np.all(o_m[~sel] == 0)
    np.testing.assert_array_equal(s_m[sel], s_full[sel])


def test_threads_do_not_change_results(oracle_lib):
    inp = inputs.generate(SMALL_BF16, seed=5)
    n0 = oracle_lib.num_threads()
    try:
        oracle_lib.set_num_threads(1)
        a = _run_stage(oracle_lib, inp, 0)
        oracle_lib.set_num_threads(max(2, n0))
        b = _run_stage(oracle_lib, inp, 0)
    finally:
        oracle_lib.set_num_threads(n0)
    assert np.array_equal(a[1], b[1]) and np.array_equal(a[0], b[0], equal_nan=True)


# -------------------------------------------------------------------------- combine
# The combine is the step after the down projection: per token, the router-weighted sum
# of its pair rows over the pairs whose base expert is local (0 <= t < E).


def _combine_case(dtype, M=13, k=4, N=40, E=6, seed=0, sentinels=True):
    rng = np.random.default_rng(seed)
    t = rng.integers(0, E, size=(M, k)).astype(np.int32)
    if sentinels:
        t.reshape(-1)[rng.choice(M * k, size=M * k // 5, replace=False)] = -1
        t.reshape(-1)[rng.choice(M * k, size=3, replace=False)] = E + 2  # no such expert
    w = rng.random((M, k), dtype=np.float32) + np.float32(0.05)
    rows = rng.standard_normal((M * k, N), dtype=np.float32)
    if dtype == "bf16":
        rows = inputs.f32_to_bf16_bits(rows)
    return t, w, rows


def _local(t, E):
    return (t >= 0) & (t < E)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_combine_is_a_batched_matvec(oracle_lib, dtype):
    # With every expert local, y[m] = w[m] @ rows[m*k:(m+1)*k]: numpy's batched matmul in
    # double, rounded once.
    M, k, N, E = 13, 4, 40, 6
    t, w, rows = _combine_case(dtype, M, k, N, E, seed=1, sentinels=False)
    y = oracle_lib.moe_combine(rows, t, w, E)
    ref = np.matmul(w.astype(np.float64)[:, None, :],
                    pins.to_f64(rows).reshape(M, k, N))[:, 0, :]
    if dtype == "f32":
        np.testing.assert_allclose(y, ref.astype(np.float32), rtol=1e-6, atol=1e-7)
    else:
        want = pins.bf16_rne_bits(ref)
        assert np.mean(y == want) > 0.999
        assert np.all(np.abs(pins.bf16_bits_to_f64(y) - ref) <= np.abs(ref) * 2.0 ** -8)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_combine_reads_only_local_pairs(oracle_lib, dtype):
    # Pairs whose expert is not local (negative sentinel, or an id >= E) have no row: NaN
    # there must not reach y, which equals the batched matvec with those weights zeroed.
    M, k, N, E = 13, 4, 40, 6
    t, w, rows = _combine_case(dtype, M, k, N, E, seed=2)
    off = ~_local(t, E).reshape(-1)
    assert off.any()
    nan = np.uint16(0x7FC0) if dtype == "bf16" else np.float32(np.nan)
    rows[off] = nan
    y = oracle_lib.moe_combine(rows, t, w, E)
    w0 = np.where(_local(t, E), w, 0).astype(np.float64)
    r0 = np.where(off[:, None], 0.0, pins.to_f64(rows)).reshape(M, k, N)
    ref = np.matmul(w0[:, None, :], r0)[:, 0, :]
    got = pins.to_f64(y)
    assert np.all(np.isfinite(got))
    np.testing.assert_allclose(got, ref, rtol=2.0 ** -8, atol=1e-30)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_combine_one_slot_unit_weight_is_the_row(oracle_lib, dtype):
    t, _, rows = _combine_case(dtype, M=9, k=1, N=33, E=4, seed=3, sentinels=False)
    w = np.ones((9, 1), np.float32)
    assert np.array_equal(oracle_lib.moe_combine(rows, t, w, 4), rows)


def _down_case(oracle_lib, cfg, seed):
    """One layer's down stage: its s (oracle shrink over the aligned blocks), B, base rows
    and router weights."""
    inp = inputs.generate(cfg, seed=seed)
    si = len(cfg.stages) - 1
    st, sin = cfg.stages[si], inp.stages[si]
    srt, eid, npp = oracle_lib.align_block_size(inp.topk_ids, inp.lora_ids, cfg.E, cfg.S,
                                                cfg.block_m)
    s = oracle_lib.lora_shrink(sin.xin, sin.row_div, sin.A, srt, eid, npp, cfg.numel,
                               cfg.block_m, slot_ranks=inp.slot_ranks, E=cfg.E)
    base = inputs.base_out(cfg, si, seed=seed)
    w = inputs.topk_weights(cfg, seed)
    return inp, st, sin, (srt, eid, npp), s, base, w


FUSED = [
    _small(configs.C0, name="fused_f32"),
    _small(SMALL_BF16, name="fused_bf16"),
]


@pytest.mark.parametrize("cfg", FUSED, ids=[c.name for c in FUSED])
def test_fused_combine_one_unit_slot_equals_expand(oracle_lib, cfg):
    # topk 1 with weight 1: each token's y is its pair's expanded row, rounded once from the
    # same double sum as the (pinned) expand.
    cfg = _small(cfg, name=cfg.name + "_k1", topk=1)
    inp, st, sin, (srt, eid, npp), s, base, _ = _down_case(oracle_lib, cfg, seed=6)
    inp.scale[:] = np.linspace(0.5, 2.0, cfg.S, dtype=np.float32)
    w = np.ones((cfg.M, 1), np.float32)
    y = oracle_lib.lora_expand_combine(np.nan_to_num(s), sin.B, inp.scale, inp.topk_ids,
                                       inp.lora_ids, w, cfg.E, cfg.S, base)
    out = oracle_lib.lora_expand(s, 1, sin.B, inp.scale, cfg.E, srt, eid, npp, cfg.numel,
                                 cfg.block_m, base.copy())
    local = _local(inp.topk_ids, cfg.E).reshape(-1)
    assert np.array_equal(y[local], out[local])
    assert np.all(pins.to_f64(y[~local]) == 0)


@pytest.mark.parametrize("cfg", FUSED, ids=[c.name for c in FUSED])
def test_fused_combine_equals_combine_of_expanded_rows(oracle_lib, cfg):
    # The fused form is the combine of the expanded rows taken before their rounding: in
    # f32 the two differ by the rows' float rounding only; in bf16 by at most one
    # rounding of each row (2^-9 relative) plus the final one.
    inp, st, sin, (srt, eid, npp), s, base, w = _down_case(oracle_lib, cfg, seed=8)
    inp.scale[:] = np.linspace(0.5, 2.0, cfg.S, dtype=np.float32)
    y = oracle_lib.lora_expand_combine(np.nan_to_num(s), sin.B, inp.scale, inp.topk_ids,
                                       inp.lora_ids, w, cfg.E, cfg.S, base)
    rows = oracle_lib.lora_expand(s, 1, sin.B, inp.scale, cfg.E, srt, eid, npp, cfg.numel,
                                  cfg.block_m, base.copy())
    y2 = oracle_lib.moe_combine(rows, inp.topk_ids, w, cfg.E)
    a, b = pins.to_f64(y), pins.to_f64(y2)
    wabs = np.abs(w).astype(np.float64)
    mag = np.matmul(wabs[:, None, :], np.abs(pins.to_f64(rows)).reshape(cfg.M, cfg.topk, -1))[:, 0]
    tol = (2.0 ** -8 if cfg.dtype == "bf16" else 2.0 ** -22) * (mag + np.abs(a))
    assert np.all(np.abs(a - b) <= tol + 1e-30)


@pytest.mark.parametrize("cfg", FUSED, ids=[c.name for c in FUSED])
def test_fused_combine_without_adapters_is_the_base_combine(oracle_lib, cfg):
    # No token has an adapter: no delta anywhere, so the fused form is the combine of the
    # base rows, term for term.
    inp, st, sin, _, s, base, w = _down_case(oracle_lib, cfg, seed=9)
    none = np.full(cfg.M, -1, np.int32)
    y = oracle_lib.lora_expand_combine(np.full_like(s, np.nan), sin.B, inp.scale,
                                       inp.topk_ids, none, w, cfg.E, cfg.S, base)
    assert np.array_equal(y, oracle_lib.moe_combine(base, inp.topk_ids, w, cfg.E))


def test_fused_combine_ranked_equals_full_rank_on_zeroed_weights(oracle_lib):
    cfg = _small(SMALL_BF16, name="fused_ranked", slot_ranks=(8, 3, 0))
    inp, st, sin, _, s, base, w = _down_case(oracle_lib, cfg, seed=10)
    assert np.isnan(pins.bf16_bits_to_f64(sin.B)).any()
    y = oracle_lib.lora_expand_combine(np.nan_to_num(s), sin.B, inp.scale, inp.topk_ids,
                                       inp.lora_ids, w, cfg.E, cfg.S, base,
                                       slot_ranks=inp.slot_ranks)
    z = _zeroed_past_rank(inp)
    y0 = oracle_lib.lora_expand_combine(np.nan_to_num(s), z.stages[-1].B, inp.scale,
                                        inp.topk_ids, inp.lora_ids, w, cfg.E, cfg.S, base)
    assert np.array_equal(y, y0)


# ------------------------------------------------------ base grouped GEMM (+ fused delta)
# The base MoE GEMM of a stage: out[p] = W[t_p] x_row(p) for pairs with a local expert,
# optionally with the LoRA delta added before the one rounding.

GEMM = [
    _small(configs.C0, name="gemm_f32"),
    _small(SMALL_BF16, name="gemm_bf16"),
    _small(SMALL_BF16, name="gemm_ranked", slot_ranks=(8, 3, 0)),
]


def _gemm_case(oracle_lib, cfg, seed, si=0):
    inp = inputs.generate(cfg, seed=seed)
    st, sin = cfg.stages[si], inp.stages[si]
    W = inputs.base_weights(cfg, si, seed)
    srt, eid, npp = oracle_lib.align_block_size(inp.topk_ids, inp.lora_ids, cfg.E, cfg.S,
                                                cfg.block_m)
    s = oracle_lib.lora_shrink(sin.xin, sin.row_div, sin.A, srt, eid, npp, cfg.numel,
                               cfg.block_m, slices=st.slices, slot_ranks=inp.slot_ranks,
                               E=cfg.E)
    base = inputs.base_out(cfg, si, seed)
    return inp, st, sin, W, (srt, eid, npp), s, base


@pytest.mark.parametrize("cfg", GEMM[:2], ids=[c.name for c in GEMM[:2]])
def test_base_gemm_is_a_per_pair_matvec(oracle_lib, cfg):
    # numpy: each local pair's row is W[t] @ x, in double, rounded once; other rows untouched
    inp, st, sin, W, _, _, start = _gemm_case(oracle_lib, cfg, seed=1)
    out = oracle_lib.moe_gemm(sin.xin, sin.row_div, W, inp.topk_ids, cfg.E, start.copy())
    t = inp.topk_ids.reshape(-1)
    local = (t >= 0) & (t < cfg.E)
    Wd, Xd = pins.to_f64(W), pins.to_f64(sin.xin)
    rows = np.arange(cfg.numel) // sin.row_div
    ref = np.einsum("pnk,pk->pn", Wd[np.where(local, t, 0)], Xd[rows])
    got = pins.to_f64(out)
    half = 2.0 ** -8 if cfg.dtype == "bf16" else 2.0 ** -23
    assert np.all(np.abs(got[local] - ref[local]) <= half * np.abs(ref[local]) + 1e-30)
    assert np.array_equal(out[~local], start[~local])
    assert local.any() and (~local).any()


@pytest.mark.parametrize("cfg", GEMM, ids=[c.name for c in GEMM])
def test_fused_gemm_reduces_to_its_parts(oracle_lib, cfg):
    inp, st, sin, W, (srt, eid, npp), s, start = _gemm_case(oracle_lib, cfg, seed=2)
    inp.scale[:] = np.linspace(0.5, 2.0, cfg.S, dtype=np.float32)
    s0 = np.nan_to_num(s)
    kw = dict(s=s0, slices=st.slices, B=sin.B, scale=inp.scale, lora_ids=inp.lora_ids,
              S=cfg.S, slot_ranks=inp.slot_ranks)
    base_only = oracle_lib.moe_gemm(sin.xin, sin.row_div, W, inp.topk_ids, cfg.E, start.copy())
    # zero scale: exactly the base GEMM
    z = dict(kw, scale=np.zeros_like(inp.scale))
    assert np.array_equal(
        oracle_lib.moe_gemm(sin.xin, sin.row_div, W, inp.topk_ids, cfg.E, start.copy(), **z),
        base_only)
    # zero base weights: exactly the expand from zero rows, on the local pairs
    fused0 = oracle_lib.moe_gemm(sin.xin, sin.row_div, np.zeros_like(W), inp.topk_ids, cfg.E,
                                 start.copy(), **kw)
    exp0 = oracle_lib.lora_expand(s, st.slices, sin.B, inp.scale, cfg.E, srt, eid, npp,
                                  cfg.numel, cfg.block_m, np.zeros_like(start),
                                  slot_ranks=inp.slot_ranks)
    t = inp.topk_ids.reshape(-1)
    local = (t >= 0) & (t < cfg.E)
    assert np.array_equal(fused0[local], exp0[local])
    # no adapters: the base GEMM
    none = dict(kw, lora_ids=np.full(cfg.M, -1, np.int32))
    assert np.array_equal(
        oracle_lib.moe_gemm(sin.xin, sin.row_div, W, inp.topk_ids, cfg.E, start.copy(), **none),
        base_only)
    # the full fused row: base + delta within one rounding of the row (and of each part)
    fused = oracle_lib.moe_gemm(sin.xin, sin.row_div, W, inp.topk_ids, cfg.E, start.copy(), **kw)
    a, b, d = pins.to_f64(fused), pins.to_f64(base_only), pins.to_f64(exp0)
    ulp = 2.0 ** -7 if cfg.dtype == "bf16" else 2.0 ** -22
    tol = ulp * (np.abs(a) + np.abs(b) + np.abs(d)) + 1e-30
    assert np.all(np.abs(a - (b + d))[local] <= tol[local])
    assert np.array_equal(fused[~local], start[~local])
