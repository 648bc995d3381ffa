"""Seeded synthetic inputs for one MoL layer.

This module only draws numbers: it holds none of the method's arithmetic (no remap, no
routing, no products). The oracle's tests and the GPU path both take their inputs from
here, so the two see bit-identical data.

Recipe (one numpy PCG64 stream per (config, seed), drawn in this fixed order):

1. top-k expert ids [M, topk] int32:
   * "iid":     independent integers in [0, E);
   * "uniform": per token, the first `topk` entries of a random permutation of the
     E experts (argsort of uniforms), i.e. uniform without replacement;
   * "zipf":    Gumbel-top-k over log p(e) with p(e) proportional to (e+1)^-zipf_s,
     which is sequential weighted sampling without replacement (expert 0 hottest).
2. `sentinel_count` distinct pair slots (chosen without replacement) set to -1, the
   id expert-parallel dispatch leaves for a pair this GPU does not own.
3. LoRA slot per token [M] int32: uniform over [0, S), or over {-1, 0, 1} ("c0").
4. `nolora_count` distinct tokens set to slot -1 (no adapter).
5. x [M, hidden] ~ N(0, x_sigma).
6. h [M*topk, K_down] ~ N(0, h_sigma) for a stage that reads pair rows (the down
   projection's input; the activation that really produces it lies outside the path).
7. For each stage in order: A [V, R, K] then B [V, N, R/slices], both N(0, w_sigma).

Outside that stream (each from its own PCG64 stream keyed by (seed, tag), so the layer's
draws above never move):
* base_out: nonzero starting rows for an expand's output, N(0, 1);
* base_weights [E, N, K]: a stage's base expert weights, N(0, w_sigma), for the base grouped
  GEMM that the delta can be fused into;
* topk_weights [M, topk] float32: the router's combine weights, a softmax over `topk`
  standard-normal logits per token (positive, summing to 1 per token, as a renormalised
  top-k softmax router gives).

Normals are drawn in float32 (numpy's standard_normal), scaled in float32, and for bf16
configs rounded to bfloat16 with round-to-nearest-even; bf16 arrays are kept as their
uint16 bit patterns. Weights are drawn in slabs of virtual experts so the float32
staging stays small; the slab size does not change the values.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .configs import LayerConfig

_SLAB_ELEMS = 1 << 24


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest, ties to even.

    Only finite draws reach this (normals), so NaN handling is not needed here."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class StageInputs:
    A: np.ndarray        # [V, R, K]  float32 or uint16 (bf16 bits)
    B: np.ndarray        # [V, N, r]
    xin: np.ndarray      # the shrink's input rows: x [M, K] or h [numel, K]
    row_div: int         # pair p reads xin row p // row_div


@dataclass
class LayerInputs:
    cfg: object
    seed: int
    topk_ids: np.ndarray     # [M, topk] int32
    lora_ids: np.ndarray     # [M] int32
    x: np.ndarray
    stages: list             # StageInputs per cfg.stages
    scale: np.ndarray        # [S] float32
    slot_ranks: np.ndarray = None  # [S] int32 or None (every slot at full rank)


def _normals(rng, shape, sigma, dtype):
    n = int(np.prod(shape))
    if dtype == "f32":
        out = np.empty(n, dtype=np.float32)
    else:
        out = np.empty(n, dtype=np.uint16)
    for s0 in range(0, n, _SLAB_ELEMS):
        s1 = min(n, s0 + _SLAB_ELEMS)
        v = rng.standard_normal(s1 - s0, dtype=np.float32)
        if sigma != 1.0:
            v *= np.float32(sigma)
        out[s0:s1] = v if dtype == "f32" else f32_to_bf16_bits(v)
    return out.reshape(shape)


def _draw_topk(rng, cfg: LayerConfig) -> np.ndarray:
    M, E, k = cfg.M, cfg.E, cfg.topk
    if cfg.expert_dist == "iid":
        t = rng.integers(0, E, size=(M, k))
    elif cfg.expert_dist == "uniform":
        t = np.argsort(rng.random((M, E)), axis=1, kind="stable")[:, :k]
    elif cfg.expert_dist == "zipf":
        logp = -cfg.zipf_s * np.log(np.arange(1, E + 1, dtype=np.float64))
        g = -np.log(-np.log(rng.random((M, E))))
        t = np.argsort(-(logp[None, :] + g), axis=1, kind="stable")[:, :k]
    else:
        raise ValueError(cfg.expert_dist)
    return np.ascontiguousarray(t, dtype=np.int32)


def generate(cfg: LayerConfig, seed: int = 0, tensors: bool = True) -> LayerInputs:
    """All of one layer's inputs. With tensors=False only the routing (steps 1-4) is
    drawn; it is identical to the routing of the full draw."""
    rng = np.random.default_rng(seed)
    topk = _draw_topk(rng, cfg)
    numel = cfg.M * cfg.topk
    if cfg.sentinel_count:
        pos = rng.choice(numel, size=cfg.sentinel_count, replace=False)
        topk.reshape(-1)[pos] = -1
    if cfg.lora_dist == "uniform":
        lora = rng.integers(0, cfg.S, size=cfg.M)
    elif cfg.lora_dist == "c0":
        lora = rng.integers(-1, 2, size=cfg.M)
    else:
        raise ValueError(cfg.lora_dist)
    lora = np.ascontiguousarray(lora, dtype=np.int32)
    if cfg.nolora_count:
        lora[rng.choice(cfg.M, size=cfg.nolora_count, replace=False)] = -1
    scale = np.full(cfg.S, cfg.scale, dtype=np.float32)
    if not tensors:
        return LayerInputs(cfg=cfg, seed=seed, topk_ids=topk, lora_ids=lora, x=None,
                           stages=[], scale=scale)
    x = _normals(rng, (cfg.M, cfg.hidden), cfg.x_sigma, cfg.dtype)
    h = {}
    for st in cfg.stages:
        if st.input == "h":
            h[st.name] = _normals(rng, (numel, st.K), cfg.h_sigma, cfg.dtype)
    stages = []
    V = cfg.V
    for st in cfg.stages:
        A = _normals(rng, (V, st.R, st.K), cfg.w_sigma, cfg.dtype)
        B = _normals(rng, (V, st.N, st.r), cfg.w_sigma, cfg.dtype)
        if st.input == "x":
            xin, row_div = x, cfg.topk
        else:
            xin, row_div = h[st.name], 1
        if cfg.slot_ranks is not None:
            _poison_past_rank(cfg, st, A, B)
        stages.append(StageInputs(A=A, B=B, xin=xin, row_div=row_div))
    ranks = None if cfg.slot_ranks is None else np.asarray(cfg.slot_ranks, dtype=np.int32)
    return LayerInputs(cfg=cfg, seed=seed, topk_ids=topk, lora_ids=lora, x=x,
                       stages=stages, scale=scale, slot_ranks=ranks)


def _poison_past_rank(cfg, st, A, B):
    """A slot of rank rl < r leaves rank dimensions [rl, r) of each slice unused; fill them
    with NaN (as stale pool memory could hold anything) so that reading them shows."""
    nan = np.uint16(0x7FC0) if cfg.dtype == "bf16" else np.float32(np.nan)
    for l, rl in enumerate(cfg.slot_ranks):
        v = slice(l * cfg.E, (l + 1) * cfg.E)
        for g in range(st.slices):
            A[v, g * st.r + rl:(g + 1) * st.r, :] = nan
        B[v, :, rl:] = nan


def base_out(cfg: LayerConfig, stage_index: int, seed: int) -> np.ndarray:
    """A nonzero starting value for an expand's output rows, ~N(0,1), from its own
    stream (seed, stage) so it does not disturb the layer's draws."""
    st = cfg.stages[stage_index]
    rng = np.random.default_rng([seed, 1000 + stage_index])
    return _normals(rng, (cfg.M * cfg.topk, st.N), 1.0, cfg.dtype)


def topk_weights(cfg: LayerConfig, seed: int) -> np.ndarray:
    """Router combine weights [M, topk] float32 from their own stream (seed, 2000)."""
    rng = np.random.default_rng([seed, 2000])
    z = rng.standard_normal((cfg.M, cfg.topk), dtype=np.float32)
    e = np.exp(z - z.max(axis=1, keepdims=True))
    return np.ascontiguousarray(e / e.sum(axis=1, keepdims=True), dtype=np.float32)


def base_weights(cfg: LayerConfig, stage_index: int, seed: int) -> np.ndarray:
    """A stage's base expert weights [E, N, K] ~ N(0, w_sigma) from their own stream
    (seed, 3000 + stage)."""
    st = cfg.stages[stage_index]
    rng = np.random.default_rng([seed, 3000 + stage_index])
    return _normals(rng, (cfg.E, st.N, st.K), cfg.w_sigma, cfg.dtype)


def sha256(inp: LayerInputs) -> str:
    """SHA-256 over every array of one layer's inputs, in a fixed order (routing ids, slot
    scales and ranks, x, then per stage its input rows, A and B), so a run's results can
    name exactly the data they were measured on."""
    import hashlib
    h = hashlib.sha256()
    arrays = [inp.topk_ids, inp.lora_ids, inp.scale]
    if inp.slot_ranks is not None:
        arrays.append(inp.slot_ranks)
    if inp.x is not None:
        arrays.append(inp.x)
    for st in inp.stages:
        arrays += [st.xin, st.A, st.B]
    for a in arrays:
        a = np.ascontiguousarray(a)
        h.update(str((a.dtype.str, a.shape)).encode())
        h.update(memoryview(a).cast("B"))
    return h.hexdigest()

