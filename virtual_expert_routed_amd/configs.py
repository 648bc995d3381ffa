"""Shapes of the synthetic MoL (multi-LoRA MoE) layers the path is exercised on: the five
workloads C0-C4 and N2, the pages' own decode shape.

A layer routes M tokens to `topk` of E base experts and gives every token one LoRA
slot out of S, so a (token, slot) pair lands on virtual expert  v = e + slot * E,
V = E * S of them (virtual-experts page, the remap passage of "sglang PR 24171").
Each stage is one shrink (K -> R) followed by one expand (R/slices -> N per slice):

* gate_up: K = hidden, R = 2r, N = 2 * moe_intermediate, 2 slices (gate, up);
* down:    K = moe_intermediate, R = r, N = hidden, 1 slice.

The tiny fp32 layer has a single stage (K = 64, R = r = 8, N = 32).
Distributions of the draws live in `inputs.py`; nothing here computes anything.
"""
from __future__ import annotations

from dataclasses import dataclass, field


@dataclass(frozen=True)
class Stage:
    name: str
    K: int          # contraction length of the shrink (input row width)
    R: int          # shrink output width (rank * slices)
    N: int          # expand output width (all slices together)
    slices: int     # expand slices; slice g uses s[:, g*r:(g+1)*r] and owns N/slices columns
    input: str      # "x": token rows (row = pair // topk); "h": pair rows (row = pair)

    @property
    def r(self) -> int:
        return self.R // self.slices


@dataclass(frozen=True)
class LayerConfig:
    name: str
    dtype: str                 # "f32" or "bf16": x, h, A, B and out all use it
    M: int                     # tokens
    hidden: int
    E: int                     # routed experts
    topk: int
    S: int                     # LoRA slots
    rank: int
    block_m: int
    stages: tuple
    expert_dist: str           # "iid" | "uniform" (no replacement) | "zipf" (no replacement)
    sentinel_count: int        # pair slots forced to -1 (expert-parallel dispatch drops)
    nolora_count: int          # tokens forced to lora = -1 (no adapter)
    lora_dist: str             # "uniform" over [0,S) or "c0" over {-1,0,1}
    x_sigma: float = 1.0
    w_sigma: float = 0.02
    h_sigma: float = 1.0
    scale: float = 1.0
    zipf_s: float = 1.1
    slot_ranks: tuple = None   # per LoRA slot rank (<= rank; 0 = no delta), None = all full
    note: str = field(default="", compare=False)

    @property
    def V(self) -> int:
        return self.E * self.S

    @property
    def numel(self) -> int:
        return self.M * self.topk


def _round_half_up(frac: float, count: int) -> int:
    # fractions of a count become exact counts, halves rounded up
    return int(frac * count + 0.5)


def _two_stage(hidden: int, inter: int, rank: int):
    return (
        Stage("gate_up", K=hidden, R=2 * rank, N=2 * inter, slices=2, input="x"),
        Stage("down", K=inter, R=rank, N=hidden, slices=1, input="h"),
    )


C0 = LayerConfig(
    name="c0_tiny_f32", dtype="f32", M=8, hidden=64, E=4, topk=2, S=2, rank=8, block_m=16,
    stages=(Stage("lora", K=64, R=8, N=32, slices=1, input="x"),),
    expert_dist="iid", sentinel_count=1, nolora_count=0, lora_dist="c0",
    w_sigma=0.1, note="tiny MoL layer, fp32, seed 0")

C1 = LayerConfig(
    name="c1_decode_bs23", dtype="bf16", M=23, hidden=2048, E=128, topk=8, S=8, rank=32,
    block_m=64, stages=_two_stage(2048, 768, 32), expert_dist="uniform",
    sentinel_count=_round_half_up(0.05, 23 * 8), nolora_count=_round_half_up(0.10, 23),
    lora_dist="uniform", note="decode bs=23, 30B-A3B-shaped MoE layer, 8 slots")

C2 = LayerConfig(
    name="c2_decode_bs128_zipf", dtype="bf16", M=128, hidden=2048, E=128, topk=8, S=16,
    rank=32, block_m=64, stages=_two_stage(2048, 768, 32), expert_dist="zipf",
    sentinel_count=_round_half_up(0.05, 128 * 8), nolora_count=_round_half_up(0.10, 128),
    lora_dist="uniform", note="decode bs=128, Zipf(1.1) experts, 16 slots")

C3 = LayerConfig(
    name="c3_prefill_4096_v8064", dtype="bf16", M=4096, hidden=2048, E=128, topk=8, S=63,
    rank=32, block_m=64, stages=_two_stage(2048, 768, 32), expert_dist="uniform",
    sentinel_count=_round_half_up(0.02, 4096 * 8), nolora_count=0, lora_dist="uniform",
    note="prefill chunk, 8064 virtual experts (near the 8191 ceiling)")

C4 = LayerConfig(
    name="c4_prefill_16384_r64", dtype="bf16", M=16384, hidden=4096, E=128, topk=8, S=16,
    rank=64, block_m=64, stages=_two_stage(4096, 1536, 64), expert_dist="zipf",
    sentinel_count=_round_half_up(0.02, 16384 * 8), nolora_count=0, lora_dist="uniform",
    note="large prefill, rank 64, Zipf(1.1) experts")

# The decode shape the MindLab sglang PR 24 page measures (its root-cause passage and the PR
# body's background section): a speculative-verify step of 23 requests with about 1.1 k routed
# (token, virtual expert) pairs, BLOCK_M = 64, rank 32; the LoRA gate and up expands have
# N = 256 each (one two-slice stage here, N = 512) and the down expand N = 6144, so the
# hidden size is 6144 and the per-GPU intermediate 256. The pages give neither the token
# count nor E and S: 138 tokens (23 x 6) at top-8 give 1104 pair slots, and E = 160, S = 10
# put the worst-case routing buffer at 1594 blocks of 64 against the page's 1604.
N2 = LayerConfig(
    name="n2_verify_h6144", dtype="bf16", M=138, hidden=6144, E=160, topk=8, S=10, rank=32,
    block_m=64, stages=_two_stage(6144, 256, 32), expert_dist="uniform",
    sentinel_count=_round_half_up(0.02, 138 * 8), nolora_count=0, lora_dist="uniform",
    note="the pages' decode shape: ~1.1 k pairs, down expand N = 6144, r = 32")

CONFIGS = (C0, C1, C2, C3, C4, N2)
BY_NAME = {c.name: c for c in CONFIGS}


def scaled(cfg: LayerConfig, **overrides) -> LayerConfig:
    """A copy of `cfg` with some fields replaced (smaller parity cases)."""
    d = {f: getattr(cfg, f) for f in cfg.__dataclass_fields__}
    d.update(overrides)
    return LayerConfig(**d)
