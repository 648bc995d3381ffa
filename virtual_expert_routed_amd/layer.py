"""One MoL layer resident on the GPU: uploaded inputs, routing buffers, workspaces and
outputs, and the calls that run the path on them through the C ABI.

Plumbing only: torch allocates device memory and supplies the stream; every step of the
path (remap, align, shrink, expand) runs in libmol's kernels.
"""
from __future__ import annotations

import numpy as np
import torch

from . import binding as mb
from .inputs import LayerInputs


def to_device(a: np.ndarray, device, bf16: bool) -> torch.Tensor:
    if bf16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(
            torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


class DeviceLayer:
    def __init__(self, inp: LayerInputs, device="cuda", outs=None, topk_weights=None,
                 use_plan=True):
        cfg = inp.cfg
        self.cfg = cfg
        self.device = torch.device(device)
        bf16 = cfg.dtype == "bf16"
        self.bf16 = bf16
        dev = self.device
        self.topk_ids = torch.from_numpy(inp.topk_ids).to(dev)
        self.lora_ids = torch.from_numpy(inp.lora_ids).to(dev)
        self.scale = torch.from_numpy(inp.scale).to(dev)
        ranks = getattr(inp, "slot_ranks", None)
        self.slot_ranks = None if ranks is None else torch.from_numpy(ranks).to(dev)
        x = to_device(inp.x, dev, bf16)
        self.A, self.B, self.xin, self.row_div = [], [], [], []
        for st, sin in zip(cfg.stages, inp.stages):
            self.A.append(to_device(sin.A, dev, bf16))
            self.B.append(to_device(sin.B, dev, bf16))
            self.xin.append(x if st.input == "x" else to_device(sin.xin, dev, bf16))
            self.row_div.append(sin.row_div)
        numel, V, BM = cfg.numel, cfg.V, cfg.block_m
        nblk = mb.mol_align_max_blocks(numel, V, BM)
        self.max_blocks = nblk
        self.sorted_ids = torch.empty(max(1, nblk * BM), dtype=torch.int32, device=dev)
        self.expert_ids = torch.empty(max(1, nblk), dtype=torch.int32, device=dev)
        self.npp = torch.empty(1, dtype=torch.int32, device=dev)
        wsb = mb.mol_align_workspace_bytes(numel, V, BM)
        self.align_ws = torch.empty(max(256, wsb), dtype=torch.uint8, device=dev)
        # the align's work plan, which the expand then takes its work items from
        self.plan = mb.new_plan(numel, V, BM, dev) if use_plan else None
        self.delta_ws = [mb.new_delta_workspace(numel, st.R, V, BM, dev) for st in cfg.stages]
        self.s = [torch.empty((max(1, numel), st.R), dtype=torch.float32, device=dev)
                  for st in cfg.stages]
        odt = torch.bfloat16 if bf16 else torch.float32
        if outs is None:
            self.out = [torch.zeros((numel, st.N), dtype=odt, device=dev) for st in cfg.stages]
        else:
            self.out = [to_device(o, dev, bf16) for o in outs]
        # the combine after the last (down) stage: router weights and per-token output
        self.topk_weights = self.y = None
        if topk_weights is not None:
            self.topk_weights = torch.from_numpy(
                np.ascontiguousarray(topk_weights, dtype=np.float32)).to(dev)
            self.y = torch.zeros((cfg.M, cfg.stages[-1].N), dtype=odt, device=dev)

    def attach_base(self, weights):
        """Base expert weights per stage ([E, N, K] each) for the base grouped GEMM, with its
        own routing buffers (by base expert: one slot)."""
        c = self.cfg
        dev = self.device
        self.W = [to_device(w, dev, self.bf16) for w in weights]
        nblk = mb.mol_align_max_blocks(c.numel, c.E, c.block_m)
        self.b_sorted = torch.empty(max(1, nblk * c.block_m), dtype=torch.int32, device=dev)
        self.b_expert = torch.empty(max(1, nblk), dtype=torch.int32, device=dev)
        self.b_npp = torch.empty(1, dtype=torch.int32, device=dev)
        wsb = mb.mol_align_workspace_bytes(c.numel, c.E, c.block_m)
        self.b_ws = torch.empty(max(256, wsb), dtype=torch.uint8, device=dev)

    def align_base(self):
        c = self.cfg
        mb.mol_align_block_size(self.topk_ids, None, c.E, 1, c.block_m, self.b_sorted,
                                self.b_expert, self.b_npp, self.b_ws)

    def base_gemm(self, si: int, fused: bool):
        """The stage's base grouped GEMM into out[si]; fused: with the LoRA delta (from this
        stage's s, computed by shrink()) in its epilogue."""
        c = self.cfg
        st = c.stages[si]
        kw = {}
        if fused:
            kw = dict(s=self.s[si], slices=st.slices, B=self.B[si], slot_scale=self.scale,
                      lora_ids=self.lora_ids, topk=c.topk, num_slots=c.S,
                      slot_ranks=self.slot_ranks)
        mb.mol_moe_gemm(self.xin[si], self.row_div[si], self.W[si], self.b_sorted, self.b_expert,
                        self.b_npp, c.numel, c.block_m, self.out[si], **kw)
        return self.out[si]

    # ---------------------------------------------------------------------------- steps
    def align(self):
        c = self.cfg
        mb.mol_align_block_size(self.topk_ids, self.lora_ids, c.E, c.S, c.block_m,
                                self.sorted_ids, self.expert_ids, self.npp, self.align_ws,
                                plan=self.plan)

    def remap(self):
        c = self.cfg
        return mb.mol_virtual_topk(self.topk_ids, self.lora_ids, c.E, c.S)

    def routing(self):
        return self.sorted_ids, self.expert_ids, self.npp

    def shrink(self, si: int):
        c = self.cfg
        mb.mol_lora_shrink(self.xin[si], self.row_div[si], self.A[si], *self.routing(),
                           c.numel, c.V, c.block_m, s=self.s[si], slices=c.stages[si].slices,
                           slot_ranks=self.slot_ranks, num_experts=c.E)
        return self.s[si]

    def expand(self, si: int):
        c = self.cfg
        st = c.stages[si]
        mb.mol_lora_expand(self.s[si], st.slices, self.B[si], self.scale, c.E, *self.routing(),
                           c.numel, c.V, c.block_m, self.out[si], slot_ranks=self.slot_ranks,
                           plan=self.plan)
        return self.out[si]

    def delta(self, si: int):
        c = self.cfg
        st = c.stages[si]
        mb.mol_lora_delta(self.xin[si], self.row_div[si], self.A[si], st.slices, self.B[si],
                          self.scale, c.E, *self.routing(), c.numel, c.V, c.block_m,
                          self.out[si], self.delta_ws[si], slot_ranks=self.slot_ranks,
                          plan=self.plan)
        return self.out[si]

    def combine(self, rows=None):
        """y = per token the router-weighted sum of its rows of the down stage's out."""
        c = self.cfg
        rows = self.out[-1] if rows is None else rows
        return mb.mol_moe_combine(rows, self.topk_ids, self.topk_weights, c.E, y=self.y)

    def expand_combine(self, base=None):
        """The down stage's expand fused with the combine: y from the down stage's s and
        the pairs' base rows (default: the down stage's out, which is not written)."""
        c = self.cfg
        base = self.out[-1] if base is None else base
        return mb.mol_lora_expand_combine(self.s[-1], self.B[-1], self.scale, self.topk_ids,
                                          self.lora_ids, self.topk_weights, c.E, c.S, base,
                                          y=self.y, slot_ranks=self.slot_ranks)

    def y_host(self) -> np.ndarray:
        if self.bf16:
            return self.y.view(torch.int16).cpu().numpy().view(np.uint16)
        return self.y.cpu().numpy()

    def run(self, fused: bool = True):
        """The whole path: align (remap inline), then every stage's shrink + expand."""
        self.align()
        for si in range(len(self.cfg.stages)):
            if fused:
                self.delta(si)
            else:
                self.shrink(si)
                self.expand(si)
        return self.out

    # ------------------------------------------------------------------------ readback
    def routing_host(self):
        npp = int(self.npp.item())
        BM = self.cfg.block_m
        return (self.sorted_ids[:npp].cpu().numpy(), self.expert_ids[: npp // BM].cpu().numpy(),
                npp)

    def out_host(self, si: int) -> np.ndarray:
        o = self.out[si]
        if self.bf16:
            return o.view(torch.int16).cpu().numpy().view(np.uint16)
        return o.cpu().numpy()
