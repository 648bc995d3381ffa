"""ctypes binding over libmol.so (include/mol.h), with the same entry point names.

Argument marshalling only: tensors become device pointers, torch's current stream becomes
the hipStream_t, missing outputs are allocated with torch. Every step of the path runs in
the HIP kernels of libmol; there is no fallback of any kind - if the library is missing or
a call fails, this raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# MOL_LIBRARY names another build of the same library (the host-sanitizer build of the CPU
# tests); by default, the one built in-tree
LIB_PATH = os.environ.get("MOL_LIBRARY") or os.path.join(_PKG, "libmol.so")

MOL_OK, MOL_E_ARG, MOL_E_LIMIT, MOL_E_DTYPE, MOL_E_ALIGN, MOL_E_WORKSPACE, MOL_E_HIP = range(7)
MOL_F32, MOL_BF16 = 0, 1
MOL_MAX_BUCKETS = 8192

# every symbol include/mol.h declares, with (restype, argtypes)
_P, _I32, _I64, _SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
SIGNATURES = {
    "mol_status_string": (ctypes.c_char_p, [_I32]),
    "mol_abi_version": (_I32, []),
    "mol_virtual_topk": (_I32, [_P, _P, _I32, _I32, _I32, _I32, _P, _P]),
    "mol_align_max_blocks": (_I64, [_I64, _I32, _I32]),
    "mol_align_workspace_bytes": (_I64, [_I64, _I32, _I32]),
    "mol_plan_bytes": (_I64, [_I64, _I32, _I32]),
    "mol_align_block_size": (_I32, [_P, _P, _I32, _I32, _I32, _I32, _I32, _P, _P, _P, _P, _SZ,
                                    _P, _SZ, _P]),
    "mol_lora_shrink": (_I32, [_I32, _P, _I64, _I32, _P, _I32, _I32, _I32, _P, _I32, _P, _P,
                               _P, _I32, _I32, _I32, _P, _P]),
    "mol_lora_expand": (_I32, [_I32, _P, _I32, _I32, _P, _I32, _P, _P, _I32, _P, _P, _P, _P,
                               _I32, _I32, _I32, _P, _I64, _P]),
    "mol_delta_workspace_bytes": (_I64, [_I32, _I32, _I32, _I32]),
    "mol_lora_delta": (_I32, [_I32, _P, _I64, _I32, _P, _I32, _I32, _I32, _P, _I32, _P, _P,
                              _I32, _P, _P, _P, _P, _I32, _I32, _I32, _P, _I64, _P, _SZ, _P]),
    "mol_lora_delta_noalloc": (_I32, [_I32, _P, _I64, _I32, _P, _I32, _I32, _I32, _P, _I32, _P,
                                      _P, _I32, _P, _P, _P, _P, _I32, _I32, _I32, _P, _I64,
                                      _P]),
    "mol_moe_gemm": (_I32, [_I32, _P, _I64, _I32, _P, _I32, _I32, _I32, _P, _P, _P, _I32, _I32,
                            _P, _I64, _P, _I32, _I32, _P, _P, _P, _P, _I32, _I32, _P]),
    "mol_moe_combine": (_I32, [_I32, _P, _I64, _P, _P, _I32, _I32, _I32, _I32, _P, _I64, _P]),
    "mol_lora_expand_combine": (_I32, [_I32, _P, _I32, _P, _I32, _P, _P, _P, _P, _P, _I32,
                                       _I32, _I32, _I32, _P, _I64, _P, _I64, _P]),
}


class MolError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {status_string(status)} (status {status})")


_lib = None


def lib() -> ctypes.CDLL:
    """Load libmol.so once (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m virtual_expert_routed_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype, fn.argtypes = res, args
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().mol_status_string(int(status)).decode()


def _check(fn: str, status: int) -> None:
    if status != MOL_OK:
        raise MolError(fn, status)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t=None):
    dev = t.device if t is not None and t.is_cuda else None
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return MOL_F32
    if t.dtype == torch.bfloat16:
        return MOL_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _need(t: torch.Tensor, name: str, dtype=None, contiguous=True):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


# ------------------------------------------------------------------------------- sizing


def mol_align_max_blocks(numel: int, num_virtual: int, block_m: int) -> int:
    v = lib().mol_align_max_blocks(numel, num_virtual, block_m)
    if v < 0:
        raise MolError("mol_align_max_blocks", -v)
    return int(v)


def mol_align_workspace_bytes(numel: int, num_virtual: int, block_m: int) -> int:
    v = lib().mol_align_workspace_bytes(numel, num_virtual, block_m)
    if v < 0:
        raise MolError("mol_align_workspace_bytes", -v)
    return int(v)


def mol_plan_bytes(numel: int, num_virtual: int, block_m: int) -> int:
    v = lib().mol_plan_bytes(numel, num_virtual, block_m)
    if v < 0:
        raise MolError("mol_plan_bytes", -v)
    return int(v)


def new_plan(numel: int, num_virtual: int, block_m: int, device):
    """A buffer for the align's work plan (int32; written by mol_align_block_size)."""
    n = mol_plan_bytes(numel, num_virtual, block_m)
    return torch.empty(max(64, n // 4), dtype=torch.int32, device=device)


def mol_delta_workspace_bytes(numel: int, R: int, num_virtual: int, block_m: int) -> int:
    v = lib().mol_delta_workspace_bytes(numel, R, num_virtual, block_m)
    if v < 0:
        raise MolError("mol_delta_workspace_bytes", -v)
    return int(v)


# -------------------------------------------------------------------------- entry points


def mol_virtual_topk(topk_ids, lora_ids, num_experts: int, num_slots: int, out=None):
    _need(topk_ids, "topk_ids", torch.int32)
    _need(lora_ids, "lora_ids", torch.int32)
    M, k = topk_ids.shape
    if out is None:
        out = torch.empty_like(topk_ids)
    _need(out, "out", torch.int32)
    _check("mol_virtual_topk", lib().mol_virtual_topk(
        _ptr(topk_ids), _ptr(lora_ids), M, k, num_experts, num_slots, _ptr(out),
        _stream(topk_ids)))
    return out


def mol_align_block_size(ids, lora_ids, num_experts: int, num_slots: int, block_m: int,
                         sorted_ids=None, expert_ids=None, num_post_padded=None,
                         workspace=None, plan=None):
    """Returns (sorted_ids, expert_ids, num_post_padded) sized by mol_align_max_blocks. With
    plan (an int32 tensor of mol_plan_bytes), the work plan is written there as well."""
    _need(ids, "ids", torch.int32)
    if lora_ids is not None:
        _need(lora_ids, "lora_ids", torch.int32)
    M, k = ids.shape
    V = num_experts * num_slots
    mb = mol_align_max_blocks(M * k, V, block_m)
    dev = ids.device
    if sorted_ids is None:
        sorted_ids = torch.empty(max(1, mb * block_m), dtype=torch.int32, device=dev)
    if expert_ids is None:
        expert_ids = torch.empty(max(1, mb), dtype=torch.int32, device=dev)
    if num_post_padded is None:
        num_post_padded = torch.empty(1, dtype=torch.int32, device=dev)
    wsb = mol_align_workspace_bytes(M * k, V, block_m)
    if wsb and workspace is None:
        workspace = torch.empty(wsb, dtype=torch.uint8, device=dev)
    if plan is not None:
        _need(plan, "plan", torch.int32)
    _check("mol_align_block_size", lib().mol_align_block_size(
        _ptr(ids), _ptr(lora_ids), M, k, num_experts, num_slots, block_m, _ptr(sorted_ids),
        _ptr(expert_ids), _ptr(num_post_padded), _ptr(plan),
        plan.numel() * 4 if plan is not None else 0, _ptr(workspace) if wsb else None,
        workspace.numel() if (wsb and workspace is not None) else 0, _stream(ids)))
    return sorted_ids, expert_ids, num_post_padded


def _ranks(slot_ranks):
    if slot_ranks is not None:
        _need(slot_ranks, "slot_ranks", torch.int32)
    return _ptr(slot_ranks)


def mol_lora_shrink(xin, row_div: int, A, sorted_ids, expert_ids, num_post_padded,
                    numel: int, num_virtual: int, block_m: int, s=None, slices: int = 1,
                    slot_ranks=None, num_experts: int = None):
    _need(xin, "xin", contiguous=False)
    _need(A, "A")
    if xin.stride(1) != 1:
        raise ValueError("xin rows must be contiguous")
    V, R, K = A.shape
    if s is None:
        s = torch.empty((max(1, numel), R), dtype=torch.float32, device=A.device)
    _need(s, "s", torch.float32)
    E = num_virtual if num_experts is None else num_experts
    _check("mol_lora_shrink", lib().mol_lora_shrink(
        _dtype_code(A), _ptr(xin), xin.stride(0), row_div, _ptr(A), R, K, slices,
        _ranks(slot_ranks), E, _ptr(sorted_ids), _ptr(expert_ids), _ptr(num_post_padded),
        numel, num_virtual, block_m, _ptr(s), _stream(A)))
    return s


def mol_lora_expand(s, slices: int, B, slot_scale, num_experts: int, sorted_ids, expert_ids,
                    num_post_padded, numel: int, num_virtual: int, block_m: int, out,
                    slot_ranks=None, plan=None):
    _need(B, "B")
    _need(s, "s", torch.float32)
    _need(slot_scale, "slot_scale", torch.float32)
    _need(out, "out", B.dtype, contiguous=False)
    if out.stride(1) != 1:
        raise ValueError("out rows must be contiguous")
    V, N, r = B.shape
    _check("mol_lora_expand", lib().mol_lora_expand(
        _dtype_code(B), _ptr(s), s.shape[1], slices, _ptr(B), N, _ptr(slot_scale),
        _ranks(slot_ranks), num_experts, _ptr(sorted_ids), _ptr(expert_ids),
        _ptr(num_post_padded), _ptr(plan), numel, num_virtual, block_m, _ptr(out),
        out.stride(0), _stream(B)))
    return out


def new_delta_workspace(numel: int, R: int, num_virtual: int, block_m: int, device):
    """A workspace for mol_lora_delta (its contents need no initialisation)."""
    n = mol_delta_workspace_bytes(numel, R, num_virtual, block_m)
    return torch.empty(max(256, n), dtype=torch.uint8, device=device)


def mol_lora_delta(xin, row_div: int, A, slices: int, B, slot_scale, num_experts: int,
                   sorted_ids, expert_ids, num_post_padded, numel: int, num_virtual: int,
                   block_m: int, out, workspace, slot_ranks=None, plan=None):
    _need(xin, "xin", contiguous=False)
    _need(A, "A")
    _need(B, "B")
    _need(slot_scale, "slot_scale", torch.float32)
    _need(out, "out", B.dtype, contiguous=False)
    _need(workspace, "workspace", torch.uint8)
    if xin.stride(1) != 1 or out.stride(1) != 1:
        raise ValueError("xin and out rows must be contiguous")
    V, R, K = A.shape
    _, N, r = B.shape
    _check("mol_lora_delta", lib().mol_lora_delta(
        _dtype_code(A), _ptr(xin), xin.stride(0), row_div, _ptr(A), R, K, slices, _ptr(B), N,
        _ptr(slot_scale), _ranks(slot_ranks), num_experts, _ptr(sorted_ids), _ptr(expert_ids),
        _ptr(num_post_padded), _ptr(plan), numel, num_virtual, block_m, _ptr(out), out.stride(0),
        _ptr(workspace), workspace.numel(), _stream(A)))
    return out


def mol_lora_delta_noalloc(xin, row_div: int, A, slices: int, B, slot_scale, num_experts: int,
                           sorted_ids, expert_ids, num_post_padded, numel: int,
                           num_virtual: int, block_m: int, out, slot_ranks=None, plan=None):
    """mol_lora_delta with s in the library's own per-GPU scratch: no workspace argument and
    nothing allocated (numel * R <= MOL_DELTA_SCRATCH_FLOATS; calls that overlap on one
    GPU race)."""
    _need(xin, "xin", contiguous=False)
    _need(A, "A")
    _need(B, "B")
    _need(slot_scale, "slot_scale", torch.float32)
    _need(out, "out", B.dtype, contiguous=False)
    if xin.stride(1) != 1 or out.stride(1) != 1:
        raise ValueError("xin and out rows must be contiguous")
    V, R, K = A.shape
    _, N, r = B.shape
    _check("mol_lora_delta_noalloc", lib().mol_lora_delta_noalloc(
        _dtype_code(A), _ptr(xin), xin.stride(0), row_div, _ptr(A), R, K, slices, _ptr(B), N,
        _ptr(slot_scale), _ranks(slot_ranks), num_experts, _ptr(sorted_ids), _ptr(expert_ids),
        _ptr(num_post_padded), _ptr(plan), numel, num_virtual, block_m, _ptr(out), out.stride(0),
        _stream(A)))
    return out


MOL_DELTA_SCRATCH_FLOATS = 4 * 1024 * 1024


def mol_moe_combine(rows, topk_ids, topk_weights, num_experts: int, y=None):
    """y [M, N] = per token the router-weighted sum of its pair rows [M*topk, N]."""
    _need(rows, "rows", contiguous=False)
    _need(topk_ids, "topk_ids", torch.int32)
    _need(topk_weights, "topk_weights", torch.float32)
    if rows.stride(1) != 1:
        raise ValueError("rows must have contiguous rows")
    M, k = topk_ids.shape
    N = rows.shape[1]
    if y is None:
        y = torch.empty((M, N), dtype=rows.dtype, device=rows.device)
    _need(y, "y", rows.dtype, contiguous=False)
    _check("mol_moe_combine", lib().mol_moe_combine(
        _dtype_code(rows), _ptr(rows), rows.stride(0), _ptr(topk_ids), _ptr(topk_weights), M,
        k, num_experts, N, _ptr(y), y.stride(0), _stream(rows)))
    return y


def mol_lora_expand_combine(s, B, slot_scale, topk_ids, lora_ids, topk_weights,
                            num_experts: int, num_slots: int, base, y=None, slot_ranks=None):
    """The down stage's expand fused with the combine: y [M, N] from s [M*topk, R], B
    [E*S, N, R] and the pairs' base rows [M*topk, N]; the rows are not written."""
    _need(B, "B")
    _need(s, "s", torch.float32)
    _need(slot_scale, "slot_scale", torch.float32)
    _need(topk_ids, "topk_ids", torch.int32)
    _need(lora_ids, "lora_ids", torch.int32)
    _need(topk_weights, "topk_weights", torch.float32)
    _need(base, "base", B.dtype, contiguous=False)
    if base.stride(1) != 1:
        raise ValueError("base must have contiguous rows")
    V, N, R = B.shape
    M, k = topk_ids.shape
    if y is None:
        y = torch.empty((M, N), dtype=B.dtype, device=B.device)
    _need(y, "y", B.dtype, contiguous=False)
    _check("mol_lora_expand_combine", lib().mol_lora_expand_combine(
        _dtype_code(B), _ptr(s), R, _ptr(B), N, _ptr(slot_scale), _ranks(slot_ranks),
        _ptr(topk_ids), _ptr(lora_ids), _ptr(topk_weights), M, k, num_experts, num_slots,
        _ptr(base), base.stride(0), _ptr(y), y.stride(0), _stream(B)))
    return y


def mol_moe_gemm(xin, row_div: int, W, sorted_ids, expert_ids, num_post_padded, numel: int,
                 block_m: int, out, s=None, slices: int = 1, B=None, slot_scale=None,
                 lora_ids=None, topk: int = 1, num_slots: int = 1, slot_ranks=None):
    """The base grouped GEMM of a stage into out [numel, N] (routing by base expert); with
    s and B the LoRA delta is added before the one rounding."""
    _need(xin, "xin", contiguous=False)
    _need(W, "W")
    _need(out, "out", W.dtype, contiguous=False)
    if xin.stride(1) != 1 or out.stride(1) != 1:
        raise ValueError("xin and out rows must be contiguous")
    E, N, K = W.shape
    R = 0
    if s is not None:
        _need(s, "s", torch.float32)
        _need(B, "B", W.dtype)
        _need(slot_scale, "slot_scale", torch.float32)
        _need(lora_ids, "lora_ids", torch.int32)
        R = s.shape[1]
    _check("mol_moe_gemm", lib().mol_moe_gemm(
        _dtype_code(W), _ptr(xin), xin.stride(0), row_div, _ptr(W), K, N, E, _ptr(sorted_ids),
        _ptr(expert_ids), _ptr(num_post_padded), numel, block_m, _ptr(out), out.stride(0),
        _ptr(s), R, slices, _ptr(B), _ptr(slot_scale), _ranks(slot_ranks), _ptr(lora_ids), topk,
        num_slots, _stream(W)))
    return out
