"""CPU oracle for the MoL delta path: a ctypes binding over `oracle.c`.

TEST INFRASTRUCTURE ONLY: imported by the tests, by the package smoke check and by the
benchmark's CPU-baseline leg, never by the GPU path. See `oracle.c` for what each
function computes and which passage of the pages it follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

F32, BF16 = 0, 1


def build(force: bool = False) -> str:
    """Compile oracle.c with the host C compiler (-O2, no -march=native, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-fopenmp",
                        "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        P, I32, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        L.oracle_num_threads.argtypes, L.oracle_num_threads.restype = [], ctypes.c_int
        L.oracle_set_num_threads.argtypes, L.oracle_set_num_threads.restype = [ctypes.c_int], None
        L.oracle_bf16_from_double.argtypes = [ctypes.c_double]
        L.oracle_bf16_from_double.restype = ctypes.c_uint16
        L.oracle_bf16_round_array.argtypes, L.oracle_bf16_round_array.restype = [P, P, I64], None
        L.oracle_virtual_topk.argtypes = [P, P, I64, I32, I32, I32, P]
        L.oracle_virtual_topk.restype = ctypes.c_int
        L.oracle_align_block_size.argtypes = [P, P, I64, I32, I32, I32, I32, P, I64, P, I64, P]
        L.oracle_align_block_size.restype = ctypes.c_int
        L.oracle_lora_shrink.argtypes = [ctypes.c_int, P, I64, I32, P, I32, I32, P, P, I32,
                                         I64, I32, P, P, I32, P, I32]
        L.oracle_lora_shrink.restype = ctypes.c_int
        L.oracle_lora_expand.argtypes = [ctypes.c_int, P, I32, I32, P, I32, P, I32, P, P, I32,
                                         I64, I32, P, P, I64, P]
        L.oracle_lora_expand.restype = ctypes.c_int
        L.oracle_moe_combine.argtypes = [ctypes.c_int, P, I64, P, P, I64, I32, I32, I32, P, I64]
        L.oracle_moe_combine.restype = ctypes.c_int
        L.oracle_lora_expand_combine.argtypes = [ctypes.c_int, P, I32, P, I32, P, P, P, P, P,
                                                 I64, I32, I32, I32, P, I64, P, I64]
        L.oracle_lora_expand_combine.restype = ctypes.c_int
        L.oracle_moe_gemm.argtypes = [ctypes.c_int, P, I64, I32, P, I32, I32, P, I64, I32, I32,
                                      P, I64, P, I32, I32, P, P, P, P, I32]
        L.oracle_moe_gemm.restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _dt(a) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError(f"oracle takes float32 or bf16 bits (uint16), not {a.dtype}")


def num_threads() -> int:
    return lib().oracle_num_threads()


def set_num_threads(n: int) -> None:
    lib().oracle_set_num_threads(int(n))


def bf16_from_double(v) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.uint16)
    lib().oracle_bf16_round_array(_ptr(v), _ptr(out), v.size)
    return out


def virtual_topk(topk_ids, lora_ids, E: int, S: int) -> np.ndarray:
    t = np.ascontiguousarray(topk_ids, dtype=np.int32)
    l = np.ascontiguousarray(lora_ids, dtype=np.int32)
    M, k = t.shape
    out = np.empty_like(t)
    rc = lib().oracle_virtual_topk(_ptr(t), _ptr(l), M, k, E, S, _ptr(out))
    if rc:
        raise ValueError(f"oracle_virtual_topk: {rc}")
    return out


def align_block_size(ids, lora_ids, E: int, S: int, block_m: int):
    """Returns (sorted_ids[:npp], expert_ids[:npp/BM], npp)."""
    t = np.ascontiguousarray(ids, dtype=np.int32)
    M, k = t.shape
    numel = M * k
    V = E * S
    nz = min(numel, V + 1)
    cap_blocks = max(1, (numel + nz * (block_m - 1) + block_m - 1) // block_m)
    sorted_ids = np.empty(cap_blocks * block_m, dtype=np.int32)
    expert_ids = np.empty(cap_blocks, dtype=np.int32)
    npp = np.zeros(1, dtype=np.int32)
    l = None if lora_ids is None else np.ascontiguousarray(lora_ids, dtype=np.int32)
    rc = lib().oracle_align_block_size(_ptr(t), _ptr(l), M, k, E, S, block_m,
                                       _ptr(sorted_ids), sorted_ids.size,
                                       _ptr(expert_ids), expert_ids.size, _ptr(npp))
    if rc:
        raise ValueError(f"oracle_align_block_size: {rc}")
    n = int(npp[0])
    return sorted_ids[:n].copy(), expert_ids[: n // block_m].copy(), n


def _ranks(slot_ranks):
    return None if slot_ranks is None else np.ascontiguousarray(slot_ranks, dtype=np.int32)


def lora_shrink(xin, row_div: int, A, sorted_ids, expert_ids, npp: int, numel: int,
                block_m: int, pair_mask=None, s=None, slices: int = 1, slot_ranks=None,
                E: int = 1) -> np.ndarray:
    """s [numel, R] float64; rows of pairs that get no delta stay as given (NaN). With
    slot_ranks (int32 [S]; slot = v / E), entries past a slot's rank in each of the
    `slices` slices are 0."""
    xin = np.ascontiguousarray(xin)
    A = np.ascontiguousarray(A)
    V, R, K = A.shape
    if s is None:
        s = np.full((numel, R), np.nan, dtype=np.float64)
    srt = np.ascontiguousarray(sorted_ids, dtype=np.int32)
    eid = np.ascontiguousarray(expert_ids, dtype=np.int32)
    mask = None if pair_mask is None else np.ascontiguousarray(pair_mask, dtype=np.uint8)
    rk = _ranks(slot_ranks)
    rc = lib().oracle_lora_shrink(_dt(A), _ptr(xin), xin.shape[1], row_div, _ptr(A), R, K,
                                  _ptr(srt), _ptr(eid), npp, numel, block_m, _ptr(mask),
                                  _ptr(s), slices, _ptr(rk), E)
    if rc:
        raise ValueError(f"oracle_lora_shrink: {rc}")
    return s


def lora_expand(s, slices: int, B, scale, E: int, sorted_ids, expert_ids, npp: int,
                numel: int, block_m: int, out, pair_mask=None, slot_ranks=None) -> np.ndarray:
    """Adds the delta into `out` [numel, N] (float32 or bf16 bits) in place; with
    slot_ranks, only a slot's first rank dimensions count and rank 0 adds nothing."""
    s = np.ascontiguousarray(s, dtype=np.float64)
    B = np.ascontiguousarray(B)
    V, N, r = B.shape
    R = s.shape[1]
    assert out.flags.c_contiguous and out.dtype == B.dtype
    sc = np.ascontiguousarray(scale, dtype=np.float32)
    srt = np.ascontiguousarray(sorted_ids, dtype=np.int32)
    eid = np.ascontiguousarray(expert_ids, dtype=np.int32)
    mask = None if pair_mask is None else np.ascontiguousarray(pair_mask, dtype=np.uint8)
    rk = _ranks(slot_ranks)
    rc = lib().oracle_lora_expand(_dt(B), _ptr(s), R, slices, _ptr(B), N, _ptr(sc), E,
                                  _ptr(srt), _ptr(eid), npp, numel, block_m, _ptr(mask),
                                  _ptr(out), out.shape[1], _ptr(rk))
    if rc:
        raise ValueError(f"oracle_lora_expand: {rc}")
    return out


def moe_combine(rows, topk_ids, topk_weights, E: int) -> np.ndarray:
    """y [M, N] (rows' dtype) = per token the weighted sum of its pair rows (rows
    [M*topk, N]) over the pairs with a local base expert, rounded once."""
    rows = np.ascontiguousarray(rows)
    t = np.ascontiguousarray(topk_ids, dtype=np.int32)
    w = np.ascontiguousarray(topk_weights, dtype=np.float32)
    M, k = t.shape
    assert w.shape == (M, k) and rows.shape[0] == M * k
    N = rows.shape[1]
    y = np.zeros((M, N), dtype=rows.dtype)
    rc = lib().oracle_moe_combine(_dt(rows), _ptr(rows), N, _ptr(t), _ptr(w), M, k, E, N,
                                  _ptr(y), N)
    if rc:
        raise ValueError(f"oracle_moe_combine: {rc}")
    return y


def lora_expand_combine(s, B, scale, topk_ids, lora_ids, topk_weights, E: int, S: int,
                        base, slot_ranks=None) -> np.ndarray:
    """The down stage's expand fused with the combine: y [M, N] from s [M*topk, R]
    (float64), B [V, N, R], base rows [M*topk, N]; nothing rounded before the end."""
    s = np.ascontiguousarray(s, dtype=np.float64)
    B = np.ascontiguousarray(B)
    base = np.ascontiguousarray(base)
    V, N, R = B.shape
    t = np.ascontiguousarray(topk_ids, dtype=np.int32)
    l = np.ascontiguousarray(lora_ids, dtype=np.int32)
    w = np.ascontiguousarray(topk_weights, dtype=np.float32)
    M, k = t.shape
    assert s.shape == (M * k, R) and base.shape == (M * k, N) and base.dtype == B.dtype
    sc = np.ascontiguousarray(scale, dtype=np.float32)
    rk = _ranks(slot_ranks)
    y = np.zeros((M, N), dtype=B.dtype)
    rc = lib().oracle_lora_expand_combine(_dt(B), _ptr(s), R, _ptr(B), N, _ptr(sc), _ptr(rk),
                                          _ptr(t), _ptr(l), _ptr(w), M, k, E, S, _ptr(base),
                                          N, _ptr(y), N)
    if rc:
        raise ValueError(f"oracle_lora_expand_combine: {rc}")
    return y


def moe_gemm(xin, row_div: int, W, topk_ids, E: int, out, s=None, slices: int = 1, B=None,
             scale=None, lora_ids=None, S: int = 1, slot_ranks=None) -> np.ndarray:
    """The base grouped GEMM of a stage into `out` [M*topk, N] (rows of pairs without a local
    expert untouched); with s (float64 [M*topk, R]) and B, the LoRA delta is added before the
    one rounding."""
    xin = np.ascontiguousarray(xin)
    W = np.ascontiguousarray(W)
    Ew, N, K = W.shape
    assert Ew == E and out.flags.c_contiguous and out.dtype == W.dtype
    t = np.ascontiguousarray(topk_ids, dtype=np.int32)
    M, k = t.shape
    args = [None, 0, 1, None, None, None, None, 1]
    if s is not None:
        s = np.ascontiguousarray(s, dtype=np.float64)
        B = np.ascontiguousarray(B)
        assert B.dtype == W.dtype
        args = [s, s.shape[1], slices, B, np.ascontiguousarray(scale, dtype=np.float32),
                _ranks(slot_ranks), np.ascontiguousarray(lora_ids, dtype=np.int32), S]
    rc = lib().oracle_moe_gemm(_dt(W), _ptr(xin), xin.shape[1], row_div, _ptr(W), K, N,
                               _ptr(t), M, k, E, _ptr(out), out.shape[1], _ptr(args[0]),
                               args[1], args[2], _ptr(args[3]), _ptr(args[4]), _ptr(args[5]),
                               _ptr(args[6]), args[7])
    if rc:
        raise ValueError(f"oracle_moe_gemm: {rc}")
    return out


def run_layer(inp, outs=None, pair_mask=None):
    """The whole path on one layer's inputs: align with the remap inline, then each
    stage's shrink and expand. `outs` (one array per stage, [numel, N]) start at zero
    unless given. Returns (routing, s per stage, out per stage)."""
    cfg = inp.cfg
    numel = cfg.numel
    srt, eid, npp = align_block_size(inp.topk_ids, inp.lora_ids, cfg.E, cfg.S, cfg.block_m)
    ss, oo = [], []
    for si, (st, sin) in enumerate(zip(cfg.stages, inp.stages)):
        ranks = getattr(inp, "slot_ranks", None)
        s = lora_shrink(sin.xin, sin.row_div, sin.A, srt, eid, npp, numel, cfg.block_m,
                        pair_mask=pair_mask, slices=st.slices, slot_ranks=ranks, E=cfg.E)
        if outs is None:
            out = np.zeros((numel, st.N), dtype=sin.B.dtype)
        else:
            out = outs[si]
        lora_expand(s, st.slices, sin.B, inp.scale, cfg.E, srt, eid, npp, numel,
                    cfg.block_m, out, pair_mask=pair_mask, slot_ranks=ranks)
        ss.append(s)
        oo.append(out)
    return (srt, eid, npp), ss, oo
