"""Host-only checks of the C ABI: the library loads, exports every declared symbol, and
rejects bad arguments before touching the device (no call here launches anything)."""
import ctypes
import os
import re

import pytest

from tests import conftest
from virtual_expert_routed_amd import binding as mb

HEADER = os.path.join(conftest.ROOT, "include", "mol.h")


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"MOL_API\s+[\w\s\*]+?\b(mol_\w+)\s*\(", text)))


def test_header_declares_the_five_path_calls():
    syms = declared_symbols()
    for name in ("mol_virtual_topk", "mol_align_block_size", "mol_lora_shrink",
                 "mol_lora_expand", "mol_lora_delta"):
        assert name in syms


def test_library_exports_every_declared_symbol():
    L = mb.lib()
    for name in declared_symbols():
        assert hasattr(L, name), name
    assert set(declared_symbols()) == set(mb.SIGNATURES)


def test_only_mol_symbols_exported():
    out = os.popen(f"nm -D --defined-only {mb.LIB_PATH}").read()
    funcs = [ln.split()[-1] for ln in out.splitlines() if " T " in ln]
    assert funcs and all(f.startswith("mol_") for f in funcs), funcs


def test_version_and_status_strings():
    L = mb.lib()
    assert L.mol_abi_version() == 7
    for code in range(7):
        assert mb.status_string(code)
    assert mb.status_string(99) == "unknown status"


def _cdiv(a, b):
    return -(-a // b)


@pytest.mark.parametrize("numel,V,BM", [(0, 8, 16), (16, 8, 16), (184, 1024, 64),
                                        (1024, 2048, 64), (32768, 8064, 64),
                                        (131072, 2048, 64), (5, 1, 1), (7, 8191, 1024)])
def test_align_max_blocks_formula(numel, V, BM):
    nz = min(numel, V + 1)
    assert mb.mol_align_max_blocks(numel, V, BM) == _cdiv(numel + nz * (BM - 1), BM)


def test_align_bucket_ceiling():
    # 8191 virtual experts + the sentinel bucket = 8192 buckets is the largest allowed
    assert mb.mol_align_max_blocks(10, 8191, 64) > 0
    with pytest.raises(mb.MolError) as e:
        mb.mol_align_max_blocks(10, 8192, 64)
    assert e.value.status == mb.MOL_E_LIMIT


def test_align_workspace_small_and_large():
    assert mb.mol_align_workspace_bytes(4096, 8191, 64) == 0
    ws = mb.mol_align_workspace_bytes(32768, 8064, 64)
    assert ws >= (16 * 8065 + 2 * 8065) * 4 and ws % 256 == 0


def test_delta_workspace_bytes():
    n = mb.mol_delta_workspace_bytes(184, 64, 1024, 64)
    assert n >= 184 * 64 * 4 and n % 256 == 0


P = ctypes.c_void_p
FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every call below fails validation


def test_align_rejects_before_launch():
    L = mb.lib()
    # too many buckets
    assert L.mol_align_block_size(FAKE, FAKE, 4, 2, 4096, 2, 64, FAKE, FAKE, FAKE, None, 0, None, 0,
                                  None) == mb.MOL_E_LIMIT
    # null outputs
    assert L.mol_align_block_size(FAKE, None, 4, 2, 8, 2, 16, None, FAKE, FAKE, None, 0, None, 0,
                                  None) == mb.MOL_E_ARG
    assert L.mol_align_block_size(FAKE, None, 4, 2, 8, 2, 16, FAKE, FAKE, None, None, 0, None, 0,
                                  None) == mb.MOL_E_ARG
    # bad sizes
    assert L.mol_align_block_size(FAKE, None, -1, 2, 8, 2, 16, FAKE, FAKE, FAKE, None, 0, None, 0,
                                  None) == mb.MOL_E_ARG
    assert L.mol_align_block_size(FAKE, None, 4, 2, 8, 2, 2048, FAKE, FAKE, FAKE, None, 0, None, 0,
                                  None) == mb.MOL_E_LIMIT
    # large path without workspace
    assert L.mol_align_block_size(FAKE, None, 5000, 1, 8, 2, 16, FAKE, FAKE, FAKE, None, 0, None, 0,
                                  None) == mb.MOL_E_WORKSPACE


def test_align_plan_sizing_and_checks():
    L = mb.lib()
    # the plan's room: a header of 8 words, then runs of 4 words, at most one per block of a
    # real bucket (every such block holds a pair): min(max_blocks, numel)
    for numel, V, bm in ((184, 1024, 64), (1024, 2048, 64), (32768, 8064, 64),
                         (131072, 2048, 64), (16, 8, 16), (0, 8, 16), (5000, 7, 1)):
        mb_ = mb.mol_align_max_blocks(numel, V, bm)
        words = 8 + 4 * min(mb_, numel)
        assert mb.mol_plan_bytes(numel, V, bm) == -(-words * 4 // 256) * 256
    # a plan buffer that is too small, or misaligned
    need = mb.mol_plan_bytes(16, 16, 16)
    assert L.mol_align_block_size(FAKE, None, 8, 2, 8, 2, 16, FAKE, FAKE, FAKE, FAKE, need - 4,
                                  None, 0, None) == mb.MOL_E_WORKSPACE
    assert L.mol_align_block_size(FAKE, None, 8, 2, 8, 2, 16, FAKE, FAKE, FAKE,
                                  ctypes.c_void_p(0x1004), need, None, 0,
                                  None) == mb.MOL_E_ALIGN


def test_remap_rejects_before_launch():
    L = mb.lib()
    assert L.mol_virtual_topk(None, FAKE, 3, 2, 4, 2, FAKE, None) == mb.MOL_E_ARG
    assert L.mol_virtual_topk(FAKE, FAKE, 3, 0, 4, 2, FAKE, None) == mb.MOL_E_ARG
    assert L.mol_virtual_topk(FAKE, FAKE, 0, 2, 4, 2, FAKE, None) == mb.MOL_OK  # M = 0


def test_shrink_expand_delta_reject_before_launch():
    L = mb.lib()
    # shrink: unknown dtype, K not a multiple of 16 bytes, misaligned pointer
    assert L.mol_lora_shrink(7, FAKE, 64, 1, FAKE, 8, 64, 1, None, 8, FAKE, FAKE, FAKE, 16, 8,
                             16, FAKE, None) == mb.MOL_E_DTYPE
    assert L.mol_lora_shrink(mb.MOL_BF16, FAKE, 68, 1, FAKE, 8, 60, 1, None, 8, FAKE, FAKE,
                             FAKE, 16, 8, 16, FAKE, None) == mb.MOL_E_ALIGN
    assert L.mol_lora_shrink(mb.MOL_F32, ctypes.c_void_p(0x1004), 64, 1, FAKE, 8, 64, 1, None,
                             8, FAKE, FAKE, FAKE, 16, 8, 16, FAKE, None) == mb.MOL_E_ALIGN
    assert L.mol_lora_shrink(mb.MOL_F32, FAKE, 32, 1, FAKE, 8, 64, 1, None, 8, FAKE, FAKE,
                             FAKE, 16, 8, 16, FAKE, None) == mb.MOL_E_ARG           # ld_x < K
    assert L.mol_lora_shrink(mb.MOL_BF16, FAKE, 64, 1, FAKE, 8, 64, 1, None, 8, FAKE, FAKE,
                             FAKE, 16, 8, 16, ctypes.c_void_p(0x1008), None) == mb.MOL_E_ALIGN
    assert L.mol_lora_shrink(mb.MOL_BF16, FAKE, 64, 1, FAKE, 8, 64, 3, None, 8, FAKE, FAKE,
                             FAKE, 16, 8, 16, FAKE, None) == mb.MOL_E_ARG     # R % slices
    assert L.mol_lora_shrink(mb.MOL_BF16, FAKE, 64, 1, FAKE, 8, 64, 1, None, 3, FAKE, FAKE,
                             FAKE, 16, 8, 16, FAKE, None) == mb.MOL_E_ARG     # V % E
    # expand: R % slices, rank too large, V not a multiple of E
    assert L.mol_lora_expand(mb.MOL_BF16, FAKE, 63, 2, FAKE, 32, FAKE, None, 4, FAKE, FAKE,
                             FAKE, None, 16, 8, 16, FAKE, 32, None) == mb.MOL_E_ARG
    assert L.mol_lora_expand(mb.MOL_BF16, FAKE, 512, 2, FAKE, 32, FAKE, None, 4, FAKE, FAKE,
                             FAKE, None, 16, 8, 16, FAKE, 32, None) == mb.MOL_E_LIMIT
    assert L.mol_lora_expand(mb.MOL_BF16, FAKE, 16, 1, FAKE, 32, FAKE, None, 3, FAKE, FAKE,
                             FAKE, None, 16, 8, 16, FAKE, 32, None) == mb.MOL_E_ARG
    assert L.mol_lora_expand(mb.MOL_BF16, ctypes.c_void_p(0x1008), 16, 1, FAKE, 32, FAKE, None,
                             4, FAKE, FAKE, FAKE, None, 16, 8, 16, FAKE, 32, None) == mb.MOL_E_ALIGN
    # delta: workspace missing or too small
    assert L.mol_lora_delta(mb.MOL_BF16, FAKE, 64, 1, FAKE, 16, 64, 1, FAKE, 32, FAKE, None, 4,
                            FAKE, FAKE, FAKE, None, 16, 8, 16, FAKE, 32, None, 0,
                            None) == mb.MOL_E_WORKSPACE
    assert L.mol_lora_delta(mb.MOL_BF16, FAKE, 64, 1, FAKE, 16, 64, 1, FAKE, 32, FAKE, None, 4,
                            FAKE, FAKE, FAKE, None, 16, 8, 16, FAKE, 32, FAKE, 64,
                            None) == mb.MOL_E_WORKSPACE
    # numel == 0 is a no-op
    assert L.mol_lora_delta(mb.MOL_BF16, None, 64, 1, None, 16, 64, 1, None, 32, None, None, 4,
                            None, None, None, None, 0, 8, 16, None, 32, None, 0, None) == mb.MOL_OK


def test_noalloc_delta_rejects_before_launch():
    L = mb.lib()

    def noalloc(numel=16, R=16, K=64, out=FAKE, dtype=mb.MOL_BF16):
        return L.mol_lora_delta_noalloc(dtype, FAKE, K, 1, FAKE, R, K, 1, FAKE, 32, FAKE, None,
                                        4, FAKE, FAKE, FAKE, None, numel, 8, 16, out, 32, None)

    # s of numel * R floats must fit the library's scratch
    assert noalloc(numel=mb.MOL_DELTA_SCRATCH_FLOATS // 16 + 1) == mb.MOL_E_LIMIT
    assert noalloc(dtype=6) == mb.MOL_E_DTYPE
    assert noalloc(out=None) == mb.MOL_E_ARG
    assert noalloc(K=60) == mb.MOL_E_ALIGN
    assert noalloc(numel=0) == mb.MOL_OK  # a no-op: nothing looked up, nothing enqueued
    text = open(HEADER).read()
    assert f"#define MOL_DELTA_SCRATCH_FLOATS (4 * 1024 * 1024)" in text
    assert mb.MOL_DELTA_SCRATCH_FLOATS == 4 * 1024 * 1024


def test_library_is_built_for_gfx950():
    from virtual_expert_routed_amd import build
    assert any("gfx950" in ln for ln in build.code_objects(mb.LIB_PATH))


def test_combine_rejects_before_launch():
    L = mb.lib()
    # combine: dtype, sizes, null pointers, 16-byte rows, misaligned base
    assert L.mol_moe_combine(5, FAKE, 64, FAKE, FAKE, 4, 2, 8, 64, FAKE, 64,
                             None) == mb.MOL_E_DTYPE
    assert L.mol_moe_combine(mb.MOL_BF16, FAKE, 64, FAKE, FAKE, 4, 0, 8, 64, FAKE, 64,
                             None) == mb.MOL_E_ARG                              # topk 0
    assert L.mol_moe_combine(mb.MOL_BF16, FAKE, 32, FAKE, FAKE, 4, 2, 8, 64, FAKE, 64,
                             None) == mb.MOL_E_ARG                              # ld_rows < N
    assert L.mol_moe_combine(mb.MOL_BF16, None, 64, FAKE, FAKE, 4, 2, 8, 64, FAKE, 64,
                             None) == mb.MOL_E_ARG
    assert L.mol_moe_combine(mb.MOL_BF16, FAKE, 60, FAKE, FAKE, 4, 2, 8, 60, FAKE, 60,
                             None) == mb.MOL_E_ALIGN                            # N % 8
    assert L.mol_moe_combine(mb.MOL_F32, ctypes.c_void_p(0x1008), 64, FAKE, FAKE, 4, 2, 8, 64,
                             FAKE, 64, None) == mb.MOL_E_ALIGN
    assert L.mol_moe_combine(mb.MOL_BF16, None, 64, None, None, 0, 2, 8, 64, None, 64,
                             None) == mb.MOL_OK                                 # M = 0
    # fused expand + combine: rank not built, rank bytes, bucket ceiling, alignment
    args = dict(s=FAKE, R=32, B=FAKE, N=64, sc=FAKE, rk=None, t=FAKE, l=FAKE, w=FAKE, M=4,
                k=2, E=8, S=2, base=FAKE, ldb=64, y=FAKE, ldy=64)

    def fused(dtype=mb.MOL_BF16, **kw):
        a = dict(args, **kw)
        return L.mol_lora_expand_combine(dtype, a["s"], a["R"], a["B"], a["N"], a["sc"],
                                         a["rk"], a["t"], a["l"], a["w"], a["M"], a["k"],
                                         a["E"], a["S"], a["base"], a["ldb"], a["y"],
                                         a["ldy"], None)

    assert fused(dtype=9) == mb.MOL_E_DTYPE
    assert fused(R=24) == mb.MOL_E_LIMIT            # 3 vectors of 8: not a power of two
    assert fused(R=256) == mb.MOL_E_LIMIT           # past 16 vectors
    assert fused(R=12) == mb.MOL_E_ALIGN            # 24 bytes
    assert fused(dtype=mb.MOL_F32, R=128) == mb.MOL_E_LIMIT
    assert fused(E=4096, S=2) == mb.MOL_E_LIMIT     # 8193 buckets
    assert fused(l=None) == mb.MOL_E_ARG
    assert fused(ldb=32) == mb.MOL_E_ARG
    assert fused(s=ctypes.c_void_p(0x1008)) == mb.MOL_E_ALIGN
    assert fused(M=0, s=None, B=None, t=None, l=None, w=None, base=None, y=None) == mb.MOL_OK


def test_moe_gemm_rejects_before_launch():
    L = mb.lib()

    def gemm(dtype=mb.MOL_BF16, xin=FAKE, ldx=64, rd=1, W=FAKE, K=64, N=32, E=8, srt=FAKE,
             eid=FAKE, npp=FAKE, numel=16, bm=16, out=FAKE, ldo=32, s=None, R=0, sl=1, B=None,
             sc=None, rk=None, lora=None, topk=1, S=1):
        return L.mol_moe_gemm(dtype, xin, ldx, rd, W, K, N, E, srt, eid, npp, numel, bm, out,
                              ldo, s, R, sl, B, sc, rk, lora, topk, S, None)

    assert gemm(dtype=4) == mb.MOL_E_DTYPE
    assert gemm(ldx=32) == mb.MOL_E_ARG                      # ld_x < K
    assert gemm(K=60, ldx=64) == mb.MOL_E_ALIGN              # 120-byte rows
    assert gemm(W=ctypes.c_void_p(0x1008)) == mb.MOL_E_ALIGN
    assert gemm(srt=None) == mb.MOL_E_ARG
    assert gemm(E=8192) == mb.MOL_E_LIMIT                    # 8193 buckets
    # fused delta: missing slots, rank bytes, misaligned s, token count
    assert gemm(s=FAKE, R=16, B=FAKE, sc=FAKE, topk=2, S=2) == mb.MOL_E_ARG
    assert gemm(s=FAKE, R=512, B=FAKE, sc=FAKE, lora=FAKE, topk=2, S=2) == mb.MOL_E_LIMIT
    assert gemm(s=ctypes.c_void_p(0x1008), R=16, B=FAKE, sc=FAKE, lora=FAKE, topk=2,
                S=2) == mb.MOL_E_ALIGN
    assert gemm(s=FAKE, R=16, B=FAKE, sc=FAKE, lora=FAKE, topk=3, S=2) == mb.MOL_E_ARG
    assert gemm(numel=0, xin=None, W=None, srt=None, eid=None, npp=None,
                out=None) == mb.MOL_OK
