"""Independent re-statements used to pin the oracle (tests only).

Each helper reaches the same result as the oracle by a different route, so that a
mistake in the oracle (a dropped term, a wrong index, a transposed operand, a broken
sort) shows up as a disagreement:

* `align_by_argsort`  - numpy's stable argsort of the bucket keys, then per-bucket
                        padding: the textbook special case of a stable counting sort.
* `delta_per_pair`    - the per-pair identity delta = scale * B_e (A_e x), computed with
                        numpy matmuls directly from the virtual ids, never touching the
                        aligned blocks.
* `bf16_rne_bits`     - double -> bfloat16 round-to-nearest-even by integer arithmetic
                        on the IEEE binary64 bit pattern (normal range only).
"""
from __future__ import annotations

import numpy as np


def bf16_bits_to_f64(b):
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(
        np.float32).astype(np.float64)


def to_f64(a):
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return bf16_bits_to_f64(a)
    return a.astype(np.float64)


def bf16_rne_bits(d):
    """double -> bf16 bits with ties to even, for finite values whose bf16 result is a
    normal number or zero (|d| >= 2^-126 or d == 0, and below the overflow threshold)."""
    d = np.ascontiguousarray(d, dtype=np.float64)
    u = d.view(np.uint64)
    sign = (u >> np.uint64(63)).astype(np.uint64)
    exp = ((u >> np.uint64(52)) & np.uint64(0x7FF)).astype(np.int64)
    man = (u & np.uint64((1 << 52) - 1)).astype(np.uint64)
    # keep 7 fraction bits out of 52: drop 45 with round-half-even
    drop = np.uint64(45)
    half = np.uint64(1 << 44)
    low = man & np.uint64((1 << 45) - 1)
    kept = man >> drop
    up = (low > half) | ((low == half) & ((kept & np.uint64(1)) == np.uint64(1)))
    kept = kept + up.astype(np.uint64)
    carry = kept >> np.uint64(7)
    kept = kept & np.uint64(0x7F)
    e8 = exp - 1023 + 127 + carry.astype(np.int64)
    bits = (sign << np.uint64(15)) | (e8.astype(np.uint64) << np.uint64(7)) | kept
    bits = np.where(d == 0.0, sign << np.uint64(15), bits)
    return bits.astype(np.uint16)


def keys_of(ids, lora_ids, E, S):
    """Bucket key per pair, restated from the remap rule: virtual id when it lands in
    [0, V), else V (the sentinel bucket)."""
    ids = np.asarray(ids, dtype=np.int64)
    M, k = ids.shape
    V = E * S
    if lora_ids is None:
        v = ids.reshape(-1)
    else:
        l = np.repeat(np.asarray(lora_ids, dtype=np.int64), k)
        t = ids.reshape(-1)
        ok = (t >= 0) & (t < E) & (l >= 0) & (l < S)
        v = np.where(t < 0, t, np.where(ok, t + l * E, -1))
    return np.where((v >= 0) & (v < V), v, V)


def align_by_argsort(ids, lora_ids, E, S, BM):
    key = keys_of(ids, lora_ids, E, S)
    numel = key.size
    V = E * S
    order = np.argsort(key, kind="stable")
    sorted_keys = key[order]
    srt, eid = [], []
    for b in range(V + 1):
        members = order[sorted_keys == b]
        if members.size == 0:
            continue
        nblk = -(-members.size // BM)
        padded = np.full(nblk * BM, numel, dtype=np.int64)
        padded[: members.size] = members
        srt.append(padded)
        eid.extend([(-1 if b == V else b)] * nblk)
    srt = np.concatenate(srt) if srt else np.zeros(0, dtype=np.int64)
    return srt.astype(np.int32), np.asarray(eid, dtype=np.int32), int(srt.size)


def delta_per_pair(cfg_E, cfg_S, topk, vids, stage, xin, row_div, A, B, scale):
    """Per pair p with a valid virtual id v: s_p = A_v @ x_row, and for slice g,
    delta[p, g*w:(g+1)*w] = scale[v // E] * B_v[g*w:(g+1)*w] @ s_p[g*r:(g+1)*r].
    Returns (s [numel, R] with NaN rows for pairs without a delta, delta [numel, N])."""
    V = cfg_E * cfg_S
    vids = np.asarray(vids).reshape(-1)
    numel = vids.size
    A64, B64, X64 = to_f64(A), to_f64(B), to_f64(xin)
    R, N, r = A.shape[1], B.shape[1], B.shape[2]
    w = N // stage.slices
    s = np.full((numel, R), np.nan)
    delta = np.zeros((numel, N))
    for p in range(numel):
        v = int(vids[p])
        if v < 0 or v >= V:
            continue
        s[p] = A64[v] @ X64[p // row_div]
        for g in range(stage.slices):
            delta[p, g * w:(g + 1) * w] = float(scale[v // cfg_E]) * (
                B64[v, g * w:(g + 1) * w] @ s[p, g * r:(g + 1) * r])
    return s, delta


def expected_plan(numel, V, block_m, sorted_ids, expert_ids, npp):
    """The work plan the align writes, rebuilt on the host from a routing (sorted_ids and
    expert_ids over [0, npp)): (written, runs). A plan is only written for a batch of at
    least 4096 pairs and 8 pairs per bucket on average (otherwise written is False and there
    are no runs). Every block of a real bucket lies in exactly one run of up to four
    consecutive blocks of that bucket, (first block, blocks, virtual expert), in bucket
    order; the sentinel bucket has none."""
    if not (numel >= 4096 and numel >= 8 * (V + 1)):
        return False, []
    nblk = npp // block_m
    eid = np.asarray(expert_ids[:nblk])
    runs = []
    i = 0
    while i < nblk:
        e = int(eid[i])
        j = i
        while j < nblk and int(eid[j]) == e:  # the bucket's blocks
            j += 1
        if e >= 0:
            for k in range(i, j, 4):
                runs.append((k, min(4, j - k), e))
        i = j
    return True, runs
