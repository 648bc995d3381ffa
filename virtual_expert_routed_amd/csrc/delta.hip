// LoRA shrink and expand over the aligned blocks (MindLab sglang PR 24: the MoL shrink
// hidden -> rank and expand rank -> N stages, weights laid out [V, N, K] with N the
// second dimension).
//
//   shrink: s[p, i]   = sum_k A[v, i, k] * xin[p / row_div, k]
//   expand: out[p, n] = round(out[p, n] + scale[v / E] * sum_j B[v, n, j] * s[p, g(n)*r + j])
//
// At decode a block holds one to a few pairs, so the work is a gather of many small
// matrix-vector products bound by streaming A_v and B_v from HBM. On MI355X one
// workgroup streams at most ~20 GB/s, so the weights of every touched virtual expert are
// spread over many workgroups and the grid follows the real blocks, not padded rows:
//  * shrink item = (block, group of RPI rows of A_v): RPI full rows of A_v (about 32 KiB)
//    read once with coalesced 16-byte buffer loads (LPR = 256/RPI lanes per row, each
//    row's lanes reading consecutive vectors), held in registers and reused for up to
//    four pairs at a time. The pairs' x segments go straight into LDS (direct-to-LDS
//    loads) once per item. The LPR partial sums are combined by a fixed butterfly, so s
//    is bit-reproducible and needs no split-K partials.
//  * expand item = (block, 256 output columns): one thread per column holds the
//    column's r weights in registers; the block's s rows are staged in LDS; out is read,
//    added to and rounded once.
// Latency chains are kept short: a block whose real pairs are within its first four
// entries (nearly every block at decode) reads those pair ids as scalars together with
// the expert id, so its weight, x, s and out loads all leave in one round trip. Loads are
// branch-free (out-of-range buffer offsets read as zero; other masked addresses are
// clamped to a valid one and their values unused), so each run of loads issues back to
// back.
//
// mol_lora_delta runs the shrink kernel then the expand kernel with s in the caller's
// workspace. A single launch that hands s between workgroups was measured to cost more
// than the kernel boundary: the handoff needs a store that reaches the coherence point, a
// counter and a poll, each a full memory round trip under load.
#include "delta_common.h"

namespace mol {
namespace {

// ------------------------------------------------------------------------------ shrink
// Lane lr of a row's LPR-lane group owns the 16-byte vectors lr, lr+LPR, lr+2*LPR, ...
// of the row, sums their products in ascending order, and the lanes are combined by a
// fixed butterfly (group_sum): the result depends only on (K, LPR).

template <int LPR>
__device__ __forceinline__ void load_a_seg(__amdgpu_buffer_rsrc_t ra, uint32_t row_off, bool row_ok,
                                           int m0, int nvec, uint4* av) {
  const int lr = threadIdx.x % LPR;
#pragma unroll
  for (int sg = 0; sg < kSeg; ++sg) {
    const int v = lr + (m0 + sg) * LPR;
    av[sg] = buf16(ra, (row_ok && v < nvec) ? row_off + (uint32_t)v * 16u : kOutOfRange);
  }
}

// Pairs whose x segments one LDS stage holds: eight where a segment is at most 2 KiB (rows
// of up to 1024 bf16, the down projection's), so a block of up to eight pairs fetches its x
// in one round trip, and four for longer segments, which keeps the stage at 16 KiB where
// the registers allow six workgroups per CU.
template <int LPR>
struct ShrinkLds {
  static constexpr int kPairs = LPR <= 16 ? 8 : 4;
  static constexpr int kVecs = kPairs * kSeg * LPR;
};

// Sixteen zero bytes in device memory: the source of the x slots past a row.
__device__ const uint4 kZero16 = {0, 0, 0, 0};

// The x vectors [m0*LPR, m0*LPR + SEGV) of the rows of pairs p[0..nq) go straight into xs
// (pair q at xs[q*SEGV]): pair by pair, each wave a run of 64 vectors. A wave whose run lies
// past the segment issues nothing; slots past the row are filled with zeros, so every slot
// of the segment holds a finite value and the products need no mask. Pair ids are indexed
// with compile-time indices only (a runtime index into them would put them in scratch
// memory).
template <bool BF16, int LPR, int NQ>
__device__ __forceinline__ void stage_x(const DeltaArgs& a, const int* p, int nq, int m0,
                                        int nvec, uint4* xs) {
  constexpr int ESZ = BF16 ? 2 : 4;
  constexpr int SEGV = kSeg * LPR;  // vectors of one x segment (a multiple of 64)
  constexpr int RUNS = (SEGV + kThreads - 1) / kThreads;
  static_assert(SEGV % 64 == 0, "x staging covers whole waves");
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const char* xbase = (const char*)a.xin;
  const int64_t xstride = a.ld_x * ESZ;
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    if (q >= nq) break;  // uniform
    const int64_t xrow = (int64_t)fdiv(p[q], a.f_rd) * xstride;
#pragma unroll
    for (int t = 0; t < RUNS; ++t) {
      const int i0 = t * kThreads + wv * 64;  // this wave's first vector of the segment
      if (i0 >= SEGV) continue;  // uniform: past the segment
      const int v = m0 * LPR + i0 + lane;
      const void* src = v < nvec ? (const void*)(xbase + xrow + (int64_t)v * 16)
                                 : (const void*)&kZero16;
      lds_dma16(src, xs + q * SEGV + i0);
    }
  }
}

// The products of NP pairs (their x staged at xs[i*SEGV]) with the held weight vectors,
// each weight vector against the pairs' x vectors read together, the rows' lanes reduced by
// the butterfly, and lane 0 of each row storing.
template <bool BF16, int LPR, int NP>
__device__ __forceinline__ void shrink_products(const DeltaArgs& a, const uint4* av, int row,
                                                bool row_in, const int* p, const uint4* xs) {
  constexpr int SEGV = kSeg * LPR;
  const int lr = threadIdx.x % LPR;
  float acc[NP];
#pragma unroll
  for (int i = 0; i < NP; ++i) acc[i] = 0.f;
#pragma unroll
  for (int sg = 0; sg < kSeg; ++sg) {
    uint4 xv[NP];
#pragma unroll
    for (int i = 0; i < NP; ++i) xv[i] = xs[i * SEGV + sg * LPR + lr];
#pragma unroll
    for (int i = 0; i < NP; ++i) acc[i] = dot16<BF16>(av[sg], xv[i], acc[i]);
  }
#pragma unroll
  for (int i = 0; i < NP; ++i) acc[i] = group_sum<LPR>(acc[i]);
  if (lr == 0 && row_in) {
#pragma unroll
    for (int i = 0; i < NP; ++i) a.s[(int64_t)p[i] * a.R + row] = acc[i];
  }
}

// Row `row` of s for the pairs p[0..nq) (nq <= NQ) from the weight vectors av[] that this
// lane holds (the lane's whole share of the row: vectors lr, lr+LPR, ... < nvec). Stages the
// pairs' x rows in one round trip, multiplies, reduces each row's LPR lanes by the fixed
// butterfly, and lane 0 of the row stores. The caller has issued the weight loads; every
// thread takes part.
template <bool BF16, int LPR, int NQ>
__device__ __forceinline__ void shrink_pairs(const DeltaArgs& a, const uint4* av, int row,
                                             bool row_in, const int* p, int nq, int nvec,
                                             uint4* xs) {
  constexpr int SEGV = kSeg * LPR;
  stage_x<BF16, LPR, NQ>(a, p, nq, 0, nvec, xs);
  __builtin_amdgcn_s_waitcnt(0);  // the x DMA (and the weights, the first time) have landed
  __syncthreads();
  // The products, kPG pairs at a time, with the group's pair count chosen by one uniform
  // switch: inside, every segment vector of every pair is multiplied with no branch, each
  // weight vector against the pairs' x vectors read together, so the LDS reads go out
  // together instead of one round trip each behind its own branch. Past the row both the
  // held weights and the staged x are zero. (The bf16 products take the packed pairs as they
  // are, so the held weights are never unpacked.) A block of one pair, the common case at
  // decode, then computes one pair's products and reduction, not four.
#pragma unroll
  for (int q0 = 0; q0 < NQ; q0 += kPG) {
    if (q0 >= nq) break;  // uniform
    const int m = nq - q0;  // uniform: pairs in this group (the last may hold fewer)
    if (m == 1)
      shrink_products<BF16, LPR, 1>(a, av, row, row_in, p + q0, xs + q0 * SEGV);
    else if (m == 2)
      shrink_products<BF16, LPR, 2>(a, av, row, row_in, p + q0, xs + q0 * SEGV);
    else if (m == 3)
      shrink_products<BF16, LPR, 3>(a, av, row, row_in, p + q0, xs + q0 * SEGV);
    else
      shrink_products<BF16, LPR, kPG>(a, av, row, row_in, p + q0, xs + q0 * SEGV);
  }
}

// Rows [rg*RPI, rg*RPI+RPI) of s for the pairs p[0..nq) (nq <= kPG) when a row is longer than
// one register segment: the weights are loaded segment by segment, for every group of pairs.
template <bool BF16, int LPR>
__device__ __forceinline__ void shrink_group_long(const DeltaArgs& a, int e, int rl, int rg,
                                                  const int* p, int nq, uint4* xs) {
  constexpr int ESZ = BF16 ? 2 : 4;
  constexpr int RPI = kThreads / LPR;
  constexpr int SEGV = kSeg * LPR;
  const int tid = threadIdx.x;
  const int lr = tid % LPR;
  const int row = rg * RPI + tid / LPR;
  const bool row_in = row < a.R;
  const bool row_ok = row_in && fmod(row, a.f_r) < rl;  // past the rank: zero, unread
  const int nvec = a.K * ESZ / 16;
  const int vpl = (nvec + LPR - 1) / LPR;
  const int64_t abytes = (int64_t)a.R * a.K * ESZ;
  const __amdgpu_buffer_rsrc_t ra = expert_rsrc((const char*)a.A + (int64_t)e * abytes, abytes);
  const uint32_t row_off = (uint32_t)(row_ok ? row : 0) * (uint32_t)(a.K * ESZ);
  float acc[kPG];
#pragma unroll
  for (int i = 0; i < kPG; ++i) acc[i] = 0.f;
  for (int m0 = 0; m0 < vpl; m0 += kSeg) {
    uint4 av[kSeg];
    load_a_seg<LPR>(ra, row_off, row_ok, m0, nvec, av);
    if (m0 > 0) __syncthreads();  // earlier readers of xs are done
    stage_x<BF16, LPR, kPG>(a, p, nq, m0, nvec, xs);
    __builtin_amdgcn_s_waitcnt(0);  // the x DMA and the weights have landed
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kPG; ++i) {
      if (i >= nq) break;
#pragma unroll
      for (int sg = 0; sg < kSeg; ++sg) {
        const int v = lr + (m0 + sg) * LPR;
        if (v < nvec) acc[i] = dot16<BF16>(av[sg], xs[i * SEGV + sg * LPR + lr], acc[i]);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < kPG; ++i) acc[i] = group_sum<LPR>(acc[i]);
  if (lr == 0 && row_in) {
#pragma unroll
    for (int i = 0; i < kPG; ++i) {
      if (i >= nq) break;
      a.s[(int64_t)p[i] * a.R + row] = acc[i];
    }
  }
}

// Shrink work item (blk, rg): all real pairs of block blk, NQ at a time. When a lane's share
// of a row fits one register segment (every row up to 8*LPR vectors: K = 2048 at 8 rows per
// item, K = 768 at 16), its weights are loaded once, together with the first group's x rows,
// and held for every group of pairs of the block. A block whose real pairs are all among its
// first NQ entries (nearly every block at decode) takes them from its head as scalars; a
// larger one stages its pair ids through pid, 64 per pass (they form a prefix of the block).
template <bool BF16, int LPR, bool HELD>
__device__ __forceinline__ void shrink_block(const DeltaArgs& a, const RouteArgs& ra_, int blk,
                                             int rg, int* pid, int& nreal, uint4* xs) {
  constexpr int ESZ = BF16 ? 2 : 4;
  constexpr int RPI = kThreads / LPR;
  constexpr int NQ = HELD ? ShrinkLds<LPR>::kPairs : kPG;  // pairs per x stage
  const BlockHeadN<NQ> h = block_head<NQ>(a, ra_, blk);
  if (h.e < 0 || h.nq == 0) return;  // no delta
  const int rl = slot_rank(a, h.e);
  const int nvec = a.K * ESZ / 16;  // HELD: nvec <= kSeg * LPR (chosen by the launcher)
  const int tid = threadIdx.x;
  const int row = rg * RPI + tid / LPR;
  const bool row_in = row < a.R;
  const bool row_ok = row_in && fmod(row, a.f_r) < rl;  // past the rank: zero, unread
  uint4 av[kSeg];
  if constexpr (HELD) {
    const int64_t abytes = (int64_t)a.R * a.K * ESZ;
    const __amdgpu_buffer_rsrc_t ra =
        expert_rsrc((const char*)a.A + (int64_t)h.e * abytes, abytes);
    load_a_seg<LPR>(ra, (uint32_t)(row_ok ? row : 0) * (uint32_t)(a.K * ESZ), row_ok, 0, nvec,
                    av);
    if (h.all_here) {  // the common decode case: the whole item is one straight run
      shrink_pairs<BF16, LPR, NQ>(a, av, row, row_in, h.p, h.nq, nvec, xs);
      return;
    }
  } else {
    if (h.all_here) {
      shrink_group_long<BF16, LPR>(a, h.e, rl, rg, h.p, h.nq, xs);
      return;
    }
  }
  for (int j0 = 0; j0 < a.BM; j0 += kPidSlots) {
    const int pv = tid < kPidSlots ? load_pid(a, blk, j0) : a.numel;
    __syncthreads();
    publish_pids(a, pv, pid, &nreal);
    __syncthreads();
    const int nr = nreal;
    for (int q0 = 0; q0 < nr; q0 += NQ) {
      int pq[NQ];
#pragma unroll
      for (int i = 0; i < NQ; ++i) pq[i] = q0 + i < nr ? pid[q0 + i] : a.numel;
      const int n = min(NQ, nr - q0);
      __syncthreads();  // xs of the previous group is no longer read
      if constexpr (HELD)
        shrink_pairs<BF16, LPR, NQ>(a, av, row, row_in, pq, n, nvec, xs);
      else
        shrink_group_long<BF16, LPR>(a, h.e, rl, rg, pq, n, xs);
    }
    if (nr < kPidSlots) return;  // the block's real entries ended in this pass
  }
}

template <bool BF16, int LPR, bool HELD>
__global__ void __launch_bounds__(kThreads) shrink_kernel(MOL_ROUTE_PARAMS, DeltaArgs a) {
  __shared__ int pid[kPidSlots];
  __shared__ int nreal;
  __shared__ uint4 xs[ShrinkLds<LPR>::kVecs];
  const RouteArgs r = MOL_ROUTE_MAKE;
  const int blk = route_block(r);
  shrink_block<BF16, LPR, HELD>(a, r, blk, (int)blockIdx.x - blk * r.per, pid, nreal, xs);
}

// ------------------------------------------------------------------------------ expand

// The weight rows of this thread's columns; vectors wholly past the slot's rank rl read as
// zero (the one that straddles rl is trimmed by trim_b_rows once the loads have landed).
template <bool BF16, int RV, int CPT>
__device__ __forceinline__ void load_b_rows(const DeltaArgs& a, int e, int rl, const int* n,
                                            uint4 (*bv)[RV]) {
  constexpr int RB = RV * 16;  // bytes of one weight row
  constexpr int VE = BF16 ? 8 : 4;
  const int64_t bbytes = (int64_t)a.N * RB;
  const __amdgpu_buffer_rsrc_t rb = expert_rsrc((const char*)a.B + (int64_t)e * bbytes, bbytes);
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    const bool ok = n[j] < a.N;
#pragma unroll
    for (int v = 0; v < RV; ++v)
      bv[j][v] = buf16(rb, ok && v * VE < rl ? (uint32_t)n[j] * RB + v * 16 : kOutOfRange);
  }
}

// Zero the elements at rank rl and past of the vector that straddles rl (a slot below full
// rank only; idempotent). Called after the weight loads have been waited for, so a full
// rank slot pays one uniform branch and a ranked one no extra round trip.
template <bool BF16, int RV, int CPT>
__device__ __forceinline__ void trim_b_rows(uint4 (*bv)[RV], int rl) {
  constexpr int VE = BF16 ? 8 : 4;
  if (rl >= RV * VE) return;  // uniform
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
#pragma unroll
    for (int v = 0; v < RV; ++v)
      if (v * VE < rl && rl < (v + 1) * VE) bv[j][v] = keep_first<BF16>(bv[j][v], rl - v * VE);
  }
}

// out[p, n] = round(out[p, n] + sc * <B_v[n], s_p[slice(n)]>) for the pairs pid[0..nr),
// kPG pairs at a time; ov holds the old values of the first kPG pairs (loaded ahead by the
// caller), and the old values of each next group are loaded while the current one is
// computed, so a block of many pairs costs one dependent round trip per kPG pairs.
template <bool BF16, int RV, int CPT>
__device__ __forceinline__ void expand_outputs(const DeltaArgs& a, const uint4 (*bv)[RV],
                                               const int* pid, int nr, const float* s_lds,
                                               const int* n, const int* soff, float sc,
                                               const float (*ov)[CPT]) {
  constexpr int VE = BF16 ? 8 : 4;
  float cur[kPG][CPT];
#pragma unroll
  for (int i = 0; i < kPG; ++i) {
#pragma unroll
    for (int j = 0; j < CPT; ++j) cur[i][j] = ov[i][j];
  }
#pragma unroll 1
  for (int q0 = 0; q0 < nr; q0 += kPG) {
    float nxt[kPG][CPT] = {};
    if (q0 + kPG < nr) {  // uniform over the workgroup
#pragma unroll
      for (int i = 0; i < kPG; ++i) {
        const int q = q0 + kPG + i;
        const bool qok = q < nr;
        const int pq = pid[qok ? q : 0];
#pragma unroll
        for (int j = 0; j < CPT; ++j) nxt[i][j] = load_out<BF16>(a, pq, n[j], qok && n[j] < a.N);
      }
    }
#pragma unroll
    for (int i = 0; i < kPG; ++i) {
      const int q = q0 + i;
      if (q >= nr) break;
      const int p = pid[q];
      const float* s_row = s_lds + q * a.R;
#pragma unroll
      for (int j = 0; j < CPT; ++j) {
        if (n[j] >= a.N) continue;
        const float* sv = s_row + soff[j];
        float acc = 0.f;
#pragma unroll
        for (int v = 0; v < RV; ++v) {
          // keep the weights packed across pairs: unpacking them once for all pairs would
          // hold RV*8 more floats per column live, for no gain at one or two pairs a block
          uint4 b = bv[j][v];
          asm volatile("" : "+v"(b.x), "+v"(b.y), "+v"(b.z), "+v"(b.w));
          acc = dot16_s<BF16>(b, sv + v * VE, acc);
        }
        store_out<BF16>(a, p, n[j], fmaf(sc, acc, cur[i][j]));
      }
    }
#pragma unroll
    for (int i = 0; i < kPG; ++i) {
#pragma unroll
      for (int j = 0; j < CPT; ++j) cur[i][j] = nxt[i][j];
    }
  }
}

// The columns n[] of the pairs p[0..n4) (n4 <= kPG real pairs of one virtual expert, weights
// bv already requested): each pair's s row goes straight into LDS (wave q takes pair q) and
// the old out values are requested in the same round trip as the weights; then the sums,
// one rounding and the stores.
template <bool BF16, int RV>
__device__ __forceinline__ void expand_pairs(const DeltaArgs& a, int rl, const int* n,
                                             const int* soff, float sc, uint4 (*bv)[RV],
                                             const int* p, int n4, int* pid, float* s_lds) {
  constexpr int CPT = cols_per_thread(RV);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rv4 = a.R / 4;  // 16-byte vectors of one s row
#pragma unroll
  for (int q = 0; q < kPG; ++q) {
    if (q < n4 && wv == (q & 3)) {  // uniform over the wave
      const float* src = a.s + (int64_t)p[q] * a.R;
      for (int t0 = 0; t0 < rv4; t0 += 64)
        if (t0 + lane < rv4) lds_dma16(src + (t0 + lane) * 4, s_lds + q * a.R + t0 * 4);
    }
  }
  if (tid < kPG) pid[tid] = tid == 0 ? p[0] : tid == 1 ? p[1] : tid == 2 ? p[2] : p[3];
  float ov[kPG][CPT];
#pragma unroll
  for (int q = 0; q < kPG; ++q) {
#pragma unroll
    for (int j = 0; j < CPT; ++j)
      ov[q][j] = load_out<BF16>(a, q < n4 ? p[q] : 0, n[j], q < n4 && n[j] < a.N);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  trim_b_rows<BF16, RV, CPT>(bv, rl);
  expand_outputs<BF16, RV, CPT>(a, bv, pid, n4, s_lds, n, soff, sc, ov);
}

// One expand work item: CPT*256 output columns for every real pair of block blk.
template <bool BF16, int RV>
__device__ __forceinline__ void expand_block(const DeltaArgs& a, const RouteArgs& ra_, int blk,
                                             int chunk, int* pid, int& nreal, float* s_lds) {
  constexpr int CPT = cols_per_thread(RV);
  constexpr int ESZ = BF16 ? 2 : 4;
  constexpr int r = RV * 16 / ESZ;
  const int tid = threadIdx.x;
  const BlockHead h = block_head(a, ra_, blk);
  const int e = h.e;
  if (e < 0 || h.nq == 0) return;  // no delta
  const int rl = slot_rank(a, e);
  if (rl == 0) return;  // a slot of rank 0 adds nothing
  int n[CPT], soff[CPT];
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    n[j] = chunk * (CPT * kThreads) + j * kThreads + tid;
    soff[j] = (n[j] < a.N ? fdiv(n[j], a.f_w) : 0) * r;
  }
  const float sc = a.scale[fdiv(e, a.f_e)];
  uint4 bv[CPT][RV];
  load_b_rows<BF16, RV, CPT>(a, e, rl, n, bv);
  if (h.all_here) {
    expand_pairs<BF16, RV>(a, rl, n, soff, sc, bv, h.p, h.nq, pid, s_lds);
    return;
  }
  const int pg = min(kPidSlots, kSLdsFloats / a.R);
  for (int j0 = 0; j0 < a.BM; j0 += pg) {
    const int pv = tid < pg ? load_pid(a, blk, j0) : a.numel;
    __syncthreads();
    publish_pids(a, pv, pid, &nreal);
    __syncthreads();
    const int nr = nreal;
    if (nr == 0) break;
    float ov[kPG][CPT];  // old out values of the first pairs, loaded before s is needed
#pragma unroll
    for (int q = 0; q < kPG; ++q) {
      const int pq = pid[q];
#pragma unroll
      for (int j = 0; j < CPT; ++j) ov[q][j] = load_out<BF16>(a, pq, n[j], q < nr && n[j] < a.N);
    }
    for (int i = tid; i < nr * a.R; i += kThreads) {
      const int q = i / a.R;
      s_lds[i] = a.s[(int64_t)pid[q] * a.R + (i - q * a.R)];
    }
    __syncthreads();
    trim_b_rows<BF16, RV, CPT>(bv, rl);
    expand_outputs<BF16, RV, CPT>(a, bv, pid, nr, s_lds, n, soff, sc, ov);
    if (nr < pg) break;  // the block's real entries ended in this pass
  }
}

template <bool BF16, int RV>
__global__ void __launch_bounds__(kThreads) expand_kernel(MOL_ROUTE_PARAMS, DeltaArgs a) {
  __shared__ int pid[kPidSlots];
  __shared__ int nreal;
  __shared__ __attribute__((aligned(16))) float s_lds[kSLdsFloats];
  const RouteArgs r = MOL_ROUTE_MAKE;
  const int blk = route_block(r);
  expand_block<BF16, RV>(a, r, blk, (int)blockIdx.x - blk * r.per, pid, nreal, s_lds);
}

template <bool BF16, bool HELD>
hipError_t shrink_dispatch(const DeltaArgs& a, int lpr, int grid, hipStream_t st) {
  switch (lpr) {
    case 8: hipLaunchKernelGGL((shrink_kernel<BF16, 8, HELD>), dim3(grid), dim3(kThreads), 0, st, MOL_ROUTE_ARGS(a, a.rgroups, a.f_rg), a); break;
    case 16: hipLaunchKernelGGL((shrink_kernel<BF16, 16, HELD>), dim3(grid), dim3(kThreads), 0, st, MOL_ROUTE_ARGS(a, a.rgroups, a.f_rg), a); break;
    case 32: hipLaunchKernelGGL((shrink_kernel<BF16, 32, HELD>), dim3(grid), dim3(kThreads), 0, st, MOL_ROUTE_ARGS(a, a.rgroups, a.f_rg), a); break;
    case 64: hipLaunchKernelGGL((shrink_kernel<BF16, 64, HELD>), dim3(grid), dim3(kThreads), 0, st, MOL_ROUTE_ARGS(a, a.rgroups, a.f_rg), a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <bool BF16>
hipError_t expand_dispatch(const DeltaArgs& a, int rv, int grid, hipStream_t st) {
  switch (rv) {
    case 1: hipLaunchKernelGGL((expand_kernel<BF16, 1>), dim3(grid), dim3(kThreads), 0, st, MOL_ROUTE_ARGS(a, a.nchunk, a.f_nc), a); break;
    case 2: hipLaunchKernelGGL((expand_kernel<BF16, 2>), dim3(grid), dim3(kThreads), 0, st, MOL_ROUTE_ARGS(a, a.nchunk, a.f_nc), a); break;
    case 4: hipLaunchKernelGGL((expand_kernel<BF16, 4>), dim3(grid), dim3(kThreads), 0, st, MOL_ROUTE_ARGS(a, a.nchunk, a.f_nc), a); break;
    case 8: hipLaunchKernelGGL((expand_kernel<BF16, 8>), dim3(grid), dim3(kThreads), 0, st, MOL_ROUTE_ARGS(a, a.nchunk, a.f_nc), a); break;
    case 16: hipLaunchKernelGGL((expand_kernel<BF16, 16>), dim3(grid), dim3(kThreads), 0, st, MOL_ROUTE_ARGS(a, a.nchunk, a.f_nc), a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

int expand_cols_per_item(int32_t R, int32_t slices, int elem_bytes) {
  const int rv = (R / slices) * elem_bytes / 16;
  return cols_per_thread(rv) * kThreads;  // = kExpandCols
}

int shrink_rows_per_item(int32_t K, int elem_bytes) {
  const int64_t row_bytes = (int64_t)K * elem_bytes;
  int rpi = 4;
  while (rpi < 32 && (int64_t)(rpi * 2) * row_bytes <= kShrinkItemBytes) rpi *= 2;
  return rpi;
}

hipError_t launch_shrink(const DeltaArgs& a, bool bf16, int rows_per_item, int grid,
                         hipStream_t stream) {
  const int lpr = kThreads / rows_per_item;
  // a lane's share of a row fits one register segment: held across the block's pairs
  const bool held = (int64_t)a.K * (bf16 ? 2 : 4) / 16 <= (int64_t)kSeg * lpr;
  if (bf16)
    return held ? shrink_dispatch<true, true>(a, lpr, grid, stream)
                : shrink_dispatch<true, false>(a, lpr, grid, stream);
  return held ? shrink_dispatch<false, true>(a, lpr, grid, stream)
              : shrink_dispatch<false, false>(a, lpr, grid, stream);
}

hipError_t launch_expand(const DeltaArgs& a, bool bf16, int grid, hipStream_t stream) {
  const int rv = (a.R / a.slices) * (bf16 ? 2 : 4) / 16;
  return bf16 ? expand_dispatch<true>(a, rv, grid, stream)
              : expand_dispatch<false>(a, rv, grid, stream);
}

}  // namespace mol
