// LoRA shrink and expand over the aligned blocks (MindLab sglang PR 24: the MoL shrink
// hidden -> rank and expand rank -> N stages, weights laid out [V, N, K] with N the
// second dimension).
//
//   shrink: s[p, i]   = sum_k A[v, i, k] * xin[p / row_div, k]
//   expand: out[p, n] = round(out[p, n] + scale[v / E] * sum_j B[v, n, j] * s[p, g(n)*r + j])
//
// At decode a block holds one to a few pairs, so the work is a gather of many small
// matrix-vector products and the bound is streaming A_v and B_v from HBM. Work is split
// so the number of work items follows the real blocks, not padded rows:
//  * shrink item = (block, group of RPI rows of A_v): the item reads RPI full rows of
//    A_v (about 32 KiB) once with coalesced 16-byte loads (LPR = 256/RPI lanes per row,
//    each row's lanes reading consecutive 16-byte vectors), keeps them in registers and
//    reuses them for up to 4 pairs at a time; the LPR partial sums are combined with a
//    fixed xor-shuffle tree, so s is bit-reproducible and needs no split-K partials;
//  * expand item = (block, 256 output columns): one thread per column holds the column's
//    r weights in registers and loops over the block's pairs, with their s rows staged in
//    LDS; out is read, added to and rounded once.
//
// The fused kernel runs both in one launch. Workgroups [0, S) are shrink items and the
// rest expand items, block by block. A shrink item publishes its rows of s with
// agent-coherent (L2-bypassing) stores, waits for them to complete, and bumps its block's
// counter; an expand item first issues its weight loads, then polls the counter and reads
// s with agent-coherent loads. No cache-wide writeback or invalidate is needed, and no
// counter is shared by all workgroups. The wait is bounded: an expand item that does not
// see its block ready in time computes the block's s itself with exactly the shrink
// arithmetic (same lanes, same order), so the result is bit-identical either way and no
// workgroup ever depends on the scheduling of another. Each block's counter packs the
// finished shrink items (low 16 bits) and expand items (high 16 bits); whichever
// participant arrives last puts it back to zero for the next call.
#include "mol_internal.h"

namespace mol {
namespace {

__device__ __forceinline__ uint4 ld16(const void* p) {
  return *reinterpret_cast<const uint4*>(p);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);  // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// acc += <a, x> over one 16-byte vector of each
template <bool BF16>
__device__ __forceinline__ float dot16(const uint4& a, const uint4& x, float acc) {
  if constexpr (BF16) {
    acc = fmaf(bf16_lo(a.x), bf16_lo(x.x), acc);
    acc = fmaf(bf16_hi(a.x), bf16_hi(x.x), acc);
    acc = fmaf(bf16_lo(a.y), bf16_lo(x.y), acc);
    acc = fmaf(bf16_hi(a.y), bf16_hi(x.y), acc);
    acc = fmaf(bf16_lo(a.z), bf16_lo(x.z), acc);
    acc = fmaf(bf16_hi(a.z), bf16_hi(x.z), acc);
    acc = fmaf(bf16_lo(a.w), bf16_lo(x.w), acc);
    acc = fmaf(bf16_hi(a.w), bf16_hi(x.w), acc);
  } else {
    acc = fmaf(__uint_as_float(a.x), __uint_as_float(x.x), acc);
    acc = fmaf(__uint_as_float(a.y), __uint_as_float(x.y), acc);
    acc = fmaf(__uint_as_float(a.z), __uint_as_float(x.z), acc);
    acc = fmaf(__uint_as_float(a.w), __uint_as_float(x.w), acc);
  }
  return acc;
}

// acc += <b, s[0:VE]> with b one 16-byte vector of weights, s fp32 in LDS
template <bool BF16>
__device__ __forceinline__ float dot16_s(const uint4& b, const float* s, float acc) {
  if constexpr (BF16) {
    acc = fmaf(bf16_lo(b.x), s[0], acc);
    acc = fmaf(bf16_hi(b.x), s[1], acc);
    acc = fmaf(bf16_lo(b.y), s[2], acc);
    acc = fmaf(bf16_hi(b.y), s[3], acc);
    acc = fmaf(bf16_lo(b.z), s[4], acc);
    acc = fmaf(bf16_hi(b.z), s[5], acc);
    acc = fmaf(bf16_lo(b.w), s[6], acc);
    acc = fmaf(bf16_hi(b.w), s[7], acc);
  } else {
    acc = fmaf(__uint_as_float(b.x), s[0], acc);
    acc = fmaf(__uint_as_float(b.y), s[1], acc);
    acc = fmaf(__uint_as_float(b.z), s[2], acc);
    acc = fmaf(__uint_as_float(b.w), s[3], acc);
  }
  return acc;
}

constexpr int kThreads = 256;
constexpr int kPidSlots = 64;     // pair ids staged per pass over a block
constexpr int kSLdsFloats = 4096; // s rows staged per expand pass (16 KiB)
constexpr int kPG = 4;            // pairs sharing one pass over the held weight vectors
constexpr int kSeg = 8;           // 16-byte weight vectors a lane holds at once

// output columns per thread of an expand item, from the 16-byte vectors per weight row
__host__ __device__ constexpr int cols_per_thread(int rv) { return rv >= 8 ? 1 : 8 / rv; }

__device__ __forceinline__ bool real_pair(int p, int numel) {
  return (unsigned)p < (unsigned)numel;
}

__device__ __forceinline__ bool real_expert(int e, int V) { return (unsigned)e < (unsigned)V; }

// blocks that carry work: [0, npp / BM) clamped to the launched bound
__device__ __forceinline__ int live_blocks(const DeltaArgs& a, int npp) {
  const int nb = npp / a.BM;
  return nb < 0 ? 0 : (nb > a.max_blocks ? a.max_blocks : nb);
}

// Expert id of block blk if the block carries work, else -1. Both loads go out together
// (blk < max_blocks, so the expert id read is in bounds even past the live blocks).
__device__ __forceinline__ int block_expert(const DeltaArgs& a, int blk) {
  const int npp = *a.npp;
  const int e = a.expert_ids[blk];
  return (blk < live_blocks(a, npp) && real_expert(e, a.V)) ? e : -1;
}

// agent-coherent accesses used to hand s from shrink to expand items of one launch
__device__ __forceinline__ void st_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_coherent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Branch-free loads: an address that is not needed is clamped to a valid one (the first
// element of the same array) and the value discarded afterwards, so a run of loads issues
// back to back instead of each sitting in its own branch with its own wait.
__device__ __forceinline__ uint4 ld16_if(const char* base, int64_t off, bool ok) {
  const uint4 v = ld16(base + (ok ? off : 0));
  return ok ? v : make_uint4(0, 0, 0, 0);
}

// Raw buffer loads over one expert's weight matrix: the resource covers exactly that
// matrix, offsets are 32-bit, and an offset past its end reads as zero in hardware, so
// masked lanes need neither a branch nor a select nor a 64-bit address of their own.
constexpr uint32_t kOutOfRange = 0x80000000u;
constexpr int kBufferFlags = 0x00020000;  // raw 32-bit-element buffer, gfx9 data format

__device__ __forceinline__ __amdgpu_buffer_rsrc_t expert_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kBufferFlags);
}

__device__ __forceinline__ uint4 buf16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return *reinterpret_cast<const uint4*>(&v);
}

// Entry j0 + lane of block blk for the lanes of wave 0 (numel for entries past the block).
__device__ __forceinline__ int load_pid(const DeltaArgs& a, int blk, int j0) {
  const int j = j0 + (int)threadIdx.x;
  const int v = a.sorted[(int64_t)blk * a.BM + (j < a.BM ? j : 0)];
  return j < a.BM ? v : a.numel;
}

// Wave 0 publishes its pair ids and the number of real ones (they form a prefix).
__device__ __forceinline__ void publish_pids(const DeltaArgs& a, int pv, int* pid, int* nreal) {
  if (threadIdx.x < kPidSlots) {
    pid[threadIdx.x] = pv;
    const uint64_t m = __builtin_amdgcn_ballot_w64(real_pair(pv, a.numel));
    if (threadIdx.x == 0) *nreal = (int)__popcll(m);
  }
}

// ------------------------------------------------------------------------------ shrink
// Lane lr of a row's LPR-lane group owns the 16-byte vectors lr, lr+LPR, lr+2*LPR, ...
// of the row, sums their products in ascending order, and the lanes are combined by a
// fixed xor tree: the result depends only on (K, LPR), not on how many vectors (kSeg) or
// pairs (kPG) are processed together, which is what lets the fallback path below
// reproduce the shrink items bit for bit.

// The kSeg vectors of one segment of this lane's row of A_e (zero past the row or matrix).
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

// One shrink work item: rows [rg*RPI, rg*RPI+RPI) of s for every real pair of block blk.
// The x segments of kPG pairs at a time are staged once in LDS (xs) instead of every row
// group of lanes reading them again.
template <bool BF16, int LPR, bool COHERENT>
__device__ __forceinline__ void shrink_item(const DeltaArgs& a, int blk, int rg, int e, int pv0,
                                            int* pid, int* nreal, uint4* xs) {
  constexpr int ESZ = BF16 ? 2 : 4;
  constexpr int RPI = kThreads / LPR;
  constexpr int SEGV = kSeg * LPR;              // vectors of one x segment
  constexpr int XPT = kPG * SEGV / kThreads;    // x vectors each thread stages
  const int tid = threadIdx.x;
  const int lr = tid % LPR;
  const int row = rg * RPI + tid / LPR;
  const bool row_ok = row < a.R;
  const int nvec = a.K * ESZ / 16;
  const int vpl = (nvec + LPR - 1) / LPR;
  const int64_t abytes = (int64_t)a.R * a.K * ESZ;
  const __amdgpu_buffer_rsrc_t ra = expert_rsrc((const char*)a.A + (int64_t)e * abytes, abytes);
  const uint32_t row_off = (uint32_t)(row_ok ? row : 0) * (uint32_t)(a.K * ESZ);
  const char* xbase = (const char*)a.xin;
  const int64_t xstride = a.ld_x * ESZ;
  for (int j0 = 0; j0 < a.BM; j0 += kPidSlots) {
    const int pv = j0 == 0 ? pv0 : (tid < kPidSlots ? load_pid(a, blk, j0) : 0);
    uint4 av[kSeg];
    load_a_seg<LPR>(ra, row_off, row_ok, 0, nvec, av);  // weights go out with the ids
    __syncthreads();
    publish_pids(a, pv, pid, nreal);
    __syncthreads();
    const int nr = *nreal;
    for (int q0 = 0; q0 < nr; q0 += kPG) {
      float acc[kPG];
#pragma unroll
      for (int i = 0; i < kPG; ++i) acc[i] = 0.f;
      for (int m0 = 0; m0 < vpl; m0 += kSeg) {
        if (m0 > 0 || q0 > 0) load_a_seg<LPR>(ra, row_off, row_ok, m0, nvec, av);
        uint4 xv[XPT];
#pragma unroll
        for (int t = 0; t < XPT; ++t) {
          const int i = tid + t * kThreads;
          const int q = i / SEGV;
          const int v = m0 * LPR + (i - q * SEGV);
          const int pq = pid[q0 + q];
          const bool ok = q0 + q < nr && v < nvec;
          xv[t] = ld16_if(xbase, (int64_t)(ok ? pq / a.row_div : 0) * xstride + (int64_t)v * 16, ok);
        }
        __syncthreads();  // earlier readers of xs are done
#pragma unroll
        for (int t = 0; t < XPT; ++t) xs[tid + t * kThreads] = xv[t];
        __syncthreads();
#pragma unroll
        for (int i = 0; i < kPG; ++i) {
          if (q0 + i >= nr) break;
#pragma unroll
          for (int sg = 0; sg < kSeg; ++sg) {
            const int v = lr + (m0 + sg) * LPR;
            if (v < nvec) acc[i] = dot16<BF16>(av[sg], xs[i * SEGV + sg * LPR + lr], acc[i]);
          }
        }
      }
#pragma unroll
      for (int i = 0; i < kPG; ++i) {
#pragma unroll
        for (int off = LPR / 2; off > 0; off >>= 1) acc[i] += __shfl_xor(acc[i], off, 64);
      }
      if (lr == 0 && row_ok) {
#pragma unroll
        for (int i = 0; i < kPG; ++i) {
          if (q0 + i >= nr) break;
          float* d = a.s + (int64_t)pid[q0 + i] * a.R + row;
          if constexpr (COHERENT) st_coherent(d, acc[i]); else *d = acc[i];
        }
      }
    }
    if (nr < kPidSlots) return;  // the block's real entries ended in this pass
  }
}

// The shrink sum of one row (lane group) for one pair, read straight from global memory
// one vector at a time: few registers, and the same sums as shrink_item.
template <bool BF16, int LPR>
__device__ __forceinline__ float shrink_one(const DeltaArgs& a, int e, int row, int p) {
  constexpr int ESZ = BF16 ? 2 : 4;
  const int lr = threadIdx.x % LPR;
  const bool row_ok = row < a.R;
  const int nvec = a.K * ESZ / 16;
  const char* arow =
      (const char*)a.A + ((int64_t)e * a.R + (row_ok ? row : 0)) * (int64_t)a.K * ESZ;
  const char* xr = (const char*)a.xin + (int64_t)(p / a.row_div) * a.ld_x * ESZ;
  float acc = 0.f;
  for (int v = lr; v < nvec; v += LPR)
    acc = dot16<BF16>(ld16_if(arow, (int64_t)v * 16, row_ok), ld16(xr + (int64_t)v * 16), acc);
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
  return acc;
}

// s rows of the pairs pid[0..nr) into s_lds [nr][R], computed here with the arithmetic of
// the shrink items (used when they are not done in time).
template <bool BF16, int LPR>
__device__ __forceinline__ void compute_s_rows(const DeltaArgs& a, int e, const int* pid, int nr,
                                               float* s_lds) {
  constexpr int RPI = kThreads / LPR;
  const int lr = threadIdx.x % LPR;
  for (int rg = 0; rg < a.rgroups; ++rg) {
    const int row = rg * RPI + threadIdx.x / LPR;
    for (int q = 0; q < nr; ++q) {
      const float acc = shrink_one<BF16, LPR>(a, e, row, pid[q]);
      if (lr == 0 && row < a.R) s_lds[q * a.R + row] = acc;
    }
  }
}

// ------------------------------------------------------------------------------ expand

// s rows of the pairs pid[0..nr) into s_lds [nr][R] (nr * R <= kSLdsFloats), read from
// a.s four loads per thread at a time.
template <bool COHERENT>
__device__ __forceinline__ void load_s_rows(const DeltaArgs& a, const int* pid, int nr,
                                            float* s_lds) {
  const int R = a.R;
  const int total = nr * R;
  for (int base = 0; base < total; base += 4 * kThreads) {
    float v[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int i = base + t * kThreads + threadIdx.x;
      const bool ok = i < total;
      const int q = ok ? i / R : 0;
      const float* src = a.s + (int64_t)pid[q] * R + (ok ? i - q * R : 0);
      v[t] = COHERENT ? ld_coherent(src) : *src;
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int i = base + t * kThreads + threadIdx.x;
      if (i < total) s_lds[i] = v[t];
    }
  }
}

template <bool BF16, int RV, int CPT>
__device__ __forceinline__ void load_b_rows(const DeltaArgs& a, int e, const int* n,
                                            uint4 (*bv)[RV]) {
  constexpr int ESZ = BF16 ? 2 : 4;
  constexpr int RB = RV * 16;  // bytes of one weight row
  const int64_t bbytes = (int64_t)a.N * RB;
  const __amdgpu_buffer_rsrc_t rb = expert_rsrc((const char*)a.B + (int64_t)e * bbytes, bbytes);
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    const bool ok = n[j] < a.N;
#pragma unroll
    for (int v = 0; v < RV; ++v)
      bv[j][v] = buf16(rb, ok ? (uint32_t)n[j] * RB + v * 16 : kOutOfRange);
  }
  (void)ESZ;
}

template <bool BF16>
__device__ __forceinline__ float load_out(const DeltaArgs& a, int p, int n, bool ok) {
  const int64_t i = ok ? (int64_t)p * a.ld_out + n : 0;
  float v;
  if constexpr (BF16)
    v = __uint_as_float((uint32_t)((const uint16_t*)a.out)[i] << 16);
  else
    v = ((const float*)a.out)[i];
  return ok ? v : 0.f;
}

template <bool BF16>
__device__ __forceinline__ void store_out(const DeltaArgs& a, int p, int n, float v) {
  if constexpr (BF16)
    ((uint16_t*)a.out)[(int64_t)p * a.ld_out + n] = f32_to_bf16_rne(v);
  else
    ((float*)a.out)[(int64_t)p * a.ld_out + n] = v;
}

// out[p, n] = round(out[p, n] + sc * <B_v[n], s_p[slice(n)]>) for this pass's pairs; the
// old values of the first kPG pairs were loaded ahead into ov.
template <bool BF16, int RV, int CPT>
__device__ __forceinline__ void expand_outputs(const DeltaArgs& a, const uint4 (*bv)[RV],
                                               const int* pid, int nr, const float* s_lds,
                                               const int* n, const int* soff, float sc,
                                               const float (*ov)[CPT]) {
  constexpr int VE = BF16 ? 8 : 4;
#pragma unroll 1
  for (int q = 0; q < nr; ++q) {
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
      float old;
      if (q < kPG) {
        old = q == 0 ? ov[0][j] : q == 1 ? ov[1][j] : q == 2 ? ov[2][j] : ov[3][j];
      } else {
        old = load_out<BF16>(a, p, n[j], true);
      }
      store_out<BF16>(a, p, n[j], fmaf(sc, acc, old));
    }
  }
}

// One expand work item: CPT*256 output columns for every real pair of block blk.
// FUSED: s comes from this launch's shrink items (or is computed here, see above).
template <bool BF16, int LPR, int RV, bool FUSED>
__device__ __forceinline__ void expand_item(const DeltaArgs& a, int blk, int chunk, int e,
                                            int pv0, int* pid, int* nreal, float* s_lds,
                                            int* flag) {
  constexpr int CPT = cols_per_thread(RV);
  constexpr int ESZ = BF16 ? 2 : 4;
  constexpr int r = RV * 16 / ESZ;
  const int tid = threadIdx.x;
  const int width = a.N / a.slices;
  const int pg = min(kPidSlots, kSLdsFloats / a.R);
  int n[CPT], soff[CPT];
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    n[j] = chunk * (CPT * kThreads) + j * kThreads + tid;
    soff[j] = (n[j] < a.N ? n[j] / width : 0) * r;
  }
  const float sc = a.scale[e / a.E];
  int pv = tid < pg ? pv0 : a.numel;
  uint4 bv[CPT][RV];
  load_b_rows<BF16, RV, CPT>(a, e, n, bv);  // the weights go out with the first ids
  bool ready = true;
  for (int j0 = 0; j0 < a.BM; j0 += pg) {
    if (j0 > 0) pv = tid < pg ? load_pid(a, blk, j0) : a.numel;
    if (tid >= pg) pv = a.numel;
    __syncthreads();
    publish_pids(a, pv, pid, nreal);
    if constexpr (FUSED) {
      if (j0 == 0 && tid == 0) {
        int ok = 0;
        for (int it = 0; it < a.spin_limit; ++it) {
          const int w =
              __hip_atomic_load(a.sync + blk, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if ((w & 0xffff) >= a.rgroups) {
            ok = 1;
            break;
          }
          __builtin_amdgcn_s_sleep(2);
        }
        *flag = ok;
      }
    }
    __syncthreads();
    const int nr = *nreal;
    if (nr == 0) break;
    if constexpr (FUSED) ready = *flag != 0;
    float ov[kPG][CPT];  // old out values of the first pairs, loaded before s is needed
#pragma unroll
    for (int q = 0; q < kPG; ++q) {
      const int p = pid[q];
#pragma unroll
      for (int j = 0; j < CPT; ++j) ov[q][j] = load_out<BF16>(a, p, n[j], q < nr && n[j] < a.N);
    }
    if (ready) {
      load_s_rows<FUSED>(a, pid, nr, s_lds);
    } else if constexpr (FUSED) {
      compute_s_rows<BF16, LPR>(a, e, pid, nr, s_lds);
    }
    __syncthreads();
    expand_outputs<BF16, RV, CPT>(a, bv, pid, nr, s_lds, n, soff, sc, ov);
    if (nr < pg) break;  // the block's real entries ended in this pass
  }
}

// block counter arrival: shrink items add 1, expand items add 1 << 16; the last of the
// rgroups + nchunk participants clears the counter
__device__ __forceinline__ void arrive(const DeltaArgs& a, int blk, int inc) {
  const int target = a.rgroups + (a.nchunk << 16);
  const int old = __hip_atomic_fetch_add(a.sync + blk, inc, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
  if (old + inc == target)
    __hip_atomic_store(a.sync + blk, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int LPR>
struct ShrinkLds {
  static constexpr int kVecs = kPG * kSeg * LPR;
};

template <bool BF16, int LPR>
__global__ void __launch_bounds__(kThreads) shrink_kernel(DeltaArgs a) {
  __shared__ int pid[kPidSlots];
  __shared__ int nreal;
  __shared__ uint4 xs[ShrinkLds<LPR>::kVecs];
  const int blk = blockIdx.x / a.rgroups, rg = blockIdx.x % a.rgroups;
  const int pv0 = threadIdx.x < kPidSlots ? load_pid(a, blk, 0) : 0;  // with the expert id
  const int e = block_expert(a, blk);
  if (e < 0) return;
  shrink_item<BF16, LPR, false>(a, blk, rg, e, pv0, pid, &nreal, xs);
}

template <bool BF16, int RV>
__global__ void __launch_bounds__(kThreads) expand_kernel(DeltaArgs a) {
  __shared__ int pid[kPidSlots];
  __shared__ int nreal;
  __shared__ float s_lds[kSLdsFloats];
  const int blk = blockIdx.x / a.nchunk, c = blockIdx.x % a.nchunk;
  const int pv0 = threadIdx.x < kPidSlots ? load_pid(a, blk, 0) : 0;
  const int e = block_expert(a, blk);
  if (e < 0) return;
  expand_item<BF16, 64, RV, false>(a, blk, c, e, pv0, pid, &nreal, s_lds, nullptr);
}

// Fused delta: block blk is served by a.nchunk consecutive workgroups (parts). Part g
// issues the weight loads of its a.cpp expand columns first, computes shrink row group g
// when g < a.rgroups and publishes it, then waits for the block's other row groups and
// expands its own columns. Parts of one block are adjacent in the grid, so they run side
// by side; no part waits for a workgroup later in the grid, and the bounded wait falls
// back to computing s in place (same sums) if the others are late.
template <bool BF16, int LPR, int RV>
__global__ void __launch_bounds__(kThreads) delta_fused_kernel(DeltaArgs a) {
  constexpr int kXsBytes = ShrinkLds<LPR>::kVecs * 16;
  constexpr int kSBytes = kSLdsFloats * 4;
  constexpr int ESZ = BF16 ? 2 : 4;
  constexpr int VE = 16 / ESZ;
  constexpr int r = RV * VE;
  __shared__ int pid[kPidSlots];
  __shared__ int nreal;
  __shared__ int flag;
  __shared__ uint4 smem[(kXsBytes > kSBytes ? kXsBytes : kSBytes) / 16];  // xs or s rows
  float* s_lds = reinterpret_cast<float*>(smem);
  const int tid = threadIdx.x;
  const int blk = blockIdx.x / a.nchunk, g = blockIdx.x % a.nchunk;
  const int pv0 = tid < kPidSlots ? load_pid(a, blk, 0) : 0;  // with the expert id
  const int e = block_expert(a, blk);
  if (e < 0) return;
  // this thread's expand column; its weights go out first
  const int n = g * a.cpp + tid;
  const bool n_ok = tid < a.cpp && n < a.N;
  int nc[1] = {n_ok ? n : a.N};
  uint4 bv[1][RV];
  load_b_rows<BF16, RV, 1>(a, e, nc, bv);
  const int soff[1] = {(n_ok ? n / (a.N / a.slices) : 0) * r};
  const bool shrinker = g < a.rgroups;
  if (shrinker) {
    shrink_item<BF16, LPR, true>(a, blk, g, e, pv0, pid, &nreal, smem);
    __builtin_amdgcn_s_waitcnt(0);  // this wave's s stores have completed
    __syncthreads();
    if (tid == 0) arrive(a, blk, 1);
  }
  const float sc = a.scale[e / a.E];
  const int pg = min(kPidSlots, kSLdsFloats / a.R);
  bool ready = true;
  for (int j0 = 0; j0 < a.BM; j0 += pg) {
    int pv = j0 == 0 ? pv0 : (tid < pg ? load_pid(a, blk, j0) : a.numel);
    if (tid >= pg) pv = a.numel;
    __syncthreads();
    publish_pids(a, pv, pid, &nreal);
    if (j0 == 0 && tid == 0) {
      int ok = 0;
      for (int it = 0; it < a.spin_limit; ++it) {
        const int w = __hip_atomic_load(a.sync + blk, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if ((w & 0xffff) >= a.rgroups) {
          ok = 1;
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
      flag = ok;
    }
    __syncthreads();
    const int nr = nreal;
    if (nr == 0) break;
    ready = flag != 0;
    float ov[kPG][1];  // old out values of the first pairs, loaded before s is needed
#pragma unroll
    for (int q = 0; q < kPG; ++q) ov[q][0] = load_out<BF16>(a, pid[q], nc[0], q < nr && n_ok);
    if (ready) {
      load_s_rows<true>(a, pid, nr, s_lds);
    } else {
      compute_s_rows<BF16, LPR>(a, e, pid, nr, s_lds);
    }
    __syncthreads();
    expand_outputs<BF16, RV, 1>(a, bv, pid, nr, s_lds, nc, soff, sc, ov);
    if (nr < pg) break;  // the block's real entries ended in this pass
  }
  __syncthreads();
  if (tid == 0) arrive(a, blk, 1 << 16);
}

template <bool BF16>
hipError_t shrink_dispatch(const DeltaArgs& a, int lpr, int grid, hipStream_t st) {
  switch (lpr) {
    case 8: hipLaunchKernelGGL((shrink_kernel<BF16, 8>), dim3(grid), dim3(256), 0, st, a); break;
    case 16: hipLaunchKernelGGL((shrink_kernel<BF16, 16>), dim3(grid), dim3(256), 0, st, a); break;
    case 32: hipLaunchKernelGGL((shrink_kernel<BF16, 32>), dim3(grid), dim3(256), 0, st, a); break;
    case 64: hipLaunchKernelGGL((shrink_kernel<BF16, 64>), dim3(grid), dim3(256), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <bool BF16>
hipError_t expand_dispatch(const DeltaArgs& a, int rv, int grid, hipStream_t st) {
  switch (rv) {
    case 1: hipLaunchKernelGGL((expand_kernel<BF16, 1>), dim3(grid), dim3(256), 0, st, a); break;
    case 2: hipLaunchKernelGGL((expand_kernel<BF16, 2>), dim3(grid), dim3(256), 0, st, a); break;
    case 4: hipLaunchKernelGGL((expand_kernel<BF16, 4>), dim3(grid), dim3(256), 0, st, a); break;
    case 8: hipLaunchKernelGGL((expand_kernel<BF16, 8>), dim3(grid), dim3(256), 0, st, a); break;
    case 16: hipLaunchKernelGGL((expand_kernel<BF16, 16>), dim3(grid), dim3(256), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <bool BF16, int LPR>
hipError_t delta_dispatch_rv(const DeltaArgs& a, int rv, int grid, hipStream_t st) {
  switch (rv) {
    case 1: hipLaunchKernelGGL((delta_fused_kernel<BF16, LPR, 1>), dim3(grid), dim3(256), 0, st, a); break;
    case 2: hipLaunchKernelGGL((delta_fused_kernel<BF16, LPR, 2>), dim3(grid), dim3(256), 0, st, a); break;
    case 4: hipLaunchKernelGGL((delta_fused_kernel<BF16, LPR, 4>), dim3(grid), dim3(256), 0, st, a); break;
    case 8: hipLaunchKernelGGL((delta_fused_kernel<BF16, LPR, 8>), dim3(grid), dim3(256), 0, st, a); break;
    case 16: hipLaunchKernelGGL((delta_fused_kernel<BF16, LPR, 16>), dim3(grid), dim3(256), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <bool BF16>
hipError_t delta_dispatch(const DeltaArgs& a, int lpr, int rv, int grid, hipStream_t st) {
  switch (lpr) {
    case 8: return delta_dispatch_rv<BF16, 8>(a, rv, grid, st);
    case 16: return delta_dispatch_rv<BF16, 16>(a, rv, grid, st);
    case 32: return delta_dispatch_rv<BF16, 32>(a, rv, grid, st);
    case 64: return delta_dispatch_rv<BF16, 64>(a, rv, grid, st);
    default: return hipErrorInvalidValue;
  }
}

int rank_vectors(const DeltaArgs& a, bool bf16) {
  return (a.R / a.slices) * (bf16 ? 2 : 4) / 16;
}

}  // namespace

int expand_cols_per_item(int32_t R, int32_t slices, int elem_bytes) {
  const int rv = (R / slices) * elem_bytes / 16;
  return cols_per_thread(rv) * kThreads;
}

int shrink_rows_per_item(int32_t K, int elem_bytes) {
  const int64_t row_bytes = (int64_t)K * elem_bytes;
  int rpi = 4;
  while (rpi < 32 && (int64_t)(rpi * 2) * row_bytes <= kShrinkItemBytes) rpi *= 2;
  return rpi;
}

hipError_t launch_shrink(const DeltaArgs& a, bool bf16, int rows_per_item, int grid,
                         hipStream_t stream) {
  const int lpr = 256 / rows_per_item;
  return bf16 ? shrink_dispatch<true>(a, lpr, grid, stream)
              : shrink_dispatch<false>(a, lpr, grid, stream);
}

hipError_t launch_expand(const DeltaArgs& a, bool bf16, int grid, hipStream_t stream) {
  const int rv = rank_vectors(a, bf16);
  return bf16 ? expand_dispatch<true>(a, rv, grid, stream)
              : expand_dispatch<false>(a, rv, grid, stream);
}

hipError_t launch_delta(const DeltaArgs& a, bool bf16, int rows_per_item, int grid,
                        hipStream_t stream) {
  const int lpr = 256 / rows_per_item;
  const int rv = rank_vectors(a, bf16);
  return bf16 ? delta_dispatch<true>(a, lpr, rv, grid, stream)
              : delta_dispatch<false>(a, lpr, rv, grid, stream);
}

}  // namespace mol
