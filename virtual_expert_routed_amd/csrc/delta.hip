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

constexpr int kPidSlots = 64;     // pair ids staged per pass over a block

__device__ __forceinline__ bool real_pair(int p, int numel) {
  return (unsigned)p < (unsigned)numel;
}

// blocks that carry work: [0, npp / BM) clamped to the launched bound
__device__ __forceinline__ int live_blocks(const DeltaArgs& a) {
  const int nb = *a.npp / a.BM;
  return nb < 0 ? 0 : (nb > a.max_blocks ? a.max_blocks : nb);
}

__device__ __forceinline__ bool real_expert(int e, int V) { return (unsigned)e < (unsigned)V; }
constexpr int kSLdsFloats = 4096; // s rows staged per expand pass (16 KiB)

constexpr int kPG = 4;  // pairs sharing one pass over the held weight vectors

// agent-coherent accesses used to hand s from shrink to expand items of one launch
__device__ __forceinline__ void st_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_coherent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Dot products of rows rg*RPI + tid/LPR of A_e with the input rows of the pairs p[0..PG)
// (ids that are not real pairs are skipped). Afterwards lane 0 of each row's lane group
// holds the full sum in acc[i]. Each lane sums its vectors lr, lr+LPR, lr+2*LPR, ... in
// ascending order and the lanes are combined by a fixed xor tree, so the result depends
// only on (K, LPR) - not on SEG (vectors held at once) or PG (pairs per pass).
template <bool BF16, int LPR, int SEG = 8, int PG = 4>
__device__ __forceinline__ void shrink_rows(const DeltaArgs& a, int e, int rg, const int* p,
                                            float* acc) {
  constexpr int ESZ = BF16 ? 2 : 4;
  constexpr int RPI = 256 / LPR;
  const int tid = threadIdx.x;
  const int lr = tid % LPR;
  const int row = rg * RPI + tid / LPR;
  const bool row_ok = row < a.R;
  const int nvec = a.K * ESZ / 16;
  const int vpl = (nvec + LPR - 1) / LPR;
  const char* arow =
      (const char*)a.A + ((int64_t)e * a.R + (row_ok ? row : 0)) * (int64_t)a.K * ESZ;
  const char* xbase = (const char*)a.xin;
  const int64_t xstride = a.ld_x * ESZ;
#pragma unroll
  for (int i = 0; i < PG; ++i) acc[i] = 0.f;
  for (int m0 = 0; m0 < vpl; m0 += SEG) {
    uint4 av[SEG];
#pragma unroll
    for (int sg = 0; sg < SEG; ++sg) {
      const int v = lr + (m0 + sg) * LPR;
      av[sg] = (row_ok && v < nvec) ? ld16(arow + (int64_t)v * 16) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < PG; ++i) {
      if (real_pair(p[i], a.numel)) {
        const char* xr = xbase + (int64_t)(p[i] / a.row_div) * xstride;
#pragma unroll
        for (int sg = 0; sg < SEG; ++sg) {
          const int v = lr + (m0 + sg) * LPR;
          if (v < nvec) acc[i] = dot16<BF16>(av[sg], ld16(xr + (int64_t)v * 16), acc[i]);
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < PG; ++i) {
#pragma unroll
    for (int off = LPR / 2; off > 0; off >>= 1) acc[i] += __shfl_xor(acc[i], off, 64);
  }
}

// Stage the ids of block entries [j0, j0 + n) into pid (numel marks a padding entry).
__device__ __forceinline__ void stage_pids(const DeltaArgs& a, int blk, int j0, int n, int* pid) {
  const int tid = threadIdx.x;
  if (tid < n) {
    const int j = j0 + tid;
    pid[tid] = j < a.BM ? a.sorted[blk * a.BM + j] : a.numel;
  }
}

// One shrink work item: rows [rg*RPI, rg*RPI+RPI) of s for every real pair of block blk.
template <bool BF16, int LPR, bool COHERENT>
__device__ __forceinline__ void shrink_item(const DeltaArgs& a, int blk, int rg, int* pid) {
  constexpr int RPI = 256 / LPR;
  const int tid = threadIdx.x;
  const int lr = tid % LPR;
  const int row = rg * RPI + tid / LPR;
  const int e = a.expert_ids[blk];
  for (int j0 = 0; j0 < a.BM; j0 += kPidSlots) {
    __syncthreads();
    stage_pids(a, blk, j0, kPidSlots, pid);
    __syncthreads();
    for (int q0 = 0; q0 < kPidSlots; q0 += kPG) {
      int p[kPG];
#pragma unroll
      for (int i = 0; i < kPG; ++i) p[i] = pid[q0 + i];
      if (!real_pair(p[0], a.numel)) return;  // real entries are a prefix of the block
      float acc[kPG];
      shrink_rows<BF16, LPR>(a, e, rg, p, acc);
      if (lr == 0 && row < a.R) {
#pragma unroll
        for (int i = 0; i < kPG; ++i) {
          if (!real_pair(p[i], a.numel)) continue;
          float* d = a.s + (int64_t)p[i] * a.R + row;
          if constexpr (COHERENT) st_coherent(d, acc[i]); else *d = acc[i];
        }
      }
    }
  }
}

// s rows of the pairs pid[0..pg) into s_lds [pg][R], read from a.s.
template <bool COHERENT>
__device__ __forceinline__ void load_s_rows(const DeltaArgs& a, const int* pid, int pg,
                                            float* s_lds) {
  const int R = a.R;
  for (int i = threadIdx.x; i < pg * R; i += blockDim.x) {
    const int q = i / R, c = i - q * R;
    const int p = pid[q];
    float v = 0.f;
    if (real_pair(p, a.numel)) {
      const float* src = a.s + (int64_t)p * R + c;
      v = COHERENT ? ld_coherent(src) : *src;
    }
    s_lds[i] = v;
  }
}

// s rows of the pairs pid[0..pg) into s_lds [pg][R], computed here with exactly the
// arithmetic of the shrink items (used when they are not done in time).
template <bool BF16, int LPR>
__device__ __forceinline__ void compute_s_rows(const DeltaArgs& a, int e, const int* pid, int pg,
                                               float* s_lds) {
  constexpr int RPI = 256 / LPR;
  const int tid = threadIdx.x;
  const int lr = tid % LPR;
  for (int rg = 0; rg < a.rgroups; ++rg) {
    const int row = rg * RPI + tid / LPR;
    for (int q = 0; q < pg; ++q) {
      const int p = pid[q];
      if (!real_pair(p, a.numel)) break;
      float acc;
      shrink_rows<BF16, LPR, 1, 1>(a, e, rg, &p, &acc);  // light on registers, same sums
      if (lr == 0 && row < a.R) s_lds[q * a.R + row] = acc;
    }
  }
}

// out[p, n] += for the pairs pid[0..pg) of this pass, s rows staged in s_lds [pg][R].
template <bool BF16, int RV>
__device__ __forceinline__ void expand_outputs(const DeltaArgs& a, const uint4* bv, const int* pid,
                                               int pg, const float* s_lds, int n, int soff,
                                               float sc) {
  constexpr int VE = BF16 ? 8 : 4;
  if (n >= a.N) return;
  for (int q = 0; q < pg; ++q) {
    const int p = pid[q];
    if (!real_pair(p, a.numel)) break;
    const float* sv = s_lds + q * a.R + soff;
    float acc = 0.f;
#pragma unroll
    for (int v = 0; v < RV; ++v) acc = dot16_s<BF16>(bv[v], sv + v * VE, acc);
    if constexpr (BF16) {
      uint16_t* o = (uint16_t*)a.out + (int64_t)p * a.ld_out + n;
      const float old = __uint_as_float((uint32_t)*o << 16);
      *o = f32_to_bf16_rne(fmaf(sc, acc, old));
    } else {
      float* o = (float*)a.out + (int64_t)p * a.ld_out + n;
      *o = fmaf(sc, acc, *o);
    }
  }
}

template <bool BF16, int RV>
__device__ __forceinline__ void load_b_row(const DeltaArgs& a, int e, int n, uint4* bv) {
  constexpr int ESZ = BF16 ? 2 : 4;
  constexpr int r = RV * 16 / ESZ;
  const bool n_ok = n < a.N;
  const char* brow = (const char*)a.B + ((int64_t)e * a.N + (n_ok ? n : 0)) * (int64_t)(r * ESZ);
#pragma unroll
  for (int v = 0; v < RV; ++v) bv[v] = n_ok ? ld16(brow + v * 16) : make_uint4(0, 0, 0, 0);
}

// One expand work item: columns [chunk*256, chunk*256+256) for every real pair of block
// blk. FUSED: s comes from this launch's shrink items (or is computed here, see above).
template <bool BF16, int LPR, int RV, bool FUSED>
__device__ __forceinline__ void expand_item(const DeltaArgs& a, int blk, int chunk, int* pid,
                                            float* s_lds, int* flag) {
  constexpr int ESZ = BF16 ? 2 : 4;
  constexpr int r = RV * 16 / ESZ;
  const int tid = threadIdx.x;
  const int n = chunk * kExpandCols + tid;
  const int e = a.expert_ids[blk];
  const int width = a.N / a.slices;
  const int soff = (n < a.N ? n / width : 0) * r;
  const float sc = a.scale[e / a.E];
  const int pg = min(kPidSlots, kSLdsFloats / a.R);
  uint4 bv[RV];
  load_b_row<BF16, RV>(a, e, n, bv);  // weights first: they do not depend on s
  bool ready = true;
  if constexpr (FUSED) {
    if (tid == 0) {
      int ok = 0;
      for (int it = 0; it < a.spin_limit; ++it) {
        const int w = __hip_atomic_load(a.sync + blk, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if ((w & 0xffff) >= a.rgroups) {
          ok = 1;
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
      *flag = ok;
    }
    __syncthreads();
    ready = *flag != 0;
  }
  if (ready) {
    for (int j0 = 0; j0 < a.BM; j0 += pg) {
      __syncthreads();
      stage_pids(a, blk, j0, pg, pid);
      __syncthreads();
      if (!real_pair(pid[0], a.numel)) break;
      load_s_rows<FUSED>(a, pid, pg, s_lds);
      __syncthreads();
      expand_outputs<BF16, RV>(a, bv, pid, pg, s_lds, n, soff, sc);
    }
  } else if constexpr (FUSED) {
    for (int j0 = 0; j0 < a.BM; j0 += pg) {
      __syncthreads();
      stage_pids(a, blk, j0, pg, pid);
      __syncthreads();
      if (!real_pair(pid[0], a.numel)) break;
      compute_s_rows<BF16, LPR>(a, e, pid, pg, s_lds);
      __syncthreads();
      uint4 bw[RV];
      load_b_row<BF16, RV>(a, e, n, bw);
      expand_outputs<BF16, RV>(a, bw, pid, pg, s_lds, n, soff, sc);
    }
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

template <bool BF16, int LPR>
__global__ void __launch_bounds__(256) shrink_kernel(DeltaArgs a) {
  __shared__ int pid[kPidSlots];
  const int blk = blockIdx.x / a.rgroups, rg = blockIdx.x % a.rgroups;
  if (blk >= live_blocks(a)) return;
  if (!real_expert(a.expert_ids[blk], a.V)) return;
  shrink_item<BF16, LPR, false>(a, blk, rg, pid);
}

template <bool BF16, int RV>
__global__ void __launch_bounds__(256) expand_kernel(DeltaArgs a) {
  __shared__ int pid[kPidSlots];
  __shared__ float s_lds[kSLdsFloats];
  const int blk = blockIdx.x / a.nchunk, c = blockIdx.x % a.nchunk;
  if (blk >= live_blocks(a)) return;
  if (!real_expert(a.expert_ids[blk], a.V)) return;
  expand_item<BF16, 64, RV, false>(a, blk, c, pid, s_lds, nullptr);
}

template <bool BF16, int LPR, int RV>
__global__ void __launch_bounds__(256) delta_fused_kernel(DeltaArgs a) {
  __shared__ int pid[kPidSlots];
  __shared__ float s_lds[kSLdsFloats];
  __shared__ int flag;
  const int nb = live_blocks(a);
  const int nshrink = a.max_blocks * a.rgroups;
  const int bid = blockIdx.x;
  if (bid < nshrink) {
    const int blk = bid / a.rgroups, rg = bid % a.rgroups;
    if (blk >= nb || !real_expert(a.expert_ids[blk], a.V)) return;
    shrink_item<BF16, LPR, true>(a, blk, rg, pid);
    __builtin_amdgcn_s_waitcnt(0);  // this wave's s stores have completed
    __syncthreads();
    if (threadIdx.x == 0) arrive(a, blk, 1);
    return;
  }
  const int u = bid - nshrink;
  const int blk = u / a.nchunk, c = u % a.nchunk;
  if (blk >= nb || !real_expert(a.expert_ids[blk], a.V)) return;
  expand_item<BF16, LPR, RV, true>(a, blk, c, pid, s_lds, &flag);
  __syncthreads();
  if (threadIdx.x == 0) arrive(a, blk, 1 << 16);
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
