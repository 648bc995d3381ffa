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
// The fused kernel runs both in one launch: work items are handed out by an ordered
// ticket (one atomic per workgroup), all shrink items first. An expand item waits for its
// block's shrink items through a per-block counter; those items hold earlier tickets, so
// they are already running and never wait themselves - every wait ends. The last
// workgroup to take a ticket and the last consumer of each block put the counters back
// to zero for the next call.
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

// One shrink work item: rows [rg*RPI, rg*RPI+RPI) of A_v for every real pair of block blk.
template <bool BF16, int LPR>
__device__ __forceinline__ void shrink_item(const DeltaArgs& a, int blk, int rg, int* pid) {
  constexpr int ESZ = BF16 ? 2 : 4;
  constexpr int RPI = 256 / LPR;
  constexpr int SEG = 8;  // 16-byte vectors per lane held at once
  constexpr int PG = 4;   // pairs sharing one pass over the held vectors
  const int tid = threadIdx.x;
  const int lr = tid % LPR;
  const int row = rg * RPI + tid / LPR;
  const bool row_ok = row < a.R;
  const int e = a.expert_ids[blk];
  const int nvec = a.K * ESZ / 16;
  const int vpl = (nvec + LPR - 1) / LPR;
  const char* arow =
      (const char*)a.A + ((int64_t)e * a.R + (row_ok ? row : 0)) * (int64_t)a.K * ESZ;
  const char* xbase = (const char*)a.xin;
  const int64_t xstride = a.ld_x * ESZ;
  const int base = blk * a.BM;
  for (int j0 = 0; j0 < a.BM; j0 += kPidSlots) {
    __syncthreads();
    if (tid < kPidSlots) {
      const int j = j0 + tid;
      pid[tid] = j < a.BM ? a.sorted[base + j] : a.numel;
    }
    __syncthreads();
    for (int q0 = 0; q0 < kPidSlots; q0 += PG) {
      int p[PG];
#pragma unroll
      for (int i = 0; i < PG; ++i) p[i] = pid[q0 + i];
      if (!real_pair(p[0], a.numel)) return;  // real entries are a prefix of the block
      float acc[PG];
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
      if (lr == 0 && row_ok) {
#pragma unroll
        for (int i = 0; i < PG; ++i)
          if (real_pair(p[i], a.numel)) a.s[(int64_t)p[i] * a.R + row] = acc[i];
      }
    }
  }
}

// One expand work item: columns [chunk*256, chunk*256+256) for every real pair of block blk.
template <bool BF16, int RV>
__device__ __forceinline__ void expand_item(const DeltaArgs& a, int blk, int chunk, int* pid,
                                            float* s_lds) {
  constexpr int ESZ = BF16 ? 2 : 4;
  constexpr int VE = 16 / ESZ;
  constexpr int r = RV * VE;
  const int tid = threadIdx.x;
  const int n = chunk * kExpandCols + tid;
  const bool n_ok = n < a.N;
  const int e = a.expert_ids[blk];
  const float sc = a.scale[e / a.E];
  const int width = a.N / a.slices;
  const int soff = (n_ok ? n / width : 0) * r;
  const int R = a.R;
  uint4 bv[RV];
  const char* brow = (const char*)a.B + ((int64_t)e * a.N + (n_ok ? n : 0)) * (int64_t)(r * ESZ);
#pragma unroll
  for (int v = 0; v < RV; ++v) bv[v] = n_ok ? ld16(brow + v * 16) : make_uint4(0, 0, 0, 0);
  const int pg = min(kPidSlots, kSLdsFloats / R);
  const int base = blk * a.BM;
  for (int j0 = 0; j0 < a.BM; j0 += pg) {
    __syncthreads();
    if (tid < pg) {
      const int j = j0 + tid;
      pid[tid] = j < a.BM ? a.sorted[base + j] : a.numel;
    }
    __syncthreads();
    if (!real_pair(pid[0], a.numel)) return;
    for (int i = tid; i < pg * R; i += blockDim.x) {
      const int q = i / R, c = i - q * R;
      const int p = pid[q];
      s_lds[i] = real_pair(p, a.numel) ? a.s[(int64_t)p * R + c] : 0.f;
    }
    __syncthreads();
    for (int q = 0; q < pg; ++q) {
      const int p = pid[q];
      if (!real_pair(p, a.numel)) break;
      const float* sv = s_lds + q * R + soff;
      float acc = 0.f;
#pragma unroll
      for (int v = 0; v < RV; ++v) acc = dot16_s<BF16>(bv[v], sv + v * VE, acc);
      if (n_ok) {
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
  }
}

template <bool BF16, int LPR>
__global__ void __launch_bounds__(256) shrink_kernel(DeltaArgs a) {
  __shared__ int pid[kPidSlots];
  const int blk = blockIdx.x / a.rgroups, rg = blockIdx.x % a.rgroups;
  if (blk >= live_blocks(a)) return;
  if (!real_expert(a.expert_ids[blk], a.V)) return;
  shrink_item<BF16, LPR>(a, blk, rg, pid);
}

template <bool BF16, int RV>
__global__ void __launch_bounds__(256) expand_kernel(DeltaArgs a) {
  __shared__ int pid[kPidSlots];
  __shared__ float s_lds[kSLdsFloats];
  const int blk = blockIdx.x / a.nchunk, c = blockIdx.x % a.nchunk;
  if (blk >= live_blocks(a)) return;
  if (!real_expert(a.expert_ids[blk], a.V)) return;
  expand_item<BF16, RV>(a, blk, c, pid, s_lds);
}

template <bool BF16, int LPR, int RV>
__global__ void __launch_bounds__(256) delta_fused_kernel(DeltaArgs a) {
  __shared__ int pid[kPidSlots];
  __shared__ float s_lds[kSLdsFloats];
  __shared__ int ticket;
  int32_t* ready = a.sync + 64;
  int32_t* consumed = a.sync + 64 + a.max_blocks;
  if (threadIdx.x == 0) {
    const int t = __hip_atomic_fetch_add(a.sync, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // the last ticket of the grid: no workgroup of this launch touches the counter again
    if (t == (int)gridDim.x - 1)
      __hip_atomic_store(a.sync, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    ticket = t;
  }
  __syncthreads();
  const int t = ticket;
  const int nb = live_blocks(a);
  const int nshrink = nb * a.rgroups;
  if (t < nshrink) {
    const int blk = t / a.rgroups, rg = t % a.rgroups;
    if (!real_expert(a.expert_ids[blk], a.V)) return;
    shrink_item<BF16, LPR>(a, blk, rg, pid);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __syncthreads();
    if (threadIdx.x == 0)
      __hip_atomic_fetch_add(ready + blk, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  const int u = t - nshrink;
  if (u >= nb * a.nchunk) return;
  const int blk = u / a.nchunk, c = u % a.nchunk;
  if (!real_expert(a.expert_ids[blk], a.V)) return;
  if (threadIdx.x == 0) {
    // producers hold earlier tickets: they are resident and never wait, so this ends
    while (__hip_atomic_load(ready + blk, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) <
           a.rgroups)
      __builtin_amdgcn_s_sleep(1);
  }
  __syncthreads();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  expand_item<BF16, RV>(a, blk, c, pid, s_lds);
  __syncthreads();
  if (threadIdx.x == 0) {
    const int old =
        __hip_atomic_fetch_add(consumed + blk, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old == a.nchunk - 1) {  // last reader of this block's s: reset for the next call
      __hip_atomic_store(ready + blk, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(consumed + blk, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
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
