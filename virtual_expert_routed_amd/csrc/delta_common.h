// Device helpers shared by the shrink/expand translation units of libmol (not installed):
// bf16 conversions, the 16-byte dot products, routing reads of an aligned block, buffer
// and direct-to-LDS loads, and out element access.
#pragma once

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

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// acc + a.lo * b.lo + a.hi * b.hi for two packed bf16 pairs, in one v_dot2c_f32_bf16 (the
// bf16 products are exact in fp32; no unpacking of either operand)
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), acc, false);
}

// acc += <a, x> over one 16-byte vector of each (element pairs in ascending order)
template <bool BF16>
__device__ __forceinline__ float dot16(const uint4& a, const uint4& x, float acc) {
  if constexpr (BF16) {
    acc = dot2_bf16(a.x, x.x, acc);
    acc = dot2_bf16(a.y, x.y, acc);
    acc = dot2_bf16(a.z, x.z, acc);
    acc = dot2_bf16(a.w, x.w, acc);
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

// Output columns per thread of an expand item. One: at decode, twice as many items of
// half the weight bytes keep more loads in flight than two columns per thread (measured
// on MI355X: 12-23 % faster expands at 23 and 128 tokens), and every rank fits.
__host__ __device__ constexpr int cols_per_thread(int /*rv*/) { return 1; }

constexpr int kExpandCols = 256;  // output columns per expand work item

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


// What a work item needs to know of its block before its first weight load: the block's
// virtual expert (e < 0: the item has nothing to do, because the block is past the live
// blocks or in the sentinel bucket), its first NH entries as scalars (numel past the
// block) and how many of them are real pairs (a prefix).
template <int NH>
struct BlockHeadN {
  int e;
  int p[NH];
  int nq;
  bool all_here;  // the block has no real pairs past its first NH entries
};
using BlockHead = BlockHeadN<kPG>;

// The routing arguments a delta item needs first. The kernels take them as their leading
// scalar parameters (MOL_ROUTE_PARAMS), and the library is built with kernel-argument
// preloading for the first eight parameters, so they arrive in scalar registers with the
// wave and the item's routing reads can leave at its first instructions, with no fetch of
// the argument buffer before them.
struct RouteArgs {
  const int32_t* sorted;
  const int32_t* expert_ids;
  const int32_t* npp;
  int32_t BM;
  FastDiv per_div;  // work items per block, as a multiply-shift divisor (m, l)
  int32_t per;      // work items per block
};

#define MOL_ROUTE_PARAMS                                                               \
  const int32_t *r_sorted, const int32_t *r_eids, const int32_t *r_npp, int32_t r_bm, \
      uint32_t r_pm, uint32_t r_pl, int32_t r_per
#define MOL_ROUTE_ARGS(a, per, div) \
  (a).sorted, (a).expert_ids, (a).npp, (a).BM, (div).m, (div).l, (per)
#define MOL_ROUTE_MAKE \
  RouteArgs{r_sorted, r_eids, r_npp, r_bm, FastDiv{(uint32_t)r_per, r_pm, r_pl}, r_per}

// The block and the item within it of this workgroup.
__device__ __forceinline__ int route_block(const RouteArgs& r) {
  return fdiv((int)blockIdx.x, r.per_div);
}

// The kernel arguments a delta item reads before its weight loads, all fetched at its start
// in one batch. (Left to itself the compiler fetches each one where it is first used, and a
// fetch that misses the scalar cache then costs one more round trip between the routing
// reads and the weight loads.)
__device__ __forceinline__ void fetch_args(const DeltaArgs& a) {
  asm volatile("" ::"s"(a.xin), "s"(a.A), "s"(a.B), "s"(a.scale), "s"(a.s), "s"(a.out),
               "s"(a.ranks), "s"(a.ld_x), "s"(a.ld_out));
  asm volatile("" ::"s"(a.row_div), "s"(a.R), "s"(a.K), "s"(a.slices), "s"(a.N), "s"(a.E),
               "s"(a.numel), "s"(a.V), "s"(a.max_blocks));
  asm volatile("" ::"s"(a.f_bm.m), "s"(a.f_bm.l), "s"(a.f_e.m), "s"(a.f_e.l), "s"(a.f_r.m),
               "s"(a.f_r.l), "s"(a.f_w.m), "s"(a.f_w.l), "s"(a.f_rd.m), "s"(a.f_rd.l),
               "s"(a.f_r4.m), "s"(a.f_r4.l));
}

// Every routing read of the head leaves in one batch: the padded count, the expert id and
// the entries are read from clamped indices with no branch between the loads, so an item
// pays one round trip to the routing before it can issue its weight loads.
template <int NH = kPG>
__device__ __forceinline__ BlockHeadN<NH> block_head(const DeltaArgs& a, const RouteArgs& r,
                                                     int blk) {
  const int32_t* sp = r.sorted + (int64_t)blk * r.BM;
  const int last = r.BM - 1;
  int v[NH];
#pragma unroll
  for (int i = 0; i < NH; ++i) v[i] = sp[i < last ? i : last];
  const int er = r.expert_ids[blk];
  const int npp = *r.npp;
  // after the routing reads, so that they stay scalar loads, and in their round trip
  fetch_args(a);
  BlockHeadN<NH> h;
  h.nq = 0;
#pragma unroll
  for (int i = 0; i < NH; ++i) {
    h.p[i] = i <= last ? v[i] : a.numel;
    h.nq += real_pair(h.p[i], a.numel) ? 1 : 0;
  }
  h.all_here = h.nq < NH || r.BM <= NH;
  const int nb = npp < 0 ? 0 : fdiv(npp, a.f_bm);
  const int live = nb > a.max_blocks ? a.max_blocks : nb;
  h.e = (blk < live && real_expert(er, a.V)) ? er : -1;
  return h;
}

// Rank of the slot of virtual expert e: its slot_ranks entry clamped to [0, r], or r = R /
// slices when there is no rank table (one load, uniform over the workgroup).
__device__ __forceinline__ int slot_rank(const DeltaArgs& a, int e) {
  const int r = a.R / a.slices;
  if (!a.ranks) return r;
  const int v = a.ranks[fdiv(e, a.f_e)];
  return v < 0 ? 0 : (v > r ? r : v);
}

// The first `keep` elements of a 16-byte weight vector (8 bf16 or 4 fp32), the rest zero.
template <bool BF16>
__device__ __forceinline__ uint4 keep_first(uint4 v, int keep) {
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (BF16) {
      const uint32_t lo = keep > 2 * i ? 0x0000ffffu : 0u;
      const uint32_t hi = keep > 2 * i + 1 ? 0xffff0000u : 0u;
      w[i] &= lo | hi;
    } else {
      w[i] = keep > i ? w[i] : 0u;
    }
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// The sum over each group of LPR consecutive lanes (LPR a power of two up to 64), left in
// every lane of the group, by a butterfly in ascending distance d: cross-lane moves inside a
// row of 16 lanes for d = 1 to 8, a swizzle for 16, a permute for 32. Before the step of
// distance d >= 4 every aligned run of d lanes holds one value, and a half-row (d = 4) or row
// (d = 8) mirror maps each run onto its neighbour, so it adds the same two values an xor
// would; the two lanes of a pair add them in either order, which gives the same sum. The
// result depends only on LPR.
template <int CTRL>
__device__ __forceinline__ float from_lane(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
template <int LPR>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (LPR >= 2) v += from_lane<0xB1>(v);   // quad_perm [1, 0, 3, 2]
  if constexpr (LPR >= 4) v += from_lane<0x4E>(v);   // quad_perm [2, 3, 0, 1]
  if constexpr (LPR >= 8) v += from_lane<0x141>(v);  // row_half_mirror
  if constexpr (LPR >= 16) v += from_lane<0x140>(v); // row_mirror
  if constexpr (LPR >= 32)                            // lanes i and i ^ 16
    v += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F));
  if constexpr (LPR >= 64) v += __shfl_xor(v, 32, 64);
  return v;
}

// Branch-free 16-byte load: a masked address is clamped to the array's first element
// and its value replaced by zero.
__device__ __forceinline__ uint4 ld16_if(const char* base, int64_t off, bool ok) {
  const uint4 v = ld16(base + (ok ? off : 0));
  return ok ? v : make_uint4(0, 0, 0, 0);
}

// Non-temporal 16-byte load and store, for a stream that is read once and written once
// (the out rows a kernel updates in place): the hint keeps those lines from evicting data
// that other workgroups re-read from L2, such as an expert's weight tile.
typedef unsigned int nt_u4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 ld16_nt_if(const char* base, int64_t off, bool ok) {
  const nt_u4 v = __builtin_nontemporal_load(reinterpret_cast<const nt_u4*>(base + (ok ? off : 0)));
  return ok ? make_uint4(v.x, v.y, v.z, v.w) : make_uint4(0, 0, 0, 0);
}

__device__ __forceinline__ void st16_nt(char* p, uint4 v) {
  const nt_u4 t = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(t, reinterpret_cast<nt_u4*>(p));
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

// Direct-to-LDS 16-byte load: lane i of the wave writes at lds_wave_base + 16*i.
__device__ __forceinline__ void lds_dma16(const void* src, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds_wave_base,
                                   16, 0, 0);
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

}  // namespace
}  // namespace mol
