// Internal declarations shared by the HIP translation units of libmol (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fastdiv.h"

namespace mol {

constexpr int kMaxBuckets = 8192;     // V + 1 <= 8192
constexpr int kAlignSmallMax = 4096;  // pairs the one-workgroup align handles

// The small align's buckets per thread (V + 1 buckets over 1024 threads, rounded up to a power
// of two) and the stride of its counter rows in ints: V + 1 rounded up to a multiple of that,
// so that one thread's buckets of one row are a single aligned LDS access.
__host__ __device__ constexpr int align_small_bpt(int nb) {
  return nb <= 1024 ? 1 : nb <= 2048 ? 2 : nb <= 4096 ? 4 : 8;
}
__host__ __device__ constexpr int align_small_stride(int nb) {
  return (nb + align_small_bpt(nb) - 1) / align_small_bpt(nb) * align_small_bpt(nb);
}
constexpr int kShrinkItemBytes = 32768;  // target weight bytes per shrink work item
constexpr int kMfmaMinNumel = 4096;      // MFMA kernels are launched from this many pairs
constexpr int kMaxRankVecs = 16;         // 16-byte vectors in one rank row slice (256 bytes)

// A batch takes the bf16 MFMA kernels for all of its blocks when it is large enough to hold
// dense blocks in numbers: from kMfmaMinNumel pairs and 8 pairs per bucket on average. Its
// VALU kernels are then not launched at all; a block of few pairs still costs less as a
// mostly empty MFMA tile than as a VALU item.
inline bool mfma_batch(int64_t numel, int64_t V) {
  return numel >= kMfmaMinNumel && numel >= 8 * (V + 1);
}

// The work plan the align writes beside the routing when asked, for such a batch (int32
// words): [0] the number of runs D, [1..7] 0; from word kPlanHeader, D runs of
// kPlanDenseInts words {first block, blocks (1..kPlanDenseBlocks), virtual expert, 0}:
// consecutive blocks of one real bucket, in bucket order, every block of a real bucket in
// exactly one run (the sentinel bucket has none). A block holds at least one real pair, so
// there are at most min(max_blocks, numel) runs.
constexpr int kPlanHeader = 8;
constexpr int kPlanDenseInts = 4;
constexpr int kPlanDenseBlocks = 4;

inline int64_t plan_max_runs(int64_t numel, int64_t max_blocks) {
  return numel < max_blocks ? numel : max_blocks;
}
inline int64_t plan_words(int64_t numel, int64_t max_blocks) {
  return kPlanHeader + kPlanDenseInts * plan_max_runs(numel, max_blocks);
}

struct AlignArgs {
  const int32_t* ids;
  const int32_t* lora;   // nullptr: ids are virtual ids
  int32_t topk;
  int32_t E;
  int32_t S;
  int32_t numel;
  int32_t V;             // number of virtual experts; bucket V is the sentinel bucket
  int32_t BM;
  int32_t bm_shift;      // log2(BM) when BM is a power of two, else -1
  int32_t* sorted;
  int32_t* expert_ids;
  int32_t* npp;
  int32_t* counts;       // three-kernel path: [ntiles][V+1] counts, then earlier-tile counts
  int32_t* totals;       // three-kernel path: [V+1] pairs per bucket
  int32_t ntiles;
  int32_t tile;          // three-kernel path: pairs per tile
  int32_t per;           // one-launch path: pairs of each walker's contiguous range
  FastDiv f_topk;        // topk (token of a pair)
  FastDiv f_per;         // per (walker of a pair)
  FastDiv f_bm;          // BM
  FastDiv f_groups;      // workgroups of the one-launch path
  int32_t* plan;         // the work plan (nullptr: none is written)
  int32_t dmax;          // runs the plan has room for
  int32_t max_blocks;    // the routing's block bound
};

// Tiles of the three-kernel align: at most 64 of them up to 1M pairs (the column scan walks
// the tiles one by one), at least 512 pairs each, a multiple of 64.
inline int64_t align_tile(int64_t numel) {
  int64_t t = (numel + 63) / 64;
  t = t < 512 ? 512 : (t > 16384 ? 16384 : t);
  return (t + 63) / 64 * 64;
}

// Arguments of the delta kernels. Laid out densely (pointers, then 64-bit strides, then
// 32-bit fields, then the divisors) so that a kernel fetches all of it in a few wide scalar
// loads, in the same round trip as its routing reads.
struct DeltaArgs {
  const void* xin;
  const void* A;
  const void* B;
  const float* scale;
  const int32_t* sorted;
  const int32_t* expert_ids;
  const int32_t* npp;
  float* s;              // [numel, R]
  void* out;
  const int32_t* ranks;  // [S] per-slot ranks (clamped to [0, R/slices]) or nullptr
  int64_t ld_x;
  int64_t ld_out;
  int32_t row_div;
  int32_t R;
  int32_t K;
  int32_t slices;
  int32_t N;
  int32_t E;
  int32_t numel;
  int32_t V;             // virtual experts: expert ids outside [0, V) are skipped
  int32_t BM;
  int32_t rgroups;       // shrink work items per block (row groups of A)
  int32_t nchunk;        // expand work items per block (column chunks of B)
  int32_t max_blocks;
  // the launch's fixed divisors, as multiply-shift constants (set by with_divisors)
  FastDiv f_rg;          // rgroups
  FastDiv f_nc;          // nchunk
  FastDiv f_bm;          // BM
  FastDiv f_e;           // E
  FastDiv f_r;           // R / slices (rank of one slice)
  FastDiv f_w;           // N / slices (columns of one slice)
  FastDiv f_rd;          // row_div
  FastDiv f_r4;          // R / 4 (16-byte vectors of one s row)
};

// Host: fill the multiply-shift divisors of a from its fields (before every launch).
inline void with_divisors(DeltaArgs& a) {
  a.f_rg = make_fastdiv((uint32_t)(a.rgroups > 0 ? a.rgroups : 1));
  a.f_nc = make_fastdiv((uint32_t)(a.nchunk > 0 ? a.nchunk : 1));
  a.f_bm = make_fastdiv((uint32_t)a.BM);
  a.f_e = make_fastdiv((uint32_t)a.E);
  a.f_r = make_fastdiv((uint32_t)(a.slices > 0 ? a.R / a.slices : a.R));
  a.f_w = make_fastdiv((uint32_t)(a.slices > 0 ? a.N / a.slices : a.N));
  a.f_rd = make_fastdiv((uint32_t)a.row_div);
  a.f_r4 = make_fastdiv((uint32_t)(a.R / 4 > 0 ? a.R / 4 : 1));
}

// The combine after the down projection, and its form fused with the down-stage expand.
struct CombineArgs {
  const void* rows;        // combine: [M*topk, N] pair rows, ld_rows apart
  int64_t ld_rows;
  const int32_t* topk_ids; // [M, topk] base expert ids; pairs outside [0, E) have no row
  const float* weights;    // [M, topk] router weights
  const int32_t* lora;     // fused: [M] LoRA slot per token
  int32_t M;
  int32_t topk;
  int32_t E;
  int32_t S;
  int32_t N;
  int32_t R;               // fused: rank (one slice)
  const float* s;          // fused: [M*topk, R]
  const void* B;           // fused: [E*S, N, R]
  const float* scale;      // fused: [S]
  const int32_t* ranks;    // fused: [S] per-slot ranks or nullptr
  const void* base;        // fused: [M*topk, N] base rows, ld_base apart
  int64_t ld_base;
  void* y;                 // [M, N], ld_y apart
  int64_t ld_y;
};

// The base MoE grouped GEMM of a stage, optionally with the LoRA delta in its epilogue.
struct GemmArgs {
  DeltaArgs route;         // routing of the base-expert blocks (V = E)
  const void* xin;
  int64_t ld_x;
  int32_t row_div;
  const void* W;           // [E, N, K]
  int32_t K;
  int32_t N;
  int32_t rgroups;         // work items per block (groups of output columns)
  void* out;               // [numel, ld_out]
  int64_t ld_out;
  const float* s;          // fused delta: [numel, R] from the LoRA shrink; nullptr: base only
  int32_t R;
  int32_t slices;
  const void* B;           // [E*S, N, R/slices]
  const float* scale;      // [S]
  const int32_t* ranks;    // [S] or nullptr
  const int32_t* lora;     // [numel / topk] slot per token
  int32_t topk;
  int32_t E;
  int32_t S;
};

// host-side launchers (return the launch status)
hipError_t launch_virtual_topk(const int32_t* topk_ids, const int32_t* lora_ids, int32_t M,
                               int32_t topk, int32_t E, int32_t S, int32_t* out,
                               hipStream_t stream);
hipError_t launch_align_small(const AlignArgs& a, int waves, int groups, size_t lds_bytes,
                              hipStream_t stream);
hipError_t launch_align_large(const AlignArgs& a, size_t scatter_lds_bytes, hipStream_t stream);

// rows per shrink item (power of two in [4, 32]) for contraction length K
int shrink_rows_per_item(int32_t K, int elem_bytes);
// output columns per expand item for rank R / slices
int expand_cols_per_item(int32_t R, int32_t slices, int elem_bytes);

hipError_t launch_shrink(const DeltaArgs& a, bool bf16, int rows_per_item, int grid,
                         hipStream_t stream);
hipError_t launch_expand(const DeltaArgs& a, bool bf16, int grid, hipStream_t stream);
// bf16 MFMA kernels, for every block of a batch that takes them (mfma_batch)
// rows of A_v per MFMA shrink work item (the grid is max_blocks * cdiv(R, this))
int shrink_mfma_row_tile(int32_t R);
hipError_t launch_shrink_mfma(const DeltaArgs& a, int items, hipStream_t stream);
hipError_t launch_expand_mfma(const DeltaArgs& a, int grid, hipStream_t stream);
// the expand over the plan's dense runs: items = dense-entry room x column chunks; entries
// past the plan's count are empty
hipError_t launch_expand_mfma_runs(const DeltaArgs& a, const int32_t* plan, int items,
                                   hipStream_t stream);
// base grouped GEMM (+ fused delta when g.s is set): rows_per_item as for the shrink
hipError_t launch_moe_gemm(const GemmArgs& g, bool bf16, int rows_per_item, int grid,
                           hipStream_t stream);
// combine: one wave per (token, 64 16-byte vectors of columns)
hipError_t launch_combine(const CombineArgs& a, bool bf16, hipStream_t stream);
// fused expand + combine: ranks it is built for (R/8 or R/4 a power of two up to 16)
bool fused_rank_supported(int32_t R, bool bf16);
hipError_t launch_expand_combine(const CombineArgs& a, bool bf16, hipStream_t stream);

}  // namespace mol
