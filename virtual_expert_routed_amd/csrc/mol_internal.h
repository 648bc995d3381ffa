// Internal declarations shared by the HIP translation units of libmol (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mol {

constexpr int kMaxBuckets = 8192;     // V + 1 <= 8192
constexpr int kAlignSmallMax = 4096;  // pairs the one-workgroup align handles
constexpr int kAlignTile = 2048;      // pairs per tile of the three-kernel align
constexpr int kShrinkItemBytes = 32768;  // target weight bytes per shrink work item

struct AlignArgs {
  const int32_t* ids;
  const int32_t* lora;   // nullptr: ids are virtual ids
  int32_t topk;
  int32_t E;
  int32_t S;
  int32_t numel;
  int32_t V;             // number of virtual experts; bucket V is the sentinel bucket
  int32_t BM;
  int32_t nbits;         // bits needed to hold a bucket id in [0, V]
  int32_t* sorted;
  int32_t* expert_ids;
  int32_t* npp;
  int32_t* counts;       // three-kernel path: [ntiles][V+1] counts, then cursors
  int32_t* bucket_off;   // three-kernel path: [V+1] padded offsets
  int32_t* bucket_cnt;   // three-kernel path: [V+1] counts
  int32_t ntiles;
};

struct DeltaArgs {
  const void* xin;
  int64_t ld_x;
  int32_t row_div;
  const void* A;
  int32_t R;
  int32_t K;
  int32_t slices;
  const void* B;
  int32_t N;
  const float* scale;
  int32_t E;
  const int32_t* sorted;
  const int32_t* expert_ids;
  const int32_t* npp;
  int32_t numel;
  int32_t V;             // virtual experts: expert ids outside [0, V) are skipped
  int32_t BM;
  int32_t rgroups;       // shrink work items per block (row groups of A)
  int32_t nchunk;        // expand work items per block (column chunks of B)
  float* s;              // [numel, R]
  void* out;
  int64_t ld_out;
  int32_t max_blocks;
};

// host-side launchers (return the launch status)
hipError_t launch_virtual_topk(const int32_t* topk_ids, const int32_t* lora_ids, int32_t M,
                               int32_t topk, int32_t E, int32_t S, int32_t* out,
                               hipStream_t stream);
hipError_t launch_align_small(const AlignArgs& a, int waves, int groups, size_t lds_bytes,
                              hipStream_t stream);
hipError_t launch_align_large(const AlignArgs& a, hipStream_t stream);

// rows per shrink item (power of two in [4, 32]) for contraction length K
int shrink_rows_per_item(int32_t K, int elem_bytes);
// output columns per expand item for rank R / slices
int expand_cols_per_item(int32_t R, int32_t slices, int elem_bytes);

hipError_t launch_shrink(const DeltaArgs& a, bool bf16, int rows_per_item, int grid,
                         hipStream_t stream);
hipError_t launch_expand(const DeltaArgs& a, bool bf16, int grid, hipStream_t stream);

}  // namespace mol
