// C ABI of libmol: host-side validation, sizing and launch (declared in include/mol.h).
// Every check happens before any HIP call, so argument errors never touch the device.
#include "mol.h"

#include <algorithm>
#include <atomic>
#include <limits>
#include <mutex>

#include "mol_internal.h"

namespace {

constexpr int64_t kI32Max = std::numeric_limits<int32_t>::max();

int64_t cdiv64(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t round256(int64_t a) { return (a + 255) / 256 * 256; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Max dynamic LDS per workgroup, cached per device (only the one-workgroup align asks).
std::atomic<int> g_lds_bytes[64];

int device_lds_bytes() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 65536;
  int v = g_lds_bytes[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    int attr = 0;
    if (hipDeviceGetAttribute(&attr, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) !=
            hipSuccess ||
        attr <= 0)
      attr = 65536;
    v = attr < 163840 ? attr : 163840;
    g_lds_bytes[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}


mol_status hip_status(hipError_t e) { return e == hipSuccess ? MOL_OK : MOL_E_HIP; }

// number of blocks any routing of numel pairs over V virtual experts can produce
int64_t max_blocks_of(int64_t numel, int64_t V, int64_t BM) {
  const int64_t nz = numel < V + 1 ? numel : V + 1;
  return cdiv64(numel + nz * (BM - 1), BM);
}

int64_t align_check(int64_t numel, int32_t V, int32_t BM) {
  if (numel < 0 || V < 1 || BM < 1) return -MOL_E_ARG;
  if ((int64_t)V + 1 > MOL_MAX_BUCKETS || BM > MOL_MAX_BLOCK_M) return -MOL_E_LIMIT;
  if (numel > kI32Max) return -MOL_E_LIMIT;
  const int64_t mb = max_blocks_of(numel, V, BM);
  if (mb * BM > kI32Max) return -MOL_E_LIMIT;
  return mb;
}

struct StageCheck {
  mol_status st;
  int64_t max_blocks;
};

// checks shared by shrink, expand and delta (routing arguments)
StageCheck routing_check(const int32_t* sorted_ids, const int32_t* expert_ids,
                         const int32_t* npp, int32_t numel, int32_t V, int32_t BM) {
  const int64_t mb = align_check(numel, V, BM);
  if (mb < 0) return {(mol_status)(-mb), 0};
  if (numel > 0 && (!sorted_ids || !expert_ids || !npp)) return {MOL_E_ARG, 0};
  return {MOL_OK, mb};
}

mol_status shrink_check(int32_t dtype, const void* xin, int64_t ld_x, int32_t row_div,
                        const void* A, int32_t R, int32_t K, int32_t numel, float* s) {
  if (dtype != MOL_F32 && dtype != MOL_BF16) return MOL_E_DTYPE;
  if (R < 1 || K < 1 || row_div < 1 || ld_x < K) return MOL_E_ARG;
  if (numel > 0 && (!xin || !A || !s)) return MOL_E_ARG;
  const int esz = dtype == MOL_BF16 ? 2 : 4;
  if (((int64_t)K * esz) % 16 || (ld_x * esz) % 16) return MOL_E_ALIGN;
  if (numel > 0 && (!aligned16(xin) || !aligned16(A) || !aligned16(s))) return MOL_E_ALIGN;
  if ((int64_t)R * K * esz >= (int64_t(1) << 31)) return MOL_E_LIMIT;  // one expert's A
  return MOL_OK;
}

mol_status expand_check(int32_t dtype, int32_t R, int32_t slices, const void* B, int32_t N,
                        const float* scale, int32_t E, int32_t V, int32_t numel,
                        const void* out, int64_t ld_out) {
  if (dtype != MOL_F32 && dtype != MOL_BF16) return MOL_E_DTYPE;
  if (R < 1 || slices < 1 || N < 1 || E < 1 || R % slices || N % slices || ld_out < N ||
      V % E)
    return MOL_E_ARG;
  if (numel > 0 && (!B || !scale || !out)) return MOL_E_ARG;
  const int esz = dtype == MOL_BF16 ? 2 : 4;
  const int64_t rbytes = (int64_t)(R / slices) * esz;
  if (rbytes % 16) return MOL_E_ALIGN;
  if (rbytes > MOL_MAX_RANK_BYTES || R > 1024) return MOL_E_LIMIT;
  if ((int64_t)N * rbytes >= (int64_t(1) << 31)) return MOL_E_LIMIT;  // one expert's B
  if (numel > 0 && (!aligned16(B) || (reinterpret_cast<uintptr_t>(out) % esz)))
    return MOL_E_ALIGN;
  return MOL_OK;
}

mol::DeltaArgs make_delta_args(const void* xin, int64_t ld_x, int32_t row_div, const void* A,
                               int32_t R, int32_t K, int32_t slices, const void* B,
                               int32_t N, const float* scale, int32_t E,
                               const int32_t* sorted_ids, const int32_t* expert_ids,
                               const int32_t* npp, int32_t numel, int32_t V, int32_t BM,
                               float* s, void* out, int64_t ld_out, int64_t max_blocks) {
  mol::DeltaArgs a{};
  a.xin = xin;
  a.ld_x = ld_x;
  a.row_div = row_div;
  a.A = A;
  a.R = R;
  a.K = K;
  a.slices = slices;
  a.B = B;
  a.N = N;
  a.scale = scale;
  a.E = E;
  a.sorted = sorted_ids;
  a.expert_ids = expert_ids;
  a.npp = npp;
  a.numel = numel;
  a.V = V;
  a.BM = BM;
  a.s = s;
  a.out = out;
  a.ld_out = ld_out;
  a.max_blocks = (int32_t)max_blocks;
  return a;
}

}  // namespace

extern "C" {

MOL_API const char* mol_status_string(mol_status status) {
  switch (status) {
    case MOL_OK: return "ok";
    case MOL_E_ARG: return "invalid argument";
    case MOL_E_LIMIT: return "size beyond a supported limit";
    case MOL_E_DTYPE: return "unsupported dtype";
    case MOL_E_ALIGN: return "pointer, row or stride not 16-byte aligned";
    case MOL_E_WORKSPACE: return "workspace missing or too small";
    case MOL_E_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

MOL_API int32_t mol_abi_version(void) { return 7; }

MOL_API mol_status mol_virtual_topk(const int32_t* topk_ids, const int32_t* lora_ids,
                                    int32_t M, int32_t topk, int32_t num_experts,
                                    int32_t num_slots, int32_t* virtual_ids, void* stream) {
  if (M < 0 || topk < 1 || num_experts < 1 || num_slots < 1) return MOL_E_ARG;
  if ((int64_t)M * topk > kI32Max || (int64_t)num_experts * num_slots > kI32Max)
    return MOL_E_LIMIT;
  if (M == 0) return MOL_OK;
  if (!topk_ids || !lora_ids || !virtual_ids) return MOL_E_ARG;
  return hip_status(mol::launch_virtual_topk(topk_ids, lora_ids, M, topk, num_experts,
                                             num_slots, virtual_ids, (hipStream_t)stream));
}

MOL_API int64_t mol_align_max_blocks(int64_t numel, int32_t num_virtual, int32_t block_m) {
  return align_check(numel, num_virtual, block_m);
}

MOL_API int64_t mol_align_workspace_bytes(int64_t numel, int32_t num_virtual,
                                          int32_t block_m) {
  const int64_t mb = align_check(numel, num_virtual, block_m);
  if (mb < 0) return mb;
  if (numel <= mol::kAlignSmallMax) return 0;
  const int64_t nb = (int64_t)num_virtual + 1;
  const int64_t ntiles = cdiv64(numel, mol::align_tile(numel));
  return round256((ntiles * nb + nb) * (int64_t)sizeof(int32_t));
}

MOL_API int64_t mol_plan_bytes(int64_t numel, int32_t num_virtual, int32_t block_m) {
  const int64_t mb = align_check(numel, num_virtual, block_m);
  if (mb < 0) return mb;
  return round256(mol::plan_words(numel, mb) * (int64_t)sizeof(int32_t));
}

MOL_API mol_status mol_align_block_size(const int32_t* ids, const int32_t* lora_ids,
                                        int32_t M, int32_t topk, int32_t num_experts,
                                        int32_t num_slots, int32_t block_m,
                                        int32_t* sorted_ids, int32_t* expert_ids,
                                        int32_t* num_post_padded, int32_t* plan,
                                        size_t plan_bytes, void* workspace,
                                        size_t workspace_bytes, void* stream) {
  if (M < 0 || topk < 1 || num_experts < 1 || num_slots < 1 || block_m < 1)
    return MOL_E_ARG;
  const int64_t V64 = (int64_t)num_experts * num_slots;
  if (V64 + 1 > MOL_MAX_BUCKETS || block_m > MOL_MAX_BLOCK_M) return MOL_E_LIMIT;
  const int64_t numel = (int64_t)M * topk;
  const int64_t mb = align_check(numel, (int32_t)V64, block_m);
  if (mb < 0) return (mol_status)(-mb);
  if (!num_post_padded) return MOL_E_ARG;
  if (numel > 0 && (!ids || !sorted_ids || !expert_ids)) return MOL_E_ARG;
  const int64_t need = mol_align_workspace_bytes(numel, (int32_t)V64, block_m);
  if (need > 0 && (!workspace || workspace_bytes < (size_t)need)) return MOL_E_WORKSPACE;
  if (plan) {
    const int64_t pneed = mol_plan_bytes(numel, (int32_t)V64, block_m);
    if (pneed < 0) return (mol_status)(-pneed);
    if (plan_bytes < (size_t)pneed) return MOL_E_WORKSPACE;
    if (!aligned16(plan)) return MOL_E_ALIGN;
  }

  mol::AlignArgs a{};
  a.plan = mol::mfma_batch(numel, V64) ? plan : nullptr;  // otherwise nothing to plan
  a.dmax = (int32_t)mol::plan_max_runs(numel, mb);
  a.max_blocks = (int32_t)mb;
  a.ids = ids;
  a.lora = lora_ids;
  a.topk = topk;
  a.E = num_experts;
  a.S = num_slots;
  a.numel = (int32_t)numel;
  a.V = (int32_t)V64;
  a.BM = block_m;
  a.bm_shift = (block_m & (block_m - 1)) == 0 ? __builtin_ctz((unsigned)block_m) : -1;
  a.f_topk = mol::make_fastdiv((uint32_t)topk);
  a.f_bm = mol::make_fastdiv((uint32_t)block_m);
  a.sorted = sorted_ids;
  a.expert_ids = expert_ids;
  a.npp = num_post_padded;
  const hipStream_t st = (hipStream_t)stream;
  const int nb = a.V + 1;
  if (numel <= mol::kAlignSmallMax) {
    // counter rows + bucket starts + scan scratch + per pair a bucket id and a rank
    // (uint16 each)
    const int64_t fixed = ((int64_t)nb + 64) * (int64_t)sizeof(int) +
                          ((numel + 1) & ~1LL) * 2 * 2;
    const int64_t row = (int64_t)mol::align_small_stride(nb) * (int64_t)sizeof(int);
    int64_t waves = (device_lds_bytes() - fixed) / row;
    // walkers: one chunk of 64 pairs each for the smallest batches, two chunks each above
    // (more walkers shorten the walk but add counter rows to every bucket's sums)
    const int64_t useful = numel <= 256 ? cdiv64(numel, 64) : cdiv64(numel, 128);
    if (waves > useful) waves = useful;
    if (waves > 16) waves = 16;
    if (waves < 1) waves = 1;
    const size_t lds = (size_t)(waves * row + fixed);
    if ((int64_t)lds > device_lds_bytes()) return MOL_E_LIMIT;
    // workgroups that split the output writes (each one rebuilds the routing in LDS)
    const int groups = (int)std::max<int64_t>(1, std::min<int64_t>(16, cdiv64(numel, 16)));
    // each walker's contiguous range of pairs: a multiple of 64
    a.per = (int32_t)(cdiv64(cdiv64(numel, waves), 64) * 64);
    a.f_per = mol::make_fastdiv((uint32_t)std::max<int64_t>(1, a.per));
    a.f_groups = mol::make_fastdiv((uint32_t)groups);
    return hip_status(mol::launch_align_small(a, (int)waves, groups, lds, st));
  }
  a.tile = (int32_t)mol::align_tile(numel);
  a.ntiles = (int32_t)cdiv64(numel, a.tile);
  int32_t* ws = static_cast<int32_t*>(workspace);
  a.counts = ws;
  a.totals = ws + (int64_t)a.ntiles * nb;
  // offsets, cursors and the tile's keys in LDS
  const size_t lds = (size_t)(2 * nb + 64) * sizeof(int) + (size_t)a.tile * 2;
  if ((int64_t)lds > device_lds_bytes()) return MOL_E_LIMIT;
  return hip_status(mol::launch_align_large(a, lds, st));
}

}  // extern "C"

namespace {

// Whether the bf16 MFMA kernels take every block (and no VALU kernel is launched), else the
// VALU kernels take every block. The MFMA kernels serve batches large enough to hold dense
// blocks in numbers (mol::mfma_batch): their grid spans every possible block, so a batch of
// small blocks would pay for empty workgroups, and a block of one or two pairs is a mostly
// empty tile.
bool shrink_uses_mfma(bool bf16, int32_t numel, int32_t num_virtual) {
  return bf16 && mol::mfma_batch(numel, num_virtual);
}

// The MFMA expand also needs whole 32-wide rank steps, s rows of at most 256 floats (they
// are staged in LDS), 64-column groups inside one slice, and 16-byte aligned groups of
// eight out elements.
bool expand_uses_mfma(bool bf16, int32_t numel, int32_t num_virtual, int32_t R, int32_t slices,
                      int32_t N, const void* out, int64_t ld_out) {
  const int32_t r = R / slices;
  const bool shape_ok = r % 32 == 0 && r <= 128 && R <= 256 && (N / slices) % 64 == 0 &&
                        ld_out % 8 == 0 && reinterpret_cast<uintptr_t>(out) % 16 == 0;
  return shape_ok && shrink_uses_mfma(bf16, numel, num_virtual);
}

// The shrink of a stage: the MFMA kernel over every block when the batch takes it (items
// ordered by XCD), else the VALU kernel over every block.
hipError_t shrink_all(mol::DeltaArgs a, bool bf16, int rpi, int64_t grid, bool mfma,
                      hipStream_t st) {
  mol::with_divisors(a);
  if (!mfma) return mol::launch_shrink(a, bf16, rpi, (int)grid, st);
  return mol::launch_shrink_mfma(
      a, (int)(a.max_blocks * cdiv64(a.R, mol::shrink_mfma_row_tile(a.R))), st);
}

// The expand of a stage: the MFMA kernel when the batch and the shape allow it, over the
// align's dense runs when a plan is given and over every block otherwise; else the VALU
// kernel over every block.
hipError_t expand_all(mol::DeltaArgs a, bool bf16, int64_t grid, bool mfma,
                      const int32_t* plan, hipStream_t st) {
  mol::with_divisors(a);
  if (!mfma) return mol::launch_expand(a, bf16, (int)grid, st);
  if (plan) {
    const int64_t runs = mol::plan_max_runs(a.numel, a.max_blocks);
    return mol::launch_expand_mfma_runs(a, plan, (int)(runs * a.nchunk), st);
  }
  return mol::launch_expand_mfma(a, (int)grid, st);
}

// Scratch of mol_lora_delta_noalloc: the fp32 rank-space rows s of one stage live here
// instead of in a caller's workspace. Each GPU holds its own copy of this array, at its own
// address, until the process ends. On the host its name stands for the symbol only: the
// device address is taken with hipGetSymbolAddress once per device and kept below.
__device__ __align__(256) float scratch[MOL_DELTA_SCRATCH_FLOATS];

std::atomic<float*> g_scratch[64];  // device address of `scratch`, per device
std::mutex g_scratch_mu;

// The current device's address of `scratch` (looked up on the first call on a device).
mol_status delta_scratch(float** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return MOL_E_HIP;
  float* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      void* q = nullptr;
      if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) return MOL_E_HIP;
      p = static_cast<float*>(q);
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return MOL_OK;
}

// Host checks of a stage delta call (every argument but the workspace).
mol_status delta_check(int32_t dtype, const void* xin, int64_t ld_x, int32_t row_div,
                       const void* A, int32_t R, int32_t K, int32_t slices, const void* B,
                       int32_t N, const float* slot_scale, int32_t num_experts,
                       const int32_t* sorted_ids, const int32_t* expert_ids,
                       const int32_t* num_post_padded, int32_t numel, int32_t num_virtual,
                       int32_t block_m, const void* out, int64_t ld_out) {
  const StageCheck rc =
      routing_check(sorted_ids, expert_ids, num_post_padded, numel, num_virtual, block_m);
  if (rc.st != MOL_OK) return rc.st;
  alignas(16) float s_probe[4] = {};  // s is checked by the caller
  mol_status c = shrink_check(dtype, xin, ld_x, row_div, A, R, K, numel, s_probe);
  if (c != MOL_OK) return c;
  c = expand_check(dtype, R, slices, B, N, slot_scale, num_experts, num_virtual, numel, out,
                   ld_out);
  if (c != MOL_OK) return c;
  const bool bf16 = dtype == MOL_BF16;
  const int esz = bf16 ? 2 : 4;
  const int64_t mb = rc.max_blocks;
  if (mb * cdiv64(R, mol::shrink_rows_per_item(K, esz)) > kI32Max ||
      mb * cdiv64(N, mol::expand_cols_per_item(R, slices, esz)) > kI32Max)
    return MOL_E_LIMIT;
  if (shrink_uses_mfma(bf16, numel, num_virtual) && mb * cdiv64(R, 64) > kI32Max)
    return MOL_E_LIMIT;
  return MOL_OK;
}

// Enqueue a checked stage delta with s at `s` (16-byte aligned, numel * R floats).
mol_status delta_enqueue(int32_t dtype, const void* xin, int64_t ld_x, int32_t row_div,
                         const void* A, int32_t R, int32_t K, int32_t slices, const void* B,
                         int32_t N, const float* slot_scale, const int32_t* slot_ranks,
                         int32_t num_experts, const int32_t* sorted_ids,
                         const int32_t* expert_ids, const int32_t* num_post_padded,
                         int32_t numel, int32_t num_virtual, int32_t block_m, void* out,
                         int64_t ld_out, float* s, const int32_t* plan, hipStream_t st) {
  const bool bf16 = dtype == MOL_BF16;
  const int esz = bf16 ? 2 : 4;
  const int64_t mb = max_blocks_of(numel, num_virtual, block_m);
  const int rpi = mol::shrink_rows_per_item(K, esz);
  mol::DeltaArgs a = make_delta_args(xin, ld_x, row_div, A, R, K, slices, B, N, slot_scale,
                                     num_experts, sorted_ids, expert_ids, num_post_padded,
                                     numel, num_virtual, block_m, s, out, ld_out, mb);
  a.ranks = slot_ranks;
  a.rgroups = (int32_t)cdiv64(R, rpi);
  a.nchunk = (int32_t)cdiv64(N, mol::expand_cols_per_item(R, slices, esz));
  const int64_t grid_s = mb * (int64_t)a.rgroups;
  const int64_t grid_e = mb * (int64_t)a.nchunk;
  const bool mm_s = shrink_uses_mfma(bf16, numel, num_virtual);
  const bool mm_e = expand_uses_mfma(bf16, numel, num_virtual, R, slices, N, out, ld_out);
  if (shrink_all(a, bf16, rpi, grid_s, mm_s, st) != hipSuccess) return MOL_E_HIP;
  return hip_status(expand_all(a, bf16, grid_e, mm_e, plan, st));
}

}  // namespace

extern "C" {

MOL_API mol_status mol_lora_shrink(int32_t dtype, const void* xin, int64_t ld_x,
                                   int32_t row_div, const void* A, int32_t R, int32_t K,
                                   int32_t slices, const int32_t* slot_ranks,
                                   int32_t num_experts, const int32_t* sorted_ids,
                                   const int32_t* expert_ids, const int32_t* num_post_padded,
                                   int32_t numel, int32_t num_virtual, int32_t block_m,
                                   float* s, void* stream) {
  const StageCheck rc =
      routing_check(sorted_ids, expert_ids, num_post_padded, numel, num_virtual, block_m);
  if (rc.st != MOL_OK) return rc.st;
  const mol_status sc = shrink_check(dtype, xin, ld_x, row_div, A, R, K, numel, s);
  if (sc != MOL_OK) return sc;
  if (slices < 1 || R % slices || num_experts < 1 || num_virtual % num_experts)
    return MOL_E_ARG;
  if (numel == 0) return MOL_OK;
  const bool bf16 = dtype == MOL_BF16;
  const int rpi = mol::shrink_rows_per_item(K, bf16 ? 2 : 4);
  const int64_t rgroups = cdiv64(R, rpi);
  const int64_t grid = rc.max_blocks * rgroups;
  if (grid > kI32Max) return MOL_E_LIMIT;
  mol::DeltaArgs a = make_delta_args(xin, ld_x, row_div, A, R, K, slices, nullptr, 1, nullptr,
                                     num_experts, sorted_ids, expert_ids, num_post_padded,
                                     numel, num_virtual, block_m, s, nullptr, 0, rc.max_blocks);
  a.ranks = slot_ranks;
  a.rgroups = (int32_t)rgroups;
  const bool mm = shrink_uses_mfma(bf16, numel, num_virtual);
  if (mm && rc.max_blocks * cdiv64(R, 64) > kI32Max) return MOL_E_LIMIT;
  return hip_status(shrink_all(a, bf16, rpi, grid, mm, (hipStream_t)stream));
}

MOL_API mol_status mol_lora_expand(int32_t dtype, const float* s, int32_t R, int32_t slices,
                                   const void* B, int32_t N, const float* slot_scale,
                                   const int32_t* slot_ranks, int32_t num_experts,
                                   const int32_t* sorted_ids,
                                   const int32_t* expert_ids,
                                   const int32_t* num_post_padded, const int32_t* plan,
                                   int32_t numel, int32_t num_virtual, int32_t block_m,
                                   void* out, int64_t ld_out, void* stream) {
  const StageCheck rc =
      routing_check(sorted_ids, expert_ids, num_post_padded, numel, num_virtual, block_m);
  if (rc.st != MOL_OK) return rc.st;
  const mol_status ec = expand_check(dtype, R, slices, B, N, slot_scale, num_experts,
                                     num_virtual, numel, out, ld_out);
  if (ec != MOL_OK) return ec;
  if (numel > 0 && !s) return MOL_E_ARG;
  if (numel > 0 && !aligned16(s)) return MOL_E_ALIGN;  // s rows are read as 16-byte vectors
  if (numel == 0) return MOL_OK;
  const bool bf16 = dtype == MOL_BF16;
  mol::DeltaArgs a = make_delta_args(nullptr, 0, 1, nullptr, R, 1, slices, B, N, slot_scale,
                                     num_experts, sorted_ids, expert_ids, num_post_padded,
                                     numel, num_virtual, block_m, const_cast<float*>(s), out,
                                     ld_out, rc.max_blocks);
  a.ranks = slot_ranks;
  a.nchunk = (int32_t)cdiv64(N, mol::expand_cols_per_item(R, slices, bf16 ? 2 : 4));
  const int64_t grid = rc.max_blocks * a.nchunk;
  if (grid > kI32Max) return MOL_E_LIMIT;
  const bool mm = expand_uses_mfma(bf16, numel, num_virtual, R, slices, N, out, ld_out);
  return hip_status(expand_all(a, bf16, grid, mm, plan, (hipStream_t)stream));
}

MOL_API int64_t mol_delta_workspace_bytes(int32_t numel, int32_t R, int32_t num_virtual,
                                          int32_t block_m) {
  const int64_t mb = align_check(numel, num_virtual, block_m);
  if (mb < 0) return mb;
  if (R < 1) return -MOL_E_ARG;
  return round256((int64_t)numel * R * (int64_t)sizeof(float));
}

MOL_API mol_status mol_lora_delta(int32_t dtype, const void* xin, int64_t ld_x,
                                  int32_t row_div, const void* A, int32_t R, int32_t K,
                                  int32_t slices, const void* B, int32_t N,
                                  const float* slot_scale, const int32_t* slot_ranks,
                                  int32_t num_experts,
                                  const int32_t* sorted_ids, const int32_t* expert_ids,
                                  const int32_t* num_post_padded, const int32_t* plan,
                                  int32_t numel, int32_t num_virtual, int32_t block_m,
                                  void* out, int64_t ld_out, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  const mol_status c =
      delta_check(dtype, xin, ld_x, row_div, A, R, K, slices, B, N, slot_scale, num_experts,
                  sorted_ids, expert_ids, num_post_padded, numel, num_virtual, block_m, out,
                  ld_out);
  if (c != MOL_OK || numel == 0) return c;
  const int64_t need = mol_delta_workspace_bytes(numel, R, num_virtual, block_m);
  if (need < 0) return (mol_status)(-need);
  if (!workspace || workspace_bytes < (size_t)need) return MOL_E_WORKSPACE;
  if (!aligned16(workspace)) return MOL_E_ALIGN;
  return delta_enqueue(dtype, xin, ld_x, row_div, A, R, K, slices, B, N, slot_scale,
                       slot_ranks, num_experts, sorted_ids, expert_ids, num_post_padded, numel,
                       num_virtual, block_m, out, ld_out, static_cast<float*>(workspace), plan,
                       (hipStream_t)stream);
}

MOL_API mol_status mol_lora_delta_noalloc(int32_t dtype, const void* xin, int64_t ld_x,
                                          int32_t row_div, const void* A, int32_t R, int32_t K,
                                          int32_t slices, const void* B, int32_t N,
                                          const float* slot_scale, const int32_t* slot_ranks,
                                          int32_t num_experts, const int32_t* sorted_ids,
                                          const int32_t* expert_ids,
                                          const int32_t* num_post_padded, const int32_t* plan,
                                          int32_t numel, int32_t num_virtual, int32_t block_m,
                                          void* out, int64_t ld_out, void* stream) {
  const mol_status c =
      delta_check(dtype, xin, ld_x, row_div, A, R, K, slices, B, N, slot_scale, num_experts,
                  sorted_ids, expert_ids, num_post_padded, numel, num_virtual, block_m, out,
                  ld_out);
  if (c != MOL_OK || numel == 0) return c;
  if ((int64_t)numel * R > MOL_DELTA_SCRATCH_FLOATS) return MOL_E_LIMIT;
  float* s = nullptr;
  const mol_status sc = delta_scratch(&s);
  if (sc != MOL_OK) return sc;
  return delta_enqueue(dtype, xin, ld_x, row_div, A, R, K, slices, B, N, slot_scale,
                       slot_ranks, num_experts, sorted_ids, expert_ids, num_post_padded, numel,
                       num_virtual, block_m, out, ld_out, s, plan, (hipStream_t)stream);
}

// ---- base grouped GEMM, alone or with the LoRA delta in its epilogue -----------------

MOL_API mol_status mol_moe_gemm(int32_t dtype, const void* xin, int64_t ld_x, int32_t row_div,
                                const void* W, int32_t K, int32_t N, int32_t num_experts,
                                const int32_t* sorted_ids, const int32_t* expert_ids,
                                const int32_t* num_post_padded, int32_t numel, int32_t block_m,
                                void* out, int64_t ld_out, const float* s, int32_t R,
                                int32_t slices, const void* B, const float* slot_scale,
                                const int32_t* slot_ranks, const int32_t* lora_ids,
                                int32_t topk, int32_t num_slots, void* stream) {
  const StageCheck rc =
      routing_check(sorted_ids, expert_ids, num_post_padded, numel, num_experts, block_m);
  if (rc.st != MOL_OK) return rc.st;
  if (dtype != MOL_F32 && dtype != MOL_BF16) return MOL_E_DTYPE;
  if (K < 1 || N < 1 || row_div < 1 || ld_x < K || ld_out < N) return MOL_E_ARG;
  if (numel > 0 && (!xin || !W || !out)) return MOL_E_ARG;
  const bool bf16 = dtype == MOL_BF16;
  const int esz = bf16 ? 2 : 4;
  if (((int64_t)K * esz) % 16 || (ld_x * esz) % 16) return MOL_E_ALIGN;
  if (numel > 0 && (!aligned16(xin) || !aligned16(W) || reinterpret_cast<uintptr_t>(out) % esz))
    return MOL_E_ALIGN;
  if ((int64_t)N * K * esz >= (int64_t(1) << 31)) return MOL_E_LIMIT;  // one expert's W
  if (s) {  // the fused delta
    if (R < 1 || slices < 1 || R % slices || N % slices || topk < 1 || num_slots < 1 ||
        numel % topk)
      return MOL_E_ARG;
    if (numel > 0 && (!B || !slot_scale || !lora_ids)) return MOL_E_ARG;
    const int64_t rbytes = (int64_t)(R / slices) * esz;
    if (rbytes % 16) return MOL_E_ALIGN;
    if (rbytes > MOL_MAX_RANK_BYTES) return MOL_E_LIMIT;
    if ((int64_t)num_experts * num_slots + 1 > MOL_MAX_BUCKETS) return MOL_E_LIMIT;
    if ((int64_t)N * rbytes >= (int64_t(1) << 31)) return MOL_E_LIMIT;  // one expert's B
    if (numel > 0 && (!aligned16(s) || !aligned16(B))) return MOL_E_ALIGN;
  }
  if (numel == 0) return MOL_OK;
  mol::GemmArgs g{};
  g.route = make_delta_args(nullptr, 0, 1, nullptr, 1, 1, 1, nullptr, 1, nullptr, num_experts,
                            sorted_ids, expert_ids, num_post_padded, numel, num_experts,
                            block_m, nullptr, nullptr, 0, rc.max_blocks);
  g.xin = xin;
  g.ld_x = ld_x;
  g.row_div = row_div;
  g.W = W;
  g.K = K;
  g.N = N;
  g.out = out;
  g.ld_out = ld_out;
  g.s = s;
  g.R = s ? R : 0;
  g.slices = s ? slices : 1;
  g.B = B;
  g.scale = slot_scale;
  g.ranks = slot_ranks;
  g.lora = lora_ids;
  g.topk = s ? topk : 1;
  g.E = num_experts;
  g.S = s ? num_slots : 1;
  const int rpi = mol::shrink_rows_per_item(K, esz);
  g.rgroups = (int32_t)cdiv64(N, rpi);
  const int64_t grid = rc.max_blocks * (int64_t)g.rgroups;
  if (grid > kI32Max) return MOL_E_LIMIT;
  // the kernel's fixed divisors: items per block, input rows, columns of a slice
  g.route.rgroups = g.rgroups;
  g.route.row_div = row_div;
  g.route.N = N;
  g.route.slices = g.slices;
  mol::with_divisors(g.route);
  return hip_status(mol::launch_moe_gemm(g, bf16, rpi, (int)grid, (hipStream_t)stream));
}

// ---- combine -----------------------------------------------------------------------

MOL_API mol_status mol_moe_combine(int32_t dtype, const void* rows, int64_t ld_rows,
                                   const int32_t* topk_ids, const float* topk_weights,
                                   int32_t M, int32_t topk, int32_t num_experts, int32_t N,
                                   void* y, int64_t ld_y, void* stream) {
  if (dtype != MOL_F32 && dtype != MOL_BF16) return MOL_E_DTYPE;
  if (M < 0 || topk < 1 || num_experts < 1 || N < 1 || ld_rows < N || ld_y < N)
    return MOL_E_ARG;
  if (M > 0 && (!rows || !topk_ids || !topk_weights || !y)) return MOL_E_ARG;
  const bool bf16 = dtype == MOL_BF16;
  const int ve = bf16 ? 8 : 4;  // elements of one 16-byte vector
  if (N % ve || ld_rows % ve || ld_y % ve) return MOL_E_ALIGN;
  if (M > 0 && (!aligned16(rows) || !aligned16(y))) return MOL_E_ALIGN;
  if ((int64_t)M * topk > kI32Max) return MOL_E_LIMIT;
  const int64_t grid = (int64_t)M * cdiv64(N, 64 * ve);
  if (grid > kI32Max) return MOL_E_LIMIT;
  if (M == 0) return MOL_OK;
  mol::CombineArgs a{};
  a.rows = rows;
  a.ld_rows = ld_rows;
  a.topk_ids = topk_ids;
  a.weights = topk_weights;
  a.M = M;
  a.topk = topk;
  a.E = num_experts;
  a.N = N;
  a.y = y;
  a.ld_y = ld_y;
  return hip_status(mol::launch_combine(a, bf16, (hipStream_t)stream));
}

MOL_API mol_status mol_lora_expand_combine(int32_t dtype, const float* s, int32_t R,
                                           const void* B, int32_t N, const float* slot_scale,
                                           const int32_t* slot_ranks, const int32_t* topk_ids,
                                           const int32_t* lora_ids,
                                           const float* topk_weights, int32_t M, int32_t topk,
                                           int32_t num_experts, int32_t num_slots,
                                           const void* base, int64_t ld_base, void* y,
                                           int64_t ld_y, void* stream) {
  if (dtype != MOL_F32 && dtype != MOL_BF16) return MOL_E_DTYPE;
  if (M < 0 || topk < 1 || num_experts < 1 || num_slots < 1 || N < 1 || R < 1 ||
      ld_base < N || ld_y < N)
    return MOL_E_ARG;
  if (M > 0 && (!s || !B || !slot_scale || !topk_ids || !lora_ids || !topk_weights || !base ||
                !y))
    return MOL_E_ARG;
  const bool bf16 = dtype == MOL_BF16;
  const int esz = bf16 ? 2 : 4;
  if (((int64_t)R * esz) % 16) return MOL_E_ALIGN;
  if (!mol::fused_rank_supported(R, bf16)) return MOL_E_LIMIT;
  if ((int64_t)num_experts * num_slots + 1 > MOL_MAX_BUCKETS) return MOL_E_LIMIT;
  if ((int64_t)N * R * esz >= (int64_t(1) << 31)) return MOL_E_LIMIT;  // one expert's B
  if ((int64_t)M * topk > kI32Max) return MOL_E_LIMIT;
  if (M > 0 && (!aligned16(s) || !aligned16(B) ||
                reinterpret_cast<uintptr_t>(base) % esz || reinterpret_cast<uintptr_t>(y) % esz))
    return MOL_E_ALIGN;
  const int64_t grid = (int64_t)M * cdiv64(N, 64);
  if (grid > kI32Max) return MOL_E_LIMIT;
  if (M == 0) return MOL_OK;
  mol::CombineArgs a{};
  a.topk_ids = topk_ids;
  a.weights = topk_weights;
  a.lora = lora_ids;
  a.M = M;
  a.topk = topk;
  a.E = num_experts;
  a.S = num_slots;
  a.N = N;
  a.R = R;
  a.s = s;
  a.B = B;
  a.scale = slot_scale;
  a.ranks = slot_ranks;
  a.base = base;
  a.ld_base = ld_base;
  a.y = y;
  a.ld_y = ld_y;
  return hip_status(mol::launch_expand_combine(a, bf16, (hipStream_t)stream));
}

}  // extern "C"
