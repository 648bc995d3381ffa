// bf16 MFMA shrink and expand for the aligned blocks that hold many pairs (MindLab sglang
// PR 24: the MoL shrink hidden -> rank and expand rank -> N stages; same definitions as
// the VALU kernels):
//
//   shrink: s[p, i]   = sum_k A[v, i, k] * xin[p / row_div, k]
//   expand: out[p, n] = round(out[p, n] + scale[v / E] * sum_j B[v, n, j] * s[p, g(n)*r + j])
//
// At prefill a hot virtual expert's block carries up to BLOCK_M real pairs, so a block is a
// real dense tile and the products run on v_mfma_f32_16x16x32_bf16 (fp32 accumulation).
// A batch large enough for them (from 4096 pairs and 8 per bucket on average) gives every
// block to these kernels and launches no VALU kernel: a block of one or two pairs still
// costs less as a mostly empty tile than a VALU launch over every possible block.
//
// MFMA 16x16x32 operand layout (lane l of a wave): A holds row l % 16, k = 8*(l/16)..+8;
// B holds column l % 16, k = 8*(l/16)..+8; the 16x16 fp32 result holds column l % 16,
// rows 4*(l/16)..+4.
//
//  * shrink item = (block, 64 or 128 rows of A_v: 128 when R > 64, so that a block with
//    R <= 128 reads its gathered x rows once); wave w owns the block's pairs 16w..16w+15
//    (MFMA A operand = their x rows, straight from global) and all the item's rows of A_v
//    (MFMA B operand), which are staged per k chunk (128 wide for 64 rows, 64 for 128) in
//    LDS by direct-to-LDS loads, double buffered, with an XOR swizzle of the 16-byte slots
//    so the fragment reads are free of bank conflicts. Pairs of a block beyond 64 are done
//    64 at a time.
//  * expand item = (block, 256 output columns); the product is taken transposed, D = B_v s^T
//    (MFMA A operand = rows of B_v, held in registers for the whole block; B operand = s
//    rows). Only the slices of s that the item's columns use are staged, once per item, in
//    LDS (swizzled like the shrink's tile), and split into a bf16 high part and a bf16
//    remainder, two MFMAs per step, which keeps s to about 16 significant bits instead of
//    bf16's 8. Each 16-pair tile of results goes through an LDS tile so that out is read and
//    written in whole 512-byte row segments (16-byte vectors); the old out values of the
//    next 16 pairs are loaded while the current 16 are multiplied.
#include "delta_common.h"

namespace mol {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

constexpr int kRowsPerPass = 64;  // pairs of a block per pass (4 waves x 16)
constexpr int kKChunk = 128;      // shrink: k elements staged per chunk at 64 rows
constexpr int kXcds = 8;          // accelerator dies (XCDs), each with its own L2

// Workgroups are handed to the XCDs in turn (workgroup i to XCD i % 8). The item of
// workgroup i is remapped so that each XCD works through one contiguous eighth of the live
// items in order: the workgroups resident on an XCD at one time then take neighbouring
// blocks, mostly of the same virtual expert, and share its weight tiles (and, in the
// expand, a block's s rows across its column chunks) through that XCD's L2. The eighths
// are of the live items (a prefix of the launched ones, counted on the device), so every
// XCD gets its share of the work. The grid covers every possible item, rounded up to a
// multiple of 8; a workgroup past the live items gets n_live, which is empty.
__device__ __forceinline__ int xcd_item(int n_live) {
  const int per = (n_live + kXcds - 1) / kXcds;
  const int wg = (int)blockIdx.x, local = wg / kXcds;
  return local < per ? (wg % kXcds) * per + local : n_live;
}
inline int xcd_grid(int n_items) { return (n_items + kXcds - 1) / kXcds * kXcds; }

__device__ __forceinline__ floatx4_t mfma16(const uint4& a, const uint4& b, floatx4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<const bf16x8_t*>(&a),
                                                 *reinterpret_cast<const bf16x8_t*>(&b), c, 0,
                                                 0, 0);
}

// The pair ids of rows j0..j0+63 of block blk into pid (numel past the block); returns the
// number of real ones (a prefix). Every thread of the workgroup takes part.
__device__ __forceinline__ int stage_rows(const DeltaArgs& a, int blk, int j0, int* pid,
                                          int* nrows_lds) {
  const int tid = threadIdx.x;
  __syncthreads();  // the previous pass is done with pid
  if (tid < kRowsPerPass) {
    const int j = j0 + tid;
    const int v = a.sorted[(int64_t)blk * a.BM + (j < a.BM ? j : 0)];
    const int pv = j < a.BM ? v : a.numel;
    pid[tid] = pv;
    const uint64_t m = __builtin_amdgcn_ballot_w64(real_pair(pv, a.numel));
    if (tid == 0) *nrows_lds = (int)__popcll(m);
  }
  __syncthreads();
  return *nrows_lds;
}

// ------------------------------------------------------------------------------ shrink

// A shrink item covers 64 * NRT rows of A_v (NRT = 2 when R > 64, so an item with R <= 128
// reads the block's gathered x rows once), staged per k chunk of kKChunk / NRT: always
// 16 KiB of LDS per buffer, i.e. 1024 slots of 16 bytes.
template <int NRT>
struct ShrinkGeom {
  static constexpr int kRows = 64 * NRT;
  static constexpr int kChunk = kKChunk / NRT;  // k elements per staged chunk
  static constexpr int kSlots = kChunk / 8;     // 16-byte slots of one staged row
  static constexpr int kSteps = kChunk / 32;    // MFMA k steps per chunk
  static_assert(kRows * kSlots == 1024, "16 KiB per buffer");
};

// A_v rows r0..r0+kRows-1, k chunk kc0.. -> LDS tile [kRows][kSlots], slot of 16-byte vector
// kv of row rr at (kv ^ (rr & (kSlots - 1))). Lane i of wave instruction t writes LDS slot
// (4t + w) * 64 + i, so it fetches the global vector that belongs there. Rows past R and
// vectors past K read a valid weight instead (finite; they meet zero x or are never stored).
template <int NRT>
__device__ __forceinline__ void stage_w(const DeltaArgs& a, const char* av, int r0, int kc0,
                                        uint4* tile) {
  using G = ShrinkGeom<NRT>;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nvec = a.K / 8;
#pragma unroll
  for (int t = 0; t < G::kRows * G::kSlots / 256; ++t) {
    const int P = (4 * t + w) * 64 + lane;
    const int rr = P / G::kSlots, slot = P % G::kSlots;
    const int kv = (kc0 / 8) + (slot ^ (rr & (G::kSlots - 1)));
    const bool ok = r0 + rr < a.R && kv < nvec;
    const int64_t off = ok ? ((int64_t)(r0 + rr) * a.K + (int64_t)kv * 8) * 2 : 0;
    lds_dma16(av + off, tile + (4 * t + w) * 64);
  }
}

// x fragments of this wave's 16 pairs for the chunk at kc0: step st holds k = kc0 + 32 st +
// 8 (l/16) .. +8 of pair row l % 16 (zero past K or for rows that are not real pairs).
template <int NRT>
__device__ __forceinline__ void load_x(const DeltaArgs& a, int p, bool real, int kc0,
                                       uint4* xf) {
  const int lane = threadIdx.x & 63;
  const int64_t rowoff = real ? (int64_t)fdiv(p, a.f_rd) * a.ld_x : 0;
  const char* xb = (const char*)a.xin;
#pragma unroll
  for (int st = 0; st < ShrinkGeom<NRT>::kSteps; ++st) {
    const int k = kc0 + 32 * st + 8 * (lane >> 4);
    const bool ok = real && k < a.K;
    xf[st] = ld16_if(xb, (rowoff + k) * 2, ok);
  }
}

// One pass: wave w's 16 entries pid[16w..16w+15] (numel: not a real pair) times rows
// r0..r0+kRows-1 of A_v, which the workgroup's four waves stream through LDS one k chunk at
// a time (double buffered: the next chunk and the next x fragments are in flight while the
// current one is multiplied). A wave with no real pair skips the loads and products but
// takes part in the staging. Results go to s (rows past the slot's rank store 0).
template <int NRT>
__device__ __forceinline__ void shrink_mfma_pass(const DeltaArgs& a, const char* av, int r0,
                                                 int rl, const int* pid, uint4 (*wt)[1024]) {
  using G = ShrinkGeom<NRT>;
  constexpr int NT = 4 * NRT;  // 16-row tiles of A_v per wave
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = a.R / a.slices;
  const int nchunks = (a.K + G::kChunk - 1) / G::kChunk;
  const int p = pid[16 * w + (lane & 15)];
  const bool real = real_pair(p, a.numel);
  const bool live = __builtin_amdgcn_ballot_w64(real) != 0;  // uniform over the wave
  floatx4_t acc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc[nt] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  uint4 xf[G::kSteps], xn[G::kSteps];
  stage_w<NRT>(a, av, r0, 0, wt[0]);
  if (live) load_x<NRT>(a, p, real, 0, xf);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int c = 0; c < nchunks; ++c) {
    const int buf = c & 1;
    if (c + 1 < nchunks) {  // next chunk in flight while this one is multiplied
      stage_w<NRT>(a, av, r0, (c + 1) * G::kChunk, wt[buf ^ 1]);
      if (live) load_x<NRT>(a, p, real, (c + 1) * G::kChunk, xn);
    }
    if (live) {
#pragma unroll
      for (int st = 0; st < G::kSteps; ++st) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const int rr = nt * 16 + (lane & 15);
          const int slot = (4 * st + (lane >> 4)) ^ (rr & (G::kSlots - 1));
          const uint4 wf = wt[buf][rr * G::kSlots + slot];
          acc[nt] = mfma16(xf[st], wf, acc[nt]);
        }
      }
    }
    if (c + 1 < nchunks) {
#pragma unroll
      for (int st = 0; st < G::kSteps; ++st) xf[st] = xn[st];
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();  // chunk c+1 has landed and chunk c is no longer read
  }
  if (live) {
    // result rows 4 (l/16) + i of this wave's tile = pairs, column l % 16 = row of A_v
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int pi = pid[16 * w + 4 * (lane >> 4) + i];
      if (real_pair(pi, a.numel)) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const int row = r0 + nt * 16 + (lane & 15);
          if (row < a.R) a.s[(int64_t)pi * a.R + row] = row % r < rl ? acc[nt][i] : 0.f;
        }
      }
    }
  }
}

// Registers for four workgroups per CU.
template <int NRT>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4)))
    shrink_mfma_kernel(DeltaArgs a, int n_items) {
  using G = ShrinkGeom<NRT>;
  __shared__ __attribute__((aligned(16))) uint4 wt[2][1024];  // 2 x 16 KiB
  __shared__ int pid[kRowsPerPass];
  __shared__ int nrows_lds;
  const int nrt = (a.R + G::kRows - 1) / G::kRows;
  const int n_live = min(n_items, live_blocks(a, *a.npp) * nrt);
  const int item = xcd_item(n_live);
  if (item >= n_live) return;
  const int blk = item / nrt, r0 = (item % nrt) * G::kRows;
  const int e = block_expert(a, blk);
  if (e < 0) return;  // past the live blocks or the sentinel bucket
  const int rl = slot_rank(a, e);
  const char* av = (const char*)a.A + (int64_t)e * a.R * a.K * 2;
  for (int j0 = 0; j0 < a.BM; j0 += kRowsPerPass) {
    const int nrows = stage_rows(a, blk, j0, pid, &nrows_lds);
    if (nrows == 0) break;
    shrink_mfma_pass<NRT>(a, av, r0, rl, pid, wt);
    if (nrows < kRowsPerPass) break;
  }
}

// ----------------------------------------------------------------- plan-driven dense runs
// With the align's work plan the MFMA expand takes the plan's runs instead of single
// blocks: up to kPlanDenseBlocks consecutive blocks of one virtual expert. A run item holds its weight columns for all of its blocks,
// where a block item loads them once per block (a hot expert's bucket of many blocks is
// read about a quarter as often). The shrink keeps its block items: a run there needs the
// accumulators of every block at once, and at the occupancy that leaves it measured
// slower than block items ordered by XCD, which share A_v through L2 instead.

// Run `run` of the plan: {first block, blocks, virtual expert}; nb = 0 past the plan's
// count (the entry read is then entry 0, a valid address).
struct DenseRun {
  int blk0, nb, e;
};
__device__ __forceinline__ DenseRun dense_run(const int32_t* plan, int run) {
  const int count = plan[0];
  const int rc = run < count ? run : 0;
  const int4 d =
      *reinterpret_cast<const int4*>(plan + kPlanHeader + (int64_t)rc * kPlanDenseInts);
  return DenseRun{d.x, run < count ? d.y : 0, d.z};
}

// ------------------------------------------------------------------------------ expand

// bf16 high part and bf16 remainder of 8 fp32 values (RNE both), packed for MFMA.
__device__ __forceinline__ void split_bf16(const uint4& f0, const uint4& f1, uint4* hi,
                                           uint4* lo) {
  const float v[8] = {__uint_as_float(f0.x), __uint_as_float(f0.y), __uint_as_float(f0.z),
                      __uint_as_float(f0.w), __uint_as_float(f1.x), __uint_as_float(f1.y),
                      __uint_as_float(f1.z), __uint_as_float(f1.w)};
  uint32_t h[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint16_t h0 = f32_to_bf16_rne(v[2 * i]), h1 = f32_to_bf16_rne(v[2 * i + 1]);
    const uint16_t l0 = f32_to_bf16_rne(v[2 * i] - __uint_as_float((uint32_t)h0 << 16));
    const uint16_t l1 = f32_to_bf16_rne(v[2 * i + 1] - __uint_as_float((uint32_t)h1 << 16));
    h[i] = (uint32_t)h0 | ((uint32_t)h1 << 16);
    l[i] = (uint32_t)l0 | ((uint32_t)l1 << 16);
  }
  *hi = make_uint4(h[0], h[1], h[2], h[3]);
  *lo = make_uint4(l[0], l[1], l[2], l[3]);
}

// s columns [cb, cb + rs) of the pass's pairs -> LDS [64 rows][rs/4 slots of 16 bytes], the
// vector kv of row m at slot kv ^ (m & mask): the fragment reads of 16 rows then hit
// distinct banks. Lane i of wave instruction t writes slot (4t + w) * 64 + i and fetches
// the vector that belongs there; rows past the real pairs copy the first pair's row (a
// written row; its products land in columns that are never stored).
__device__ __forceinline__ void stage_s(const DeltaArgs& a, const int* pid, int nrows, int cb,
                                       int rs, int mask, uint4* s_lds) {
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int spr = rs / 4;
  const char* sb = (const char*)a.s;
  for (int t = 0; t < rs / 16; ++t) {
    const int P = (4 * t + w) * 64 + lane;
    const int m = P / spr, slot = P % spr;
    const int kv = slot ^ (m & mask);
    const int pm = pid[m < nrows ? m : 0];
    lds_dma16(sb + ((int64_t)pm * a.R + cb + 4 * kv) * 4, s_lds + (4 * t + w) * 64);
  }
}

constexpr int kTileStride = kExpandCols + 4;  // fp32 result tile row, padded against conflicts

// The out rows of pair tile pt as the epilogue reads them: thread t holds the 16-byte
// vectors t and t + 256 of the tile's 16 rows x 32 vectors (8 bf16 each), so every wave
// reads two rows' 512 contiguous bytes. Vectors of rows that are not real pairs read zero.
// The rows are read and written non-temporally: each is touched once by this workgroup,
// while the weight tile of a virtual expert is re-read by its other column chunks' blocks.
__device__ __forceinline__ void load_out_tile(const DeltaArgs& a, const int* pid, int nrows,
                                              int pt, int chunk, uint4* ov) {
  const int t = threadIdx.x;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int v = t + 256 * h;
    const int m = 16 * pt + v / 32;
    const int n = chunk * kExpandCols + (v % 32) * 8;
    const bool ok = m < nrows && n < a.N;
    const int64_t off = ok ? ((int64_t)pid[m] * a.ld_out + n) * 2 : 0;
    ov[h] = ld16_nt_if((const char*)a.out, off, ok);
  }
}

// Blocks blk0..blk0+nb-1 (of virtual expert e) for output columns chunk: the weights are
// loaded once and held for every block.
template <int KS>
__device__ __forceinline__ void expand_mfma_blocks(const DeltaArgs& a, int blk0, int nb,
                                                   int chunk, int e, int rl, int* pid,
                                                   int* nrows_lds, uint4* s_lds, float* tile) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = a.R / a.slices, width = a.N / a.slices;
  const float sc = a.scale[fdiv(e, a.f_e)];
  // the slices this item's columns fall in: only their part of s is staged
  const int cfirst = chunk * kExpandCols;
  const int clast = min(a.N, cfirst + kExpandCols) - 1;
  const int g0 = cfirst / width, cb = g0 * r, rs = (clast / width - g0 + 1) * r;
  const int c0 = cfirst + 64 * w;  // this wave's 64 columns, one slice
  const int g = c0 < a.N ? c0 / width : g0;
  const int spr = rs / 4;
  const int mask = min(16, spr & -spr) - 1;
  // rows of B_v for the wave's columns: A operand, tile nt, step st
  const int64_t bbytes = (int64_t)a.N * r * 2;
  const __amdgpu_buffer_rsrc_t rb = expert_rsrc((const char*)a.B + (int64_t)e * bbytes, bbytes);
  uint4 bf[4][KS];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const int n = c0 + 16 * nt + (lane & 15);
#pragma unroll
    for (int st = 0; st < KS; ++st) {
      const int k = 32 * st + 8 * (lane >> 4);  // rank dimensions past rl are zero
      bf[nt][st] = buf16(rb, n < a.N && k < rl ? (uint32_t)((n * r + k) * 2) : kOutOfRange);
    }
  }
  for (int b = 0; b < nb; ++b)
  for (int j0 = 0; j0 < a.BM; j0 += kRowsPerPass) {
    const int nrows = stage_rows(a, blk0 + b, j0, pid, nrows_lds);
    if (nrows == 0) break;
    stage_s(a, pid, nrows, cb, rs, mask, s_lds);
    uint4 ov[2];
    load_out_tile(a, pid, nrows, 0, chunk, ov);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (rl < r) {  // uniform; after the wait, so the weight loads stay in one round trip
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
#pragma unroll
        for (int st = 0; st < KS; ++st)
          bf[nt][st] = keep_first<true>(bf[nt][st], rl - (32 * st + 8 * (lane >> 4)));
      }
    }
    const int ntiles = (nrows + 15) / 16;
#pragma unroll 1
    for (int pt = 0; pt < ntiles; ++pt) {
      uint4 ovn[2];
      if (pt + 1 < ntiles) load_out_tile(a, pid, nrows, pt + 1, chunk, ovn);  // uniform
      const int m = 16 * pt + (lane & 15);
      // s row of pair m, slice g: B operand (k = 32 st + 8 (l/16) .. +8), split hi + lo
      uint4 sh[KS], sl[KS];
#pragma unroll
      for (int st = 0; st < KS; ++st) {
        const int kv0 = ((g - g0) * r + 32 * st + 8 * (lane >> 4)) / 4;
        const uint4 f0 = s_lds[m * spr + (kv0 ^ (m & mask))];
        const uint4 f1 = s_lds[m * spr + ((kv0 + 1) ^ (m & mask))];
        split_bf16(f0, f1, &sh[st], &sl[st]);
      }
      // out^T tile: lane l holds pair l % 16, columns 16 nt + 4 (l/16) .. +4 of the wave's 64
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        floatx4_t acc = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < KS; ++st) {
          acc = mfma16(bf[nt][st], sh[st], acc);
          acc = mfma16(bf[nt][st], sl[st], acc);
        }
        *reinterpret_cast<floatx4_t*>(tile + (lane & 15) * kTileStride + 64 * w + 16 * nt +
                                      4 * (lane >> 4)) = acc;
      }
      __syncthreads();
      // epilogue over whole rows: thread t owns vectors t and t + 256 of the 16 x 32 grid
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int v = tid + 256 * h;
        const int q = v / 32, cv = v % 32;
        const int mq = 16 * pt + q;
        const int n = chunk * kExpandCols + cv * 8;
        if (mq < nrows && n < a.N) {
          const float* d = tile + q * kTileStride + cv * 8;
          const uint4 o = ov[h];
          const uint32_t ow[4] = {o.x, o.y, o.z, o.w};
          uint32_t res[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float lo = fmaf(sc, d[2 * i], bf16_lo(ow[i]));
            const float hi = fmaf(sc, d[2 * i + 1], bf16_hi(ow[i]));
            res[i] = (uint32_t)f32_to_bf16_rne(lo) | ((uint32_t)f32_to_bf16_rne(hi) << 16);
          }
          st16_nt((char*)a.out + ((int64_t)pid[mq] * a.ld_out + n) * 2,
                  make_uint4(res[0], res[1], res[2], res[3]));
        }
      }
      __syncthreads();  // the tile is rewritten by the next pair tile
      if (pt + 1 < ntiles) {
        ov[0] = ovn[0];
        ov[1] = ovn[1];
      }
    }
    if (nrows < kRowsPerPass) break;
  }
}

template <int KS>
__global__ void __launch_bounds__(256) expand_mfma_kernel(DeltaArgs a) {
  extern __shared__ uint4 s_lds[];  // [64][(slices of the item) * r / 4]
  __shared__ __attribute__((aligned(16))) float tile[16 * kTileStride];
  __shared__ int pid[kRowsPerPass];
  __shared__ int nrows_lds;
  const int blk = fdiv((int)blockIdx.x, a.f_nc), chunk = (int)blockIdx.x - blk * a.nchunk;
  const int e = block_expert(a, blk);
  if (e < 0) return;  // past the live blocks or the sentinel bucket
  const int rl = slot_rank(a, e);
  if (rl == 0) return;  // a slot of rank 0 adds nothing
  expand_mfma_blocks<KS>(a, blk, 1, chunk, e, rl, pid, &nrows_lds, s_lds, tile);
}

// Expand over the plan's dense runs: item = (run, 256 output columns).
template <int KS>
__global__ void __launch_bounds__(256) expand_mfma_run_kernel(const int32_t* plan,
                                                              int n_items, DeltaArgs a) {
  extern __shared__ uint4 s_lds[];
  __shared__ __attribute__((aligned(16))) float tile[16 * kTileStride];
  __shared__ int pid[kRowsPerPass];
  __shared__ int nrows_lds;
  const int n_live = min(n_items, plan[0] * a.nchunk);  // the plan's runs x column chunks
  const int item = xcd_item(n_live);
  if (item >= n_live) return;
  const int run = fdiv(item, a.f_nc), chunk = item - run * a.nchunk;
  const DenseRun d = dense_run(plan, run);
  if (d.nb == 0) return;
  const int rl = slot_rank(a, d.e);
  if (rl == 0) return;  // a slot of rank 0 adds nothing
  expand_mfma_blocks<KS>(a, d.blk0, d.nb, chunk, d.e, rl, pid, &nrows_lds, s_lds, tile);
}

}  // namespace

int shrink_mfma_row_tile(int32_t R) { return R > 64 ? 128 : 64; }

hipError_t launch_shrink_mfma(const DeltaArgs& a, int items, hipStream_t stream) {
  const dim3 grid(xcd_grid(items));
  if (shrink_mfma_row_tile(a.R) == 128)
    hipLaunchKernelGGL((shrink_mfma_kernel<2>), grid, dim3(256), 0, stream, a, items);
  else
    hipLaunchKernelGGL((shrink_mfma_kernel<1>), grid, dim3(256), 0, stream, a, items);
  return hipGetLastError();
}

// Slices of s the widest item needs: an item's kExpandCols columns can straddle slice
// boundaries. Only those columns of s are staged, so LDS is sized by them (at gate_up with
// slice widths that are multiples of kExpandCols, one slice: half of R), which leaves room
// for more workgroups per CU.
int expand_mfma_span(const DeltaArgs& a) {
  const int width = a.N / a.slices;
  int span = 1;
  for (int c0 = 0; c0 < a.N; c0 += kExpandCols) {
    const int c1 = (c0 + kExpandCols < a.N ? c0 + kExpandCols : a.N) - 1;
    const int sp = c1 / width - c0 / width + 1;
    span = sp > span ? sp : span;
  }
  return span;
}

hipError_t launch_expand_mfma(const DeltaArgs& a, int grid, hipStream_t stream) {
  // s rows of one pass, the columns of the slices one item spans
  const size_t lds =
      (size_t)kRowsPerPass * (a.R / a.slices) * expand_mfma_span(a) * sizeof(float);
  switch ((a.R / a.slices) / 32) {
    case 1: hipLaunchKernelGGL((expand_mfma_kernel<1>), dim3(grid), dim3(256), lds, stream, a); break;
    case 2: hipLaunchKernelGGL((expand_mfma_kernel<2>), dim3(grid), dim3(256), lds, stream, a); break;
    case 3: hipLaunchKernelGGL((expand_mfma_kernel<3>), dim3(grid), dim3(256), lds, stream, a); break;
    case 4: hipLaunchKernelGGL((expand_mfma_kernel<4>), dim3(grid), dim3(256), lds, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_expand_mfma_runs(const DeltaArgs& a, const int32_t* plan, int items,
                                   hipStream_t stream) {
  const dim3 grid(xcd_grid(items));
  // s rows of one pass, the columns of the slices one item spans
  const size_t lds =
      (size_t)kRowsPerPass * (a.R / a.slices) * expand_mfma_span(a) * sizeof(float);
  switch ((a.R / a.slices) / 32) {
    case 1: hipLaunchKernelGGL((expand_mfma_run_kernel<1>), grid, dim3(256), lds, stream, plan, items, a); break;
    case 2: hipLaunchKernelGGL((expand_mfma_run_kernel<2>), grid, dim3(256), lds, stream, plan, items, a); break;
    case 3: hipLaunchKernelGGL((expand_mfma_run_kernel<3>), grid, dim3(256), lds, stream, plan, items, a); break;
    case 4: hipLaunchKernelGGL((expand_mfma_run_kernel<4>), grid, dim3(256), lds, stream, plan, items, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace mol
