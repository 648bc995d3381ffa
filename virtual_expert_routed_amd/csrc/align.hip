// Remap and align_block_size for the MoL delta path on gfx950.
//
// align_block_size groups the (token, slot) pairs by virtual expert into BLOCK_M-padded
// buckets: histogram -> padded exclusive prefix sum -> one expert id per block -> scatter
// of the pair indices, with one extra sentinel bucket (id V) whose blocks are tagged -1
// (sglang PR 24262 page, implementation item 1; PR 24171 page, the sentinel-bucket
// snippet and risk item 2). Inside a bucket the pairs keep ascending order, so the
// result is unique and reproducible.
//
// Design (the order of the pairs never depends on atomics or on timing):
//  * the pairs are cut into contiguous ranges; one wave64 walks a range in chunks of 64
//    in ascending order;
//  * inside a chunk, lanes holding the same bucket find each other with one ballot per
//    key bit (13 ballots); the lowest lane of a group is its leader and the rank of a
//    lane is the number of group members below it (mbcnt);
//  * each range has a private per-bucket counter row (LDS), so a walk only touches its
//    own row;
//  * cursor[range][b] = off_b + (pairs of bucket b in earlier ranges): prefix sums in
//    range order, which gives the stable order across ranges.
// numel <= 4096 runs as up to 16 workgroups that each build the whole routing in LDS and
// split the writes (one launch); larger inputs run three kernels (count per tile -> scan
// over tiles -> scatter) through a workspace. The only atomics are the LDS histogram adds
// of the count kernel, whose result does not depend on their order.
#include "mol_internal.h"

namespace mol {
namespace {

__device__ __forceinline__ uint64_t wave_ballot(bool p) {
  return __builtin_amdgcn_ballot_w64(p);
}

// number of set bits of m in lanes below this lane
__device__ __forceinline__ int lanes_below(uint64_t m) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                        __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

__device__ __forceinline__ int remap_one(int32_t t, int32_t l, int32_t E, int32_t S) {
  return t < 0 ? t : ((t >= E || l < 0 || l >= S) ? -1 : t + l * E);
}

__device__ __forceinline__ int bucket_of(const AlignArgs& a, int p) {
  const int32_t t = a.ids[p];
  const int32_t v = a.lora ? remap_one(t, a.lora[fdiv(p, a.f_topk)], a.E, a.S) : t;
  return (v >= 0 && v < a.V) ? v : a.V;
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP: shifts of 1, 2, 4, 8 inside
// each row of 16 lanes, then the row broadcasts of lane 15 and lane 31 carry the row
// totals into the rows above. Lanes with no source lane take 0.
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return v;
}

// Exclusive prefix sum of one int per thread over the workgroup (<= 16 waves).
// `sh` is >= 33 ints of LDS; *total gets the sum over all threads.
__device__ __forceinline__ int block_excl_scan(int v, int* sh, int* total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  const int inc = wave_incl_scan(v);
  if (lane == 63) sh[wid] = inc;
  __syncthreads();
  if (wid == 0) {
    const int w = lane < nw ? sh[lane] : 0;
    const int winc = wave_incl_scan(w);
    if (lane < nw) sh[16 + lane] = winc - w;
    if (lane == 63) sh[32] = winc;
  }
  __syncthreads();
  *total = sh[32];
  return sh[16 + wid] + inc - v;
}

// x / BLOCK_M and c rounded up to a multiple of BLOCK_M (shifts when BLOCK_M is a power of 2)
__device__ __forceinline__ int bm_div(const AlignArgs& a, int x) {
  return a.bm_shift >= 0 ? x >> a.bm_shift : fdiv(x, a.f_bm);
}
__device__ __forceinline__ int bm_round(const AlignArgs& a, int c) {
  return a.bm_shift >= 0 ? (c + a.BM - 1) & -a.BM : fdiv(c + a.BM - 1, a.f_bm) * a.BM;
}

// ---------------------------------------------------------------------- the work plan
// A bucket of c real pairs has cdiv(c, BM) blocks, listed in the plan as runs of up to
// kPlanDenseBlocks consecutive blocks (layout in mol_internal.h); the sentinel bucket and
// empty buckets have none.
__device__ __forceinline__ int bucket_runs(const AlignArgs& a, int b, int c) {
  if (b >= a.V || c <= 0) return 0;
  return (bm_div(a, c + a.BM - 1) + kPlanDenseBlocks - 1) / kPlanDenseBlocks;
}

__device__ __forceinline__ int32_t* plan_run(const AlignArgs& a, int j) {
  return a.plan + kPlanHeader + (int64_t)j * kPlanDenseInts;
}

// Run jj of bucket b (first slot off_b, c real pairs) into plan entry j.
__device__ __forceinline__ void write_run(const AlignArgs& a, int b, int off_b, int c, int jj,
                                          int j) {
  const int nblk = bm_div(a, c + a.BM - 1);
  const int first = jj * kPlanDenseBlocks;
  *reinterpret_cast<int4*>(plan_run(a, j)) =
      make_int4(bm_div(a, off_b) + first, min(kPlanDenseBlocks, nblk - first), b, 0);
}

__global__ void __launch_bounds__(256) virtual_topk_kernel(const int32_t* __restrict__ topk,
                                                         const int32_t* __restrict__ lora,
                                                         int32_t numel, int32_t k, int32_t E,
                                                         int32_t S, int32_t* __restrict__ out) {
  const int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (p >= numel) return;
  out[p] = remap_one(topk[p], lora[p / k], E, S);
}

// All 13 key bits, unrolled: bits above the largest bucket id are zero for every lane
// and leave the mask unchanged.
__device__ __forceinline__ uint64_t match_key13(int key, bool valid) {
  uint64_t peers = wave_ballot(valid);
#pragma unroll
  for (int b = 0; b < 13; ++b) {
    const bool bit = (key >> b) & 1;
    const uint64_t ones = wave_ballot(valid && bit);
    peers &= bit ? ones : ~ones;
  }
  return peers;
}

// N consecutive ints of LDS at an N-int-aligned address (N a power of two), moved as one
// access of up to 16 bytes at a time.
template <int N>
struct LdsInts {
  int v[N];
  __device__ __forceinline__ void load(const int* p) {
    if constexpr (N == 1) {
      v[0] = p[0];
    } else if constexpr (N == 2) {
      const int2 t = *reinterpret_cast<const int2*>(p);
      v[0] = t.x; v[1] = t.y;
    } else {
#pragma unroll
      for (int j = 0; j < N; j += 4) {
        const int4 t = *reinterpret_cast<const int4*>(p + j);
        v[j] = t.x; v[j + 1] = t.y; v[j + 2] = t.z; v[j + 3] = t.w;
      }
    }
  }
  __device__ __forceinline__ void store(int* p) const {
    if constexpr (N == 1) {
      p[0] = v[0];
    } else if constexpr (N == 2) {
      *reinterpret_cast<int2*>(p) = make_int2(v[0], v[1]);
    } else {
#pragma unroll
      for (int j = 0; j < N; j += 4)
        *reinterpret_cast<int4*>(p + j) = make_int4(v[j], v[j + 1], v[j + 2], v[j + 3]);
    }
  }
};

// numel <= 4096: G workgroups of 1024 threads. Every workgroup builds the whole routing in
// its own LDS (the ids are a few KiB, so the repeated reads hit L2), then writes only
// its share of the outputs: the pairs p with p % G == g, and the expert ids and padding
// of the buckets b with b % G == g. No workgroup waits for another.
// LDS: `waves` counter rows of V+1 ints (each padded to a multiple of BPT), the V+1 bucket
// starts, 64 ints of scan scratch, then per pair its bucket id and its rank among the earlier
// pairs of the same bucket in its wave's range (uint16 each).
//   A  every thread: bucket ids of its pairs (ids and slots loaded together) -> LDS;
//      counter rows zeroed.
//   B  wave w walks its contiguous range in chunks of 64, in order: ballot-matched peers
//      give each pair's rank in the chunk, the group leader adds the group to row w and
//      hands the row's previous value to its peers, so rank_in_range = old + rank.
//   C  thread t owns BPT consecutive buckets, one aligned BPT-int access per row (the
//      threads of a wave read and write consecutive 4*BPT-byte pieces, so no LDS bank is
//      hit twice). One pass over the rows, four at a time, every read of a round issued
//      together: row w of bucket b becomes the pairs of b in ranges before w, and b's total
//      stays in a register. After the
//      padded exclusive scan, start[b] = off_b and the expert ids are written; nothing
//      is read back from LDS.
//   D  sorted[start[b(p)] + row[w(p)][b(p)] + rank_in_range(p)] = p for this workgroup's
//      pairs; each wave writes the padding of this workgroup's non-empty buckets its
//      threads own.
// The leading eight parameters (everything phase A needs: the ids, the slots, the pair
// count, the token divisor, the key array's LDS offset and the remap's E and S) arrive
// preloaded in scalar registers, so phase A's loads leave at the kernel's first
// instructions, before the argument struct has been fetched.
template <int BPT>
__global__ void __launch_bounds__(1024)
    align_small_kernel(const int32_t* ids, const int32_t* lora, int32_t numel_, uint32_t tk_m,
                       uint32_t tk_l, int32_t keys_off, int32_t E, int32_t S, AlignArgs a,
                       int waves) {
  extern __shared__ __attribute__((aligned(16))) int lds[];
  const int NB = a.V + 1;
  const int NBP = align_small_stride(NB);             // = NB rounded up to a multiple of BPT
  int* table = lds;                                   // [waves][NBP]
  int* start = lds + waves * NBP;                     // [NB] padded bucket starts
  int* sh = start + NB;                               // scan scratch (64 ints)
  uint16_t* keys = reinterpret_cast<uint16_t*>(lds + keys_off);  // = sh + 64
  uint16_t* rel = keys + ((numel_ + 1) & ~1);
  const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63;
  const int numel = numel_;
  const int g = blockIdx.x, G = gridDim.x;
  const FastDiv f_topk{(uint32_t)a.topk, tk_m, tk_l};

  // A: up to four pairs per thread (numel <= 4096 on this path), every load of ids and
  // slots issued together from the preloaded leading parameters, at unconditional clamped
  // addresses (an empty batch may come with no ids at all, so it loads nothing)
  if (numel > 0) {
    const int32_t* lsrc = lora ? lora : ids;  // a valid address either way
    int t[4], l[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int p = i * 1024 + tid;
      const int pc = p < numel ? p : 0;
      t[i] = ids[pc];
      l[i] = lsrc[lora ? fdiv(pc, f_topk) : pc];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int p = i * 1024 + tid;
      if (p < numel) {
        const int v = lora ? remap_one(t[i], l[i], E, S) : t[i];
        const int V = E * S;
        keys[p] = (uint16_t)((v >= 0 && v < V) ? v : V);
      }
    }
  }
  // the rows as 16-byte stores (the last one may run up to 3 ints into start, set later)
  for (int i = tid; i < (waves * NBP + 3) / 4; i += blockDim.x)
    reinterpret_cast<int4*>(table)[i] = make_int4(0, 0, 0, 0);
  __syncthreads();

  // B
  const int per = a.per;  // a multiple of 64, per * waves >= numel
  if (wid < waves) {
    int* row = table + wid * NBP;
    const int begin = min(numel, wid * per);
    const int end = min(numel, begin + per);
    for (int c = begin; c < end; c += 64) {
      const int p = c + lane;
      const bool valid = p < end;
      const int key = valid ? keys[p] : 0;
      const uint64_t peers = match_key13(key, valid);
      const int rank = lanes_below(peers);
      const int leader = valid ? __builtin_ctzll(peers) : lane;
      int old = 0;
      if (valid && rank == 0) {
        old = row[key];
        row[key] = old + __popcll(peers);
      }
      old = __shfl(old, leader, 64);
      if (valid) rel[p] = (uint16_t)(old + rank);
    }
  }
  __syncthreads();

  // C
  const int b0 = min(NB, tid * BPT);
  const int nown = min(NB, b0 + BPT) - b0;  // buckets this thread owns (uniform bound BPT)
  int run[BPT];
#pragma unroll
  for (int k = 0; k < BPT; ++k) run[k] = 0;
  if (nown > 0) {
    // b0 is a multiple of BPT below NB, so b0 + BPT <= NBP: the access stays in the row; the
    // row's padding entries are never incremented, so they read 0 and add nothing
    for (int w0 = 0; w0 < waves; w0 += 4) {
      LdsInts<BPT> x[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i].load(table + min(w0 + i, waves - 1) * NBP + b0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (w0 + i < waves) {
          LdsInts<BPT> y;
#pragma unroll
          for (int k = 0; k < BPT; ++k) {
            y.v[k] = run[k];
            run[k] += x[i].v[k];
          }
          y.store(table + (w0 + i) * NBP + b0);
        }
      }
    }
  }
  int mine = 0;
#pragma unroll
  for (int k = 0; k < BPT; ++k) mine += bm_round(a, run[k]);  // 0 past the owned buckets
  int total;
  int off = block_excl_scan(mine, sh, &total);
  // padding of this thread's buckets, kept as (first slot, count) per owned bucket
  int pad_from[BPT], pad_cnt[BPT];
  int bmod = fmod(b0, a.f_groups);  // b % G for b = b0, b0 + 1, ...
#pragma unroll
  for (int k = 0; k < BPT; ++k) {
    pad_cnt[k] = 0;
    pad_from[k] = 0;
    if (k < nown) {
      const int b = b0 + k;
      const int c = run[k];
      const int pc = bm_round(a, c);
      start[b] = off;
      if (bmod == g) {
        const int eid = (b == a.V) ? -1 : b;
        const int blk0 = bm_div(a, off), nblk = bm_div(a, pc);
        for (int j = 0; j < nblk; ++j) a.expert_ids[blk0 + j] = eid;
        pad_from[k] = off + c;
        pad_cnt[k] = pc - c;
      }
      off += pc;
      bmod = bmod + 1 == G ? 0 : bmod + 1;
    }
  }
  if (tid == 0 && g == 0) *a.npp = total;
  if (a.plan) {
    // the plan: each owned bucket's runs, at offsets from one more block scan, written by
    // the bucket's owning workgroup
    int nr = 0;
#pragma unroll
    for (int k = 0; k < BPT; ++k) nr += k < nown ? bucket_runs(a, b0 + k, run[k]) : 0;
    int rtotal;
    int pre = block_excl_scan(nr, sh, &rtotal);
    int bm2 = fmod(b0, a.f_groups);
#pragma unroll
    for (int k = 0; k < BPT; ++k) {
      if (k < nown) {
        const int b = b0 + k;
        const int nk = bucket_runs(a, b, run[k]);
        if (bm2 == g)
          for (int jj = 0; jj < nk; ++jj) write_run(a, b, start[b], run[k], jj, pre + jj);
        pre += nk;
        bm2 = bm2 + 1 == G ? 0 : bm2 + 1;
      }
    }
    if (tid == 0 && g == 0) {
      reinterpret_cast<int4*>(a.plan)[0] = make_int4(rtotal, 0, 0, 0);
      reinterpret_cast<int4*>(a.plan)[1] = make_int4(0, 0, 0, 0);
    }
  }
  __syncthreads();

  // D
  for (int p = g + tid * G; p < numel; p += (int)blockDim.x * G) {
    const int w = fdiv(p, a.f_per);
    const int key = keys[p];
    const int r = table[w * NBP + key] + rel[p];  // the pair's rank within its bucket
    a.sorted[start[key] + r] = p;
  }
  // padding: the wave's lanes fill one padded bucket after another
#pragma unroll
  for (int k = 0; k < BPT; ++k) {
    uint64_t todo = wave_ballot(pad_cnt[k] > 0);
    while (todo) {
      const int src = __builtin_ctzll(todo);
      todo &= todo - 1;
      const int from = __builtin_amdgcn_readlane(pad_from[k], src);
      const int cnt = __builtin_amdgcn_readlane(pad_cnt[k], src);
      for (int j = lane; j < cnt; j += 64) a.sorted[from + j] = numel;
    }
  }
}

// numel > 4096: three kernels over a workspace, the pairs cut into ntiles tiles.
//   count    one workgroup per tile: the tile's histogram in LDS (counts commute, so LDS
//            atomics are exact here) -> counts[t][b].
//   scan     one thread per bucket: counts[t][b] becomes the number of pairs of bucket b
//            in the tiles before t; totals[b] = all pairs of b.
//   scatter  one workgroup per tile: each one scans the padded totals itself (bucket
//            offsets in LDS, no extra launch), then wave 0 walks the tile in ascending
//            order and puts pair p at off_b + (pairs of b in earlier tiles) + (rank of p
//            among the earlier pairs of b in the tile), while the other waves write the
//            expert ids and the padding of this tile's share of the buckets.
__global__ void __launch_bounds__(256) align_count_kernel(AlignArgs a) {
  extern __shared__ int hist[];
  const int NB = a.V + 1;
  const int t = blockIdx.x, tid = threadIdx.x;
  for (int i = tid; i < NB; i += 256) hist[i] = 0;
  __syncthreads();
  const int begin = t * a.tile;
  const int end = min(a.numel, begin + a.tile);
  for (int base = begin; base < end; base += 4 * 256) {
    int key[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int p = base + i * 256 + tid;
      key[i] = p < end ? bucket_of(a, p) : -1;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (key[i] >= 0) atomicAdd(&hist[key[i]], 1);
  }
  __syncthreads();
  int32_t* row = a.counts + (int64_t)t * NB;
  for (int i = tid; i < NB; i += 256) row[i] = hist[i];
}

__global__ void __launch_bounds__(256) align_scan_kernel(AlignArgs a) {
  const int NB = a.V + 1;
  const int b = blockIdx.x * 256 + threadIdx.x;
  if (b >= NB) return;
  int run = 0;
  for (int t0 = 0; t0 < a.ntiles; t0 += 8) {
    int c[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {  // eight independent reads per round trip
      const int t = t0 + i < a.ntiles ? t0 + i : 0;
      c[i] = a.counts[(int64_t)t * NB + b];
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (t0 + i < a.ntiles) {
        a.counts[(int64_t)(t0 + i) * NB + b] = run;
        run += c[i];
      }
    }
  }
  a.totals[b] = run;
}

constexpr int kScanBucketsPerThread = kMaxBuckets / 256;  // 32

__global__ void __launch_bounds__(256) align_scatter_kernel(AlignArgs a) {
  extern __shared__ int lds[];
  const int NB = a.V + 1;
  int* off = lds;               // [NB] padded offset of each bucket
  int* cur = lds + NB;          // [NB] next slot of each bucket for this tile
  int* sh = lds + 2 * NB;       // scan scratch (64)
  uint16_t* keys = reinterpret_cast<uint16_t*>(sh + 64);  // [tile]
  const int t = blockIdx.x, tid = threadIdx.x;
  const int wid = tid >> 6, lane = tid & 63;
  const int begin = t * a.tile;
  const int end = min(a.numel, begin + a.tile);
  for (int p = begin + tid; p < end; p += 256) keys[p - begin] = (uint16_t)bucket_of(a, p);
  // padded exclusive scan of the totals: thread tid owns buckets [b0, b1)
  const int bpt = (NB + 255) / 256;
  const int b0 = min(NB, tid * bpt), b1 = min(NB, b0 + bpt);
  int cnt[kScanBucketsPerThread];
  int mine = 0;
#pragma unroll
  for (int k = 0; k < kScanBucketsPerThread; ++k) {
    const int b = b0 + k;
    cnt[k] = b < b1 ? a.totals[b] : 0;
    mine += bm_round(a, cnt[k]);
  }
  int total;
  int o = block_excl_scan(mine, sh, &total);
#pragma unroll
  for (int k = 0; k < kScanBucketsPerThread; ++k) {
    const int b = b0 + k;
    if (b < b1) {
      off[b] = o;
      o += bm_round(a, cnt[k]);
    }
  }
  if (t == 0 && tid == 0) *a.npp = total;
  __syncthreads();
  // this tile's cursors: all of the thread's counter reads issued together
  const int32_t* row = a.counts + (int64_t)t * NB;
  {
    int rv[kScanBucketsPerThread];
#pragma unroll
    for (int k = 0; k < kScanBucketsPerThread; ++k) {
      const int b = tid + 256 * k;
      rv[k] = row[b < NB ? b : 0];
    }
#pragma unroll
    for (int k = 0; k < kScanBucketsPerThread; ++k) {
      const int b = tid + 256 * k;
      if (b < NB) cur[b] = off[b] + rv[k];
    }
  }
  __syncthreads();
  if (wid == 0) {
    for (int c = begin; c < end; c += 64) {
      const int p = c + lane;
      const bool valid = p < end;
      const int key = valid ? keys[p - begin] : 0;
      const uint64_t peers = match_key13(key, valid);
      if (valid) {
        const int rank = lanes_below(peers);
        const int base = cur[key];  // every member reads before the leader writes
        if (rank == 0) cur[key] = base + __popcll(peers);
        a.sorted[base + rank] = p;
      }
    }
  } else {
    // expert ids and padding of this tile's share of the buckets: lane i of wave w takes
    // bucket bb0 + 64 (w - 1) + i of each pass (its total read with the others, not one
    // bucket after another), writes its expert ids, and the wave fills the padding of its
    // buckets one after another with all lanes
    const int bb0 = (int)((int64_t)NB * t / a.ntiles);
    const int bb1 = (int)((int64_t)NB * (t + 1) / a.ntiles);
    for (int base = bb0 + 64 * (wid - 1); base < bb1; base += 192) {
      const int b = base + lane;
      const bool own = b < bb1;
      const int c = own ? a.totals[b] : 0;
      const int o = own ? off[b] : 0;
      const int pc = bm_round(a, c);
      if (own) {
        const int eid = (b == a.V) ? -1 : b;
        const int blk0 = bm_div(a, o), nblk = bm_div(a, pc);
        for (int j = 0; j < nblk; ++j) a.expert_ids[blk0 + j] = eid;
      }
      uint64_t todo = wave_ballot(own && pc > c);
      while (todo) {
        const int src = __builtin_ctzll(todo);
        todo &= todo - 1;
        const int from = __builtin_amdgcn_readlane(o + c, src);
        const int cnt = __builtin_amdgcn_readlane(pc - c, src);
        for (int j = lane; j < cnt; j += 64) a.sorted[from + j] = a.numel;
      }
    }
  }
}

// numel > 4096, after the column scan: the work plan, by one 1024-thread workgroup. Thread t
// owns consecutive buckets, reads their totals, and two block scans (padded sizes and run
// counts) give each owned bucket its first slot and its first run; the thread then writes
// the bucket's runs.
__global__ void __launch_bounds__(1024) align_plan_kernel(AlignArgs a) {
  __shared__ int sh[64];
  const int NB = a.V + 1;
  const int tid = threadIdx.x;
  const int bpt = (NB + 1023) / 1024;
  const int b0 = min(NB, tid * bpt), b1 = min(NB, b0 + bpt);
  int pc = 0, nr = 0;
  for (int b = b0; b < b1; ++b) {
    const int c = a.totals[b];
    pc += bm_round(a, c);
    nr += bucket_runs(a, b, c);
  }
  int tp, tr;
  int po = block_excl_scan(pc, sh, &tp);
  __syncthreads();
  int ro = block_excl_scan(nr, sh, &tr);
  for (int b = b0; b < b1; ++b) {
    const int c = a.totals[b];
    const int nk = bucket_runs(a, b, c);
    for (int jj = 0; jj < nk; ++jj) write_run(a, b, po, c, jj, ro + jj);
    po += bm_round(a, c);
    ro += nk;
  }
  if (tid == 0) {
    reinterpret_cast<int4*>(a.plan)[0] = make_int4(tr, 0, 0, 0);
    reinterpret_cast<int4*>(a.plan)[1] = make_int4(0, 0, 0, 0);
  }
}

}  // namespace

hipError_t launch_virtual_topk(const int32_t* topk_ids, const int32_t* lora_ids, int32_t M,
                               int32_t topk, int32_t E, int32_t S, int32_t* out,
                               hipStream_t stream) {
  const int32_t numel = M * topk;
  const unsigned grid = (unsigned)((numel + 255) / 256);
  hipLaunchKernelGGL(virtual_topk_kernel, dim3(grid), dim3(256), 0, stream, topk_ids,
                     lora_ids, numel, topk, E, S, out);
  return hipGetLastError();
}

hipError_t launch_align_small(const AlignArgs& a, int waves, int groups, size_t lds_bytes,
                              hipStream_t stream) {
  // buckets per thread, a power of two (V + 1 <= 8192 = 8 x 1024)
  const int bpt = align_small_bpt(a.V + 1);
  const dim3 grid(groups), block(1024);
  // ints before the key array: counter rows, bucket starts, scan scratch
  const int keys_off = waves * align_small_stride(a.V + 1) + (a.V + 1) + 64;
#define MOL_ALIGN_SMALL(BPT)                                                                \
  hipLaunchKernelGGL(align_small_kernel<BPT>, grid, block, lds_bytes, stream, a.ids, a.lora, \
                     a.numel, a.f_topk.m, a.f_topk.l, keys_off, a.lora ? a.E : a.V,       \
                     a.lora ? a.S : 1, a, waves)
  if (bpt <= 1)
    MOL_ALIGN_SMALL(1);
  else if (bpt <= 2)
    MOL_ALIGN_SMALL(2);
  else if (bpt <= 4)
    MOL_ALIGN_SMALL(4);
  else
    MOL_ALIGN_SMALL(8);
#undef MOL_ALIGN_SMALL
  return hipGetLastError();
}

hipError_t launch_align_large(const AlignArgs& a, size_t scatter_lds_bytes,
                              hipStream_t stream) {
  const size_t nb_bytes = (size_t)(a.V + 1) * sizeof(int);
  hipLaunchKernelGGL(align_count_kernel, dim3(a.ntiles), dim3(256), nb_bytes, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(align_scan_kernel, dim3((a.V + 1 + 255) / 256), dim3(256), 0, stream, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(align_scatter_kernel, dim3(a.ntiles), dim3(256), scatter_lds_bytes,
                     stream, a);
  e = hipGetLastError();
  if (e != hipSuccess || !a.plan) return e;
  hipLaunchKernelGGL(align_plan_kernel, dim3(1), dim3(1024), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mol
