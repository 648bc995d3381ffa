// The base MoE grouped GEMM of a stage, with the LoRA delta optionally fused into its
// epilogue. The pages' layer runs base grouped-GEMM launches and, after them, the LoRA
// shrink/expand launches that add the delta into the same output rows (MindLab sglang
// PR 24, the PR body's per-layer launch count). Here the delta can be added before the
// base result is rounded, so the output rows are written once instead of written, read back
// and written again.
//
//   out[p, n] = round( sum_k W[t_p, n, k] * xin[p / row_div, k]
//                      + [fused, slot l valid, rank rl > 0]
//                        scale[l] * sum_{j < rl} B[t_p + l*E, n, j] * s[p, g(n)*r + j] )
//
// for every pair whose base expert t_p is local (0 <= t_p < E); other rows are untouched.
// The pairs come grouped by base expert (align_block_size over the base ids, one slot).
//
// At decode this is the same gather of matrix-vector products as the LoRA shrink, over
// far larger weights (W_t is N x K), so it is built the same way: a work item is (block,
// RPI consecutive output columns), each column's row of W_t read once with coalesced
// 16-byte buffer loads by LPR lanes and reused for up to four pairs, the pairs' input
// rows staged in LDS, the lanes' partial sums combined by a fixed butterfly. The fused
// delta costs, per pair, the B row slices of the item's columns and the s row, moved into
// LDS by direct-to-LDS loads in the last weight segment's round trip, and each lane adds its
// part of the rank sum to its partial before the tree: the delta needs no extra pass over
// the output and no extra write. (Measured at decode on MI355X it is still slower than the
// base GEMM followed by a separate expand: the base GEMM streams its weights at about
// 6 TB/s in items of eight columns, and the delta's extra bytes per item show.)
#include "delta_common.h"

namespace mol {
namespace {

// The fused delta's operands in (dynamic) LDS: per pair, the B row slices of the item's
// columns and the s row (R <= 256 floats).
constexpr int kSRowBytes = 1024;
__host__ __device__ inline int gemm_bslice_bytes(int rpi, int rbytes) { return rpi * rbytes; }
static_assert(kThreads / 64 == kPG, "wave q stages pair q's delta operands");

template <bool BF16, int LPR, bool FUSED>
__device__ __forceinline__ void gemm_group(const GemmArgs& g, int e, int rg, const int* p,
                                           int nq, uint4* xs, char* dl) {
  constexpr int ESZ = BF16 ? 2 : 4;
  constexpr int VE = BF16 ? 8 : 4;  // elements of one 16-byte vector
  constexpr int RPI = kThreads / LPR;
  constexpr int SEGV = kSeg * LPR;
  constexpr int XPT = kPG * SEGV / kThreads;
  static_assert(XPT >= 1 && kPG * SEGV % kThreads == 0, "x staging covers whole waves");
  const int tid = threadIdx.x;
  const int lr = tid % LPR;
  const int n = rg * RPI + tid / LPR;  // this row group's output column
  const bool n_ok = n < g.N;
  const int nvec = g.K * ESZ / 16;
  const int vpl = (nvec + LPR - 1) / LPR;
  const int64_t wbytes = (int64_t)g.N * g.K * ESZ;
  const __amdgpu_buffer_rsrc_t rw = expert_rsrc((const char*)g.W + (int64_t)e * wbytes, wbytes);
  const uint32_t row_off = (uint32_t)(n_ok ? n : 0) * (uint32_t)(g.K * ESZ);
  const char* xbase = (const char*)g.xin;
  const int64_t xstride = g.ld_x * ESZ;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  float acc[kPG];
#pragma unroll
  for (int i = 0; i < kPG; ++i) acc[i] = 0.f;

  // The fused delta. Its per-pair slot, rank and scale are uniform over the workgroup and
  // read up front. Its vector operands go straight to LDS in the last weight segment's round
  // trip (wave q: pair q's B row slices for the item's columns, one contiguous run, and its
  // s row), so the delta adds neither a dependent round trip nor registers to the weight
  // loop. After the products, lane lr takes 16-byte vectors lr, lr + LPR, ... of its
  // column's B row slice and the matching s values, and adds its share of the rank sum to
  // its partial before the butterfly.
  int rlq[kPG], vq[kPG];
  float scq[kPG];
  if constexpr (FUSED) {
    const int r = g.R / g.slices;
#pragma unroll
    for (int i = 0; i < kPG; ++i) {
      const int pq = i < nq ? (i == 0 ? p[0] : i == 1 ? p[1] : i == 2 ? p[2] : p[3]) : 0;
      const int l = i < nq ? g.lora[pq / g.topk] : -1;
      const bool lv = l >= 0 && l < g.S;
      rlq[i] = lv ? (g.ranks ? min(max(g.ranks[l], 0), r) : r) : 0;
      vq[i] = lv ? e + l * g.E : 0;
      scq[i] = lv ? g.scale[l] : 0.f;
    }
  }

  for (int m0 = 0; m0 < vpl; m0 += kSeg) {
    uint4 wvec[kSeg];
#pragma unroll
    for (int sg = 0; sg < kSeg; ++sg) {
      const int v = lr + (m0 + sg) * LPR;
      wvec[sg] = buf16(rw, (n_ok && v < nvec) ? row_off + (uint32_t)v * 16u : kOutOfRange);
    }
    if (m0 > 0) __syncthreads();  // earlier readers of xs are done
#pragma unroll
    for (int t = 0; t < XPT; ++t) {
      const int i = tid + t * kThreads;
      const int q = i / SEGV;
      const int v = m0 * LPR + (i - q * SEGV);
      const bool ok = q < nq && v < nvec;
      const int pq = !ok ? 0 : q == 0 ? p[0] : q == 1 ? p[1] : q == 2 ? p[2] : p[3];
      lds_dma16(xbase + (ok ? (int64_t)fdiv(pq, g.route.f_rd) * xstride + (int64_t)v * 16 : 0),
                xs + wv * 64 + t * kThreads);
    }
    if constexpr (FUSED) {
      if (m0 + kSeg >= vpl && wv < nq) {  // wave q takes pair q (uniform)
        const int r = g.R / g.slices, rb = r * ESZ;
        const int bsz = gemm_bslice_bytes(RPI, rb);
        const int lane = tid & 63;
        const int v = wv == 0 ? vq[0] : wv == 1 ? vq[1] : wv == 2 ? vq[2] : vq[3];
        const int pq = wv == 0 ? p[0] : wv == 1 ? p[1] : wv == 2 ? p[2] : p[3];
        // the item's columns n0.. are consecutive rows of B_v: one contiguous slice (the
        // columns past N are not loaded; their lanes never read them)
        const int64_t mat = (int64_t)g.N * rb;
        const char* bsrc = (const char*)g.B + (int64_t)v * mat;
        const int64_t first = (int64_t)rg * RPI * rb;
        const int nv = (int)(min<int64_t>(mat - first, bsz) / 16);
        char* bdst = dl + wv * bsz;
        for (int t0 = 0; t0 < nv; t0 += 64)
          if (t0 + lane < nv) lds_dma16(bsrc + first + (int64_t)(t0 + lane) * 16, bdst + t0 * 16);
        const float* srow = g.s + (int64_t)pq * g.R;
        if (lane < g.R / 4) lds_dma16(srow + lane * 4, dl + kPG * bsz + wv * kSRowBytes);
      }
    }
    __builtin_amdgcn_s_waitcnt(0);  // the x DMA and the weights have landed
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kPG; ++i) {
      if (i >= nq) break;
#pragma unroll
      for (int sg = 0; sg < kSeg; ++sg) {
        const int v = lr + (m0 + sg) * LPR;
        if (v < nvec) acc[i] = dot16<BF16>(wvec[sg], xs[i * SEGV + sg * LPR + lr], acc[i]);
      }
    }
  }
  if constexpr (FUSED) {
    const int r = g.R / g.slices, rb = r * ESZ;
    const int bsz = gemm_bslice_bytes(RPI, rb);
    const int gs = n_ok ? fdiv(n, g.route.f_w) : 0;
    const int c = tid / LPR;  // this lane's column within the item
    constexpr int NVL = (kMaxRankVecs + LPR - 1) / LPR;
#pragma unroll
    for (int i = 0; i < kPG; ++i) {
      if (i >= nq || rlq[i] == 0 || !n_ok || lr * VE >= rlq[i]) continue;  // no part here
      const char* bsl = dl + i * bsz + c * rb;
      const float* sp0 = reinterpret_cast<const float*>(dl + kPG * bsz + i * kSRowBytes) + gs * r;
      float d = 0.f;
#pragma unroll
      for (int w = 0; w < NVL; ++w) {
        const int vi = lr + w * LPR;
        if (vi * VE >= rlq[i]) break;
        const uint4 braw = *reinterpret_cast<const uint4*>(bsl + vi * 16);
        const float4 s0 = *reinterpret_cast<const float4*>(sp0 + vi * VE);
        const float4 s1 = BF16 ? *reinterpret_cast<const float4*>(sp0 + vi * VE + 4)
                               : make_float4(0.f, 0.f, 0.f, 0.f);  // fp32: 4 per vector
        const float sv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
        // the vector that straddles the slot's rank is trimmed
        const uint4 b = rlq[i] < (vi + 1) * VE ? keep_first<BF16>(braw, rlq[i] - vi * VE) : braw;
        d = dot16_s<BF16>(b, sv, d);
      }
      acc[i] = fmaf(scq[i], d, acc[i]);
    }
  }
#pragma unroll
  for (int i = 0; i < kPG; ++i) acc[i] = group_sum<LPR>(acc[i]);
  if (lr == 0 && n_ok) {
#pragma unroll
    for (int i = 0; i < kPG; ++i) {
      if (i >= nq) break;
      const int64_t o = (int64_t)p[i] * g.ld_out + n;
      if constexpr (BF16)
        ((uint16_t*)g.out)[o] = f32_to_bf16_rne(acc[i]);
      else
        ((float*)g.out)[o] = acc[i];
    }
  }
}

template <bool BF16, int LPR, bool FUSED>
__global__ void __launch_bounds__(kThreads) gemm_kernel(MOL_ROUTE_PARAMS, GemmArgs g) {
  __shared__ int pid[kPidSlots];
  __shared__ int nreal;
  __shared__ uint4 xs[kPG * kSeg * LPR];
  extern __shared__ __attribute__((aligned(16))) char dl[];  // the fused delta's operands
  const DeltaArgs& a = g.route;
  const RouteArgs r = MOL_ROUTE_MAKE;
  const int blk = route_block(r), rg = (int)blockIdx.x - blk * r.per;
  const BlockHead h = block_head(a, r, blk);
  const int e = h.e;
  if (e < 0) return;  // sentinel block (no local expert) or past the live blocks
  if (h.all_here) {
    if (h.nq > 0) gemm_group<BF16, LPR, FUSED>(g, e, rg, h.p, h.nq, xs, dl);
    return;
  }
  for (int j0 = 0; j0 < a.BM; j0 += kPidSlots) {
    const int pv = threadIdx.x < kPidSlots ? load_pid(a, blk, j0) : a.numel;
    __syncthreads();
    publish_pids(a, pv, pid, &nreal);
    __syncthreads();
    const int nr = nreal;
    for (int q0 = 0; q0 < nr; q0 += kPG) {
      int pq[kPG];
#pragma unroll
      for (int i = 0; i < kPG; ++i) pq[i] = q0 + i < nr ? pid[q0 + i] : a.numel;
      __syncthreads();  // xs of the previous group is no longer read
      gemm_group<BF16, LPR, FUSED>(g, e, rg, pq, min(kPG, nr - q0), xs, dl);
    }
    if (nr < kPidSlots) return;  // the block's real entries ended in this pass
  }
}

template <bool BF16, bool FUSED>
hipError_t gemm_dispatch(const GemmArgs& g, int lpr, int grid, hipStream_t st) {
  const size_t dyn =
      FUSED ? (size_t)kPG * (gemm_bslice_bytes(kThreads / lpr, (g.R / g.slices) * (BF16 ? 2 : 4)) +
                             kSRowBytes)
            : 0;
  switch (lpr) {
    case 8: hipLaunchKernelGGL((gemm_kernel<BF16, 8, FUSED>), dim3(grid), dim3(kThreads), dyn, st, MOL_ROUTE_ARGS(g.route, g.rgroups, g.route.f_rg), g); break;
    case 16: hipLaunchKernelGGL((gemm_kernel<BF16, 16, FUSED>), dim3(grid), dim3(kThreads), dyn, st, MOL_ROUTE_ARGS(g.route, g.rgroups, g.route.f_rg), g); break;
    case 32: hipLaunchKernelGGL((gemm_kernel<BF16, 32, FUSED>), dim3(grid), dim3(kThreads), dyn, st, MOL_ROUTE_ARGS(g.route, g.rgroups, g.route.f_rg), g); break;
    case 64: hipLaunchKernelGGL((gemm_kernel<BF16, 64, FUSED>), dim3(grid), dim3(kThreads), dyn, st, MOL_ROUTE_ARGS(g.route, g.rgroups, g.route.f_rg), g); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_moe_gemm(const GemmArgs& g, bool bf16, int rows_per_item, int grid,
                           hipStream_t stream) {
  const int lpr = kThreads / rows_per_item;
  const bool fused = g.s != nullptr;
  if (bf16)
    return fused ? gemm_dispatch<true, true>(g, lpr, grid, stream)
                 : gemm_dispatch<true, false>(g, lpr, grid, stream);
  return fused ? gemm_dispatch<false, true>(g, lpr, grid, stream)
               : gemm_dispatch<false, false>(g, lpr, grid, stream);
}

}  // namespace mol
