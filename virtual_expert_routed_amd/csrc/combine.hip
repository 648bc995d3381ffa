// The step after the down projection: each token's output is the router-weighted sum of
// its top-k pair rows, over the pairs whose base expert is local (0 <= t < E; a negative
// id is an expert-parallel sentinel whose expert lives on another GPU, so the pair has no
// row here). The pages leave this step implicit; it is the combine that consumes the
// rows the down stage's delta was added into.
//
//   combine:        y[m, n] = round( sum_k w[m, k] * rows[m*topk + k, n] )
//   expand_combine: y[m, n] = round( sum_k w[m, k] * (base[p, n] + d_p[n]) ),  p = m*topk + k
//                   d_p[n]  = scale[l] * sum_{j < rl} B[v, n, j] * s[p, j]  for a pair with
//                             virtual expert v = t + l*E (slot l of the token) and rank rl > 0
//
// Both sum in fp32 and round once. The fused form never writes the per-pair rows: at
// decode a token's pairs almost never share a virtual expert, so reading B_v per pair
// instead of per aligned block costs no extra weight bytes, and the rows' read-modify-
// write plus one launch go away. (With many tokens per expert, as in prefill, it would
// re-read each B_v once per token; there the aligned expand followed by the combine is
// the right pair of calls.)
#include "delta_common.h"

namespace mol {
namespace {

__device__ __forceinline__ bool local_expert(int t, int E) { return (unsigned)t < (unsigned)E; }

// ------------------------------------------------------------------------------ combine
// One wave per (token, VE*64 columns); lane owns one 16-byte vector (8 bf16 or 4 fp32).
// The pair rows' loads go out kCombineBatch at a time before any is summed.
constexpr int kCombineBatch = 8;

template <bool BF16>
__global__ void __launch_bounds__(64) combine_kernel(CombineArgs a) {
  constexpr int VE = BF16 ? 8 : 4;
  constexpr int ESZ = BF16 ? 2 : 4;
  const int chunks = (a.N + 64 * VE - 1) / (64 * VE);
  const int m = blockIdx.x / chunks;
  const int n = (blockIdx.x % chunks) * 64 * VE + (int)threadIdx.x * VE;
  const bool col_ok = n < a.N;
  const char* rows = (const char*)a.rows;
  float acc[VE];
#pragma unroll
  for (int i = 0; i < VE; ++i) acc[i] = 0.f;
  for (int k0 = 0; k0 < a.topk; k0 += kCombineBatch) {
    uint4 v[kCombineBatch];
    float w[kCombineBatch];
#pragma unroll
    for (int i = 0; i < kCombineBatch; ++i) {
      const int k = k0 + i;
      const int64_t p = (int64_t)m * a.topk + (k < a.topk ? k : 0);
      const bool ok = k < a.topk && local_expert(a.topk_ids[p], a.E);
      w[i] = ok ? a.weights[p] : 0.f;
      v[i] = ld16_if(rows, (p * a.ld_rows + n) * ESZ, ok && col_ok);
    }
#pragma unroll
    for (int i = 0; i < kCombineBatch; ++i) {
      const uint32_t u[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if constexpr (BF16) {
          acc[2 * q] = fmaf(w[i], bf16_lo(u[q]), acc[2 * q]);
          acc[2 * q + 1] = fmaf(w[i], bf16_hi(u[q]), acc[2 * q + 1]);
        } else {
          acc[q] = fmaf(w[i], __uint_as_float(u[q]), acc[q]);
        }
      }
    }
  }
  if (!col_ok) return;
  char* y = (char*)a.y + ((int64_t)m * a.ld_y + n) * ESZ;
  if constexpr (BF16) {
    uint32_t o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      o[q] = (uint32_t)f32_to_bf16_rne(acc[2 * q]) |
             ((uint32_t)f32_to_bf16_rne(acc[2 * q + 1]) << 16);
    *reinterpret_cast<uint4*>(y) = make_uint4(o[0], o[1], o[2], o[3]);
  } else {
    *reinterpret_cast<uint4*>(y) = make_uint4(__float_as_uint(acc[0]), __float_as_uint(acc[1]),
                                              __float_as_uint(acc[2]), __float_as_uint(acc[3]));
  }
}

// ----------------------------------------------------------------------- expand_combine
// Work item = (token m, 64 output columns), four waves. Wave w takes the pairs
// k = w, w + 4, ... two at a time; lane c owns column n = 64*chunk + c and holds that
// column's R weights of the pair's B_v. The s rows of the wave's two pairs go to LDS
// (one 16-byte vector per lane), so the dot products read them as broadcasts. Each wave
// leaves its partial sum per column in LDS; wave 0 adds them in wave order and rounds.
constexpr int kFusedWaves = 4;
constexpr int kFusedPairs = 2;  // pairs per wave per round
constexpr int kFusedMaxR = 128;

template <bool BF16, int RV>
__global__ void __launch_bounds__(256) expand_combine_kernel(CombineArgs a) {
  constexpr int VE = BF16 ? 8 : 4;
  constexpr int ESZ = BF16 ? 2 : 4;
  constexpr int R = RV * VE;  // the rank this instance is built for (a.R == R)
  __shared__ __attribute__((aligned(16))) float s_lds[kFusedWaves][kFusedPairs][R];
  __shared__ float part[kFusedWaves][64];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int chunks = (a.N + 63) / 64;
  const int m = blockIdx.x / chunks;
  const int n = (blockIdx.x % chunks) * 64 + lane;
  const bool col_ok = n < a.N;
  const int64_t bbytes = (int64_t)a.N * R * ESZ;
  const int lm = a.lora[m];
  float acc = 0.f;
  for (int k0 = w; k0 < a.topk; k0 += kFusedWaves * kFusedPairs) {
    uint4 bv[kFusedPairs][RV];
    float base[kFusedPairs], wk[kFusedPairs], sc[kFusedPairs];
    int rl[kFusedPairs];
    bool has[kFusedPairs];
#pragma unroll
    for (int i = 0; i < kFusedPairs; ++i) {
      const int k = k0 + i * kFusedWaves;
      const int64_t p = (int64_t)m * a.topk + (k < a.topk ? k : 0);
      const int t = a.topk_ids[p];
      const bool row = k < a.topk && local_expert(t, a.E);
      const bool lora = row && lm >= 0 && lm < a.S;  // a valid virtual expert t + l*E
      const int v = lora ? t + lm * a.E : 0;
      rl[i] = lora ? (a.ranks ? min(max(a.ranks[lm], 0), R) : R) : 0;
      has[i] = rl[i] > 0;
      wk[i] = row ? a.weights[p] : 0.f;
      sc[i] = has[i] ? a.scale[lm] : 0.f;
      const __amdgpu_buffer_rsrc_t rb =
          expert_rsrc((const char*)a.B + (int64_t)v * bbytes, bbytes);
#pragma unroll
      for (int q = 0; q < RV; ++q)
        bv[i][q] = buf16(rb, has[i] && col_ok && q * VE < rl[i]
                                 ? (uint32_t)((n * R + q * VE) * ESZ) : kOutOfRange);
      base[i] = 0.f;
      if (row && col_ok) {
        const int64_t bi = p * a.ld_base + n;
        base[i] = BF16 ? __uint_as_float((uint32_t)((const uint16_t*)a.base)[bi] << 16)
                       : ((const float*)a.base)[bi];
      }
      // the pair's s row: lanes [0, R/4) move one 16-byte vector each
      if (has[i] && lane < R / 4)
        *reinterpret_cast<float4*>(&s_lds[w][i][lane * 4]) =
            *reinterpret_cast<const float4*>(a.s + p * a.R + lane * 4);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int i = 0; i < kFusedPairs; ++i) {
      float d = 0.f;
      if (has[i]) {  // uniform over the wave
#pragma unroll
        for (int q = 0; q < RV; ++q) {
          uint4 b = bv[i][q];
          if (rl[i] < (q + 1) * VE) b = keep_first<BF16>(b, rl[i] - q * VE);
          d = dot16_s<BF16>(b, &s_lds[w][i][q * VE], d);
        }
      }
      acc = fmaf(wk[i], fmaf(sc[i], d, base[i]), acc);
    }
    __builtin_amdgcn_wave_barrier();  // the next round rewrites this wave's s rows
  }
  part[w][lane] = acc;
  __syncthreads();
  if (w != 0 || !col_ok) return;
  const float sum = ((part[0][lane] + part[1][lane]) + part[2][lane]) + part[3][lane];
  const int64_t yi = (int64_t)m * a.ld_y + n;
  if constexpr (BF16)
    ((uint16_t*)a.y)[yi] = f32_to_bf16_rne(sum);
  else
    ((float*)a.y)[yi] = sum;
}

template <bool BF16>
hipError_t fused_dispatch(const CombineArgs& a, int grid, hipStream_t st) {
  constexpr int VE = BF16 ? 8 : 4;
  switch (a.R / VE) {
    case 1: hipLaunchKernelGGL((expand_combine_kernel<BF16, 1>), dim3(grid), dim3(256), 0, st, a); break;
    case 2: hipLaunchKernelGGL((expand_combine_kernel<BF16, 2>), dim3(grid), dim3(256), 0, st, a); break;
    case 4: hipLaunchKernelGGL((expand_combine_kernel<BF16, 4>), dim3(grid), dim3(256), 0, st, a); break;
    case 8: hipLaunchKernelGGL((expand_combine_kernel<BF16, 8>), dim3(grid), dim3(256), 0, st, a); break;
    case 16: hipLaunchKernelGGL((expand_combine_kernel<BF16, 16>), dim3(grid), dim3(256), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

bool fused_rank_supported(int32_t R, bool bf16) {
  const int ve = bf16 ? 8 : 4;
  if (R <= 0 || R > kFusedMaxR || R % ve) return false;
  const int rv = R / ve;  // 16-byte weight vectors per column: a power of two up to 16
  return rv == 1 || rv == 2 || rv == 4 || rv == 8 || rv == 16;
}

hipError_t launch_combine(const CombineArgs& a, bool bf16, hipStream_t stream) {
  const int ve = bf16 ? 8 : 4;
  const int64_t grid = (int64_t)a.M * ((a.N + 64 * ve - 1) / (64 * ve));
  if (bf16)
    hipLaunchKernelGGL(combine_kernel<true>, dim3((unsigned)grid), dim3(64), 0, stream, a);
  else
    hipLaunchKernelGGL(combine_kernel<false>, dim3((unsigned)grid), dim3(64), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_expand_combine(const CombineArgs& a, bool bf16, hipStream_t stream) {
  const int64_t grid = (int64_t)a.M * ((a.N + 63) / 64);
  return bf16 ? fused_dispatch<true>(a, (int)grid, stream)
              : fused_dispatch<false>(a, (int)grid, stream);
}

}  // namespace mol
