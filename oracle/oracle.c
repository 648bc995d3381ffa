/*
 * Plain CPU oracle for the multi-LoRA MoE ("MoL", virtual-experts) delta path.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the package's smoke check and the
 * benchmark's CPU-baseline leg may load this library. The GPU path shares no code,
 * header, table or constant with it, and never calls it.
 *
 * It is the plain definition of what the path computes, with nothing blocked, fused
 * or reordered, accumulating in double precision:
 *
 *   remap   - virtual id  v = t + l*E  for base expert t of a token with LoRA slot l;
 *             a negative t (an expert-parallel dispatch sentinel) is kept as it is.
 *             (sglang PR 24171 summary, "implementation" item 2 and its
 *             virtual_experts snippet; the -1 "no adapter" slot contract is the
 *             "base takes no pool slot" and "-1 guards" commits of MindLab sglang PR 24.)
 *   align   - counting sort of the pairs by virtual id into BLOCK_M-padded buckets,
 *             with one extra sentinel bucket (id V) for every pair that has no valid
 *             virtual expert; its blocks are tagged -1 and skipped downstream
 *             (PR 24171 summary, the _align_block_size_torch snippet and risk item 2;
 *             PR 24262 summary, implementation item 1).
 *   shrink  - s[p, i] = sum_k A[v_p, i, k] * xin[row(p), k]
 *   expand  - out[p, n] += scale[v_p / E] * sum_j B[v_p, n, j] * s[p, g(n)*r + j]
 *             (MindLab sglang PR 24, the "...and grid blowup" commit and the PR body:
 *             shrink hidden -> rank, expand rank -> N, weights laid out [E, N, K]
 *             with N = shape[1] per the code-review commit.)
 *
 * Per-slot ranks (optional): a slot of rank rl < r uses rank dimensions [0, rl) of each
 * slice; s is 0 past it, and a slot of rank 0 gets no delta.
 *
 *   base    - the base MoE grouped GEMM of a stage, which the pages run as the base
 *             fused_moe_kernel launches the LoRA delta is added to: out[p, n] =
 *             sum_k W[t_p, n, k] * xin[row(p), k] for a pair whose base expert t_p is local
 *             (0 <= t_p < E), rounded once; with the LoRA delta fused in, out[p, n] = round(base
 *             + delta) with the delta of the expand above (MindLab sglang PR 24, the PR body's
 *             count of base and LoRA grouped-GEMM launches per layer).
 *   combine - the step after the down projection, which the pages leave implicit: each
 *             token's output is the router-weighted sum of its top-k pair rows,
 *             y[m, n] = sum_k w[m, k] * rows[m*topk + k, n], over the pairs whose base
 *             expert is local (0 <= t < E; a negative t is an expert-parallel sentinel
 *             whose expert lives on another GPU). The fused form takes the down stage's
 *             rows as base + delta, never rounded in between.
 *
 * Readings taken where the pages leave a step open (each is listed with its reason in
 * the design notes): a token with no adapter (slot -1) or a slot >= S, and a base id
 * >= E, map to virtual id -1; pairs inside a bucket keep ascending pair order; padding
 * entries of sorted_ids hold numel; gate_up uses two expand slices, slice g reading
 * s[:, g*r:(g+1)*r]; scale is per LoRA slot; bf16 outputs are rounded once, to nearest
 * even, from the exact double sum out + delta.
 *
 * Threading: the shrink and expand loop over aligned blocks with an OpenMP
 * "parallel for"; every output element is produced by one thread in a fixed order, so
 * the result does not depend on the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_OK = 0, OR_E_ARG = 1, OR_E_CAP = 2 };
enum { OR_F32 = 0, OR_BF16 = 1 };

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_num_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* ---- element access --------------------------------------------------------------- */

/* bfloat16 is the top half of an IEEE binary32; widening it is exact. */
static double bf16_to_double(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Round a double to the nearest bfloat16 (8 significant bits, exponent range of
 * binary32), ties to even, straight from its value: the spacing of representable
 * numbers in [2^(e-1), 2^e) is 2^(e-8), and 2^-133 below the smallest normal 2^-126.
 * Magnitudes that round past the largest finite value (255 * 2^120) become infinity. */
uint16_t oracle_bf16_from_double(double v) {
    uint16_t sign = signbit(v) ? 0x8000u : 0u;
    if (isnan(v)) return (uint16_t)(sign | 0x7FC0u);
    double a = fabs(v);
    if (isinf(a)) return (uint16_t)(sign | 0x7F80u);
    if (a == 0.0) return sign;
    int e;
    (void)frexp(a, &e);               /* a = m * 2^e, 0.5 <= m < 1 */
    int q = e - 8;
    if (q < -133) q = -133;
    double k = nearbyint(ldexp(a, -q)); /* default rounding mode: nearest, ties to even */
    double r = ldexp(k, q);
    if (r > 255.0 * ldexp(1.0, 120)) return (uint16_t)(sign | 0x7F80u);
    float f = (float)r;                  /* exact: r has at most 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(sign | (u >> 16));
}

void oracle_bf16_round_array(const double *in, uint16_t *out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_bf16_from_double(in[i]);
}

static double load_elem(const void *base, int64_t idx, int dtype) {
    if (dtype == OR_F32) return (double)((const float *)base)[idx];
    return bf16_to_double(((const uint16_t *)base)[idx]);
}

/* ---- remap ------------------------------------------------------------------------ */

/* Virtual id of one pair: a negative base id stays as it is; a base id past the
 * routed experts, or a slot outside [0, S) (slot -1 = no adapter), gives -1;
 * otherwise t + l*E. */
static int32_t virtual_id(int32_t t, int32_t l, int32_t E, int32_t S) {
    if (t < 0) return t;
    if (t >= E || l < 0 || l >= S) return -1;
    return t + l * E;
}

int oracle_virtual_topk(const int32_t *topk_ids, const int32_t *lora_ids, int64_t M,
                        int32_t topk, int32_t E, int32_t S, int32_t *out) {
    if (M < 0 || topk <= 0 || E <= 0 || S <= 0) return OR_E_ARG;
    if (M > 0 && (!topk_ids || !lora_ids || !out)) return OR_E_ARG;
    for (int64_t p = 0; p < M * topk; ++p)
        out[p] = virtual_id(topk_ids[p], lora_ids[p / topk], E, S);
    return OR_OK;
}

/* ---- align_block_size ------------------------------------------------------------- */

/* ids: base ids with lora_ids != NULL (remapped first), or virtual ids when NULL.
 * Bucket of a pair: its virtual id when in [0, V), else the sentinel bucket V.
 * Writes sorted_ids[0, npp), expert_ids[0, npp/BM) and *npp; capacities are checked. */
int oracle_align_block_size(const int32_t *ids, const int32_t *lora_ids, int64_t M,
                            int32_t topk, int32_t E, int32_t S, int32_t BM,
                            int32_t *sorted_ids, int64_t sorted_cap,
                            int32_t *expert_ids, int64_t expert_cap, int32_t *npp_out) {
    if (M < 0 || topk <= 0 || E <= 0 || S <= 0 || BM <= 0 || !npp_out) return OR_E_ARG;
    const int64_t numel = M * topk;
    const int64_t V = (int64_t)E * S;
    if (numel > 0 && !ids) return OR_E_ARG;

    int32_t *key = (int32_t *)malloc(sizeof(int32_t) * (size_t)(numel > 0 ? numel : 1));
    int64_t *count = (int64_t *)calloc((size_t)(V + 1), sizeof(int64_t));
    int64_t *offset = (int64_t *)malloc(sizeof(int64_t) * (size_t)(V + 1));
    int64_t *fill = (int64_t *)calloc((size_t)(V + 1), sizeof(int64_t));
    if (!key || !count || !offset || !fill) {
        free(key); free(count); free(offset); free(fill);
        return OR_E_ARG;
    }

    /* keys */
    for (int64_t p = 0; p < numel; ++p) {
        int32_t v = lora_ids ? virtual_id(ids[p], lora_ids[p / topk], E, S) : ids[p];
        key[p] = (v >= 0 && v < V) ? v : (int32_t)V;
        count[key[p]] += 1;
    }
    /* padded sizes and their exclusive prefix sum */
    int64_t total = 0;
    for (int64_t b = 0; b <= V; ++b) {
        offset[b] = total;
        total += (count[b] + BM - 1) / BM * BM;
    }
    int rc = OR_OK;
    if (total > sorted_cap || total / BM > expert_cap) {
        rc = OR_E_CAP;
    } else {
        /* padding entries first, then the pairs in ascending order: a stable sort */
        for (int64_t i = 0; i < total; ++i) sorted_ids[i] = (int32_t)numel;
        for (int64_t p = 0; p < numel; ++p) {
            int32_t b = key[p];
            sorted_ids[offset[b] + fill[b]] = (int32_t)p;
            fill[b] += 1;
        }
        /* one expert id per block; the sentinel bucket's blocks are -1 */
        for (int64_t b = 0; b <= V; ++b) {
            int64_t nblk = (count[b] + BM - 1) / BM;
            for (int64_t j = 0; j < nblk; ++j)
                expert_ids[offset[b] / BM + j] = (b == V) ? -1 : (int32_t)b;
        }
        *npp_out = (int32_t)total;
    }
    free(key); free(count); free(offset); free(fill);
    return rc;
}

/* ---- shrink ----------------------------------------------------------------------- */

/* For every real pair p of every aligned block with expert id e >= 0 (and, if
 * pair_mask is given, pair_mask[p] != 0):  s[p*R + i] = sum_k A[e][i][k] * xin[p/row_div][k],
 * k ascending, in double.  A is [V, R, K] row-major; xin rows are ld_x elements apart. */
/* Rank of LoRA slot l: slot_ranks[l] clamped to [0, r], or r when no ranks are given.
 * An adapter of rank rl uses the first rl rank dimensions of each slice of its weights;
 * rank 0 means no delta at all, like a pair with no adapter (MindLab sglang PR 24: the
 * lora_ranks table and its rank == 0 early return, which the "-1 guards" commit extends to
 * the -1 slot). */
static int32_t slot_rank(const int32_t *slot_ranks, int32_t slot, int32_t r) {
    if (!slot_ranks) return r;
    const int32_t v = slot_ranks[slot];
    return v < 0 ? 0 : (v > r ? r : v);
}

int oracle_lora_shrink(int dtype, const void *xin, int64_t ld_x, int32_t row_div,
                       const void *A, int32_t R, int32_t K,
                       const int32_t *sorted_ids, const int32_t *expert_ids, int32_t npp,
                       int64_t numel, int32_t BM, const uint8_t *pair_mask, double *s,
                       int32_t slices, const int32_t *slot_ranks, int32_t E) {
    if ((dtype != OR_F32 && dtype != OR_BF16) || R <= 0 || K <= 0 || BM <= 0 ||
        row_div <= 0 || ld_x < K || npp < 0 || npp % BM || slices <= 0 || R % slices ||
        E <= 0)
        return OR_E_ARG;
    const int32_t r = R / slices;
    const int64_t nblocks = npp / BM;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t blk = 0; blk < nblocks; ++blk) {
        const int32_t e = expert_ids[blk];
        if (e < 0) continue;
        const int32_t rl = slot_rank(slot_ranks, e / E, r);
        for (int32_t j = 0; j < BM; ++j) {
            const int64_t p = sorted_ids[blk * BM + j];
            if (p < 0 || p >= numel) continue;
            if (pair_mask && !pair_mask[p]) continue;
            const int64_t xrow = (p / row_div) * ld_x;
            for (int32_t i = 0; i < R; ++i) {
                if (i % r >= rl) {  /* past the adapter's rank in this slice */
                    s[p * R + i] = 0.0;
                    continue;
                }
                const int64_t arow = ((int64_t)e * R + i) * K;
                double acc = 0.0;
                for (int32_t k = 0; k < K; ++k)
                    acc += load_elem(A, arow + k, dtype) * load_elem(xin, xrow + k, dtype);
                s[p * R + i] = acc;
            }
        }
    }
    return OR_OK;
}

/* ---- expand ----------------------------------------------------------------------- */

/* For the same pairs:  d = scale[e / E] * sum_{j < rl} B[e][n][j] * s[p*R + g*r + j], j
 * ascending, with r = R/slices, g = n / (N/slices) and rl the slot's rank (r without
 * ranks; a slot of rank 0 gets no delta); then
 *   bf16: out[p][n] = round_bf16(out[p][n] + d)   (sum and rounding from double)
 *   f32:  out[p][n] = (float)(out[p][n] + d)
 * B is [V, N, r] row-major; out rows are ld_out elements apart. Every other row of out
 * is left untouched. */
int oracle_lora_expand(int dtype, const double *s, int32_t R, int32_t slices,
                       const void *B, int32_t N, const float *scale, int32_t E,
                       const int32_t *sorted_ids, const int32_t *expert_ids, int32_t npp,
                       int64_t numel, int32_t BM, const uint8_t *pair_mask,
                       void *out, int64_t ld_out, const int32_t *slot_ranks) {
    if ((dtype != OR_F32 && dtype != OR_BF16) || R <= 0 || slices <= 0 || R % slices ||
        N <= 0 || N % slices || E <= 0 || BM <= 0 || ld_out < N || npp < 0 || npp % BM)
        return OR_E_ARG;
    const int32_t r = R / slices;
    const int32_t width = N / slices;
    const int64_t nblocks = npp / BM;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t blk = 0; blk < nblocks; ++blk) {
        const int32_t e = expert_ids[blk];
        if (e < 0) continue;
        const double sc = (double)scale[e / E];
        const int32_t rl = slot_rank(slot_ranks, e / E, r);
        if (rl == 0) continue;  /* rank 0: no delta, rows untouched */
        for (int32_t j = 0; j < BM; ++j) {
            const int64_t p = sorted_ids[blk * BM + j];
            if (p < 0 || p >= numel) continue;
            if (pair_mask && !pair_mask[p]) continue;
            for (int32_t n = 0; n < N; ++n) {
                const int32_t g = n / width;
                const int64_t brow = ((int64_t)e * N + n) * r;
                double acc = 0.0;
                for (int32_t jj = 0; jj < rl; ++jj)
                    acc += load_elem(B, brow + jj, dtype) * s[p * R + (int64_t)g * r + jj];
                const double d = sc * acc;
                const int64_t o = p * ld_out + n;
                if (dtype == OR_F32) {
                    float *of = (float *)out;
                    of[o] = (float)((double)of[o] + d);
                } else {
                    uint16_t *ob = (uint16_t *)out;
                    ob[o] = oracle_bf16_from_double(bf16_to_double(ob[o]) + d);
                }
            }
        }
    }
    return OR_OK;
}

/* ---- combine ---------------------------------------------------------------------- */

static void store_rounded(int dtype, double v, void *y, int64_t o) {
    if (dtype == OR_F32) {
        ((float *)y)[o] = (float)v;
    } else {
        ((uint16_t *)y)[o] = oracle_bf16_from_double(v);
    }
}

/* y[m][n] = round( sum over k ascending with 0 <= t[m][k] < E of
 *                  w[m][k] * rows[m*topk + k][n] )
 * summed in double, rounded once (bf16 to nearest even, or to float). Rows of pairs with no
 * local expert are never read. rows are ld_rows elements apart, y rows ld_y. */
int oracle_moe_combine(int dtype, const void *rows, int64_t ld_rows, const int32_t *topk_ids,
                       const float *topk_weights, int64_t M, int32_t topk, int32_t E,
                       int32_t N, void *y, int64_t ld_y) {
    if ((dtype != OR_F32 && dtype != OR_BF16) || M < 0 || topk <= 0 || E <= 0 || N <= 0 ||
        ld_rows < N || ld_y < N)
        return OR_E_ARG;
    if (M > 0 && (!rows || !topk_ids || !topk_weights || !y)) return OR_E_ARG;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        for (int32_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int32_t k = 0; k < topk; ++k) {
                const int64_t p = m * topk + k;
                const int32_t t = topk_ids[p];
                if (t < 0 || t >= E) continue;  /* no local expert: no row */
                acc += (double)topk_weights[p] * load_elem(rows, p * ld_rows + n, dtype);
            }
            store_rounded(dtype, acc, y, m * ld_y + n);
        }
    }
    return OR_OK;
}

/* The down stage's expand fused with the combine (one slice, rank r = R):
 *   y[m][n] = round( sum over k ascending with 0 <= t < E of
 *                    w[m][k] * (base[p][n] + d_p[n]) ),   p = m*topk + k,
 * where d_p[n] = scale[l] * sum_{j < rl} B[v][n][j] * s[p*R + j] for a pair with a valid
 * virtual expert v = t + l*E (l = lora[m] in [0, S)) and slot rank rl > 0, else 0. Nothing
 * is rounded before the final sum. */
int oracle_lora_expand_combine(int dtype, const double *s, int32_t R, const void *B,
                               int32_t N, const float *scale, const int32_t *slot_ranks,
                               const int32_t *topk_ids, const int32_t *lora_ids,
                               const float *topk_weights, int64_t M, int32_t topk, int32_t E,
                               int32_t S, const void *base, int64_t ld_base, void *y,
                               int64_t ld_y) {
    if ((dtype != OR_F32 && dtype != OR_BF16) || R <= 0 || N <= 0 || M < 0 || topk <= 0 ||
        E <= 0 || S <= 0 || ld_base < N || ld_y < N)
        return OR_E_ARG;
    if (M > 0 && (!s || !B || !scale || !topk_ids || !lora_ids || !topk_weights || !base || !y))
        return OR_E_ARG;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        for (int32_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int32_t k = 0; k < topk; ++k) {
                const int64_t p = m * topk + k;
                const int32_t t = topk_ids[p];
                if (t < 0 || t >= E) continue;
                double row = load_elem(base, p * ld_base + n, dtype);
                const int32_t v = virtual_id(t, lora_ids[m], E, S);
                if (v >= 0) {
                    const int32_t l = v / E;
                    const int32_t rl = slot_rank(slot_ranks, l, R);
                    const int64_t brow = ((int64_t)v * N + n) * R;
                    double d = 0.0;
                    for (int32_t j = 0; j < rl; ++j) d += load_elem(B, brow + j, dtype) * s[p * R + j];
                    row += (double)scale[l] * d;
                }
                acc += (double)topk_weights[p] * row;
            }
            store_rounded(dtype, acc, y, m * ld_y + n);
        }
    }
    return OR_OK;
}

/* ---- base grouped GEMM, alone or with the LoRA delta in its epilogue ------------------ */

/* For every pair p with a local base expert t = topk_ids[p] (0 <= t < E):
 *   acc = sum_k W[t][n][k] * xin[(p / row_div) * ld_x + k]              (k ascending)
 *   if s != NULL and the token's slot l = lora_ids[p / topk] is in [0, S) and its rank
 *   rl > 0:  acc += scale[l] * sum_{j < rl} B[t + l*E][n][j] * s[p*R + g(n)*r + j]
 *   out[p][n] = round(acc)   (bf16 RNE from the double, or (float))
 * with r = R / slices and g(n) = n / (N / slices). W is [E, N, K], B is [E*S, N, r]. Rows of
 * pairs without a local expert are left untouched. */
int oracle_moe_gemm(int dtype, const void *xin, int64_t ld_x, int32_t row_div, const void *W,
                    int32_t K, int32_t N, const int32_t *topk_ids, int64_t M, int32_t topk,
                    int32_t E, void *out, int64_t ld_out, const double *s, int32_t R,
                    int32_t slices, const void *B, const float *scale,
                    const int32_t *slot_ranks, const int32_t *lora_ids, int32_t S) {
    if ((dtype != OR_F32 && dtype != OR_BF16) || K <= 0 || N <= 0 || M < 0 || topk <= 0 ||
        E <= 0 || row_div <= 0 || ld_x < K || ld_out < N)
        return OR_E_ARG;
    if (s && (R <= 0 || slices <= 0 || R % slices || N % slices || !B || !scale ||
              !lora_ids || S <= 0))
        return OR_E_ARG;
    const int64_t numel = M * topk;
    const int32_t r = s ? R / slices : 0;
    const int32_t width = s ? N / slices : N;
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t p = 0; p < numel; ++p) {
        const int32_t t = topk_ids[p];
        if (t < 0 || t >= E) continue;  /* no local expert: row untouched */
        const int64_t xrow = (p / row_div) * ld_x;
        int32_t v = -1, rl = 0, l = -1;
        if (s) {
            l = lora_ids[p / topk];
            v = virtual_id(t, l, E, S);
            rl = v >= 0 ? slot_rank(slot_ranks, l, r) : 0;
        }
        for (int32_t n = 0; n < N; ++n) {
            const int64_t wrow = ((int64_t)t * N + n) * K;
            double acc = 0.0;
            for (int32_t k = 0; k < K; ++k)
                acc += load_elem(W, wrow + k, dtype) * load_elem(xin, xrow + k, dtype);
            if (rl > 0) {
                const int32_t g = n / width;
                const int64_t brow = ((int64_t)v * N + n) * r;
                double d = 0.0;
                for (int32_t j = 0; j < rl; ++j)
                    d += load_elem(B, brow + j, dtype) * s[p * R + (int64_t)g * r + j];
                acc += (double)scale[l] * d;
            }
            store_rounded(dtype, acc, out, p * ld_out + n);
        }
    }
    return OR_OK;
}
