/*
 * mol.h - C ABI of the multi-LoRA MoE ("MoL", virtual experts) delta path on MI355X.
 *
 * One MoE layer with S LoRA adapters loaded into slots treats every (routed expert e,
 * slot l) combination as a "virtual expert" v = e + l*E, V = E*S of them. A layer pass is
 *   1. remap  - top-k base ids -> virtual ids (mol_virtual_topk, or inline in 2);
 *   2. align  - bucket the (token, slot) pairs by virtual expert into BLOCK_M-padded
 *               blocks (mol_align_block_size);
 *   3. delta  - per stage, shrink s = x A_v^T (hidden -> rank) and expand
 *               out += scale * s B_v^T (rank -> N) over the aligned blocks
 *               (mol_lora_shrink + mol_lora_expand, or fused: mol_lora_delta);
 *   4. combine - per token, the router-weighted sum of its down-stage rows
 *               (mol_moe_combine, or fused with the down expand: mol_lora_expand_combine).
 * Sources: the sglang virtual-experts kernels as summarised on the PR 24171 page
 * (remap keeping negative sentinels, sentinel bucket, -1 blocks skipped), the PR 24262
 * page (align as histogram -> prefix sum -> expert ids -> scatter, no host sync, the
 * 8192-bucket ceiling), and MindLab sglang PR 24 (shrink/expand stage shapes, weights
 * laid out [E, N, K] with N = shape[1], the "-1 = no adapter" slot contract).
 *
 * Conventions for every entry point:
 *  - Pointers are DEVICE pointers unless marked (host). The caller owns every buffer,
 *    including workspaces; the library keeps no device memory of its own.
 *  - Calls only validate host-side scalars and pointers, then enqueue kernels on
 *    `stream` (a hipStream_t; NULL = the legacy default stream) and return. No call
 *    allocates, synchronises, or reads device memory on the host, so a sequence of calls
 *    can be captured into a hipGraph.
 *  - Bad *device data* cannot be reported without a sync; it has defined behaviour
 *    instead: a base id >= E, a slot outside [0, S) and any negative id never reach a
 *    real virtual expert (they land in the sentinel bucket and get no delta).
 *  - Matrices are row-major; "ld" arguments are row strides in elements.
 *  - Returns MOL_OK or an error code; nothing is enqueued when an error is returned
 *    (except MOL_E_HIP, which reports a failed launch).
 */
#ifndef MOL_H
#define MOL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define MOL_API __attribute__((visibility("default")))
#else
#define MOL_API
#endif

typedef int32_t mol_status;

enum {
    MOL_OK = 0,
    MOL_E_ARG = 1,       /* NULL pointer, negative or zero size, inconsistent shapes   */
    MOL_E_LIMIT = 2,     /* more than MOL_MAX_BUCKETS buckets, rank or block too large */
    MOL_E_DTYPE = 3,     /* unknown dtype                                              */
    MOL_E_ALIGN = 4,     /* a row, stride or base pointer not 16-byte aligned          */
    MOL_E_WORKSPACE = 5, /* workspace missing or smaller than the size query says      */
    MOL_E_HIP = 6        /* a HIP call or kernel launch failed                         */
};

enum { MOL_F32 = 0, MOL_BF16 = 1 };

/* At most 8192 buckets = 8191 virtual experts + the sentinel bucket (the align kernel
 * ceiling on the PR 24262 page). */
#define MOL_MAX_BUCKETS 8192
#define MOL_MAX_BLOCK_M 1024
/* expand: r * sizeof(elem) <= 256 bytes (rank <= 128 in bf16, <= 64 in fp32) */
#define MOL_MAX_RANK_BYTES 256
/* floats of the library's own per-GPU scratch behind mol_lora_delta_noalloc (16 MiB) */
#define MOL_DELTA_SCRATCH_FLOATS (4 * 1024 * 1024)

/* (host) Static description of a status code. Never NULL. */
MOL_API const char *mol_status_string(mol_status status);

/* (host) ABI version of this header, 7 (2 added the per-slot ranks, 3 the combine, 4 the
 * base grouped GEMM with the fused delta, 5 the allocation-free stage delta, 6 the work
 * plan, 7 the plan as runs of blocks only, read by the expand). */
MOL_API int32_t mol_abi_version(void);

/* ---------------------------------------------------------------------------------
 * mol_virtual_topk - remap base top-k ids to virtual ids (PR 24171 page: the fused
 * virtual top-k ids kernel keeps a negative id and shifts the others by slot * E).
 *   topk_ids     int32 [M, topk]   base expert ids; negative = expert-parallel sentinel
 *   lora_ids     int32 [M]         LoRA slot per token; -1 = no adapter
 *   virtual_ids  int32 [M, topk]   out: t if t < 0; -1 if t >= E or slot outside [0, S);
 *                                  else t + slot * E. May not alias the inputs.
 * M == 0 is valid and enqueues nothing. Errors: MOL_E_ARG.
 * ------------------------------------------------------------------------------- */
MOL_API mol_status mol_virtual_topk(const int32_t *topk_ids, const int32_t *lora_ids,
                                    int32_t M, int32_t topk, int32_t num_experts,
                                    int32_t num_slots, int32_t *virtual_ids, void *stream);

/* ---------------------------------------------------------------------------------
 * Align sizing (host, pure). num_virtual = V = E * S.
 *   mol_align_max_blocks: an upper bound on the number of BLOCK_M blocks any routing
 *     of `numel` pairs can produce, cdiv(numel + min(numel, V+1) * (block_m - 1),
 *     block_m). sorted_ids needs max_blocks * block_m entries, expert_ids max_blocks.
 *   mol_align_workspace_bytes: device workspace mol_align_block_size needs (0 when the
 *     one-workgroup kernel handles numel).
 * Both return a negative -mol_status on invalid arguments (e.g. -MOL_E_LIMIT when
 * V + 1 > MOL_MAX_BUCKETS).
 * ------------------------------------------------------------------------------- */
MOL_API int64_t mol_align_max_blocks(int64_t numel, int32_t num_virtual, int32_t block_m);
MOL_API int64_t mol_align_workspace_bytes(int64_t numel, int32_t num_virtual, int32_t block_m);

/* ---------------------------------------------------------------------------------
 * The work plan (optional). A batch of at least 4096 pairs and 8 pairs per bucket on average
 * (numel >= 8 (V + 1)) is dense enough for the bf16 matrix-core kernels, which then take
 * every block (no VALU kernel is launched). For such a batch, mol_align_block_size can write
 * beside the routing a plan of its blocks: runs of up to four consecutive blocks of one
 * virtual expert, every block of a real bucket in exactly one run. The expand then takes
 * whole runs as work items and loads each weight column once per run instead of once per
 * block. For other batches nothing is written and the calls ignore a plan. Layout (int32
 * words): [0] the number of runs, [1..7] 0; from word 8, runs of 4 words {first block,
 * blocks (1..4), virtual expert, 0} in bucket order, at most min(max_blocks, numel). The
 * sentinel bucket has none.
 *   mol_plan_bytes: bytes of a plan buffer (a multiple of 256), or -mol_status.
 * ------------------------------------------------------------------------------- */
MOL_API int64_t mol_plan_bytes(int64_t numel, int32_t num_virtual, int32_t block_m);

/* ---------------------------------------------------------------------------------
 * mol_align_block_size - bucket the numel = M * topk pairs by virtual expert (PR 24262
 * page: histogram, padded prefix sum, per-block expert ids, token scatter; PR 24171
 * page: the extra sentinel bucket whose blocks are -1).
 *   ids            int32 [M, topk]  base ids (lora_ids != NULL: remapped inline exactly
 *                                   as mol_virtual_topk) or virtual ids (lora_ids == NULL)
 *   lora_ids       int32 [M] or NULL
 *   Bucket of a pair = its virtual id if in [0, V), else V (the sentinel bucket, last).
 *   With c_b pairs in bucket b, pc_b = ceil(c_b / block_m) * block_m and off_b the
 *   exclusive prefix sum of pc:
 *   sorted_ids       int32 [max_blocks * block_m] out: sorted_ids[off_b + j] = the j-th
 *                    pair of bucket b in ascending pair order (j < c_b); entries
 *                    [off_b + c_b, off_b + pc_b) = numel (padding).
 *   expert_ids       int32 [max_blocks] out: block i in [off_b, off_b + pc_b)/block_m
 *                    gets b, or -1 for the sentinel bucket.
 *   num_post_padded  int32 [1] out: sum_b pc_b.
 *   Entries past num_post_padded (resp. num_post_padded / block_m) are left undefined.
 *   plan, plan_bytes the work plan out (see above; 16-byte aligned, at least
 *                    mol_plan_bytes()), or NULL (0). Written only for a batch that takes
 *                    the matrix-core kernels; the buffer is left untouched otherwise.
 *   workspace        device scratch of mol_align_workspace_bytes(), or NULL when that is 0.
 * No atomics are used; results are bit-for-bit reproducible. M == 0 writes
 * num_post_padded = 0 (sorted_ids and expert_ids may then be NULL).
 * Errors: MOL_E_ARG, MOL_E_LIMIT (V + 1 > MOL_MAX_BUCKETS, block_m > MOL_MAX_BLOCK_M),
 * MOL_E_WORKSPACE, MOL_E_HIP.
 * ------------------------------------------------------------------------------- */
MOL_API mol_status mol_align_block_size(const int32_t *ids, const int32_t *lora_ids,
                                        int32_t M, int32_t topk, int32_t num_experts,
                                        int32_t num_slots, int32_t block_m,
                                        int32_t *sorted_ids, int32_t *expert_ids,
                                        int32_t *num_post_padded, int32_t *plan,
                                        size_t plan_bytes, void *workspace,
                                        size_t workspace_bytes, void *stream);

/* ---------------------------------------------------------------------------------
 * Per-slot ranks (all three delta calls). slot_ranks, int32 [num_virtual / num_experts] or
 * NULL, gives the rank rl of each LoRA slot (MindLab sglang PR 24: the lora_ranks table and
 * its rank == 0 early return): an adapter of rank rl uses rank dimensions [0, rl) of each
 * slice of its weights, r = R / slices. Values are clamped to [0, r]; NULL means every slot
 * has rank r. Weights past a slot's rank are never read, whatever they hold.
 * ------------------------------------------------------------------------------- */

/* ---------------------------------------------------------------------------------
 * mol_lora_shrink - s[p, i] = sum_k A[v, i, k] * xin[p / row_div, k] for every real pair
 * p of every block with expert id v >= 0 (MindLab sglang PR 24: the MoL shrink stage,
 * hidden -> rank). fp32 accumulation.
 *   dtype        MOL_F32 or MOL_BF16 (xin and A)
 *   xin          [rows, ld_x] input rows; pair p reads row p / row_div (row_div = topk
 *                for token rows, 1 for per-pair rows)
 *   A            [V, R, K] weights, rows of K contiguous elements
 *   slices       R = slices * r; slice g holds rank dimensions [g r, g r + r)
 *   slot_ranks, num_experts: the per-slot ranks above (slot of v = v / num_experts);
 *                s[p, g r + i] = 0 for i >= rl
 *   sorted_ids, expert_ids, num_post_padded: the outputs of mol_align_block_size for
 *                `numel` pairs, V = num_virtual virtual experts and this block_m
 *   s            float32 [numel, R] out, 16-byte aligned; rows of pairs that get no delta are
 *                untouched
 * Requires K * elem and ld_x * elem to be multiples of 16 bytes, R % slices == 0, and xin,
 * A, s 16-byte aligned (MOL_E_ALIGN). numel == 0 enqueues nothing.
 * ------------------------------------------------------------------------------- */
MOL_API mol_status mol_lora_shrink(int32_t dtype, const void *xin, int64_t ld_x,
                                   int32_t row_div, const void *A, int32_t R, int32_t K,
                                   int32_t slices, const int32_t *slot_ranks,
                                   int32_t num_experts, const int32_t *sorted_ids,
                                   const int32_t *expert_ids, const int32_t *num_post_padded,
                                   int32_t numel, int32_t num_virtual, int32_t block_m,
                                   float *s, void *stream);

/* ---------------------------------------------------------------------------------
 * mol_lora_expand - for the same pairs, with r = R / slices, w = N / slices and rl the
 * slot's rank,
 *   out[p, n] = round(out[p, n] + slot_scale[v / E] * sum_{j < rl} B[v, n, j] * s[p, (n / w) * r + j])
 * (MindLab sglang PR 24: expand rank -> N; gate_up expands as two slices, gate from
 * s[:, :r] and up from s[:, r:]). Sum in fp32, one fused multiply-add into the fp32 value
 * of out, then round to nearest even for bf16. A slot of rank 0 adds nothing.
 *   s            float32 [numel, R] from mol_lora_shrink, 16-byte aligned
 *   B            [V, N, r] weights (dtype as out)
 *   slot_scale   float32 [num_virtual / num_experts]
 *   slot_ranks   int32 [num_virtual / num_experts] or NULL (see above)
 *   out          [numel, ld_out] read and written in place; rows of pairs without a
 *                delta are left bit-for-bit untouched
 *   plan         the work plan the same align call wrote, or NULL. When the matrix-core
 *                kernels take the batch, their items are then the plan's runs (same
 *                results); otherwise it is not read. (mol_lora_delta and
 *                mol_lora_delta_noalloc take the same argument for their expand.)
 * Requires R % slices == 0, N % slices == 0, r * elem a multiple of 16 bytes and at most
 * MOL_MAX_RANK_BYTES, B and s 16-byte aligned (MOL_E_ALIGN), out aligned to its element.
 * ------------------------------------------------------------------------------- */
MOL_API mol_status mol_lora_expand(int32_t dtype, const float *s, int32_t R, int32_t slices,
                                   const void *B, int32_t N, const float *slot_scale,
                                   const int32_t *slot_ranks, int32_t num_experts,
                                   const int32_t *sorted_ids, const int32_t *expert_ids,
                                   const int32_t *num_post_padded, const int32_t *plan,
                                   int32_t numel, int32_t num_virtual, int32_t block_m,
                                   void *out, int64_t ld_out, void *stream);

/* ---------------------------------------------------------------------------------
 * mol_lora_delta - one stage: shrink then expand, with s kept in the caller's workspace.
 * Same arguments and results as mol_lora_shrink followed by mol_lora_expand (bit-identical
 * to them; they are the same kernels, enqueued back to back).
 *   workspace    device scratch of at least mol_delta_workspace_bytes(), 16-byte aligned;
 *                no initial contents are required. Calls that may overlap must not share
 *                a workspace.
 * ------------------------------------------------------------------------------- */
MOL_API int64_t mol_delta_workspace_bytes(int32_t numel, int32_t R, int32_t num_virtual,
                                          int32_t block_m);
MOL_API mol_status mol_lora_delta(int32_t dtype, const void *xin, int64_t ld_x,
                                  int32_t row_div, const void *A, int32_t R, int32_t K,
                                  int32_t slices, const void *B, int32_t N,
                                  const float *slot_scale, const int32_t *slot_ranks,
                                  int32_t num_experts, const int32_t *sorted_ids,
                                  const int32_t *expert_ids, const int32_t *num_post_padded,
                                  const int32_t *plan, int32_t numel, int32_t num_virtual,
                                  int32_t block_m, void *out, int64_t ld_out, void *workspace,
                                  size_t workspace_bytes, void *stream);

/* ---------------------------------------------------------------------------------
 * mol_lora_delta_noalloc - mol_lora_delta for callers that cannot allocate device memory
 * (code under hipGraph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same checks, kernels and results (bit-identical), but s lives in a scratch array that the
 * library itself holds on each GPU, so no workspace is passed and nothing is allocated.
 *   Limit: numel * R <= MOL_DELTA_SCRATCH_FLOATS (16 MiB of float32), else MOL_E_LIMIT
 *          before anything is enqueued. The scratch needs no initial contents.
 *   Every call on one GPU shares that GPU's scratch and leaves its contents behind: calls
 *   that may overlap on one GPU (other streams, other threads) race and must not be made.
 *   The first call on a device looks up the scratch's address there (no allocation); a
 *   failure of that lookup returns MOL_E_HIP. Other errors as for mol_lora_delta.
 * ------------------------------------------------------------------------------- */
MOL_API mol_status mol_lora_delta_noalloc(int32_t dtype, const void *xin, int64_t ld_x,
                                          int32_t row_div, const void *A, int32_t R,
                                          int32_t K, int32_t slices, const void *B, int32_t N,
                                          const float *slot_scale, const int32_t *slot_ranks,
                                          int32_t num_experts, const int32_t *sorted_ids,
                                          const int32_t *expert_ids,
                                          const int32_t *num_post_padded,
                                          const int32_t *plan, int32_t numel,
                                          int32_t num_virtual, int32_t block_m, void *out,
                                          int64_t ld_out, void *stream);

/* ---------------------------------------------------------------------------------
 * mol_moe_gemm - the base MoE grouped GEMM of a stage, with the LoRA delta optionally fused
 * into its epilogue. The pages' layer runs the base grouped-GEMM launches and then the LoRA
 * launches that add the delta into the same rows (MindLab sglang PR 24, the PR body's count
 * of base and LoRA launches per layer); fused, the rows are written once:
 *   out[p, n] = round( sum_k W[t, n, k] * xin[p / row_div, k]
 *                      + slot_scale[l] * sum_{j < rl} B[t + l*E, n, j] * s[p, (n / w) * r + j] )
 * for every pair p with a local base expert t = topk id in [0, E) (other rows untouched),
 * with l the token's slot (lora_ids[p / topk]; the delta term only for l in [0, S) and slot
 * rank rl > 0), r = R / slices, w = N / slices. Summed in fp32, rounded once (bf16 RNE).
 *   sorted_ids, expert_ids, num_post_padded
 *                 the routing by BASE expert: mol_align_block_size over the top-k ids with
 *                 lora_ids = NULL and num_slots = 1 (num_virtual = num_experts)
 *   W             [E, N, K] base weights (dtype), 16-byte aligned, K * elem a multiple of 16
 *   xin           rows of ld_x elements (16-byte multiple), row p / row_div for pair p
 *   out           [numel, ld_out] (dtype), aligned to its element
 *   s             NULL: the base GEMM alone. Else the fused delta: float32 [numel, R] from
 *                 mol_lora_shrink of the same stage (16-byte aligned), B [E*S, N, r] (dtype,
 *                 16-byte aligned), slot_scale [S], slot_ranks [S] or NULL, lora_ids [numel /
 *                 topk]; r * elem a multiple of 16 and at most MOL_MAX_RANK_BYTES
 * Built for decode-sized batches (a gather of matrix-vector products over the touched
 * experts' weights, like the shrink). Errors as for mol_lora_shrink / mol_lora_expand.
 * ------------------------------------------------------------------------------- */
MOL_API mol_status mol_moe_gemm(int32_t dtype, const void *xin, int64_t ld_x, int32_t row_div,
                                const void *W, int32_t K, int32_t N, int32_t num_experts,
                                const int32_t *sorted_ids, const int32_t *expert_ids,
                                const int32_t *num_post_padded, int32_t numel, int32_t block_m,
                                void *out, int64_t ld_out, const float *s, int32_t R,
                                int32_t slices, const void *B, const float *slot_scale,
                                const int32_t *slot_ranks, const int32_t *lora_ids,
                                int32_t topk, int32_t num_slots, void *stream);

/* ---------------------------------------------------------------------------------
 * The combine after the down projection. The pages stop at the per-pair rows the down
 * stage's delta is added into (the layer's grouped-GEMM launches counted on the MindLab
 * sglang PR 24 page end with the down expand); the next step of an MoE layer sums each
 * token's pair rows with its router weights. A pair whose base id is outside [0, E) has no
 * local expert (a negative id is an expert-parallel sentinel: the expert lives on another
 * GPU) and contributes nothing; its row is never read.
 *
 * mol_moe_combine -
 *   y[m, n] = round( sum_{k ascending, 0 <= topk_ids[m, k] < E} w[m, k] * rows[m*topk + k, n] )
 * summed in fp32 and rounded once (bf16: to nearest even).
 *   rows          [M*topk, ld_rows] pair rows (dtype), e.g. the down stage's out
 *   topk_ids      int32 [M, topk] base expert ids
 *   topk_weights  float32 [M, topk] router weights
 *   y             [M, ld_y] out (dtype); every element of [M, N] is written
 * Requires N, ld_rows and ld_y multiples of 16 bytes' worth of elements (8 bf16, 4 fp32)
 * and rows, y 16-byte aligned (MOL_E_ALIGN). M = 0 is a no-op.
 * ------------------------------------------------------------------------------- */
MOL_API mol_status mol_moe_combine(int32_t dtype, const void *rows, int64_t ld_rows,
                                   const int32_t *topk_ids, const float *topk_weights,
                                   int32_t M, int32_t topk, int32_t num_experts, int32_t N,
                                   void *y, int64_t ld_y, void *stream);

/* ---------------------------------------------------------------------------------
 * mol_lora_expand_combine - the down stage's expand (one slice) fused with the combine;
 * the per-pair rows are never written:
 *   y[m, n] = round( sum_{k, 0 <= t < E} w[m, k] * (base[p, n] + d_p[n]) ),  p = m*topk + k,
 *   d_p[n]  = slot_scale[l] * sum_{j < rl} B[v, n, j] * s[p, j]
 * for a pair whose token has slot l in [0, S) (virtual expert v = t + l*E, slot rank rl >
 * 0); otherwise d_p = 0. Summed in fp32, rounded once. It reads each pair's B_v columns,
 * which at decode (almost every pair its own virtual expert) are the same bytes the aligned
 * expand reads; with many tokens per virtual expert (prefill) mol_lora_expand followed by
 * mol_moe_combine reads far fewer.
 *   s             float32 [M*topk, R] from mol_lora_shrink of the down stage, 16-byte
 *                 aligned; rows of pairs without a delta are not read
 *   B             [E*S, N, R] (dtype), 16-byte aligned
 *   slot_scale    float32 [S];  slot_ranks  int32 [S] or NULL (clamped to [0, R])
 *   lora_ids      int32 [M] LoRA slot per token (-1: no adapter, base row only)
 *   base          [M*topk, ld_base] the pairs' base rows (read only)
 *   y             [M, ld_y] out
 * Requires R * elem a multiple of 16 bytes with R / (16 / elem) a power of two up to 16
 * (bf16 ranks 8..128, fp32 ranks 4..64; else MOL_E_LIMIT), E*S + 1 <= MOL_MAX_BUCKETS.
 * ------------------------------------------------------------------------------- */
MOL_API mol_status mol_lora_expand_combine(int32_t dtype, const float *s, int32_t R,
                                           const void *B, int32_t N, const float *slot_scale,
                                           const int32_t *slot_ranks, const int32_t *topk_ids,
                                           const int32_t *lora_ids,
                                           const float *topk_weights, int32_t M, int32_t topk,
                                           int32_t num_experts, int32_t num_slots,
                                           const void *base, int64_t ld_base, void *y,
                                           int64_t ld_y, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MOL_H */
