/*
 * amla.h — C ABI of the folded split-KV absorbed-MLA decode for AMD MI355X (gfx950).
 *
 * The operation (page "vllm.models.kimi_k3.nvidia.specialized_decode.drafter.attention",
 * module docstring; page "...cutedsl.mla.balanced", module docstring):
 *
 *   Absorbed MLA decode is MQA over a single latent KV head.  A speculative draft block of
 *   k query tokens per request is non-causal: every token sees the request's whole cache.
 *   The k tokens are folded into the head axis, q [R*k, H, 576] viewed as [R, k*H, 576]
 *   (row i = t*H + h), so each request's paged FP8 latent cache is read once instead of
 *   k times.  Each request's keys are split into a planned number of chunks; each chunk
 *   yields FP32 partials plus a log2 LSE; a reducer merges them into BF16 out
 *   [R, k*H, 512] and FP32 log2 LSE [R, k*H], the same memory order as the stock
 *   [R*k, H, 512] / [R*k, H].
 *
 * Fixed geometry: pages of 64 tokens; a token row is 576 bytes of float8 E4M3FN (OCP),
 * the 512 latent dims first, then the 64 rope dims; the value is the 512 latent dims.
 *
 * Calling convention for every entry point:
 *   - pointers named d_* are device pointers, owned by the caller;
 *   - the library never allocates device memory, never synchronises and keeps no global
 *     state (except the static device scratch of amla_folded_decode_noalloc); all work is
 *     enqueued on `stream` (a hipStream_t, NULL = the null stream), so the calls can be
 *     captured into a HIP graph;
 *   - the return value is AMLA_OK (0) or a negative AMLA_ERR_* code; on error nothing has
 *     been enqueued;
 *   - values that only live on the device (lengths, block-table entries, the work list)
 *     are checked by the kernels, which record a nonzero code in the workspace's device
 *     status word (int32 at byte AMLA_WS_STATUS of the workspace) and skip the bad work
 *     instead of reading out of bounds.
 */
#ifndef AMLA_H
#define AMLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define AMLA_PAGE 64          /* tokens per cache page */
#define AMLA_KDIM 576         /* bytes (E4M3 codes) per token row: 512 latent + 64 rope */
#define AMLA_VDIM 512         /* value dims: the latent part */
#define AMLA_UVDIM 128        /* output dims per head of the W_UV up-projection */
#define AMLA_MAX_ROWS 1024    /* most folded rows per request (k*H) */
#define AMLA_MAX_REQS 4096    /* most requests one plan takes */
#define AMLA_MAX_SPLITS 256   /* most splits per request */
#define AMLA_MAX_SPLIT_COST 4096  /* largest split_cost_pages */
#define AMLA_SPLIT_COST_ONE_TILE 8    /* measured split cost when a split is one row tile */
#define AMLA_SPLIT_COST_MULTI_TILE 4  /* measured split cost when a split has several tiles */

#define AMLA_MAX_SOURCES 64   /* most DCP sources amla_merge_sources takes */

/* Host status codes. */
#define AMLA_OK 0
#define AMLA_ERR_INVALID (-1)   /* null pointer, size or parameter out of range */
#define AMLA_ERR_WORKSPACE (-2) /* workspace smaller than amla_workspace_bytes() */
#define AMLA_ERR_LIST (-3)      /* list_len < 2 * (num_reqs + 2 * workers) */
#define AMLA_ERR_HIP (-4)       /* a kernel launch failed */

/* Device status word (int32 at byte AMLA_WS_STATUS of the workspace), bit flags. */
#define AMLA_WS_STATUS 0
#define AMLA_DEV_BAD_LENGTH 1   /* plan: a length < 0 or more pages than table columns;
                                   the plan is then empty (every count 0) */
#define AMLA_DEV_BAD_PAGE 2     /* decode: a block-table entry outside [0, pool_pages) */
#define AMLA_DEV_BAD_ITEM 4     /* decode: a work item or plan that does not match the call */
#define AMLA_DEV_BAD_POSITION 8 /* query build: a position outside the rotary table (row 0
                                   used instead) */

/* Split-plan modes (page "...cutedsl.mla.balanced", module docstring). */
#define AMLA_PLAN_BALANCED 0    /* split counts planned from the lengths */
#define AMLA_PLAN_FIXED 1       /* every request in the same number of chunks */

/*
 * Plan / decode parameters; one value of this struct must be used for a plan and for the
 * decode and combine calls that consume it.
 *   rows_per_req      M = folded rows per request (k*H after folding), 1..AMLA_MAX_ROWS
 *   mtile             MT = rows per decode work unit: 32, 64 or 128
 *   workers           W = persistent decode workgroups (normally one per compute unit)
 *   min_split_tokens  no split is planned shorter than this (rounded up to pages), >= 0
 *   max_splits        most splits per request, 1..AMLA_MAX_SPLITS
 *   mode              AMLA_PLAN_BALANCED or AMLA_PLAN_FIXED
 *   split_cost_pages  BALANCED: what one split costs its worker beyond its pages (loading
 *                     its query rows, writing its partials), in pages, 0..AMLA_MAX_SPLIT_COST;
 *                     this library's measured figures for gfx950: AMLA_SPLIT_COST_ONE_TILE
 *                     when M <= MT (one worker per split), AMLA_SPLIT_COST_MULTI_TILE
 *                     otherwise
 */
typedef struct amla_plan_params {
    int32_t rows_per_req;
    int32_t mtile;
    int32_t workers;
    int32_t min_split_tokens;
    int32_t max_splits;
    int32_t mode;
    int32_t split_cost_pages;
} amla_plan_params;

/*
 * Fold plan of a decode batch (host only, no device work).
 * Page "drafter.attention", sections foldable and fold_plan.
 *   k_out:    query tokens per request when the batch folds, else 0: the batch must be
 *             non-causal, num_rows == num_decode_tokens, num_rows divisible by
 *             num_reqs with k >= 2, at least num_reqs block-table rows, and
 *             max_query_len == k.
 *   fold_out: tokens folded into one decode row (0 when k_out is 0): k without an LSE;
 *             with one, the largest divisor f of k with f*heads <= max_fold_heads.
 * Returns AMLA_ERR_INVALID for null outputs, heads < 1 or max_fold_heads < heads
 * when an LSE is needed.
 */
int amla_fold_plan(int32_t causal, int32_t num_reqs, int32_t num_rows,
                   int32_t num_decode_tokens, int32_t block_table_rows,
                   int32_t max_query_len, int32_t heads, int32_t need_lse,
                   int32_t max_fold_heads, int32_t *k_out, int32_t *fold_out);

/*
 * Scale composition of the stock decode for an FP8 cache (host only).
 * Page "drafter.attention", section _scales: bmm1 = softmax_scale * q_scale * k_scale,
 * bmm2 = k_scale.  Outputs in dequantised value units.
 */
int amla_bmm_scales(float softmax_scale, float q_scale, float k_scale,
                    float *bmm1_out, float *bmm2_out);

/*
 * Decode launch shape for a device (host only).  No passage of the pages fixes it: this is
 * the library's own choice for gfx950 (the pages' counterpart, the worker count of the
 * balanced core's persistent launch, page "...cutedsl.mla.balanced", module docstring, is
 * a property of their GPU).  The pages' device query becomes an argument so that a plan
 * can be reproduced off the device.
 *   compute_units  CUs of the device (hipDeviceProp_t::multiProcessorCount), >= 1
 *   rows_per_req   M, 1..AMLA_MAX_ROWS
 *   workers_out    = compute_units: one persistent workgroup per CU
 *   mtile_out      rows per work unit: 32 for M <= 32, 64 for M <= 64; above, 128 unless
 *                  64-row tiles leave fewer padding rows in a request's last tile (measured on
 *                  gfx950: M = 448, 7 tiles of 64 rows against 3.5 of 128, decodes 10-15 %
 *                  faster on 64-row tiles; M = 256 alike on both)
 * Returns AMLA_ERR_INVALID for null outputs or arguments out of range.
 */
int amla_decode_config(int32_t compute_units, int32_t rows_per_req,
                       int32_t *workers_out, int32_t *mtile_out);

/*
 * D512 bands per row for the reducer (host only).  Page "...cutedsl.mla.balanced",
 * section reducer_d_tiles: 2 when ceil(2*rows/units) < 2*ceil(rows/units), else 1.
 */
int amla_reducer_bands(int32_t rows, int32_t compute_units, int32_t *bands_out);

/*
 * Workspace bytes for up to num_reqs requests (host only).  Precedent: page
 * "drafter.attention", tier_workspace_bytes (the split-KV workspace is sized on the host
 * from the batch shape before any launch, so it can be allocated once, ahead of graph
 * capture); the layout is the library's own: a 256-byte header (device status, plan
 * summary), then FP32 partials [num_reqs + 2 * workers][rows_per_req][512] and FP32 log2
 * LSE [num_reqs + 2 * workers][rows_per_req] (every plan has fewer than
 * num_reqs + workers splits).  The caller allocates and owns the workspace.
 * Returns 0 for arguments out of range.
 */
size_t amla_workspace_bytes(int32_t num_reqs, int32_t rows_per_req, int32_t workers);

/*
 * Plan the splits of one decode step from the KV lengths (one kernel, one workgroup).
 * Page "...cutedsl.mla.balanced", module docstring and BalancedMla.plan: split counts are
 * planned on the device from this step's lengths, once per step, and reused by every
 * layer's decode.
 *   d_lengths  int32 [num_reqs]: keys per request, including the draft block
 *   bt_cols    columns of the block table (pages a request may have)
 *   d_counts   int32 [num_reqs]  out: splits per request (0 for an empty request)
 *   d_offsets  int32 [num_reqs+1] out: exclusive prefix sum of the counts; item (and
 *              workspace slot) offsets[r] + s is split s of r; offsets[num_reqs] = N items
 *   d_work     int32 [list_len] out: item i as (request, first page) at [2i, 2i+1], items in
 *              request order, splits of a request in page order; -1 up to 2 * (R + W); then
 *              at 2 * (R + W) + g the first item of worker group g (g = 0..G, entry G = N),
 *              G = max(1, W / mt); then -1.  Item i ends where item i+1 starts if that is of
 *              the same request, else at the request's last page.
 *   list_len   >= 2 * (num_reqs + 2 * workers)
 *   d_workspace / ws_bytes: the workspace (header written here)
 * The split rule (the pages leave it open; this is the library's reading): pages_r =
 * ceil(L_r/64), P = sum_r pages_r, mt = ceil(M/MT) row tiles per split, one worker per tile:
 * worker group g is workers [g*mt, (g+1)*mt).  minp = max(1, ceil(min_split_tokens/64)),
 * a = split_cost_pages.  BALANCED: every non-empty request is laid out as a head of a pages
 * and its pages_r pages, the requests end to end (request r from voff_r, V in all), and V
 * is cut into Gp = min(G, max_splits, max(1, floor(V/minp))) ranges at c_g = floor(g*V/Gp).
 * A cut strictly inside request r at page x = c_g - voff_r - a of it (negative in the
 * head) moves to the request's start if x < minp, to its end if pages_r - x < minp, else
 * cuts r at page x.  The splits of r start at page 0 and at each cut left inside it; group
 * g takes the items starting in [C_g, C_{g+1}) of the moved cuts (a request's first item
 * starts at its head; groups g >= Gp take none), so every group costs about V/Gp.
 * FIXED: count_r = min(pages_r, clamp(floor(W/(R*mt)), 1, max_splits)) splits, split s with
 * q + (s < rem) pages from page s*q + min(s, rem), q = pages_r / count_r, rem = pages_r %
 * count_r; group g takes items [floor(g*N/G), floor((g+1)*N/G)).
 */
int amla_plan_splits(const int32_t *d_lengths, int32_t num_reqs, int32_t bt_cols,
                     const amla_plan_params *params, int32_t *d_counts, int32_t *d_offsets,
                     int32_t *d_work, int32_t list_len, void *d_workspace, size_t ws_bytes,
                     void *stream);

/*
 * Folded split-KV decode: one persistent kernel of `workers` workgroups; each worker group
 * walks its items of the planned work list; every (request, split, row tile) stages its
 * pages in LDS, computes S = Q K^T
 * and O += P V on FP8 MFMA with an online softmax, and writes FP32 partials and the log2
 * LSE of its split into the workspace.  Page "...cutedsl.mla.balanced", module docstring
 * (FP32 split partials; the row max is kept lazily and P is fed to the MMA as E4M3).
 *   d_q          E4M3 [num_reqs][rows_per_req][576], row i = t*H + h
 *   d_kv         E4M3 [pool_pages][64][576]
 *   d_block_table int32 [num_reqs][bt_stride]; entries for pages [0, ceil(L_r/64)) must
 *                be in [0, pool_pages) (others are never read)
 *   d_lengths    int32 [num_reqs] (the lengths the plan was made from)
 *   bmm1_scale   softmax_scale * q_scale * k_scale (finite, > 0);  bmm2_scale  k_scale
 *   d_counts, d_offsets, d_work, list_len: the plan of amla_plan_splits with `params`
 */
int amla_folded_decode(const uint8_t *d_q, const uint8_t *d_kv, int64_t pool_pages,
                       const int32_t *d_block_table, int32_t bt_stride,
                       const int32_t *d_lengths, int32_t num_reqs,
                       const amla_plan_params *params, float bmm1_scale, float bmm2_scale,
                       const int32_t *d_counts, const int32_t *d_offsets,
                       const int32_t *d_work, int32_t list_len, void *d_workspace,
                       size_t ws_bytes, void *stream);

/*
 * Decode context parallelism (page "...cutedsl.mla.balanced", module docstring and
 * BalancedMla.decode: under DCP the decode reads this rank's KV shard, masks causally in
 * global positions from the requests' global lengths, and returns the log2 LSE the head
 * owner merges; page "drafter.attention", DraftDcp).  A rank holds the global positions p
 * with (p / interleave) % world == rank, in global order: local position
 * (p / (interleave * world)) * interleave + p % interleave.
 *   heads       H: folded row i = t*H + h is draft token t = i / H (rows_per_req % H == 0)
 *   causal      0: every row sees the rank's whole shard (the draft block is non-causal);
 *               1: token t of a request of `total` global keys sits at position
 *               total - k + t (k = rows_per_req / H) and sees the positions up to it
 *   world, rank, interleave: the shard, 0 <= rank < world, interleave >= 1,
 *               interleave * world <= 2^30
 */
typedef struct amla_dcp_params {
    int32_t heads;
    int32_t causal;
    int32_t world;
    int32_t rank;
    int32_t interleave;
} amla_dcp_params;

/*
 * amla_folded_decode over one rank's KV shard: d_lengths are the local lengths (keys of
 * the shard, what the plan was made from), d_block_table the shard's pages, d_totals int32
 * [num_reqs] the global lengths (needed when causal; may be NULL otherwise).  A row that
 * sees none of a split's keys gets partial 0 and LSE -inf.  The device status word gets
 * AMLA_DEV_BAD_LENGTH when a local length is not the shard's share of its total.
 * AMLA_ERR_INVALID for a NULL dcp, out-of-range fields, or causal without d_totals; the
 * other arguments and errors are those of amla_folded_decode.
 */
int amla_folded_decode_dcp(const uint8_t *d_q, const uint8_t *d_kv, int64_t pool_pages,
                           const int32_t *d_block_table, int32_t bt_stride,
                           const int32_t *d_lengths, int32_t num_reqs,
                           const amla_plan_params *params, float bmm1_scale, float bmm2_scale,
                           const int32_t *d_counts, const int32_t *d_offsets,
                           const int32_t *d_work, int32_t list_len, void *d_workspace,
                           size_t ws_bytes, const amla_dcp_params *dcp, const int32_t *d_totals,
                           void *stream);

/*
 * Merge over DCP sources (page "drafter.attention", DraftDcp: the head owner merges each
 * row over the sources, exp2(lse_s - max) weights over their sum in FP32, one BF16
 * rounding):
 *   d_rows     BF16 [n_src][n_rows][512], 16-byte aligned: each source's merged rows
 *   d_lse      FP32 log2 [n_src][n_rows]; -inf marks a row a source has no key for
 *   d_out      BF16 [n_rows][512], 16-byte aligned;  d_lse_out FP32 [n_rows]
 * Rows every source leaves empty get 0 and -inf.  1 <= n_src <= 64.
 */
int amla_merge_sources(int32_t n_src, const uint16_t *d_rows, const float *d_lse, int64_t n_rows,
                       uint16_t *d_out, float *d_lse_out, void *stream);

/*
 * Reducer: merges each row's split partials (page "drafter.attention", DraftDcp: exp2
 * weights of lse_s - max over their sum, in FP32, one BF16 rounding) into
 *   d_out  BF16 (uint16 bits, round to nearest even) [num_reqs][rows_per_req][512]
 *   d_lse  FP32 log2 LSE [num_reqs][rows_per_req]
 * Requests with count 0 get out = 0 and lse = -inf.  compute_units feeds
 * amla_reducer_bands.
 */
int amla_combine(const void *d_workspace, size_t ws_bytes, const int32_t *d_counts,
                 const int32_t *d_offsets, int32_t num_reqs, const amla_plan_params *params,
                 int32_t compute_units, uint16_t *d_out, float *d_lse, void *stream);

/*
 * Reducer fused with the W_UV up-projection (the value stage after the merge; page
 * "drafter.attention", DraftDcp and latent_major).  Each row's split partials are merged
 * exactly as amla_combine does (one BF16 rounding of the merged latent), then multiplied by
 * its head's W_UV on BF16 MFMA with FP32 accumulation and rounded to BF16:
 *   attn_out[r*k + t][h*128 + v] = sum_c latent[r][t*H + h][c] * W_UV[h][c][v]
 *   d_w_uv      BF16 bits, W_UV [heads][512][128] stored latent-contiguous, i.e. the
 *               memory is [heads][128][512] (the 512 latent weights of one (h, v) are
 *               adjacent); 16-byte aligned
 *   d_attn_out  BF16 [num_reqs * k][heads * 128] (k = rows_per_req / heads), 8-byte aligned
 *   d_out       optional (NULL: not written): the merged BF16 latent [num_reqs][M][512]
 *   d_lse       optional (NULL: not written): the merged FP32 log2 LSE [num_reqs][M]
 * heads must divide rows_per_req.  Requests with count 0 give zero rows (lse -inf).
 * AMLA_ERR_INVALID for null or misaligned pointers, heads < 1 or heads not dividing M.
 */
int amla_combine_uv(const void *d_workspace, size_t ws_bytes, const int32_t *d_counts,
                    const int32_t *d_offsets, int32_t num_reqs, const amla_plan_params *params,
                    int32_t heads, const uint16_t *d_w_uv, uint16_t *d_attn_out,
                    uint16_t *d_out, float *d_lse, void *stream);

/*
 * The step before the decode (page "drafter.attention", DraftDcp._forward): the absorbed
 * decode query and the new tokens' cache rows, in one launch.
 *   d_q          BF16 [n][H][192]: per head q_nope (128) then q_pe (64); 16-byte aligned
 *   d_w_uk       BF16 W_UK_T [H][128][512] stored [H][512][128] (element (h, l, c) =
 *                W_UK_T[h][c][l]: the 128 nope weights of a latent dim adjacent);
 *                16-byte aligned
 *   d_kv_c       BF16 [n][512]: each token's normalised latent; 16-byte aligned
 *   d_k_pe       BF16 [n][64]: its rope key before the rotation
 *   d_positions  int64 [n]: rotary positions, in [0, max_pos)
 *   d_cos_sin    FP32 [max_pos][64]: cos of the 32 angles of a position, then their sin
 *   d_slot_mapping int64 [n]: cache slot of each token (page = slot / 64, row = slot % 64);
 *                negative: no cache row (padding)
 *   neox         0: rotary pairs (2i, 2i+1); 1: pairs (i, i + 32)
 *   q_scale, k_scale  per-tensor FP8 scales (code = E4M3(x / scale), saturated at 448)
 *   d_q_out      E4M3 [n][H][576]: ql_nope = q_nope W_UK_T (512) then rope(q_pe) (64);
 *                4-byte aligned
 *   d_kv_cache   E4M3 [pool_pages][64][576]: rows kv_c (512) then rope(k_pe) (64) are
 *                written at the tokens' slots, nothing else; 8-byte aligned
 *   d_status     int32 status word or NULL: AMLA_DEV_BAD_PAGE for a slot past the pool (row
 *                skipped), AMLA_DEV_BAD_POSITION for a position outside the table
 * Every value is rounded to BF16 before the cast (ql_nope after its FP32 accumulation).
 */
int amla_build_query_cache(const uint16_t *d_q, const uint16_t *d_w_uk, const uint16_t *d_kv_c,
                           const uint16_t *d_k_pe, const int64_t *d_positions,
                           const float *d_cos_sin, int32_t max_pos,
                           const int64_t *d_slot_mapping, int32_t n_tokens, int32_t heads,
                           int32_t neox, float q_scale, float k_scale, uint8_t *d_q_out,
                           uint8_t *d_kv_cache, int64_t pool_pages, int32_t *d_status,
                           void *stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): amla_plan_splits, amla_folded_decode and
 * amla_combine in one call, with the plan buffers and the split workspace in the library's
 * own static device scratch (AMLA_NOALLOC_SCRATCH_BYTES per device, held by every device
 * the library runs on until the process ends) instead of caller memory.  It allocates
 * nothing: no hipMalloc, hipFree or allocating library routine.
 *   arguments   as amla_folded_decode (bt_stride is also the plan's table width) and
 *               amla_combine; d_out BF16 [num_reqs][rows_per_req][512], d_lse FP32 log2
 *               [num_reqs][rows_per_req]
 *   d_status    NULL, or one int32 that receives the call's device status word (the bits
 *               of AMLA_DEV_*), written on the stream after the merge
 *   stream      must belong to the current device (the scratch copy used is the current
 *               device's)
 * Every call on one device shares that device's scratch, and each call leaves its plan and
 * partials there: calls that overlap in time on one device (several streams or host
 * threads) race and must not be issued.  Each call rewrites all the scratch state it reads.
 * The scratch a call needs is amla_workspace_bytes(num_reqs, rows_per_req, workers) plus
 * the plan buffers (counts, offsets and the work list of 2 * (num_reqs + 2 * workers)
 * entries, each rounded up to 256 bytes).  Returns AMLA_ERR_WORKSPACE when that exceeds
 * AMLA_NOALLOC_SCRATCH_BYTES, AMLA_ERR_INVALID for bad arguments (nothing enqueued),
 * AMLA_ERR_HIP when the scratch address cannot be found or a launch fails.
 */
#define AMLA_NOALLOC_SCRATCH_BYTES (64u << 20)
int amla_folded_decode_noalloc(const uint8_t *d_q, const uint8_t *d_kv, int64_t pool_pages,
                               const int32_t *d_block_table, int32_t bt_stride,
                               const int32_t *d_lengths, int32_t num_reqs,
                               const amla_plan_params *params, float bmm1_scale,
                               float bmm2_scale, int32_t compute_units, uint16_t *d_out,
                               float *d_lse, int32_t *d_status, void *stream);

/* Static text for a host status code or a device status word. */
const char *amla_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* AMLA_H */
