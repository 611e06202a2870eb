// Folded split-KV absorbed-MLA decode for MI355X (gfx950): plan, decode and combine
// kernels, and the steps next to them, behind the C ABI declared in include/amla.h.
//
// Method (page "vllm.models.kimi_k3.nvidia.specialized_decode.drafter.attention", module
// docstring; page "...cutedsl.mla.balanced", module docstring): MQA over one latent head
// of 576 FP8 dims per token (value = the first 512), the k draft tokens of a request
// folded into its head axis, each request's keys cut into planned splits that produce
// FP32 partials and a log2 LSE, and a reducer merging the splits into BF16 rows.
//
// gfx950 mapping (this library's design, not the pages'):
//   * plan    (this file) one 256-thread workgroup: the requests' pages (each charged a
//             head of a few pages for its split's overhead) laid end to end and cut into
//             equal ranges, one per group of workers; counts, items and group starts in
//             closed form per request (block scans, no sort).
//   * decode  one persistent workgroup per CU; each group of ceil(M/MT) workers walks its
//             items, a work unit being (item, row tile of MT rows); pages (64 tokens x 576 B)
//             go HBM -> LDS by global_load_lds_dwordx4 into a ring of page slots; S^T = K Q^T
//             and O^T += V^T P^T on v_mfma_f32_32x32x64_f8f6f4 (the accumulator layout puts
//             one query row per lane); P in E4M3 against a per-row reference, each key
//             block's P scaled by its own E8M0 byte in the P V MFMA.  decode_stream.hip:
//             MT = 32, 64 (score and value waves one entry apart, two waves per SIMD, a
//             stream of entries across work units); decode128.hip: MT = 128 (four waves,
//             each owning 32 rows end to end, 256 output accumulators per lane in AGPRs).
//   * combine (this file) one wave per (row, band); merges the splits of a row with exp2
//             weights.
//   * combine_uv  the merge fused with the W_UV up-projection (BF16 MFMA).
//   * merge_sources  a head owner's merge of rows computed on several DCP shards.
//   * build_query_cache  the step before the decode: the absorbed query (W_UK_T on BF16
//             MFMA, rotary embedding, E4M3 cast) and the new tokens' cache rows.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>
#include <type_traits>

#include "common.h"


namespace {

using namespace amla;

// ------------------------------------------------------------------ block utilities

// All-lane max (MAX) or sum of a wave without LDS traffic: DPP within rows of 16 lanes, then
// v_permlane16_swap / v_permlane32_swap across rows.
template <bool MAX>
__device__ float wave_allf(float v)
{
    auto op = [](float x, float y) { return MAX ? fmaxf(x, y) : x + y; };
    v = op(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x128, 0xf, 0xf, false)));
    v = op(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x124, 0xf, 0xf, false)));
    v = op(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4e, 0xf, 0xf, false)));
    v = op(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xb1, 0xf, 0xf, false)));
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = op(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return op(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Exclusive scan over the workgroup of one value per thread (thread order); returns the
// thread's exclusive prefix and writes the grand total to *total.
__device__ int32_t block_exclusive_scan(int32_t v, int32_t *scratch, int32_t *total)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int32_t incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        int32_t t = __shfl_up(incl, o);
        if (lane >= o) incl += t;
    }
    __syncthreads();
    if (lane == 63) scratch[wave] = incl;
    __syncthreads();
    int32_t before = 0, all = 0;
    for (int i = 0; i < kPlanThreads / 64; ++i) {
        if (i < wave) before += scratch[i];
        all += scratch[i];
    }
    *total = all;
    return before + incl - v;
}

// ---------------------------------------------------------------------- plan kernel

struct PlanArgs {
    const int32_t *lengths;
    int32_t *counts;
    int32_t *offsets;
    int32_t *work;
    int32_t *header;
    int32_t reqs, bt_cols, rows, mtile, workers, min_pages, max_splits, mode, list_len;
    int32_t split_cost;
};

__device__ inline int64_t pages_of(int32_t len) { return ((int64_t)len + kPage - 1) / kPage; }

// Exclusive scan of one int64 per thread (thread order) over the workgroup; the grand
// total goes to *total.
__device__ int64_t block_exclusive_scan64(int64_t v, int64_t *scratch, int64_t *total)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int64_t incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int64_t t = __shfl_up(incl, o);
        if (lane >= o) incl += t;
    }
    __syncthreads();
    if (lane == 63) scratch[wave] = incl;
    __syncthreads();
    int64_t before = 0, all = 0;
    for (int i = 0; i < kPlanThreads / 64; ++i) {
        if (i < wave) before += scratch[i];
        all += scratch[i];
    }
    *total = all;
    return before + incl - v;
}

// x / y for 0 <= x, 0 < y: 32-bit division when both fit (a 64-bit one is a long software
// sequence; the plan's products fit 32 bits for any realistic batch)
__device__ inline int64_t udiv64(int64_t x, int64_t y)
{
    if ((uint64_t)x <= 0xFFFFFFFFull && (uint64_t)y <= 0xFFFFFFFFull)
        return (int64_t)((uint32_t)x / (uint32_t)y);
    return x / y;
}

// ceil(x / y) for x >= 0, y > 0
__device__ inline int64_t cdiv64(int64_t x, int64_t y) { return x == 0 ? 0 : udiv64(x - 1, y) + 1; }

// The split plan, one workgroup; thread t owns the requests [t * per, (t + 1) * per).
// BALANCED (page "...cutedsl.mla.balanced", module docstring: split counts planned on the
// device from the KV lengths, one wave of persistent workers walking a work list; the rule
// is this library's reading): every non-empty request is laid out as a head of a =
// split_cost pages (what a split costs beyond its pages) and its pages, end to end, V in
// all, and V is cut into Gp = min(W / mt, max_splits, V / minp) equal ranges, one per group
// of mt = ceil(M / MT) workers (one per row tile), at c_g = floor(g V / Gp).  A cut inside
// request r less than minp pages into its pages (or in its head) moves to its start, less
// than minp from its end to its end; the others cut it, so the splits of r start at 0 and
// at the cuts with voff_r + a + minp <= c_g <= voff_r + a + pages_r - minp, which are
// g = g0(r) .. g1(r) in closed form (the cuts are at least minp apart since V / Gp >= minp).
// Group g takes the items starting in [C_g, C_{g+1}) of the moved cuts.
// FIXED: min(pages_r, W / (R mt)) equal splits per request, group g taking items
// [g N / G, (g + 1) N / G).
// Work list: (request, first page) per item in request order (item offsets[r] + s is split
// s of request r and its workspace slot), -1 up to 2 (R + W), the G + 1 group starts, -1.
__global__ __launch_bounds__(kPlanThreads) void plan_kernel(PlanArgs a)
{
    __shared__ int64_t voff[AMLA_MAX_REQS + 1];    // virtual pages before request r
    __shared__ int32_t ioff[AMLA_MAX_REQS + 1];    // items before request r
    __shared__ int64_t red64[kPlanThreads / 64];
    __shared__ int32_t red32[kPlanThreads / 64];
    const int tid = threadIdx.x;
    const int R = a.reqs;
    const int per = ceil_div(R > 0 ? R : 1, kPlanThreads);
    const int r0 = tid * per < R ? tid * per : R, r1 = r0 + per < R ? r0 + per : R;
    const int64_t mt = ceil_div(a.rows, a.mtile);
    const int64_t G = a.workers / mt > 0 ? a.workers / mt : 1;
    const int64_t minp = a.min_pages > 0 ? a.min_pages : 1;
    const int64_t head = a.split_cost;

    // 1. pages, validity, virtual offsets
    int64_t mine = 0;
    int bad_l = 0;
    for (int r = r0; r < r1; ++r) {
        const int32_t L = a.lengths[r];
        const int64_t p = pages_of(L);
        bad_l |= L < 0 || p > a.bt_cols;
        mine += L <= 0 ? 0 : head + p;
    }
    const bool bad = __syncthreads_or(bad_l) != 0;
    // virtual length of request r (0 for an empty one or a bad batch)
    auto vlen = [&](int r) -> int64_t {
        const int32_t L = a.lengths[r];
        return bad || L <= 0 ? 0 : head + pages_of(L);
    };
    int64_t V = 0;
    int64_t run = block_exclusive_scan64(bad ? 0 : mine, red64, &V);
    for (int r = r0; r < r1; ++r) {
        voff[r] = run;
        run += vlen(r);
    }
    if (tid == 0) voff[R] = V;

    // 2. counts and item offsets
    int64_t Gp = udiv64(V, minp);
    Gp = Gp < 1 ? 1 : Gp;
    Gp = Gp < G ? Gp : G;
    Gp = Gp < a.max_splits ? Gp : a.max_splits;
    int64_t fixed = R > 0 ? (int64_t)a.workers / ((int64_t)R * mt) : 1;
    fixed = fixed < 1 ? 1 : (fixed > a.max_splits ? a.max_splits : fixed);
    const bool balanced = a.mode == AMLA_PLAN_BALANCED;
    // the first and last cut inside the pages of a request whose pages start at virtual
    // position s (g1 < g0: none)
    auto cut_range = [&](int64_t s, int64_t p, int64_t &g0, int64_t &g1) {
        g0 = cdiv64((s + minp) * Gp, V);
        g1 = cdiv64((s + p - minp + 1) * Gp, V) - 1;
    };
    int32_t icount = 0;
    for (int r = r0; r < r1; ++r) {
        const int64_t p = bad ? 0 : pages_of(a.lengths[r]);
        int64_t c = 0;
        if (p > 0) {
            if (balanced) {
                int64_t g0, g1;
                cut_range(voff[r] + head, p, g0, g1);
                c = 1 + (g1 >= g0 ? g1 - g0 + 1 : 0);
            } else {
                c = p < fixed ? p : fixed;
            }
        }
        a.counts[r] = (int32_t)c;
        icount += (int32_t)c;
    }
    int32_t N = 0;
    int32_t irun = block_exclusive_scan(icount, red32, &N);

    // 3. the items of each request
    for (int r = r0; r < r1; ++r) {
        const int64_t p = bad ? 0 : pages_of(a.lengths[r]);
        ioff[r] = irun;
        a.offsets[r] = irun;
        if (p == 0) continue;
        int32_t *w = a.work + 2 * (int64_t)irun;
        if (balanced) {
            const int64_t s = voff[r] + head;
            int64_t g0, g1;
            cut_range(s, p, g0, g1);
            w[0] = r;
            w[1] = 0;
            for (int64_t g = g0; g <= g1; ++g) {
                w[2 * (g - g0 + 1)] = r;
                w[2 * (g - g0 + 1) + 1] = (int32_t)(udiv64(g * V, Gp) - s);
            }
            irun += (int32_t)(1 + (g1 >= g0 ? g1 - g0 + 1 : 0));
        } else {
            const int64_t c = p < fixed ? p : fixed, q = p / c, rem = p % c;
            for (int64_t k = 0; k < c; ++k) {
                w[2 * k] = r;
                w[2 * k + 1] = (int32_t)(k * q + (k < rem ? k : rem));
            }
            irun += (int32_t)c;
        }
    }
    if (tid == 0) {
        ioff[R] = N;
        a.offsets[R] = N;
    }
    const int64_t gbase = 2 * ((int64_t)R + a.workers);
    for (int64_t i = 2 * (int64_t)N + tid; i < gbase; i += kPlanThreads) a.work[i] = -1;
    for (int64_t i = gbase + G + 1 + tid; i < a.list_len; i += kPlanThreads) a.work[i] = -1;
    __syncthreads();   // voff and ioff complete

    // 4. the first item of each group
    for (int64_t g = tid; g <= G; g += kPlanThreads) {
        int32_t first = N;
        if (!balanced) {
            first = (int32_t)udiv64(g * N, G);
        } else if (g < Gp && V > 0) {
            const int64_t c = udiv64(g * V, Gp);
            int lo = 1, hi = R;                 // the first request with voff > c ...
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if (voff[mid] > c) hi = mid;
                else lo = mid + 1;
            }
            const int r = lo - 1;               // ... less one holds position c
            const int64_t x = c - voff[r] - head, p = voff[r + 1] - voff[r] - head;
            if (x < minp) {
                first = ioff[r];
            } else if (p - x < minp) {
                first = ioff[r + 1];
            } else {
                int64_t g0, g1;
                cut_range(voff[r] + head, p, g0, g1);
                first = ioff[r] + 1 + (int32_t)(g - g0);
            }
        }
        a.work[gbase + g] = first;
    }

    if (tid == 0) {
        a.header[kHdrStatus] = bad ? AMLA_DEV_BAD_LENGTH : 0;
        a.header[kHdrItems] = N;
        a.header[kHdrRows] = a.rows;
        a.header[kHdrMtile] = a.mtile;
        a.header[kHdrWorkers] = a.workers;
        a.header[kHdrMode] = a.mode;
        a.header[kHdrReqs] = R;
        a.header[kHdrPlanned] = kPlannedMagic;
    }
}

// ------------------------------------------------------------------- combine kernel

struct CombineArgs {
    const float *partial;
    const float *lse;
    const int32_t *counts;
    const int32_t *offsets;
    uint16_t *out;
    float *out_lse;
    int32_t reqs, rows, bands, slots;
};

__device__ inline uint16_t bf16_rne(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu))
        return (uint16_t)((u >> 16) | 0x40);  // quiet NaN
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// One wave per (row, band): band b covers dims [b*512/bands, (b+1)*512/bands).  The
// request's count and offset are loaded together; then the LSE of every split (lane s, and
// s + 64j, holds split s + 64j's) and the first batch of partials are in flight at once,
// so the wave waits for memory twice before its first output, and the split weights are
// broadcast from the lanes that computed them.
constexpr int kCombineBatch = 8;
constexpr int kLsePerLane = AMLA_MAX_SPLITS / 64;

template <int PER_LANE>
__device__ __forceinline__ void combine_row(const CombineArgs &a, int64_t g, int band, int lane,
                                            int i, int c, int64_t base)
{
    const int width = 256 * PER_LANE;
    uint16_t *out = a.out + g * kVDim + band * width;
    // the next batch of split rows (past the last split: zeros, no load; c is uniform)
    auto load_batch = [&](int s0, v4f (&part)[kCombineBatch][PER_LANE]) {
#pragma unroll
        for (int b = 0; b < kCombineBatch; ++b) {
            const float *p = a.partial + ((base + s0 + b) * a.rows + i) * kVDim + band * width;
#pragma unroll
            for (int k = 0; k < PER_LANE; ++k)
                part[b][k] = s0 + b < c ? *(const v4f *)(p + 4 * (lane + 64 * k)) : v4f{0, 0, 0, 0};
        }
    };
    float ls[kLsePerLane];
#pragma unroll
    for (int j = 0; j < kLsePerLane; ++j) {
        const int s = lane + 64 * j;
        ls[j] = s < c ? a.lse[(base + s) * a.rows + i] : -INFINITY;
    }
    v4f part[kCombineBatch][PER_LANE];
    load_batch(0, part);
    // weights exp2(lse_s - max) / sum_s exp2(lse_s - max)
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < kLsePerLane; ++j) mx = fmaxf(mx, ls[j]);
    mx = wave_allf<true>(mx);
    float wt[kLsePerLane], sum = 0.f;
#pragma unroll
    for (int j = 0; j < kLsePerLane; ++j) {
        // a row with no key in any split (possible under a causal mask) has mx = -inf
        wt[j] = lane + 64 * j < c && mx != -INFINITY ? __builtin_amdgcn_exp2f(ls[j] - mx) : 0.f;
        sum += wt[j];
    }
    sum = wave_allf<false>(sum);
    const float inv = sum > 0.f ? 1.0f / sum : 0.f;

    v4f acc[PER_LANE];
#pragma unroll
    for (int k = 0; k < PER_LANE; ++k) acc[k] = v4f{0, 0, 0, 0};
    for (int s0 = 0; s0 < c; s0 += kCombineBatch) {
        const int j = s0 >> 6;   // the batch lies in one 64-split group (64 % batch == 0)
        const float wj = j == 0 ? wt[0] : j == 1 ? wt[1] : j == 2 ? wt[2] : wt[3];
#pragma unroll
        for (int b = 0; b < kCombineBatch; ++b) {
            const float w = s0 + b < c
                                ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wj), (s0 + b) & 63)) * inv
                                : 0.f;
#pragma unroll
            for (int k = 0; k < PER_LANE; ++k) acc[k] += w * part[b][k];
        }
        if (s0 + kCombineBatch < c) load_batch(s0 + kCombineBatch, part);
    }
#pragma unroll
    for (int k = 0; k < PER_LANE; ++k) {
        const uint32_t lo = bf16_rne(acc[k][0]) | ((uint32_t)bf16_rne(acc[k][1]) << 16);
        const uint32_t hi = bf16_rne(acc[k][2]) | ((uint32_t)bf16_rne(acc[k][3]) << 16);
        *(uint2 *)(out + 4 * (lane + 64 * k)) = make_uint2(lo, hi);
    }
    if (band == 0 && lane == 0) a.out_lse[g] = mx + __builtin_amdgcn_logf(sum);
}
static_assert(64 % kCombineBatch == 0, "a batch of splits must not straddle a lane group");
static_assert(AMLA_MAX_SPLITS <= 4 * 64, "combine_row holds at most four LSEs per lane");

__global__ __launch_bounds__(64) void combine_kernel(CombineArgs a)
{
    const int lane = threadIdx.x;
    const int64_t g = blockIdx.x / a.bands;       // folded row, request-major
    const int band = blockIdx.x % a.bands;
    const int r = (int)(g / a.rows), i = (int)(g % a.rows);
    const int c = ldc(&a.counts[r]);
    const int64_t base = ldc(&a.offsets[r]);
    asm volatile("" ::"s"(c), "s"(base));
    const int width = kVDim / a.bands;            // 512 or 256
    const int per_lane = width / 256;             // float4s per lane: 2 or 1
    uint16_t *out = a.out + g * kVDim + band * width;

    if (c <= 0) {
        for (int k = 0; k < per_lane; ++k)
            *(uint2 *)(out + 4 * (lane + 64 * k)) = make_uint2(0u, 0u);
        if (band == 0 && lane == 0) a.out_lse[g] = -INFINITY;
        return;
    }
    if (c > AMLA_MAX_SPLITS || base < 0 || base + c > a.slots) {
        // not a plan of these sizes: flag the row as NaN rather than read out of bounds
        for (int k = 0; k < per_lane; ++k)
            *(uint2 *)(out + 4 * (lane + 64 * k)) = make_uint2(0x7FC07FC0u, 0x7FC07FC0u);
        if (band == 0 && lane == 0) a.out_lse[g] = NAN;
        return;
    }
    if (per_lane == 2)
        combine_row<2>(a, g, band, lane, i, c, base);
    else
        combine_row<1>(a, g, band, lane, i, c, base);
}

// ------------------------------------------------------- merge + W_UV (value stage)

// Page "drafter.attention", DraftDcp (value stage): each row's split partials merged as in
// combine_kernel, the merged latent rounded once to BF16, then multiplied by its head's
// W_UV [H, 512, 128] on BF16 MFMA with FP32 accumulation, into the attention output
// [R*k, H*128] (the same bytes as [R][M][128] in folded row order).  W_UV is stored
// latent-contiguous ([H][128][512]; page "drafter.attention", latent_major), so every
// MFMA operand fragment is 16 adjacent bytes.
// One workgroup of 8 waves per (head h, ROWS = 32, 16 or 8 rows of that head); row j of
// head h is draft token t = j % k of request r = j / k, folded row i = t*H + h.  512 / ROWS
// threads merge one row; the BF16 latent tile goes through LDS into the B operand of
// D[v][row] = W^T lat^T, wave w computing output dims [16w, 16w + 16) for every 16-row
// block of the tile with the same W_UV fragments, so each lane ends with four adjacent
// output dims of one row per block.
constexpr int kUvDim = 128;
constexpr int kUvRows = 16;
constexpr int kUvStride = kVDim + 8;   // BF16 per LDS latent row: 16 B of padding moves
                                       // each row four banks on (conflict-free B reads)
constexpr int kUvBatch = 4;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

struct UvArgs {
    const float *partial;
    const float *lse;
    const int32_t *counts;
    const int32_t *offsets;
    const uint16_t *w_uv;
    uint16_t *attn_out;
    uint16_t *out;       // merged BF16 latent, or null
    float *out_lse;      // merged log2 LSE, or null
    int32_t reqs, rows, heads, k, slots;
};

template <int ROWS>
__global__ __launch_bounds__(512) void combine_uv_kernel(UvArgs a)
{
    constexpr int TILE = ROWS > kUvRows ? ROWS : kUvRows;   // LDS latent rows: 16 or 32
    constexpr int RB = TILE / 16;          // 16-row column blocks of the MFMA
    constexpr int TPR = 512 / ROWS;        // threads per row: 16, 32 or 64
    constexpr int NJ = kVDim / 4 / TPR;    // float4s per thread and split: 8, 4 or 2
    constexpr int BATCH = ROWS > kUvRows ? 2 : kUvBatch;   // splits in flight per thread
    __shared__ __attribute__((aligned(16))) uint16_t lat[TILE * kUvStride];
    __shared__ float wts[TILE][AMLA_MAX_SPLITS];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int h = blockIdx.y;
    const int per_head = a.reqs * a.k;
    const int j0 = blockIdx.x * ROWS;

    // W_UV fragments of this wave's 16 output dims for all 16 K-steps, loaded first (they
    // do not depend on the merge).  A operand of the 16x16x32 MFMA: lane l holds
    // W[h][v = 16 wave + l%16][c = 32 s + 8 (l/16) .. +7].
    bf16x8 wf[16];
    {
        const uint16_t *wv = a.w_uv + ((size_t)h * kUvDim + 16 * wave + (lane & 15)) * kVDim +
                             8 * (lane >> 4);
#pragma unroll
        for (int s = 0; s < 16; ++s) wf[s] = *(const bf16x8 *)(wv + 32 * s);
    }

    // merge (the weights of combine_row): TPR threads per row; thread tr of row rho holds
    // float4s tr + TPR jj (jj < NJ).  The row's first LSEs and its first batch of partials
    // are loaded together, right after the request's count and offset.
    const int rho = tid / TPR, tr = tid % TPR;
    const int j = j0 + rho;
    int r = 0, i = 0, c = 0;
    int64_t base = 0;
    if (j < per_head) {
        r = j / a.k;
        i = (j - r * a.k) * a.heads + h;
        c = a.counts[r];
        base = a.offsets[r];
    }
    const bool bad = c < 0 || c > AMLA_MAX_SPLITS || base < 0 || base + c > a.slots;
    if (bad) c = 0;   // not a plan of these sizes: the row becomes NaN, nothing is read
    if (c == 0) base = 0;   // every address formed below stays inside slot 0
    const int64_t g = (int64_t)r * a.rows + i;
    const float *lrow_g = a.lse + base * a.rows + i;              // split s at s * rows
    const float *prow = a.partial + (base * a.rows + i) * kVDim + 4 * tr;
    const int64_t pstride = (int64_t)a.rows * kVDim;

    float ls = tr < c ? lrow_g[(int64_t)tr * a.rows] : -INFINITY;
    v4f p[BATCH][NJ];
#pragma unroll
    for (int b = 0; b < BATCH; ++b) {
        const int sb = b < c ? b : (c > 0 ? c - 1 : 0);
#pragma unroll
        for (int jj = 0; jj < NJ; ++jj)
            p[b][jj] = c > 0 ? *(const v4f *)(prow + sb * pstride + 4 * TPR * jj) : v4f{0, 0, 0, 0};
    }
    float mx = ls;
    for (int s = tr + TPR; s < c; s += TPR) mx = fmaxf(mx, lrow_g[(int64_t)s * a.rows]);
#pragma unroll
    for (int o = TPR / 2; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    float sum = 0.f;
    if (tr < c) {
        // a row with no key in any split (possible under a causal mask) has mx = -inf
        const float w = mx != -INFINITY ? __builtin_amdgcn_exp2f(ls - mx) : 0.f;
        wts[rho][tr] = w;
        sum = w;
    }
    for (int s = tr + TPR; s < c; s += TPR) {
        const float w = mx != -INFINITY ? __builtin_amdgcn_exp2f(lrow_g[(int64_t)s * a.rows] - mx) : 0.f;
        wts[rho][s] = w;
        sum += w;
    }
#pragma unroll
    for (int o = TPR / 2; o > 0; o >>= 1) sum += __shfl_xor(sum, o);
    __syncthreads();
    const float inv = sum > 0.f ? 1.0f / sum : 0.f;

    v4f acc[NJ];
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj) acc[jj] = v4f{0, 0, 0, 0};
    for (int s0 = 0; s0 < c; s0 += BATCH) {
        if (s0 > 0) {
#pragma unroll
            for (int b = 0; b < BATCH; ++b) {
                const int sb = s0 + b < c ? s0 + b : c - 1;
#pragma unroll
                for (int jj = 0; jj < NJ; ++jj)
                    p[b][jj] = *(const v4f *)(prow + sb * pstride + 4 * TPR * jj);
            }
        }
#pragma unroll
        for (int b = 0; b < BATCH; ++b) {
            const float w = s0 + b < c ? wts[rho][s0 + b] * inv : 0.f;
#pragma unroll
            for (int jj = 0; jj < NJ; ++jj) acc[jj] += w * p[b][jj];
        }
    }

    // one BF16 rounding: the latent tile in LDS (and the optional global copy)
    uint16_t *lrow = lat + rho * kUvStride + 4 * tr;
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj) {
        uint32_t lo = 0x7FC07FC0u, hi = 0x7FC07FC0u;
        if (!bad) {
            lo = bf16_rne(acc[jj][0]) | ((uint32_t)bf16_rne(acc[jj][1]) << 16);
            hi = bf16_rne(acc[jj][2]) | ((uint32_t)bf16_rne(acc[jj][3]) << 16);
        }
        *(uint2 *)(lrow + 4 * TPR * jj) = make_uint2(lo, hi);
        if (a.out && j < per_head)
            *(uint2 *)(a.out + g * kVDim + 4 * tr + 4 * TPR * jj) = make_uint2(lo, hi);
    }
    if (ROWS < TILE) {   // the MFMA's 16 rows: the tile's unused rows are zero
        for (int x = tid; x < (TILE - ROWS) * kVDim / 4; x += 512)
            *(uint2 *)(lat + (ROWS + x / (kVDim / 4)) * kUvStride + 4 * (x % (kVDim / 4))) =
                make_uint2(0u, 0u);
    }
    if (a.out_lse && j < per_head && tr == 0)
        a.out_lse[g] = bad ? NAN : c > 0 ? mx + __builtin_amdgcn_logf(sum) : -INFINITY;
    __syncthreads();

    // D[v][row] over K = 512 in 16 steps for each 16-row block rb (the W_UV fragments serve
    // every block); B operand: lane l holds lat[row 16 rb + l%16][c = 32 s + 8 (l/16) .. +7]
    v4f d[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) d[rb] = v4f{0, 0, 0, 0};
#pragma unroll
    for (int s = 0; s < 16; ++s) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            const uint16_t *lb = lat + (16 * rb + (lane & 15)) * kUvStride + 8 * (lane >> 4);
            const bf16x8 bfr = *(const bf16x8 *)(lb + 32 * s);
            d[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[s], bfr, d[rb], 0, 0, 0);
        }
    }
    // lane l holds D[v = 16 wave + 4 (l/16) + e][row 16 rb + l%16], e < 4
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const int jl = 16 * rb + (lane & 15), jr = j0 + jl;
        if (jl < ROWS && jr < per_head) {
            const int rr = jr / a.k;
            const int64_t gr = (int64_t)rr * a.rows + (int64_t)(jr - rr * a.k) * a.heads + h;
            const uint32_t lo = bf16_rne(d[rb][0]) | ((uint32_t)bf16_rne(d[rb][1]) << 16);
            const uint32_t hi = bf16_rne(d[rb][2]) | ((uint32_t)bf16_rne(d[rb][3]) << 16);
            *(uint2 *)(a.attn_out + gr * kUvDim + 16 * wave + 4 * (lane >> 4)) = make_uint2(lo, hi);
        }
    }
}

// ------------------------------------------------------------ merge over DCP sources

// Page "drafter.attention", DraftDcp (value stage): a head owner merges each row over the
// DCP sources that computed it on their KV shards, with the combine math (exp2(lse_s - max)
// weights over their sum in FP32, one BF16 rounding).  One wave per row: lane s holds
// source s's LSE, and every lane merges 8 adjacent dims (16 bytes per source row), four
// source rows in flight at a time.
constexpr int kMaxSources = 64;

__global__ __launch_bounds__(256) void merge_sources_kernel(const uint16_t *__restrict__ rows,
                                                            const float *__restrict__ lse,
                                                            int n_src, int64_t n_rows,
                                                            uint16_t *__restrict__ out,
                                                            float *__restrict__ out_lse)
{
    const int lane = threadIdx.x & 63;
    const int64_t g = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (g >= n_rows) return;   // whole waves
    const float ls = lane < n_src ? lse[(int64_t)lane * n_rows + g] : -INFINITY;
    const float mx = wave_allf<true>(ls);
    const float w = lane < n_src && mx != -INFINITY ? __builtin_amdgcn_exp2f(ls - mx) : 0.f;
    const float sum = wave_allf<false>(w);
    const float inv = sum > 0.f ? 1.0f / sum : 0.f;
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    const uint16_t *src = rows + g * kVDim + 8 * lane;
    for (int s0 = 0; s0 < n_src; s0 += 4) {
        uint4 v[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int sb = s0 + b < n_src ? s0 + b : n_src - 1;
            v[b] = *(const uint4 *)(src + (int64_t)sb * n_rows * kVDim);
        }
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const float ws =
                s0 + b < n_src
                    ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), s0 + b)) * inv
                    : 0.f;
            const uint32_t u[4] = {v[b].x, v[b].y, v[b].z, v[b].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc[2 * e] += ws * __uint_as_float(u[e] << 16);
                acc[2 * e + 1] += ws * __uint_as_float(u[e] & 0xFFFF0000u);
            }
        }
    }
    uint4 o;
    o.x = bf16_rne(acc[0]) | ((uint32_t)bf16_rne(acc[1]) << 16);
    o.y = bf16_rne(acc[2]) | ((uint32_t)bf16_rne(acc[3]) << 16);
    o.z = bf16_rne(acc[4]) | ((uint32_t)bf16_rne(acc[5]) << 16);
    o.w = bf16_rne(acc[6]) | ((uint32_t)bf16_rne(acc[7]) << 16);
    *(uint4 *)(out + g * kVDim + 8 * lane) = o;
    if (lane == 0) out_lse[g] = mx == -INFINITY ? -INFINITY : mx + __builtin_amdgcn_logf(sum);
}

// --------------------------------------------- absorbed query build and cache write

// Page "drafter.attention", DraftDcp._forward (the step before the decode): per head,
// ql_nope = q_nope W_UK_T ([H, 128, 512]; BF16 MMA, FP32 accumulation), the query row is
// ql_nope ++ rope(q_pe) and each new token's cache row is kv_c ++ rope(k_pe), both cast to
// E4M3 with their per-tensor scales; the cache row goes to its slot (page slot / 64, row
// slot % 64), the query row to [n, H, 576].  Every value passes through BF16 (the model
// dtype) before the cast.  W_UK_T arrives stored [H][512][128] (the 128 nope weights of a
// latent dim adjacent), so MFMA operand fragments are 16 adjacent bytes.
// One launch, two roles: blocks [0, query_blocks) build the query of (TOK = 16 or 32
// tokens, head h), the W_UK fragments of each MFMA serving every 16-token block; the others
// write the cache rows of 4 tokens (one wave each).
constexpr int kQbTokens = 16;

struct BuildArgs {
    const uint16_t *q;          // [n][H][192]
    const uint16_t *w_uk;       // [H][512][128]
    const uint16_t *kv_c;       // [n][512]
    const uint16_t *k_pe;       // [n][64]
    const int64_t *positions;   // [n]
    const float *cos_sin;       // [max_pos][64]
    const int64_t *slots;       // [n]
    uint8_t *q_out;             // [n][H][576]
    uint8_t *cache;             // [pool_pages][64][576]
    int32_t *status;            // device status word or null
    int64_t pool_pages;
    int32_t n, heads, neox, max_pos, query_blocks;
    float q_inv, k_inv;         // 1 / scale
};

__device__ __forceinline__ float bf16_round(float x) { return __uint_as_float((uint32_t)bf16_rne(x) << 16); }

// four values -> four E4M3 bytes (x * inv_scale, saturated at +-448, nearest even)
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d, float inv)
{
    auto sat = [&](float v) { return fminf(fmaxf(v * inv, -448.f), 448.f); };
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(sat(a), sat(b), 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(sat(c), sat(d), w, true);
    return (uint32_t)w;
}

// rotary pair i of a 64-dim rope vector: its two dims
__device__ __forceinline__ void rope_dims(int i, bool neox, int &d0, int &d1)
{
    d0 = neox ? i : 2 * i;
    d1 = neox ? i + 32 : 2 * i + 1;
}

template <int TOK>
__global__ __launch_bounds__(256) void build_query_cache_kernel(BuildArgs a)
{
    constexpr int TB = TOK / 16;   // 16-token column blocks of the MFMA
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const bool neox = a.neox != 0;
    auto bf = [](uint16_t u) { return __uint_as_float((uint32_t)u << 16); };
    auto cos_sin_row = [&](int64_t tok) {
        int64_t p = a.positions[tok];
        if (p < 0 || p >= a.max_pos) {
            if (a.status) atomicOr(a.status, AMLA_DEV_BAD_POSITION);
            p = 0;
        }
        return a.cos_sin + p * 64;
    };

    if ((int)blockIdx.x < a.query_blocks) {
        const int h = blockIdx.x % a.heads;
        const int t0 = (blockIdx.x / a.heads) * TOK;
        // B operand (q_nope^T) of token block tb: lane l holds q_nope[token t0 + 16 tb + l%16]
        // [c = 32 ks + 8 (l/16) ..+7]
        bf16x8 qb[TB][4];
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) {
            const int tok = t0 + 16 * tb + (lane & 15);
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                if (tok < a.n)
                    qb[tb][ks] = *(const bf16x8 *)(a.q + ((int64_t)tok * a.heads + h) * 192 + 32 * ks + 8 * (lane >> 4));
                else
                    qb[tb][ks] = bf16x8{};
            }
        }
        // A operand (W_UK): lane l holds W[h][l = 128 wave + 16 mt + l%16][c = 32 ks + 8 (l/16) ..]
        const uint16_t *wh = a.w_uk + ((int64_t)h * kVDim + 128 * wave + (lane & 15)) * 128 + 8 * (lane >> 4);
        v4f d[TB][8];
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
#pragma unroll
            for (int tb = 0; tb < TB; ++tb) d[tb][mt] = v4f{0, 0, 0, 0};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const bf16x8 wa = *(const bf16x8 *)(wh + 16 * 128 * mt + 32 * ks);
#pragma unroll
                for (int tb = 0; tb < TB; ++tb)
                    d[tb][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa, qb[tb][ks], d[tb][mt], 0, 0, 0);
            }
        }
        // lane l holds ql[token t0 + 16 tb + l%16][latent 128 wave + 16 mt + 4 (l/16) + e]
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) {
            const int tok = t0 + 16 * tb + (lane & 15);
            if (tok < a.n) {
                uint8_t *qo = a.q_out + ((int64_t)tok * a.heads + h) * kKDim + 128 * wave + 4 * (lane >> 4);
#pragma unroll
                for (int mt = 0; mt < 8; ++mt)
                    *(uint32_t *)(qo + 16 * mt) =
                        e4m3x4(bf16_round(d[tb][mt][0]), bf16_round(d[tb][mt][1]),
                               bf16_round(d[tb][mt][2]), bf16_round(d[tb][mt][3]), a.q_inv);
            }
        }
        // rope(q_pe): thread (token t0 + 16 tb + tid/16, pairs 2 (tid%16) and 2 (tid%16) + 1)
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) {
        const int rt = t0 + 16 * tb + (tid >> 4);
        if (rt < a.n) {
            const float *cs = cos_sin_row(rt);
            const uint16_t *pe = a.q + ((int64_t)rt * a.heads + h) * 192 + 128;
            uint8_t *qo = a.q_out + ((int64_t)rt * a.heads + h) * kKDim + kVDim;
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int i = 2 * (tid & 15) + u;
                int d0, d1;
                rope_dims(i, neox, d0, d1);
                const float x0 = bf(pe[d0]), x1 = bf(pe[d1]), c = cs[i], sn = cs[32 + i];
                const float y0 = bf16_round(x0 * c - x1 * sn), y1 = bf16_round(x1 * c + x0 * sn);
                const uint32_t w = e4m3x4(y0, y1, 0.f, 0.f, a.q_inv);
                qo[d0] = (uint8_t)(w & 0xFF);
                qo[d1] = (uint8_t)((w >> 8) & 0xFF);
            }
        }
        }
        return;
    }

    // cache rows: one wave per token
    const int64_t tok = ((int64_t)blockIdx.x - a.query_blocks) * 4 + wave;
    if (tok >= a.n) return;
    const int64_t slot = a.slots[tok];
    if (slot < 0) return;                       // a padding token: no cache row
    const int64_t page = slot >> 6;
    if (page >= a.pool_pages) {
        if (lane == 0 && a.status) atomicOr(a.status, AMLA_DEV_BAD_PAGE);
        return;
    }
    uint8_t *dst = a.cache + slot * kKDim;      // page * 64 + row, rows of 576 bytes
    {
        const uint4 v = *(const uint4 *)(a.kv_c + tok * kVDim + 8 * lane);
        const uint32_t u[4] = {v.x, v.y, v.z, v.w};
        float f[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            f[2 * e] = __uint_as_float(u[e] << 16);
            f[2 * e + 1] = __uint_as_float(u[e] & 0xFFFF0000u);
        }
        *(uint2 *)(dst + 8 * lane) = make_uint2(e4m3x4(f[0], f[1], f[2], f[3], a.k_inv),
                                                e4m3x4(f[4], f[5], f[6], f[7], a.k_inv));
    }
    if (lane < 32) {
        const float *cs = cos_sin_row(tok);
        int d0, d1;
        rope_dims(lane, neox, d0, d1);
        const uint16_t *pe = a.k_pe + tok * 64;
        const float x0 = bf(pe[d0]), x1 = bf(pe[d1]), c = cs[lane], sn = cs[32 + lane];
        const float y0 = bf16_round(x0 * c - x1 * sn), y1 = bf16_round(x1 * c + x0 * sn);
        const uint32_t w = e4m3x4(y0, y1, 0.f, 0.f, a.k_inv);
        dst[kVDim + d0] = (uint8_t)(w & 0xFF);
        dst[kVDim + d1] = (uint8_t)((w >> 8) & 0xFF);
    }
}

// ----------------------------------------------------------------------- host helpers

bool params_ok(const amla_plan_params *p)
{
    return p && p->rows_per_req >= 1 && p->rows_per_req <= AMLA_MAX_ROWS &&
           (p->mtile == 32 || p->mtile == 64 || p->mtile == 128) && p->workers >= 1 &&
           p->workers <= 65536 && p->min_split_tokens >= 0 && p->max_splits >= 1 &&
           p->max_splits <= AMLA_MAX_SPLITS &&
           (p->mode == AMLA_PLAN_BALANCED || p->mode == AMLA_PLAN_FIXED) &&
           p->split_cost_pages >= 0 && p->split_cost_pages <= AMLA_MAX_SPLIT_COST;
}

// ------------------------------------------------- allocation-free entry: static scratch

// The plan buffers and the split workspace of amla_folded_decode_noalloc live in this
// file-scope array, one copy per device the library runs on, held until the process ends.
// Host code never passes `scratch` itself to a kernel (on the host it is only a stand-in
// for the symbol): it uses the address hipGetSymbolAddress returns for the current device.
constexpr size_t kScratchBytes = (size_t)AMLA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

struct ScratchLayout {
    size_t counts, offsets, work, workspace, ws_bytes, total;
    int32_t list_len;
};

inline size_t align256(size_t x) { return (x + 255) / 256 * 256; }

inline ScratchLayout scratch_layout(int32_t reqs, int32_t rows, int32_t workers)
{
    ScratchLayout l;
    l.list_len = 2 * (reqs + kPlanSlack * workers);
    l.counts = 0;
    l.offsets = align256((size_t)(reqs > 0 ? reqs : 1) * 4);
    l.work = l.offsets + align256((size_t)(reqs + 1) * 4);
    l.workspace = l.work + align256((size_t)l.list_len * 4);
    l.ws_bytes = ws_layout(reqs, rows, workers).total;
    l.total = l.workspace + l.ws_bytes;
    return l;
}

__global__ void copy_status_kernel(const int32_t *__restrict__ header, int32_t *__restrict__ out)
{
    if (threadIdx.x == 0) *out = header[kHdrStatus];
}

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxScratchDevices];

// The device address of `scratch` on the current device, looked up on the first call made
// with that device current and kept for the later ones.
int scratch_address(void **out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return AMLA_ERR_HIP;
    if (dev < 0 || dev >= kMaxScratchDevices) return AMLA_ERR_INVALID;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress((void **)&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr)
            return AMLA_ERR_HIP;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return AMLA_OK;
}

}  // namespace

// ============================================================================ C ABI

extern "C" {

int amla_fold_plan(int32_t causal, int32_t num_reqs, int32_t num_rows, int32_t num_decode_tokens,
                   int32_t block_table_rows, int32_t max_query_len, int32_t heads,
                   int32_t need_lse, int32_t max_fold_heads, int32_t *k_out, int32_t *fold_out)
{
    if (!k_out || !fold_out || heads < 1 || (need_lse && max_fold_heads < heads))
        return AMLA_ERR_INVALID;
    // A non-causal draft block folds when every request has the same k >= 2 decode tokens
    // (the rows split evenly over the requests and the longest block is that share) and a
    // block-table row.
    const int32_t k = num_reqs > 0 ? num_rows / num_reqs : 0;
    const bool uniform = num_reqs > 0 && (int64_t)k * num_reqs == num_rows &&
                         max_query_len == k && num_rows == num_decode_tokens;
    const bool folds = !causal && uniform && k >= 2 && block_table_rows >= num_reqs;
    // Tokens per folded row: all k without an LSE; with one, the largest divisor of k
    // that keeps the row within max_fold_heads heads.
    int32_t f = k;
    if (need_lse)
        while (f > 1 && (k % f != 0 || (int64_t)f * heads > max_fold_heads)) --f;
    *k_out = folds ? k : 0;
    *fold_out = folds ? f : 0;
    return AMLA_OK;
}

int amla_bmm_scales(float softmax_scale, float q_scale, float k_scale, float *bmm1_out,
                    float *bmm2_out)
{
    if (!bmm1_out || !bmm2_out) return AMLA_ERR_INVALID;
    *bmm1_out = softmax_scale * q_scale * k_scale;
    *bmm2_out = k_scale;
    return AMLA_OK;
}

int amla_decode_config(int32_t compute_units, int32_t rows_per_req, int32_t *workers_out,
                       int32_t *mtile_out)
{
    if (!workers_out || !mtile_out || compute_units < 1 || rows_per_req < 1 ||
        rows_per_req > AMLA_MAX_ROWS)
        return AMLA_ERR_INVALID;
    *workers_out = compute_units;
    if (rows_per_req <= 64) {
        *mtile_out = rows_per_req <= 32 ? 32 : 64;
    } else {
        // 128-row tiles unless 64-row tiles leave fewer padding rows in the last tile
        const int pad64 = ceil_div(rows_per_req, 64) * 64 - rows_per_req;
        const int pad128 = ceil_div(rows_per_req, 128) * 128 - rows_per_req;
        *mtile_out = pad128 <= pad64 ? 128 : 64;
    }
    return AMLA_OK;
}

int amla_reducer_bands(int32_t rows, int32_t compute_units, int32_t *bands_out)
{
    if (!bands_out || rows < 0 || compute_units < 1) return AMLA_ERR_INVALID;
    const int64_t a = ((int64_t)rows * 2 + compute_units - 1) / compute_units;
    const int64_t b = 2 * (((int64_t)rows + compute_units - 1) / compute_units);
    *bands_out = a < b ? 2 : 1;
    return AMLA_OK;
}

size_t amla_workspace_bytes(int32_t num_reqs, int32_t rows_per_req, int32_t workers)
{
    if (num_reqs < 0 || num_reqs > AMLA_MAX_REQS || rows_per_req < 1 ||
        rows_per_req > AMLA_MAX_ROWS || workers < 1 || workers > 65536)
        return 0;
    return ws_layout(num_reqs, rows_per_req, workers).total;
}

int amla_plan_splits(const int32_t *d_lengths, int32_t num_reqs, int32_t bt_cols,
                     const amla_plan_params *params, int32_t *d_counts, int32_t *d_offsets,
                     int32_t *d_work, int32_t list_len, void *d_workspace, size_t ws_bytes,
                     void *stream)
{
    if (!params_ok(params) || num_reqs < 0 || num_reqs > AMLA_MAX_REQS || bt_cols < 0 ||
        !d_offsets || !d_work || !d_workspace || (num_reqs > 0 && (!d_lengths || !d_counts)))
        return AMLA_ERR_INVALID;
    if (ws_bytes < amla_workspace_bytes(num_reqs, params->rows_per_req, params->workers))
        return AMLA_ERR_WORKSPACE;
    if ((int64_t)list_len < 2 * ((int64_t)num_reqs + kPlanSlack * params->workers)) return AMLA_ERR_LIST;
    PlanArgs a;
    a.lengths = d_lengths;
    a.counts = d_counts;
    a.offsets = d_offsets;
    a.work = d_work;
    a.header = (int32_t *)d_workspace;
    a.reqs = num_reqs;
    a.bt_cols = bt_cols;
    a.rows = params->rows_per_req;
    a.mtile = params->mtile;
    a.workers = params->workers;
    a.min_pages = ceil_div(params->min_split_tokens, kPage);
    a.max_splits = params->max_splits;
    a.mode = params->mode;
    a.list_len = list_len;
    a.split_cost = params->split_cost_pages;
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, (hipStream_t)stream, a);
    return hipGetLastError() == hipSuccess ? AMLA_OK : AMLA_ERR_HIP;
}

static int decode_launch(const uint8_t *d_q, const uint8_t *d_kv, int64_t pool_pages,
                         const int32_t *d_block_table, int32_t bt_stride,
                         const int32_t *d_lengths, int32_t num_reqs,
                         const amla_plan_params *params, float bmm1_scale, float bmm2_scale,
                         const int32_t *d_counts, const int32_t *d_offsets,
                         const int32_t *d_work, int32_t list_len, void *d_workspace,
                         size_t ws_bytes, const amla_dcp_params *dcp, const int32_t *d_totals,
                         void *stream)
{
    if (dcp && (dcp->heads < 1 || dcp->causal < 0 || dcp->causal > 1 || dcp->world < 1 ||
                dcp->rank < 0 || dcp->rank >= dcp->world || dcp->interleave < 1 ||
                (int64_t)dcp->interleave * dcp->world > (1 << 30) || !params ||
                params->rows_per_req % dcp->heads != 0 ||
                (dcp->causal && num_reqs > 0 && !d_totals)))
        return AMLA_ERR_INVALID;
    if (!params_ok(params) || num_reqs < 0 || num_reqs > AMLA_MAX_REQS || pool_pages < 1 ||
        bt_stride < 1 || !d_kv || !d_offsets || !d_work || !d_workspace ||
        (num_reqs > 0 && (!d_q || !d_block_table || !d_lengths || !d_counts)) ||
        !std::isfinite(bmm1_scale) || !(bmm1_scale > 0.f) || !std::isfinite(bmm2_scale))
        return AMLA_ERR_INVALID;
    const WsLayout lay = ws_layout(num_reqs, params->rows_per_req, params->workers);
    if (ws_bytes < lay.total) return AMLA_ERR_WORKSPACE;
    if ((int64_t)list_len < 2 * ((int64_t)num_reqs + kPlanSlack * params->workers)) return AMLA_ERR_LIST;
    if (num_reqs == 0) return AMLA_OK;
    DecodeArgs a;
    a.pool_pages = pool_pages;
    a.bt_stride = bt_stride;
    a.reqs = num_reqs;
    a.rows = params->rows_per_req;
    a.mtile = params->mtile;
    a.workers = params->workers;
    a.list_len = list_len;
    a.score_scale = bmm1_scale * kLog2e;
    a.out_scale = bmm2_scale;
    a.totals = d_totals;
    a.causal = dcp ? dcp->causal : 0;
    a.heads = dcp ? dcp->heads : 1;
    a.k_tokens = dcp ? params->rows_per_req / dcp->heads : 1;
    a.cp_world = dcp ? dcp->world : 1;
    a.cp_rank = dcp ? dcp->rank : 0;
    a.cp_interleave = dcp ? dcp->interleave : 1;
    int32_t *hdr = (int32_t *)d_workspace;
    float *part = (float *)((char *)d_workspace + lay.partial_off);
    float *lse = (float *)((char *)d_workspace + lay.lse_off);
    const dim3 grid(params->workers);
    hipStream_t st = (hipStream_t)stream;
#define AMLA_DECODE_ARGS d_q, d_kv, d_block_table, d_lengths, d_counts, d_offsets, d_work, hdr, part, lse, a
    switch (params->mtile) {
    case 32:
    case 64:
        if (launch_decode_stream(params->mtile, grid, st, AMLA_DECODE_ARGS) != hipSuccess)
            return AMLA_ERR_HIP;
        break;
    default:
        if (launch_decode128(grid, st, AMLA_DECODE_ARGS) != hipSuccess) return AMLA_ERR_HIP;
        break;
    }
#undef AMLA_DECODE_ARGS
    return hipGetLastError() == hipSuccess ? AMLA_OK : AMLA_ERR_HIP;
}

int amla_folded_decode(const uint8_t *d_q, const uint8_t *d_kv, int64_t pool_pages,
                       const int32_t *d_block_table, int32_t bt_stride, const int32_t *d_lengths,
                       int32_t num_reqs, const amla_plan_params *params, float bmm1_scale,
                       float bmm2_scale, const int32_t *d_counts, const int32_t *d_offsets,
                       const int32_t *d_work, int32_t list_len, void *d_workspace,
                       size_t ws_bytes, void *stream)
{
    return decode_launch(d_q, d_kv, pool_pages, d_block_table, bt_stride, d_lengths, num_reqs,
                         params, bmm1_scale, bmm2_scale, d_counts, d_offsets, d_work, list_len,
                         d_workspace, ws_bytes, nullptr, nullptr, stream);
}

int amla_folded_decode_dcp(const uint8_t *d_q, const uint8_t *d_kv, int64_t pool_pages,
                           const int32_t *d_block_table, int32_t bt_stride,
                           const int32_t *d_lengths, int32_t num_reqs,
                           const amla_plan_params *params, float bmm1_scale, float bmm2_scale,
                           const int32_t *d_counts, const int32_t *d_offsets,
                           const int32_t *d_work, int32_t list_len, void *d_workspace,
                           size_t ws_bytes, const amla_dcp_params *dcp, const int32_t *d_totals,
                           void *stream)
{
    if (!dcp) return AMLA_ERR_INVALID;
    return decode_launch(d_q, d_kv, pool_pages, d_block_table, bt_stride, d_lengths, num_reqs,
                         params, bmm1_scale, bmm2_scale, d_counts, d_offsets, d_work, list_len,
                         d_workspace, ws_bytes, dcp, d_totals, stream);
}

int amla_merge_sources(int32_t n_src, const uint16_t *d_rows, const float *d_lse, int64_t n_rows,
                       uint16_t *d_out, float *d_lse_out, void *stream)
{
    if (n_src < 1 || n_src > kMaxSources || n_rows < 0 ||
        (n_rows > 0 && (!d_rows || !d_lse || !d_out || !d_lse_out)) ||
        ((uintptr_t)d_rows & 15) || ((uintptr_t)d_out & 15) ||
        n_rows > ((int64_t)1 << 40) / n_src)
        return AMLA_ERR_INVALID;
    if (n_rows == 0) return AMLA_OK;
    hipLaunchKernelGGL(merge_sources_kernel, dim3((unsigned)((n_rows + 3) / 4)), dim3(256), 0,
                       (hipStream_t)stream, d_rows, d_lse, (int)n_src, n_rows, d_out, d_lse_out);
    return hipGetLastError() == hipSuccess ? AMLA_OK : AMLA_ERR_HIP;
}

int amla_build_query_cache(const uint16_t *d_q, const uint16_t *d_w_uk, const uint16_t *d_kv_c,
                           const uint16_t *d_k_pe, const int64_t *d_positions,
                           const float *d_cos_sin, int32_t max_pos,
                           const int64_t *d_slot_mapping, int32_t n_tokens, int32_t heads,
                           int32_t neox, float q_scale, float k_scale, uint8_t *d_q_out,
                           uint8_t *d_kv_cache, int64_t pool_pages, int32_t *d_status,
                           void *stream)
{
    if (n_tokens < 0 || heads < 1 || heads > 1024 || max_pos < 1 || pool_pages < 0 ||
        (neox != 0 && neox != 1) || !std::isfinite(q_scale) || !(q_scale > 0.f) ||
        !std::isfinite(k_scale) || !(k_scale > 0.f) ||
        (n_tokens > 0 && (!d_q || !d_w_uk || !d_kv_c || !d_k_pe || !d_positions || !d_cos_sin ||
                          !d_slot_mapping || !d_q_out || !d_kv_cache)) ||
        ((uintptr_t)d_q & 15) || ((uintptr_t)d_w_uk & 15) || ((uintptr_t)d_kv_c & 15) ||
        ((uintptr_t)d_q_out & 3) || ((uintptr_t)d_kv_cache & 7))
        return AMLA_ERR_INVALID;
    if (n_tokens == 0) return AMLA_OK;
    BuildArgs a;
    a.q = d_q;
    a.w_uk = d_w_uk;
    a.kv_c = d_kv_c;
    a.k_pe = d_k_pe;
    a.positions = d_positions;
    a.cos_sin = d_cos_sin;
    a.slots = d_slot_mapping;
    a.q_out = d_q_out;
    a.cache = d_kv_cache;
    a.status = d_status;
    a.pool_pages = pool_pages;
    a.n = n_tokens;
    a.heads = heads;
    a.neox = neox;
    a.max_pos = max_pos;
    a.q_inv = 1.0f / q_scale;
    a.k_inv = 1.0f / k_scale;
    // 32-token query blocks (each W_UK fragment serves two MFMAs) when they give at least
    // three quarters of the 256 compute units a block, else 16-token blocks
    const int64_t qblocks32 = (int64_t)((n_tokens + 2 * kQbTokens - 1) / (2 * kQbTokens)) * heads;
    const bool wide = qblocks32 >= 192;
    const int64_t qblocks =
        wide ? qblocks32 : (int64_t)((n_tokens + kQbTokens - 1) / kQbTokens) * heads;
    const int64_t cblocks = (n_tokens + 3) / 4;
    if (qblocks + cblocks > 0x7FFFFFFF) return AMLA_ERR_INVALID;
    a.query_blocks = (int32_t)qblocks;
    if (wide)
        hipLaunchKernelGGL(build_query_cache_kernel<2 * kQbTokens>, dim3((unsigned)(qblocks + cblocks)),
                           dim3(256), 0, (hipStream_t)stream, a);
    else
        hipLaunchKernelGGL(build_query_cache_kernel<kQbTokens>, dim3((unsigned)(qblocks + cblocks)),
                           dim3(256), 0, (hipStream_t)stream, a);
    return hipGetLastError() == hipSuccess ? AMLA_OK : AMLA_ERR_HIP;
}

int amla_combine(const void *d_workspace, size_t ws_bytes, const int32_t *d_counts,
                 const int32_t *d_offsets, int32_t num_reqs, const amla_plan_params *params,
                 int32_t compute_units, uint16_t *d_out, float *d_lse, void *stream)
{
    if (!params_ok(params) || num_reqs < 0 || num_reqs > AMLA_MAX_REQS || compute_units < 1 ||
        !d_workspace || (num_reqs > 0 && (!d_counts || !d_offsets || !d_out || !d_lse)))
        return AMLA_ERR_INVALID;
    const WsLayout lay = ws_layout(num_reqs, params->rows_per_req, params->workers);
    if (ws_bytes < lay.total) return AMLA_ERR_WORKSPACE;
    if (num_reqs == 0) return AMLA_OK;
    const int64_t rows = (int64_t)num_reqs * params->rows_per_req;
    int32_t bands = 1;
    amla_reducer_bands((int32_t)rows, compute_units, &bands);
    CombineArgs a;
    a.partial = (const float *)((const char *)d_workspace + lay.partial_off);
    a.lse = (const float *)((const char *)d_workspace + lay.lse_off);
    a.counts = d_counts;
    a.offsets = d_offsets;
    a.out = d_out;
    a.out_lse = d_lse;
    a.reqs = num_reqs;
    a.rows = params->rows_per_req;
    a.bands = bands;
    a.slots = num_reqs + kPlanSlack * params->workers;
    hipLaunchKernelGGL(combine_kernel, dim3((unsigned)(rows * bands)), dim3(64), 0,
                       (hipStream_t)stream, a);
    return hipGetLastError() == hipSuccess ? AMLA_OK : AMLA_ERR_HIP;
}

int amla_combine_uv(const void *d_workspace, size_t ws_bytes, const int32_t *d_counts,
                    const int32_t *d_offsets, int32_t num_reqs, const amla_plan_params *params,
                    int32_t heads, const uint16_t *d_w_uv, uint16_t *d_attn_out,
                    uint16_t *d_out, float *d_lse, void *stream)
{
    if (!params_ok(params) || num_reqs < 0 || num_reqs > AMLA_MAX_REQS || heads < 1 ||
        params->rows_per_req % heads != 0 || !d_workspace ||
        (num_reqs > 0 && (!d_counts || !d_offsets || !d_w_uv || !d_attn_out)) ||
        ((uintptr_t)d_w_uv & 15) || ((uintptr_t)d_attn_out & 7) || ((uintptr_t)d_out & 7))
        return AMLA_ERR_INVALID;
    const WsLayout lay = ws_layout(num_reqs, params->rows_per_req, params->workers);
    if (ws_bytes < lay.total) return AMLA_ERR_WORKSPACE;
    if (num_reqs == 0) return AMLA_OK;
    UvArgs a;
    a.partial = (const float *)((const char *)d_workspace + lay.partial_off);
    a.lse = (const float *)((const char *)d_workspace + lay.lse_off);
    a.counts = d_counts;
    a.offsets = d_offsets;
    a.w_uv = d_w_uv;
    a.attn_out = d_attn_out;
    a.out = d_out;
    a.out_lse = d_lse;
    a.reqs = num_reqs;
    a.rows = params->rows_per_req;
    a.heads = heads;
    a.k = params->rows_per_req / heads;
    a.slots = num_reqs + kPlanSlack * params->workers;
    const int64_t per_head = (int64_t)num_reqs * a.k;
    // 32-row tiles (each wave's W_UV fragments serve twice the rows) when they give at least
    // three quarters of the 256 compute units a workgroup (c3's 224 tiles: 17-18 us against
    // 21-24 us as 448 16-row tiles), else 16-row tiles when those fill them, else 8-row tiles
    const int64_t tiles32 = (per_head + 2 * kUvRows - 1) / (2 * kUvRows);
    const int64_t tiles16 = (per_head + kUvRows - 1) / kUvRows;
    if (tiles32 * heads >= 192)
        hipLaunchKernelGGL(combine_uv_kernel<2 * kUvRows>, dim3((unsigned)tiles32, (unsigned)heads),
                           dim3(512), 0, (hipStream_t)stream, a);
    else if (tiles16 * heads >= 256)
        hipLaunchKernelGGL(combine_uv_kernel<kUvRows>, dim3((unsigned)tiles16, (unsigned)heads),
                           dim3(512), 0, (hipStream_t)stream, a);
    else
        hipLaunchKernelGGL(combine_uv_kernel<kUvRows / 2>,
                           dim3((unsigned)((per_head + kUvRows / 2 - 1) / (kUvRows / 2)),
                                (unsigned)heads),
                           dim3(512), 0, (hipStream_t)stream, a);
    return hipGetLastError() == hipSuccess ? AMLA_OK : AMLA_ERR_HIP;
}

int amla_folded_decode_noalloc(const uint8_t *d_q, const uint8_t *d_kv, int64_t pool_pages,
                               const int32_t *d_block_table, int32_t bt_stride,
                               const int32_t *d_lengths, int32_t num_reqs,
                               const amla_plan_params *params, float bmm1_scale,
                               float bmm2_scale, int32_t compute_units, uint16_t *d_out,
                               float *d_lse, int32_t *d_status, void *stream)
{
    // every argument is checked before the first launch, so an error enqueues nothing
    if (!params_ok(params) || num_reqs < 0 || num_reqs > AMLA_MAX_REQS || pool_pages < 1 ||
        bt_stride < 1 || compute_units < 1 || !d_kv ||
        (num_reqs > 0 && (!d_q || !d_block_table || !d_lengths || !d_out || !d_lse)) ||
        !std::isfinite(bmm1_scale) || !(bmm1_scale > 0.f) || !std::isfinite(bmm2_scale))
        return AMLA_ERR_INVALID;
    const ScratchLayout l = scratch_layout(num_reqs, params->rows_per_req, params->workers);
    if (l.total > kScratchBytes) return AMLA_ERR_WORKSPACE;
    void *base = nullptr;
    const int rc = scratch_address(&base);
    if (rc != AMLA_OK) return rc;
    uint8_t *b = (uint8_t *)base;
    int32_t *counts = (int32_t *)(b + l.counts), *offsets = (int32_t *)(b + l.offsets);
    int32_t *work = (int32_t *)(b + l.work);
    void *ws = b + l.workspace;
    // the plan rewrites the header (status included), the counts, offsets and the whole
    // work list, and the decode writes every planned slot the merge reads: nothing left
    // by an earlier call is read
    int st = amla_plan_splits(d_lengths, num_reqs, bt_stride, params, counts, offsets, work,
                              l.list_len, ws, l.ws_bytes, stream);
    if (st == AMLA_OK)
        st = amla_folded_decode(d_q, d_kv, pool_pages, d_block_table, bt_stride, d_lengths,
                                num_reqs, params, bmm1_scale, bmm2_scale, counts, offsets, work,
                                l.list_len, ws, l.ws_bytes, stream);
    if (st == AMLA_OK)
        st = amla_combine(ws, l.ws_bytes, counts, offsets, num_reqs, params, compute_units,
                          d_out, d_lse, stream);
    if (st == AMLA_OK && d_status) {
        hipLaunchKernelGGL(copy_status_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream,
                           (const int32_t *)ws, d_status);
        st = hipGetLastError() == hipSuccess ? AMLA_OK : AMLA_ERR_HIP;
    }
    return st;
}

const char *amla_status_string(int status)
{
    switch (status) {
    case AMLA_OK: return "ok";
    case AMLA_ERR_INVALID: return "invalid argument";
    case AMLA_ERR_WORKSPACE: return "workspace too small";
    case AMLA_ERR_LIST: return "work list too short";
    case AMLA_ERR_HIP: return "kernel launch failed";
    default: break;
    }
    if (status > 0) {
        if (status & AMLA_DEV_BAD_LENGTH) return "device: bad length (plan is empty)";
        if (status & AMLA_DEV_BAD_PAGE) return "device: block-table entry out of range";
        if (status & AMLA_DEV_BAD_ITEM) return "device: work item or plan does not match";
        if (status & AMLA_DEV_BAD_POSITION) return "device: position outside the rotary table";
    }
    return "unknown status";
}

}  // extern "C"
