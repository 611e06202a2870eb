// Folded split-KV absorbed-MLA decode for MI355X (gfx950): plan, decode and combine
// kernels, and the steps next to them, behind the C ABI declared in include/amla.h.
//
// Method (page "vllm.models.kimi_k3.nvidia.specialized_decode.drafter.attention", module
// docstring; page "...cutedsl.mla.balanced", module docstring): MQA over one latent head
// of 576 FP8 dims per token (value = the first 512), the k draft tokens of a request
// folded into its head axis, each request's keys cut into planned splits that produce
// FP32 partials and a log2 LSE, and a reducer merging the splits into BF16 rows.
//
// gfx950 mapping (this file's design, not the pages'):
//   * plan    one 256-thread workgroup.  Up to 256 requests: every wave derives the chunk
//             and the scans by itself (DPP, no barrier), then each thread places one run of
//             equal-size splits by counting the runs that sort before it.  More requests:
//             block reductions and scans, a rank or bitonic sort of the runs.
//   * decode  one persistent 256-thread workgroup per CU.  A work unit is (request, split,
//             row tile of MT rows).  Pages (64 tokens x 576 B) go HBM -> LDS by
//             global_load_lds_dwordx4 into a ring of four page slots.  Per page and 32 rows:
//               S^T[64 keys x 32 rows] = K Q^T : 18 x v_mfma_f32_32x32x64_f8f6f4, K read
//                                                 from LDS, Q^T resident in VGPRs;
//               softmax in log2 units, lazy row max (rescale O only when the page max
//               exceeds it by more than 2^TAU), P = exp2(t - m) to E4M3 in-lane;
//               O^T[dims x 32 rows] += V^T P^T : V^T fragments come from LDS through
//                                                 ds_read_b64_tr_b8 transposed reads.
//             The accumulator layout puts one query row per lane, so the running max,
//             sum, rescale and the per-row key limit (causal mask over a DCP shard) are
//             lane-local; one lane-swap merges the two key halves.  Three kernels:
//             decode32 (MT = 32: wave pairs on alternate pages), decode64 (MT = 64: pairs
//             on alternate pages, partners swapping P) and decode128 (MT = 128: the four
//             waves on every page, partners swapping P).
//   * combine one wave per (row, band); merges the splits of a row with exp2 weights.
//   * combine_uv  the merge fused with the W_UV up-projection (BF16 MFMA).
//   * merge_sources  a head owner's merge of rows computed on several DCP shards.
//   * build_query_cache  the step before the decode: the absorbed query (W_UK_T on BF16
//             MFMA, rotary embedding, E4M3 cast) and the new tokens' cache rows.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>
#include <type_traits>

#include "../../include/amla.h"

namespace {

constexpr int kPage = AMLA_PAGE;
constexpr int kKDim = AMLA_KDIM;
constexpr int kVDim = AMLA_VDIM;
constexpr int kPageBytes = kPage * kKDim;      // 36864
constexpr int kSlots = 4;                      // LDS page ring
constexpr int kDecodeThreads = 256;            // 4 waves
constexpr int kChunksPerWave = kPageBytes / (4 * 1024);  // 9 x 1 KiB DMA per wave per page
constexpr int kHeaderBytes = 256;
constexpr int kPlanThreads = 256;
// A plan may use up to kPlanSlack * W units (see the rebalancing rule in the plan kernels):
// the work list and the workspace hold num_reqs + kPlanSlack * workers splits.
constexpr int kPlanSlack = 2;
constexpr int kMaxRuns = 2 * AMLA_MAX_REQS;    // two split-size runs per request
constexpr float kLog2e = 1.4426950408889634f;
// Lazy max: the running row max is only raised when a page's max exceeds it by more
// than 2^kTau, so p = 2^(t - m) <= 2^kTau; P is scaled by 2^kPScale before the E4M3
// cast (kTau + kPScale <= 8 keeps it <= 256 < 448) to keep small weights out of the
// subnormal range.
constexpr float kTau = 2.0f;
constexpr float kPScale = 6.0f;

// Workspace header words (int32).
enum HeaderWord {
    kHdrStatus = 0,
    kHdrItems = 1,
    kHdrRows = 2,
    kHdrMtile = 3,
    kHdrWorkers = 4,
    kHdrMode = 5,
    kHdrReqs = 6,
    kHdrPlanned = 7,  // 0x600DF00D after a successful plan
};
constexpr int kPlannedMagic = 0x600DF00D;

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
#define LDS_AS __attribute__((address_space(3)))
#define CONST_AS __attribute__((address_space(4)))

// A uniform read of memory that no kernel of this file writes while reading it: through
// the constant address space it is always a scalar load (lgkmcnt), never a vector load,
// whose vmcnt wait would also wait for the page DMAs in flight.
template <typename T>
__device__ __forceinline__ T ldc(const T *p)
{
    return *(const CONST_AS T *)p;
}

// f(std::integral_constant<int, I>) for I in [I0, N): a loop whose index is a constant in
// every step, so register arrays indexed by it stay in registers.
template <int I0, int N, typename F>
__device__ __forceinline__ void static_for(F &&f)
{
    if constexpr (I0 < N) {
        f(std::integral_constant<int, I0>{});
        static_for<I0 + 1, N>(f);
    }
}

struct WsLayout {
    size_t partial_off;  // FP32 [slots][M][512]
    size_t lse_off;      // FP32 [slots][M]
    size_t total;
};

__host__ __device__ inline WsLayout ws_layout(int64_t reqs, int64_t rows, int64_t workers)
{
    WsLayout w;
    const int64_t slots = reqs + kPlanSlack * workers;
    w.partial_off = kHeaderBytes;
    w.lse_off = w.partial_off + (size_t)(slots * rows * kVDim * 4);
    w.total = w.lse_off + (size_t)(((slots * rows * 4) + 255) / 256 * 256);
    return w;
}

__host__ __device__ inline int ceil_div(int a, int b) { return (a + b - 1) / b; }

// ------------------------------------------------------------------ block utilities

template <typename T>
__device__ inline T wave_sum(T v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

template <typename T>
__device__ inline T wave_max(T v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        T w = __shfl_xor(v, o);
        v = w > v ? w : v;
    }
    return v;
}

// All-lane reductions of a wave without LDS traffic: DPP within rows of 16 lanes, then
// v_permlane16_swap / v_permlane32_swap across rows.  64-bit values move as two halves.
template <int CTRL>
__device__ __forceinline__ int64_t dpp64(int64_t v)
{
    const int lo = __builtin_amdgcn_mov_dpp((int)v, CTRL, 0xf, 0xf, false);
    const int hi = __builtin_amdgcn_mov_dpp((int)(v >> 32), CTRL, 0xf, 0xf, false);
    return ((int64_t)hi << 32) | (uint32_t)lo;
}

template <bool MAX>
__device__ __forceinline__ int64_t op64(int64_t a, int64_t b)
{
    return MAX ? (a > b ? a : b) : a + b;
}

template <bool MAX>
__device__ int64_t wave_all64(int64_t v)
{
    v = op64<MAX>(v, dpp64<0x128>(v));   // row_ror:8
    v = op64<MAX>(v, dpp64<0x124>(v));   // row_ror:4
    v = op64<MAX>(v, dpp64<0x4e>(v));    // quad_perm [2,3,0,1]
    v = op64<MAX>(v, dpp64<0xb1>(v));    // quad_perm [1,0,3,2]
    {
        const auto lo = __builtin_amdgcn_permlane16_swap((uint32_t)v, (uint32_t)v, false, false);
        const auto hi = __builtin_amdgcn_permlane16_swap((uint32_t)(v >> 32), (uint32_t)(v >> 32), false, false);
        v = op64<MAX>(((int64_t)hi[0] << 32) | lo[0], ((int64_t)hi[1] << 32) | lo[1]);
    }
    {
        const auto lo = __builtin_amdgcn_permlane32_swap((uint32_t)v, (uint32_t)v, false, false);
        const auto hi = __builtin_amdgcn_permlane32_swap((uint32_t)(v >> 32), (uint32_t)(v >> 32), false, false);
        v = op64<MAX>(((int64_t)hi[0] << 32) | lo[0], ((int64_t)hi[1] << 32) | lo[1]);
    }
    return v;
}

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
};

__device__ inline int64_t pages_of(int32_t len) { return ((int64_t)len + kPage - 1) / kPage; }

// Sort key of a run of equal-size splits of request r: size descending, then r ascending.
__device__ inline uint64_t run_key(int64_t size, int32_t r)
{
    return ((uint64_t)(0x7FFFFFFFll - size) << 32) | (uint32_t)r;
}

// Reduces four values over the workgroup at once (max, max, sum, sum).
__device__ void block_reduce4(int64_t &mx0, int64_t &mx1, int64_t &sm0, int64_t &sm1,
                              int64_t (*scratch)[4])
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    mx0 = wave_all64<true>(mx0);
    mx1 = wave_all64<true>(mx1);
    sm0 = wave_all64<false>(sm0);
    sm1 = wave_all64<false>(sm1);
    if (lane == 0) {
        scratch[wave][0] = mx0;
        scratch[wave][1] = mx1;
        scratch[wave][2] = sm0;
        scratch[wave][3] = sm1;
    }
    __syncthreads();
    mx0 = mx1 = sm0 = sm1 = 0;
    for (int w = 0; w < kPlanThreads / 64; ++w) {
        mx0 = scratch[w][0] > mx0 ? scratch[w][0] : mx0;
        mx1 = scratch[w][1] > mx1 ? scratch[w][1] : mx1;
        sm0 += scratch[w][2];
        sm1 += scratch[w][3];
    }
}

constexpr int kRankSortRuns = kPlanThreads;   // rank sort up to this many runs, else bitonic

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(PlanArgs a)
{
    __shared__ int32_t pg[AMLA_MAX_REQS];            // pages per request
    __shared__ int32_t cnt[AMLA_MAX_REQS];           // splits per request
    __shared__ uint64_t keys[kMaxRuns];              // run keys (sorted in place: bitonic)
    __shared__ uint64_t ranked[kRankSortRuns];       // run keys in order (rank sort)
    __shared__ int64_t red4[kPlanThreads / 64][4];
    __shared__ int32_t red32[kPlanThreads / 64];
    __shared__ int32_t ok[2][16];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int R = a.reqs;
    const int64_t mt = ceil_div(a.rows, a.mtile);
    const int64_t budget = (int64_t)a.workers / mt;  // most splits the workers take at once
    const int64_t budget2 = (int64_t)kPlanSlack * a.workers / mt;

    // 1. pages per request, validity, longest request, total pages, non-empty requests
    int64_t bad = 0, pmax = 0, total = 0, nz = 0;
    for (int r = tid; r < R; r += kPlanThreads) {
        const int32_t L = a.lengths[r];
        const int64_t p = pages_of(L);
        const bool b = L < 0 || p > a.bt_cols;
        bad |= b;
        pg[r] = b ? 0 : (int32_t)p;
        pmax = p > pmax ? p : pmax;
        total += b ? 0 : p;
        nz += (!b && p > 0);
    }
    block_reduce4(bad, pmax, total, nz, red4);

    // 2. BALANCED: the smallest chunk c with sum_r ceil(pages_r / c) <= budget.  Since
    //    total/c <= sum <= total/c + nz, it lies in [ceil(total/budget),
    //    ceil(total/(budget - nz))]; a 16-way search (one candidate per wave) narrows that.
    // the smallest chunk with sum_r ceil(pages_r / c) <= b, at least the minimum split
    auto search = [&](int64_t b) {
        int64_t chunk;
        __syncthreads();   // the candidate flags of an earlier search are read by now
        if (b < nz) {
            chunk = pmax;                         // no chunk fits: one split per request
        } else {
            int64_t lo = (total + b - 1) / b, hi = pmax;
            if (b > nz) {
                const int64_t h = (total + (b - nz) - 1) / (b - nz);
                hi = h < hi ? h : hi;
            }
            lo = lo < 1 ? 1 : (lo > hi ? hi : lo);
            constexpr int kCand = 16, kPerWave = kCand / (kPlanThreads / 64);
            int round = 0;
            while (lo < hi) {
                const int64_t span = hi - lo;
#pragma unroll
                for (int k = 0; k < kPerWave; ++k) {
                    const int cand = wave * kPerWave + k;
                    const uint32_t c = (uint32_t)(lo + span * cand / kCand);
                    int64_t u = 0;
                    for (int r = lane; r < R; r += 64) u += ((uint32_t)pg[r] + c - 1u) / c;
                    u = wave_all64<false>(u);
                    if (lane == 0) ok[round & 1][cand] = u <= b;
                }
                __syncthreads();
                int first = -1;
                for (int w = kCand - 1; w >= 0; --w)
                    if (ok[round & 1][w]) first = w;
                if (first >= 0) {
                    const int64_t cf = lo + span * first / kCand;
                    const int64_t cp = first > 0 ? lo + span * (first - 1) / kCand + 1 : lo;
                    hi = cf;
                    lo = cp < cf ? cp : cf;
                } else {
                    lo = lo + span * (kCand - 1) / kCand + 1;
                }
                ++round;
            }
            chunk = hi;
        }
        return chunk > a.min_pages ? chunk : (int64_t)a.min_pages;
    };
    int64_t chunk = 1, fixed = 1;
    if (!bad && a.mode == AMLA_PLAN_BALANCED && pmax > 0) {
        chunk = search(budget);
        // rebalance (see plan_small_kernel): the longest split against the mean per worker
        int64_t longest = 0;
        for (int r = tid; r < R; r += kPlanThreads) {
            const uint32_t p = (uint32_t)pg[r];
            if (p == 0) continue;
            uint32_t cc = (p + (uint32_t)chunk - 1u) / (uint32_t)chunk;
            cc = cc < (uint32_t)a.max_splits ? cc : (uint32_t)a.max_splits;
            const int64_t sz = (p + cc - 1u) / cc;
            longest = sz > longest ? sz : longest;
        }
        longest = wave_all64<true>(longest);
        if (lane == 0) red32[wave] = (int32_t)longest;
        __syncthreads();
        longest = 0;
        for (int w = 0; w < kPlanThreads / 64; ++w) longest = red32[w] > longest ? red32[w] : longest;
        __syncthreads();   // red32 is reused below
        if (4 * longest * (int64_t)a.workers > 5 * mt * total) chunk = search(budget2);
    } else if (!bad && a.mode == AMLA_PLAN_FIXED) {
        fixed = R > 0 ? (int64_t)a.workers / ((int64_t)R * mt) : 1;
        fixed = fixed < 1 ? 1 : (fixed > a.max_splits ? a.max_splits : fixed);
    }

    // 3. counts and their exclusive scan: thread t owns requests [t*per, (t+1)*per)
    const int per = ceil_div(R > 0 ? R : 1, kPlanThreads);
    int32_t mine = 0;
    for (int i = 0; i < per; ++i) {
        const int r = tid * per + i;
        if (r >= R) break;
        const uint32_t p = (uint32_t)pg[r];
        int64_t c = 0;
        if (!bad && p > 0) {
            if (a.mode == AMLA_PLAN_BALANCED) {
                c = (p + (uint32_t)chunk - 1u) / (uint32_t)chunk;
                c = c < a.max_splits ? c : a.max_splits;
            } else {
                c = (int64_t)p < fixed ? (int64_t)p : fixed;
            }
        }
        cnt[r] = (int32_t)c;
        a.counts[r] = (int32_t)c;
        mine += (int32_t)c;
    }
    int32_t n_items = 0;
    int32_t run = block_exclusive_scan(mine, red32, &n_items);
    for (int i = 0; i < per; ++i) {
        const int r = tid * per + i;
        if (r >= R) break;
        a.offsets[r] = run;
        run += cnt[r];
    }
    if (tid == 0) a.offsets[R] = n_items;

    // 4. runs of equal-size splits, (q+1) x rem from s = 0 then q x (c-rem) from s = rem,
    //    keyed (size descending, request ascending), sorted ascending
    const int runs = 2 * R;
    const uint64_t *sorted;
    auto key_of = [&](int x) -> uint64_t {
        const int r = x >> 1;
        const int c = cnt[r];
        if (c == 0) return ~0ull;
        const int q = pg[r] / c, rem = pg[r] % c;
        if ((x & 1) == 0) return rem > 0 ? run_key(q + 1, r) : ~0ull;
        return run_key(q, r);
    };
    if (runs <= kRankSortRuns) {
        const uint64_t mykey = tid < runs ? key_of(tid) : ~0ull;
        if (tid < runs) keys[tid] = mykey;
        __syncthreads();
        if (tid < runs && mykey != ~0ull) {
            int rank = 0;
            for (int y = 0; y < runs; ++y) rank += keys[y] < mykey;
            ranked[rank] = mykey;
        }
        // empty runs sort last: fill the tail so the positions below see count 0
        int nonempty = 0;
        {
            int64_t z0 = 0, z1 = 0, e0 = (tid < runs && mykey != ~0ull), e1 = 0;
            block_reduce4(z0, z1, e0, e1, red4);
            nonempty = (int)e0;
        }
        for (int i = nonempty + tid; i < kRankSortRuns; i += kPlanThreads) ranked[i] = ~0ull;
        __syncthreads();
        sorted = ranked;
    } else {
        int n = 2;
        while (n < runs) n <<= 1;
        for (int x = tid; x < n; x += kPlanThreads) keys[x] = x < runs ? key_of(x) : ~0ull;
        __syncthreads();
        for (int k = 2; k <= n; k <<= 1) {
            for (int j = k >> 1; j > 0; j >>= 1) {
                for (int i = tid; i < n; i += kPlanThreads) {
                    const int ixj = i ^ j;
                    if (ixj > i) {
                        const uint64_t x = keys[i], y = keys[ixj];
                        const bool up = (i & k) == 0;
                        if ((x > y) == up) {
                            keys[i] = y;
                            keys[ixj] = x;
                        }
                    }
                }
                __syncthreads();
            }
        }
        sorted = keys;
    }

    // 5. positions of the runs in sorted order, then the (r, s) pairs
    int n_sorted = 2;
    while (n_sorted < runs) n_sorted <<= 1;
    if (runs <= kRankSortRuns) n_sorted = kRankSortRuns;
    const int per_run = n_sorted / kPlanThreads > 0 ? n_sorted / kPlanThreads : 1;
    constexpr int kMaxPerRun = kMaxRuns / kPlanThreads;
    int32_t cnt_local[kMaxPerRun], s0_local[kMaxPerRun], r_local[kMaxPerRun];
    int32_t my_items = 0;
    for (int i = 0; i < per_run; ++i) {
        const int idx = tid * per_run + i;
        cnt_local[i] = 0;
        s0_local[i] = 0;
        r_local[i] = 0;
        if (idx >= n_sorted) continue;
        const uint64_t key = sorted[idx];
        if (key == ~0ull) continue;
        const int64_t size = 0x7FFFFFFFll - (int64_t)(key >> 32);
        const int32_t r = (int32_t)(key & 0xFFFFFFFFu);
        const int32_t c = cnt[r];
        const int32_t q = pg[r] / c, rem = pg[r] % c;
        if (rem > 0 && size == q + 1) {
            cnt_local[i] = rem;
            s0_local[i] = 0;
        } else {
            cnt_local[i] = c - rem;
            s0_local[i] = rem;
        }
        r_local[i] = r;
        my_items += cnt_local[i];
    }
    int32_t total_items = 0;
    int32_t pos = block_exclusive_scan(my_items, red32, &total_items);
    for (int i = 0; i < per_run && 2 * total_items <= a.list_len; ++i) {
        for (int32_t e = 0; e < cnt_local[i]; ++e) {
            a.work[2 * (pos + e)] = r_local[i];
            a.work[2 * (pos + e) + 1] = s0_local[i] + e;
        }
        pos += cnt_local[i];
    }
    for (int i = 2 * total_items + tid; i < a.list_len; i += kPlanThreads) a.work[i] = -1;

    if (tid == 0) {
        a.header[kHdrStatus] = bad ? AMLA_DEV_BAD_LENGTH : 0;
        a.header[kHdrItems] = n_items;
        a.header[kHdrRows] = a.rows;
        a.header[kHdrMtile] = a.mtile;
        a.header[kHdrWorkers] = a.workers;
        a.header[kHdrMode] = a.mode;
        a.header[kHdrReqs] = R;
        a.header[kHdrPlanned] = kPlannedMagic;
    }
}

// Inclusive scan over the 64 lanes of a wave: DPP row shifts within rows of 16 lanes,
// then the row broadcasts of lanes 15 and 31 into the rows above them.
__device__ __forceinline__ int32_t wave_incl_scan(int32_t v)
{
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, true);   // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, true);   // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, true);   // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, true);   // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15 -> rows 1, 3
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31 -> rows 2, 3
    return v;
}

__device__ __forceinline__ int32_t wave_total(int32_t incl)
{
    return __builtin_amdgcn_readlane(incl, 63);
}

// Plan of up to kSmallReqs requests.  Every wave derives the whole plan summary by itself
// (lane l holds requests l, l+64, l+128, l+192), so the chunk search and the scans need
// no barrier; one barrier publishes the runs, whose list positions the 256 threads then
// compute one run each.  Same result as plan_kernel.
constexpr int kSmallReqs = 256;
constexpr int kSmallPer = kSmallReqs / 64;

__global__ __launch_bounds__(kPlanThreads) void plan_small_kernel(PlanArgs a)
{
    // runs in request order, packed (0x7FFFFFFF - size) << 32 | r << 18 | s0 << 9 | length
    // (s0 = its first split): the order of the packed words is the list order (size
    // descending, then r; a request has one run per size)
    __shared__ uint64_t runs[2 * kSmallReqs];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int R = a.reqs;
    const int64_t mt = ceil_div(a.rows, a.mtile);
    const int64_t budget = (int64_t)a.workers / mt;          // splits W workers take at once
    const int64_t budget2 = (int64_t)kPlanSlack * a.workers / mt;

    // 1. pages per request (every wave reads all lengths); kn = request groups in use
    const int kn = (R + 63) >> 6;
    int32_t pg[kSmallPer];
    int32_t len[kSmallPer];
#pragma unroll
    for (int k = 0; k < kSmallPer; ++k) {
        const int r = lane + 64 * k;
        len[k] = k < kn && r < R ? a.lengths[r] : 0;
    }
    bool bad_l = false;
    int32_t pmax_l = 0, nz_l = 0;
    int64_t total_l = 0;
#pragma unroll
    for (int k = 0; k < kSmallPer; ++k) {
        const int32_t L = len[k];
        const int32_t p = (L >> 6) + ((L & 63) != 0);   // ceil(L / 64) without overflow
        const bool b = L < 0 || p > a.bt_cols;
        bad_l |= b;
        pg[k] = b ? 0 : p;
        pmax_l = pg[k] > pmax_l ? pg[k] : pmax_l;
        total_l += pg[k];
        nz_l += pg[k] > 0;
    }
    const bool bad = __any(bad_l);
    const int64_t pmax = wave_all64<true>(pmax_l);
    const int64_t total = wave_all64<false>(total_l);
    const int64_t nz = wave_all64<false>(nz_l);
    if (bad) {
#pragma unroll
        for (int k = 0; k < kSmallPer; ++k) pg[k] = 0;
    }

    // 2. chunk (BALANCED) or fixed count.  units(c) = sum_r ceil(pages_r / c) falls with c
    //    and total/c <= units(c) <= total/c + nz, so the smallest c with units(c) <= budget
    //    lies in [ceil(total/budget), ceil(total/(budget - nz))]: binary search, trying the
    //    lower bound first (the answer for near-uniform lengths)
    auto units = [&](int64_t c) {
        int64_t u = 0;
#pragma unroll
        for (int k = 0; k < kSmallPer; ++k)
            if (k < kn) u += ((uint32_t)pg[k] + (uint32_t)c - 1u) / (uint32_t)c;
        return wave_all64<false>(u);
    };
    // ceil(x / y) for x >= 0, y > 0, in 32 bits when both fit
    auto cdiv = [](int64_t x, int64_t y) -> int64_t {
        if (x == 0) return 0;
        if ((uint64_t)x <= 0xFFFFFFFFull && (uint64_t)y <= 0xFFFFFFFFull)
            return (int64_t)((uint32_t)(x - 1) / (uint32_t)y) + 1;
        return (x - 1) / y + 1;
    };
    // the smallest chunk with units(c) <= b, at least the minimum split
    auto search = [&](int64_t b) {
        int64_t c;
        if (b < nz) {
            c = pmax;
        } else {
            int64_t lo = cdiv(total, b), hi = pmax;
            if (b > nz) {
                const int64_t h = cdiv(total, b - nz);
                hi = h < hi ? h : hi;
            }
            lo = lo < 1 ? 1 : (lo > hi ? hi : lo);
            if (lo < hi && units(lo) <= b) hi = lo;
            else if (lo < hi) ++lo;
            while (lo < hi) {
                const int64_t mid = lo + (hi - lo) / 2;
                if (units(mid) <= b) hi = mid;
                else lo = mid + 1;
            }
            c = hi;
        }
        return c > a.min_pages ? c : (int64_t)a.min_pages;
    };
    int64_t chunk = 1, fixed = 1;
    if (!bad && a.mode == AMLA_PLAN_BALANCED && pmax > 0) {
        chunk = search(budget);
        // rebalance: when the longest split exceeds the mean work per worker by more than a
        // quarter, plan for twice the workers (about two units per worker)
        int64_t longest = 0;
#pragma unroll
        for (int k = 0; k < kSmallPer; ++k) {
            if (k >= kn || pg[k] == 0) continue;
            const uint32_t p = (uint32_t)pg[k];
            uint32_t cc = (p + (uint32_t)chunk - 1u) / (uint32_t)chunk;
            cc = cc < (uint32_t)a.max_splits ? cc : (uint32_t)a.max_splits;
            const int64_t sz = (p + cc - 1u) / cc;
            longest = sz > longest ? sz : longest;
        }
        longest = wave_all64<true>(longest);
        if (4 * longest * (int64_t)a.workers > 5 * mt * total) chunk = search(budget2);
    } else if (!bad && a.mode == AMLA_PLAN_FIXED) {
        fixed = R > 0 ? (int64_t)a.workers / ((int64_t)R * mt) : 1;
        fixed = fixed < 1 ? 1 : (fixed > a.max_splits ? a.max_splits : fixed);
    }

    // 3. counts, offsets (request order = k-major lane order) and the runs of each request:
    //    (q+1) x rem from s = 0, then q x (c - rem) from s = rem
    int32_t cnt[kSmallPer], off[kSmallPer], rbase[kSmallPer];
    int32_t carry = 0, rcarry = 0;
#pragma unroll
    for (int k = 0; k < kSmallPer; ++k) {
        cnt[k] = off[k] = rbase[k] = 0;
        if (k >= kn) continue;
        const uint32_t p = (uint32_t)pg[k];
        int32_t c = 0;
        if (p > 0) {
            if (a.mode == AMLA_PLAN_BALANCED) {
                const uint32_t cc = (p + (uint32_t)chunk - 1u) / (uint32_t)chunk;
                c = (int32_t)(cc < (uint32_t)a.max_splits ? cc : (uint32_t)a.max_splits);
            } else {
                c = (int32_t)((int64_t)p < fixed ? (int64_t)p : fixed);
            }
        }
        cnt[k] = c;
        const int32_t rem = c > 0 ? (int32_t)(p % (uint32_t)c) : 0;
        const int32_t nruns = (rem > 0) + (c - rem > 0);
        const int32_t ci = wave_incl_scan(c), ri = wave_incl_scan(nruns);
        off[k] = carry + ci - c;
        rbase[k] = rcarry + ri - nruns;
        carry += wave_total(ci);
        rcarry += wave_total(ri);
    }
    const int32_t n_items = carry, n_runs = rcarry;
    if (wave == 0) {
#pragma unroll
        for (int k = 0; k < kSmallPer; ++k) {
            const int r = lane + 64 * k;
            if (r < R) {
                a.counts[r] = cnt[k];
                a.offsets[r] = off[k];
                const int32_t c = cnt[k];
                if (c > 0) {
                    const uint32_t p = (uint32_t)pg[k];
                    const int32_t q = (int32_t)(p / (uint32_t)c), rem = (int32_t)(p % (uint32_t)c);
                    int idx = rbase[k];
                    if (rem > 0)
                        runs[idx++] = ((uint64_t)(0x7FFFFFFF - (q + 1)) << 32) | ((uint32_t)r << 18) |
                                      (uint32_t)rem;
                    if (c - rem > 0)
                        runs[idx] = ((uint64_t)(0x7FFFFFFF - q) << 32) | ((uint32_t)r << 18) |
                                    ((uint32_t)rem << 9) | (uint32_t)(c - rem);
                }
            }
        }
        if (lane == 0) a.offsets[R] = n_items;
    }
    __syncthreads();

    // 4. list position of each run: the lengths of the runs that sort before it; then its
    //    (r, s) pairs.  Up to 64 runs, the four threads of a quad count over every fourth
    //    run and sum in the quad (all 256 threads busy); more, one thread per run.
    auto place = [&](uint64_t key, int32_t pos, int e0, int de) {
        const int32_t r = (int32_t)((key >> 18) & 0xFF), s0 = (int32_t)((key >> 9) & 0x1FF);
        const int32_t n = (int32_t)(key & 0x1FF);
        for (int e = e0; e < n && 2 * n_items <= a.list_len; e += de) {
            a.work[2 * (pos + e)] = r;
            a.work[2 * (pos + e) + 1] = s0 + e;
        }
    };
    if (n_runs <= kPlanThreads / 4) {
        const int part = tid & 3, x = tid >> 2;
        const uint64_t key = x < n_runs ? runs[x] : ~0ull;
        int32_t pos = 0;
        for (int y0 = 0; y0 < n_runs; y0 += 16) {   // uniform trip count, four reads in flight
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int y = y0 + 4 * j + part;
                const uint64_t o = runs[y < n_runs ? y : 0];
                pos += y < n_runs && o < key ? (int32_t)(o & 0x1FF) : 0;
            }
        }
        pos += __builtin_amdgcn_mov_dpp(pos, 0xb1, 0xf, 0xf, false);   // quad_perm [1,0,3,2]
        pos += __builtin_amdgcn_mov_dpp(pos, 0x4e, 0xf, 0xf, false);   // quad_perm [2,3,0,1]
        if (x < n_runs) place(key, pos, part, 4);
    } else {
        for (int x = tid; x < n_runs; x += kPlanThreads) {
            const uint64_t key = runs[x];
            int32_t pos = 0;
            int y = 0;
            for (; y + 4 <= n_runs; y += 4) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint64_t o = runs[y + j];
                    pos += o < key ? (int32_t)(o & 0x1FF) : 0;
                }
            }
            for (; y < n_runs; ++y) {
                const uint64_t o = runs[y];
                pos += o < key ? (int32_t)(o & 0x1FF) : 0;
            }
            place(key, pos, 0, 1);
        }
    }
    for (int i = 2 * n_items + tid; i < a.list_len; i += kPlanThreads) a.work[i] = -1;

    if (tid == 0) {
        a.header[kHdrStatus] = bad ? AMLA_DEV_BAD_LENGTH : 0;
        a.header[kHdrItems] = n_items;
        a.header[kHdrRows] = a.rows;
        a.header[kHdrMtile] = a.mtile;
        a.header[kHdrWorkers] = a.workers;
        a.header[kHdrMode] = a.mode;
        a.header[kHdrReqs] = R;
        a.header[kHdrPlanned] = kPlannedMagic;
    }
}

// -------------------------------------------------------------------- decode kernel

struct DecodeArgs {
    int64_t pool_pages;
    int32_t bt_stride, reqs, rows, mtile, workers, list_len;
    float score_scale;  // bmm1 * log2(e)
    float out_scale;    // bmm2
    // causal mask in global positions over a DCP shard (causal == 0: every row sees the
    // request's whole local length; the other fields are then unused)
    const int32_t *totals;
    int32_t causal, heads, k_tokens, cp_world, cp_rank, cp_interleave;
};

// Keys of the local shard that folded row `row` may see.  Page "...cutedsl.mla.balanced",
// module docstring and BalancedMla.decode: under DCP the decode reads this rank's shard
// and masks causally in global positions, from the requests' global lengths.  Draft token
// t = row / H of a request of `total` global keys sits at position total - k + t and sees
// the g = total - k + t + 1 positions before it and itself; the rank holds blocks of
// `interleave` positions dealt round-robin over `world` ranks, in global order, so the
// visible keys are the first (g / span) * interleave + clamp(g % span - rank * interleave,
// 0, interleave) of its shard (span = interleave * world).
__device__ __forceinline__ int shard_count(const DecodeArgs &a, int g)
{
    if (g <= 0) return 0;
    const uint32_t span = (uint32_t)a.cp_interleave * (uint32_t)a.cp_world;
    const int rem = (int)((uint32_t)g % span) - a.cp_rank * a.cp_interleave;
    return (int)((uint32_t)g / span) * a.cp_interleave +
           (rem < 0 ? 0 : rem > a.cp_interleave ? a.cp_interleave : rem);
}

__device__ __forceinline__ int row_key_limit(const DecodeArgs &a, int total, int L, int row)
{
    if (!a.causal) return L;
    int t = row / a.heads;
    t = t < a.k_tokens - 1 ? t : a.k_tokens - 1;   // rows past M: any limit will do
    const int n = shard_count(a, total - a.k_tokens + t + 1);
    return n < L ? n : L;
}

// s_waitcnt immediates for gfx9: vmcnt in [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8].
constexpr int waitcnt_imm(int vm, int lgkm)
{
    return (vm & 0xF) | ((vm >> 4) << 14) | (0x7 << 4) | ((lgkm & 0xF) << 8);
}

__device__ __forceinline__ void wait_pages_then_barrier(int pages_after)
{
    // Every wave waits for its own page DMAs except the `pages_after` newest pages, and
    // for its LDS traffic, then the workgroup meets.  No release fence: it would also
    // wait for the in-flight prefetch.
    if (pages_after >= 2)
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(2 * kChunksPerWave, 0));
    else if (pages_after == 1)
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(kChunksPerWave, 0));
    else
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
    asm volatile("s_barrier" ::: "memory");
}

__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
    asm volatile("s_barrier" ::: "memory");
}

// LDS page layout: token row t occupies bytes [576t, 576t+576) of its slot, and within
// the row the 16-byte chunk c is stored at chunk position c ^ ((t >> 2) & 3).  Rows are
// 576 B apart, so without the swizzle 16 lanes reading one chunk of 16 consecutive rows
// hit only 4 of the 16 bank groups; with it they hit all 16, and so do the transposed V
// reads (8 keys x 2 chunks per 16 lanes).
__device__ __forceinline__ int swz(int row) { return (row >> 2) & 3; }

// One wave's 9 KiB share of a page, HBM -> LDS (global_load_lds_dwordx4: lane i's 16 bytes
// land at M0 + 16*i, the source is the page base in SGPRs plus the lane's offset).  LDS
// chunk position p of the slot receives the page's chunk (p / 36, (p % 36) ^ swz(p / 36));
// the per-lane source offsets are the same for every page and are computed once.  Issued as
// inline asm so that the compiler does not count these loads (it would otherwise wait for
// all of them before every transposed LDS read); completion is awaited explicitly with
// s_waitcnt vmcnt before the barrier that publishes a page.  The s_nop covers the
// SALU-write-M0 -> LDS-DMA hazard.  M0 is not listed as clobbered (clang reserves it); no
// compiler-generated code in these kernels reads M0.
struct DmaOffsets {
    uint32_t v[(kChunksPerWave + 1) / 2];   // two 16-bit offsets per register
    __device__ __forceinline__ uint32_t get(int i) const
    {
        return (i & 1) ? (v[i >> 1] >> 16) : (v[i >> 1] & 0xFFFFu);
    }
};

__device__ __forceinline__ DmaOffsets dma_offsets(int wave, int lane)
{
    DmaOffsets o;
#pragma unroll
    for (int i = 0; i < (kChunksPerWave + 1) / 2; ++i) o.v[i] = 0;
#pragma unroll
    for (int i = 0; i < kChunksPerWave; ++i) {
        const int p = (wave * kChunksPerWave + i) * 64 + lane;
        const int row = p / (kKDim / 16), q = p - row * (kKDim / 16);
        o.v[i >> 1] |= (uint32_t)(row * kKDim + 16 * (q ^ swz(row))) << (16 * (i & 1));
    }
    return o;
}

// A wave-uniform pointer, pinned to scalar registers for an inline-asm "s" operand.
__device__ __forceinline__ const uint8_t *uniform_ptr(const uint8_t *p)
{
    const uint64_t v = (uint64_t)(uintptr_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return (const uint8_t *)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ void issue_page(const uint8_t *page_base, uint32_t lds_dst,
                                           const DmaOffsets &o)
{
    page_base = uniform_ptr(page_base);
    lds_dst = __builtin_amdgcn_readfirstlane(lds_dst);
    asm volatile(
        "s_mov_b32 m0, %[m]\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %[o0], %[b]\n\t"
        "s_add_u32 m0, %[m], 0x400\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %[o1], %[b]\n\t"
        "s_add_u32 m0, %[m], 0x800\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %[o2], %[b]\n\t"
        "s_add_u32 m0, %[m], 0xc00\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %[o3], %[b]\n\t"
        "s_add_u32 m0, %[m], 0x1000\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %[o4], %[b]\n\t"
        "s_add_u32 m0, %[m], 0x1400\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %[o5], %[b]\n\t"
        "s_add_u32 m0, %[m], 0x1800\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %[o6], %[b]\n\t"
        "s_add_u32 m0, %[m], 0x1c00\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %[o7], %[b]\n\t"
        "s_add_u32 m0, %[m], 0x2000\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %[o8], %[b]"
        :
        : [o0] "v"(o.get(0)), [o1] "v"(o.get(1)), [o2] "v"(o.get(2)), [o3] "v"(o.get(3)),
          [o4] "v"(o.get(4)), [o5] "v"(o.get(5)), [o6] "v"(o.get(6)), [o7] "v"(o.get(7)),
          [o8] "v"(o.get(8)), [b] "s"(page_base), [m] "s"(lds_dst)
        : "memory");
}
static_assert(kChunksPerWave == 9, "issue_page is written for 9 DMA instructions per wave");

// A work unit's Q rows (MT rows x 576 B, contiguous in q) HBM -> LDS at `lds_dst`, same
// layout; chunks of rows at or past `valid_rows` are not loaded.
template <int MT>
__device__ __forceinline__ void issue_q(const uint8_t *q_rows, uint32_t lds_dst, int valid_rows,
                                        int wave, int lane)
{
    constexpr int kChunks = MT * (kKDim / 16);
    constexpr int kPerWave = (kChunks / 4 + 63) / 64;
    static_assert(kChunks * 16 <= kPageBytes, "Q rows must fit one ring slot");
    q_rows = uniform_ptr(q_rows);
    lds_dst = __builtin_amdgcn_readfirstlane(lds_dst);
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
        const int p = (wave * kPerWave + i) * 64 + lane;
        if (p < kChunks && p < valid_rows * (kKDim / 16)) {
            asm volatile("s_mov_b32 m0, %[m]\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %[o], %[b]"
                         :
                         : [o] "v"(p * 16), [b] "s"(q_rows),
                           [m] "s"(lds_dst + (uint32_t)((wave * kPerWave + i) * 1024))
                         : "memory");
        }
    }
}

__device__ __forceinline__ v8i lds_read2x16(const uint8_t *p0, const uint8_t *p1)
{
    const v4i a = *(const v4i *)p0;
    const v4i b = *(const v4i *)p1;
    return v8i{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// Lanes l and l ^ 32 hold the two key halves of one row: v_permlane32_swap gives every
// lane both values.
__device__ __forceinline__ float half_pair_max(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float half_pair_sum(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ v2i lds_read_tr8(const uint8_t *p)
{
    return __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS_AS v2i *)p);
}

// blockIdx -> virtual worker: hardware hands workgroups to the 8 XCDs round-robin, so
// virtual workers v and v+1 (the row tiles of one split) are put on the same XCD and
// share its L2.
__device__ __forceinline__ int virtual_worker(int b, int W, int mt)
{
    // with one row tile per split there is nothing to share: workgroups take the list in
    // order, so those that start first (and those started as CUs free up) take the
    // longest items
    if (mt == 1 || W % 8 != 0) return b;
    return (b % 8) * (W / 8) + b / 8;
}

__device__ __forceinline__ v16f mfma(v8i a, v8i b, v16f c)
{
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// 128-row tiles, paired waves sharing each page: wave w computes the scores, running
// max/sum and P of row block w; it accumulates O^T for the rows of blocks {2p, 2p+1}
// (p = w/2) and the dims [256h, +256) (h = w%2), so every V^T fragment read from LDS feeds
// two MFMAs.  Partners (w, w^1) swap P, the per-row rescale factor and a rescale flag
// through LDS each page.  The DMA of page t+3 goes into the slot page t-1 used.  Read-only
// inputs are separate __restrict__ arguments; their uniform reads go through the constant
// address space (scalar loads, which do not wait on the in-flight page DMAs).
__global__ __launch_bounds__(kDecodeThreads, 1) void decode128_kernel(
    const uint8_t *__restrict__ q_in, const uint8_t *__restrict__ kv_in,
    const int32_t *__restrict__ block_table, const int32_t *__restrict__ lengths,
    const int32_t *__restrict__ counts, const int32_t *__restrict__ offsets,
    const int32_t *__restrict__ work, int32_t *__restrict__ header, float *__restrict__ partial,
    float *__restrict__ lse_out, DecodeArgs a)
{
    constexpr int MT = 128;          // rows per work unit
    constexpr int NT = 16;           // accumulator tiles per wave: 2 row blocks x 8 dim tiles
    __shared__ __attribute__((aligned(1024))) uint8_t lds[kSlots * kPageBytes];
    // per wave: its P fragment (64 lanes x 32 B), per-row rescale factor, rescale flag
    __shared__ __attribute__((aligned(16))) int32_t xch_p[4][64 * 8];
    __shared__ float xch_alpha[4][32];
    __shared__ int32_t xch_flag[4];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, half = lane >> 5;
    const int R = a.reqs, M = a.rows;
    const int mt = ceil_div(M, MT);
    const int W = a.workers;

    // The plan summary, the item count and the first unit's work pair do not depend on
    // each other, so they are loaded together and their latencies overlap.  The pair is
    // inside the list: its item is below W and list_len >= 2 * (reqs + 2 * workers).
    const int vw = virtual_worker(blockIdx.x, W, mt);
    const int h_planned = ldc(&header[kHdrPlanned]), h_rows = ldc(&header[kHdrRows]);
    const int h_mtile = ldc(&header[kHdrMtile]), h_workers = ldc(&header[kHdrWorkers]);
    const int h_reqs = ldc(&header[kHdrReqs]);
    const int n_items = ldc(&offsets[R]);
    int r_first = ldc(&work[2 * (vw / mt)]), s_first = ldc(&work[2 * (vw / mt) + 1]);
    // consume every value here so that the compiler cannot sink a load past the checks
    // below (it would otherwise chain them one behind the other)
    asm volatile("" ::"s"(h_planned), "s"(h_rows), "s"(h_mtile), "s"(h_workers), "s"(h_reqs),
                 "s"(n_items), "s"(r_first), "s"(s_first), "s"(q_in), "s"(kv_in), "s"(block_table),
                 "s"(lengths), "s"(counts));
    if (h_planned != kPlannedMagic || h_rows != M || h_mtile != MT || h_workers != W ||
        h_reqs != R || n_items < 0 || 2 * n_items > a.list_len || n_items > R + kPlanSlack * W) {
        if (tid == 0 && blockIdx.x == 0) atomicOr(&header[kHdrStatus], AMLA_DEV_BAD_ITEM);
        return;
    }
    const int units = n_items * mt;

    const DmaOffsets dmao = dma_offsets(wave, lane);
    const uint32_t lds_base = (uint32_t)(uintptr_t)(LDS_AS uint8_t *)lds + wave * (kChunksPerWave * 1024);

    // V^T fragment reads (ds_read_b64_tr_b8): within each 16-lane group, source lane i
    // supplies key row b = i/2 and dims [8*(i%2), +8) of a 16-dim column block.  Keys are
    // tr_key + 16*w2; dims [32*tile + 16*(g16&1) + 8*(i16&1), +8) lie in chunk
    // 2*tile + (g16&1), swizzled by the key row (the same for the four w2 rows).
    const int g16 = lane >> 4, i16 = lane & 15;
    const int tr_key = 8 * (i16 >> 3) + 4 * half + ((i16 >> 1) & 3);
    int tr_off[2];
#pragma unroll
    for (int par = 0; par < 2; ++par)
        tr_off[par] = tr_key * kKDim + 16 * ((2 * par + (g16 & 1)) ^ swz(tr_key)) + 8 * (i16 & 1);
    // K fragment reads: row l32 (+32 per key block), chunks 4k + 2*half + e, e = 0, 1
    int k_off[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) k_off[e] = l32 * kKDim + 16 * ((2 * half + e) ^ swz(l32));

    for (int u = vw; u < units; u += W) {
        const int item = u / mt, jt = u - item * mt;
        const int r = u == vw ? r_first : ldc(&work[2 * item]);
        const int s = u == vw ? s_first : ldc(&work[2 * item + 1]);
        // the request's count, length and slot offset, loaded together (index clamped so
        // that the loads stay in bounds before r is checked)
        const int rc = r >= 0 && r < R ? r : 0;
        const int c = ldc(&counts[rc]), L = ldc(&lengths[rc]), off_r = ldc(&offsets[rc]);
        const int total = a.causal ? ldc(&a.totals[rc]) : L;
        asm volatile("" ::"s"(c), "s"(L), "s"(off_r), "s"(total));
        const int pages = ceil_div(L, kPage);
        const int q = c > 0 ? pages / c : 0, rem = c > 0 ? pages % c : 0;
        const int first = s * q + (s < rem ? s : rem);
        const int size = q + (s < rem ? 1 : 0);
        if (r != rc || s < 0 || s >= c || L <= 0 || pages > a.bt_stride || size <= 0 ||
            off_r + s >= n_items) {
            if (tid == 0) atomicOr(&header[kHdrStatus], AMLA_DEV_BAD_ITEM);
            continue;
        }
        if (a.causal && tid == 0 && shard_count(a, total) != L)   // shard and totals disagree
            atomicOr(&header[kHdrStatus], AMLA_DEV_BAD_LENGTH);
        const int row0 = jt * MT + 32 * wave;   // this wave's score rows
        const int lim = row_key_limit(a, total, L, row0 + l32);   // keys this lane's row sees
        const bool active = row0 < M;
        const int32_t *bt = block_table + (size_t)r * a.bt_stride + first;

        v8i qf[9];   // Q^T fragments, loaded below once the first pages are in flight

        bool page_bad = false;
        auto page_at = [&](int32_t pid) {
            if (pid < 0 || pid >= a.pool_pages) {
                page_bad = true;
                pid = 0;
            }
            return kv_in + (int64_t)pid * kPageBytes;
        };
        // block-table entry of page min(t, size - 1)
        auto page_id = [&](int t) { return ldc(&bt[t < size ? t : size - 1]); };
        // keys past the request's length (only on its last page): zero the rows in LDS so
        // that P*V stays finite; scores there are masked by key index
        auto zero_tail = [&](int t) {
            const int valid = L - (first + t) * kPage;
            if (valid < kPage) {
                uint8_t *slot = lds + (t % kSlots) * kPageBytes;
                for (int off = valid * kKDim + tid * 16; off < kPageBytes; off += kDecodeThreads * 16)
                    *(v4i *)(slot + off) = v4i{0, 0, 0, 0};
                lds_barrier();
            }
        };

        // l_run: row sum of the FP32 P (for the LSE); lq_run: of the E4M3 P that the MMA
        // uses (O is normalised by it, so the weights of the output rows sum to one)
        float m_run = -INFINITY, l_run = 0.f, lq_run = 0.f;
        v16f acc[NT];
#pragma unroll
        for (int n = 0; n < NT; ++n) acc[n] = v16f{0};
        v16f sc[2];          // the scores of the page

        // S^T[64 keys x 32 rows] of the page in `slot`: 9 MFMAs per 32-key block, each fed
        // by two 16-byte LDS reads of a key row.  Step j issues the reads of fragment j+2,
        // then MFMA j, then `valu(j)` (other work to overlap with the MFMA); a scheduling
        // fence after each step keeps that order, so the reads stay two MFMAs ahead.
        auto scores = [&](const uint8_t *slot, v16f (&out)[2], auto &&valu) {
            const uint8_t *kp0 = slot + k_off[0], *kp1 = slot + k_off[1];
            out[0] = v16f{0};
            out[1] = v16f{0};
            v8i kf0 = lds_read2x16(kp0, kp1);
            v8i kf1 = lds_read2x16(kp0 + 64, kp1 + 64);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < 18; ++j) {
                const int b = j / 9, k = j % 9;
                const v8i cur = (j & 1) ? kf1 : kf0;
                if (j + 2 < 18) {
                    const int o = 32 * ((j + 2) / 9) * kKDim + 64 * ((j + 2) % 9);
                    if (j & 1)
                        kf1 = lds_read2x16(kp0 + o, kp1 + o);
                    else
                        kf0 = lds_read2x16(kp0 + o, kp1 + o);
                }
                out[b] = mfma(cur, qf[k], out[b]);
                valu(j);
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        // P = 2^(s*scale - m + kPScale): FP32 into the row sum, E4M3 into the P^T operand;
        // lane (l32, half) byte 16b + e holds key 32b + 8(e/4) + 4*half + e%4.  Group g of 8
        // makes fragment dword g (four keys).
        v8i pf;
        float psum = 0.f, qsum = 0.f, bias = 0.f;
        auto probs_begin = [&]() {
            bias = m_run == -INFINITY ? 0.f : kPScale - m_run;   // no key seen: P = 0
            psum = 0.f;
            qsum = 0.f;
        };
        auto probs_group = [&](const v16f (&sv)[2], int g) {
            const int b = g >> 2, qd = g & 3;
            float p[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[b][4 * qd + e], a.score_scale, bias));
                psum += p[e];
            }
            int w = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], 0, false);
            w = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], w, true);
            pf[g] = w;
            const v2f q0 = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
            const v2f q1 = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
            qsum += (q0[0] + q0[1]) + (q1[0] + q1[1]);
        };
        auto probs_end = [&]() {
            l_run += psum;
            lq_run += qsum;
        };
        // The first pages' block-table entries, loaded together.
        int32_t pid0[kSlots - 1];
#pragma unroll
        for (int d = 0; d < kSlots - 1; ++d) pid0[d] = page_id(d);
        asm volatile("" ::"s"(pid0[0]), "s"(pid0[1]), "s"(pid0[2]));
        // the entry of the next page to fetch, read one fetch ahead
        int32_t pid_next = page_id(kSlots - 1);
        // The first pages' DMA, then the Q^T fragments from global memory, so that
        // both latencies overlap; then wait for all of it (the compiler tracks the Q
        // loads, not the DMA).
#pragma unroll
        for (int d = 0; d < kSlots - 1; ++d)
            if (d < size) issue_page(page_at(pid0[d]), lds_base + d * kPageBytes, dmao);
        const int row = row0 + l32;
        if (row < M) {
            const uint8_t *qp = q_in + ((size_t)r * M + row) * kKDim + 32 * half;
#pragma unroll
            for (int k = 0; k < 9; ++k) {
                const v4i x = *(const v4i *)(qp + 64 * k);
                const v4i y = *(const v4i *)(qp + 64 * k + 16);
                qf[k] = v8i{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
            }
        } else {
#pragma unroll
            for (int k = 0; k < 9; ++k) qf[k] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
        }
        wait_pages_then_barrier(0);

        auto no_valu = [](int) {};
        // 128-row tiles, paired waves.  Wave w computes the scores, running max/sum and
        // P of row block w; it owns O for the 64 rows of blocks {2p, 2p+1} (p = w/2) and
        // the 256 dims [256*hw, +256) (hw = w%2).  Partners (w, w^1) swap their P
        // fragments and rescale factors through LDS each page, so every V^T fragment
        // read from LDS feeds two MFMAs (one per row block).
        const int hw = wave & 1, pair = wave >> 1;
        const bool o_active = jt * MT + 64 * pair < M;
        // acc[n]: own row block (2p + hw), acc[8 + n]: the partner's (2p + 1 - hw);
        // dim tile 8*hw + n in both
        for (int t = 0; t < size; ++t) {
            const int after = size - 1 - t;
            wait_pages_then_barrier(after < kSlots - 2 ? after : kSlots - 2);
            if (t + kSlots - 1 < size) {
                issue_page(page_at(pid_next),
                           lds_base + ((t + kSlots - 1) % kSlots) * kPageBytes, dmao);
                pid_next = page_id(t + kSlots);
            }
            zero_tail(t);
            const uint8_t *slot = lds + (t % kSlots) * kPageBytes;
            float alpha = 1.f;
            bool any_grow = false;
            pf = v8i{0, 0, 0, 0, 0, 0, 0, 0};
            if (active) {
                scores(slot, sc, no_valu);
                const int valid = lim - (first + t) * kPage;   // keys of the page the row sees
                if (__any(valid < kPage)) {
#pragma unroll
                    for (int b = 0; b < 2; ++b)
#pragma unroll
                        for (int e = 0; e < 16; ++e)
                            if (32 * b + 8 * (e >> 2) + 4 * half + (e & 3) >= valid)
                                sc[b][e] = -INFINITY;
                }
                float smax = -INFINITY;
#pragma unroll
                for (int b = 0; b < 2; ++b)
#pragma unroll
                    for (int e = 0; e < 16; ++e) smax = fmaxf(smax, sc[b][e]);
                const float mx = half_pair_max(smax) * a.score_scale;
                const bool grow = mx > m_run + kTau;
                any_grow = __any(grow);
                if (any_grow) {
                    const float m_new = grow ? mx : m_run;
                    // rows whose max stays keep factor 1 (exp2(m - m) would be NaN for a
                    // row that has seen no key yet, m = -inf)
                    alpha = grow ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
                    l_run *= alpha;
                    lq_run *= alpha;
                    m_run = m_new;
                }
                probs_begin();
#pragma unroll
                for (int g = 0; g < 8; ++g) probs_group(sc, g);
                probs_end();
            }
            // swap with the partner: P fragment, per-row rescale factor, rescale flag
            *(v8i *)&xch_p[wave][lane * 8] = pf;
            if (half == 0) xch_alpha[wave][l32] = alpha;
            if (lane == 0) xch_flag[wave] = any_grow ? 1 : 0;
            lds_barrier();
            if (!o_active) continue;
            const v8i pf_other = *(const v8i *)&xch_p[wave ^ 1][lane * 8];
            const float alpha_other = xch_alpha[wave ^ 1][l32];
            const bool grow_other = xch_flag[wave ^ 1] != 0;
            if (any_grow) {
#pragma unroll
                for (int n = 0; n < 8; ++n) acc[n] *= alpha;
            }
            if (grow_other) {
#pragma unroll
                for (int n = 0; n < 8; ++n) acc[8 + n] *= alpha_other;
            }
            const uint8_t *vp0 = slot + tr_off[0] + 64 * (4 * hw);
            const uint8_t *vp1 = slot + tr_off[1] + 64 * (4 * hw);
            auto vtile = [&](int n) {
                v8i f;
                const uint8_t *vp = (n & 1) ? vp1 : vp0;
#pragma unroll
                for (int w2 = 0; w2 < 4; ++w2) {
                    const v2i x = lds_read_tr8(vp + 16 * w2 * kKDim + 64 * (n >> 1));
                    f[2 * w2] = x[0];
                    f[2 * w2 + 1] = x[1];
                }
                return f;
            };
            v8i vf = vtile(0);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int n = 0; n < 8; ++n) {
                const v8i cur = vf;
                if (n + 1 < 8) vf = vtile(n + 1);
                acc[n] = mfma(cur, pf, acc[n]);
                acc[8 + n] = mfma(cur, pf_other, acc[8 + n]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }

        if (page_bad && tid == 0) atomicOr(&header[kHdrStatus], AMLA_DEV_BAD_PAGE);

        // epilogue: normalise and store this split's FP32 partial and log2 LSE.
        // l_run is scaled by 2^kPScale like P, so the scale cancels in O / l.
        const size_t slot_idx = (size_t)off_r + s;
        const float l_tot = half_pair_sum(l_run), lq_tot = half_pair_sum(lq_run);
        if (half == 0) xch_alpha[wave][l32] = lq_tot;
        lds_barrier();
        const float lq_other = xch_alpha[wave ^ 1][l32];
        if (active && half == 0 && row0 + l32 < M)
            lse_out[slot_idx * M + row0 + l32] = m_run + __builtin_amdgcn_logf(l_tot) - kPScale;
#pragma unroll
        for (int own = 1; own >= 0; --own) {
            const int row = jt * MT + 32 * (2 * pair + (own ? hw : 1 - hw)) + l32;
            if (row < M) {
                float *po = partial + (slot_idx * M + row) * kVDim;
                const float lq = own ? lq_tot : lq_other;
                const float inv = lq > 0.f ? a.out_scale / lq : 0.f;   // no key: O = 0
#pragma unroll
                for (int n = 0; n < 8; ++n) {
                    const int dim = 32 * (8 * hw + n) + 4 * half;
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4) {
                        const v16f &t16 = acc[(own ? 0 : 8) + n];
                        const v4f o = v4f{t16[4 * q4], t16[4 * q4 + 1], t16[4 * q4 + 2],
                                          t16[4 * q4 + 3]} * inv;
                        *(v4f *)(po + dim + 8 * q4) = o;
                    }
                }
            }
        }

        lds_barrier();  // the next unit's prologue overwrites the ring
    }
}


// 32-row tiles, wave pairs on alternate pages.  Pair p (waves 2p, 2p+1) computes the pages
// t = p (mod 2) of the split: both waves of the pair compute the page's scores for all 32
// rows and the same P, and wave 2p+h accumulates O^T for the dims [256h, +256).  Each page's
// scores are computed twice instead of four times (once per wave of a shared page stream),
// which halves the MFMA and LDS work per page.  The two pairs' (max, sum, O) are merged
// through LDS at the end of the unit.  Per iteration: pages 2i and 2i+1 are computed while
// pages 2i+2 and 2i+3 are fetched into the other two ring slots.
constexpr int kMergeStride = kVDim / 2 + 4;   // floats per row of a merge region (+16 B pad)
static_assert(4 * 32 * kMergeStride * 4 <= kSlots * kPageBytes, "merge regions must fit the ring");

__global__ __launch_bounds__(kDecodeThreads, 1) void decode32_kernel(
    const uint8_t *__restrict__ q_in, const uint8_t *__restrict__ kv_in,
    const int32_t *__restrict__ block_table, const int32_t *__restrict__ lengths,
    const int32_t *__restrict__ counts, const int32_t *__restrict__ offsets,
    const int32_t *__restrict__ work, int32_t *__restrict__ header, float *__restrict__ partial,
    float *__restrict__ lse_out, DecodeArgs a)
{
    constexpr int MT = 32;
    constexpr int NT = kVDim / 64;   // 8 output tiles of 32 dims per wave
    __shared__ __attribute__((aligned(1024))) uint8_t lds[kSlots * kPageBytes];
    __shared__ float xm[2][32], xl[2][32], xq[2][32];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int pair = wave >> 1, hw = wave & 1;
    const int l32 = lane & 31, half = lane >> 5;
    const int R = a.reqs, M = a.rows;
    const int mt = ceil_div(M, MT);
    const int W = a.workers;

    // plan summary, item count and the first unit's work pair, loaded together (see
    // decode_kernel)
    const int vw = virtual_worker(blockIdx.x, W, mt);
    const int h_planned = ldc(&header[kHdrPlanned]), h_rows = ldc(&header[kHdrRows]);
    const int h_mtile = ldc(&header[kHdrMtile]), h_workers = ldc(&header[kHdrWorkers]);
    const int h_reqs = ldc(&header[kHdrReqs]);
    const int n_items = ldc(&offsets[R]);
    int r_first = ldc(&work[2 * (vw / mt)]), s_first = ldc(&work[2 * (vw / mt) + 1]);
    asm volatile("" ::"s"(h_planned), "s"(h_rows), "s"(h_mtile), "s"(h_workers), "s"(h_reqs),
                 "s"(n_items), "s"(r_first), "s"(s_first), "s"(q_in), "s"(kv_in), "s"(block_table),
                 "s"(lengths), "s"(counts));
    if (h_planned != kPlannedMagic || h_rows != M || h_mtile != MT || h_workers != W ||
        h_reqs != R || n_items < 0 || 2 * n_items > a.list_len || n_items > R + kPlanSlack * W) {
        if (tid == 0 && blockIdx.x == 0) atomicOr(&header[kHdrStatus], AMLA_DEV_BAD_ITEM);
        return;
    }
    const int units = n_items * mt;

    const DmaOffsets dmao = dma_offsets(wave, lane);
    const uint32_t lds_base = (uint32_t)(uintptr_t)(LDS_AS uint8_t *)lds + wave * (kChunksPerWave * 1024);

    // V^T fragment reads of this wave's tile n (dims 256*hw + 32n): vp[n & 1] + 64 * (n >> 1)
    // (layout as in decode_kernel)
    const int g16 = lane >> 4, i16 = lane & 15;
    const int tr_key = 8 * (i16 >> 3) + 4 * half + ((i16 >> 1) & 3);
    int tr_off[2];
#pragma unroll
    for (int par = 0; par < 2; ++par)
        tr_off[par] = tr_key * kKDim + 16 * ((2 * par + (g16 & 1)) ^ swz(tr_key)) + 8 * (i16 & 1) +
                      64 * (hw * NT / 2);
    int k_off[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) k_off[e] = l32 * kKDim + 16 * ((2 * half + e) ^ swz(l32));

    for (int u = vw; u < units; u += W) {
        const int item = u / mt, jt = u - item * mt;
        const int r = u == vw ? r_first : ldc(&work[2 * item]);
        const int s = u == vw ? s_first : ldc(&work[2 * item + 1]);
        const int rc = r >= 0 && r < R ? r : 0;
        const int c = ldc(&counts[rc]), L = ldc(&lengths[rc]), off_r = ldc(&offsets[rc]);
        const int total = a.causal ? ldc(&a.totals[rc]) : L;
        asm volatile("" ::"s"(c), "s"(L), "s"(off_r), "s"(total));
        const int pages = ceil_div(L, kPage);
        const int q = c > 0 ? pages / c : 0, rem = c > 0 ? pages % c : 0;
        const int first = s * q + (s < rem ? s : rem);
        const int size = q + (s < rem ? 1 : 0);
        if (r != rc || s < 0 || s >= c || L <= 0 || pages > a.bt_stride || size <= 0 ||
            off_r + s >= n_items) {
            if (tid == 0) atomicOr(&header[kHdrStatus], AMLA_DEV_BAD_ITEM);
            continue;
        }
        if (a.causal && tid == 0 && shard_count(a, total) != L)   // shard and totals disagree
            atomicOr(&header[kHdrStatus], AMLA_DEV_BAD_LENGTH);
        const int32_t *bt = block_table + (size_t)r * a.bt_stride + first;
        const int row = jt * MT + l32;
        const int lim = row_key_limit(a, total, L, row);   // keys this lane's row sees

        bool page_bad = false;
        auto page_at = [&](int32_t pid) {
            if (pid < 0 || pid >= a.pool_pages) {
                page_bad = true;
                pid = 0;
            }
            return kv_in + (int64_t)pid * kPageBytes;
        };
        auto page_id = [&](int t) { return ldc(&bt[t < size ? t : size - 1]); };
        auto issue = [&](int t, int32_t pid) {
            issue_page(page_at(pid), lds_base + (t % kSlots) * kPageBytes, dmao);
        };

        // Prologue: the unit's Q rows by DMA into the last ring slot, pages 0..2 into the
        // others; once Q and pages 0, 1 are in, every wave reads its Q^T fragments (lane
        // (row l32, half) holds dims [64k + 32*half, +32)), and page 3 then takes the slot.
        int32_t pid0[kSlots];
#pragma unroll
        for (int d = 0; d < kSlots; ++d) pid0[d] = page_id(d);
        asm volatile("" ::"s"(pid0[0]), "s"(pid0[1]), "s"(pid0[2]), "s"(pid0[3]));
        issue_q<MT>(q_in + ((size_t)r * M + (size_t)jt * MT) * kKDim,
                    (uint32_t)(uintptr_t)(LDS_AS uint8_t *)lds + (kSlots - 1) * kPageBytes, M - jt * MT,
                    wave, lane);
#pragma unroll
        for (int d = 0; d < kSlots - 1; ++d)
            if (d < size) issue(d, pid0[d]);
        int32_t pid_a = page_id(kSlots), pid_b = page_id(kSlots + 1);
        wait_pages_then_barrier(size > 2 ? 1 : 0);
        v8i qf[9];
        {
            // the lane index is re-read here rather than kept live across the unit loop
            int ln;
            asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
            const uint8_t *qs = lds + (kSlots - 1) * kPageBytes + (ln & 31) * kKDim + 32 * (ln >> 5);
            const bool row_ok = jt * MT + (ln & 31) < M;
#pragma unroll
            for (int k = 0; k < 9; ++k) {
                const v8i x = lds_read2x16(qs + 64 * k, qs + 64 * k + 16);
                qf[k] = row_ok ? x : v8i{0, 0, 0, 0, 0, 0, 0, 0};
            }
        }
        lds_barrier();  // every wave has its Q^T: page 3 may overwrite it
        if (kSlots - 1 < size) issue(kSlots - 1, pid0[kSlots - 1]);

        // l_run: row sum of the FP32 P (for the LSE); lq_run: of the E4M3 P that the MMA
        // uses (O is normalised by it, so the weights of the output rows sum to one)
        float m_run = -INFINITY, l_run = 0.f, lq_run = 0.f;
        v16f acc[NT];
#pragma unroll
        for (int n = 0; n < NT; ++n) acc[n] = v16f{0};

        for (int t0 = 0; t0 < size; t0 += 2) {
            if (t0 > 0) {
                // pages t0, t0+1 resident (nothing newer in flight); every wave is past
                // pages t0-2, t0-1, whose slots take pages t0+2, t0+3
                wait_pages_then_barrier(0);
                if (t0 + 2 < size) issue(t0 + 2, pid_a);
                if (t0 + 3 < size) issue(t0 + 3, pid_b);
                pid_a = page_id(t0 + 4);
                pid_b = page_id(t0 + 5);
            }
            // keys past the request's length (its last page only): zero their rows so that
            // P V stays finite; their scores are masked by key index below
            const int last_valid = L - (first + (t0 + 1 < size ? t0 + 1 : t0)) * kPage;
            if (last_valid < kPage) {
                const int tz = t0 + 1 < size ? t0 + 1 : t0;
                uint8_t *zs = lds + (tz % kSlots) * kPageBytes;
                for (int off = last_valid * kKDim + tid * 16; off < kPageBytes; off += kDecodeThreads * 16)
                    *(v4i *)(zs + off) = v4i{0, 0, 0, 0};
                lds_barrier();
            }
            const int t = t0 + pair;
            if (t >= size) continue;
            const uint8_t *slot = lds + (t % kSlots) * kPageBytes;
            const int valid = lim - (first + t) * kPage;   // keys of the page the row sees

            // S^T[64 keys x 32 rows]: 18 MFMAs, K fragment reads two ahead
            v16f sc[2];
            {
                const uint8_t *kp0 = slot + k_off[0], *kp1 = slot + k_off[1];
                sc[0] = v16f{0};
                sc[1] = v16f{0};
                v8i kf0 = lds_read2x16(kp0, kp1);
                v8i kf1 = lds_read2x16(kp0 + 64, kp1 + 64);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int j = 0; j < 18; ++j) {
                    const int b = j / 9, k = j % 9;
                    const v8i cur = (j & 1) ? kf1 : kf0;
                    if (j + 2 < 18) {
                        const int o = 32 * ((j + 2) / 9) * kKDim + 64 * ((j + 2) % 9);
                        if (j & 1)
                            kf1 = lds_read2x16(kp0 + o, kp1 + o);
                        else
                            kf0 = lds_read2x16(kp0 + o, kp1 + o);
                    }
                    sc[b] = mfma(cur, qf[k], sc[b]);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            // page max (masked), lazy running max and O rescale
            if (__any(valid < kPage)) {
#pragma unroll
                for (int b = 0; b < 2; ++b)
#pragma unroll
                    for (int e = 0; e < 16; ++e)
                        if (32 * b + 8 * (e >> 2) + 4 * half + (e & 3) >= valid) sc[b][e] = -INFINITY;
            }
            float smax = -INFINITY;
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int e = 0; e < 16; ++e) smax = fmaxf(smax, sc[b][e]);
            const float mx = half_pair_max(smax) * a.score_scale;
            const bool grow = mx > m_run + kTau;
            if (__any(grow)) {
                const float m_new = grow ? mx : m_run;
                // rows whose max stays keep factor 1 (exp2(m - m) would be NaN for a
                // row that has seen no key yet, m = -inf)
                const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
                l_run *= alpha;
                lq_run *= alpha;
#pragma unroll
                for (int n = 0; n < NT; ++n) acc[n] *= alpha;
                m_run = m_new;
            }
            // P = 2^(s*scale - m + kPScale): FP32 into the row sum, E4M3 into P^T
            v8i pf;
            {
                const float bias = m_run == -INFINITY ? 0.f : kPScale - m_run;   // no key seen: P = 0
                float psum = 0.f, qsum = 0.f;
#pragma unroll
                for (int g = 0; g < 8; ++g) {
                    const int b = g >> 2, qd = g & 3;
                    float p4[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        p4[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[b][4 * qd + e], a.score_scale, bias));
                        psum += p4[e];
                    }
                    int w4 = __builtin_amdgcn_cvt_pk_fp8_f32(p4[0], p4[1], 0, false);
                    w4 = __builtin_amdgcn_cvt_pk_fp8_f32(p4[2], p4[3], w4, true);
                    pf[g] = w4;
                    const v2f q0 = __builtin_amdgcn_cvt_pk_f32_fp8(w4, false);
                    const v2f q1 = __builtin_amdgcn_cvt_pk_f32_fp8(w4, true);
                    qsum += (q0[0] + q0[1]) + (q1[0] + q1[1]);
                }
                l_run += psum;
                lq_run += qsum;
            }
            // O^T += V^T P^T over this wave's 8 tiles, transposed V reads one tile ahead
            {
                const uint8_t *vp0 = slot + tr_off[0], *vp1 = slot + tr_off[1];
                auto vtile = [&](int n) {
                    v8i f;
                    const uint8_t *vp = (n & 1) ? vp1 : vp0;
#pragma unroll
                    for (int w2 = 0; w2 < 4; ++w2) {
                        const v2i x = lds_read_tr8(vp + 16 * w2 * kKDim + 64 * (n >> 1));
                        f[2 * w2] = x[0];
                        f[2 * w2 + 1] = x[1];
                    }
                    return f;
                };
                v8i vf = vtile(0);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int n = 0; n < NT; ++n) {
                    const v8i cur = vf;
                    if (n + 1 < NT) vf = vtile(n + 1);
                    acc[n] = mfma(cur, pf, acc[n]);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
        if (page_bad && tid == 0) atomicOr(&header[kHdrStatus], AMLA_DEV_BAD_PAGE);

        // merge the two pairs: m = max_p m_p, l = sum_p l_p 2^(m_p - m) (likewise lq) and
        // O = sum_p O_p 2^(m_p - m) / lq (the sums carry P's 2^kPScale, which cancels)
        const float l_tot = half_pair_sum(l_run), lq_tot = half_pair_sum(lq_run);
        if (hw == 0 && half == 0) {
            xm[pair][l32] = m_run;
            xl[pair][l32] = l_tot;
            xq[pair][l32] = lq_tot;
        }
        lds_barrier();  // also: every wave is done with the ring
        const float m0 = xm[0][l32], m1 = xm[1][l32];
        const float m_all = fmaxf(m0, m1);
        const float e0 = m0 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m0 - m_all);
        const float e1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - m_all);
        const float l_all = xl[0][l32] * e0 + xl[1][l32] * e1;
        const float lq_all = xq[0][l32] * e0 + xq[1][l32] * e1;
        const float f_own =
            m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m_all) * (a.out_scale / lq_all);
        const size_t slot_idx = (size_t)off_r + s;
        if (wave == 0 && half == 0 && row < M)
            lse_out[slot_idx * M + row] = m_all + __builtin_amdgcn_logf(l_all) - kPScale;
        // every wave stores its scaled O (32 rows x 256 dims) in region `wave`; then wave w
        // adds dims [128w, +128) of the two pairs' regions and stores them
        float *const region = (float *)(void *)lds;
        {
            float *mine = region + wave * (32 * kMergeStride) + l32 * kMergeStride + 4 * half;
#pragma unroll
            for (int n = 0; n < NT; ++n) {
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4)
                    *(v4f *)(mine + 32 * n + 8 * q4) =
                        v4f{acc[n][4 * q4], acc[n][4 * q4 + 1], acc[n][4 * q4 + 2], acc[n][4 * q4 + 3]} * f_own;
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        lds_barrier();
        {
            const int hsel = wave >> 1, dbase = 128 * (wave & 1);
            const float *r0 = region + hsel * (32 * kMergeStride);         // pair 0, half hsel
            const float *r1 = region + (2 + hsel) * (32 * kMergeStride);   // pair 1, half hsel
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int f = i * 64 + lane, rr = f >> 5, d = dbase + 4 * (f & 31);
                const v4f sum = *(const v4f *)(r0 + rr * kMergeStride + d) +
                                *(const v4f *)(r1 + rr * kMergeStride + d);
                if (jt * MT + rr < M)
                    *(v4f *)(partial + (slot_idx * M + jt * MT + rr) * kVDim + 256 * hsel + d) = sum;
            }
        }
        lds_barrier();  // the next unit's pages overwrite the regions
    }
}

// 64-row tiles, wave pairs on alternate pages.  Pair p (waves 2p, 2p+1) computes the pages
// t = p (mod 2) of the split for all 64 rows: wave 2p+h computes the scores, running
// max/sum and P of row block h and accumulates O^T for both row blocks and the dims
// [256h, +256), so every V^T fragment read from LDS feeds two MFMAs; the partners swap P,
// the per-row rescale factor and a rescale flag through LDS.  Each page's scores are
// computed once (with one shared page stream the two waves of each row block would both
// compute them).  At the end the two pairs' (max, sum, O) are merged through LDS: pair p
// merges and stores row block p.
__global__ __launch_bounds__(kDecodeThreads, 1) void decode64_kernel(
    const uint8_t *__restrict__ q_in, const uint8_t *__restrict__ kv_in,
    const int32_t *__restrict__ block_table, const int32_t *__restrict__ lengths,
    const int32_t *__restrict__ counts, const int32_t *__restrict__ offsets,
    const int32_t *__restrict__ work, int32_t *__restrict__ header, float *__restrict__ partial,
    float *__restrict__ lse_out, DecodeArgs a)
{
    constexpr int MT = 64;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[kSlots * kPageBytes];
    __shared__ __attribute__((aligned(16))) int32_t xch_p[4][64 * 8];  // per wave: its P fragment
    __shared__ float xch_alpha[4][32];                                  // per-row rescale factor
    __shared__ int32_t xch_flag[4];                                     // any row rescaled
    __shared__ float xm[2][2][32], xl[2][2][32], xq[2][2][32];          // [pair][block][row]

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int pair = wave >> 1, hw = wave & 1;
    const int l32 = lane & 31, half = lane >> 5;
    const int R = a.reqs, M = a.rows;
    const int mt = ceil_div(M, MT);
    const int W = a.workers;

    const int vw = virtual_worker(blockIdx.x, W, mt);
    const int h_planned = ldc(&header[kHdrPlanned]), h_rows = ldc(&header[kHdrRows]);
    const int h_mtile = ldc(&header[kHdrMtile]), h_workers = ldc(&header[kHdrWorkers]);
    const int h_reqs = ldc(&header[kHdrReqs]);
    const int n_items = ldc(&offsets[R]);
    int r_first = ldc(&work[2 * (vw / mt)]), s_first = ldc(&work[2 * (vw / mt) + 1]);
    asm volatile("" ::"s"(h_planned), "s"(h_rows), "s"(h_mtile), "s"(h_workers), "s"(h_reqs),
                 "s"(n_items), "s"(r_first), "s"(s_first), "s"(q_in), "s"(kv_in), "s"(block_table),
                 "s"(lengths), "s"(counts));
    if (h_planned != kPlannedMagic || h_rows != M || h_mtile != MT || h_workers != W ||
        h_reqs != R || n_items < 0 || 2 * n_items > a.list_len || n_items > R + kPlanSlack * W) {
        if (tid == 0 && blockIdx.x == 0) atomicOr(&header[kHdrStatus], AMLA_DEV_BAD_ITEM);
        return;
    }
    const int units = n_items * mt;

    const DmaOffsets dmao = dma_offsets(wave, lane);
    const uint32_t lds_base = (uint32_t)(uintptr_t)(LDS_AS uint8_t *)lds + wave * (kChunksPerWave * 1024);
    const int g16 = lane >> 4, i16 = lane & 15;
    const int tr_key = 8 * (i16 >> 3) + 4 * half + ((i16 >> 1) & 3);
    int tr_off[2];
#pragma unroll
    for (int par = 0; par < 2; ++par)
        tr_off[par] = tr_key * kKDim + 16 * ((2 * par + (g16 & 1)) ^ swz(tr_key)) + 8 * (i16 & 1) +
                      64 * (4 * hw);
    int k_off[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) k_off[e] = l32 * kKDim + 16 * ((2 * half + e) ^ swz(l32));

    for (int u = vw; u < units; u += W) {
        const int item = u / mt, jt = u - item * mt;
        const int r = u == vw ? r_first : ldc(&work[2 * item]);
        const int s = u == vw ? s_first : ldc(&work[2 * item + 1]);
        const int rc = r >= 0 && r < R ? r : 0;
        const int c = ldc(&counts[rc]), L = ldc(&lengths[rc]), off_r = ldc(&offsets[rc]);
        const int total = a.causal ? ldc(&a.totals[rc]) : L;
        asm volatile("" ::"s"(c), "s"(L), "s"(off_r), "s"(total));
        const int pages = ceil_div(L, kPage);
        const int q = c > 0 ? pages / c : 0, rem = c > 0 ? pages % c : 0;
        const int first = s * q + (s < rem ? s : rem);
        const int size = q + (s < rem ? 1 : 0);
        if (r != rc || s < 0 || s >= c || L <= 0 || pages > a.bt_stride || size <= 0 ||
            off_r + s >= n_items) {
            if (tid == 0) atomicOr(&header[kHdrStatus], AMLA_DEV_BAD_ITEM);
            continue;
        }
        if (a.causal && tid == 0 && shard_count(a, total) != L)   // shard and totals disagree
            atomicOr(&header[kHdrStatus], AMLA_DEV_BAD_LENGTH);
        const int row0 = jt * MT + 32 * hw;     // this wave's score rows (block hw)
        const int lim = row_key_limit(a, total, L, row0 + l32);   // keys this lane's row sees
        const bool active = row0 < M;
        const int32_t *bt = block_table + (size_t)r * a.bt_stride + first;

        bool page_bad = false;
        auto page_at = [&](int32_t pid) {
            if (pid < 0 || pid >= a.pool_pages) {
                page_bad = true;
                pid = 0;
            }
            return kv_in + (int64_t)pid * kPageBytes;
        };
        auto page_id = [&](int t) { return ldc(&bt[t < size ? t : size - 1]); };

        // the first pages' DMA, then the Q^T fragments of the score rows; wait for all of
        // it (the compiler tracks the Q loads, not the DMA)
        int32_t pid0[kSlots - 1];
#pragma unroll
        for (int d = 0; d < kSlots - 1; ++d) pid0[d] = page_id(d);
        asm volatile("" ::"s"(pid0[0]), "s"(pid0[1]), "s"(pid0[2]));
#pragma unroll
        for (int d = 0; d < kSlots - 1; ++d)
            if (d < size) issue_page(page_at(pid0[d]), lds_base + d * kPageBytes, dmao);
        int32_t pid_a = page_id(kSlots - 1), pid_b = page_id(kSlots);
        v8i qf[9];
        if (active && row0 + l32 < M) {
            const uint8_t *qp = q_in + ((size_t)r * M + row0 + l32) * kKDim + 32 * half;
#pragma unroll
            for (int k = 0; k < 9; ++k) {
                const v4i x = *(const v4i *)(qp + 64 * k);
                const v4i y = *(const v4i *)(qp + 64 * k + 16);
                qf[k] = v8i{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
            }
        } else {
#pragma unroll
            for (int k = 0; k < 9; ++k) qf[k] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
        }
        wait_pages_then_barrier(0);

        // l_run: row sum of the FP32 P (for the LSE); lq_run: of the E4M3 P that the MMA
        // uses (O is normalised by it, so the weights of the output rows sum to one)
        float m_run = -INFINITY, l_run = 0.f, lq_run = 0.f;
        v16f acc[16];   // [0, 8): row block hw, [8, 16): block 1 - hw; dim tile 8*hw + n
#pragma unroll
        for (int n = 0; n < 16; ++n) acc[n] = v16f{0};

        for (int t0 = 0; t0 < size; t0 += 2) {
            if (t0 > 0) {
                // pages t0, t0+1 resident; every wave is past pages t0-2, t0-1, whose slots
                // take pages t0+2, t0+3 (page 3 goes into slot 3, untouched so far)
                wait_pages_then_barrier(0);
                if (t0 + 2 < size) {
                    issue_page(page_at(pid_a), lds_base + ((t0 + 2) % kSlots) * kPageBytes, dmao);
                    pid_a = page_id(t0 + 4);
                }
                if (t0 + 3 < size) {
                    issue_page(page_at(pid_b), lds_base + ((t0 + 3) % kSlots) * kPageBytes, dmao);
                    pid_b = page_id(t0 + 5);
                }
            } else if (kSlots - 1 < size) {
                // page 3 into the free fourth slot
                issue_page(page_at(pid_a), lds_base + (kSlots - 1) * kPageBytes, dmao);
                pid_a = page_id(kSlots + 1);
                // (pid_b already holds page 4's entry, fetched at the next iteration)
                const int32_t swap = pid_a;
                pid_a = pid_b;
                pid_b = swap;
            }
            // keys past the request's length (its last page only): zero their rows so that
            // P V stays finite; their scores are masked by key index below
            const int tz = t0 + 1 < size ? t0 + 1 : t0;
            const int last_valid = L - (first + tz) * kPage;
            if (last_valid < kPage) {
                uint8_t *zs = lds + (tz % kSlots) * kPageBytes;
                for (int off = last_valid * kKDim + tid * 16; off < kPageBytes; off += kDecodeThreads * 16)
                    *(v4i *)(zs + off) = v4i{0, 0, 0, 0};
                lds_barrier();
            }
            const int t = t0 + pair;
            const bool has = t < size;
            const uint8_t *slot = lds + (t % kSlots) * kPageBytes;
            float alpha = 1.f;
            bool any_grow = false;
            v8i pf = v8i{0, 0, 0, 0, 0, 0, 0, 0};
            if (has && active) {
                // S^T[64 keys x 32 rows]: 18 MFMAs, K fragment reads two ahead
                v16f sc[2];
                const uint8_t *kp0 = slot + k_off[0], *kp1 = slot + k_off[1];
                sc[0] = v16f{0};
                sc[1] = v16f{0};
                v8i kf0 = lds_read2x16(kp0, kp1);
                v8i kf1 = lds_read2x16(kp0 + 64, kp1 + 64);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int j = 0; j < 18; ++j) {
                    const int b = j / 9, k = j % 9;
                    const v8i cur = (j & 1) ? kf1 : kf0;
                    if (j + 2 < 18) {
                        const int o = 32 * ((j + 2) / 9) * kKDim + 64 * ((j + 2) % 9);
                        if (j & 1)
                            kf1 = lds_read2x16(kp0 + o, kp1 + o);
                        else
                            kf0 = lds_read2x16(kp0 + o, kp1 + o);
                    }
                    sc[b] = mfma(cur, qf[k], sc[b]);
                    __builtin_amdgcn_sched_barrier(0);
                }
                const int valid = lim - (first + t) * kPage;   // keys of the page the row sees
                if (__any(valid < kPage)) {
#pragma unroll
                    for (int b = 0; b < 2; ++b)
#pragma unroll
                        for (int e = 0; e < 16; ++e)
                            if (32 * b + 8 * (e >> 2) + 4 * half + (e & 3) >= valid) sc[b][e] = -INFINITY;
                }
                float smax = -INFINITY;
#pragma unroll
                for (int b = 0; b < 2; ++b)
#pragma unroll
                    for (int e = 0; e < 16; ++e) smax = fmaxf(smax, sc[b][e]);
                const float mx = half_pair_max(smax) * a.score_scale;
                const bool grow = mx > m_run + kTau;
                any_grow = __any(grow);
                if (any_grow) {
                    const float m_new = grow ? mx : m_run;
                    // rows whose max stays keep factor 1 (exp2(m - m) would be NaN for a
                    // row that has seen no key yet, m = -inf)
                    alpha = grow ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
                    l_run *= alpha;
                    lq_run *= alpha;
                    m_run = m_new;
                }
                const float bias = m_run == -INFINITY ? 0.f : kPScale - m_run;   // no key seen: P = 0
                float psum = 0.f, qsum = 0.f;
#pragma unroll
                for (int g = 0; g < 8; ++g) {
                    const int b = g >> 2, qd = g & 3;
                    float p4[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        p4[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[b][4 * qd + e], a.score_scale, bias));
                        psum += p4[e];
                    }
                    int w4 = __builtin_amdgcn_cvt_pk_fp8_f32(p4[0], p4[1], 0, false);
                    w4 = __builtin_amdgcn_cvt_pk_fp8_f32(p4[2], p4[3], w4, true);
                    pf[g] = w4;
                    const v2f q0 = __builtin_amdgcn_cvt_pk_f32_fp8(w4, false);
                    const v2f q1 = __builtin_amdgcn_cvt_pk_f32_fp8(w4, true);
                    qsum += (q0[0] + q0[1]) + (q1[0] + q1[1]);
                }
                l_run += psum;
                lq_run += qsum;
            }
            // swap with the partner: P fragment, per-row rescale factor, rescale flag
            *(v8i *)&xch_p[wave][lane * 8] = pf;
            if (half == 0) xch_alpha[wave][l32] = alpha;
            if (lane == 0) xch_flag[wave] = any_grow ? 1 : 0;
            lds_barrier();
            if (has) {
                const v8i pf_other = *(const v8i *)&xch_p[wave ^ 1][lane * 8];
                const float alpha_other = xch_alpha[wave ^ 1][l32];
                const bool grow_other = xch_flag[wave ^ 1] != 0;
                if (any_grow) {
#pragma unroll
                    for (int n = 0; n < 8; ++n) acc[n] *= alpha;
                }
                if (grow_other) {
#pragma unroll
                    for (int n = 0; n < 8; ++n) acc[8 + n] *= alpha_other;
                }
                const uint8_t *vp0 = slot + tr_off[0], *vp1 = slot + tr_off[1];
                auto vtile = [&](int n) {
                    v8i f;
                    const uint8_t *vp = (n & 1) ? vp1 : vp0;
#pragma unroll
                    for (int w2 = 0; w2 < 4; ++w2) {
                        const v2i x = lds_read_tr8(vp + 16 * w2 * kKDim + 64 * (n >> 1));
                        f[2 * w2] = x[0];
                        f[2 * w2 + 1] = x[1];
                    }
                    return f;
                };
                v8i vf = vtile(0);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int n = 0; n < 8; ++n) {
                    const v8i cur = vf;
                    if (n + 1 < 8) vf = vtile(n + 1);
                    acc[n] = mfma(cur, pf, acc[n]);
                    acc[8 + n] = mfma(cur, pf_other, acc[8 + n]);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
        if (page_bad && tid == 0) atomicOr(&header[kHdrStatus], AMLA_DEV_BAD_PAGE);

        // merge the pairs.  Block b's state of pair p (m, l over its pages) is in wave
        // 2p + b; its O for dims half h is in wave 2p + h (slot own if b == h).
        const float l_tot = half_pair_sum(l_run), lq_tot = half_pair_sum(lq_run);
        lds_barrier();   // every wave is done with the ring and the exchange
        if (half == 0) {
            xm[pair][hw][l32] = m_run;
            xl[pair][hw][l32] = l_tot;
            xq[pair][hw][l32] = lq_tot;
        }
        lds_barrier();
        float f_blk[2];          // this pair's factor for block hw (own) and 1 - hw
        float m_blk[2], l_blk[2];
#pragma unroll
        for (int o = 0; o < 2; ++o) {
            const int b = o == 0 ? hw : 1 - hw;
            const float m0 = xm[0][b][l32], m1 = xm[1][b][l32];
            const float mm = fmaxf(m0, m1);
            const float e0 = m0 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m0 - mm);
            const float e1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - mm);
            const float ll = xl[0][b][l32] * e0 + xl[1][b][l32] * e1;
            const float lq = xq[0][b][l32] * e0 + xq[1][b][l32] * e1;
            const float mine = xm[pair][b][l32];
            f_blk[o] = mine == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mine - mm) * (a.out_scale / lq);
            m_blk[o] = mm;
            l_blk[o] = ll;
        }
        const size_t slot_idx = (size_t)off_r + s;
        // LSE of block `pair`, by the wave of this pair that holds it as its own block
        if (hw == pair && half == 0 && jt * MT + 32 * pair + l32 < M)
            lse_out[slot_idx * M + jt * MT + 32 * pair + l32] = m_blk[0] + __builtin_amdgcn_logf(l_blk[0]) - kPScale;
        // every wave stores its scaled O of block 1 - pair (the block the other pair
        // stores) in region [1 - pair][hw]; then it adds the other pair's O of block `pair`
        constexpr int kRegion = 32 * kMergeStride;
        float *const region = (float *)(void *)lds;
        {
            const int b = 1 - pair;
            const int o = b == hw ? 0 : 1;           // acc slot of block b
            float *mine = region + (b * 2 + hw) * kRegion + l32 * kMergeStride + 4 * half;
#pragma unroll
            for (int n = 0; n < 8; ++n) {
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const v16f &t16 = acc[8 * o + n];
                    *(v4f *)(mine + 32 * n + 8 * q4) =
                        v4f{t16[4 * q4], t16[4 * q4 + 1], t16[4 * q4 + 2], t16[4 * q4 + 3]} * f_blk[o];
                }
            }
        }
        lds_barrier();
        {
            const int b = pair;
            const int o = b == hw ? 0 : 1;
            const int row = jt * MT + 32 * b + l32;
            const float *theirs = region + (b * 2 + hw) * kRegion + l32 * kMergeStride + 4 * half;
            if (row < M) {
                float *po = partial + (slot_idx * M + row) * kVDim + 256 * hw;
#pragma unroll
                for (int n = 0; n < 8; ++n) {
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4) {
                        const v16f &t16 = acc[8 * o + n];
                        const v4f sum = v4f{t16[4 * q4], t16[4 * q4 + 1], t16[4 * q4 + 2], t16[4 * q4 + 3]} * f_blk[o] +
                                        *(const v4f *)(theirs + 32 * n + 8 * q4);
                        *(v4f *)(po + 32 * n + 8 * q4 + 4 * half) = sum;
                    }
                }
            }
        }
        lds_barrier();  // the next unit's pages overwrite the regions
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
    auto load_batch = [&](int s0, v4f (&part)[kCombineBatch][PER_LANE]) {
#pragma unroll
        for (int b = 0; b < kCombineBatch; ++b) {
            const int s = s0 + b < c ? s0 + b : c - 1;
            const float *p = a.partial + ((base + s) * a.rows + i) * kVDim + band * width;
#pragma unroll
            for (int k = 0; k < PER_LANE; ++k) part[b][k] = *(const v4f *)(p + 4 * (lane + 64 * k));
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
// One workgroup of 8 waves per (head h, 16 rows of that head); row j of head h is draft
// token t = j % k of request r = j / k, folded row i = t*H + h.  32 threads merge one row;
// the BF16 latent tile goes through LDS into the B operand of D[v][row] = W^T lat^T, wave w
// computing output dims [16w, 16w + 16), so each lane ends with four adjacent output dims
// of one row.
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
    constexpr int TPR = 512 / ROWS;        // threads per row: 32 or 64
    constexpr int NJ = kVDim / 4 / TPR;    // float4s per thread and split: 4 or 2
    __shared__ __attribute__((aligned(16))) uint16_t lat[kUvRows * kUvStride];
    __shared__ float wts[kUvRows][AMLA_MAX_SPLITS];
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
    v4f p[kUvBatch][NJ];
#pragma unroll
    for (int b = 0; b < kUvBatch; ++b) {
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
    for (int s0 = 0; s0 < c; s0 += kUvBatch) {
        if (s0 > 0) {
#pragma unroll
            for (int b = 0; b < kUvBatch; ++b) {
                const int sb = s0 + b < c ? s0 + b : c - 1;
#pragma unroll
                for (int jj = 0; jj < NJ; ++jj)
                    p[b][jj] = *(const v4f *)(prow + sb * pstride + 4 * TPR * jj);
            }
        }
#pragma unroll
        for (int b = 0; b < kUvBatch; ++b) {
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
    if (ROWS < kUvRows) {   // the MFMA's 16 rows: the tile's unused rows are zero
        for (int x = tid; x < (kUvRows - ROWS) * kVDim / 4; x += 512)
            *(uint2 *)(lat + (ROWS + x / (kVDim / 4)) * kUvStride + 4 * (x % (kVDim / 4))) =
                make_uint2(0u, 0u);
    }
    if (a.out_lse && j < per_head && tr == 0)
        a.out_lse[g] = bad ? NAN : c > 0 ? mx + __builtin_amdgcn_logf(sum) : -INFINITY;
    __syncthreads();

    // D[v][row] over K = 512 in 16 steps; B operand: lane l holds lat[row l%16][c = 32 s +
    // 8 (l/16) .. +7]
    v4f d = v4f{0, 0, 0, 0};
    const uint16_t *lb = lat + (lane & 15) * kUvStride + 8 * (lane >> 4);
#pragma unroll
    for (int s = 0; s < 16; ++s) {
        const bf16x8 bfr = *(const bf16x8 *)(lb + 32 * s);
        d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[s], bfr, d, 0, 0, 0);
    }
    // lane l holds D[v = 16 wave + 4 (l/16) + e][row l%16], e < 4
    const int jr = j0 + (lane & 15);
    if ((lane & 15) < ROWS && jr < per_head) {
        const int rr = jr / a.k;
        const int64_t gr = (int64_t)rr * a.rows + (int64_t)(jr - rr * a.k) * a.heads + h;
        const uint32_t lo = bf16_rne(d[0]) | ((uint32_t)bf16_rne(d[1]) << 16);
        const uint32_t hi = bf16_rne(d[2]) | ((uint32_t)bf16_rne(d[3]) << 16);
        *(uint2 *)(a.attn_out + gr * kUvDim + 16 * wave + 4 * (lane >> 4)) = make_uint2(lo, hi);
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
// One launch, two roles: blocks [0, query_blocks) build the query of (16 tokens, head h);
// the others write the cache rows of 4 tokens (one wave each).
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

__global__ __launch_bounds__(256) void build_query_cache_kernel(BuildArgs a)
{
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
        const int t0 = (blockIdx.x / a.heads) * kQbTokens;
        // B operand (q_nope^T): lane l holds q_nope[token t0 + l%16][c = 32 ks + 8 (l/16) ..+7]
        const int tok = t0 + (lane & 15);
        bf16x8 qb[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            if (tok < a.n)
                qb[ks] = *(const bf16x8 *)(a.q + ((int64_t)tok * a.heads + h) * 192 + 32 * ks + 8 * (lane >> 4));
            else
                qb[ks] = bf16x8{};
        }
        // A operand (W_UK): lane l holds W[h][l = 128 wave + 16 mt + l%16][c = 32 ks + 8 (l/16) ..]
        const uint16_t *wh = a.w_uk + ((int64_t)h * kVDim + 128 * wave + (lane & 15)) * 128 + 8 * (lane >> 4);
        v4f d[8];
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
            d[mt] = v4f{0, 0, 0, 0};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const bf16x8 wa = *(const bf16x8 *)(wh + 16 * 128 * mt + 32 * ks);
                d[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa, qb[ks], d[mt], 0, 0, 0);
            }
        }
        // lane l holds ql[token t0 + l%16][latent 128 wave + 16 mt + 4 (l/16) + e]
        if (tok < a.n) {
            uint8_t *qo = a.q_out + ((int64_t)tok * a.heads + h) * kKDim + 128 * wave + 4 * (lane >> 4);
#pragma unroll
            for (int mt = 0; mt < 8; ++mt)
                *(uint32_t *)(qo + 16 * mt) =
                    e4m3x4(bf16_round(d[mt][0]), bf16_round(d[mt][1]), bf16_round(d[mt][2]),
                           bf16_round(d[mt][3]), a.q_inv);
        }
        // rope(q_pe): thread (token t0 + tid/16, pairs 2 (tid%16) and 2 (tid%16) + 1)
        const int rt = t0 + (tid >> 4);
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
           (p->mode == AMLA_PLAN_BALANCED || p->mode == AMLA_PLAN_FIXED);
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
    *mtile_out = rows_per_req <= 32 ? 32 : (rows_per_req <= 64 ? 64 : 128);
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
    if (num_reqs <= kSmallReqs)
        hipLaunchKernelGGL(plan_small_kernel, dim3(1), dim3(kPlanThreads), 0, (hipStream_t)stream, a);
    else
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
    const dim3 grid(params->workers), block(kDecodeThreads);
    hipStream_t st = (hipStream_t)stream;
#define AMLA_DECODE_ARGS d_q, d_kv, d_block_table, d_lengths, d_counts, d_offsets, d_work, hdr, part, lse, a
    switch (params->mtile) {
    case 32: hipLaunchKernelGGL(decode32_kernel, grid, block, 0, st, AMLA_DECODE_ARGS); break;
    case 64: hipLaunchKernelGGL(decode64_kernel, grid, block, 0, st, AMLA_DECODE_ARGS); break;
    default: hipLaunchKernelGGL(decode128_kernel, grid, block, 0, st, AMLA_DECODE_ARGS); break;
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
    const int64_t qblocks = (int64_t)((n_tokens + kQbTokens - 1) / kQbTokens) * heads;
    const int64_t cblocks = (n_tokens + 3) / 4;
    if (qblocks + cblocks > 0x7FFFFFFF) return AMLA_ERR_INVALID;
    a.query_blocks = (int32_t)qblocks;
    hipLaunchKernelGGL(build_query_cache_kernel, dim3((unsigned)(qblocks + cblocks)), dim3(256), 0,
                       (hipStream_t)stream, a);
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
    // 16-row tiles, or 8-row tiles when 16-row tiles would leave compute units idle
    const int64_t tiles16 = (per_head + kUvRows - 1) / kUvRows;
    if (tiles16 * heads >= 256)
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
