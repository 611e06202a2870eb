// Folded split-KV absorbed-MLA decode for MI355X (gfx950): plan, decode and combine
// kernels behind the C ABI declared in include/amla.h.
//
// Method (page "vllm.models.kimi_k3.nvidia.specialized_decode.drafter.attention", module
// docstring; page "...cutedsl.mla.balanced", module docstring): MQA over one latent head
// of 576 FP8 dims per token (value = the first 512), the k draft tokens of a request
// folded into its head axis, each request's keys cut into planned splits that produce
// FP32 partials and a log2 LSE, and a reducer merging the splits into BF16 rows.
//
// gfx950 mapping (this file's design, not the pages'):
//   * plan    one 1024-thread workgroup; binary search for the split chunk, block scans,
//             an LDS bitonic sort of per-request split runs to build the work list.
//   * decode  one persistent 256-thread workgroup per CU.  A work unit is (request, split,
//             row tile of MT = 32*G rows).  The four waves share one page stream: pages
//             (64 tokens x 576 B) go HBM -> LDS by global_load_lds_dwordx4 into a ring of
//             four page slots, three pages ahead of the one being computed.  Wave w owns
//             the 32-row group w / (4/G) and 512*G/4 of the output dims.  Per page:
//               S^T[64 keys x 32 rows] = K Q^T : 18 x v_mfma_f32_32x32x64_f8f6f4, K read
//                                                 from LDS, Q^T resident in VGPRs;
//               softmax in log2 units, lazy row max (rescale O only when the page max
//               exceeds it by more than 2^TAU), P = exp2(t - m) to E4M3 in-lane;
//               O^T[dims x 32 rows] += V^T P^T : V^T fragments come from LDS through
//                                                 ds_read_b64_tr_b8 transposed reads.
//             The accumulator layout puts one query row per lane, so the running max,
//             sum and rescale are lane-local; one lane-swap merges the two key halves.
//   * combine one wave per (row, band); merges the splits of a row with exp2 weights.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

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
constexpr int kPlanThreads = 1024;
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
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
#define LDS_AS __attribute__((address_space(3)))

struct WsLayout {
    size_t partial_off;  // FP32 [slots][M][512]
    size_t lse_off;      // FP32 [slots][M]
    size_t total;
};

__host__ __device__ inline WsLayout ws_layout(int64_t reqs, int64_t rows, int64_t workers)
{
    WsLayout w;
    const int64_t slots = reqs + workers;
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

// Sum over the 1024-thread plan workgroup; every thread gets the total.
__device__ int64_t block_sum64(int64_t v, int64_t *scratch)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    v = wave_sum(v);
    __syncthreads();
    if (lane == 0) scratch[wave] = v;
    __syncthreads();
    int64_t t = 0;
    for (int i = 0; i < kPlanThreads / 64; ++i) t += scratch[i];
    return t;
}

__device__ int64_t block_max64(int64_t v, int64_t *scratch)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    v = wave_max(v);
    __syncthreads();
    if (lane == 0) scratch[wave] = v;
    __syncthreads();
    int64_t t = scratch[0];
    for (int i = 1; i < kPlanThreads / 64; ++i) t = scratch[i] > t ? scratch[i] : t;
    return t;
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

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(PlanArgs a)
{
    __shared__ uint64_t keys[kMaxRuns];
    __shared__ int64_t red64[kPlanThreads / 64];
    __shared__ int32_t red32[kPlanThreads / 64];
    const int tid = threadIdx.x;
    const int R = a.reqs;
    const int64_t mt = ceil_div(a.rows, a.mtile);

    // 1. validate lengths, longest request
    int64_t bad = 0, pmax = 0;
    for (int r = tid; r < R; r += kPlanThreads) {
        const int32_t L = a.lengths[r];
        const int64_t p = pages_of(L);
        if (L < 0 || p > a.bt_cols) bad = 1;
        pmax = p > pmax ? p : pmax;
    }
    bad = block_max64(bad, red64);
    pmax = block_max64(pmax, red64);

    // 2. split chunk (BALANCED) or fixed split count
    int64_t chunk = 1, fixed = 1;
    if (!bad && a.mode == AMLA_PLAN_BALANCED) {
        int64_t lo = 1, hi = pmax > 0 ? pmax : 1;
        // units(c) = mt * sum_r ceil(p_r / c) is non-increasing in c: smallest c that fits.
        auto units = [&](int64_t c) {
            int64_t u = 0;
            for (int r = tid; r < R; r += kPlanThreads) u += (pages_of(a.lengths[r]) + c - 1) / c;
            return block_sum64(u, red64) * mt;
        };
        if (units(hi) <= a.workers) {
            while (lo < hi) {
                const int64_t mid = lo + (hi - lo) / 2;
                if (units(mid) <= a.workers) hi = mid; else lo = mid + 1;
            }
        }
        chunk = hi > a.min_pages ? hi : a.min_pages;
        if (chunk < 1) chunk = 1;
    } else if (!bad) {
        fixed = R > 0 ? (int64_t)a.workers / ((int64_t)R * mt) : 1;
        fixed = fixed < 1 ? 1 : (fixed > a.max_splits ? a.max_splits : fixed);
    }

    // 3. counts and offsets: thread t owns requests [t*per, (t+1)*per)
    const int per = ceil_div(R > 0 ? R : 1, kPlanThreads);
    int32_t mine = 0;
    for (int i = 0; i < per; ++i) {
        const int r = tid * per + i;
        if (r >= R) break;
        const int64_t p = pages_of(a.lengths[r]);
        int64_t c = 0;
        if (!bad && p > 0) {
            if (a.mode == AMLA_PLAN_BALANCED) {
                c = (p + chunk - 1) / chunk;
                c = c < a.max_splits ? c : a.max_splits;
            } else {
                c = p < fixed ? p : fixed;
            }
        }
        a.counts[r] = (int32_t)c;
        mine += (int32_t)c;
    }
    int32_t n_items = 0;
    int32_t run = block_exclusive_scan(mine, red32, &n_items);
    for (int i = 0; i < per; ++i) {
        const int r = tid * per + i;
        if (r >= R) break;
        a.offsets[r] = run;
        const int64_t p = pages_of(a.lengths[r]);
        int64_t c = 0;
        if (!bad && p > 0) {
            if (a.mode == AMLA_PLAN_BALANCED) {
                c = (p + chunk - 1) / chunk;
                c = c < a.max_splits ? c : a.max_splits;
            } else {
                c = p < fixed ? p : fixed;
            }
        }
        run += (int32_t)c;
    }
    if (tid == 0) a.offsets[R] = n_items;

    // 4. runs of equal-size splits: (q+1) x rem from s = 0, then q x (c - rem) from s = rem
    int n = 2;
    while (n < 2 * R) n <<= 1;
    for (int i = tid; i < n; i += kPlanThreads) keys[i] = ~0ull;
    __syncthreads();
    for (int r = tid; r < R && !bad; r += kPlanThreads) {
        const int64_t p = pages_of(a.lengths[r]);
        if (p == 0) continue;
        int64_t c;
        if (a.mode == AMLA_PLAN_BALANCED) {
            c = (p + chunk - 1) / chunk;
            c = c < a.max_splits ? c : a.max_splits;
        } else {
            c = p < fixed ? p : fixed;
        }
        const int64_t q = p / c, rem = p % c;
        if (rem > 0) keys[2 * r] = run_key(q + 1, r);
        keys[2 * r + 1] = run_key(q, r);
    }
    __syncthreads();

    // 5. bitonic sort of the run keys, ascending
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

    // 6. positions of the runs in sorted order, then the (r, s) pairs
    const int per_run = n / kPlanThreads > 0 ? n / kPlanThreads : 1;
    int32_t cnt_local[kMaxRuns / kPlanThreads > 0 ? kMaxRuns / kPlanThreads : 1];
    int32_t s0_local[kMaxRuns / kPlanThreads > 0 ? kMaxRuns / kPlanThreads : 1];
    int32_t r_local[kMaxRuns / kPlanThreads > 0 ? kMaxRuns / kPlanThreads : 1];
    int32_t my_items = 0;
    for (int i = 0; i < per_run; ++i) {
        const int idx = tid * per_run + i;
        cnt_local[i] = 0;
        s0_local[i] = 0;
        r_local[i] = 0;
        if (idx >= n) continue;
        const uint64_t key = keys[idx];
        if (key == ~0ull) continue;
        const int64_t size = 0x7FFFFFFFll - (int64_t)(key >> 32);
        const int32_t r = (int32_t)(key & 0xFFFFFFFFu);
        const int64_t p = pages_of(a.lengths[r]);
        const int32_t c = a.counts[r];
        const int64_t q = p / c, rem = p % c;
        if (rem > 0 && size == q + 1) {
            cnt_local[i] = (int32_t)rem;
            s0_local[i] = 0;
        } else {
            cnt_local[i] = (int32_t)(c - rem);
            s0_local[i] = (int32_t)rem;
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

// -------------------------------------------------------------------- decode kernel

struct DecodeArgs {
    int64_t pool_pages;
    int32_t bt_stride, reqs, rows, mtile, workers, list_len;
    float score_scale;  // bmm1 * log2(e)
    float out_scale;    // bmm2
};

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

// This wave's 9 KiB share of one page, HBM -> LDS, 16 B per lane per instruction
// (global_load_lds_dwordx4: lane i's 16 bytes land at M0 + 16*i).  Issued as inline asm
// so that the compiler does not count these loads: otherwise it waits for all of them
// before every transposed LDS read.  Completion is awaited explicitly with s_waitcnt
// vmcnt before the barrier that publishes a page.  The s_nop covers the SALU-write-M0 ->
// LDS-DMA hazard.
__device__ __forceinline__ void issue_page(const uint8_t *kv, int64_t page, uint8_t *slot, int wave,
                                           int lane)
{
    const uint8_t *src = kv + page * kPageBytes + wave * (kChunksPerWave * 1024) + lane * 16;
    const uint32_t dst = (uint32_t)(uintptr_t)(LDS_AS uint8_t *)slot + wave * (kChunksPerWave * 1024);
#pragma unroll
    for (int i = 0; i < kChunksPerWave; ++i) {
        const uint32_t m0 = __builtin_amdgcn_readfirstlane(dst + i * 1024);
        asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                     :
                     : "v"(src + i * 1024), "s"(m0)
                     : "memory", "m0");
    }
}

__device__ __forceinline__ v8i lds_read32(const uint8_t *p)
{
    const v4i a = *(const v4i *)p;
    const v4i b = *(const v4i *)(p + 16);
    return v8i{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

__device__ __forceinline__ v2i lds_read_tr8(const uint8_t *p)
{
    return __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS_AS v2i *)p);
}

// blockIdx -> virtual worker: hardware hands workgroups to the 8 XCDs round-robin, so
// virtual workers v and v+1 (the row tiles of one split) are put on the same XCD and
// share its L2.
__device__ __forceinline__ int virtual_worker(int b, int W)
{
    if (W % 8 != 0) return b;
    return (b % 8) * (W / 8) + b / 8;
}

// Read-only inputs are separate __restrict__ arguments so that the uniform reads
// (work list, counts, block table) become scalar loads, which do not wait on the
// in-flight page DMAs.
template <int G>
__global__ __launch_bounds__(kDecodeThreads, 1) void decode_kernel(
    const uint8_t *__restrict__ q_in, const uint8_t *__restrict__ kv_in,
    const int32_t *__restrict__ block_table, const int32_t *__restrict__ lengths,
    const int32_t *__restrict__ counts, const int32_t *__restrict__ offsets,
    const int32_t *__restrict__ work, int32_t *__restrict__ header, float *__restrict__ partial,
    float *__restrict__ lse_out, DecodeArgs a)
{
    constexpr int DS = 4 / G;        // waves per row group (they split the output dims)
    constexpr int NT = 16 / DS;      // 32-dim output tiles per wave
    constexpr int MT = 32 * G;       // rows per work unit
    __shared__ __attribute__((aligned(1024))) uint8_t lds[kSlots * kPageBytes];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int grp = wave / DS, dsi = wave % DS;
    const int l32 = lane & 31, half = lane >> 5;
    const int R = a.reqs, M = a.rows;
    const int mt = ceil_div(M, MT);
    const int W = a.workers;

    if (header[kHdrPlanned] != kPlannedMagic || header[kHdrRows] != M ||
        header[kHdrMtile] != MT || header[kHdrWorkers] != W || header[kHdrReqs] != R) {
        if (tid == 0 && blockIdx.x == 0) atomicOr(&header[kHdrStatus], AMLA_DEV_BAD_ITEM);
        return;
    }
    const int n_items = offsets[R];
    if (n_items < 0 || 2 * n_items > a.list_len || n_items > R + W) {
        if (tid == 0 && blockIdx.x == 0) atomicOr(&header[kHdrStatus], AMLA_DEV_BAD_ITEM);
        return;
    }
    const int units = n_items * mt;

    // tr8 read geometry (independent of the page): within each 16-lane group, source
    // lane i supplies key row b = i/2 and dims [8*(i%2), +8) of a 16-dim column block.
    const int g16 = lane >> 4, i16 = lane & 15;
    const int tr_dim = 16 * (g16 & 1) + 8 * (i16 & 1);                 // + 32 * tile
    const int tr_key = 8 * (i16 >> 3) + 4 * half + ((i16 >> 1) & 3);    // + 16 * w2

    for (int u = virtual_worker(blockIdx.x, W); u < units; u += W) {
        const int item = u / mt, jt = u - item * mt;
        const int r = work[2 * item], s = work[2 * item + 1];
        const bool item_ok = r >= 0 && r < R && s >= 0 && s < counts[r];
        if (!item_ok) {
            if (tid == 0) atomicOr(&header[kHdrStatus], AMLA_DEV_BAD_ITEM);
            continue;
        }
        const int L = lengths[r];
        const int c = counts[r];
        const int pages = ceil_div(L, kPage);
        const int q = pages / c, rem = pages % c;
        const int first = s * q + (s < rem ? s : rem);
        const int size = q + (s < rem ? 1 : 0);
        if (L <= 0 || pages > a.bt_stride || size <= 0 || offsets[r] + s >= n_items) {
            if (tid == 0) atomicOr(&header[kHdrStatus], AMLA_DEV_BAD_ITEM);
            continue;
        }
        const int row0 = jt * MT + 32 * grp;
        const bool active = row0 < M;
        const int32_t *bt = block_table + (size_t)r * a.bt_stride + first;

        // Q^T fragments: lane (row l32, half) holds dims [64k + 32*half, +32), k < 9.
        v8i qf[9];
        {
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
        }

        // The Q fragments are the only vector loads the compiler tracks; wait for them
        // here, before any page DMA is in flight, so that no later wait drains the ring.
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 63));

        float m_run = -INFINITY, l_run = 0.f;
        v16f acc[NT];
#pragma unroll
        for (int n = 0; n < NT; ++n) acc[n] = v16f{0};

        // prologue: up to kSlots-1 pages in flight
        bool page_bad = false;
        for (int d = 0; d < kSlots - 1 && d < size; ++d) {
            int64_t pid = bt[d];
            if (pid < 0 || pid >= a.pool_pages) { page_bad = true; pid = 0; }
            issue_page(kv_in, pid, lds + d * kPageBytes, wave, lane);
        }

        for (int t = 0; t < size; ++t) {
            const int after = size - 1 - t;
            wait_pages_then_barrier(after < kSlots - 2 ? after : kSlots - 2);
            if (t + kSlots - 1 < size) {
                int64_t pid = bt[t + kSlots - 1];
                if (pid < 0 || pid >= a.pool_pages) { page_bad = true; pid = 0; }
                issue_page(kv_in, pid, lds + ((t + kSlots - 1) % kSlots) * kPageBytes, wave, lane);
            }
            uint8_t *slot = lds + (t % kSlots) * kPageBytes;
            const int valid = L - (first + t) * kPage;   // >= 1
            if (valid < kPage) {
                // keys past the request's length: zero the rows so P*V stays finite
                for (int off = valid * kKDim + tid * 16; off < kPageBytes; off += kDecodeThreads * 16)
                    *(v4i *)(slot + off) = v4i{0, 0, 0, 0};
                lds_barrier();
            }
            if (!active) continue;

            // S^T = K Q^T for the page's two 32-key blocks: 18 MFMAs, each fed by two
            // 16-byte LDS reads of one key row; the reads run two fragments ahead.
            v16f sacc[2] = {v16f{0}, v16f{0}};
            {
                const uint8_t *kp = slot + l32 * kKDim + 32 * half;
                v8i kf[2];
                kf[0] = lds_read32(kp);
                kf[1] = lds_read32(kp + 64);
#pragma unroll
                for (int j = 0; j < 18; ++j) {
                    const int b = j / 9, k = j % 9;
                    const v8i cur = kf[j & 1];
                    if (j + 2 < 18) {
                        const int b2 = (j + 2) / 9, k2 = (j + 2) % 9;
                        kf[j & 1] = lds_read32(kp + 32 * b2 * kKDim + 64 * k2);
                    }
                    sacc[b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(cur, qf[k], sacc[b],
                                                                             0, 0, 0, 0, 0, 0);
                }
                // keep the reads two MFMAs ahead (and no further: registers)
                __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
                for (int j = 0; j < 18; ++j) {
                    if (j + 2 < 18) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                }
            }

            // scores in log2 units; lane holds row l32 and keys 32b + 8(e/4) + 4*half + e%4
            float mx = -INFINITY;
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int key = 32 * b + 8 * (e >> 2) + 4 * half + (e & 3);
                    const float tv = key < valid ? sacc[b][e] * a.score_scale : -INFINITY;
                    sacc[b][e] = tv;
                    mx = fmaxf(mx, tv);
                }
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const bool grow = mx > m_run + kTau;
            if (__any(grow)) {
                const float m_new = grow ? mx : m_run;
                const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
                l_run *= alpha;
#pragma unroll
                for (int n = 0; n < NT; ++n) acc[n] *= alpha;
                m_run = m_new;
            }

            // P = 2^(t - m): FP32 into the row sum, E4M3 (scaled by 2^kPScale) into P^T
            v8i pf;
            float psum = 0.f;
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int qd = 0; qd < 4; ++qd) {
                    float p[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        p[e] = __builtin_amdgcn_exp2f(sacc[b][4 * qd + e] - m_run + kPScale);
                        psum += p[e];
                    }
                    int w = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], 0, false);
                    w = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], w, true);
                    pf[4 * b + qd] = w;
                }
            l_run += psum;

            // O^T += V^T P^T: per 32-dim tile, four transposed LDS reads build the V^T
            // fragment; the reads run one tile ahead of the MFMAs.
            {
                const uint8_t *vp = slot + tr_key * kKDim + 32 * dsi * NT + tr_dim;
                auto vtile = [&](int n) {
                    v8i f;
#pragma unroll
                    for (int w2 = 0; w2 < 4; ++w2) {
                        const v2i x = lds_read_tr8(vp + 16 * w2 * kKDim + 32 * n);
                        f[2 * w2] = x[0];
                        f[2 * w2 + 1] = x[1];
                    }
                    return f;
                };
                v8i vf = vtile(0);
#pragma unroll
                for (int n = 0; n < NT; ++n) {
                    const v8i cur = vf;
                    if (n + 1 < NT) vf = vtile(n + 1);
                    acc[n] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(cur, pf, acc[n], 0, 0,
                                                                            0, 0, 0, 0);
                }
                __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
                for (int n = 0; n < NT; ++n) {
                    if (n + 1 < NT) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                }
            }
        }
        if (page_bad && tid == 0) atomicOr(&header[kHdrStatus], AMLA_DEV_BAD_PAGE);

        // epilogue: normalise and store this split's FP32 partial and log2 LSE.
        // l_run is scaled by 2^kPScale like P, so the scale cancels in O / l.
        if (active) {
            const float l_tot = l_run + __shfl_xor(l_run, 32);
            const int row = row0 + l32;
            if (row < M) {
                const size_t slot_idx = (size_t)offsets[r] + s;
                float *po = partial + (slot_idx * M + row) * kVDim;
                const float inv = a.out_scale / l_tot;
#pragma unroll
                for (int n = 0; n < NT; ++n) {
                    const int dim = 32 * (dsi * NT + n) + 4 * half;
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4) {
                        const v4f o = v4f{acc[n][4 * q4], acc[n][4 * q4 + 1], acc[n][4 * q4 + 2],
                                          acc[n][4 * q4 + 3]} * inv;
                        *(v4f *)(po + dim + 8 * q4) = o;
                    }
                }
                if (dsi == 0 && half == 0)
                    lse_out[slot_idx * M + row] =
                        m_run + __builtin_amdgcn_logf(l_tot) - kPScale;
            }
        }
        lds_barrier();  // the next unit's prologue overwrites the ring
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

// One wave per (row, band): band b covers dims [b*512/bands, (b+1)*512/bands).
__global__ __launch_bounds__(64) void combine_kernel(CombineArgs a)
{
    __shared__ float weight[AMLA_MAX_SPLITS];
    const int lane = threadIdx.x;
    const int64_t g = blockIdx.x / a.bands;       // folded row, request-major
    const int band = blockIdx.x % a.bands;
    const int r = (int)(g / a.rows), i = (int)(g % a.rows);
    const int c = a.counts[r];
    const int width = kVDim / a.bands;            // 512 or 256
    const int per_lane = width / 256;             // float4s per lane: 2 or 1
    uint16_t *out = a.out + g * kVDim + band * width;

    if (c <= 0) {
        for (int k = 0; k < per_lane; ++k)
            *(uint2 *)(out + 4 * (lane + 64 * k)) = make_uint2(0u, 0u);
        if (band == 0 && lane == 0) a.out_lse[g] = -INFINITY;
        return;
    }
    const int64_t base = a.offsets[r];
    if (c > AMLA_MAX_SPLITS || base < 0 || base + c > a.slots) {
        // not a plan of these sizes: flag the row as NaN rather than read out of bounds
        for (int k = 0; k < per_lane; ++k)
            *(uint2 *)(out + 4 * (lane + 64 * k)) = make_uint2(0x7FC07FC0u, 0x7FC07FC0u);
        if (band == 0 && lane == 0) a.out_lse[g] = NAN;
        return;
    }
    float mx = -INFINITY;
    for (int s = lane; s < c; s += 64) mx = fmaxf(mx, a.lse[(base + s) * a.rows + i]);
    mx = wave_max(mx);
    float sum = 0.f;
    for (int s = lane; s < c; s += 64) sum += __builtin_amdgcn_exp2f(a.lse[(base + s) * a.rows + i] - mx);
    sum = wave_sum(sum);
    for (int s = lane; s < c; s += 64)
        weight[s] = __builtin_amdgcn_exp2f(a.lse[(base + s) * a.rows + i] - mx) / sum;
    __syncthreads();

    v4f acc[2] = {v4f{0, 0, 0, 0}, v4f{0, 0, 0, 0}};
    for (int s = 0; s < c; ++s) {
        const float w = weight[s];
        const float *p = a.partial + ((base + s) * a.rows + i) * kVDim + band * width;
        for (int k = 0; k < per_lane; ++k) acc[k] += w * *(const v4f *)(p + 4 * (lane + 64 * k));
    }
    for (int k = 0; k < per_lane; ++k) {
        const uint32_t lo = bf16_rne(acc[k][0]) | ((uint32_t)bf16_rne(acc[k][1]) << 16);
        const uint32_t hi = bf16_rne(acc[k][2]) | ((uint32_t)bf16_rne(acc[k][3]) << 16);
        *(uint2 *)(out + 4 * (lane + 64 * k)) = make_uint2(lo, hi);
    }
    if (band == 0 && lane == 0) a.out_lse[g] = mx + __builtin_amdgcn_logf(sum);
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

}  // namespace

// ============================================================================ C ABI

extern "C" {

int amla_fold_plan(int32_t causal, int32_t num_reqs, int32_t num_rows, int32_t num_decode_tokens,
                   int32_t block_table_rows, int32_t max_query_len, int32_t heads,
                   int32_t need_lse, int32_t max_fold_heads, int32_t *k_out, int32_t *fold_out)
{
    if (!k_out || !fold_out || heads < 1 || (need_lse && max_fold_heads < heads))
        return AMLA_ERR_INVALID;
    *k_out = 0;
    *fold_out = 0;
    if (causal || num_reqs <= 0 || num_rows != num_decode_tokens || num_rows % num_reqs != 0)
        return AMLA_OK;
    const int32_t k = num_rows / num_reqs;
    if (k < 2 || block_table_rows < num_reqs || max_query_len != k) return AMLA_OK;
    int32_t f = 1;
    if (!need_lse) {
        f = k;
    } else {
        for (int32_t d = 1; d <= k; ++d)
            if (k % d == 0 && (int64_t)d * heads <= max_fold_heads) f = d;
    }
    *k_out = k;
    *fold_out = f;
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
    if ((int64_t)list_len < 2 * ((int64_t)num_reqs + params->workers)) return AMLA_ERR_LIST;
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
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, (hipStream_t)stream, a);
    return hipGetLastError() == hipSuccess ? AMLA_OK : AMLA_ERR_HIP;
}

int amla_folded_decode(const uint8_t *d_q, const uint8_t *d_kv, int64_t pool_pages,
                       const int32_t *d_block_table, int32_t bt_stride, const int32_t *d_lengths,
                       int32_t num_reqs, const amla_plan_params *params, float bmm1_scale,
                       float bmm2_scale, const int32_t *d_counts, const int32_t *d_offsets,
                       const int32_t *d_work, int32_t list_len, void *d_workspace,
                       size_t ws_bytes, void *stream)
{
    if (!params_ok(params) || num_reqs < 0 || num_reqs > AMLA_MAX_REQS || pool_pages < 1 ||
        bt_stride < 1 || !d_kv || !d_offsets || !d_work || !d_workspace ||
        (num_reqs > 0 && (!d_q || !d_block_table || !d_lengths || !d_counts)) ||
        !std::isfinite(bmm1_scale) || !std::isfinite(bmm2_scale))
        return AMLA_ERR_INVALID;
    const WsLayout lay = ws_layout(num_reqs, params->rows_per_req, params->workers);
    if (ws_bytes < lay.total) return AMLA_ERR_WORKSPACE;
    if ((int64_t)list_len < 2 * ((int64_t)num_reqs + params->workers)) return AMLA_ERR_LIST;
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
    int32_t *hdr = (int32_t *)d_workspace;
    float *part = (float *)((char *)d_workspace + lay.partial_off);
    float *lse = (float *)((char *)d_workspace + lay.lse_off);
    const dim3 grid(params->workers), block(kDecodeThreads);
    hipStream_t st = (hipStream_t)stream;
#define AMLA_DECODE_ARGS d_q, d_kv, d_block_table, d_lengths, d_counts, d_offsets, d_work, hdr, part, lse, a
    switch (params->mtile) {
    case 32: hipLaunchKernelGGL(decode_kernel<1>, grid, block, 0, st, AMLA_DECODE_ARGS); break;
    case 64: hipLaunchKernelGGL(decode_kernel<2>, grid, block, 0, st, AMLA_DECODE_ARGS); break;
    default: hipLaunchKernelGGL(decode_kernel<4>, grid, block, 0, st, AMLA_DECODE_ARGS); break;
    }
#undef AMLA_DECODE_ARGS
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
    a.slots = num_reqs + params->workers;
    hipLaunchKernelGGL(combine_kernel, dim3((unsigned)(rows * bands)), dim3(64), 0,
                       (hipStream_t)stream, a);
    return hipGetLastError() == hipSuccess ? AMLA_OK : AMLA_ERR_HIP;
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
    }
    return "unknown status";
}

}  // extern "C"
