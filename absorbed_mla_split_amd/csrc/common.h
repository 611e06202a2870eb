// Definitions shared by the translation units of the decode library: geometry, the
// workspace layout, vector types and the device helpers of the decode kernels (page DMA
// into LDS, the LDS layout, the lane-pair reductions, the MFMA wrappers).
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <type_traits>

#include "../../include/amla.h"

namespace amla {

constexpr int kPage = AMLA_PAGE;
constexpr int kKDim = AMLA_KDIM;
constexpr int kVDim = AMLA_VDIM;
constexpr int kPageBytes = kPage * kKDim;      // 36864
constexpr int kSlots = 4;                      // LDS page ring
constexpr int kDecodeThreads = 256;            // 4 waves
constexpr int kChunksPerWave = kPageBytes / (4 * 1024);  // 9 x 1 KiB DMA per wave per page
constexpr int kHeaderBytes = 256;
constexpr int kPlanThreads = 256;
// The work list and the workspace are sized for num_reqs + kPlanSlack * workers splits; a
// plan uses at most num_reqs + workers - 1 (one per request and one per cut between worker
// groups), and the list holds the group starts after its first 2 (num_reqs + workers)
// entries.
constexpr int kPlanSlack = 2;
constexpr float kLog2e = 1.4426950408889634f;
// Softmax of the decode kernels: P = 2^(s - m + kPExp) with m the row's reference plus a
// whole number per key block, at or above that block's running max, so P <= 2^8 < 448 (the
// E4M3 range); the output stays relative to the reference, which only moves when the
// running max passes it by more than kRefGap (FP32 headroom for the unnormalised O).
constexpr float kPExp = 8.0f;
constexpr int kRefGap = 64;

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

// issue_page with the lane's offsets taken through opaque copies: the compiler cannot
// hoist their unpacking out of a page loop (nine live or spilled registers instead of five).
__device__ __forceinline__ void issue_page_opaque(const uint8_t *page_base, uint32_t lds_dst,
                                                  const DmaOffsets &o)
{
    DmaOffsets c = o;
#pragma unroll
    for (int i = 0; i < (kChunksPerWave + 1) / 2; ++i) asm volatile("" : "+v"(c.v[i]));
    issue_page(page_base, lds_dst, c);
}

// DMA of one ring entry: 64 rows of 576 bytes, row i at `base + 576 i`, into the ring slot
// at `lds_dst` in the swizzled layout (`o`: the lane's offsets from dma_offsets).  Rows at or
// past `valid` (1..64) take a copy of row valid-1, so the slot holds only codes that belong
// to the entry and nothing past its valid rows is read.  OPAQUE: the offsets are computed
// from opaque copies of the lane's values (see issue_page_opaque).
template <bool OPAQUE = false>
__device__ __forceinline__ void issue_rows(const uint8_t *base, uint32_t lds_dst, int valid,
                                           const DmaOffsets &o, int wave, int lane)
{
    if (valid >= kPage) {
        if constexpr (OPAQUE)
            issue_page_opaque(base, lds_dst, o);
        else
            issue_page(base, lds_dst, o);
        return;
    }
    int ln = lane;
    if constexpr (OPAQUE) asm volatile("" : "+v"(ln));
    DmaOffsets c;
#pragma unroll
    for (int i = 0; i < (kChunksPerWave + 1) / 2; ++i) c.v[i] = 0;
#pragma unroll
    for (int i = 0; i < kChunksPerWave; ++i) {
        const int p = (wave * kChunksPerWave + i) * 64 + ln;
        const int row = p / (kKDim / 16), q = p - row * (kKDim / 16);
        const int src = row < valid ? row : valid - 1;
        c.v[i >> 1] |= (uint32_t)(src * kKDim + 16 * (q ^ swz(row))) << (16 * (i & 1));
    }
    issue_page(base, lds_dst, c);
}

// One of the nine DMA instructions of a wave's share of a ring entry: 1 KiB, lane l's 16
// bytes from `base` + `off` to `lds_dst` + 16 l (see issue_page), so that a caller can spread
// a page's DMA between other work instead of stalling on nine issues in a row.
__device__ __forceinline__ void issue_chunk(const uint8_t *base, uint32_t lds_dst, uint32_t off)
{
    base = uniform_ptr(base);
    lds_dst = __builtin_amdgcn_readfirstlane(lds_dst);
    asm volatile("s_mov_b32 m0, %[m]\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %[o], %[b]"
                 :
                 : [o] "v"(off), [b] "s"(base), [m] "s"(lds_dst)
                 : "memory");
}

// The lane's source offset of chunk i of a ring entry whose rows at or past `valid` repeat row
// valid-1 (see issue_rows), computed from opaque copies (see issue_page_opaque).
__device__ __forceinline__ uint32_t chunk_offset(const DmaOffsets &o, int i, int valid, int wave,
                                                 int lane)
{
    if (valid >= kPage) {
        uint32_t v = o.v[i >> 1];
        asm volatile("" : "+v"(v));
        return (i & 1) ? (v >> 16) : (v & 0xFFFFu);
    }
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int p = (wave * kChunksPerWave + i) * 64 + ln;
    const int row = p / (kKDim / 16), q = p - row * (kKDim / 16);
    const int src = row < valid ? row : valid - 1;
    return (uint32_t)(src * kKDim + 16 * (q ^ swz(row)));
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
// consecutive virtual workers (the row tiles of one worker group, which read the same
// pages) are put on the same XCD and share its L2.
__device__ __forceinline__ int virtual_worker(int b, int W, int mt)
{
    // with one row tile per split there is nothing to share
    if (mt == 1 || W % 8 != 0) return b;
    return (b % 8) * (W / 8) + b / 8;
}

// The worker groups of a plan (plan kernel): G = max(1, W / mt) groups of min(W, mt)
// workers; group g takes the items [work[2 (R + W) + g], work[2 (R + W) + g + 1]) of the
// work list, each with its mt row tiles, as units (item-major, tile-minor) that its workers
// take in turn.  Workers beyond the groups (W % mt of them) are idle.
struct WorkerGroup {
    int groups;      // G
    int list_at;     // 2 (R + W) + g: where the group's first item is listed
    int first_tile;  // the worker's first unit within an item's tiles
    int step;        // units between the worker's units
    bool active;
};

__device__ __forceinline__ WorkerGroup worker_group(int vw, int W, int mt, int R)
{
    WorkerGroup w;
    w.groups = W / mt > 0 ? W / mt : 1;
    w.step = W < mt ? W : mt;
    const int g = vw / w.step;
    w.active = g < w.groups;
    w.first_tile = vw - g * w.step;
    w.list_at = 2 * (R + W) + (w.active ? g : 0);
    return w;
}

__device__ __forceinline__ v16f mfma(v8i a, v8i b, v16f c)
{
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// The same product with B's column j scaled by 2^(sb - 127) (E8M0 byte sb of lane j and of
// lane j + 32, which hold that column), A unscaled (127: 2^0).
__device__ __forceinline__ v16f mfma_scaled_b(v8i a, v8i b, v16f c, int sb)
{
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, sb);
}

// S^T += K Q^T for the two row blocks of one k-step, VGPR results.  The 128-row decode
// holds its 256 output accumulators in AGPRs (the compiler's MFMAs there use the AGPR
// form); the score tiles must stay in VGPRs for the softmax, so these MFMAs are written
// here.  The compiler does not see them as MFMAs: the last step of a page pads 24 wait
// states after its MFMAs (a 16-pass XDL result read by VALU code needs fewer).
template <bool FIRST, bool LAST>
__device__ __forceinline__ void score_step(v16f &s0, v16f &s1, v8i k, v8i q0, v8i q1)
{
    if constexpr (FIRST && LAST) {
        asm volatile("v_mfma_f32_32x32x64_f8f6f4 %0, %2, %3, 0\n\t"
                     "v_mfma_f32_32x32x64_f8f6f4 %1, %2, %4, 0\n\t"
                     "s_nop 7\n\ts_nop 7\n\ts_nop 7"
                     : "=&v"(s0), "=&v"(s1) : "v"(k), "v"(q0), "v"(q1));
    } else if constexpr (FIRST) {
        asm volatile("v_mfma_f32_32x32x64_f8f6f4 %0, %2, %3, 0\n\t"
                     "v_mfma_f32_32x32x64_f8f6f4 %1, %2, %4, 0"
                     : "=&v"(s0), "=&v"(s1) : "v"(k), "v"(q0), "v"(q1));
    } else if constexpr (LAST) {
        asm volatile("v_mfma_f32_32x32x64_f8f6f4 %0, %2, %3, %0\n\t"
                     "v_mfma_f32_32x32x64_f8f6f4 %1, %2, %4, %1\n\t"
                     "s_nop 7\n\ts_nop 7\n\ts_nop 7"
                     : "+v"(s0), "+v"(s1) : "v"(k), "v"(q0), "v"(q1));
    } else {
        asm volatile("v_mfma_f32_32x32x64_f8f6f4 %0, %2, %3, %0\n\t"
                     "v_mfma_f32_32x32x64_f8f6f4 %1, %2, %4, %1"
                     : "+v"(s0), "+v"(s1) : "v"(k), "v"(q0), "v"(q1));
    }
}

// acc *= f for an accumulator tile held in AGPRs, eight registers per asm statement through
// eight VGPRs, so that the tile never leaves its AGPRs (the compiler would otherwise copy
// whole tiles between the register classes) and the reads, multiplies and writes of the
// eight registers pipeline.  The caller pads the hazard wait states around a run of these
// (an MFMA that has just written a tile; an MFMA reading a tile just written here).
__device__ __forceinline__ void scale_acc(v16f &t, float f)
{
#pragma unroll
    for (int h = 0; h < 16; h += 8) {
        float x0 = t[h], x1 = t[h + 1], x2 = t[h + 2], x3 = t[h + 3];
        float x4 = t[h + 4], x5 = t[h + 5], x6 = t[h + 6], x7 = t[h + 7];
        float y0, y1, y2, y3, y4, y5, y6, y7;
        asm volatile(
            "v_accvgpr_read_b32 %8, %0\n\tv_accvgpr_read_b32 %9, %1\n\t"
            "v_accvgpr_read_b32 %10, %2\n\tv_accvgpr_read_b32 %11, %3\n\t"
            "v_accvgpr_read_b32 %12, %4\n\tv_accvgpr_read_b32 %13, %5\n\t"
            "v_accvgpr_read_b32 %14, %6\n\tv_accvgpr_read_b32 %15, %7\n\t"
            "v_mul_f32 %8, %8, %16\n\tv_mul_f32 %9, %9, %16\n\t"
            "v_mul_f32 %10, %10, %16\n\tv_mul_f32 %11, %11, %16\n\t"
            "v_mul_f32 %12, %12, %16\n\tv_mul_f32 %13, %13, %16\n\t"
            "v_mul_f32 %14, %14, %16\n\tv_mul_f32 %15, %15, %16\n\t"
            "v_accvgpr_write_b32 %0, %8\n\tv_accvgpr_write_b32 %1, %9\n\t"
            "v_accvgpr_write_b32 %2, %10\n\tv_accvgpr_write_b32 %3, %11\n\t"
            "v_accvgpr_write_b32 %4, %12\n\tv_accvgpr_write_b32 %5, %13\n\t"
            "v_accvgpr_write_b32 %6, %14\n\tv_accvgpr_write_b32 %7, %15"
            : "+a"(x0), "+a"(x1), "+a"(x2), "+a"(x3), "+a"(x4), "+a"(x5), "+a"(x6), "+a"(x7),
              "=&v"(y0), "=&v"(y1), "=&v"(y2), "=&v"(y3), "=&v"(y4), "=&v"(y5), "=&v"(y6), "=&v"(y7)
            : "v"(f));
        t[h] = x0; t[h + 1] = x1; t[h + 2] = x2; t[h + 3] = x3;
        t[h + 4] = x4; t[h + 5] = x5; t[h + 6] = x6; t[h + 7] = x7;
    }
}

// An accumulator tile held in AGPRs, copied to VGPRs eight registers per asm statement.
// The AGPR operands keep the tile in its AGPRs up to this point (read as plain values, the
// compiler may move whole tiles into VGPRs at a loop exit).  The caller pads the wait states
// after the MFMA that last wrote the tile.
__device__ __forceinline__ v16f acc_read(const v16f &t)
{
    v16f o;
#pragma unroll
    for (int h = 0; h < 16; h += 8) {
        float y0, y1, y2, y3, y4, y5, y6, y7;
        asm volatile(
            "v_accvgpr_read_b32 %0, %8\n\tv_accvgpr_read_b32 %1, %9\n\t"
            "v_accvgpr_read_b32 %2, %10\n\tv_accvgpr_read_b32 %3, %11\n\t"
            "v_accvgpr_read_b32 %4, %12\n\tv_accvgpr_read_b32 %5, %13\n\t"
            "v_accvgpr_read_b32 %6, %14\n\tv_accvgpr_read_b32 %7, %15"
            : "=v"(y0), "=v"(y1), "=v"(y2), "=v"(y3), "=v"(y4), "=v"(y5), "=v"(y6), "=v"(y7)
            : "a"(t[h]), "a"(t[h + 1]), "a"(t[h + 2]), "a"(t[h + 3]), "a"(t[h + 4]),
              "a"(t[h + 5]), "a"(t[h + 6]), "a"(t[h + 7]));
        o[h] = y0; o[h + 1] = y1; o[h + 2] = y2; o[h + 3] = y3;
        o[h + 4] = y4; o[h + 5] = y5; o[h + 6] = y6; o[h + 7] = y7;
    }
    return o;
}

// Launches decode128_kernel (defined in decode128.hip, compiled with MFMA accumulators in
// AGPRs) on `stream`.
hipError_t launch_decode128(dim3 grid, hipStream_t stream, const uint8_t *q, const uint8_t *kv,
                            const int32_t *block_table, const int32_t *lengths,
                            const int32_t *counts, const int32_t *offsets, const int32_t *work,
                            int32_t *header, float *partial, float *lse, const DecodeArgs &a);

// Launches decode_stream_kernel<mtile> (32 or 64; defined in decode_stream.hip) on
// `stream`.
hipError_t launch_decode_stream(int mtile, dim3 grid, hipStream_t stream, const uint8_t *q,
                                const uint8_t *kv, const int32_t *block_table,
                                const int32_t *lengths, const int32_t *counts,
                                const int32_t *offsets, const int32_t *work, int32_t *header,
                                float *partial, float *lse, const DecodeArgs &a);

}  // namespace amla
