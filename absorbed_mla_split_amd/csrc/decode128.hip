// The 128-row decode kernel (row tiles of 128 folded rows: the compute-bound shapes).
// It is its own translation unit because it is compiled with MFMA accumulators in AGPRs
// (the other kernels keep the VGPR form): see decode128_kernel.
#include "common.h"

namespace amla {
namespace {

// S^T of both key blocks of a page for one k-step: key block kb's K fragment (A) times the
// row block's Q^T fragment (B, shared), VGPR results.  The kernel's output accumulators
// are AGPR-form MFMAs; these are written here so that the score tiles stay in VGPRs.  The
// compiler does not see them as MFMAs: PAD adds 24 wait states after them, for a result
// read by VALU code right after (a 16-pass XDL result read by VALU code needs fewer).
template <bool FIRST, bool PAD>
__device__ __forceinline__ void score_kpair(v16f &s0, v16f &s1, v8i k0, v8i k1, v8i q)
{
    if constexpr (FIRST) {
        asm volatile("v_mfma_f32_32x32x64_f8f6f4 %0, %2, %4, 0\n\t"
                     "v_mfma_f32_32x32x64_f8f6f4 %1, %3, %4, 0"
                     : "=&v"(s0), "=&v"(s1) : "v"(k0), "v"(k1), "v"(q));
    } else {
        asm volatile("v_mfma_f32_32x32x64_f8f6f4 %0, %2, %4, %0\n\t"
                     "v_mfma_f32_32x32x64_f8f6f4 %1, %3, %4, %1"
                     : "+v"(s0), "+v"(s1) : "v"(k0), "v"(k1), "v"(q));
    }
    if constexpr (PAD) asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
}

// 128-row tiles, four waves, each owning 32 rows of the tile end to end: wave w computes
// S^T (the page's 64 keys, two key blocks of 32, x its rows [32w, +32)), the softmax of its
// rows, and O^T (the 512 value dims, sixteen 32-dim tiles in AGPRs, x its rows).  The lane
// that holds a row's scores (column l % 32 of S^T) is the lane that supplies that row's
// column of the P^T operand, so P goes from the exponentials to the P V MFMA in registers:
// the waves exchange nothing, and meet only once per page, where the page ring advances.
//
// Each wave software-pipelines its pages: while the MFMAs of page t+1's scores run, the
// VALU computes page t's softmax (mask, row max, reference, exponentials, E4M3 P), and
// while page t's P V MFMAs run, the VALU adds up page t's E4M3 P.  The LDS ring holds
// four pages: V of page t, K of page t+1 and two pages in flight; the DMA of page t+3 goes
// into the slot that page t-1 used.  Read-only inputs are separate __restrict__
// arguments; their uniform reads go through the constant address space (scalar loads,
// which do not wait on the in-flight page DMAs).
//
// Softmax in log2 units against a per-row reference (page "...cutedsl.mla.balanced",
// module docstring: the row max is kept lazily and P is fed to the MMA in E4M3): m_ref is
// the row's max over the unit's first page, and on each page key block kb's P is
// 2^(s - m_ref - g_kb + kPExp) <= 2^8 with g_kb the smallest whole number at or above that
// block's max over the page minus m_ref (at least -127).  The P V MFMA scales K block kb of
// its B operand by the E8M0 byte 127 + g_kb, so O and the row sums stay relative to m_ref
// with no rescaling, while each page's P uses the E4M3 range from its own max down.  A
// page whose max passes m_ref by more than kRefGap (log2 units; practically never) moves
// the reference up and rescales the wave's tiles.
__global__ __launch_bounds__(kDecodeThreads, 1) void decode128_kernel(
    const uint8_t *__restrict__ q_in, const uint8_t *__restrict__ kv_in,
    const int32_t *__restrict__ block_table, const int32_t *__restrict__ lengths,
    const int32_t *__restrict__ counts, const int32_t *__restrict__ offsets,
    const int32_t *__restrict__ work, int32_t *__restrict__ header, float *__restrict__ partial,
    float *__restrict__ lse_out, DecodeArgs a)
{
    constexpr int MT = 128;          // rows per work unit
    __shared__ __attribute__((aligned(1024))) uint8_t lds[kSlots * kPageBytes];

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
    // tr_key + 16*w2; dims [32*T + 16*(g16&1) + 8*(i16&1), +8) of dim tile T lie in chunk
    // 2*T + (g16&1), swizzled by the key row (the same for the four w2 rows).
    const int g16 = lane >> 4, i16 = lane & 15;
    const int tr_key = 8 * (i16 >> 3) + 4 * half + ((i16 >> 1) & 3);
    int tr_off[2];
#pragma unroll
    for (int par = 0; par < 2; ++par)
        tr_off[par] = tr_key * kKDim + 16 * ((2 * par + (g16 & 1)) ^ swz(tr_key)) + 8 * (i16 & 1);
    // K fragment reads: key l32 of key block 0 (block 1: 32 rows further, the same swizzle),
    // chunks 4k + 2*half + e
    const int k_off0 = l32 * kKDim + 16 * ((2 * half) ^ swz(l32));
    const int k_off1 = l32 * kKDim + 16 * ((2 * half + 1) ^ swz(l32));
    constexpr int kBlock1 = 32 * kKDim;

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
        const int rbase = jt * MT + 32 * wave;   // this wave's rows: [rbase, +32)
        const int row = rbase + l32;
        const int lim = row_key_limit(a, total, L, row);   // keys the lane's row sees
        const int32_t *bt = block_table + (size_t)r * a.bt_stride + first;

        bool page_bad = false;
        // page t of the split into its ring slot; rows past the request's length (only on
        // its last page) repeat the last valid row, so that P*V reads no foreign codes
        auto issue = [&](int t, int32_t pid) {
            if (pid < 0 || pid >= a.pool_pages) {
                page_bad = true;
                pid = 0;
            }
            const int valid = L - (first + t) * kPage;
            issue_rows<true>(kv_in + (int64_t)pid * kPageBytes, lds_base + (t % kSlots) * kPageBytes,
                       valid < kPage ? valid : kPage, dmao, wave, lane);
        };
        // block-table entry of page min(t, size - 1)
        auto page_id = [&](int t) { return ldc(&bt[t < size ? t : size - 1]); };

        // The first two pages' block-table entries, loaded together, and the entry of the
        // next page to fetch; the first pages' DMA, then the Q^T fragments of the wave's rows
        // from global memory, so that both latencies overlap; then wait for all of it (the
        // compiler tracks the Q loads, not the DMA).
        const int32_t pid_a = page_id(0), pid_b = page_id(1);
        asm volatile("" ::"s"(pid_a), "s"(pid_b));
        int32_t pid_next = page_id(2);
        issue(0, pid_a);
        if (size > 1) issue(1, pid_b);
        // Q^T fragment of k-step k: row `row`, bytes [64k + 32*half, +32); a row past M (in
        // a last tile) reads row M-1: its scores are computed and never stored
        v8i qf[9];
        {
            const uint8_t *qp = q_in + ((size_t)r * M + (row < M ? row : M - 1)) * kKDim + 32 * half;
#pragma unroll
            for (int k = 0; k < 9; ++k) {
                const v4i x = *(const v4i *)(qp + 64 * k);
                const v4i y = *(const v4i *)(qp + 64 * k + 16);
                qf[k] = v8i{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
            }
        }
        wait_pages_then_barrier(0);

        // the row's reference and its sums relative to it: FP32 P (for the LSE) and E4M3 P
        // (O is normalised by the sum of the P it was built from); per lane the keys of
        // its half, added over the lane pair at the end
        float m_ref = -INFINITY, l_run = 0.f, lq_run = 0.f;
        v16f acc[16];   // O^T of dim tile n (dims [32n, +32)) x the wave's rows
#pragma unroll
        for (int n = 0; n < 16; ++n) acc[n] = v16f{0};

        // S^T of the page in ring slot `slot` into sc (both key blocks).  The K fragments of
        // k-step k+1 are read into the registers of k-step k once its MFMAs are issued (an
        // MFMA reads its A and B operands at issue); `work(k)` runs after them, so that its
        // VALU work overlaps the MFMAs and the reads.
        v16f sc[2];
        auto score = [&](const uint8_t *slot, auto &&work) {
            v8i kf0 = lds_read2x16(slot + k_off0, slot + k_off1);
            v8i kf1 = lds_read2x16(slot + kBlock1 + k_off0, slot + kBlock1 + k_off1);
            static_for<0, 9>([&](auto kk) {
                constexpr int k = decltype(kk)::value;
                score_kpair<k == 0, false>(sc[0], sc[1], kf0, kf1, qf[k]);
                __builtin_amdgcn_sched_barrier(0);
                if constexpr (k + 1 < 9) {
                    kf0 = lds_read2x16(slot + 64 * (k + 1) + k_off0, slot + 64 * (k + 1) + k_off1);
                    kf1 = lds_read2x16(slot + kBlock1 + 64 * (k + 1) + k_off0,
                                       slot + kBlock1 + 64 * (k + 1) + k_off1);
                }
                work(kk);
                __builtin_amdgcn_sched_barrier(0);
            });
        };
        // O^T[dims 32n.., rows] += V^T (P^T, K block h scaled by 2^(sbv_h - 127)) for the page
        // in `slot`, the V^T fragments read one tile ahead; `work(n)` runs after the MFMA of
        // dim tile n is issued.
        auto pv = [&](const uint8_t *slot, const v8i &pfv, int sbv, auto &&work) {
            auto vtile = [&](int n) {
                const uint8_t *vp = slot + tr_off[n & 1] + 64 * (n >> 1);
                v8i f;
#pragma unroll
                for (int w2 = 0; w2 < 4; ++w2) {
                    const v2i x = lds_read_tr8(vp + 16 * w2 * kKDim);
                    f[2 * w2] = x[0];
                    f[2 * w2 + 1] = x[1];
                }
                return f;
            };
            v8i vf = vtile(0);
            static_for<0, 16>([&](auto nn) {
                constexpr int n = decltype(nn)::value;
                v8i cv = vf;
                if constexpr (n + 1 < 16) vf = vtile(n + 1);
                // operands in VGPRs (the allocator would otherwise load some into AGPRs,
                // which the sixteen accumulator tiles fill)
                asm volatile("" : "+v"(cv));
                acc[n] = mfma_scaled_b(cv, pfv, acc[n], sbv);
                __builtin_amdgcn_sched_barrier(0);
                work(nn);
                __builtin_amdgcn_sched_barrier(0);
            });
        };

        // Page t: its scores (with page t-1's E4M3 sum), then page t-1's P V MFMAs with page
        // t's softmax: mask, row max, reference, exponentials, E4M3 P.
        v8i pf, pf_prev;          // P^T fragments: bytes [16kb, +16) are key block kb
        int g0 = 0, g1 = 0;       // page t's whole-number gaps (key blocks 0, 1)
        int gp0 = 0, gp1 = 0;     // page t-1's
        auto page = [&](int t, auto has_prev) {
            constexpr bool PREV = decltype(has_prev)::value;
            if (t > 0) {
                wait_pages_then_barrier(t + 1 < size ? 1 : 0);
            }
            if (t + 2 < size) issue(t + 2, pid_next);
            {
                const uint8_t *slot_t = lds + (t % kSlots) * kPageBytes;
                float qs0 = 0.f, qs1 = 0.f;
                // page t-1's E4M3 P dwords, added up for lq while the score MFMAs run
                score(slot_t, [&](auto kk) {
                    constexpr int k = decltype(kk)::value;
                    if constexpr (PREV && k < 8) {
                        const v2f x0 = __builtin_amdgcn_cvt_pk_f32_fp8(pf_prev[k], false);
                        const v2f x1 = __builtin_amdgcn_cvt_pk_f32_fp8(pf_prev[k], true);
                        const float d4 = (x0[0] + x0[1]) + (x1[0] + x1[1]);
                        if constexpr (k < 4) qs0 += d4; else qs1 += d4;
                    }
                });
                if constexpr (PREV)
                    lq_run += __builtin_amdgcn_ldexpf(qs0, gp0) + __builtin_amdgcn_ldexpf(qs1, gp1);

                // keys of the page the lane's row sees, counted from the lane's first key
                // (4*half): element e of key block kb holds key 32kb + 8(e/4) + e%4 past it
                const int valid = lim - (first + t) * kPage - 4 * half;
                float mx0 = -INFINITY, mx1 = -INFINITY;
                float b0 = 0.f, b1 = 0.f, ps0 = 0.f, ps1 = 0.f;
                int moved = 0;   // log2 step of the reference on this page
                auto softmax = [&](auto nn) {
                    constexpr int n = decltype(nn)::value;
                    if constexpr (n == 0) {
                        // the score MFMAs' results, read by VALU code: wait states the
                        // compiler does not count for their asm
                        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
                        if (__any(valid < kPage)) {
#pragma unroll
                            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                                for (int e = 0; e < 16; ++e)
                                    if (32 * kb + 8 * (e >> 2) + (e & 3) >= valid) sc[kb][e] = -INFINITY;
                        }
#pragma unroll
                        for (int e = 0; e < 16; ++e) mx0 = fmaxf(mx0, sc[0][e]);
                    } else if constexpr (n == 1) {
#pragma unroll
                        for (int e = 0; e < 16; ++e) mx1 = fmaxf(mx1, sc[1][e]);
                        mx0 = half_pair_max(mx0) * a.score_scale;
                        mx1 = half_pair_max(mx1) * a.score_scale;
                    } else if constexpr (n == 2) {
                        // -inf while the row sees no key: with visible keys a prefix of the
                        // shard, a row that sees no key of its split's first page sees none
                        if (t == 0) m_ref = fmaxf(mx0, mx1);
                        const bool none = m_ref == -INFINITY;
                        g0 = none ? 0 : (int)__builtin_ceilf(fmaxf(mx0 - m_ref, -127.f));
                        g1 = none ? 0 : (int)__builtin_ceilf(fmaxf(mx1 - m_ref, -127.f));
                        // a block more than kRefGap above the reference moves it up by the
                        // larger block's gap (the tiles follow once page t-1's MFMAs are done)
                        const int gmax = g0 > g1 ? g0 : g1;
                        moved = gmax > kRefGap ? gmax : 0;
                        const float f = __builtin_amdgcn_ldexpf(1.f, -moved);
                        m_ref += (float)moved;
                        g0 = g0 - moved < -127 ? -127 : g0 - moved;
                        g1 = g1 - moved < -127 ? -127 : g1 - moved;
                        l_run *= f;
                        lq_run *= f;
                        b0 = none ? 0.f : (kPExp - (float)g0) - m_ref;
                        b1 = none ? 0.f : (kPExp - (float)g1) - m_ref;
                    } else if constexpr (n >= 3 && n <= 10) {
                        // P = 2^(s*scale - m_ref - g + kPExp) for 4 elements: FP32 into the
                        // block's sum, E4M3 into one dword of the fragment
                        constexpr int kb = (n - 3) >> 2, e0 = 4 * ((n - 3) & 3);
                        const float bias = kb ? b1 : b0;
                        float p[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kb][e0 + i], a.score_scale, bias));
                        const float sum = (p[0] + p[1]) + (p[2] + p[3]);
                        if constexpr (kb == 0) ps0 += sum; else ps1 += sum;
                        int w4 = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], 0, false);
                        w4 = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], w4, true);
                        pf[4 * kb + e0 / 4] = w4;
                    }
                };
                if constexpr (PREV) {
                    pv(lds + ((t - 1) % kSlots) * kPageBytes, pf_prev, 127 + (half ? gp1 : gp0),
                       softmax);
                } else {
                    static_for<0, 16>([&](auto nn) { softmax(nn); });
                }
                l_run += __builtin_amdgcn_ldexpf(ps0, g0) + __builtin_amdgcn_ldexpf(ps1, g1);
                if (__any(moved != 0)) {
                    // page t-1's tiles follow the reference.  An MFMA that has just written
                    // a tile, then an MFMA reading a tile written through v_accvgpr_write:
                    // wait states the compiler does not count for the asm of scale_acc
                    const float f = __builtin_amdgcn_ldexpf(1.f, -moved);
                    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
                    for (int n = 0; n < 16; ++n) scale_acc(acc[n], f);
                    asm volatile("s_nop 7" ::: "memory");
                }
                pf_prev = pf;
                gp0 = g0;
                gp1 = g1;
            }
            // the block-table entry of the page after the next refill, loaded after the last
            // LDS read of the page (a scalar load in flight makes every LDS wait a full one)
            pid_next = page_id(t + 3);
        };
        page(0, std::false_type{});
        for (int t = 1; t < size; ++t) page(t, std::true_type{});
        {
            // page size-1's P V MFMAs, with its E4M3 sum
            float qs0 = 0.f, qs1 = 0.f;
            pv(lds + ((size - 1) % kSlots) * kPageBytes, pf_prev, 127 + (half ? gp1 : gp0),
               [&](auto nn) {
                   constexpr int n = decltype(nn)::value;
                   if constexpr (n < 8) {
                       const v2f x0 = __builtin_amdgcn_cvt_pk_f32_fp8(pf_prev[n], false);
                       const v2f x1 = __builtin_amdgcn_cvt_pk_f32_fp8(pf_prev[n], true);
                       const float d4 = (x0[0] + x0[1]) + (x1[0] + x1[1]);
                       if constexpr (n < 4) qs0 += d4; else qs1 += d4;
                   }
               });
            lq_run += __builtin_amdgcn_ldexpf(qs0, gp0) + __builtin_amdgcn_ldexpf(qs1, gp1);
        }

        if (page_bad && tid == 0) atomicOr(&header[kHdrStatus], AMLA_DEV_BAD_PAGE);

        // epilogue: the lane pair's sums; LSE from the FP32 sum, O normalised by the E4M3
        // sum (both carry P's 2^kPExp, which cancels in O / lq)
        const size_t slot_idx = (size_t)off_r + s;
        const float l = half_pair_sum(l_run), lq = half_pair_sum(lq_run);
        // (the last P V MFMAs wrote the tiles read below through asm)
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
        if (row < M) {
            if (half == 0) lse_out[slot_idx * M + row] = m_ref + __builtin_amdgcn_logf(l) - kPExp;
            const float inv = lq > 0.f ? a.out_scale / lq : 0.f;   // no key: O = 0
            float *po = partial + (slot_idx * M + row) * kVDim;
#pragma unroll
            for (int n = 0; n < 16; ++n) {
                const int dim = 32 * n + 4 * half;
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const v16f t16 = acc_read(acc[n]);
                    const v4f o = v4f{t16[4 * q4], t16[4 * q4 + 1], t16[4 * q4 + 2],
                                      t16[4 * q4 + 3]} * inv;
                    *(v4f *)(po + dim + 8 * q4) = o;
                }
                // one tile at a time out of the AGPRs (all at once they would not fit)
                __builtin_amdgcn_sched_barrier(0);
            }
        }

        lds_barrier();  // the next unit's prologue overwrites the ring
    }
}

}  // namespace

hipError_t launch_decode128(dim3 grid, hipStream_t stream, const uint8_t *q, const uint8_t *kv,
                            const int32_t *block_table, const int32_t *lengths,
                            const int32_t *counts, const int32_t *offsets, const int32_t *work,
                            int32_t *header, float *partial, float *lse, const DecodeArgs &a)
{
    hipLaunchKernelGGL(decode128_kernel, grid, dim3(kDecodeThreads), 0, stream, q, kv, block_table,
                       lengths, counts, offsets, work, header, partial, lse, a);
    return hipGetLastError();
}

}  // namespace amla
