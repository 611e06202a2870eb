// The 128-row decode kernel (row tiles of 128 folded rows: the compute-bound shapes).
// It is its own translation unit because it is compiled with MFMA accumulators in AGPRs
// (the other kernels keep the VGPR form): see decode128_kernel.
#include "common.h"

namespace amla {
namespace {

// An empty asm that takes x and gives it back: whatever computes x stays before this point.
template <typename T>
__device__ __forceinline__ void pin_vgpr(T &x)
{
    asm volatile("" : "+v"(x));
}

// S^T of one key block of a page for one k-step: the key block's K fragment (A) times the
// row block's Q^T fragment (B), VGPR results.  The kernel's output accumulators are
// AGPR-form MFMAs; this one is written here so that the score tile stays in VGPRs.  The
// compiler does not see it as an MFMA: its readers pad the wait states.
template <bool FIRST>
__device__ __forceinline__ void score_one(v16f &s, v8i k, v8i q)
{
    if constexpr (FIRST)
        asm volatile("v_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, 0" : "=&v"(s) : "v"(k), "v"(q));
    else
        asm volatile("v_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, %0" : "+v"(s) : "v"(k), "v"(q));
}

// The row sums of the P that a P V MFMA takes, by the same MFMA with an all-ones A operand
// (E4M3 1.0 in every byte) and the same B operand and scales: every element of lane l's
// tile is the sum over the page's keys of row l % 32, as the P V MFMA weighs them.  VGPR
// results, written here for the same reason as score_one.  The compiler does not see it as
// an MFMA either, so it may write the operands with VALU instructions right before it: the
// leading s_nop gives that write the wait states an MFMA operand read needs.
__device__ __forceinline__ void psum_mfma(v16f &s, v8i ones, v8i p, int sa, int sb)
{
    asm volatile("s_nop 4\n\tv_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0]"
                 : "+v"(s)
                 : "v"(ones), "v"(p), "v"(sa), "v"(sb));
}

// The page slots (score slots 0-17, then P V slots 18-33) that issue the ring refill's nine
// DMA instructions, one each.  Score slots 9-17 measured best: slots 0-8 (next to the
// exponentials) 8 % slower; every other score slot, or the chunks spread over both phases,
// no faster.
constexpr int kRefillSlots[kChunksPerWave] = {9, 10, 11, 12, 13, 14, 15, 16, 17};
// the refill chunk issued in page slot `slot`, or -1
constexpr int refill_chunk_at(int slot)
{
    for (int c = 0; c < kChunksPerWave; ++c)
        if (kRefillSlots[c] == slot) return c;
    return -1;
}

// 128-row tiles, four waves, each owning 32 rows of the tile end to end: wave w computes
// S^T (the page's 64 keys, two key blocks of 32, x its rows [32w, +32)), the softmax of its
// rows, and O^T (the 512 value dims, sixteen 32-dim tiles in AGPRs, x its rows).  The lane
// that holds a row's scores (column l % 32 of S^T) is the lane that supplies that row's
// column of the P^T operand, so P goes from the exponentials to the P V MFMA in registers:
// the waves exchange nothing, and meet only once per page, where the page ring advances.
//
// Each wave software-pipelines its pages: while the MFMAs of page t+1's scores run, the
// VALU computes page t's softmax (mask, row max, reference, exponentials, E4M3 P); page
// t's P V MFMAs are followed by one more that sums that P per row (psum_mfma), so that O
// is normalised by exactly the P it was built from.  The LDS ring holds
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
    // the unit's block-table entries, 64 pages per half, one copy per wave (each wave reads
    // the entries it DMA'd itself: a scalar load of an entry in flight would turn every LDS
    // wait of the page into a full wait)
    __shared__ int32_t bt_lds[4][2][64];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, half = lane >> 5;
    const int R = a.reqs, M = a.rows;
    const int mt = ceil_div(M, MT);
    const int W = a.workers;

    // The plan summary, the item count and the group's item range do not depend on each
    // other, so they are loaded together and their latencies overlap (the range is inside
    // the list, which holds at least 2 (R + 2 W) entries).
    const int vw = virtual_worker(blockIdx.x, W, mt);
    const WorkerGroup wg = worker_group(vw, W, mt, R);
    const int h_planned = ldc(&header[kHdrPlanned]), h_rows = ldc(&header[kHdrRows]);
    const int h_mtile = ldc(&header[kHdrMtile]), h_workers = ldc(&header[kHdrWorkers]);
    const int h_reqs = ldc(&header[kHdrReqs]);
    const int n_items = ldc(&offsets[R]);
    const int g_begin = ldc(&work[wg.list_at]), g_end = ldc(&work[wg.list_at + 1]);
    // consume every value here so that the compiler cannot sink a load past the checks
    // below (it would otherwise chain them one behind the other)
    asm volatile("" ::"s"(h_planned), "s"(h_rows), "s"(h_mtile), "s"(h_workers), "s"(h_reqs),
                 "s"(n_items), "s"(g_begin), "s"(g_end), "s"(q_in), "s"(kv_in), "s"(block_table),
                 "s"(lengths), "s"(counts));
    if (h_planned != kPlannedMagic || h_rows != M || h_mtile != MT || h_workers != W ||
        h_reqs != R || n_items < 0 || n_items > R + W || 2 * (R + W) + wg.groups >= a.list_len ||
        g_begin < 0 || g_begin > g_end || g_end > n_items) {
        if (tid == 0) atomicOr(&header[kHdrStatus], AMLA_DEV_BAD_ITEM);
        return;
    }
    if (!wg.active) return;
    const int units = g_end * mt;   // the group's units, item-major; this worker's: every
                                    // wg.step-th from its own tile

    const DmaOffsets dmao = dma_offsets(wave, lane);
    // the pool bound as a 32-bit scalar (page ids are 32-bit)
    const int pool32 = a.pool_pages < 0x7FFFFFFF ? (int)a.pool_pages : 0x7FFFFFFF;
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

    for (int u = g_begin * mt + wg.first_tile; u < units; u += wg.step) {
        const int item = u / mt, jt = u - item * mt;
        // the work pair, the next one (where the item ends), the request's count, length and
        // item offset, loaded together (index clamped so that the loads stay in bounds
        // before r is checked)
        const int r = ldc(&work[2 * item]), first = ldc(&work[2 * item + 1]);
        const int r_next = ldc(&work[2 * item + 2]), f_next = ldc(&work[2 * item + 3]);
        const int rc = r >= 0 && r < R ? r : 0;
        const int c = ldc(&counts[rc]), L = ldc(&lengths[rc]), off_r = ldc(&offsets[rc]);
        const int total = a.causal ? ldc(&a.totals[rc]) : L;
        asm volatile("" ::"s"(r), "s"(first), "s"(r_next), "s"(f_next), "s"(c), "s"(L),
                     "s"(off_r), "s"(total));
        const int pages = ceil_div(L, kPage);
        const int end = item + 1 < n_items && r_next == r ? f_next : pages;
        const int size = end - first;
        if (r != rc || L <= 0 || pages > a.bt_stride || first < 0 || size <= 0 || end > pages ||
            item < off_r || item >= off_r + c) {
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
            if (pid < 0 || pid >= pool32) {
                page_bad = true;
                pid = 0;
            }
            const int valid = L - (first + t) * kPage;
            issue_rows<true>(kv_in + (int64_t)pid * kPageBytes, lds_base + (t % kSlots) * kPageBytes,
                       valid < kPage ? valid : kPage, dmao, wave, lane);
        };
        // block-table entry of page min(t, size - 1)
        auto page_id = [&](int t) { return ldc(&bt[t < size ? t : size - 1]); };
        // the entries of pages [64b, +64) (clamped to the unit) into bt_lds[wave][b & 1]:
        // one DMA instruction, lane l's entry to bt_lds[wave][b & 1][l]
        const uint32_t bt_lds_base = (uint32_t)(uintptr_t)(LDS_AS int32_t *)&bt_lds[wave][0][0];
        auto issue_bt = [&](int b) {
            const int e = 64 * b + lane;
            const uint32_t off = 4u * (uint32_t)(e < size ? e : size - 1);
            const uint8_t *base = uniform_ptr((const uint8_t *)bt);
            const uint32_t m = __builtin_amdgcn_readfirstlane(bt_lds_base + 256u * (uint32_t)(b & 1));
            asm volatile("s_mov_b32 m0, %[m]\n\ts_nop 0\n\tglobal_load_lds_dword %[o], %[b]"
                         :
                         : [o] "v"(off), [b] "s"(base), [m] "s"(m)
                         : "memory");
        };

        // The first two pages' block-table entries, loaded together, and the entry of the
        // next page to fetch; the first pages' DMA, then the Q^T fragments of the wave's rows
        // from global memory, so that both latencies overlap; then wait for all of it (the
        // compiler tracks the Q loads, not the DMA).
        const int32_t pid_a = page_id(0), pid_b = page_id(1);
        asm volatile("" ::"s"(pid_a), "s"(pid_b));
        int32_t pid_next = page_id(2);
        issue_bt(0);
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

        // the row's reference and the FP32 sum of P relative to it, for the LSE (per lane
        // the keys of its half, added over the lane pair at the end)
        float m_ref = -INFINITY, l_run = 0.f;
        // the sums of the E4M3 P by the P V MFMAs' weights, in every element (psum_mfma):
        // O is normalised by the sum of the P it was built from
        v16f lq_acc = v16f{0};
        v8i ones;
#pragma unroll
        for (int w = 0; w < 8; ++w) ones[w] = 0x38383838;
        pin_vgpr(ones);   // kept in registers, not rebuilt for every page
        int scale_one = 127;
        v16f acc[16];   // O^T of dim tile n (dims [32n, +32)) x the wave's rows
#pragma unroll
        for (int n = 0; n < 16; ++n) acc[n] = v16f{0};

        // An MFMA may still read its A and B registers after it is issued, and the data of an
        // LDS load is written to its registers when it returns, with no interlock between the
        // two.  So no load may target the operand registers of the MFMA issued last: each
        // MFMA's operands are kept live (an empty asm using them) until the next MFMA is
        // issued, and fragments are read into registers freed that way.
        //
        // A wave issues in order, and an MFMA waits at issue until the one before it is done,
        // so VALU work overlaps an MFMA only when it stands between two MFMAs.  A page is
        // therefore 34 slots of one MFMA followed by at most about one MFMA's worth of VALU
        // work: 18 score slots (page t's S^T, key block 0 then key block 1, k-steps 0-8)
        // carrying page t-1's key-block-1 exponentials and the ring refill, then
        // 16 P V slots (page t-1's O^T update, dim tiles 0-15) carrying page t's mask, row max,
        // reference and key-block-0 exponentials, and one MFMA for page t-1's row sums.

        v16f sc[2];   // S^T of the page in flight: key blocks 0, 1
        // K fragment of score slot i (key block i / 9, k-step i % 9) of the page in `slot`
        auto kfrag = [&](const uint8_t *slot, int i) {
            const uint8_t *kp = slot + (i / 9) * kBlock1 + 64 * (i % 9);
            return lds_read2x16(kp + k_off0, kp + k_off1);
        };
        // V^T fragment of dim tile n (dims [32n, +32)) of the page in `slot`
        auto vtile = [&](const uint8_t *slot, int n) {
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

        // Score slots of the page in `slot` (SCORE) with `work(i)` after slot i's MFMA.  The
        // K fragments go round a ring of three, read two slots ahead into the registers of
        // slot i-1 once slot i's MFMA is issued.
        v8i kf[3];
        auto score_slots = [&](auto score, const uint8_t *slot, auto &&work) {
            constexpr bool SCORE = decltype(score)::value;
            if constexpr (SCORE) {
                kf[0] = kfrag(slot, 0);
                kf[1] = kfrag(slot, 1);
            }
            static_for<0, 18>([&](auto ii) {
                constexpr int i = decltype(ii)::value;
                if constexpr (SCORE) {
                    score_one<i % 9 == 0>(sc[i / 9], kf[i % 3], qf[i % 9]);
                    __builtin_amdgcn_sched_barrier(0);
                    if constexpr (i >= 1) asm volatile("" ::"v"(kf[(i - 1) % 3]));
                    if constexpr (i + 2 < 18) kf[(i + 2) % 3] = kfrag(slot, i + 2);
                }
                work(ii);
                __builtin_amdgcn_sched_barrier(0);
            });
        };
        // P V slots of the page in `slot` (PV; fragment pfv, E8M0 scales sbv) with `work(n)`
        // after dim tile n's MFMA.  The V^T fragments go round a ring of three (tile n in
        // vr[n % 3]; the caller reads tiles 0 and 1), two tiles ahead into the registers of
        // tile n-1 once tile n's MFMA is issued.  The last MFMA's operands are kept live for
        // 64 cycles after it.
        v8i vr[3];
        auto pv_slots = [&](auto pvb, const uint8_t *slot, const v8i &pfv, int sbv, auto &&work) {
            constexpr bool PV = decltype(pvb)::value;
            static_for<0, 16>([&](auto nn) {
                constexpr int n = decltype(nn)::value;
                if constexpr (PV) {
                    // operands in VGPRs (the allocator would otherwise load some into AGPRs,
                    // which the sixteen accumulator tiles fill)
                    asm volatile("" : "+v"(vr[n % 3]));
                    acc[n] = mfma_scaled_b(vr[n % 3], pfv, acc[n], sbv);
                    __builtin_amdgcn_sched_barrier(0);
                    if constexpr (n >= 1) asm volatile("" ::"v"(vr[(n - 1) % 3]));
                    if constexpr (n + 2 < 16) vr[(n + 2) % 3] = vtile(slot, n + 2);
                }
                work(nn);
                __builtin_amdgcn_sched_barrier(0);
            });
            if constexpr (PV) {
                // the row sums of this P (after the last tile, whose operands it shares)
                psum_mfma(lq_acc, ones, pfv, scale_one, sbv);
                asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\t"
                             "s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::"v"(vr[15 % 3]), "v"(pfv),
                             "v"(ones), "v"(scale_one), "v"(sbv));
            }
        };

        // Softmax state.  Page t's key block kb has whole-number gap g_kb and bias b_kb (P =
        // 2^(s*scale + b_kb)); the previous page's (gp, bp1) are kept for its key-block-1
        // exponentials, its sums and its P V MFMAs.  pf: the P^T fragment being built (bytes
        // [16kb, +16) are key block kb; key block 0 is written with the page's softmax, key
        // block 1 one page later); pfa: the previous page's, complete once its key-block-1
        // exponentials are done.
        v8i pf, pfa;
        int g0 = 0, g1 = 0, gp0 = 0, gp1 = 0;
        // A slot's results are first read after the rare reference-move branch, and the
        // compiler would sink the work that makes them below that branch, out of the MFMA
        // slots; an empty asm that redefines them keeps the work in its slot.
        auto here = [](auto &...x) { (pin_vgpr(x), ...); };
        float b0 = 0.f, b1 = 0.f, bp1 = 0.f;

        // Score-slot work for the previous page (PREV): its key-block-1 exponentials (two per
        // slot, slots 0-7), their FP32 sum into l (slot 8); the ring refill (one DMA
        // instruction per slot, by kRefillSlots) and the first V^T fragments of the previous
        // page (slots 16, 17).
        float ps1 = 0.f;
        float pt[4];
        bool bt_next = false;
        int bt_block = 0;
        auto prev_work = [&](auto ii, auto dma, const uint8_t *src, uint32_t dst, const uint32_t *co,
                             const uint8_t *slot_p, auto prev) {
            constexpr int i = decltype(ii)::value;
            constexpr bool PREV = decltype(prev)::value;
            if constexpr (PREV && i < 8) {
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[1][2 * i + e], a.score_scale, bp1));
                    pt[2 * (i & 1) + e] = p;
                    ps1 += p;
                }
                here(ps1);
                if constexpr (i & 1) {
                    // (both halves are written: the old dword only saves a zeroing move)
                    int w4 = __builtin_amdgcn_cvt_pk_fp8_f32(pt[0], pt[1], pfa[4 + (i >> 1)], false);
                    w4 = __builtin_amdgcn_cvt_pk_fp8_f32(pt[2], pt[3], w4, true);
                    pfa[4 + (i >> 1)] = w4;
                    here(pfa);
                }
            }
            if constexpr (PREV && i == 8) {
                l_run += __builtin_amdgcn_ldexpf(ps1, gp1);
                here(l_run);
            }
            if constexpr (i == 0) {
                // the next 64 block-table entries, well before they are read (and before
                // this page's refill, so that the barrier's vmcnt wait still counts the
                // refill as the newest nine)
                if (bt_next) issue_bt(bt_block);
            }
            if constexpr (decltype(dma)::value && refill_chunk_at(i) >= 0)
                issue_chunk(src, dst + 1024 * refill_chunk_at(i), co[refill_chunk_at(i)]);
            if constexpr (PREV && i >= 16) vr[i - 16] = vtile(slot_p, i - 16);
        };

        // P-V-slot work for page t (SOFTMAX): mask and key-block-0 max (slot 0), key-block-1
        // max (1), gaps and the reference move (2), biases (3), key-block-0 exponentials (two
        // per slot, 4-11), their FP32 sum into l (12).
        float mx0 = -INFINITY, mx1 = -INFINITY, ps0 = 0.f;
        int32_t bt_v = 0;
        int moved = 0;   // log2 step of the reference on this page
        auto cur_work = [&](auto nn, int t, int valid, auto softmax, auto dma, const uint8_t *src,
                            uint32_t dst, const uint32_t *co) {
            constexpr int n = decltype(nn)::value;
            if constexpr (decltype(dma)::value && refill_chunk_at(18 + n) >= 0)
                issue_chunk(src, dst + 1024 * refill_chunk_at(18 + n), co[refill_chunk_at(18 + n)]);
            if constexpr (decltype(softmax)::value) {
                if constexpr (n == 0) {
                    // the score MFMAs' results, read by VALU code: wait states the compiler
                    // does not count for their asm
                    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
                    if (__any(valid < kPage)) {
#pragma unroll
                        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                            for (int e = 0; e < 16; ++e)
                                if (32 * kb + 8 * (e >> 2) + (e & 3) >= valid) sc[kb][e] = -INFINITY;
                    }
                    mx0 = -INFINITY;
#pragma unroll
                    for (int e = 0; e < 16; ++e) mx0 = fmaxf(mx0, sc[0][e]);
                } else if constexpr (n == 1) {
                    mx1 = -INFINITY;
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
                } else if constexpr (n == 3) {
                    const float f = __builtin_amdgcn_ldexpf(1.f, -moved);
                    m_ref += (float)moved;
                    g0 = g0 - moved < -127 ? -127 : g0 - moved;
                    g1 = g1 - moved < -127 ? -127 : g1 - moved;
                    l_run *= f;
                    const bool none = m_ref == -INFINITY;
                    b0 = none ? 0.f : (kPExp - (float)g0) - m_ref;
                    b1 = none ? 0.f : (kPExp - (float)g1) - m_ref;
                    ps0 = 0.f;
                    here(l_run, b0, b1);
                } else if constexpr (n >= 4 && n <= 11) {
                    constexpr int i = n - 4;
#pragma unroll
                    for (int e = 0; e < 2; ++e) {
                        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[0][2 * i + e], a.score_scale, b0));
                        pt[2 * (i & 1) + e] = p;
                        ps0 += p;
                    }
                    here(ps0);
                    if constexpr (i & 1) {
                        int w4 = __builtin_amdgcn_cvt_pk_fp8_f32(pt[0], pt[1], pf[i >> 1], false);
                        w4 = __builtin_amdgcn_cvt_pk_fp8_f32(pt[2], pt[3], w4, true);
                        pf[i >> 1] = w4;
                        here(pf);
                    }
                } else if constexpr (n == 12) {
                    l_run += __builtin_amdgcn_ldexpf(ps0, g0);
                    here(l_run);
                }
            }
            if constexpr (n == 13) {
                // the block-table entry of the page after the next refill
                const int tt = t + 3 < size ? t + 3 : size - 1;
                bt_v = bt_lds[wave][(tt >> 6) & 1][tt & 63];
            }
        };

        // Page t: wait for it and refill the ring, its score slots, the previous page's P V
        // slots, then (rarely) the tiles follow a reference move, and the page's state becomes
        // the previous page's.
        auto page = [&](int t, auto prev) {
            // page t has landed (the newest nine DMAs, page t+1's or a spare copy, may not)
            if (t > 0) wait_pages_then_barrier(1);
            const uint8_t *slot_t = lds + (t % kSlots) * kPageBytes;
            const uint8_t *slot_p = lds + ((t + kSlots - 1) % kSlots) * kPageBytes;
            // the ring refill: page t+2, into the slot that page t-2 used; past the unit's end
            // a spare copy of its last page (the entry pid_next then holds) goes into that
            // free slot, so that every page issues the same nine DMA instructions with no
            // branch between the MFMA slots
            const bool refill = t + 2 < size;
            int32_t pid = pid_next;
            if (pid < 0 || pid >= pool32) {
                if (refill) page_bad = true;
                pid = 0;
            }
            const uint8_t *src = kv_in + (int64_t)pid * kPageBytes;
            const uint32_t dst = lds_base + ((t + 2) % kSlots) * kPageBytes;
            const int rvalid = refill ? L - (first + t + 2) * kPage : kPage;
            // the lane's source offsets of the refill's nine chunks, chosen once per page
            uint32_t co[kChunksPerWave];
            if (rvalid >= kPage) {
#pragma unroll
                for (int i = 0; i < kChunksPerWave; ++i) co[i] = chunk_offset(dmao, i, kPage, wave, lane);
            } else {
#pragma unroll
                for (int i = 0; i < kChunksPerWave; ++i) co[i] = chunk_offset(dmao, i, rvalid, wave, lane);
            }
            bt_block = (t >> 6) + 1;
            bt_next = (t & 63) == 8 && 64 * bt_block < size;
            ps1 = 0.f;
            score_slots(std::true_type{}, slot_t, [&](auto ii) {
                prev_work(ii, std::true_type{}, src, dst, co, slot_p, prev);
            });
            // keys of the page the lane's row sees, counted from the lane's first key
            // (4*half): element e of key block kb holds key 32kb + 8(e/4) + e%4 past it
            const int valid = lim - (first + t) * kPage - 4 * half;
            pv_slots(prev, slot_p, pfa, 127 + (half ? gp1 : gp0), [&](auto nn) {
                cur_work(nn, t, valid, std::true_type{}, std::true_type{}, src, dst, co);
            });
            if (__any(moved != 0)) {
                // the previous page's tiles follow the reference.  An MFMA that has just
                // written a tile, then an MFMA reading a tile written through
                // v_accvgpr_write: wait states the compiler does not count for scale_acc
                const float f = __builtin_amdgcn_ldexpf(1.f, -moved);
                asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
                for (int n = 0; n < 16; ++n) scale_acc(acc[n], f);
                lq_acc *= f;
                asm volatile("s_nop 7" ::: "memory");
            }
#pragma unroll
            for (int w = 0; w < 4; ++w) pfa[w] = pf[w];
            gp0 = g0;
            gp1 = g1;
            bp1 = b1;
            pid_next = __builtin_amdgcn_readfirstlane(bt_v);
        };
        page(0, std::false_type{});
        for (int t = 1; t < size; ++t) page(t, std::true_type{});
        {
            // the last page's key-block-1 exponentials, then its P V MFMAs; the
            // spare copy issued by the last page lands first (the next unit's DMA reuses the
            // ring)
            __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 15));
            const uint8_t *slot_l = lds + ((size - 1) % kSlots) * kPageBytes;
            ps1 = 0.f;
            score_slots(std::false_type{}, slot_l, [&](auto ii) {
                prev_work(ii, std::false_type{}, slot_l, 0u, nullptr, slot_l, std::true_type{});
            });
            pv_slots(std::true_type{}, slot_l, pfa, 127 + (half ? gp1 : gp0), [&](auto nn) {
                cur_work(nn, 0, 0, std::false_type{}, std::false_type{}, slot_l, 0u, nullptr);
            });
        }

        if (page_bad && tid == 0) atomicOr(&header[kHdrStatus], AMLA_DEV_BAD_PAGE);

        // epilogue: LSE from the FP32 sum (the lane pair's), O normalised by the E4M3 sum
        // (both carry P's 2^kPExp, which cancels in O / lq)
        const size_t slot_idx = (size_t)item;
        const float l = half_pair_sum(l_run);
        // (the last P V MFMAs and psum_mfma wrote the tiles read below through asm)
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
        const float lq = lq_acc[0];
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
