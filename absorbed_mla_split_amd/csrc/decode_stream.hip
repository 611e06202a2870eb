// The 32- and 64-row decode kernels (row tiles of up to 64 folded rows: the shapes whose
// time is the KV stream from HBM).
//
// A workgroup's work units form one stream of ring entries: each unit contributes its query
// rows (one entry: the tile's rows laid out like a page) and then its pages.  The four LDS
// ring slots are refilled in stream order across unit boundaries, so the next unit's query
// rows and first pages arrive while the current unit finishes and a unit costs no
// pipeline drain.
//
// Eight waves, two per SIMD, in two roles one entry apart, so that each SIMD overlaps one
// role's MFMAs with the other role's softmax, LDS traffic and waits:
//   score waves (0-3)  wave (rb, kb) computes S^T for key block kb (keys [32kb, +32) of the
//                      page) and the 32 rows of row block rb, the key block's softmax and
//                      its half of the E4M3 P^T fragment, published in LDS (double
//                      buffered).  MT = 32 has one row block: waves 2, 3 repeat waves 0, 1,
//                      which alone publish.
//   value waves (4-7)  one entry behind, O^T += V^T P^T for one row block and NT 32-dim
//                      tiles (MT = 64: 256 dims, MT = 32: 128 dims), and the unit's FP32
//                      partial and log2 LSE; they also issue the ring's DMA (a wave stalls
//                      on DMA issue, and the value waves have the slack).
// One barrier per entry (plus one at a unit's first page, where the two key blocks agree on
// the row reference).
//
// Softmax in log2 units against a per-row reference (page "...cutedsl.mla.balanced", module
// docstring: the row max is kept lazily and P is fed to the MMA in E4M3): m_ref is the row's
// max over the unit's first page and key block kb's P is 2^(s - m_ref - gap_kb + kPExp)
// <= 2^8, gap_kb the smallest whole number keeping that block's running max at or below
// m_ref + gap_kb.  The P V MFMA scales each K block of its B operand by its own E8M0 byte, so
// key block kb's P is scaled by 2^gap_kb and O and the row sums stay relative to m_ref with
// no rescaling and no per-page agreement between the two key blocks.
#include "common.h"

namespace amla {
namespace {

// One work unit as the stream sees it.
struct Unit {
    int r, L, total, slot, first, size, jt;
    bool ok;
};

template <int MT>
__global__ __launch_bounds__(2 * kDecodeThreads, 1) void decode_stream_kernel(
    const uint8_t *__restrict__ q_in, const uint8_t *__restrict__ kv_in,
    const int32_t *__restrict__ block_table, const int32_t *__restrict__ lengths,
    const int32_t *__restrict__ counts, const int32_t *__restrict__ offsets,
    const int32_t *__restrict__ work, int32_t *__restrict__ header, float *__restrict__ partial,
    float *__restrict__ lse_out, DecodeArgs a)
{
    static_assert(MT == 32 || MT == 64, "32- or 64-row tiles");
    constexpr int NT = MT == 32 ? 4 : 8;   // 32-dim output tiles per value wave
    __shared__ __attribute__((aligned(1024))) uint8_t lds[kSlots * kPageBytes];
    // P^T fragments of an entry by (buffer, row block, lane): dwords [4kb, +4) come from the
    // score wave of key block kb (the MFMA takes bytes [16kb, +16) of both lanes of a column
    // as its K block kb, each K block with its own E8M0 scale)
    __shared__ __attribute__((aligned(16))) int32_t xch_p[2][2][64][8];
    // the whole-number gap of each key block's P reference, by (buffer, row block, key
    // block, row)
    __shared__ int32_t xch_gap[2][2][2][32];
    // key-block maxima at a unit's first page; at its last page the row sums of each key
    // block and the row reference
    __shared__ float xch_max[2][2][32];
    __shared__ float xch_l[2][2][32];
    __shared__ float xch_lq[2][2][32];
    __shared__ float xch_mref[2][32];
    // per (row block, key block, row): the unit's last page's FP32 and E4M3 P sums (relative
    // to the reference plus that page's gap), added in by the value waves
    __shared__ float xch_ps[2][2][32];
    __shared__ float xch_qs[2][2][32];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, half = lane >> 5;
    const int R = a.reqs, M = a.rows;
    const int mt = ceil_div(M, MT);
    const int W = a.workers;

    const int vw = virtual_worker(blockIdx.x, W, mt);
    const int h_planned = ldc(&header[kHdrPlanned]), h_rows = ldc(&header[kHdrRows]);
    const int h_mtile = ldc(&header[kHdrMtile]), h_workers = ldc(&header[kHdrWorkers]);
    const int h_reqs = ldc(&header[kHdrReqs]);
    const int n_items = ldc(&offsets[R]);
    // this worker's group and the group's item range (inside the list, which holds at least
    // 2 (R + 2 W) entries)
    const WorkerGroup wg = worker_group(vw, W, mt, R);
    const int g_begin = ldc(&work[wg.list_at]), g_end = ldc(&work[wg.list_at + 1]);
    asm volatile("" ::"s"(h_planned), "s"(h_rows), "s"(h_mtile), "s"(h_workers), "s"(h_reqs),
                 "s"(n_items), "s"(g_begin), "s"(g_end));
    if (h_planned != kPlannedMagic || h_rows != M || h_mtile != MT || h_workers != W ||
        h_reqs != R || n_items < 0 || n_items > R + W || 2 * (R + W) + wg.groups >= a.list_len ||
        g_begin < 0 || g_begin > g_end || g_end > n_items) {
        if (tid == 0) atomicOr(&header[kHdrStatus], AMLA_DEV_BAD_ITEM);
        return;
    }
    if (!wg.active) return;
    // the group's units, item-major: this worker takes every wg.step-th from its own tile
    const int units = g_end * mt, ustep = wg.step;

    // The descriptor of unit u: its work pair and the next one (where the item ends), then
    // the request's count, length, item offset (and global length under DCP); index clamped
    // so the loads stay in bounds.
    auto load_unit = [&](int u) {
        Unit d;
        const int uu = u < units ? u : 0;
        const int item = uu / mt;
        d.jt = uu - item * mt;
        d.r = ldc(&work[2 * item]);
        d.first = ldc(&work[2 * item + 1]);
        const int r_next = ldc(&work[2 * item + 2]), f_next = ldc(&work[2 * item + 3]);
        const int rc = d.r >= 0 && d.r < R ? d.r : 0;
        const int c = ldc(&counts[rc]);
        d.L = ldc(&lengths[rc]);
        const int off = ldc(&offsets[rc]);
        d.total = a.causal ? ldc(&a.totals[rc]) : d.L;
        const int pages = ceil_div(d.L, kPage);
        const int end = item + 1 < n_items && r_next == d.r ? f_next : pages;
        d.size = end - d.first;
        d.slot = item;
        d.ok = d.r == rc && d.L > 0 && pages <= a.bt_stride && d.first >= 0 && d.size > 0 &&
               end <= pages && item >= off && item < off + c;
        return d;
    };
    // A cursor over the workgroup's entries: the unit (skipping bad work items, which have
    // no entries) and the entry within it (0: query rows, 1 + t: page t).
    struct Cursor {
        int u, e;
        Unit d, next;
    };
    auto cursor_skip = [&](Cursor &c, bool flag) {
        while (c.u < units && !c.d.ok) {
            if (flag && tid == 0) atomicOr(&header[kHdrStatus], AMLA_DEV_BAD_ITEM);
            c.u += ustep;
            c.d = c.next;
            c.next = load_unit(c.u + ustep);
        }
    };
    auto cursor_init = [&](Cursor &c, bool flag) {
        c.u = g_begin * mt + wg.first_tile;
        c.e = 0;
        c.d = load_unit(c.u);
        c.next = load_unit(c.u + ustep);
        cursor_skip(c, flag);
    };
    auto cursor_advance = [&](Cursor &c, bool flag) {
        if (++c.e > c.d.size) {
            c.u += ustep;
            c.d = c.next;
            c.next = load_unit(c.u + ustep);
            c.e = 0;
            cursor_skip(c, flag);
        }
    };

    if (wave < 4) {
        // ================================================================ score waves
        const int srb = MT == 64 ? (wave & 1) : 0;
        const int skb = MT == 64 ? (wave >> 1) : (wave & 1);
        const bool writer = MT == 64 || wave < 2;

        // K and Q fragment reads: key 32 skb + l32 / row 32 srb + l32, chunks 4k + 2*half + e
        // (rows 32 apart share the swizzle)
        int k_off[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) k_off[e] = l32 * kKDim + 16 * ((2 * half + e) ^ swz(l32));
        v8i qf[9];
        // the row's reference (log2 units, the same for both key blocks), this key block's
        // P-reference gap above it, FP32 and E4M3 P sums of the key block relative to m_ref
        float m_ref = -INFINITY, l_run = 0.f, lq_run = 0.f;
        int gap = 0, lim = 0;
        // the latest page's sums and gap: added to l_run / lq_run at the next page, once the
        // move of the reference that page may cause is known (ldexp by a gap above kRefGap
        // could overflow)
        float pend_ps = 0.f, pend_qs = 0.f;
        int pend_gap = 0;

        Cursor cs;
        cursor_init(cs, true);
        for (int step = 0;; ++step) {
            const bool have = cs.u < units;
            // the value waves wait for this step's entry; this wave's LDS traffic is done
            __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
            asm volatile("s_barrier" ::: "memory");
            if (!have) break;
            const uint8_t *slot = lds + (step % kSlots) * kPageBytes;
            const Unit &u = cs.d;
            if (cs.e == 0) {
                // the unit's query rows: Q^T fragments of row block srb (lane (l32, half):
                // row 32 srb + l32, dims [64k + 32 half, +32))
                const uint8_t *qs = slot + 32 * srb * kKDim;
#pragma unroll
                for (int k = 0; k < 9; ++k)
                    qf[k] = lds_read2x16(qs + k_off[0] + 64 * k, qs + k_off[1] + 64 * k);
                m_ref = -INFINITY;
                l_run = lq_run = 0.f;
                gap = 0;
                lim = row_key_limit(a, u.total, u.L, u.jt * MT + 32 * srb + l32);
                if (a.causal && tid == 0 && shard_count(a, u.total) != u.L)
                    atomicOr(&header[kHdrStatus], AMLA_DEV_BAD_LENGTH);
            } else {
                const int t = cs.e - 1;
                const int buf = step & 1;
                // a reference more than 2^kRefGap below a key block's running max (practically
                // never): both key blocks and the value waves move it up by the larger gap of
                // the previous page, whose sums are added here relative to the moved reference
                if (t > 0) {
                    const int g0 = xch_gap[buf ^ 1][srb][0][l32], g1 = xch_gap[buf ^ 1][srb][1][l32];
                    const int gmax = g0 > g1 ? g0 : g1;
                    const int d = gmax > kRefGap ? gmax : 0;
                    l_run = __builtin_amdgcn_ldexpf(l_run, -d) +
                            __builtin_amdgcn_ldexpf(pend_ps, pend_gap - d);
                    lq_run = __builtin_amdgcn_ldexpf(lq_run, -d) +
                             __builtin_amdgcn_ldexpf(pend_qs, pend_gap - d);
                    m_ref += (float)d;
                    gap -= d;
                }
                // S^T[32 keys of block skb x 32 rows] = K Q^T: 9 MFMAs.  An MFMA may still read
                // its operands after it is issued and a returning LDS load is not held back,
                // so the K fragments go round a ring of three, read two ahead into the
                // registers of the k-step before once k-step k's MFMA is issued (kept live
                // until then).
                v16f sc = v16f{0};
                {
                    const uint8_t *kp0 = slot + 32 * skb * kKDim + k_off[0];
                    const uint8_t *kp1 = slot + 32 * skb * kKDim + k_off[1];
                    v8i kf[3];
                    kf[0] = lds_read2x16(kp0, kp1);
                    kf[1] = lds_read2x16(kp0 + 64, kp1 + 64);
                    __builtin_amdgcn_sched_barrier(0);
                    static_for<0, 9>([&](auto kk) {
                        constexpr int k = decltype(kk)::value;
                        sc = mfma(kf[k % 3], qf[k], sc);
                        __builtin_amdgcn_sched_barrier(0);
                        if constexpr (k >= 1) asm volatile("" ::"v"(kf[(k - 1) % 3]));
                        if constexpr (k + 2 < 9)
                            kf[(k + 2) % 3] = lds_read2x16(kp0 + 64 * (k + 2), kp1 + 64 * (k + 2));
                        __builtin_amdgcn_sched_barrier(0);
                    });
                }
                // keys of the page the row sees, counted from this lane's first key
                // (32 skb + 4 half): element e holds key 8(e/4) + e%4 past it
                const int valid = lim - (u.first + t) * kPage - 32 * skb - 4 * half;
                if (__any(valid < 32)) {
#pragma unroll
                    for (int e = 0; e < 16; ++e)
                        if (8 * (e >> 2) + (e & 3) >= valid) sc[e] = -INFINITY;
                }
                float smax = -INFINITY;
#pragma unroll
                for (int e = 0; e < 16; ++e) smax = fmaxf(smax, sc[e]);
                const float mx = half_pair_max(smax) * a.score_scale;   // the key block's max
                if (t == 0) {
                    // the unit's first page: the row reference is the page max over both key
                    // blocks (-inf while the row sees no key: with visible keys a prefix of
                    // the shard, a row that sees no key of its split's first page sees none)
                    if (writer && half == 0) xch_max[srb][skb][l32] = mx;
                    lds_barrier();
                    m_ref = fmaxf(mx, xch_max[srb][skb ^ 1][l32]);
                    gap = 0;
                } else if (mx > m_ref + (float)gap) {
                    gap = (int)__builtin_ceilf(mx - m_ref);
                }
                const float bias = m_ref == -INFINITY ? 0.f : (kPExp - (float)gap) - m_ref;
                // P = 2^(s*scale - m_ref - gap + kPExp) <= 2^8: FP32 into the row sum, E4M3
                // into this lane's 16 bytes of key block skb (byte 4g + e: key 32 skb + 8g +
                // 4 half + e)
                float psum = 0.f, qsum = 0.f;
                v4i pw;
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    float p4[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        p4[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[4 * g + e], a.score_scale, bias));
                        psum += p4[e];
                    }
                    int w4 = __builtin_amdgcn_cvt_pk_fp8_f32(p4[0], p4[1], 0, false);
                    w4 = __builtin_amdgcn_cvt_pk_fp8_f32(p4[2], p4[3], w4, true);
                    pw[g] = w4;
                    const v2f q0 = __builtin_amdgcn_cvt_pk_f32_fp8(w4, false);
                    const v2f q1 = __builtin_amdgcn_cvt_pk_f32_fp8(w4, true);
                    qsum += (q0[0] + q0[1]) + (q1[0] + q1[1]);
                }
                pend_ps = psum;
                pend_qs = qsum;
                pend_gap = gap;
                if (writer) {
                    *(v4i *)&xch_p[buf][srb][lane][4 * skb] = pw;
                    if (half == 0) xch_gap[buf][srb][skb][l32] = gap;
                }
                if (cs.e == u.size) {
                    // the unit's last page: its row sums before that page and that page's
                    // sums (both lane halves: every lane takes part in the swaps) and the
                    // reference, for the value waves
                    const float l_tot = half_pair_sum(l_run), lq_tot = half_pair_sum(lq_run);
                    const float ps_tot = half_pair_sum(pend_ps), qs_tot = half_pair_sum(pend_qs);
                    if (writer && half == 0) {
                        xch_l[srb][skb][l32] = l_tot;
                        xch_lq[srb][skb][l32] = lq_tot;
                        xch_ps[srb][skb][l32] = ps_tot;
                        xch_qs[srb][skb][l32] = qs_tot;
                        if (skb == 0) xch_mref[srb][l32] = m_ref;
                    }
                }
            }
            cursor_advance(cs, true);
        }
    } else {
        // ================================================================ value waves
        const int vwv = wave - 4;
        // the value waves go first where both waves of a SIMD could issue (measured on c3:
        // decode 248-249 against 250-251 us; raising the score waves instead: 251-258)
        __builtin_amdgcn_s_setprio(1);
        const int prb = MT == 64 ? (vwv & 1) : 0;
        const int tile0 = MT == 64 ? NT * (vwv >> 1) : NT * vwv;
        const bool lse_writer = MT == 64 ? (vwv >> 1) == 0 : vwv == 0;

        // V^T fragment reads (ds_read_b64_tr_b8): within each 16-lane group, source lane i
        // supplies key row b = i/2 and dims [8*(i%2), +8) of a 16-dim column block; keys are
        // tr_key + 16*w2, dims of tile T lie in chunk 2T + (g16&1), swizzled by the key row.
        // Byte 16b + e of lane half h is then key 32b + 8(e/4) + 4h + e%4, as in P^T.
        const int g16 = lane >> 4, i16 = lane & 15;
        const int tr_key = 8 * (i16 >> 3) + 4 * half + ((i16 >> 1) & 3);
        int tr_off[2];
#pragma unroll
        for (int par = 0; par < 2; ++par)
            tr_off[par] = tr_key * kKDim + 16 * ((2 * par + (g16 & 1)) ^ swz(tr_key)) +
                          8 * (i16 & 1) + 64 * (tile0 >> 1);
        // ---- the ring's DMA, two entries ahead of the score waves' entry (the value waves
        // have the slack: their P V MFMAs are half of a step's)
        const DmaOffsets dmao = dma_offsets(vwv, lane);
        const uint32_t lds_base = (uint32_t)(uintptr_t)(LDS_AS uint8_t *)lds + vwv * (kChunksPerWave * 1024);
        bool page_bad = false;
        Cursor ci;
        cursor_init(ci, false);
        int issued = 0;
        int32_t pid_next = 0;
        auto prefetch_pid = [&]() {
            const int t = ci.e >= 1 ? ci.e - 1 : 0;   // the page of the next page entry
            if (ci.u < units)
                pid_next = ldc(&block_table[(size_t)ci.d.r * a.bt_stride + ci.d.first +
                                            (t < ci.d.size ? t : ci.d.size - 1)]);
        };
        prefetch_pid();
        // The next entry's DMA, right after the barrier that frees its slot (the sooner it is
        // issued, the more of the HBM latency it hides): prepare_next issues its scalar loads
        // (the cursor's next unit, the block-table entry after it) first, then dma_all its nine
        // DMA instructions, which stall the wave a while, so that the scalar loads are back by
        // the next LDS wait (every LDS wait is a full one while a scalar load is in flight).
        // Each is called from one place in the loop: every inlined copy of the cursor code
        // adds registers next to the output tiles.
        bool dma_on = false;
        const uint8_t *dma_base = kv_in;
        uint32_t dma_dst = 0;
        int dma_valid = kPage;
        auto prepare_next = [&]() {
            dma_on = ci.u < units;
            if (!dma_on) return;
            dma_dst = lds_base + (uint32_t)(issued % kSlots) * kPageBytes;
            if (ci.e == 0) {
                const int rows = M - ci.d.jt * MT;
                dma_base = q_in + ((size_t)ci.d.r * M + (size_t)ci.d.jt * MT) * kKDim;
                dma_valid = rows < MT ? rows : MT;
            } else {
                const int t = ci.e - 1;
                int32_t pid = pid_next;
                if (pid < 0 || pid >= a.pool_pages) {
                    page_bad = true;
                    pid = 0;
                }
                const int v = ci.d.L - (ci.d.first + t) * kPage;
                dma_base = kv_in + (int64_t)pid * kPageBytes;
                dma_valid = v < kPage ? v : kPage;
            }
            ++issued;
            cursor_advance(ci, false);
            prefetch_pid();
        };
        auto dma_all = [&]() {
            if (dma_on) issue_rows(dma_base, dma_dst, dma_valid, dmao, vwv, lane);
        };
        v16f acc[NT];
        Cursor cv;
        cursor_init(cv, false);
        prepare_next();
        dma_all();
        prepare_next();
        dma_all();
        for (int step = 0;; ++step) {
            // step s: this role's entry is the one the score waves took at step s - 1
            if (step > 0 && cv.u >= units) break;
            // the score waves' entry of this step has landed (every value wave waits for its
            // own DMA share) and every wave is done with the entry two before it, whose slot
            // is refilled after the barrier
            if (issued > step && issued - step - 1 >= 1)
                __builtin_amdgcn_s_waitcnt(waitcnt_imm(kChunksPerWave, 0));
            else
                __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
            asm volatile("s_barrier" ::: "memory");
            // the ring refill, before the step's first LDS wait
            prepare_next();
            dma_all();
            if (step == 0) continue;
            const Unit &u = cv.d;
            if (cv.e == 0) {
                // the query rows: nothing here, but the score waves now agree on the first
                // page's reference (one more barrier on both sides)
#pragma unroll
                for (int n = 0; n < NT; ++n) acc[n] = v16f{0};
                lds_barrier();
            } else {
                const int buf = (step - 1) & 1;
                const uint8_t *slot = lds + ((step - 1) % kSlots) * kPageBytes;
                // the row block's P^T fragment and the E8M0 scale of K block `half` (lane
                // half h supplies the scale of K block h of its column: 2^gap of key block h)
                const v8i pf = *(const v8i *)&xch_p[buf][prb][lane][0];
                int g_own = xch_gap[buf][prb][half][l32];
                const int gl0 = xch_gap[buf][prb][0][l32], gl1 = xch_gap[buf][prb][1][l32];
                {
                    const int gmax = gl0 > gl1 ? gl0 : gl1;
                    if (__any(gmax > kRefGap)) {
                        // the score waves move the reference up by the larger gap (see
                        // there): O follows, before this page is added
                        const int d = gmax > kRefGap ? gmax : 0;
                        const float f = __builtin_amdgcn_ldexpf(1.f, -d);
#pragma unroll
                        for (int n = 0; n < NT; ++n) acc[n] *= f;
                        g_own -= d;
                    }
                }
                const int sb = 127 + (g_own < -127 ? -127 : g_own);
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
                // (V^T fragments round a ring of three as the K fragments above; the last
                // MFMA's operands stay live for 64 cycles after it)
                v8i vr[3];
                vr[0] = vtile(0);
                vr[1] = vtile(1);
                __builtin_amdgcn_sched_barrier(0);
                static_for<0, NT>([&](auto nn) {
                    constexpr int n = decltype(nn)::value;
                    acc[n] = mfma_scaled_b(vr[n % 3], pf, acc[n], sb);
                    __builtin_amdgcn_sched_barrier(0);
                    if constexpr (n >= 1) asm volatile("" ::"v"(vr[(n - 1) % 3]));
                    if constexpr (n + 2 < NT) vr[(n + 2) % 3] = vtile(n + 2);
                    __builtin_amdgcn_sched_barrier(0);
                });
                asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\t"
                             "s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::"v"(vr[(NT - 1) % 3]), "v"(pf));
                if (cv.e == u.size) {
                    // the unit's last page: normalise and store the row block's FP32 partial
                    // (this wave's dims) and the log2 LSE; l and lq carry P's 2^kPExp, which
                    // cancels in O / lq
                    // (the sums before the last page, and the last page's relative to the
                    // reference plus its gaps; a move caused by that page applies to all)
                    // (the row index is an opaque copy here: addresses kept across the page
                    // loop would be spilled, and a reload waits for the DMA in flight)
                    int rl = l32;
                    asm volatile("" : "+v"(rl));
                    const int g0 = xch_gap[buf][prb][0][rl], g1 = xch_gap[buf][prb][1][rl];
                    const int gmax = g0 > g1 ? g0 : g1;
                    const int d = gmax > kRefGap ? gmax : 0;
                    const float l_tot =
                        __builtin_amdgcn_ldexpf(xch_l[prb][0][rl] + xch_l[prb][1][rl], -d) +
                        __builtin_amdgcn_ldexpf(xch_ps[prb][0][rl], g0 - d) +
                        __builtin_amdgcn_ldexpf(xch_ps[prb][1][rl], g1 - d);
                    const float lq_tot =
                        __builtin_amdgcn_ldexpf(xch_lq[prb][0][rl] + xch_lq[prb][1][rl], -d) +
                        __builtin_amdgcn_ldexpf(xch_qs[prb][0][rl], g0 - d) +
                        __builtin_amdgcn_ldexpf(xch_qs[prb][1][rl], g1 - d);
                    const float mref = xch_mref[prb][rl] + (float)d;
                    const size_t slot_idx = (size_t)u.slot;
                    const int row = u.jt * MT + 32 * prb + l32;
                    if (row < M) {
                        if (lse_writer && half == 0)
                            lse_out[slot_idx * M + row] = mref + __builtin_amdgcn_logf(l_tot) - kPExp;
                        const float inv = lq_tot > 0.f ? a.out_scale / lq_tot : 0.f;   // no key: O = 0
                        float *po = partial + (slot_idx * M + row) * kVDim;
#pragma unroll
                        for (int n = 0; n < NT; ++n) {
                            const int dim = 32 * (tile0 + n) + 4 * half;
#pragma unroll
                            for (int q4 = 0; q4 < 4; ++q4)
                                *(v4f *)(po + dim + 8 * q4) =
                                    v4f{acc[n][4 * q4], acc[n][4 * q4 + 1], acc[n][4 * q4 + 2],
                                        acc[n][4 * q4 + 3]} * inv;
                        }
                    }
                }
            }
            cursor_advance(cv, false);
        }
        if (page_bad && lane == 0) atomicOr(&header[kHdrStatus], AMLA_DEV_BAD_PAGE);
    }
}

}  // namespace

hipError_t launch_decode_stream(int mtile, dim3 grid, hipStream_t stream, const uint8_t *q,
                                const uint8_t *kv, const int32_t *block_table,
                                const int32_t *lengths, const int32_t *counts,
                                const int32_t *offsets, const int32_t *work, int32_t *header,
                                float *partial, float *lse, const DecodeArgs &a)
{
    if (mtile == 32)
        hipLaunchKernelGGL(decode_stream_kernel<32>, grid, dim3(2 * kDecodeThreads), 0, stream, q,
                           kv, block_table, lengths, counts, offsets, work, header, partial, lse, a);
    else
        hipLaunchKernelGGL(decode_stream_kernel<64>, grid, dim3(2 * kDecodeThreads), 0, stream, q,
                           kv, block_table, lengths, counts, offsets, work, header, partial, lse, a);
    return hipGetLastError();
}

}  // namespace amla
