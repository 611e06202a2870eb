// The 128-row decode kernel (row tiles of 128 folded rows: the compute-bound shapes).
// It is its own translation unit because it is compiled with MFMA accumulators in AGPRs
// (the other kernels keep the VGPR form): see decode128_kernel.
#include "common.h"

namespace amla {
namespace {

// 128-row tiles, the four waves on every page.  Wave w = 2p + kb computes the scores of key
// block kb (keys [32kb, +32) of the page) for the 64 rows [64p, +64) of the tile, so each
// K fragment read from LDS feeds two MFMAs (one per row block); the two waves of a row
// pair swap their key-block row maxima through LDS, so both take the same lazy max, then
// each writes its half of the E4M3 P^T fragments of its rows.  Wave w owns O^T for the
// 128 dims [128w, +128) of all 128 rows: after a second barrier it reads the P^T
// fragments of the four row blocks and each V^T fragment read from LDS feeds four MFMAs.
// The DMA of page t+3 goes into the slot page t-1 used.  Read-only inputs are separate
// __restrict__ arguments; their uniform reads go through the constant address space
// (scalar loads, which do not wait on the in-flight page DMAs).
__global__ __launch_bounds__(kDecodeThreads, 1) void decode128_kernel(
    const uint8_t *__restrict__ q_in, const uint8_t *__restrict__ kv_in,
    const int32_t *__restrict__ block_table, const int32_t *__restrict__ lengths,
    const int32_t *__restrict__ counts, const int32_t *__restrict__ offsets,
    const int32_t *__restrict__ work, int32_t *__restrict__ header, float *__restrict__ partial,
    float *__restrict__ lse_out, DecodeArgs a)
{
    constexpr int MT = 128;          // rows per work unit
    __shared__ __attribute__((aligned(1024))) uint8_t lds[kSlots * kPageBytes];
    // P^T fragments of the page: [row block][key block][lane][16 B]
    __shared__ __attribute__((aligned(16))) int32_t xch_p[4][2][64 * 4];
    // per (key block, row block, row): the key block's max on a unit's first page; at the
    // end its P sums
    __shared__ float xch_max[2][4][32];
    __shared__ float xch_lq[2][4][32];
    // per (row block, key block, row): the whole-number gap of the key block's P reference
    __shared__ int32_t xch_gap[4][2][32];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kb = wave & 1, rp = wave >> 1;
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
    // K fragment reads: key 32kb + l32 (same swizzle as key l32), chunks 4k + 2*half + e
    int k_off[2];
#pragma unroll
    for (int e = 0; e < 2; ++e)
        k_off[e] = (32 * kb + l32) * kKDim + 16 * ((2 * half + e) ^ swz(l32));

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
        const int row0 = jt * MT + 64 * rp;   // this wave's score rows: [row0, +64)
        int lim[2];   // keys each of this lane's two score rows sees
#pragma unroll
        for (int j = 0; j < 2; ++j) lim[j] = row_key_limit(a, total, L, row0 + 32 * j + l32);
        const int32_t *bt = block_table + (size_t)r * a.bt_stride + first;

        v8i qf[2][9];   // Q^T fragments of the two row blocks, loaded below

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

        // per score row block j: the row's reference and the whole-number gap of its P
        // reference above it (log2 units, shared by the two key-block waves), this key
        // block's FP32 P sum (for the LSE) and E4M3 P sum (O is normalised by the E4M3 sum
        // of both key blocks), both relative to m_ref
        float m_ref[2] = {-INFINITY, -INFINITY};
        int gap[2] = {0, 0};
        float l_run[2] = {0.f, 0.f}, lq_run[2] = {0.f, 0.f};
        v16f acc[4][4];   // O^T of row block rb, dim tile 4*wave + n
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
#pragma unroll
            for (int n = 0; n < 4; ++n) acc[rb][n] = v16f{0};

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
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int row = row0 + 32 * j + l32;
            if (row < M) {
                const uint8_t *qp = q_in + ((size_t)r * M + row) * kKDim + 32 * half;
#pragma unroll
                for (int k = 0; k < 9; ++k) {
                    const v4i x = *(const v4i *)(qp + 64 * k);
                    const v4i y = *(const v4i *)(qp + 64 * k + 16);
                    qf[j][k] = v8i{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
                }
            } else {
#pragma unroll
                for (int k = 0; k < 9; ++k) qf[j][k] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
            }
        }
        wait_pages_then_barrier(0);

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

            // S^T[32 keys of block kb x 32 rows] for the two row blocks: 9 K fragments,
            // each feeding two MFMAs, read one k-step ahead
            v16f sc[2];
            {
                const uint8_t *kp0 = slot + k_off[0], *kp1 = slot + k_off[1];
                v8i kf = lds_read2x16(kp0, kp1);
                __builtin_amdgcn_sched_barrier(0);
                static_for<0, 9>([&](auto kk) {
                    constexpr int k = decltype(kk)::value;
                    const v8i cur = kf;
                    if constexpr (k + 1 < 9) kf = lds_read2x16(kp0 + 64 * (k + 1), kp1 + 64 * (k + 1));
                    score_step<k == 0, k == 8>(sc[0], sc[1], cur, qf[0][k], qf[1][k]);
                    __builtin_amdgcn_sched_barrier(0);
                });
            }
            // key-block max of each row (masked by the row's key limit)
            float kmax[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                // keys of the page the row sees, counted from this lane's first key
                // (32kb + 4*half): element e holds key 8(e/4) + e%4 past it
                const int valid = lim[j] - (first + t) * kPage - (32 * kb + 4 * half);
                if (__any(valid < 32)) {
#pragma unroll
                    for (int e = 0; e < 16; ++e)
                        if (8 * (e >> 2) + (e & 3) >= valid) sc[j][e] = -INFINITY;
                }
                float mx = -INFINITY;
#pragma unroll
                for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sc[j][e]);
                kmax[j] = half_pair_max(mx) * a.score_scale;
            }
            // Reference of each row (log2 units, the same in both waves of the row pair):
            // m_ref is the row's max over the unit's first page (both key blocks, exchanged
            // once), and key block kb's P is 2^(s - m_ref - gap + kPExp) <= 2^8, gap the
            // smallest whole number keeping that block's running max at or below m_ref +
            // gap.  The P V MFMA scales each K block of its B operand by its own E8M0 byte,
            // so key block kb's P is scaled by 2^gap and O and the row sums stay relative to
            // m_ref with no rescaling and no agreement between the key blocks on later pages.
            if (t == 0) {
                // the row index is recomputed here (an opaque copy): a value kept across the
                // page loop would be spilled, and its reload waits for the page DMAs
                int row_l = lane & 31;
                asm volatile("" : "+v"(row_l));
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    if (half == 0) xch_max[kb][2 * rp + j][row_l] = kmax[j];
                lds_barrier();
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    // -inf while the row sees no key: with visible keys a prefix of the
                    // shard, a row that sees no key of its split's first page sees none
                    m_ref[j] = fmaxf(kmax[j], xch_max[kb ^ 1][2 * rp + j][row_l]);
                    gap[j] = 0;
                }
            } else {
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    if (kmax[j] > m_ref[j] + (float)gap[j]) gap[j] = (int)__builtin_ceilf(kmax[j] - m_ref[j]);
            }
            // P = 2^(s*scale - m_ref - gap + kPExp): FP32 into the row sum, E4M3 into this key
            // block's half of the P^T fragment (lane (l32, half) byte 4g + e, g < 4, holds
            // key 32kb + 8g + 4*half + e); the sums are kept relative to m_ref
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const float bias = m_ref[j] == -INFINITY ? 0.f : (kPExp - (float)gap[j]) - m_ref[j];
                float psum = 0.f, qsum = 0.f;
                v4i pw;
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    float p[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[j][4 * g + e], a.score_scale, bias));
                        psum += p[e];
                    }
                    int w4 = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], 0, false);
                    w4 = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], w4, true);
                    pw[g] = w4;
                    const v2f q0 = __builtin_amdgcn_cvt_pk_f32_fp8(w4, false);
                    const v2f q1 = __builtin_amdgcn_cvt_pk_f32_fp8(w4, true);
                    qsum += (q0[0] + q0[1]) + (q1[0] + q1[1]);
                }
                l_run[j] += __builtin_amdgcn_ldexpf(psum, gap[j]);
                lq_run[j] += __builtin_amdgcn_ldexpf(qsum, gap[j]);
                *(v4i *)&xch_p[2 * rp + j][kb][lane * 4] = pw;
                if (half == 0) xch_gap[2 * rp + j][kb][l32] = gap[j];
            }
            lds_barrier();

            // The row blocks' P^T fragments and the E8M0 scale of K block `half` (lane half h
            // supplies the scale of K block h of its column: 2^gap of key block h).  A
            // reference more than 2^64 below a key block's running max (practically never)
            // moves up by the larger gap: the row block's tiles in every wave, and its score
            // state in the two waves that own it.
            v8i pf[4];
            int sb[4];
            bool moved = false;
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) {
                const v4i lo = *(const v4i *)&xch_p[rb][0][lane * 4];
                const v4i hi = *(const v4i *)&xch_p[rb][1][lane * 4];
                pf[rb] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                const int g0 = xch_gap[rb][0][l32], g1 = xch_gap[rb][1][l32];
                moved = moved || (g0 > kRefGap || g1 > kRefGap);
                sb[rb] = 127 + (half ? g1 : g0);
            }
            if (__any(moved)) {
                // an MFMA that has just written a tile, then an MFMA reading a tile written
                // through v_accvgpr_write: wait states the compiler does not count for the
                // asm of scale_acc
                asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
                for (int rb = 0; rb < 4; ++rb) {
                    const int g0 = xch_gap[rb][0][l32], g1 = xch_gap[rb][1][l32];
                    const int gmax = g0 > g1 ? g0 : g1;
                    const int d = gmax > kRefGap ? gmax : 0;
                    const int g = sb[rb] - 127 - d;
                    sb[rb] = 127 + (g < -127 ? -127 : g);
                    if (rb >> 1 == rp) {   // this wave's score rows
                        const int j = rb & 1;
                        const float f = __builtin_amdgcn_ldexpf(1.f, -d);
                        l_run[j] *= f;
                        lq_run[j] *= f;
                        if (d > 0) m_ref[j] += (float)d;
                        gap[j] -= d;
                    }
                    if (!__any(d != 0)) continue;
                    const float f = __builtin_amdgcn_ldexpf(1.f, -d);
#pragma unroll
                    for (int n = 0; n < 4; ++n) scale_acc(acc[rb][n], f);
                }
                asm volatile("s_nop 7" ::: "memory");
            }
            // O^T[dims 128w + 32n, rows of block rb] += V^T (P^T, K block h scaled by 2^gap_h)
            auto vtile = [&](int n) {
                const int T = 4 * wave + n;
                const uint8_t *vp = slot + tr_off[T & 1] + 64 * (T >> 1);
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
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int n = 0; n < 4; ++n) {
                const v8i cur = vf;
                if (n + 1 < 4) vf = vtile(n + 1);
                // all four row blocks, also in a last tile with fewer rows: the accumulators
                // stay in their registers only when every page updates all of them
#pragma unroll
                for (int rb = 0; rb < 4; ++rb) acc[rb][n] = mfma_scaled_b(cur, pf[rb], acc[rb][n], sb[rb]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }

        if (page_bad && tid == 0) atomicOr(&header[kHdrStatus], AMLA_DEV_BAD_PAGE);

        // epilogue: the key-block sums are added over the row pair; each wave normalises
        // and stores its dims of all rows.  l and lq carry P's 2^kPExp, which cancels
        // in O / lq.
        const size_t slot_idx = (size_t)off_r + s;
        float l_tot[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            l_tot[j] = half_pair_sum(l_run[j]);
            const float lq_tot = half_pair_sum(lq_run[j]);
            if (half == 0) {
                xch_max[kb][2 * rp + j][l32] = l_tot[j];
                xch_lq[kb][2 * rp + j][l32] = lq_tot;
            }
        }
        lds_barrier();
        if (kb == 0 && half == 0) {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int row = row0 + 32 * j + l32;
                if (row < M) {
                    const float l = l_tot[j] + xch_max[1][2 * rp + j][l32];
                    lse_out[slot_idx * M + row] = m_ref[j] + __builtin_amdgcn_logf(l) - kPExp;
                }
            }
        }
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
            const int row = jt * MT + 32 * rb + l32;
            if (row < M) {
                const float lq = xch_lq[0][rb][l32] + xch_lq[1][rb][l32];
                const float inv = lq > 0.f ? a.out_scale / lq : 0.f;   // no key: O = 0
                float *po = partial + (slot_idx * M + row) * kVDim;
#pragma unroll
                for (int n = 0; n < 4; ++n) {
                    const int dim = 32 * (4 * wave + n) + 4 * half;
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4) {
                        const v16f &t16 = acc[rb][n];
                        const v4f o = v4f{t16[4 * q4], t16[4 * q4 + 1], t16[4 * q4 + 2],
                                          t16[4 * q4 + 3]} * inv;
                        *(v4f *)(po + dim + 8 * q4) = o;
                    }
                }
            }
        }

        lds_barrier();  // the next unit's prologue overwrites the ring and the exchange
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
