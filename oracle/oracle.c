/*
 * CPU oracle for the folded split-KV absorbed-MLA decode.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or call
 * this file: only the tests, the smoke check and the benchmark's CPU-baseline leg
 * use it.  It shares no code, header, table or constant generator with the HIP
 * library; it is plain C99 + OpenMP and computes in double precision.
 *
 * What it computes, and where the pages state it:
 *
 *  - oracle_e4m3_value: the OCP float8 E4M3FN code -> real value.  The cache and
 *    the query are torch.float8_e4m3fn (page "drafter.attention", cake_supported:
 *    FP8 query and cache).  Format: 1 sign, 4 exponent (bias 7), 3 mantissa bits;
 *    exponent 0 is subnormal; S.1111.111 is NaN; there is no infinity.
 *
 *  - oracle_attend: exact softmax attention of one folded query row over a key
 *    range of one request.  Absorbed MLA decode is MQA over a single latent KV
 *    head, every (token, head) row has its own full softmax over the request's
 *    keys, and folding the k tokens into heads changes nothing of that (page
 *    "drafter.attention", module docstring).  Keys are 576 bytes (512 latent then
 *    64 rope), the value is the first 512 (page "drafter.attention", folded_decode:
 *    output width kv_lora_rank).  Scores use the dequantized operands and the
 *    softmax scale; the stock bmm1 = scale * q_scale * k_scale and bmm2 = k_scale
 *    (page "drafter.attention", _scales) are the same numbers regrouped, so the
 *    oracle takes q_scale, k_scale and sm_scale separately.  The LSE returned is
 *    log2 of sum_j exp(s_j) (page "cutedsl.mla.balanced", BalancedMla.decode:
 *    log2 lse).  An empty range gives out = 0 and lse = -inf (zero-length rows do
 *    no work: page "drafter.attention", balanced_decode).
 *
 *  - oracle_merge: the LSE merge of partial results, exp2(lse_s - max) weights
 *    normalised by their sum (page "drafter.attention", DraftDcp: the merge over
 *    sources in FP32 with exp2 weights).
 *
 *  - oracle_plan: the integer split plan.  The pages only say that each request's
 *    split count is planned from the KV lengths on the device and that one wave of
 *    persistent workers walks a work list (page "cutedsl.mla.balanced", module
 *    docstring); fixed equal splits per batch shape are the comparator there.  The
 *    exact rule is this project's reading and is written out at oracle_plan.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <omp.h>

#define ORACLE_PAGE 64
#define ORACLE_KDIM 576
#define ORACLE_VDIM 512

/* Threads the oracle's parallel loops use (OpenMP's current maximum). */
int oracle_threads(void)
{
    return omp_get_max_threads();
}

/* Sets the threads later parallel loops use (n >= 1); returns the previous count. */
int oracle_set_threads(int n)
{
    const int prev = omp_get_max_threads();
    if (n >= 1) omp_set_num_threads(n);
    return prev;
}

/* ---------------------------------------------------------------- E4M3FN */

double oracle_e4m3_value(uint8_t code)
{
    int sign = code >> 7;
    int exponent = (code >> 3) & 0xF;
    int mantissa = code & 0x7;
    double magnitude;
    if (exponent == 0xF && mantissa == 0x7)
        return NAN;
    if (exponent == 0)
        magnitude = ldexp((double)mantissa / 8.0, -6);
    else
        magnitude = ldexp(1.0 + (double)mantissa / 8.0, exponent - 7);
    return sign ? -magnitude : magnitude;
}

void oracle_e4m3_table(double *out256)
{
    for (int c = 0; c < 256; ++c)
        out256[c] = oracle_e4m3_value((uint8_t)c);
}

/* ------------------------------------------------------------- attention */

/*
 * tasks: ntasks x 4 int32 (request r, folded row i, key begin a, key end b).
 * q8:  [R][M][576] E4M3 codes, row i = t*H + h (token-major, then head).
 * kv8: [pool_pages][64][576] E4M3 codes.
 * block_table: [R][bt_stride] physical page of each 64-key page of the request.
 * out: ntasks x 512 doubles; lse: ntasks doubles (log2 units).
 * Returns 0, or -1 on an out-of-range task, length or page id.
 */
int oracle_attend(const uint8_t *q8, const uint8_t *kv8, int64_t pool_pages,
                  const int32_t *block_table, int32_t bt_stride,
                  const int32_t *lengths, int32_t R, int32_t M,
                  double q_scale, double k_scale, double sm_scale,
                  const int32_t *tasks, int32_t ntasks,
                  double *out, double *lse)
{
    double table[256];
    int bad = 0;
    oracle_e4m3_table(table);

    for (int32_t t = 0; t < ntasks; ++t) {
        int32_t r = tasks[4 * t], i = tasks[4 * t + 1];
        int32_t a = tasks[4 * t + 2], b = tasks[4 * t + 3];
        if (r < 0 || r >= R || i < 0 || i >= M || a < 0 || b < a || b > lengths[r])
            return -1;
        for (int32_t j = a; j < b; ++j) {
            int32_t page = block_table[(int64_t)r * bt_stride + j / ORACLE_PAGE];
            if (page < 0 || page >= pool_pages)
                return -1;
        }
    }

#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int32_t t = 0; t < ntasks; ++t) {
        int32_t r = tasks[4 * t], i = tasks[4 * t + 1];
        int32_t a = tasks[4 * t + 2], b = tasks[4 * t + 3];
        double *o = out + (int64_t)t * ORACLE_VDIM;
        const uint8_t *qrow = q8 + ((int64_t)r * M + i) * ORACLE_KDIM;
        double qhat[ORACLE_KDIM];
        double *score;
        double m = -INFINITY, l = 0.0;

        for (int c = 0; c < ORACLE_VDIM; ++c)
            o[c] = 0.0;
        if (a == b) {
            lse[t] = -INFINITY;
            continue;
        }
        score = (double *)malloc(sizeof(double) * (size_t)(b - a));
        if (!score) {
            bad |= 1;
            continue;
        }
        for (int d = 0; d < ORACLE_KDIM; ++d)
            qhat[d] = q_scale * table[qrow[d]];

        /* s_j = sm_scale * <q_hat, k_hat_j> over all 576 dims */
        for (int32_t j = a; j < b; ++j) {
            int32_t page = block_table[(int64_t)r * bt_stride + j / ORACLE_PAGE];
            const uint8_t *krow = kv8 + ((int64_t)page * ORACLE_PAGE + j % ORACLE_PAGE) * ORACLE_KDIM;
            double dot = 0.0;
            for (int d = 0; d < ORACLE_KDIM; ++d)
                dot += qhat[d] * (k_scale * table[krow[d]]);
            score[j - a] = sm_scale * dot;
            if (score[j - a] > m)
                m = score[j - a];
        }
        /* softmax weights exp(s_j - m), their sum l, and the weighted values */
        for (int32_t j = a; j < b; ++j) {
            int32_t page = block_table[(int64_t)r * bt_stride + j / ORACLE_PAGE];
            const uint8_t *vrow = kv8 + ((int64_t)page * ORACLE_PAGE + j % ORACLE_PAGE) * ORACLE_KDIM;
            double w = exp(score[j - a] - m);
            l += w;
            for (int c = 0; c < ORACLE_VDIM; ++c)
                o[c] += w * (k_scale * table[vrow[c]]);
        }
        for (int c = 0; c < ORACLE_VDIM; ++c)
            o[c] /= l;
        /* log2 sum_j exp(s_j) = (m + ln l) / ln 2 */
        lse[t] = (m + log(l)) / log(2.0);
        free(score);
    }
    return bad ? -1 : 0;
}

/* ------------------------------------------------------------------ merge */

/*
 * n partials (o_s: n x 512, lse_s: n, log2 units) -> one (out, lse).
 * Mx = max_s lse_s; lse = Mx + log2 sum_s 2^(lse_s - Mx); out = sum_s 2^(lse_s - lse) o_s.
 * Partials with lse_s = -inf carry no weight; with none left, out = 0, lse = -inf.
 */
void oracle_merge(const double *o, const double *lse, int32_t n, double *out, double *lse_out)
{
    double mx = -INFINITY, total = 0.0;
    for (int c = 0; c < ORACLE_VDIM; ++c)
        out[c] = 0.0;
    for (int32_t s = 0; s < n; ++s)
        if (lse[s] > mx)
            mx = lse[s];
    if (mx == -INFINITY) {
        *lse_out = -INFINITY;
        return;
    }
    for (int32_t s = 0; s < n; ++s)
        total += exp2(lse[s] - mx);
    *lse_out = mx + log2(total);
    for (int32_t s = 0; s < n; ++s) {
        double w = exp2(lse[s] - *lse_out);
        if (w == 0.0)
            continue;
        for (int c = 0; c < ORACLE_VDIM; ++c)
            out[c] += w * o[(int64_t)s * ORACLE_VDIM + c];
    }
}

/* ------------------------------------------------------------------- plan */

/*
 * The split plan (this project's reading; the pages leave the formula open: per-request
 * split counts planned from the KV lengths on the device, one wave of persistent workers
 * walking a work list, fixed equal splits per batch shape as the comparator).
 *
 *   pages_r = ceil(L_r / 64); mt = ceil(M / MT) row tiles per split; the mt row tiles of a
 *   split go to the mt workers of one group, G = max(1, floor(W / mt)) groups;
 *   minp = max(1, ceil(min_split_tokens / 64)); a = split_cost, what one split costs a
 *   worker beyond its pages (its query rows and its partial output), in pages.
 *   BALANCED: each non-empty request is laid out as a head of a pages followed by its
 *     pages_r pages, the requests end to end (request r from voff_r; V in all), and V is
 *     cut into Gp = min(G, max_splits, max(1, floor(V / minp))) ranges at
 *     c_g = floor(g * V / Gp), g = 0..Gp.  A cut strictly inside request r at page
 *     x = c_g - voff_r - a of it (negative in the head) moves to the request's start when
 *     x < minp and to its end when pages_r - x < minp; otherwise it cuts r at page x.
 *     A request's splits start at page 0 and at each cut left inside it (every piece is
 *     then at least minp pages or the whole request); group g takes the items starting in
 *     [C_g, C_{g+1}) of the moved cuts (an item's start being voff_r for a request's first
 *     item, voff_r + a + its first page for the others), so every group costs about V / Gp.
 *   FIXED: count_r = min(pages_r, clamp(floor(W / (R * mt)), 1, max_splits)) equal splits,
 *     split s covering pages [s*q + min(s, rem), +q + (s < rem)), q = pages_r / count_r,
 *     rem = pages_r % count_r; group g takes items [floor(g * N / G), floor((g+1) * N / G)).
 *   count_r = 0 when pages_r = 0.  offsets = exclusive prefix sum of counts.  Items are in
 *   request order, item offsets[r] + s being split s of request r (and its workspace slot):
 *   work[2i] = r, work[2i+1] = its first page (i < N), then -1 up to 2 * (R + W); then
 *   work[2 * (R + W) + g] = the first item of group g, g = 0..G (group g takes items
 *   [that, the next group's)); the rest of the list is -1.  Item i covers pages
 *   [first_i, first_{i+1}) when item i+1 is of the same request, else [first_i, pages_r).
 *
 * Returns N, the number of items, -1 on invalid arguments (negative length, pages_r >
 * bt_cols, bad sizes), -2 if list_len < 2 * (R + 2 * W).
 */
int oracle_plan(const int32_t *lengths, int32_t R, int32_t bt_cols, int32_t M, int32_t MT,
                int32_t W, int32_t min_split_tokens, int32_t max_splits, int32_t split_cost,
                int32_t mode, int32_t *counts, int32_t *offsets, int32_t *work,
                int32_t list_len)
{
    int64_t V = 0, n = 0, G, minp, mt, a = split_cost;
    int64_t *pages, *voff, *cut = NULL;
    int32_t *gstart;

    if (R < 0 || M < 1 || MT < 1 || W < 1 || max_splits < 1 || min_split_tokens < 0 ||
        split_cost < 0 || (mode != 0 && mode != 1))
        return -1;
    for (int32_t r = 0; r < R; ++r)
        if (lengths[r] < 0 || ((int64_t)lengths[r] + ORACLE_PAGE - 1) / ORACLE_PAGE > bt_cols)
            return -1;
    if ((int64_t)list_len < 2 * ((int64_t)R + 2 * (int64_t)W))
        return -2;
    mt = (M + MT - 1) / MT;
    G = W / mt < 1 ? 1 : W / mt;
    minp = ((int64_t)min_split_tokens + ORACLE_PAGE - 1) / ORACLE_PAGE;
    if (minp < 1)
        minp = 1;

    pages = (int64_t *)malloc(sizeof(int64_t) * (size_t)(R + 1));
    voff = (int64_t *)malloc(sizeof(int64_t) * (size_t)(R + 1));
    if (!pages || !voff) {
        free(pages);
        free(voff);
        return -1;
    }
    for (int32_t r = 0; r < R; ++r) {
        pages[r] = ((int64_t)lengths[r] + ORACLE_PAGE - 1) / ORACLE_PAGE;
        voff[r] = V;
        V += pages[r] > 0 ? a + pages[r] : 0;
    }
    voff[R] = V;
    for (int32_t k = 0; k < list_len; ++k)
        work[k] = -1;
    gstart = work + 2 * ((int64_t)R + W);

    if (mode == 0) {
        int64_t Gp = V / minp;
        if (Gp < 1)
            Gp = 1;
        if (Gp > G)
            Gp = G;
        if (Gp > max_splits)
            Gp = max_splits;
        /* the moved cuts C_0..C_Gp */
        cut = (int64_t *)malloc(sizeof(int64_t) * (size_t)(Gp + 1));
        if (!cut) {
            free(pages);
            free(voff);
            return -1;
        }
        for (int64_t g = 0; g <= Gp; ++g) {
            int64_t c = g * V / Gp;
            cut[g] = c;
            for (int32_t r = 0; r < R; ++r) {
                int64_t end = voff[r] + (pages[r] > 0 ? a + pages[r] : 0);
                if (voff[r] < c && c < end) {                    /* inside request r */
                    int64_t x = c - voff[r] - a;
                    if (x < minp)
                        cut[g] = voff[r];
                    else if (pages[r] - x < minp)
                        cut[g] = end;
                    break;
                }
            }
        }
        /* each request's splits: its pieces between the distinct moved cuts inside it */
        for (int32_t r = 0; r < R; ++r) {
            int64_t last = -1, end = voff[r] + a + pages[r];
            offsets[r] = (int32_t)n;
            counts[r] = 0;
            if (pages[r] == 0)
                continue;
            work[2 * n] = r;
            work[2 * n + 1] = 0;
            ++n;
            counts[r] = 1;
            for (int64_t g = 0; g <= Gp; ++g) {
                if (voff[r] < cut[g] && cut[g] < end && cut[g] != last) {
                    work[2 * n] = r;
                    work[2 * n + 1] = (int32_t)(cut[g] - voff[r] - a);
                    ++n;
                    ++counts[r];
                    last = cut[g];
                }
            }
        }
        /* group g takes the items starting in [C_g, C_{g+1}) */
        for (int64_t g = 0; g <= G; ++g) {
            int64_t first = n;
            if (g <= Gp) {
                for (int64_t i = 0; i < n; ++i) {
                    int32_t r = work[2 * i];
                    int64_t start = voff[r] + (work[2 * i + 1] > 0 ? a + work[2 * i + 1] : 0);
                    if (start >= cut[g]) {
                        first = i;
                        break;
                    }
                }
            }
            gstart[g] = (int32_t)first;
        }
    } else {
        int64_t fixed = R > 0 ? (int64_t)W / ((int64_t)R * mt) : 1;
        if (fixed < 1)
            fixed = 1;
        if (fixed > max_splits)
            fixed = max_splits;
        for (int32_t r = 0; r < R; ++r) {
            int64_t c = pages[r] < fixed ? pages[r] : fixed;
            offsets[r] = (int32_t)n;
            counts[r] = (int32_t)c;
            for (int64_t s = 0; s < c; ++s) {
                int64_t q = pages[r] / c, rem = pages[r] % c;
                work[2 * n] = r;
                work[2 * n + 1] = (int32_t)(s * q + (s < rem ? s : rem));
                ++n;
            }
        }
        for (int64_t g = 0; g <= G; ++g)
            gstart[g] = (int32_t)(g * n / G);
    }
    offsets[R] = (int32_t)n;
    free(cut);
    free(pages);
    free(voff);
    return (int32_t)n;
}

/* The request and token range [*a, *b) of item i of a plan (work list of N items). */
int oracle_item_range(const int32_t *work, int32_t N, const int32_t *lengths, int32_t R,
                      int32_t i, int32_t *r, int32_t *a, int32_t *b)
{
    int64_t pages, end;
    if (i < 0 || i >= N || work[2 * i] < 0 || work[2 * i] >= R)
        return -1;
    *r = work[2 * i];
    pages = ((int64_t)lengths[*r] + ORACLE_PAGE - 1) / ORACLE_PAGE;
    end = (i + 1 < N && work[2 * i + 2] == *r) ? work[2 * i + 3] : pages;
    if (work[2 * i + 1] < 0 || work[2 * i + 1] >= end || end > pages)
        return -1;
    *a = work[2 * i + 1] * ORACLE_PAGE;
    *b = (int32_t)(end * ORACLE_PAGE < lengths[*r] ? end * ORACLE_PAGE : lengths[*r]);
    return 0;
}
