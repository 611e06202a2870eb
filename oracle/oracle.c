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

typedef struct {
    int32_t size, r, s;
} oracle_item;

static int oracle_item_order(const void *x, const void *y)
{
    const oracle_item *p = (const oracle_item *)x, *q = (const oracle_item *)y;
    if (p->size != q->size)
        return p->size > q->size ? -1 : 1; /* longest first */
    if (p->r != q->r)
        return p->r < q->r ? -1 : 1; /* ties: the lower request first */
    return p->s < q->s ? -1 : (p->s > q->s);
}

/*
 * The split plan (this project's reading; the pages leave the formula open).
 *
 *   pages_r = ceil(L_r / 64); mt = ceil(M / MT) row tiles per split.
 *   BALANCED: chunk(B) = the smallest c >= 1 with mt * sum_r ceil(pages_r / c) <= B
 *             (c = max pages if none), raised to at least ceil(min_split_tokens / 64);
 *             count_r = min(max_splits, ceil(pages_r / chunk)), with chunk = chunk(W);
 *             but when the longest split, max_r ceil(pages_r / count_r), exceeds 5/4 of the
 *             mean work per worker, mt * sum_r pages_r / W (that is, 4 * longest * W >
 *             5 * mt * total), chunk = chunk(2 W): finer splits, about two per worker,
 *             so that a batch of very different lengths does not wait on its longest
 *             split.
 *   FIXED:    count_r = min(pages_r, clamp(floor(W / (R * mt)), 1, max_splits)).
 *   count_r = 0 when pages_r = 0.
 *   offsets = exclusive prefix sum of counts (workspace slot of (r, s) = offsets[r] + s).
 *   Split s of r covers pages [s*q + min(s, rem), +q + (s < rem)) with q = pages_r / count_r,
 *   rem = pages_r % count_r.
 *   work = (r, s) pairs sorted by split size, longest first, ties by r then s
 *   (the tie rule of the host tiering: page "drafter.attention", _plan_kernel),
 *   then -1 up to list_len.
 *
 * Returns the number of items, -1 on invalid arguments (negative length,
 * pages_r > bt_cols, bad sizes), -2 if list_len < 2 * items.
 */
/* The smallest chunk c >= 1 with mt * sum_r ceil(pages_r / c) <= budget (the longest
   request's pages if none), raised to min_pages; by trying every c in turn. */
static int32_t oracle_chunk(const int32_t *lengths, int32_t R, int32_t mt, int64_t pmax,
                            int64_t budget, int32_t min_pages)
{
    int32_t chunk = (int32_t)(pmax > 0 ? pmax : 1);
    for (int64_t c = 1; c <= pmax; ++c) {
        int64_t units = 0;
        for (int32_t r = 0; r < R; ++r) {
            int64_t pages = ((int64_t)lengths[r] + ORACLE_PAGE - 1) / ORACLE_PAGE;
            units += mt * ((pages + c - 1) / c);
        }
        if (units <= budget) {
            chunk = (int32_t)c;
            break;
        }
    }
    return chunk < min_pages ? min_pages : chunk;
}

int oracle_plan(const int32_t *lengths, int32_t R, int32_t bt_cols, int32_t M, int32_t MT,
                int32_t W, int32_t min_split_tokens, int32_t max_splits, int32_t mode,
                int32_t *counts, int32_t *offsets, int32_t *work, int32_t list_len)
{
    int64_t pmax = 0, n = 0;
    int32_t mt, min_pages, chunk;
    oracle_item *items;

    if (R < 0 || M < 1 || MT < 1 || W < 1 || max_splits < 1 || min_split_tokens < 0 ||
        (mode != 0 && mode != 1))
        return -1;
    mt = (M + MT - 1) / MT;
    min_pages = (min_split_tokens + ORACLE_PAGE - 1) / ORACLE_PAGE;
    for (int32_t r = 0; r < R; ++r) {
        int64_t pages;
        if (lengths[r] < 0)
            return -1;
        pages = ((int64_t)lengths[r] + ORACLE_PAGE - 1) / ORACLE_PAGE;
        if (pages > bt_cols)
            return -1;
        if (pages > pmax)
            pmax = pages;
    }

    if (mode == 0) {
        int64_t total = 0, longest = 0;
        chunk = oracle_chunk(lengths, R, mt, pmax, (int64_t)W, min_pages);
        for (int32_t r = 0; r < R; ++r) {
            int64_t pages = ((int64_t)lengths[r] + ORACLE_PAGE - 1) / ORACLE_PAGE;
            int64_t c = (pages + chunk - 1) / chunk, size;
            total += pages;
            if (pages == 0)
                continue;
            if (c > max_splits)
                c = max_splits;
            size = (pages + c - 1) / c;
            if (size > longest)
                longest = size;
        }
        if (4 * longest * (int64_t)W > 5 * (int64_t)mt * total)
            chunk = oracle_chunk(lengths, R, mt, pmax, 2 * (int64_t)W, min_pages);
        for (int32_t r = 0; r < R; ++r) {
            int64_t pages = ((int64_t)lengths[r] + ORACLE_PAGE - 1) / ORACLE_PAGE;
            int64_t c = pages == 0 ? 0 : (pages + chunk - 1) / chunk;
            counts[r] = (int32_t)(c < max_splits ? c : max_splits);
        }
    } else {
        int64_t fixed = R > 0 ? (int64_t)W / ((int64_t)R * mt) : 1;
        if (fixed < 1)
            fixed = 1;
        if (fixed > max_splits)
            fixed = max_splits;
        for (int32_t r = 0; r < R; ++r) {
            int64_t pages = ((int64_t)lengths[r] + ORACLE_PAGE - 1) / ORACLE_PAGE;
            counts[r] = (int32_t)(pages < fixed ? pages : fixed);
        }
    }

    for (int32_t r = 0; r < R; ++r) {
        offsets[r] = (int32_t)n;
        n += counts[r];
    }
    offsets[R] = (int32_t)n;
    if (2 * n > list_len)
        return -2;

    items = (oracle_item *)malloc(sizeof(oracle_item) * (size_t)(n > 0 ? n : 1));
    if (!items)
        return -1;
    n = 0;
    for (int32_t r = 0; r < R; ++r) {
        int64_t pages = ((int64_t)lengths[r] + ORACLE_PAGE - 1) / ORACLE_PAGE;
        for (int32_t s = 0; s < counts[r]; ++s) {
            int64_t q = pages / counts[r], rem = pages % counts[r];
            items[n].size = (int32_t)(q + (s < rem));
            items[n].r = r;
            items[n].s = s;
            ++n;
        }
    }
    qsort(items, (size_t)n, sizeof(oracle_item), oracle_item_order);
    for (int32_t k = 0; k < list_len; ++k)
        work[k] = -1;
    for (int64_t k = 0; k < n; ++k) {
        work[2 * k] = items[k].r;
        work[2 * k + 1] = items[k].s;
    }
    free(items);
    return (int32_t)n;
}

/* The token range [*a, *b) of split s of request r under a plan (counts). */
int oracle_split_range(int32_t length, int32_t count, int32_t s, int32_t *a, int32_t *b)
{
    int64_t pages = ((int64_t)length + ORACLE_PAGE - 1) / ORACLE_PAGE;
    int64_t q, rem, first, size, end;
    if (count < 1 || s < 0 || s >= count || length < 0)
        return -1;
    q = pages / count;
    rem = pages % count;
    first = s * q + (s < rem ? s : rem);
    size = q + (s < rem);
    end = (first + size) * ORACLE_PAGE;
    *a = (int32_t)(first * ORACLE_PAGE);
    *b = (int32_t)(end < length ? end : length);
    return 0;
}
