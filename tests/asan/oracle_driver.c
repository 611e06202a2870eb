/*
 * Runs the oracle's entry points on inputs read from a file and writes their results to
 * another, so that a build of oracle.c with the address and undefined-behaviour
 * sanitizers can be exercised on the inputs the tests use and its results compared with
 * the regular build's.  Test infrastructure only.
 *
 * usage: oracle_driver attend|plan|merge <in> <out>
 *   attend in:  int32 R, M, cols, pool, ntasks; double q_scale, k_scale, sm_scale;
 *               uint8 q8[R*M*576], kv8[pool*64*576]; int32 bt[R*cols], lengths[R],
 *               tasks[ntasks*4]
 *          out: int32 rc; double out[ntasks*512], lse[ntasks]
 *   plan   in:  int32 R, bt_cols, M, MT, W, min_split_tokens, max_splits, mode, list_len,
 *               lengths[R]
 *          out: int32 rc, counts[R], offsets[R+1], work[list_len]
 *   merge  in:  int32 n; double o[n*512], lse[n]
 *          out: double out[512], lse
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_attend(const uint8_t *q8, const uint8_t *kv8, int64_t pool_pages,
                  const int32_t *block_table, int32_t bt_stride, const int32_t *lengths,
                  int32_t R, int32_t M, double q_scale, double k_scale, double sm_scale,
                  const int32_t *tasks, int32_t ntasks, double *out, double *lse);
int oracle_plan(const int32_t *lengths, int32_t R, int32_t bt_cols, int32_t M, int32_t MT,
                int32_t W, int32_t min_split_tokens, int32_t max_splits, int32_t split_cost,
                int32_t mode, int32_t *counts, int32_t *offsets, int32_t *work,
                int32_t list_len);
void oracle_merge(const double *o, const double *lse, int32_t n, double *out, double *lse_out);

static void *take(FILE *f, size_t bytes)
{
    void *p = malloc(bytes ? bytes : 1);
    if (!p || fread(p, 1, bytes, f) != bytes) {
        fprintf(stderr, "short input\n");
        exit(2);
    }
    return p;
}

int main(int argc, char **argv)
{
    if (argc != 4) return 2;
    FILE *in = fopen(argv[2], "rb"), *out = fopen(argv[3], "wb");
    if (!in || !out) return 2;
    if (!strcmp(argv[1], "attend")) {
        int32_t *h = take(in, 5 * sizeof(int32_t));
        double *sc = take(in, 3 * sizeof(double));
        const int32_t R = h[0], M = h[1], cols = h[2], pool = h[3], nt = h[4];
        uint8_t *q8 = take(in, (size_t)R * M * 576);
        uint8_t *kv8 = take(in, (size_t)pool * 64 * 576);
        int32_t *bt = take(in, (size_t)R * cols * sizeof(int32_t));
        int32_t *len = take(in, (size_t)R * sizeof(int32_t));
        int32_t *tasks = take(in, (size_t)nt * 4 * sizeof(int32_t));
        double *o = malloc((size_t)nt * 512 * sizeof(double) + 8);
        double *l = malloc((size_t)nt * sizeof(double) + 8);
        int32_t rc = oracle_attend(q8, kv8, pool, bt, cols, len, R, M, sc[0], sc[1], sc[2],
                                   tasks, nt, o, l);
        fwrite(&rc, sizeof rc, 1, out);
        fwrite(o, sizeof(double), (size_t)nt * 512, out);
        fwrite(l, sizeof(double), (size_t)nt, out);
        free(h); free(sc); free(q8); free(kv8); free(bt); free(len); free(tasks); free(o); free(l);
    } else if (!strcmp(argv[1], "plan")) {
        int32_t *h = take(in, 10 * sizeof(int32_t));
        const int32_t R = h[0], list_len = h[9];
        int32_t *len = take(in, (size_t)R * sizeof(int32_t));
        int32_t *counts = malloc((size_t)R * sizeof(int32_t) + 4);
        int32_t *offsets = malloc((size_t)(R + 1) * sizeof(int32_t));
        int32_t *work = malloc((size_t)list_len * sizeof(int32_t) + 4);
        int32_t rc = oracle_plan(len, R, h[1], h[2], h[3], h[4], h[5], h[6], h[7], h[8],
                                 counts, offsets, work, list_len);
        fwrite(&rc, sizeof rc, 1, out);
        fwrite(counts, sizeof(int32_t), (size_t)R, out);
        fwrite(offsets, sizeof(int32_t), (size_t)R + 1, out);
        fwrite(work, sizeof(int32_t), (size_t)list_len, out);
        free(h); free(len); free(counts); free(offsets); free(work);
    } else if (!strcmp(argv[1], "merge")) {
        int32_t *h = take(in, sizeof(int32_t));
        const int32_t n = h[0];
        double *o = take(in, (size_t)n * 512 * sizeof(double));
        double *l = take(in, (size_t)n * sizeof(double));
        double res[513];
        oracle_merge(o, l, n, res, res + 512);
        fwrite(res, sizeof(double), 513, out);
        free(h); free(o); free(l);
    } else {
        return 2;
    }
    fclose(in);
    fclose(out);
    return 0;
}
