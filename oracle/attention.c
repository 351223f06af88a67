/*
 * fp64 reference for single-token decode attention over a paged KV cache.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is part of the oracle: a plain, slow
 * CPU statement of what the decode path computes.  Only the test suite, the
 * smoke check and the CPU-baseline leg of the benchmark may load it; the
 * product library never does, and the two share no code.
 *
 * What is computed (the plain definition; split-K, grouping and page layout
 * do not change it):
 *   For every active sequence s, query head r and its KV head h, over the
 *   token list T of that head -- the retained tokens 0..L-1 (Tangram,
 *   abstract: attention over each head's retained entries under a fixed
 *   per-head budget) or an explicit list of critical entries (KVDrive,
 *   Fig 1: sparse attention over selected entries) --
 *       z_t = scale * sum_d q[s][r][d] * K_t[d]
 *       m   = max_t z_t,   l = sum_t exp(z_t - m)
 *       out = sum_t exp(z_t - m) * V_t / l,   lse = m + ln l
 *   K_t / V_t is the bf16 row stored at page table entry t / P of the head's
 *   group, head slot inside the page, row t % P (KV-RM, abstract: logical
 *   histories decoupled from physical storage through a block pager;
 *   Tangram, Fig 8: one page table per head group).  An empty token list
 *   gives out = 0 and lse = -inf.
 * Everything is evaluated in double precision, summing in token-list order,
 * with two passes (maximum first, then the sums).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static double bf16_to_f64(uint16_t b) {
    uint32_t u = ((uint32_t)b) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Address of row t of KV head h of sequence s in a pool laid out as
 * [num_pages][heads_per_group][page_size][head_dim]. */
static const uint16_t *row_ptr(const uint16_t *pool, const int32_t *page_table,
                               int s, int h, long t, int B, int P, int G_h,
                               int max_pages, int D, const int32_t *group_of_head,
                               const int32_t *slot_of_head) {
    int g = group_of_head[h];
    long page = page_table[((long)g * B + s) * max_pages + t / P];
    long off = ((page * G_h + slot_of_head[h]) * P + t % P) * (long)D;
    return pool + off;
}

/*
 * tokens == NULL: token list is 0..lengths[s][h]-1.
 * tokens != NULL: token list is tokens[s][h][0..K-1] (logical positions).
 * Returns 0, or -1 when a token position is outside 0..lengths-1.
 */
int oracle_decode(int B, int Hq, int Hkv, int D, int P, int G_h, int max_pages,
                  const uint16_t *q, const uint16_t *pool_k, const uint16_t *pool_v,
                  const int32_t *page_table, const int32_t *lengths,
                  const int32_t *group_of_head, const int32_t *slot_of_head,
                  const int32_t *tokens, int K, double scale,
                  double *out, double *lse, int num_threads) {
    int gqa = Hq / Hkv;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(num_threads) reduction(| : bad)
    for (long sr = 0; sr < (long)B * Hq; ++sr) {
        int s = (int)(sr / Hq), r = (int)(sr % Hq), h = r / gqa;
        long L = lengths[s * Hkv + h];
        long n = tokens ? (L > 0 ? K : 0) : L;
        double *o = out + sr * D;
        for (int d = 0; d < D; ++d) o[d] = 0.0;
        if (n <= 0) {
            lse[sr] = -INFINITY;
            continue;
        }
        double *z = (double *)malloc(sizeof(double) * n);
        const uint16_t *qr = q + sr * D;
        double m = -INFINITY;
        for (long i = 0; i < n; ++i) {
            long t = tokens ? tokens[((long)s * Hkv + h) * K + i] : i;
            if (t < 0 || t >= L) { bad = 1; t = 0; }
            const uint16_t *kr = row_ptr(pool_k, page_table, s, h, t, B, P, G_h,
                                         max_pages, D, group_of_head, slot_of_head);
            double acc = 0.0;
            for (int d = 0; d < D; ++d) acc += bf16_to_f64(qr[d]) * bf16_to_f64(kr[d]);
            z[i] = scale * acc;
            if (z[i] > m) m = z[i];
        }
        double l = 0.0;
        for (long i = 0; i < n; ++i) {
            long t = tokens ? tokens[((long)s * Hkv + h) * K + i] : i;
            if (t < 0 || t >= L) t = 0;
            const uint16_t *vr = row_ptr(pool_v, page_table, s, h, t, B, P, G_h,
                                         max_pages, D, group_of_head, slot_of_head);
            double p = exp(z[i] - m);
            l += p;
            for (int d = 0; d < D; ++d) o[d] += p * bf16_to_f64(vr[d]);
        }
        for (int d = 0; d < D; ++d) o[d] /= l;
        lse[sr] = m + log(l);
        free(z);
    }
    return bad ? -1 : 0;
}
