/*
 * seer_oracle.c -- plain fp64 CPU oracle (TEST INFRASTRUCTURE ONLY; see seer_oracle.h).
 *
 * Written for a reader checking it against the pages by eye: every step is
 * the definition written out with loops, in the order the method applies
 * them, with no blocking, fusion or reassociation beyond that definition.
 * The attention part (D6, P4) is textbook softmax attention restricted to a
 * token set; the gate and selection parts (D1-D4, P1-P3) follow the gating
 * steps of the SeerAttention pages.  Only OpenMP over independent heads is
 * added, which changes no result.
 */
#include "seer_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

double so_bf16_to_f64(uint16_t bits)
{
    /* bf16 is the upper half of an IEEE binary32; widening is exact. */
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

int so_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ---------------------------------------------------------------- D1 ---- */
/* The gate pools keys along the sequence dimension, one vector per block
 * (SeerAttention v1 abstract); the pooling operator is the mean.  Only
 * complete blocks have a pooled key. */
int so_pool_k(const uint16_t *k, int64_t row_stride, int L, int d, int bs, double *kpool)
{
    if (!k || !kpool || L < 0 || d <= 0 || bs <= 0 || row_stride < d)
        return -1;
    int nc = L / bs;
    for (int j = 0; j < nc; ++j) {
        for (int c = 0; c < d; ++c) {
            double sum = 0.0;
            for (int t = j * bs; t < (j + 1) * bs; ++t)
                sum += so_bf16_to_f64(k[(int64_t)t * row_stride + c]);
            kpool[(int64_t)j * d + c] = sum / bs;
        }
    }
    return 0;
}

/* ------------------------------------------------------------ D2 + D3 --- */
/* Gate of SeerAttention-R (abstract): SeerAttention's gate (v1 abstract:
 * learnable linear layers applied to the pooled query and pooled key, the
 * two results multiplied into gating scores) with query pooling removed, so
 * each decode query row is projected as it is.  Under GQA one selection is
 * shared by the KV head's group: its score is the mean over the group's
 * query heads of their own gate logits. */
int so_gate_scores(const uint16_t *q, int64_t q_row_stride, int G, int d,
                   const uint16_t *wq, const uint16_t *wk, int dg,
                   const double *kpool, int nc, double gate_scale,
                   double *s_head, double *S)
{
    if (!q || !wq || !wk || !S || (nc > 0 && !kpool) || G <= 0 || d <= 0 || dg <= 0 || nc < 0)
        return -1;
    double *a = (double *)malloc(sizeof(double) * (size_t)G * dg);   /* a_h = Wq q_h   */
    double *c = (double *)malloc(sizeof(double) * (size_t)dg);       /* c_j = Wk kp_j  */
    if (!a || !c) {
        free(a);
        free(c);
        return -2;
    }
    for (int h = 0; h < G; ++h)
        for (int r = 0; r < dg; ++r) {
            double acc = 0.0;
            for (int e = 0; e < d; ++e)
                acc += so_bf16_to_f64(wq[(int64_t)r * d + e]) * so_bf16_to_f64(q[h * q_row_stride + e]);
            a[(int64_t)h * dg + r] = acc;
        }
    for (int j = 0; j < nc; ++j) {
        for (int r = 0; r < dg; ++r) {
            double acc = 0.0;
            for (int e = 0; e < d; ++e)
                acc += so_bf16_to_f64(wk[(int64_t)r * d + e]) * kpool[(int64_t)j * d + e];
            c[r] = acc;
        }
        double mean = 0.0;
        for (int h = 0; h < G; ++h) {
            double s = 0.0;
            for (int r = 0; r < dg; ++r)
                s += a[(int64_t)h * dg + r] * c[r];
            s *= gate_scale;
            if (s_head)
                s_head[(int64_t)h * nc + j] = s;
            mean += s;
        }
        S[j] = mean / G;
    }
    free(a);
    free(c);
    return 0;
}

/* ---------------------------------------------------------------- D4 ---- */
/* Token-budget selection (SeerAttention-R abstract: a fixed token budget at
 * 64- or 128-token block granularity): keep the k highest-scoring blocks,
 * equal scores ordered by the lower block index, output ascending. */
/* Stable merge sort of block ids by descending score: equal scores keep
 * their original (ascending id) order, which is the lower-index tie rule. */
static void stable_sort_desc(int32_t *ids, int32_t *tmp, int n, const double *S)
{
    if (n < 2)
        return;
    int h = n / 2;
    stable_sort_desc(ids, tmp, h, S);
    stable_sort_desc(ids + h, tmp, n - h, S);
    int a = 0, b = h, o = 0;
    while (a < h && b < n)
        tmp[o++] = (S[ids[b]] > S[ids[a]]) ? ids[b++] : ids[a++];
    while (a < h)
        tmp[o++] = ids[a++];
    while (b < n)
        tmp[o++] = ids[b++];
    memcpy(ids, tmp, sizeof(int32_t) * (size_t)n);
}

static int by_index(const void *pa, const void *pb)
{
    int32_t ia = *(const int32_t *)pa, ib = *(const int32_t *)pb;
    return (ia > ib) - (ia < ib);
}

int so_select_blocks(const double *S, int nc, int k, int32_t *idx)
{
    if (nc < 0 || k < 0 || (nc > 0 && !S) || (k > 0 && !idx))
        return -1;
    for (int j = 0; j < nc; ++j)
        if (isnan(S[j]))
            return -1;
    int n = k < nc ? k : nc;
    if (n == 0)
        return 0;
    int32_t *order = (int32_t *)malloc(sizeof(int32_t) * (size_t)nc);
    int32_t *tmp = (int32_t *)malloc(sizeof(int32_t) * (size_t)nc);
    if (!order || !tmp) {
        free(order);
        free(tmp);
        return -2;
    }
    for (int j = 0; j < nc; ++j)
        order[j] = j;
    stable_sort_desc(order, tmp, nc, S);
    memcpy(idx, order, sizeof(int32_t) * (size_t)n);
    qsort(idx, (size_t)n, sizeof(int32_t), by_index);
    free(tmp);
    free(order);
    return n;
}

/* ------------------------------------------------------------------ S1 --- */
int so_select_policy(const double *S, int nc, int policy, int k_max, int num, int den, double tau, int32_t *idx)
{
    if (nc < 0 || k_max < 0 || (nc > 0 && !S))
        return -1;
    int k;
    if (policy == 0) {
        k = nc;
    } else if (policy == 1) {
        if (num < 0 || den <= 0)
            return -1;
        k = (int)(((int64_t)nc * num + den - 1) / den);
    } else if (policy == 2) {
        if (isnan(tau))
            return -1;
        double m = -INFINITY, z = 0.0;
        for (int j = 0; j < nc; ++j)
            if (S[j] > m)
                m = S[j];
        for (int j = 0; j < nc; ++j)
            z += exp(S[j] - m);
        k = 0;
        for (int j = 0; j < nc; ++j)
            if (exp(S[j] - m) / z >= tau)
                ++k;
    } else {
        return -1;
    }
    if (k > nc)
        k = nc;
    if (k > k_max)
        k = k_max;
    return so_select_blocks(S, nc, k, idx);
}

/* ------------------------------------------------------------ D5 + D6 --- */
/* Scaled dot-product softmax attention of each query row over the token set
 * T = (kept complete blocks) + (incomplete tail).  The tail has no pooled key
 * yet, so it is never gated; it is always attended, as it holds the current
 * token.  Dropped blocks get zero weight (SeerAttention v2 abstract: the
 * unselected blocks are treated as sparse). */
int so_sparse_attention(const uint16_t *q, int64_t q_row_stride, int G, int d,
                        const uint16_t *k, const uint16_t *v, int64_t kv_row_stride,
                        int L, int bs, const int32_t *idx, int n_idx, double scale,
                        double *out, double *lse, double *w)
{
    if (!q || !out || !lse || G <= 0 || d <= 0 || bs <= 0 || L < 0 || n_idx < 0 ||
        (L > 0 && (!k || !v)) || (n_idx > 0 && !idx) || kv_row_stride < d)
        return -1;
    int nc = L / bs;
    for (int i = 0; i < n_idx; ++i)
        if (idx[i] < 0 || idx[i] >= nc || (i > 0 && idx[i] <= idx[i - 1]))
            return -1;

    /* D5: membership of every token of the context in T */
    unsigned char *in_t = (unsigned char *)calloc((size_t)(L > 0 ? L : 1), 1);
    double *z = (double *)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
    if (!in_t || !z) {
        free(in_t);
        free(z);
        return -2;
    }
    for (int i = 0; i < n_idx; ++i)
        for (int t = idx[i] * bs; t < (idx[i] + 1) * bs; ++t)
            in_t[t] = 1;
    for (int t = nc * bs; t < L; ++t)
        in_t[t] = 1;

    /* D6: z_t = scale * q.K_t ; w_t = exp(z_t - m) / sum ; o = sum_t w_t V_t */
    for (int h = 0; h < G; ++h) {
        const uint16_t *qh = q + h * q_row_stride;
        double m = -INFINITY;
        for (int t = 0; t < L; ++t) {
            if (!in_t[t])
                continue;
            double dot = 0.0;
            for (int c = 0; c < d; ++c)
                dot += so_bf16_to_f64(qh[c]) * so_bf16_to_f64(k[(int64_t)t * kv_row_stride + c]);
            z[t] = scale * dot;
            if (z[t] > m)
                m = z[t];
        }
        double *oh = out + (int64_t)h * d;
        for (int c = 0; c < d; ++c)
            oh[c] = 0.0;
        if (w)
            for (int t = 0; t < L; ++t)
                w[(int64_t)h * L + t] = 0.0;
        if (m == -INFINITY) { /* empty token set */
            lse[h] = -INFINITY;
            continue;
        }
        double denom = 0.0;
        for (int t = 0; t < L; ++t)
            if (in_t[t])
                denom += exp(z[t] - m);
        for (int t = 0; t < L; ++t) {
            if (!in_t[t])
                continue;
            double wt = exp(z[t] - m) / denom;
            if (w)
                w[(int64_t)h * L + t] = wt;
            for (int c = 0; c < d; ++c)
                oh[c] += wt * so_bf16_to_f64(v[(int64_t)t * kv_row_stride + c]);
        }
        lse[h] = m + log(denom);
    }
    free(in_t);
    free(z);
    return 0;
}

/* ---------------------------------------------------------- ground truth --- */
int so_decode_block_mass(const uint16_t *q, int64_t q_row_stride, int G, int d,
                         const uint16_t *k, const uint16_t *v, int64_t kv_row_stride,
                         int L, int bs, double scale, double *out, double *lse, double *mass)
{
    if (!mass || G <= 0 || bs <= 0 || L < 0)
        return -1;
    const int nc = L / bs;
    int32_t *all = (int32_t *)malloc(sizeof(int32_t) * (size_t)(nc > 0 ? nc : 1));
    double *w = (double *)malloc(sizeof(double) * (size_t)G * (size_t)(L > 0 ? L : 1));
    if (!all || !w) {
        free(all);
        free(w);
        return -2;
    }
    for (int j = 0; j < nc; ++j)
        all[j] = j;
    /* every complete block kept: T is the whole context */
    int rc = so_sparse_attention(q, q_row_stride, G, d, k, v, kv_row_stride, L, bs, all, nc, scale, out, lse, w);
    if (rc == 0) {
        for (int j = 0; j <= nc; ++j) {
            const int t0 = j * bs, t1 = j < nc ? (j + 1) * bs : L;
            double sum = 0.0;
            for (int h = 0; h < G; ++h)
                for (int t = t0; t < t1; ++t)
                    sum += w[(int64_t)h * L + t];
            mass[j] = sum / G;
        }
    }
    free(all);
    free(w);
    return rc;
}

/* ------------------------------------------------------ batched decode --- */
int so_pool_cache(const uint16_t *k, int64_t sk_b, int64_t sk_h, int64_t sk_t,
                  const int32_t *seqlens, int B, int Hkv, int d, int bs, int nb_max,
                  double *kpool)
{
    if (!k || !seqlens || !kpool || B <= 0 || Hkv <= 0 || d <= 0 || bs <= 0 || nb_max < 0)
        return -1;
    for (int b = 0; b < B; ++b)
        if (seqlens[b] < 0 || seqlens[b] / bs > nb_max)
            return -1;
    int bad = 0;
#pragma omp parallel for schedule(dynamic) reduction(| : bad)
    for (int p = 0; p < B * Hkv; ++p) {
        int b = p / Hkv, g = p % Hkv;
        double *dst = kpool + ((int64_t)b * Hkv + g) * nb_max * d;
        memset(dst, 0, sizeof(double) * (size_t)nb_max * d);
        bad |= so_pool_k(k + b * sk_b + g * sk_h, sk_t, seqlens[b], d, bs, dst) != 0;
    }
    return bad ? -1 : 0;
}

int so_decode_step(const uint16_t *q, int64_t sq_b, int64_t sq_h,
                   const uint16_t *k, const uint16_t *v, int64_t skv_b, int64_t skv_h, int64_t skv_t,
                   const int32_t *seqlens, int B, int Hq, int Hkv, int d, int bs, int budget,
                   const uint16_t *wq, const uint16_t *wk, int dg, double gate_scale,
                   const double *kpool, int nb_max, double softmax_scale,
                   double *scores, int32_t *idx, int32_t *n_sel, double *out, double *lse)
{
    if (!q || !k || !v || !seqlens || !wq || !wk || !kpool || !idx || !n_sel || !out || !lse ||
        B <= 0 || Hkv <= 0 || Hq <= 0 || Hq % Hkv || d <= 0 || bs <= 0 || budget < 0 || dg <= 0)
        return -1;
    for (int b = 0; b < B; ++b)
        if (seqlens[b] < 0 || seqlens[b] / bs > nb_max)
            return -1;
    int G = Hq / Hkv, kmax = budget / bs, bad = 0;
#pragma omp parallel for schedule(dynamic) reduction(| : bad)
    for (int p = 0; p < B * Hkv; ++p) {
        int b = p / Hkv, g = p % Hkv, L = seqlens[b], nc = L / bs;
        const uint16_t *qg = q + b * sq_b + (int64_t)g * G * sq_h;
        double *S = (double *)malloc(sizeof(double) * (size_t)(nc > 0 ? nc : 1));
        int32_t *sel = idx + ((int64_t)b * Hkv + g) * kmax;
        if (!S) {
            bad = 1;
            continue;
        }
        bad |= so_gate_scores(qg, sq_h, G, d, wq + (int64_t)g * dg * d, wk + (int64_t)g * dg * d, dg,
                              kpool + ((int64_t)b * Hkv + g) * nb_max * d, nc, gate_scale, NULL, S) != 0;
        if (scores)
            for (int j = 0; j < nb_max; ++j)
                scores[((int64_t)b * Hkv + g) * nb_max + j] = j < nc ? S[j] : -INFINITY;
        for (int i = 0; i < kmax; ++i)
            sel[i] = -1;
        int n = so_select_blocks(S, nc, kmax, sel);
        bad |= n < 0;
        n_sel[(int64_t)b * Hkv + g] = n < 0 ? 0 : n;
        if (n >= 0)
            bad |= so_sparse_attention(qg, sq_h, G, d, k + b * skv_b + g * skv_h, v + b * skv_b + g * skv_h,
                                       skv_t, L, bs, sel, n, softmax_scale,
                                       out + ((int64_t)b * Hq + (int64_t)g * G) * d,
                                       lse + (int64_t)b * Hq + (int64_t)g * G, NULL) != 0;
        free(S);
    }
    return bad ? -1 : 0;
}

/* ------------------------------------------------------------------ V1 --- */
int so_decode_step_per_head(const uint16_t *q, int64_t sq_b, int64_t sq_h,
                            const uint16_t *k, const uint16_t *v, int64_t skv_b, int64_t skv_h, int64_t skv_t,
                            const int32_t *seqlens, int B, int Hq, int Hkv, int d, int bs, int budget,
                            const uint16_t *wq, const uint16_t *wk, int dg, double gate_scale,
                            const double *kpool, int nb_max, double softmax_scale,
                            double *scores, int32_t *idx, int32_t *n_sel, double *out, double *lse)
{
    if (!q || !k || !v || !seqlens || !wq || !wk || !kpool || !idx || !n_sel || !out || !lse ||
        B <= 0 || Hkv <= 0 || Hq <= 0 || Hq % Hkv || d <= 0 || bs <= 0 || budget < 0 || dg <= 0)
        return -1;
    for (int b = 0; b < B; ++b)
        if (seqlens[b] < 0 || seqlens[b] / bs > nb_max)
            return -1;
    int G = Hq / Hkv, kmax = budget / bs, bad = 0;
#pragma omp parallel for schedule(dynamic) reduction(| : bad)
    for (int p = 0; p < B * Hkv; ++p) {
        int b = p / Hkv, g = p % Hkv, L = seqlens[b], nc = L / bs;
        const uint16_t *qg = q + b * sq_b + (int64_t)g * G * sq_h;
        double *sh = (double *)malloc(sizeof(double) * (size_t)G * (size_t)(nc > 0 ? nc : 1));
        double *S = (double *)malloc(sizeof(double) * (size_t)(nc > 0 ? nc : 1));
        if (!sh || !S) {
            free(sh);
            free(S);
            bad = 1;
            continue;
        }
        /* D2 per head (the group mean S is not used) */
        bad |= so_gate_scores(qg, sq_h, G, d, wq + (int64_t)g * dg * d, wk + (int64_t)g * dg * d, dg,
                              kpool + ((int64_t)b * Hkv + g) * nb_max * d, nc, gate_scale, sh, S) != 0;
        for (int h = 0; h < G; ++h) {
            const int64_t row = (int64_t)b * Hq + (int64_t)g * G + h;
            if (scores)
                for (int j = 0; j < nb_max; ++j)
                    scores[row * nb_max + j] = j < nc ? sh[(int64_t)h * nc + j] : -INFINITY;
            int32_t *sel = idx + row * kmax;
            for (int i = 0; i < kmax; ++i)
                sel[i] = -1;
            int n = so_select_blocks(sh + (int64_t)h * nc, nc, kmax, sel);
            bad |= n < 0;
            n_sel[row] = n < 0 ? 0 : n;
            if (n >= 0)
                bad |= so_sparse_attention(qg + h * sq_h, sq_h, 1, d, k + b * skv_b + g * skv_h,
                                           v + b * skv_b + g * skv_h, skv_t, L, bs, sel, n, softmax_scale,
                                           out + row * d, lse + row, NULL) != 0;
        }
        free(sh);
        free(S);
    }
    return bad ? -1 : 0;
}

/* ------------------------------------------------------------ prefill --- */
/* k_i = ceil((i + 1) * num / den) in integers, kept within [1, i + 1]. */
static int keep_count(int i, int keep_num, int keep_den)
{
    int64_t kk = ((int64_t)(i + 1) * keep_num + keep_den - 1) / keep_den;
    if (kk < 1) kk = 1;
    if (kk > i + 1) kk = i + 1;
    return (int)kk;
}

/* Mean over the rows of block j that exist (the last block may be partial). */
static void pool_block_rows(const uint16_t *x, int64_t row_stride, int L, int d, int bs, int j, double *dst)
{
    int t0 = j * bs, t1 = (j + 1) * bs < L ? (j + 1) * bs : L;
    for (int c = 0; c < d; ++c) {
        double sum = 0.0;
        for (int t = t0; t < t1; ++t)
            sum += so_bf16_to_f64(x[(int64_t)t * row_stride + c]);
        dst[c] = sum / (t1 - t0);
    }
}

/* SeerAttention v1 gate for prefill: pool Q and K per block, project each
 * through its linear layer, multiply into a block score matrix; causal rows
 * keep their diagonal block and their best earlier blocks. */
int so_prefill_gate(const uint16_t *q, const uint16_t *k, int64_t row_stride, int L, int d, int bs,
                    const uint16_t *wq, const uint16_t *wk, int dg, double gate_scale,
                    int keep_num, int keep_den, double *S, int32_t *kv_blocks, int32_t *kv_count,
                    int kmax_row)
{
    if (!q || !k || !wq || !wk || !kv_blocks || !kv_count || L <= 0 || d <= 0 || bs <= 0 || dg <= 0 ||
        keep_num < 0 || keep_den <= 0 || row_stride < d)
        return -1;
    int nb = (L + bs - 1) / bs;
    if (kmax_row < keep_count(nb - 1, keep_num, keep_den))
        return -1;
    double *qbar = (double *)malloc(sizeof(double) * (size_t)d);
    double *kbar = (double *)malloc(sizeof(double) * (size_t)d);
    double *a = (double *)malloc(sizeof(double) * (size_t)nb * dg);  /* Wq Qbar_i */
    double *c = (double *)malloc(sizeof(double) * (size_t)nb * dg);  /* Wk Kbar_j */
    double *row = (double *)malloc(sizeof(double) * (size_t)nb);
    int32_t *cand = (int32_t *)malloc(sizeof(int32_t) * (size_t)nb);
    int rc = 0;
    if (!qbar || !kbar || !a || !c || !row || !cand) {
        rc = -2;
        goto done;
    }
    for (int i = 0; i < nb; ++i) {                                   /* P1 + projections */
        pool_block_rows(q, row_stride, L, d, bs, i, qbar);
        pool_block_rows(k, row_stride, L, d, bs, i, kbar);
        for (int r = 0; r < dg; ++r) {
            double sa = 0.0, sc = 0.0;
            for (int e = 0; e < d; ++e) {
                sa += so_bf16_to_f64(wq[(int64_t)r * d + e]) * qbar[e];
                sc += so_bf16_to_f64(wk[(int64_t)r * d + e]) * kbar[e];
            }
            a[(int64_t)i * dg + r] = sa;
            c[(int64_t)i * dg + r] = sc;
        }
    }
    for (int i = 0; i < nb; ++i) {
        for (int j = 0; j < nb; ++j) {                               /* P2 */
            double s = -INFINITY;
            if (j <= i) {
                s = 0.0;
                for (int r = 0; r < dg; ++r)
                    s += a[(int64_t)i * dg + r] * c[(int64_t)j * dg + r];
                s *= gate_scale;
            }
            row[j] = s;
            if (S)
                S[(int64_t)i * nb + j] = s;
        }
        int ki = keep_count(i, keep_num, keep_den);                 /* P3 */
        int32_t *dst = kv_blocks + (int64_t)i * kmax_row;
        for (int m = 0; m < kmax_row; ++m)
            dst[m] = -1;
        int n = so_select_blocks(row, i, ki - 1, cand);              /* best of j < i */
        if (n < 0) {
            rc = -1;
            goto done;
        }
        for (int m = 0; m < n; ++m)
            dst[m] = cand[m];
        dst[n] = i;                                                  /* diagonal, largest id */
        kv_count[i] = n + 1;
    }
done:
    free(qbar);
    free(kbar);
    free(a);
    free(c);
    free(row);
    free(cand);
    return rc;
}

/* Causal attention of query token t (in block i) over keys t' <= t that lie
 * in the kept blocks of row i; scale 1/sqrt(d) unless given otherwise. */
int so_prefill_attention(const uint16_t *q, const uint16_t *k, const uint16_t *v, int64_t row_stride,
                         int L, int d, int bs, const int32_t *kv_blocks, const int32_t *kv_count,
                         int kmax_row, double scale, int t_lo, int t_hi, double *out, double *lse)
{
    if (!q || !k || !v || !kv_blocks || !kv_count || !out || !lse || L <= 0 || d <= 0 || bs <= 0 ||
        t_lo < 0 || t_hi > L || t_lo > t_hi || row_stride < d)
        return -1;
    double *z = (double *)malloc(sizeof(double) * (size_t)L);
    unsigned char *in_row = (unsigned char *)malloc((size_t)L);
    if (!z || !in_row) {
        free(z);
        free(in_row);
        return -2;
    }
    int rc = 0, cur_row = -1;
    for (int t = t_lo; t < t_hi; ++t) {
        int i = t / bs;
        if (i != cur_row) {
            memset(in_row, 0, (size_t)L);
            if (kv_count[i] < 1 || kv_count[i] > kmax_row) {
                rc = -1;
                break;
            }
            for (int m = 0; m < kv_count[i]; ++m) {
                int j = kv_blocks[(int64_t)i * kmax_row + m];
                if (j < 0 || j > i) {
                    rc = -1;
                    break;
                }
                for (int tt = j * bs; tt < (j + 1) * bs && tt < L; ++tt)
                    in_row[tt] = 1;
            }
            if (rc)
                break;
            cur_row = i;
        }
        const uint16_t *qt = q + (int64_t)t * row_stride;
        double m = -INFINITY;
        for (int tt = 0; tt <= t; ++tt) {
            if (!in_row[tt])
                continue;
            double dot = 0.0;
            for (int c = 0; c < d; ++c)
                dot += so_bf16_to_f64(qt[c]) * so_bf16_to_f64(k[(int64_t)tt * row_stride + c]);
            z[tt] = scale * dot;
            if (z[tt] > m)
                m = z[tt];
        }
        double *ot = out + (int64_t)(t - t_lo) * d;
        for (int c = 0; c < d; ++c)
            ot[c] = 0.0;
        if (m == -INFINITY) {
            lse[t - t_lo] = -INFINITY;
            continue;
        }
        double denom = 0.0;
        for (int tt = 0; tt <= t; ++tt)
            if (in_row[tt])
                denom += exp(z[tt] - m);
        for (int tt = 0; tt <= t; ++tt) {
            if (!in_row[tt])
                continue;
            double wt = exp(z[tt] - m) / denom;
            for (int c = 0; c < d; ++c)
                ot[c] += wt * so_bf16_to_f64(v[(int64_t)tt * row_stride + c]);
        }
        lse[t - t_lo] = m + log(denom);
    }
    free(z);
    free(in_row);
    return rc;
}

int so_prefill(const uint16_t *q, const uint16_t *k, const uint16_t *v, int B, int H, int L, int d,
               int bs, const uint16_t *wq, const uint16_t *wk, int dg, double gate_scale,
               int keep_num, int keep_den, int32_t *kv_blocks, int32_t *kv_count, int kmax_row,
               double scale, int t_lo, int t_hi, double *out, double *lse)
{
    if (B <= 0 || H <= 0 || L <= 0 || bs <= 0 || t_lo < 0 || t_hi > L || t_lo > t_hi)
        return -1;
    int nb = (L + bs - 1) / bs, nt = t_hi - t_lo, bad = 0;
    int64_t head = (int64_t)L * d;
#pragma omp parallel for schedule(dynamic) reduction(| : bad)
    for (int p = 0; p < B * H; ++p) {
        int h = p % H;
        int32_t *blk = kv_blocks + (int64_t)p * nb * kmax_row;
        int32_t *cnt = kv_count + (int64_t)p * nb;
        bad |= so_prefill_gate(q + p * head, k + p * head, d, L, d, bs, wq + (int64_t)h * dg * d,
                               wk + (int64_t)h * dg * d, dg, gate_scale, keep_num, keep_den, NULL,
                               blk, cnt, kmax_row) != 0;
        if (!bad)
            bad |= so_prefill_attention(q + p * head, k + p * head, v + p * head, d, L, d, bs, blk, cnt,
                                        kmax_row, scale, t_lo, t_hi, out + (int64_t)p * nt * d,
                                        lse + (int64_t)p * nt) != 0;
    }
    return bad ? -1 : 0;
}

/* ---------------------------------------------------------------- G2 --- */
int so_prefill_block_mass(const uint16_t *q, const uint16_t *k, int64_t row_stride, int L, int d, int bs,
                          double scale, int i_lo, int i_hi, double *mass)
{
    const int nb = L > 0 && bs > 0 ? (L + bs - 1) / bs : 0;
    if (!q || !k || !mass || L <= 0 || d <= 0 || bs <= 0 || row_stride < d || i_lo < 0 || i_hi > nb ||
        i_lo > i_hi)
        return -1;
    double *z = (double *)malloc(sizeof(double) * (size_t)L);
    if (!z)
        return -2;
    for (int i = i_lo; i < i_hi; ++i) {
        double *row = mass + (int64_t)(i - i_lo) * nb;
        for (int j = 0; j < nb; ++j)
            row[j] = 0.0;
        const int t0 = i * bs, t1 = (i + 1) * bs < L ? (i + 1) * bs : L;
        for (int t = t0; t < t1; ++t) {
            /* dense causal softmax of row t over tokens 0..t */
            double m = -INFINITY;
            for (int tt = 0; tt <= t; ++tt) {
                double dot = 0.0;
                for (int c = 0; c < d; ++c)
                    dot += so_bf16_to_f64(q[(int64_t)t * row_stride + c]) *
                           so_bf16_to_f64(k[(int64_t)tt * row_stride + c]);
                z[tt] = scale * dot;
                if (z[tt] > m)
                    m = z[tt];
            }
            double denom = 0.0;
            for (int tt = 0; tt <= t; ++tt)
                denom += exp(z[tt] - m);
            for (int tt = 0; tt <= t; ++tt)
                row[tt / bs] += exp(z[tt] - m) / denom / (t1 - t0);
        }
    }
    free(z);
    return 0;
}
