/*
 * pma_oracle.c -- plain CPU reference for packed multi-head attention over
 * live edges, in double precision.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the bench's
 * CPU-baseline leg load this file's library. It shares no code with the GPU
 * library: no kernels, headers, helpers or tables.
 *
 * It follows the "Notes" of the kpnn2 PackedMultiheadAttention page (one
 * forward pass, for one sample and one head), step by step:
 *   1. project every token with the four nn.Linear maps (y = x W^T + b, W
 *      stored [out][in]), each split into num_heads contiguous slices of
 *      d = E / H channels;
 *   2. score each live edge e from source s to target t:
 *      score[e] = dot(q[t], k[s]) / sqrt(d);
 *   3. softmax over the edges into each target only (eval mode: no dropout);
 *   4. mixed[t] = sum over the edges e into t of weight[e] * v[s];
 *   5. join the heads' slices and apply out_proj.
 * A target with no live edge mixes to zeros, so its output is the out_proj
 * bias (same page, Notes, on queries with no live keys).
 *
 * key_padding_mask (same page, forward parameter table and Notes step 3):
 * for sample b, a key s with mask[b][s] set takes no part; the edges from it
 * drop out of that sample's softmax (weight 0), and a target left with no
 * edge mixes to zeros as above.
 *
 * Every computed row is independent, so rows may be computed in parallel
 * (OpenMP); each row's arithmetic is sequential in edge order.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* nn.Linear on one row: y[o] = sum_i x[i] * w[o][i] + b[o]  (b may be NULL). */
static void linear_row(int64_t E, const double *x, const double *w, const double *b, double *y)
{
    for (int64_t o = 0; o < E; ++o) {
        double acc = 0.0;
        for (int64_t i = 0; i < E; ++i)
            acc += x[i] * w[o * E + i];
        y[o] = acc + (b ? b[o] : 0.0);
    }
}

int oracle_num_threads(int nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0)
        return nthreads;
    return omp_get_max_threads();
#else
    (void)nthreads;
    return 1;
#endif
}

/*
 * Forward pass for the requested (sample, target) rows.
 *
 *   xq (B, L, E), xk (B, S, E), xv (B, S, E): tokens, row-major, double.
 *   w* (E, E) [out][in]; b* (E) or NULL (all four NULL <=> bias=False).
 *   src, tgt (nnz): the final live edges (given pairs, then any appended
 *     self-loops); their position is the edge id.
 *   rows: nrows pairs (row_b[i], row_t[i]); all rows when row_b == NULL
 *     (then nrows must be B * L, in order b-major).
 *   out (nrows, E): the layer output at each requested row.
 *   mixed (nrows, E) or NULL: the joined heads before out_proj.
 *   weights (B, nnz, H) or NULL: per-head softmax weight of every edge into a
 *     requested row; entries of other edges are left untouched.
 *   kpm: NULL, or key_padding_mask bytes, sample b's at kpm + b * kpm_bstride
 *     (kpm_bstride = 0: one mask for every sample), S per sample; nonzero
 *     means the key is left out.
 *
 * Returns 0, or -1 when memory runs out.
 */
int oracle_forward(int64_t B, int64_t L, int64_t S, int64_t E, int64_t H,
                   const double *xq, const double *xk, const double *xv,
                   const double *wq, const double *bq, const double *wk, const double *bk,
                   const double *wv, const double *bv, const double *wo, const double *bo,
                   int64_t nnz, const int64_t *src, const int64_t *tgt,
                   int64_t nrows, const int64_t *row_b, const int64_t *row_t,
                   double *out, double *mixed, double *weights,
                   const unsigned char *kpm, int64_t kpm_bstride, int nthreads)
{
    const int64_t d = E / H;
    const double sqrt_d = sqrt((double)d);
    int rc = -1;

    /* The edges into each target, in edge-id order: the set each softmax
       runs over. first[t] .. first[t+1] indexes into into_t[]. */
    int64_t *first = calloc((size_t)L + 1, sizeof(int64_t));
    int64_t *into_t = malloc((size_t)(nnz > 0 ? nnz : 1) * sizeof(int64_t));
    int64_t *fill = calloc((size_t)L + 1, sizeof(int64_t));
    unsigned char *need = calloc((size_t)(B * S > 0 ? B * S : 1), 1);
    double *K = malloc((size_t)(B * S * E > 0 ? B * S * E : 1) * sizeof(double));
    double *V = malloc((size_t)(B * S * E > 0 ? B * S * E : 1) * sizeof(double));
    if (!first || !into_t || !fill || !need || !K || !V)
        goto done;

    for (int64_t e = 0; e < nnz; ++e)
        first[tgt[e] + 1] += 1;
    for (int64_t t = 0; t < L; ++t)
        first[t + 1] += first[t];
    for (int64_t e = 0; e < nnz; ++e) {
        int64_t t = tgt[e];
        into_t[first[t] + fill[t]++] = e;
    }

    /* Which key/value rows the requested rows read. */
    for (int64_t i = 0; i < nrows; ++i) {
        int64_t b = row_b ? row_b[i] : i / L;
        int64_t t = row_b ? row_t[i] : i % L;
        for (int64_t j = first[t]; j < first[t + 1]; ++j)
            need[b * S + src[into_t[j]]] = 1;
    }

    /* Step 1 for keys and values. */
#pragma omp parallel for schedule(dynamic, 64) num_threads(oracle_num_threads(nthreads))
    for (int64_t bs = 0; bs < B * S; ++bs) {
        if (!need[bs])
            continue;
        linear_row(E, xk + bs * E, wk, bk, K + bs * E);
        linear_row(E, xv + bs * E, wv, bv, V + bs * E);
    }

    int failed = 0;
#pragma omp parallel num_threads(oracle_num_threads(nthreads))
    {
        double *q = malloc((size_t)E * sizeof(double));
        double *mix = malloc((size_t)E * sizeof(double));
        int64_t cap = 0;
        double *score = NULL, *w = NULL;
        if (!q || !mix)
            failed = 1;
#pragma omp for schedule(dynamic, 16)
        for (int64_t i = 0; i < nrows; ++i) {
            if (failed)
                continue;
            int64_t b = row_b ? row_b[i] : i / L;
            int64_t t = row_b ? row_t[i] : i % L;
            int64_t deg = first[t + 1] - first[t];
            if (deg > cap) {
                free(score);
                free(w);
                cap = deg;
                score = malloc((size_t)cap * sizeof(double));
                w = malloc((size_t)cap * sizeof(double));
                if (!score || !w) {
                    failed = 1;
                    cap = 0;
                    continue;
                }
            }
            /* Step 1 for the query. */
            linear_row(E, xq + (b * L + t) * E, wq, bq, q);
            for (int64_t h = 0; h < H; ++h) {
                const double *qh = q + h * d;
                /* Step 2: one score per live edge into t (left out: keys that
                   the mask drops for this sample). */
                int64_t live = 0;
                for (int64_t j = 0; j < deg; ++j) {
                    const int64_t s = src[into_t[first[t] + j]];
                    if (kpm && kpm[b * kpm_bstride + s]) {
                        score[j] = -INFINITY;
                        continue;
                    }
                    ++live;
                    const double *kh = K + (b * S + s) * E + h * d;
                    double dot = 0.0;
                    for (int64_t c = 0; c < d; ++c)
                        dot += qh[c] * kh[c];
                    score[j] = dot / sqrt_d;
                }
                /* Step 3: softmax over those edges only. */
                double m = -INFINITY;
                for (int64_t j = 0; j < deg; ++j)
                    if (score[j] > m)
                        m = score[j];
                double den = 0.0;
                for (int64_t j = 0; j < deg; ++j)
                    if (score[j] != -INFINITY)
                        den += exp(score[j] - m);
                for (int64_t j = 0; j < deg; ++j)
                    w[j] = (live > 0 && score[j] != -INFINITY) ? exp(score[j] - m) / den : 0.0;
                /* Step 4: mix the sources' values (zeros with no edge). */
                for (int64_t c = 0; c < d; ++c) {
                    double acc = 0.0;
                    for (int64_t j = 0; j < deg; ++j)
                        if (w[j] != 0.0)
                            acc += w[j] * V[(b * S + src[into_t[first[t] + j]]) * E + h * d + c];
                    mix[h * d + c] = acc;
                }
                if (weights)
                    for (int64_t j = 0; j < deg; ++j)
                        weights[(b * nnz + into_t[first[t] + j]) * H + h] = w[j];
            }
            /* Step 5: the heads' slices are already joined in mix; out_proj. */
            linear_row(E, mix, wo, bo, out + i * E);
            if (mixed)
                memcpy(mixed + i * E, mix, (size_t)E * sizeof(double));
        }
        free(q);
        free(mix);
        free(score);
        free(w);
    }
    rc = failed ? -1 : 0;

done:
    free(first);
    free(into_t);
    free(fill);
    free(need);
    free(K);
    free(V);
    return rc;
}
