/*
 * Draft-correction oracle: a plain, slow, obviously correct CPU implementation
 * of one corrector pass over a batch of draft blocks.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header or constant with the GPU library and never calls it.
 *
 * What it computes, in the order and notation of the DCOCO page ("Contextual
 * Correction of Parallel Drafts for Speculative Decoding", method details,
 * steps (1)-(5)):
 *   (1) per drafted slot, the top-K candidate ids and their drafter logits l;
 *   (2) b = LN(W_cand E[c]) and g = LN(W_ctx h) with a non-affine LayerNorm,
 *       z = LN_{gamma,beta}(W_fuse [b; g]) of width r;
 *   (3) pair state s_p = W_pair [h_p; h_{p+1}], once per adjacent slot pair;
 *   (4) S_p(a,b) = l_{p+1}(b) + Delta([s_p; z_p^a; z_{p+1}^b; l_p(a); l_{p+1}(b)]),
 *       Delta a two-layer GELU MLP (3r+2) -> h -> 1;
 *   (5) the prefix-first walk: slot 1 takes the drafter argmax, then
 *       k_{p+1} = argmax_b S_p(k_p, b).
 * The Global-Sum path rule (LiLiCorr, appendix E, Eq. 12) replaces (5) by the
 * path with the largest summed transition score, by dynamic programming; a
 * narrow beam search over the same score is a further rule.
 * The cosine variant (LiLiCorr, section 3.2, Eq. 1) replaces (3)-(4) by
 *   S_p(a,b) = l_{p+1}(b) + sigma * cos(W_out z_p^a, W_in z_{p+1}^b).
 * Beside step (1), the log-normaliser of each slot row over the whole
 * vocabulary (LiLiCorr appendix A), from which the candidates' log-probs and
 * confidence scalars follow.
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *   - top-K order is value descending, ties to the lowest token id; values
 *     compare numerically (-0 == +0, -inf sorts last); NaN is rejected;
 *   - the walk breaks ties to the lowest candidate index;
 *   - the Global-Sum path keeps slot 1 at rank 0 like the walk, and breaks
 *     ties to the lowest predecessor index in the sweep and the lowest
 *     candidate index in the last slot;
 *   - LayerNorm uses the biased variance over the r features and eps from the
 *     descriptor; GELU is the exact erf form;
 *   - the cosine normalises v / max(|v|, 1e-12).
 *
 * Precision: every input is read from its stored bits (bfloat16 widened
 * exactly, or float32); all arithmetic is double precision, with dot products
 * accumulated in index order.  Every function here is pinned by the CPU test
 * suite to something other than itself (brute force, closed forms, special
 * cases, hand-worked examples).  One rule is a reading rather than a formula
 * of the pages: the Geometric path (a lambda^p-discounted sum, named by the
 * DCOCO page's path-rule table without a formula) is pinned to that reading,
 * but whether the reading is the page's rule is parity unpinned.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORA_OK = 0, ORA_E_ARG = 1, ORA_E_NAN = 2, ORA_E_NOMEM = 3 };
enum { ORA_MLP = 0, ORA_COSINE = 1 };
enum { ORA_BF16 = 0, ORA_F32 = 1 };

typedef struct {
    int64_t V;
    int32_t B, K, d, de, r, h, dvec, variant, logits_dtype;
    double eps, sigma;
    int32_t top_m;   /* successors scored per predecessor (0: all K) */
} oracle_desc;

/* Matrices are bfloat16 bit patterns, row-major [out][in]; vectors are float32. */
typedef struct {
    const uint16_t *embed, *w_cand, *w_ctx, *w_fuse, *w_pair, *w1, *w_out, *w_in;
    const float *gamma, *beta, *b1, *w2, *b2;
} oracle_weights;

static double bf(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double logit_at(const void *row, int dtype, int64_t v)
{
    if (dtype == ORA_BF16) return bf(((const uint16_t *)row)[v]);
    return (double)((const float *)row)[v];
}

void oracle_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int oracle_get_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Number of trainable parameters the MLP corrector reads, from the shapes of
 * the arrays this file indexes below. */
int64_t oracle_param_count(const oracle_desc *D)
{
    int64_t r = D->r, d = D->d, de = D->de, h = D->h;
    int64_t n = 0;
    n += r * de;          /* W_cand */
    n += r * d;           /* W_ctx */
    n += r * (2 * r);     /* W_fuse */
    n += r * (2 * d);     /* W_pair */
    n += r + r;           /* LN gamma, beta */
    n += h * (3 * r + 2); /* MLP layer 1 */
    n += h;               /* b1 */
    n += h;               /* w2 */
    n += 1;               /* b2 */
    return n;
}

/* ---------------------------------------------------------------- top-K -- */

typedef struct {
    double v;
    int32_t id;
} cand_t;

/* Value descending, then token id ascending: a total order on distinct ids,
 * so a full sort gives the same result as a stable sort by value. */
static int cand_cmp(const void *pa, const void *pb)
{
    const cand_t *a = (const cand_t *)pa, *b = (const cand_t *)pb;
    if (a->v > b->v) return -1;
    if (a->v < b->v) return 1;
    return (a->id > b->id) - (a->id < b->id);
}

/* Step (1): the K largest logits of one slot row, full sort of the row. */
int oracle_topk_row(const void *row, int dtype, int64_t V, int32_t K,
                    int32_t *ids, double *vals)
{
    if (!row || !ids || !vals || V <= 0 || K <= 0 || K > V) return ORA_E_ARG;
    cand_t *c = (cand_t *)malloc(sizeof(cand_t) * (size_t)V);
    if (!c) return ORA_E_NOMEM;
    for (int64_t v = 0; v < V; ++v) {
        double x = logit_at(row, dtype, v);
        if (isnan(x)) {
            free(c);
            return ORA_E_NAN;
        }
        c[v].v = x;
        c[v].id = (int32_t)v;
    }
    qsort(c, (size_t)V, sizeof(cand_t), cand_cmp);
    for (int32_t k = 0; k < K; ++k) {
        ids[k] = c[k].id;
        vals[k] = c[k].v;
    }
    free(c);
    return ORA_OK;
}

/* Top-K of every drafted slot of n blocks.  Row (i, s) starts at
 * logits + i*req_stride + s*slot_stride elements (the caller skips the anchor).
 * ids/vals are [n][B][K]. */
int oracle_topk(const oracle_desc *D, int32_t n, const void *logits,
                int64_t req_stride, int64_t slot_stride, int32_t *ids, double *vals)
{
    if (!D || !logits || !ids || !vals || n < 0) return ORA_E_ARG;
    const size_t esz = D->logits_dtype == ORA_BF16 ? 2 : 4;
    int err = ORA_OK;
#pragma omp parallel for schedule(dynamic) reduction(| : err)
    for (int64_t t = 0; t < (int64_t)n * D->B; ++t) {
        int64_t i = t / D->B, s = t % D->B;
        const char *row = (const char *)logits + (size_t)(i * req_stride + s * slot_stride) * esz;
        err |= oracle_topk_row(row, D->logits_dtype, D->V, D->K,
                               ids + t * D->K, vals + t * D->K);
    }
    return err;
}

/* ------------------------------------------- vocabulary normalisation -- */

/* LiLiCorr appendix A (Architecture; Serving): the drafter's distribution at a
 * slot is the softmax of its logits over the whole vocabulary, so every
 * log-probability needs the row's log-normaliser log Z = log sum_v exp(l_v).
 * It is computed as m + log sum_v exp(l_v - m) with m the row maximum (the
 * same quantity, free of overflow), summing in index order.  A row of -inf
 * gives -inf.  NaN and +inf logits are rejected (ORA_E_NAN). */
int oracle_log_normaliser_row(const void *row, int dtype, int64_t V, double *logz)
{
    if (!row || !logz || V <= 0) return ORA_E_ARG;
    double m = -INFINITY;
    for (int64_t v = 0; v < V; ++v) {
        double x = logit_at(row, dtype, v);
        if (isnan(x) || x == INFINITY) return ORA_E_NAN;
        if (x > m) m = x;
    }
    if (m == -INFINITY) {
        *logz = -INFINITY;
        return ORA_OK;
    }
    double sum = 0.0;
    for (int64_t v = 0; v < V; ++v) sum += exp(logit_at(row, dtype, v) - m);
    *logz = m + log(sum);
    return ORA_OK;
}

/* The log-normaliser of every drafted slot row of n blocks, rows addressed as
 * in oracle_topk; logz is [n][B]. */
int oracle_log_normaliser(const oracle_desc *D, int32_t n, const void *logits,
                          int64_t req_stride, int64_t slot_stride, double *logz)
{
    if (!D || !logits || !logz || n < 0) return ORA_E_ARG;
    const size_t esz = D->logits_dtype == ORA_BF16 ? 2 : 4;
    int err = ORA_OK;
#pragma omp parallel for schedule(dynamic) reduction(| : err)
    for (int64_t t = 0; t < (int64_t)n * D->B; ++t) {
        int64_t i = t / D->B, s = t % D->B;
        const char *row = (const char *)logits + (size_t)(i * req_stride + s * slot_stride) * esz;
        err |= oracle_log_normaliser_row(row, D->logits_dtype, D->V, logz + t);
    }
    return err;
}

/* ------------------------------------------------------- dense helpers -- */

/* y[o] = sum_i W[o][i] x[i] for a bfloat16 matrix with row stride ld. */
static void matvec_bf(const uint16_t *W, int64_t ld, int rows, int cols,
                      const double *x, double *y)
{
    for (int o = 0; o < rows; ++o) {
        double acc = 0.0;
        const uint16_t *w = W + (size_t)o * ld;
        for (int i = 0; i < cols; ++i) acc += bf(w[i]) * x[i];
        y[o] = acc;
    }
}

/* LayerNorm over m features: (x - mean) / sqrt(var + eps), biased variance;
 * then gamma * . + beta when gamma is given. */
void oracle_layernorm(double *x, int m, double eps, const float *gamma, const float *beta)
{
    double mean = 0.0, var = 0.0;
    for (int i = 0; i < m; ++i) mean += x[i];
    mean /= m;
    for (int i = 0; i < m; ++i) var += (x[i] - mean) * (x[i] - mean);
    var /= m;
    double inv = 1.0 / sqrt(var + eps);
    for (int i = 0; i < m; ++i) {
        double y = (x[i] - mean) * inv;
        if (gamma) y = (double)gamma[i] * y + (double)beta[i];
        x[i] = y;
    }
}

/* GELU(t) = t * Phi(t) = 0.5 t (1 + erf(t / sqrt 2)). */
double oracle_gelu(double t)
{
    return 0.5 * t * (1.0 + erf(t / sqrt(2.0)));
}

/* ------------------------------------------------ steps (2) and (3) -- */

/* For every block i and drafted slot s (0-based; slot s is the page's slot s+1):
 *   b[i][s][k] = LN(W_cand E[ids[i][s][k]])            [n][B][K][r]
 *   g[i][s]    = LN(W_ctx h_s)                          [n][B][r]
 *   z[i][s][k] = gamma * LN(W_fuse [b; g]) + beta       [n][B][K][r]
 *   s[i][p]    = W_pair [h_p; h_{p+1}], p = 0..B-2      [n][B-1][r]
 * Hidden row (i, s) starts at hidden + i*h_req_stride + s*h_slot_stride.
 * Any output pointer may be NULL. */
int oracle_represent(const oracle_desc *D, const oracle_weights *W, int32_t n,
                     const int32_t *ids, const uint16_t *hidden,
                     int64_t h_req_stride, int64_t h_slot_stride,
                     double *b_out, double *g_out, double *z_out, double *s_out)
{
    if (!D || !W || !ids || !hidden || n < 0) return ORA_E_ARG;
    const int B = D->B, K = D->K, r = D->r, d = D->d, de = D->de;
    int err = ORA_OK;
#pragma omp parallel for schedule(dynamic) reduction(| : err)
    for (int64_t t = 0; t < (int64_t)n * B; ++t) {
        int64_t i = t / B, s = t % B;
        double *x = (double *)malloc(sizeof(double) * (size_t)(2 * (d > de ? d : de) + 3 * r));
        if (!x) {
            err |= ORA_E_NOMEM;
            continue;
        }
        double *hx = x;                         /* [h_s; h_{s+1}], later E[c] */
        double *bg = x + 2 * (d > de ? d : de); /* [b; g] */
        double *u = bg + 2 * r;                 /* W_fuse [b; g], then z */

        const uint16_t *hs = hidden + (size_t)(i * h_req_stride + s * h_slot_stride);
        for (int j = 0; j < d; ++j) hx[j] = bf(hs[j]);

        /* g = LN(W_ctx h) */
        double *g = bg + r;
        matvec_bf(W->w_ctx, d, r, d, hx, g);
        oracle_layernorm(g, r, D->eps, NULL, NULL);
        if (g_out)
            for (int j = 0; j < r; ++j) g_out[(size_t)t * r + j] = g[j];

        /* s_p = W_pair [h_p; h_{p+1}] for the pair that starts at this slot */
        if (s + 1 < B && s_out) {
            const uint16_t *hn = hs + h_slot_stride;
            for (int j = 0; j < d; ++j) hx[d + j] = bf(hn[j]);
            double *sp = s_out + ((size_t)i * (B - 1) + s) * r;
            matvec_bf(W->w_pair, 2 * (int64_t)d, r, 2 * d, hx, sp);
        }

        for (int k = 0; k < K; ++k) {
            int32_t tok = ids[t * K + k];
            if (tok < 0 || tok >= D->V) {
                err |= ORA_E_ARG;
                break;
            }
            const uint16_t *e = W->embed + (size_t)tok * de;
            for (int j = 0; j < de; ++j) hx[j] = bf(e[j]);
            /* b = LN(W_cand e) */
            double *b = bg;
            matvec_bf(W->w_cand, de, r, de, hx, b);
            oracle_layernorm(b, r, D->eps, NULL, NULL);
            if (b_out)
                for (int j = 0; j < r; ++j) b_out[((size_t)t * K + k) * r + j] = b[j];
            /* z = LN_{gamma,beta}(W_fuse [b; g]) */
            matvec_bf(W->w_fuse, 2 * r, r, 2 * r, bg, u);
            oracle_layernorm(u, r, D->eps, W->gamma, W->beta);
            if (z_out)
                for (int j = 0; j < r; ++j) z_out[((size_t)t * K + k) * r + j] = u[j];
        }
        free(x);
    }
    return err;
}

/* ---------------------------------------------------------- step (4) -- */

/* Transition scores for every block i, pair p = 0..B-2 (slots p and p+1),
 * predecessor candidate a and successor candidate b:
 *   MLP:    delta = w2 . GELU(W1 x + b1) + b2,
 *           x = [s_p; z_p^a; z_{p+1}^b; l_p(a); l_{p+1}(b)]
 *   COSINE: delta = sigma * <o_p^a, i_{p+1}^b>, o = unit(W_out z), i = unit(W_in z)
 *   S = l_{p+1}(b) + delta.
 * vals [n][B][K], z [n][B][K][r], s [n][B-1][r] (MLP only);
 * delta and scores are [n][B-1][K][K] indexed [i][p][a][b]; either may be NULL. */
int oracle_score(const oracle_desc *D, const oracle_weights *W, int32_t n,
                 const double *vals, const double *z, const double *s,
                 double *delta_out, double *scores_out)
{
    if (!D || !W || !vals || !z || n < 0) return ORA_E_ARG;
    const int B = D->B, K = D->K, r = D->r, h = D->h, dv = D->dvec;
    if (D->variant == ORA_MLP && !s) return ORA_E_ARG;
    const int nin = 3 * r + 2;
    /* Top-m successor sparsification (the DCOCO page's critique, weakness 3:
     * keep only the top-m successors of each predecessor, O(B K m) instead of
     * O(B K^2)).  The successors kept are the first m of the next slot's
     * top-K, i.e. ranked by the drafter; the others are not scored and get
     * S = Delta = -inf, so no path rule can choose them. */
    const int mk = (D->top_m > 0 && D->top_m < K) ? D->top_m : K;
    int err = ORA_OK;
#pragma omp parallel for schedule(dynamic) reduction(| : err)
    for (int64_t t = 0; t < (int64_t)n * (B - 1); ++t) {
        int64_t i = t / (B - 1), p = t % (B - 1);
        const double *zp = z + ((size_t)i * B + p) * K * r;
        const double *zq = z + ((size_t)i * B + p + 1) * K * r;
        const double *lp = vals + ((size_t)i * B + p) * K;
        const double *lq = vals + ((size_t)i * B + p + 1) * K;
        double *buf = (double *)malloc(sizeof(double) * (size_t)(nin + h + 2 * K * (dv > 0 ? dv : 1)));
        if (!buf) {
            err |= ORA_E_NOMEM;
            continue;
        }
        double *x = buf, *u = buf + nin;
        double *ov = u + h, *iv = ov + (size_t)K * (dv > 0 ? dv : 1);
        if (D->variant == ORA_COSINE) {
            for (int k = 0; k < K; ++k) {
                matvec_bf(W->w_out, r, dv, r, zp + (size_t)k * r, ov + (size_t)k * dv);
                matvec_bf(W->w_in, r, dv, r, zq + (size_t)k * r, iv + (size_t)k * dv);
                double no = 0.0, ni = 0.0;
                for (int j = 0; j < dv; ++j) {
                    no += ov[(size_t)k * dv + j] * ov[(size_t)k * dv + j];
                    ni += iv[(size_t)k * dv + j] * iv[(size_t)k * dv + j];
                }
                no = fmax(sqrt(no), 1e-12);
                ni = fmax(sqrt(ni), 1e-12);
                for (int j = 0; j < dv; ++j) {
                    ov[(size_t)k * dv + j] /= no;
                    iv[(size_t)k * dv + j] /= ni;
                }
            }
        }
        for (int a = 0; a < K; ++a) {
            for (int b = 0; b < K; ++b) {
                double delta;
                if (b >= mk) {
                    size_t o = (((size_t)i * (B - 1) + p) * K + a) * K + b;
                    if (delta_out) delta_out[o] = -INFINITY;
                    if (scores_out) scores_out[o] = -INFINITY;
                    continue;
                }
                if (D->variant == ORA_MLP) {
                    const double *sp = s + ((size_t)i * (B - 1) + p) * r;
                    for (int j = 0; j < r; ++j) x[j] = sp[j];
                    for (int j = 0; j < r; ++j) x[r + j] = zp[(size_t)a * r + j];
                    for (int j = 0; j < r; ++j) x[2 * r + j] = zq[(size_t)b * r + j];
                    x[3 * r] = lp[a];
                    x[3 * r + 1] = lq[b];
                    matvec_bf(W->w1, nin, h, nin, x, u);
                    delta = 0.0;
                    for (int j = 0; j < h; ++j)
                        delta += (double)W->w2[j] * oracle_gelu(u[j] + (double)W->b1[j]);
                    delta += (double)W->b2[0];
                } else {
                    double c = 0.0;
                    for (int j = 0; j < dv; ++j) c += ov[(size_t)a * dv + j] * iv[(size_t)b * dv + j];
                    delta = D->sigma * c;
                }
                size_t o = (((size_t)i * (B - 1) + p) * K + a) * K + b;
                if (delta_out) delta_out[o] = delta;
                if (scores_out) scores_out[o] = lq[b] + delta;
            }
        }
        free(buf);
    }
    return err;
}

/* ---------------------------------------------------------- step (5) -- */

/* Prefix-first walk.  choice[i][0] = 0 (rank 0 is the drafter argmax of slot 1);
 * choice[i][p+1] = smallest b attaining max_b S[i][p][choice[i][p]][b];
 * tokens[i][s] = ids[i][s][choice[i][s]].  scores [n][B-1][K][K]. */
int oracle_walk(const oracle_desc *D, int32_t n, const double *scores, const int32_t *ids,
                int32_t *tokens, int32_t *choice)
{
    if (!D || !scores || !ids || !tokens || !choice || n < 0) return ORA_E_ARG;
    const int B = D->B, K = D->K;
    for (int32_t i = 0; i < n; ++i) {
        int32_t k = 0;
        choice[(size_t)i * B] = 0;
        for (int p = 0; p + 1 < B; ++p) {
            const double *row = scores + ((((size_t)i * (B - 1) + p) * K) + k) * K;
            int32_t best = 0;
            for (int b = 1; b < K; ++b)
                if (row[b] > row[best]) best = b;
            k = best;
            choice[(size_t)i * B + p + 1] = k;
        }
        for (int sl = 0; sl < B; ++sl)
            tokens[(size_t)i * B + sl] = ids[((size_t)i * B + sl) * K + choice[(size_t)i * B + sl]];
    }
    return ORA_OK;
}

/* ------------------------------------------------- Global-Sum path rule -- */

/* The path through the candidate lattice with the largest summed transition
 * score (LiLiCorr, appendix E, Eq. 12: a path scores as the sum of its
 * adjacent-slot terms), found exactly by dynamic programming (the Viterbi
 * algorithm the appendix names).  Slot 1 is fixed at rank 0 (the drafter's
 * argmax), as in the walk.  Sweeping left to right, best[b] is the largest
 * score of a path ending at candidate b of the current slot and from[p][b]
 * the smallest predecessor index attaining it; the last slot takes the
 * smallest b attaining the largest best[b], and the path is traced back
 * through `from`.  total[i] (optional) receives the path's summed score.
 *
 * lambda weights pair p's term by lambda^p.  lambda = 1 is the Global-Sum
 * rule of Eq. 12.  The DCOCO page's Geometric rule (lambda = 0.75) is named
 * there without a formula; it is read here as this geometrically discounted
 * sum, which favours the early slots that prefix acceptance rewards. */
int oracle_viterbi(const oracle_desc *D, int32_t n, const double *scores, const int32_t *ids,
                   double lambda, int32_t *tokens, int32_t *choice, double *total)
{
    if (!D || !scores || !ids || !tokens || !choice || n < 0 || !(lambda > 0.0)) return ORA_E_ARG;
    const int B = D->B, K = D->K;
    double *best = malloc(sizeof(double) * (size_t)K);
    double *next = malloc(sizeof(double) * (size_t)K);
    int32_t *from = malloc(sizeof(int32_t) * (size_t)(B > 1 ? B - 1 : 1) * K);
    if (!best || !next || !from) {
        free(best); free(next); free(from);
        return ORA_E_NOMEM;
    }
    for (int32_t i = 0; i < n; ++i) {
        for (int a = 0; a < K; ++a) best[a] = a == 0 ? 0.0 : -INFINITY;
        for (int p = 0; p + 1 < B; ++p) {
            const double *Sp = scores + ((size_t)i * (B - 1) + p) * K * K;
            const double wp = pow(lambda, p);
            for (int b = 0; b < K; ++b) {
                int32_t arg = 0;
                double v = best[0] + wp * Sp[b];
                for (int a = 1; a < K; ++a) {
                    const double w = best[a] + wp * Sp[(size_t)a * K + b];
                    if (w > v) { v = w; arg = a; }
                }
                next[b] = v;
                from[(size_t)p * K + b] = arg;
            }
            for (int b = 0; b < K; ++b) best[b] = next[b];
        }
        int32_t k = 0;
        for (int b = 1; b < K; ++b)
            if (best[b] > best[k]) k = b;
        if (total) total[i] = best[k];
        for (int sl = B - 1; sl >= 1; --sl) {
            choice[(size_t)i * B + sl] = k;
            k = from[(size_t)(sl - 1) * K + k];
        }
        choice[(size_t)i * B] = 0;
        for (int sl = 0; sl < B; ++sl)
            tokens[(size_t)i * B + sl] = ids[((size_t)i * B + sl) * K + choice[(size_t)i * B + sl]];
    }
    free(best); free(next); free(from);
    return ORA_OK;
}

/* Beam search over the candidate lattice (the critique on the DCOCO page,
 * weakness (2): the single-path walk cannot look ahead, so widen it into a
 * narrow beam of 2-4 paths at O(B K beam) cost).  The page gives no path
 * score; the one read here is the summed transition score of the Global-Sum
 * rule, slot 1 fixed at rank 0 as in the walk.  The beam starts as the single
 * path (0) with score 0; at pair p every beam path i extends by every
 * successor b with score g_i + S_p(last_i, b), and the W best extensions are
 * kept, ordered by score descending, then beam index ascending, then b
 * ascending.  The answer is the first path of the final beam.  Scores are
 * float32 and each extension's score is one float32 addition (the kernel's
 * precision, so that both sides rank the same numbers).  W = 1 is the greedy
 * walk; a W of at least K^(B-1) keeps every path.  total[i] (optional)
 * receives the chosen path's score. */
typedef struct {
    float g;
    int32_t beam, b;
} beam_cand_t;

static int beam_cmp(const void *pa, const void *pb)
{
    const beam_cand_t *a = (const beam_cand_t *)pa, *b = (const beam_cand_t *)pb;
    if (a->g > b->g) return -1;
    if (a->g < b->g) return 1;
    if (a->beam != b->beam) return a->beam < b->beam ? -1 : 1;
    return (a->b > b->b) - (a->b < b->b);
}

int oracle_beam(const oracle_desc *D, int32_t n, const float *scores, const int32_t *ids, int32_t W,
                int32_t *tokens, int32_t *choice, float *total)
{
    if (!D || !scores || !ids || !tokens || !choice || n < 0 || W < 1) return ORA_E_ARG;
    const int B = D->B, K = D->K;
    const size_t ncand = (size_t)W * K;
    float *g = malloc(sizeof(float) * W), *g2 = malloc(sizeof(float) * W);
    int32_t *path = malloc(sizeof(int32_t) * W * B), *path2 = malloc(sizeof(int32_t) * W * B);
    beam_cand_t *cand = malloc(sizeof(beam_cand_t) * ncand);
    if (!g || !g2 || !path || !path2 || !cand) {
        free(g); free(g2); free(path); free(path2); free(cand);
        return ORA_E_NOMEM;
    }
    for (int32_t i = 0; i < n; ++i) {
        int nb = 1;
        g[0] = 0.f;
        path[0] = 0;
        for (int p = 0; p + 1 < B; ++p) {
            const float *Sp = scores + ((size_t)i * (B - 1) + p) * K * K;
            size_t nc = 0;
            for (int bi = 0; bi < nb; ++bi) {
                const int last = path[(size_t)bi * B + p];
                for (int b = 0; b < K; ++b) {
                    cand[nc].g = g[bi] + Sp[(size_t)last * K + b];   /* one float32 addition */
                    cand[nc].beam = bi;
                    cand[nc].b = b;
                    ++nc;
                }
            }
            qsort(cand, nc, sizeof(beam_cand_t), beam_cmp);
            const int keep = (int)(nc < (size_t)W ? nc : (size_t)W);
            for (int k = 0; k < keep; ++k) {
                g2[k] = cand[k].g;
                memcpy(path2 + (size_t)k * B, path + (size_t)cand[k].beam * B, sizeof(int32_t) * (p + 1));
                path2[(size_t)k * B + p + 1] = cand[k].b;
            }
            nb = keep;
            float *tg = g; g = g2; g2 = tg;
            int32_t *tp = path; path = path2; path2 = tp;
        }
        if (total) total[i] = g[0];
        for (int sl = 0; sl < B; ++sl) {
            choice[(size_t)i * B + sl] = path[sl];
            tokens[(size_t)i * B + sl] = ids[((size_t)i * B + sl) * K + path[sl]];
        }
    }
    free(g); free(g2); free(path); free(path2); free(cand);
    return ORA_OK;
}

/* Length of the accepted prefix under a greedy verifier (Faster Decoding,
 * "Greedy verification"): the number of leading slots whose proposed token
 * equals the target token. accepted[i] in [0, B]. */
int oracle_accepted(int32_t n, int32_t B, const int32_t *tokens, const int32_t *targets,
                    int32_t *accepted)
{
    if (!tokens || !targets || !accepted || n < 0 || B < 0) return ORA_E_ARG;
    for (int32_t i = 0; i < n; ++i) {
        int32_t a = 0;
        while (a < B && tokens[(size_t)i * B + a] == targets[(size_t)i * B + a]) ++a;
        accepted[i] = a;
    }
    return ORA_OK;
}
