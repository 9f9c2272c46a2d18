/*
 * hils_oracle.c -- plain fp64 CPU oracle of the HiLS (Hierarchical Landmark
 * Sparse) attention forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may load, link or
 * call this file; it exists so that tests, the smoke check and the CPU
 * baseline leg of the benchmark can compare the GPU library against a slow,
 * obviously correct implementation.  It shares no code, header, table or
 * helper with the GPU library.
 *
 * Source of the method: "HiLS: Hierarchical Landmark Sparse Attention"
 * (hyper.ai paper summary, section "方法"):
 *   - uniform chunks of S tokens; per query a chunk-aligned causal sliding
 *     window of size W plus the top-K distant chunks (naive-BSA paragraph);
 *   - landmark query q'_c of chunk c induces a distribution p over the chunk's
 *     keys; compressed key k'_c = sum_j p_j k_j; bias b'_c = entropy of p;
 *     surrogate score s^_{i,c} = q_i.k'_c / sqrt(d) + b'_c (surrogate-score
 *     equation and the paragraph after it);
 *   - partition estimate Z^_i = sum_{c in I_i} exp(s^_{i,c}) + Z_{i,swa};
 *     attention weight = (exp(s_ij)/Z_{i,c(j)}) * (Z^_{i,c(j)}/Z^_i)
 *     (hierarchical factorisation equation);
 *   - Q-Cal: scoring query q_i + W_up W_down h_i (practical design choices);
 *   - GQA: per-head chunk scores, max over the heads of a group, one top-K
 *     per group (same paragraph).
 * Readings where the pages are silent (window bounds, candidate set, logit
 * scale inside the landmark softmax, tie-break, landmark heads under GQA)
 * are stated next to the code that takes them.
 *
 * Everything is computed in double.  Array inputs that are data (q, k, v,
 * landmark queries, hidden states, Q-Cal weights, decode caches) are taken
 * as float: the caller promotes bf16/fp32 data to float exactly, and every
 * read here promotes float to double exactly.  Computed quantities
 * (summaries) are double.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "hils_oracle.h"

/* ------------------------------------------------------------------ */
/* shape helpers                                                      */
/* ------------------------------------------------------------------ */

/* Completed chunks of a length-n sequence: chunk c holds tokens
 * [c*S, c*S + S).  Only completed chunks get a landmark and a summary. */
static int64_t completed_chunks(const hils_ref_cfg *cfg, int64_t n)
{
    return n / cfg->S;
}

/* Reading of "a local sliding window of size W aligned to chunk
 * boundaries": the causal prefix of the query's own chunk plus the W/S
 * complete chunks before it, i.e. keys [max(0, floor(i/S)*S - W), i]. */
static int64_t window_start(const hils_ref_cfg *cfg, int64_t i)
{
    int64_t s = (i / cfg->S) * cfg->S - cfg->W;
    return s < 0 ? 0 : s;
}

/* Reading of "the top-K distant chunks": the candidates are the completed
 * chunks lying entirely before the window, c < floor(i/S) - W/S. */
static int64_t num_candidates(const hils_ref_cfg *cfg, int64_t i)
{
    int64_t n = i / cfg->S - cfg->W / cfg->S;
    return n < 0 ? 0 : n;
}

/* Landmark head used by query head h, and kv head read by landmark head l.
 * With H_lm == H_q every query head has its own landmark; with
 * H_lm == H_kv the heads of a GQA group share one. */
static int64_t lm_head_of(const hils_ref_cfg *cfg, int64_t h)
{
    return h * cfg->H_lm / cfg->H_q;
}
static int64_t kv_head_of_lm(const hils_ref_cfg *cfg, int64_t l)
{
    return l * cfg->H_kv / cfg->H_lm;
}

static double dot_fd(const float *a, const float *b, int64_t d)
{
    double s = 0.0;
    for (int64_t t = 0; t < d; ++t)
        s += (double)a[t] * (double)b[t];
    return s;
}
static double dot_dd(const double *a, const double *b, int64_t d)
{
    double s = 0.0;
    for (int64_t t = 0; t < d; ++t)
        s += a[t] * b[t];
    return s;
}
static double dot_df(const double *a, const float *b, int64_t d)
{
    double s = 0.0;
    for (int64_t t = 0; t < d; ++t)
        s += a[t] * (double)b[t];
    return s;
}

/* log(sum_j exp(x_j)), written out with the max shifted out. */
static double log_sum_exp(const double *x, int64_t n)
{
    if (n <= 0)
        return -INFINITY;
    double m = -INFINITY;
    for (int64_t j = 0; j < n; ++j)
        if (x[j] > m)
            m = x[j];
    if (m == -INFINITY)
        return -INFINITY;
    double z = 0.0;
    for (int64_t j = 0; j < n; ++j)
        z += exp(x[j] - m);
    return m + log(z);
}

/* ------------------------------------------------------------------ */
/* landmark summary: (k'_c, b'_c) from the landmark query q'_c         */
/* ------------------------------------------------------------------ */

/* One chunk: keys[j*d ...] for j < S, landmark query ql (double).
 * p_j = softmax_j(scale * ql.k_j); k' = sum_j p_j k_j; b' = -sum_j p_j log p_j.
 * The logit scale inside the landmark softmax is taken to be the attention
 * scale 1/sqrt(d); with it, s^ equals the chunk log-mass exactly when the
 * query equals the landmark query (first-order Taylor expansion of
 * log-sum-exp at the landmark point). */
static void summarize_one(const hils_ref_cfg *cfg, const double *ql,
                          const float *keys, int64_t key_stride,
                          double *a /* scratch S */, double *k_out,
                          double *b_out)
{
    const int64_t S = cfg->S, d = cfg->d;
    for (int64_t j = 0; j < S; ++j)
        a[j] = cfg->scale * dot_df(ql, keys + j * key_stride, d);
    const double lse = log_sum_exp(a, S);
    for (int64_t t = 0; t < d; ++t)
        k_out[t] = 0.0;
    double entropy = 0.0;
    for (int64_t j = 0; j < S; ++j) {
        const double log_p = a[j] - lse;
        const double p = exp(log_p);
        for (int64_t t = 0; t < d; ++t)
            k_out[t] += p * (double)keys[j * key_stride + t];
        if (p > 0.0)
            entropy -= p * log_p;
    }
    *b_out = entropy;
}

int hils_ref_summarize(const hils_ref_cfg *cfg, const float *k,
                       const float *q_lm, double *k_sum, double *b_sum)
{
    const int64_t B = cfg->B, N = cfg->N, H_kv = cfg->H_kv, H_lm = cfg->H_lm;
    const int64_t d = cfg->d, S = cfg->S;
    const int64_t C = completed_chunks(cfg, N);
    if (C <= 0)
        return 0;
#pragma omp parallel
    {
        double *a = (double *)malloc(sizeof(double) * S);
        double *ql = (double *)malloc(sizeof(double) * d);
#pragma omp for collapse(3) schedule(static)
        for (int64_t b = 0; b < B; ++b)
            for (int64_t l = 0; l < H_lm; ++l)
                for (int64_t c = 0; c < C; ++c) {
                    const int64_t g = kv_head_of_lm(cfg, l);
                    const float *qsrc = q_lm + ((b * H_lm + l) * C + c) * d;
                    for (int64_t t = 0; t < d; ++t)
                        ql[t] = (double)qsrc[t];
                    const float *keys = k + ((b * H_kv + g) * N + c * S) * d;
                    summarize_one(cfg, ql, keys, d, a,
                                  k_sum + ((b * H_lm + l) * C + c) * d,
                                  b_sum + (b * H_lm + l) * C + c);
                }
        free(a);
        free(ql);
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* Q-Cal: scoring query q_i + W_up (W_down h_i)                        */
/* ------------------------------------------------------------------ */

/* h_i: [d_model]; w_down: [r, d_model]; w_up: [H_q*d, r].  Writes
 * delta[H_q*d], laid out head-major (h*d + t). */
static void qcal_delta(int64_t d_model, int64_t r, int64_t hd, const float *h_i,
                       const float *w_down, const float *w_up, double *u,
                       double *delta)
{
    for (int64_t a = 0; a < r; ++a)
        u[a] = dot_fd(w_down + a * d_model, h_i, d_model);
    for (int64_t e = 0; e < hd; ++e) {
        double s = 0.0;
        for (int64_t a = 0; a < r; ++a)
            s += (double)w_up[e * r + a] * u[a];
        delta[e] = s;
    }
}

int hils_ref_qcal_rows(const hils_ref_cfg *cfg, int64_t d_model, int64_t r,
                       const float *q, const float *h, const float *w_down,
                       const float *w_up, int64_t R, const int64_t *rows,
                       double *q_s /* [B, H_q, R, d] */)
{
    const int64_t B = cfg->B, N = cfg->N, H_q = cfg->H_q, d = cfg->d;
#pragma omp parallel
    {
        double *u = (double *)malloc(sizeof(double) * (r > 0 ? r : 1));
        double *delta = (double *)malloc(sizeof(double) * H_q * d);
#pragma omp for collapse(2) schedule(static)
        for (int64_t b = 0; b < B; ++b)
            for (int64_t ri = 0; ri < R; ++ri) {
                const int64_t i = rows[ri];
                qcal_delta(d_model, r, H_q * d, h + (b * N + i) * d_model,
                           w_down, w_up, u, delta);
                for (int64_t hh = 0; hh < H_q; ++hh)
                    for (int64_t t = 0; t < d; ++t)
                        q_s[((b * H_q + hh) * R + ri) * d + t] =
                            (double)q[((b * H_q + hh) * N + i) * d + t] +
                            delta[hh * d + t];
            }
        free(u);
        free(delta);
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* selection: first min(K, n) candidates by (score desc, index asc)    */
/* ------------------------------------------------------------------ */

typedef struct {
    double score;
    int64_t index;
} scored_chunk;

static int by_score_then_index(const void *x, const void *y)
{
    const scored_chunk *a = (const scored_chunk *)x;
    const scored_chunk *b = (const scored_chunk *)y;
    if (a->score > b->score)
        return -1;
    if (a->score < b->score)
        return 1;
    return (a->index < b->index) ? -1 : (a->index > b->index);
}
static int by_int_asc(const void *x, const void *y)
{
    int32_t a = *(const int32_t *)x, b = *(const int32_t *)y;
    return (a > b) - (a < b);
}

/* Sorts agg[0..n) (in a scratch copy) and writes the selected chunk ids,
 * ascending and padded with -1, to sel[0..K).  kth[0] = K-th largest
 * score, kth[1] = (K+1)-th (NaN where absent); used by the tests' near-tie
 * exemption. */
static void select_top_k(const double *agg, int64_t n, int64_t K,
                         scored_chunk *scratch, int32_t *sel, double *kth)
{
    for (int64_t c = 0; c < n; ++c) {
        scratch[c].score = agg[c];
        scratch[c].index = c;
    }
    qsort(scratch, (size_t)n, sizeof(scored_chunk), by_score_then_index);
    const int64_t take = n < K ? n : K;
    for (int64_t k = 0; k < K; ++k)
        sel[k] = (k < take) ? (int32_t)scratch[k].index : -1;
    qsort(sel, (size_t)take, sizeof(int32_t), by_int_asc);
    if (kth) {
        kth[0] = (K >= 1 && n >= K) ? scratch[K - 1].score : NAN;
        kth[1] = (n >= K + 1) ? scratch[K].score : NAN;
    }
}

/* ------------------------------------------------------------------ */
/* exact softmax attention over an explicit key range                  */
/* ------------------------------------------------------------------ */

/* keys/values: pointers to token j's rows via the accessor callbacks of the
 * caller (prefill: contiguous; decode: through the block table).  Computes
 * lse = log sum_j exp(s_j) and o = sum_j softmax(s)_j v_j over tokens
 * [j0, j1]. */
typedef const float *(*row_fn)(const void *ctx, int64_t j);

static void attend_range(const hils_ref_cfg *cfg, const double *q, row_fn key,
                         row_fn val, const void *ctx, int64_t j0, int64_t j1,
                         double *s /* scratch */, double *o, double *lse)
{
    const int64_t d = cfg->d;
    const int64_t n = j1 - j0 + 1;
    for (int64_t t = 0; t < d; ++t)
        o[t] = 0.0;
    if (n <= 0) {
        *lse = -INFINITY;
        return;
    }
    for (int64_t j = 0; j < n; ++j)
        s[j] = cfg->scale * dot_df(q, key(ctx, j0 + j), d);
    const double L = log_sum_exp(s, n);
    for (int64_t j = 0; j < n; ++j) {
        const double w = exp(s[j] - L);
        const float *vj = val(ctx, j0 + j);
        for (int64_t t = 0; t < d; ++t)
            o[t] += w * (double)vj[t];
    }
    *lse = L;
}

/* ------------------------------------------------------------------ */
/* per-query forward (shared by prefill rows and decode)               */
/* ------------------------------------------------------------------ */

typedef struct {
    const hils_ref_cfg *cfg;
    /* prefill: contiguous k, v of one (b, kv head) */
    const float *k_bg, *v_bg;
    /* decode: paged caches */
    const float *k_cache, *v_cache;
    const int32_t *pages; /* block-table row of this sequence */
    int64_t g;            /* kv head */
} kv_ctx;

static const float *prefill_key(const void *p, int64_t j)
{
    const kv_ctx *c = (const kv_ctx *)p;
    return c->k_bg + j * c->cfg->d;
}
static const float *prefill_val(const void *p, int64_t j)
{
    const kv_ctx *c = (const kv_ctx *)p;
    return c->v_bg + j * c->cfg->d;
}
/* paged cache layout: [page, H_kv, S, d]; token j lives in logical chunk
 * j / S, i.e. physical page pages[j / S], slot j % S. */
static const float *paged_key(const void *p, int64_t j)
{
    const kv_ctx *c = (const kv_ctx *)p;
    const hils_ref_cfg *cfg = c->cfg;
    const int64_t page = c->pages[j / cfg->S];
    return c->k_cache + ((page * cfg->H_kv + c->g) * cfg->S + j % cfg->S) * cfg->d;
}
static const float *paged_val(const void *p, int64_t j)
{
    const kv_ctx *c = (const kv_ctx *)p;
    const hils_ref_cfg *cfg = c->cfg;
    const int64_t page = c->pages[j / cfg->S];
    return c->v_cache + ((page * cfg->H_kv + c->g) * cfg->S + j % cfg->S) * cfg->d;
}

/* Chunk-score provider: returns s^ for (query head h, chunk c) given the
 * scoring query of head h. */
typedef struct {
    const hils_ref_cfg *cfg;
    int mode;
    /* landmark mode, prefill: double summaries [B,H_lm,C,d], [B,H_lm,C] */
    const double *k_sum, *b_sum;
    int64_t C; /* chunk stride of the summaries */
    /* landmark mode, decode: float caches [P,H_lm,d], [P,H_lm] */
    const float *ksum_cache, *bsum_cache;
    int64_t b;
    kv_ctx *kv;
    double *a_scratch, *kp_scratch; /* S and d doubles */
    const int32_t *sum_pages;       /* decode: chunk -> page of the summaries */
} score_ctx;

static double chunk_score(score_ctx *sc, int64_t h, const double *q_s,
                          int64_t c)
{
    const hils_ref_cfg *cfg = sc->cfg;
    const int64_t d = cfg->d, S = cfg->S;
    const int64_t l = lm_head_of(cfg, h);
    if (sc->mode == HILS_REF_SCORE_LANDMARK) {
        if (sc->ksum_cache) {
            const int64_t page = sc->sum_pages[c];
            const float *kp = sc->ksum_cache + (page * cfg->H_lm + l) * d;
            return cfg->scale * dot_df(q_s, kp, d) +
                   (double)sc->bsum_cache[page * cfg->H_lm + l];
        }
        const double *kp = sc->k_sum + ((sc->b * cfg->H_lm + l) * sc->C + c) * d;
        return cfg->scale * dot_dd(q_s, kp, d) +
               sc->b_sum[(sc->b * cfg->H_lm + l) * sc->C + c];
    }
    /* gather the chunk's keys */
    row_fn key = sc->kv->pages ? paged_key : prefill_key;
    if (sc->mode == HILS_REF_SCORE_SELF_LANDMARK) {
        /* landmark query := the scoring query itself */
        double *a = sc->a_scratch, *kp = sc->kp_scratch;
        for (int64_t j = 0; j < S; ++j)
            a[j] = cfg->scale * dot_df(q_s, key(sc->kv, c * S + j), d);
        const double lse = log_sum_exp(a, S);
        for (int64_t t = 0; t < d; ++t)
            kp[t] = 0.0;
        double entropy = 0.0;
        for (int64_t j = 0; j < S; ++j) {
            const double log_p = a[j] - lse;
            const double p = exp(log_p);
            const float *kj = key(sc->kv, c * S + j);
            for (int64_t t = 0; t < d; ++t)
                kp[t] += p * (double)kj[t];
            if (p > 0.0)
                entropy -= p * log_p;
        }
        return cfg->scale * dot_dd(q_s, kp, d) + entropy;
    }
    /* HILS_REF_SCORE_EXACT_MASS: log of the true chunk mass */
    double *a = sc->a_scratch;
    for (int64_t j = 0; j < S; ++j)
        a[j] = cfg->scale * dot_df(q_s, key(sc->kv, c * S + j), d);
    return log_sum_exp(a, S);
}

/* One (b, kv group g, query position i): score -> select -> attend ->
 * fuse, for the G query heads of the group.
 *   q_rows  [G][d]   raw queries (double)
 *   qs_rows [G][d]   scoring queries (double; == q_rows without Q-Cal)
 *   given   [K] or NULL
 *   outputs: sel[K], sel_score[G][K], kth[2], out[G][d], lse[G]
 *   agg_all[n_cand] optional (all candidate group scores) */
static void forward_one(const hils_ref_cfg *cfg, score_ctx *sc, kv_ctx *kv,
                        row_fn key, row_fn val, int64_t i,
                        const double *q_rows, const double *qs_rows,
                        const int32_t *given, int32_t *sel, double *sel_score,
                        double *kth, double *out, double *lse, double *agg_all,
                        double *scratch_scores /* G * nc */,
                        scored_chunk *scratch_sort, double *s_scratch,
                        double *o_tmp, int do_attend)
{
    const int64_t G = cfg->H_q / cfg->H_kv, K = cfg->K, d = cfg->d;
    const int64_t S = cfg->S;
    const int64_t nc = num_candidates(cfg, i);
    const int64_t h0 = kv->g * G;

    /* per-head surrogate scores of every candidate chunk */
    for (int64_t c = 0; c < nc; ++c)
        for (int64_t e = 0; e < G; ++e)
            scratch_scores[e * nc + c] = chunk_score(sc, h0 + e, qs_rows + e * d, c);
    /* group score: the max over the heads of the group of each head's chunk
     * weight -- its raw s^ (agg_mode 0), or (agg_mode 1) its log-softmax
     * over the row's candidates, s^ - log sum_c' exp(s^_c').  The fusion
     * below always uses the raw s^. */
    double *agg = agg_all;
    for (int64_t c = 0; c < nc; ++c)
        agg[c] = -INFINITY;
    for (int64_t e = 0; e < G; ++e) {
        const double norm =
            cfg->agg_mode == 1 ? log_sum_exp(scratch_scores + e * nc, nc) : 0.0;
        for (int64_t c = 0; c < nc; ++c) {
            const double v = scratch_scores[e * nc + c] - norm;
            if (v > agg[c])
                agg[c] = v;
        }
    }

    if (given) {
        for (int64_t k = 0; k < K; ++k)
            sel[k] = given[k];
        kth[0] = kth[1] = NAN;
    } else {
        select_top_k(agg, nc, K, scratch_sort, sel, kth);
    }

    for (int64_t e = 0; e < G; ++e) {
        for (int64_t k = 0; k < K; ++k)
            sel_score[e * K + k] =
                sel[k] < 0 ? -INFINITY : scratch_scores[e * nc + sel[k]];
    }
    if (!do_attend)
        return;

    for (int64_t e = 0; e < G; ++e) {
        const double *q = q_rows + e * d;
        /* window part */
        double o_sw[HILS_REF_MAX_D], lse_sw;
        attend_range(cfg, q, key, val, kv, window_start(cfg, i), i, s_scratch,
                     o_sw, &lse_sw);
        /* L = log(sum_c exp(s^_c) + exp(lse_swa)) */
        double terms[HILS_REF_MAX_K + 1];
        int64_t nt = 0;
        for (int64_t k = 0; k < K; ++k)
            if (sel[k] >= 0)
                terms[nt++] = sel_score[e * K + k];
        terms[nt++] = lse_sw;
        const double L = log_sum_exp(terms, nt);
        double *o = out + e * d;
        const double w_sw = exp(lse_sw - L);
        for (int64_t t = 0; t < d; ++t)
            o[t] = w_sw * o_sw[t];
        for (int64_t k = 0; k < K; ++k) {
            if (sel[k] < 0)
                continue;
            const int64_t c = sel[k];
            double lse_c;
            attend_range(cfg, q, key, val, kv, c * S, c * S + S - 1, s_scratch,
                         o_tmp, &lse_c);
            /* exact intra-chunk softmax, weighted by the learned surrogate
             * mass exp(s^_c) / Z^ */
            const double w = exp(sel_score[e * K + k] - L);
            for (int64_t t = 0; t < d; ++t)
                o[t] += w * o_tmp[t];
        }
        lse[e] = L;
    }
}

static int check_cfg(const hils_ref_cfg *cfg)
{
    if (cfg->B < 0 || cfg->N < 0 || cfg->H_q <= 0 || cfg->H_kv <= 0 ||
        cfg->H_lm <= 0 || cfg->d <= 0 || cfg->S <= 0 || cfg->W < 0 ||
        cfg->K < 0)
        return -1;
    if (cfg->H_q % cfg->H_kv != 0 || cfg->W % cfg->S != 0)
        return -1;
    if (!(cfg->H_lm == cfg->H_q || cfg->H_lm == cfg->H_kv))
        return -1;
    if (cfg->d > HILS_REF_MAX_D || cfg->K > HILS_REF_MAX_K)
        return -1;
    if (cfg->agg_mode != 0 && cfg->agg_mode != 1)
        return -1;
    return 0;
}

int hils_ref_forward_rows(const hils_ref_cfg *cfg, int mode, const float *q,
                          const float *k, const float *v, const double *k_sum,
                          const double *b_sum, int64_t d_model, int64_t r,
                          const float *h, const float *w_down,
                          const float *w_up, int64_t R, const int64_t *rows,
                          const int32_t *given_sel, int32_t *sel_idx,
                          double *sel_score, double *kth, double *out,
                          double *lse, double *agg_out)
{
    if (check_cfg(cfg))
        return -1;
    const int64_t B = cfg->B, N = cfg->N, H_q = cfg->H_q, H_kv = cfg->H_kv;
    const int64_t d = cfg->d, K = cfg->K, G = H_q / H_kv;
    const int64_t C = completed_chunks(cfg, N);
    const int64_t nc_max = num_candidates(cfg, N > 0 ? N - 1 : 0);
    const int64_t n_s = (cfg->W + cfg->S > cfg->S) ? cfg->W + cfg->S : cfg->S;
#pragma omp parallel
    {
        double *q_rows = (double *)malloc(sizeof(double) * G * d);
        double *qs_rows = (double *)malloc(sizeof(double) * G * d);
        double *scores = (double *)malloc(sizeof(double) * (G * nc_max + 1));
        double *agg = (double *)malloc(sizeof(double) * (nc_max + 1));
        scored_chunk *srt =
            (scored_chunk *)malloc(sizeof(scored_chunk) * (nc_max + 1));
        double *s_scr = (double *)malloc(sizeof(double) * (n_s + cfg->S));
        double *o_tmp = (double *)malloc(sizeof(double) * d);
        double *a_scr = (double *)malloc(sizeof(double) * cfg->S);
        double *kp_scr = (double *)malloc(sizeof(double) * d);
        double *u = (double *)malloc(sizeof(double) * (r > 0 ? r : 1));
        double *delta = (double *)malloc(sizeof(double) * H_q * d);
        int32_t *sel = (int32_t *)malloc(sizeof(int32_t) * (K + 1));
        double *ss = (double *)malloc(sizeof(double) * (G * K + 1));
        double *o = (double *)malloc(sizeof(double) * G * d);
        double l_out[HILS_REF_MAX_G];
        double kt[2];
#pragma omp for collapse(3) schedule(dynamic, 4)
        for (int64_t b = 0; b < B; ++b)
            for (int64_t g = 0; g < H_kv; ++g)
                for (int64_t ri = 0; ri < R; ++ri) {
                    const int64_t i = rows[ri];
                    kv_ctx kv = {cfg, k + (b * H_kv + g) * N * d,
                                 v + (b * H_kv + g) * N * d, NULL, NULL, NULL, g};
                    score_ctx sc = {cfg,  mode, k_sum, b_sum, C,     NULL,
                                    NULL, b,    &kv,   a_scr, kp_scr, NULL};
                    if (h)
                        qcal_delta(d_model, r, H_q * d, h + (b * N + i) * d_model,
                                   w_down, w_up, u, delta);
                    for (int64_t e = 0; e < G; ++e)
                        for (int64_t t = 0; t < d; ++t) {
                            const double x =
                                (double)q[((b * H_q + g * G + e) * N + i) * d + t];
                            q_rows[e * d + t] = x;
                            qs_rows[e * d + t] =
                                h ? x + delta[(g * G + e) * d + t] : x;
                        }
                    const int32_t *given =
                        given_sel ? given_sel + ((b * H_kv + g) * R + ri) * K : NULL;
                    forward_one(cfg, &sc, &kv, prefill_key, prefill_val, i, q_rows,
                                qs_rows, given, sel, ss, kt, o, l_out, agg, scores,
                                srt, s_scr, o_tmp, out != NULL || lse != NULL);
                    const int64_t nc = num_candidates(cfg, i);
                    if (sel_idx)
                        for (int64_t kk = 0; kk < K; ++kk)
                            sel_idx[((b * H_kv + g) * R + ri) * K + kk] = sel[kk];
                    if (kth) {
                        kth[((b * H_kv + g) * R + ri) * 2 + 0] = kt[0];
                        kth[((b * H_kv + g) * R + ri) * 2 + 1] = kt[1];
                    }
                    if (agg_out)
                        for (int64_t c = 0; c < C; ++c)
                            agg_out[((b * H_kv + g) * R + ri) * C + c] =
                                c < nc ? agg[c] : NAN;
                    for (int64_t e = 0; e < G; ++e) {
                        const int64_t hh = g * G + e;
                        if (sel_score)
                            for (int64_t kk = 0; kk < K; ++kk)
                                sel_score[((b * H_q + hh) * R + ri) * K + kk] =
                                    ss[e * K + kk];
                        if (out)
                            for (int64_t t = 0; t < d; ++t)
                                out[((b * H_q + hh) * R + ri) * d + t] = o[e * d + t];
                        if (lse)
                            lse[(b * H_q + hh) * R + ri] = l_out[e];
                    }
                }
        free(q_rows);
        free(qs_rows);
        free(scores);
        free(agg);
        free(srt);
        free(s_scr);
        free(o_tmp);
        free(a_scr);
        free(kp_scr);
        free(u);
        free(delta);
        free(sel);
        free(ss);
        free(o);
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* decode over a paged KV / summary cache                              */
/* ------------------------------------------------------------------ */

int hils_ref_decode(const hils_ref_cfg *cfg, int64_t num_seqs, const float *q,
                    const float *k_cache, const float *v_cache,
                    const float *ksum_cache, const float *bsum_cache,
                    const int32_t *block_table, int64_t max_pages,
                    const int32_t *seq_lens, int64_t d_model, int64_t r,
                    const float *h, const float *w_down, const float *w_up,
                    const int32_t *kv_block_table, const int32_t *given_sel,
                    int32_t *sel_idx, double *sel_score, double *kth,
                    double *out, double *lse, double *agg_out,
                    int64_t agg_stride)
{
    /* kv_block_table (optional) maps logical chunks to pages of k_cache /
     * v_cache when those caches hold only a subset of the pages of the
     * summary cache; NULL means both are indexed by block_table. */
    if (!kv_block_table)
        kv_block_table = block_table;
    if ((out || lse) && (!k_cache || !v_cache))
        return -1;
    if (check_cfg(cfg))
        return -1;
    const int64_t H_q = cfg->H_q, H_kv = cfg->H_kv, d = cfg->d, K = cfg->K;
    const int64_t G = H_q / H_kv, S = cfg->S;
    int64_t nc_max = 0;
    for (int64_t b = 0; b < num_seqs; ++b) {
        if (seq_lens[b] <= 0 || (seq_lens[b] + S - 1) / S > max_pages)
            return -1;
        const int64_t n = num_candidates(cfg, seq_lens[b] - 1);
        if (n > nc_max)
            nc_max = n;
    }
    const int64_t n_s = cfg->W + 2 * S;
#pragma omp parallel
    {
        double *q_rows = (double *)malloc(sizeof(double) * G * d);
        double *qs_rows = (double *)malloc(sizeof(double) * G * d);
        double *scores = (double *)malloc(sizeof(double) * (G * nc_max + 1));
        double *agg = (double *)malloc(sizeof(double) * (nc_max + 1));
        scored_chunk *srt =
            (scored_chunk *)malloc(sizeof(scored_chunk) * (nc_max + 1));
        double *s_scr = (double *)malloc(sizeof(double) * n_s);
        double *o_tmp = (double *)malloc(sizeof(double) * d);
        double *a_scr = (double *)malloc(sizeof(double) * S);
        double *kp_scr = (double *)malloc(sizeof(double) * d);
        double *u = (double *)malloc(sizeof(double) * (r > 0 ? r : 1));
        double *delta = (double *)malloc(sizeof(double) * H_q * d);
        int32_t *sel = (int32_t *)malloc(sizeof(int32_t) * (K + 1));
        double *ss = (double *)malloc(sizeof(double) * (G * K + 1));
        double *o = (double *)malloc(sizeof(double) * G * d);
        double l_out[HILS_REF_MAX_G];
        double kt[2];
#pragma omp for collapse(2) schedule(dynamic, 1)
        for (int64_t b = 0; b < num_seqs; ++b)
            for (int64_t g = 0; g < H_kv; ++g) {
                const int64_t t_pos = seq_lens[b] - 1;
                kv_ctx kv = {cfg,     NULL, NULL, k_cache, v_cache,
                             kv_block_table + b * max_pages, g};
                const int32_t *sum_pages = block_table + b * max_pages;
                score_ctx sc = {cfg,        HILS_REF_SCORE_LANDMARK,
                                NULL,       NULL,
                                0,          ksum_cache,
                                bsum_cache, b,
                                &kv,        a_scr,
                                kp_scr,     sum_pages};
                if (h)
                    qcal_delta(d_model, r, H_q * d, h + b * d_model, w_down, w_up,
                               u, delta);
                for (int64_t e = 0; e < G; ++e)
                    for (int64_t t = 0; t < d; ++t) {
                        const double x = (double)q[(b * H_q + g * G + e) * d + t];
                        q_rows[e * d + t] = x;
                        qs_rows[e * d + t] = h ? x + delta[(g * G + e) * d + t] : x;
                    }
                const int32_t *given =
                    given_sel ? given_sel + (b * H_kv + g) * K : NULL;
                forward_one(cfg, &sc, &kv, paged_key, paged_val, t_pos, q_rows,
                            qs_rows, given, sel, ss, kt, o, l_out, agg, scores,
                            srt, s_scr, o_tmp, out != NULL || lse != NULL);
                const int64_t nc = num_candidates(cfg, t_pos);
                if (sel_idx)
                    for (int64_t kk = 0; kk < K; ++kk)
                        sel_idx[(b * H_kv + g) * K + kk] = sel[kk];
                if (kth) {
                    kth[(b * H_kv + g) * 2 + 0] = kt[0];
                    kth[(b * H_kv + g) * 2 + 1] = kt[1];
                }
                if (agg_out)
                    for (int64_t c = 0; c < agg_stride; ++c)
                        agg_out[(b * H_kv + g) * agg_stride + c] =
                            c < nc ? agg[c] : NAN;
                for (int64_t e = 0; e < G; ++e) {
                    const int64_t hh = g * G + e;
                    if (sel_score)
                        for (int64_t kk = 0; kk < K; ++kk)
                            sel_score[(b * H_q + hh) * K + kk] = ss[e * K + kk];
                    if (out)
                        for (int64_t t = 0; t < d; ++t)
                            out[(b * H_q + hh) * d + t] = o[e * d + t];
                    if (lse)
                        lse[b * H_q + hh] = l_out[e];
                }
            }
        free(q_rows);
        free(qs_rows);
        free(scores);
        free(agg);
        free(srt);
        free(s_scr);
        free(o_tmp);
        free(a_scr);
        free(kp_scr);
        free(u);
        free(delta);
        free(sel);
        free(ss);
        free(o);
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* textbook dense causal attention (for the special-case pins)          */
/* ------------------------------------------------------------------ */

int hils_ref_dense_causal_rows(const hils_ref_cfg *cfg, const float *q,
                               const float *k, const float *v, int64_t R,
                               const int64_t *rows, double *out, double *lse)
{
    const int64_t B = cfg->B, N = cfg->N, H_q = cfg->H_q, H_kv = cfg->H_kv;
    const int64_t d = cfg->d, G = H_q / H_kv;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (N + 1));
        double *qd = (double *)malloc(sizeof(double) * d);
#pragma omp for collapse(3) schedule(dynamic, 4)
        for (int64_t b = 0; b < B; ++b)
            for (int64_t hh = 0; hh < H_q; ++hh)
                for (int64_t ri = 0; ri < R; ++ri) {
                    const int64_t i = rows[ri], g = hh / G;
                    kv_ctx kv = {cfg, k + (b * H_kv + g) * N * d,
                                 v + (b * H_kv + g) * N * d, NULL, NULL, NULL, g};
                    for (int64_t t = 0; t < d; ++t)
                        qd[t] = (double)q[((b * H_q + hh) * N + i) * d + t];
                    attend_range(cfg, qd, prefill_key, prefill_val, &kv, 0, i, s,
                                 out + ((b * H_q + hh) * R + ri) * d,
                                 lse + (b * H_q + hh) * R + ri);
                }
        free(s);
        free(qd);
    }
    return 0;
}

int hils_ref_version(void) { return 1; }
