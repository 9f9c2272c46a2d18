/*
 * hils_oracle.h -- interface of the fp64 CPU oracle (test infrastructure
 * only; see hils_oracle.c).  Independent of the GPU library's header.
 */
#ifndef HILS_ORACLE_H
#define HILS_ORACLE_H

#include <stdint.h>

#define HILS_REF_MAX_D 256
#define HILS_REF_MAX_K 256
#define HILS_REF_MAX_G 64

/* how chunk scores are obtained */
enum {
    HILS_REF_SCORE_LANDMARK = 0,      /* s^ = q.k'/sqrt(d) + b' from summaries */
    HILS_REF_SCORE_SELF_LANDMARK = 1, /* summaries recomputed with q' := q_i */
    HILS_REF_SCORE_EXACT_MASS = 2     /* log of the true chunk mass (naive BSA) */
};

typedef struct {
    int64_t B, N, H_q, H_kv, H_lm, d, S, W, K;
    double scale;
    /* 0: a group's chunk score is the max of its heads' s^ (GQA paragraph);
     * 1: the max of each head's s^ minus its log-sum-exp over the row's
     *    candidate chunks (per-head normalised weights) */
    int64_t agg_mode;
} hils_ref_cfg;

int hils_ref_summarize(const hils_ref_cfg *cfg, const float *k,
                       const float *q_lm, double *k_sum, double *b_sum);

int hils_ref_qcal_rows(const hils_ref_cfg *cfg, int64_t d_model, int64_t r,
                       const float *q, const float *h, const float *w_down,
                       const float *w_up, int64_t R, const int64_t *rows,
                       double *q_s);

int hils_ref_forward_rows(const hils_ref_cfg *cfg, int mode, const float *q,
                          const float *k, const float *v, const double *k_sum,
                          const double *b_sum, int64_t d_model, int64_t r,
                          const float *h, const float *w_down,
                          const float *w_up, int64_t R, const int64_t *rows,
                          const int32_t *given_sel, int32_t *sel_idx,
                          double *sel_score, double *kth, double *out,
                          double *lse, double *agg_out);

int hils_ref_decode(const hils_ref_cfg *cfg, int64_t num_seqs, const float *q,
                    const float *k_cache, const float *v_cache,
                    const float *ksum_cache, const float *bsum_cache,
                    const int32_t *block_table, int64_t max_pages,
                    const int32_t *seq_lens, int64_t d_model, int64_t r,
                    const float *h, const float *w_down, const float *w_up,
                    const int32_t *kv_block_table, const int32_t *given_sel,
                    int32_t *sel_idx, double *sel_score, double *kth,
                    double *out, double *lse, double *agg_out,
                    int64_t agg_stride);

int hils_ref_dense_causal_rows(const hils_ref_cfg *cfg, const float *q,
                               const float *k, const float *v, int64_t R,
                               const int64_t *rows, double *out, double *lse);

int hils_ref_version(void);

#endif
