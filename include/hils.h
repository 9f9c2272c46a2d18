/*
 * hils.h -- C ABI of libhils, an MI355X (gfx950) implementation of the
 * HiLS (Hierarchical Landmark Sparse) attention forward pass.
 *
 * Method source: "HiLS: Hierarchical Landmark Sparse Attention", paper
 * summary on hyper.ai, section 方法:
 *   - the sequence is cut into chunks of S tokens; each query attends a
 *     causal sliding window of W tokens aligned to chunk boundaries plus the
 *     top-K distant chunks (naive block-sparse attention paragraph);
 *   - a landmark query q'_c per chunk induces a distribution p over the
 *     chunk's keys; the compressed key is k'_c = sum_j p_j k_j and the bias
 *     b'_c is the entropy of p (paragraph after the surrogate-score
 *     equation);
 *   - surrogate chunk score s^_ic = q_i.k'_c / sqrt(d) + b'_c (surrogate-score
 *     equation); chunks are ranked by it and the top K kept;
 *   - partition estimate Z^_i = sum_{c in I_i} exp(s^_ic) + Z_{i,swa}, and the
 *     attention weight of a selected key is its intra-chunk softmax weight
 *     times exp(s^_ic) / Z^_i (hierarchical factorisation equation);
 *   - Q-Cal: the scoring query is q_i + W_up W_down h_i (low-rank query
 *     calibration paragraph);
 *   - GQA: per-head chunk scores are max-aggregated over the heads of a
 *     group and one top-K set is chosen per group (same paragraph).
 *
 * Conventions shared by every entry point:
 *   - All array pointers are caller-owned DEVICE pointers (hipMalloc or
 *     torch CUDA tensors), contiguous in the stated layout, 16-byte aligned.
 *     The library never allocates, frees or keeps a pointer beyond the work
 *     it enqueues on `stream`.
 *   - Work is enqueued asynchronously on `stream`; results are ready when
 *     the stream is synchronised.  Asynchronous device faults surface there.
 *   - Every argument is validated on the host before anything is launched;
 *     on a non-OK status nothing has been written.  hils_last_error() then
 *     returns a message (thread-local).
 *   - Results are deterministic run to run (no atomics in accumulation).
 *   - Calls are thread-safe; concurrent calls must not share output or
 *     workspace buffers.
 *
 * Layouts (row-major, innermost last):
 *   q      [B, H_q,  N, d]        k, v   [B, H_kv, N, d]
 *   q_lm   [B, H_lm, C, d]        k_sum  [B, H_lm, C, d]   b_sum [B, H_lm, C]
 *   sel_idx   [B, H_kv, N, K] int32 -- ascending chunk ids, -1 padded
 *   sel_score [B, H_q,  N, K] fp32  -- s^ of each selected chunk, -inf padded
 *   out    [B, H_q,  N, d]        lse    [B, H_q, N] fp32
 * with C = floor(N / S) completed chunks.  Query head h belongs to GQA
 * group g = h / (H_q / H_kv); it scores with landmark head
 * l = h * H_lm / H_q; landmark head l reads kv head l * H_kv / H_lm.
 *
 * Window and candidates (the pages leave the bounds open; reading adopted):
 * query i attends keys [max(0, floor(i/S)*S - W), i] exactly; its candidate
 * chunks are c < floor(i/S) - W/S; it selects min(K, #candidates) of them by
 * (group score descending, chunk index ascending).
 */
#ifndef HILS_H
#define HILS_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    HILS_OK = 0,
    HILS_ERR_INVALID_ARG = 1, /* null/misaligned pointer, inconsistent shape */
    HILS_ERR_UNSUPPORTED = 2, /* valid but outside what the kernels cover   */
    HILS_ERR_WORKSPACE = 3,   /* workspace missing or smaller than needed    */
    HILS_ERR_HIP = 4          /* a HIP launch or runtime call failed         */
} hils_status_t;

typedef enum { HILS_F32 = 0, HILS_BF16 = 1 } hils_dtype_t;

/* Where the landmark query q'_c of a chunk comes from (hyper.ai summary,
 * 方法: the landmark paragraph, and the landmark-free variant named after the
 * GQA paragraph). */
typedef enum {
    HILS_LM_CHUNK = 0,  /* one landmark query per chunk: q_lm [B, H_lm, C, d]      */
    HILS_LM_SHARED = 1, /* landmark-free variant: one query per landmark head
                           shared by every chunk and sequence: q_lm [H_lm, d]   */
    HILS_LM_MEAN = 2    /* q'_c = 0: mean-pooled keys, b'_c = log S; q_lm unused */
} hils_landmark_mode_t;

/* How the heads of a GQA group combine their chunk scores before the shared
 * top-K (hyper.ai summary, 方法, GQA paragraph: per-head chunk weights,
 * max-aggregated over the group). */
typedef enum {
    HILS_AGG_MAX = 0,       /* max over the group's heads of s^[h,c]                   */
    HILS_AGG_NORMALIZED = 1 /* max over the heads of the per-head normalised weight
                               s^[h,c] - log sum_{c' candidate} exp(s^[h,c'])          */
} hils_agg_mode_t;

typedef struct {
    int32_t B;    /* batch (prefill); ignored by hils_decode                 */
    int32_t N;    /* tokens per sequence (prefill); ignored by hils_decode   */
    int32_t H_q;  /* query heads                                             */
    int32_t H_kv; /* key/value heads; H_q % H_kv == 0, G = H_q/H_kv in {1,2,4,8} */
    int32_t H_lm; /* landmark heads: H_q or H_kv                             */
    int32_t d;    /* head dim: 64 or 128                                     */
    int32_t S;    /* chunk size: 64 or 128                                   */
    int32_t W;    /* window in tokens, W % S == 0                            */
    int32_t K;    /* chunks kept per query and group, 0..128                 */
    int32_t M;    /* query-group size: a schedule hint; results never depend on it */
    int32_t io_dtype;      /* hils_dtype_t of q, k, v, q_lm, h, W, out, caches */
    int32_t summary_dtype; /* hils_dtype_t of k_sum / ksum_cache; b_sum is fp32 */
    float scale;           /* logit scale; 0 selects 1/sqrt(d)               */
    int32_t landmark_mode; /* hils_landmark_mode_t; 0 (per-chunk queries) by default */
    int32_t agg_mode;      /* hils_agg_mode_t; 0 (max of raw scores) by default   */
    int32_t wait_spins;    /* bound on each internal wait of the bf16 fused-attention
                              kernel, in pauses of the waiting wave; 0 selects the
                              default (2^18).  A wait that reaches it gives up, and
                              the call reports it in its status word (see
                              hils_sparse_attend_fused).  Smaller values only serve
                              to exercise that report. */
    int32_t score_mode;    /* hils_score_mode_t: how hils_score_select (and the
                              paged prefill) ranks the candidates; 0 (auto) by
                              default */
    int32_t attend_mode;   /* hils_attend_mode_t: how hils_sparse_attend_fused
                              visits the selected chunks; 0 (auto) by default */
    int32_t attend_slab;   /* chunk-major form: query rows per slab, rounded up to
                              a multiple of S; 0 bounds the slab's partial buffer
                              by 32 GiB.  Results do not depend on it. */
} hils_config_t;

/* Forms of the selected-chunk attention of hils_sparse_attend_fused (bf16
 * I/O; same definition, outputs equal up to fp32 rounding order and the fp16
 * rounding of each chunk's weighted output).  WALK: a block of adjacent
 * queries stages the union of their selected chunks once and walks it, then
 * the window.  CHUNK_MAJOR: the selections are inverted into per-chunk lists
 * of (query, slot); each chunk is staged once per list segment for every
 * query that selected it, its weighted output exp(s^_c - m^) o_c goes to an
 * fp16 partial buffer, and the window pass starts each row from the sum of
 * its partials; it pays when adjacent queries select different chunks.
 * Workspace grows by about B * H_q * min(N, slab) * K * (d * 2 + 8) bytes
 * (32 GiB of partials at most with the default slab).  fp32 I/O always
 * walks.  hils_prefill_paged takes the same form as the whole-sequence call
 * (and its rows equal that call's bitwise).  AUTO takes CHUNK_MAJOR wherever
 * it runs (faster on both measured workloads: 128K tokens with 64-key
 * chunks, 512K with 128-key chunks). */
typedef enum {
    HILS_ATTEND_AUTO = 0,
    HILS_ATTEND_WALK = 1,
    HILS_ATTEND_CHUNK_MAJOR = 2
} hils_attend_mode_t;

/* Score-and-select forms (same selection, same scores up to fp32 rounding
 * order).  TWO_PASS writes approximate scores of every candidate (a ragged
 * array of about B * H_kv * N * C / 2 floats) and selects from them; it is
 * the faster form.  STREAMING keeps per-row candidate lists on chip and
 * O(B * H_kv * N * K) workspace; it covers every shape except d = 128 with
 * G = 8, fp32 summaries and K > 32, whose per-block working set exceeds the
 * LDS (HILS_ERR_UNSUPPORTED).  AUTO takes TWO_PASS unless its score array
 * would exceed 32 GiB and STREAMING covers the shape. */
typedef enum {
    HILS_SCORE_AUTO = 0,
    HILS_SCORE_TWO_PASS = 1,
    HILS_SCORE_STREAMING = 2
} hils_score_mode_t;

/* Workspace kinds for hils_workspace_size(). */
enum {
    HILS_WS_SCORE = 0,      /* hils_score_select without Q-Cal            */
    HILS_WS_SCORE_QCAL = 1, /* hils_score_select with Q-Cal               */
    HILS_WS_FUSED = 2,      /* hils_sparse_attend_fused                   */
    HILS_WS_DECODE = 3,     /* hils_decode                                */
    HILS_WS_BACKWARD = 4,   /* hils_sparse_attend_backward                */
    HILS_WS_DENSE = 5,      /* hils_dense_causal_attend                   */
    HILS_WS_DENSE_DECODE = 6 /* hils_dense_decode                         */
};

/* Landmark summary (compressed keys).  For every completed chunk c and
 * landmark head l: p = softmax_j(scale * q_lm[l,c] . k[g(l), cS+j]) over the
 * chunk's S keys, k_sum[l,c] = sum_j p_j k_j, b_sum[l,c] = -sum_j p_j log p_j
 * (hyper.ai summary, 方法: the compressed key and its entropy bias).
 *   k     [B, H_kv, N, d]  io_dtype
 *   q_lm  [B, H_lm, C, d]  io_dtype ([H_lm, d] with HILS_LM_SHARED; unused,
 *                          may be NULL, with HILS_LM_MEAN)
 *   k_sum [B, H_lm, C, d]  summary_dtype (written)
 *   b_sum [B, H_lm, C]     fp32          (written)
 * Also usable on a paged cache [P, H_kv, S, d] by passing B = P, N = S. */
hils_status_t hils_landmark_summarize(const hils_config_t *cfg, const void *k, const void *q_lm, void *k_sum,
                                      float *b_sum, hipStream_t stream);

/* Surrogate chunk scores, GQA max-aggregation and top-K selection
 * (hyper.ai summary, 方法: surrogate-score equation, partition estimate,
 * Q-Cal and GQA paragraphs).  For every query i, group g and candidate
 * chunk c: s^[h,c] = scale * qs[h,i] . k_sum[l(h),c] + b_sum[l(h),c] for the
 * heads h of g, group score max_h s^[h,c]; the first min(K, #candidates)
 * chunks by (group score desc, index asc) are written ascending to sel_idx
 * (-1 padded) and each head's s^ of them to sel_score (-inf padded).
 * qs = q, or with Q-Cal (h != NULL) qs = q + reshape(W_up (W_down h_i)),
 * used for scoring only.
 *   q        [B, H_q, N, d]        io_dtype
 *   k_sum    [B, H_lm, C, d]       summary_dtype,  b_sum [B, H_lm, C] fp32
 *   h        [B, N, d_model]       io_dtype or NULL (then w_down, w_up unused)
 *   w_down   [r, d_model]          io_dtype
 *   w_up     [H_q * d, r]          io_dtype (row h*d + t feeds head h, dim t)
 *   sel_idx  [B, H_kv, N, K] int32 (written)
 *   sel_score[B, H_q, N, K]  fp32  (written)
 *   workspace: hils_workspace_size(cfg, HILS_WS_SCORE[_QCAL], 0, 0) bytes. */
hils_status_t hils_score_select(const hils_config_t *cfg, const void *q, const void *k_sum, const float *b_sum,
                                const void *h, const void *w_down, const void *w_up, int32_t d_model, int32_t r,
                                int32_t *sel_idx, float *sel_score, void *workspace, size_t workspace_bytes,
                                hipStream_t stream);

/* Exact attention inside each selected chunk and inside the chunk-aligned
 * causal window, fused by the surrogate masses (hyper.ai summary, 方法:
 * partition estimate and hierarchical factorisation equation):
 *   L_i = log(sum_{c in I} exp(s^_c) + exp(lse_swa)),
 *   out_i = sum_c exp(s^_c - L_i) o_c + exp(lse_swa - L_i) o_swa,
 * where o_c / lse_c are the softmax output / log-mass of q_i over chunk c's
 * S keys and o_swa / lse_swa those over the window.  Uses the raw q.
 *   q [B,H_q,N,d], k, v [B,H_kv,N,d] io_dtype; sel_idx / sel_score as
 *   written by hils_score_select; out [B,H_q,N,d] io_dtype (written);
 *   lse [B,H_q,N] fp32 (written, may be NULL).
 *   workspace: hils_workspace_size(cfg, HILS_WS_FUSED, 0, 0) bytes (0 for
 *   fp32 I/O).  bf16 I/O: bytes 0..255 are a status block, followed by a
 *   transposed fp16 copy of v and, in the chunk-major form (attend_mode),
 *   the chunk lists and the fp16 partial buffer of one slab of rows.
 *   Word 0 of the status block (uint32) is written by the call; read it
 *   once the stream is synchronised.  0: the
 *   call completed normally.  Bit 0: an internal wait of the kernel gave up
 *   after cfg->wait_spins pauses; the rows of the waves that gave up hold
 *   NaN in out and lse.  Bit 1: some value of v is not finite or has
 *   magnitude >= 65520, beyond fp16's range.  With either bit set the
 *   outputs of the call are unreliable.
 *   bf16 path: v enters the probability-weighted sum as fp16.  A bf16 value
 *   converts exactly when 2^-14 <= |v| <= 65280 (the largest bf16 value
 *   below fp16's maximum 65504).  Below 2^-14 it rounds to fp16's subnormal
 *   grid, an absolute error of at most 2^-25, and a magnitude of at most
 *   2^-25 becomes 0. */
hils_status_t hils_sparse_attend_fused(const hils_config_t *cfg, const void *q, const void *k, const void *v,
                                       const int32_t *sel_idx, const float *sel_score, void *out, float *lse,
                                       void *workspace, size_t workspace_bytes, hipStream_t stream);

/* One decode step per sequence over a paged KV / summary cache: the steps
 * of hils_score_select and hils_sparse_attend_fused for the single query at
 * position t = seq_lens[b] - 1, whose own key/value are already in the
 * cache.  Summaries are read from the cache, never recomputed.
 *   q           [num_seqs, H_q, d]        io_dtype
 *   k_cache,
 *   v_cache     [P, H_kv, S, d]           io_dtype (one page = one chunk)
 *   ksum_cache  [P, H_lm, d]              summary_dtype
 *   bsum_cache  [P, H_lm]                 fp32
 *   block_table [num_seqs, max_pages]     int32: logical chunk -> page
 *   seq_lens    [num_seqs]                int32, >= 1, tokens incl. the new one
 *   h           [num_seqs, d_model] or NULL (Q-Cal, as in hils_score_select)
 *   out         [num_seqs, H_q, d]        io_dtype (written)
 *   lse         [num_seqs, H_q] fp32      (written, may be NULL)
 *   sel_idx     [num_seqs, H_kv, K] int32 (written, may be NULL)
 *   workspace: hils_workspace_size(cfg, HILS_WS_DECODE, num_seqs, max_pages).
 * Page ids outside [0, P) are not checked on the device: the caller owns
 * the block table.  cfg->B and cfg->N are ignored. */
hils_status_t hils_decode(const hils_config_t *cfg, int32_t num_seqs, const void *q, const void *k_cache,
                          const void *v_cache, const void *ksum_cache, const float *bsum_cache,
                          const int32_t *block_table, int32_t max_pages, const int32_t *seq_lens, const void *h,
                          const void *w_down, const void *w_up, int32_t d_model, int32_t r, void *out, float *lse,
                          int32_t *sel_idx, void *workspace, size_t workspace_bytes, hipStream_t stream);

/* hils_decode without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  Arguments, layouts and results are
 * those of hils_decode.  Its scratch is a static device array of
 * HILS_DECODE_NOALLOC_SCRATCH_BYTES inside the library, one per GPU, held
 * until the process ends; its address is looked up on the first call on
 * each device.  A call whose scratch need (hils_workspace_size(cfg,
 * HILS_WS_DECODE, num_seqs, max_pages)) exceeds that size returns
 * HILS_ERR_UNSUPPORTED.  The call allocates nothing.  Every call on one GPU
 * shares that GPU's array: calls that overlap in time on one GPU (other
 * streams, other threads) race and must be serialised by the caller.  The
 * stream must belong to the current device. */
#define HILS_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
hils_status_t hils_decode_noalloc(const hils_config_t *cfg, int32_t num_seqs, const void *q, const void *k_cache,
                                  const void *v_cache, const void *ksum_cache, const float *bsum_cache,
                                  const int32_t *block_table, int32_t max_pages, const int32_t *seq_lens,
                                  const void *h, const void *w_down, const void *w_up, int32_t d_model, int32_t r,
                                  void *out, float *lse, int32_t *sel_idx, hipStream_t stream);

/* Landmark summaries of chunks that complete while a sequence is served:
 * item i summarises the S keys held by page pages[i] of the paged key cache
 * with the landmark queries q_lm[i] (the summary definition of
 * hils_landmark_summarize: hyper.ai summary, 方法, the compressed key and
 * its entropy bias; the landmark query of a chunk exists once its S tokens
 * have arrived) and writes row pages[i] of the summary caches.
 *   k_cache     [num_pages, H_kv, S, d]   io_dtype; the page must be full
 *   q_lm        [num_items, H_lm, d]      io_dtype (as in hils_landmark_summarize
 *               for the other landmark modes)
 *   pages       [num_items] int32 (device); an id outside [0, num_pages)
 *               skips the item (nothing written), so a batch may carry -1
 *               for sequences with no completed chunk this step
 *   ksum_cache  [num_pages, H_lm, d]      summary_dtype (rows written)
 *   bsum_cache  [num_pages, H_lm]         fp32 (rows written)
 * Two items naming the same page race; the caller keeps ids distinct.
 * cfg->B and cfg->N are ignored. */
hils_status_t hils_summarize_pages(const hils_config_t *cfg, int32_t num_items, const void *k_cache,
                                   int32_t num_pages, const void *q_lm, const int32_t *pages, void *ksum_cache,
                                   float *bsum_cache, hipStream_t stream);

/* Chunked prefill over the paged cache: for each of cfg->B sequences, the
 * cfg->N new tokens at positions q_start .. q_start + N - 1 take the steps
 * of hils_score_select and hils_sparse_attend_fused (hyper.ai summary,
 * 方法: surrogate score, top-K, partition estimate and hierarchical
 * factorisation), with keys, values and summaries read through the block
 * table.  Row t of the result equals row q_start + t of a whole-sequence
 * prefill (and the decode step at that position).
 *   q_start     multiple of S, >= 0 (host value, shared by the B sequences)
 *   q           [B, H_q, N, d]            io_dtype, the new tokens
 *   k_cache,
 *   v_cache     [num_pages, H_kv, S, d]   io_dtype: keys 0 .. q_start+N-1
 *               already written (the new tokens' too)
 *   ksum_cache  [num_pages, H_lm, d]      summary_dtype; bsum_cache
 *               [num_pages, H_lm] fp32: rows of every chunk
 *               c < floor((q_start + N - 1) / S) - W/S already written
 *               (hils_summarize_pages / hils_landmark_summarize)
 *   block_table [B, max_pages] int32: logical chunk -> page; entries of
 *               chunks 0 .. ceil((q_start + N)/S) - 1 must lie in
 *               [0, num_pages) (not checked on the device)
 *   h, w_down, w_up, d_model, r: Q-Cal as in hils_score_select, h rows
 *               [B, N, d_model] of the new tokens (or NULL)
 *   sel_idx     [B, H_kv, N, K] int32, sel_score [B, H_q, N, K] fp32
 *               (written; may be NULL when K = 0)
 *   out         [B, H_q, N, d] io_dtype (written); lse [B, H_q, N] fp32
 *               (written, may be NULL)
 *   workspace   hils_prefill_paged_workspace_size(cfg, q_start, max_pages,
 *               h != NULL) bytes; with bf16 I/O its word 0 is the status
 *               word of hils_sparse_attend_fused.
 * num_pages <= 262144; q_start + N <= 8192 * S. */
hils_status_t hils_prefill_paged(const hils_config_t *cfg, int32_t q_start, const void *q, const void *k_cache,
                                 const void *v_cache, const void *ksum_cache, const float *bsum_cache,
                                 int32_t num_pages, const int32_t *block_table, int32_t max_pages, const void *h,
                                 const void *w_down, const void *w_up, int32_t d_model, int32_t r, int32_t *sel_idx,
                                 float *sel_score, void *out, float *lse, void *workspace, size_t workspace_bytes,
                                 hipStream_t stream);

/* Workspace bytes of hils_prefill_paged (0 with hils_last_error() set when
 * the configuration is rejected). */
size_t hils_prefill_paged_workspace_size(const hils_config_t *cfg, int32_t q_start, int32_t max_pages,
                                         int32_t with_qcal);

/* Gradients of the fused forward (hils_landmark_summarize ->
 * hils_score_select -> hils_sparse_attend_fused) with the selection held
 * fixed, for the loss sum(dout * out) + sum(dlse * lse) (hyper.ai summary,
 * 方法: the factorised attention weight makes the chunk scores, and through
 * them the landmark summaries, differentiable; the top-K choice is not).
 * The scoring query is q (Q-Cal's parameters get no gradient here).
 *   q, k, v, dout: as in the forward, io_dtype; lse [B,H_q,N] fp32 and
 *   sel_idx / sel_score: the forward's outputs (dout.out is formed from
 *   the recomputed weights, so out itself is not read); k_sum [B,H_lm,C,d] fp32
 *   (summary_dtype must be F32); q_lm as for hils_landmark_summarize;
 *   dlse [B,H_q,N] fp32 or NULL (zero).
 *   dq [B,H_q,N,d], dk, dv [B,H_kv,N,d], dq_lm [B,H_lm,C,d] ([H_lm,d] with
 *   HILS_LM_SHARED: summed over every sequence and chunk): fp32, written
 *   (dq_lm unused, may be NULL, with HILS_LM_MEAN).
 *   workspace: hils_workspace_size(cfg, HILS_WS_BACKWARD, 0, 0) bytes.
 * G <= 8.  Deterministic (no atomics). */
hils_status_t hils_sparse_attend_backward(const hils_config_t *cfg, const void *q, const void *k, const void *v,
                                          const void *q_lm, const float *k_sum, const int32_t *sel_idx,
                                          const float *sel_score, const float *lse, const void *dout,
                                          const float *dlse, float *dq, float *dk, float *dv, float *dq_lm,
                                          void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Dense causal attention, the full-attention baseline that the pages quote
 * HiLS's prefill speed against (wmrh.cn article on HiLS-Attention, results
 * table: prefill at a 512K context; hyper.ai summary, experiments paragraph
 * on inference efficiency).  For every query head h (kv head h / G):
 *   out[b,h,i] = sum_{j<=i} softmax_j(scale q[b,h,i] . k[b,g,j]) v[b,g,j]
 *   lse[b,h,i] = log sum_{j<=i} exp(scale q[b,h,i] . k[b,g,j])
 * i.e. the hyper.ai summary's block-sparse attention (方法, naive block-sparse
 * paragraph) with every key kept.
 *   q [B,H_q,N,d], k, v [B,H_kv,N,d]  bf16 (io_dtype must be BF16)
 *   out [B,H_q,N,d] bf16 (written); lse [B,H_q,N] fp32 (written, may be NULL)
 *   workspace: hils_workspace_size(cfg, HILS_WS_DENSE, 0, 0) bytes; word 0
 *   is the call's status word, as for hils_sparse_attend_fused (bit 1: a
 *   value of v beyond fp16's range; v enters the weighted sum as fp16).
 * d must be 64 or 128 (else HILS_ERR_UNSUPPORTED).  cfg's S, W, K, H_lm and
 * the landmark, aggregation and score modes are validated as for every call
 * and otherwise ignored. */
hils_status_t hils_dense_causal_attend(const hils_config_t *cfg, const void *q, const void *k, const void *v,
                                       void *out, float *lse, void *workspace, size_t workspace_bytes,
                                       hipStream_t stream);

/* Dense decode step, the full-attention baseline of the pages' decode speed
 * comparison (wmrh.cn article on HiLS-Attention, results table: decode at a
 * 512K context): the query at t = seq_lens[b] - 1 attends every key 0 .. t
 * of its sequence in the paged cache,
 *   out[b,h] = sum_{j<=t} softmax_j(scale q[b,h] . k_j) v_j over kv head h / G,
 *   lse[b,h] = log sum_{j<=t} exp(scale q[b,h] . k_j).
 *   q [num_seqs,H_q,d], k_cache, v_cache [P,H_kv,S,d], block_table
 *   [num_seqs,max_pages], seq_lens [num_seqs]: as for hils_decode (bf16)
 *   out [num_seqs,H_q,d] bf16 (written); lse [num_seqs,H_q] fp32 (written, may
 *   be NULL)
 *   workspace: hils_workspace_size(cfg, HILS_WS_DENSE_DECODE, num_seqs,
 *   max_pages) bytes.
 * Requires bf16 I/O, d = 128 and S = 64 (else HILS_ERR_UNSUPPORTED).  Page
 * ids are not checked on the device; seq_lens are clamped to [1, max_pages *
 * S].  cfg->B, N, W, K and the summary fields are ignored. */
hils_status_t hils_dense_decode(const hils_config_t *cfg, int32_t num_seqs, const void *q, const void *k_cache,
                                const void *v_cache, const int32_t *block_table, int32_t max_pages,
                                const int32_t *seq_lens, void *out, float *lse, void *workspace,
                                size_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace the given call needs (0 if none); 0 with
 * hils_last_error() set when the configuration is rejected.  num_seqs and
 * max_pages are used by HILS_WS_DECODE only. */
size_t hils_workspace_size(const hils_config_t *cfg, int which, int32_t num_seqs, int32_t max_pages);

/* Thread-local message describing the last non-OK status of this thread. */
const char *hils_last_error(void);

/* Library version: major * 10000 + minor * 100 + patch. */
int hils_version(void);

#ifdef __cplusplus
}
#endif

#endif /* HILS_H */
