// hils_internal.hpp -- host-side launcher interface between the C ABI layer
// (hils_api.cpp) and the kernel translation units.  Every launcher assumes
// its arguments were validated by the ABI layer and only enqueues work.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

#include <algorithm>
#include <stdint.h>

namespace hils {

// Validated, resolved configuration.
struct Shape {
    int B, N, H_q, H_kv, H_lm, D, S, W, K, M;
    int G;      // H_q / H_kv
    int GLM;    // landmark heads per kv head: H_lm / H_kv (1 or G)
    int C;      // floor(N / S) completed chunks
    int CA;     // ceil(N / S) chunks incl. a partial last one
    bool io_bf16, sum_bf16;
    float scale;
    int lm_mode;   // landmark queries: 0 per chunk, 1 one shared per landmark head, 2 none (q' = 0)
    int agg_mode;  // group aggregation: 0 max of s^, 1 max of s^ - LSE over the candidates
    int wait_spins;  // bound on each wait of the fused kernel (pauses)
    int score_mode;  // score/select form: 0 auto, 1 two-pass, 2 streaming
    int attend_mode; // selected-chunk attention form: 0 auto, 1 query-major walk, 2 chunk-major
    int attend_slab; // chunk-major: query rows per slab (0: bounded by the partial buffer cap)
    // Paged prefill (q0 = 0, Nk = N, bt = null for the contiguous layout):
    // the N query rows are positions q0 .. q0 + N - 1 (q0 % S == 0) of
    // sequences whose keys 0 .. Nk - 1 = q0 + N - 1 live in a paged cache
    // [P, H_kv, S, D]; chunk c of sequence b is page bt[b * max_pages + c],
    // and its summaries are row bt[b * max_pages + c] of the paged summary
    // cache.  C is then the candidate bound of the last row and CA the
    // chunks holding keys 0 .. Nk - 1.  max_pages > 0 marks the paged layout.
    int q0, Nk;
    const int32_t *bt;
    int max_pages;
};

// ---- kernel 1: landmark summary
// pages == null: every completed chunk of k [B, H_kv, N, D].  Otherwise
// item b < B summarises page pages[b] of a paged cache (N = S, C = 1) with
// landmark queries q_lm[b] and writes summary row pages[b]; items whose id
// is outside [0, num_pages) are skipped.
hipError_t launch_landmark_summary(const Shape &s, const void *k, const void *q_lm, void *k_sum, float *b_sum,
                                   const int32_t *pages, int num_pages, hipStream_t st);

// ---- kernel 2: score + select
struct ScoreWorkspace {
    bool topk;          // streaming top-K kernel (no per-candidate scores in memory)
    void *ksb;          // [B,H_lm,C,D] bf16 k1 = bf16(k_sum)
    void *ksb2;         // [B,H_lm,C,D] bf16 k2 = bf16(k_sum - k1) (fp32 summaries)
    void *ksb3;         // [B,H_lm,C,D] bf16 k3 = bf16(k_sum - k1 - k2) (fp32 summaries, streaming kernel)
    float *heads;       // [B,H_kv,N,CAP,G] per-head scores of each row's listed chunks (streaming kernel)
    float *kcm;         // [B,H_kv,C,GLM,D] fp32 chunk-major copy of k_sum (two-kernel path)
    float *knorm;       // [B,H_lm] max_c ||k'_c||
    float *err;         // [B,H_kv,N] per-row bound of the approximate group score
    float *agg;         // ragged approximate group scores, per (b,g): per_bg entries
    int64_t per_bg;     // entries per (b, g)
    float *q_s;         // [B,H_q,N,D] Q-Cal scoring queries (fp32) or null
    float *bsum;        // [B,H_lm,C] b_sum gathered from the paged cache (paged prefill) or null
    float *lse;         // [B,H_q,N] per-head log-sum-exp over the candidates (normalised aggregation) or null
};
int64_t score_agg_entries_per_bg(const Shape &s);
// streaming top-K kernel (score_topk.hip): whether its LDS fits the shape,
// its per-row list capacity, and the launch (qv: bf16 q or fp32 scoring
// queries)
bool score_topk_supported(const Shape &s);
int score_topk_capacity(const Shape &s);
// whether score/select runs the streaming kernel for this shape and mode
bool score_use_topk(const Shape &s);
hipError_t launch_score_topk(const Shape &s, const void *qv, bool q_fp32, const ScoreWorkspace &ws,
                             const float *b_sum, int32_t *sel_idx, float *sel_score, hipStream_t st);
size_t score_workspace_bytes(const Shape &s, bool qcal);
void score_workspace_carve(const Shape &s, bool qcal, void *base, ScoreWorkspace &ws);
hipError_t launch_score_select(const Shape &s, const void *q, const void *k_sum, const float *b_sum, const void *h,
                               const void *w_down, const void *w_up, int d_model, int r, int32_t *sel_idx,
                               float *sel_score, const ScoreWorkspace &ws, hipStream_t st);

// ---- kernel 3: fused sparse attention
// bf16 I/O: a 256-byte status block (word 0: bit 0 set when a bounded wait
// of the kernel gave up, bit 1 when a value of v is beyond fp16's range)
// followed by the transposed fp16 copy of v; fp32: none.
constexpr size_t FUSED_STATUS_BYTES = 256;
size_t fused_workspace_bytes(const Shape &s);
// Whether the fused kernel has a block shape whose LDS fits this shape
// (every combination with K <= 32 does; large K with G = 1 at S = 128 may not).
bool sparse_attend_supported(const Shape &s);
// status: word zeroed by the launch and set when a wait gives up (bf16 I/O);
// vt_ws: room for the transposed copy of v.
hipError_t launch_sparse_attend(const Shape &s, const void *q, const void *k, const void *v, const int32_t *sel_idx,
                                const float *sel_score, void *out, float *lse, uint32_t *status, void *vt_ws,
                                hipStream_t st);

// Chunk-major form of the selected chunks (attend_cm.hip): whether it runs
// for this shape and mode, its workspace (after the V^T copy: chunk lists,
// row maxima and the fp16 partial buffer of one slab), the slab rows, and
// the launch (V^T pre-pass, then per slab: count, scan, fill, chunk-major
// attention, and the window kernel started from the partials).
bool attend_use_cm(const Shape &s);
size_t cm_workspace_bytes(const Shape &s);
int cm_slab_rows(const Shape &s);
hipError_t launch_sparse_attend_cm(const Shape &s, const void *q, const void *k, const void *v,
                                   const int32_t *sel_idx, const float *sel_score, void *out, float *lse,
                                   uint32_t *status, void *vt_ws, void *cm_ws, hipStream_t st);
// The window kernel's chunk-major variant (attend.hip): rows s0 .. s0 + NS - 1
// start from the summed partials part [B, H_kv, NS, K, G D] and walk the window.
bool window_after_cm_supported(const Shape &s);
hipError_t launch_window_after_cm(const Shape &s, const void *q, const void *k, const void *vt,
                                  const int32_t *sel_idx, const float *sel_score, void *out, float *lse,
                                  uint32_t *status, const void *part, int s0, int NS, hipStream_t st);

// Status word cleared, then v [B, H_kv, Nk, D] (or the paged cache with
// s.bt) copied to vt as fp16 [B, H_kv, CA, D, S] with the keys of each 32-key
// step in MFMA accumulator order; bit 1 of *status is set for a value beyond
// fp16's range.
hipError_t launch_vt_prepass(const Shape &s, const void *v, void *vt, uint32_t *status, hipStream_t st);

// ---- dense causal attention (bf16, d = 64 or 128): the full-attention
// point of comparison.  Workspace: the status block, then the fp16 V^T copy
// in 64-key tiles.
bool dense_attend_supported(const Shape &s);
size_t dense_workspace_bytes(const Shape &s);
hipError_t launch_dense_attend(const Shape &s, const void *q, const void *k, const void *v, void *out, float *lse,
                               void *workspace, hipStream_t st);

// ---- kernel 4: decode
size_t decode_workspace_bytes(const Shape &s, int num_seqs, int max_pages);
// Largest candidate range one phase-A block may own (LDS capacity).
constexpr int DECODE_SPLIT_CAP = 512;
int decode_splits(const Shape &s, int max_pages);
hipError_t launch_decode(const Shape &s, int num_seqs, const void *q, const void *k_cache, const void *v_cache,
                         const void *ksum_cache, const float *bsum_cache, const int32_t *block_table, int max_pages,
                         const int32_t *seq_lens, int max_seq_len, const void *h, const void *w_down,
                         const void *w_up, int d_model, int r, void *out, float *lse, int32_t *sel_idx,
                         void *workspace, hipStream_t st);

// Dense decode (bf16, d = 128, S = 64 pages): the query at seq_len - 1 over
// every key of its sequence; the full-attention point of comparison for a
// decode step.  Workspace: per-split partial states.
bool dense_decode_supported(const Shape &s);
size_t dense_decode_workspace_bytes(const Shape &s, int num_seqs, int max_pages);
hipError_t launch_dense_decode(const Shape &s, int num_seqs, const void *q, const void *k_cache,
                               const void *v_cache, const int32_t *block_table, int max_pages,
                               const int32_t *seq_lens, void *out, float *lse, void *workspace, hipStream_t st);

// ---- backward of the fused attention (fixed selection), incl. the summary
size_t backward_workspace_bytes(const Shape &s);
hipError_t launch_backward(const Shape &s, const void *q, const void *k, const void *v, const void *q_lm,
                           const float *k_sum, const int32_t *sel_idx, const float *sel_score, const float *lse,
                           const void *dout, const float *dlse, float *dq, float *dk, float *dv, float *dq_lm,
                           void *workspace, hipStream_t st);

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Record msg as the calling thread's last error (hils_last_error) and
// return status.
int report_error(int status, const char *msg);

}  // namespace hils
