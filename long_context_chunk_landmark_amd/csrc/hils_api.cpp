// hils_api.cpp -- the C ABI of libhils: argument validation, workspace
// accounting and dispatch to the kernel launchers.  Validation happens on
// the host before anything is enqueued; on failure nothing is written.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "../../include/hils.h"
#include "hils_internal.hpp"

namespace {

thread_local char g_err[512] = "";

hils_status_t fail(hils_status_t st, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return st;
}

hils_status_t ok() {
    g_err[0] = '\0';
    return HILS_OK;
}

hils_status_t hip_status(hipError_t e, const char *what) {
    if (e == hipSuccess) return ok();
    return fail(HILS_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Resolve and validate the configuration.  need_seq: B and N matter.
hils_status_t resolve(const hils_config_t *cfg, bool need_seq, hils::Shape &s) {
    if (!cfg) return fail(HILS_ERR_INVALID_ARG, "cfg is NULL");
    s.B = need_seq ? cfg->B : 1;
    s.N = need_seq ? cfg->N : 0;
    s.H_q = cfg->H_q;
    s.H_kv = cfg->H_kv;
    s.H_lm = cfg->H_lm;
    s.D = cfg->d;
    s.S = cfg->S;
    s.W = cfg->W;
    s.K = cfg->K;
    s.M = cfg->M;
    if (need_seq && (s.B < 0 || s.N < 0)) return fail(HILS_ERR_INVALID_ARG, "B=%d N=%d must be >= 0", s.B, s.N);
    if (s.H_q <= 0 || s.H_kv <= 0 || s.H_lm <= 0 || s.D <= 0 || s.S <= 0 || s.W < 0 || s.K < 0)
        return fail(HILS_ERR_INVALID_ARG, "head counts, d and S must be > 0; W, K must be >= 0");
    if (s.H_q % s.H_kv) return fail(HILS_ERR_INVALID_ARG, "H_q=%d is not a multiple of H_kv=%d", s.H_q, s.H_kv);
    if (s.H_lm != s.H_q && s.H_lm != s.H_kv)
        return fail(HILS_ERR_INVALID_ARG, "H_lm=%d must equal H_q=%d or H_kv=%d", s.H_lm, s.H_q, s.H_kv);
    if (s.W % s.S) return fail(HILS_ERR_INVALID_ARG, "W=%d is not a multiple of S=%d", s.W, s.S);
    if (cfg->io_dtype != HILS_F32 && cfg->io_dtype != HILS_BF16)
        return fail(HILS_ERR_INVALID_ARG, "io_dtype=%d unknown", cfg->io_dtype);
    if (cfg->summary_dtype != HILS_F32 && cfg->summary_dtype != HILS_BF16)
        return fail(HILS_ERR_INVALID_ARG, "summary_dtype=%d unknown", cfg->summary_dtype);
    if (!(cfg->scale >= 0.f) || !isfinite(cfg->scale)) return fail(HILS_ERR_INVALID_ARG, "scale must be finite, >= 0");
    s.G = s.H_q / s.H_kv;
    s.GLM = s.H_lm / s.H_kv;
    if (s.D != 64 && s.D != 128) return fail(HILS_ERR_UNSUPPORTED, "d=%d: supported 64, 128", s.D);
    if (s.S != 64 && s.S != 128) return fail(HILS_ERR_UNSUPPORTED, "S=%d: supported 64, 128", s.S);
    if (s.G != 1 && s.G != 2 && s.G != 4 && s.G != 8)
        return fail(HILS_ERR_UNSUPPORTED, "G=H_q/H_kv=%d: supported 1, 2, 4, 8", s.G);
    if (s.K > 128) return fail(HILS_ERR_UNSUPPORTED, "K=%d: supported 0..128", s.K);
    s.C = s.S ? s.N / s.S : 0;
    s.CA = s.S ? (s.N + s.S - 1) / s.S : 0;
    if (need_seq && s.C > 8192) return fail(HILS_ERR_UNSUPPORTED, "N/S=%d chunks: supported up to 8192", s.C);
    if (cfg->landmark_mode < HILS_LM_CHUNK || cfg->landmark_mode > HILS_LM_MEAN)
        return fail(HILS_ERR_INVALID_ARG, "landmark_mode=%d unknown", cfg->landmark_mode);
    if (cfg->agg_mode != HILS_AGG_MAX && cfg->agg_mode != HILS_AGG_NORMALIZED)
        return fail(HILS_ERR_INVALID_ARG, "agg_mode=%d unknown", cfg->agg_mode);
    if (cfg->wait_spins < 0) return fail(HILS_ERR_INVALID_ARG, "wait_spins=%d must be >= 0", cfg->wait_spins);
    if (cfg->score_mode < HILS_SCORE_AUTO || cfg->score_mode > HILS_SCORE_STREAMING)
        return fail(HILS_ERR_INVALID_ARG, "score_mode=%d unknown", cfg->score_mode);
    s.score_mode = cfg->score_mode;
    if (cfg->attend_mode < HILS_ATTEND_AUTO || cfg->attend_mode > HILS_ATTEND_CHUNK_MAJOR)
        return fail(HILS_ERR_INVALID_ARG, "attend_mode=%d unknown", cfg->attend_mode);
    if (cfg->attend_slab < 0) return fail(HILS_ERR_INVALID_ARG, "attend_slab=%d must be >= 0", cfg->attend_slab);
    s.attend_mode = cfg->attend_mode;
    s.attend_slab = cfg->attend_slab;
    s.lm_mode = cfg->landmark_mode;
    s.agg_mode = cfg->agg_mode;
    s.wait_spins = cfg->wait_spins > 0 ? cfg->wait_spins : (1 << 18);
    s.io_bf16 = cfg->io_dtype == HILS_BF16;
    s.sum_bf16 = cfg->summary_dtype == HILS_BF16;
    s.scale = cfg->scale > 0.f ? cfg->scale : 1.0f / sqrtf((float)s.D);
    s.q0 = 0;
    s.Nk = s.N;
    s.bt = nullptr;
    s.max_pages = 0;
    return ok();
}

// Largest page count of a paged cache the walk entries of the fused kernel
// can address (18 bits above a 14-bit chunk id).
constexpr int32_t PAGED_MAX_PAGES = 1 << 18;

// Paged prefill: B sequences, N new rows each at positions q_start ..
// q_start + N - 1, keys 0 .. q_start + N - 1 in the paged cache.
hils_status_t resolve_paged(const hils_config_t *cfg, int32_t q_start, int32_t num_pages, int32_t max_pages,
                            hils::Shape &s) {
    hils_status_t st = resolve(cfg, true, s);
    if (st) return st;
    if (q_start < 0 || q_start % s.S)
        return fail(HILS_ERR_INVALID_ARG, "q_start=%d must be >= 0 and a multiple of S=%d", q_start, s.S);
    if (num_pages <= 0 || max_pages <= 0)
        return fail(HILS_ERR_INVALID_ARG, "num_pages=%d, max_pages=%d must be >= 1", num_pages, max_pages);
    if (num_pages > PAGED_MAX_PAGES)
        return fail(HILS_ERR_UNSUPPORTED, "num_pages=%d: supported up to %d", num_pages, PAGED_MAX_PAGES);
    const int64_t Nk = (int64_t)q_start + s.N;
    const int64_t CA = (Nk + s.S - 1) / s.S;
    if (CA > 8192) return fail(HILS_ERR_UNSUPPORTED, "q_start + N = %lld keys: supported up to 8192 chunks", (long long)Nk);
    if (CA > max_pages)
        return fail(HILS_ERR_INVALID_ARG, "q_start + N = %lld keys need %lld pages, block table has %d", (long long)Nk,
                    (long long)CA, max_pages);
    s.q0 = q_start;
    s.Nk = (int)Nk;
    s.CA = (int)CA;
    // candidates of the last row: chunks below its window
    s.C = s.N > 0 ? std::max(0, (int)((Nk - 1) / s.S) - s.W / s.S) : 0;
    s.max_pages = max_pages;
    return ok();
}

// [fused status block][score workspace][transposed v]: the status word sits
// at offset 0 as in the fused entry point's workspace.
size_t paged_workspace_bytes(const hils::Shape &s, bool qcal) {
    return hils::align_up(hils::score_workspace_bytes(s, qcal), 256) + hils::fused_workspace_bytes(s) +
           (s.io_bf16 ? 0 : hils::FUSED_STATUS_BYTES);
}

// An explicit streaming score/select on a shape its kernel does not cover.
hils_status_t check_score_mode(const hils::Shape &s) {
    if (s.score_mode == HILS_SCORE_STREAMING && !hils::score_topk_supported(s))
        return fail(HILS_ERR_UNSUPPORTED, "streaming score/select does not cover d=%d, G=%d, K=%d", s.D, s.G, s.K);
    return HILS_OK;
}

hils_status_t check_ptr(const void *p, const char *name) {
    if (!p) return fail(HILS_ERR_INVALID_ARG, "%s is NULL", name);
    if (!aligned16(p)) return fail(HILS_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
    return HILS_OK;
}

hils_status_t check_qcal(const void *h, const void *w_down, const void *w_up, int32_t d_model, int32_t r) {
    if (!h) return HILS_OK;
    hils_status_t st;
    if ((st = check_ptr(h, "h")) || (st = check_ptr(w_down, "w_down")) || (st = check_ptr(w_up, "w_up"))) return st;
    if (d_model <= 0 || r <= 0) return fail(HILS_ERR_INVALID_ARG, "d_model=%d, r=%d must be > 0", d_model, r);
    if (r > 64) return fail(HILS_ERR_UNSUPPORTED, "Q-Cal rank r=%d: supported up to 64", r);
    return HILS_OK;
}

}  // namespace

namespace hils {
int report_error(int status, const char *msg) {
    snprintf(g_err, sizeof(g_err), "%s", msg);
    return status;
}
}  // namespace hils

extern "C" {

const char *hils_last_error(void) { return g_err; }

int hils_version(void) { return 10100; }

size_t hils_workspace_size(const hils_config_t *cfg, int which, int32_t num_seqs, int32_t max_pages) {
    hils::Shape s;
    const bool seq = which != HILS_WS_DECODE && which != HILS_WS_DENSE_DECODE;
    if (resolve(cfg, seq, s) != HILS_OK) return 0;
    switch (which) {
        case HILS_WS_SCORE: return hils::score_workspace_bytes(s, false);
        case HILS_WS_SCORE_QCAL: return hils::score_workspace_bytes(s, true);
        case HILS_WS_FUSED: return hils::fused_workspace_bytes(s);
        case HILS_WS_BACKWARD: return hils::backward_workspace_bytes(s);
        case HILS_WS_DENSE: return hils::dense_workspace_bytes(s);
        case HILS_WS_DENSE_DECODE:
            if (num_seqs < 0 || max_pages < 1) {
                fail(HILS_ERR_INVALID_ARG, "num_seqs must be >= 0 and max_pages >= 1");
                return 0;
            }
            return hils::dense_decode_workspace_bytes(s, num_seqs, max_pages);
        case HILS_WS_DECODE:
            if (num_seqs < 0 || max_pages < 0) {
                fail(HILS_ERR_INVALID_ARG, "num_seqs, max_pages must be >= 0");
                return 0;
            }
            return hils::decode_workspace_bytes(s, num_seqs, max_pages);
        default: fail(HILS_ERR_INVALID_ARG, "unknown workspace kind %d", which); return 0;
    }
}

hils_status_t hils_landmark_summarize(const hils_config_t *cfg, const void *k, const void *q_lm, void *k_sum,
                                      float *b_sum, hipStream_t stream) {
    hils::Shape s;
    hils_status_t st = resolve(cfg, true, s);
    if (st) return st;
    if ((int64_t)s.B * s.H_lm * s.C == 0) return ok();
    if ((st = check_ptr(k, "k")) || (st = check_ptr(k_sum, "k_sum")) || (st = check_ptr(b_sum, "b_sum"))) return st;
    if (s.lm_mode != HILS_LM_MEAN && (st = check_ptr(q_lm, "q_lm"))) return st;
    return hip_status(hils::launch_landmark_summary(s, k, q_lm, k_sum, b_sum, nullptr, 0, stream),
                      "landmark summary launch");
}

hils_status_t hils_summarize_pages(const hils_config_t *cfg, int32_t num_items, const void *k_cache,
                                   int32_t num_pages, const void *q_lm, const int32_t *pages, void *ksum_cache,
                                   float *bsum_cache, hipStream_t stream) {
    hils::Shape s;
    hils_status_t st = resolve(cfg, false, s);
    if (st) return st;
    if (num_items < 0 || num_pages < 0) return fail(HILS_ERR_INVALID_ARG, "num_items, num_pages must be >= 0");
    if (num_items == 0 || num_pages == 0) return ok();
    if ((st = check_ptr(k_cache, "k_cache")) || (st = check_ptr(pages, "pages")) ||
        (st = check_ptr(ksum_cache, "ksum_cache")) || (st = check_ptr(bsum_cache, "bsum_cache")))
        return st;
    if (s.lm_mode != HILS_LM_MEAN && (st = check_ptr(q_lm, "q_lm"))) return st;
    // item b = one "sequence" of a single S-key chunk (page pages[b])
    s.B = num_items;
    s.N = s.S;
    s.C = s.CA = 1;
    s.Nk = s.N;
    return hip_status(hils::launch_landmark_summary(s, k_cache, q_lm, ksum_cache, bsum_cache, pages, num_pages, stream),
                      "paged landmark summary launch");
}

hils_status_t hils_score_select(const hils_config_t *cfg, const void *q, const void *k_sum, const float *b_sum,
                                const void *h, const void *w_down, const void *w_up, int32_t d_model, int32_t r,
                                int32_t *sel_idx, float *sel_score, void *workspace, size_t workspace_bytes,
                                hipStream_t stream) {
    hils::Shape s;
    hils_status_t st = resolve(cfg, true, s);
    if (st) return st;
    if ((int64_t)s.B * s.N == 0 || s.K == 0) return ok();
    if ((st = check_score_mode(s))) return st;
    if ((st = check_ptr(q, "q")) || (st = check_ptr(sel_idx, "sel_idx")) || (st = check_ptr(sel_score, "sel_score")))
        return st;
    if (s.C > 0 && ((st = check_ptr(k_sum, "k_sum")) || (st = check_ptr(b_sum, "b_sum")))) return st;
    if ((st = check_qcal(h, w_down, w_up, d_model, r))) return st;
    const bool qcal = h != nullptr;
    const size_t need = hils::score_workspace_bytes(s, qcal);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(HILS_ERR_WORKSPACE, "score_select needs %zu workspace bytes, got %zu", need,
                    workspace ? workspace_bytes : (size_t)0);
    if (need > 0 && !aligned16(workspace)) return fail(HILS_ERR_INVALID_ARG, "workspace is not 16-byte aligned");
    hils::ScoreWorkspace ws;
    hils::score_workspace_carve(s, qcal, workspace, ws);
    return hip_status(hils::launch_score_select(s, q, k_sum, b_sum, h, w_down, w_up, d_model, r, sel_idx, sel_score,
                                                ws, stream),
                      "score/select launch");
}

hils_status_t hils_sparse_attend_fused(const hils_config_t *cfg, const void *q, const void *k, const void *v,
                                       const int32_t *sel_idx, const float *sel_score, void *out, float *lse,
                                       void *workspace, size_t workspace_bytes, hipStream_t stream) {
    hils::Shape s;
    hils_status_t st = resolve(cfg, true, s);
    if (st) return st;
    if ((int64_t)s.B * s.N == 0) return ok();
    if ((st = check_ptr(q, "q")) || (st = check_ptr(k, "k")) || (st = check_ptr(v, "v")) ||
        (st = check_ptr(out, "out")))
        return st;
    if (s.K > 0 && ((st = check_ptr(sel_idx, "sel_idx")) || (st = check_ptr(sel_score, "sel_score")))) return st;
    if (lse && !aligned16(lse)) return fail(HILS_ERR_INVALID_ARG, "lse is not 16-byte aligned");
    if (!hils::sparse_attend_supported(s))
        return fail(HILS_ERR_UNSUPPORTED, "no fused-attention block shape fits LDS for G=%d, S=%d, d=%d, K=%d", s.G, s.S,
                    s.D, s.K);
    const size_t need = hils::fused_workspace_bytes(s);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(HILS_ERR_WORKSPACE, "sparse_attend_fused needs %zu workspace bytes, got %zu", need,
                    workspace ? workspace_bytes : (size_t)0);
    if (need > 0 && !aligned16(workspace)) return fail(HILS_ERR_INVALID_ARG, "workspace is not 16-byte aligned");
    uint32_t *status = s.io_bf16 ? (uint32_t *)workspace : nullptr;
    void *vt_ws = s.io_bf16 ? (char *)workspace + hils::FUSED_STATUS_BYTES : nullptr;
    return hip_status(hils::launch_sparse_attend(s, q, k, v, sel_idx, sel_score, out, lse, status, vt_ws, stream),
                      "sparse attention launch");
}

hils_status_t hils_dense_causal_attend(const hils_config_t *cfg, const void *q, const void *k, const void *v,
                                       void *out, float *lse, void *workspace, size_t workspace_bytes,
                                       hipStream_t stream) {
    hils::Shape s;
    hils_status_t st = resolve(cfg, true, s);
    if (st) return st;
    if (!hils::dense_attend_supported(s))
        return fail(HILS_ERR_UNSUPPORTED, "dense attention covers bf16 I/O with d = 64 or 128 (io_dtype=%d, d=%d)",
                    cfg->io_dtype, s.D);
    if ((int64_t)s.B * s.N == 0) return ok();
    if ((st = check_ptr(q, "q")) || (st = check_ptr(k, "k")) || (st = check_ptr(v, "v")) ||
        (st = check_ptr(out, "out")))
        return st;
    if (lse && !aligned16(lse)) return fail(HILS_ERR_INVALID_ARG, "lse is not 16-byte aligned");
    const size_t need = hils::dense_workspace_bytes(s);
    if (!workspace || workspace_bytes < need)
        return fail(HILS_ERR_WORKSPACE, "dense_causal_attend needs %zu workspace bytes, got %zu", need,
                    workspace ? workspace_bytes : (size_t)0);
    if (!aligned16(workspace)) return fail(HILS_ERR_INVALID_ARG, "workspace is not 16-byte aligned");
    return hip_status(hils::launch_dense_attend(s, q, k, v, out, lse, workspace, stream), "dense attention launch");
}

hils_status_t hils_decode(const hils_config_t *cfg, int32_t num_seqs, const void *q, const void *k_cache,
                          const void *v_cache, const void *ksum_cache, const float *bsum_cache,
                          const int32_t *block_table, int32_t max_pages, const int32_t *seq_lens, const void *h,
                          const void *w_down, const void *w_up, int32_t d_model, int32_t r, void *out, float *lse,
                          int32_t *sel_idx, void *workspace, size_t workspace_bytes, hipStream_t stream) {
    hils::Shape s;
    hils_status_t st = resolve(cfg, false, s);
    if (st) return st;
    if (num_seqs < 0 || max_pages < 0) return fail(HILS_ERR_INVALID_ARG, "num_seqs, max_pages must be >= 0");
    if (num_seqs == 0) return ok();
    if (max_pages == 0) return fail(HILS_ERR_INVALID_ARG, "max_pages must be >= 1");
    if ((int64_t)max_pages > 65536) return fail(HILS_ERR_UNSUPPORTED, "max_pages=%d: supported up to 65536", max_pages);
    if ((max_pages + hils::decode_splits(s, max_pages) - 1) / hils::decode_splits(s, max_pages) >
        hils::DECODE_SPLIT_CAP)
        return fail(HILS_ERR_UNSUPPORTED, "max_pages=%d with K=%d exceeds the decode scoring split capacity",
                    max_pages, s.K);
    if ((st = check_ptr(q, "q")) || (st = check_ptr(k_cache, "k_cache")) || (st = check_ptr(v_cache, "v_cache")) ||
        (st = check_ptr(ksum_cache, "ksum_cache")) || (st = check_ptr(bsum_cache, "bsum_cache")) ||
        (st = check_ptr(block_table, "block_table")) || (st = check_ptr(seq_lens, "seq_lens")) ||
        (st = check_ptr(out, "out")))
        return st;
    if (lse && !aligned16(lse)) return fail(HILS_ERR_INVALID_ARG, "lse is not 16-byte aligned");
    if (sel_idx && !aligned16(sel_idx)) return fail(HILS_ERR_INVALID_ARG, "sel_idx is not 16-byte aligned");
    if ((st = check_qcal(h, w_down, w_up, d_model, r))) return st;
    const size_t need = hils::decode_workspace_bytes(s, num_seqs, max_pages);
    if (!workspace || workspace_bytes < need)
        return fail(HILS_ERR_WORKSPACE, "decode needs %zu workspace bytes, got %zu", need,
                    workspace ? workspace_bytes : (size_t)0);
    if (!aligned16(workspace)) return fail(HILS_ERR_INVALID_ARG, "workspace is not 16-byte aligned");
    return hip_status(hils::launch_decode(s, num_seqs, q, k_cache, v_cache, ksum_cache, bsum_cache, block_table,
                                          max_pages, seq_lens, 0, h, w_down, w_up, d_model, r, out, lse, sel_idx,
                                          workspace, stream),
                      "decode launch");
}

hils_status_t hils_dense_decode(const hils_config_t *cfg, int32_t num_seqs, const void *q, const void *k_cache,
                                const void *v_cache, const int32_t *block_table, int32_t max_pages,
                                const int32_t *seq_lens, void *out, float *lse, void *workspace,
                                size_t workspace_bytes, hipStream_t stream) {
    hils::Shape s;
    hils_status_t st = resolve(cfg, false, s);
    if (st) return st;
    if (!hils::dense_decode_supported(s))
        return fail(HILS_ERR_UNSUPPORTED, "dense decode covers bf16 I/O with d = 128 and S = 64 (io_dtype=%d, d=%d, S=%d)",
                    cfg->io_dtype, s.D, s.S);
    if (num_seqs < 0 || max_pages < 0) return fail(HILS_ERR_INVALID_ARG, "num_seqs, max_pages must be >= 0");
    if (num_seqs == 0) return ok();
    if (max_pages == 0) return fail(HILS_ERR_INVALID_ARG, "max_pages must be >= 1");
    if (num_seqs > 65535) return fail(HILS_ERR_UNSUPPORTED, "num_seqs=%d: supported up to 65535", num_seqs);
    if ((st = check_ptr(q, "q")) || (st = check_ptr(k_cache, "k_cache")) || (st = check_ptr(v_cache, "v_cache")) ||
        (st = check_ptr(block_table, "block_table")) || (st = check_ptr(seq_lens, "seq_lens")) ||
        (st = check_ptr(out, "out")))
        return st;
    if (lse && !aligned16(lse)) return fail(HILS_ERR_INVALID_ARG, "lse is not 16-byte aligned");
    const size_t need = hils::dense_decode_workspace_bytes(s, num_seqs, max_pages);
    if (!workspace || workspace_bytes < need)
        return fail(HILS_ERR_WORKSPACE, "dense decode needs %zu workspace bytes, got %zu", need,
                    workspace ? workspace_bytes : (size_t)0);
    if (!aligned16(workspace)) return fail(HILS_ERR_INVALID_ARG, "workspace is not 16-byte aligned");
    return hip_status(hils::launch_dense_decode(s, num_seqs, q, k_cache, v_cache, block_table, max_pages, seq_lens,
                                                out, lse, workspace, stream),
                      "dense decode launch");
}

hils_status_t hils_sparse_attend_backward(const hils_config_t *cfg, const void *q, const void *k, const void *v,
                                          const void *q_lm, const float *k_sum, const int32_t *sel_idx,
                                          const float *sel_score, const float *lse, const void *dout,
                                          const float *dlse, float *dq, float *dk, float *dv, float *dq_lm,
                                          void *workspace, size_t workspace_bytes, hipStream_t stream) {
    hils::Shape s;
    hils_status_t st = resolve(cfg, true, s);
    if (st) return st;
    if (s.sum_bf16) return fail(HILS_ERR_UNSUPPORTED, "backward: summary_dtype must be F32");
    if (s.G > 8) return fail(HILS_ERR_UNSUPPORTED, "backward: G=%d, supported up to 8", s.G);
    if ((int64_t)s.B * s.N == 0) return ok();
    if ((st = check_ptr(q, "q")) || (st = check_ptr(k, "k")) || (st = check_ptr(v, "v")) ||
        (st = check_ptr(lse, "lse")) || (st = check_ptr(dout, "dout")) || (st = check_ptr(dq, "dq")) ||
        (st = check_ptr(dk, "dk")) || (st = check_ptr(dv, "dv")))
        return st;
    if (s.K > 0 && ((st = check_ptr(sel_idx, "sel_idx")) || (st = check_ptr(sel_score, "sel_score")))) return st;
    if (s.C > 0 && ((st = check_ptr(k_sum, "k_sum")) || (s.lm_mode != HILS_LM_MEAN && (st = check_ptr(q_lm, "q_lm"))) ||
                    (s.lm_mode != HILS_LM_MEAN && (st = check_ptr(dq_lm, "dq_lm")))))
        return st;
    if (dlse && !aligned16(dlse)) return fail(HILS_ERR_INVALID_ARG, "dlse is not 16-byte aligned");
    const size_t need = hils::backward_workspace_bytes(s);
    if (!workspace || workspace_bytes < need)
        return fail(HILS_ERR_WORKSPACE, "backward needs %zu workspace bytes, got %zu", need,
                    workspace ? workspace_bytes : (size_t)0);
    if (!aligned16(workspace)) return fail(HILS_ERR_INVALID_ARG, "workspace is not 16-byte aligned");
    return hip_status(hils::launch_backward(s, q, k, v, q_lm, k_sum, sel_idx, sel_score, lse, dout, dlse, dq, dk, dv,
                                            dq_lm, workspace, stream),
                      "backward launch");
}

size_t hils_prefill_paged_workspace_size(const hils_config_t *cfg, int32_t q_start, int32_t max_pages,
                                         int32_t with_qcal) {
    hils::Shape s;
    if (resolve_paged(cfg, q_start, 1, max_pages, s) != HILS_OK) return 0;
    return paged_workspace_bytes(s, with_qcal != 0);
}

hils_status_t hils_prefill_paged(const hils_config_t *cfg, int32_t q_start, const void *q, const void *k_cache,
                                 const void *v_cache, const void *ksum_cache, const float *bsum_cache,
                                 int32_t num_pages, const int32_t *block_table, int32_t max_pages, const void *h,
                                 const void *w_down, const void *w_up, int32_t d_model, int32_t r, int32_t *sel_idx,
                                 float *sel_score, void *out, float *lse, void *workspace, size_t workspace_bytes,
                                 hipStream_t stream) {
    hils::Shape s;
    hils_status_t st = resolve_paged(cfg, q_start, num_pages, max_pages, s);
    if (st) return st;
    if ((int64_t)s.B * s.N == 0) return ok();
    if ((st = check_ptr(q, "q")) || (st = check_ptr(k_cache, "k_cache")) || (st = check_ptr(v_cache, "v_cache")) ||
        (st = check_ptr(block_table, "block_table")) || (st = check_ptr(out, "out")))
        return st;
    if (s.K > 0 && ((st = check_ptr(sel_idx, "sel_idx")) || (st = check_ptr(sel_score, "sel_score")))) return st;
    if (s.K > 0 && s.C > 0 && ((st = check_ptr(ksum_cache, "ksum_cache")) || (st = check_ptr(bsum_cache, "bsum_cache"))))
        return st;
    if (lse && !aligned16(lse)) return fail(HILS_ERR_INVALID_ARG, "lse is not 16-byte aligned");
    if ((st = check_qcal(h, w_down, w_up, d_model, r))) return st;
    if (s.K > 0 && (st = check_score_mode(s))) return st;
    s.bt = block_table;
    if (!hils::sparse_attend_supported(s))
        return fail(HILS_ERR_UNSUPPORTED, "no fused-attention block shape fits LDS for G=%d, S=%d, d=%d, K=%d", s.G, s.S,
                    s.D, s.K);
    const bool qcal = h != nullptr;
    const size_t need = paged_workspace_bytes(s, qcal);
    if (!workspace || workspace_bytes < need)
        return fail(HILS_ERR_WORKSPACE, "prefill_paged needs %zu workspace bytes, got %zu", need,
                    workspace ? workspace_bytes : (size_t)0);
    if (!aligned16(workspace)) return fail(HILS_ERR_INVALID_ARG, "workspace is not 16-byte aligned");
    const size_t score_bytes = hils::align_up(hils::score_workspace_bytes(s, qcal), 256);
    char *score_ws = (char *)workspace + hils::FUSED_STATUS_BYTES;
    if (s.K > 0) {
        hils::ScoreWorkspace ws;
        hils::score_workspace_carve(s, qcal, score_ws, ws);
        if ((st = hip_status(hils::launch_score_select(s, q, ksum_cache, bsum_cache, h, w_down, w_up, d_model, r,
                                                       sel_idx, sel_score, ws, stream),
                             "paged score/select launch")))
            return st;
    }
    return hip_status(hils::launch_sparse_attend(s, q, k_cache, v_cache, sel_idx, sel_score, out, lse,
                                                 (uint32_t *)workspace, score_ws + score_bytes, stream),
                      "paged sparse attention launch");
}

}  // extern "C"
