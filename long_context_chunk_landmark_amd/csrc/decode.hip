// decode.hip -- kernel 4: one HiLS decode step over a paged KV/summary cache.
//
// hyper.ai HiLS summary, section 方法 (same computation as prefill, for the
// query at t = seq_len - 1 whose own key/value are already in the cache):
// score every candidate chunk's cached summary (k'_c, b'_c), max over the
// heads of the GQA group, keep the top K; attend exactly inside each
// selected chunk and the chunk-aligned window; fuse with exp(s^)/Z^.
//
// MI355X design: decode is HBM-bound on two streams -- the summaries of
// every candidate chunk and the K/V pages of the selected + window chunks.
// With one query per (sequence, group) there is too little parallelism per
// unit, so both phases split their ranges across many blocks:
//   A  decode_score    candidate range split: fp32 dots of the cached
//                      summaries (coalesced 16-byte loads, several
//                      candidates per wave), local top-K per block
//   A2 decode_merge    one wave per (seq, group): global top-K of the
//                      partial lists, ascending ids + per-head s^
//   B  decode_attend   chunk-list split: each block stages its pages' K/V
//                      in LDS and returns a partial (max, mass, output)
//   B2 decode_combine  log-sum-exp merge of the partials per (seq, head)
// A selected chunk enters as the state (max = s^_c, mass = 1, out = its
// normalised intra-chunk output); window chunks enter with their raw
// softmax statistics; the merge of all states is exactly the fused output.
#include <type_traits>

#include "hils_device.hpp"
#include "hils_internal.hpp"

namespace hils {

constexpr int DECODE_PAGES_CAP = 256;  // candidates per block of the page-contiguous scorer

namespace {

struct DecodeLayout {
    int splits;  // phase A blocks per (seq, group)
    int nsb;     // phase B blocks per (seq, group) (generic attend)
    int np;      // partial (m, l, o) slots per (seq, query head)
    bool fast;   // bf16, d = 128, S = 64: one wave per chunk of the list
    bool pages;  // bf16 summaries, d = 128, H_lm = H_q: page-contiguous scoring
    size_t off_qs, off_pkey, off_psc, off_sel, off_selsc, off_pm, off_pl, off_po, off_plse, total;
};

DecodeLayout decode_layout(const Shape &s, int num_seqs, int max_pages) {
    DecodeLayout L;
    L.splits = decode_splits(s, max_pages);
    L.nsb = std::max(1, std::min(16, (s.K + s.W / s.S + 1 + 3) / 4));
    L.fast = s.io_bf16 && s.D == 128 && s.S == 64;
    L.np = L.fast ? s.K + s.W / s.S + 1 : L.nsb;
    L.pages = s.sum_bf16 && s.D == 128 && s.H_lm == s.H_q && (s.H_q == 8 || s.H_q == 16 || s.H_q == 32) &&
              (max_pages + L.splits - 1) / L.splits <= DECODE_PAGES_CAP && s.agg_mode == 0;
    size_t o = 0;
    auto take = [&](size_t bytes) {
        const size_t at = o;
        o += align_up(bytes, 256);
        return at;
    };
    const size_t NS = (size_t)num_seqs;
    L.off_qs = take(NS * s.H_q * s.D * 4);
    L.off_pkey = take(NS * s.H_kv * L.splits * s.K * 8);
    L.off_psc = take(NS * s.H_kv * L.splits * s.K * s.G * 4);
    L.off_sel = take(NS * s.H_kv * s.K * 4);
    L.off_selsc = take(NS * s.H_q * s.K * 4);
    L.off_pm = take(NS * s.H_q * L.np * 4);
    L.off_pl = take(NS * s.H_q * L.np * 4);
    L.off_po = take(NS * s.H_q * L.np * s.D * 4);
    // normalised aggregation: per (seq, head, split) partial (max, sum) of exp(s^)
    L.off_plse = take(s.agg_mode == 1 ? NS * s.H_q * L.splits * 2 * 4 : 0);
    L.total = o;
    return L;
}

__device__ __forceinline__ int clamp_len(int len, int max_pages, int S) {
    return min(max(len, 1), max_pages * S);
}

__device__ __forceinline__ uint64_t dec_key(float s, int idx) {
    return ((uint64_t)ord_key(s) << 32) | (uint64_t)(0xffffffffu - (uint32_t)idx);
}

}  // namespace

// Phase-A blocks per (seq, group): about 256 candidates each, and at most
// 2048 partial entries for the merge wave (splits * K <= 2048).
int decode_splits(const Shape &s, int max_pages) {
    const int cap = std::max(1, 2048 / std::max(1, s.K));
    return std::max(1, std::min(cap, (max_pages + 255) / 256));
}

// q_s[seq, h, :] = q (+ W_up W_down h_seq), fp32.  One block per sequence.
template <typename T>
__global__ __launch_bounds__(256) void decode_qprep_kernel(const T *__restrict__ q, const T *__restrict__ h,
                                                           const T *__restrict__ w_down, const T *__restrict__ w_up,
                                                           float *__restrict__ qs, int H_q, int D, int d_model,
                                                           int r) {
    __shared__ float u[64];
    const int64_t seq = blockIdx.x;
    const int HD = H_q * D;
    if (h) {
        for (int a = threadIdx.x; a < r; a += blockDim.x) {
            float acc = 0.f;
            for (int x = 0; x < d_model; ++x)
                acc = fmaf(to_f32(w_down[(int64_t)a * d_model + x]), to_f32(h[seq * d_model + x]), acc);
            u[a] = acc;
        }
        __syncthreads();
    }
    for (int e = threadIdx.x; e < HD; e += blockDim.x) {
        float acc = to_f32(q[seq * HD + e]);
        if (h) {
            float dq = 0.f;
            for (int a = 0; a < r; ++a) dq = fmaf(to_f32(w_up[(int64_t)e * r + a]), u[a], dq);
            acc += dq;
        }
        qs[seq * HD + e] = acc;
    }
}

// Phase A.  LPR lanes cover one landmark row (16-byte loads), CPS = 64/LPR
// candidates per wave step.  GLM = landmark rows per candidate (G when
// every query head has its own landmark, 1 when the group shares one).
//
// AM (aggregation mode): 0 ranks by the group max of s^; 1 (first pass of
// the normalised aggregation) writes, per head, the split's partial (max,
// sum of exp) of s^ over its candidates into plse; 2 ranks by the group
// max of s^ - LSE_h, LSE_h combined from all splits' partials.  psc keeps
// the raw s^ in every mode.
template <typename TS, int D, int G, int GLM, int AM = 0>
__global__ __launch_bounds__(256) void decode_score_kernel(
    const float *__restrict__ qs, const TS *__restrict__ ksum_cache, const float *__restrict__ bsum_cache,
    const int32_t *__restrict__ block_table, int max_pages, const int32_t *__restrict__ seq_lens, uint64_t *pkey,
    float *psc, int H_q, int H_kv, int H_lm, int S, int W, int K, int splits, float scale,
    float *__restrict__ plse) {
    constexpr int E = 16 / sizeof(TS);
    constexpr int LPR = D / E;
    constexpr int CPS = WAVE / LPR;
    constexpr int CAPL = DECODE_SPLIT_CAP;
    __shared__ float agg_l[CAPL];
    __shared__ float sc_l[CAPL][G];
    __shared__ float lse_l[G];
    __shared__ float pm_l[4][G], pz_l[4][G];

    const int sp = blockIdx.x, g = blockIdx.y, seq = blockIdx.z;
    const int wave = threadIdx.x / WAVE, lane = lane_id();
    const int t = clamp_len(seq_lens[seq], max_pages, S) - 1;
    const int n = max(0, t / S - W / S);
    const int c_lo = (int)((int64_t)sp * n / splits), c_hi = (int)((int64_t)(sp + 1) * n / splits);
    const int cnt = c_hi - c_lo;
    const int col = lane % LPR, cs = lane / LPR;
    if constexpr (AM == 2) {
        // each head's log-sum-exp over all candidates, from the splits' partials
        if (threadIdx.x < G) {
            const float *pp = plse + ((int64_t)seq * H_q + g * G + threadIdx.x) * splits * 2;
            float m = -INFINITY, z = 0.f;
            for (int x = 0; x < splits; ++x) {
                const float mo = pp[2 * x], zo = pp[2 * x + 1];
                const float mn = fmaxf(m, mo);
                if (mn == -INFINITY) continue;
                z = (m == -INFINITY ? 0.f : z * expf(m - mn)) + (mo == -INFINITY ? 0.f : zo * expf(mo - mn));
                m = mn;
            }
            lse_l[threadIdx.x] = m + logf(z);
        }
        __syncthreads();
    }
    float lm[G], lz[G];  // AM == 1: this lane's running max / sum per head
#pragma unroll
    for (int e = 0; e < G; ++e) lm[e] = -INFINITY, lz[e] = 0.f;

    float qv[G][E];
#pragma unroll
    for (int e = 0; e < G; ++e)
#pragma unroll
        for (int x = 0; x < E; ++x) qv[e][x] = qs[((int64_t)seq * H_q + g * G + e) * D + col * E + x];
    const int32_t *bt = block_table + (int64_t)seq * max_pages;
    const int lbase = g * G * H_lm / H_q;  // first landmark head of the group

    // each wave scores a contiguous range of the split (at most 128
    // candidates); its block-table entries are fetched once, then U steps
    // of CPS candidates have their summary rows in flight together
    constexpr int U = 4;
    const int per_w = (cnt + 3) / 4;
    const int w_lo = min(cnt, wave * per_w), w_hi = min(cnt, w_lo + per_w);
    const int pg0 = w_lo + lane < w_hi ? bt[c_lo + w_lo + lane] : 0;
    const int pg1 = w_lo + 64 + lane < w_hi ? bt[c_lo + w_lo + 64 + lane] : 0;
    for (int base = w_lo; base < w_hi; base += U * CPS) {
        Vec16<TS> kv[U][GLM];
        float bias[U][GLM];
        bool okv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int lc = base + u * CPS + cs;
            okv[u] = lc < w_hi;
            const int rel = (okv[u] ? lc : w_lo) - w_lo;
            const int p0 = __shfl(pg0, rel & 63, WAVE), p1 = __shfl(pg1, rel & 63, WAVE);
            const int64_t page = rel < 64 ? p0 : p1;
#pragma unroll
            for (int e = 0; e < GLM; ++e) {
                kv[u][e] = load16(ksum_cache + (page * H_lm + lbase + e) * D + col * E);
                bias[u][e] = bsum_cache[page * H_lm + lbase + e];
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int lc = base + u * CPS + cs;
            float agg = -INFINITY;
            float sc[G];
#pragma unroll
            for (int e = 0; e < G; ++e) {
                const int le = GLM == 1 ? 0 : e;
                float part = 0.f;
#pragma unroll
                for (int x = 0; x < E; ++x) part = fmaf(qv[e][x], kv[u][le].get(x), part);
                part = seg_sum<LPR>(part);
                sc[e] = fmaf(scale, part, bias[u][le]);
                if constexpr (AM == 2) agg = fmaxf(agg, sc[e] - lse_l[e]);
                else agg = fmaxf(agg, sc[e]);
                if constexpr (AM == 1) {
                    if (okv[u] && col == 0) {
                        const float mn = fmaxf(lm[e], sc[e]);
                        lz[e] = lz[e] * expf(lm[e] - mn) + expf(sc[e] - mn);
                        lm[e] = mn;
                    }
                }
            }
            if (AM != 1 && okv[u] && col == 0) {
                agg_l[lc] = agg;
#pragma unroll
                for (int e = 0; e < G; ++e) sc_l[lc][e] = sc[e];
            }
        }
    }
    if constexpr (AM == 1) {
        // (max, sum) per head: over the wave's lanes, then the block's waves
#pragma unroll
        for (int e = 0; e < G; ++e) {
            float m = lm[e], z = lz[e];
#pragma unroll
            for (int off = 1; off < WAVE; off <<= 1) {
                const float mo = __shfl_xor(m, off, WAVE), zo = __shfl_xor(z, off, WAVE);
                const float mn = fmaxf(m, mo);
                z = (m == -INFINITY ? 0.f : z * expf(m - mn)) + (mo == -INFINITY ? 0.f : zo * expf(mo - mn));
                m = mn;
            }
            if (lane == 0) pm_l[wave][e] = m, pz_l[wave][e] = z;
        }
        __syncthreads();
        if (threadIdx.x < G) {
            float m = -INFINITY, z = 0.f;
            for (int w = 0; w < 4; ++w) {
                const float mo = pm_l[w][threadIdx.x], zo = pz_l[w][threadIdx.x];
                const float mn = fmaxf(m, mo);
                if (mn == -INFINITY) continue;
                z = (m == -INFINITY ? 0.f : z * expf(m - mn)) + (mo == -INFINITY ? 0.f : zo * expf(mo - mn));
                m = mn;
            }
            float *pp = plse + (((int64_t)seq * H_q + g * G + threadIdx.x) * splits + sp) * 2;
            pp[0] = m;
            pp[1] = z;
        }
        return;
    }
    __syncthreads();
    if (wave != 0) return;
    // local top-K over cnt <= CAPL entries (CAPL / 64 per lane)
    uint64_t keys[CAPL / WAVE];
#pragma unroll
    for (int v = 0; v < CAPL / WAVE; ++v) {
        const int lc = v * WAVE + lane;
        keys[v] = lc < cnt ? dec_key(agg_l[lc], c_lo + lc) : 0ull;
    }
    const uint64_t T = cnt > K ? kth_largest64<CAPL / WAVE>(keys, K) : 1ull;
    const int64_t pbase = (((int64_t)seq * H_kv + g) * splits + sp) * K;
    int outc = 0;
#pragma unroll
    for (int v = 0; v < CAPL / WAVE; ++v) {
        const bool keep = keys[v] >= T && keys[v] != 0ull;
        const uint64_t m = __ballot(keep);
        const int pos = outc + __popcll(m & lanemask_lt());
        if (keep && pos < K) {
            pkey[pbase + pos] = keys[v];
            const int lc = v * WAVE + lane;
#pragma unroll
            for (int e = 0; e < G; ++e) psc[(pbase + pos) * G + e] = sc_l[lc][e];
        }
        outc += __popcll(m);
    }
    for (int k = min(outc, K) + lane; k < K; k += WAVE) pkey[pbase + k] = 0ull;
}

// Phase A, page-contiguous variant (bf16 summaries, d = 128, one landmark
// head per query head).  A block scores a candidate range of one sequence
// for every kv group at once, so each candidate's summary row of all HQ
// landmark heads (HQ * 256 bytes, contiguous in the page) is read in one
// sweep.  Lane (slice, rg) holds dims 8slice..8slice+7 of landmark rows
// rg + 4k (k < HQ / 4) and the matching query slices.  Per-head scores and
// group maxima go to LDS; then each kv group takes its local top-K.
template <int HQ, int G>
__global__ __launch_bounds__(256) void decode_score_pages_kernel(
    const float *__restrict__ qs, const bf16 *__restrict__ q_raw, const bf16 *__restrict__ ksum_cache,
    const float *__restrict__ bsum_cache, const int32_t *__restrict__ block_table, int max_pages,
    const int32_t *__restrict__ seq_lens, uint64_t *pkey, float *psc, int S, int W, int K, int splits,
    float scale) {
    constexpr int D = 128, NR = HQ / 4, NG = HQ / G, CAP = DECODE_PAGES_CAP;
    __shared__ float sc_l[CAP][HQ];
    __shared__ float agg_l[NG][CAP];
    const int sp = blockIdx.x, seq = blockIdx.y;
    const int wave = threadIdx.x / WAVE, lane = lane_id();
    const int slice = lane & 15, rg = lane >> 4;
    const int t = clamp_len(seq_lens[seq], max_pages, S) - 1;
    const int n = max(0, t / S - W / S);
    const int c_lo = (int)((int64_t)sp * n / splits), c_hi = (int)((int64_t)(sp + 1) * n / splits);
    const int cnt = c_hi - c_lo;

    // scoring query slices of heads rg + 4k (calibrated fp32 when given)
    float qv[NR][8];
#pragma unroll
    for (int k = 0; k < NR; ++k) {
        const int64_t off = ((int64_t)seq * HQ + rg + 4 * k) * D + slice * 8;
#pragma unroll
        for (int x = 0; x < 8; ++x) qv[k][x] = qs ? qs[off + x] : (float)q_raw[off + x];
    }
    const int32_t *bt = block_table + (int64_t)seq * max_pages;
    const int per_w = (cnt + 3) / 4;
    const int w_lo = min(cnt, wave * per_w), w_hi = min(cnt, w_lo + per_w);  // <= 64 candidates
    const int pg = w_lo + lane < w_hi ? bt[c_lo + w_lo + lane] : 0;
    constexpr int U = 2;
    for (int base = w_lo; base < w_hi; base += U) {
        u32x4 kv[U][NR];
        float bias[U][NR];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int lc = min(base + u, w_hi - 1);
            const int64_t page = __shfl(pg, lc - w_lo, WAVE);
            const bf16 *row = ksum_cache + page * HQ * D + slice * 8;
#pragma unroll
            for (int k = 0; k < NR; ++k) {
                kv[u][k] = *(const u32x4 *)(row + (rg + 4 * k) * D);
                bias[u][k] = bsum_cache[page * HQ + rg + 4 * k];
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int lc = base + u;
            float sc[NR];
#pragma unroll
            for (int k = 0; k < NR; ++k) {
                float part = 0.f;
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    const uint32_t w = kv[u][k][x];
                    part = fmaf(qv[k][2 * x], __uint_as_float(w << 16), part);
                    part = fmaf(qv[k][2 * x + 1], __uint_as_float(w & 0xffff0000u), part);
                }
                sc[k] = fmaf(scale, seg_sum<16>(part), bias[u][k]);
            }
            // group maxima: head h = rg + 4k belongs to group h / G
            float ag[NR];
#pragma unroll
            for (int k = 0; k < NR; ++k) {
                float a = sc[k];
                if constexpr (G >= 2) {
                    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(a), false, false);
                    a = fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
                }
                if constexpr (G >= 4) {
                    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(a), false, false);
                    a = fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
                }
                ag[k] = a;
            }
            if (lc < w_hi && slice == 0) {
#pragma unroll
                for (int k = 0; k < NR; ++k) sc_l[lc][rg + 4 * k] = sc[k];
#pragma unroll
                for (int k = 0; k < NR; ++k) {
                    if constexpr (G == 1) {
                        agg_l[rg + 4 * k][lc] = ag[k];
                    } else if constexpr (G == 2) {
                        if ((rg & 1) == 0) agg_l[(rg + 4 * k) / 2][lc] = ag[k];
                    } else if constexpr (G == 4) {
                        if (rg == 0) agg_l[k][lc] = ag[k];
                    } else {  // G == 8: heads 8gg .. 8gg+7 are rows k = 2gg, 2gg+1
                        if (rg == 0 && (k & 1)) agg_l[k / 2][lc] = fmaxf(ag[k], ag[k - 1]);
                    }
                }
            }
        }
    }
    __syncthreads();
    // local top-K of each kv group (groups wave, wave + 4, ...)
    for (int gg = wave; gg < NG; gg += 4) {
        uint64_t keys[CAP / WAVE];
#pragma unroll
        for (int v = 0; v < CAP / WAVE; ++v) {
            const int lc = v * WAVE + lane;
            keys[v] = lc < cnt ? dec_key(agg_l[gg][lc], c_lo + lc) : 0ull;
        }
        const uint64_t T = cnt > K ? kth_largest64<CAP / WAVE>(keys, K) : 1ull;
        const int64_t pbase = (((int64_t)seq * NG + gg) * splits + sp) * K;
        int outc = 0;
#pragma unroll
        for (int v = 0; v < CAP / WAVE; ++v) {
            const bool keep = keys[v] >= T && keys[v] != 0ull;
            const uint64_t m = __ballot(keep);
            const int pos = outc + __popcll(m & lanemask_lt());
            if (keep && pos < K) {
                pkey[pbase + pos] = keys[v];
                const int lc = v * WAVE + lane;
#pragma unroll
                for (int e = 0; e < G; ++e) psc[(pbase + pos) * G + e] = sc_l[lc][gg * G + e];
            }
            outc += __popcll(m);
        }
        for (int k = min(outc, K) + lane; k < K; k += WAVE) pkey[pbase + k] = 0ull;
    }
}

// Phase A2.  One wave per (seq, group): top-K of splits*K partial entries.
template <int G, int NVMAX>
__global__ __launch_bounds__(64) void decode_merge_kernel(const uint64_t *__restrict__ pkey,
                                                          const float *__restrict__ psc, int32_t *sel_ws,
                                                          float *selsc_ws, int32_t *sel_user, int H_q, int H_kv,
                                                          int K, int splits) {
    // NVMAX * 64 >= splits * K partial entries
    __shared__ uint64_t kept[128];
    __shared__ int kept_at[128];
    const int g = blockIdx.x, seq = blockIdx.y, lane = lane_id();
    const int total = splits * K;
    const int64_t pbase = ((int64_t)seq * H_kv + g) * splits * K;
    uint64_t keys[NVMAX];
#pragma unroll
    for (int v = 0; v < NVMAX; ++v) {
        const int idx = v * WAVE + lane;
        keys[v] = idx < total ? pkey[pbase + idx] : 0ull;
    }
    int nonempty = 0;
#pragma unroll
    for (int v = 0; v < NVMAX; ++v) nonempty += __popcll(__ballot(keys[v] != 0ull));
    const uint64_t T = nonempty > K ? kth_largest64<NVMAX>(keys, K) : 1ull;
    int outc = 0;
#pragma unroll
    for (int v = 0; v < NVMAX; ++v) {
        const bool keep = keys[v] >= T && keys[v] != 0ull;
        const uint64_t m = __ballot(keep);
        const int pos = outc + __popcll(m & lanemask_lt());
        if (keep && pos < 128) {
            kept[pos] = keys[v];
            kept_at[pos] = v * WAVE + lane;
        }
        outc += __popcll(m);
    }
    wave_sync();
    const int cnt = min(outc, K);
    const int64_t sbase = ((int64_t)seq * H_kv + g) * K;
    for (int t = lane; t < 128; t += WAVE) {
        if (t < cnt) {
            const int my = (int)(0xffffffffu - (uint32_t)kept[t]);
            int rank = 0;
            for (int u = 0; u < cnt; ++u) rank += (int)(0xffffffffu - (uint32_t)kept[u]) < my;
            sel_ws[sbase + rank] = my;
            if (sel_user) sel_user[sbase + rank] = my;
#pragma unroll
            for (int e = 0; e < G; ++e)
                selsc_ws[((int64_t)seq * H_q + g * G + e) * K + rank] = psc[(pbase + kept_at[t]) * G + e];
        }
    }
    for (int k = cnt + lane; k < K; k += WAVE) {
        sel_ws[sbase + k] = -1;
        if (sel_user) sel_user[sbase + k] = -1;
#pragma unroll
        for (int e = 0; e < G; ++e) selsc_ws[((int64_t)seq * H_q + g * G + e) * K + k] = -INFINITY;
    }
}

// Phase B.  Block (split, group, seq) attends positions [lo, hi) of the
// list "selected chunks, then window chunks".
template <typename T, int D, int S, int G>
__global__ __launch_bounds__(256) void decode_attend_kernel(
    const T *__restrict__ q_raw, const T *__restrict__ k_cache, const T *__restrict__ v_cache,
    const int32_t *__restrict__ block_table, int max_pages, const int32_t *__restrict__ seq_lens,
    const int32_t *__restrict__ sel_ws, const float *__restrict__ selsc_ws, float *pm, float *pl, float *po,
    int H_q, int H_kv, int W, int K, int nsb, float scale) {
    constexpr int DPL = D / WAVE;  // consecutive dims per lane (1 or 2)
    constexpr int KPL = S / WAVE;  // keys per lane
    constexpr int E = 16 / sizeof(T);
    extern __shared__ float dyn_f[];
    float(*k_l)[D + 1] = (float(*)[D + 1])dyn_f;            // [S][D+1]: lane-per-key rows, no bank conflicts
    float(*v_l)[D] = (float(*)[D])(dyn_f + S * (D + 1));    // [S][D]
    __shared__ float q_l[G][D];
    __shared__ float p_l[4][S];

    const int sp = blockIdx.x, g = blockIdx.y, seq = blockIdx.z;
    const int tid = threadIdx.x, wave = tid / WAVE, lane = lane_id();
    const int t = clamp_len(seq_lens[seq], max_pages, S) - 1;
    const int tc = t / S;
    const int wc0 = max(0, tc - W / S);
    const int32_t *sl = sel_ws + ((int64_t)seq * H_kv + g) * K;
    // chunk list: selected (ascending, -1 padded) then window
    int nsel = 0;
    for (int kk = 0; kk < K; ++kk) nsel += sl[kk] >= 0;
    const int total = nsel + (tc - wc0 + 1);
    const int lo = (int)((int64_t)sp * total / nsb), hi = (int)((int64_t)(sp + 1) * total / nsb);
    // exact attention uses the raw query (the calibration is for scoring only)
    for (int x = tid; x < G * D; x += blockDim.x) q_l[x / D][x % D] = to_f32(q_raw[((int64_t)seq * H_q + g * G) * D + x]);

    // per-head running state, heads e = wave, wave + 4, ...
    constexpr int HPW = (G + 3) / 4;
    float m_s[HPW], l_s[HPW], o_s[HPW][DPL];
#pragma unroll
    for (int a = 0; a < HPW; ++a) {
        m_s[a] = -INFINITY;
        l_s[a] = 0.f;
#pragma unroll
        for (int y = 0; y < DPL; ++y) o_s[a][y] = 0.f;
    }
    const int32_t *bt = block_table + (int64_t)seq * max_pages;
    for (int pos = lo; pos < hi; ++pos) {
        const bool is_sel = pos < nsel;
        const int c = is_sel ? sl[pos] : wc0 + (pos - nsel);
        const int64_t page = bt[c];
        __syncthreads();
        const T *kp = k_cache + (page * H_kv + g) * (int64_t)S * D;
        const T *vp = v_cache + (page * H_kv + g) * (int64_t)S * D;
        for (int idx = tid; idx < S * D / E; idx += blockDim.x) {
            const int j = idx / (D / E), x0 = (idx % (D / E)) * E;
            const Vec16<T> kk = load16(kp + (int64_t)j * D + x0);
            const Vec16<T> vv = load16(vp + (int64_t)j * D + x0);
#pragma unroll
            for (int x = 0; x < E; ++x) {
                k_l[j][x0 + x] = kk.get(x);
                v_l[j][x0 + x] = vv.get(x);
            }
        }
        __syncthreads();
#pragma unroll
        for (int a = 0; a < HPW; ++a) {
            const int e = wave + 4 * a;
            if (e >= G) break;
            float lg[KPL];
            float cm = -INFINITY;
#pragma unroll
            for (int u = 0; u < KPL; ++u) {
                const int j = u * WAVE + lane;
                float dot = 0.f;
                for (int x = 0; x < D; ++x) dot = fmaf(q_l[e][x], k_l[j][x], dot);
                const bool masked = !is_sel && (c * S + j > t);
                lg[u] = masked ? -INFINITY : dot * scale;
                cm = fmaxf(cm, lg[u]);
            }
            cm = wave_max(cm);
            float ls = 0.f;
#pragma unroll
            for (int u = 0; u < KPL; ++u) {
                const float p = expf(lg[u] - cm);
                p_l[wave][u * WAVE + lane] = p;
                ls += p;
            }
            ls = xor_sum<1, 32>(ls);
            wave_sync();
            float oc[DPL];
#pragma unroll
            for (int y = 0; y < DPL; ++y) oc[y] = 0.f;
            for (int j = 0; j < S; ++j) {
                const float p = p_l[wave][j];
#pragma unroll
                for (int y = 0; y < DPL; ++y) oc[y] = fmaf(p, v_l[j][lane * DPL + y], oc[y]);
            }
            wave_sync();
            // state of this chunk: selected -> (s^_c, 1, o_c / l_c); window -> (cm, ls, oc)
            float cmx, cl, cscale;
            if (is_sel) {
                cmx = selsc_ws[((int64_t)seq * H_q + g * G + e) * K + pos];
                cl = 1.f;
                cscale = 1.f / ls;
            } else {
                cmx = cm;
                cl = ls;
                cscale = 1.f;
            }
            const float mn = fmaxf(m_s[a], cmx);
            const float a0 = expf(m_s[a] - mn), a1 = expf(cmx - mn);
            l_s[a] = l_s[a] * a0 + cl * a1;
#pragma unroll
            for (int y = 0; y < DPL; ++y) o_s[a][y] = o_s[a][y] * a0 + oc[y] * cscale * a1;
            m_s[a] = mn;
        }
    }
#pragma unroll
    for (int a = 0; a < HPW; ++a) {
        const int e = wave + 4 * a;
        if (e >= G) break;
        const int64_t hb = ((int64_t)seq * H_q + g * G + e) * nsb + sp;
        if (lane == 0) {
            pm[hb] = m_s[a];
            pl[hb] = l_s[a];
        }
#pragma unroll
        for (int y = 0; y < DPL; ++y) po[hb * D + lane * DPL + y] = o_s[a][y];
    }
}

// Phase B, fast path (bf16 caches, d = 128, S = 64).  One wave per entry
// pos of the list "selected chunks, then window chunks" of (seq, group),
// writing that chunk's partial state per query head: a selected chunk
// enters as (s^_c, 1, o_c) with o_c its normalised intra-chunk output, a
// window chunk as its raw softmax statistics (max, mass, unnormalised sum).
// Lane (col, rsub) holds key rows 4t + rsub, dims 8col..8col+7, of K and V.
// Logits: packed bf16 dot2 of the raw query with the key slice,
// transpose-reduced over the 16-lane DPP row (afterwards the lane holds
// key 4col + rsub).  PV: V rows are repacked as fp16 pairs (keys t, t+1)
// and combined with fp16 pairs of p by fp16 dot2 with fp32 accumulation;
// p is exchanged through LDS.  (fp16 holds bf16 values below 65504 exactly;
// p lies in [0, 1].)
template <int G>
__global__ __launch_bounds__(256) void decode_attend_fast_kernel(
    const bf16 *__restrict__ q_raw, const bf16 *__restrict__ k_cache, const bf16 *__restrict__ v_cache,
    const int32_t *__restrict__ block_table, int max_pages, const int32_t *__restrict__ seq_lens,
    const int32_t *__restrict__ sel_ws, const float *__restrict__ selsc_ws, float *pm, float *pl, float *po,
    int H_q, int H_kv, int W, int K, int np, float scale) {
    constexpr int D = 128, S = 64;
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
    __shared__ float p_l[4][G][4][16];  // [wave][head][rsub][t]
    const int g = blockIdx.y, seq = blockIdx.z;
    const int wave = threadIdx.x / WAVE, lane = lane_id();
    const int col = lane & 15, rsub = lane >> 4;
    const int pos = blockIdx.x * 4 + wave;
    if (pos >= np) return;
    const int t_last = clamp_len(seq_lens[seq], max_pages, S) - 1;
    const int tc = t_last / S;
    const int wc0 = max(0, tc - W / S);
    const int32_t *sl = sel_ws + ((int64_t)seq * H_kv + g) * K;
    int nsel = 0;
    for (int k0 = 0; k0 < K; k0 += WAVE) nsel += __popcll(__ballot(k0 + lane < K && sl[k0 + lane] >= 0));
    const int total = nsel + (tc - wc0 + 1);
    const int64_t hrow0 = (int64_t)seq * H_q + g * G;  // first query head of the group
    if (pos >= total) {
        // unused slot: an empty state
#pragma unroll
        for (int e = 0; e < G; ++e) {
            const int64_t hb = (hrow0 + e) * np + pos;
            if (lane == 0) {
                pm[hb] = -INFINITY;
                pl[hb] = 0.f;
            }
            po[hb * D + lane] = 0.f;
            po[hb * D + 64 + lane] = 0.f;
        }
        return;
    }
    const bool is_sel = pos < nsel;
    const int c = is_sel ? sl[pos] : wc0 + (pos - nsel);
    const int64_t page = block_table[(int64_t)seq * max_pages + c];
    const bf16 *kp = k_cache + (page * H_kv + g) * (int64_t)S * D + col * 8;
    const bf16 *vp = v_cache + (page * H_kv + g) * (int64_t)S * D + col * 8;
    u32x4 kx[16], vx[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) kx[t] = *(const u32x4 *)(kp + (t * 4 + rsub) * D);
#pragma unroll
    for (int t = 0; t < 16; ++t) vx[t] = *(const u32x4 *)(vp + (t * 4 + rsub) * D);
    const float sl2 = scale * LOG2E;
    const int j = 4 * col + rsub;  // key of this lane after the transpose-reduce
    const bool masked = !is_sel && (c * S + j > t_last);

    float (*pw)[4][16] = p_l[wave];
    float lsum[G], mx[G];
#pragma unroll
    for (int e = 0; e < G; ++e) {
        const u32x4 qr = *(const u32x4 *)(q_raw + (hrow0 + e) * D + col * 8);
        float part[16];
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            float acc = 0.f;
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                const uint32_t qa = qr[x], kb2 = kx[t][x];
                bf16x2 a2, b2;
                __builtin_memcpy(&a2, &qa, 4);
                __builtin_memcpy(&b2, &kb2, 4);
                acc = __builtin_amdgcn_fdot2_f32_bf16(a2, b2, acc, false);
            }
            part[t] = acc;
        }
        // the cross-lane reduction runs on every lane; masking comes after
        // (inside a conditional it would run with masked lanes disabled)
        const float tr = transpose_sum16(part, col);
        const float lg = masked ? -INFINITY : tr * sl2;
        const float m2 = wave_max_f(lg);
        const float ex = exp2f(lg - m2);
        const float l = wave_sum_f(ex);
        mx[e] = m2;
        lsum[e] = l;
        pw[e][rsub][col] = is_sel ? ex / l : ex;
    }
    wave_sync();
    // V as fp16 pairs of consecutive rows: vh[tp][d] = (v[2tp][d], v[2tp+1][d])
    f16x2 vh[8][8];
#pragma unroll
    for (int tp = 0; tp < 8; ++tp)
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            const uint32_t a = vx[2 * tp][x], b = vx[2 * tp + 1][x];
            vh[tp][2 * x] = f16x2{(_Float16)__uint_as_float(a << 16), (_Float16)__uint_as_float(b << 16)};
            vh[tp][2 * x + 1] =
                f16x2{(_Float16)__uint_as_float(a & 0xffff0000u), (_Float16)__uint_as_float(b & 0xffff0000u)};
        }
#pragma unroll
    for (int e = 0; e < G; ++e) {
        f16x2 bp[8];
#pragma unroll
        for (int t0 = 0; t0 < 16; t0 += 4) {
            const f32x4 p4 = *(const f32x4 *)&pw[e][rsub][t0];
            bp[t0 / 2] = f16x2{(_Float16)p4[0], (_Float16)p4[1]};
            bp[t0 / 2 + 1] = f16x2{(_Float16)p4[2], (_Float16)p4[3]};
        }
        float o[8];
#pragma unroll
        for (int d = 0; d < 8; ++d) {
            float acc = 0.f;
#pragma unroll
            for (int tp = 0; tp < 8; ++tp) acc = __builtin_amdgcn_fdot2(vh[tp][d], bp[tp], acc, false);
            o[d] = rows4_sum(acc);
        }
        const int64_t hb = (hrow0 + e) * np + pos;
        if (rsub == 0) {
            float *dst = po + hb * D + col * 8;
            *(f32x4 *)dst = f32x4{o[0], o[1], o[2], o[3]};
            *(f32x4 *)(dst + 4) = f32x4{o[4], o[5], o[6], o[7]};
        }
        if (lane == 0) {
            pm[hb] = is_sel ? selsc_ws[(hrow0 + e) * K + pos] : mx[e] * LN2;
            pl[hb] = is_sel ? 1.f : lsum[e];
        }
    }
}

// Phase B2.  One wave per (seq, head): the wave's four 16-lane groups
// each merge every fourth partial state (lane covering D/16 dims), then
// the four group states are joined with lane swaps.
template <typename T, int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(const float *__restrict__ pm, const float *__restrict__ pl,
                                                             const float *__restrict__ po, T *__restrict__ out,
                                                             float *__restrict__ lse, int64_t rows, int np) {
    constexpr int DPL = D / 16;
    const int lane = lane_id(), sub = lane & 15, pgp = lane >> 4;
    const int64_t row = (int64_t)blockIdx.x * 4 + threadIdx.x / WAVE;
    if (row >= rows) return;
    float m = -INFINITY, l = 0.f, o[DPL];
#pragma unroll
    for (int y = 0; y < DPL; ++y) o[y] = 0.f;
    auto add = [&](float ms, float ls, const float (&os)[DPL]) {
        if (ms == -INFINITY) return;
        const float mn = fmaxf(m, ms);
        const float a0 = m == -INFINITY ? 0.f : expf(m - mn), a1 = expf(ms - mn);
        l = l * a0 + ls * a1;
#pragma unroll
        for (int y = 0; y < DPL; ++y) o[y] = o[y] * a0 + os[y] * a1;
        m = mn;
    };
    constexpr int U = 4;
    for (int s0 = pgp; s0 < np; s0 += 4 * U) {
        float ms[U], ls[U], os[U][DPL];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int sidx = min(s0 + 4 * u, np - 1);
            const bool ok = s0 + 4 * u < np;
            ms[u] = ok ? pm[row * np + sidx] : -INFINITY;
            ls[u] = pl[row * np + sidx];
            const float *src = po + (row * np + sidx) * D + sub * DPL;
#pragma unroll
            for (int y = 0; y < DPL; y += 4) {
                const f32x4 v = *(const f32x4 *)(src + y);
                os[u][y] = v[0], os[u][y + 1] = v[1], os[u][y + 2] = v[2], os[u][y + 3] = v[3];
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) add(ms[u], ls[u], os[u]);
    }
    // join the four groups (lanes sub, sub + 16, sub + 32, sub + 48)
    const float M = rows4_max(m);
    const float a = m == -INFINITY ? 0.f : expf(m - M);
    const float L = rows4_sum(l * a);
    float r[DPL];
#pragma unroll
    for (int y = 0; y < DPL; ++y) r[y] = rows4_sum(o[y] * a);
    if (pgp == 0) {
        const float inv = 1.f / L;
#pragma unroll
        for (int y = 0; y < DPL; ++y) out[row * D + sub * DPL + y] = from_f32<T>(r[y] * inv);
        if (lse && sub == 0) lse[row] = M + logf(L);
    }
}

// Dense decode, the full-attention point of comparison for one decode step:
// the query at t = seq_len - 1 attends every key 0 .. t of its sequence.
// Grid (splits, H_kv, num_seqs) of 4-wave blocks; block x owns chunks
// [x cps, (x + 1) cps) of its (seq, group), its waves take every fourth
// chunk and carry one running softmax state per query head of the group
// (base-2 max, mass, and output sums left unreduced over the lane's four
// key rows until the end).  The block joins its four wave states into one
// partial (max, mass, sum) per head, and decode_combine_kernel merges the
// splits.  The per-chunk arithmetic is the fast attend path's: packed bf16
// dot2 logits, fp16 dot2 products of p and V.
template <int G>
__global__ __launch_bounds__(256) void dense_decode_kernel(
    const bf16 *__restrict__ q_raw, const bf16 *__restrict__ k_cache, const bf16 *__restrict__ v_cache,
    const int32_t *__restrict__ block_table, int max_pages, const int32_t *__restrict__ seq_lens, float *pm,
    float *pl, float *po, int H_q, int H_kv, int splits, int cps, float scale) {
    constexpr int D = 128, S = 64;
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
    __shared__ float p_l[4][G][4][16];  // [wave][head][rsub][t]
    __shared__ float st_m[4][G], st_l[4][G];
    __shared__ float st_o[4][G][D];
    const int split = blockIdx.x, g = blockIdx.y, seq = blockIdx.z;
    const int wave = threadIdx.x / WAVE, lane = lane_id();
    const int col = lane & 15, rsub = lane >> 4;
    const int t_last = clamp_len(seq_lens[seq], max_pages, S) - 1;
    const int c0 = split * cps, c1 = min(t_last / S + 1, c0 + cps);
    const int64_t hrow0 = (int64_t)seq * H_q + g * G;  // first query head of the group
    const float sl2 = scale * LOG2E;
    const int j = 4 * col + rsub;  // key of this lane after the transpose-reduce

    u32x4 qr[G];
#pragma unroll
    for (int e = 0; e < G; ++e) qr[e] = *(const u32x4 *)(q_raw + (hrow0 + e) * D + col * 8);
    float m[G], l[G], oacc[G][8];
#pragma unroll
    for (int e = 0; e < G; ++e) {
        m[e] = -INFINITY;
        l[e] = 0.f;
#pragma unroll
        for (int d = 0; d < 8; ++d) oacc[e][d] = 0.f;
    }
    float (*pw)[4][16] = p_l[wave];
    for (int c = c0 + wave; c < c1; c += 4) {
        const int64_t page = block_table[(int64_t)seq * max_pages + c];
        const bf16 *kp = k_cache + (page * H_kv + g) * (int64_t)S * D + col * 8;
        const bf16 *vp = v_cache + (page * H_kv + g) * (int64_t)S * D + col * 8;
        u32x4 kx[16], vx[16];
#pragma unroll
        for (int t = 0; t < 16; ++t) kx[t] = *(const u32x4 *)(kp + (t * 4 + rsub) * D);
#pragma unroll
        for (int t = 0; t < 16; ++t) vx[t] = *(const u32x4 *)(vp + (t * 4 + rsub) * D);
        const bool masked = c * S + j > t_last;
#pragma unroll
        for (int e = 0; e < G; ++e) {
            float part[16];
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                float acc = 0.f;
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    const uint32_t qa = qr[e][x], kb2 = kx[t][x];
                    bf16x2 a2, b2;
                    __builtin_memcpy(&a2, &qa, 4);
                    __builtin_memcpy(&b2, &kb2, 4);
                    acc = __builtin_amdgcn_fdot2_f32_bf16(a2, b2, acc, false);
                }
                part[t] = acc;
            }
            // the cross-lane reduction runs on every lane; masking comes after
            const float tr = transpose_sum16(part, col);
            const float lg = masked ? -INFINITY : tr * sl2;
            // key c S is visible, so the chunk's maximum is finite
            const float mnew = fmaxf(m[e], wave_max_f(lg));
            const float alpha = exp2_hw(m[e] - mnew);
            const float ex = exp2_hw(lg - mnew);
            l[e] = fmaf(l[e], alpha, wave_sum_f(ex));
            m[e] = mnew;
#pragma unroll
            for (int d = 0; d < 8; ++d) oacc[e][d] *= alpha;
            pw[e][rsub][col] = ex;
        }
        wave_sync();
        // V as fp16 pairs of consecutive rows: vh[tp][d] = (v[2tp][d], v[2tp+1][d])
        f16x2 vh[8][8];
#pragma unroll
        for (int tp = 0; tp < 8; ++tp)
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                const uint32_t a = vx[2 * tp][x], b = vx[2 * tp + 1][x];
                vh[tp][2 * x] = f16x2{(_Float16)__uint_as_float(a << 16), (_Float16)__uint_as_float(b << 16)};
                vh[tp][2 * x + 1] =
                    f16x2{(_Float16)__uint_as_float(a & 0xffff0000u), (_Float16)__uint_as_float(b & 0xffff0000u)};
            }
#pragma unroll
        for (int e = 0; e < G; ++e) {
            f16x2 bp[8];
#pragma unroll
            for (int t0 = 0; t0 < 16; t0 += 4) {
                const f32x4 p4 = *(const f32x4 *)&pw[e][rsub][t0];
                bp[t0 / 2] = f16x2{(_Float16)p4[0], (_Float16)p4[1]};
                bp[t0 / 2 + 1] = f16x2{(_Float16)p4[2], (_Float16)p4[3]};
            }
#pragma unroll
            for (int d = 0; d < 8; ++d)
#pragma unroll
                for (int tp = 0; tp < 8; ++tp) oacc[e][d] = __builtin_amdgcn_fdot2(vh[tp][d], bp[tp], oacc[e][d], false);
        }
        wave_sync();  // the next chunk's p overwrites this one's
    }
    // the wave's state: lane (col, 0) holds dims 8 col .. +7 of each head
#pragma unroll
    for (int e = 0; e < G; ++e) {
#pragma unroll
        for (int d = 0; d < 8; ++d) {
            const float o = rows4_sum(oacc[e][d]);
            if (rsub == 0) st_o[wave][e][col * 8 + d] = o;
        }
        if (lane == 0) {
            st_m[wave][e] = m[e];
            st_l[wave][e] = l[e];
        }
    }
    __syncthreads();
    // join the four wave states: thread (e, dim) pairs, base-2 maxima
    for (int x = threadIdx.x; x < G * D; x += 256) {
        const int e = x / D, dim = x % D;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < 4; ++w) M = fmaxf(M, st_m[w][e]);
        float L = 0.f, O = 0.f;
        if (M != -INFINITY) {
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const float a = st_m[w][e] == -INFINITY ? 0.f : exp2_hw(st_m[w][e] - M);
                L = fmaf(st_l[w][e], a, L);
                O = fmaf(st_o[w][e][dim], a, O);
            }
        }
        const int64_t hb = (hrow0 + e) * splits + split;
        po[hb * D + dim] = O;
        if (dim == 0) {
            pm[hb] = M == -INFINITY ? -INFINITY : M * LN2;
            pl[hb] = L;
        }
    }
}

// Splits of the dense decode: about 8192 blocks in all, at least 4 chunks each.
static void dense_decode_split(int num_seqs, int H_kv, int max_pages, int &splits, int &cps) {
    const int units = std::max(1, num_seqs * H_kv);
    splits = std::max(1, std::min((max_pages + 3) / 4, (8192 + units - 1) / units));
    cps = (max_pages + splits - 1) / splits;
    splits = (max_pages + cps - 1) / cps;
}

size_t dense_decode_workspace_bytes(const Shape &s, int num_seqs, int max_pages) {
    if (!dense_decode_supported(s)) return 0;
    int splits, cps;
    dense_decode_split(num_seqs, s.H_kv, max_pages, splits, cps);
    const size_t rows = (size_t)num_seqs * s.H_q * splits;
    return align_up(rows * 4, 256) * 2 + align_up(rows * s.D * 4, 256);
}

bool dense_decode_supported(const Shape &s) {
    return s.io_bf16 && s.D == 128 && s.S == 64 && (s.G == 1 || s.G == 2 || s.G == 4 || s.G == 8);
}

hipError_t launch_dense_decode(const Shape &s, int num_seqs, const void *q, const void *k_cache,
                               const void *v_cache, const int32_t *block_table, int max_pages,
                               const int32_t *seq_lens, void *out, float *lse, void *workspace, hipStream_t st) {
    if (num_seqs == 0) return hipSuccess;
    int splits, cps;
    dense_decode_split(num_seqs, s.H_kv, max_pages, splits, cps);
    const size_t rows = (size_t)num_seqs * s.H_q * splits;
    char *ws = (char *)workspace;
    float *pm = (float *)ws, *pl = (float *)(ws + align_up(rows * 4, 256));
    float *po = (float *)(ws + 2 * align_up(rows * 4, 256));
    const dim3 grid((unsigned)splits, (unsigned)s.H_kv, (unsigned)num_seqs);
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, grid, dim3(256), 0, st, (const bf16 *)q, (const bf16 *)k_cache,
                           (const bf16 *)v_cache, block_table, max_pages, seq_lens, pm, pl, po, s.H_q, s.H_kv, splits,
                           cps, s.scale);
    };
    switch (s.G) {
        case 1: go(dense_decode_kernel<1>); break;
        case 2: go(dense_decode_kernel<2>); break;
        case 4: go(dense_decode_kernel<4>); break;
        case 8: go(dense_decode_kernel<8>); break;
        default: return hipErrorInvalidValue;
    }
    const int64_t hrows = (int64_t)num_seqs * s.H_q;
    hipLaunchKernelGGL((decode_combine_kernel<bf16, 128>), dim3((unsigned)((hrows + 3) / 4)), dim3(256), 0, st, pm, pl,
                       po, (bf16 *)out, lse, hrows, splits);
    return hipGetLastError();
}

size_t decode_workspace_bytes(const Shape &s, int num_seqs, int max_pages) {
    return decode_layout(s, num_seqs, max_pages).total;
}

template <typename T, typename TS, int D, int S, int G>
static hipError_t go_decode(const Shape &s, const DecodeLayout &L, int num_seqs, const void *q, const void *k_cache,
                            const void *v_cache, const void *ksum_cache, const float *bsum_cache,
                            const int32_t *block_table, int max_pages, const int32_t *seq_lens, const void *h,
                            const void *w_down, const void *w_up, int d_model, int r, void *out, float *lse,
                            int32_t *sel_idx, char *ws, hipStream_t st) {
    float *qs = (float *)(ws + L.off_qs);
    uint64_t *pkey = (uint64_t *)(ws + L.off_pkey);
    float *psc = (float *)(ws + L.off_psc);
    int32_t *sel = (int32_t *)(ws + L.off_sel);
    float *selsc = (float *)(ws + L.off_selsc);
    float *pm = (float *)(ws + L.off_pm), *pl = (float *)(ws + L.off_pl), *po = (float *)(ws + L.off_po);
    const bool pages = std::is_same<T, bf16>::value && std::is_same<TS, bf16>::value && D == 128 && L.pages;
    if (!pages || h)
        hipLaunchKernelGGL(decode_qprep_kernel<T>, dim3(num_seqs), dim3(256), 0, st, (const T *)q, (const T *)h,
                           (const T *)w_down, (const T *)w_up, qs, s.H_q, s.D, d_model, r);
    const dim3 ga(L.splits, s.H_kv, num_seqs);
    if constexpr (std::is_same<T, bf16>::value && std::is_same<TS, bf16>::value && D == 128) {
        if (pages) {
            const float *qsp = h ? qs : nullptr;
            auto sc = [&](auto kern) {
                hipLaunchKernelGGL(kern, dim3(L.splits, num_seqs), dim3(256), 0, st, qsp, (const bf16 *)q,
                                   (const bf16 *)ksum_cache, bsum_cache, block_table, max_pages, seq_lens, pkey, psc,
                                   s.S, s.W, s.K, L.splits, s.scale);
            };
            if (s.H_q == 8) sc(decode_score_pages_kernel<8, G>);
            else if (s.H_q == 16) sc(decode_score_pages_kernel<16, G>);
            else sc(decode_score_pages_kernel<32, G>);
        }
    }
    float *plse = (float *)(ws + L.off_plse);
    auto gscore = [&](auto kern) {
        hipLaunchKernelGGL(kern, ga, dim3(256), 0, st, qs, (const TS *)ksum_cache, bsum_cache, block_table, max_pages,
                           seq_lens, pkey, psc, s.H_q, s.H_kv, s.H_lm, s.S, s.W, s.K, L.splits, s.scale, plse);
    };
    if (pages) {
    } else if (s.agg_mode == 1) {
        // normalised aggregation: each head's log-sum-exp first, then the ranking pass
        if (s.GLM == 1) {
            gscore(decode_score_kernel<TS, D, G, 1, 1>);
            gscore(decode_score_kernel<TS, D, G, 1, 2>);
        } else {
            gscore(decode_score_kernel<TS, D, G, G, 1>);
            gscore(decode_score_kernel<TS, D, G, G, 2>);
        }
    } else if (s.GLM == 1) {
        gscore(decode_score_kernel<TS, D, G, 1>);
    } else {
        gscore(decode_score_kernel<TS, D, G, G>);
    }
    {
        const int nv = (L.splits * s.K + WAVE - 1) / WAVE;
        auto mg = [&](auto kern) {
            hipLaunchKernelGGL(kern, dim3(s.H_kv, num_seqs), dim3(64), 0, st, pkey, psc, sel, selsc, sel_idx, s.H_q,
                               s.H_kv, s.K, L.splits);
        };
        if (nv <= 4) mg(decode_merge_kernel<G, 4>);
        else if (nv <= 8) mg(decode_merge_kernel<G, 8>);
        else if (nv <= 16) mg(decode_merge_kernel<G, 16>);
        else mg(decode_merge_kernel<G, 32>);
    }
    if constexpr (std::is_same<T, bf16>::value && D == 128 && S == 64) {
        hipLaunchKernelGGL(decode_attend_fast_kernel<G>, dim3((L.np + 3) / 4, s.H_kv, num_seqs), dim3(256), 0, st,
                           (const bf16 *)q, (const bf16 *)k_cache, (const bf16 *)v_cache, block_table, max_pages,
                           seq_lens, sel, selsc, pm, pl, po, s.H_q, s.H_kv, s.W, s.K, L.np, s.scale);
    } else {
        const size_t dyn = (size_t)S * (D + 1) * 4 + (size_t)S * D * 4;
        auto att = decode_attend_kernel<T, D, S, G>;
        if (dyn > 48 * 1024) {
            const hipError_t e =
                hipFuncSetAttribute((const void *)att, hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn);
            if (e != hipSuccess) return e;
        }
        hipLaunchKernelGGL(att, dim3(L.nsb, s.H_kv, num_seqs), dim3(256), dyn, st, (const T *)q,
                           (const T *)k_cache, (const T *)v_cache, block_table, max_pages, seq_lens, sel, selsc, pm,
                           pl, po, s.H_q, s.H_kv, s.W, s.K, L.nsb, s.scale);
    }
    const int64_t rows = (int64_t)num_seqs * s.H_q;
    hipLaunchKernelGGL((decode_combine_kernel<T, D>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st, pm, pl, po,
                       (T *)out, lse, rows, L.np);
    return hipGetLastError();
}

template <typename T, typename TS>
static hipError_t dispatch_decode(const Shape &s, const DecodeLayout &L, int num_seqs, const void *q,
                                  const void *k_cache, const void *v_cache, const void *ksum_cache,
                                  const float *bsum_cache, const int32_t *block_table, int max_pages,
                                  const int32_t *seq_lens, const void *h, const void *w_down, const void *w_up,
                                  int d_model, int r, void *out, float *lse, int32_t *sel_idx, char *ws,
                                  hipStream_t st) {
#define HILS_DEC(DD, SS, GG)                                                                                    \
    if (s.D == DD && s.S == SS && s.G == GG)                                                                    \
        return go_decode<T, TS, DD, SS, GG>(s, L, num_seqs, q, k_cache, v_cache, ksum_cache, bsum_cache,         \
                                            block_table, max_pages, seq_lens, h, w_down, w_up, d_model, r, out, \
                                            lse, sel_idx, ws, st);
    HILS_DEC(64, 64, 1) HILS_DEC(64, 64, 2) HILS_DEC(64, 64, 4) HILS_DEC(64, 64, 8)
    HILS_DEC(64, 128, 1) HILS_DEC(64, 128, 2) HILS_DEC(64, 128, 4) HILS_DEC(64, 128, 8)
    HILS_DEC(128, 64, 1) HILS_DEC(128, 64, 2) HILS_DEC(128, 64, 4) HILS_DEC(128, 64, 8)
    HILS_DEC(128, 128, 1) HILS_DEC(128, 128, 2) HILS_DEC(128, 128, 4) HILS_DEC(128, 128, 8)
#undef HILS_DEC
    return hipErrorInvalidValue;
}

hipError_t launch_decode(const Shape &s, int num_seqs, const void *q, const void *k_cache, const void *v_cache,
                         const void *ksum_cache, const float *bsum_cache, const int32_t *block_table, int max_pages,
                         const int32_t *seq_lens, int max_seq_len, const void *h, const void *w_down,
                         const void *w_up, int d_model, int r, void *out, float *lse, int32_t *sel_idx,
                         void *workspace, hipStream_t st) {
    (void)max_seq_len;
    if (num_seqs == 0) return hipSuccess;
    const DecodeLayout L = decode_layout(s, num_seqs, max_pages);
    char *ws = (char *)workspace;
    if (s.io_bf16)
        return s.sum_bf16 ? dispatch_decode<bf16, bf16>(s, L, num_seqs, q, k_cache, v_cache, ksum_cache, bsum_cache,
                                                        block_table, max_pages, seq_lens, h, w_down, w_up, d_model,
                                                        r, out, lse, sel_idx, ws, st)
                          : dispatch_decode<bf16, float>(s, L, num_seqs, q, k_cache, v_cache, ksum_cache,
                                                         bsum_cache, block_table, max_pages, seq_lens, h, w_down,
                                                         w_up, d_model, r, out, lse, sel_idx, ws, st);
    return s.sum_bf16 ? dispatch_decode<float, bf16>(s, L, num_seqs, q, k_cache, v_cache, ksum_cache, bsum_cache,
                                                     block_table, max_pages, seq_lens, h, w_down, w_up, d_model, r,
                                                     out, lse, sel_idx, ws, st)
                      : dispatch_decode<float, float>(s, L, num_seqs, q, k_cache, v_cache, ksum_cache, bsum_cache,
                                                      block_table, max_pages, seq_lens, h, w_down, w_up, d_model, r,
                                                      out, lse, sel_idx, ws, st);
}

}  // namespace hils
