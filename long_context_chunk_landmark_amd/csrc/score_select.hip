// score_select.hip -- kernel 2: surrogate chunk scores, GQA max, top-K.
//
// hyper.ai HiLS summary, section 方法: s^_ic = q_i . k'_c / sqrt(d) + b'_c;
// chunks are ranked by s^ and the top K kept; under GQA the per-head scores
// are max-aggregated over the heads of a group and one top-K set is taken
// per group; Q-Cal replaces the scoring query by q_i + W_up W_down h_i.
//
// Design (MI355X): the scoring contraction is dense (every query of a chunk
// scores the same candidate set), so it runs on bf16 MFMA.  fp32 operands
// (k', a Q-Cal or fp32 query) enter as two-term bf16 splits, so the MFMA
// scores are approximate within a rigorous bound E on |approx - exact|
// (a two-term split is within 2^-16 |x| of x, fp32 accumulation,
// Cauchy-Schwarz: E = scale * kappa * ||q|| * max_c ||k'_c||).  The select kernel then
// takes a lower bound tau' of the K-th largest approximate group score,
// keeps every candidate whose approximate score is >= tau' - 2E (a superset
// of the exact top-K, about K + 1 candidates), recomputes those in fp32 on
// the vector ALUs, and takes the exact top-K by (score desc, index asc).
// Bit-exact selection, MFMA-rate scoring.
//
// Kernels:
//   ksum_prep        bf16 split k1 + k2 of k', its fp32 chunk-major copy,
//                    and per-(b, landmark head) max ||k'||
//   qcal_mfma        fp32 scoring queries q + W_up (W_down h), bf16 MFMA
//   qcal             the same for other shapes and fp32 inputs (VALU)
//   score_approx     bf16 MFMA scores -> ragged approximate group scores
//   select           exact refine + top-K per (b, g, query)
#include "hils_device.hpp"
#include "hils_internal.hpp"

namespace hils {

// ------------------------------------------------------------ workspace

int64_t score_agg_entries_per_bg(const Shape &s) {
    // rows of the query positions q0 .. q0 + N - 1, each padded to 16
    const int64_t w = s.W / s.S;
    return cand_row_offset((int64_t)s.q0 + s.N, w, s.S) - cand_row_offset(s.q0, w, s.S);
}

// Two-pass form (faster): two bf16 split terms of k', a chunk-major fp32
// copy of k', per-row bounds and the ragged approximate scores of every
// candidate (O(N^2 / S) per kv head).  Streaming form: the split terms of k'
// (three for fp32 summaries), max ||k'|| and the per-head scores of each
// row's listed chunks (O(N K) per head).  Auto takes the two-pass form
// unless its score array would exceed 32 GiB.
constexpr size_t SCORE_TWO_PASS_BUDGET = (size_t)32 << 30;

bool score_use_topk(const Shape &s) {
    if (s.score_mode == 1 || !score_topk_supported(s)) return false;
    if (s.score_mode == 2) return true;
    return (size_t)s.B * s.H_kv * score_agg_entries_per_bg(s) * 4 > SCORE_TWO_PASS_BUDGET;
}

size_t score_workspace_bytes(const Shape &s, bool qcal) {
    const size_t kr = (size_t)s.B * s.H_lm * s.C * s.D * 2;  // one bf16 term
    size_t b = 0;
    if (score_use_topk(s)) {
        b += align_up(kr * (s.sum_bf16 ? 1 : 3), 256);
        b += align_up((size_t)s.B * s.H_lm * 4, 256);  // knorm
        b += align_up((size_t)s.B * s.H_kv * s.N * score_topk_capacity(s) * s.G * 4, 256);  // heads
    } else {
        b += align_up(kr * 2, 256);                                  // ksb: two bf16 terms
        b += align_up((size_t)s.B * s.H_lm * s.C * s.D * 4, 256);  // kcm
        b += align_up((size_t)s.B * s.H_lm * 4, 256);               // knorm
        b += align_up((size_t)s.B * s.H_kv * s.N * 4, 256);         // err
        b += align_up((size_t)s.B * s.H_kv * score_agg_entries_per_bg(s) * 4, 256);
    }
    if (qcal) b += align_up((size_t)s.B * s.H_q * s.N * s.D * 4, 256);
    if (s.max_pages > 0) b += align_up((size_t)s.B * s.H_lm * s.C * 4, 256);  // paged: gathered b_sum
    if (s.agg_mode == 1) b += align_up((size_t)s.B * s.H_q * s.N * 4, 256);    // per-head log-sum-exp
    return b;
}

void score_workspace_carve(const Shape &s, bool qcal, void *base, ScoreWorkspace &ws) {
    char *p = (char *)base;
    const size_t kr = (size_t)s.B * s.H_lm * s.C * s.D * 2;
    ws.topk = score_use_topk(s);
    ws.ksb = p;
    ws.ksb2 = s.sum_bf16 ? nullptr : p + kr;
    ws.ksb3 = nullptr;
    ws.heads = nullptr;
    ws.kcm = nullptr;
    ws.err = nullptr;
    ws.agg = nullptr;
    ws.per_bg = 0;
    if (ws.topk) {
        ws.ksb3 = s.sum_bf16 ? nullptr : p + 2 * kr;
        p += align_up(kr * (s.sum_bf16 ? 1 : 3), 256);
        ws.knorm = (float *)p;
        p += align_up((size_t)s.B * s.H_lm * 4, 256);
        ws.heads = (float *)p;
        p += align_up((size_t)s.B * s.H_kv * s.N * score_topk_capacity(s) * s.G * 4, 256);
    } else {
        ws.ksb2 = p + kr;
        p += align_up(kr * 2, 256);
        ws.kcm = (float *)p;
        p += align_up((size_t)s.B * s.H_lm * s.C * s.D * 4, 256);
        ws.knorm = (float *)p;
        p += align_up((size_t)s.B * s.H_lm * 4, 256);
        ws.err = (float *)p;
        p += align_up((size_t)s.B * s.H_kv * s.N * 4, 256);
        ws.per_bg = score_agg_entries_per_bg(s);
        ws.agg = (float *)p;
        p += align_up((size_t)s.B * s.H_kv * ws.per_bg * 4, 256);
    }
    ws.q_s = qcal ? (float *)p : nullptr;
    if (qcal) p += align_up((size_t)s.B * s.H_q * s.N * s.D * 4, 256);
    ws.bsum = s.max_pages > 0 ? (float *)p : nullptr;
    if (s.max_pages > 0) p += align_up((size_t)s.B * s.H_lm * s.C * 4, 256);
    ws.lse = s.agg_mode == 1 ? (float *)p : nullptr;
}

// ------------------------------------------------------------ k' prep

constexpr int KPREP_ROWS = 32;  // k' rows per wave in ksum_prep

// Copy NB bytes (a multiple of 8; both pointers aligned to min(NB, 16)) with
// 16-byte (or 8-byte) accesses.
template <int NB>
__device__ __forceinline__ void copy_bytes(void *dst, const void *src) {
    static_assert(NB % 8 == 0, "whole 8-byte pieces");
    if constexpr (NB % 16 == 0) {
#pragma unroll
        for (int q = 0; q < NB / 16; ++q) ((u32x4 *)dst)[q] = ((const u32x4 *)src)[q];
    } else {
#pragma unroll
        for (int q = 0; q < NB / 8; ++q) ((uint2 *)dst)[q] = ((const uint2 *)src)[q];
    }
}

__global__ void fill_zero_kernel(float *p, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0.f;
}

// 16 lanes per k' row (D/16 elements each), 4 rows per wave.  Writes the
// two-term bf16 split k1 = bf16(k'), k2 = bf16(k' - k1) (same layout; k2
// only for fp32 summaries) for the MFMA pass, an fp32 chunk-major copy
// [B, H_kv, C, GLM, D] (the GLM landmark rows of a group contiguous per
// chunk) for the exact refinement, and the max norm per (b, landmark head).
// With a block table (bt != null) the summaries come from a paged cache
// [P, H_lm, D] (chunk c of sequence b is row bt[b * max_pages + c]), and
// b_sum [P, H_lm] is gathered into bsum_out [B, H_lm, C] as well.
template <typename TS, int D>
__global__ __launch_bounds__(256) void ksum_prep_kernel(const TS *__restrict__ k_sum, bf16 *__restrict__ ksb,
                                                        bf16 *__restrict__ ksb2, bf16 *__restrict__ ksb3,
                                                        float *__restrict__ kcm,
                                                        float *__restrict__ knorm, int C, int GLM, int64_t rows,
                                                        const int32_t *__restrict__ bt, int max_pages, int H_lm,
                                                        const float *__restrict__ bsum_in,
                                                        float *__restrict__ bsum_out) {
    constexpr int EL = D / 16;
    const int lane = lane_id();
    // each wave: KPREP_ROWS consecutive rows, four per step; the max norm
    // of its (b, l) run is kept in a register and flushed with one atomic
    // when the run ends (the knorm words see few atomics)
    const int64_t wrow0 = ((int64_t)blockIdx.x * (blockDim.x / WAVE) + threadIdx.x / WAVE) * KPREP_ROWS;
    int64_t cur_bl = -1;
    float wmax = 0.f;
    auto flush = [&]() {
        if (cur_bl >= 0 && lane == 0) atomicMax((unsigned int *)(knorm + cur_bl), __float_as_uint(wmax));
    };
    for (int step = 0; step < KPREP_ROWS / 4; ++step) {
        const int64_t row0 = wrow0 + step * 4;
        if (row0 >= rows) break;
        const int64_t row = row0 + (lane >> 4);
        const bool ok = row < rows;
        float ss = 0.f;
        if (ok) {
            // row = (b * H_lm + l) * C + c with l = g * GLM + e
            const int64_t c = row % C, bl = row / C;
            const int64_t e = bl % GLM, bg = bl / GLM;
            int64_t src_row = row;
            if (bt) {
                const int64_t b = bl / H_lm, l = bl % H_lm;
                src_row = (int64_t)bt[b * max_pages + c] * H_lm + l;
                if ((lane & 15) == 0) bsum_out[row] = bsum_in[src_row];
            }
            const TS *src = k_sum + src_row * D + (lane & 15) * EL;
            bf16 *dst = ksb + row * D + (lane & 15) * EL;
            // whole-slice vector loads and stores (the slices are 16-byte aligned)
            TS in[EL];
            bf16 o1[EL], o2[EL], o4[EL];
            float o3[EL];
            copy_bytes<EL * sizeof(TS)>(in, src);
#pragma unroll
            for (int x = 0; x < EL; ++x) {
                const float v = to_f32(in[x]);
                ss = fmaf(v, v, ss);
                o1[x] = (bf16)v;
                const float r1 = v - (float)o1[x];  // exact
                o2[x] = (bf16)r1;
                o4[x] = (bf16)(r1 - (float)o2[x]);
                o3[x] = v;
            }
            copy_bytes<EL * 2>(dst, o1);
            if constexpr (std::is_same<TS, float>::value) {
                copy_bytes<EL * 2>(ksb2 + row * D + (lane & 15) * EL, o2);
                if (ksb3) copy_bytes<EL * 2>(ksb3 + row * D + (lane & 15) * EL, o4);
            }
            if (kcm) copy_bytes<EL * 4>(kcm + ((bg * C + c) * GLM + e) * D + (lane & 15) * EL, o3);
        }
        ss = xor_sum<1, 8>(ss);
        const float nrm = ok ? sqrtf(ss) : 0.f;
        const int64_t last = min(row0 + 3, rows - 1);
        if (row0 / C == last / C) {  // the four rows share (b, l)
            const float m = xor_max<16, 32>(nrm);
            if (row0 / C != cur_bl) {
                flush();
                cur_bl = row0 / C;
                wmax = m;
            } else {
                wmax = fmaxf(wmax, m);
            }
        } else {  // a run boundary inside the step: per-row atomics
            flush();
            cur_bl = -1;
            if (ok && (lane & 15) == 0) atomicMax((unsigned int *)(knorm + row / C), __float_as_uint(nrm));
        }
    }
    flush();
}

// ------------------------------------------------------------ Q-Cal

// q_s[b,h,i,:] = q[b,h,i,:] + (W_up (W_down h[b,i]))[h*D : h*D + D]
// One block per 16 tokens.  Phase 1: u = W_down h for the 16 tokens (fp32,
// LDS).  Phase 2: each thread owns rows e of W_up and writes 16 tokens.
template <typename T>
__global__ __launch_bounds__(256) void qcal_kernel(const T *__restrict__ q, const T *__restrict__ h,
                                                   const T *__restrict__ w_down, const T *__restrict__ w_up,
                                                   float *__restrict__ q_s, int N, int H_q, int D, int d_model,
                                                   int r) {
    constexpr int TB = 16;
    extern __shared__ float u_lds[];  // [TB][r]
    const int64_t b = blockIdx.y;
    const int i0 = blockIdx.x * TB;
    const int nt = min(TB, N - i0);
    // phase 1: 256 threads over (token, a) pairs, each a d_model-long dot
    for (int p = threadIdx.x; p < TB * r; p += blockDim.x) {
        const int t = p / r, a = p % r;
        float acc = 0.f;
        if (t < nt) {
            const T *hr = h + (b * N + i0 + t) * (int64_t)d_model;
            const T *wr = w_down + (int64_t)a * d_model;
            for (int x = 0; x < d_model; ++x) acc = fmaf(to_f32(hr[x]), to_f32(wr[x]), acc);
        }
        u_lds[t * r + a] = acc;
    }
    __syncthreads();
    const int HD = H_q * D;
    for (int e = threadIdx.x; e < HD; e += blockDim.x) {
        float wrow[64];
        for (int a = 0; a < r; ++a) wrow[a] = to_f32(w_up[(int64_t)e * r + a]);
        const int hh = e / D, x = e % D;
        for (int t = 0; t < nt; ++t) {
            float acc = 0.f;
            for (int a = 0; a < r; ++a) acc = fmaf(wrow[a], u_lds[t * r + a], acc);
            const int64_t o = ((b * H_q + hh) * N + i0 + t) * (int64_t)D + x;
            q_s[o] = to_f32(q[o]) + acc;
        }
    }
}

// Split an fp32 value into three bf16 terms whose sum is the value (exact
// for normal values: each residual carries the next 8 significand bits).
__device__ __forceinline__ void split_bf16x3(float v, bf16 &a, bf16 &b, bf16 &c) {
    a = (bf16)v;
    const float r1 = v - (float)a;
    b = (bf16)r1;
    c = (bf16)(r1 - (float)b);
}

// bf16 Q-Cal on MFMA (r % 16 == 0, r <= 64, d_model % 32 == 0).  One wave
// owns 64 tokens as four 16-token column tiles.
//   Phase 1: U^T = W_down h^T, rows a padded to RP (rows >= r read as 0).
//     Products of bf16 values are exact in fp32, so this equals an fp32 FMA
//     chain up to the summation order.
//   Phase 2: Delta^T = W_up U^T over K = RP.  U (fp32) enters the bf16 MFMA
//     as its exact three-term split, so again only the fp32 accumulation
//     rounds.  The accumulator starts at q, so the chain yields q + Delta.
// An MFMA sums its K slots in any order, so lane group j of the phase-2
// operands carries U's rows 32s + 4j + {0..3} and 32s + 16 + 4j + {0..3}:
// exactly the rows phase 1 left in that lane (no data movement), with the
// W_up fragment read in the same order.
template <int RP>
__global__ __launch_bounds__(256) void qcal_mfma_kernel(const bf16 *__restrict__ q, const bf16 *__restrict__ h,
                                                        const bf16 *__restrict__ w_down,
                                                        const bf16 *__restrict__ w_up, float *__restrict__ q_s,
                                                        int N, int H_q, int D, int d_model, int r) {
    constexpr int NA = RP / 16;  // phase-1 row tiles
    constexpr int NK = RP / 32;  // phase-2 k-steps
    constexpr int NT = 4;        // 16-token column tiles per wave
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int col = lane & 15, j = lane >> 4;
    const int64_t b = blockIdx.y;
    const int t0 = (blockIdx.x * 4 + wave) * (16 * NT);
    if (t0 >= N) return;

    int tok[NT];
    const bf16 *hrow[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
        tok[n] = t0 + 16 * n + col;
        hrow[n] = h + (b * N + min(tok[n], N - 1)) * (int64_t)d_model + 8 * j;  // clamped rows are never stored
    }
    const bf16 *wrow[NA];
    bool a_ok[NA];
#pragma unroll
    for (int m = 0; m < NA; ++m) {
        a_ok[m] = 16 * m + col < r;
        wrow[m] = w_down + (int64_t)min(16 * m + col, r - 1) * d_model + 8 * j;
    }
    f32x4 acc[NA][NT];
#pragma unroll
    for (int m = 0; m < NA; ++m)
#pragma unroll
        for (int n = 0; n < NT; ++n) acc[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};
    const bf16x8 zero8 = {};
#pragma unroll 2
    for (int x = 0; x < d_model; x += 32) {
        bf16x8 af[NA], bfr[NT];
#pragma unroll
        for (int m = 0; m < NA; ++m) {
            const bf16x8 t = *(const bf16x8 *)(wrow[m] + x);
            af[m] = a_ok[m] ? t : zero8;
        }
#pragma unroll
        for (int n = 0; n < NT; ++n) bfr[n] = *(const bf16x8 *)(hrow[n] + x);
#pragma unroll
        for (int m = 0; m < NA; ++m)
#pragma unroll
            for (int n = 0; n < NT; ++n) acc[m][n] = mfma16(af[m], bfr[n], acc[m][n]);
    }

    // phase-2 B operands: split U into bf16 terms in the K order above
    bf16x8 u[NT][NK][3];
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
        for (int s = 0; s < NK; ++s)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float v = i < 4 ? acc[2 * s][n][i] : acc[2 * s + 1][n][i - 4];
                bf16 x1, x2, x3;
                split_bf16x3(v, x1, x2, x3);
                u[n][s][0][i] = x1;
                u[n][s][1][i] = x2;
                u[n][s][2][i] = x3;
            }

    const int HD = H_q * D;
    for (int e0 = 0; e0 < HD; e0 += 16) {
        const bf16 *wr = w_up + (int64_t)(e0 + col) * r;
        bf16x8 wf[NK];
#pragma unroll
        for (int s = 0; s < NK; ++s) {
            const int alo = 32 * s + 4 * j, ahi = alo + 16;
            bf16x4 lo = {}, hi = {};
            if (alo < r) lo = *(const bf16x4 *)(wr + alo);
            if (ahi < r) hi = *(const bf16x4 *)(wr + ahi);
            wf[s] = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
        const int hh = e0 / D, x0 = e0 % D + 4 * j;  // a 16-row tile stays inside one head (D % 16 == 0)
        const int64_t hb = (b * H_q + hh) * (int64_t)N;
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            const bool ok = tok[n] < N;
            const int64_t o = (hb + min(tok[n], N - 1)) * D + x0;
            const bf16x4 qv = *(const bf16x4 *)(q + o);
            f32x4 c = {(float)qv[0], (float)qv[1], (float)qv[2], (float)qv[3]};
#pragma unroll
            for (int s = 0; s < NK; ++s)
#pragma unroll
                for (int k = 0; k < 3; ++k) c = mfma16(wf[s], u[n][s][k], c);
            if (ok) *(f32x4 *)(q_s + o) = c;
        }
    }
}

// ------------------------------------------------------------ approximate scores (MFMA)

// One block = 64 NQP consecutive queries (NQP = 1 or 2; 64 queries lie in
// one query chunk, S being a multiple of 64) for one (b, g): 2 NQP G waves,
// wave (qp, e) owns query tiles 2qp, 2qp+1 (16 queries each) of head e of
// the group.  Query chunks are nested in their candidates (chunk qc has
// candidates 0 .. n(qc) - 1), so two chunks share every k' tile up to the
// smaller count: the block walks the larger one and each row keeps its own.  The B operands of the
// 16x16x32 MFMAs are q^T of those 32 queries (bf16 terms, in registers);
// the A operand is a 16-candidate k' tile staged in LDS, each fragment read
// feeding both query tiles.  D: lane l holds candidates 4*(l/16)+i of query
// l%16; the G heads of a query pair meet through LDS and wave (qp, 0) stores
// 16 contiguous bytes of each query's ragged score row.
//
// Split products: the scoring query q_s = t1 + t2 and k' = k1 + k2 with
// t1 = bf16(q_s), t2 = bf16(q_s - t1) (k likewise); the MFMAs sum
// t1 k1 + t1 k2 + t2 k1.  Terms that are exactly zero are skipped: bf16
// queries have t2 = 0, bf16 summaries k2 = 0.  A bf16 rounding is within
// 2^-8 of its argument, so each two-term split is within 2^-16 |x| of x
// and the dropped t2 k2 term within 2^-16 (1 + 2^-8)^2 |q_j||k_j|
// elementwise; by Cauchy-Schwarz |exact - approx| <= scale * kappa *
// ||q_s|| * max_c ||k'_c|| with kappa (set by the launcher) adding those
// terms to a bound on the fp32 accumulation.
//
// AM selects what the block produces: 0 the group max of the approximate
// scores; 1 (first pass of the normalised aggregation) each head's
// log-sum-exp of its approximate scores over the row's candidates, into
// lse [B, H_q, N]; 2 the group max of the scores minus those log-sum-exps.
// The subtracted constant is the same in the exact pass, so E still bounds
// |exact - approximate| of what is ranked.
template <typename TQ, int D, int G, bool KSPLIT, int AM, int NQP>
__global__ __launch_bounds__(128 * G * NQP) void score_approx_kernel(
    const TQ *__restrict__ q, const bf16 *__restrict__ ksb, const bf16 *__restrict__ ksb2,
    const float *__restrict__ b_sum, const float *__restrict__ knorm, float *__restrict__ agg_out,
    float *__restrict__ err_out, int N, int H_q, int H_kv, int H_lm, int C, int S, int W, int K, float scale,
    float kappa, int64_t per_bg, int q0, float *__restrict__ lse) {
    constexpr bool QSPLIT = std::is_same<TQ, float>::value;
    constexpr int NQT = QSPLIT ? 2 : 1;   // query terms
    constexpr int NKT = KSPLIT ? 2 : 1;   // k' terms
    constexpr int NT = 128 * G * NQP;
    constexpr int NPAIR = 2 * NQP;        // 32-query pairs per head
    constexpr int KS = D / 32;            // MFMA k-steps over the head dim
    constexpr int NB = D / 8;             // 16-byte blocks per k' row
    __shared__ u32x4 kt[NKT][G][16][NB];
    __shared__ float bt[G][16];
    __shared__ f32x4 px[G > 1 ? G - 1 : 1][NPAIR][2][WAVE];

    const int g = blockIdx.y;
    const int64_t b = blockIdx.z;
    const int i0 = blockIdx.x * 64 * NQP;  // local row; position q0 + i0 (q0 % S == 0)
    const int w = W / S;
    // candidates of the block's last row (the most of its rows)
    const int n = max(0, (q0 + min(N - 1, i0 + 64 * NQP - 1)) / S - w);
    if (n <= K) return;  // every candidate is selected; nothing to rank

    const int wave = threadIdx.x / WAVE, lane = lane_id();
    const int qp = wave % NPAIR, e = wave / NPAIR;
    const int grp = lane >> 4;
    const int n_row = max(0, (q0 + i0 + 32 * qp) / S - w);  // candidates of this wave's rows
    int iq[2], iqc[2];
    bool qvalid[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        iq[u] = i0 + (2 * qp + u) * 16 + (lane & 15);
        qvalid[u] = iq[u] < N;
        iqc[u] = qvalid[u] ? iq[u] : N - 1;
    }

    bf16x8 qf[2][NQT][KS];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const TQ *qr = q + (((int64_t)b * H_q + g * G + e) * N + iqc[u]) * D;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const int d0 = 32 * s + 8 * grp;
#pragma unroll
            for (int x = 0; x < 8; ++x) {
                const float v = to_f32(qr[d0 + x]);
                const bf16 v1 = (bf16)v;
                qf[u][0][s][x] = v1;
                if constexpr (QSPLIT) qf[u][NQT - 1][s][x] = (bf16)(v - (float)v1);
            }
        }
    }
    // normalised aggregation: this wave's head's log-sum-exp of its rows
    float lsev[2] = {0.f, 0.f};
    if constexpr (AM == 2) {
#pragma unroll
        for (int u = 0; u < 2; ++u) lsev[u] = lse[((int64_t)b * H_q + g * G + e) * N + iqc[u]];
    }
    float lm[2] = {-INFINITY, -INFINITY}, lz[2] = {0.f, 0.f};  // AM == 1: running max and sum
    if (AM != 1 && e == 0) {
        // bound of the group score: the largest per-head bound of the group
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            float emax = 0.f;
            for (int h = 0; h < G; ++h) {
                const int hd = g * G + h;
                const TQ *qr = q + (((int64_t)b * H_q + hd) * N + iqc[u]) * D;
                float ss = 0.f;
#pragma unroll
                for (int s = 0; s < KS; ++s)
#pragma unroll
                    for (int x = 0; x < 8; ++x) {
                        const float v = to_f32(qr[32 * s + 8 * grp + x]);
                        ss = fmaf(v, v, ss);
                    }
                ss = xor_sum<16, 32>(ss);
                emax = fmaxf(emax, sqrtf(ss) * knorm[b * H_lm + hd * H_lm / H_q]);
            }
            const float err = scale * kappa * emax + 1e-5f;
            if (qvalid[u] && grp == 0) err_out[((int64_t)b * H_kv + g) * N + iq[u]] = err;
        }
    }

    float *row[2];
#pragma unroll
    for (int u = 0; u < 2; ++u)
        row[u] = agg_out + ((int64_t)b * H_kv + g) * per_bg + cand_row_offset((int64_t)q0 + iqc[u], w, S) -
                 cand_row_offset(q0, w, S);
    const int cr = lane & 15;

    // k' tiles are staged through registers one tile ahead: the loads of
    // tile c0 + 16 are in flight while tile c0 is multiplied
    constexpr int NPRE = NKT * G * 16 * NB / NT;  // 16-byte pieces per thread and tile
    static_assert(NKT * G * 16 * NB == NPRE * NT, "staging pieces");
    u32x4 pre[NPRE];
    float bpre = 0.f;
    auto fetch = [&](int c0) {
#pragma unroll
        for (int j = 0; j < NPRE; ++j) {
            const int idx = threadIdx.x + j * NT;
            const int kk = idx / (G * 16 * NB), rem0 = idx % (G * 16 * NB);
            const int h = rem0 / (16 * NB), rem = rem0 % (16 * NB);
            const int rr = rem / NB, cb = rem % NB;
            const int c = c0 + rr;
            const int l = (g * G + h) * H_lm / H_q;
            pre[j] = u32x4{0u, 0u, 0u, 0u};
            if (c < n) pre[j] = *(const u32x4 *)((kk ? ksb2 : ksb) + (((int64_t)b * H_lm + l) * C + c) * D + cb * 8);
        }
        if (threadIdx.x < G * 16) {
            const int h = threadIdx.x / 16, rr = threadIdx.x % 16;
            const int c = c0 + rr;
            const int l = (g * G + h) * H_lm / H_q;
            bpre = c < n ? b_sum[((int64_t)b * H_lm + l) * C + c] : 0.f;
        }
    };
    fetch(0);
    for (int c0 = 0; c0 < n; c0 += 16) {
        __syncthreads();
#pragma unroll
        for (int j = 0; j < NPRE; ++j) {
            const int idx = threadIdx.x + j * NT;
            const int kk = idx / (G * 16 * NB), rem0 = idx % (G * 16 * NB);
            const int h = rem0 / (16 * NB), rem = rem0 % (16 * NB);
            const int rr = rem / NB, cb = rem % NB;
            kt[kk][h][rr][cb ^ (rr & 7)] = pre[j];
        }
        if (threadIdx.x < G * 16) bt[threadIdx.x / 16][threadIdx.x % 16] = bpre;
        if (c0 + 16 < n) fetch(c0 + 16);
        __syncthreads();
        f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const int blk = (4 * s + grp) ^ (cr & 7);
            bf16x8 a1;
            const u32x4 raw1 = kt[0][e][cr][blk];
            __builtin_memcpy(&a1, &raw1, 16);
#pragma unroll
            for (int u = 0; u < 2; ++u) acc[u] = mfma16(a1, qf[u][0][s], acc[u]);
            if constexpr (KSPLIT) {
                bf16x8 a2;
                const u32x4 raw2 = kt[NKT - 1][e][cr][blk];
                __builtin_memcpy(&a2, &raw2, 16);
#pragma unroll
                for (int u = 0; u < 2; ++u) acc[u] = mfma16(a2, qf[u][0][s], acc[u]);
            }
            if constexpr (QSPLIT) {
#pragma unroll
                for (int u = 0; u < 2; ++u) acc[u] = mfma16(a1, qf[u][NQT - 1][s], acc[u]);
            }
        }
        f32x4 best[2];
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int i = 0; i < 4; ++i) best[u][i] = fmaf(scale, acc[u][i], bt[e][4 * grp + i]) - lsev[u];
        if constexpr (AM == 1) {
            // running log-sum-exp over this lane's candidates c < n
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                float v[4], tm = -INFINITY;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    v[i] = c0 + 4 * grp + i < n_row ? best[u][i] : -INFINITY;
                    tm = fmaxf(tm, v[i]);
                }
                const float mn = fmaxf(lm[u], tm);
                if (mn != -INFINITY) {
                    float z = lz[u] * expf(lm[u] - mn);
#pragma unroll
                    for (int i = 0; i < 4; ++i) z += expf(v[i] - mn);
                    lz[u] = z;
                    lm[u] = mn;
                }
            }
            continue;
        }
        if constexpr (G > 1) {
            if (e > 0) {
                px[e - 1][qp][0][lane] = best[0];
                px[e - 1][qp][1][lane] = best[1];
            }
            __syncthreads();
            if (e == 0) {
#pragma unroll
                for (int x = 0; x < G - 1; ++x)
#pragma unroll
                    for (int u = 0; u < 2; ++u) {
                        const f32x4 o = px[x][qp][u][lane];
#pragma unroll
                        for (int i = 0; i < 4; ++i) best[u][i] = fmaxf(best[u][i], o[i]);
                    }
            }
        }
        if (e == 0 && c0 < n_row) {  // (c0 < n_row keeps the store inside the row's pad16(n_row))
#pragma unroll
            for (int u = 0; u < 2; ++u)
                if (qvalid[u]) *(f32x4 *)(row[u] + c0 + 4 * grp) = best[u];
        }
    }
    if constexpr (AM == 1) {
        // combine the four lane groups holding a query's candidates
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            float m = lm[u], z = lz[u];
#pragma unroll
            for (int off = 16; off <= 32; off <<= 1) {
                const float mo = __shfl_xor(m, off, WAVE), zo = __shfl_xor(z, off, WAVE);
                const float mn = fmaxf(m, mo);
                z = (m == -INFINITY ? 0.f : z * expf(m - mn)) + (mo == -INFINITY ? 0.f : zo * expf(mo - mn));
                m = mn;
            }
            if (qvalid[u] && grp == 0) lse[((int64_t)b * H_q + g * G + e) * N + iq[u]] = m + logf(z);
        }
    }
}

// ------------------------------------------------------------ exact refine + top-K


// 64-bit ranking key: larger score first, then lower chunk index first.
__device__ __forceinline__ uint64_t rank_key(float s, int idx) {
    return ((uint64_t)ord_key(s) << 32) | (uint64_t)(0xffffffffu - (uint32_t)idx);
}

// Sum over aligned groups of L lanes (L = 2..64), result in every lane.
template <int L>
__device__ __forceinline__ float group_sum(float v) {
    if constexpr (L >= 16) {
        v = row_sum16(v);
        if constexpr (L >= 32) v += __shfl_xor(v, 16, WAVE);
        if constexpr (L >= 64) v += __shfl_xor(v, 32, WAVE);
        return v;
    } else {
        return xor_sum<1, L / 2>(v);
    }
}

// Per-wave survivor list: chunk ids in ascending order, their exact
// ranking keys and per-head exact scores.  Entries [0, nref) are refined.
constexpr int SEL_CAP = 3 * WAVE;
template <int G>
struct SelLds {
    int idx[SEL_CAP];
    uint64_t key[SEL_CAP];
    float sc[SEL_CAP][G];
};

// One wave per (b, g, query).  SHARED: the G heads of a group share one
// landmark (H_lm == H_kv); otherwise each head has its own.
//
// 1. Threshold from the approximate group scores: tau' = K-th largest of the
//    per-lane top-4 (a lower bound of the K-th largest approximate score).
// 2. Survivors: approximate score >= tau' - 2E, a superset of the exact
//    top-K (E bounds |exact - approx|).  They are appended to the list in
//    ascending chunk order.
// 3. Exact refinement of the survivors from the fp32 chunk-major copy of k'
//    (the GLM rows of a group are contiguous: one coalesced read spread over
//    the wave, EPL elements per lane, reduced with DPP).
// 4. When the list would overflow, it is refined and cut in place to its
//    exact top-K (order kept); at the end the exact top-K of the list are
//    emitted in list order, i.e. ascending.
template <typename TQ, int D, int G, bool SHARED>
__global__ __launch_bounds__(256) void select_kernel(const TQ *__restrict__ q, const float *__restrict__ kcm,
                                                     const float *__restrict__ b_sum,
                                                     const float *__restrict__ agg_in,
                                                     const float *__restrict__ err_in, int32_t *__restrict__ sel_idx,
                                                     float *__restrict__ sel_score, int B, int N, int H_q, int H_kv,
                                                     int H_lm, int C, int S, int W, int K, float scale,
                                                     int64_t per_bg, int q0, const float *__restrict__ lse) {
    constexpr int GLM = SHARED ? 1 : G;
    constexpr int EPL = GLM * D / WAVE;   // elements of a survivor row per lane
    constexpr int LR = D / EPL;           // lanes covering one landmark row
    static_assert(EPL >= 1 && EPL <= 16 && (EPL % 4 == 0 || EPL < 4), "lane slice");
    __shared__ SelLds<G> lds_all[4];
    const int wave = threadIdx.x / WAVE, lane = lane_id();
    SelLds<G> &L = lds_all[wave];
    const int64_t row = (int64_t)blockIdx.x * 4 + wave;  // (b*H_kv + g)*N + i
    if (row >= (int64_t)B * H_kv * N) return;
    const int i = (int)(row % N);
    const int64_t bg = row / N;
    const int g = (int)(bg % H_kv);
    const int64_t b = bg / H_kv;
    const int w = W / S;
    const int n = max(0, (q0 + i) / S - w);  // row i is position q0 + i

    int32_t *out_idx = sel_idx + row * K;
    const int64_t sc_base = (b * H_q + (int64_t)g * G) * N + i;  // + e*N, then * K
    if (n == 0) {
        for (int k = lane; k < K; k += WAVE) out_idx[k] = -1;
        for (int e = 0; e < G; ++e)
            for (int k = lane; k < K; k += WAVE) sel_score[(sc_base + (int64_t)e * N) * K + k] = -INFINITY;
        return;
    }

    // scoring-query slices: lane covers elements [lane*EPL, lane*EPL + EPL)
    // of a survivor row, i.e. landmark row el = lane / LR, dims d0..d0+EPL
    const int el = lane / LR, d0 = (lane % LR) * EPL;
    float qv[SHARED ? G : 1][EPL];
#pragma unroll
    for (int e = 0; e < (SHARED ? G : 1); ++e) {
        const int head = SHARED ? e : el;
        const TQ *qr = q + ((b * H_q + (int64_t)g * G + head) * N + i) * D + d0;
#pragma unroll
        for (int x = 0; x < EPL; ++x) qv[e][x] = to_f32(qr[x]);
    }
    // normalised aggregation: each head's log-sum-exp over the candidates
    // (from the approximate pass) is subtracted before the group max
    float lsev[G];
#pragma unroll
    for (int e = 0; e < G; ++e) lsev[e] = (lse && n > K) ? lse[(b * H_q + (int64_t)g * G + e) * N + i] : 0.f;
    const float *kcm_g = kcm + bg * (int64_t)C * GLM * D;
    const float *bs_g = b_sum + (b * (int64_t)H_lm + (int64_t)g * GLM) * C;  // + e*C + c

    // ---- threshold of the approximate pass.  Rows of up to 64 * JR
    // candidates keep their approximate keys in registers (all loads in
    // flight at once, no second read); longer rows stream twice.
    constexpr int JR = 32;
    const int J = (n + WAVE - 1) / WAVE;
    const bool cached = J <= JR;
    const float *ar = agg_in + bg * per_bg + cand_row_offset((int64_t)q0 + i, w, S) - cand_row_offset(q0, w, S);
    uint32_t kreg[JR];
    if (cached) {
#pragma unroll
        for (int j = 0; j < JR; ++j) {
            const int c = j * WAVE + lane;
            kreg[j] = (j < J && c < n) ? ord_key(ar[c]) : 0u;
        }
    }
    uint32_t thr_key = 0;
    const bool rank_needed = n > K;
    if (rank_needed) {
        // tau' = K-th largest of the multiset of per-lane top-4 approximate
        // scores: those entries are distinct candidates, so at least K
        // candidates score >= tau' and tau' <= the K-th largest approximate
        // score (equal to it unless a lane holds more than four of the top K)
        uint32_t m0 = 0u, m1 = 0u, m2 = 0u, m3 = 0u;
        auto insert = [&](uint32_t x) {
            m3 = max(m3, min(m2, x));
            m2 = max(m2, min(m1, x));
            m1 = max(m1, min(m0, x));
            m0 = max(m0, x);
        };
        if (cached) {
#pragma unroll
            for (int j = 0; j < JR; ++j) insert(kreg[j]);
        } else {
            for (int j = 0; j < J; ++j) {
                const int c = j * WAVE + lane;
                insert(c < n ? ord_key(ar[c]) : 0u);
            }
        }
        uint32_t T = 0;
        for (int bit = 31; bit >= 0; --bit) {
            const uint32_t cand = T | (1u << bit);
            const int cnt = __popcll(__ballot(m0 >= cand)) + __popcll(__ballot(m1 >= cand)) +
                            __popcll(__ballot(m2 >= cand)) + __popcll(__ballot(m3 >= cand));
            if (cnt >= K) T = cand;
        }
        // every exact top-K member has approximate score >= tau' - 2E
        thr_key = ord_key(ord_key_inv(T) - 2.f * err_in[row]);
        if (thr_key == 0u) thr_key = 1u;
    }

    // ---- exact refinement of list entries [k0, k1): per-head s^ into
    // L.sc, ranking key into L.key.  RB rows are loaded before any is
    // reduced; one row at a time measured fastest (fewer registers, more
    // rows in flight per SIMD than a batch of loads per wave buys).
    constexpr int RB = 1;
    auto refine = [&](int k0, int k1) {
        for (int kb = k0; kb < k1; kb += RB) {
            const int cnt = min(RB, k1 - kb);
            float kx[RB][EPL];
            int cs[RB];
#pragma unroll
            for (int u = 0; u < RB; ++u) {
                cs[u] = L.idx[kb + min(u, cnt - 1)];
                const float *kr = kcm_g + (int64_t)cs[u] * GLM * D + lane * EPL;
                if constexpr (EPL >= 4) {
#pragma unroll
                    for (int x = 0; x < EPL; x += 4) {
                        const f32x4 v4 = *(const f32x4 *)(kr + x);
                        kx[u][x] = v4[0], kx[u][x + 1] = v4[1], kx[u][x + 2] = v4[2], kx[u][x + 3] = v4[3];
                    }
                } else {
#pragma unroll
                    for (int x = 0; x < EPL; ++x) kx[u][x] = kr[x];
                }
            }
#pragma unroll
            for (int u = 0; u < RB; ++u) {
                if (u >= cnt) break;
                const int c = cs[u], slot = kb + u;
                float agg = -INFINITY;
                if constexpr (SHARED) {
                    const float bb = bs_g[c];
#pragma unroll
                    for (int e = 0; e < G; ++e) {
                        float part = 0.f;
#pragma unroll
                        for (int x = 0; x < EPL; ++x) part = fmaf(qv[e][x], kx[u][x], part);
                        const float sc = fmaf(scale, group_sum<WAVE>(part), bb);
                        if (lane == 0) L.sc[slot][e] = sc;
                        agg = fmaxf(agg, sc - lsev[e]);
                    }
                } else {
                    float part = 0.f;
#pragma unroll
                    for (int x = 0; x < EPL; ++x) part = fmaf(qv[0][x], kx[u][x], part);
                    const float sc = fmaf(scale, group_sum<LR>(part), bs_g[(int64_t)el * C + c]);
                    if (lane % LR == 0) L.sc[slot][el] = sc;
                    float sub = lsev[0];
#pragma unroll
                    for (int e = 1; e < G; ++e) sub = el == e ? lsev[e] : sub;
                    agg = sc - sub;
#pragma unroll
                    for (int m = LR; m < WAVE; m <<= 1) agg = fmaxf(agg, __shfl_xor(agg, m, WAVE));
                }
                if (lane == 0) L.key[slot] = rank_key(agg, c);
            }
        }
    };
    // keys of the (refined) list, three slots per lane, 0 past cnt
    auto list_keys = [&](int cnt, uint64_t (&keys)[3]) {
#pragma unroll
        for (int v = 0; v < 3; ++v) keys[v] = lane + WAVE * v < cnt ? L.key[lane + WAVE * v] : 0ull;
    };

    int cnt = 0, nref = 0;
    // cut the list to its exact top K, keeping the order
    auto shrink = [&]() {
        wave_sync();
        refine(nref, cnt);
        wave_sync();
        uint64_t keys[3];
        list_keys(cnt, keys);
        const uint64_t T = kth_largest64<3>(keys, K);
        // forward compaction: a kept entry moves to pos <= its slot, and
        // every slot of a 64-slot round is read before the round writes
        int base = 0;
#pragma unroll
        for (int v = 0; v < 3; ++v) {
            const int slot = lane + WAVE * v;
            const bool keep = keys[v] >= T && keys[v] != 0ull;
            const uint64_t m = __ballot(keep);
            const int pos = base + __popcll(m & lanemask_lt());
            int id = 0;
            float scv[G];
            if (keep) {
                id = L.idx[slot];
#pragma unroll
                for (int e = 0; e < G; ++e) scv[e] = L.sc[slot][e];
            }
            wave_sync();
            if (keep) {
                L.idx[pos] = id;
                L.key[pos] = keys[v];
#pragma unroll
                for (int e = 0; e < G; ++e) L.sc[pos][e] = scv[e];
            }
            wave_sync();
            base += __popcll(m);
        }
        cnt = nref = base;
        wave_sync();
    };
    // append the candidates whose lanes hold surv (one 64-candidate slice)
    auto push = [&](int c, bool surv) {
        const uint64_t m = __ballot(surv);
        if (surv) L.idx[cnt + __popcll(m & lanemask_lt())] = c;
        cnt += __popcll(m);
    };
    auto take = [&](int c, bool surv) {
        if (cnt + __popcll(__ballot(surv)) > SEL_CAP) shrink();
        push(c, surv);
    };

    if (!rank_needed) {
        for (int c0 = 0; c0 < n; c0 += WAVE) push(c0 + lane, c0 + lane < n);  // n <= K < SEL_CAP
    } else {
        // survivors straight from the cached keys when the list holds them
        // all (the usual case); otherwise stream them, cutting the list to
        // its top K whenever it fills
        int total = SEL_CAP + 1;
        if (cached) {
            total = 0;
#pragma unroll
            for (int j = 0; j < JR; ++j) total += __popcll(__ballot(j < J && kreg[j] >= thr_key));
        }
        if (total <= SEL_CAP) {
#pragma unroll
            for (int j = 0; j < JR; ++j) push(j * WAVE + lane, j < J && kreg[j] >= thr_key);  // kreg = 0 past n
        } else {
            for (int j = 0; j < J; ++j) {
                const int c = j * WAVE + lane;
                take(c, c < n && ord_key(ar[c]) >= thr_key);
            }
        }
    }
    wave_sync();
    refine(nref, cnt);
    wave_sync();

    // ---- emit the exact top K of the list, in list (= ascending) order
    uint64_t keys[3];
    list_keys(cnt, keys);
    const uint64_t T = cnt > K ? kth_largest64<3>(keys, K) : 1ull;
    int base = 0;
#pragma unroll
    for (int v = 0; v < 3; ++v) {
        const int slot = lane + WAVE * v;
        const bool win = keys[v] >= T && keys[v] != 0ull;
        const uint64_t m = __ballot(win);
        const int pos = base + __popcll(m & lanemask_lt());
        if (win) {
            out_idx[pos] = L.idx[slot];
#pragma unroll
            for (int e = 0; e < G; ++e) sel_score[(sc_base + (int64_t)e * N) * K + pos] = L.sc[slot][e];
        }
        base += __popcll(m);
    }
    for (int k = base + lane; k < K; k += WAVE) {
        out_idx[k] = -1;
#pragma unroll
        for (int e = 0; e < G; ++e) sel_score[(sc_base + (int64_t)e * N) * K + k] = -INFINITY;
    }
}

// ------------------------------------------------------------ launch

template <typename TQ, int D, int G, int AM>
static void go_approx_m(const Shape &s, const TQ *qv, const float *b_sum, const ScoreWorkspace &ws, float kappa,
                        hipStream_t st) {
    // 128-query blocks while they fit 1024 threads and the k' tile still
    // gives every thread whole 16-byte pieces to stage
    constexpr int NQP = (G <= 4 && D == 128) ? 2 : 1;
    const dim3 grid((unsigned)((s.N + 64 * NQP - 1) / (64 * NQP)), (unsigned)s.H_kv, (unsigned)s.B),
        block(128 * G * NQP);
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, grid, block, 0, st, qv, (const bf16 *)ws.ksb, (const bf16 *)ws.ksb2, b_sum,
                           ws.knorm, ws.agg, ws.err, s.N, s.H_q, s.H_kv, s.H_lm, s.C, s.S, s.W, s.K, s.scale, kappa,
                           ws.per_bg, s.q0, ws.lse);
    };
    if (s.sum_bf16) go(score_approx_kernel<TQ, D, G, false, AM, NQP>);
    else go(score_approx_kernel<TQ, D, G, true, AM, NQP>);
}

template <typename TQ, int D, int G>
static void go_approx(const Shape &s, const TQ *qv, const float *b_sum, const ScoreWorkspace &ws, float kappa,
                      hipStream_t st) {
    if (s.agg_mode == 1) {
        go_approx_m<TQ, D, G, 1>(s, qv, b_sum, ws, kappa, st);  // per-head log-sum-exp
        // normalised group max (the streaming kernel ranks by it itself)
        if (!ws.topk) go_approx_m<TQ, D, G, 2>(s, qv, b_sum, ws, kappa, st);
    } else {
        go_approx_m<TQ, D, G, 0>(s, qv, b_sum, ws, kappa, st);
    }
}

template <typename TQ>
static hipError_t dispatch_approx(const Shape &s, const TQ *qv, const float *b_sum, const ScoreWorkspace &ws,
                                  float kappa, hipStream_t st) {
#define HILS_APPROX(DD, GG)                                                  \
    if (s.D == DD && s.G == GG) {                                            \
        go_approx<TQ, DD, GG>(s, qv, b_sum, ws, kappa, st);                  \
        return hipGetLastError();                                            \
    }
    HILS_APPROX(64, 1) HILS_APPROX(64, 2) HILS_APPROX(64, 4) HILS_APPROX(64, 8)
    HILS_APPROX(128, 1) HILS_APPROX(128, 2) HILS_APPROX(128, 4) HILS_APPROX(128, 8)
#undef HILS_APPROX
    return hipErrorInvalidValue;
}

template <typename TQ, int D, int G>
static void go_select(const Shape &s, const TQ *qv, const float *b_sum, const ScoreWorkspace &ws, int32_t *sel_idx,
                      float *sel_score, hipStream_t st) {
    const int64_t rows = (int64_t)s.B * s.H_kv * s.N;
    const dim3 grid((unsigned)((rows + 3) / 4)), block(256);
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, grid, block, 0, st, qv, (const float *)ws.kcm, b_sum, (const float *)ws.agg,
                           (const float *)ws.err, sel_idx, sel_score, s.B, s.N, s.H_q, s.H_kv, s.H_lm, s.C, s.S, s.W,
                           s.K, s.scale, ws.per_bg, s.q0, (const float *)ws.lse);
    };
    if (s.GLM == 1 && G > 1) go(select_kernel<TQ, D, G, true>);
    else go(select_kernel<TQ, D, G, false>);
}

template <typename TQ>
static hipError_t dispatch_select(const Shape &s, const TQ *qv, const float *b_sum, const ScoreWorkspace &ws,
                                  int32_t *sel_idx, float *sel_score, hipStream_t st) {
#define HILS_SEL(DD, GG)                                                     \
    if (s.D == DD && s.G == GG) {                                            \
        go_select<TQ, DD, GG>(s, qv, b_sum, ws, sel_idx, sel_score, st);     \
        return hipGetLastError();                                            \
    }
    HILS_SEL(64, 1) HILS_SEL(64, 2) HILS_SEL(64, 4) HILS_SEL(64, 8)
    HILS_SEL(128, 1) HILS_SEL(128, 2) HILS_SEL(128, 4) HILS_SEL(128, 8)
#undef HILS_SEL
    return hipErrorInvalidValue;
}

hipError_t launch_score_select(const Shape &s, const void *q, const void *k_sum, const float *b_sum, const void *h,
                               const void *w_down, const void *w_up, int d_model, int r, int32_t *sel_idx,
                               float *sel_score, const ScoreWorkspace &ws, hipStream_t st) {
    if ((int64_t)s.B * s.N == 0) return hipSuccess;
    hipError_t e;
    // k' prep: bf16 copy + max norm per (b, landmark head)
    const int64_t nl = (int64_t)s.B * s.H_lm;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)((nl + 255) / 256)), dim3(256), 0, st, ws.knorm, nl);
    const int64_t krows = (int64_t)s.B * s.H_lm * s.C;
    if (krows > 0) {
        const dim3 grid((unsigned)((krows + 4 * KPREP_ROWS - 1) / (4 * KPREP_ROWS))), block(256);
        auto prep = [&](auto kern, auto *src) {
            hipLaunchKernelGGL(kern, grid, block, 0, st, src, (bf16 *)ws.ksb, (bf16 *)ws.ksb2, (bf16 *)ws.ksb3,
                               ws.kcm, ws.knorm, s.C, s.GLM, krows, s.bt, s.max_pages, s.H_lm, b_sum, ws.bsum);
        };
        if (s.sum_bf16) {
            if (s.D == 64) prep(ksum_prep_kernel<bf16, 64>, (const bf16 *)k_sum);
            else prep(ksum_prep_kernel<bf16, 128>, (const bf16 *)k_sum);
        } else {
            if (s.D == 64) prep(ksum_prep_kernel<float, 64>, (const float *)k_sum);
            else prep(ksum_prep_kernel<float, 128>, (const float *)k_sum);
        }
    }
    // paged prefill: the scorers read the gathered b_sum
    if (s.bt) b_sum = ws.bsum;
    if ((e = hipGetLastError()) != hipSuccess) return e;

    // scoring queries
    const bool qcal = h != nullptr;
    if (qcal) {
        const dim3 grid((unsigned)((s.N + 15) / 16), (unsigned)s.B), block(256);
        const size_t lds = (size_t)16 * r * sizeof(float);
        const dim3 mgrid((unsigned)((s.N + 255) / 256), (unsigned)s.B);
        if (s.io_bf16 && r % 16 == 0 && r <= 32 && d_model % 32 == 0)
            hipLaunchKernelGGL(qcal_mfma_kernel<32>, mgrid, block, 0, st, (const bf16 *)q, (const bf16 *)h,
                               (const bf16 *)w_down, (const bf16 *)w_up, ws.q_s, s.N, s.H_q, s.D, d_model, r);
        else if (s.io_bf16 && r % 16 == 0 && r <= 64 && d_model % 32 == 0)
            hipLaunchKernelGGL(qcal_mfma_kernel<64>, mgrid, block, 0, st, (const bf16 *)q, (const bf16 *)h,
                               (const bf16 *)w_down, (const bf16 *)w_up, ws.q_s, s.N, s.H_q, s.D, d_model, r);
        else if (s.io_bf16)
            hipLaunchKernelGGL(qcal_kernel<bf16>, grid, block, lds, st, (const bf16 *)q, (const bf16 *)h,
                               (const bf16 *)w_down, (const bf16 *)w_up, ws.q_s, s.N, s.H_q, s.D, d_model, r);
        else
            hipLaunchKernelGGL(qcal_kernel<float>, grid, block, lds, st, (const float *)q, (const float *)h,
                               (const float *)w_down, (const float *)w_up, ws.q_s, s.N, s.H_q, s.D, d_model, r);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }

    // kappa, relative to ||q_s|| ||k'||.  Accumulation: the products of
    // bf16 terms are exact in fp32 and at most 3 d <= 384 of them are summed,
    // so fp32 rounding stays within gamma_384 (1 + 2^-7) < 2.4e-5, bounded
    // here by 2^-14 whatever order the MFMA sums in.  Representation: each
    // two-term split (fp32 queries, fp32 summaries) and the dropped t2 k2
    // term add at most 2^-16 (1 + 2^-7) each.
    const int nq = (qcal || !s.io_bf16) ? 1 : 0, nk = s.sum_bf16 ? 0 : 1;
    const float kappa = 1.0f / 16384.f + (float)(nq + nk + nq * nk) * (1.f + 1.f / 128.f) / 65536.f;

    if (ws.topk) {
        // normalised aggregation: each head's log-sum-exp over the candidates first
        const bool qf32 = qcal || !s.io_bf16;
        const void *qv = qcal ? (const void *)ws.q_s : q;
        if (s.agg_mode == 1) {
            if (qf32) e = dispatch_approx<float>(s, (const float *)qv, b_sum, ws, kappa, st);
            else e = dispatch_approx<bf16>(s, (const bf16 *)qv, b_sum, ws, kappa, st);
            if (e != hipSuccess) return e;
        }
        return launch_score_topk(s, qv, qf32, ws, b_sum, sel_idx, sel_score, st);
    }
    if (qcal || !s.io_bf16) {
        const float *qv = qcal ? ws.q_s : (const float *)q;
        if ((e = dispatch_approx<float>(s, qv, b_sum, ws, kappa, st)) != hipSuccess) return e;
        return dispatch_select<float>(s, qv, b_sum, ws, sel_idx, sel_score, st);
    }
    const bf16 *qv = (const bf16 *)q;
    if ((e = dispatch_approx<bf16>(s, qv, b_sum, ws, kappa, st)) != hipSuccess) return e;
    return dispatch_select<bf16>(s, qv, b_sum, ws, sel_idx, sel_score, st);
}

}  // namespace hils
