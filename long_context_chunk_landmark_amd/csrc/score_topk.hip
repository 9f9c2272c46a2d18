// score_topk.hip -- kernel 2 in streaming form: surrogate chunk scores, the
// GQA group max and the exact top-K of every query in one kernel, with no
// per-candidate score written to memory.
//
// hyper.ai HiLS summary, section 方法: s^_ic = q_i . k'_c / sqrt(d) + b'_c
// (surrogate-score equation); the heads of a GQA group rank the chunks by
// the max of their scores and keep one top-K set (Q-Cal and GQA paragraph);
// Q-Cal only changes the scoring query.
//
// A block owns 64 NQP consecutive queries of one kv group: wave (qp, e)
// holds the query fragments of 32 of them (one query chunk: they share the
// candidate set c < n) for head e of the group.  Query chunks are nested in
// their candidates, so the block walks the candidates of its last rows and
// each row uses its own.  The candidates are walked twice in tiles of 16
// chunks staged in LDS, the next tile's loads in flight while the current
// one is multiplied (bf16 split terms of k', A operand of 16x16x32 MFMAs;
// D: lane l holds candidates 4(l/16)+i of query l%16):
//   pass 1  two-term products (t1 k1 + t1 k2, and t2 k1 for an fp32 query,
//           with t1, t2 and k1, k2 the leading bf16 terms of q_s and k'),
//           within E1 of the exact scores.  Each row's candidates are dealt to 16 streams (the 4
//           lane groups x the 4 accumulator slots, spread over the waves),
//           and each stream keeps its T largest group scores.  The K-th
//           largest of those 16 T values (distinct candidates, 16 T >= K) is
//           a lower bound tau of the row's K-th largest pass-1 score.
//   pass 2  the products of the split terms that make up q_s . k' exactly
//           (k' = k1 + k2 + k3 holds an fp32 value to 2^-24; an fp32 query
//           likewise, the three smallest cross terms, below 2^-23 together,
//           dropped), summed in fp32: the scores the selection ranks by,
//           within E2 of the exact ones.  A chunk can be among the row's top
//           K only if its score is >= tau - E1 - E2 (the K chunks with the
//           largest pass-1 scores all score at least that), so only those
//           are listed, in ascending chunk order, in the row's LDS list; their
//           per-head scores go to a scratch array.
//   emit    the exact top K of each list by (group score desc, chunk index
//           asc), written ascending with each head's score.
// A list about to overflow is first cut to its exact top K (a dropped chunk
// has K better ones), so the result does not depend on the list capacity.
// The group scores of identical chunks are computed by identical
// arithmetic, so exact ties keep the lower index.
#include <type_traits>

#include "hils_device.hpp"
#include "hils_internal.hpp"

namespace hils {

namespace {

// ranking key: larger score first, then the lower chunk index
__device__ __forceinline__ uint64_t topk_key(float s, int idx) {
    return ((uint64_t)ord_key(s) << 32) | (uint64_t)(0xffffffffu - (uint32_t)idx);
}

// kk-th largest (kk >= 1) of the 32-bit keys held NV per lane (0 = empty):
// bisection over the bits, counting with ballots.
template <int NV>
__device__ __forceinline__ uint32_t kth_largest32(const uint32_t (&keys)[NV], int kk) {
    uint32_t hi = 0;
    for (int bit = 31; bit >= 0; --bit) {
        const uint32_t cand = hi | (1u << bit);
        int cnt = 0;
#pragma unroll
        for (int v = 0; v < NV; ++v) cnt += __popcll(__ballot(keys[v] >= cand));
        if (cnt >= kk) hi = cand;
    }
    return hi;
}

// The values of x held by the four lanes of this lane's row (lanes l % 16 +
// 16 j, j = 0..3), in lane-group order, with the gfx950 lane swaps.
__device__ __forceinline__ void row_lanes4(int x, int (&v)[4]) {
    const auto a = __builtin_amdgcn_permlane16_swap((uint32_t)x, (uint32_t)x, false, false);  // groups 2j, 2j+1
    const auto lo = __builtin_amdgcn_permlane32_swap(a[0], a[0], false, false);               // groups 0, 2
    const auto hi = __builtin_amdgcn_permlane32_swap(a[1], a[1], false, false);               // groups 1, 3
    v[0] = (int)lo[0];
    v[1] = (int)hi[0];
    v[2] = (int)lo[1];
    v[3] = (int)hi[1];
}

}  // namespace

// Compile-time layout of one instantiation: 64 NQP rows per block (two
// 32-query pairs per 64; 128-query blocks where they fit 1024 threads and
// the LDS).
template <int D, int G, int NKT, int KC, int NQP_ = 0>
struct TopkPlan {
    static constexpr int NQP = NQP_ ? NQP_ : ((G <= 4 && KC <= 32) ? 2 : 1);
    static constexpr int ROWS = 64 * NQP;                   // queries per block
    static constexpr int NPAIR = 2 * NQP;                   // 32-query pairs per block
    static constexpr int KS = D / 32;                       // MFMA k-steps over the head dim
    static constexpr int NB = D / 8;                        // 16-byte blocks per k' row
    static constexpr int NW = NPAIR * G;                    // waves
    static constexpr int NT = NW * WAVE;
    static constexpr int T = KC / 8 < 2 ? 2 : (KC / 8 > 8 ? 8 : KC / 8);  // stream depth (16 T >= KC)
    static constexpr int CAP = KC + 16;                     // list capacity per row
    static constexpr int NV = (CAP + WAVE - 1) / WAVE;      // list entries per lane
    static constexpr int NVG = (16 * T + WAVE - 1) / WAVE;  // stream values per lane
    static constexpr int SPW = G >= 4 ? 1 : 4 / G;          // pass-1 accumulator slots per wave
    static constexpr int PIECES1 = G * 16 * NB;             // 16-byte pieces of one term of a tile
    static constexpr int NPRE = (NKT * PIECES1 + NT - 1) / NT;  // pieces per thread and tile
    static constexpr size_t kt_bytes = (size_t)NKT * PIECES1 * 16;
    static constexpr size_t px_bytes = (size_t)G * NPAIR * 2 * WAVE * 16;
    static constexpr size_t region_words =
        (size_t)ROWS * 16 * T > (size_t)ROWS * CAP * 2 ? (size_t)ROWS * 16 * T : (size_t)ROWS * CAP * 2;
    static constexpr size_t lds_bytes = kt_bytes + (size_t)G * 16 * 4 + px_bytes + ROWS * 12 + region_words * 4;
};

template <typename TQ, int D, int G, int NKT, int KC>
__global__ __launch_bounds__((TopkPlan<D, G, NKT, KC>::NT)) void score_topk_kernel(
    const TQ *__restrict__ q, const bf16 *__restrict__ ks, int64_t kterm, const float *__restrict__ b_sum,
    const float *__restrict__ knorm,
    const float *__restrict__ lse, float *__restrict__ heads, int32_t *__restrict__ sel_idx,
    float *__restrict__ sel_score, int N, int H_q, int H_kv, int H_lm, int C, int S, int W, int K, float scale,
    float kappa, int q0) {
    using P = TopkPlan<D, G, NKT, KC>;
    constexpr bool QSPLIT = std::is_same<TQ, float>::value;
    constexpr int NQT = QSPLIT ? 3 : 1;  // query terms in pass 2
    constexpr int KS = P::KS, NB = P::NB, NW = P::NW, NT = P::NT, T = P::T, CAP = P::CAP, NV = P::NV;
    constexpr int NVG = P::NVG, SPW = P::SPW, ROWS = P::ROWS, NPAIR = P::NPAIR;
    constexpr int PIECES1 = P::PIECES1, NPRE = P::NPRE;
    __shared__ u32x4 kt[NKT][G][16][NB];     // staged split terms of the tile's k' rows
    __shared__ float bt[G][16];              // and their b'
    __shared__ f32x4 px[G][NPAIR][2][WAVE];  // per-head scores of the tile, exchanged between the waves
    __shared__ float rowE[ROWS];             // bound of |pass-1 - pass-2| per row
    __shared__ float thr[ROWS];              // listing threshold per row
    __shared__ int rcnt[ROWS];               // list length per row
    __shared__ uint32_t region[P::region_words];  // pass 1: stream values; pass 2: the lists
    float *gat = (float *)region;                           // [row][16 T]
    int *lidx = (int *)region;                              // [row][CAP] chunk ids
    float *lkey = (float *)(region + ROWS * CAP);           // [row][CAP] group scores

    const int g = blockIdx.y;
    const int64_t b = blockIdx.z;
    const int i0 = blockIdx.x * ROWS;  // local row; position q0 + i0 (q0 % S == 0, S >= 64)
    const int w = W / S;
    const int tid = threadIdx.x, wave = tid / WAVE, lane = lane_id(), grp = lane >> 4, cr = lane & 15;
    const int qp = wave % NPAIR, e = wave / NPAIR;
    // candidates of this wave's rows, and of the block's last rows (the most)
    const int n_row = max(0, (q0 + i0 + 32 * qp) / S - w);
    const int n = max(0, (q0 + min(N - 1, i0 + ROWS - 1)) / S - w);
    const int GLM = H_lm == H_q ? G : 1;     // landmark rows of the group
    const int el = GLM == G ? e : 0;         // head e's landmark row within them
    const int64_t bg = b * H_kv + g;
    const int64_t hq0 = b * H_q + (int64_t)g * G;  // first query head of the group
    const int64_t lm0 = b * H_lm + (int64_t)g * GLM;

    if (n == 0) {  // no candidates: every slot is padding
        for (int t = tid; t < ROWS * K; t += NT) {
            const int iq = i0 + t / K, kk = t % K;
            if (iq >= N) continue;
            sel_idx[(bg * N + iq) * K + kk] = -1;
            for (int h = 0; h < G; ++h) sel_score[((hq0 + h) * N + iq) * K + kk] = -INFINITY;
        }
        return;
    }
    const bool rank = n > K;             // some row of the block ranks
    const bool rank_row = n_row > K;     // this wave's rows rank

    // ---- query fragments of head e for rows u = 0, 1 (16 queries each)
    int iq[2];
    bool qvalid[2];
    bf16x8 qf[2][NQT][KS];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        iq[u] = i0 + qp * 32 + u * 16 + cr;
        qvalid[u] = iq[u] < N;
        const TQ *qr = q + ((hq0 + e) * N + min(iq[u], N - 1)) * D;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
#pragma unroll
            for (int x = 0; x < 8; ++x) {
                const float v = to_f32(qr[32 * s + 8 * grp + x]);
                const bf16 t1 = (bf16)v;
                qf[u][0][s][x] = t1;
                if constexpr (QSPLIT) {
                    const float r1 = v - (float)t1;
                    const bf16 t2 = (bf16)r1;
                    qf[u][1][s][x] = t2;
                    qf[u][2][s][x] = (bf16)(r1 - (float)t2);
                }
            }
        }
    }
    // per-head log-sum-exp of the normalised aggregation (0 otherwise)
    float lsev[2][G];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int h = 0; h < G; ++h) lsev[u][h] = (lse && rank_row) ? lse[(hq0 + h) * N + min(iq[u], N - 1)] : 0.f;
    if (tid < ROWS) {
        rcnt[tid] = 0;
        thr[tid] = -INFINITY;
    }
    if (rank && e == 0) {
        // E1 + E2 of each row: scale * kappa * max over the heads of
        // ||q_h|| * max_c ||k'_c|| (Cauchy-Schwarz), plus the rounding of
        // the b' additions
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            float emax = 0.f;
            for (int h = 0; h < G; ++h) {
                const TQ *qr = q + ((hq0 + h) * N + min(iq[u], N - 1)) * D;
                float ss = 0.f;
#pragma unroll
                for (int s = 0; s < KS; ++s)
#pragma unroll
                    for (int x = 0; x < 8; ++x) {
                        const float v = to_f32(qr[32 * s + 8 * grp + x]);
                        ss = fmaf(v, v, ss);
                    }
                ss = xor_sum<16, 32>(ss);
                emax = fmaxf(emax, sqrtf(ss) * knorm[lm0 + (GLM == G ? h : 0)]);
            }
            if (grp == 0) rowE[qp * 32 + u * 16 + cr] = scale * kappa * emax + 2e-5f;
        }
    }

    // ---- tile staging: nterms split terms of k' rows c0 .. c0 + 15 (zero
    // past n) go to registers (fetch, issued a tile ahead), then to LDS
    // XOR-swizzled by row so the fragment reads are conflict-free (commit)
    u32x4 pre[NPRE];
    float bpre = 0.f;
    auto fetch = [&](int c0, int nterms) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < NPRE; ++j) {
            const int p = tid + j * NT;
            const int kk = p / PIECES1, h = (p / (16 * NB)) % G, rr = (p / NB) % 16, cb = p % NB;
            const int c = c0 + rr;
            pre[j] = u32x4{0u, 0u, 0u, 0u};
            if (kk < nterms && h < GLM && c < n)
                pre[j] = *(const u32x4 *)(ks + kk * kterm + ((lm0 + h) * C + c) * D + cb * 8);
        }
        if (tid < G * 16) {
            const int h = tid / 16, rr = tid % 16, c = c0 + rr;
            bpre = (h < GLM && c < n) ? b_sum[(lm0 + h) * C + c] : 0.f;
        }
    };
    auto commit = [&](int nterms) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < NPRE; ++j) {
            const int p = tid + j * NT;
            const int kk = p / PIECES1, h = (p / (16 * NB)) % G, rr = (p / NB) % 16, cb = p % NB;
            if (kk < nterms && h < GLM) kt[kk][h][rr][cb ^ (rr & 7)] = pre[j];
        }
        if (tid < G * 16) bt[tid / 16][tid % 16] = bpre;
    };
    // raw s^ of head e for the lane's 4 candidates of rows u, from the term
    // pairs (tq, tk) with tq + tk <= LV among the available ones
    auto scores = [&](auto nkt_c, auto nqt_c, auto lv_c, f32x4 (&val)[2]) __attribute__((always_inline)) {
        constexpr int MK = decltype(nkt_c)::value, MQ = decltype(nqt_c)::value, LV = decltype(lv_c)::value;
        f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const int blk = (4 * s + grp) ^ (cr & 7);
            bf16x8 ak[MK];
#pragma unroll
            for (int kk = 0; kk < MK; ++kk) {
                const u32x4 raw = kt[kk][el][cr][blk];
                __builtin_memcpy(&ak[kk], &raw, 16);
            }
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int tq = 0; tq < MQ; ++tq)
#pragma unroll
                    for (int tk = 0; tk < MK; ++tk)
                        if (tq + tk <= LV) acc[u] = mfma16(ak[tk], qf[u][tq][s], acc[u]);
        }
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int i = 0; i < 4; ++i) val[u][i] = fmaf(scale, acc[u][i], bt[el][4 * grp + i]);
    };

    // ---- pass 1: threshold
    if (rank) {
        float top[SPW][2][T];
#pragma unroll
        for (int j = 0; j < SPW; ++j)
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int t = 0; t < T; ++t) top[j][u][t] = -INFINITY;
        constexpr int NK1 = NKT < 2 ? NKT : 2, NQ1 = NQT < 2 ? NQT : 2;  // pass-1 terms
        fetch(0, NK1);
        for (int c0 = 0; c0 < n; c0 += 16) {
            __syncthreads();  // the previous tile's reads of kt and px are done
            commit(NK1);
            if (c0 + 16 < n) fetch(c0 + 16, NK1);
            __syncthreads();
            f32x4 val[2];
            scores(std::integral_constant<int, NK1>{}, std::integral_constant<int, NQ1>{},
                   std::integral_constant<int, 1>{}, val);
#pragma unroll
            for (int u = 0; u < 2; ++u) px[e][qp][u][lane] = val[u];
            __syncthreads();
            // wave e keeps the streams of accumulator slots e, e + G, ...
#pragma unroll
            for (int j = 0; j < SPW; ++j) {
                const int i = e + G * j;
                if (i >= 4) continue;
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    float gv = -INFINITY;
#pragma unroll
                    for (int h = 0; h < G; ++h) gv = fmaxf(gv, px[h][qp][u][lane][i] - lsev[u][h]);
                    if (c0 + 4 * grp + i >= n_row) gv = -INFINITY;
#pragma unroll
                    for (int t = 0; t < T; ++t) {
                        const float hi = fmaxf(top[j][u][t], gv);
                        gv = fminf(top[j][u][t], gv);
                        top[j][u][t] = hi;
                    }
                }
            }
        }
        // the streams meet in LDS; the K-th largest of each row's 16 T values
#pragma unroll
        for (int j = 0; j < SPW; ++j) {
            const int i = e + G * j;
            if (i >= 4) continue;
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int t = 0; t < T; ++t)
                    gat[((qp * 32 + u * 16 + cr) * 16 + grp * 4 + i) * T + t] = top[j][u][t];
        }
        __syncthreads();
        for (int r = wave; r < ROWS; r += NW) {
            if ((q0 + i0 + r) / S - w <= K) continue;  // all of this row's candidates are kept
            uint32_t kv[NVG];
#pragma unroll
            for (int v = 0; v < NVG; ++v) {
                const int x = lane + WAVE * v;
                kv[v] = x < 16 * T ? ord_key(gat[r * 16 * T + x]) : 0u;
            }
            const float tau = ord_key_inv(kth_largest32<NVG>(kv, K));
            if (lane == 0) thr[r] = tau - rowE[r];
        }
        __syncthreads();  // thresholds are in; the stream values are no longer read
    }

    // ---- pass 2: list the chunks that can be in the top K.  The list of
    // rows (qp, u) is kept by wave (qp, u % G); its length is held in the
    // row's four lanes.
    __syncthreads();  // thr and rcnt are initialised
    int cnt[2] = {0, 0};
    float th[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) th[u] = thr[qp * 32 + u * 16 + cr];
    // cut row r's list (length m) to its exact top K, keeping the order;
    // returns the K-th largest score
    auto cut = [&](int r, int64_t rowg, bool rvalid, int m) __attribute__((always_inline)) -> float {
        uint64_t keys[NV];
        int ids[NV];
        float kv[NV], hh[NV][G];
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const int slot = lane + WAVE * v;
            const bool ok = slot < m;
            ids[v] = ok ? lidx[r * CAP + slot] : 0;
            kv[v] = ok ? lkey[r * CAP + slot] : 0.f;
            keys[v] = ok ? topk_key(kv[v], ids[v]) : 0ull;
#pragma unroll
            for (int h = 0; h < G; ++h) hh[v][h] = (ok && rvalid) ? heads[(rowg * CAP + slot) * G + h] : 0.f;
        }
        const uint64_t kth = kth_largest64<NV>(keys, K);
        wave_sync();
        int base = 0;
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const bool keep = keys[v] >= kth && keys[v] != 0ull;
            const uint64_t mk = __ballot(keep);
            const int pos = base + __popcll(mk & lanemask_lt());
            if (keep) {
                lidx[r * CAP + pos] = ids[v];
                lkey[r * CAP + pos] = kv[v];
                if (rvalid) {
#pragma unroll
                    for (int h = 0; h < G; ++h) heads[(rowg * CAP + pos) * G + h] = hh[v][h];
                }
            }
            base += __popcll(mk);
        }
        wave_sync();
        return ord_key_inv((uint32_t)(kth >> 32));
    };
    fetch(0, NKT);
    for (int c0 = 0; c0 < n; c0 += 16) {
        __syncthreads();
        commit(NKT);
        if (c0 + 16 < n) fetch(c0 + 16, NKT);
        __syncthreads();
        f32x4 val[2];
        scores(std::integral_constant<int, NKT>{}, std::integral_constant<int, NQT>{},
               std::integral_constant<int, 2>{}, val);
#pragma unroll
        for (int u = 0; u < 2; ++u) px[e][qp][u][lane] = val[u];
        __syncthreads();
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            if (e != u % G) continue;
            const int row = qp * 32 + u * 16 + cr;
            const int64_t rowg = bg * N + iq[u];
            float hs[G][4], key[4];
            bool sv[4];
            int k = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                key[i] = -INFINITY;
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    hs[h][i] = px[h][qp][u][lane][i];
                    key[i] = fmaxf(key[i], hs[h][i] - lsev[u][h]);
                }
                sv[i] = c0 + 4 * grp + i < n_row && key[i] >= th[u];
                k += sv[i];
            }
            int kv4[4];
            row_lanes4(k, kv4);
            const int total = kv4[0] + kv4[1] + kv4[2] + kv4[3];
            int before = 0;
#pragma unroll
            for (int j = 0; j < 3; ++j) before += j < grp ? kv4[j] : 0;
            // a row about to overflow is cut to its top K first
            uint64_t om = __ballot(grp == 0 && cnt[u] + total > CAP);
            while (om) {
                const int r16 = __builtin_ffsll((long long)om) - 1;
                om &= om - 1;
                const int m = __builtin_amdgcn_readlane(cnt[u], r16);
                const bool rv = __builtin_amdgcn_readlane((int)qvalid[u], r16) != 0;
                const int64_t rg = bg * N + (i0 + qp * 32 + u * 16 + r16);
                const float kth = cut(qp * 32 + u * 16 + r16, rg, rv, m);
                if (cr == r16) {
                    cnt[u] = K;
                    th[u] = fmaxf(th[u], kth);
                }
            }
            int pos = cnt[u] + before;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (!sv[i]) continue;
                lidx[row * CAP + pos] = c0 + 4 * grp + i;
                lkey[row * CAP + pos] = key[i];
                if (qvalid[u]) {
#pragma unroll
                    for (int h = 0; h < G; ++h) heads[(rowg * CAP + pos) * G + h] = hs[h][i];
                }
                ++pos;
            }
            cnt[u] += total;
        }
    }
#pragma unroll
    for (int u = 0; u < 2; ++u)
        if (e == u % G && grp == 0) rcnt[qp * 32 + u * 16 + cr] = cnt[u];
    __syncthreads();

    // ---- emit: the exact top K of each list, ascending
    for (int r = wave; r < ROWS; r += NW) {
        const int iqr = i0 + r;
        if (iqr >= N) continue;
        const int m = rcnt[r];
        const int64_t rowg = bg * N + iqr;
        uint64_t keys[NV];
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const int slot = lane + WAVE * v;
            keys[v] = slot < m ? topk_key(lkey[r * CAP + slot], lidx[r * CAP + slot]) : 0ull;
        }
        const uint64_t kth = m > K ? kth_largest64<NV>(keys, K) : 1ull;
        int base = 0;
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const int slot = lane + WAVE * v;
            const bool win = keys[v] >= kth && keys[v] != 0ull;
            const uint64_t mk = __ballot(win);
            const int pos = base + __popcll(mk & lanemask_lt());
            if (win) {
                sel_idx[rowg * K + pos] = lidx[r * CAP + slot];
#pragma unroll
                for (int h = 0; h < G; ++h)
                    sel_score[((hq0 + h) * N + iqr) * K + pos] = heads[(rowg * CAP + slot) * G + h];
            }
            base += __popcll(mk);
        }
        for (int kk = base + lane; kk < K; kk += WAVE) {
            sel_idx[rowg * K + kk] = -1;
#pragma unroll
            for (int h = 0; h < G; ++h) sel_score[((hq0 + h) * N + iqr) * K + kk] = -INFINITY;
        }
    }
}

// ---------------------------------------------------------------- launch

namespace {

int topk_class(int K) { return K <= 32 ? 32 : (K <= 64 ? 64 : 128); }

template <int D, int G, int NKT>
size_t topk_lds(int kc) {
    switch (kc) {
        case 32: return TopkPlan<D, G, NKT, 32>::lds_bytes;
        case 64: return TopkPlan<D, G, NKT, 64>::lds_bytes;
        default: return TopkPlan<D, G, NKT, 128>::lds_bytes;
    }
}

template <int D, int G>
size_t topk_lds_g(const Shape &s) {
    return s.sum_bf16 ? topk_lds<D, G, 1>(topk_class(s.K)) : topk_lds<D, G, 3>(topk_class(s.K));
}

}  // namespace

int score_topk_capacity(const Shape &s) { return topk_class(s.K) + 16; }

bool score_topk_supported(const Shape &s) {
    if (s.K <= 0 || s.K > 128) return false;
    size_t lds = 0;
#define HILS_TKL(DD, GG) \
    if (s.D == DD && s.G == GG) lds = topk_lds_g<DD, GG>(s);
    HILS_TKL(64, 1) HILS_TKL(64, 2) HILS_TKL(64, 4) HILS_TKL(64, 8)
    HILS_TKL(128, 1) HILS_TKL(128, 2) HILS_TKL(128, 4) HILS_TKL(128, 8)
#undef HILS_TKL
    return lds > 0 && lds <= 160 * 1024;
}

template <typename TQ, int D, int G, int NKT, int KC>
static void go_topk_k(const Shape &s, const TQ *qv, const ScoreWorkspace &ws, const float *b_sum, float kappa,
                      int32_t *sel_idx, float *sel_score, hipStream_t st) {
    using P = TopkPlan<D, G, NKT, KC>;
    // (instantiations whose LDS does not fit are never launched:
    // score_topk_supported sends those shapes to the two-kernel path)
    if constexpr (P::lds_bytes <= 160 * 1024) {
        const dim3 grid((unsigned)((s.N + P::ROWS - 1) / P::ROWS), (unsigned)s.H_kv, (unsigned)s.B), block(P::NT);
        // the split terms lie one after another, kterm elements apart
        const int64_t kterm = (int64_t)s.B * s.H_lm * s.C * s.D;
        hipLaunchKernelGGL((score_topk_kernel<TQ, D, G, NKT, KC>), grid, block, 0, st, qv, (const bf16 *)ws.ksb, kterm,
                           b_sum, ws.knorm, ws.lse, ws.heads, sel_idx, sel_score, s.N, s.H_q, s.H_kv, s.H_lm, s.C,
                           s.S, s.W, s.K, s.scale, kappa, s.q0);
    }
}

template <typename TQ, int D, int G, int NKT>
static hipError_t go_topk(const Shape &s, const TQ *qv, const ScoreWorkspace &ws, const float *b_sum, float kappa,
                          int32_t *sel_idx, float *sel_score, hipStream_t st) {
    switch (topk_class(s.K)) {
        case 32: go_topk_k<TQ, D, G, NKT, 32>(s, qv, ws, b_sum, kappa, sel_idx, sel_score, st); break;
        case 64: go_topk_k<TQ, D, G, NKT, 64>(s, qv, ws, b_sum, kappa, sel_idx, sel_score, st); break;
        default: go_topk_k<TQ, D, G, NKT, 128>(s, qv, ws, b_sum, kappa, sel_idx, sel_score, st); break;
    }
    return hipGetLastError();
}

template <typename TQ>
static hipError_t dispatch_topk(const Shape &s, const TQ *qv, const ScoreWorkspace &ws, const float *b_sum,
                                float kappa, int32_t *sel_idx, float *sel_score, hipStream_t st) {
#define HILS_TK(DD, GG)                                                                               \
    if (s.D == DD && s.G == GG)                                                                       \
        return s.sum_bf16 ? go_topk<TQ, DD, GG, 1>(s, qv, ws, b_sum, kappa, sel_idx, sel_score, st)   \
                          : go_topk<TQ, DD, GG, 3>(s, qv, ws, b_sum, kappa, sel_idx, sel_score, st);
    HILS_TK(64, 1) HILS_TK(64, 2) HILS_TK(64, 4) HILS_TK(64, 8)
    HILS_TK(128, 1) HILS_TK(128, 2) HILS_TK(128, 4) HILS_TK(128, 8)
#undef HILS_TK
    return hipErrorInvalidValue;
}

hipError_t launch_score_topk(const Shape &s, const void *qv, bool q_fp32, const ScoreWorkspace &ws,
                             const float *b_sum, int32_t *sel_idx, float *sel_score, hipStream_t st) {
    // kappa relative to ||q_s|| ||k'||.  Pass 1: fp32 accumulation of at
    // most 3 d exact products (bounded by 2^-14) plus 2^-16 (1 + 2^-7) for
    // each two-term split operand (an fp32 query, fp32 summaries) and for the
    // dropped t2 k2 term.  Pass 2: fp32 accumulation of at most 6 d exact
    // products (2^-14 bounds gamma_768 with room to spare) plus 2^-22 for the
    // split terms left out.
    const int nq = q_fp32 ? 1 : 0, nk = s.sum_bf16 ? 0 : 1;
    const float kappa1 = 1.f / 16384.f + (float)(nq + nk + nq * nk) * (1.f + 1.f / 128.f) / 65536.f;
    const float kappa2 = 1.f / 16384.f + 1.f / 4194304.f;
    const float kappa = kappa1 + kappa2;
    if (q_fp32) return dispatch_topk<float>(s, (const float *)qv, ws, b_sum, kappa, sel_idx, sel_score, st);
    return dispatch_topk<bf16>(s, (const bf16 *)qv, ws, b_sum, kappa, sel_idx, sel_score, st);
}

}  // namespace hils
