// attend.hip -- kernel 3: fused sparse attention (selected chunks + window).
//
// hyper.ai HiLS summary, section 方法: each query attends exactly inside each
// selected chunk (intra-chunk softmax) and inside a chunk-aligned causal
// window; the per-chunk outputs are fused with weights exp(s^_c) / Z^ where
// Z^ = sum_c exp(s^_c) + Z_swa (partition estimate and the hierarchical
// factorisation of the attention weight).  Same page, kernel paragraph:
// M adjacent queries x G heads of a GQA group share one pass over the union
// of their selected chunks, so a loaded K/V chunk serves many rows.
//
// MI355X design (bf16 path):
//   * A block owns QB consecutive queries of one query chunk x the G heads
//     of one kv group; 16-row MFMA tiles hold 16/G queries x G heads, each
//     wave owns TPW tiles.  Every query of the block shares the candidate
//     set and the window, so one staged K/V chunk tile in LDS serves all
//     tiles that need it.
//   * The block builds the ascending union of its queries' selections
//     (bitmap + prefix scan in LDS) and walks it; each row keeps a cursor
//     into its own ascending selection list, so a row only takes the chunks
//     it selected (the union is a schedule, the result is per query).
//   * Transposed products keep every per-row quantity in lane l%16:
//     S^T = K Q^T (A = K tile from LDS, B = Q^T in registers) and
//     O^T += V^T P^T (A = V^T tile, B = P^T packed straight from the S^T
//     accumulators).  V^T comes from a pre-pass that writes each chunk as
//     [d][key] with keys of every 32-key group stored in the order the S^T
//     accumulator layout delivers them, so P^T needs no cross-lane moves.
//   * Q K^T runs on bf16 operands (exact products of the bf16 inputs).  The
//     probabilities P lie in [0, 1]; they are rounded to fp16 (11-bit
//     significand, 8x finer than bf16) and V^T is stored as fp16 (exact for
//     bf16 values of magnitude below 65504), so V^T P^T runs on fp16 MFMA:
//     bf16 rounding of P alone can miss a 2e-3 absolute bound on rows with
//     few keys whose values cancel.
//   * Selected chunk c of a row: exact softmax over its S keys, scaled by
//     exp(s^_c - m^) where m^ = max of the row's selected s^ (known up
//     front); the accumulator then starts the window's online softmax with
//     running max m^ and running mass sum_c exp(s^_c - m^).  All exps are
//     exp2 with log2(e) folded into the scales.
#include "hils_device.hpp"
#include "hils_internal.hpp"

namespace hils {

// Key held by slot p of a chunk's transposed V rows.  In the S^T
// accumulators of 16-key tiles 2s and 2s+1, lane group gq holds keys
// 32s + 4gq + {0..3} and 32s + 16 + 4gq + {0..3}; those become the eight
// B-operand slots 8gq..8gq+7 of k-step s.
__host__ __device__ __forceinline__ int vt_slot_key(int p) {
    const int s = p >> 5, qd = p & 31, gq = qd >> 3, j = qd & 7;
    return 32 * s + (j < 4 ? 4 * gq + j : 16 + 4 * gq + (j - 4));
}

// vt[b, g, c, d, slot] = fp16(v[b, g, c*S + vt_slot_key(slot), d]) (0 past N).
template <int D, int S>
__global__ __launch_bounds__(256) void v_transpose_kernel(const bf16 *__restrict__ v, f16 *__restrict__ vt, int N,
                                                          int CA, int H_kv) {
    __shared__ bf16 tile[S][D + 8];
    const int c = blockIdx.x;
    const int64_t bg = (int64_t)blockIdx.z * H_kv + blockIdx.y;
    const bf16 *src = v + (bg * N + (int64_t)c * S) * D;
    for (int idx = threadIdx.x; idx < S * (D / 8); idx += blockDim.x) {
        const int j = idx / (D / 8), cb = idx % (D / 8);
        u32x4 val = {0u, 0u, 0u, 0u};
        if (c * S + j < N) val = *(const u32x4 *)(src + (int64_t)j * D + cb * 8);
        bf16x8 x;
        __builtin_memcpy(&x, &val, 16);
#pragma unroll
        for (int e = 0; e < 8; ++e) tile[j][cb * 8 + e] = x[e];
    }
    __syncthreads();
    f16 *dst = vt + (bg * CA + c) * (int64_t)D * S;
    for (int idx = threadIdx.x; idx < D * (S / 8); idx += blockDim.x) {
        const int d = idx / (S / 8), blk = idx % (S / 8);
        f16x8 x;
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = (f16)(float)tile[vt_slot_key(blk * 8 + e)][d];
        *(f16x8 *)(dst + (int64_t)d * S + blk * 8) = x;
    }
}

template <int D, int S, int G, int TPW>
struct AttendCfg {
    static constexpr int QPT = 16 / G;          // queries per 16-row tile
    static constexpr int QB = 4 * TPW * QPT;    // queries per block
    static constexpr int KS = D / 32;           // k-steps of Q K^T
    static constexpr int KT = S / 16;           // 16-key tiles per chunk
    static constexpr int PS = S / 32;           // k-steps of V^T P^T
    static constexpr int DT = D / 16;           // 16-dim tiles of O^T
    static constexpr int NBK = D / 8;           // 16-byte blocks per K row
    static constexpr int NBV = S / 8;           // 16-byte blocks per V^T row
};

// Dynamic LDS layout after the static K/V tiles:
//   int   sel[QB*K]        selections of the block's queries
//   float sc[QB*G*K]       their s^ (log2 units), per head
//   uint  bitmap[NW]       union bitmap over candidate chunks
//   int   ulist[UCAP]      ascending union
//   int   scan[8]          wave totals of the prefix scan
template <int D, int S, int G, int TPW>
__global__ __launch_bounds__(256) void sparse_attend_kernel(
    const bf16 *__restrict__ q, const bf16 *__restrict__ k, const f16 *__restrict__ vt,
    const int32_t *__restrict__ sel_idx, const float *__restrict__ sel_score, bf16 *__restrict__ out,
    float *__restrict__ lse, int N, int H_q, int H_kv, int CA, int W, int K, float scale_log2, int NW, int UCAP) {
    using Cf = AttendCfg<D, S, G, TPW>;
    constexpr int QPT = Cf::QPT, QB = Cf::QB, KS = Cf::KS, KT = Cf::KT, PS = Cf::PS, DT = Cf::DT;
    constexpr int NBK = Cf::NBK, NBV = Cf::NBV;
    __shared__ u32x4 k_lds[S][NBK];
    __shared__ u32x4 v_lds[D][NBV];
    extern __shared__ int dyn[];
    int *sel_l = dyn;
    float *sc_l = (float *)(sel_l + QB * K);
    uint32_t *bitmap = (uint32_t *)(sc_l + QB * G * K);
    int *ulist = (int *)(bitmap + NW);
    int *scan = ulist + UCAP;

    const int g = blockIdx.y;
    const int64_t b = blockIdx.z;
    const int i0 = blockIdx.x * QB;
    const int qc = i0 / S;
    const int n = max(0, qc - W / S);
    const int tid = threadIdx.x, wave = tid / WAVE, lane = lane_id(), grp = lane >> 4;
    const int64_t bg = b * H_kv + g;

    // ---- selections of the block's queries
    for (int t = tid; t < QB * K; t += blockDim.x) {
        const int m = t / K, kk = t % K, iq = i0 + m;
        sel_l[t] = iq < N ? sel_idx[(bg * N + iq) * K + kk] : -1;
    }
    for (int t = tid; t < QB * G * K; t += blockDim.x) {
        const int m = t / (G * K), rem = t % (G * K), e = rem / K, kk = rem % K, iq = i0 + m;
        sc_l[t] = iq < N ? sel_score[((b * H_q + g * G + e) * N + iq) * K + kk] * LOG2E : -INFINITY;
    }
    for (int t = tid; t < NW; t += blockDim.x) bitmap[t] = 0u;
    __syncthreads();
    for (int t = tid; t < QB * K; t += blockDim.x) {
        const int c = sel_l[t];
        if (c >= 0 && c < n) atomicOr(&bitmap[c >> 5], 1u << (c & 31));
    }
    __syncthreads();
    // ---- ascending union: exclusive prefix sum of per-word popcounts
    int U = 0;
    {
        int base = 0;
        for (int w0 = 0; w0 < NW; w0 += blockDim.x) {
            const int wi = w0 + tid;
            const uint32_t word = wi < NW ? bitmap[wi] : 0u;
            const int cnt = __popc(word);
            int incl = cnt;
#pragma unroll
            for (int o = 1; o < WAVE; o <<= 1) {
                const int y = __shfl_up(incl, o, WAVE);
                if (lane >= o) incl += y;
            }
            if (lane == WAVE - 1) scan[wave] = incl;
            __syncthreads();
            int wbase = 0, tot = 0;
            for (int x = 0; x < 4; ++x) {
                if (x < wave) wbase += scan[x];
                tot += scan[x];
            }
            int pos = base + wbase + incl - cnt;
            uint32_t wv = word;
            while (wv) {
                const int bit = __ffs(wv) - 1;
                wv &= wv - 1;
                if (pos < UCAP) ulist[pos] = wi * 32 + bit;
                ++pos;
            }
            base += tot;
            __syncthreads();
        }
        U = min(base, UCAP);
    }

    // ---- per-tile row state
    const int r = lane & 15;
    bf16x8 qf[TPW][KS];
    f32x4 O[TPW][DT];
    float mrun[TPW], lrun[TPW];
    int cur[TPW], nsel[TPW], qrow[TPW], hrow[TPW];
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
        const int m = (wave * TPW + t) * QPT + r / G;
        const int e = r % G;
        const int iq = i0 + m;
        qrow[t] = m;
        hrow[t] = g * G + e;
        const bf16 *qr = q + ((b * H_q + hrow[t]) * N + min(iq, N - 1)) * D;
#pragma unroll
        for (int s = 0; s < KS; ++s) qf[t][s] = *(const bf16x8 *)(qr + 32 * s + 8 * grp);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) O[t][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
        float mh = -INFINITY;
        int ns = 0;
        for (int kk = 0; kk < K; ++kk) {
            const int c = sel_l[m * K + kk];
            if (c >= 0) {
                ++ns;
                mh = fmaxf(mh, sc_l[(m * G + e) * K + kk]);
            }
        }
        float z = 0.f;
        for (int kk = 0; kk < ns; ++kk) z += exp2f(sc_l[(m * G + e) * K + kk] - mh);
        mrun[t] = mh;
        lrun[t] = z;
        cur[t] = 0;
        nsel[t] = ns;
    }

    const bf16 *kbase = k + bg * (int64_t)N * D;
    const f16 *vtbase = vt + bg * (int64_t)CA * D * S;

    auto stage = [&](int c) {
        __syncthreads();
        const bf16 *ks = kbase + (int64_t)c * S * D;
        for (int idx = tid; idx < S * NBK; idx += blockDim.x) {
            const int row = idx / NBK, cb = idx % NBK;
            u32x4 val = {0u, 0u, 0u, 0u};
            if ((int64_t)c * S + row < N) val = *(const u32x4 *)(ks + (int64_t)row * D + cb * 8);
            k_lds[row][cb ^ (row & 7)] = val;
        }
        const f16 *vs = vtbase + (int64_t)c * D * S;
        for (int idx = tid; idx < D * NBV; idx += blockDim.x) {
            const int row = idx / NBV, cb = idx % NBV;
            v_lds[row][cb ^ (row & 7)] = *(const u32x4 *)(vs + (int64_t)row * S + cb * 8);
        }
        __syncthreads();
    };

    // S^T tile of one 16-row MFMA tile: acc[kt][i] = q_row . k_{16kt + 4grp + i}
    auto qk = [&](const bf16x8 (&qt)[KS], f32x4 (&acc)[KT]) {
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
            acc[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
            const int row = 16 * kt + r;
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                const u32x4 raw = k_lds[row][(4 * s + grp) ^ (row & 7)];
                bf16x8 a;
                __builtin_memcpy(&a, &raw, 16);
                acc[kt] = mfma16(a, qt[s], acc[kt]);
            }
        }
    };
    // O^T += V^T P^T with P^T taken from the (already exponentiated) S^T
    auto pv = [&](const f32x4 (&p)[KT], f32x4 (&o)[DT]) {
#pragma unroll
        for (int ps = 0; ps < PS; ++ps) {
            f16x8 bp;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                bp[i] = (f16)p[2 * ps][i];
                bp[4 + i] = (f16)p[2 * ps + 1][i];
            }
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const int row = 16 * dt + r;
                const u32x4 raw = v_lds[row][(4 * ps + grp) ^ (row & 7)];
                f16x8 a;
                __builtin_memcpy(&a, &raw, 16);
                o[dt] = mfma16h(a, bp, o[dt]);
            }
        }
    };

    // ---- selected chunks (union walk)
    for (int u = 0; u < U; ++u) {
        const int c = ulist[u];
        stage(c);
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
            const int m = qrow[t], e = hrow[t] - g * G;
            const bool active = cur[t] < nsel[t] && sel_l[m * K + cur[t]] == c;
            if (__ballot(active) == 0ull) continue;
            f32x4 acc[KT];
            qk(qf[t], acc);
            float cmax = -INFINITY;
#pragma unroll
            for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    acc[kt][i] *= scale_log2;
                    cmax = fmaxf(cmax, acc[kt][i]);
                }
            cmax = xor_max<16, 32>(cmax);
            float lc = 0.f;
#pragma unroll
            for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    acc[kt][i] = exp2f(acc[kt][i] - cmax);
                    lc += acc[kt][i];
                }
            lc = xor_sum<16, 32>(lc);
            const float f = active ? exp2f(sc_l[(m * G + e) * K + cur[t]] - mrun[t]) / lc : 0.f;
#pragma unroll
            for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[kt][i] *= f;
            pv(acc, O[t]);
            cur[t] += active ? 1 : 0;
        }
    }

    // ---- chunk-aligned causal window: online softmax continuing the state
    const int wc0 = max(0, qc - W / S);
    for (int c = wc0; c <= qc; ++c) {
        stage(c);
        const bool diag = c == qc;
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
            const int iq = i0 + qrow[t];
            f32x4 acc[KT];
            qk(qf[t], acc);
            float cmax = -INFINITY;
#pragma unroll
            for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int j = c * S + 16 * kt + 4 * grp + i;
                    const float x = (diag && j > iq) ? -INFINITY : acc[kt][i] * scale_log2;
                    acc[kt][i] = x;
                    cmax = fmaxf(cmax, x);
                }
            cmax = xor_max<16, 32>(cmax);
            const float mnew = fmaxf(mrun[t], cmax);
            const float alpha = exp2f(mrun[t] - mnew);
            float ls = 0.f;
#pragma unroll
            for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    acc[kt][i] = exp2f(acc[kt][i] - mnew);
                    ls += acc[kt][i];
                }
            ls = xor_sum<16, 32>(ls);
            lrun[t] = lrun[t] * alpha + ls;
            mrun[t] = mnew;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) O[t][dt] *= alpha;
            pv(acc, O[t]);
        }
    }

    // ---- epilogue
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
        const int iq = i0 + qrow[t];
        if (iq >= N) continue;
        const float inv = 1.f / lrun[t];
        bf16 *orow = out + ((b * H_q + hrow[t]) * N + iq) * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            bf16x4 y;
#pragma unroll
            for (int i = 0; i < 4; ++i) y[i] = (bf16)(O[t][dt][i] * inv);
            *(bf16x4 *)(orow + 16 * dt + 4 * grp) = y;
        }
        if (lse && grp == 0) lse[(b * H_q + hrow[t]) * N + iq] = (mrun[t] + log2f(lrun[t])) * LN2;
    }
}

// ---------------------------------------------------------------- fp32 path
//
// One wave per (b, query head, query); fp32 throughout (expf / logf), in
// the order of the definition: window part first, then
// L = log(sum_c exp(s^_c) + exp(lse_swa)), then the selected chunks'
// normalised outputs weighted by exp(s^_c - L).
template <int D>
__global__ __launch_bounds__(256) void sparse_attend_f32_kernel(const float *__restrict__ q,
                                                                const float *__restrict__ k,
                                                                const float *__restrict__ v,
                                                                const int32_t *__restrict__ sel_idx,
                                                                const float *__restrict__ sel_score,
                                                                float *__restrict__ out, float *__restrict__ lse,
                                                                int B, int N, int H_q, int H_kv, int S, int W, int K,
                                                                float scale) {
    constexpr int DPL = D / WAVE;  // dims per lane (1 or 2)
    __shared__ float q_l[4][D];
    __shared__ float p_l[4][128];
    const int wave = threadIdx.x / WAVE, lane = lane_id();
    const int64_t row = (int64_t)blockIdx.x * 4 + wave;  // (b*H_q + h)*N + i
    if (row >= (int64_t)B * H_q * N) return;
    const int i = (int)(row % N);
    const int64_t bh = row / N;
    const int h = (int)(bh % H_q);
    const int64_t b = bh / H_q;
    const int G = H_q / H_kv, g = h / G;
    const float *kb = k + (b * H_kv + g) * (int64_t)N * D;
    const float *vb = v + (b * H_kv + g) * (int64_t)N * D;
    for (int x = lane; x < D; x += WAVE) q_l[wave][x] = q[row * D + x];
    wave_sync();

    // exact softmax over keys [j0, j1] (j1 - j0 < 2*WAVE per call) merged
    // into (m, l, o) with online rescaling
    auto attend_block = [&](int j0, int j1, float &m, float &l, float (&o)[DPL]) {
        float lg[2];
        float bm = -INFINITY;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int j = j0 + u * WAVE + lane;
            lg[u] = -INFINITY;
            if (j <= j1) {
                const float *kr = kb + (int64_t)j * D;
                float dot = 0.f;
                for (int x = 0; x < D; ++x) dot = fmaf(q_l[wave][x], kr[x], dot);
                lg[u] = dot * scale;
            }
            bm = fmaxf(bm, lg[u]);
        }
        bm = wave_max(bm);
        const float mn = fmaxf(m, bm);
        const float alpha = expf(m - mn);
        float ls = 0.f;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const float p = (j0 + u * WAVE + lane <= j1) ? expf(lg[u] - mn) : 0.f;
            p_l[wave][u * WAVE + lane] = p;
            ls += p;
        }
        ls = xor_sum<1, 32>(ls);
        wave_sync();
        l = l * alpha + ls;
        m = mn;
#pragma unroll
        for (int y = 0; y < DPL; ++y) {
            float acc = o[y] * alpha;
            const int x = lane + y * WAVE;
            for (int j = j0; j <= j1; ++j) acc = fmaf(p_l[wave][j - j0], vb[(int64_t)j * D + x], acc);
            o[y] = acc;
        }
        wave_sync();
    };

    const int w0 = max(0, (i / S) * S - W);
    float mw = -INFINITY, lw = 0.f, ow[DPL];
#pragma unroll
    for (int y = 0; y < DPL; ++y) ow[y] = 0.f;
    for (int j = w0; j <= i; j += 2 * WAVE) attend_block(j, min(i, j + 2 * WAVE - 1), mw, lw, ow);
    const float lse_sw = mw + logf(lw);

    const int32_t *sl = sel_idx + ((b * H_kv + g) * N + i) * K;
    const float *ss = sel_score + row * K;
    float mx = lse_sw;
    for (int kk = 0; kk < K; ++kk)
        if (sl[kk] >= 0) mx = fmaxf(mx, ss[kk]);
    float z = expf(lse_sw - mx);
    for (int kk = 0; kk < K; ++kk)
        if (sl[kk] >= 0) z += expf(ss[kk] - mx);
    const float L = mx + logf(z);

    float o[DPL];
    const float wsw = expf(lse_sw - L) / lw;
#pragma unroll
    for (int y = 0; y < DPL; ++y) o[y] = wsw * ow[y];
    for (int kk = 0; kk < K; ++kk) {
        const int c = sl[kk];
        if (c < 0) continue;
        float mc = -INFINITY, lc = 0.f, oc[DPL];
#pragma unroll
        for (int y = 0; y < DPL; ++y) oc[y] = 0.f;
        for (int j = c * S; j < c * S + S; j += 2 * WAVE) attend_block(j, min(c * S + S - 1, j + 2 * WAVE - 1), mc, lc, oc);
        const float wc = expf(ss[kk] - L) / lc;
#pragma unroll
        for (int y = 0; y < DPL; ++y) o[y] = fmaf(wc, oc[y], o[y]);
    }
#pragma unroll
    for (int y = 0; y < DPL; ++y) out[row * D + lane + y * WAVE] = o[y];
    if (lse && lane == 0) lse[row] = L;
}

// ---------------------------------------------------------------- launch

size_t fused_workspace_bytes(const Shape &s) {
    if (!s.io_bf16) return 0;
    return align_up((size_t)s.B * s.H_kv * s.CA * s.D * s.S * 2, 256);
}

static int pick_tpw(const Shape &s) {
    // queries per block = 4 * TPW * 16 / G must divide S; two tiles per
    // wave only while the S^T and O^T accumulators fit the register file
    const int qpt = 16 / s.G;
    int tpw = 1;
    if (s.D * s.S > 128 * 64) return 1;
    while (tpw < 2 && 4 * (tpw * 2) * qpt <= s.S && s.S % (4 * tpw * 2 * qpt) == 0) tpw *= 2;
    return tpw;
}

template <int D, int S, int G, int TPW>
static hipError_t go_attend(const Shape &s, const void *q, const void *k, const void *vt, const int32_t *sel_idx,
                            const float *sel_score, void *out, float *lse, hipStream_t st) {
    using Cf = AttendCfg<D, S, G, TPW>;
    const int QB = Cf::QB;
    const int NW = (s.C + 31) / 32 + 1;
    const int UCAP = std::min(s.C + 1, QB * s.K + 1);  // union size bound
    const size_t dyn = (size_t)QB * s.K * 4 + (size_t)QB * G * s.K * 4 + (size_t)NW * 4 + (size_t)UCAP * 4 + 8 * 4;
    const dim3 grid((unsigned)((s.N + QB - 1) / QB), (unsigned)s.H_kv, (unsigned)s.B), block(256);
    auto kern = sparse_attend_kernel<D, S, G, TPW>;
    // static K/V tiles plus this dynamic part may exceed 64 KB at S = 128
    hipError_t e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, grid, block, dyn, st, (const bf16 *)q, (const bf16 *)k, (const f16 *)vt, sel_idx,
                       sel_score, (bf16 *)out, lse, s.N, s.H_q, s.H_kv, s.CA, s.W, s.K, s.scale * LOG2E, NW, UCAP);
    return hipGetLastError();
}

template <int D, int S>
static hipError_t dispatch_g(const Shape &s, const void *q, const void *k, const void *vt, const int32_t *sel_idx,
                             const float *sel_score, void *out, float *lse, hipStream_t st) {
    const int tpw = pick_tpw(s);
#define HILS_ATT(GG, TT)                                                                       \
    if (s.G == GG && tpw == TT) return go_attend<D, S, GG, TT>(s, q, k, vt, sel_idx, sel_score, out, lse, st);
    HILS_ATT(1, 1) HILS_ATT(1, 2) HILS_ATT(2, 1) HILS_ATT(2, 2) HILS_ATT(4, 1) HILS_ATT(4, 2) HILS_ATT(8, 1) HILS_ATT(8, 2)
#undef HILS_ATT
    return hipErrorInvalidValue;
}

hipError_t launch_sparse_attend(const Shape &s, const void *q, const void *k, const void *v, const int32_t *sel_idx,
                                const float *sel_score, void *out, float *lse, void *workspace, hipStream_t st) {
    if ((int64_t)s.B * s.N == 0) return hipSuccess;
    if (!s.io_bf16) {
        const int64_t rows = (int64_t)s.B * s.H_q * s.N;
        const dim3 grid((unsigned)((rows + 3) / 4)), block(256);
        if (s.D == 64)
            hipLaunchKernelGGL(sparse_attend_f32_kernel<64>, grid, block, 0, st, (const float *)q, (const float *)k,
                               (const float *)v, sel_idx, sel_score, (float *)out, lse, s.B, s.N, s.H_q, s.H_kv, s.S,
                               s.W, s.K, s.scale);
        else
            hipLaunchKernelGGL(sparse_attend_f32_kernel<128>, grid, block, 0, st, (const float *)q, (const float *)k,
                               (const float *)v, sel_idx, sel_score, (float *)out, lse, s.B, s.N, s.H_q, s.H_kv, s.S,
                               s.W, s.K, s.scale);
        return hipGetLastError();
    }
    // V^T pre-pass into the workspace (fp16)
    f16 *vt = (f16 *)workspace;
    {
        const dim3 grid((unsigned)s.CA, (unsigned)s.H_kv, (unsigned)s.B), block(256);
        if (s.D == 64 && s.S == 64) hipLaunchKernelGGL((v_transpose_kernel<64, 64>), grid, block, 0, st, (const bf16 *)v, vt, s.N, s.CA, s.H_kv);
        else if (s.D == 64) hipLaunchKernelGGL((v_transpose_kernel<64, 128>), grid, block, 0, st, (const bf16 *)v, vt, s.N, s.CA, s.H_kv);
        else if (s.S == 64) hipLaunchKernelGGL((v_transpose_kernel<128, 64>), grid, block, 0, st, (const bf16 *)v, vt, s.N, s.CA, s.H_kv);
        else hipLaunchKernelGGL((v_transpose_kernel<128, 128>), grid, block, 0, st, (const bf16 *)v, vt, s.N, s.CA, s.H_kv);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (s.D == 64 && s.S == 64) return dispatch_g<64, 64>(s, q, k, vt, sel_idx, sel_score, out, lse, st);
    if (s.D == 64 && s.S == 128) return dispatch_g<64, 128>(s, q, k, vt, sel_idx, sel_score, out, lse, st);
    if (s.D == 128 && s.S == 64) return dispatch_g<128, 64>(s, q, k, vt, sel_idx, sel_score, out, lse, st);
    if (s.D == 128 && s.S == 128) return dispatch_g<128, 128>(s, q, k, vt, sel_idx, sel_score, out, lse, st);
    return hipErrorInvalidValue;
}

}  // namespace hils
