// summary.hip -- kernel 1: landmark summaries (k'_c, b'_c).
//
// hyper.ai HiLS summary, section 方法: the landmark query q'_c of chunk c
// induces a distribution p over the chunk's keys; the compressed key is the
// p-weighted key sum and the bias is the entropy of p.  The logit scale of
// that softmax is the attention scale (the reading under which the score is
// the first-order Taylor expansion of the chunk log-mass at q'_c).
//
// HBM-bound: every key is read exactly once.  One wavefront owns one
// (batch, kv head, chunk) and produces the summaries of all landmark heads
// that read that kv head, so the S x d key tile is loaded once into
// registers with 16-byte loads and reused GLM times.  Reductions over the
// chunk's keys are butterfly shuffles inside the wavefront; no LDS.
#include <type_traits>

#include "hils_device.hpp"
#include "hils_internal.hpp"

namespace hils {


template <typename T, typename TS, int D, int S, int GLM>
__global__ __launch_bounds__(256) void landmark_summary_kernel(const T *__restrict__ k, const T *__restrict__ q_lm,
                                                               TS *__restrict__ k_sum, float *__restrict__ b_sum,
                                                               int H_kv, int N, int C, float scale,
                                                               int64_t total_units, const int32_t *__restrict__ pages,
                                                               int num_pages, int lm_mode) {
    constexpr int E = 16 / sizeof(T);  // elements per 16-byte load
    constexpr int LPR = D / E;         // lanes covering one key row
    constexpr int RPL = WAVE / LPR;    // key rows per wave-wide load
    constexpr int NL = S / RPL;        // loads per lane for the whole chunk
    static_assert(WAVE % LPR == 0 && S % RPL == 0, "tile shape");

    const int lane = lane_id();
    const int64_t unit = (int64_t)blockIdx.x * (blockDim.x / WAVE) + threadIdx.x / WAVE;
    if (unit >= total_units) return;
    const int c = (int)(unit % C);
    const int64_t bg = unit / C;  // b * H_kv + g
    const int g = (int)(bg % H_kv);
    const int64_t b = bg / H_kv;
    // paged: item b summarises page pb (keys and summary row); else pb = b
    const int64_t pb = pages ? (int64_t)pages[b] : b;
    if (pb < 0 || (pages && pb >= num_pages)) return;
    const int col = lane % LPR;
    const int rsub = lane / LPR;

    const T *kb = k + ((pb * H_kv + g) * N + (int64_t)c * S) * D;
    Vec16<T> kr[NL];
#pragma unroll
    for (int t = 0; t < NL; ++t) kr[t] = load16(kb + (int64_t)(t * RPL + rsub) * D + col * E);

    const int H_lm = H_kv * GLM;
    // one landmark head at a time keeps the key tile as the only large
    // register array
#pragma unroll 1
    for (int e = 0; e < GLM; ++e) {
        const int64_t lrow = (b * H_lm + (int64_t)g * GLM + e) * C + c;   // landmark query
        const int64_t orow = (pb * H_lm + (int64_t)g * GLM + e) * C + c;  // summary
        // landmark query: per chunk, shared by all chunks of head l, or zero
        Vec16<T> qv;
        if (lm_mode == 2) qv = Vec16<T>{};
        else qv = load16(q_lm + (lm_mode == 1 ? (int64_t)g * GLM + e : lrow) * D + col * E);
        float a[NL];
        float m = -INFINITY;
#pragma unroll
        for (int t = 0; t < NL; ++t) {
            float part = 0.f;
#pragma unroll
            for (int x = 0; x < E; ++x) part = fmaf(qv.get(x), kr[t].get(x), part);
            a[t] = xor_sum<1, LPR / 2>(part) * scale;
            m = fmaxf(m, a[t]);
        }
        m = xor_max<LPR, WAVE / 2>(m);
        float z = 0.f;
#pragma unroll
        for (int t = 0; t < NL; ++t) {
            a[t] -= m;  // shifted logits
            z += expf(a[t]);
        }
        z = xor_sum<LPR, WAVE / 2>(z);
        const float inv_z = 1.f / z;
        const float log_z = logf(z);
        // entropy: -sum p log p with log p = (a - m) - log Z
        float ent = 0.f;
        float acc[E];
#pragma unroll
        for (int x = 0; x < E; ++x) acc[x] = 0.f;
#pragma unroll
        for (int t = 0; t < NL; ++t) {
            const float p = expf(a[t]) * inv_z;
            ent = fmaf(p, log_z - a[t], ent);
#pragma unroll
            for (int x = 0; x < E; ++x) acc[x] = fmaf(p, kr[t].get(x), acc[x]);
        }
        ent = xor_sum<LPR, WAVE / 2>(ent);
#pragma unroll
        for (int x = 0; x < E; ++x) acc[x] = xor_sum<LPR, WAVE / 2>(acc[x]);
        if (rsub == 0) {
            TS *dst = k_sum + orow * D + col * E;
#pragma unroll
            for (int x = 0; x < E; ++x) dst[x] = from_f32<TS>(acc[x]);
            if (col == 0) b_sum[orow] = ent;
        }
    }
}

// Fast path for bf16 keys at d = 128 (16 lanes per key row).  A chunk's keys
// go in blocks of 64 rows, one block per wave (S / 64 waves per chunk, in
// one workgroup of 4 waves), loaded once: lane (col, rsub) holds rows
// 4t + rsub of its block, t < 16, as packed bf16.  Per landmark head, the
// partial dots (packed bf16 dot2 instructions, fp32 accumulation) are
// transpose-reduced over the 16 lanes of the DPP row, after which the lane
// holds the logit of block row 4*col + rsub (base-2 scaled).  The waves of a
// 128-key chunk combine their softmax statistics (max, mass, mass-weighted
// logit) through LDS.  p goes through LDS, transposed per rsub, to every
// lane of its wave for the weighted key sum; the second wave's partial k'
// is added by the first, which writes the summary.
template <typename TS, int S, int GLM>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void landmark_summary_d128_kernel(
    const bf16 *__restrict__ k, const bf16 *__restrict__ q_lm, TS *__restrict__ k_sum, float *__restrict__ b_sum,
    int H_kv, int N, int C, float scale, int64_t total_units, const int32_t *__restrict__ pages, int num_pages,
    int lm_mode) {
    constexpr int D = 128, NB = S / 64, CPB = 4 / NB;  // waves per chunk, chunks per workgroup
    static_assert(NB == 1 || NB == 2, "64- or 128-key chunks");
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    __shared__ float p_lds[4][4][16];  // [wave][rsub][t]: p of block row 4t + rsub
    __shared__ float stat[4][4];       // [wave]: max, mass, mass-weighted logit (base 2)
    __shared__ float part[4][D];       // [wave]: partial k' of a chunk's second block
    const int lane = lane_id(), wv = threadIdx.x / WAVE, half = wv % NB;
    const int64_t unit = (int64_t)blockIdx.x * CPB + wv / NB;
    bool live = unit < total_units;
    const int c = live ? (int)(unit % C) : 0;
    const int64_t bg = live ? unit / C : 0;  // b * H_kv + g
    const int g = (int)(bg % H_kv);
    const int64_t b = bg / H_kv;
    // paged: item b summarises page pb (keys and summary row); else pb = b
    const int64_t pb = (pages && live) ? (int64_t)pages[b] : b;
    live = live && pb >= 0 && !(pages && pb >= num_pages);
    // a dead wave of a 128-key chunk still takes part in the barriers
    if (NB == 1 && !live) return;
    const int col = lane & 15, rsub = lane >> 4;
    float(*pw)[16] = p_lds[wv];
    const bf16 *kb = k + ((pb * H_kv + g) * N + (int64_t)c * S + 64 * half) * D + col * 8;
    const float sl2 = scale * LOG2E;
    const int H_lm = H_kv * GLM;

    u32x4 kx[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) kx[t] = u32x4{0u, 0u, 0u, 0u};
    if (live) {
#pragma unroll
        for (int t = 0; t < 16; ++t) kx[t] = *(const u32x4 *)(kb + (t * 4 + rsub) * D);
    }
#pragma unroll 1
    for (int e = 0; e < GLM; ++e) {
        const int64_t lrow = (b * H_lm + (int64_t)g * GLM + e) * C + c;   // landmark query
        const int64_t orow = (pb * H_lm + (int64_t)g * GLM + e) * C + c;  // summary
        // landmark query: per chunk, shared by all chunks of head l, or zero
        u32x4 qr = u32x4{0u, 0u, 0u, 0u};
        if (live && lm_mode != 2)
            qr = *(const u32x4 *)(q_lm + (lm_mode == 1 ? (int64_t)g * GLM + e : lrow) * D + col * 8);
        float prt[16];
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
            prt[t] = acc;
        }
        const float lg = transpose_sum16(prt, col) * sl2;
        float m = wave_max_f(lg);
        float ex = exp2f(lg - m);
        float z = wave_sum_f(ex);
        float ez = wave_sum_f(ex * (lg - m));
        if constexpr (NB == 2) {
            // both waves combine the two blocks' statistics in the same order
            if (lane == 0) {
                stat[wv][0] = m;
                stat[wv][1] = z;
                stat[wv][2] = ez;
            }
            __syncthreads();
            const int w0 = wv & ~1;
            const float m0 = stat[w0][0], z0 = stat[w0][1], ez0 = stat[w0][2];
            const float m1 = stat[w0 + 1][0], z1 = stat[w0 + 1][1], ez1 = stat[w0 + 1][2];
            const float mn = fmaxf(m0, m1);
            const float a0 = exp2f(m0 - mn), a1 = exp2f(m1 - mn);
            // sum_j 2^(lg_j - mn) (lg_j - mn) = a (ez + (m - mn) z) per block
            ez = a0 * fmaf(m0 - mn, z0, ez0) + a1 * fmaf(m1 - mn, z1, ez1);
            z = a0 * z0 + a1 * z1;
            ex *= half ? a1 : a0;
        }
        const float inv_z = 1.f / z;
        // entropy = ln 2 * (log2 Z - sum_j p_j (a2_j - m)), a2 = base-2 logits
        const float ent = LN2 * (log2f(z) - ez * inv_z);
        wave_sync();
        pw[rsub][col] = ex * inv_z;
        wave_sync();
        float acc[8];
#pragma unroll
        for (int x = 0; x < 8; ++x) acc[x] = 0.f;
        // widen inside the head loop: an opaque shift and mask keep the
        // compiler from hoisting 128 widened values out of it (without
        // copying the keys)
        uint32_t sh = 16, mk = 0xffff0000u;
        asm volatile("" : "+v"(sh), "+v"(mk));
#pragma unroll
        for (int t0 = 0; t0 < 16; t0 += 4) {
            const f32x4 p4 = *(const f32x4 *)&pw[rsub][t0];
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    const uint32_t w = kx[t0 + u][x];
                    acc[2 * x] = fmaf(p4[u], __uint_as_float(w << sh), acc[2 * x]);
                    acc[2 * x + 1] = fmaf(p4[u], __uint_as_float(w & mk), acc[2 * x + 1]);
                }
        }
#pragma unroll
        for (int x = 0; x < 8; ++x) acc[x] = rows4_sum(acc[x]);
        if constexpr (NB == 2) {
            if (half == 1 && rsub == 0) {
#pragma unroll
                for (int x = 0; x < 8; ++x) part[wv][col * 8 + x] = acc[x];
            }
            __syncthreads();
            if (half == 0) {
#pragma unroll
                for (int x = 0; x < 8; ++x) acc[x] += part[wv + 1][col * 8 + x];
            }
        }
        if (live && half == 0 && rsub == 0) {
            TS *dst = k_sum + orow * D + col * 8;
#pragma unroll
            for (int x = 0; x < 8; ++x) dst[x] = from_f32<TS>(acc[x]);
            if (col == 0) b_sum[orow] = ent;
        }
    }
}

template <typename T, typename TS, int D, int S>
static hipError_t launch_s(const Shape &s, const void *k, const void *q_lm, void *k_sum, float *b_sum,
                           const int32_t *pages, int num_pages, hipStream_t st) {
    const int64_t units = (int64_t)s.B * s.H_kv * s.C;
    if (units == 0) return hipSuccess;
    // four waves per workgroup: one chunk each, or, on the bf16 d = 128 path,
    // S / 64 waves per chunk
    const int cpb = (std::is_same<T, bf16>::value && D == 128) ? 4 / (S / 64) : 4;
    const dim3 grid((unsigned)((units + cpb - 1) / cpb)), block(256);
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, grid, block, 0, st, (const T *)k, (const T *)q_lm, (TS *)k_sum, b_sum, s.H_kv, s.N,
                           s.C, s.scale, units, pages, num_pages, s.lm_mode);
    };
    if constexpr (std::is_same<T, bf16>::value && D == 128) {
        switch (s.GLM) {
            case 1: go(landmark_summary_d128_kernel<TS, S, 1>); break;
            case 2: go(landmark_summary_d128_kernel<TS, S, 2>); break;
            case 4: go(landmark_summary_d128_kernel<TS, S, 4>); break;
            case 8: go(landmark_summary_d128_kernel<TS, S, 8>); break;
            default: return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
    switch (s.GLM) {
        case 1: go(landmark_summary_kernel<T, TS, D, S, 1>); break;
        case 2: go(landmark_summary_kernel<T, TS, D, S, 2>); break;
        case 4: go(landmark_summary_kernel<T, TS, D, S, 4>); break;
        case 8: go(landmark_summary_kernel<T, TS, D, S, 8>); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename T, typename TS>
static hipError_t launch_t(const Shape &s, const void *k, const void *q_lm, void *k_sum, float *b_sum,
                           const int32_t *pages, int num_pages, hipStream_t st) {
    if (s.D == 64 && s.S == 64) return launch_s<T, TS, 64, 64>(s, k, q_lm, k_sum, b_sum, pages, num_pages, st);
    if (s.D == 64 && s.S == 128) return launch_s<T, TS, 64, 128>(s, k, q_lm, k_sum, b_sum, pages, num_pages, st);
    if (s.D == 128 && s.S == 64) return launch_s<T, TS, 128, 64>(s, k, q_lm, k_sum, b_sum, pages, num_pages, st);
    if (s.D == 128 && s.S == 128) return launch_s<T, TS, 128, 128>(s, k, q_lm, k_sum, b_sum, pages, num_pages, st);
    return hipErrorInvalidValue;
}

hipError_t launch_landmark_summary(const Shape &s, const void *k, const void *q_lm, void *k_sum, float *b_sum,
                                   const int32_t *pages, int num_pages, hipStream_t st) {
    if (s.io_bf16)
        return s.sum_bf16 ? launch_t<bf16, bf16>(s, k, q_lm, k_sum, b_sum, pages, num_pages, st)
                          : launch_t<bf16, float>(s, k, q_lm, k_sum, b_sum, pages, num_pages, st);
    return s.sum_bf16 ? launch_t<float, bf16>(s, k, q_lm, k_sum, b_sum, pages, num_pages, st)
                      : launch_t<float, float>(s, k, q_lm, k_sum, b_sum, pages, num_pages, st);
}

}  // namespace hils
