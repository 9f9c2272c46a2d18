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
// that read that kv head, so the S x d key tile is loaded once and reused
// GLM times.  bf16 keys at d = 128 take the matrix-core kernel (the tile in
// LDS, logits and the weighted key sum on MFMA); other shapes keep the tile
// in registers and reduce with butterfly shuffles inside the wavefront.
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

// Matrix-core path for bf16 keys at d = 128.  One wave per (batch, kv
// head, chunk), for all GLM landmark heads of that kv head at once:
//   * the chunk's S x 128 key tile goes global -> LDS by buffer_load ... lds
//     (row-major, 16-byte blocks XOR-swizzled by row & 15, the swizzle
//     applied through the per-lane source offset);
//   * logits A = K Q'^T on bf16 MFMA (exact products, fp32 sums): the A
//     operand is K read row-major, the B operand holds the landmark queries,
//     one per column (columns >= GLM are zero);
//   * the per-head softmax in base 2, reductions across the four 16-lane
//     rows of the accumulator layout;
//   * k'^T = K^T P on bf16 MFMA: the A operand K^T is read from the same
//     tile with the transposing LDS read, in the k-slot order in which two
//     16-key accumulator tiles deliver their keys, so P enters straight from
//     the softmax registers, as three bf16 terms (residual below 2^-26 |p|).
// The waves of a block are independent (each has its own LDS tile; no
// barrier), so one that has no chunk returns at once.
constexpr int SUM_RSRC_WORD3 = 0x00020000;  // raw buffer: 32-bit dwords, no swizzle, no stride

template <typename TS, int S, int GLM>
__global__ __launch_bounds__(S == 64 ? 128 : 64) void landmark_summary_mfma_kernel(
    const bf16 *__restrict__ k, const bf16 *__restrict__ q_lm, TS *__restrict__ k_sum, float *__restrict__ b_sum,
    int H_kv, int N, int C, float scale, int64_t total_units, const int32_t *__restrict__ pages, int num_pages,
    int lm_mode) {
    constexpr int D = 128, NB = D / 8, KT = S / 16, PS = S / 32, DT = D / 16, KS = D / 32;
    constexpr int WPB = S == 64 ? 2 : 1;  // waves per block: 32 KB of key tiles per block
    constexpr int NP = S * D * 2 / 1024;  // 1 KB DMA pieces per chunk, 4 rows each
    static_assert(GLM <= 16, "one landmark head per MFMA column");
    typedef short v4i16 __attribute__((ext_vector_type(4)));
    __shared__ u32x4 tile[WPB][S][NB];
    const int lane = lane_id(), wv = __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE);
    const int64_t unit = (int64_t)blockIdx.x * WPB + wv;
    if (unit >= total_units) return;
    const int c = (int)(unit % C);
    const int64_t bg = unit / C;  // b * H_kv + g
    const int g = (int)(bg % H_kv);
    const int64_t b = bg / H_kv;
    // paged: item b summarises page pb (keys and summary row); else pb = b
    const int64_t pb = pages ? (int64_t)pages[b] : b;
    if (pb < 0 || (pages && pb >= num_pages)) return;
    const int r = lane & 15, grp = lane >> 4;
    u32x4(*kt)[NB] = tile[wv];

    // the chunk's keys -> LDS
    {
        const bf16 *kb = k + ((pb * H_kv + g) * N + (int64_t)c * S) * D;
        const __amdgpu_buffer_rsrc_t kr =
            __builtin_amdgcn_make_buffer_rsrc((void *)kb, (short)0, S * D * 2, SUM_RSRC_WORD3);
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const int row = 4 * p + grp, blk = r;
            const int off = (row * D + (blk ^ (row & 15)) * 8) * 2;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (void __attribute__((address_space(3))) *)&kt[4 * p][0], 16,
                                                     off, 0, 0, 0);
        }
    }
    // B operand of the logits: lane (r, grp) holds dims 32 s + 8 grp .. +7 of
    // landmark head r (zero for r >= GLM and for mean pooling)
    const int H_lm = H_kv * GLM;
    bf16x8 qb[KS];
    {
        u32x4 qr[KS];
#pragma unroll
        for (int s2 = 0; s2 < KS; ++s2) qr[s2] = u32x4{0u, 0u, 0u, 0u};
        if (r < GLM && lm_mode != 2) {
            const int64_t qrow = lm_mode == 1 ? (int64_t)g * GLM + r : (b * H_lm + (int64_t)g * GLM + r) * C + c;
#pragma unroll
            for (int s2 = 0; s2 < KS; ++s2) qr[s2] = *(const u32x4 *)(q_lm + qrow * D + 32 * s2 + 8 * grp);
        }
#pragma unroll
        for (int s2 = 0; s2 < KS; ++s2) __builtin_memcpy(&qb[s2], &qr[s2], 16);
    }
    // the tile is in LDS once this wave's loads have completed (the memory
    // clobber keeps the tile reads below this point)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    // logits: acc[kt][i] = q'_r . k_(16 kt + 4 grp + i)
    f32x4 acc[KT];
#pragma unroll
    for (int kt2 = 0; kt2 < KT; ++kt2) acc[kt2] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2)
#pragma unroll
        for (int kt2 = 0; kt2 < KT; ++kt2) {
            const int row = 16 * kt2 + r;
            const u32x4 raw = kt[row][(4 * s2 + grp) ^ (row & 15)];
            bf16x8 a;
            __builtin_memcpy(&a, &raw, 16);
            acc[kt2] = mfma16(a, qb[s2], acc[kt2]);
        }
    // softmax of head r in base 2: x = a log2 e, e_j = 2^(x_j - max x)
    const float sl2 = scale * LOG2E;
    float m = -INFINITY;
#pragma unroll
    for (int kt2 = 0; kt2 < KT; ++kt2)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            acc[kt2][i] *= sl2;
            m = fmaxf(m, acc[kt2][i]);
        }
    m = rows4_max(m);
    float z = 0.f, ez = 0.f;
#pragma unroll
    for (int kt2 = 0; kt2 < KT; ++kt2)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float d2 = acc[kt2][i] - m;
            const float ex = exp2_hw(d2);
            z += ex;
            ez = fmaf(ex, d2, ez);
            acc[kt2][i] = ex;
        }
    z = rows4_sum(z);  // >= 1: the largest key contributes 2^0
    ez = rows4_sum(ez);
    const float inv_z = 1.f / z;
    // entropy = ln 2 (log2 Z - sum_j p_j (x_j - max x))
    const float ent = LN2 * (log2f(z) - ez * inv_z);

    // k'^T = K^T P: three bf16 terms of p in k-slot order (slots 8 grp .. +3:
    // keys 32 ps + 4 grp + i of tile 2 ps; slots 8 grp + 4 .. +7: tile 2 ps + 1)
    const int tsub = r & 3, trow = r >> 2;
    f32x4 o[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ps = 0; ps < PS; ++ps) {
        bf16x8 p1, p2, p3;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float x = acc[2 * ps + (j >> 2)][j & 3] * inv_z;
            const bf16 h1 = (bf16)x;
            const float r1 = x - (float)h1;
            const bf16 h2 = (bf16)r1;
            p1[j] = h1;
            p2[j] = h2;
            p3[j] = (bf16)(r1 - (float)h2);
        }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            // K^T fragment: in each 16-lane group the transposing read gives
            // lane i element i of the 16 values that lanes 4 q .. 4 q + 3
            // address; lane 4 q + tsub addresses dims x0 .. x0 + 3 of key row q
            const int x0 = 16 * dt + 4 * tsub;
            bf16x8 a;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int key = 32 * ps + 16 * h + 4 * grp + trow;
                const short *src = (const short *)&kt[key][(x0 >> 3) ^ (key & 15)] + (x0 & 7);
                const v4i16 v4 =
                    __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16 *)src);
                __builtin_memcpy((char *)&a + 8 * h, &v4, 8);
            }
            o[dt] = mfma16(a, p1, o[dt]);
            o[dt] = mfma16(a, p2, o[dt]);
            o[dt] = mfma16(a, p3, o[dt]);
        }
    }
    // lane (r, grp) holds dims 16 dt + 4 grp + i of head r's k'
    if (r < GLM) {
        const int64_t orow = (pb * H_lm + (int64_t)g * GLM + r) * C + c;
        TS *dst = k_sum + orow * D + 4 * grp;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            if constexpr (std::is_same<TS, float>::value) {
                *(f32x4 *)(dst + 16 * dt) = o[dt];
            } else {
                bf16x4 y;
#pragma unroll
                for (int i = 0; i < 4; ++i) y[i] = (bf16)o[dt][i];
                *(bf16x4 *)(dst + 16 * dt) = y;
            }
        }
        if (grp == 0) b_sum[orow] = ent;
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
        constexpr int WPB = S == 64 ? 2 : 1;  // the MFMA kernel's waves per block (one chunk each)
        const dim3 mgrid((unsigned)((units + WPB - 1) / WPB)), mblock(64 * WPB);
        auto gm = [&](auto kern) {
            hipLaunchKernelGGL(kern, mgrid, mblock, 0, st, (const bf16 *)k, (const bf16 *)q_lm, (TS *)k_sum, b_sum,
                               s.H_kv, s.N, s.C, s.scale, units, pages, num_pages, s.lm_mode);
        };
        switch (s.GLM) {
            case 1: gm(landmark_summary_mfma_kernel<TS, S, 1>); break;
            case 2: gm(landmark_summary_mfma_kernel<TS, S, 2>); break;
            case 4: gm(landmark_summary_mfma_kernel<TS, S, 4>); break;
            case 8: gm(landmark_summary_mfma_kernel<TS, S, 8>); break;
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
