// attend.hip -- kernel 3: fused sparse attention (selected chunks + window).
//
// hyper.ai HiLS summary, section 方法: each query attends exactly inside each
// selected chunk (intra-chunk softmax) and inside a chunk-aligned causal
// window; the per-chunk outputs are fused with weights exp(s^_c) / Z^ where
// Z^ = sum_c exp(s^_c) + Z_swa (partition estimate and the hierarchical
// factorisation of the attention weight).  Same page, kernel paragraph:
// adjacent queries x the G heads of a GQA group share one pass over the
// union of their selected chunks, so a loaded K/V chunk serves many rows.
//
// MI355X design (bf16 path):
//   * A block owns QB consecutive queries of one query chunk x the G heads
//     of one kv group (up to 16 waves x one MFMA tile of 16 rows; 16/G
//     queries x G heads per tile; QB = 64 for G = 4).  The queries share the candidate
//     set and the window, so one staged K/V chunk serves every tile that
//     needs it.  On the measured workload the union of 64 adjacent queries'
//     selections is ~5.6 chunks per query instead of 32 for separate
//     queries: the gather traffic, not the MFMA work, bounds this kernel.
//   * The block builds the ascending union of its queries' selections
//     (bitmap + prefix scan in LDS) and walks it, then the window chunks.
//     Every row keeps its next selected chunk and score in registers, so a
//     row only takes the chunks it selected (the union is a schedule; the
//     result is per query).  A tile with no selecting row skips the chunk.
//   * K and V^T chunk tiles are copied global -> LDS by buffer_load_lds
//     (16 bytes per lane, no register staging) into a ring of NSTAGE
//     stages.  There is no block barrier in the walk: a wave waits only for
//     the chunks its tiles compute (a flag the DMA writes behind the data),
//     counts itself out of each stage, and the last wave out refills the
//     stage NSTAGE chunks ahead, so waves drift up to NSTAGE - 1 chunks
//     apart and the uneven per-chunk work of the tiles evens out.  The
//     waves behind (those most of the block has passed) take issue priority,
//     since the last of them gates the next refill.  A
//     16-byte-block XOR swizzle by
//     row (applied through the per-lane source address, since the DMA
//     writes lane-contiguous LDS) keeps the MFMA operand reads free of
//     bank conflicts.
//   * Transposed products keep every per-row quantity in lane l%16:
//     S^T = K Q^T (A = K tile, B = Q^T in registers) and O^T += V^T P^T
//     (A = V^T tile, B = P^T packed straight from the S^T accumulators).  A
//     pre-pass writes V^T per chunk as fp16 [d][slot] with the keys of each
//     32-key group in the order the S^T accumulators deliver them.
//   * Q K^T runs on bf16 operands (exact products of the bf16 inputs).  P
//     lies in [0, 1] and is rounded to fp16 (8x finer than bf16), V^T is
//     fp16, so V^T P^T runs on fp16 MFMA: bf16 rounding of P alone can miss
//     a 2e-3 absolute bound on rows with few keys whose values cancel.  A
//     bf16 value of v converts to fp16 exactly when 2^-14 <= |v| < 65504
//     (fp16 normals keep 11 significant bits); below 2^-14 it rounds to the
//     fp16 subnormal grid (absolute error <= 2^-25), so a magnitude of at most
//     2^-25 becomes 0.  A value beyond fp16's range sets bit 1 of the
//     call's status word (V^T pre-pass).
//   * Selected chunk c of a row: exact softmax over its S keys, scaled by
//     exp(s^_c - m^) where m^ = max of the row's selected s^ (known up
//     front); the window then continues as an online softmax from running
//     max m^ and running mass sum_c exp(s^_c - m^).  exp2 throughout with
//     log2(e) folded into the scales.
//   * Blocks are mapped XCD-aware: the 8 XCDs each walk a contiguous range
//     of (batch, group, query block) work items, so the blocks resident on
//     one XCD's L2 are neighbouring query blocks whose unions overlap.
#include "hils_device.hpp"
#include <type_traits>

#include "hils_internal.hpp"

#define HILS_GPTR(p) ((const void __attribute__((address_space(1))) *)(p))
#define HILS_LPTR(p) ((void __attribute__((address_space(3))) *)(p))
// Word 3 of a raw buffer resource on CDNA: 32-bit data format (untyped
// dword loads), no swizzle, no index stride.
#define BUF_RSRC_WORD3 0x00020000

namespace hils {

// Source of the ring flags: the parity of a stage's lap (read by DMA).
__device__ int32_t ring_parity[2] = {0, 1};

// Key held by slot p of a chunk's transposed V rows.  In the S^T
// accumulators of 16-key tiles 2s and 2s+1, lane group gq holds keys
// 32s + 4gq + {0..3} and 32s + 16 + 4gq + {0..3}; those become the eight
// B-operand slots 8gq..8gq+7 of k-step s.
__host__ __device__ __forceinline__ int vt_slot_key(int p) {
    const int s = p >> 5, qd = p & 31, gq = qd >> 3, j = qd & 7;
    return 32 * s + (j < 4 ? 4 * gq + j : 16 + 4 * gq + (j - 4));
}

// vt[b, g, c, d, slot] = fp16(v[b, g, c*S + vt_slot_key(slot), d]), 0 past
// key Nk.  With a block table, chunk c of sequence b is page
// bt[b * max_pages + c] of a paged cache [P, H_kv, S, D].
// A value of v that fp16 cannot hold (|v| >= 65520, or not finite) sets bit
// 1 of the call's status word: the probability-weighted sum would then be
// wrong.
template <int D, int S>
__global__ __launch_bounds__(256) void v_transpose_kernel(const bf16 *__restrict__ v, f16 *__restrict__ vt, int Nk,
                                                          int CA, int H_kv, const int32_t *__restrict__ bt,
                                                          int max_pages, uint32_t *__restrict__ status) {
    __shared__ bf16 tile[S][D + 8];
    const int c = blockIdx.x;
    const int64_t bg = (int64_t)blockIdx.z * H_kv + blockIdx.y;
    const bf16 *src = bt ? v + ((int64_t)bt[(int64_t)blockIdx.z * max_pages + c] * H_kv + blockIdx.y) * S * D
                         : v + (bg * Nk + (int64_t)c * S) * D;
    bool range_bad = false;
    for (int idx = threadIdx.x; idx < S * (D / 8); idx += blockDim.x) {
        const int j = idx / (D / 8), cb = idx % (D / 8);
        u32x4 val = {0u, 0u, 0u, 0u};
        if ((int64_t)c * S + j < Nk) val = *(const u32x4 *)(src + (int64_t)j * D + cb * 8);
        bf16x8 x;
        __builtin_memcpy(&x, &val, 16);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            tile[j][cb * 8 + e] = x[e];
            range_bad |= !(fabsf((float)x[e]) < 65520.f);
        }
    }
    if (__ballot(range_bad) != 0ull && lane_id() == 0) atomicOr(status, 2u);
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

// Zeroes the status word of a call (the first kernel of the call).
__global__ void status_clear_kernel(uint32_t *status) {
    if (threadIdx.x == 0) *status = 0u;
}

// s_waitcnt with vmcnt = n (expcnt / lgkmcnt not waited).
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(n >= 0 && n < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// XOR swizzle of the 16-byte block index within an LDS row so that the 16
// lanes of one 128-bit read phase (rows r..r+15, same block) hit distinct
// bank groups, and so do the two 8-lane halves: rows of 16 blocks use
// r & 15; rows of 8 blocks (two rows per 256 bytes) use (r & 7) ^ ((r >> 3) & 1).
template <int NB>
__host__ __device__ __forceinline__ int swz(int row) {
    static_assert(NB == 8 || NB == 16, "rows of 8 or 16 blocks");
    return NB == 16 ? (row & 15) : ((row & 7) ^ ((row >> 3) & 1));
}

#ifndef LA_QK
#define LA_QK 4
#endif
#ifndef LA_PV
#define LA_PV 4
#endif
template <int D, int S, int G, int TPW, int NWAVE, int NSTAGE>
struct AttendCfg {
    static constexpr int QPT = 16 / G;               // queries per 16-row tile
    static constexpr int QB = NWAVE * TPW * QPT;     // queries per block
    static constexpr int KS = D / 32;                // k-steps of Q K^T
    static constexpr int KT = S / 16;                // 16-key tiles per chunk
    static constexpr int PS = S / 32;                // k-steps of V^T P^T
    static constexpr int DT = D / 16;                // 16-dim tiles of O^T
    static constexpr int NBK = D / 8;                // 16-byte blocks per K row
    static constexpr int NBV = S / 8;                // 16-byte blocks per V^T row
    static constexpr int PK = S * D * 2 / 1024;      // 1 KB pieces of a K tile
    static constexpr int PV = D * S * 2 / 1024;      // 1 KB pieces of a V^T tile
    static constexpr int NP = PK + PV;               // 1 KB DMA pieces per chunk
};

// Dynamic LDS: int16 sel[QB*K] (chunk ids, -1 padded); fp16 wt[QB*G*K]
// (fusion weights exp(s^ - m^) of each row's selections); uint bitmap[NW];
// int ulist[UCAP + W/S + 1] (the walk: union chunks, then window chunks;
// chunk id in the low 14 bits, its page of a paged cache above); int
// scan[16].  Selections live in LDS so that reading a
// row's next selection never waits on the vector-memory counter that
// tracks the chunk DMA.
// CM (chunk-major variant): the selected chunks were computed by
// cm_attend_kernel into weighted fp16 partials part[B, H_kv, NS, K, G D]
// (piece j of head e and lane group grp at 32 (G j + e) + 8 grp within a
// selection's region); the block starts
// each row from their sum and walks the window only.  Rows are the slab
// s0 = qb0 * QB .. s0 + NS - 1.
template <int D, int S, int G, int TPW, int NWAVE, int NSTAGE, bool CM>
__global__ __launch_bounds__(NWAVE * 64) void sparse_attend_kernel(
    const bf16 *__restrict__ q, const bf16 *__restrict__ k, const f16 *__restrict__ vt,
    const int32_t *__restrict__ sel_idx, const float *__restrict__ sel_score, bf16 *__restrict__ out,
    float *__restrict__ lse, int N, int H_q, int H_kv, int CA, int W, int K, float scale_log2, int NW, int UCAP,
    int nqb, int64_t n_items, int64_t per_xcd, int q0, int Nk, const int32_t *__restrict__ bt, int max_pages,
    int wait_spins, uint32_t *__restrict__ status, const f16 *__restrict__ part, int qb0, int NS) {
    using Cf = AttendCfg<D, S, G, TPW, NWAVE, NSTAGE>;
    constexpr int QPT = Cf::QPT, QB = Cf::QB, KS = Cf::KS, KT = Cf::KT, PS = Cf::PS, DT = Cf::DT;
    constexpr int NBK = Cf::NBK, NBV = Cf::NBV, PK = Cf::PK, NP = Cf::NP;
    constexpr int NT = NWAVE * 64;
    // chunk ring: stage s holds the K tile [S][NBK] then the V^T tile [D][NBV]
    __shared__ u32x4 ring[NSTAGE][S * NBK + D * NBV];
    // ring protocol: rel[s] counts the waves done with the chunks stage s
    // has held; flag[s] is written by DMA behind the data of each chunk
    // loaded into stage s (the parity of its lap through the ring)
    __shared__ int rel[NSTAGE];
    __shared__ int flag[NSTAGE];
    auto k_tile = [&](int buf) { return reinterpret_cast<u32x4(*)[NBK]>(&ring[buf][0]); };
    auto v_tile = [&](int buf) { return reinterpret_cast<u32x4(*)[NBV]>(&ring[buf][S * NBK]); };
    extern __shared__ int dyn[];
    int16_t *sel_l = (int16_t *)dyn;
    f16 *wt_l = (f16 *)(sel_l + QB * K);
    uint32_t *bitmap = (uint32_t *)(wt_l + QB * G * K);
    int *ulist = (int *)(bitmap + NW);
    int *scan = ulist + UCAP + W / S + 1;

    // ---- XCD-aware work item: consecutive blocks on one XCD take
    // consecutive (b, g, query block) items
    const int64_t item = (int64_t)(blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
    if (item >= n_items) return;
    const int qb = qb0 + (int)(item % nqb);
    const int64_t bg = item / nqb;
    const int g = (int)(bg % H_kv);
    const int64_t b = bg / H_kv;
    const int i0 = qb * QB;        // local row; rows are positions q0 + i (q0 % S == 0)
    const int qc = (q0 + i0) / S;  // query chunk
    const int n = max(0, qc - W / S);
    const int tid = threadIdx.x, wave = tid / WAVE, lane = lane_id(), grp = lane >> 4;
    const int r = lane & 15;

    // ---- setup: selections and scores of the block's queries.  The fp32
    // scores are first staged in the (still idle) chunk ring; the launcher
    // checks QB * G * K * 4 <= sizeof(ring).
    float *sc_tmp = (float *)&ring[0][0];
    if (tid < NSTAGE) {
        rel[tid] = 0;
        flag[tid] = -1;
    }
    if constexpr (!CM)
        for (int t = tid; t < NW; t += NT) bitmap[t] = 0u;
    for (int t = tid; t < QB * K; t += NT) {
        const int iq = i0 + t / K;
        const int c = iq < N ? sel_idx[(bg * N + iq) * K + t % K] : -1;
        sel_l[t] = (int16_t)c;
    }
    for (int t = tid; t < QB * G * K; t += NT) {
        const int m = t / (G * K), rem = t % (G * K), e = rem / K, iq = i0 + m;
        sc_tmp[t] = iq < N ? sel_score[((b * H_q + g * G + e) * N + iq) * K + rem % K] * LOG2E : -INFINITY;
    }
    __syncthreads();
    if constexpr (!CM)
        for (int t = tid; t < QB * K; t += NT) {
            const int c = sel_l[t];
            if (c >= 0 && c < n) atomicOr(&bitmap[c >> 5], 1u << (c & 31));
        }

    // per-tile row state; rows convert their scores to fp16 weights
    bf16x8 qf[TPW][KS];
    f32x4 O[TPW][DT];
    float mrun[TPW], lrun[TPW], nwt[TPW];
    int cur[TPW], nsel[TPW], nch[TPW], qrow[TPW], hrow[TPW];
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
        // selections are ascending with -1 padding at the end
        const int16_t *sl = sel_l + m * K;
        const float *sc = sc_tmp + (m * G + e) * K;
        float mh = -INFINITY;
        int ns = 0;
        for (int kk = 0; kk < K; ++kk) {
            const bool ok = sl[kk] >= 0;
            ns += ok;
            mh = ok ? fmaxf(mh, sc[kk]) : mh;
        }
        float z = 0.f;
        for (int kk = 0; kk < K; ++kk) {
            const float wv = sl[kk] >= 0 ? exp2f(sc[kk] - mh) : 0.f;
            z += wv;
            if (!CM && grp == 0) wt_l[(m * G + e) * K + kk] = (f16)wv;
        }
        mrun[t] = mh;
        lrun[t] = z;
        cur[t] = 0;
        nsel[t] = ns;
        nch[t] = ns > 0 ? sl[0] : 0x7fffffff;
        nwt[t] = ns > 0 ? exp2f(sc[0] - mh) : 0.f;
    }
    __syncthreads();

    // a walk entry: chunk id, and above it the chunk's page (paged cache)
    const int32_t *btb = bt ? bt + b * (int64_t)max_pages : nullptr;
    auto entry = [&](int c) { return btb ? (int)(((uint32_t)btb[c] << 14) | (uint32_t)c) : c; };

    // ---- ascending union: exclusive prefix sum of per-word popcounts
    int U = 0;
    if constexpr (!CM) {
        int base = 0;
        for (int w0 = 0; w0 < NW; w0 += NT) {
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
            for (int x = 0; x < NWAVE; ++x) {
                if (x < wave) wbase += scan[x];
                tot += scan[x];
            }
            int pos = base + wbase + incl - cnt;
            uint32_t wv = word;
            while (wv) {
                const int bit = __ffs(wv) - 1;
                wv &= wv - 1;
                if (pos < UCAP) ulist[pos] = entry(wi * 32 + bit);
                ++pos;
            }
            base += tot;
            __syncthreads();
        }
        U = min(base, UCAP);
    }
    const int wc0 = max(0, qc - W / S);
    const int T = U + (qc - wc0 + 1);
    for (int t = tid; t < T - U; t += NT) ulist[U + t] = entry(wc0 + t);
    __syncthreads();

    const bf16 *kbase = k + bg * (int64_t)Nk * D;
    const f16 *vtbase = vt + bg * (int64_t)CA * D * S;
    auto chunk_of = [&](int it) { return ulist[it] & 0x3fff; };

    // ---- DMA of one chunk into its ring stage by one wave: NP pieces of
    // 1 KB, 16 bytes per lane, then (lane 0 only) the stage's flag from
    // the parity table.  A wave's loads complete in issue order, so the
    // flag lands after the data.  Buffer loads: K resources end at key Nk,
    // so rows of a partial last chunk read as zeros (those keys are
    // masked), and the per-lane address is 32 bits.
    const __amdgpu_buffer_rsrc_t par_rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void *)&ring_parity[0], (short)0, 8, BUF_RSRC_WORD3);
    auto issue = [&](int it) {
        const int ent = __builtin_amdgcn_readfirstlane(ulist[it]);
        const int c = ent & 0x3fff;
        const bf16 *kc = btb ? k + ((int64_t)((uint32_t)ent >> 14) * H_kv + g) * S * D : kbase + (int64_t)c * S * D;
        const int buf = __builtin_amdgcn_readfirstlane(it % NSTAGE);
        const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(vtbase + (int64_t)c * D * S), (short)0, D * S * 2, BUF_RSRC_WORD3);
        // The swizzle repeats every 16 rows, so the lane part of a piece's
        // source offset takes PPx distinct values.  The rest of a V^T
        // piece's offset goes in the scalar offset.  That one is not
        // range-checked, so the K tile instead takes one resource per 16
        // rows, each ending at key Nk: rows past Nk read as zeros.
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            if (p < PK) {
                constexpr int RPP = 1024 / (D * 2), PPK = 16 / RPP;  // K rows per piece, pieces per 16 rows
                const int r16 = (p / PPK) * 16;
                const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
                    (void *)(kc + (int64_t)r16 * D), (short)0, max(0, Nk - c * S - r16) * D * 2, BUF_RSRC_WORD3);
                const int row = (p % PPK) * RPP + lane / NBK, blk = lane % NBK;
                const int off = (row * D + (blk ^ swz<NBK>(row)) * 8) * 2;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, HILS_LPTR(&k_tile(buf)[p * RPP][0]), 16, off, 0, 0, 0);
            } else {
                constexpr int RPP = 1024 / (S * 2), PPV = 16 / RPP;  // V^T rows per piece, pieces per 16 rows
                const int pv = p - PK;
                const int row = (pv % PPV) * RPP + lane / NBV, blk = lane % NBV;
                const int off = (row * S + (blk ^ swz<NBV>(row)) * 8) * 2;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, HILS_LPTR(&v_tile(buf)[pv * RPP][0]), 16, off,
                                                         (pv / PPV) * 16 * S * 2, 0, 0);
            }
        }
        if (lane == 0)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(par_rsrc, HILS_LPTR(&flag[buf]), 4, ((it / NSTAGE) & 1) * 4, 0,
                                                     0, 0);
    };
    // Software pipeline of n LDS fragment reads, each feeding M MFMAs (one
    // per tile of the wave): the scheduler issues LA reads ahead, then
    // alternates M MFMAs with one read, so about LA fragments are live.
    auto pipeline = [&](auto n_c, auto m_c, auto la_c) {
        constexpr int n = decltype(n_c)::value, M = decltype(m_c)::value, LA = decltype(la_c)::value;
        __builtin_amdgcn_sched_group_barrier(0x100, LA, 0);  // DS reads
#pragma unroll
        for (int i = 0; i < n - LA; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, M, 0);  // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, M * LA, 0);
    };
    // S^T tiles: acc[t][kt][i] = q_row(t) . k_{16kt + 4grp + i}.  One K
    // fragment read feeds the MFMA of every tile of the wave; the KT key
    // tiles are independent accumulators, visited k-step major.
    auto qk = [&](auto mask_c, const u32x4 (*kt_lds)[NBK], f32x4 (&acc)[TPW][KT]) {
        constexpr int MASK = decltype(mask_c)::value, NM = __builtin_popcount(MASK);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < TPW; ++t)
#pragma unroll
            for (int kt = 0; kt < KT; ++kt) acc[t][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
        (void)NM;
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
            for (int kt = 0; kt < KT; ++kt) {
                const int row = 16 * kt + r;
                const u32x4 raw = kt_lds[row][(4 * s + grp) ^ swz<NBK>(row)];
                bf16x8 a;
                __builtin_memcpy(&a, &raw, 16);
#pragma unroll
                for (int t = 0; t < TPW; ++t)
                    if ((MASK >> t) & 1) acc[t][kt] = mfma16(a, qf[t][s], acc[t][kt]);
            }
        pipeline(std::integral_constant<int, KS * KT>{}, std::integral_constant<int, NM>{},
                 std::integral_constant<int, LA_QK>{});
        __builtin_amdgcn_sched_barrier(0);
    };
    // O^T += V^T P^T for every tile of the wave, P^T packed from the
    // exponentiated S^T; one V^T fragment read feeds every tile.
    auto pv = [&](auto mask_c, const u32x4 (*vt_lds)[NBV], const f32x4 (&p)[TPW][KT]) {
        constexpr int MASK = decltype(mask_c)::value, NM = __builtin_popcount(MASK);
        f16x8 bp[TPW][PS];
#pragma unroll
        for (int t = 0; t < TPW; ++t)
#pragma unroll
            for (int ps = 0; ps < PS; ++ps)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    bp[t][ps][i] = (f16)p[t][2 * ps][i];
                    bp[t][ps][4 + i] = (f16)p[t][2 * ps + 1][i];
                }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ps = 0; ps < PS; ++ps)
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const int row = 16 * dt + r;
                const u32x4 raw = vt_lds[row][(4 * ps + grp) ^ swz<NBV>(row)];
                f16x8 a;
                __builtin_memcpy(&a, &raw, 16);
#pragma unroll
                for (int t = 0; t < TPW; ++t)
                    if ((MASK >> t) & 1) O[t][dt] = mfma16h(a, bp[t][ps], O[t][dt]);
            }
        pipeline(std::integral_constant<int, PS * DT>{}, std::integral_constant<int, NM>{},
                 std::integral_constant<int, LA_PV>{});
        __builtin_amdgcn_sched_barrier(0);
    };

    // ---- walk: union chunks, then the window.  Waves are decoupled: a
    // wave waits only for each chunk's data to land (its flag), and
    // announces in rel when it is done with a stage; the last wave to leave
    // a stage refills it with the chunk NSTAGE steps ahead.  So a wave runs
    // up to NSTAGE - 1 chunks ahead of the slowest, and the work of the
    // tiles that a chunk activates spreads over several chunks' time.
    // Every wait is bounded, and the slowest wave never waits on another
    // wave: its chunk was issued when it left that chunk's stage.
    // A wait that runs out of pauses gives up: the wave goes on, marks its
    // rows NaN and sets the call's status word (the protocol's counters stay
    // exact, so every wave still reaches the end).
    bool expired = false;
    for (int j = wave; j < NSTAGE && j < T; j += NWAVE) issue(j);
    if constexpr (CM) {
        // the selected chunks' weighted outputs, summed in slot order while
        // the first window chunks land.  Piece j of a lane (dims of dt = 2j,
        // 2j + 1) sits at 32 j + 8 grp of the row; four slots per round keep
        // 4 * D / 32 loads of 16 bytes in flight.
        // 8-wave blocks alone on a CU (64 KB chunks) have the registers for 8
        constexpr int NV = D / 32, UR = (NWAVE <= 8 && S * D > 128 * 64) ? 8 : 4;
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
            const int m = qrow[t], iq = i0 + m;
            const int16_t *sl = sel_l + m * K;
            // partial regions [B, H_kv, NS, K, G D], ordered [piece j][head][grp][8]
            const f16 *pr = part + (bg * NS + (iq - qb0 * QB)) * (int64_t)K * G * D + 32 * (hrow[t] - g * G) + 8 * grp;
            const int ns = iq < N ? nsel[t] : 0;
            for (int k0 = 0; k0 < ns; k0 += UR) {
                f16x8 y[UR][NV];
#pragma unroll
                for (int u = 0; u < UR; ++u) {
                    const int kk = k0 + u;
                    const bool use = kk < ns && sl[min(kk, K - 1)] < n;
#pragma unroll
                    for (int j = 0; j < NV; ++j)
                        y[u][j] = use ? *(const f16x8 *)(pr + (int64_t)kk * G * D + 32 * G * j) : f16x8{};
                }
#pragma unroll
                for (int u = 0; u < UR; ++u)
#pragma unroll
                    for (int j = 0; j < NV; ++j)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            O[t][2 * j][i] += (float)y[u][j][i];
                            O[t][2 * j + 1][i] += (float)y[u][j][4 + i];
                        }
            }
        }
    }
    for (int it = 0; it < T; ++it) {
        const int buf = it % NSTAGE;
        const int c = chunk_of(it);
        const bool window = it >= U;
        bool act[TPW];
        bool any = false;
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
            act[t] = window || nch[t] == c;
            any |= act[t];
        }
        // Every wave waits for every chunk to land, also one it skips: so no
        // wave leaves a stage before its current lap is in (a wave can
        // lead the slowest by at most NSTAGE - 1 chunks, rel[s] never mixes
        // laps) and, having seen the previous lap's flag, a wave only
        // finds this lap's or the previous lap's parity in flag[buf].
        // (LDS operations of a wave execute in order, so a plain flag read
        // orders the flag before the data reads, and those before the
        // release below; the asm statements are compiler barriers.)
        int rel_seen = 0;  // rel[buf] read just after the flag
        {
            const int want = (it / NSTAGE) & 1;
            const uint32_t faddr = (uint32_t)(uintptr_t)&flag[buf];  // LDS offsets
            const uint32_t raddr = (uint32_t)(uintptr_t)&rel[buf];
            bool landed = false;
            for (int spin = 0; spin < wait_spins; ++spin) {
                // read in asm: the compiler would otherwise first wait for
                // all of this wave's DMA in flight (the flag is a DMA target).
                // The stage's leave counter comes in the same round trip
                // (early-clobber outputs: the first load's destination must
                // not be the second load's address register).
                int fv, rv;
                asm volatile("ds_read_b32 %0, %2\n\tds_read_b32 %1, %3\n\ts_waitcnt lgkmcnt(0)"
                             : "=&v"(fv), "=&v"(rv)
                             : "v"(faddr), "v"(raddr)
                             : "memory");
                rel_seen = rv;
                if (fv == want) {
                    landed = true;
                    break;
                }
                // a waiting wave yields its SIMD to the working ones (the
                // longer pause suits the deeper ring: its waits are longer)
                __builtin_amdgcn_s_sleep(NSTAGE >= 4 ? 8 : 1);
            }
            expired |= !landed;
        }
        // A stage is refilled only when its last wave leaves it, so the
        // waves that at least half of the block has already passed are on
        // the refill's critical path: they take issue priority over the
        // waves running ahead for this chunk.  rel[buf] holds NWAVE * lap +
        // the waves that have left this lap's chunk; read after this lap's
        // flag, it is at least NWAVE * lap (the lap's DMA was issued once
        // the previous lap's last wave left).
        {
            const int left = __builtin_amdgcn_readfirstlane(rel_seen) - NWAVE * (it / NSTAGE);
            if (left >= NWAVE / 2) __builtin_amdgcn_s_setprio(3);
            else __builtin_amdgcn_s_setprio(0);
        }
        if (__ballot(any) != 0ull) {
            f32x4 acc[TPW][KT];
            if (!window) {
                // a wave computes its tiles when one of its rows selected chunk c;
                // rows that did not select it get weight 0 (exact zeros in O)
                int wmask = 0;
#pragma unroll
                for (int t = 0; t < TPW; ++t) wmask |= (__ballot(act[t]) != 0ull) << t;
                auto sel_step = [&](auto mask_c) {
                    constexpr int MASK = decltype(mask_c)::value;
                    qk(mask_c, k_tile(buf), acc);
#pragma unroll
                    for (int t = 0; t < TPW; ++t) {
                        if (!((MASK >> t) & 1)) continue;
                        float cmax = -INFINITY;
#pragma unroll
                        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                            for (int i = 0; i < 4; ++i) cmax = fmaxf(cmax, acc[t][kt][i]);
                        cmax = rows4_max(cmax) * scale_log2;
                        float lc = 0.f;
#pragma unroll
                        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                acc[t][kt][i] = exp2_hw(fmaf(acc[t][kt][i], scale_log2, -cmax));
                                lc += acc[t][kt][i];
                            }
                        lc = rows4_sum(lc);  // >= 1: the largest key contributes 2^0
                        const float f = act[t] ? nwt[t] * __builtin_amdgcn_rcpf(lc) : 0.f;
#pragma unroll
                        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                            for (int i = 0; i < 4; ++i) acc[t][kt][i] *= f;
                    }
                    pv(mask_c, v_tile(buf), acc);
                };
                if constexpr (TPW == 1) {
                    sel_step(std::integral_constant<int, 1>{});
                } else {
                    if (wmask == 1) sel_step(std::integral_constant<int, 1>{});
                    else if (wmask == 2) sel_step(std::integral_constant<int, 2>{});
                    else sel_step(std::integral_constant<int, 3>{});
                }
#pragma unroll
                for (int t = 0; t < TPW; ++t)
                    if (act[t]) {
                        const int nx = ++cur[t];
                        const int m = qrow[t], e = hrow[t] - g * G;
                        nch[t] = nx < nsel[t] ? (int)sel_l[m * K + nx] : 0x7fffffff;
                        nwt[t] = nx < nsel[t] ? (float)wt_l[(m * G + e) * K + nx] : 0.f;
                    }
            } else {
                const bool diag = c == qc;
                constexpr int ALL = (1 << TPW) - 1;
                qk(std::integral_constant<int, ALL>{}, k_tile(buf), acc);
#pragma unroll
                for (int t = 0; t < TPW; ++t) {
                    const int iq = i0 + qrow[t];
                    // only the query's own chunk holds keys after the row: lim is
                    // the last key offset (from the lane's first) the row sees
                    const int lim = diag ? q0 + iq - c * S - 4 * grp : S;
                    float cmax = -INFINITY;
#pragma unroll
                    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const float x = 16 * kt + i > lim ? -INFINITY : acc[t][kt][i] * scale_log2;
                            acc[t][kt][i] = x;
                            cmax = fmaxf(cmax, x);
                        }
                    cmax = rows4_max(cmax);
                    const float mnew = fmaxf(mrun[t], cmax);
                    const float alpha = exp2_hw(mrun[t] - mnew);
                    const bool rescale = __ballot(mnew > mrun[t]) != 0ull;
                    float ls = 0.f;
#pragma unroll
                    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            acc[t][kt][i] = exp2_hw(acc[t][kt][i] - mnew);
                            ls += acc[t][kt][i];
                        }
                    ls = rows4_sum(ls);
                    lrun[t] = lrun[t] * alpha + ls;
                    mrun[t] = mnew;
                    // alpha = 1 exactly in every lane whose max held
                    if (rescale) {
#pragma unroll
                        for (int dt = 0; dt < DT; ++dt) O[t][dt] *= alpha;
                    }
                }
                pv(std::integral_constant<int, ALL>{}, v_tile(buf), acc);
            }
        }
        // leave the stage (after this wave's reads of it: LDS operations of
        // a wave complete in order); the last wave out refills it
        // (in asm for the same reason as the flag read)
        int old = 0;
        if (lane == 0) {
            const uint32_t raddr = (uint32_t)(uintptr_t)&rel[buf];
            asm volatile("ds_add_rtn_u32 %0, %1, %2\n\ts_waitcnt lgkmcnt(0)" : "=v"(old) : "v"(raddr), "v"(1)
                         : "memory");
        }
        old = __builtin_amdgcn_readfirstlane(old);
        if (old == NWAVE * (it / NSTAGE + 1) - 1 && it + NSTAGE < T) issue(it + NSTAGE);
    }
    wait_vmcnt<0>();  // no DMA outstanding when the wave retires
    if (expired && lane == 0) atomicOr(status, 1u);

    // ---- epilogue
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
        const int iq = i0 + qrow[t];
        if (iq >= N) continue;
        const float inv = expired ? __builtin_nanf("") : 1.f / lrun[t];
        bf16 *orow = out + ((b * H_q + hrow[t]) * N + iq) * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            bf16x4 y;
#pragma unroll
            for (int i = 0; i < 4; ++i) y[i] = (bf16)(O[t][dt][i] * inv);
            *(bf16x4 *)(orow + 16 * dt + 4 * grp) = y;
        }
        if (lse && grp == 0)
            lse[(b * H_q + hrow[t]) * N + iq] = expired ? __builtin_nanf("") : (mrun[t] + log2f(lrun[t])) * LN2;
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
                                                                float scale, int q0, int Nk,
                                                                const int32_t *__restrict__ bt, int max_pages) {
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
    const int pi = q0 + i;  // position of row i
    // key / value row j: contiguous [B, H_kv, Nk, D] or paged [P, H_kv, S, D]
    auto kv_row = [&](const float *base, int j) -> const float * {
        if (!bt) return base + ((b * H_kv + g) * (int64_t)Nk + j) * D;
        return base + (((int64_t)bt[b * max_pages + j / S] * H_kv + g) * S + j % S) * D;
    };
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
                const float *kr = kv_row(k, j);
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
            for (int j = j0; j <= j1; ++j) acc = fmaf(p_l[wave][j - j0], kv_row(v, j)[x], acc);
            o[y] = acc;
        }
        wave_sync();
    };

    const int w0 = max(0, (pi / S) * S - W);
    float mw = -INFINITY, lw = 0.f, ow[DPL];
#pragma unroll
    for (int y = 0; y < DPL; ++y) ow[y] = 0.f;
    for (int j = w0; j <= pi; j += 2 * WAVE) attend_block(j, min(pi, j + 2 * WAVE - 1), mw, lw, ow);
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
    const size_t base = FUSED_STATUS_BYTES + align_up((size_t)s.B * s.H_kv * s.CA * s.D * s.S * 2, 256);
    return attend_use_cm(s) ? base + cm_workspace_bytes(s) : base;
}

// Block shapes: NWAVE waves of one 16-row tile each (QB = NWAVE * 16/G
// queries, dividing S).  16 waves leave 128 registers per wave, enough for
// 64-key chunks at d = 128 only.  The ring holds 4 chunks when a chunk is
// 32 KB, else 2.
// The window pass after the chunk-major form (CMF) walks ~W/S chunks per
// block: it keeps two stages, so that two blocks share a CU and one block's
// partial reads overlap the other's chunks.
template <int D, int S, int G, int NWAVE, int TPW_ = 1, bool CMF = false>
struct AttendPlan {
    static constexpr int TPW = TPW_;
    static constexpr int QB = NWAVE * TPW * (16 / G);
    static constexpr bool valid = QB <= S && S % QB == 0 && !(NWAVE == 16 && D * S > 128 * 64) &&
                                  !(TPW == 2 && D * S > 128 * 64);
    static constexpr int NSTAGE = (!CMF && S * D * 4 <= 32 * 1024) ? 4 : 2;
    static constexpr size_t ring_bytes = (size_t)NSTAGE * 2 * S * D * 2;
    static constexpr size_t static_lds = ring_bytes + 64;
};

constexpr size_t LDS_BYTES = 160 * 1024;

// The chunk-major variant's extra arguments (part == null: the walk).
struct WinArgs {
    const f16 *part;
    int s0, NS;
};

// Bitmap words and union capacity of a block's walk (none in the
// chunk-major variant: it walks the window only).
template <int QB>
static void walk_sizes(const Shape &s, bool cm, int &NW, int &UCAP) {
    NW = cm ? 0 : (s.C + 31) / 32 + 1;
    UCAP = cm ? 0 : std::min(s.C + 1, QB * s.K + 1);
}

template <int D, int S, int G, int NWAVE, int TPW>
static size_t attend_dyn_lds(const Shape &s, bool cm) {
    constexpr int QB = AttendPlan<D, S, G, NWAVE, TPW>::QB;
    int NW, UCAP;
    walk_sizes<QB>(s, cm, NW, UCAP);
    return align_up((size_t)QB * s.K * 2 + (size_t)QB * G * s.K * 2, 16) + (size_t)NW * 4 +
           (size_t)(UCAP + s.W / s.S + 1) * 4 + 16 * 4;
}

template <int D, int S, int G, int NWAVE, int TPW, bool CM>
static hipError_t go_attend(const Shape &s, const void *q, const void *k, const void *vt, const int32_t *sel_idx,
                            const float *sel_score, void *out, float *lse, uint32_t *status, const WinArgs &wa,
                            hipStream_t st) {
    using P = AttendPlan<D, S, G, NWAVE, TPW, CM>;
    const int QB = P::QB;
    int NW, UCAP;
    walk_sizes<P::QB>(s, CM, NW, UCAP);
    const size_t dyn = attend_dyn_lds<D, S, G, NWAVE, TPW>(s, CM);
    // query blocks of the rows s0 .. s0 + rows - 1 (s0 % S == 0, QB | S)
    const int rows = CM ? std::min(wa.NS, s.N - wa.s0) : s.N;
    const int qb0 = CM ? wa.s0 / QB : 0;
    const int nqb = (rows + QB - 1) / QB;
    const int64_t n_items = (int64_t)s.B * s.H_kv * nqb;
    const int64_t per_xcd = (n_items + 7) / 8;
    const dim3 grid((unsigned)(8 * per_xcd)), block(NWAVE * 64);
    auto kern = sparse_attend_kernel<D, S, G, TPW, NWAVE, P::NSTAGE, CM>;
    hipError_t e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, grid, block, dyn, st, (const bf16 *)q, (const bf16 *)k, (const f16 *)vt, sel_idx,
                       sel_score, (bf16 *)out, lse, s.N, s.H_q, s.H_kv, s.CA, s.W, s.K, s.scale * LOG2E, NW, UCAP,
                       nqb, n_items, per_xcd, s.q0, s.Nk, s.bt, s.max_pages, s.wait_spins, status, wa.part, qb0,
                       wa.NS);
    return hipGetLastError();
}

template <int D, int S, int G, int NWAVE, int TPW, bool CM>
static bool fits_plan(const Shape &s) {
    using P = AttendPlan<D, S, G, NWAVE, TPW, CM>;
    if constexpr (!P::valid) return false;
    else
        return P::static_lds + attend_dyn_lds<D, S, G, NWAVE, TPW>(s, CM) <= LDS_BYTES &&
               (size_t)P::QB * G * s.K * 4 <= P::ring_bytes;  // setup staging of the scores
}

template <int D, int S, int G, int NWAVE, int TPW>
static bool fits(const Shape &s, bool cm) {
    return cm ? fits_plan<D, S, G, NWAVE, TPW, true>(s) : fits_plan<D, S, G, NWAVE, TPW, false>(s);
}

// Largest block whose LDS (chunk ring + selections + union) fits.
template <int D, int S, int G, int NWAVE, int TPW, bool CM>
static bool try_attend(const Shape &s, const void *q, const void *k, const void *vt, const int32_t *sel_idx,
                       const float *sel_score, void *out, float *lse, uint32_t *status, const WinArgs &wa,
                       hipStream_t st, hipError_t &err) {
    if constexpr (!AttendPlan<D, S, G, NWAVE, TPW>::valid) {
        return false;
    } else {
        if (!fits<D, S, G, NWAVE, TPW>(s, CM)) return false;
        err = go_attend<D, S, G, NWAVE, TPW, CM>(s, q, k, vt, sel_idx, sel_score, out, lse, status, wa, st);
        return true;
    }
}

template <int D, int S, int G, bool CM>
static hipError_t dispatch_w(const Shape &s, const void *q, const void *k, const void *vt, const int32_t *sel_idx,
                             const float *sel_score, void *out, float *lse, uint32_t *status, const WinArgs &wa,
                             hipStream_t st) {
    hipError_t err = hipErrorInvalidValue;
    // the window pass prefers 8-wave blocks (two per CU with its 2-stage ring)
    if (CM && try_attend<D, S, G, 8, 1, CM>(s, q, k, vt, sel_idx, sel_score, out, lse, status, wa, st, err)) return err;
    if (try_attend<D, S, G, 16, 1, CM>(s, q, k, vt, sel_idx, sel_score, out, lse, status, wa, st, err)) return err;
    if (try_attend<D, S, G, 8, 1, CM>(s, q, k, vt, sel_idx, sel_score, out, lse, status, wa, st, err)) return err;
    if (try_attend<D, S, G, 4, 1, CM>(s, q, k, vt, sel_idx, sel_score, out, lse, status, wa, st, err)) return err;
    if (try_attend<D, S, G, 2, 1, CM>(s, q, k, vt, sel_idx, sel_score, out, lse, status, wa, st, err)) return err;
    return hipErrorInvalidValue;
}

template <int D, int S, int G>
static bool fits_any(const Shape &s, bool cm) {
    return fits<D, S, G, 16, 1>(s, cm) || fits<D, S, G, 8, 1>(s, cm) || fits<D, S, G, 4, 1>(s, cm) ||
           fits<D, S, G, 2, 1>(s, cm);
}

template <int D, int S>
static bool fits_g(const Shape &s, bool cm) {
    switch (s.G) {
        case 1: return fits_any<D, S, 1>(s, cm);
        case 2: return fits_any<D, S, 2>(s, cm);
        case 4: return fits_any<D, S, 4>(s, cm);
        case 8: return fits_any<D, S, 8>(s, cm);
        default: return false;
    }
}

static bool fits_shape(const Shape &s, bool cm) {
    if (s.D == 64 && s.S == 64) return fits_g<64, 64>(s, cm);
    if (s.D == 64 && s.S == 128) return fits_g<64, 128>(s, cm);
    if (s.D == 128 && s.S == 64) return fits_g<128, 64>(s, cm);
    if (s.D == 128 && s.S == 128) return fits_g<128, 128>(s, cm);
    return false;
}

bool window_after_cm_supported(const Shape &s) { return s.io_bf16 && fits_shape(s, true); }

bool sparse_attend_supported(const Shape &s) {
    if (!s.io_bf16) return true;
    return attend_use_cm(s) || fits_shape(s, false);
}

template <int D, int S, bool CM>
static hipError_t dispatch_g(const Shape &s, const void *q, const void *k, const void *vt, const int32_t *sel_idx,
                             const float *sel_score, void *out, float *lse, uint32_t *status, const WinArgs &wa,
                             hipStream_t st) {
    switch (s.G) {
        case 1: return dispatch_w<D, S, 1, CM>(s, q, k, vt, sel_idx, sel_score, out, lse, status, wa, st);
        case 2: return dispatch_w<D, S, 2, CM>(s, q, k, vt, sel_idx, sel_score, out, lse, status, wa, st);
        case 4: return dispatch_w<D, S, 4, CM>(s, q, k, vt, sel_idx, sel_score, out, lse, status, wa, st);
        case 8: return dispatch_w<D, S, 8, CM>(s, q, k, vt, sel_idx, sel_score, out, lse, status, wa, st);
        default: return hipErrorInvalidValue;
    }
}

template <bool CM>
static hipError_t dispatch_shape(const Shape &s, const void *q, const void *k, const void *vt,
                                 const int32_t *sel_idx, const float *sel_score, void *out, float *lse,
                                 uint32_t *status, const WinArgs &wa, hipStream_t st) {
    if (s.D == 64 && s.S == 64) return dispatch_g<64, 64, CM>(s, q, k, vt, sel_idx, sel_score, out, lse, status, wa, st);
    if (s.D == 64 && s.S == 128) return dispatch_g<64, 128, CM>(s, q, k, vt, sel_idx, sel_score, out, lse, status, wa, st);
    if (s.D == 128 && s.S == 64) return dispatch_g<128, 64, CM>(s, q, k, vt, sel_idx, sel_score, out, lse, status, wa, st);
    if (s.D == 128 && s.S == 128)
        return dispatch_g<128, 128, CM>(s, q, k, vt, sel_idx, sel_score, out, lse, status, wa, st);
    return hipErrorInvalidValue;
}

hipError_t launch_window_after_cm(const Shape &s, const void *q, const void *k, const void *vt,
                                  const int32_t *sel_idx, const float *sel_score, void *out, float *lse,
                                  uint32_t *status, const void *part, int s0, int NS, hipStream_t st) {
    const WinArgs wa{(const f16 *)part, s0, NS};
    return dispatch_shape<true>(s, q, k, vt, sel_idx, sel_score, out, lse, status, wa, st);
}

hipError_t launch_vt_prepass(const Shape &s, const void *v, void *vt, uint32_t *status, hipStream_t st) {
    // clear the call's status word, then the V^T pre-pass (fp16, slot order)
    hipLaunchKernelGGL(status_clear_kernel, dim3(1), dim3(64), 0, st, status);
    const dim3 grid((unsigned)s.CA, (unsigned)s.H_kv, (unsigned)s.B), block(256);
    auto vtr = [&](auto kern) {
        hipLaunchKernelGGL(kern, grid, block, 0, st, (const bf16 *)v, (f16 *)vt, s.Nk, s.CA, s.H_kv, s.bt,
                           s.max_pages, status);
    };
    if (s.D == 64 && s.S == 64) vtr(v_transpose_kernel<64, 64>);
    else if (s.D == 64) vtr(v_transpose_kernel<64, 128>);
    else if (s.S == 64) vtr(v_transpose_kernel<128, 64>);
    else vtr(v_transpose_kernel<128, 128>);
    return hipGetLastError();
}

hipError_t launch_sparse_attend(const Shape &s, const void *q, const void *k, const void *v, const int32_t *sel_idx,
                                const float *sel_score, void *out, float *lse, uint32_t *status, void *vt_ws,
                                hipStream_t st) {
    if ((int64_t)s.B * s.N == 0) return hipSuccess;
    if (!s.io_bf16) {
        const int64_t rows = (int64_t)s.B * s.H_q * s.N;
        const dim3 grid((unsigned)((rows + 3) / 4)), block(256);
        if (s.D == 64)
            hipLaunchKernelGGL(sparse_attend_f32_kernel<64>, grid, block, 0, st, (const float *)q, (const float *)k,
                               (const float *)v, sel_idx, sel_score, (float *)out, lse, s.B, s.N, s.H_q, s.H_kv, s.S,
                               s.W, s.K, s.scale, s.q0, s.Nk, s.bt, s.max_pages);
        else
            hipLaunchKernelGGL(sparse_attend_f32_kernel<128>, grid, block, 0, st, (const float *)q, (const float *)k,
                               (const float *)v, sel_idx, sel_score, (float *)out, lse, s.B, s.N, s.H_q, s.H_kv, s.S,
                               s.W, s.K, s.scale, s.q0, s.Nk, s.bt, s.max_pages);
        return hipGetLastError();
    }
    f16 *vt = (f16 *)vt_ws;
    if (attend_use_cm(s)) {
        char *cm_ws = (char *)vt_ws + align_up((size_t)s.B * s.H_kv * s.CA * s.D * s.S * 2, 256);
        return launch_sparse_attend_cm(s, q, k, v, sel_idx, sel_score, out, lse, status, vt_ws, cm_ws, st);
    }
    {
        const hipError_t e = launch_vt_prepass(s, v, vt, status, st);
        if (e != hipSuccess) return e;
    }
    const WinArgs wa{nullptr, 0, s.N};
    return dispatch_shape<false>(s, q, k, vt, sel_idx, sel_score, out, lse, status, wa, st);
}

}  // namespace hils
