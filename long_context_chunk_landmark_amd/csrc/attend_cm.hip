// attend_cm.hip -- chunk-major form of the selected-chunk part of kernel 3.
//
// hyper.ai HiLS summary, section 方法 (partition estimate and hierarchical
// factorisation): every selected chunk c of a query contributes its own
// exact softmax output o_c, weighted by exp(s^_c) / Z^.  The contributions
// of different chunks never interact before that weighted sum, so they can
// be computed in any order.
//
// The query-major walk (attend.hip) reuses a staged chunk only across the
// queries of one block.  When selections scatter (i.i.d. inputs select
// nearly disjoint chunks even for adjacent queries), a staged 32-64 KB chunk
// then serves a handful of rows.  This form turns the loop around:
//   1. cm_count: per (b, g) and chunk, how many rows of the slab selected it;
//      per row and head, the max of the row's selected scores (log2 units);
//   2. cm_scan: per (b, g), exclusive offsets of every chunk's list and of
//      its fixed-size segments (SEG entries each);
//   3. cm_fill: each selection (row i, slot kk) is written into its chunk's
//      list (order within a list is arbitrary: a row's result never depends
//      on the other rows of its MFMA tile);
//   4. cm_attend: one block per segment stages chunk c (K bf16, V^T fp16) in
//      LDS once and runs packed 16-row tiles (16/G entries x the G heads of
//      the group) over the segment: S^T = K Q^T on bf16 MFMA, the exact
//      softmax over the chunk's S keys, O^T = V^T P^T on fp16 MFMA, then the
//      row's weight exp(s^_c - m^) / l_c, where m^ is the row's largest
//      selected score.  The weighted output goes to a partial buffer
//      [B, H_kv, slab rows, K, G d] in fp16, one region of G d values per
//      (query, slot) holding the G heads' outputs;
//   5. the window kernel (attend.hip, chunk-major variant) starts each row
//      from O = sum over its slots of the partials (fp32, slot order),
//      running max m^ and mass sum_c exp(s^_c - m^), exactly the state the
//      query-major walk reaches after its selected chunks, and continues
//      with the window's online softmax.
// Rows are processed in slabs of NS queries so that the partial buffer
// stays bounded; every slab runs steps 1-5.
#include "hils_device.hpp"

#include "hils_internal.hpp"

namespace hils {

namespace {

constexpr int CM_SCAN_THREADS = 1024;

// 16-byte-block XOR swizzle of an LDS row (same rule as the walk kernel's
// ring): rows of 16 blocks use r & 15, rows of 8 blocks (r & 7) ^ ((r >> 3) & 1).
template <int NB>
__device__ __forceinline__ int cm_swz(int row) {
    static_assert(NB == 8 || NB == 16, "rows of 8 or 16 blocks");
    return NB == 16 ? (row & 15) : ((row & 7) ^ ((row >> 3) & 1));
}

// Schedule of n LDS fragment reads each feeding one MFMA: LA reads issued
// ahead, then one MFMA per read, so about LA fragments are live (the
// scheduler would otherwise hoist every read and run out of registers).
template <int n, int LA>
__device__ __forceinline__ void cm_pipeline() {
    __builtin_amdgcn_sched_group_barrier(0x100, LA, 0);  // DS reads
#pragma unroll
    for (int i = 0; i < n - LA; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, LA, 0);
}

}  // namespace

__global__ void cm_zero_kernel(int32_t *__restrict__ p, int64_t n) {
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < n; t += (int64_t)gridDim.x * blockDim.x)
        p[t] = 0;
}

// Row blocks: one block takes CM_RB consecutive rows of one (b, g) and
// counts their selections in an LDS histogram over the C chunks, so global
// atomics are one per (block, chunk) instead of one per selection.
constexpr int CM_RB = 1024;

// Rows of block (bg, x) inside the slab and below N: [i0, i0 + nr).
__device__ __forceinline__ int cm_block_rows(int N, int s0, int NS, int r0) {
    return max(0, min(min(CM_RB, NS - r0), N - s0 - r0));
}

__global__ __launch_bounds__(256) void cm_count_kernel(const int32_t *__restrict__ sel_idx, int32_t *__restrict__ cnt,
                                                       int N, int K, int C, int S, int W, int s0, int NS, int q0) {
    extern __shared__ int hist[];  // [C]
    const int64_t bg = blockIdx.y;
    const int r0 = blockIdx.x * CM_RB, nr = cm_block_rows(N, s0, NS, r0);
    for (int c = threadIdx.x; c < C; c += blockDim.x) hist[c] = 0;
    __syncthreads();
    const int32_t *base = sel_idx + (bg * N + s0 + r0) * K;
    for (int e = threadIdx.x; e < nr * K; e += blockDim.x) {
        const int i = s0 + r0 + e / K;
        const int c = base[e];
        if (c >= 0 && c < max(0, (q0 + i) / S - W / S)) atomicAdd(&hist[c], 1);
    }
    __syncthreads();
    for (int c = threadIdx.x; c < C; c += blockDim.x)
        if (hist[c]) atomicAdd(&cnt[bg * C + c], hist[c]);
}

// m^ of every (b, h, row) of the slab: the largest selected score, in log2
// units.  16 lanes per row, reading its K scores 16 at a time.
__global__ __launch_bounds__(256) void cm_rowmax_kernel(const int32_t *__restrict__ sel_idx,
                                                        const float *__restrict__ sel_score,
                                                        float *__restrict__ mhat, int N, int H_q, int H_kv, int G,
                                                        int K, int s0, int NS, int64_t npairs) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t pair = t >> 4;
    const int j = (int)(t & 15);
    float mh = -INFINITY;
    int64_t hr = 0;
    int il = 0;
    bool ok = false;
    if (pair < npairs) {
        hr = pair / NS;
        il = (int)(pair % NS);
        const int i = s0 + il;
        ok = i < N;
        if (ok) {
            const int h = (int)(hr % H_q);
            const int64_t b = hr / H_q;
            const float *sc = sel_score + (hr * N + i) * K;
            const int32_t *sl = sel_idx + ((b * H_kv + h / G) * N + i) * K;
            for (int kk = j; kk < K; kk += 16)
                if (sl[kk] >= 0) mh = fmaxf(mh, sc[kk] * LOG2E);
        }
    }
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) mh = fmaxf(mh, __shfl_xor(mh, o, 16));
    if (ok && j == 0) mhat[hr * NS + il] = mh;
}

typedef int32_t cm_i32x4 __attribute__((ext_vector_type(4)));

// The same with 16-byte reads (K % 4 == 0, 16-byte aligned sel_idx and
// sel_score): 4 lanes per row, each reading 4 slots at a time.
__global__ __launch_bounds__(256) void cm_rowmax4_kernel(const int32_t *__restrict__ sel_idx,
                                                         const float *__restrict__ sel_score,
                                                         float *__restrict__ mhat, int N, int H_q, int H_kv, int G,
                                                         int K, int s0, int NS, int64_t npairs) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t pair = t >> 2;
    const int j = (int)(t & 3);
    float mh = -INFINITY;
    int64_t hr = 0;
    int il = 0;
    bool ok = false;
    if (pair < npairs) {
        hr = pair / NS;
        il = (int)(pair % NS);
        const int i = s0 + il;
        ok = i < N;
        if (ok) {
            const int h = (int)(hr % H_q);
            const int64_t b = hr / H_q;
            const f32x4 *sc = (const f32x4 *)(sel_score + (hr * N + i) * K);
            const cm_i32x4 *sl = (const cm_i32x4 *)(sel_idx + ((b * H_kv + h / G) * N + i) * K);
            for (int kq = j; kq < K / 4; kq += 4) {
                const f32x4 v = sc[kq];
                const cm_i32x4 c = sl[kq];
#pragma unroll
                for (int x = 0; x < 4; ++x)
                    if (c[x] >= 0) mh = fmaxf(mh, v[x] * LOG2E);
            }
        }
    }
    mh = fmaxf(mh, __shfl_xor(mh, 2, 4));
    mh = fmaxf(mh, __shfl_xor(mh, 1, 4));
    if (ok && j == 0) mhat[hr * NS + il] = mh;
}

// One block per (b, g): exclusive scans of the chunk counts (list offsets)
// and of their segment counts ceil(cnt / SEG).  off and segoff hold C + 1
// entries each; entry C is the total.
__global__ __launch_bounds__(CM_SCAN_THREADS) void cm_scan_kernel(const int32_t *__restrict__ cnt,
                                                                  int32_t *__restrict__ off,
                                                                  int32_t *__restrict__ segoff, int C, int SEG) {
    __shared__ int wa[CM_SCAN_THREADS / WAVE], ws[CM_SCAN_THREADS / WAVE];
    const int64_t bg = blockIdx.x;
    const int tid = threadIdx.x, lane = lane_id(), wave = tid / WAVE;
    const int per = (C + CM_SCAN_THREADS - 1) / CM_SCAN_THREADS;
    const int c0 = min(C, tid * per), c1 = min(C, c0 + per);
    const int32_t *cb = cnt + bg * C;
    int a = 0, sg = 0;
    for (int c = c0; c < c1; ++c) {
        a += cb[c];
        sg += (cb[c] + SEG - 1) / SEG;
    }
    int ia = a, is = sg;
#pragma unroll
    for (int o = 1; o < WAVE; o <<= 1) {
        const int ya = __shfl_up(ia, o, WAVE), ys = __shfl_up(is, o, WAVE);
        if (lane >= o) {
            ia += ya;
            is += ys;
        }
    }
    if (lane == WAVE - 1) {
        wa[wave] = ia;
        ws[wave] = is;
    }
    __syncthreads();
    int ba = 0, bs = 0, ta = 0, ts = 0;
    for (int x = 0; x < CM_SCAN_THREADS / WAVE; ++x) {
        if (x < wave) {
            ba += wa[x];
            bs += ws[x];
        }
        ta += wa[x];
        ts += ws[x];
    }
    int pa = ba + ia - a, ps = bs + is - sg;
    int32_t *ob = off + bg * (C + 1), *sb = segoff + bg * (C + 1);
    for (int c = c0; c < c1; ++c) {
        ob[c] = pa;
        sb[c] = ps;
        pa += cb[c];
        ps += (cb[c] + SEG - 1) / SEG;
    }
    if (tid == 0) {
        ob[C] = ta;
        sb[C] = ts;
    }
}

// Same row blocks as cm_count; each selection takes a place in its chunk's
// list.  The block reserves a range per chunk with one global atomic
// (counting cnt back down to zero), then ranks its own selections in LDS.
// Entry = (slab row << 8) | slot; beside it, wl holds the weights
// exp2(s^ - m^) of the entry's G heads (the row's chunk masses relative to
// its largest selected one), so the attention reads them with the entry.
__global__ __launch_bounds__(256) void cm_fill_kernel(const int32_t *__restrict__ sel_idx, int32_t *__restrict__ cnt,
                                                      const int32_t *__restrict__ off, int32_t *__restrict__ list,
                                                      float *__restrict__ wl, const float *__restrict__ sel_score,
                                                      const float *__restrict__ mhat, int N, int H_q, int H_kv,
                                                      int G, int K, int C, int S, int W, int s0, int NS,
                                                      int64_t lstride, int q0) {
    extern __shared__ int sh[];  // hist[C], then base[C]
    int *hist = sh, *basep = sh + C;
    const int64_t bg = blockIdx.y;
    const int r0 = blockIdx.x * CM_RB, nr = cm_block_rows(N, s0, NS, r0);
    for (int c = threadIdx.x; c < C; c += blockDim.x) hist[c] = 0;
    __syncthreads();
    const int32_t *base = sel_idx + (bg * N + s0 + r0) * K;
    for (int e = threadIdx.x; e < nr * K; e += blockDim.x) {
        const int i = s0 + r0 + e / K;
        const int c = base[e];
        if (c >= 0 && c < max(0, (q0 + i) / S - W / S)) atomicAdd(&hist[c], 1);
    }
    __syncthreads();
    const int32_t *ob = off + bg * (C + 1);
    for (int c = threadIdx.x; c < C; c += blockDim.x) {
        const int h = hist[c];
        basep[c] = h ? ob[c] + atomicSub(&cnt[bg * C + c], h) - h : 0;
        hist[c] = 0;
    }
    __syncthreads();
    int32_t *lb = list + bg * lstride;
    float *wb = wl + bg * lstride * G;
    const int64_t hr0 = (bg / H_kv) * H_q + (bg % H_kv) * G;  // first head of the group
    for (int e = threadIdx.x; e < nr * K; e += blockDim.x) {
        const int il = r0 + e / K, i = s0 + il, kk = e % K;
        const int c = base[e];
        if (c >= 0 && c < max(0, (q0 + i) / S - W / S)) {
            const int p = basep[c] + atomicAdd(&hist[c], 1);
            lb[p] = (il << 8) | kk;
            // the G weights of the entry, stored four at a time (16 bytes)
            for (int x0 = 0; x0 < G; x0 += 4) {
                float w4[4];
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    const int64_t hr = hr0 + min(x0 + x, G - 1);
                    w4[x] = exp2_hw(sel_score[(hr * N + i) * K + kk] * LOG2E - mhat[hr * NS + il]);
                }
                float *dst = wb + (int64_t)p * G + x0;
                if (G >= 4) *(f32x4 *)dst = f32x4{w4[0], w4[1], w4[2], w4[3]};
                else
                    for (int x = 0; x < G; ++x) dst[x] = w4[x];
            }
        }
    }
}

// q [B, H_q, N, D] copied once per call into per-query regions
// qt [B, H_kv, N, G D]: the G heads of a query side by side, ordered
// [k-step s][head][lane group][8] so that the Q K^T fragment load for k-step s
// reads 64 G contiguous bytes of each query of a tile (as the partial stores).
// One thread per 16-byte piece of qt.
__global__ __launch_bounds__(256) void cm_qt_kernel(const bf16 *__restrict__ q, bf16 *__restrict__ qt, int N,
                                                    int H_q, int H_kv, int G, int D, int64_t npieces) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= npieces) return;
    const int grp = (int)(t & 3);
    const int64_t r1 = t >> 2;
    const int e = (int)(r1 % G);
    const int64_t r2 = r1 / G;
    const int KS = D / 32;
    const int s = (int)(r2 % KS);
    const int64_t r3 = r2 / KS;  // (b * H_kv + g) * N + i
    const int i = (int)(r3 % N);
    const int64_t bg = r3 / N;
    const int64_t b = bg / H_kv, g = bg % H_kv;
    const bf16 *src = q + ((b * H_q + g * G + e) * N + i) * D + 32 * s + 8 * grp;
    *(u32x4 *)(qt + t * 8) = *(const u32x4 *)src;
}

// Per-tile operands gathered from global memory: the Q fragments of the
// tile's rows, and where the row's partial goes.
template <int KS>
struct CmTile {
    bf16x8 qf[KS];
    int64_t pent;   // element offset of the selection's partial region (the trash region for an empty row)
};

// Tiles per wave per segment.
constexpr int CM_TPW = 8;

template <int D, int S, int G, int NWAVE>
__global__ __launch_bounds__(NWAVE * 64) void cm_attend_kernel(
    const bf16 *__restrict__ qt, const bf16 *__restrict__ k, const f16 *__restrict__ vt,
    const int32_t *__restrict__ list, const float *__restrict__ wl, const int32_t *__restrict__ off,
    const int32_t *__restrict__ segoff, f16 *__restrict__ part, int N, int H_q, int H_kv, int CA, int C, int K,
    float scale_log2, int s0, int NS, int64_t lstride, int SEG, int per_xcd, int64_t trash, int Nk,
    const int32_t *__restrict__ bt, int max_pages) {
    constexpr int TE = 16 / G;      // entries (queries) per 16-row tile
    constexpr int KS = D / 32;      // k-steps of Q K^T
    constexpr int KT = S / 16;      // 16-key tiles of S^T
    constexpr int PS = S / 32;      // k-steps of V^T P^T
    constexpr int DT = D / 16;      // 16-dim tiles of O^T
    constexpr int NBK = D / 8;      // 16-byte blocks per K row
    constexpr int NBV = S / 8;      // 16-byte blocks per V^T row
    constexpr int NT = NWAVE * 64;
    __shared__ u32x4 kt_l[S][NBK];
    __shared__ u32x4 vt_l[D][NBV];

    const int64_t bg = blockIdx.y;
    // XCD-aware: consecutive segments (mostly of one chunk) on one XCD's L2
    const int x = (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8);
    const int32_t *sb = segoff + bg * (C + 1);
    if (x >= sb[C]) return;
    // chunk c: the largest with sb[c] <= x (chunks without entries have
    // sb[c] == sb[c + 1] and are passed over)
    int lo = 0, hi = C - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (sb[mid] <= x) lo = mid;
        else hi = mid - 1;
    }
    const int c = lo;
    const int32_t *ob = off + bg * (C + 1);
    const int e0 = ob[c] + (x - sb[c]) * SEG;
    const int e1 = min(ob[c + 1], e0 + SEG);
    const int g = (int)(bg % H_kv);
    const int64_t b = bg / H_kv;
    const int tid = threadIdx.x, wave = tid / WAVE, lane = lane_id(), grp = lane >> 4, r = lane & 15;
    const int e = r % G;
    const int64_t hr = b * H_q + g * G + e;  // row's (batch, head)

    // Every global load and store below is issued unconditionally (empty
    // rows read row 0 and write the trash region): the compiler then counts the
    // loads in flight exactly and waits only for the ones a step needs.
    // ---- the list entries of this wave's tiles (tile wave + NWAVE u), all
    // loaded at once so that no Q gather waits on its entry's load
    int ent[CM_TPW + 2];
    float wt[CM_TPW + 2];  // the row's weight exp2(s^ - m^) for this slot
#pragma unroll
    for (int u = 0; u < CM_TPW; ++u) {
        const int ei = e0 + (wave + NWAVE * u) * TE + r / G;
        const int64_t ec = bg * lstride + min(ei, e1 - 1);
        const int en = list[ec];
        const float w = wl[ec * G + e];
        ent[u] = ei < e1 ? en : -1;
        wt[u] = w;
    }
    ent[CM_TPW] = ent[CM_TPW + 1] = -1;
    wt[CM_TPW] = wt[CM_TPW + 1] = 0.f;
    auto gather = [&](int u, CmTile<KS> &tl) {
        const int en = ent[u];
        const int il = en >= 0 ? en >> 8 : 0, kk = en >= 0 ? en & 255 : 0;
        // the query's region of qt: piece (s, e, grp) at 32 (G s + e) + 8 grp
        const bf16 *qr = qt + (bg * N + s0 + il) * (int64_t)G * D + 32 * e + 8 * grp;
#pragma unroll
        for (int s = 0; s < KS; ++s) tl.qf[s] = *(const bf16x8 *)(qr + 32 * G * s);
        tl.pent = (en >= 0 ? (bg * NS + il) * K + kk : trash) * G * D;
    };
    const int nu = ((e1 - e0 + TE - 1) / TE - wave + NWAVE - 1) / NWAVE;  // this wave's tiles

    // ---- stage the chunk: K rows (bf16) and its V^T copy (fp16, slot
    // order); every piece is loaded before any is written to LDS
    constexpr int NPK = (S * NBK + NT - 1) / NT, NPV = (D * NBV + NT - 1) / NT;
    u32x4 kst[NPK], vst[NPV];
    {
        // chunk c of k [B, H_kv, Nk, D], or page bt[b, c] of a paged cache [P, H_kv, S, D]
        const u32x4 *ks = (const u32x4 *)(bt ? k + ((int64_t)bt[b * max_pages + c] * H_kv + g) * S * D
                                             : k + (bg * Nk + (int64_t)c * S) * D);
        const u32x4 *vs = (const u32x4 *)(vt + (bg * CA + c) * (int64_t)D * S);
#pragma unroll
        for (int p = 0; p < NPK; ++p) kst[p] = ks[min(tid + p * NT, S * NBK - 1)];
#pragma unroll
        for (int p = 0; p < NPV; ++p) vst[p] = vs[min(tid + p * NT, D * NBV - 1)];
    }
    CmTile<KS> ta, tb;
    gather(0, ta);
    gather(1, tb);
#pragma unroll
    for (int p = 0; p < NPK; ++p) {
        const int t = tid + p * NT, row = t / NBK, blk = t % NBK;
        if (t < S * NBK) kt_l[row][blk ^ cm_swz<NBK>(row)] = kst[p];
    }
#pragma unroll
    for (int p = 0; p < NPV; ++p) {
        const int t = tid + p * NT, row = t / NBV, blk = t % NBV;
        if (t < D * NBV) vt_l[row][blk ^ cm_swz<NBV>(row)] = vst[p];
    }
    __syncthreads();

    auto compute = [&](const CmTile<KS> &cur, float w) {
        // S^T = K Q^T: acc[kt][i] = q_row . k_{16 kt + 4 grp + i}
        f32x4 acc[KT];
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) acc[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
            for (int kt = 0; kt < KT; ++kt) {
                const int row = 16 * kt + r;
                const u32x4 raw = kt_l[row][(4 * s + grp) ^ cm_swz<NBK>(row)];
                bf16x8 a;
                __builtin_memcpy(&a, &raw, 16);
                acc[kt] = mfma16(a, cur.qf[s], acc[kt]);
            }
        cm_pipeline<KS * KT, 4>();
        __builtin_amdgcn_sched_barrier(0);
        // exact softmax over the chunk's S keys, per row (lane column)
        float cmax = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i) cmax = fmaxf(cmax, acc[kt][i]);
        cmax = rows4_max(cmax) * scale_log2;
        float lc = 0.f;
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                acc[kt][i] = exp2_hw(fmaf(acc[kt][i], scale_log2, -cmax));
                lc += acc[kt][i];
            }
        lc = rows4_sum(lc);  // >= 1: the largest key contributes 2^0
        // O^T = V^T P^T, P^T packed from the S^T accumulators (fp16 in [0, 1])
        f16x8 bp[PS];
#pragma unroll
        for (int ps = 0; ps < PS; ++ps)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                bp[ps][i] = (f16)acc[2 * ps][i];
                bp[ps][4 + i] = (f16)acc[2 * ps + 1][i];
            }
        f32x4 O[DT];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) O[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ps = 0; ps < PS; ++ps)
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const int row = 16 * dt + r;
                const u32x4 raw = vt_l[row][(4 * ps + grp) ^ cm_swz<NBV>(row)];
                f16x8 a;
                __builtin_memcpy(&a, &raw, 16);
                O[dt] = mfma16h(a, bp[ps], O[dt]);
            }
        cm_pipeline<PS * DT, 4>();
        __builtin_amdgcn_sched_barrier(0);
        // weighted partial, fp16: lane (r, grp) holds dims 16 dt + 4 grp + i
        // of its row (head e).  A selection's G heads share one region of
        // G d values, ordered [piece j][head][grp][8]: piece j holds the dims
        // of dt = 2j, 2j + 1, so store j writes 64 G contiguous bytes (two
        // full cache lines at G = 4) of each selection of the tile
        {
            const float f = w * __builtin_amdgcn_rcpf(lc);
            f16 *pr = part + cur.pent + 32 * e + 8 * grp;
#pragma unroll
            for (int j = 0; j < DT / 2; ++j) {
                f16x8 y;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    y[i] = (f16)(O[2 * j][i] * f);
                    y[4 + i] = (f16)(O[2 * j + 1][i] * f);
                }
                *(f16x8 *)(pr + 32 * G * j) = y;
            }
        }
    };
    // two tile buffers in turn: a buffer is refilled right after its tile's
    // products have read it, so each gather has a whole tile of slack
    // (with an odd count the last round's second tile is an empty one)
    // (unrolled: the entry index stays a compile-time register index)
#pragma unroll
    for (int u = 0; u < CM_TPW; u += 2) {
        if (u >= nu) break;
        compute(ta, wt[u]);
        gather(u + 2, ta);
        compute(tb, wt[u + 1]);
        gather(u + 3 < CM_TPW + 2 ? u + 3 : CM_TPW + 1, tb);
    }
}

// ---------------------------------------------------------------- launch

namespace {

constexpr size_t CM_PART_CAP = (size_t)32 << 30;  // partial buffer bound (bytes)

struct CmLayout {
    int NS;               // slab rows (multiple of S)
    int SEG;              // entries per cm_attend block
    size_t qt, cnt, off, segoff, mhat, list, wl, part, total;  // byte offsets after the V^T copy
};

template <int G>
constexpr int cm_seg() {
    return 8 * CM_TPW * (16 / G);  // 8 waves x CM_TPW tiles of 16/G entries
}

CmLayout cm_layout(const Shape &s) {
    CmLayout L{};
    const int64_t per_row = (int64_t)s.B * s.H_q * s.K * s.D * 2;  // partial bytes per slab row
    int64_t ns = ((int64_t)s.N + s.S - 1) / s.S * s.S;
    if (s.attend_slab > 0) {
        ns = std::min<int64_t>(ns, ((int64_t)s.attend_slab + s.S - 1) / s.S * s.S);
    } else if (per_row > 0 && (size_t)(ns * per_row) > CM_PART_CAP) {
        ns = std::max<int64_t>(s.S, (int64_t)(CM_PART_CAP / per_row) / s.S * s.S);
    }
    L.NS = (int)std::max<int64_t>(ns, s.S);
    switch (s.G) {
        case 1: L.SEG = cm_seg<1>(); break;
        case 2: L.SEG = cm_seg<2>(); break;
        case 4: L.SEG = cm_seg<4>(); break;
        default: L.SEG = cm_seg<8>(); break;
    }
    const size_t bg = (size_t)s.B * s.H_kv;
    size_t o = 0;
    L.qt = o;  // q regrouped per query (all rows of the call)
    o = align_up(o + (size_t)s.B * s.H_q * s.N * s.D * 2, 256);
    L.cnt = o;
    o = align_up(o + bg * s.C * 4, 256);
    L.off = o;
    o = align_up(o + bg * (s.C + 1) * 4, 256);
    L.segoff = o;
    o = align_up(o + bg * (s.C + 1) * 4, 256);
    L.mhat = o;
    o = align_up(o + (size_t)s.B * s.H_q * L.NS * 4, 256);
    L.list = o;
    o = align_up(o + bg * (size_t)L.NS * s.K * 4, 256);
    L.wl = o;
    o = align_up(o + bg * (size_t)L.NS * s.K * s.G * 4, 256);
    L.part = o;  // one region past the partials: the trash region of empty tile rows
    o = align_up(o + ((size_t)s.B * s.H_kv * L.NS * s.K + 1) * s.G * s.D * 2, 256);
    L.total = o;
    return L;
}

template <int D, int S, int G>
hipError_t go_cm_attend(const Shape &s, const CmLayout &L, const void *q, const void *k, const f16 *vt,
                        const int32_t *list, const float *wl, const int32_t *off, const int32_t *segoff, f16 *part,
                        int s0, hipStream_t st) {
    constexpr int NWAVE = 8;
    const int rows = std::min(L.NS, s.N - s0);
    // segments per (b, g) are at most ceil(entries / SEG) + C
    const int64_t bound = ((int64_t)rows * s.K + L.SEG - 1) / L.SEG + s.C;
    const int per_xcd = (int)((bound + 7) / 8);
    const dim3 grid((unsigned)(8 * per_xcd), (unsigned)(s.B * s.H_kv)), block(NWAVE * 64);
    hipLaunchKernelGGL((cm_attend_kernel<D, S, G, NWAVE>), grid, block, 0, st, (const bf16 *)q, (const bf16 *)k, vt,
                       list, wl, off, segoff, part, s.N, s.H_q, s.H_kv, s.CA, s.C, s.K, s.scale * LOG2E, s0, L.NS,
                       (int64_t)L.NS * s.K, L.SEG, per_xcd, (int64_t)s.B * s.H_kv * L.NS * s.K, s.Nk, s.bt,
                       s.max_pages);
    return hipGetLastError();
}

template <int D, int S>
hipError_t cm_attend_g(const Shape &s, const CmLayout &L, const void *q, const void *k, const f16 *vt,
                       const int32_t *list, const float *wl, const int32_t *off, const int32_t *segoff, f16 *part,
                       int s0, hipStream_t st) {
    switch (s.G) {
        case 1: return go_cm_attend<D, S, 1>(s, L, q, k, vt, list, wl, off, segoff, part, s0, st);
        case 2: return go_cm_attend<D, S, 2>(s, L, q, k, vt, list, wl, off, segoff, part, s0, st);
        case 4: return go_cm_attend<D, S, 4>(s, L, q, k, vt, list, wl, off, segoff, part, s0, st);
        case 8: return go_cm_attend<D, S, 8>(s, L, q, k, vt, list, wl, off, segoff, part, s0, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool attend_use_cm(const Shape &s) {
    if (!s.io_bf16 || s.K == 0 || s.C == 0) return false;
    if (s.attend_mode == 1) return false;                 // the query-major walk
    if (!window_after_cm_supported(s)) return false;
    if (s.attend_mode == 2) return true;                  // chunk-major, asked for
    // auto: chunk-major wherever it runs.  Measured against the walk: 101-102
    // against 497 ms at 512K tokens (i.i.d. inputs, S = 128, K = 64: a
    // 32-query block's union is about 1100 chunks, so the walk stages each
    // 64 KB chunk for ~2 queries) and 23.2 against 25.2-25.5 ms at 128K
    // tokens (drifting inputs, S = 64, K = 32).
    (void)s;
    return true;
}

size_t cm_workspace_bytes(const Shape &s) { return cm_layout(s).total; }

int cm_slab_rows(const Shape &s) { return cm_layout(s).NS; }

hipError_t launch_sparse_attend_cm(const Shape &s, const void *q, const void *k, const void *v,
                                   const int32_t *sel_idx, const float *sel_score, void *out, float *lse,
                                   uint32_t *status, void *vt_ws, void *cm_ws, hipStream_t st) {
    f16 *vt = (f16 *)vt_ws;
    hipError_t e = launch_vt_prepass(s, v, vt, status, st);
    if (e != hipSuccess) return e;
    const CmLayout L = cm_layout(s);
    char *base = (char *)cm_ws;
    int32_t *cnt = (int32_t *)(base + L.cnt);
    int32_t *off = (int32_t *)(base + L.off);
    int32_t *segoff = (int32_t *)(base + L.segoff);
    float *mhat = (float *)(base + L.mhat);
    bf16 *qt = (bf16 *)(base + L.qt);
    int32_t *list = (int32_t *)(base + L.list);
    float *wl = (float *)(base + L.wl);
    f16 *part = (f16 *)(base + L.part);
    const int64_t ncnt = (int64_t)s.B * s.H_kv * s.C;
    {
        const int64_t npieces = (int64_t)s.B * s.H_q * s.N * (s.D / 8);
        hipLaunchKernelGGL(cm_qt_kernel, dim3((unsigned)((npieces + 255) / 256)), dim3(256), 0, st, (const bf16 *)q, qt,
                           s.N, s.H_q, s.H_kv, s.G, s.D, npieces);
    }
    // the histogram kernels' LDS: up to 2 x 8192 chunk counters
    hipFuncSetAttribute((const void *)cm_count_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, s.C * 4);
    hipFuncSetAttribute((const void *)cm_fill_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, s.C * 8);
    for (int s0 = 0; s0 < s.N; s0 += L.NS) {
        hipLaunchKernelGGL(cm_zero_kernel, dim3((unsigned)std::min<int64_t>(1024, (ncnt + 255) / 256)), dim3(256), 0,
                           st, cnt, ncnt);
        // row blocks of CM_RB rows per (b, g); LDS histograms over the C chunks
        const dim3 bgrid((unsigned)((L.NS + CM_RB - 1) / CM_RB), (unsigned)(s.B * s.H_kv));
        hipLaunchKernelGGL(cm_count_kernel, bgrid, dim3(256), (size_t)s.C * 4, st, sel_idx, cnt, s.N, s.K, s.C, s.S,
                           s.W, s0, L.NS, s.q0);
        const int64_t npairs = (int64_t)s.B * s.H_q * L.NS;
        if (s.K % 4 == 0 && (((uintptr_t)sel_idx | (uintptr_t)sel_score) & 15) == 0)
            hipLaunchKernelGGL(cm_rowmax4_kernel, dim3((unsigned)((npairs * 4 + 255) / 256)), dim3(256), 0, st,
                               sel_idx, sel_score, mhat, s.N, s.H_q, s.H_kv, s.G, s.K, s0, L.NS, npairs);
        else
            hipLaunchKernelGGL(cm_rowmax_kernel, dim3((unsigned)((npairs * 16 + 255) / 256)), dim3(256), 0, st,
                               sel_idx, sel_score, mhat, s.N, s.H_q, s.H_kv, s.G, s.K, s0, L.NS, npairs);
        hipLaunchKernelGGL(cm_scan_kernel, dim3((unsigned)(s.B * s.H_kv)), dim3(CM_SCAN_THREADS), 0, st, cnt, off,
                           segoff, s.C, L.SEG);
        hipLaunchKernelGGL(cm_fill_kernel, bgrid, dim3(256), (size_t)s.C * 8, st, sel_idx, cnt, off, list, wl,
                           sel_score, mhat, s.N, s.H_q, s.H_kv, s.G, s.K, s.C, s.S, s.W, s0, L.NS,
                           (int64_t)L.NS * s.K, s.q0);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if (s.D == 64 && s.S == 64) e = cm_attend_g<64, 64>(s, L, qt, k, vt, list, wl, off, segoff, part, s0, st);
        else if (s.D == 64) e = cm_attend_g<64, 128>(s, L, qt, k, vt, list, wl, off, segoff, part, s0, st);
        else if (s.S == 64) e = cm_attend_g<128, 64>(s, L, qt, k, vt, list, wl, off, segoff, part, s0, st);
        else e = cm_attend_g<128, 128>(s, L, qt, k, vt, list, wl, off, segoff, part, s0, st);
        if (e != hipSuccess) return e;
        e = launch_window_after_cm(s, q, k, vt, sel_idx, sel_score, out, lse, status, part, s0, L.NS, st);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace hils
