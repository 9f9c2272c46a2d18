// dense.hip -- dense causal attention, the full-attention point of
// comparison.
//
// The pages quote HiLS's prefill and decode speed as multiples of full
// attention at a 512K context (wmrh.cn article "HiLS-Attention 腾讯开源稀疏
// 注意力…", results table; hyper.ai HiLS summary, experiments paragraph on
// inference efficiency).  This file computes that baseline on the same chip:
//   out_i = sum_{j <= i} softmax_j(scale q_i . k_j) v_j
//   lse_i = log sum_{j <= i} exp(scale q_i . k_j)
// for every query head h over kv head h / G (hyper.ai summary, 方法: the
// naive block-sparse paragraph's attention with every key kept).
//
// MI355X design (bf16 in and out, fp32 accumulation):
//   * A block is 8 waves x two 16-row MFMA tiles = 256 rows: QB = 256 / G
//     consecutive queries x the G heads of one kv group.  Each 64-key tile
//     of K and V staged in LDS serves all 256 rows; a wave owns 32
//     consecutive queries of one head, so every LDS fragment it reads feeds
//     two MFMAs (one per tile).
//   * Transposed products, as in the fused sparse kernel: S^T = K Q^T (A = K
//     tile from LDS, B = Q^T in registers) and O^T += V^T P^T (A = fp16 V^T
//     from LDS, B = P^T packed from the S^T accumulators).  V^T comes from
//     the fused path's pre-pass (fp16, the keys of each 32-key step in the
//     order the accumulators hold them); P is rounded to fp16.
//   * Key tiles stream global -> LDS by buffer_load_lds (16 bytes per lane,
//     XOR swizzle through the source offset) through a ring of NSTAGE stages,
//     NSTAGE - 1 tiles ahead, with one block barrier per tile.  The tiles
//     below a wave's queries take no mask; its last tile (the one holding
//     its own positions) is masked per row.
//   * Online softmax in base 2 (log2 e folded into the scale); the rescale
//     of O is skipped when no row's maximum moved.
//   * Work is longest first: the causal work of a query block grows with
//     its position, so blocks are dispatched from the last query block down
//     (every (batch, group) pair of a query block side by side, which spreads
//     long and short blocks evenly over the XCDs), and the short blocks fill
//     the tail.
#include "hils_device.hpp"
#include <type_traits>

#include "hils_internal.hpp"

#define DENSE_LPTR(p) ((void __attribute__((address_space(3))) *)(p))

namespace hils {

namespace {

// raw buffer resource word 3: 32-bit dwords, no swizzle, no index stride
constexpr int DENSE_RSRC_WORD3 = 0x00020000;

// s_waitcnt immediate that waits for vmcnt <= n only
constexpr int dense_vmcnt(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }

// XOR swizzle of the 16-byte block index within an LDS row, so that the 16
// rows of one 128-bit read phase hit distinct bank groups: rows of 16 blocks
// use row & 15, rows of 8 blocks (two rows per 256 bytes) (row & 7) ^ bit 3.
template <int NB>
__device__ __forceinline__ int dswz(int row) {
    static_assert(NB == 8 || NB == 16, "rows of 8 or 16 blocks");
    return NB == 16 ? (row & 15) : ((row & 7) ^ ((row >> 3) & 1));
}

// Block barrier with no memory fence.  __syncthreads() releases every
// memory operation of the wave first, so the compiler would wait there for
// all tile loads in flight; here each wave waits for its own pieces of the
// tile in use (vmcnt) before the barrier, and the LDS reads of the previous
// tile have all returned (their MFMAs consumed them).  The memory clobber
// keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void dense_barrier() { asm volatile("s_barrier" ::: "memory"); }

#ifndef DENSE_NSTAGE
#define DENSE_NSTAGE 4  // ring stages (tiles in flight + the one in use)
#endif
#ifndef DENSE_LA
#define DENSE_LA 4  // LDS fragment reads issued ahead of their MFMAs
#endif

template <int D, int G>
struct DenseCfg {
    static constexpr int KB = 64;                     // keys per tile (one V^T pre-pass chunk)
    static constexpr int NWAVE = 8, TPW = 2;          // waves per block, 16-row tiles per wave
    static constexpr int QB = NWAVE * TPW * 16 / G;   // queries per block
    static constexpr int WPH = QB / 32;               // waves per head (32 queries each)
    static constexpr int KS = D / 32, KT = KB / 16, PS = KB / 32, DT = D / 16;
    static constexpr int NBK = D / 8, NBV = KB / 8;   // 16-byte blocks per K row, per V^T row
    static constexpr int PK = KB * D * 2 / 1024, PV = D * KB * 2 / 1024, NP = PK + PV;  // 1 KB pieces
    static constexpr int PPW = NP / NWAVE;            // pieces per wave per tile
    static constexpr int NSTAGE = DENSE_NSTAGE;
    static_assert(QB % 32 == 0 && NP % NWAVE == 0, "block shape");
};

}  // namespace

template <int D, int G>
__global__ __launch_bounds__(512) void dense_attend_kernel(const bf16 *__restrict__ q, const bf16 *__restrict__ k,
                                                           const f16 *__restrict__ vt, bf16 *__restrict__ out,
                                                           float *__restrict__ lse, int N, int H_q, int H_kv, int CA,
                                                           float scale_log2, int nqb, int64_t n_items) {
    using Cf = DenseCfg<D, G>;
    constexpr int KB = Cf::KB, TPW = Cf::TPW, NWAVE = Cf::NWAVE, QB = Cf::QB, WPH = Cf::WPH;
    constexpr int KS = Cf::KS, KT = Cf::KT, PS = Cf::PS, DT = Cf::DT, NBK = Cf::NBK, NBV = Cf::NBV;
    constexpr int PK = Cf::PK, PPW = Cf::PPW, NSTAGE = Cf::NSTAGE;
    // ring stage: the K tile [KB][NBK], then the V^T tile [D][NBV]
    __shared__ u32x4 ring[NSTAGE][KB * NBK + D * NBV];

    // ---- work item: in dispatch order the query blocks go from the last
    // (longest) down, the (batch, group) pairs of one query block side by
    // side.  Blocks reach the XCDs round robin, so every XCD gets the same
    // mix of long and short blocks, and with 8 or fewer pairs (or a multiple
    // of 8) each XCD keeps to fixed pairs, whose K/V its L2 serves.
    const int64_t item = blockIdx.x;
    if (item >= n_items) return;
    const int64_t nbg = n_items / nqb;
    const int qb = nqb - 1 - (int)(item / nbg);
    const int64_t bg = item % nbg;
    const int g = (int)(bg % H_kv);
    const int64_t b = bg / H_kv;
    const int i0 = qb * QB;
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid / WAVE), lane = lane_id();
    const int grp = lane >> 4, r = lane & 15;
    const int h = g * G + wave / WPH;          // the wave's head
    const int qw = i0 + 32 * (wave % WPH);     // the wave's first query
    // key tiles the block stages, and the wave's last one (its queries qw ..
    // qw + 31 lie in one 64-key span); a wave past the end computes none
    const int T = (min(N, i0 + QB) - 1) / KB + 1;
    const int wlast = qw < N ? qw / KB : -1;

    // Q^T fragments (B operand): lane (r, grp) holds dims 32 s + 8 grp .. +7
    // of query qw + 16 t + r
    bf16x8 qf[TPW][KS];
    const bf16 *qh = q + (b * H_q + h) * (int64_t)N * D;
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
        const bf16 *qr = qh + (int64_t)min(qw + 16 * t + r, N - 1) * D;
#pragma unroll
        for (int s = 0; s < KS; ++s) qf[t][s] = *(const bf16x8 *)(qr + 32 * s + 8 * grp);
    }
    // the fragments are in registers before any tile load is issued: the
    // walk's only vector-memory operations are then the tile loads, whose
    // counts the walk waits on itself
    __builtin_amdgcn_s_waitcnt(dense_vmcnt(0));
    f32x4 O[TPW][DT];
    float mrun[TPW], lrun[TPW];
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) O[t][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
        mrun[t] = -INFINITY;
        lrun[t] = 0.f;
    }

    // ---- DMA of key tile kc into stage buf: PPW pieces of 1 KB per wave.
    // The K resource ends at key N (rows past it read as zeros and are
    // masked); the V^T pre-pass holds zeros past key N.
    const bf16 *kbase = k + bg * (int64_t)N * D;
    const f16 *vbase = vt + bg * (int64_t)CA * D * KB;
    auto issue = [&](int kc, int buf) __attribute__((always_inline)) {
        const int nk = min(KB, N - kc * KB);
        const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(kbase + (int64_t)kc * KB * D), (short)0, nk * D * 2, DENSE_RSRC_WORD3);
        const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(vbase + (int64_t)kc * D * KB), (short)0, D * KB * 2, DENSE_RSRC_WORD3);
#pragma unroll
        for (int x = 0; x < PPW; ++x) {
            const int pc = wave + x * NWAVE;  // piece 0 .. NP - 1
            if (pc < PK) {
                constexpr int RPP = 1024 / (D * 2);  // K rows per piece
                const int row = pc * RPP + lane / NBK, blk = lane % NBK;
                const int off = (row * D + (blk ^ dswz<NBK>(row)) * 8) * 2;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, DENSE_LPTR(&ring[buf][pc * 64]), 16, off, 0, 0, 0);
            } else {
                constexpr int RPP = 1024 / (KB * 2);  // V^T rows per piece
                const int pv = pc - PK;
                const int row = pv * RPP + lane / NBV, blk = lane % NBV;
                const int off = (row * KB + (blk ^ dswz<NBV>(row)) * 8) * 2;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, DENSE_LPTR(&ring[buf][KB * NBK + pv * 64]), 16, off, 0,
                                                         0, 0);
            }
        }
    };
    // Software pipeline of n LDS fragment reads, each feeding TPW MFMAs:
    // LA reads ahead, then TPW MFMAs per further read.
    auto pipeline = [&](auto n_c, auto la_c) __attribute__((always_inline)) {
        constexpr int n = decltype(n_c)::value, LA = decltype(la_c)::value;
        __builtin_amdgcn_sched_group_barrier(0x100, LA, 0);  // DS reads
#pragma unroll
        for (int i = 0; i < n - LA; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, TPW, 0);  // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, TPW * LA, 0);
    };

    // ---- one key tile: S^T, online softmax, O^T += V^T P^T
    auto step = [&](auto diag_c, int buf, int kc) __attribute__((always_inline)) {
        constexpr bool DIAG = decltype(diag_c)::value;
        const u32x4(*kl)[NBK] = reinterpret_cast<const u32x4(*)[NBK]>(&ring[buf][0]);
        const u32x4(*vl)[NBV] = reinterpret_cast<const u32x4(*)[NBV]>(&ring[buf][KB * NBK]);
        // acc[t][kt][i] = q_(qw + 16 t + r) . k_(kc KB + 16 kt + 4 grp + i)
        f32x4 acc[TPW][KT];
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < TPW; ++t)
#pragma unroll
            for (int kt = 0; kt < KT; ++kt) acc[t][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
            for (int kt = 0; kt < KT; ++kt) {
                const int row = 16 * kt + r;
                const u32x4 raw = kl[row][(4 * s + grp) ^ dswz<NBK>(row)];
                bf16x8 a;
                __builtin_memcpy(&a, &raw, 16);
#pragma unroll
                for (int t = 0; t < TPW; ++t) acc[t][kt] = mfma16(a, qf[t][s], acc[t][kt]);
            }
        pipeline(std::integral_constant<int, KS * KT>{}, std::integral_constant<int, DENSE_LA>{});
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
            if constexpr (DIAG) {
                // keys after the row's own position are masked: lim is the last
                // visible key offset from the lane's first (16 kt + i)
                const int lim = qw + 16 * t + r - kc * KB - 4 * grp;
#pragma unroll
                for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[t][kt][i] = 16 * kt + i > lim ? -INFINITY : acc[t][kt][i];
            }
            float cmax = -INFINITY;
#pragma unroll
            for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                for (int i = 0; i < 4; ++i) cmax = fmaxf(cmax, acc[t][kt][i]);
            // every row sees key kc * KB (its position is at least that), so
            // the maximum is finite
            const float mnew = fmaxf(mrun[t], rows4_max(cmax) * scale_log2);
            const float alpha = exp2_hw(mrun[t] - mnew);
            const bool rescale = __ballot(mnew > mrun[t]) != 0ull;
            float ls = 0.f;
#pragma unroll
            for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    acc[t][kt][i] = exp2_hw(fmaf(acc[t][kt][i], scale_log2, -mnew));
                    ls += acc[t][kt][i];
                }
            lrun[t] = fmaf(lrun[t], alpha, rows4_sum(ls));
            mrun[t] = mnew;
            // alpha = 1 exactly in every lane whose maximum held
            if (rescale) {
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) O[t][dt] *= alpha;
            }
        }
        // P^T in k-slot order: slots 8 grp .. +3 are keys 32 ps + 4 grp + i
        // (tile 2 ps), slots 8 grp + 4 .. +7 the same of tile 2 ps + 1
        f16x8 bp[TPW][PS];
#pragma unroll
        for (int t = 0; t < TPW; ++t)
#pragma unroll
            for (int ps = 0; ps < PS; ++ps)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    bp[t][ps][i] = (f16)acc[t][2 * ps][i];
                    bp[t][ps][4 + i] = (f16)acc[t][2 * ps + 1][i];
                }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ps = 0; ps < PS; ++ps)
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const int row = 16 * dt + r;
                const u32x4 raw = vl[row][(4 * ps + grp) ^ dswz<NBV>(row)];
                f16x8 a;
                __builtin_memcpy(&a, &raw, 16);
#pragma unroll
                for (int t = 0; t < TPW; ++t) O[t][dt] = mfma16h(a, bp[t][ps], O[t][dt]);
            }
        pipeline(std::integral_constant<int, PS * DT>{}, std::integral_constant<int, DENSE_LA>{});
        __builtin_amdgcn_sched_barrier(0);
    };

    // ---- walk the key tiles: NSTAGE - 1 in flight ahead of the one in use
    for (int j = 0; j < NSTAGE - 1 && j < T; ++j) issue(j, j);
    for (int it = 0; it < T; ++it) {
        // this wave's pieces of tile it have landed once at most the later
        // tiles' pieces are outstanding
        const int later = min(NSTAGE - 2, T - 1 - it);
        static_assert(NSTAGE <= 5, "the waits below cover up to 3 later tiles");
        if (later >= 3) __builtin_amdgcn_s_waitcnt(dense_vmcnt(3 * PPW));
        else if (later == 2) __builtin_amdgcn_s_waitcnt(dense_vmcnt(2 * PPW));
        else if (later == 1) __builtin_amdgcn_s_waitcnt(dense_vmcnt(PPW));
        else __builtin_amdgcn_s_waitcnt(dense_vmcnt(0));
        // every wave's pieces of tile it are in; every wave is done with tile
        // it - 1, whose stage the next issue refills
        dense_barrier();
        if (it + NSTAGE - 1 < T) issue(it + NSTAGE - 1, (it + NSTAGE - 1) % NSTAGE);
        if (it < wlast) step(std::false_type{}, it % NSTAGE, it);
        else if (it == wlast) step(std::true_type{}, it % NSTAGE, it);
    }

    // ---- epilogue: lane (r, grp) holds dims 16 dt + 4 grp + i of its row
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
        const int iq = qw + 16 * t + r;
        if (iq >= N) continue;
        const float inv = 1.f / lrun[t];
        bf16 *orow = out + ((b * H_q + h) * N + iq) * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            bf16x4 y;
#pragma unroll
            for (int i = 0; i < 4; ++i) y[i] = (bf16)(O[t][dt][i] * inv);
            *(bf16x4 *)(orow + 16 * dt + 4 * grp) = y;
        }
        if (lse && grp == 0) lse[(b * H_q + h) * N + iq] = (mrun[t] + log2f(lrun[t])) * LN2;
    }
}

// ---------------------------------------------------------------- launch

namespace {

constexpr int DENSE_KB = 64;

Shape dense_vt_shape(const Shape &s) {
    Shape t = s;
    t.S = DENSE_KB;
    t.C = s.N / DENSE_KB;
    t.CA = (s.N + DENSE_KB - 1) / DENSE_KB;
    t.q0 = 0;
    t.Nk = s.N;
    t.bt = nullptr;
    t.max_pages = 0;
    return t;
}

template <int D, int G>
hipError_t go_dense(const Shape &s, const void *q, const void *k, const f16 *vt, void *out, float *lse,
                    hipStream_t st) {
    constexpr int QB = DenseCfg<D, G>::QB;
    const int nqb = (s.N + QB - 1) / QB;
    const int64_t n_items = (int64_t)s.B * s.H_kv * nqb;
    const int CA = (s.N + DENSE_KB - 1) / DENSE_KB;
    hipLaunchKernelGGL((dense_attend_kernel<D, G>), dim3((unsigned)n_items), dim3(512), 0, st, (const bf16 *)q,
                       (const bf16 *)k, vt, (bf16 *)out, lse, s.N, s.H_q, s.H_kv, CA, s.scale * LOG2E, nqb,
                       n_items);
    return hipGetLastError();
}

template <int D>
hipError_t dense_g(const Shape &s, const void *q, const void *k, const f16 *vt, void *out, float *lse,
                   hipStream_t st) {
    switch (s.G) {
        case 1: return go_dense<D, 1>(s, q, k, vt, out, lse, st);
        case 2: return go_dense<D, 2>(s, q, k, vt, out, lse, st);
        case 4: return go_dense<D, 4>(s, q, k, vt, out, lse, st);
        case 8: return go_dense<D, 8>(s, q, k, vt, out, lse, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool dense_attend_supported(const Shape &s) {
    return s.io_bf16 && (s.D == 64 || s.D == 128) && (s.G == 1 || s.G == 2 || s.G == 4 || s.G == 8);
}

size_t dense_workspace_bytes(const Shape &s) {
    if (!dense_attend_supported(s)) return 0;
    const Shape t = dense_vt_shape(s);
    return FUSED_STATUS_BYTES + align_up((size_t)t.B * t.H_kv * t.CA * t.D * t.S * 2, 256);
}

hipError_t launch_dense_attend(const Shape &s, const void *q, const void *k, const void *v, void *out, float *lse,
                               void *workspace, hipStream_t st) {
    if ((int64_t)s.B * s.N == 0) return hipSuccess;
    uint32_t *status = (uint32_t *)workspace;
    f16 *vt = (f16 *)((char *)workspace + FUSED_STATUS_BYTES);
    hipError_t e = launch_vt_prepass(dense_vt_shape(s), v, vt, status, st);
    if (e != hipSuccess) return e;
    return s.D == 64 ? dense_g<64>(s, q, k, vt, out, lse, st) : dense_g<128>(s, q, k, vt, out, lse, st);
}

}  // namespace hils
