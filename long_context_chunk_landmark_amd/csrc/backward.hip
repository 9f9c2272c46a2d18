// backward.hip -- gradients of the fused HiLS attention forward.
//
// hyper.ai HiLS summary, section 方法: the fused output is a softmax over the
// window keys and the selected chunks' keys whose logits are s_ij for window
// keys and s_ij + s^_c - lse_c for the keys of chunk c (the hierarchical
// factorisation: intra-chunk softmax times the surrogate mass); s^_c =
// scale q.k'_c + b'_c with the landmark summary (k'_c, b'_c) of the chunk.
// The selection is held fixed.  With P_j the fused weight of key j, dO the
// output gradient, D = dO.o - dlse:
//   window key j:       ds_j = P_j (dO.v_j - D)      (D = dO.o - dlse, from the recomputed weights)
//   key j of chunk c:   ds_j = w_c p_cj (dO.v_j - dO.o_c),  w_c = e^{s^_c - L}
//   chunk score:        ds^_c = w_c (dO.o_c - D)
//   dv_j += P_j dO, dk_j += scale ds_j q, dq += scale (sum_j ds_j k_j + sum_c ds^_c k'_c)
//   dk'_c += scale ds^_c q, db'_c += ds^_c
// and through the summary (a_j = scale q'.k_j, p = softmax a):
//   da_j = p_j dk'.(k_j - k') - db' p_j (a_j - p.a)
//   dq' = scale sum_j da_j k_j, dk_j += p_j dk' + scale da_j q'.
//
// Two passes, deterministic (every sum has one owner; the only atomics
// are the order-free ORs of the selection bitmap):
//   rows   dq, and per selected slot ds^, the chunk's log-weight
//          m = s^ - L - lse_c and g = dO.o_c
//   keys   dk, dv of a chunk's keys from the window rows and the rows that
//          selected it, the chunk's dk', db' of its landmark heads, and then
//          the summary backward into dk and dq'.
// bf16 I/O runs them on MFMA (bwd_rows_mfma_kernel: a block per 32 queries
// walking the union of their selections through an LDS ring;
// bwd_selbits_kernel: a bitmap of each chunk's selecting rows;
// bwd_keys_mfma_kernel: a block per chunk, rows in tiles of 32 pairs), with
// P and dS entering their products as two bf16 terms each.  fp32 I/O runs
// the first, fp32 VALU kernels (bwd_rows_kernel, bwd_keys_kernel: selecting
// rows found by a binary search in each later row's ascending selection).
#include <type_traits>

#include "hils_device.hpp"
#include "hils_internal.hpp"

#define BWD_LPTR(p) ((void __attribute__((address_space(3))) *)(p))
// Word 3 of a raw buffer resource on CDNA: 32-bit data format (untyped
// dword loads), no swizzle, no index stride.
#define BWD_RSRC_WORD3 0x00020000

namespace hils {

// dot of an fp32 vector in LDS with a row of T in global memory (16-byte loads)
template <typename T, int D>
__device__ __forceinline__ float dot_row(const float *__restrict__ x, const T *__restrict__ row) {
    constexpr int E = 16 / sizeof(T);
    float acc = 0.f;
#pragma unroll 4
    for (int c = 0; c < D; c += E) {
        const Vec16<T> r = load16(row + c);
#pragma unroll
        for (int e = 0; e < E; ++e) acc = fmaf(x[c + e], r.get(e), acc);
    }
    return acc;
}

// One block per (b, kv head g, row i), one wave per query head of the
// group: the G heads share the row's window and selection, so each tile of
// S keys (and values) is staged in LDS once for all of them.  D = dO.o is
// formed in the same pass from the recomputed fp32 weights (D = sum_j P_j
// dO.v_j), not from the stored output, so the rounding of a bf16 output
// does not enter the gradients.  Every term of dq that carries D is split
// off: dq = scale (A - D' Bv) with A = sum_window P_j (dO.v_j) k_j +
// sum_c [sum_j w_c p_j (dO.v_j - g_c) k_j + w_c g_c k'_c] and Bv =
// sum_window P_j k_j + sum_c w_c k'_c, D' = D - dlse.
template <typename T, int D, int S, int G>
__global__ __launch_bounds__(64 * G) void bwd_rows_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v, const float *__restrict__ k_sum,
    const int32_t *__restrict__ sel_idx, const float *__restrict__ sel_score, const float *__restrict__ lse,
    const T *__restrict__ dout, const float *__restrict__ dlse, float *__restrict__ dq, float *__restrict__ dsel,
    float *__restrict__ mlog, float *__restrict__ gdo, float *__restrict__ dcoef, int N, int H_q, int H_kv,
    int H_lm, int C, int W, int K, float scale) {
    constexpr int E = 16 / sizeof(T);    // elements per 16-byte piece
    constexpr int RP = D + E;            // padded LDS row (one extra piece)
    constexpr int NU = S / WAVE;         // keys per lane in a tile
    constexpr int DPL = D / WAVE;        // dims per lane in the gathers
    constexpr int NT = 64 * G;
    __shared__ T k_t[S][RP];
    __shared__ T v_t[S][RP];
    __shared__ float q_l[G][D];
    __shared__ float do_l[G][D];
    __shared__ float ca_l[G][S];  // per-key coefficient of A
    __shared__ float cb_l[G][S];  // per-key coefficient of Bv
    const int e = threadIdx.x / WAVE, lane = lane_id(), t = threadIdx.x;
    const int64_t bgi = blockIdx.x;  // (b*H_kv + g)*N + i
    const int i = (int)(bgi % N);
    const int64_t bg = bgi / N;
    const int g = (int)(bg % H_kv);
    const int64_t b = bg / H_kv;
    const int h = g * G + e, l = h * H_lm / H_q;
    const int64_t row = (b * H_q + h) * N + i;
    const T *kb = k + bg * (int64_t)N * D;
    const T *vb = v + bg * (int64_t)N * D;
    for (int x = lane; x < D; x += WAVE) {
        q_l[e][x] = to_f32(q[row * D + x]);
        do_l[e][x] = to_f32(dout[row * D + x]);
    }
    const float L = lse[row];

    // stage keys / values j0 .. j0 + n - 1 (n <= S) in LDS
    auto stage = [&](int64_t j0, int n) {
        __syncthreads();  // the previous tile is no longer read
        for (int idx = t; idx < n * (D / E); idx += NT) {
            const int r = idx / (D / E), cpc = idx % (D / E);
            *(u32x4 *)&k_t[r][cpc * E] = *(const u32x4 *)(kb + (j0 + r) * D + cpc * E);
            *(u32x4 *)&v_t[r][cpc * E] = *(const u32x4 *)(vb + (j0 + r) * D + cpc * E);
        }
        __syncthreads();
    };
    // q.k_r and dO.v_r from the staged tile
    // (partly unrolled: the query and gradient rows stay in LDS, read as
    // broadcasts, instead of occupying 2 D registers per lane)
    auto dots = [&](int r, float &s, float &dpv) {
        float a = 0.f, c = 0.f;
#pragma unroll 2
        for (int x = 0; x < D; x += E) {
            const Vec16<T> kr = *(const Vec16<T> *)&k_t[r][x];
            const Vec16<T> vr = *(const Vec16<T> *)&v_t[r][x];
#pragma unroll
            for (int y = 0; y < E; y += 4) {
                const f32x4 qv = *(const f32x4 *)&q_l[e][x + y];
                const f32x4 dv = *(const f32x4 *)&do_l[e][x + y];
#pragma unroll
                for (int z = 0; z < 4; ++z) {
                    a = fmaf(qv[z], kr.get(y + z), a);
                    c = fmaf(dv[z], vr.get(y + z), c);
                }
            }
        }
        s = scale * a;
        dpv = c;
    };

    float accA[DPL], accB[DPL];
#pragma unroll
    for (int y = 0; y < DPL; ++y) accA[y] = accB[y] = 0.f;
    // accA += sum_r ca_r k_r, accB += sum_r cb_r k_r over the first n staged keys
    auto gather = [&](int n, bool with_b) {
        wave_sync();
#pragma unroll 4
        for (int r = 0; r < n; ++r) {
            const float ca = ca_l[e][r], cb = cb_l[e][r];
#pragma unroll
            for (int y = 0; y < DPL; ++y) {
                const float kx = to_f32(k_t[r][lane * DPL + y]);
                accA[y] = fmaf(ca, kx, accA[y]);
                if (with_b) accB[y] = fmaf(cb, kx, accB[y]);
            }
        }
        wave_sync();
    };

    // window [w0, i], in tiles of S keys: ds_j = P_j (dO.v_j - D')
    float dpart = 0.f;  // this lane's share of sum_window P_j dO.v_j
    const int w0 = max(0, (i / S) * S - W);
    for (int j0 = w0; j0 <= i; j0 += S) {
        const int n = min(S, i - j0 + 1);
        stage(j0, n);
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            const int r = u * WAVE + lane;
            float P = 0.f, dpv = 0.f;
            if (r < n) {
                float s;
                dots(r, s, dpv);
                P = expf(s - L);
            }
            dpart = fmaf(P, dpv, dpart);
            ca_l[e][r] = P * dpv;
            cb_l[e][r] = P;
        }
        gather(n, true);
    }

    // selected chunks (shared by the group's heads)
    const int32_t *sl = sel_idx + bgi * K;
    const float *ss = sel_score + row * K;
    float dsel_sum = 0.f;  // sum_c w_c g_c (wave-uniform)
    for (int kk = 0; kk < K; ++kk) {
        const int c = sl[kk];
        if (c < 0) {
            if (lane == 0) dsel[row * K + kk] = 0.f, mlog[row * K + kk] = -INFINITY, gdo[row * K + kk] = 0.f;
            continue;
        }
        stage((int64_t)c * S, S);
        float s[NU], dpv[NU];
        float m = -INFINITY;
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            dots(u * WAVE + lane, s[u], dpv[u]);
            m = fmaxf(m, s[u]);
        }
        m = wave_max(m);
        float z = 0.f;
#pragma unroll
        for (int u = 0; u < NU; ++u) z += expf(s[u] - m);
        const float lse_c = m + logf(wave_sum_f(z));
        float p[NU], gpart = 0.f;
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            p[u] = expf(s[u] - lse_c);
            gpart = fmaf(p[u], dpv[u], gpart);
        }
        const float gc = wave_sum_f(gpart);  // dO.o_c
        const float shat = ss[kk];
        const float wc = expf(shat - L);
        dsel_sum = fmaf(wc, gc, dsel_sum);
#pragma unroll
        for (int u = 0; u < NU; ++u) ca_l[e][u * WAVE + lane] = wc * p[u] * (dpv[u] - gc);
        gather(S, false);
        // score term: ds^_c k'_c = w_c (g_c - D') k'_c
        const float *kp = k_sum + (((int64_t)b * H_lm + l) * C + c) * D;
#pragma unroll
        for (int y = 0; y < DPL; ++y) {
            const float kx = kp[lane * DPL + y];
            accA[y] = fmaf(wc * gc, kx, accA[y]);
            accB[y] = fmaf(wc, kx, accB[y]);
        }
        if (lane == 0) {
            dsel[row * K + kk] = wc;  // w_c for now; ds^_c once D' is known
            mlog[row * K + kk] = shat - L - lse_c;
            gdo[row * K + kk] = gc;
        }
    }
    const float Dp = wave_sum_f(dpart) + dsel_sum - (dlse ? dlse[row] : 0.f);
#pragma unroll
    for (int y = 0; y < DPL; ++y) dq[row * D + lane * DPL + y] = scale * fmaf(-Dp, accB[y], accA[y]);
    if (lane == 0) {
        dcoef[row] = Dp;
        for (int kk = 0; kk < K; ++kk)
            if (sl[kk] >= 0) dsel[row * K + kk] = dsel[row * K + kk] * (gdo[row * K + kk] - Dp);
    }
}

// Block (chunk c, kv head g, batch b) of NT = 4 S threads: thread (jj, qd)
// owns key c*S + jj and dims [qd*DPT, qd*DPT + DPT) (DPT = D / 4), holding
// that slice of k, v and of the gradients in registers.  Rows are visited
// one at a time with the group's G query heads staged in LDS.
template <typename T, int D, int S>
__global__ __launch_bounds__(4 * S) void bwd_keys_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v, const T *__restrict__ q_lm,
    const int32_t *__restrict__ sel_idx, const float *__restrict__ lse, const T *__restrict__ dout,
    const float *__restrict__ dcoef, const float *__restrict__ dsel, const float *__restrict__ mlog,
    const float *__restrict__ gdo, float *__restrict__ dk, float *__restrict__ dv, float *__restrict__ dq_lm, int N,
    int H_q, int H_kv, int H_lm, int C, int W, int K, float scale, int lm_mode) {
    constexpr int NT = 4 * S, NQ = 4, DPT = D / NQ, NWV = NT / WAVE;
    constexpr int GMAX = 8;
    constexpr int RB = 4;  // rows staged per barrier round
    __shared__ float qs_l[RB][GMAX][D];
    __shared__ float do_l[RB][GMAX][D];
    __shared__ float sc_l[RB][GMAX][3];
    __shared__ int list_i[NT];
    __shared__ int list_k[NT];
    __shared__ int wcnt[NWV];
    __shared__ float red[S][D + 1];  // summary backward: per-key partial rows
    __shared__ float a_l[S], p_l[S], kd_l[S];
    __shared__ float dkp_l[GMAX][D];
    __shared__ float dbp_l[GMAX];

    const int c = blockIdx.x, g = blockIdx.y;
    const int64_t b = blockIdx.z;
    const int G = H_q / H_kv, GLM = H_lm / H_kv;
    const int t = threadIdx.x, jj = t / NQ, qd = t % NQ, x0 = qd * DPT;
    const int wave = t / WAVE, lane = lane_id();
    const int64_t j = (int64_t)c * S + jj;
    const bool valid_j = j < N;
    const int64_t kvrow = ((b * H_kv + g) * N + j) * D;

    float kr[DPT], vr[DPT], dka[DPT], dva[DPT];
#pragma unroll
    for (int x = 0; x < DPT; ++x) {
        kr[x] = valid_j ? to_f32(k[kvrow + x0 + x]) : 0.f;
        vr[x] = valid_j ? to_f32(v[kvrow + x0 + x]) : 0.f;
        dka[x] = dva[x] = 0.f;
    }
    // dk', db' of the chunk's landmark heads, accumulated in LDS by their
    // owner threads (key row jj == landmark index, each its dim slice)
    for (int idx = t; idx < GLM * D; idx += NT) dkp_l[idx / D][idx % D] = 0.f;
    if (t < GLM) dbp_l[t] = 0.f;
    auto quad_sum = [&](float a) {
        a += __shfl_xor(a, 1, WAVE);
        a += __shfl_xor(a, 2, WAVE);
        return a;
    };

    // up to RB query rows (all G heads each): window rows (selected =
    // false) or rows that selected chunk c, row_of(rr) -> (i, slot)
    auto process_rows = [&](int nr, bool selected, auto row_of) {
        __syncthreads();  // the previous rows are done with the staged heads
        for (int idx = t; idx < nr * G * D; idx += NT) {
            const int rr = idx / (G * D), rem = idx % (G * D), e = rem / D, x = rem % D;
            const int i = row_of(rr).x;
            const int64_t rh = ((b * H_q + (int64_t)g * G + e) * N + i);
            qs_l[rr][e][x] = to_f32(q[rh * D + x]);
            do_l[rr][e][x] = to_f32(dout[rh * D + x]);
        }
        if (t < nr * G) {
            const int rr = t / G, e = t % G;
            const int2 ik = row_of(rr);
            const int64_t rh = ((b * H_q + (int64_t)g * G + e) * N + ik.x);
            if (selected) {
                sc_l[rr][e][0] = mlog[rh * K + ik.y];  // log of w_c / e^{lse_c}: P_j = e^{s_j + m}
                sc_l[rr][e][1] = gdo[rh * K + ik.y];
                sc_l[rr][e][2] = dsel[rh * K + ik.y];
            } else {
                sc_l[rr][e][0] = -lse[rh];
                sc_l[rr][e][1] = dcoef[rh];
                sc_l[rr][e][2] = 0.f;
            }
        }
        __syncthreads();
#pragma unroll 1
        for (int rr = 0; rr < nr; ++rr) {
            const bool live = valid_j && (selected || j <= row_of(rr).x);
#pragma unroll 1
            for (int e = 0; e < G; ++e) {
                float ps = 0.f, pd = 0.f;
#pragma unroll
                for (int x = 0; x < DPT; ++x) {
                    ps = fmaf(qs_l[rr][e][x0 + x], kr[x], ps);
                    pd = fmaf(do_l[rr][e][x0 + x], vr[x], pd);
                }
                const float s = scale * quad_sum(ps), dpv = quad_sum(pd);
                const float P = live ? expf(s + sc_l[rr][e][0]) : 0.f;
                const float ds = P * (dpv - sc_l[rr][e][1]);
#pragma unroll
                for (int x = 0; x < DPT; ++x) {
                    dva[x] = fmaf(P, do_l[rr][e][x0 + x], dva[x]);
                    dka[x] = fmaf(scale * ds, qs_l[rr][e][x0 + x], dka[x]);
                }
                if (selected) {
                    // landmark head of query head e: its local index le gets
                    // the score gradient (thread rows jj == le hold dk' slices)
                    const int le = (g * G + e) * H_lm / H_q - g * GLM;
                    if (jj == le) {
                        const float dsh = sc_l[rr][e][2];
#pragma unroll
                        for (int x = 0; x < DPT; ++x)
                            dkp_l[le][x0 + x] = fmaf(scale * dsh, qs_l[rr][e][x0 + x], dkp_l[le][x0 + x]);
                        if (qd == 0) dbp_l[le] += dsh;
                    }
                }
            }
        }
    };

    const int wc = W / (S);
    // window rows: query chunks c .. c + W/S
    const int r_end = (int)min((int64_t)N, (int64_t)(c + wc + 1) * S);
    for (int i0 = c * S; i0 < r_end; i0 += RB)
        process_rows(min(RB, r_end - i0), false, [&](int rr) { return make_int2(i0 + rr, 0); });

    // rows of later query chunks that selected chunk c
    if (K > 0 && c < C) {
        for (int i0 = r_end; i0 < N; i0 += NT) {
            const int i = i0 + t;
            int found = -1;
            if (i < N) {
                const int32_t *sr = sel_idx + ((b * H_kv + g) * N + i) * K;
                int lo = 0, hi = K;  // entries ascending, -1 padding last
                while (lo < hi) {
                    const int mid = (lo + hi) >> 1;
                    const int x = sr[mid];
                    if (x >= 0 && x < c) lo = mid + 1;
                    else hi = mid;
                }
                if (lo < K && sr[lo] == c) found = lo;
            }
            const uint64_t m = __ballot(found >= 0);
            __syncthreads();  // the previous batch's list is consumed
            if (lane == 0) wcnt[wave] = __popcll(m);
            __syncthreads();
            int base = 0, tot = 0;
            for (int w = 0; w < NWV; ++w) {
                base += w < wave ? wcnt[w] : 0;
                tot += wcnt[w];
            }
            if (found >= 0) {
                const int pos = base + __popcll(m & lanemask_lt());
                list_i[pos] = i;
                list_k[pos] = found;
            }
            __syncthreads();
            for (int r0 = 0; r0 < tot; r0 += RB)
                process_rows(min(RB, tot - r0), true, [&](int rr) { return make_int2(list_i[r0 + rr], list_k[r0 + rr]); });
        }
    }

    // ---- summary backward of the chunk's landmark heads (completed chunks)
    if (c < C) {
        __syncthreads();  // dk', db' complete
        for (int e = 0; e < GLM; ++e) {
            const int lh = g * GLM + e;
            const int64_t lrow = ((b * H_lm + lh) * C + c) * D;
            float qp[DPT];
            // landmark query: per chunk, one shared by the chunks of head lh, or zero
            const int64_t qrow = lm_mode == 1 ? (int64_t)lh * D : lrow;
#pragma unroll
            for (int x = 0; x < DPT; ++x) qp[x] = lm_mode == 2 ? 0.f : to_f32(q_lm[qrow + x0 + x]);
            float pa = 0.f, pk = 0.f;
#pragma unroll
            for (int x = 0; x < DPT; ++x) {
                pa = fmaf(qp[x], kr[x], pa);
                pk = fmaf(dkp_l[e][x0 + x], kr[x], pk);
            }
            const float a = scale * quad_sum(pa), kdk = quad_sum(pk);  // a_j, dk'.k_j
            __syncthreads();  // previous head done with a_l / p_l / red
            if (qd == 0) a_l[jj] = a, kd_l[jj] = kdk;
            __syncthreads();
            float mx = -INFINITY;
            for (int r = 0; r < S; ++r) mx = fmaxf(mx, a_l[r]);
            float z = 0.f, za = 0.f, zk = 0.f;
            for (int r = 0; r < S; ++r) {
                const float ex = expf(a_l[r] - mx);
                z += ex;
                za = fmaf(ex, a_l[r], za);
                zk = fmaf(ex, kd_l[r], zk);
            }
            const float p = expf(a - mx) / z;
            const float abar = za / z, kpdk = zk / z;  // p.a, dk'.k'
            const float da = p * (kdk - kpdk) - dbp_l[e] * p * (a - abar);
#pragma unroll
            for (int x = 0; x < DPT; ++x) {
                dka[x] = fmaf(p, dkp_l[e][x0 + x], dka[x]);
                dka[x] = fmaf(scale * da, qp[x], dka[x]);
                red[jj][x0 + x] = da * kr[x];
            }
            __syncthreads();
            if (lm_mode != 2 && t < D) {
                float sum = 0.f;
                for (int r = 0; r < S; ++r) sum += red[r][t];
                dq_lm[lrow + t] = scale * sum;
            }
        }
    }

    if (valid_j) {
#pragma unroll
        for (int x = 0; x < DPT; ++x) {
            dk[kvrow + x0 + x] = dka[x];
            dv[kvrow + x0 + x] = dva[x];
        }
    }
}

typedef short v4i16 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- MFMA key pass (bf16 I/O)
//
// The key-side pass on the matrix cores.  Block (chunk c, kv head g, batch
// b) of S / 16 waves; wave w owns keys c*S + 16w .. +15 and keeps their K
// and V slices in registers as B operands, with dK^T and dV^T of those keys
// as fp32 accumulators (lane l: key 16w + l%16, dims 16dt + 4(l/16) + i).
// The rows that attend chunk c (the window rows, then the later rows that
// selected it) go in tiles of 32 (row, head) pairs staged in LDS, row-major
// (A operand of S = Q K^T and dP = dO V^T) and transposed (A operand of
// dK^T += Q^T dS and dV^T += dO^T P).  The accumulators of S for pairs 0-15
// and 16-31 hold, in lane group gq, pairs 4gq + i and 16 + 4gq + i of key
// l%16: as the B operand of the second products they are k-slots 8gq + i
// and 8gq + 4 + i, the order the transposed tiles are written in.  P and
// dS enter those products as two bf16 terms each (hi + lo, within 2^-16 of
// the fp32 value); q, k, v and dO are bf16 inputs, so every product is
// exact and the sums are fp32.

namespace {

// 16-byte block swizzle of an LDS row of NB blocks, by row, so the 16 rows
// of one MFMA operand read fall in distinct bank groups
template <int NB>
__device__ __forceinline__ int bswz(int row) {
    return NB == 16 ? (row & 15) : ((row & 7) ^ ((row >> 3) & 1));
}

}  // namespace

template <int D, int S, int G>
__global__ __launch_bounds__(4 * S) __attribute__((amdgpu_waves_per_eu(2))) void bwd_keys_mfma_kernel(
    const bf16 *__restrict__ q, const bf16 *__restrict__ k, const bf16 *__restrict__ v,
    const bf16 *__restrict__ q_lm, const int32_t *__restrict__ sel_idx, const uint64_t *__restrict__ selbits,
    const float *__restrict__ lse, const bf16 *__restrict__ dout, const float *__restrict__ dcoef,
    const float *__restrict__ dsel, const float *__restrict__ mlog, const float *__restrict__ gdo,
    float *__restrict__ dk, float *__restrict__ dv, float *__restrict__ dq_lm, int N, int H_q, int H_kv, int H_lm,
    int C, int W, int K, float scale, int lm_mode) {
    constexpr int NT = 4 * S;                     // one wave per 16 keys
    constexpr int BW = 16, LCAP = BW * 64 + 32;  // bitmap words per batch; row list capacity
    constexpr int KS = D / 32, DT = D / 16, NB = D / 8;
    constexpr int RT = 32, RPT = RT / G;  // pairs and rows per row tile
    constexpr int NQ = 4, DPT = D / NQ;   // summary backward: four threads per key
    __shared__ u32x4 q_t[RT][NB];         // tile rows of q (bf16, swizzled by pair)
    __shared__ u32x4 do_t[RT][NB];        // and of dO
    // per pair (16-byte aligned: a lane reads four consecutive pairs at once)
    __shared__ __attribute__((aligned(16))) float pbias[RT];  // log-weight (base 2) added to the scaled logit
    __shared__ __attribute__((aligned(16))) float pdc[RT];    // the term subtracted from dO.v (D' or dO.o_c)
    __shared__ __attribute__((aligned(16))) float pdsh[RT];   // ds^_c of a selecting pair (0 for window pairs)
    __shared__ __attribute__((aligned(16))) int prow[RT];     // last key the pair may see (its row; selected: all)
    __shared__ int list_i[LCAP];
    __shared__ int list_k[LCAP];
    __shared__ int nlist;
    __shared__ float red[S][D + 1];  // summary backward: per-key partial rows
    __shared__ float a_l[S], p_l[S], kd_l[S], da_l[S];
    __shared__ float dkp_l[G][D];
    __shared__ float dbp_l[G];
    __shared__ float qp_l[D];

    const int c = blockIdx.x, g = blockIdx.y;
    const int64_t b = blockIdx.z;
    const int GLM = H_lm / H_kv;
    const int t = threadIdx.x, wave = t / WAVE, lane = lane_id(), grp = lane >> 4, r16 = lane & 15;
    const int64_t kvb = (b * H_kv + g) * (int64_t)N;  // first key row of (b, g)
    const int keyl = 16 * wave + r16;                  // the lane's key within the chunk
    const int key = c * S + keyl;
    const bool key_ok = key < N;
    const float scale2 = scale * LOG2E;

    bf16x8 kf[KS], vf[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        u32x4 kr = {0u, 0u, 0u, 0u}, vr = {0u, 0u, 0u, 0u};
        if (key_ok) {
            kr = *(const u32x4 *)(k + (kvb + key) * D + 32 * s + 8 * grp);
            vr = *(const u32x4 *)(v + (kvb + key) * D + 32 * s + 8 * grp);
        }
        __builtin_memcpy(&kf[s], &kr, 16);
        __builtin_memcpy(&vf[s], &vr, 16);
    }
    f32x4 accK[DT], accV[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) accK[dt] = accV[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    // dk'^T of the chunk's landmark heads (dims x heads, head = MFMA column):
    // wave w accumulates the dim tiles dt = w, w + NWV, ...; db' as a sum
    constexpr int NWV = S / 16, KPN = (DT + NWV - 1) / NWV;
    f32x4 accKP[KPN];
#pragma unroll
    for (int j = 0; j < KPN; ++j) accKP[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    float dbacc = 0.f;

    // A tile: nrows rows x G heads; pair p is row p / G, head p % G;
    // row_of(rr) -> (row, selection slot).  fetch loads a tile's rows and
    // per-pair values into registers, commit stores them (and the
    // transposed rows) in LDS, compute runs the products; the next tile is
    // fetched while the current one computes.
    constexpr int NPT = (2 * RT * NB + NT - 1) / NT;  // 16-byte row pieces per thread
    u32x4 tv[NPT];
    float tbias = -INFINITY, tdc = 0.f, tdsh = 0.f;
    int tlim = -1;
    auto fetch = [&](int nrows, bool selected, auto row_of) __attribute__((always_inline)) {
        const int np = nrows * G;
#pragma unroll
        for (int j = 0; j < NPT; ++j) {
            const int idx = t + j * NT;
            const int which = idx / (RT * NB), rem = idx % (RT * NB), p = rem / NB, cb = rem % NB;
            tv[j] = u32x4{0u, 0u, 0u, 0u};
            if (idx < 2 * RT * NB && p < np) {
                const int64_t rh = (b * H_q + (int64_t)g * G + p % G) * N + row_of(p / G).x;
                tv[j] = *(const u32x4 *)((which ? dout : q) + rh * D + cb * 8);
            }
        }
        tbias = -INFINITY, tdc = 0.f, tdsh = 0.f, tlim = -1;
        if (t < np) {
            const int2 ik = row_of(t / G);
            const int64_t rh = (b * H_q + (int64_t)g * G + t % G) * N + ik.x;
            if (selected) {
                tbias = mlog[rh * K + ik.y] * LOG2E;  // P_j = e^{s_j + m}, m = s^_c - L - lse_c
                tdc = gdo[rh * K + ik.y];
                tdsh = dsel[rh * K + ik.y];
                tlim = 0x7fffffff;
            } else {
                tbias = -lse[rh] * LOG2E;
                tdc = dcoef[rh];
                tlim = ik.x;
            }
        }
    };
    auto commit = [&]() __attribute__((always_inline)) {
        __syncthreads();  // the previous tile is no longer read
#pragma unroll
        for (int j = 0; j < NPT; ++j) {
            const int idx = t + j * NT;
            const int which = idx / (RT * NB), rem = idx % (RT * NB), p = rem / NB, cb = rem % NB;
            if (idx < 2 * RT * NB) (which ? do_t : q_t)[p][cb ^ bswz<NB>(p)] = tv[j];
        }
        if (t < RT) {
            pbias[t] = tbias;
            pdc[t] = tdc;
            pdsh[t] = tdsh;
            prow[t] = tlim;
        }
        __syncthreads();
    };
    // The A operands Q^T and dO^T (dims 16 dt + l%16 x k-slots 8 grp .. +7)
    // read transposed from the row-major tiles: in each 16-lane group, the
    // transpose read gives lane i element i of the 16 values that lanes
    // 4r .. 4r+3 address; lane 4r + sub addresses 4 dims of pair row r.
    // Slots 8grp .. 8grp+3 are pairs 4grp + r, slots 8grp+4 .. +7 pairs
    // 16 + 4grp + r.
    const int tsub = r16 & 3, trow = r16 >> 2;
    auto t_frag = [&](const u32x4 (*src)[NB], int dt) __attribute__((always_inline)) {
        const int x0 = 16 * dt + 4 * tsub;
        bf16x8 a;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int p = 16 * h + 4 * grp + trow;
            const short *at = (const short *)&src[p][(x0 >> 3) ^ bswz<NB>(p)] + (x0 & 7);
            const v4i16 v4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16 *)at);
            __builtin_memcpy((char *)&a + 8 * h, &v4, 8);
        }
        return a;
    };
    auto compute = [&](bool selected) __attribute__((always_inline)) {
        f32x4 sacc[2], dacc[2];
#pragma unroll
        for (int rg = 0; rg < 2; ++rg) {
            sacc[rg] = dacc[rg] = f32x4{0.f, 0.f, 0.f, 0.f};
            const int pr = 16 * rg + r16;
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                const int blk = (4 * s + grp) ^ bswz<NB>(pr);
                bf16x8 qa, da;
                const u32x4 rq = q_t[pr][blk], rd = do_t[pr][blk];
                __builtin_memcpy(&qa, &rq, 16);
                __builtin_memcpy(&da, &rd, 16);
                sacc[rg] = mfma16(qa, kf[s], sacc[rg]);
                dacc[rg] = mfma16(da, vf[s], dacc[rg]);
            }
        }
        // the lane's k-slots 4 rg + i are pairs 16 rg + 4 grp + i
        bf16x8 ph, pl, sh, sl;
#pragma unroll
        for (int rg = 0; rg < 2; ++rg) {
            const int p0 = 16 * rg + 4 * grp;
            const f32x4 pb = *(const f32x4 *)&pbias[p0], pc = *(const f32x4 *)&pdc[p0];
            const int4 pr = *(const int4 *)&prow[p0];
            const int lim[4] = {pr.x, pr.y, pr.z, pr.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float ex = exp2_hw(fmaf(sacc[rg][i], scale2, pb[i]));
                const float P = (key_ok && key <= lim[i]) ? ex : 0.f;
                const float ds = scale * P * (dacc[rg][i] - pc[i]);
                const bf16 p1 = (bf16)P, d1 = (bf16)ds;
                ph[4 * rg + i] = p1;
                pl[4 * rg + i] = (bf16)(P - (float)p1);
                sh[4 * rg + i] = d1;
                sl[4 * rg + i] = (bf16)(ds - (float)d1);
            }
        }
        // V and K alternate, so consecutive MFMAs write different accumulators
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const bf16x8 ad = t_frag(do_t, dt), aq = t_frag(q_t, dt);
            accV[dt] = mfma16(ad, ph, accV[dt]);
            accK[dt] = mfma16(aq, sh, accK[dt]);
            accV[dt] = mfma16(ad, pl, accV[dt]);
            accK[dt] = mfma16(aq, sl, accK[dt]);
        }
        if (selected) {
            // dk'^T += Q^T X with X[pair][head] = scale ds^ when the pair's
            // query head feeds landmark head `head` (all pairs when there is
            // one landmark head per kv head); column r16 is head r16
            bf16x8 kh, kl;
            float dbs = 0.f;
#pragma unroll
            for (int rg = 0; rg < 2; ++rg) {
                const f32x4 pd = *(const f32x4 *)&pdsh[16 * rg + 4 * grp];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int lm = GLM == G ? (4 * grp + i) % G : 0;
                    const float x = lm == r16 ? pd[i] : 0.f;
                    dbs += x;
                    const float xs = scale * x;
                    const bf16 x1 = (bf16)xs;
                    kh[4 * rg + i] = x1;
                    kl[4 * rg + i] = (bf16)(xs - (float)x1);
                }
            }
#pragma unroll
            for (int j = 0; j < KPN; ++j) {
                const int dt = wave + NWV * j;
                if (dt < DT) {
                    const bf16x8 aq = t_frag(q_t, dt);
                    accKP[j] = mfma16(aq, kh, accKP[j]);
                    accKP[j] = mfma16(aq, kl, accKP[j]);
                }
            }
            dbacc += rows4_sum(dbs);  // this tile's ds^ of head r16
        }
    };

    // ntile tiles: tile j has nrows_of(j) rows, row_of(j, rr)
    auto run_tiles = [&](int ntile, bool selected, auto nrows_of, auto row_of) __attribute__((always_inline)) {
        if (ntile <= 0) return;
        fetch(nrows_of(0), selected, [&](int rr) { return row_of(0, rr); });
        for (int j = 0; j < ntile; ++j) {
            commit();
            if (j + 1 < ntile) fetch(nrows_of(j + 1), selected, [&](int rr) { return row_of(j + 1, rr); });
            compute(selected);
        }
    };

    // window rows: query chunks c .. c + W/S
    const int r_end = (int)min((int64_t)N, (int64_t)(c + W / S + 1) * S);
    run_tiles((r_end - c * S + RPT - 1) / RPT, false, [&](int j) { return min(RPT, r_end - c * S - j * RPT); },
              [&](int j, int rr) { return make_int2(c * S + j * RPT + rr, 0); });

    // rows of later query chunks that selected chunk c, in row order, from
    // the chunk's row bitmap: BW words per batch go to the row list (wave
    // 0); each listed row finds the chunk's slot in its selection (the count
    // of its entries below c: the lists are ascending); full tiles run, and
    // the rows of a partial tile carry over to the next batch
    if (K > 0 && c < C) {
        const int NWB = (N + 63) / 64;
        const uint64_t *bw = selbits + ((b * H_kv + g) * (int64_t)C + c) * NWB;
        if (t == 0) nlist = 0;
        for (int w0 = r_end / 64; w0 < NWB; w0 += BW) {
            __syncthreads();  // nlist and the carried rows are in place
            const int carry = nlist;
            if (wave == 0) {
                uint64_t word = 0ull;
                if (lane < BW && w0 + lane < NWB) {
                    word = bw[w0 + lane];
                    if (w0 + lane == r_end / 64) word &= ~0ull << (r_end & 63);  // rows >= r_end only
                }
                const int cnt = __popcll(word);
                int incl = cnt;
#pragma unroll
                for (int o = 1; o < WAVE; o <<= 1) {
                    const int y = __shfl_up(incl, o, WAVE);
                    if (lane >= o) incl += y;
                }
                int pos = carry + incl - cnt;
                while (word) {
                    const int bit = __builtin_ffsll((long long)word) - 1;
                    word &= word - 1;
                    list_i[pos++] = (w0 + lane) * 64 + bit;
                }
                if (lane == WAVE - 1) nlist = carry + incl;
            }
            __syncthreads();
            const int tot = nlist;
            for (int x = carry + t; x < tot; x += NT) {
                const int32_t *sr = sel_idx + ((b * H_kv + g) * N + list_i[x]) * K;
                int below = 0;
#pragma unroll 8
                for (int kk = 0; kk < K; ++kk) {
                    const int y = sr[kk];
                    below += (y >= 0 && y < c) ? 1 : 0;
                }
                list_k[x] = below;
            }
            __syncthreads();
            const bool last = w0 + BW >= NWB;
            const int nfull = last ? tot : tot / RPT * RPT;
            run_tiles((nfull + RPT - 1) / RPT, true, [&](int j) { return min(RPT, nfull - j * RPT); },
                      [&](int j, int rr) { return make_int2(list_i[j * RPT + rr], list_k[j * RPT + rr]); });
            __syncthreads();  // the tiles are done with the list
            const bool mv = t < tot - nfull;
            int li = 0, lk = 0;
            if (mv) li = list_i[nfull + t], lk = list_k[nfull + t];
            __syncthreads();
            if (mv) list_i[t] = li, list_k[t] = lk;
            if (t == 0) nlist = tot - nfull;
        }
    }

    // dk' and db' of the landmark heads: lane l holds dims 16 dt + 4 grp + i
    // of head l % 16
    if (r16 < GLM) {
#pragma unroll
        for (int j = 0; j < KPN; ++j) {
            const int dt = wave + NWV * j;
            if (dt < DT) {
#pragma unroll
                for (int i = 0; i < 4; ++i) dkp_l[r16][16 * dt + 4 * grp + i] = accKP[j][i];
            }
        }
        if (wave == 0 && grp == 0) dbp_l[r16] = dbacc;
    }

    // dv is final (the summary does not involve v)
    if (key_ok) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) *(f32x4 *)(dv + (kvb + key) * D + 16 * dt + 4 * grp) = accV[dt];
    }

    // ---- summary backward of the chunk's landmark heads (completed chunks):
    // a_j = scale q'.k_j, p = softmax a; da_j = p_j dk'.(k_j - k') -
    // db' p_j (a_j - p.a); dk_j += p_j dk' + scale da_j q'; dq' = scale sum_j da_j k_j
    if (c < C) {
        __syncthreads();  // dk', db' complete
        const int jj = t / NQ, qd = t % NQ, x0 = qd * DPT;
        const int64_t jrow = (int64_t)c * S + jj;  // completed chunk: jrow < N
        float kr[DPT];
#pragma unroll
        for (int x = 0; x < DPT; ++x) kr[x] = (float)k[(kvb + jrow) * D + x0 + x];
        auto quad_sum = [&](float a) {
            a += __shfl_xor(a, 1, WAVE);
            a += __shfl_xor(a, 2, WAVE);
            return a;
        };
        for (int e = 0; e < GLM; ++e) {
            const int lh = g * GLM + e;
            const int64_t lrow = ((b * H_lm + lh) * C + c) * D;
            // landmark query: per chunk, one shared by the chunks of head lh, or zero
            const int64_t qrow = lm_mode == 1 ? (int64_t)lh * D : lrow;
            float pa = 0.f, pk = 0.f;
#pragma unroll
            for (int x = 0; x < DPT; ++x) {
                const float qx = lm_mode == 2 ? 0.f : (float)q_lm[qrow + x0 + x];
                pa = fmaf(qx, kr[x], pa);
                pk = fmaf(dkp_l[e][x0 + x], kr[x], pk);
            }
            const float a = scale * quad_sum(pa), kdk = quad_sum(pk);  // a_j, dk'.k_j
            __syncthreads();  // the previous head is done with the LDS rows
            if (qd == 0) a_l[jj] = a, kd_l[jj] = kdk;
            if (t < D) qp_l[t] = lm_mode == 2 ? 0.f : (float)q_lm[qrow + t];
            __syncthreads();
            float mx = -INFINITY;
            for (int r = 0; r < S; ++r) mx = fmaxf(mx, a_l[r]);
            float z = 0.f, za = 0.f, zk = 0.f;
            for (int r = 0; r < S; ++r) {
                const float ex = expf(a_l[r] - mx);
                z += ex;
                za = fmaf(ex, a_l[r], za);
                zk = fmaf(ex, kd_l[r], zk);
            }
            const float p = expf(a - mx) / z;
            const float abar = za / z, kpdk = zk / z;  // p.a, dk'.k'
            const float da = p * (kdk - kpdk) - dbp_l[e] * p * (a - abar);
            if (qd == 0) p_l[jj] = p, da_l[jj] = da;
#pragma unroll
            for (int x = 0; x < DPT; ++x) red[jj][x0 + x] = da * kr[x];
            __syncthreads();
            // dk_j += p_j dk' + scale da_j q' in the accumulator layout
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int x = 16 * dt + 4 * grp + i;
                    accK[dt][i] = fmaf(p_l[keyl], dkp_l[e][x], accK[dt][i]);
                    accK[dt][i] = fmaf(scale * da_l[keyl], qp_l[x], accK[dt][i]);
                }
            if (lm_mode != 2 && t < D) {
                float sum = 0.f;
                for (int r = 0; r < S; ++r) sum += red[r][t];
                dq_lm[lrow + t] = scale * sum;
            }
        }
    }

    if (key_ok) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) *(f32x4 *)(dk + (kvb + key) * D + 16 * dt + 4 * grp) = accK[dt];
    }
}

// ---------------------------------------------------------------- MFMA row pass (bf16 I/O)
//
// s_waitcnt immediate that waits for vmcnt <= n only (gfx9 encoding)
constexpr int bwd_vmcnt(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }

// Block (query block, kv head g, batch b): NWAVE waves, each one MFMA tile
// of 16 (row, head) pairs (16/G consecutive rows x the G heads; lane l is
// pair l%16).  The block walks the ascending union of its rows' selections,
// then the window chunks.  Per chunk it stages K and V row-major (A operands
// of S^T = K Q^T and dP^T = V dO^T; the A operand K^T of dq^T += K^T dS^T
// is read from the K tile with transposing LDS reads) through a ring of
// NSTG stages, so several chunks' loads are in flight while one is used.  A wave computes the chunk when one of its pairs
// selected it (window: always).  The accumulators A^T and Bv^T hold, in
// lane l, dims 16dt + 4(l/16) + i of pair l%16:
//   window key j:       A += P_j (dO.v_j) k_j,  Bv += P_j k_j
//   key j of chunk c:   A += w_c p_cj (dO.v_j - g_c) k_j
// and, once the walk is done, A += sum_c w_c g_c k'_c, Bv += sum_c w_c k'_c,
// D' = sum_window P_j dO.v_j + sum_c w_c g_c - dlse, dq = scale (A - D' Bv).
// P and the ds operands enter as two bf16 terms each.
template <int D, int S, int G, int NWAVE, int NSTG>
__global__ __launch_bounds__(NWAVE * 64) void bwd_rows_mfma_kernel(
    const bf16 *__restrict__ q, const bf16 *__restrict__ k, const bf16 *__restrict__ v,
    const float *__restrict__ k_sum, const int32_t *__restrict__ sel_idx,
    const float *__restrict__ sel_score, const float *__restrict__ lse, const bf16 *__restrict__ dout,
    const float *__restrict__ dlse, float *__restrict__ dq, float *__restrict__ dsel, float *__restrict__ mlog,
    float *__restrict__ gdo, float *__restrict__ dcoef, int N, int H_q, int H_kv, int H_lm, int C, int W, int K,
    float scale, int NW, int UCAP) {
    constexpr int QPT = 16 / G, QB = NWAVE * QPT, NT = NWAVE * 64;
    constexpr int KS = D / 32, KT = S / 16, PS = S / 32, DT = D / 16, NB = D / 8;
    constexpr int TK = S * NB, TV = S * NB, STAGE = TK + TV;  // 16-byte units
    constexpr int PK = TK / 64, NPC = STAGE / 64;  // 1 KB DMA pieces: of a K (or V) tile, of a chunk
    constexpr int PPW = NPC / NWAVE;               // pieces per wave and chunk
    static_assert(NPC % NWAVE == 0, "every wave issues the same number of pieces");
    __shared__ u32x4 stg[NSTG][STAGE];
    extern __shared__ int dyn[];
    int16_t *sel_l = (int16_t *)dyn;                                      // [QB][K]
    float *sc_l = (float *)(dyn + (QB * K + 1) / 2);                       // [QB * G][K] s^ of each pair's slots
    uint32_t *bitmap = (uint32_t *)(sc_l + QB * G * K);                    // [NW]
    int *ulist = (int *)(bitmap + NW);                                     // [UCAP + W/S + 1]
    int *scan = ulist + UCAP + W / S + 1;                                  // [16]

    const int qb = blockIdx.x, g = blockIdx.y;
    const int64_t b = blockIdx.z, bg = b * H_kv + g;
    const int i0 = qb * QB, qc = i0 / S, n = max(0, qc - W / S);
    const int tid = threadIdx.x, wave = tid / WAVE, lane = lane_id(), grp = lane >> 4, r = lane & 15;
    const int GLM = H_lm / H_kv;

    // ---- setup: selections, scores, union of the block's selections
    for (int t = tid; t < NW; t += NT) bitmap[t] = 0u;
    for (int t = tid; t < QB * K; t += NT) {
        const int iq = i0 + t / K;
        sel_l[t] = (int16_t)(iq < N ? sel_idx[(bg * N + iq) * K + t % K] : -1);
    }
    for (int t = tid; t < QB * G * K; t += NT) {
        const int m = t / (G * K), rem = t % (G * K), e = rem / K, iq = i0 + m;
        sc_l[t] = iq < N ? sel_score[((b * H_q + g * G + e) * N + iq) * K + rem % K] : -INFINITY;
    }
    __syncthreads();
    for (int t = tid; t < QB * K; t += NT) {
        const int c = sel_l[t];
        if (c >= 0 && c < n) atomicOr(&bitmap[c >> 5], 1u << (c & 31));
    }
    __syncthreads();
    int U = 0;
    {
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
                if (pos < UCAP) ulist[pos] = wi * 32 + bit;
                ++pos;
            }
            base += tot;
            __syncthreads();
        }
        U = min(base, UCAP);
    }
    const int wc0 = max(0, qc - W / S);
    const int T = U + (qc - wc0 + 1);
    for (int t = tid; t < T - U; t += NT) ulist[U + t] = wc0 + t;

    // ---- per-pair state
    const int m = wave * QPT + r / G, e = r % G, iq = i0 + m, h = g * G + e;
    const bool rv = iq < N;
    const int64_t row = (b * H_q + h) * N + min(iq, N - 1);
    bf16x8 qf[KS], df[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        const u32x4 a = *(const u32x4 *)(q + row * D + 32 * s + 8 * grp);
        const u32x4 c2 = *(const u32x4 *)(dout + row * D + 32 * s + 8 * grp);
        __builtin_memcpy(&qf[s], &a, 16);
        __builtin_memcpy(&df[s], &c2, 16);
    }
    const float L = lse[row];
    const float scale2 = scale * LOG2E, L2 = rv ? L * LOG2E : INFINITY;
    f32x4 accA[DT], accB[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) accA[dt] = accB[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float dpart = 0.f;
    __syncthreads();  // sel_l, sc_l, ulist complete
    const int16_t *sl = sel_l + m * K;
    const float *scp = sc_l + (m * G + e) * K;
    int cur = 0, nsel = 0;
    for (int kk = 0; kk < K; ++kk) nsel += sl[kk] >= 0;
    int nch = (rv && nsel > 0) ? sl[0] : 0x7fffffff;

    const bf16 *kb = k + bg * (int64_t)N * D, *vb = v + bg * (int64_t)N * D;
    // DMA of chunk ulist[it] into ring stage buf: 1 KB pieces, 16 bytes
    // per lane into lane-contiguous LDS, the XOR swizzle applied through the
    // per-lane source offset; the resources end at key N (rows past it read
    // as zeros).  Every wave issues PPW pieces per chunk.
    auto issue = [&](int it, int buf) __attribute__((always_inline)) {
        const int c = __builtin_amdgcn_readfirstlane(ulist[it]);
        const int kbytes = max(0, min(S, N - c * S)) * D * 2;
        const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(kb + (int64_t)c * S * D), (short)0, kbytes, BWD_RSRC_WORD3);
        const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(vb + (int64_t)c * S * D), (short)0, kbytes, BWD_RSRC_WORD3);
        constexpr int RPP = 1024 / (D * 2);  // key rows per piece
#pragma unroll
        for (int x = 0; x < PPW; ++x) {
            const int pc = wave + x * NWAVE;
            const int pp = pc % PK, row = pp * RPP + lane / NB, blk = lane % NB;
            const int off = (row * D + (blk ^ bswz<NB>(row)) * 8) * 2;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(pc < PK ? kr : vr, BWD_LPTR(&stg[buf][pc * 64]), 16, off, 0, 0, 0);
        }
    };
    // wait until at most n pieces groups (PPW each) of this wave are in flight
    auto wait_groups = [&](int n) __attribute__((always_inline)) {
        if (n <= 0) __builtin_amdgcn_s_waitcnt(bwd_vmcnt(0));
        else if (n == 1) __builtin_amdgcn_s_waitcnt(bwd_vmcnt(PPW));
        else __builtin_amdgcn_s_waitcnt(bwd_vmcnt(2 * PPW));
    };
    // ds (or P) operand of a 32-key step from two 16-key accumulator tiles,
    // as hi and lo bf16 terms
    auto split_op = [&](const f32x4 &a0, const f32x4 &a1, bf16x8 &hi, bf16x8 &lo) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bf16 h0 = (bf16)a0[i], h1 = (bf16)a1[i];
            hi[i] = h0;
            hi[4 + i] = h1;
            lo[i] = (bf16)(a0[i] - (float)h0);
            lo[4 + i] = (bf16)(a1[i] - (float)h1);
        }
    };
    // acc^T += K^T X^T over the chunk, X given per 16-key tile in the S^T layout
    // The A operand K^T (dims 16 dt + l%16 x k-slots 8 grp .. +7 of step
    // ps) read transposed from the row-major K tile: in each 16-lane group,
    // the transpose read gives lane i element i of the 16 values that lanes
    // 4r .. 4r+3 address, r = 0..3; lane 4r + sub addresses 4 dims of key
    // row r, so lane i gets dim 16 dt + i of four consecutive keys.  Slots
    // 8grp .. 8grp+3 are keys 32ps + 4grp + r, slots 8grp+4 .. +7 keys
    // 32ps + 16 + 4grp + r.
    const int tsub = r & 3, trow = r >> 2;
    auto kt_frag = [&](const u32x4 (*k_l)[NB], int ps, int dt) __attribute__((always_inline)) {
        const int x0 = 16 * dt + 4 * tsub;  // the 4 dims this lane addresses
        bf16x8 a;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int key = 32 * ps + 16 * h + 4 * grp + trow;
            const short *src = (const short *)&k_l[key][(x0 >> 3) ^ bswz<NB>(key)] + (x0 & 7);
            const v4i16 v4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16 *)src);
            __builtin_memcpy((char *)&a + 8 * h, &v4, 8);
        }
        return a;
    };
    // acc1^T += K^T X1^T and acc2^T += K^T X2^T from one read of each K^T
    // fragment (the window: X1 = P o dP, X2 = P)
    auto ktx2 = [&](const f32x4 (&x1)[KT], f32x4 (&acc1)[DT], const f32x4 (&x2)[KT], f32x4 (&acc2)[DT],
                    const u32x4 (*k_l)[NB]) __attribute__((always_inline)) {
#pragma unroll
        for (int ps = 0; ps < PS; ++ps) {
            bf16x8 hi1, lo1, hi2, lo2;
            split_op(x1[2 * ps], x1[2 * ps + 1], hi1, lo1);
            split_op(x2[2 * ps], x2[2 * ps + 1], hi2, lo2);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const bf16x8 a = kt_frag(k_l, ps, dt);
                acc1[dt] = mfma16(a, hi1, acc1[dt]);
                acc2[dt] = mfma16(a, hi2, acc2[dt]);
                acc1[dt] = mfma16(a, lo1, acc1[dt]);
                acc2[dt] = mfma16(a, lo2, acc2[dt]);
            }
        }
    };
    auto ktx = [&](const f32x4 (&x)[KT], f32x4 (&acc)[DT], const u32x4 (*k_l)[NB]) __attribute__((always_inline)) {
#pragma unroll
        for (int ps = 0; ps < PS; ++ps) {
            bf16x8 hi, lo;
            split_op(x[2 * ps], x[2 * ps + 1], hi, lo);
            // the hi terms of every dim tile, then the lo terms: consecutive
            // MFMAs write different accumulators
            bf16x8 a[DT];
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                a[dt] = kt_frag(k_l, ps, dt);
                acc[dt] = mfma16(a[dt], hi, acc[dt]);
            }
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) acc[dt] = mfma16(a[dt], lo, acc[dt]);
        }
    };

    // ---- the walk, through a ring of NSTG stages: chunk it + NSTG - 1 is
    // issued at the start of step it, into the stage every wave released at
    // the end of step it - 1; a step ends once chunk it + 1 has landed (this
    // wave's later pieces may stay in flight; other vector-memory operations
    // issued after them only make the wait longer)
    // one step of the walk: chunk it, staged in ring stage it % NSTG
    auto step = [&](int it) __attribute__((always_inline)) {
        const u32x4(*k_l)[NB] = reinterpret_cast<const u32x4(*)[NB]>(&stg[it % NSTG][0]);
        const u32x4(*v_l)[NB] = reinterpret_cast<const u32x4(*)[NB]>(&stg[it % NSTG][TK]);
        const int c = ulist[it];
        const bool window = it >= U;
        const bool act = rv && (window || nch == c);
        if (__ballot(act) != 0ull) {
        f32x4 sacc[KT], dacc[KT];
#pragma unroll
        for (int kt2 = 0; kt2 < KT; ++kt2) sacc[kt2] = dacc[kt2] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
            for (int kt2 = 0; kt2 < KT; ++kt2) {
                const int kr = 16 * kt2 + r, blk = (4 * s + grp) ^ bswz<NB>(kr);
                const u32x4 rk = k_l[kr][blk], rvv = v_l[kr][blk];
                bf16x8 ak, av;
                __builtin_memcpy(&ak, &rk, 16);
                __builtin_memcpy(&av, &rvv, 16);
                sacc[kt2] = mfma16(ak, qf[s], sacc[kt2]);
                dacc[kt2] = mfma16(av, df[s], dacc[kt2]);
            }
        if (!window) {
            // the chunk's softmax in base 2: e_j = 2^(x_j - max x), x = s log2 e,
            // p_cj = e_j / z, lse_c = (max x + log2 z) ln 2
            float cmax = -INFINITY;
#pragma unroll
            for (int kt2 = 0; kt2 < KT; ++kt2)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    sacc[kt2][i] *= scale2;
                    cmax = fmaxf(cmax, sacc[kt2][i]);
                }
            cmax = rows4_max(cmax);
            float z = 0.f, gp = 0.f;
#pragma unroll
            for (int kt2 = 0; kt2 < KT; ++kt2)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float ex = exp2_hw(sacc[kt2][i] - cmax);
                    sacc[kt2][i] = ex;
                    z += ex;
                    gp = fmaf(ex, dacc[kt2][i], gp);
                }
            z = rows4_sum(z);  // >= 1: the largest key contributes 2^0
            const float rz = __builtin_amdgcn_rcpf(z);
            const float lse_c = (cmax + log2f(z)) * LN2;
            const float gc = rows4_sum(gp) * rz;  // dO.o_c
            const float shat = act ? scp[cur] : 0.f;
            const float f = act ? expf(shat - L) * rz : 0.f;  // w_c / z
#pragma unroll
            for (int kt2 = 0; kt2 < KT; ++kt2)
#pragma unroll
                for (int i = 0; i < 4; ++i) sacc[kt2][i] = f * sacc[kt2][i] * (dacc[kt2][i] - gc);
            ktx(sacc, accA, k_l);
            if (act) {
                if (grp == 0) {
                    mlog[row * K + cur] = shat - L - lse_c;
                    gdo[row * K + cur] = gc;
                }
                ++cur;
                nch = cur < nsel ? (int)sl[cur] : 0x7fffffff;
            }
        } else {
            // P = 2^(s scale log2 e - L log2 e); a row past N has L2 = +inf (P = 0).
            // Keys of a window chunk below the query chunk all precede the
            // row; in the query's own chunk, keys after the row are masked.
#pragma unroll
            for (int kt2 = 0; kt2 < KT; ++kt2)
#pragma unroll
                for (int i = 0; i < 4; ++i) sacc[kt2][i] = exp2_hw(fmaf(sacc[kt2][i], scale2, -L2));
            if (c == qc) {
#pragma unroll
                for (int kt2 = 0; kt2 < KT; ++kt2)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (c * S + 16 * kt2 + 4 * grp + i > iq) sacc[kt2][i] = 0.f;
            }
#pragma unroll
            for (int kt2 = 0; kt2 < KT; ++kt2)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    dpart = fmaf(sacc[kt2][i], dacc[kt2][i], dpart);
                    dacc[kt2][i] *= sacc[kt2][i];
                }
            ktx2(dacc, accA, sacc, accB, k_l);
        }
        }
    };
    __syncthreads();  // the walk list is complete
    if constexpr (NSTG == 4) {
        // steps in pairs, one barrier per pair: chunks it + 2 and it + 3 are
        // issued at the start of the pair into the stages the previous
        // barrier released, and have landed at its end
        for (int j = 0; j < 2 && j < T; ++j) issue(j, j);
        wait_groups(0);
        __syncthreads();
        for (int it = 0; it < T; it += 2) {
            for (int j = it + 2; j < it + 4 && j < T; ++j) issue(j, j % NSTG);
            step(it);
            if (it + 1 < T) step(it + 1);
            wait_groups(0);
            __syncthreads();
        }
    } else {
        for (int j = 0; j < NSTG - 1 && j < T; ++j) issue(j, j);
        wait_groups(min(NSTG - 2, T - 1));
        __syncthreads();
        for (int it = 0; it < T; ++it) {
            if (it + NSTG - 1 < T) issue(it + NSTG - 1, (it + NSTG - 1) % NSTG);
            step(it);
            // chunk it + 1 has landed once at most the groups issued after it
            // (chunks it + 2 .. min(it + NSTG - 1, T - 1)) are in flight
            wait_groups(min(NSTG - 2, T - 2 - it));
            __syncthreads();
        }
    }

    // ---- epilogue: the summary terms, D', dq, ds^ of each slot
    __syncthreads();  // this wave's gdo writes are visible to its other lanes
    const int lh = GLM == G ? h : g;  // landmark head of the pair
    float dsum = 0.f;
    for (int kk = 0; kk < nsel; ++kk) {
        const int c = sl[kk];
        const float wc = expf(scp[kk] - L), gc = gdo[row * K + kk];
        dsum = fmaf(wc, gc, dsum);
        const float *kp = k_sum + ((b * H_lm + lh) * (int64_t)C + c) * D + 4 * grp;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const f32x4 kv = *(const f32x4 *)(kp + 16 * dt);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                accA[dt][i] = fmaf(wc * gc, kv[i], accA[dt][i]);
                accB[dt][i] = fmaf(wc, kv[i], accB[dt][i]);
            }
        }
    }
    if (!rv) return;
    const float Dp = rows4_sum(dpart) + dsum - (dlse ? dlse[row] : 0.f);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
        f32x4 o;
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = scale * fmaf(-Dp, accB[dt][i], accA[dt][i]);
        *(f32x4 *)(dq + row * D + 16 * dt + 4 * grp) = o;
    }
    if (grp == 0) {
        dcoef[row] = Dp;
        for (int kk = 0; kk < K; ++kk) {
            if (kk < nsel) {
                dsel[row * K + kk] = expf(scp[kk] - L) * (gdo[row * K + kk] - Dp);
            } else {
                dsel[row * K + kk] = 0.f;
                mlog[row * K + kk] = -INFINITY;
                gdo[row * K + kk] = 0.f;
            }
        }
    }
}

// Row bitmap of each chunk's selecting rows: bit i of row c of (b, g) is
// set when row i selected chunk c (order-free ORs, so the map is
// deterministic).  Thread per row.
__global__ __launch_bounds__(256) void bwd_selbits_kernel(const int32_t *__restrict__ sel_idx,
                                                          uint64_t *__restrict__ selbits, int N, int H_kv, int C,
                                                          int K) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    const int64_t bg = (int64_t)blockIdx.z * H_kv + blockIdx.y;
    if (i >= N) return;
    const int NWB = (N + 63) / 64;
    const int32_t *sr = sel_idx + (bg * N + i) * K;
    for (int kk = 0; kk < K; ++kk) {
        const int c = sr[kk];
        if (c >= 0 && c < C) atomicOr((unsigned long long *)&selbits[(bg * C + c) * NWB + i / 64], 1ull << (i & 63));
    }
}

__global__ __launch_bounds__(256) void bwd_zero_u64_kernel(uint64_t *__restrict__ p, int64_t n) {
    for (int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x; x < n; x += (int64_t)gridDim.x * 256) p[x] = 0ull;
}

// Shared landmark query: the gradient of the one query of head l is the sum
// of the per-chunk gradients over every sequence and chunk, in a fixed order.
__global__ __launch_bounds__(256) void bwd_shared_query_kernel(const float *__restrict__ per_chunk,
                                                               float *__restrict__ dq_lm, int B, int H_lm, int C,
                                                               int D) {
    const int idx = blockIdx.x * blockDim.x + threadIdx.x;  // l * D + x
    if (idx >= H_lm * D) return;
    const int l = idx / D, x = idx % D;
    float acc = 0.f;
    for (int b = 0; b < B; ++b)
        for (int c = 0; c < C; ++c) acc += per_chunk[(((int64_t)b * H_lm + l) * C + c) * D + x];
    dq_lm[idx] = acc;
}

// bf16 I/O: one bit per (chunk, row) of each (b, kv head)
static size_t selbits_bytes(const Shape &s) {
    if (!s.io_bf16 || s.K == 0) return 0;
    return (size_t)s.B * s.H_kv * s.C * ((s.N + 63) / 64) * 8;
}

size_t backward_workspace_bytes(const Shape &s) {
    const size_t rows = (size_t)s.B * s.H_q * s.N;
    size_t b = 3 * align_up(rows * s.K * 4, 256) + align_up(rows * 4, 256);
    if (s.lm_mode == 1) b += align_up((size_t)s.B * s.H_lm * s.C * s.D * 4, 256);  // per-chunk dq'
    b += align_up(selbits_bytes(s), 256);
    return b;
}

// The MFMA row pass when its LDS fits the shape (false: not launched): the
// deepest ring (4, 3 or 2 stages of K and V) that fits beside the block's
// selections, scores and walk list.  64-key chunks; 128-key chunks take the
// fp32 VALU row pass.
template <int D, int S, int G, int NWAVE, int NSTG>
static bool go_rows_mfma(const Shape &s, const void *q, const void *k, const void *v, const float *k_sum,
                         const int32_t *sel_idx, const float *sel_score, const float *lse, const void *dout,
                         const float *dlse, float *dq, float *dsel, float *mlog, float *gdo, float *dcoef,
                         size_t dyn, int NW, int UCAP, hipStream_t st) {
    constexpr int QB = NWAVE * (16 / G);
    constexpr size_t stage = (size_t)NSTG * 2 * S * (D / 8) * 16;
    if constexpr (stage > 160 * 1024) {
        return false;
    } else {
        if (stage + dyn > 160 * 1024) return false;
        auto kern = bwd_rows_mfma_kernel<D, S, G, NWAVE, NSTG>;
        if (hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn) !=
            hipSuccess)
            return false;
        const dim3 grid((unsigned)((s.N + QB - 1) / QB), (unsigned)s.H_kv, (unsigned)s.B);
        hipLaunchKernelGGL(kern, grid, dim3(NWAVE * 64), dyn, st, (const bf16 *)q, (const bf16 *)k, (const bf16 *)v,
                           k_sum, sel_idx, sel_score, lse, (const bf16 *)dout, dlse, dq, dsel, mlog, gdo, dcoef, s.N,
                           s.H_q, s.H_kv, s.H_lm, s.C, s.W, s.K, s.scale, NW, UCAP);
        return true;
    }
}

template <int D, int S, int G>
static bool try_rows_mfma(const Shape &s, const void *q, const void *k, const void *v, const float *k_sum,
                          const int32_t *sel_idx, const float *sel_score, const float *lse, const void *dout,
                          const float *dlse, float *dq, float *dsel, float *mlog, float *gdo, float *dcoef,
                          hipStream_t st) {
    if constexpr (S != 64) {
        return false;
    } else {
        constexpr int NWAVE = S * G / 16 < 8 ? S * G / 16 : 8;
        constexpr int QB = NWAVE * (16 / G);
        const int NW = (s.C + 31) / 32 + 1;
        const int UCAP = std::min(s.C + 1, QB * s.K + 1);
        const size_t dyn = (size_t)((QB * s.K + 1) / 2) * 4 + (size_t)QB * G * s.K * 4 + (size_t)NW * 4 +
                           (size_t)(UCAP + s.W / s.S + 1) * 4 + 16 * 4;
        return go_rows_mfma<D, S, G, NWAVE, 4>(s, q, k, v, k_sum, sel_idx, sel_score, lse, dout, dlse, dq, dsel,
                                               mlog, gdo, dcoef, dyn, NW, UCAP, st) ||
               go_rows_mfma<D, S, G, NWAVE, 3>(s, q, k, v, k_sum, sel_idx, sel_score, lse, dout, dlse, dq, dsel,
                                               mlog, gdo, dcoef, dyn, NW, UCAP, st) ||
               go_rows_mfma<D, S, G, NWAVE, 2>(s, q, k, v, k_sum, sel_idx, sel_score, lse, dout, dlse, dq, dsel,
                                               mlog, gdo, dcoef, dyn, NW, UCAP, st);
    }
}

template <typename T, int D, int S>
static hipError_t go_backward(const Shape &s, const void *q, const void *k, const void *v, const void *q_lm,
                              const float *k_sum, const int32_t *sel_idx, const float *sel_score, const float *lse,
                              const void *dout, const float *dlse, float *dq, float *dk, float *dv, float *dq_lm,
                              void *workspace, hipStream_t st) {
    const size_t rows = (size_t)s.B * s.H_q * s.N;
    char *p = (char *)workspace;
    float *dsel = (float *)p;
    p += align_up(rows * s.K * 4, 256);
    float *mlog = (float *)p;
    p += align_up(rows * s.K * 4, 256);
    float *gdo = (float *)p;
    p += align_up(rows * s.K * 4, 256);
    float *dcoef = (float *)p;
    p += align_up(rows * 4, 256);
    // shared landmark query: per-chunk gradients first, summed afterwards
    float *dql_chunks = s.lm_mode == 1 ? (float *)p : dq_lm;
    if (s.lm_mode == 1) p += align_up((size_t)s.B * s.H_lm * s.C * s.D * 4, 256);
    uint64_t *selbits = (uint64_t *)p;  // bf16 I/O with K > 0
    const int64_t nbits = (int64_t)(selbits_bytes(s) / 8);
    p += align_up(selbits_bytes(s), 256);
    bool rows_done = false;
    if constexpr (std::is_same<T, bf16>::value) {
        switch (s.G) {
            case 1: rows_done = try_rows_mfma<D, S, 1>(s, q, k, v, k_sum, sel_idx, sel_score, lse, dout, dlse, dq,
                                                        dsel, mlog, gdo, dcoef, st); break;
            case 2: rows_done = try_rows_mfma<D, S, 2>(s, q, k, v, k_sum, sel_idx, sel_score, lse, dout, dlse, dq,
                                                        dsel, mlog, gdo, dcoef, st); break;
            case 4: rows_done = try_rows_mfma<D, S, 4>(s, q, k, v, k_sum, sel_idx, sel_score, lse, dout, dlse, dq,
                                                        dsel, mlog, gdo, dcoef, st); break;
            default: rows_done = try_rows_mfma<D, S, 8>(s, q, k, v, k_sum, sel_idx, sel_score, lse, dout, dlse, dq,
                                                         dsel, mlog, gdo, dcoef, st); break;
        }
    }
    if (!rows_done) {
        const dim3 rgrid((unsigned)((int64_t)s.B * s.H_kv * s.N));
        auto go_rows = [&](auto kern, int G) {
            hipLaunchKernelGGL(kern, rgrid, dim3(64 * G), 0, st, (const T *)q, (const T *)k, (const T *)v, k_sum,
                               sel_idx, sel_score, lse, (const T *)dout, dlse, dq, dsel, mlog, gdo, dcoef, s.N, s.H_q,
                               s.H_kv, s.H_lm, s.C, s.W, s.K, s.scale);
        };
        switch (s.G) {
            case 1: go_rows(bwd_rows_kernel<T, D, S, 1>, 1); break;
            case 2: go_rows(bwd_rows_kernel<T, D, S, 2>, 2); break;
            case 4: go_rows(bwd_rows_kernel<T, D, S, 4>, 4); break;
            case 8: go_rows(bwd_rows_kernel<T, D, S, 8>, 8); break;
            default: return hipErrorInvalidValue;
        }
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 kgrid((unsigned)s.CA, (unsigned)s.H_kv, (unsigned)s.B);
    if constexpr (std::is_same<T, bf16>::value) {
        if (nbits > 0) {
            hipLaunchKernelGGL(bwd_zero_u64_kernel, dim3((unsigned)std::min<int64_t>(4096, (nbits + 255) / 256)),
                               dim3(256), 0, st, selbits, nbits);
            hipLaunchKernelGGL(bwd_selbits_kernel, dim3((unsigned)((s.N + 255) / 256), (unsigned)s.H_kv, (unsigned)s.B),
                               dim3(256), 0, st, sel_idx, selbits, s.N, s.H_kv, s.C, s.K);
        }
        auto go_keys = [&](auto kern) {
            hipLaunchKernelGGL(kern, kgrid, dim3(4 * S), 0, st, (const bf16 *)q, (const bf16 *)k, (const bf16 *)v,
                               (const bf16 *)q_lm, sel_idx, (const uint64_t *)selbits, lse, (const bf16 *)dout, dcoef,
                               dsel, mlog, gdo, dk, dv, dql_chunks, s.N, s.H_q, s.H_kv, s.H_lm, s.C, s.W, s.K, s.scale,
                               s.lm_mode);
        };
        switch (s.G) {
            case 1: go_keys(bwd_keys_mfma_kernel<D, S, 1>); break;
            case 2: go_keys(bwd_keys_mfma_kernel<D, S, 2>); break;
            case 4: go_keys(bwd_keys_mfma_kernel<D, S, 4>); break;
            default: go_keys(bwd_keys_mfma_kernel<D, S, 8>); break;
        }
    } else {
        hipLaunchKernelGGL((bwd_keys_kernel<T, D, S>), kgrid, dim3(4 * S), 0, st, (const T *)q, (const T *)k,
                           (const T *)v, (const T *)q_lm, sel_idx, lse, (const T *)dout, dcoef, dsel, mlog, gdo, dk,
                           dv, dql_chunks, s.N, s.H_q, s.H_kv, s.H_lm, s.C, s.W, s.K, s.scale, s.lm_mode);
    }
    if (s.lm_mode == 1) {
        if ((e = hipGetLastError()) != hipSuccess) return e;
        hipLaunchKernelGGL(bwd_shared_query_kernel, dim3((unsigned)((s.H_lm * s.D + 255) / 256)), dim3(256), 0, st,
                           (const float *)dql_chunks, dq_lm, s.B, s.H_lm, s.C, s.D);
    }
    return hipGetLastError();
}

template <typename T>
static hipError_t dispatch_backward(const Shape &s, const void *q, const void *k, const void *v, const void *q_lm,
                                    const float *k_sum, const int32_t *sel_idx, const float *sel_score,
                                    const float *lse, const void *dout, const float *dlse, float *dq, float *dk,
                                    float *dv, float *dq_lm, void *ws, hipStream_t st) {
#define HILS_BWD(DD, SS)                                                                                      \
    if (s.D == DD && s.S == SS)                                                                               \
        return go_backward<T, DD, SS>(s, q, k, v, q_lm, k_sum, sel_idx, sel_score, lse, dout, dlse, dq, dk, dv, \
                                      dq_lm, ws, st);
    HILS_BWD(64, 64) HILS_BWD(64, 128) HILS_BWD(128, 64) HILS_BWD(128, 128)
#undef HILS_BWD
    return hipErrorInvalidValue;
}

hipError_t launch_backward(const Shape &s, const void *q, const void *k, const void *v, const void *q_lm,
                           const float *k_sum, const int32_t *sel_idx, const float *sel_score, const float *lse,
                           const void *dout, const float *dlse, float *dq, float *dk, float *dv, float *dq_lm,
                           void *workspace, hipStream_t st) {
    if ((int64_t)s.B * s.N == 0) return hipSuccess;
    if (s.io_bf16)
        return dispatch_backward<bf16>(s, q, k, v, q_lm, k_sum, sel_idx, sel_score, lse, dout, dlse, dq, dk, dv, dq_lm,
                                       workspace, st);
    return dispatch_backward<float>(s, q, k, v, q_lm, k_sum, sel_idx, sel_score, lse, dout, dlse, dq, dk, dv, dq_lm,
                                    workspace, st);
}

}  // namespace hils
