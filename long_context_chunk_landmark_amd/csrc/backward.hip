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
// Two kernels, deterministic (every sum has one owner, no atomics):
//   bwd_rows   one block per (b, kv head, row), a wave per query head of
//              the group: dq, and per selected slot ds^, the chunk's
//              log-weight m = s^ - L - lse_c and g = dO.o_c
//   bwd_keys   one block per (b, kv head, chunk): dk, dv of the chunk's keys
//              from the window rows and the rows that selected it (found by
//              a binary search in each later row's ascending selection),
//              the chunk's dk', db' of its landmark heads, and then the
//              summary backward into dk and dq'.
// fp32 VALU throughout: a first, exact backward; the forward's MFMA
// schedule is not carried over.
#include "hils_device.hpp"
#include "hils_internal.hpp"

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

size_t backward_workspace_bytes(const Shape &s) {
    const size_t rows = (size_t)s.B * s.H_q * s.N;
    size_t b = 3 * align_up(rows * s.K * 4, 256) + align_up(rows * 4, 256);
    if (s.lm_mode == 1) b += align_up((size_t)s.B * s.H_lm * s.C * s.D * 4, 256);  // per-chunk dq'
    return b;
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
    const dim3 rgrid((unsigned)((int64_t)s.B * s.H_kv * s.N));
    auto go_rows = [&](auto kern, int G) {
        hipLaunchKernelGGL(kern, rgrid, dim3(64 * G), 0, st, (const T *)q, (const T *)k, (const T *)v, k_sum, sel_idx,
                           sel_score, lse, (const T *)dout, dlse, dq, dsel, mlog, gdo, dcoef, s.N, s.H_q, s.H_kv,
                           s.H_lm, s.C, s.W, s.K, s.scale);
    };
    switch (s.G) {
        case 1: go_rows(bwd_rows_kernel<T, D, S, 1>, 1); break;
        case 2: go_rows(bwd_rows_kernel<T, D, S, 2>, 2); break;
        case 4: go_rows(bwd_rows_kernel<T, D, S, 4>, 4); break;
        case 8: go_rows(bwd_rows_kernel<T, D, S, 8>, 8); break;
        default: return hipErrorInvalidValue;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_keys_kernel<T, D, S>), dim3((unsigned)s.CA, (unsigned)s.H_kv, (unsigned)s.B), dim3(4 * S), 0,
                       st, (const T *)q, (const T *)k, (const T *)v, (const T *)q_lm, sel_idx, lse, (const T *)dout,
                       dcoef, dsel, mlog, gdo, dk, dv, dql_chunks, s.N, s.H_q, s.H_kv, s.H_lm, s.C, s.W, s.K, s.scale,
                       s.lm_mode);
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
