// hils_device.hpp -- device-side helpers shared by the HiLS kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hils {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int WAVE = 64;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }

template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

// 16-byte vector of T: 8 bf16 or 4 fp32.
template <typename T>
struct Vec16;
template <>
struct Vec16<bf16> {
    static constexpr int E = 8;
    bf16x8 v;
    __device__ __forceinline__ float get(int i) const { return (float)v[i]; }
};
template <>
struct Vec16<float> {
    static constexpr int E = 4;
    f32x4 v;
    __device__ __forceinline__ float get(int i) const { return v[i]; }
};

template <typename T>
__device__ __forceinline__ Vec16<T> load16(const T *p) {
    Vec16<T> r;
    r.v = *reinterpret_cast<const decltype(r.v) *>(p);
    return r;
}

// Butterfly reductions over lanes that differ in the bits [lo_mask, hi_mask].
template <int FROM, int TO>
__device__ __forceinline__ float xor_max(float v) {
#pragma unroll
    for (int m = FROM; m <= TO; m <<= 1) v = fmaxf(v, __shfl_xor(v, m, WAVE));
    return v;
}
template <int FROM, int TO>
__device__ __forceinline__ float xor_sum(float v) {
#pragma unroll
    for (int m = FROM; m <= TO; m <<= 1) v += __shfl_xor(v, m, WAVE);
    return v;
}
template <int FROM, int TO>
__device__ __forceinline__ int xor_sum_i(int v) {
#pragma unroll
    for (int m = FROM; m <= TO; m <<= 1) v += __shfl_xor(v, m, WAVE);
    return v;
}

// 2^x by the hardware instruction alone (v_exp_f32, about 1 ulp).  Unlike
// exp2f it skips the rescaling that keeps results below 2^-126 denormal
// instead of zero: softmax weights that small change no sum they enter.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// Reductions across the four 16-lane rows of a wave (lanes l, l^16, l^32,
// l^48) with the gfx950 lane-swap instructions, which stay in the VALU
// instead of a ds_bpermute round trip.  Swapping a register with itself
// leaves each lane holding both values of its pair (l, l^32) resp.
// (l, l^16), lower-numbered lane's value first.
__device__ __forceinline__ float rows4_max(float v) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float rows4_sum(float v) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// DPP move within 16-lane rows (CTRL: quad_perm 0x00-0xFF, row_mirror
// 0x140, row_half_mirror 0x141).
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
// Sum / max over the 16 lanes of a DPP row (every lane gets the result).
__device__ __forceinline__ float row_sum16(float v) {
    v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
    v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
    v += dpp<0x141>(v);  // row_half_mirror
    v += dpp<0x140>(v);  // row_mirror
    return v;
}
__device__ __forceinline__ float row_max16(float v) {
    v = fmaxf(v, dpp<0xB1>(v));
    v = fmaxf(v, dpp<0x4E>(v));
    v = fmaxf(v, dpp<0x141>(v));
    v = fmaxf(v, dpp<0x140>(v));
    return v;
}
__device__ __forceinline__ float wave_sum_f(float v) { return rows4_sum(row_sum16(v)); }
__device__ __forceinline__ float wave_max_f(float v) { return rows4_max(row_max16(v)); }

// Transpose-reduce over the 16 lanes of a DPP row: lane c of the row holds
// v[0..15]; on return it holds sum over the row's lanes of v[c].  Four
// butterfly steps; each partner differs in the bit of c that picks which
// half of the remaining values a lane keeps (row_mirror flips bit 3,
// row_half_mirror bit 2, the quad permutations bits 1 and 0).
__device__ __forceinline__ float transpose_sum16(const float (&v)[16], int c) {
    float w[8], x[4], y[2];
    const bool b3 = (c >> 3) & 1, b2 = (c >> 2) & 1, b1 = (c >> 1) & 1, b0 = c & 1;
#pragma unroll
    for (int j = 0; j < 8; ++j) w[j] = (b3 ? v[j + 8] : v[j]) + dpp<0x140>(b3 ? v[j] : v[j + 8]);
#pragma unroll
    for (int j = 0; j < 4; ++j) x[j] = (b2 ? w[j + 4] : w[j]) + dpp<0x141>(b2 ? w[j] : w[j + 4]);
#pragma unroll
    for (int j = 0; j < 2; ++j) y[j] = (b1 ? x[j + 2] : x[j]) + dpp<0x4E>(b1 ? x[j] : x[j + 2]);
    return (b0 ? y[1] : y[0]) + dpp<0xB1>(b0 ? y[0] : y[1]);
}

__device__ __forceinline__ int wave_sum_i(int v) { return xor_sum_i<1, 32>(v); }
__device__ __forceinline__ float wave_max(float v) { return xor_max<1, 32>(v); }

__device__ __forceinline__ int lane_id() { return threadIdx.x & (WAVE - 1); }

// Orders LDS traffic between lanes of one wavefront (lanes run in lockstep;
// this keeps the compiler from moving LDS accesses across the point).
__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

// Order-preserving map float -> uint32 (larger float -> larger key).
__device__ __forceinline__ uint32_t ord_key(float x) {
    uint32_t u = __float_as_uint(x);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float ord_key_inv(uint32_t k) {
    uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
    return __uint_as_float(u);
}

__device__ __forceinline__ uint64_t lanemask_lt() {
    const int l = lane_id();
    return l == 0 ? 0ull : (~0ull >> (64 - l));
}

// MFMA 16x16x32 bf16 -> fp32.  A: lane l holds row l%16, k = 8*(l/16)..+7.
// B: lane l holds col l%16, k = 8*(l/16)..+7.  D: lane l holds rows
// 4*(l/16)+i (i = 0..3) of col l%16.
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// Same layout, fp16 operands.
__device__ __forceinline__ f32x4 mfma16h(f16x8 a, f16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// kk-th largest of the non-zero 64-bit keys held NV per lane (keys == 0 are
// empty slots): bisection on the upper 32 bits (the score), then on the low
// bits (the inverted chunk index) only when the score ties at the boundary.
// Counting is ballot + popcount (scalar), no cross-lane data movement.
template <int NV>
__device__ __forceinline__ uint64_t kth_largest64(const uint64_t (&keys)[NV], int kk) {
    uint32_t hi = 0;
    for (int bit = 31; bit >= 0; --bit) {
        const uint32_t cand = hi | (1u << bit);
        int cnt = 0;
#pragma unroll
        for (int v = 0; v < NV; ++v) cnt += __popcll(__ballot((uint32_t)(keys[v] >> 32) >= cand));
        if (cnt >= kk) hi = cand;
    }
    int above = 0, tied = 0;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        const uint32_t h = (uint32_t)(keys[v] >> 32);
        above += __popcll(__ballot(h > hi));
        tied += __popcll(__ballot(h == hi && keys[v] != 0ull));
    }
    const int need = kk - above;  // 1 <= need <= tied
    if (tied == need) return (uint64_t)hi << 32;
    uint32_t lo = 0;
    for (int bit = 31; bit >= 0; --bit) {
        const uint32_t cand = lo | (1u << bit);
        int cnt = 0;
#pragma unroll
        for (int v = 0; v < NV; ++v)
            cnt += __popcll(__ballot((uint32_t)(keys[v] >> 32) == hi && (uint32_t)keys[v] >= cand));
        if (cnt >= need) lo = cand;
    }
    return ((uint64_t)hi << 32) | lo;
}

// Sum over aligned segments of L lanes (L = 4..64), every lane of a
// segment gets the segment total.  DPP within 16-lane rows, lane swaps
// across rows.
template <int L>
__device__ __forceinline__ float seg_sum(float v) {
    static_assert(L == 4 || L == 8 || L == 16 || L == 32 || L == 64, "segment width");
    v += dpp<0xB1>(v);  // quad_perm [1,0,3,2]
    v += dpp<0x4E>(v);  // quad_perm [2,3,0,1]
    if constexpr (L >= 8) v += dpp<0x141>(v);   // row_half_mirror
    if constexpr (L >= 16) v += dpp<0x140>(v);  // row_mirror
    if constexpr (L >= 32) {
        const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        v = __uint_as_float(b[0]) + __uint_as_float(b[1]);
    }
    if constexpr (L >= 64) {
        const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    }
    return v;
}

// Ragged row offsets of the per-query candidate lists.  All queries of
// query chunk qc have n(qc) = max(0, qc - w) candidates (w = W / S); each
// row is padded to a multiple of 16 entries.
__host__ __device__ __forceinline__ int64_t pad16(int64_t n) { return (n + 15) & ~int64_t(15); }
// sum_{m=1}^{M} pad16(m) / 16 for M >= 0, i.e. sum of ceil(m/16).
__host__ __device__ __forceinline__ int64_t sum_ceil16(int64_t M) {
    if (M <= 0) return 0;
    const int64_t A = M / 16, r = M % 16;
    return 8 * A * (A + 1) + (A + 1) * r;
}
// Offset (in entries) of the first row of query chunk qc within one (b, g).
__host__ __device__ __forceinline__ int64_t cand_chunk_offset(int64_t qc, int64_t w, int64_t S) {
    // rows of chunks qc' < qc; chunk qc' contributes S * pad16(max(0, qc' - w)).
    const int64_t M = qc - 1 - w;  // largest candidate count among them
    return S * 16 * sum_ceil16(M);
}
__host__ __device__ __forceinline__ int64_t cand_row_offset(int64_t i, int64_t w, int64_t S) {
    const int64_t qc = i / S;
    const int64_t n = qc - w > 0 ? qc - w : 0;
    return cand_chunk_offset(qc, w, S) + (i % S) * pad16(n);
}

}  // namespace hils
