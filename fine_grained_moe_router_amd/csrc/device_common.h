// device_common.h -- gfx950 device helpers shared by the kernels: FP8 and bf16
// conversions, packed bf16 dot products, fixed-order DPP reductions and the top-K
// selection rounds.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {
namespace dev {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------ scalar helpers

__device__ __forceinline__ float bf2f(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// fp32 -> bf16, round to nearest even.
__device__ __forceinline__ uint16_t f2bf(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ bf16x2 as_bf2(uint32_t v) { return __builtin_bit_cast(bf16x2, v); }

// Two E4M3FN codes (bytes 0-1 or 2-3 of v) to two bf16, exactly (scale 1).
template <bool HI>
__device__ __forceinline__ bf16x2 fp8x2_to_bf16(uint32_t v) {
    return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v, 1.0f, HI);
}

// Two E4M3FN codes (word HI of v) to two fp32.
template <bool HI>
__device__ __forceinline__ f32x2 fp8x2_to_f32(uint32_t v) {
    return __builtin_amdgcn_cvt_pk_f32_fp8((int)v, HI);
}

__device__ __forceinline__ float dot2(bf16x2 a, bf16x2 b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(a, b, c, false);
}

// 16 codes (one uint4) -> 8 bf16 pairs in column order.
__device__ __forceinline__ void decode16_bf16(const uint4 q, bf16x2 (&w)[8]) {
    w[0] = fp8x2_to_bf16<false>(q.x); w[1] = fp8x2_to_bf16<true>(q.x);
    w[2] = fp8x2_to_bf16<false>(q.y); w[3] = fp8x2_to_bf16<true>(q.y);
    w[4] = fp8x2_to_bf16<false>(q.z); w[5] = fp8x2_to_bf16<true>(q.z);
    w[6] = fp8x2_to_bf16<false>(q.w); w[7] = fp8x2_to_bf16<true>(q.w);
}

// 8 bf16 weight pairs . 16 bf16 activations (two uint4), accumulated into acc.
__device__ __forceinline__ float dot16(const bf16x2 (&w)[8], const uint4 x0, const uint4 x1, float acc) {
    acc = dot2(w[0], as_bf2(x0.x), acc);
    acc = dot2(w[1], as_bf2(x0.y), acc);
    acc = dot2(w[2], as_bf2(x0.z), acc);
    acc = dot2(w[3], as_bf2(x0.w), acc);
    acc = dot2(w[4], as_bf2(x1.x), acc);
    acc = dot2(w[5], as_bf2(x1.y), acc);
    acc = dot2(w[6], as_bf2(x1.z), acc);
    acc = dot2(w[7], as_bf2(x1.w), acc);
    return acc;
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over the 4 lanes of a quad; every lane of the quad gets the same bits.
__device__ __forceinline__ float quad_sum(float v) {
    v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
    v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
    return v;
}

// Sum over the 16 lanes of a DPP row; every lane of the row gets the same bits.
__device__ __forceinline__ float row16_sum(float v) {
    v = quad_sum(v);
    v += dpp<0x141>(v);  // row_half_mirror: combines the two quads of each half row
    v += dpp<0x140>(v);  // row_mirror: combines the two half rows
    return v;
}

// ------------------------------------------------------------ cross-lane helpers

// Order-preserving map of a float onto uint32 (larger float -> larger integer).
__device__ __forceinline__ uint32_t ordered(float v) {
    const uint32_t b = __float_as_uint(v);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float unordered(uint32_t o) {
    return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}

__device__ __forceinline__ float readlane(float v, int lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// Sum over the 64 lanes in a fixed order; the result is wave-uniform.
__device__ __forceinline__ float wave_sum(float v) {
    v = row16_sum(v);
    return ((readlane(v, 0) + readlane(v, 16)) + readlane(v, 32)) + readlane(v, 48);
}

template <int CTRL>
__device__ __forceinline__ uint32_t dppu(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

__device__ __forceinline__ void kmax_step(uint32_t &hi, uint32_t &lo, uint32_t oh, uint32_t ol) {
    const bool gt = oh > hi || (oh == hi && ol > lo);
    hi = gt ? oh : hi;
    lo = gt ? ol : lo;
}

// Largest 64-bit key over the 64 lanes (all lanes active); wave-uniform result.
__device__ __forceinline__ uint64_t wave_max_key(uint64_t k) {
    uint32_t hi = (uint32_t)(k >> 32), lo = (uint32_t)k;
    kmax_step(hi, lo, dppu<0xB1>(hi), dppu<0xB1>(lo));     // quad_perm [1,0,3,2]
    kmax_step(hi, lo, dppu<0x4E>(hi), dppu<0x4E>(lo));     // quad_perm [2,3,0,1]
    kmax_step(hi, lo, dppu<0x141>(hi), dppu<0x141>(lo));   // row_half_mirror
    kmax_step(hi, lo, dppu<0x140>(hi), dppu<0x140>(lo));   // row_mirror
    uint64_t best = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const uint64_t v = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)hi, 16 * r) << 32) |
                           (uint32_t)__builtin_amdgcn_readlane((int)lo, 16 * r);
        best = v > best ? v : best;
    }
    return best;
}

__device__ __forceinline__ int lanes_below(unsigned long long m) {
    return (int)__builtin_amdgcn_mbcnt_hi((unsigned)(m >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)m, 0u));
}

// Top-K selection by one wave for NT tokens at once. o[t][i] holds the order-preserving
// key of expert lane + 64 i of token t (0 where there is no expert). K rounds each take
// the largest remaining key over the wave (a DPP maximum and four lane reads) and select
// the lowest expert id holding it (the first 64-expert word with a lane equal to it, and
// that word's lowest such lane, picked with wave-uniform selects). On return bit i of
// sel[t] marks expert lane + 64 i as selected for token t, and wmax[t] is the first
// round's key (the token's largest). A round is a chain of dependent cross-lane steps, so
// the NT tokens' rounds are interleaved.
template <int NT, int NE>
__device__ __forceinline__ void topk_rounds(uint32_t (&o)[NT][NE], int K, int lane, unsigned (&sel)[NT],
                                            uint32_t (&wmax)[NT]) {
#pragma unroll
    for (int t = 0; t < NT; ++t) sel[t] = 0u;
    for (int k = 0; k < K; ++k) {
        uint32_t v[NT], W[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            v[t] = o[t][0];
#pragma unroll
            for (int i = 1; i < NE; ++i) v[t] = max(v[t], o[t][i]);
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) v[t] = max(v[t], dppu<0xB1>(v[t]));    // quad_perm [1,0,3,2]
#pragma unroll
        for (int t = 0; t < NT; ++t) v[t] = max(v[t], dppu<0x4E>(v[t]));    // quad_perm [2,3,0,1]
#pragma unroll
        for (int t = 0; t < NT; ++t) v[t] = max(v[t], dppu<0x141>(v[t]));   // row_half_mirror
#pragma unroll
        for (int t = 0; t < NT; ++t) v[t] = max(v[t], dppu<0x140>(v[t]));   // row_mirror
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            W[t] = max(max((uint32_t)__builtin_amdgcn_readlane((int)v[t], 0), (uint32_t)__builtin_amdgcn_readlane((int)v[t], 16)),
                       max((uint32_t)__builtin_amdgcn_readlane((int)v[t], 32), (uint32_t)__builtin_amdgcn_readlane((int)v[t], 48)));
            if (k == 0) wmax[t] = W[t];
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            unsigned long long bm[NE];
#pragma unroll
            for (int i = 0; i < NE; ++i) bm[i] = __ballot(o[t][i] == W[t]);
            int wsel = NE - 1;
            unsigned long long bw = bm[NE - 1];
#pragma unroll
            for (int i = NE - 2; i >= 0; --i) {
                wsel = bm[i] ? i : wsel;
                bw = bm[i] ? bm[i] : bw;
            }
            const int lsel = __ffsll((long long)bw) - 1;
#pragma unroll
            for (int i = 0; i < NE; ++i) {
                const bool take = i == wsel && lane == lsel;
                o[t][i] = take ? 0u : o[t][i];
                sel[t] |= take ? 1u << i : 0u;
            }
        }
    }
}

// Top-K selection by one wave for NT tokens at once, by bisection on the key value; same
// contract as topk_rounds. For each token, 32 steps from the top bit find T, the K-th
// largest key (the largest value with at least K keys at or above it): each step counts
// the keys at or above a trial value with one ballot and popcount per 64-expert word, all
// wave-uniform scalar work, and the NT tokens' chains are interleaved. Then every key
// above T is selected, and of the keys equal to T the lowest ids, as many as K still
// needs (the ids of word i are lane + 64 i, so the lowest ids are the lowest set bits of
// the lowest words). wmax[t] is the token's largest key (a DPP maximum).
template <int NT, int NE>
__device__ __forceinline__ void topk_bisect(const uint32_t (&o)[NT][NE], int K, int lane, unsigned (&sel)[NT],
                                            uint32_t (&wmax)[NT]) {
    uint32_t T[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) T[t] = 0u;
#pragma unroll 4
    for (int b = 31; b >= 0; --b) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const uint32_t trial = T[t] | (1u << b);
            int cnt = 0;
#pragma unroll
            for (int i = 0; i < NE; ++i) cnt += __popcll(__ballot(o[t][i] >= trial));
            T[t] = cnt >= K ? trial : T[t];
        }
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        int gt = 0;
        unsigned long long eq[NE];
#pragma unroll
        for (int i = 0; i < NE; ++i) {
            gt += __popcll(__ballot(o[t][i] > T[t]));
            eq[i] = __ballot(o[t][i] == T[t]);
        }
        const int need = K - gt;   // keys equal to T still to take (at least one)
        unsigned s = 0u;
        int before = 0;
#pragma unroll
        for (int i = 0; i < NE; ++i) {
            const bool take = o[t][i] > T[t] || (((eq[i] >> lane) & 1ull) && before + lanes_below(eq[i]) < need);
            s |= take ? 1u << i : 0u;
            before += __popcll(eq[i]);
        }
        sel[t] = s;
        uint32_t v = o[t][0];
#pragma unroll
        for (int i = 1; i < NE; ++i) v = max(v, o[t][i]);
        v = max(v, dppu<0xB1>(v));    // quad_perm [1,0,3,2]
        v = max(v, dppu<0x4E>(v));    // quad_perm [2,3,0,1]
        v = max(v, dppu<0x141>(v));   // row_half_mirror
        v = max(v, dppu<0x140>(v));   // row_mirror
        wmax[t] = max(max((uint32_t)__builtin_amdgcn_readlane((int)v, 0), (uint32_t)__builtin_amdgcn_readlane((int)v, 16)),
                      max((uint32_t)__builtin_amdgcn_readlane((int)v, 32), (uint32_t)__builtin_amdgcn_readlane((int)v, 48)));
    }
}

__device__ __forceinline__ float gelu_tanh(float z) {
    const float k0 = 0.7978845608028654f;  // sqrt(2/pi)
    return 0.5f * z * (1.0f + tanhf(k0 * (z + 0.044715f * z * z * z)));
}

}  // namespace dev
}  // namespace moe
