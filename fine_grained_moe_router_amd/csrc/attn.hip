// attn.hip -- one attention layer of the decode step with a KV cache (gfx950).
//
// Page "LLM decoding", "The exact architecture": 25 sliding-window layers and 5 global
// ones under grouped-query attention; "Where the 7.36 GB goes": q, k and o projections
// (no v projection: the cached key is also the value) holding about 966M parameters;
// "Lever 1" and "What we learned": an FP8 KV cache halves the KV reads. Per layer, four
// launches:
//   k_attn_proj    q = bf16(q_s (q_w u)) and k = bf16(k_s (k_w u)) for the M tokens, one
//                  GEMV over the two matrices' rows; the bf16 cache takes the new keys here
//   k_attn_part    per (KV head, tile of 16 queries, stripe of 16-position chunks): the
//                  scores of the tile's queries against the chunk's keys, an online softmax
//                  over the stripe, and the weighted key sum; a record (max, sum, 2 unused,
//                  acc[dh]) per query and stripe. The FP8 cache takes the new keys here (quantised once
//                  per (position, head) row by the workgroup whose chunk holds them).
//   k_attn_combine one workgroup per query: the stripes' records in stripe order -> o
//   k_attn_proj    out = bf16(o_s (o_w o))
// Queries of KV head g are ordered qi = m G + (h - g G) (token-major); token m sees the
// positions [lo_m, pos + m], lo_m = max(0, pos + m - window + 1) on sliding layers, 0 on
// global ones. The cache is a ring: position p in slot p mod capacity.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <type_traits>

#include "device_common.h"
#include "internal.h"
#include "pieces.h"

namespace moe {
namespace {

using namespace dev;

constexpr int kChunk = 16;       // positions per chunk: one per lane of a query's 16-lane row
constexpr int kQTile = 16;       // queries per k_attn_part workgroup

// E4M3FN code of an fp32 value: nearest, ties to even, saturating at 448 (0x7E); NaN 0x7F.
// Below 2^-6 the codes are m 2^-9; above, 2^E (1 + r/8 - 1) with r = rint(a 2^(3 - E)) in
// [8, 16]; both scalings are exact powers of two and rintf rounds to nearest even.
__device__ __forceinline__ uint32_t fp8_encode(float v) {
    if (v != v) return 0x7Fu;
    const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
    const float a = fabsf(v);
    if (a >= 448.0f) return sign | 0x7Eu;
    if (a < 0.015625f) return sign | (uint32_t)rintf(a * 512.0f);
    int E = (int)((__float_as_uint(a) >> 23) & 0xFFu) - 127;   // a is normal here
    int r = (int)rintf(a * __uint_as_float((uint32_t)(127 + 3 - E) << 23));
    if (r == 16) {
        r = 8;
        ++E;
    }
    if (E > 8 || (E == 8 && r > 14)) return sign | 0x7Eu;
    return sign | (uint32_t)(((E + 7) << 3) | (r - 8));
}

// value of an E4M3FN code (scale 1), via the hardware conversion (exact)
__device__ __forceinline__ float fp8_value(uint32_t code) { return fp8x2_to_f32<false>(code).x; }

// -------------------------------------------------------------------- projections

struct ProjArgs {
    const uint8_t *wa;   // rows [0, na): [na][K] FP8
    const float *sa;
    const uint8_t *wb;   // rows [na, na + nb): [nb][K] FP8 (nb may be 0)
    const float *sb;
    int na, nb, K, M;
    const uint16_t *x;   // [M][K] bf16
    uint16_t *outa;      // [M][na]
    uint16_t *outb;      // [M][nb]
    uint16_t *cache;     // bf16 cache to append the b rows to (rows g dh + d), or null
    int cap, dh, pos;
};

// Row n of the two stacked matrices against the M token vectors, staged in LDS a group of
// tokens at a time (at most 32 KiB); the row's pieces stay in registers across groups.
template <int LPR, int MAXCH>
__global__ __launch_bounds__(256) void k_attn_proj(ProjArgs a) {
    extern __shared__ uint4 xs[];
    const int tid = threadIdx.x, li = tid & (LPR - 1), n = blockIdx.x * (256 / LPR) + tid / LPR;
    const int ch = a.K / (16 * LPR);
    const bool in_b = n >= a.na;
    const uint8_t *row = in_b ? a.wb + (size_t)(n - a.na) * a.K : a.wa + (size_t)n * a.K;
    Pieces<LPR, MAXCH> w;
    w.load(row, li, ch);
    const float sc = in_b ? a.sb[n - a.na] : a.sa[n];
    const int tg = max(1, 16384 / a.K);   // tokens per LDS group (K bf16 each, 32 KiB)
    for (int m0 = 0; m0 < a.M; m0 += tg) {
        const int nt = min(tg, a.M - m0);
        __syncthreads();
        stage16(xs, reinterpret_cast<const uint4 *>(a.x + (size_t)m0 * a.K), nt * a.K / 8);
        __syncthreads();
        for (int t = 0; t < nt; ++t) {
            const float acc = group_sum<LPR>(w.dot_bf16(xs + (size_t)t * (a.K / 8), li, ch));
            if (li == 0) {
                const uint16_t v = f2bf(sc * acc);
                const int m = m0 + t;
                if (in_b) {
                    const int r = n - a.na;
                    a.outb[(size_t)m * a.nb + r] = v;
                    if (a.cache) {
                        const int g = r / a.dh, d = r - g * a.dh;
                        const int slot = (a.pos + m) % a.cap;
                        a.cache[((size_t)g * a.cap + slot) * a.dh + d] = v;
                    }
                } else {
                    a.outa[(size_t)m * a.na + n] = v;
                }
            }
        }
    }
}

// -------------------------------------------------------------------- attention

struct PartArgs {
    const uint16_t *q;      // [M][NQ] bf16
    const uint16_t *knew;   // [M][NK] bf16, the new keys
    void *cache;            // bf16 [nkv][cap][dh], or FP8 codes of that shape
    float *kscale;          // FP8: [nkv][cap]
    int fp8;
    int nkv, G, M, pos, window, cap, lo0, nch, nwg, Q, qsplit;
    float inv_sqrt;
    float *part;            // records [nkv][Q][nwg][dh + 4]: max, sum, -, -, acc[dh]
};

__device__ __forceinline__ float row16_max(float v) {
    v = fmaxf(v, dpp<0xB1>(v));
    v = fmaxf(v, dpp<0x4E>(v));
    v = fmaxf(v, dpp<0x141>(v));
    v = fmaxf(v, dpp<0x140>(v));
    return v;
}

// The block-wide maximum of one value per thread (256 threads), every thread gets it.
__device__ __forceinline__ float block_max(float v, float *red) {
    v = row16_max(v);
    v = fmaxf(v, __shfl_xor(v, 16));
    v = fmaxf(v, __shfl_xor(v, 32));
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// One (position, head) row of the FP8 cache, by the whole workgroup: thread t holds
// elements t and t + 256 of the bf16 row src[0..n) (n <= 512) in x[]; returns the row's
// scale max|x| / 448 (fp32 division), and code(i) = fp8_encode(x_i / scale) (0 when the
// row is zero) gives its codes.
__device__ __forceinline__ float fp8_row(const uint16_t *src, int n, float (&x)[2], float *red) {
    float amax = 0.0f;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const int d = threadIdx.x + 256 * e;
        x[e] = d < n ? bf2f(src[d]) : 0.0f;
        amax = fmaxf(amax, fabsf(x[e]));
    }
    return __fdiv_rn(block_max(amax, red), 448.0f);
}
// The same for a workgroup of NT threads (NT / 64 waves, red[] one entry per wave): thread t
// holds elements t, t + NT, ... (n <= 512).
template <int NT>
__device__ __forceinline__ float fp8_row_t(const uint16_t *src, int n, float (&x)[512 / NT], float *red) {
    float amax = 0.0f;
#pragma unroll
    for (int e = 0; e < 512 / NT; ++e) {
        const int d = threadIdx.x + NT * e;
        x[e] = d < n ? bf2f(src[d]) : 0.0f;
        amax = fmaxf(amax, fabsf(x[e]));
    }
    amax = row16_max(amax);
    amax = fmaxf(amax, __shfl_xor(amax, 16));
    amax = fmaxf(amax, __shfl_xor(amax, 32));
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
    __syncthreads();
    float m = red[0];
#pragma unroll
    for (int w = 1; w < NT / 64; ++w) m = fmaxf(m, red[w]);
    return __fdiv_rn(m, 448.0f);
}
__device__ __forceinline__ uint32_t fp8_row_code(float x, float scale) {
    return scale > 0.0f ? fp8_encode(__fdiv_rn(x, scale)) : 0u;
}

// A chunk's cached keys in registers: requested a chunk ahead of their use, so the loads of
// chunk c + nwg are in flight while chunk c is computed. bf16 cache: 16 B of a row per
// thread and request; FP8 cache: 16 codes per request and the row scale (threads 0..15).
// Positions past the last token (bf16) or from pos on (FP8: the new rows, quantised in the
// workgroup) read as zero; every address stays inside the cache (the position is clamped).
template <int DH, int NT = 256>
struct KStage {
    static constexpr int KB = DH + 8;
    static constexpr int NB = (kChunk * DH / 8 + NT - 1) / NT;
    static constexpr int N8 = (kChunk * DH / 16 + NT - 1) / NT;
    static constexpr int NV = NB > N8 ? NB : N8;
    uint4 v[NV];
    float sc;
    __device__ __forceinline__ void load(const PartArgs &a, int g, int p0, int last) {
        const int tid = threadIdx.x;
        const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
        if (!a.fp8) {
            const uint16_t *cb = reinterpret_cast<const uint16_t *>(a.cache);
#pragma unroll
            for (int e = 0; e < NB; ++e) {
                const int i = min(tid + NT * e, kChunk * DH / 8 - 1);
                const int j = i / (DH / 8), cc = i - j * (DH / 8), p = p0 + j;
                const uint4 t = reinterpret_cast<const uint4 *>(cb + ((size_t)g * a.cap + min(p, last) % a.cap) * DH)[cc];
                v[e] = p <= last ? t : zero;
            }
            sc = 1.0f;
        } else {
            const uint8_t *c8 = reinterpret_cast<const uint8_t *>(a.cache);
            const int lim = a.pos > 0 ? a.pos - 1 : 0;
#pragma unroll
            for (int e = 0; e < N8; ++e) {
                const int i = min(tid + NT * e, kChunk * DH / 16 - 1);
                const int j = i / (DH / 16), cc = i - j * (DH / 16), p = p0 + j;
                const uint4 t = reinterpret_cast<const uint4 *>(c8 + ((size_t)g * a.cap + min(p, lim) % a.cap) * DH)[cc];
                v[e] = p < a.pos ? t : zero;
            }
            const int p = p0 + (tid & (kChunk - 1));
            const float t = a.kscale[(size_t)g * a.cap + min(p, lim) % a.cap];
            sc = p < a.pos ? t : 0.0f;
        }
    }
    // the chunk as bf16 rows in LDS (the FP8 codes' values are exact in bf16) and its scales
    __device__ __forceinline__ void store(const PartArgs &a, uint4 *kb4, float *ksc) const {
        const int tid = threadIdx.x;
        if (!a.fp8) {
#pragma unroll
            for (int e = 0; e < NB; ++e) {
                const int i = tid + NT * e;
                if (i < kChunk * DH / 8) {
                    const int j = i / (DH / 8), cc = i - j * (DH / 8);
                    kb4[(j * KB) / 8 + cc] = v[e];
                }
            }
        } else {
#pragma unroll
            for (int e = 0; e < N8; ++e) {
                const int i = tid + NT * e;
                if (i < kChunk * DH / 16) {
                    const int j = i / (DH / 16), cc = i - j * (DH / 16);
                    const uint32_t vw[4] = {v[e].x, v[e].y, v[e].z, v[e].w};
                    uint32_t bw[8];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const f32x2 lo = fp8x2_to_f32<false>(vw[q]), hi = fp8x2_to_f32<true>(vw[q]);
                        bw[2 * q] = (__float_as_uint(lo.x) >> 16) | (__float_as_uint(lo.y) & 0xFFFF0000u);
                        bw[2 * q + 1] = (__float_as_uint(hi.x) >> 16) | (__float_as_uint(hi.y) & 0xFFFF0000u);
                    }
                    kb4[(j * KB) / 8 + 2 * cc] = make_uint4(bw[0], bw[1], bw[2], bw[3]);
                    kb4[(j * KB) / 8 + 2 * cc + 1] = make_uint4(bw[4], bw[5], bw[6], bw[7]);
                }
            }
        }
        if (tid < kChunk) ksc[tid] = sc;
    }
};

template <int DH>
__global__ __launch_bounds__(256) void k_attn_part(PartArgs a) {
    constexpr int KB = DH + 8;   // bf16 row stride of the staged keys (padding spreads the banks)
    __shared__ uint4 qs4[kQTile * DH / 8];
    __shared__ uint4 kb4[kChunk * KB / 8];
    __shared__ float pw[kQTile][kChunk];
    __shared__ float ksc[kChunk];
    __shared__ float red[4];
    uint16_t *kb = reinterpret_cast<uint16_t *>(kb4);

    const int tid = threadIdx.x, ql = tid >> 4, l = tid & 15;
    const int g = blockIdx.y / a.qsplit, s = blockIdx.y - g * a.qsplit, w = blockIdx.x;
    const int qi0 = s * kQTile, nql = min(kQTile, a.Q - qi0);
    const int NQ = a.G * a.nkv * DH, NK = a.nkv * DH;
    const int last = a.pos + a.M - 1;

    // the tile's queries
    for (int i = tid; i < kQTile * DH / 8; i += 256) {
        const int qq = i / (DH / 8), c = i - qq * (DH / 8);
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (qq < nql) {
            const int qi = qi0 + qq, m = qi / a.G, h = g * a.G + (qi - m * a.G);
            v = reinterpret_cast<const uint4 *>(a.q + (size_t)m * NQ + (size_t)h * DH)[c];
        }
        qs4[i] = v;
    }
    const bool active = ql < nql;
    const int my_m = active ? (qi0 + ql) / a.G : 0;
    const int hi_m = a.pos + my_m;
    const int lo_m = a.window > 0 ? max(0, hi_m - a.window + 1) : 0;

    float m_run = -INFINITY, l_run = 0.0f;
    float acc[DH / 16];
#pragma unroll
    for (int i = 0; i < DH / 16; ++i) acc[i] = 0.0f;

    uint8_t *c8 = reinterpret_cast<uint8_t *>(a.cache);
    KStage<DH> ks;
    if (w < a.nch) ks.load(a, g, a.lo0 + w * kChunk, last);
    for (int c = w; c < a.nch; c += a.nwg) {
        const int p0 = a.lo0 + c * kChunk;
        __syncthreads();
        ks.store(a, kb4, ksc);
        if (a.fp8) {
            // new positions in this chunk: quantise the key rows, store them, stage them
            const int jn0 = max(0, a.pos - p0), jn1 = min(kChunk, last - p0 + 1);
            for (int j = jn0; j < jn1; ++j) {
                const int p = p0 + j, m = p - a.pos;
                float x[2];
                const float scale = fp8_row(a.knew + (size_t)m * NK + (size_t)g * DH, DH, x, red);
                const size_t slot = (size_t)g * a.cap + p % a.cap;
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const int d = tid + 256 * e;
                    if (d < DH) {
                        const uint32_t code = fp8_row_code(x[e], scale);
                        const float v = fp8_value(code);
                        if (s == 0) c8[slot * DH + d] = (uint8_t)code;
                        kb[j * KB + d] = (uint16_t)(__float_as_uint(v) >> 16);
                    }
                }
                if (tid == 0) {
                    ksc[j] = scale;
                    if (s == 0) a.kscale[slot] = scale;
                }
            }
        }
        __syncthreads();
        if (c + a.nwg < a.nch) ks.load(a, g, p0 + a.nwg * kChunk, last);
        // scores: lane l of query ql takes position p0 + l
        float pj = 0.0f, alpha = 1.0f;
        if (active) {
            const uint4 *qr = qs4 + ql * (DH / 8);
            const uint4 *kr = kb4 + (l * KB) / 8;
            float d = 0.0f;
#pragma unroll 8
            for (int cc = 0; cc < DH / 8; ++cc) {
                const uint4 qv = qr[cc], kv = kr[cc];
                d = dot2(as_bf2(qv.x), as_bf2(kv.x), d);
                d = dot2(as_bf2(qv.y), as_bf2(kv.y), d);
                d = dot2(as_bf2(qv.z), as_bf2(kv.z), d);
                d = dot2(as_bf2(qv.w), as_bf2(kv.w), d);
            }
            const int p = p0 + l;
            const bool valid = p >= lo_m && p <= hi_m;
            const float sc = valid ? d * ksc[l] * a.inv_sqrt : -INFINITY;
            const float m_new = fmaxf(m_run, row16_max(sc));
            if (m_new != -INFINITY) {
                alpha = expf(m_run - m_new);
                pj = valid ? expf(sc - m_new) : 0.0f;
                l_run = l_run * alpha + row16_sum(pj);
                m_run = m_new;
            }
            pw[ql][l] = pj * ksc[l];
        }
        __syncthreads();
        // weighted key sum: lane l holds dims l 8 + 128 k + e (e < 8)
        if (active) {
#pragma unroll
            for (int i = 0; i < DH / 16; ++i) acc[i] *= alpha;
            for (int j = 0; j < kChunk; ++j) {
                const float wj = pw[ql][j];
                const uint4 *kr = kb4 + (j * KB) / 8 + l;
#pragma unroll
                for (int k = 0; k < DH / 128; ++k) {
                    const uint4 v = kr[16 * k];
                    const uint32_t vw[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        acc[8 * k + 2 * e] = fmaf(wj, __uint_as_float(vw[e] << 16), acc[8 * k + 2 * e]);
                        acc[8 * k + 2 * e + 1] = fmaf(wj, __uint_as_float(vw[e] & 0xFFFF0000u), acc[8 * k + 2 * e + 1]);
                    }
                }
            }
        }
    }
    if (active) {
        float *rec = a.part + (((size_t)g * a.Q + qi0 + ql) * a.nwg + w) * (DH + 4);
        if (l == 0) {
            rec[0] = m_run;
            rec[1] = l_run;
        }
#pragma unroll
        for (int k = 0; k < DH / 128; ++k) {
            *reinterpret_cast<float4 *>(rec + 4 + l * 8 + 128 * k) =
                make_float4(acc[8 * k], acc[8 * k + 1], acc[8 * k + 2], acc[8 * k + 3]);
            *reinterpret_cast<float4 *>(rec + 4 + l * 8 + 128 * k + 4) =
                make_float4(acc[8 * k + 4], acc[8 * k + 5], acc[8 * k + 6], acc[8 * k + 7]);
        }
    }
}

// ------------------------------------------------- attention on the matrix cores

// The same partial softmax as k_attn_part for every query of one KV head at once, as small
// dense contractions on gfx950's matrix cores (v_mfma_f32_16x16x32_bf16: lane l holds row
// l % 16, k 8 (l / 16) .. + 7 of A, k 8 (l / 16) .. + 7, column l % 16 of B, and rows
// 4 (l / 16) .. + 3, column l % 16 of C). Per 32-position chunk of the stripe:
//   S = Q K^T        wave v < 4 takes query tile v (16 queries, its A operands held in
//                    registers for the whole stripe) against both 16-position halves of the
//                    chunk, while waves 4..7 write the transposed copy of the chunk
//   softmax          each lane owns four query rows of S; the row maximum and sum go over the
//                    16 lanes of its DPP row; the weights p (times the FP8 row scale) are
//                    split into bf16 high and low parts (16 bits of mantissa together)
//   O += P V         wave v takes an eighth of the head's 16-dimension tiles for every query
//                    tile, V being the chunk's keys (the cached key is also the value), read
//                    from the transposed copy; a tile's accumulators are rescaled only when
//                    one of its rows' maxima moved
// Eight waves (two per SIMD) so that one wave's LDS and matrix latencies hide behind another's.
// The records have k_attn_part's layout, so k_attn_combine finishes both. Bf16 products are
// exact in fp32; the sums run in the matrix cores' order (fixed, so the result does not
// depend on timing).
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f32x4_t mma16(const uint4 a, const uint4 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                    0, 0, 0);
}
constexpr int kMmaChunk = 32;    // positions per chunk
constexpr int kMmaMaxQt = 4;     // query tiles of 16 (one per wave)

template <int DH>
struct MmaLds {
    static constexpr int KB = DH + 8;          // [position][dimension] row stride (bf16)
    static constexpr int TB = kMmaChunk + 8;   // [dimension][position] and [query][position] row stride
    uint16_t kp[kMmaChunk * KB];
    uint16_t kt[DH * TB];
    uint16_t ph[16 * kMmaMaxQt * TB];
    uint16_t pl[16 * kMmaMaxQt * TB];
    float al[16 * kMmaMaxQt];
    float ksc[kMmaChunk];
    float red[8];
};
constexpr int kMmaThreads = 512;

template <int DH>
__global__ __launch_bounds__(kMmaThreads, 2) void k_attn_part_mma(PartArgs a) {
    using LDS = MmaLds<DH>;
    constexpr int NT = kMmaThreads, KB = LDS::KB, TB = LDS::TB, NKK = DH / 32, DTW = DH / 16 / (NT / 64);
    __shared__ __align__(16) LDS L;
    uint4 *kb4 = reinterpret_cast<uint4 *>(L.kp);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, r16 = lane & 15, k8 = lane >> 4;
    const int g = blockIdx.y, w = blockIdx.x;
    const int Q = a.Q, Qt = (Q + 15) / 16;
    const int NQ = a.G * a.nkv * DH, NK = a.nkv * DH;
    const int last = a.pos + a.M - 1;
    const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
    const bool sw = wave < Qt;   // this wave scores query tile `wave`

    // query tile `wave`: A operands of every 32-dimension step, and the rows' token bounds
    uint4 qa[NKK];
    float m_run[4], l_run[4];
    int lo_r[4], hi_r[4];
    bool rv[4];
    {
        const int qi = wave * 16 + r16;
        const bool on = sw && qi < Q;
        const int m = on ? qi / a.G : 0, h = g * a.G + (on ? qi - m * a.G : 0);
        const uint16_t *qp = a.q + (size_t)m * NQ + (size_t)h * DH + 8 * k8;
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) qa[kk] = on ? *reinterpret_cast<const uint4 *>(qp + 32 * kk) : zero;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = wave * 16 + 4 * k8 + i;
            rv[i] = sw && r < Q;
            const int tok = rv[i] ? r / a.G : 0;
            hi_r[i] = a.pos + tok;
            lo_r[i] = a.window > 0 ? max(0, hi_r[i] - a.window + 1) : 0;
            m_run[i] = -INFINITY;
            l_run[i] = 0.0f;
        }
    }
    f32x4_t o[kMmaMaxQt][DTW];
#pragma unroll
    for (int mt = 0; mt < kMmaMaxQt; ++mt)
#pragma unroll
        for (int j = 0; j < DTW; ++j) o[mt][j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

    uint8_t *c8 = reinterpret_cast<uint8_t *>(a.cache);
    KStage<DH, NT> k0, k1;
    if (w < a.nch) {
        k0.load(a, g, a.lo0 + w * kMmaChunk, last);
        k1.load(a, g, a.lo0 + w * kMmaChunk + kChunk, last);
    }
    for (int c = w; c < a.nch; c += a.nwg) {
        const int p0 = a.lo0 + c * kMmaChunk;
        // the chunk's keys as bf16 rows [position][dimension] and their scales
        k0.store(a, kb4, L.ksc);
        k1.store(a, kb4 + kChunk * KB / 8, L.ksc + kChunk);
        if (a.fp8) {
            // new positions in this chunk: quantise the key rows, store them, stage them
            __syncthreads();
            const int jn0 = max(0, a.pos - p0), jn1 = min(kMmaChunk, last - p0 + 1);
            for (int j = jn0; j < jn1; ++j) {
                const int p = p0 + j, m = p - a.pos;
                float x[512 / NT];
                const float scale = fp8_row_t<NT>(a.knew + (size_t)m * NK + (size_t)g * DH, DH, x, L.red);
                const size_t slot = (size_t)g * a.cap + p % a.cap;
#pragma unroll
                for (int e = 0; e < 512 / NT; ++e) {
                    const int d = tid + NT * e;
                    if (d < DH) {
                        const uint32_t code = fp8_row_code(x[e], scale);
                        c8[slot * DH + d] = (uint8_t)code;
                        L.kp[j * KB + d] = (uint16_t)(__float_as_uint(fp8_value(code)) >> 16);
                    }
                }
                if (tid == 0) {
                    L.ksc[j] = scale;
                    a.kscale[slot] = scale;
                }
            }
        }
        __syncthreads();
        // the next chunk's keys are requested now, so they arrive during this one
        if (c + a.nwg < a.nch) {
            k0.load(a, g, p0 + a.nwg * kMmaChunk, last);
            k1.load(a, g, p0 + a.nwg * kMmaChunk + kChunk, last);
        }
        if (wave >= 4) {
            // the transposed copy [dimension][position] for the V operand
            for (int i = tid - 256; i < kMmaChunk * DH / 8; i += NT - 256) {
                const int pp = i % kMmaChunk, d0 = 8 * (i / kMmaChunk);
                const uint4 v = *reinterpret_cast<const uint4 *>(L.kp + pp * KB + d0);
                const uint32_t vw[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    L.kt[(d0 + 2 * e) * TB + pp] = (uint16_t)(vw[e] & 0xffffu);
                    L.kt[(d0 + 2 * e + 1) * TB + pp] = (uint16_t)(vw[e] >> 16);
                }
            }
        } else if (sw) {
            // scores of query tile `wave` against positions p0 + r16 and p0 + 16 + r16
            f32x4_t s0 = {0.0f, 0.0f, 0.0f, 0.0f}, s1 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) {
                const uint4 b0 = *reinterpret_cast<const uint4 *>(L.kp + r16 * KB + 32 * kk + 8 * k8);
                const uint4 b1 = *reinterpret_cast<const uint4 *>(L.kp + (kChunk + r16) * KB + 32 * kk + 8 * k8);
                s0 = mma16(qa[kk], b0, s0);
                s1 = mma16(qa[kk], b1, s1);
            }
            const int pA = p0 + r16, pB = p0 + kChunk + r16;
            const float scA = L.ksc[r16] * a.inv_sqrt, scB = L.ksc[kChunk + r16] * a.inv_sqrt;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = wave * 16 + 4 * k8 + i;
                const bool vA = rv[i] && pA >= lo_r[i] && pA <= hi_r[i];
                const bool vB = rv[i] && pB >= lo_r[i] && pB <= hi_r[i];
                const float sA = vA ? s0[i] * scA : -INFINITY, sB = vB ? s1[i] * scB : -INFINITY;
                const float m_new = fmaxf(m_run[i], row16_max(fmaxf(sA, sB)));
                const bool live = m_new != -INFINITY;
                const float alpha = live ? expf(m_run[i] - m_new) : 1.0f;
                const float eA = vA && live ? expf(sA - m_new) : 0.0f;
                const float eB = vB && live ? expf(sB - m_new) : 0.0f;
                l_run[i] = l_run[i] * alpha + row16_sum(eA + eB);
                m_run[i] = m_new;
                // the weights with the FP8 row scale, as bf16 high and low parts
                const float wA = eA * L.ksc[r16], wB = eB * L.ksc[kChunk + r16];
                const uint16_t hA = f2bf(wA), hB = f2bf(wB);
                L.ph[r * TB + r16] = hA;
                L.ph[r * TB + kChunk + r16] = hB;
                L.pl[r * TB + r16] = f2bf(wA - bf2f(hA));
                L.pl[r * TB + kChunk + r16] = f2bf(wB - bf2f(hB));
                if (r16 == 0) L.al[r] = alpha;
            }
        }
        __syncthreads();
        // O += P V over this wave's dimension tiles
#pragma unroll
        for (int mt = 0; mt < kMmaMaxQt; ++mt) {
            if (mt < Qt) {
                const float4 al = *reinterpret_cast<const float4 *>(L.al + mt * 16 + 4 * k8);
                const uint4 ah = *reinterpret_cast<const uint4 *>(L.ph + (mt * 16 + r16) * TB + 8 * k8);
                const uint4 alo = *reinterpret_cast<const uint4 *>(L.pl + (mt * 16 + r16) * TB + 8 * k8);
                // a row's accumulators change only when its maximum moved (alpha != 1)
                const bool rescale = __any(al.x != 1.0f || al.y != 1.0f || al.z != 1.0f || al.w != 1.0f);
#pragma unroll
                for (int j = 0; j < DTW; ++j) {
                    const int dt = wave * DTW + j;
                    const uint4 bv = *reinterpret_cast<const uint4 *>(L.kt + (dt * 16 + r16) * TB + 8 * k8);
                    f32x4_t acc = o[mt][j];
                    if (rescale) {
                        acc[0] *= al.x;
                        acc[1] *= al.y;
                        acc[2] *= al.z;
                        acc[3] *= al.w;
                    }
                    acc = mma16(ah, bv, acc);
                    o[mt][j] = mma16(alo, bv, acc);
                }
            }
        }
        __syncthreads();
    }
    // records: (max, sum, -, -, acc[DH]) per query, in k_attn_part's layout
    const size_t R = DH + 4;
    float *recs = a.part + ((size_t)g * a.Q * a.nwg + w) * R;   // query q at recs + q nwg R
    if (sw && r16 == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = wave * 16 + 4 * k8 + i;
            if (r < Q) {
                recs[(size_t)r * a.nwg * R] = m_run[i];
                recs[(size_t)r * a.nwg * R + 1] = l_run[i];
            }
        }
    }
#pragma unroll
    for (int mt = 0; mt < kMmaMaxQt; ++mt) {
        if (mt < Qt) {
#pragma unroll
            for (int j = 0; j < DTW; ++j) {
                const int d = (wave * DTW + j) * 16 + r16;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = mt * 16 + 4 * k8 + i;
                    if (r < Q) recs[(size_t)r * a.nwg * R + 4 + d] = o[mt][j][i];
                }
            }
        }
    }
}

struct CombArgs {
    const float *part;
    int nkv, G, Q, nwg, dh;
    uint16_t *o;       // [M][NQ] bf16 (workspace)
    uint16_t *o_user;  // or null
};

// Query (g, qi), dims 64 b .. 64 b + 63 (b = blockIdx.y): the stripes' records combined,
//   mx = max_w m_w, L = sum_w l_w e^(m_w - mx), o = sum_w acc_w e^(m_w - mx) / L,
// every sum in a fixed order (thread t takes stripes t, t + 256, ... in turn, then a fixed
// tree over the threads; wave v takes stripes v, v + 4, ... for the outputs, eight records
// requested at a time, then the four waves in turn), so the result does not depend on timing.
__global__ __launch_bounds__(256) void k_attn_combine(CombArgs a) {
    __shared__ float wt[kAttnMaxWG];
    __shared__ float po[4][64];
    __shared__ float red[4];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int g = blockIdx.x / a.Q, qi = blockIdx.x - g * a.Q, d = 64 * blockIdx.y + lane;
    const int R = a.dh + 4;
    const float *rec = a.part + ((size_t)g * a.Q + qi) * a.nwg * R;
    const float *col = rec + 4 + d;
    // Every load of the first pass is issued at once: this thread's stripes' (max, sum) pairs
    // (stripes t and t + 256) and the wave's first eight output values (stripes v, v + 4, ...,
    // v + 28), so that a stripe count up to 32 costs one memory latency.
    static_assert(kAttnMaxWG <= 512, "two stripes per thread");
    float mv[2], lv[2], v0[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const int w = wv + 4 * k;
        v0[k] = w < a.nwg ? col[(size_t)w * R] : 0.0f;
    }
#pragma unroll
    for (int j2 = 0; j2 < 2; ++j2) {
        const int w = tid + 256 * j2;
        mv[j2] = w < a.nwg ? rec[(size_t)w * R] : -INFINITY;
        lv[j2] = w < a.nwg ? rec[(size_t)w * R + 1] : 0.0f;
    }
    const float mx = block_max(fmaxf(mv[0], mv[1]), red);
    float ls = 0.0f;
#pragma unroll
    for (int j2 = 0; j2 < 2; ++j2) {
        const int w = tid + 256 * j2;
        if (w < a.nwg) {
            const float e = mv[j2] == -INFINITY ? 0.0f : expf(mv[j2] - mx);
            wt[w] = e;
            ls = fmaf(lv[j2], e, ls);
        }
    }
    ls = row16_sum(ls);
    ls += __shfl_xor(ls, 16);
    ls += __shfl_xor(ls, 32);
    __syncthreads();
    if (lane == 0) red[wv] = ls;
    __syncthreads();
    const float L = (red[0] + red[1]) + (red[2] + red[3]);
    // the weighted sum over the wave's stripes, in stripe order: the prefetched eight, then
    // eight records requested at a time
    float acc = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const int w = wv + 4 * k;
        if (w < a.nwg) acc = fmaf(v0[k], wt[w], acc);
    }
    int w = wv + 32;
    for (; w + 28 < a.nwg; w += 32) {
        float v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = col[(size_t)(w + 4 * k) * R];
#pragma unroll
        for (int k = 0; k < 8; ++k) acc = fmaf(v[k], wt[w + 4 * k], acc);
    }
    for (; w < a.nwg; w += 4) acc = fmaf(col[(size_t)w * R], wt[w], acc);
    po[wv][lane] = acc;
    __syncthreads();
    if (tid < 64) {
        const int m = qi / a.G, h = g * a.G + (qi - m * a.G), NQ = a.G * a.nkv * a.dh;
        const float o = ((po[0][tid] + po[1][tid]) + po[2][tid]) + po[3][tid];
        const uint16_t v = f2bf(o / L);
        a.o[(size_t)m * NQ + (size_t)h * a.dh + d] = v;
        if (a.o_user) a.o_user[(size_t)m * NQ + (size_t)h * a.dh + d] = v;
    }
}

// -------------------------------------------------------------------- cache writes

// Row (position first + i, head g) of the cache from bf16 keys k [n][nkv][dh].
__global__ __launch_bounds__(256) void k_kv_write(const uint16_t *k, int first, int nkv, int dh, int cap, int fp8,
                                                  void *cache, float *kscale) {
    __shared__ float red[4];
    const int i = blockIdx.x / nkv, g = blockIdx.x - i * nkv, tid = threadIdx.x;
    const uint16_t *src = k + ((size_t)i * nkv + g) * dh;
    const size_t slot = (size_t)g * cap + (first + i) % cap;
    if (!fp8) {
        uint16_t *dst = reinterpret_cast<uint16_t *>(cache) + slot * dh;
        for (int d = tid; d < dh; d += 256) dst[d] = src[d];
        return;
    }
    float x[2];
    const float scale = fp8_row(src, dh, x, red);
    uint8_t *dst = reinterpret_cast<uint8_t *>(cache) + slot * dh;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const int d = tid + 256 * e;
        if (d < dh) dst[d] = (uint8_t)fp8_row_code(x[e], scale);
    }
    if (tid == 0) kscale[slot] = scale;
}

inline hipStream_t S(void *p) { return reinterpret_cast<hipStream_t>(p); }

template <int V>
using IC = std::integral_constant<int, V>;

template <class F>
bool by_dh(int dh, F f) {
    switch (dh) {
        case 128: f(IC<128>{}); return true;
        case 256: f(IC<256>{}); return true;
        case 512: f(IC<512>{}); return true;
        default: return false;
    }
}

template <class F>
void by_lpr(int lpr, F f) {
    if (lpr == 16) f(IC<16>{});
    else if (lpr == 32) f(IC<32>{});
    else f(IC<64>{});
}

int launch_proj(const ProjArgs &a, void *stream) {
    const int rows = a.na + a.nb;
    const int lpr = draft_lpr(rows, a.K, kDraftMaxCh);
    if (!lpr || rows % (256 / lpr)) return MOE_EINVAL;
    const size_t lds = (size_t)min(a.M, max(1, 16384 / a.K)) * a.K * 2;
    by_lpr(lpr, [&](auto L) {
        constexpr int l = decltype(L)::value;
        hipLaunchKernelGGL((k_attn_proj<l, kDraftMaxCh>), dim3(rows * l / 256), dim3(256), lds, S(stream), a);
    });
    return MOE_OK;
}

}  // namespace

int launch_kv_write(const moe_attn_desc &d, int first_pos, int n, const uint16_t *k, char *cache, void *stream) {
    (void)hipGetLastError();
    const AttnCache C = attn_cache(d);
    hipLaunchKernelGGL(k_kv_write, dim3(n * d.kv_heads), dim3(256), 0, S(stream), k, first_pos, d.kv_heads, d.head_dim,
                       d.capacity, d.kv_type == MOE_KV_FP8 ? 1 : 0, (void *)cache,
                       reinterpret_cast<float *>(cache + C.scales));
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ELAUNCH;
}

int launch_attn_decode(const moe_attn_desc &d, const moe_attn_weights &w, int M, int pos, const uint16_t *u,
                       char *cache, uint16_t *out, uint16_t *o_user, char *ws, void *stream) {
    (void)hipGetLastError();
    const AttnPlan P = attn_plan(d, M, pos);
    const AttnWs W = attn_ws(d, M);
    const AttnCache C = attn_cache(d);
    const int NQ = d.q_heads * d.head_dim, NK = d.kv_heads * d.head_dim;
    const bool fp8 = d.kv_type == MOE_KV_FP8;
    uint16_t *q = reinterpret_cast<uint16_t *>(ws + W.q), *k = reinterpret_cast<uint16_t *>(ws + W.k);
    uint16_t *o = reinterpret_cast<uint16_t *>(ws + W.o);
    float *part = reinterpret_cast<float *>(ws + W.part);

    ProjArgs pa{w.q_w, w.q_s, w.k_w, w.k_s, NQ, NK, d.hidden, M, u, q, k,
                fp8 ? nullptr : reinterpret_cast<uint16_t *>(cache), d.capacity, d.head_dim, pos};
    int rc = launch_proj(pa, stream);
    if (rc != MOE_OK) return rc;

    PartArgs ta{q, k, cache, reinterpret_cast<float *>(cache + C.scales), fp8 ? 1 : 0, d.kv_heads, P.G, M, pos,
                d.window, d.capacity, P.lo0, P.nch, P.nwg, P.Q, P.qsplit, 1.0f / sqrtf((float)d.head_dim), part};
    int nwg = P.nwg;
    if (P.Q <= 16 * kMmaMaxQt && (d.head_dim == 512 || (d.head_dim == 256 && P.Q >= 8))) {
        // 512-wide heads (the global layers) with at most four tiles of queries per KV head:
        // every query of a KV head in one workgroup, on the matrix cores, 32-position chunks;
        // as many stripes per KV head as the records allow. A single token's 8 queries per KV
        // head fill half a tile and still run faster here than on the vector units (32K
        // context: 55.3 against 85.5 us per layer). 256-wide heads (the sliding layers, 2 query
        // heads per KV head) take it from 8 queries per KV head (M >= 4): at M = 5 the 30-layer
        // attention step measured 2-3 % faster with it, at M = 1 (2 queries) 2-4 % slower.
        int dev = 0, cus = 0;
        if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return MOE_ELAUNCH;
        const int nch = (pos + M - P.lo0 + kMmaChunk - 1) / kMmaChunk;
        const int cap = std::max(1, std::min({kAttnMaxWG, kAttnRecords / (d.kv_heads * P.Q), cus / d.kv_heads}));
        nwg = std::min(nch, cap);
        ta.nch = nch;
        ta.nwg = nwg;
        ta.qsplit = 1;
        if (d.head_dim == 512)
            hipLaunchKernelGGL((k_attn_part_mma<512>), dim3(nwg, d.kv_heads), dim3(kMmaThreads), 0, S(stream), ta);
        else
            hipLaunchKernelGGL((k_attn_part_mma<256>), dim3(nwg, d.kv_heads), dim3(kMmaThreads), 0, S(stream), ta);
    } else if (!by_dh(d.head_dim, [&](auto D) {
                   constexpr int dh = decltype(D)::value;
                   hipLaunchKernelGGL((k_attn_part<dh>), dim3(P.nwg, d.kv_heads * P.qsplit), dim3(256), 0, S(stream), ta);
               })) {
        return MOE_EINVAL;
    }

    CombArgs ca{part, d.kv_heads, P.G, P.Q, nwg, d.head_dim, o, o_user};
    hipLaunchKernelGGL(k_attn_combine, dim3(d.kv_heads * P.Q, d.head_dim / 64), dim3(256), 0, S(stream), ca);

    ProjArgs po{w.o_w, w.o_s, nullptr, nullptr, d.hidden, 0, NQ, M, o, out, nullptr, nullptr, 0, 0, 0};
    rc = launch_proj(po, stream);
    if (rc != MOE_OK) return rc;
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ELAUNCH;
}

}  // namespace moe
