// sample.hip -- stochastic speculative acceptance on the lm_head logits (gfx950).
//
// Page "LLM decoding", "What we learned, and where this goes": a drafted token is kept
// only if it passes the distribution the target would have sampled from, and a rejected
// one falls back to a real model step, so the output is distributed as ordinary decoding
// (the temperature-0.7 column of "The ladder, every rung"). The rule taken:
//   p_i = softmax(logits_i / T); draft d_i (drawn from the drafter's q_i) is kept iff
//   u_i q_i(d_i) < p_{i-1}(d_i); at the first rejection (row n) the last token is drawn
//   from max(0, p_n - q_{n+1}), after gamma acceptances from p_gamma (the bonus token).
// The draw is the Gumbel-max rule, argmax_v log r_v - log(-log U_v), with U_v from
// Philox4x32-10 (Salmon et al., SC 2011) on a counter of (v / 4, row, step), keyed by the
// seed: a parallel argmax over the vocabulary instead of a prefix scan, and a decision
// whose margin (the gap between the two largest perturbed values) is of order one.
//
// Kernels, after k_lmhead<true> has written every logit:
//   k_sample_stats   V / 1024 workgroups: per 1024-entry chunk and row, the maximum of
//                    logit / T and the sum of exp(logit / T - maximum)
//   k_sample_accept  one workgroup: log normalisers of all rows, the accept tests -> n
//   k_sample_draw    V / 1024 workgroups, 4 entries per thread (one Philox call): the
//                    residual (or bonus) candidates' perturbed values -> per-workgroup keys
//   k_sample_final   one workgroup: the largest key -> the token; the outputs.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "internal.h"

namespace moe {
namespace {

using namespace dev;

struct SampleArgs {
    const float *logits;    // [M][V]
    float2 *stats;          // [nsg][M]: (maximum, sum) per chunk and row
    const int32_t *draft;   // [gamma]
    const float *q;         // [gamma][V]
    const float *u_acc;     // [gamma]
    int *acc;               // n, then float logZ[M]
    unsigned long long *keys;   // [nsg][2]
    int32_t *accepted_len;
    int32_t *out_tokens;
    uint64_t seed, step;
    float inv_t;
    int M, V, nwg, nsg;
};

// Philox4x32-10: ten rounds of (hi(M0 c0) ^ c1 ^ k0, lo(M1 c2), hi(M1 c2) ^ c3 ^ k1, lo(M0 c0)),
// the key advanced by the Weyl constants between rounds.
__device__ __forceinline__ uint4 philox4x32_10(uint4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        const uint32_t lo0 = 0xD2511F53u * c.x, hi0 = __umulhi(0xD2511F53u, c.x);
        const uint32_t lo1 = 0xCD9E8D57u * c.z, hi1 = __umulhi(0xCD9E8D57u, c.z);
        c = make_uint4(hi1 ^ c.y ^ k0, lo1, hi0 ^ c.w ^ k1, lo0);
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    return c;
}

// -log(-log U) for U = (w + 1/2) / 2^32. -log U is formed from whichever of U and 1 - U is
// small, each exact up to one rounding, so the value keeps its relative precision near
// both ends (near U = 1 through log1p of the exact complement).
__device__ __forceinline__ float gumbel(uint32_t w) {
    constexpr float k2m32 = 2.3283064365386963e-10f;   // 2^-32
    float e;
    if (w >= 0x80000000u)
        e = -log1pf(-(((float)(~w) + 0.5f) * k2m32));
    else
        e = -logf(((float)w + 0.5f) * k2m32);
    return -logf(e);
}

__device__ __forceinline__ unsigned long long key_of(float val, int v) {
    return ((unsigned long long)ordered(val) << 32) | (unsigned long long)(0xffffffffu - (uint32_t)v);
}

__device__ __forceinline__ float wave_max_f(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}
__device__ __forceinline__ float wave_sum_f(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// Chunk b (entries 1024 b ..): per row, the maximum of logit / T over the chunk and the
// sum of exp(logit / T - maximum); thread t holds entries 1024 b + 4 t .. + 3.
__global__ __launch_bounds__(256) void k_sample_stats(SampleArgs a) {
    __shared__ float wm[4][kMaxM], ws[4][kMaxM];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, M = a.M;
    const int v0 = (blockIdx.x * 256 + tid) * 4;
    float4 l4[kMaxM];
#pragma unroll
    for (int m = 0; m < kMaxM; ++m)
        if (m < M) l4[m] = v0 < a.V ? *reinterpret_cast<const float4 *>(a.logits + (size_t)m * a.V + v0)
                                    : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
#pragma unroll
    for (int m = 0; m < kMaxM; ++m) {
        if (m < M) {
            const float z = wave_max_f(fmaxf(fmaxf(l4[m].x, l4[m].y), fmaxf(l4[m].z, l4[m].w)) * a.inv_t);
            if (lane == 0) wm[wave][m] = z;
        }
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < kMaxM; ++m) {
        if (m < M) {
            const float mx = fmaxf(fmaxf(wm[0][m], wm[1][m]), fmaxf(wm[2][m], wm[3][m]));
            float e = 0.0f;
            if (v0 < a.V)
                e = (__expf(l4[m].x * a.inv_t - mx) + __expf(l4[m].y * a.inv_t - mx)) +
                    (__expf(l4[m].z * a.inv_t - mx) + __expf(l4[m].w * a.inv_t - mx));
            e = wave_sum_f(e);
            if (lane == 0) ws[wave][m] = e;
        }
    }
    __syncthreads();
    if (tid < M) {
        const int m = tid;
        const float mx = fmaxf(fmaxf(wm[0][m], wm[1][m]), fmaxf(wm[2][m], wm[3][m]));
        a.stats[(size_t)blockIdx.x * M + m] = make_float2(mx, (ws[0][m] + ws[1][m]) + (ws[2][m] + ws[3][m]));
    }
}

// log normaliser of every row from the chunks' states (wave w combines rows w and w + 4),
// then the accept tests
__global__ __launch_bounds__(256) void k_sample_accept(SampleArgs a) {
    __shared__ float logz[kMaxM];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, M = a.M;
    for (int m = wave; m < M; m += 4) {
        float mx = -INFINITY;
        for (int i = lane; i < a.nsg; i += 64) mx = fmaxf(mx, a.stats[(size_t)i * M + m].x);
        mx = wave_max_f(mx);
        float sm = 0.0f;
        for (int i = lane; i < a.nsg; i += 64) {
            const float2 st = a.stats[(size_t)i * M + m];
            sm += st.y * __expf(st.x - mx);
        }
        sm = wave_sum_f(sm);
        if (lane == 0) logz[m] = mx + logf(sm);
    }
    __syncthreads();
    if (tid == 0) {
        const int gamma = M - 1;
        int n = 0;
        while (n < gamma) {
            const int d = a.draft[n];
            if (d < 0 || d >= a.V) break;
            const float lp = a.logits[(size_t)n * a.V + d] * a.inv_t - logz[n];
            const float lq = logf(a.u_acc[n] * a.q[(size_t)n * a.V + d]);
            if (!(lq < lp)) break;
            ++n;
        }
        a.acc[0] = n;
        float *lz = reinterpret_cast<float *>(a.acc + 1);
        for (int m = 0; m < M; ++m) lz[m] = logz[m];
    }
}

// Sampling workgroup b: entries 1024 b + 4 t .. + 3 for thread t. Keys: the residual
// candidates' best (0 if none) and the target row's best (for the bonus token, and for a
// residual that is zero everywhere).
__global__ __launch_bounds__(256) void k_sample_draw(SampleArgs a) {
    __shared__ unsigned long long kr[256], kp[256];
    const int tid = threadIdx.x;
    const int n = a.acc[0];
    const float lz = reinterpret_cast<const float *>(a.acc + 1)[n];
    const bool residual = n < a.M - 1;
    const int v0 = (blockIdx.x * 256 + tid) * 4;
    unsigned long long br = 0ull, bp = 0ull;
    if (v0 < a.V) {
        const float4 l4 = *reinterpret_cast<const float4 *>(a.logits + (size_t)n * a.V + v0);
        float4 q4 = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        if (residual) q4 = *reinterpret_cast<const float4 *>(a.q + (size_t)n * a.V + v0);
        const uint4 w = philox4x32_10(make_uint4((uint32_t)v0 >> 2, (uint32_t)n, (uint32_t)a.step,
                                                 (uint32_t)(a.step >> 32)),
                                      (uint32_t)a.seed, (uint32_t)(a.seed >> 32));
        const float lv[4] = {l4.x, l4.y, l4.z, l4.w}, qv[4] = {q4.x, q4.y, q4.z, q4.w};
        const uint32_t wv[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float g = gumbel(wv[j]);
            const float lp = lv[j] * a.inv_t - lz;
            const unsigned long long kpj = key_of(lp + g, v0 + j);
            bp = kpj > bp ? kpj : bp;
            if (residual) {
                const float r = __expf(lp) - qv[j];
                if (r > 0.0f) {
                    const unsigned long long krj = key_of(logf(r) + g, v0 + j);
                    br = krj > br ? krj : br;
                }
            }
        }
        if (!residual) br = bp;
    }
    kr[tid] = br;
    kp[tid] = bp;
    __syncthreads();
    for (int off = 128; off >= 1; off >>= 1) {
        if (tid < off) {
            kr[tid] = kr[tid + off] > kr[tid] ? kr[tid + off] : kr[tid];
            kp[tid] = kp[tid + off] > kp[tid] ? kp[tid + off] : kp[tid];
        }
        __syncthreads();
    }
    if (tid == 0) {
        a.keys[2 * (size_t)blockIdx.x] = kr[0];
        a.keys[2 * (size_t)blockIdx.x + 1] = kp[0];
    }
}

__global__ __launch_bounds__(256) void k_sample_final(SampleArgs a) {
    __shared__ unsigned long long kr[256], kp[256];
    const int tid = threadIdx.x;
    unsigned long long br = 0ull, bp = 0ull;
    for (int i = tid; i < a.nsg; i += 256) {
        const unsigned long long r = a.keys[2 * (size_t)i], p = a.keys[2 * (size_t)i + 1];
        br = r > br ? r : br;
        bp = p > bp ? p : bp;
    }
    kr[tid] = br;
    kp[tid] = bp;
    __syncthreads();
    for (int off = 128; off >= 1; off >>= 1) {
        if (tid < off) {
            kr[tid] = kr[tid + off] > kr[tid] ? kr[tid + off] : kr[tid];
            kp[tid] = kp[tid + off] > kp[tid] ? kp[tid + off] : kp[tid];
        }
        __syncthreads();
    }
    if (tid == 0) {
        const int n = a.acc[0];
        const unsigned long long k = kr[0] ? kr[0] : kp[0];
        const int t = (int)(0xffffffffu - (uint32_t)(k & 0xffffffffull));
        for (int i = 0; i < a.M; ++i) a.out_tokens[i] = i < n ? a.draft[i] : (i == n ? t : -1);
        *a.accepted_len = n;
    }
}

inline hipStream_t S(void *p) { return reinterpret_cast<hipStream_t>(p); }

}  // namespace

int launch_spec_sample(int M, int V, float inv_t, const int32_t *draft, const float *q, const float *u_acc,
                       uint64_t seed, uint64_t step, int32_t *accepted_len, int32_t *out_tokens,
                       const SampleWs &L, char *ws, void *stream) {
    (void)hipGetLastError();
    SampleArgs a{};
    a.logits = reinterpret_cast<const float *>(ws + L.logits);
    a.stats = reinterpret_cast<float2 *>(ws + L.stats);
    a.draft = draft;
    a.q = q;
    a.u_acc = u_acc;
    a.acc = reinterpret_cast<int *>(ws + L.acc);
    a.keys = reinterpret_cast<unsigned long long *>(ws + L.keys);
    a.accepted_len = accepted_len;
    a.out_tokens = out_tokens;
    a.seed = seed;
    a.step = step;
    a.inv_t = inv_t;
    a.M = M;
    a.V = V;
    a.nwg = L.nwg;
    a.nsg = L.nsg;
    hipLaunchKernelGGL(k_sample_stats, dim3(L.nsg), dim3(256), 0, S(stream), a);
    hipLaunchKernelGGL(k_sample_accept, dim3(1), dim3(256), 0, S(stream), a);
    hipLaunchKernelGGL(k_sample_draw, dim3(L.nsg), dim3(256), 0, S(stream), a);
    hipLaunchKernelGGL(k_sample_final, dim3(1), dim3(256), 0, S(stream), a);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ELAUNCH;
}

}  // namespace moe
