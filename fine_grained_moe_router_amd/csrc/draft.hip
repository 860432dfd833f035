// draft.hip -- the MTP drafter's step on gfx950: gamma drafts in sequence, each a chain of
// small launches (graph-capturable; the drafted token stays on the device and feeds the
// next draft's embedding row).
//
// Page "LLM decoding", "The one-line shape bug that disabled the model's own drafter": the
// head's pre_projection takes 5632 = 2 x 2816 inputs (the target's embedding of the token
// and a 2816-wide hidden state) down to its 1024-wide width, and the head has its own
// 1024-wide embedding table; "Lever 2": a 430M head proposes the tokens the target then
// verifies in one pass. The rest of the head is a reading: a body of dense GELU-gated
// blocks (pre-RMSNorm, residual) and a post-projection back to 2816 for the next draft.
// Per draft:
//   k_draft_embed   e = bf16(s_t * dec(Q[t])) (the product exact in fp64, one rounding),
//                   x = [e | g]
//   k_draft_gemv    z = bf16(pre_proj x)
//   per block       k_draft_gateup (u = rmsnorm(z; g_b) per workgroup, h = gelu(gate u) * up u)
//                   k_draft_down   (z = bf16(z + down h))
//   k_draft_norm    zf = rmsnorm(z; g_final)
//   lm_head argmax  over the head's own table -> the draft
//   k_draft_gemv    g = bf16(post_proj zf)
// Every matrix is FP8 with per-row fp32 scales; arithmetic is fp32 (FP8 and bf16 products
// are exact), the vectors between stages bf16 (h stays fp32).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "internal.h"

namespace moe {
namespace {

using namespace dev;

constexpr int kDraftRows = 16;   // output rows per workgroup: one per 16-lane group

// bf16 (round to nearest even) of a double that is a product of an fp32 and an FP8 value
// (at most 28 significant bits, normal range): round the mantissa at bit 45 in the integer
// bits, after which the value is exact in fp32.
__device__ __forceinline__ uint16_t d2bf(double d) {
    unsigned long long b = (unsigned long long)__double_as_longlong(d);
    b += ((b >> 45) & 1ull) + (1ull << 44) - 1ull;
    b &= ~((1ull << 45) - 1ull);
    return (uint16_t)(__float_as_uint((float)__longlong_as_double((long long)b)) >> 16);
}

// x = [bf16(s_t * dec(Q[t])) | g], t = *tok (the target's tied embedding row of the token)
__global__ __launch_bounds__(256) void k_draft_embed(const int32_t *tok, const uint8_t *emb_w, const float *emb_s,
                                                     const uint16_t *g, uint16_t *x, int H, int V) {
    int t = *tok;
    t = t < 0 ? 0 : (t >= V ? V - 1 : t);
    const double s = (double)emb_s[t];
    for (int c = threadIdx.x; c < H; c += 256) {
        const float dv = fp8x2_to_f32<false>((uint32_t)emb_w[(size_t)t * H + c]).x;
        x[c] = d2bf(s * (double)dv);
        x[H + c] = g[c];
    }
}

// out[n] = bf16(s[n] * sum_c dec(Q[n][c]) x[c]) for rows n of this workgroup; lane li of
// group r reads 16 bytes of every 256-column chunk of row 16 b + r, x in LDS.
__global__ __launch_bounds__(256) void k_draft_gemv(const uint8_t *Q, const float *s, const uint16_t *x,
                                                    uint16_t *out, int N, int K) {
    extern __shared__ uint4 xs[];   // [K / 8]
    const int tid = threadIdx.x;
    for (int i = tid; i < K / 8; i += 256) xs[i] = reinterpret_cast<const uint4 *>(x)[i];
    __syncthreads();
    const int li = tid & 15, n = blockIdx.x * kDraftRows + (tid >> 4);
    const uint8_t *wr = Q + (size_t)n * K + li * 16;
    float acc = 0.0f;
    for (int k = 0; k < K / 256; ++k) {
        bf16x2 wv[8];
        decode16_bf16(*reinterpret_cast<const uint4 *>(wr + (size_t)k * 256), wv);
        acc = dot16(wv, xs[(k * 256 + li * 16) / 8], xs[(k * 256 + li * 16) / 8 + 1], acc);
    }
    acc = row16_sum(acc);
    if (li == 0 && n < N) out[n] = f2bf(s[n] * acc);
}

// rmsnorm of one bf16 vector of D (a multiple of 256) elements into LDS, in the fixed order
// of k_add_rmsnorm: per-thread sums, DPP rows, the rows of a wave, then the waves.
__device__ __forceinline__ void rmsnorm_lds(const uint16_t *z, const uint16_t *gain, int D, float eps, uint16_t *u) {
    __shared__ float wsum[4];
    float ss = 0.0f;
    for (int c = threadIdx.x; c < D; c += 256) {
        const float v = bf2f(z[c]);
        ss = fmaf(v, v, ss);
    }
    ss = row16_sum(ss);
    ss += __shfl_xor(ss, 16);
    ss += __shfl_xor(ss, 32);
    if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = ss;
    __syncthreads();
    const float r = rsqrtf(((wsum[0] + wsum[1]) + (wsum[2] + wsum[3])) / (float)D + eps);
    for (int c = threadIdx.x; c < D; c += 256) u[c] = f2bf(bf2f(z[c]) * r * bf2f(gain[c]));
    __syncthreads();
}

// h[j] = gelu_tanh(sg[j] (G_j . u)) * (su[j] (U_j . u)), u = rmsnorm(z; gain), rows j of
// this workgroup (one per 16-lane group), the D columns in 256-column chunks.
__global__ __launch_bounds__(256) void k_draft_gateup(const uint8_t *G, const float *sg, const uint8_t *U,
                                                      const float *su, const uint16_t *z, const uint16_t *gain,
                                                      float eps, float *h, int F, int D) {
    extern __shared__ uint4 us[];   // [D / 8]
    rmsnorm_lds(z, gain, D, eps, reinterpret_cast<uint16_t *>(us));
    const int tid = threadIdx.x, li = tid & 15, j = blockIdx.x * kDraftRows + (tid >> 4);
    const uint8_t *gr = G + (size_t)j * D + li * 16, *ur = U + (size_t)j * D + li * 16;
    float ag = 0.0f, au = 0.0f;
    for (int k = 0; k < D / 256; ++k) {
        const uint4 x0 = us[(k * 256 + li * 16) / 8], x1 = us[(k * 256 + li * 16) / 8 + 1];
        bf16x2 wg[8], wu[8];
        decode16_bf16(*reinterpret_cast<const uint4 *>(gr + (size_t)k * 256), wg);
        decode16_bf16(*reinterpret_cast<const uint4 *>(ur + (size_t)k * 256), wu);
        ag = dot16(wg, x0, x1, ag);
        au = dot16(wu, x0, x1, au);
    }
    ag = row16_sum(ag);
    au = row16_sum(au);
    if (li == 0 && j < F) h[j] = gelu_tanh(sg[j] * ag) * (su[j] * au);
}

// z[c] = bf16(z[c] + sd[c] (Dn_c . h)) for rows c of this workgroup, h fp32 [F] in LDS;
// lane li reads 16 codes of every 256-column chunk of the row.
__global__ __launch_bounds__(256) void k_draft_down(const uint8_t *Dn, const float *sd, const float *h, uint16_t *z,
                                                    int D, int F) {
    extern __shared__ float4 hs[];   // [F / 4]
    const int tid = threadIdx.x;
    for (int i = tid; i < F / 4; i += 256) hs[i] = reinterpret_cast<const float4 *>(h)[i];
    __syncthreads();
    const int li = tid & 15, c = blockIdx.x * kDraftRows + (tid >> 4);
    const uint8_t *dr = Dn + (size_t)c * F + li * 16;
    float acc = 0.0f;
    for (int k = 0; k < F / 256; ++k) {
        const uint4 q = *reinterpret_cast<const uint4 *>(dr + (size_t)k * 256);
        const uint32_t qw[4] = {q.x, q.y, q.z, q.w};
        const float4 *hp = hs + (k * 256 + li * 16) / 4;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const f32x2 lo = fp8x2_to_f32<false>(qw[u]), hi = fp8x2_to_f32<true>(qw[u]);
            const float4 hv = hp[u];
            acc = fmaf(lo.x, hv.x, acc);
            acc = fmaf(lo.y, hv.y, acc);
            acc = fmaf(hi.x, hv.z, acc);
            acc = fmaf(hi.y, hv.w, acc);
        }
    }
    acc = row16_sum(acc);
    if (li == 0 && c < D) z[c] = f2bf(bf2f(z[c]) + sd[c] * acc);
}

__global__ __launch_bounds__(256) void k_draft_norm(const uint16_t *z, const uint16_t *gain, float eps, uint16_t *zf,
                                                    int D) {
    extern __shared__ uint4 us[];
    uint16_t *u = reinterpret_cast<uint16_t *>(us);
    rmsnorm_lds(z, gain, D, eps, u);
    for (int c = threadIdx.x; c < D; c += 256) zf[c] = u[c];
}

inline hipStream_t S(void *p) { return reinterpret_cast<hipStream_t>(p); }

}  // namespace

int launch_draft_step(const moe_draft_desc &d, const moe_draft_weights &w, int gamma, const int32_t *tok0,
                      const uint16_t *hidden0, const uint8_t *emb_w, const float *emb_s, int32_t *drafts,
                      char *ws, void *stream) {
    (void)hipGetLastError();
    const int H = d.hidden, D = d.width, F = d.ffn, B = d.blocks, V = d.vocab;
    const DraftWs W = draft_ws(d);
    uint16_t *x = reinterpret_cast<uint16_t *>(ws + W.x);
    uint16_t *z = reinterpret_cast<uint16_t *>(ws + W.z);
    uint16_t *zf = reinterpret_cast<uint16_t *>(ws + W.zf);
    uint16_t *g = reinterpret_cast<uint16_t *>(ws + W.g);
    float *h = reinterpret_cast<float *>(ws + W.h);
    char *lmws = ws + W.lm;
    for (int i = 0; i < gamma; ++i) {
        const int32_t *tok = i == 0 ? tok0 : drafts + i - 1;
        hipLaunchKernelGGL(k_draft_embed, dim3(1), dim3(256), 0, S(stream), tok, emb_w, emb_s, i == 0 ? hidden0 : g,
                           x, H, V);
        hipLaunchKernelGGL(k_draft_gemv, dim3(D / kDraftRows), dim3(256), (size_t)2 * H * 2, S(stream), w.pre_w,
                           w.pre_s, x, z, D, 2 * H);
        for (int b = 0; b < B; ++b) {
            hipLaunchKernelGGL(k_draft_gateup, dim3(F / kDraftRows), dim3(256), (size_t)D * 2, S(stream),
                               w.gate_w + (size_t)b * F * D, w.gate_s + (size_t)b * F, w.up_w + (size_t)b * F * D,
                               w.up_s + (size_t)b * F, z, w.gains + (size_t)b * D, d.eps, h, F, D);
            hipLaunchKernelGGL(k_draft_down, dim3(D / kDraftRows), dim3(256), (size_t)F * 4, S(stream),
                               w.down_w + (size_t)b * D * F, w.down_s + (size_t)b * D, h, z, D, F);
        }
        hipLaunchKernelGGL(k_draft_norm, dim3(1), dim3(256), (size_t)D * 2, S(stream), z, w.gains + (size_t)B * D,
                           d.eps, zf, D);
        if (hipGetLastError() != hipSuccess) return MOE_ELAUNCH;   // launch_lm_head clears the error state
        const int st = launch_lm_head(1, D, V, zf, w.table_w, w.table_s, drafts + i, nullptr, lmws, stream);
        if (st != MOE_OK) return st;
        if (i + 1 < gamma)
            hipLaunchKernelGGL(k_draft_gemv, dim3(H / kDraftRows), dim3(256), (size_t)D * 2, S(stream), w.post_w,
                               w.post_s, zf, g, H, D);
    }
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ELAUNCH;
}

}  // namespace moe
