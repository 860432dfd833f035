// draft.hip -- the MTP drafter's step on gfx950 as a chain of launches: gamma drafts in
// sequence, each a chain of small launches (graph-capturable; the drafted token stays on
// the device and feeds the next draft's embedding row). Heads and devices that fit it run
// the one-launch form of draft_fused.hip instead.
//
// Page "LLM decoding", "The one-line shape bug that disabled the model's own drafter": the
// head's pre_projection takes 5632 = 2 x 2816 inputs (the target's embedding of the token
// and a 2816-wide hidden state) down to its 1024-wide width, and the head has its own
// 1024-wide embedding table; "Lever 2": a 430M head proposes the tokens the target then
// verifies in one pass. The rest of the head is a reading: a body of dense GELU-gated
// blocks (pre-RMSNorm, residual) and a post-projection back to 2816 for the next draft.
// Per draft (every kernel issues its weight loads first, so the weight stream overlaps
// the wait for the vector it multiplies):
//   k_draft_pre     x = [e | g], e = bf16(s_t * dec(E[t])) (the product exact in fp64, one
//                   rounding), z = bf16(pre_proj x)
//   per block       k_draft_gateup (u = rmsnorm(z; g_b) per workgroup, h = gelu(gate u) * up u)
//                   k_draft_down   (z = bf16(z + down h))
//   k_draft_post    zf = rmsnorm(z; g_final) per workgroup, g = bf16(post_proj zf) for the
//                   next draft (k_draft_norm, zf alone, after the last)
//   lm_head argmax  over the head's own table -> the draft
// Every matrix is FP8 with per-row fp32 scales; arithmetic is fp32 (FP8 and bf16 products
// are exact), the vectors between stages bf16 (h stays fp32). A matrix of N rows of K
// codes is read by 16, 32 or 64 lanes per row, as many as give the launch 256 workgroups.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "device_common.h"
#include "internal.h"
#include "pieces.h"

namespace moe {
namespace {

using namespace dev;

// bf16 (round to nearest even) of a double that is a product of an fp32 and an FP8 value
// (at most 28 significant bits, normal range): round the mantissa at bit 45 in the integer
// bits, after which the value is exact in fp32.
__device__ __forceinline__ uint16_t d2bf(double d) {
    unsigned long long b = (unsigned long long)__double_as_longlong(d);
    b += ((b >> 45) & 1ull) + (1ull << 44) - 1ull;
    b &= ~((1ull << 45) - 1ull);
    return (uint16_t)(__float_as_uint((float)__longlong_as_double((long long)b)) >> 16);
}

// z = bf16(pre_proj [e | g]), e = bf16(s_t * dec(E[t])) (the target's tied embedding row of
// t = *tok, the product exact in fp64 and rounded once), g the hidden state.
template <int LPR, int MAXCH>
__global__ __launch_bounds__(256) void k_draft_pre(const int32_t *tok, const uint8_t *emb_w, const float *emb_s,
                                                   const uint16_t *g, const uint8_t *Q, const float *s, uint16_t *z,
                                                   int H, int V) {
    extern __shared__ uint4 xs[];   // [2H / 8]
    const int tid = threadIdx.x, li = tid & (LPR - 1), n = blockIdx.x * (256 / LPR) + tid / LPR;
    const int K = 2 * H, ch = K / (16 * LPR);
    Pieces<LPR, MAXCH> w;
    w.load(Q + (size_t)n * K, li, ch);
    int t = *tok;
    t = t < 0 ? 0 : (t >= V ? V - 1 : t);
    // thread c < H / 16: codes 16 c .. 16 c + 15 of the row, two uint4 of e
    const bool emb = tid < H / 16;
    uint4 q = {0u, 0u, 0u, 0u};
    if (emb) q = reinterpret_cast<const uint4 *>(emb_w + (size_t)t * H)[tid];
    const double st = (double)emb_s[t];
    stage16(xs + H / 8, reinterpret_cast<const uint4 *>(g), H / 8);
    if (emb) {
        const uint32_t qw[4] = {q.x, q.y, q.z, q.w};
        uint32_t e[8];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const f32x2 lo = fp8x2_to_f32<false>(qw[u]), hi = fp8x2_to_f32<true>(qw[u]);
            e[2 * u] = (uint32_t)d2bf(st * (double)lo.x) | ((uint32_t)d2bf(st * (double)lo.y) << 16);
            e[2 * u + 1] = (uint32_t)d2bf(st * (double)hi.x) | ((uint32_t)d2bf(st * (double)hi.y) << 16);
        }
        xs[2 * tid] = make_uint4(e[0], e[1], e[2], e[3]);
        xs[2 * tid + 1] = make_uint4(e[4], e[5], e[6], e[7]);
    }
    __syncthreads();
    const float acc = group_sum<LPR>(w.dot_bf16(xs, li, ch));
    if (li == 0) z[n] = f2bf(s[n] * acc);
}

// u = bf16(z * r * gain), r = 1 / sqrt(mean(z^2) + eps), for one bf16 vector of D (a
// multiple of 256, at most 4096) elements, into LDS. z and the gain are read once, eight
// elements a thread at a time; the sum of squares goes per thread in element order, then
// over each 16-lane row, the wave and the four waves in a fixed order.
__device__ __forceinline__ void rmsnorm_lds(const uint16_t *z, const uint16_t *gain, int D, float eps, uint16_t *u) {
    __shared__ float wsum[4];
    constexpr int MAXV = 2;
    const int tid = threadIdx.x, nv = D / 8;
    uint4 zv[MAXV], gv[MAXV];
#pragma unroll
    for (int i = 0; i < MAXV; ++i)
        if (tid + 256 * i < nv) {
            zv[i] = reinterpret_cast<const uint4 *>(z)[tid + 256 * i];
            gv[i] = reinterpret_cast<const uint4 *>(gain)[tid + 256 * i];
        }
    float ss = 0.0f;
#pragma unroll
    for (int i = 0; i < MAXV; ++i)
        if (tid + 256 * i < nv) {
            const uint32_t zw[4] = {zv[i].x, zv[i].y, zv[i].z, zv[i].w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const float a = bf2f(zw[k] & 0xffffu), b = bf2f(zw[k] >> 16);
                ss = fmaf(a, a, ss);
                ss = fmaf(b, b, ss);
            }
        }
    ss = row16_sum(ss);
    ss += __shfl_xor(ss, 16);
    ss += __shfl_xor(ss, 32);
    if ((tid & 63) == 0) wsum[tid >> 6] = ss;
    __syncthreads();
    const float r = rsqrtf(((wsum[0] + wsum[1]) + (wsum[2] + wsum[3])) / (float)D + eps);
#pragma unroll
    for (int i = 0; i < MAXV; ++i)
        if (tid + 256 * i < nv) {
            const uint32_t zw[4] = {zv[i].x, zv[i].y, zv[i].z, zv[i].w};
            const uint32_t gw[4] = {gv[i].x, gv[i].y, gv[i].z, gv[i].w};
            uint32_t o[4];
#pragma unroll
            for (int k = 0; k < 4; ++k)
                o[k] = (uint32_t)f2bf(bf2f(zw[k] & 0xffffu) * r * bf2f(gw[k] & 0xffffu)) |
                       ((uint32_t)f2bf(bf2f(zw[k] >> 16) * r * bf2f(gw[k] >> 16)) << 16);
            reinterpret_cast<uint4 *>(u)[tid + 256 * i] = make_uint4(o[0], o[1], o[2], o[3]);
        }
    __syncthreads();
}

// h[j] = gelu_tanh(sg[j] (G_j . u)) * (su[j] (U_j . u)), u = rmsnorm(z; gain) (each
// workgroup forms it in LDS while its gate and up pieces are in flight).
template <int LPR, int MAXCH>
__global__ __launch_bounds__(256) void k_draft_gateup(const uint8_t *G, const float *sg, const uint8_t *U,
                                                      const float *su, const uint16_t *z, const uint16_t *gain,
                                                      float eps, float *h, int D) {
    extern __shared__ uint4 us[];   // [D / 8]
    const int tid = threadIdx.x, li = tid & (LPR - 1), j = blockIdx.x * (256 / LPR) + tid / LPR;
    const int ch = D / (16 * LPR);
    Pieces<LPR, MAXCH> wg, wu;
    wg.load(G + (size_t)j * D, li, ch);
    wu.load(U + (size_t)j * D, li, ch);
    rmsnorm_lds(z, gain, D, eps, reinterpret_cast<uint16_t *>(us));
    const float ag = group_sum<LPR>(wg.dot_bf16(us, li, ch));
    const float au = group_sum<LPR>(wu.dot_bf16(us, li, ch));
    if (li == 0) h[j] = gelu_tanh(sg[j] * ag) * (su[j] * au);
}

// z[c] = bf16(z[c] + sd[c] (Dn_c . h)), h fp32 [F] in LDS.
template <int LPR, int MAXCH>
__global__ __launch_bounds__(256) void k_draft_down(const uint8_t *Dn, const float *sd, const float *h, uint16_t *z,
                                                    int F) {
    extern __shared__ float4 hs[];   // [F / 4]
    const int tid = threadIdx.x, li = tid & (LPR - 1), c = blockIdx.x * (256 / LPR) + tid / LPR;
    const int ch = F / (16 * LPR);
    Pieces<LPR, MAXCH> w;
    w.load(Dn + (size_t)c * F, li, ch);
    stage16(reinterpret_cast<uint4 *>(hs), reinterpret_cast<const uint4 *>(h), F / 4);
    __syncthreads();
    const float acc = group_sum<LPR>(w.dot_f32(hs, li, ch));
    if (li == 0) z[c] = f2bf(bf2f(z[c]) + sd[c] * acc);
}

// g = bf16(post_proj zf), zf = rmsnorm(z; final gain) formed by each workgroup in LDS;
// workgroup 0 also stores zf for the table's argmax.
template <int LPR, int MAXCH>
__global__ __launch_bounds__(256) void k_draft_post(const uint8_t *P, const float *s, const uint16_t *z,
                                                    const uint16_t *gain, float eps, uint16_t *zf, uint16_t *g,
                                                    int D) {
    extern __shared__ uint4 us[];   // [D / 8]
    const int tid = threadIdx.x, li = tid & (LPR - 1), n = blockIdx.x * (256 / LPR) + tid / LPR;
    const int ch = D / (16 * LPR);
    Pieces<LPR, MAXCH> w;
    w.load(P + (size_t)n * D, li, ch);
    rmsnorm_lds(z, gain, D, eps, reinterpret_cast<uint16_t *>(us));
    if (blockIdx.x == 0)
        for (int i = tid; i < D / 8; i += 256) reinterpret_cast<uint4 *>(zf)[i] = us[i];
    const float acc = group_sum<LPR>(w.dot_bf16(us, li, ch));
    if (li == 0) g[n] = f2bf(s[n] * acc);
}

__global__ __launch_bounds__(256) void k_draft_norm(const uint16_t *z, const uint16_t *gain, float eps, uint16_t *zf,
                                                    int D) {
    extern __shared__ uint4 us[];
    uint16_t *u = reinterpret_cast<uint16_t *>(us);
    rmsnorm_lds(z, gain, D, eps, u);
    for (int c = threadIdx.x; c < D; c += 256) zf[c] = u[c];
}

inline hipStream_t S(void *p) { return reinterpret_cast<hipStream_t>(p); }

template <int V>
using IC = std::integral_constant<int, V>;

// f(IC<lpr>) for a lanes-per-row value from draft_lpr
template <class F>
void by_lpr(int lpr, F f) {
    if (lpr == 16) f(IC<16>{});
    else if (lpr == 32) f(IC<32>{});
    else f(IC<64>{});
}

}  // namespace

int launch_draft_step(const moe_draft_desc &d, const moe_draft_weights &w, int gamma, const int32_t *tok0,
                      const uint16_t *hidden0, const uint8_t *emb_w, const float *emb_s, int32_t *drafts,
                      char *ws, void *stream) {
    // the one-launch form where the shape and the device fit it
    const int rc = launch_draft_fused(d, w, gamma, tok0, hidden0, emb_w, emb_s, drafts, ws, stream);
    if (rc != MOE_EUNSUPPORTED) return rc;
    (void)hipGetLastError();
    const int H = d.hidden, D = d.width, F = d.ffn, B = d.blocks, V = d.vocab;
    const int l_pre = draft_lpr(D, 2 * H, kDraftMaxCh), l_gu = draft_lpr(F, D, kDraftGateUpMaxCh),
              l_dn = draft_lpr(D, F, kDraftMaxCh), l_post = draft_lpr(H, D, kDraftMaxCh);
    if (!l_pre || !l_gu || !l_dn || !l_post) return MOE_EINVAL;
    const DraftWs W = draft_ws(d);
    uint16_t *z = reinterpret_cast<uint16_t *>(ws + W.z);
    uint16_t *zf = reinterpret_cast<uint16_t *>(ws + W.zf);
    uint16_t *g = reinterpret_cast<uint16_t *>(ws + W.g);
    float *h = reinterpret_cast<float *>(ws + W.h);
    char *lmws = ws + W.lm;
    hipStream_t st = S(stream);
    for (int i = 0; i < gamma; ++i) {
        const int32_t *tok = i == 0 ? tok0 : drafts + i - 1;
        const uint16_t *gi = i == 0 ? hidden0 : g;
        by_lpr(l_pre, [&](auto L) {
            constexpr int lpr = decltype(L)::value;
            hipLaunchKernelGGL((k_draft_pre<lpr, kDraftMaxCh>), dim3(D * lpr / 256), dim3(256), (size_t)4 * H, st,
                               tok, emb_w, emb_s, gi, w.pre_w, w.pre_s, z, H, V);
        });
        for (int b = 0; b < B; ++b) {
            by_lpr(l_gu, [&](auto L) {
                constexpr int lpr = decltype(L)::value;
                hipLaunchKernelGGL((k_draft_gateup<lpr, kDraftGateUpMaxCh>), dim3(F * lpr / 256), dim3(256),
                                   (size_t)D * 2, st, w.gate_w + (size_t)b * F * D, w.gate_s + (size_t)b * F,
                                   w.up_w + (size_t)b * F * D, w.up_s + (size_t)b * F, z, w.gains + (size_t)b * D,
                                   d.eps, h, D);
            });
            by_lpr(l_dn, [&](auto L) {
                constexpr int lpr = decltype(L)::value;
                hipLaunchKernelGGL((k_draft_down<lpr, kDraftMaxCh>), dim3(D * lpr / 256), dim3(256), (size_t)F * 4,
                                   st, w.down_w + (size_t)b * D * F, w.down_s + (size_t)b * D, h, z, F);
            });
        }
        // the final norm, with the post-projection for the next draft's hidden state
        if (i + 1 < gamma)
            by_lpr(l_post, [&](auto L) {
                constexpr int lpr = decltype(L)::value;
                hipLaunchKernelGGL((k_draft_post<lpr, kDraftMaxCh>), dim3(H * lpr / 256), dim3(256), (size_t)D * 2,
                                   st, w.post_w, w.post_s, z, w.gains + (size_t)B * D, d.eps, zf, g, D);
            });
        else
            hipLaunchKernelGGL(k_draft_norm, dim3(1), dim3(256), (size_t)D * 2, st, z, w.gains + (size_t)B * D,
                               d.eps, zf, D);
        if (hipGetLastError() != hipSuccess) return MOE_ELAUNCH;   // launch_lm_head clears the error state
        const int rc = launch_lm_head(1, D, V, zf, w.table_w, w.table_s, drafts + i, nullptr, lmws, stream);
        if (rc != MOE_OK) return rc;
    }
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ELAUNCH;
}

}  // namespace moe
