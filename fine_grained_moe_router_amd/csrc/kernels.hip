// kernels.hip -- gfx950 (CDNA4) kernels of the batch-1 fine-grained MoE decode step.
//
// Every weight matrix is streamed from HBM once per call with 16-byte loads, for all
// the tokens that need it. FP8 codes are decoded in registers by the gfx950
// conversion instructions (two codes per instruction) and multiplied against bf16
// activations held in LDS with the packed bf16 dot product, accumulating in fp32
// (page "LLM decoding", "Lever 1: fewer bytes (FP8 weights)": the 8-bit format only
// saves HBM bytes; the arithmetic runs in a wider type). Per-output-row scales are
// applied in fp32 after the dot product. Reductions across the lanes that share a
// row use DPP row operations in a fixed order, so results are deterministic and a
// token's output never depends on the other tokens of the call.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "device_common.h"
#include "handoff.h"
#include "internal.h"

namespace moe {
namespace {

using namespace dev;

// -------------------------------------------------------------------- router

struct RouterArgs {
    const uint16_t *x;   // [M][H]
    const uint16_t *w;   // [H][E]
    float *partial;      // [NB][M][E]
    int M, H, E;
};

// Partial router logits of one block of kRouterRows rows of W: thread (grp, e)
// accumulates rows grp, grp + G, ... of its column; groups are summed in order.
__global__ __launch_bounds__(256) void k_router(RouterArgs a) {
    __shared__ float xs[kMaxM][kRouterRows];
    __shared__ float red[256][kMaxM];
    const int b = blockIdx.x, tid = threadIdx.x;
    const int r0 = b * kRouterRows;
    const int nr = min(kRouterRows, a.H - r0);
    for (int i = tid; i < a.M * kRouterRows; i += 256) {
        const int m = i / kRouterRows, r = i % kRouterRows;
        xs[m][r] = r < nr ? bf2f(a.x[(size_t)m * a.H + r0 + r]) : 0.0f;
    }
    __syncthreads();
    const int E = a.E, G = 256 / E;
    const int e = tid % E, grp = tid / E;
    float acc[kMaxM];
#pragma unroll
    for (int m = 0; m < kMaxM; ++m) acc[m] = 0.0f;
    if (grp < G) {
        for (int r = grp; r < nr; r += G) {
            const float wv = bf2f(a.w[(size_t)(r0 + r) * E + e]);
#pragma unroll
            for (int m = 0; m < kMaxM; ++m)
                if (m < a.M) acc[m] = fmaf(xs[m][r], wv, acc[m]);
        }
    }
#pragma unroll
    for (int m = 0; m < kMaxM; ++m) red[tid][m] = acc[m];
    __syncthreads();
    if (tid < E) {
        for (int m = 0; m < a.M; ++m) {
            float s = 0.0f;
            for (int g = 0; g < G; ++g) s += red[g * E + tid][m];
            a.partial[((size_t)b * a.M + m) * E + tid] = s;
        }
    }
}

// ---------------------------------------------------------- top-K and union

struct TopkArgs {
    const float *partial;  // [NB][M][E]
    const float *bias;     // [E] or null
    int32_t *topk_idx;     // [M][K] or null
    float *topk_w;         // [M][K] or null
    int32_t *n_slots;
    int32_t *slot_expert;
    uint32_t *slot_mask;
    float *slot_w;         // [S][M]
    int M, E, K, NB, shared;
};

// One workgroup: wave m selects token m's top K (K rounds of a wave argmax with
// ties to the lower id), then all threads build the union of selected experts in
// ascending id, each with its token mask and combine weights; the shared expert
// (id E) is appended last with weight 1 for every token.
__global__ __launch_bounds__(512) void k_topk(TopkArgs a) {
    __shared__ float wsel[kMaxM][kMaxExperts];
    __shared__ unsigned long long bal_m[kMaxM][4];   // bit e % 64 of word e / 64: token m selected e
    __shared__ int wave_cnt[4];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int E = a.E, K = a.K, M = a.M;
    for (int i = tid; i < kMaxM * kMaxExperts; i += 512) (&wsel[0][0])[i] = 0.0f;
    if (tid < kMaxM * 4) (&bal_m[0][0])[tid] = 0ull;
    __syncthreads();
    if (wave < M) {
        const int m = wave;
        float l[4];
        // the logits: each expert's row-block partials summed in block order; the
        // partials are requested kChunk blocks at a time for all of the lane's experts,
        // so that a batch costs one memory latency
        constexpr int kChunk = 22;
#pragma unroll
        for (int i = 0; i < 4; ++i) l[i] = 0.0f;
        for (int b0 = 0; b0 < a.NB; b0 += kChunk) {
            float t[4][kChunk];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < kChunk; ++j) {
                    const int e = lane + 64 * i, b = b0 + j;
                    t[i][j] = e < E && b < a.NB ? a.partial[((size_t)b * M + m) * E + e] : 0.0f;
                }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < kChunk; ++j)
                    if (b0 + j < a.NB) l[i] += t[i][j];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = lane + 64 * i;
            if (e < E) {
                if (a.bias) l[i] += a.bias[e];
            } else {
                l[i] = -INFINITY;
            }
        }
        // K rounds of a wave-wide maximum over order-preserving keys, ties to the lower id;
        // the selected experts' softmax weights renormalised over the K (the full softmax
        // denominator cancels), the denominator summed over the wave in a fixed order
        uint32_t o[1][4];
#pragma unroll
        for (int i = 0; i < 4; ++i) o[0][i] = lane + 64 * i < E ? ordered(l[i]) : 0u;
        unsigned sel[1];
        uint32_t wmax[1];
        topk_rounds<1, 4>(o, K, lane, sel, wmax);
        const float lmax = unordered(wmax[0]);
        float ev[4], zl = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            ev[i] = (sel[0] >> i) & 1u ? expf(l[i] - lmax) : 0.0f;
            zl += ev[i];
        }
        const float z = wave_sum(zl);
        int before = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool si = (sel[0] >> i) & 1u;
            const unsigned long long bm = __ballot(si);
            if (lane == 0) bal_m[m][i] = bm;
            if (si) {
                // outputs in ascending expert id
                const int e = lane + 64 * i, pos = before + lanes_below(bm);
                const float wk = ev[i] / z;
                wsel[m][e] = wk;
                if (a.topk_idx) a.topk_idx[m * K + pos] = e;
                if (a.topk_w) a.topk_w[m * K + pos] = wk;
            }
            before += __popcll(bm);
        }
    }
    __syncthreads();
    // union over tokens, slots in ascending expert id
    uint32_t mask = 0;
    if (tid < 256 && tid < E)
        for (int m = 0; m < M; ++m) mask |= (unsigned)((bal_m[m][wave] >> lane) & 1ull) << m;
    const unsigned long long bal = __ballot(mask != 0);
    if (tid < 256 && lane == 0) wave_cnt[wave] = __popcll(bal);
    __syncthreads();
    if (tid < 256 && mask) {
        int base = 0;
        for (int w = 0; w < wave; ++w) base += wave_cnt[w];
        const int slot = base + __popcll(bal & ((1ull << lane) - 1ull));
        a.slot_expert[slot] = tid;
        a.slot_mask[slot] = mask;
        for (int m = 0; m < M; ++m) a.slot_w[slot * M + m] = wsel[m][tid];
    }
    if (tid == 0) {
        const int nr = wave_cnt[0] + wave_cnt[1] + wave_cnt[2] + wave_cnt[3];
        int ns = nr;
        if (a.shared) {
            a.slot_expert[ns] = E;
            a.slot_mask[ns] = (1u << M) - 1u;
            for (int m = 0; m < M; ++m) a.slot_w[ns * M + m] = 1.0f;
            ++ns;
        }
        *a.n_slots = ns;
    }
}

// ------------------------------------------------------------ expert gate/up

struct ExpertArgs {
    const uint16_t *x;        // [M][H] layer input
    const uint8_t *gate, *up, *down;          // routed [E][D][H], [E][D][H], [E][H][D]
    const float *gate_s, *up_s, *down_s;      // [E][D], [E][D], [E][H]
    const uint8_t *sh_gate, *sh_up, *sh_down;
    const float *sh_gate_s, *sh_up_s, *sh_down_s;
    const int32_t *n_slots;
    const int32_t *slot_expert;
    const uint32_t *slot_mask;
    const float *slot_w;      // [S][M]
    float *h;                 // [S][M][F]
    float *ypart;             // [S][M][H]
    int M, H, E, D, Ds, F;
    int down_lds;             // bytes of dynamic LDS given to k_down
};

constexpr int kGateUpRows = 16;   // rows of gate (and of up) per workgroup
constexpr int kGateUpUnroll = 6;  // 16-byte chunks per lane in flight, per matrix

// Workgroup (row block, slot): 4 waves x 4 groups of 16 lanes; each group owns one
// row j of gate and up; lane li reads bytes [256 i + 16 li, +16) of the row for
// i = 0..(row bytes)/256-1 (each load instruction reads 4 rows x 256 contiguous bytes):
// 16 columns per piece for FP8 codes, 8 for bf16 weights (BF).
// h[slot][t][j] = gelu_tanh(s_g[j] (G_j . x_t)) * (s_u[j] (U_j . x_t)), scales 1 for bf16.
template <bool BF>
__global__ __launch_bounds__(256) void k_gateup(ExpertArgs a) {
    extern __shared__ uint4 xs[];  // [ntok][H/8]
    const int s = blockIdx.y;
    if (s >= *a.n_slots) return;
    const int e = a.slot_expert[s];
    const bool shared = e == a.E;
    const int F = shared ? a.Ds : a.D;
    const int row0 = blockIdx.x * kGateUpRows;
    if (row0 >= F) return;
    const uint32_t mask = a.slot_mask[s];
    const int ntok = __popc(mask);
    const int H = a.H, hv = H / 8;
    {
        uint32_t mm = mask;
        for (int t = 0; mm; mm &= mm - 1u, ++t) {
            const int tok = __ffs(mm) - 1;
            const uint4 *src = reinterpret_cast<const uint4 *>(a.x + (size_t)tok * H);
            for (int i = threadIdx.x; i < hv; i += 256) xs[t * hv + i] = src[i];
        }
    }
    __syncthreads();
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, li = lane & 15;
    const int row = row0 + wave * 4 + g;
    constexpr int EB = BF ? 2 : 1;   // bytes per weight
    const size_t eoff = (size_t)e * a.D * H * EB;
    const uint8_t *gw = (shared ? a.sh_gate : a.gate + eoff) + (size_t)row * H * EB + li * 16;
    const uint8_t *uw = (shared ? a.sh_up : a.up + eoff) + (size_t)row * H * EB + li * 16;
    float accg[kMaxM], accu[kMaxM];
#pragma unroll
    for (int t = 0; t < kMaxM; ++t) accg[t] = accu[t] = 0.0f;
    const int NC = H * EB / 256;
    for (int i0 = 0; i0 < NC; i0 += kGateUpUnroll) {
        uint4 qg[kGateUpUnroll], qu[kGateUpUnroll];
#pragma unroll
        for (int k = 0; k < kGateUpUnroll; ++k) {
            if (i0 + k < NC) {
                qg[k] = ld16nt(gw + (size_t)(i0 + k) * 256);
                qu[k] = ld16nt(uw + (size_t)(i0 + k) * 256);
            }
        }
#pragma unroll
        for (int k = 0; k < kGateUpUnroll; ++k) {
            if (i0 + k < NC) {
                if constexpr (BF) {
                    // 8 bf16 weights: columns 128 i + 8 li .. + 7
                    const int xv = ((i0 + k) * 128 + li * 8) / 8;
#pragma unroll
                    for (int t = 0; t < kMaxM; ++t) {
                        if (t < ntok) {
                            const uint4 x0 = xs[t * hv + xv];
                            accg[t] = dot2(as_bf2(qg[k].x), as_bf2(x0.x), accg[t]);
                            accg[t] = dot2(as_bf2(qg[k].y), as_bf2(x0.y), accg[t]);
                            accg[t] = dot2(as_bf2(qg[k].z), as_bf2(x0.z), accg[t]);
                            accg[t] = dot2(as_bf2(qg[k].w), as_bf2(x0.w), accg[t]);
                            accu[t] = dot2(as_bf2(qu[k].x), as_bf2(x0.x), accu[t]);
                            accu[t] = dot2(as_bf2(qu[k].y), as_bf2(x0.y), accu[t]);
                            accu[t] = dot2(as_bf2(qu[k].z), as_bf2(x0.z), accu[t]);
                            accu[t] = dot2(as_bf2(qu[k].w), as_bf2(x0.w), accu[t]);
                        }
                    }
                } else {
                    bf16x2 wg[8], wu[8];
                    decode16_bf16(qg[k], wg);
                    decode16_bf16(qu[k], wu);
                    const int xv = ((i0 + k) * 256 + li * 16) / 8;
#pragma unroll
                    for (int t = 0; t < kMaxM; ++t) {
                        if (t < ntok) {
                            const uint4 x0 = xs[t * hv + xv], x1 = xs[t * hv + xv + 1];
                            accg[t] = dot16(wg, x0, x1, accg[t]);
                            accu[t] = dot16(wu, x0, x1, accu[t]);
                        }
                    }
                }
            }
        }
    }
    const float sg = BF ? 1.0f : (shared ? a.sh_gate_s : a.gate_s + (size_t)e * a.D)[row];
    const float su = BF ? 1.0f : (shared ? a.sh_up_s : a.up_s + (size_t)e * a.D)[row];
#pragma unroll
    for (int t = 0; t < kMaxM; ++t) {
        if (t < ntok) {
            const float ga = row16_sum(accg[t]);
            const float ub = row16_sum(accu[t]);
            if (li == 0)
                a.h[((size_t)s * a.M + t) * a.F + row] = gelu_tanh(sg * ga) * (su * ub);
        }
    }
}

// --------------------------------------------------------------- expert down

constexpr int kDownRows = 64;    // output rows per workgroup
constexpr int kDownUnroll = 6;
constexpr int kDownLdsBytes = 64 * 1024;

// Workgroup (row block, slot): wave w owns rows c0 + 16 w .. +16, 4 lanes per row;
// lane q reads bytes [64 i + 16 q, +16) of the row (i = 0..(row bytes)/64-1): 16
// columns per piece for FP8 codes, 8 for bf16 weights (BF). h of the slot's tokens is
// staged in LDS (fp32). ypart[slot][m][c] = w[slot][m] * s_d[c] (Dn_c . h), s_d = 1 for bf16.
template <bool BF>
__global__ __launch_bounds__(256) void k_down(ExpertArgs a) {
    extern __shared__ float4 hs4[];  // [tp][F/4]
    const int s = blockIdx.y;
    if (s >= *a.n_slots) return;
    const int e = a.slot_expert[s];
    const bool shared = e == a.E;
    const int F = shared ? a.Ds : a.D;
    const uint32_t mask = a.slot_mask[s];
    const int ntok = __popc(mask);
    const int H = a.H;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int q = lane & 3;
    const int c = blockIdx.x * kDownRows + wave * 16 + (lane >> 2);
    constexpr int EB = BF ? 2 : 1;   // bytes per weight
    const uint8_t *dw = (shared ? a.sh_down : a.down + (size_t)e * H * a.D * EB) + (size_t)c * F * EB + q * 16;
    const float sd = BF ? 1.0f : (shared ? a.sh_down_s : a.down_s + (size_t)e * H)[c];
    const int f4 = F / 4;
    const int tp = min(ntok, a.down_lds / (F * 4));
    const int NI = F * EB / 64;
    uint32_t mrem = mask;
    for (int t0 = 0; t0 < ntok; t0 += tp) {
        const int tn = min(tp, ntok - t0);
        __syncthreads();
        for (int i = threadIdx.x; i < tn * f4; i += 256) {
            const int t = i / f4, j = i % f4;
            hs4[t * f4 + j] = reinterpret_cast<const float4 *>(a.h + ((size_t)s * a.M + t0 + t) * a.F)[j];
        }
        __syncthreads();
        float acc[kMaxM];
#pragma unroll
        for (int t = 0; t < kMaxM; ++t) acc[t] = 0.0f;
        for (int i0 = 0; i0 < NI; i0 += kDownUnroll) {
            uint4 qd[kDownUnroll];
#pragma unroll
            for (int k = 0; k < kDownUnroll; ++k)
                if (i0 + k < NI) qd[k] = ld16nt(dw + (size_t)(i0 + k) * 64);
#pragma unroll
            for (int k = 0; k < kDownUnroll; ++k) {
                if (i0 + k < NI) {
                    constexpr int NW = BF ? 8 : 16;   // weights in the piece
                    float wv[NW];
                    const uint32_t qw[4] = {qd[k].x, qd[k].y, qd[k].z, qd[k].w};
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        if constexpr (BF) {
                            wv[2 * u + 0] = __uint_as_float(qw[u] << 16);
                            wv[2 * u + 1] = __uint_as_float(qw[u] & 0xffff0000u);
                        } else {
                            const f32x2 lo = fp8x2_to_f32<false>(qw[u]);
                            const f32x2 hi = fp8x2_to_f32<true>(qw[u]);
                            wv[4 * u + 0] = lo.x; wv[4 * u + 1] = lo.y;
                            wv[4 * u + 2] = hi.x; wv[4 * u + 3] = hi.y;
                        }
                    }
                    const int cv = ((i0 + k) * (64 / EB) + q * NW) / 4;
#pragma unroll
                    for (int t = 0; t < kMaxM; ++t) {
                        if (t < tn) {
#pragma unroll
                            for (int u = 0; u < NW / 4; ++u) {
                                const float4 hv = hs4[t * f4 + cv + u];
                                acc[t] = fmaf(wv[4 * u + 0], hv.x, acc[t]);
                                acc[t] = fmaf(wv[4 * u + 1], hv.y, acc[t]);
                                acc[t] = fmaf(wv[4 * u + 2], hv.z, acc[t]);
                                acc[t] = fmaf(wv[4 * u + 3], hv.w, acc[t]);
                            }
                        }
                    }
                }
            }
        }
#pragma unroll
        for (int t = 0; t < kMaxM; ++t) {
            if (t < tn) {
                const int m = __ffs(mrem) - 1;
                mrem &= mrem - 1u;
                const float v = quad_sum(acc[t]);
                if (q == 0)
                    a.ypart[((size_t)s * a.M + m) * H + c] = a.slot_w[s * a.M + m] * (sd * v);
            }
        }
    }
}

// ------------------------------------------------------------------- combine

struct CombineArgs {
    const int32_t *n_slots;
    const uint32_t *slot_mask;
    const float *ypart;  // [S][M][H]
    uint16_t *y;         // [M][H]
    int M, H;
};

// y[m][c] = bf16( sum over the slots of token m, ascending expert id, shared last ).
__global__ __launch_bounds__(256) void k_combine(CombineArgs a) {
    const int c = blockIdx.x * 256 + threadIdx.x;
    const int m = blockIdx.y;
    const int ns = *a.n_slots;
    float acc = 0.0f;
    for (int s = 0; s < ns; ++s)
        if ((a.slot_mask[s] >> m) & 1u) acc += a.ypart[((size_t)s * a.M + m) * a.H + c];
    a.y[(size_t)m * a.H + c] = f2bf(acc);
}

// ------------------------------------------------------------------- lm_head

struct LmArgs {
    const uint16_t *x;  // [M][H]
    const uint8_t *w;   // [V][H]
    const float *s;     // [V]
    float *best_v;      // [grid][M]
    int32_t *best_i;    // [grid][M]
    int32_t *token;
    float *max_logit;
    int M, H, V, nwg;
    float *logits;      // with logits (the sampling path): every logit, [M][V]
};

constexpr int kLmRowsPerLane = 4;
constexpr int kLmUnroll = 2;

__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
    return v > bv || (v == bv && i < bi);
}

// Workgroups stride over 64-row blocks. Lane (wave w, group g, li) owns rows
// blk*64 + 16 w + 4 g + r (r = 0..3) and reads the same 16-byte column chunk of all
// four, so each bf16 activation chunk read from LDS serves 4 rows. Row sums go
// through the 16-lane DPP reduction; each group keeps its running best per token.
// WBF: bf16 weights ([V][H] bf16, no scales): a 16-byte piece holds 8 columns, so a
// 16-lane chunk of a row covers 128 columns instead of 256 and a row has twice the chunks.
template <bool LOGITS, bool WBF>
__global__ __launch_bounds__(256) void k_lmhead(LmArgs a) {
    extern __shared__ uint4 xs[];  // [M][H/8]; reused at the end for the per-group bests
    const int H = a.H, hv = H / 8, M = a.M;
    for (int i = threadIdx.x; i < M * hv; i += 256)
        xs[i] = reinterpret_cast<const uint4 *>(a.x)[i];
    __syncthreads();
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, li = lane & 15;
    float bv[kMaxM];
    int bi[kMaxM];
#pragma unroll
    for (int t = 0; t < kMaxM; ++t) {
        bv[t] = -INFINITY;
        bi[t] = 0x7fffffff;
    }
    constexpr int EB = WBF ? 2 : 1;          // bytes per weight
    constexpr int CPC = 256 / EB;            // columns per 16-lane chunk of a row
    const int NC = H / CPC;
    const int nblk = a.V / kLmRowsPerWG;
    for (int blk = blockIdx.x; blk < nblk; blk += gridDim.x) {
        const int rbase = blk * kLmRowsPerWG + wave * 16 + g * 4;
        const uint8_t *wr = a.w + (size_t)rbase * H * EB + li * 16;
        float acc[kLmRowsPerLane][kMaxM];
#pragma unroll
        for (int r = 0; r < kLmRowsPerLane; ++r)
#pragma unroll
            for (int t = 0; t < kMaxM; ++t) acc[r][t] = 0.0f;
        for (int i0 = 0; i0 < NC; i0 += kLmUnroll) {
            uint4 q[kLmUnroll][kLmRowsPerLane];
#pragma unroll
            for (int k = 0; k < kLmUnroll; ++k)
#pragma unroll
                for (int r = 0; r < kLmRowsPerLane; ++r)
                    if (i0 + k < NC)
                        q[k][r] = ld16nt(wr + (size_t)r * H * EB + (size_t)(i0 + k) * 256);
#pragma unroll
            for (int k = 0; k < kLmUnroll; ++k) {
                if (i0 + k < NC) {
                    if constexpr (WBF) {
                        const int xv = ((i0 + k) * CPC + li * 8) / 8;
#pragma unroll
                        for (int t = 0; t < kMaxM; ++t) {
                            if (t < M) {
                                const uint4 x0 = xs[t * hv + xv];
#pragma unroll
                                for (int r = 0; r < kLmRowsPerLane; ++r) {
                                    float v = acc[r][t];
                                    v = dot2(as_bf2(q[k][r].x), as_bf2(x0.x), v);
                                    v = dot2(as_bf2(q[k][r].y), as_bf2(x0.y), v);
                                    v = dot2(as_bf2(q[k][r].z), as_bf2(x0.z), v);
                                    acc[r][t] = dot2(as_bf2(q[k][r].w), as_bf2(x0.w), v);
                                }
                            }
                        }
                    } else {
                        bf16x2 wv[kLmRowsPerLane][8];
#pragma unroll
                        for (int r = 0; r < kLmRowsPerLane; ++r) decode16_bf16(q[k][r], wv[r]);
                        const int xv = ((i0 + k) * CPC + li * 16) / 8;
#pragma unroll
                        for (int t = 0; t < kMaxM; ++t) {
                            if (t < M) {
                                const uint4 x0 = xs[t * hv + xv], x1 = xs[t * hv + xv + 1];
#pragma unroll
                                for (int r = 0; r < kLmRowsPerLane; ++r) acc[r][t] = dot16(wv[r], x0, x1, acc[r][t]);
                            }
                        }
                    }
                }
            }
        }
        float sc[kLmRowsPerLane];
#pragma unroll
        for (int r = 0; r < kLmRowsPerLane; ++r) sc[r] = WBF ? 1.0f : a.s[rbase + r];
#pragma unroll
        for (int t = 0; t < kMaxM; ++t) {
            if (t < M) {
                float lg[kLmRowsPerLane];
#pragma unroll
                for (int r = 0; r < kLmRowsPerLane; ++r) {
                    lg[r] = sc[r] * row16_sum(acc[r][t]);
                    if (better(lg[r], rbase + r, bv[t], bi[t])) {
                        bv[t] = lg[r];
                        bi[t] = rbase + r;
                    }
                }
                if constexpr (LOGITS) {
                    // every lane of the group holds the group's 4 logits of token t: lane
                    // r < 4 stores row rbase + r, 16 contiguous bytes per group and token
                    const float sel = li == 0 ? lg[0] : li == 1 ? lg[1] : li == 2 ? lg[2] : lg[3];
                    if (li < kLmRowsPerLane) a.logits[(size_t)t * a.V + rbase + li] = sel;
                }
            }
        }
    }
    // 16 groups x M (value, row) pairs = 128 M bytes <= the M * H * 2 bytes of xs
    __syncthreads();
    float *gv = reinterpret_cast<float *>(xs);
    int *gi = reinterpret_cast<int *>(xs) + 16 * M;
    if (li == 0) {
#pragma unroll
        for (int t = 0; t < kMaxM; ++t) {
            if (t < M) {
                gv[(wave * 4 + g) * M + t] = bv[t];
                gi[(wave * 4 + g) * M + t] = bi[t];
            }
        }
    }
    __syncthreads();
    if (threadIdx.x < M) {
        const int t = threadIdx.x;
        float v = gv[t];
        int i = gi[t];
        for (int k = 1; k < 16; ++k)
            if (better(gv[k * M + t], gi[k * M + t], v, i)) {
                v = gv[k * M + t];
                i = gi[k * M + t];
            }
        a.best_v[blockIdx.x * M + t] = v;
        a.best_i[blockIdx.x * M + t] = i;
    }
}

__global__ __launch_bounds__(256) void k_argmax_final(LmArgs a) {
    // every token's best (logit, row) over the workgroups' keys; all keys are requested up
    // front, then one tree reduction serves every token
    constexpr int kPer = (kLmMaxWG + 255) / 256;
    __shared__ float rv[kMaxM][256];
    __shared__ int ri[kMaxM][256];
    const int M = a.M, tid = threadIdx.x;
    float v[kMaxM];
    int i[kMaxM];
    float kv[kPer][kMaxM];
    int ki[kPer][kMaxM];
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
        const int k = tid + 256 * q;
#pragma unroll
        for (int t = 0; t < kMaxM; ++t) {
            const bool ok = k < a.nwg && t < M;
            kv[q][t] = ok ? a.best_v[k * M + t] : -INFINITY;
            ki[q][t] = ok ? a.best_i[k * M + t] : 0x7fffffff;
        }
    }
#pragma unroll
    for (int t = 0; t < kMaxM; ++t) {
        v[t] = -INFINITY;
        i[t] = 0x7fffffff;
#pragma unroll
        for (int q = 0; q < kPer; ++q) {
            if (better(kv[q][t], ki[q][t], v[t], i[t])) {
                v[t] = kv[q][t];
                i[t] = ki[q][t];
            }
        }
        rv[t][tid] = v[t];
        ri[t][tid] = i[t];
    }
    __syncthreads();
    for (int off = 128; off >= 1; off >>= 1) {
        if (tid < off) {
#pragma unroll
            for (int t = 0; t < kMaxM; ++t) {
                if (t < M && better(rv[t][tid + off], ri[t][tid + off], rv[t][tid], ri[t][tid])) {
                    rv[t][tid] = rv[t][tid + off];
                    ri[t][tid] = ri[t][tid + off];
                }
            }
        }
        __syncthreads();
    }
    if (tid < M) {
        a.token[tid] = ri[tid][0];
        if (a.max_logit) a.max_logit[tid] = rv[tid][0];
    }
}

// ------------------------------------------------------------- acceptance

__global__ void k_spec_accept(int gamma, const int32_t *draft, const int32_t *target,
                              int32_t *accepted_len, int32_t *out_tokens) {
    if (threadIdx.x != 0) return;
    int n = 0;
    while (n < gamma && draft[n] == target[n]) ++n;
    for (int i = 0; i <= gamma; ++i) out_tokens[i] = i <= n ? target[i] : -1;
    *accepted_len = n;
}

// ------------------------------------------------------- residual + RMSNorm

// One workgroup per token: h_out = bf16(h_in + a0 + a1); u = bf16(h_out * rsqrt(mean h_out^2 + eps) * g).
__global__ __launch_bounds__(256) void k_add_rmsnorm(int H, const uint16_t *h_in, const uint16_t *a0,
                                                     const uint16_t *a1, const uint16_t *gain,
                                                     float eps, uint16_t *h_out, uint16_t *u) {
    __shared__ float wsum[4];
    const int m = blockIdx.x;
    const size_t o = (size_t)m * H;
    float ss = 0.0f;
    for (int c = threadIdx.x; c < H; c += 256) {
        float v = bf2f(h_in[o + c]) + bf2f(a0[o + c]);
        if (a1) v += bf2f(a1[o + c]);
        const uint16_t hb = f2bf(v);
        h_out[o + c] = hb;
        const float hf = bf2f(hb);
        ss = fmaf(hf, hf, ss);
    }
    // fixed-order reduction: DPP rows, then the four rows of a wave, then waves
    ss = row16_sum(ss);
    ss += __shfl_xor(ss, 16);
    ss += __shfl_xor(ss, 32);
    if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = ss;
    __syncthreads();
    const float tot = (wsum[0] + wsum[1]) + (wsum[2] + wsum[3]);
    const float r = rsqrtf(tot / (float)H + eps);
    for (int c = threadIdx.x; c < H; c += 256)
        u[o + c] = f2bf(bf2f(h_out[o + c]) * r * bf2f(gain[c]));
}

// Each thread decodes 4 codes through both conversion paths of the GEMV kernels.
__global__ __launch_bounds__(256) void k_fp8_decode(int n, const uint32_t *codes, float4 *via_bf16,
                                                    float4 *via_f32) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i * 4 >= n) return;
    const uint32_t v = codes[i];
    const bf16x2 lo = fp8x2_to_bf16<false>(v), hi = fp8x2_to_bf16<true>(v);
    const uint32_t ulo = __builtin_bit_cast(uint32_t, lo), uhi = __builtin_bit_cast(uint32_t, hi);
    via_bf16[i] = make_float4(bf2f(ulo & 0xffffu), bf2f(ulo >> 16), bf2f(uhi & 0xffffu), bf2f(uhi >> 16));
    const f32x2 flo = fp8x2_to_f32<false>(v), fhi = fp8x2_to_f32<true>(v);
    via_f32[i] = make_float4(flo.x, flo.y, fhi.x, fhi.y);
}

inline hipStream_t S(void *p) { return reinterpret_cast<hipStream_t>(p); }

inline int launched() { return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ELAUNCH; }

}  // namespace

int launch_moe_layer(const moe_layer_desc &d, const moe_layer_weights &w, int M,
                     const uint16_t *x, uint16_t *y, int32_t *topk_idx, float *topk_w,
                     char *ws, const LayerWs &L, void *stream) {
    (void)hipGetLastError();
    const int H = d.hidden, E = d.num_experts;
    RouterArgs ra{x, static_cast<const uint16_t *>(w.router_w), reinterpret_cast<float *>(ws + L.partial), M, H, E};
    hipLaunchKernelGGL(k_router, dim3(L.nb), dim3(256), 0, S(stream), ra);
    TopkArgs ta{reinterpret_cast<const float *>(ws + L.partial), w.router_bias, topk_idx, topk_w,
                reinterpret_cast<int32_t *>(ws + L.n_slots), reinterpret_cast<int32_t *>(ws + L.slot_expert),
                reinterpret_cast<uint32_t *>(ws + L.slot_mask), reinterpret_cast<float *>(ws + L.slot_w),
                M, E, d.top_k, L.nb, d.shared_width > 0 ? 1 : 0};
    hipLaunchKernelGGL(k_topk, dim3(1), dim3(512), 0, S(stream), ta);
    const int S_ = max_slots(M, d.top_k, E, d.shared_width);
    ExpertArgs ea{x,
                  static_cast<const uint8_t *>(w.gate_w), static_cast<const uint8_t *>(w.up_w),
                  static_cast<const uint8_t *>(w.down_w), w.gate_s, w.up_s, w.down_s,
                  static_cast<const uint8_t *>(w.sh_gate_w), static_cast<const uint8_t *>(w.sh_up_w),
                  static_cast<const uint8_t *>(w.sh_down_w), w.sh_gate_s, w.sh_up_s, w.sh_down_s,
                  reinterpret_cast<const int32_t *>(ws + L.n_slots),
                  reinterpret_cast<const int32_t *>(ws + L.slot_expert),
                  reinterpret_cast<const uint32_t *>(ws + L.slot_mask),
                  reinterpret_cast<const float *>(ws + L.slot_w),
                  reinterpret_cast<float *>(ws + L.h), reinterpret_cast<float *>(ws + L.ypart),
                  M, H, E, d.expert_width, d.shared_width, L.F,
                  min(M, kDownLdsBytes / (L.F * 4)) * L.F * 4};
    if (d.wtype == MOE_W_BF16) {
        hipLaunchKernelGGL(k_gateup<true>, dim3(L.F / kGateUpRows, S_), dim3(256), (size_t)M * H * 2, S(stream), ea);
        hipLaunchKernelGGL(k_down<true>, dim3(H / kDownRows, S_), dim3(256), (size_t)ea.down_lds, S(stream), ea);
    } else {
        hipLaunchKernelGGL(k_gateup<false>, dim3(L.F / kGateUpRows, S_), dim3(256), (size_t)M * H * 2, S(stream), ea);
        hipLaunchKernelGGL(k_down<false>, dim3(H / kDownRows, S_), dim3(256), (size_t)ea.down_lds, S(stream), ea);
    }
    CombineArgs ca{reinterpret_cast<const int32_t *>(ws + L.n_slots),
                   reinterpret_cast<const uint32_t *>(ws + L.slot_mask),
                   reinterpret_cast<const float *>(ws + L.ypart), y, M, H};
    hipLaunchKernelGGL(k_combine, dim3(H / 256, M), dim3(256), 0, S(stream), ca);
    return launched();
}

int launch_lm_head(int M, int H, int V, const uint16_t *x, const uint8_t *w, const float *s,
                   int32_t *token, float *max_logit, char *ws, void *stream) {
    (void)hipGetLastError();
    const int nwg = lm_grid(V);
    LmArgs a{x, w, s, reinterpret_cast<float *>(ws),
             reinterpret_cast<int32_t *>(ws + align256((size_t)nwg * M * sizeof(float))),
             token, max_logit, M, H, V, nwg};
    hipLaunchKernelGGL((k_lmhead<false, false>), dim3(nwg), dim3(256), (size_t)M * H * 2, S(stream), a);
    hipLaunchKernelGGL(k_argmax_final, dim3(1), dim3(256), 0, S(stream), a);
    return launched();
}

int launch_lm_head_bf16(int M, int H, int V, const uint16_t *x, const uint16_t *w, int32_t *token, float *max_logit,
                        char *ws, void *stream) {
    (void)hipGetLastError();
    const int nwg = lm_grid(V);
    LmArgs a{x, reinterpret_cast<const uint8_t *>(w), nullptr, reinterpret_cast<float *>(ws),
             reinterpret_cast<int32_t *>(ws + align256((size_t)nwg * M * sizeof(float))),
             token, max_logit, M, H, V, nwg};
    hipLaunchKernelGGL((k_lmhead<false, true>), dim3(nwg), dim3(256), (size_t)M * H * 2, S(stream), a);
    hipLaunchKernelGGL(k_argmax_final, dim3(1), dim3(256), 0, S(stream), a);
    return launched();
}

int launch_lm_head_logits(int M, int H, int V, const uint16_t *x, const uint8_t *w, const float *s,
                          const SampleWs &L, char *ws, void *stream) {
    (void)hipGetLastError();
    LmArgs a{x, w, s, reinterpret_cast<float *>(ws + L.best_v), reinterpret_cast<int32_t *>(ws + L.best_i),
             nullptr, nullptr, M, H, V, L.nwg, reinterpret_cast<float *>(ws + L.logits)};
    hipLaunchKernelGGL((k_lmhead<true, false>), dim3(L.nwg), dim3(256), (size_t)M * H * 2, S(stream), a);
    return launched();
}

// ------------------------------------------------ lm_head without allocation

// The scratch of lm_head_argmax_noalloc: the per-workgroup best logits and rows that
// k_lmhead leaves for k_argmax_final, in a file-scope device array instead of a caller
// workspace. Each device the library runs on holds its own copy until the process ends.
// Host code never passes the array's name to a kernel (on the host it only stands in for
// the symbol): its device address is looked up once per device with hipGetSymbolAddress
// and kept below.
static __device__ __align__(256) char g_lm_scratch[kLmNoallocScratch];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];   // device address of g_lm_scratch, per device (set once)
}  // namespace

int launch_lm_head_noalloc(int M, int H, int V, const uint16_t *x, const uint8_t *w, const float *s,
                           int32_t *token, float *max_logit, void *stream) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_EUNSUPPORTED;
    void *ptr = nullptr;
    {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        if (!g_scratch_ptr[dev]) {
            void *p = nullptr;
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(g_lm_scratch)) != hipSuccess || !p) return MOE_ELAUNCH;
            g_scratch_ptr[dev] = p;
        }
        ptr = g_scratch_ptr[dev];
    }
    return launch_lm_head(M, H, V, x, w, s, token, max_logit, static_cast<char *>(ptr), stream);
}

int launch_spec_accept(int gamma, const int32_t *draft, const int32_t *target,
                       int32_t *accepted_len, int32_t *out_tokens, void *stream) {
    (void)hipGetLastError();
    hipLaunchKernelGGL(k_spec_accept, dim3(1), dim3(64), 0, S(stream), gamma, draft, target,
                       accepted_len, out_tokens);
    return launched();
}

int launch_add_rmsnorm(int M, int H, const uint16_t *h_in, const uint16_t *a0, const uint16_t *a1,
                       const uint16_t *g, float eps, uint16_t *h_out, uint16_t *u, void *stream) {
    (void)hipGetLastError();
    hipLaunchKernelGGL(k_add_rmsnorm, dim3(M), dim3(256), 0, S(stream), H, h_in, a0, a1, g, eps, h_out, u);
    return launched();
}

// --------------------------------------------------------- HBM read probe

// Thread t of the grid reads 16-byte pieces t, t + T, t + 2T, ... (T threads in all),
// kProbeDepth in flight at a time, and XORs their words; each workgroup leaves the XOR of
// its threads' words in sink[w].
constexpr int kProbeDepth = 8;
__global__ __launch_bounds__(256) void k_read_probe(const uint4 *__restrict__ src, size_t n, uint32_t *sink) {
    __shared__ uint32_t red[256];
    const size_t T = (size_t)gridDim.x * blockDim.x;
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    uint32_t acc = 0;
    for (; i + (kProbeDepth - 1) * T < n; i += kProbeDepth * T) {
        uint4 p[kProbeDepth];
#pragma unroll
        for (int k = 0; k < kProbeDepth; ++k) p[k] = ld16nt(src + i + k * T);
#pragma unroll
        for (int k = 0; k < kProbeDepth; ++k) acc ^= p[k].x ^ p[k].y ^ p[k].z ^ p[k].w;
    }
    for (; i < n; i += T) {
        const uint4 p0 = ld16nt(src + i);
        acc ^= p0.x ^ p0.y ^ p0.z ^ p0.w;
    }
    red[threadIdx.x] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t x = 0;
        for (int j = 0; j < 256; ++j) x ^= red[j];
        sink[blockIdx.x] = x;
    }
}

int launch_fp8_decode(int n, const uint8_t *codes, float *via_bf16, float *via_f32, void *stream) {
    (void)hipGetLastError();
    const int threads = n / 4;
    hipLaunchKernelGGL(k_fp8_decode, dim3((threads + 255) / 256), dim3(256), 0, S(stream), n,
                       reinterpret_cast<const uint32_t *>(codes), reinterpret_cast<float4 *>(via_bf16),
                       reinterpret_cast<float4 *>(via_f32));
    return launched();
}

int launch_read_probe(const void *src, size_t bytes, uint32_t *sink, void *stream) {
    (void)hipGetLastError();
    hipLaunchKernelGGL(k_read_probe, dim3(MOE_PROBE_GRID), dim3(256), 0, S(stream),
                       reinterpret_cast<const uint4 *>(src), bytes / 16, sink);
    return launched();
}

}  // namespace moe
