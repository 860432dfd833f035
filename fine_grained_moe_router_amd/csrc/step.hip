// step.hip -- the stacked batch-1 decode step as one persistent gfx950 kernel.
//
// A decode step at batch 1 is a chain of small, memory-bound GEMV phases (page "LLM
// decoding", us-homepage.pages.dev/blog/llm-decoding: "First principles" and the
// remark under "Where the 7.36 GB goes" that a fine-grained MoE step launches
// thousands of tiny kernels, which graph replay only partly hides). Here the whole
// step is one launch of G co-resident workgroups. The work is a fixed list of items:
//
//   per layer l:  NB router row blocks | S x NG gate/up row blocks | S x ND down row blocks
//   then:         NLM lm_head row blocks
//
// (S = the most expert slots M tokens can select, plus the shared expert; slots the
// routing did not fill are skipped.) Workgroup w takes items w, w + G, w + 2G, ... in
// order, and an item waits only on items earlier in the list, so the earliest
// unfinished item can always run: with every workgroup resident the step cannot
// deadlock, and every wait is bounded anyway (a timed-out wait raises the error flag
// instead of hanging).
//
// Hand-off between items goes through device memory with relaxed agent-scope atomic
// loads and stores (coherent across the XCDs without writing back or invalidating the
// L2): a producer's waves wait for their stores to complete, then thread 0 bumps a
// counter; a consumer's thread 0 polls the counter and the workgroup then reads.
//
//  router item (l, b): residual add + RMSNorm of rows 64b.., router partial logits of
//     those rows. The last router item of the layer sums the partials in block order,
//     selects the top K per token and builds the union of selected experts (slots in
//     ascending expert id, the shared expert last).
//  gate/up item (l, s, rb): waves 0-1 stream 8 rows of the slot's gate matrix, waves
//     2-3 the same 8 rows of up, for the slot's tokens; h = gelu_tanh(gate) * up.
//  down item (l, s, cb): 64 rows of the slot's down matrix (loaded before h is ready),
//     weighted by the token's combine weight. The last down item of a row block sums
//     the slots in fixed order into y_l (bf16), adds the residual and the next noise
//     and leaves the row block's sum of squares for the next layer's norm.
//  lm_head item (i): 64 vocabulary rows for all M tokens; per-token maxima are merged
//     with 64-bit atomic maxima of (ordered logit, inverted row) in 32 groups -- order
//     independent, ties to the lower row. The last item writes the tokens and runs the
//     greedy acceptance.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "device_common.h"
#include "internal.h"

namespace moe {
namespace {

using namespace dev;

struct StepArgs {
    const moe_layer_weights *layers;   // device table [L]
    const uint16_t *gains;             // [L+1][H]
    const uint16_t *x;                 // [M][H]
    const uint16_t *noise;             // [L][M][H]
    const uint8_t *lm_w;               // [V][H]
    const float *lm_s;                 // [V]
    const int32_t *draft;              // [M-1]
    int32_t *token;
    float *max_logit;
    int32_t *accepted;
    int32_t *out_tokens;
    uint16_t *y;                       // layer l, token m at y + l * y_ls + m * H
    int32_t *topk_idx;                 // [L][M][K] or null
    float *topk_w;
    uint16_t *x_final;                 // [M][H] or null
    char *ws;
    size_t o_ctr, o_lmkey, o_hres, o_u, o_sumsq, o_partial, o_nslots, o_sexp, o_smask, o_sw, o_h, o_ypart;
    size_t y_ls;
    int M, Mx, H, E, K, D, Ds, F, L, V, S, Sx, NB, NG, ND, NLM, P, T, nctr;
    float eps;
    unsigned spin_limit;
};

constexpr int kWG = 256;

// The item functions are inlined into the kernel and read the kernel arguments on
// demand through a pointer into the kernel-argument segment, made opaque to the
// optimiser per item so that argument fields are not held in registers across items.
typedef const __attribute__((address_space(4))) StepArgs *AP;

__device__ __forceinline__ AP uniform(AP p) {
    const unsigned long long v = (unsigned long long)p;
    const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)v);
    const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(v >> 32));
    return (AP)(((unsigned long long)hi << 32) | lo);
}

extern __shared__ __align__(16) char smem[];

// -------------------------------------------------------- coherent hand-off access

__device__ __forceinline__ void st32(void *p, uint32_t v) {
    __hip_atomic_store(reinterpret_cast<uint32_t *>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld32(const void *p) {
    return __hip_atomic_load(reinterpret_cast<const uint32_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void stf(float *p, float v) { st32(p, __float_as_uint(v)); }
__device__ __forceinline__ float ldf(const float *p) { return __uint_as_float(ld32(p)); }
__device__ __forceinline__ int ldi(const int *p) { return (int)ld32(p); }
__device__ __forceinline__ uint64_t ld64(const void *p) {
    return __hip_atomic_load(reinterpret_cast<const uint64_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// The hand-off loads are atomic, so the compiler waits for each before its first use;
// code below issues them in unrolled batches (loads first, uses after) so that a batch
// costs one memory latency.
__device__ __forceinline__ uint32_t pack2(uint16_t lo, uint16_t hi) { return (uint32_t)lo | ((uint32_t)hi << 16); }

// ------------------------------------------------------------ workspace views

__device__ __forceinline__ int *ctr(AP a, int i) {
    return reinterpret_cast<int *>(a->ws + a->o_ctr) + (size_t)i * kCtrStride;
}
__device__ __forceinline__ unsigned long long *lmkey(AP a, int grp, int m) {
    return reinterpret_cast<unsigned long long *>(a->ws + a->o_lmkey) + (size_t)grp * kMaxM + m;
}
__device__ __forceinline__ uint16_t *hres(AP a, int l, int m) {
    return reinterpret_cast<uint16_t *>(a->ws + a->o_hres) + ((size_t)l * a->Mx + m) * a->H;
}
__device__ __forceinline__ uint16_t *uin(AP a, int l, int m) {
    return reinterpret_cast<uint16_t *>(a->ws + a->o_u) + ((size_t)l * a->Mx + m) * a->H;
}
__device__ __forceinline__ float *sumsq(AP a, int l, int cb) {
    return reinterpret_cast<float *>(a->ws + a->o_sumsq) + ((size_t)l * a->ND + cb) * a->Mx;
}
__device__ __forceinline__ float *partial(AP a, int l, int m, int e) {
    return reinterpret_cast<float *>(a->ws + a->o_partial) + (((size_t)l * a->Mx + m) * a->E + e) * a->NB;
}
__device__ __forceinline__ int *nslots(AP a, int l) {
    return reinterpret_cast<int *>(a->ws + a->o_nslots) + (size_t)l * kCtrStride;
}
__device__ __forceinline__ int *slot_expert(AP a, int l) {
    return reinterpret_cast<int *>(a->ws + a->o_sexp) + (size_t)l * a->Sx;
}
__device__ __forceinline__ unsigned *slot_mask(AP a, int l) {
    return reinterpret_cast<unsigned *>(a->ws + a->o_smask) + (size_t)l * a->Sx;
}
__device__ __forceinline__ float *slot_w(AP a, int l, int s) {
    return reinterpret_cast<float *>(a->ws + a->o_sw) + ((size_t)l * a->Sx + s) * a->Mx;
}
__device__ __forceinline__ float *hbuf(AP a, int l, int s, int t) {
    return reinterpret_cast<float *>(a->ws + a->o_h) + (((size_t)l * a->Sx + s) * a->Mx + t) * a->F;
}
__device__ __forceinline__ float *ypart(AP a, int l, int s, int m) {
    return reinterpret_cast<float *>(a->ws + a->o_ypart) + (((size_t)l * a->Sx + s) * a->Mx + m) * a->H;
}

// counter slots after the fixed ones (their count is StepWs::nctr)
__device__ __forceinline__ int ctr_router(int l) { return kCtrFixed + l; }
__device__ __forceinline__ int ctr_routed(int L, int l) { return kCtrFixed + L + l; }
__device__ __forceinline__ int ctr_ydone(int L, int l) { return kCtrFixed + 2 * L + l; }
__device__ __forceinline__ int ctr_h(int L, int Sx, int l, int s) { return kCtrFixed + 3 * L + l * Sx + s; }
__device__ __forceinline__ int ctr_rb(int L, int Sx, int ND, int l, int cb) {
    return kCtrFixed + 3 * L + L * Sx + l * ND + cb;
}

// ------------------------------------------------------------ wait / publish

struct Shared {
    int slot;       // broadcast of an atomic's result
};
__shared__ Shared g_sh;

// Every thread: wait until *c >= target (thread 0 polls). A wait that exceeds the spin
// limit sets the error flag and gives up, so the step always finishes.
__device__ __forceinline__ void wg_wait(AP a, int *c, int target) {
    if (threadIdx.x == 0) {
        unsigned n = 0;
        while (ldi(c) < target) {
            __builtin_amdgcn_s_sleep(1);
            if (++n >= a->spin_limit) {
                st32(ctr(a, kError), 1u);
                break;
            }
        }
    }
    __syncthreads();
}

// Every thread: wait for this wave's memory operations (its hand-off stores) to
// complete, then thread 0 adds 1 to *c; returns the old value to every thread.
__device__ __forceinline__ int wg_publish(int *c) {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __syncthreads();
    if (threadIdx.x == 0)
        g_sh.slot = __hip_atomic_fetch_add(c, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    return g_sh.slot;
}

// Order-preserving map of a float onto uint32 (larger float -> larger integer).
__device__ __forceinline__ uint32_t ordered(float v) {
    const uint32_t b = __float_as_uint(v);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float unordered(uint32_t o) {
    return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}

// ------------------------------------------------------------------ router

constexpr int kRowsPerThread = 16;   // router rows prefetched per thread (E <= 128: all of them)
constexpr int kMaxRouterBlocks = kStepMaxHidden / kRouterRows;   // 48: partial logits per expert
constexpr int kQuadsPerThread = kStepMaxHidden / 4 / kWG;         // 3: bf16 quads of a row per thread

__device__ __forceinline__ void router_topk(AP a, int l);

// Router partial logits of rows 64 b .. 64 b + 63 for every token. Thread (grp, p)
// owns experts 2p, 2p+1 (one 4-byte load per row) and rows grp, grp + G, ...
__device__ __forceinline__ void item_router(AP a0, int l, int b) {
    const AP a = uniform(a0);
    const int H = a->H, E = a->E, M = a->M, tid = threadIdx.x;
    const int r0 = b * kRouterRows;   // H is a multiple of 256: every block has 64 rows
    const moe_layer_weights &w = a->layers[l];
    const uint32_t *Wr = reinterpret_cast<const uint32_t *>(w.router_w);   // [H][E/2] pairs
    const int E2 = E / 2, G = kWG / E2, p = tid % E2, grp = tid / E2;
    const bool act = grp < G;
    uint32_t wv[kRowsPerThread];
#pragma unroll
    for (int k = 0; k < kRowsPerThread; ++k) {
        const int r = grp + G * k;
        wv[k] = (act && r < kRouterRows) ? Wr[(size_t)(r0 + r) * E2 + p] : 0u;
    }
    float *xs = reinterpret_cast<float *>(smem);             // [M][64] u of this block (fp32)
    float *rsum = xs + kMaxM * kRouterRows;                  // [M] norm factors
    float *red = rsum + kMaxM;                               // [256][2][M] / [ND][M]
    if (l > 0) wg_wait(a, ctr(a, ctr_ydone(a->L, l - 1)), a->ND);

    // norm factor r_m = rsqrt(mean(h^2) + eps)
    if (l == 0) {
        // h_0 = bf16(x + noise_0): the whole row is needed for the sum of squares
        for (int m = 0; m < M; ++m) {
            const uint16_t *xm = a->x + (size_t)m * H, *nm = a->noise + (size_t)m * H;
            float ss = 0.0f;
            for (int c = tid; c < H; c += kWG) {
                const float hv = bf2f(f2bf(bf2f(xm[c]) + bf2f(nm[c])));
                ss = fmaf(hv, hv, ss);
            }
            red[tid * kMaxM + m] = ss;
        }
        __syncthreads();
        if (tid < M) {
            float ss = 0.0f;
            for (int t = 0; t < kWG; ++t) ss += red[t * kMaxM + tid];
            rsum[tid] = rsqrtf(ss / (float)H + a->eps);
        }
    } else {
        for (int i = tid; i < a->ND * M; i += kWG) {
            const int cb = i / M, m = i % M;
            red[cb * kMaxM + m] = ldf(sumsq(a, l, cb) + m);
        }
        __syncthreads();
        if (tid < M) {
            float ss = 0.0f;
            for (int cb = 0; cb < a->ND; ++cb) ss += red[cb * kMaxM + tid];
            rsum[tid] = rsqrtf(ss / (float)H + a->eps);
        }
    }
    __syncthreads();
    // u rows of this block, two rows per thread: bf16(h * r * g), kept in LDS (fp32)
    // and published for the expert items
    const uint16_t *g = a->gains + (size_t)l * H;
    for (int i = tid; i < M * (kRouterRows / 2); i += kWG) {
        const int m = i / (kRouterRows / 2), r = 2 * (i % (kRouterRows / 2)), c = r0 + r;
        uint16_t h0, h1;
        if (l == 0) {
            h0 = f2bf(bf2f(a->x[(size_t)m * H + c]) + bf2f(a->noise[(size_t)m * H + c]));
            h1 = f2bf(bf2f(a->x[(size_t)m * H + c + 1]) + bf2f(a->noise[(size_t)m * H + c + 1]));
            st32(hres(a, 0, m) + c, pack2(h0, h1));
        } else {
            const uint32_t hp = ld32(hres(a, l, m) + c);
            h0 = (uint16_t)(hp & 0xffffu);
            h1 = (uint16_t)(hp >> 16);
        }
        const uint16_t u0 = f2bf(bf2f(h0) * rsum[m] * bf2f(g[c]));
        const uint16_t u1 = f2bf(bf2f(h1) * rsum[m] * bf2f(g[c + 1]));
        st32(uin(a, l, m) + c, pack2(u0, u1));
        xs[m * kRouterRows + r] = bf2f(u0);
        xs[m * kRouterRows + r + 1] = bf2f(u1);
    }
    __syncthreads();
    float acc0[kMaxM], acc1[kMaxM];
#pragma unroll
    for (int m = 0; m < kMaxM; ++m) acc0[m] = acc1[m] = 0.0f;
    if (act) {
#pragma unroll
        for (int k = 0; k < kRowsPerThread; ++k) {
            const int r = grp + G * k;
            if (r < kRouterRows) {
                const float w0 = bf2f(wv[k] & 0xffffu), w1 = bf2f(wv[k] >> 16);
#pragma unroll
                for (int m = 0; m < kMaxM; ++m) {
                    if (m < M) {
                        acc0[m] = fmaf(xs[m * kRouterRows + r], w0, acc0[m]);
                        acc1[m] = fmaf(xs[m * kRouterRows + r], w1, acc1[m]);
                    }
                }
            }
        }
        // rows beyond the prefetched ones (E > 128)
        for (int r = grp + G * kRowsPerThread; r < kRouterRows; r += G) {
            const uint32_t wp = Wr[(size_t)(r0 + r) * E2 + p];
            const float w0 = bf2f(wp & 0xffffu), w1 = bf2f(wp >> 16);
#pragma unroll
            for (int m = 0; m < kMaxM; ++m) {
                if (m < M) {
                    acc0[m] = fmaf(xs[m * kRouterRows + r], w0, acc0[m]);
                    acc1[m] = fmaf(xs[m * kRouterRows + r], w1, acc1[m]);
                }
            }
        }
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < kMaxM; ++m) {
        red[(tid * 2 + 0) * kMaxM + m] = acc0[m];
        red[(tid * 2 + 1) * kMaxM + m] = acc1[m];
    }
    __syncthreads();
    if (tid < E) {
        const int pp = tid >> 1, half = tid & 1;
        for (int m = 0; m < M; ++m) {
            float sum = 0.0f;
            for (int q = 0; q < G; ++q) sum += red[((q * E2 + pp) * 2 + half) * kMaxM + m];
            stf(partial(a, l, m, tid) + b, sum);
        }
    }
    if (wg_publish(ctr(a, ctr_router(l))) != a->NB - 1) return;
    router_topk(a, l);
}

// The last router item of a layer: logits = partials summed in block order (+ bias);
// per token the K largest (wave argmax K times, ties to the lower id); weights are
// the softmax renormalised over the K (the full softmax denominator cancels); the
// union of selected experts becomes the slot table (ascending id, shared expert last).
__device__ __forceinline__ void router_topk(AP a, int l) {
    const int E = a->E, M = a->M, K = a->K, tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    float *wsel = reinterpret_cast<float *>(smem);                       // [M][E]
    int *sel_e = reinterpret_cast<int *>(wsel + kMaxM * kMaxExperts);   // [M][16]
    float *sel_l = reinterpret_cast<float *>(sel_e + kMaxM * kMaxTopK);
    int *wave_cnt = reinterpret_cast<int *>(sel_l + kMaxM * kMaxTopK);
    __syncthreads();
    for (int i = tid; i < kMaxM * kMaxExperts; i += kWG) wsel[i] = 0.0f;
    __syncthreads();
    const float *bias = a->layers[l].router_bias;
    const int NB = a->NB;
    for (int m = wave; m < M; m += 4) {
        float lg[4];
        bool taken[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int ee = lane + 64 * i;
            taken[i] = false;
            lg[i] = -INFINITY;
            if (ee < E) {
                const float *pp = partial(a, l, m, ee);
                uint64_t v[kMaxRouterBlocks / 2];
#pragma unroll
                for (int q = 0; q < kMaxRouterBlocks / 2; ++q)
                    if (2 * q < NB) v[q] = ld64(pp + 2 * q);
                float sum = 0.0f;
#pragma unroll
                for (int q = 0; q < kMaxRouterBlocks / 2; ++q) {
                    if (2 * q < NB) sum += __uint_as_float((uint32_t)v[q]);
                    if (2 * q + 1 < NB) sum += __uint_as_float((uint32_t)(v[q] >> 32));
                }
                if (bias) sum += bias[ee];
                lg[i] = sum;
            }
        }
        for (int k = 0; k < K; ++k) {
            float bv = -INFINITY;
            int bi = 0x7fffffff;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int ee = lane + 64 * i;
                if (ee < E && !taken[i] && (lg[i] > bv || (lg[i] == bv && ee < bi))) {
                    bv = lg[i];
                    bi = ee;
                }
            }
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) {
                const float ov = __shfl_xor(bv, off);
                const int oi = __shfl_xor(bi, off);
                if (ov > bv || (ov == bv && oi < bi)) {
                    bv = ov;
                    bi = oi;
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (lane + 64 * i == bi) taken[i] = true;
            if (lane == 0) {
                sel_e[m * kMaxTopK + k] = bi;
                sel_l[m * kMaxTopK + k] = bv;
            }
        }
        if (lane == 0) {
            int *se = sel_e + m * kMaxTopK;
            float *sl = sel_l + m * kMaxTopK;
            const float lmax = sl[0];
            float z = 0.0f;
            for (int k = 0; k < K; ++k) z += expf(sl[k] - lmax);
            for (int k = 1; k < K; ++k) {
                const int ek = se[k];
                const float lk = sl[k];
                int j = k - 1;
                while (j >= 0 && se[j] > ek) {
                    se[j + 1] = se[j];
                    sl[j + 1] = sl[j];
                    --j;
                }
                se[j + 1] = ek;
                sl[j + 1] = lk;
            }
            for (int k = 0; k < K; ++k) {
                const float wk = expf(sl[k] - lmax) / z;
                wsel[m * kMaxExperts + se[k]] = wk;
                if (a->topk_idx) a->topk_idx[((size_t)l * M + m) * K + k] = se[k];
                if (a->topk_w) a->topk_w[((size_t)l * M + m) * K + k] = wk;
            }
        }
    }
    __syncthreads();
    unsigned mask = 0;
    if (tid < E)
        for (int m = 0; m < M; ++m)
            for (int k = 0; k < K; ++k)
                if (sel_e[m * kMaxTopK + k] == tid) mask |= 1u << m;
    const unsigned long long bal = __ballot(mask != 0);
    if (lane == 0) wave_cnt[wave] = __popcll(bal);
    __syncthreads();
    int *se_out = slot_expert(a, l);
    unsigned *sm_out = slot_mask(a, l);
    if (mask) {
        int base = 0;
        for (int q = 0; q < wave; ++q) base += wave_cnt[q];
        const int slot = base + __popcll(bal & ((1ull << lane) - 1ull));
        st32(se_out + slot, (uint32_t)tid);
        st32(sm_out + slot, mask);
        for (int m = 0; m < M; ++m) stf(slot_w(a, l, slot) + m, wsel[m * kMaxExperts + tid]);
    }
    if (tid == 0) {
        int ns = wave_cnt[0] + wave_cnt[1] + wave_cnt[2] + wave_cnt[3];
        if (a->Ds > 0) {
            st32(se_out + ns, (uint32_t)E);
            st32(sm_out + ns, (1u << M) - 1u);
            for (int m = 0; m < M; ++m) stf(slot_w(a, l, ns) + m, 1.0f);
            ++ns;
        }
        st32(nslots(a, l), (uint32_t)ns);
    }
    wg_publish(ctr(a, ctr_routed(a->L, l)));
}

// ----------------------------------------------------------------- gate / up

constexpr int kGURows = 8;      // rows of gate and of up per item
constexpr int kGUChunks = 12;   // 16-byte chunks of a row per lane held in registers (H <= 3072)

struct SlotInfo {
    int ns, e, F, ntok;
    unsigned mask;
    bool shared;
};

__device__ __forceinline__ SlotInfo read_slot(AP a, int l, int s) {
    SlotInfo si;
    // s < S <= Sx, so the slot's entries can be read before knowing whether s is used
    const int ns = ldi(nslots(a, l));
    const int e = ldi(slot_expert(a, l) + s);
    const unsigned mask = ld32(slot_mask(a, l) + s);
    si.ns = ns;
    si.e = 0;
    si.mask = 0;
    si.F = 0;
    si.ntok = 0;
    si.shared = false;
    if (s < ns) {
        // clamped so that even a stale table (after a timed-out wait) names an existing expert
        si.e = min(max(e, 0), a->Ds > 0 ? a->E : a->E - 1);
        si.mask = mask & ((1u << a->M) - 1u);
        si.shared = si.e == a->E;
        si.F = si.shared ? a->Ds : a->D;
        si.ntok = __popc(si.mask);
    }
    return si;
}

// Gate/up item: waves 0-1 stream rows row0..row0+7 of the gate matrix, waves 2-3 the
// same rows of up (16 lanes per row, 256 contiguous bytes per row per load), so each
// lane holds one row's H/256 chunks.
__device__ __forceinline__ void item_gateup(AP a0, int l, int s, int rb) {
    const AP a = uniform(a0);
    wg_wait(a, ctr(a, ctr_routed(a->L, l)), 1);
    const SlotInfo si = read_slot(a, l, s);
    const int row0 = rb * kGURows;
    if (s >= si.ns || row0 >= si.F) return;
    const int H = a->H, hv = H / 8, hw = H / 2, NC = H / 256;
    (void)hw;
    const moe_layer_weights &w = a->layers[l];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, li = lane & 15, up = wave >> 1;
    const int rloc = (wave & 1) * 4 + g, row = row0 + rloc;
    const size_t eoff = (size_t)si.e * a->D * H;
    const uint8_t *mat = up ? (si.shared ? (const uint8_t *)w.sh_up_w : (const uint8_t *)w.up_w + eoff)
                            : (si.shared ? (const uint8_t *)w.sh_gate_w : (const uint8_t *)w.gate_w + eoff);
    const uint8_t *wp = mat + (size_t)row * H + li * 16;
    uint4 q[kGUChunks];
#pragma unroll
    for (int k = 0; k < kGUChunks; ++k)
        if (k < NC) q[k] = *reinterpret_cast<const uint4 *>(wp + (size_t)k * 256);
    const float *sc = up ? (si.shared ? w.sh_up_s : w.up_s + (size_t)si.e * a->D)
                         : (si.shared ? w.sh_gate_s : w.gate_s + (size_t)si.e * a->D);
    const float srow = sc[row];
    uint32_t *xw = reinterpret_cast<uint32_t *>(smem);                      // [ntok][H/2] bf16 pairs
    float *red = reinterpret_cast<float *>(smem + (size_t)a->Mx * H * 2);   // [2][8][M]
    {
        // token t's row is H/4 quads; thread i loads quads i, i + 256, ... of every token
        const int hq = H / 4;
        int toks[kMaxM];
        {
            unsigned mm = si.mask;
#pragma unroll
            for (int t = 0; t < kMaxM; ++t) {
                toks[t] = mm ? __ffs(mm) - 1 : 0;
                mm &= mm - 1u;
            }
        }
        uint64_t v[kMaxM][kQuadsPerThread];
#pragma unroll
        for (int t = 0; t < kMaxM; ++t)
#pragma unroll
            for (int k = 0; k < kQuadsPerThread; ++k) {
                const int i = threadIdx.x + k * kWG;
                if (t < si.ntok && i < hq) v[t][k] = ld64(uin(a, l, toks[t]) + 4 * i);
            }
        uint64_t *xq = reinterpret_cast<uint64_t *>(xw);
#pragma unroll
        for (int t = 0; t < kMaxM; ++t)
#pragma unroll
            for (int k = 0; k < kQuadsPerThread; ++k) {
                const int i = threadIdx.x + k * kWG;
                if (t < si.ntok && i < hq) xq[t * hq + i] = v[t][k];
            }
    }
    __syncthreads();
    const uint4 *xs = reinterpret_cast<const uint4 *>(xw);
    float acc[kMaxM];
#pragma unroll
    for (int t = 0; t < kMaxM; ++t) acc[t] = 0.0f;
#pragma unroll
    for (int k = 0; k < kGUChunks; ++k) {
        if (k < NC) {
            bf16x2 wv[8];
            decode16_bf16(q[k], wv);
            const int xv = (k * 256 + li * 16) / 8;
#pragma unroll
            for (int t = 0; t < kMaxM; ++t) {
                if (t < si.ntok) {
                    const uint4 x0 = xs[t * hv + xv], x1 = xs[t * hv + xv + 1];
                    acc[t] = dot16(wv, x0, x1, acc[t]);
                }
            }
        }
    }
#pragma unroll
    for (int t = 0; t < kMaxM; ++t) {
        if (t < si.ntok) {
            const float v = row16_sum(acc[t]);
            if (li == 0) red[(up * kGURows + rloc) * kMaxM + t] = srow * v;
        }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < kGURows * si.ntok; i += kWG) {
        const int r = i / si.ntok, t = i % si.ntok;
        stf(hbuf(a, l, s, t) + row0 + r, gelu_tanh(red[r * kMaxM + t]) * red[(kGURows + r) * kMaxM + t]);
    }
    wg_publish(ctr(a, ctr_h(a->L, a->Sx, l, s)));
}

// --------------------------------------------------------------------- down

constexpr int kDNRows = 64;
constexpr int kDNChunks = 11;   // 16-byte chunks per lane in registers (F = 704: the whole row)
constexpr int kDownLdsBytes = 32 * 1024;   // h of the slot's tokens staged per pass

__device__ __forceinline__ void item_down(AP a0, int l, int s, int cb) {
    const AP a = uniform(a0);
    wg_wait(a, ctr(a, ctr_routed(a->L, l)), 1);
    const SlotInfo si = read_slot(a, l, s);
    if (s >= si.ns) return;
    const int H = a->H, F = si.F, NI = F / 64, f4 = F / 4;
    const moe_layer_weights &w = a->layers[l];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, q = lane & 3;
    const int c = cb * kDNRows + wave * 16 + (lane >> 2);
    const uint8_t *dw = (si.shared ? (const uint8_t *)w.sh_down_w
                                   : (const uint8_t *)w.down_w + (size_t)si.e * H * a->D) +
                        (size_t)c * F + q * 16;
    // the first block of this lane's chunks is loaded before h is ready
    uint4 qd[kDNChunks];
#pragma unroll
    for (int k = 0; k < kDNChunks; ++k)
        if (k < NI) qd[k] = *reinterpret_cast<const uint4 *>(dw + (size_t)k * 64);
    const float sd = (si.shared ? w.sh_down_s : w.down_s + (size_t)si.e * H)[c];
    wg_wait(a, ctr(a, ctr_h(a->L, a->Sx, l, s)), F / kGURows);

    float4 *hs4 = reinterpret_cast<float4 *>(smem);
    float *hsf = reinterpret_cast<float *>(smem);
    const int tp = min(si.ntok, (int)(kDownLdsBytes / (F * 4)));
    // the combine weights of the slot's tokens
    float cw[kMaxM];
    {
        const float *swp = slot_w(a, l, s);
        uint32_t v[kMaxM];
#pragma unroll
        for (int m = 0; m < kMaxM; ++m)
            if (m < a->M) v[m] = ld32(swp + m);
#pragma unroll
        for (int m = 0; m < kMaxM; ++m) cw[m] = m < a->M ? __uint_as_float(v[m]) : 0.0f;
    }
    unsigned mrem = si.mask;
    bool fresh = true;   // qd holds chunks 0.. of the row
    for (int t0 = 0; t0 < si.ntok; t0 += tp) {
        const int tn = min(tp, si.ntok - t0);
        __syncthreads();
        {
            // tn * F / 2 float pairs (at most kDownLdsBytes / 8): thread i takes pairs i, i + 256, ...
            const int F2 = F / 2, np = tn * F2;
            uint64_t *hq = reinterpret_cast<uint64_t *>(hsf);
#pragma unroll 1
            for (int k0 = 0; k0 * kWG < np; k0 += 8) {   // rounds of 8 loads per thread
                uint64_t v[8];
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const int i = threadIdx.x + (k0 + k) * kWG;
                    if (i < np) v[k] = ld64(hbuf(a, l, s, t0 + i / F2) + 2 * (i % F2));
                }
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const int i = threadIdx.x + (k0 + k) * kWG;
                    if (i < np) hq[i] = v[k];
                }
            }
        }
        __syncthreads();
        float acc[kMaxM];
#pragma unroll
        for (int t = 0; t < kMaxM; ++t) acc[t] = 0.0f;
        for (int i0 = 0; i0 < NI; i0 += kDNChunks) {
            if (!fresh || i0 > 0) {
#pragma unroll
                for (int k = 0; k < kDNChunks; ++k)
                    if (i0 + k < NI) qd[k] = *reinterpret_cast<const uint4 *>(dw + (size_t)(i0 + k) * 64);
            }
            fresh = false;
#pragma unroll
            for (int k = 0; k < kDNChunks; ++k) {
                if (i0 + k < NI) {
                    float wv[16];
                    const uint32_t qw[4] = {qd[k].x, qd[k].y, qd[k].z, qd[k].w};
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const f32x2 lo = fp8x2_to_f32<false>(qw[u]);
                        const f32x2 hi = fp8x2_to_f32<true>(qw[u]);
                        wv[4 * u + 0] = lo.x;
                        wv[4 * u + 1] = lo.y;
                        wv[4 * u + 2] = hi.x;
                        wv[4 * u + 3] = hi.y;
                    }
                    const int cv = ((i0 + k) * 64 + q * 16) / 4;
#pragma unroll
                    for (int t = 0; t < kMaxM; ++t) {
                        if (t < tn) {
#pragma unroll
                            for (int u = 0; u < 4; ++u) {
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
                float wm = 0.0f;
#pragma unroll
                for (int mm = 0; mm < kMaxM; ++mm)
                    if (mm == m) wm = cw[mm];
                if (q == 0) stf(ypart(a, l, s, m) + c, wm * (sd * v));
            }
        }
    }
    if (wg_publish(ctr(a, ctr_rb(a->L, a->Sx, a->ND, l, cb))) != si.ns - 1) return;

    // ---- the last down item of row block cb: combine, residual, next norm's partial sum
    const int M = a->M, tid = threadIdx.x;
    unsigned *masks = reinterpret_cast<unsigned *>(smem);           // [ns <= kMaxSlots]
    int *slist = reinterpret_cast<int *>(masks + kMaxSlots);        // [M][kMaxTopK + 1]
    int *scount = slist + kMaxM * (kMaxTopK + 1);                   // [M]
    float *sq = reinterpret_cast<float *>(scount + kMaxM);          // [M][64]
    __syncthreads();
    {
        uint32_t v[kMaxSlots / kWG + 1];
#pragma unroll
        for (int k = 0; k < kMaxSlots / kWG + 1; ++k)
            if (tid + k * kWG < si.ns) v[k] = ld32(slot_mask(a, l) + tid + k * kWG);
#pragma unroll
        for (int k = 0; k < kMaxSlots / kWG + 1; ++k)
            if (tid + k * kWG < si.ns) masks[tid + k * kWG] = v[k];
    }
    __syncthreads();
    if (tid < M) {   // the slots of token tid in ascending order (K routed + the shared one)
        int n = 0;
        for (int s2 = 0; s2 < si.ns; ++s2)
            if (((masks[s2] >> tid) & 1u) && n < kMaxTopK + 1) slist[tid * (kMaxTopK + 1) + n++] = s2;
        scount[tid] = n;
    }
    __syncthreads();
    const bool last_layer = l == a->L - 1;
    for (int i = tid; i < M * (kDNRows / 2); i += kWG) {
        const int m = i / (kDNRows / 2), r = 2 * (i % (kDNRows / 2)), cc = cb * kDNRows + r;
        const int n = scount[m];
        uint64_t v[kMaxTopK + 1];
#pragma unroll
        for (int j = 0; j < kMaxTopK + 1; ++j)
            if (j < n) v[j] = ld64(ypart(a, l, slist[m * (kMaxTopK + 1) + j], m) + cc);
        float acc0 = 0.0f, acc1 = 0.0f;
#pragma unroll
        for (int j = 0; j < kMaxTopK + 1; ++j) {
            if (j < n) {
                acc0 += __uint_as_float((uint32_t)v[j]);
                acc1 += __uint_as_float((uint32_t)(v[j] >> 32));
            }
        }
        const uint16_t y0 = f2bf(acc0), y1 = f2bf(acc1);
        *reinterpret_cast<uint32_t *>(a->y + (size_t)l * a->y_ls + (size_t)m * H + cc) = pack2(y0, y1);
        const uint32_t hp = ld32(hres(a, l, m) + cc);
        float hv0 = bf2f(hp & 0xffffu), hv1 = bf2f(hp >> 16);
        if (!last_layer) {
            const uint16_t *nz = a->noise + ((size_t)(l + 1) * M + m) * H + cc;
            hv0 += bf2f(nz[0]);
            hv1 += bf2f(nz[1]);
        }
        const uint16_t hn0 = f2bf(hv0 + bf2f(y0)), hn1 = f2bf(hv1 + bf2f(y1));
        st32(hres(a, l + 1, m) + cc, pack2(hn0, hn1));
        const float f0 = bf2f(hn0), f1 = bf2f(hn1);
        sq[m * kDNRows + r] = f0 * f0;
        sq[m * kDNRows + r + 1] = f1 * f1;
    }
    __syncthreads();
    if (tid < M) {
        float ss = 0.0f;
        for (int r = 0; r < kDNRows; ++r) ss += sq[tid * kDNRows + r];
        stf(sumsq(a, l + 1, cb) + tid, ss);
    }
    wg_publish(ctr(a, ctr_ydone(a->L, l)));
}

// ------------------------------------------------------------------ lm_head

constexpr int kLmRows = 4;   // rows per lane (same column chunk)

__device__ __forceinline__ void item_lm(AP a0, int i) {
    const AP a = uniform(a0);
    const int H = a->H, hv = H / 8, M = a->M, NC = H / 256, tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6, g = lane >> 4, li = lane & 15;
    const int rbase = i * kLmRowsPerWG + wave * 16 + g * kLmRows;
    const uint8_t *wr = a->lm_w + (size_t)rbase * H + li * 16;
    uint4 pre[kLmRows];
#pragma unroll
    for (int r = 0; r < kLmRows; ++r) pre[r] = *reinterpret_cast<const uint4 *>(wr + (size_t)r * H);
    wg_wait(a, ctr(a, ctr_ydone(a->L, a->L - 1)), a->ND);

    // x_f = bf16(h_L * rsqrt(mean h_L^2 + eps) * g_L), staged in LDS
    uint32_t *xw = reinterpret_cast<uint32_t *>(smem);              // [M][H/2] bf16 pairs
    float *rs = reinterpret_cast<float *>(xw + (size_t)M * (H / 2));  // [M]
    float *tmp = rs + kMaxM;                                          // [ND][M]
    for (int j = tid; j < a->ND * M; j += kWG) tmp[(j / M) * kMaxM + j % M] = ldf(sumsq(a, a->L, j / M) + j % M);
    __syncthreads();
    if (tid < M) {
        float ss = 0.0f;
        for (int cb = 0; cb < a->ND; ++cb) ss += tmp[cb * kMaxM + tid];
        rs[tid] = rsqrtf(ss / (float)H + a->eps);
    }
    __syncthreads();
    const uint16_t *gL = a->gains + (size_t)a->L * H;
    {
        // M * H / 4 quads of h_L: thread tid takes quads tid, tid + 256, ...
        const int hq = H / 4, nq = M * hq;
        uint64_t v[kMaxM * kQuadsPerThread];
#pragma unroll
        for (int k = 0; k < kMaxM * kQuadsPerThread; ++k) {
            const int j = tid + k * kWG;
            if (j < nq) v[k] = ld64(hres(a, a->L, j / hq) + 4 * (j % hq));
        }
#pragma unroll
        for (int k = 0; k < kMaxM * kQuadsPerThread; ++k) {
            const int j = tid + k * kWG;
            if (j < nq) {
                const int m = j / hq, c = 4 * (j % hq);
                uint16_t xq[4];
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    xq[u] = f2bf(bf2f((uint32_t)(v[k] >> (16 * u)) & 0xffffu) * rs[m] * bf2f(gL[c + u]));
                const uint32_t p0 = pack2(xq[0], xq[1]), p1 = pack2(xq[2], xq[3]);
                xw[2 * j] = p0;
                xw[2 * j + 1] = p1;
                if (i == 0 && a->x_final) {
                    uint32_t *xo = reinterpret_cast<uint32_t *>(a->x_final + (size_t)m * H + c);
                    xo[0] = p0;
                    xo[1] = p1;
                }
            }
        }
    }
    __syncthreads();
    const uint4 *xs4 = reinterpret_cast<const uint4 *>(xw);
    float acc[kLmRows][kMaxM];
#pragma unroll
    for (int r = 0; r < kLmRows; ++r)
#pragma unroll
        for (int t = 0; t < kMaxM; ++t) acc[r][t] = 0.0f;
    for (int k = 0; k < NC; ++k) {
        uint4 qv[kLmRows];
#pragma unroll
        for (int r = 0; r < kLmRows; ++r)
            qv[r] = (k == 0) ? pre[r] : *reinterpret_cast<const uint4 *>(wr + (size_t)r * H + (size_t)k * 256);
        bf16x2 wv[kLmRows][8];
#pragma unroll
        for (int r = 0; r < kLmRows; ++r) decode16_bf16(qv[r], wv[r]);
        const int xv = (k * 256 + li * 16) / 8;
#pragma unroll
        for (int t = 0; t < kMaxM; ++t) {
            if (t < M) {
                const uint4 x0 = xs4[t * hv + xv], x1 = xs4[t * hv + xv + 1];
#pragma unroll
                for (int r = 0; r < kLmRows; ++r) acc[r][t] = dot16(wv[r], x0, x1, acc[r][t]);
            }
        }
    }
    unsigned long long best[kMaxM];
#pragma unroll
    for (int t = 0; t < kMaxM; ++t) best[t] = 0ull;
#pragma unroll
    for (int r = 0; r < kLmRows; ++r) {
        const int v = rbase + r;
        const float sc = a->lm_s[v];
#pragma unroll
        for (int t = 0; t < kMaxM; ++t) {
            if (t < M) {
                const float lg = sc * row16_sum(acc[r][t]);
                const unsigned long long key =
                    ((unsigned long long)ordered(lg) << 32) | (unsigned long long)(0xffffffffu - (uint32_t)v);
                best[t] = key > best[t] ? key : best[t];
            }
        }
    }
    // reduce the 16 lane groups of the workgroup, then one atomic max per token into
    // this item's group slot
    __syncthreads();
    unsigned long long *gb = reinterpret_cast<unsigned long long *>(smem);  // [16][M]
    if (li == 0)
        for (int t = 0; t < M; ++t) gb[(wave * 4 + g) * kMaxM + t] = best[t];
    __syncthreads();
    const int grp = i % kLmGroups;
    if (tid < M) {
        unsigned long long bk = gb[tid];
        for (int k = 1; k < 16; ++k) bk = gb[k * kMaxM + tid] > bk ? gb[k * kMaxM + tid] : bk;
        __hip_atomic_fetch_max(lmkey(a, grp, tid), bk, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    const int in_grp = (a->NLM - grp + kLmGroups - 1) / kLmGroups;
    if (wg_publish(ctr(a, kLmSub + grp)) != in_grp - 1) return;
    const int ngroups = min(a->NLM, kLmGroups);
    if (wg_publish(ctr(a, kLmTop)) != ngroups - 1) return;
    if (tid == 0) {
        int tok[kMaxM];
        for (int t = 0; t < M; ++t) {
            unsigned long long key = 0ull;
            for (int q = 0; q < ngroups; ++q) {
                const unsigned long long kq =
                    __hip_atomic_load(lmkey(a, q, t), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                key = kq > key ? kq : key;
            }
            tok[t] = (int)(0xffffffffu - (uint32_t)(key & 0xffffffffull));
            a->token[t] = tok[t];
            if (a->max_logit) a->max_logit[t] = unordered((uint32_t)(key >> 32));
        }
        const int gamma = M - 1;
        int n = 0;
        while (n < gamma && a->draft[n] == tok[n]) ++n;
        for (int t = 0; t < M; ++t) a->out_tokens[t] = t <= n ? tok[t] : -1;
        *a->accepted = n;
    }
}

// ------------------------------------------------------------------- kernel

#ifndef MOE_STEP_MIN_BLOCKS
#define MOE_STEP_MIN_BLOCKS 2
#endif
__global__ __launch_bounds__(256, MOE_STEP_MIN_BLOCKS) void k_step(StepArgs args) {
    (void)args;
    const AP base = (AP)__builtin_amdgcn_kernarg_segment_ptr();
    for (int t = blockIdx.x;; t += gridDim.x) {
        // The argument pointer is made opaque each iteration so that argument fields
        // are re-read by each item instead of being held in registers across items.
        AP a = base;
        asm volatile("" : "+s"(a));
        const int T = a->T, L = a->L, P = a->P, NB = a->NB, S = a->S, NG = a->NG, ND = a->ND;
        if (t >= T) break;
        if (t < L * P) {
            const int l = t / P, i = t % P;
            if (i < NB) {
                item_router(a, l, i);
            } else if (i < NB + S * NG) {
                const int j = i - NB;
                item_gateup(a, l, j / NG, j % NG);
            } else {
                const int j = i - NB - S * NG;
                item_down(a, l, j / ND, j % ND);
            }
        } else {
            item_lm(a, t - L * P);
        }
        __syncthreads();
    }
    // the last workgroup to leave returns every counter to zero for the next step
    const AP a = base;
    if (wg_publish(ctr(a, kExit)) != (int)gridDim.x - 1) return;
    const int nctr = a->nctr;
    for (int i = threadIdx.x; i < nctr; i += kWG)
        if (i != kError) st32(ctr(a, i), 0u);
    for (int i = threadIdx.x; i < kLmGroups * kMaxM; i += kWG)
        __hip_atomic_store(lmkey(a, i / kMaxM, i % kMaxM), 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

inline hipStream_t Sm(void *p) { return reinterpret_cast<hipStream_t>(p); }

size_t step_lds_bytes(const moe_step_desc &d, const StepWs &W) {
    const int H = d.layer.hidden, Mx = d.max_tokens;
    size_t router = sizeof(float) * (kMaxM * kRouterRows + kMaxM + 2 * kWG * kMaxM);
    size_t topk = sizeof(float) * kMaxM * kMaxExperts + 2 * sizeof(int) * kMaxM * kMaxTopK + 16;
    size_t gu = (size_t)Mx * H * 2 + sizeof(float) * 2 * kGURows * kMaxM;
    // a slot of width F stages min(ntok, kDownLdsBytes / (4 F)) tokens of h
    size_t dn = std::min((size_t)Mx * W.F * 4, (size_t)kDownLdsBytes);
    size_t comb = sizeof(unsigned) * kMaxSlots + sizeof(int) * (kMaxM * (kMaxTopK + 1) + kMaxM) +
                  sizeof(float) * kMaxM * kDNRows;
    size_t lm = (size_t)Mx * H * 2 + sizeof(float) * (kMaxM + (size_t)W.ND * kMaxM);
    size_t mx = router;
    for (size_t v : {topk, gu, dn, comb, lm, (size_t)16 * kMaxM * 8}) mx = v > mx ? v : mx;
    return (mx + 15) & ~(size_t)15;
}

}  // namespace

int step_prepare(const StepWs &W, const moe_layer_weights *layers, char *ws) {
    if (hipMemset(ws, 0, W.total) != hipSuccess) return MOE_ELAUNCH;
    if (hipMemcpy(ws + W.table, layers, sizeof(moe_layer_weights) * W.L, hipMemcpyHostToDevice) != hipSuccess)
        return MOE_ELAUNCH;
    return hipDeviceSynchronize() == hipSuccess ? MOE_OK : MOE_ELAUNCH;
}

int step_status(const StepWs &W, char *ws) {
    int err = 0;
    char *flag = ws + W.ctr + sizeof(int) * kCtrStride * kError;
    if (hipMemcpy(&err, flag, sizeof(int), hipMemcpyDeviceToHost) != hipSuccess) return MOE_ELAUNCH;
    if (!err) return MOE_OK;
    const int zero = 0;
    if (hipMemcpy(flag, &zero, sizeof(int), hipMemcpyHostToDevice) != hipSuccess) return MOE_ELAUNCH;
    return MOE_ETIMEOUT;
}

int launch_step(const moe_step_desc &d, const StepWs &W, int M, const uint16_t *gains,
                const uint8_t *lm_w, const float *lm_s, const uint16_t *x, const uint16_t *noise,
                const int32_t *draft, int32_t *token, float *max_logit, int32_t *accepted_len,
                int32_t *out_tokens, uint16_t *y_layers, int32_t *topk_idx, float *topk_w,
                uint16_t *x_final, char *ws, void *stream) {
    (void)hipGetLastError();
    const moe_layer_desc &ld = d.layer;
    StepArgs a{};
    a.layers = reinterpret_cast<const moe_layer_weights *>(ws + W.table);
    a.gains = gains;
    a.x = x;
    a.noise = noise;
    a.lm_w = lm_w;
    a.lm_s = lm_s;
    a.draft = draft;
    a.token = token;
    a.max_logit = max_logit;
    a.accepted = accepted_len;
    a.out_tokens = out_tokens;
    a.y = y_layers ? y_layers : reinterpret_cast<uint16_t *>(ws + W.y);
    a.y_ls = y_layers ? (size_t)M * ld.hidden : (size_t)W.Mx * ld.hidden;
    a.topk_idx = topk_idx;
    a.topk_w = topk_w;
    a.x_final = x_final;
    a.ws = ws;
    a.o_ctr = W.ctr;
    a.o_lmkey = W.lmkey;
    a.o_hres = W.hres;
    a.o_u = W.u;
    a.o_sumsq = W.sumsq;
    a.o_partial = W.partial;
    a.o_nslots = W.nslots;
    a.o_sexp = W.slot_expert;
    a.o_smask = W.slot_mask;
    a.o_sw = W.slot_w;
    a.o_h = W.h;
    a.o_ypart = W.ypart;
    a.M = M;
    a.Mx = W.Mx;
    a.H = ld.hidden;
    a.E = ld.num_experts;
    a.K = ld.top_k;
    a.D = ld.expert_width;
    a.Ds = ld.shared_width;
    a.F = W.F;
    a.L = d.num_layers;
    a.V = d.vocab;
    a.S = max_slots(M, ld.top_k, ld.num_experts, ld.shared_width);
    a.Sx = W.Sx;
    a.NB = W.NB;
    a.NG = W.F / kGURows;
    a.ND = W.ND;
    a.NLM = d.vocab / kLmRowsPerWG;
    a.P = a.NB + a.S * a.NG + a.S * a.ND;
    a.T = a.L * a.P + a.NLM;
    a.nctr = W.nctr;
    a.eps = d.eps;
    a.spin_limit = d.spin_limit ? d.spin_limit : kDefaultSpin;

    // every workgroup must be resident at once (items wait on other workgroups'
    // items): the grid is the occupancy of this kernel times the compute units
    const size_t lds = step_lds_bytes(d, W);
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_step, kWG, lds) != hipSuccess || per_cu < 1)
        return MOE_ELAUNCH;
    int grid = cus * per_cu;
    if (grid > a.T) grid = a.T;
    hipLaunchKernelGGL(k_step, dim3(grid), dim3(kWG), lds, Sm(stream), a);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ELAUNCH;
}

}  // namespace moe
