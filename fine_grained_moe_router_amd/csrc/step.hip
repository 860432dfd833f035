// step.hip -- the stacked batch-1 decode step as one persistent gfx950 kernel.
//
// A decode step at batch 1 is a chain of small, memory-bound GEMVs (page "LLM
// decoding", us-homepage.pages.dev/blog/llm-decoding: "First principles" and the
// remark under "Where the 7.36 GB goes" that a fine-grained MoE step is thousands of
// tiny kernels, which graph replay only partly hides). Here the whole step is one
// launch of G co-resident workgroups (the compute units times the occupancy), and
// every workgroup takes part in every phase of every layer:
//
//  router   workgroups 0..NR-1 each own 8 experts (router weights re-laid out as
//           [E][H] at prepare time, loaded before the wait). Each forms the whole
//           normalised input u_l as soon as the previous layer's residual rows are
//           in, and writes its experts' logits for all tokens.
//  route    every workgroup reads the E x M logits and selects the top K per token
//           itself (one wave per token: the K-th largest logit by a 32-step bisection
//           of ballots and popcounts, ties to the lower id), so nothing stands between
//           the logits and the expert weight loads. The union of selected experts becomes the slot list: the shared
//           expert first, then the routed experts in ascending id.
//  units    the layer's work is a list: 8-row gate/up units (gate and up rows of one
//           slot), 64-row down units (one slot, one row block), then 64-row combine
//           units. Unit i belongs to workgroup i mod G, which keeps two of its units'
//           weights in flight (one, with one token). A gate/up unit writes
//           h = gelu_tanh(gate) * up for the slot's tokens; a down unit reads the
//           slot's h, multiplies and writes its weighted partial sums; a combine unit
//           sums a row block's sub-slots into y_l (each token's routed experts in
//           ascending id, then the shared expert's column segments), adds the
//           residual and the next layer's noise and writes the next residual rows.
//  lm_head  every workgroup forms x_f itself, streams an equal share of the
//           vocabulary rows with three steps in flight, and leaves its per-token best
//           (ordered logit, inverted row) key; workgroup 0 reduces the keys, writes
//           the tokens and runs the greedy acceptance.
//
// Hand-off data between workgroups travels as 64-bit words: the value in the low half,
// the step's tag (epoch + 1) in the high half, written and read with relaxed
// agent-scope atomics (coherent across the XCDs without writing back or invalidating
// the L2). A consumer polls the words it needs until every tag is current, so a
// producer never waits for its own stores and there are no separate flags inside a
// layer. Every unit waits only on units that come earlier in the list, and a
// workgroup runs its units in list order, so with all workgroups resident the earliest
// unfinished unit can always run: the step cannot deadlock. Every poll is also bounded
// (one that exceeds the spin limit raises the error flag and moves on, so the step
// always ends). The epoch, read by every workgroup when it starts, is advanced by
// workgroup 0 at the very end, after every workgroup has signalled its lm_head share.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "device_common.h"
#include "handoff.h"
#include "internal.h"

namespace moe {
namespace {

using namespace dev;

struct StepArgs {
    const moe_layer_weights *layers;   // device table [L]
    const uint16_t *rt;                // router weights [L][E][H] (bf16, or FP8 codes): the prepared copy;
                                       // layer mode: the caller's expert-major router, or null for [H][E]
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
    uint16_t *y;                       // layer l, token m at y + l * y_ls + m * H, or null
    int32_t *topk_idx;                 // [L][M][K] or null
    float *topk_w;
    uint16_t *x_final;                 // [M][H] or null
    char *ws;
    size_t o_ctr, o_flags, o_logits, o_hres, o_hact, o_ypart, o_lmbest;
    size_t y_ls;
    int f_lm, f_epoch;                 // uint32 offsets inside the flag region
    int l_scr, l_slot;                 // LDS offsets (bytes) of the scratch and slot areas
    int M, Mx, H, E, K, D, Ds, L, V, Sx, NR, ND, NSUBx, Fmax, nseg_r, nseg_s, NLU;
    float eps;
    unsigned spin_limit;
    int layer_mode;                    // 1: one MoE layer from x (already normalised) to y (moe_decode_layer)
    int lm_bf;                         // 1: lm_w holds bf16 weights without scales
    int router_fp8;                    // 1: FP8 router codes with per-expert scales (router_s)
    moe_layer_weights lw;              // layer mode: the layer's weights (router as given, [H][E])
};

constexpr int kWG = 256;
constexpr int kNC = kStepChunks;                // 256-column chunks of a row of H (router, lm_head)
constexpr int kPc = 6;                          // 16-byte pieces of a unit row per lane
constexpr int kUS = kPc * 32 * 16;              // 3072: LDS row stride of u (bf16); columns H.. hold zeros
constexpr int kDS = kPc * 8 * 16;               // 768: LDS row stride of a down unit's staged h (fp32)
constexpr int kW = (kUS / 2 + kWG - 1) / kWG;   // residual words (2 x bf16) of a row per thread
static_assert(kUS >= kStepMaxHidden && kDS >= kStepMaxWidth, "unit rows must fit the padded LDS rows");

// The phase functions are inlined into the kernel and read the kernel arguments on
// demand through a pointer into the kernel-argument segment, made opaque to the
// optimiser per layer so that argument fields are not held in registers across phases.
typedef const __attribute__((address_space(4))) StepArgs *AP;
// The weight-pointer table, read through the constant address space: it is written
// before the launch and never during it, so its fields load through the scalar cache
// and a use of them never waits on the vector loads in flight.
typedef const __attribute__((address_space(4))) moe_layer_weights *WP;
__device__ __forceinline__ WP layer_w(AP a, int l) { return a->layer_mode ? &a->lw : (WP)(a->layers) + l; }

__device__ __forceinline__ AP uniform(AP p) {
    const unsigned long long v = (unsigned long long)p;
    const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)v);
    const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(v >> 32));
    return (AP)(((unsigned long long)hi << 32) | lo);
}

extern __shared__ __align__(16) char smem[];

// eight FP8 router codes (column order) -> eight bf16 (exact: scale 1)
__device__ __forceinline__ uint4 widen8(uint2 q) {
    return make_uint4(__builtin_bit_cast(uint32_t, fp8x2_to_bf16<false>(q.x)),
                      __builtin_bit_cast(uint32_t, fp8x2_to_bf16<true>(q.x)),
                      __builtin_bit_cast(uint32_t, fp8x2_to_bf16<false>(q.y)),
                      __builtin_bit_cast(uint32_t, fp8x2_to_bf16<true>(q.y)));
}

// The thread index, made opaque so that values derived from it are formed where a
// phase needs them rather than hoisted out of the layer loop and kept live (in
// registers, or spilled) across every phase.
__device__ __forceinline__ int ltid() {
    int t = threadIdx.x;
    asm volatile("" : "+v"(t));
    return t;
}

// ------------------------------------------------------------ workspace views

constexpr int kErrCtr = 0;

__device__ __forceinline__ int *ctr(AP a, int i) {
    return reinterpret_cast<int *>(a->ws + a->o_ctr) + (size_t)i * kCtrStride;
}
__device__ __forceinline__ uint32_t *flags(AP a) { return reinterpret_cast<uint32_t *>(a->ws + a->o_flags); }
__device__ __forceinline__ uint64_t *logits(AP a, int l) {
    return reinterpret_cast<uint64_t *>(a->ws + a->o_logits) + (size_t)l * a->Mx * a->E;
}
__device__ __forceinline__ uint64_t *hres(AP a, int l, int m) {   // words of bf16 pairs
    return reinterpret_cast<uint64_t *>(a->ws + a->o_hres) + ((size_t)l * a->Mx + m) * (a->H / 2);
}
__device__ __forceinline__ uint64_t *hact(AP a, int l, int s, int m) {
    return reinterpret_cast<uint64_t *>(a->ws + a->o_hact) + (((size_t)l * a->Sx + s) * a->Mx + m) * a->Fmax;
}
__device__ __forceinline__ uint64_t *ypart(AP a, int l, int js, int m) {
    return reinterpret_cast<uint64_t *>(a->ws + a->o_ypart) + (((size_t)l * a->NSUBx + js) * a->Mx + m) * a->H;
}
__device__ __forceinline__ uint64_t *lmbest(AP a, int w) {
    return reinterpret_cast<uint64_t *>(a->ws + a->o_lmbest) + (size_t)w * kMaxM;
}

// ------------------------------------------------------------ LDS

// The slot area: the routing of the current layer, as every workgroup computes it.
constexpr int kMaxSub = 24;   // sub-slots (slot, column segment) per token: K + shared segments
struct SlotLds {
    int se[kMaxSlots + 3];                 // expert of slot s (E: the shared expert)
    unsigned sm[kMaxSlots + 3];            // bit m: token m uses slot s
    float sw[kMaxSlots + 3][kMaxM];        // combine weight of token m in slot s
    int tsub[kMaxM][kMaxSub];              // token m's sub-slots, in summation order
    unsigned long long bal[kMaxM][4];      // bit e % 64 of word e / 64: token m selected e
    float red[4][kMaxM];                   // per-wave partial sums of squares
};

__device__ __forceinline__ SlotLds &slots(AP a) { return *reinterpret_cast<SlotLds *>(smem + a->l_slot); }
__device__ __forceinline__ uint16_t *ulds() { return reinterpret_cast<uint16_t *>(smem); }   // [M][kUS] bf16
__device__ __forceinline__ char *scratch(AP a) { return smem + a->l_scr; }

// ------------------------------------------------------------ polling

// A wave's polling loop: done() is true once every lane's words are current (or the
// spin limit is reached, which raises the error flag); otherwise it sleeps SLEEP x 64
// cycles and the loop reloads.
// Once any wait of the step has given up, every other wait gives up within 256 polls
// (it checks the error flag that often), so a step whose workgroups cannot all make
// progress ends after about one spin limit rather than one per wait.
template <int SLEEP>
struct PollS {
    unsigned spins = 0;
    __device__ __forceinline__ bool done(AP a, bool ok) {
        if (__all(ok)) return true;
        if (++spins >= a->spin_limit) {
            if ((ltid() & 63) == 0) st32(ctr(a, kErrCtr), 1u);
            return true;
        }
        if ((spins & 255u) == 0u && __builtin_amdgcn_readfirstlane(ld32(ctr(a, kErrCtr))) != 0u) return true;
        __builtin_amdgcn_s_sleep(SLEEP);
        return false;
    }
};
typedef PollS<1> Poll;

// Wait until all n flags hold a value >= tgt (wrap-safe); wave 0 polls.
__device__ __forceinline__ void wait_flags(AP a, const uint32_t *f, int n, uint32_t tgt) {
    const int tid = ltid();
    if (tid < 64) {
        const int lane = tid;
        Poll pl;
        bool ok;
        do {
            ok = true;
            for (int i0 = 0; i0 < n; i0 += 64 * 8) {
                uint32_t v[8];
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const int i = i0 + lane + 64 * k;
                    v[k] = i < n ? ld32(f + i) : tgt;
                }
#pragma unroll
                for (int k = 0; k < 8; ++k) ok = ok && (int)(v[k] - tgt) >= 0;
            }
        } while (!pl.done(a, ok));
    }
    __syncthreads();
}

// Every thread: once every wave's outstanding memory operations (its stores among
// them) are complete, thread 0 raises the flag.
__device__ __forceinline__ void publish(uint32_t *f, uint32_t tgt) {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __syncthreads();
    if (ltid() == 0) st32(f, tgt);
}

// ------------------------------------------------------------ cross-lane helpers

// Sum over each half-wave (32 lanes); valid in lanes 16..31 and 48..63.
__device__ __forceinline__ float half_sum(float v) {
    v = row16_sum(v);
    // row_bcast:15 into rows 1 and 3 only: lane 15 of the row below
    return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xA, 0xF, false));
}

// ------------------------------------------------------------ norm

// h_0 = bf16(x + noise_0) for the pair of columns (2 word, 2 word + 1) of token m
__device__ __forceinline__ uint32_t h0_pair(AP a, int m, int word) {
    const uint32_t xv = *glb(reinterpret_cast<const uint32_t *>(a->x + (size_t)m * a->H + 2 * word));
    const uint32_t nv = *glb(reinterpret_cast<const uint32_t *>(a->noise + (size_t)m * a->H + 2 * word));
    return pack2(f2bf(bf2f(xv & 0xffffu) + bf2f(nv & 0xffffu)), f2bf(bf2f(xv >> 16) + bf2f(nv >> 16)));
}

// u = bf16(h_l * rsqrt(mean(h_l^2) + eps) * g) for the M tokens, into the u area of
// LDS. h_0 comes from the inputs; h_l (l >= 1) from the residual words, polled until
// current, four tokens at a time. Thread t owns words t, t+256, ... of every token and
// the sums of squares are reduced in a fixed order, so every workgroup forms
// bit-identical u. h is staged in the u area and rewritten in place; the columns from H
// to the row stride are zeroed, so unit and router loops can run over whole padded
// rows without bounds checks.
constexpr int kNormTok = 4;
template <int MT, int SLEEP = 1>
__device__ __forceinline__ void norm_to_lds(AP a, int l, const uint16_t *g, uint32_t tgt) {
    const int H = a->H, M = MT, tid = ltid(), hw = H / 2, lane = tid & 63, wave = tid >> 6;
    uint32_t *uw = reinterpret_cast<uint32_t *>(ulds());   // [M][kUS/2] bf16 pairs
    // the gains are requested first, so that they arrive while h is awaited
    uint32_t gv[kW];
#pragma unroll
    for (int k = 0; k < kW; ++k) {
        const int q = tid + k * kWG;
        gv[k] = q < hw ? *glb(reinterpret_cast<const uint32_t *>(g + 2 * q)) : 0u;
    }
    float ss[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) ss[m] = 0.0f;
#pragma unroll
    for (int m0 = 0; m0 < MT; m0 += kNormTok) {
        if (m0 >= M) break;
        uint32_t hp[kNormTok][kW];
        if (l == 0) {
            uint32_t xv[kNormTok][kW], nv[kNormTok][kW];
#pragma unroll
            for (int mm = 0; mm < kNormTok; ++mm)
#pragma unroll
                for (int k = 0; k < kW; ++k) {
                    const int m = m0 + mm, q = tid + k * kWG;
                    if (m < M && q < hw) {
                        xv[mm][k] = *glb(reinterpret_cast<const uint32_t *>(a->x + (size_t)m * H + 2 * q));
                        nv[mm][k] = *glb(reinterpret_cast<const uint32_t *>(a->noise + (size_t)m * H + 2 * q));
                    }
                }
#pragma unroll
            for (int mm = 0; mm < kNormTok; ++mm)
#pragma unroll
                for (int k = 0; k < kW; ++k)
                    hp[mm][k] = pack2(f2bf(bf2f(xv[mm][k] & 0xffffu) + bf2f(nv[mm][k] & 0xffffu)),
                                      f2bf(bf2f(xv[mm][k] >> 16) + bf2f(nv[mm][k] >> 16)));
        } else {
            PollS<SLEEP> pl;
            bool ok;
            do {
                uint64_t v[kNormTok][kW];
#pragma unroll
                for (int mm = 0; mm < kNormTok; ++mm)
#pragma unroll
                    for (int k = 0; k < kW; ++k) {
                        const int m = m0 + mm, q = tid + k * kWG;
                        if (m < M && q < hw) v[mm][k] = ld64(hres(a, l, m) + q);
                    }
                ok = true;
#pragma unroll
                for (int mm = 0; mm < kNormTok; ++mm)
#pragma unroll
                    for (int k = 0; k < kW; ++k) {
                        const int m = m0 + mm, q = tid + k * kWG;
                        if (m < M && q < hw) {
                            hp[mm][k] = (uint32_t)v[mm][k];
                            ok = ok && current(v[mm][k], tgt);
                        }
                    }
            } while (!pl.done(a, ok));
        }
#pragma unroll
        for (int mm = 0; mm < kNormTok; ++mm) {
            const int m = m0 + mm;
#pragma unroll
            for (int k = 0; k < kW; ++k) {
                const int q = tid + k * kWG;
                if (m < M && q < hw) {
                    const float f0 = bf2f(hp[mm][k] & 0xffffu), f1 = bf2f(hp[mm][k] >> 16);
                    ss[m0 + mm] = fmaf(f0, f0, ss[m0 + mm]);
                    ss[m0 + mm] = fmaf(f1, f1, ss[m0 + mm]);
                    uw[m * (kUS / 2) + q] = hp[mm][k];
                }
            }
        }
    }
    SlotLds &S = slots(a);
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        if (m < M) {
            const float t = wave_sum(ss[m]);
            if (lane == 0) S.red[wave][m] = t;
        }
    }
    __syncthreads();
    // every word of the padded row is in range (kW * kWG == kUS / 2): the row's words
    // are read together and the padding is written with a select, without branches
    static_assert(kW * kWG == kUS / 2, "one pass of the normalisation covers the padded row");
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        const float r = rsqrtf((S.red[0][m] + S.red[1][m] + S.red[2][m] + S.red[3][m]) / (float)H + a->eps);
        uint32_t hv[kW];
#pragma unroll
        for (int k = 0; k < kW; ++k) hv[k] = uw[m * (kUS / 2) + tid + k * kWG];
#pragma unroll
        for (int k = 0; k < kW; ++k) {
            const uint16_t u0 = f2bf(bf2f(hv[k] & 0xffffu) * r * bf2f(gv[k] & 0xffffu));
            const uint16_t u1 = f2bf(bf2f(hv[k] >> 16) * r * bf2f(gv[k] >> 16));
            uw[m * (kUS / 2) + tid + k * kWG] = tid + k * kWG < hw ? pack2(u0, u1) : 0u;
        }
    }
    __syncthreads();
}

// Layer mode: the layer input x (already normalised) into the u area as it is, zeros
// past H, in place of the norm.
template <int MT>
__device__ __forceinline__ void x_to_lds(AP a) {
    const int H = a->H, hw = H / 2, tid = ltid();
    uint32_t *uw = reinterpret_cast<uint32_t *>(ulds());   // [M][kUS/2] bf16 pairs
    uint32_t v[MT][kW];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int k = 0; k < kW; ++k) {
            const int q = tid + k * kWG;
            v[m][k] = q < hw ? *glb(reinterpret_cast<const uint32_t *>(a->x + (size_t)m * H + 2 * q)) : 0u;
        }
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int k = 0; k < kW; ++k) uw[m * (kUS / 2) + tid + k * kWG] = v[m][k];
    __syncthreads();
}

template <int MT, int SLEEP = 1>
__device__ __forceinline__ void layer_input(AP a, int l, uint32_t tgt) {
    if (a->layer_mode)
        x_to_lds<MT>(a);
    else
        norm_to_lds<MT, SLEEP>(a, l, a->gains + (size_t)l * a->H, tgt);
}

// ------------------------------------------------------------------ router

// Router workgroup j's weights for layer l: experts 8j .. 8j+7, one half-wave (32
// lanes) per expert, each lane 8 bf16 of every 256-column chunk of the expert's row
// (zeros past H).
__device__ __forceinline__ void router_load(AP a, int l, int j, uint4 (&wq)[kNC]) {
    const int H = a->H, E = a->E, NC = H / 256, tid = ltid();
    const int e = min(8 * j + (tid >> 5), E - 1);
    if (a->router_fp8) {   // codes [L][E][H]: eight per piece, widened to bf16
        const uint8_t *wr8 = reinterpret_cast<const uint8_t *>(a->rt) + ((size_t)l * E + e) * H + (tid & 31) * 8;
#pragma unroll
        for (int k = 0; k < kNC; ++k) wq[k] = k < NC ? widen8(ld8(wr8 + k * 256)) : make_uint4(0u, 0u, 0u, 0u);
        return;
    }
    const uint16_t *wr = a->rt + ((size_t)l * E + e) * H + (tid & 31) * 8;
#pragma unroll
    for (int k = 0; k < kNC; ++k)
        wq[k] = k < NC ? ld16(wr + k * 256) : make_uint4(0u, 0u, 0u, 0u);
}

// Layer mode, FP8 router codes [H][E] (bytes): as router_load_hxe with 8-byte loads (the
// codes of experts 8 j .. 8 j + 7 in one row) through an LDS tile, the pieces widened to
// bf16; rows that are not 8-byte aligned (E not a multiple of 8) take one byte per load.
__device__ __forceinline__ void router_load_hxe8(AP a, int j, uint4 (&wq)[kNC]) {
    const int H = a->H, E = a->E, NC = H / 256, tid = ltid();
    const uint8_t *w8 = static_cast<const uint8_t *>(layer_w(a, 0)->router_w);
    const int e = tid >> 5, l8 = (tid & 31) * 8;
    if (E % 8) {
        const int ee = min(8 * j + e, E - 1);
#pragma unroll
        for (int k = 0; k < kNC; ++k) {
            uint32_t c[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) c[i] = k < NC ? *glb(w8 + ((size_t)k * 256 + l8 + i) * E + ee) : 0u;
            wq[k] = widen8(make_uint2(c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24),
                                      c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24)));
        }
        return;
    }
    uint2 r[kNC];
#pragma unroll
    for (int k = 0; k < kNC; ++k) r[k] = ld8(w8 + ((size_t)min(k, NC - 1) * 256 + tid) * E + 8 * j);
    uint2 *tile = reinterpret_cast<uint2 *>(ulds());   // kNC x 288 x 8 bytes
    const uint8_t *t8 = reinterpret_cast<const uint8_t *>(ulds());
#pragma unroll
    for (int k = 0; k < kNC; ++k)
        if (k < NC) tile[k * 288 + tid + (tid >> 3)] = r[k];
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kNC; ++k) {
        if (k < NC) {
            uint32_t c[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) c[i] = t8[(k * 288 + l8 + i + ((l8 + i) >> 3)) * 8 + e];
            wq[k] = widen8(make_uint2(c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24),
                                      c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24)));
        } else {
            wq[k] = make_uint4(0u, 0u, 0u, 0u);
        }
    }
    __syncthreads();
}

// Layer mode: the same per-lane pieces gathered from the router weights as given, [H][E]
// (element (c, e) at c * E + e): piece k of expert e holds columns k * 256 + 8 lane + 0..7,
// eight 2-byte loads at a stride of one row. The arithmetic that follows is the fused
// step's, so both give the same logits for the same u.
__device__ __forceinline__ void router_load_hxe(AP a, int j, uint4 (&wq)[kNC]) {
    const int H = a->H, E = a->E, NC = H / 256, tid = ltid();
    if (a->router_fp8) {
        router_load_hxe8(a, j, wq);
        return;
    }
    if (E % 8) {
        // rows not 16-byte aligned: one element per load
        const int e = min(8 * j + (tid >> 5), E - 1);
        const uint16_t *base = static_cast<const uint16_t *>(layer_w(a, 0)->router_w) + e + (size_t)(tid & 31) * 8 * E;
#pragma unroll
        for (int k = 0; k < kNC; ++k) {
            uint32_t v[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = k < NC ? *glb(base + ((size_t)k * 256 + i) * E) : 0u;
            wq[k] = make_uint4(v[0] | (v[1] << 16), v[2] | (v[3] << 16), v[4] | (v[5] << 16), v[6] | (v[7] << 16));
        }
        return;
    }
    // Block k covers rows 256 k .. 256 k + 255: thread t requests the 16 bytes of row 256 k + t
    // that hold experts 8 j .. 8 j + 7 (every block's load is issued first); all blocks then go
    // into one LDS tile (H / 256 blocks of 288 x 16 bytes at the head of LDS, which the one-layer launch provides;
    // rows padded by 16 bytes every 8 rows, which spreads the banks), from which thread (expert
    // tid / 32, lane l = tid % 32) takes rows 8 l .. 8 l + 7 of its expert in every block. The
    // tile lies in LDS that layer_input and the routing fill only after this.
    const uint16_t *col = static_cast<const uint16_t *>(layer_w(a, 0)->router_w) + 8 * j;
    uint4 r[kNC];
#pragma unroll
    for (int k = 0; k < kNC; ++k) r[k] = ld16(col + ((size_t)min(k, NC - 1) * 256 + tid) * E);
    uint4 *tile = reinterpret_cast<uint4 *>(ulds());   // kNC x 288 x 16 bytes
    const uint16_t *t16 = reinterpret_cast<const uint16_t *>(ulds());
    const int e = tid >> 5, l8 = (tid & 31) * 8;
#pragma unroll
    for (int k = 0; k < kNC; ++k)
        if (k < NC) tile[k * 288 + tid + (tid >> 3)] = r[k];
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kNC; ++k) {
        if (k < NC) {
            uint32_t v[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = t16[(k * 288 + l8 + i + ((l8 + i) >> 3)) * 8 + e];
            wq[k] = make_uint4(v[0] | (v[1] << 16), v[2] | (v[3] << 16), v[4] | (v[5] << 16), v[6] | (v[7] << 16));
        } else {
            wq[k] = make_uint4(0u, 0u, 0u, 0u);
        }
    }
    __syncthreads();
}

// Router workgroup j, layer l: u_l, then the logits of experts 8j .. 8j+7 for every
// token (weights already in wq).
template <int MT>
__device__ __forceinline__ void router_phase(AP a0, int l, int j, const uint4 (&wq)[kNC], uint32_t tgt) {
    const AP a = uniform(a0);
    const int E = a->E, tid = ltid(), lane32 = tid & 31;
    const int e = 8 * j + (tid >> 5);
    const bool valid = e < E;
    const float *bias = layer_w(a, l)->router_bias;
    const float bv = (bias && valid) ? glb(bias)[e] : 0.0f;   // requested before the norm's polls
    const float *rsp = layer_w(a, l)->router_s;
    const float rs = (a->router_fp8 && valid) ? glb(rsp)[e] : 1.0f;   // FP8 router: the expert's scale
    layer_input<MT>(a, l, tgt);
    const uint16_t *u = ulds();
    float acc[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m] = 0.0f;
    int off = lane32 * 8;   // this lane's columns of the token's row of u
#pragma unroll
    for (int m = 0; m < MT; m += 2) {
        // two tokens' rows at a time: their reads are issued together and their sums
        // interleave; the row offset depends on the previous pair's sums, so the next
        // pair's reads are not hoisted into this pair's registers
#pragma unroll
        for (int k = 0; k < kNC; ++k) {
#pragma unroll
            for (int mm = 0; mm < 2; ++mm) {
                if (m + mm < MT) {
                    const uint4 xv = *reinterpret_cast<const uint4 *>(u + off + mm * kUS + k * 256);
                    acc[m + mm] = dot2(as_bf2(wq[k].x), as_bf2(xv.x), acc[m + mm]);
                    acc[m + mm] = dot2(as_bf2(wq[k].y), as_bf2(xv.y), acc[m + mm]);
                    acc[m + mm] = dot2(as_bf2(wq[k].z), as_bf2(xv.z), acc[m + mm]);
                    acc[m + mm] = dot2(as_bf2(wq[k].w), as_bf2(xv.w), acc[m + mm]);
                }
            }
        }
        off += 2 * kUS;
        asm volatile("" : "+v"(off) : "v"(acc[m]), "v"(acc[m + 1 < MT ? m + 1 : m]));
    }
    // every logit is formed before the first store: stores count against the same
    // in-order counter as loads, so a wait placed between two stores would also wait
    // for the first store to complete
    float v[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) v[m] = half_sum(acc[m]) * rs + bv;
    uint64_t *lg = logits(a, l);
    if (lane32 == 16 && valid) {
#pragma unroll
        for (int m = 0; m < MT; ++m) st64(lg + (size_t)m * E + e, tagged(__float_as_uint(v[m]), tgt));
    }
}

// ------------------------------------------------------------------ route

constexpr int kEI = kMaxExperts / 64;   // experts per lane in the top-K selection

// Every workgroup, layer l: route. Wave w selects the top K of tokens w and w+4 (in the
// same rounds): each lane
// holds the (ordered logit, inverted id) keys of experts lane, lane+64, ..., and K
// rounds of a wave-wide maximum take the largest remaining key (ties to the lower id).
// The selected experts' softmax weights are renormalised over the K (the full softmax
// denominator cancels). Then every thread e builds expert e's slot from the per-token
// selection masks: the slot list is the shared expert, then the union of selected
// experts in ascending id. Returns the number of slots.
template <int MT>
__device__ __forceinline__ int route_phase(AP a0, int l, uint32_t tgt, bool outputs) {
    const AP a = uniform(a0);
    const int E = a->E, M = MT, K = a->K, tid = ltid(), lane = tid & 63, wave = tid >> 6;
    SlotLds &S = slots(a);
    float *wt = reinterpret_cast<float *>(scratch(a));   // [M][E] weight of expert e for token m
    const uint64_t *src = logits(a, l);
    // Wave w selects token w and, with more than four tokens, token w + 4 in the same
    // rounds: a round is a chain of dependent cross-lane steps, so two tokens' chains
    // interleaved take about as long as one.
    constexpr int NT = MT > 4 ? 2 : 1;
    if (wave < M) {   // waves without a token skip the selection
        float lgv[NT][kEI];
        {
            Poll pl;
            bool ok;
            do {
                uint64_t v[NT][kEI];
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    const int m = wave + 4 * t;
#pragma unroll
                    for (int i = 0; i < kEI; ++i)
                        if (m < M && lane + 64 * i < E) v[t][i] = ld64(src + (size_t)m * E + lane + 64 * i);
                }
                ok = true;
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    const int m = wave + 4 * t;
#pragma unroll
                    for (int i = 0; i < kEI; ++i) {
                        lgv[t][i] = 0.0f;
                        if (m < M && lane + 64 * i < E) {
                            lgv[t][i] = __uint_as_float((uint32_t)v[t][i]);
                            ok = ok && current(v[t][i], tgt);
                        }
                    }
                }
            } while (!pl.done(a, ok));
        }
        // the K largest ordered logits over the wave (ties: lower id), by bisection on the value
        uint32_t o[NT][kEI];
        unsigned sel[NT];   // bit i: this lane's expert lane + 64 i is selected
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int i = 0; i < kEI; ++i) o[t][i] = wave + 4 * t < M && lane + 64 * i < E ? ordered(lgv[t][i]) : 0u;
        uint32_t wmax[NT];
        if (E <= 128) {   // two 64-expert words suffice: the bisection counts only those
            uint32_t o2[NT][2];
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                o2[t][0] = o[t][0];
                o2[t][1] = o[t][1];
            }
            topk_bisect<NT, 2>(o2, K, lane, sel, wmax);
        } else {
            topk_bisect<NT, kEI>(o, K, lane, sel, wmax);
        }
        float lmax[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) lmax[t] = unordered(wmax[t]);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const int m = wave + 4 * t;
            if (m >= M) break;
            float ev[kEI], zl = 0.0f;
#pragma unroll
            for (int i = 0; i < kEI; ++i) {
                ev[i] = (sel[t] >> i) & 1u ? expf(lgv[t][i] - lmax[t]) : 0.0f;
                zl += ev[i];
            }
            const float z = wave_sum(zl);
            int before = 0;
#pragma unroll
            for (int i = 0; i < kEI; ++i) {
                const bool si = (sel[t] >> i) & 1u;
                const unsigned long long bm = __ballot(si);
                if (lane == 0) S.bal[m][i] = bm;
                if (si) {
                    const int e = lane + 64 * i, pos = before + lanes_below(bm);
                    const float wv = ev[i] / z;
                    wt[m * E + e] = wv;
                    if (outputs) {
                        if (a->topk_idx) glb(a->topk_idx)[((size_t)l * M + m) * K + pos] = e;
                        if (a->topk_w) glb(a->topk_w)[((size_t)l * M + m) * K + pos] = wv;
                    }
                }
                before += __popcll(bm);
            }
        }
    }
    __syncthreads();
    const int has_sh = a->Ds > 0, nsh = has_sh ? a->nseg_s : 0, nsr = a->nseg_r;
    // union of the selections, and for expert tid = lane + 64 * wave its selection mask
    // word and the number of experts each token selected below its word; every mask word
    // is read once, all together (register arrays are only indexed by constants)
    unsigned long long U[kEI], Bw[MT];
    int pre[MT];
#pragma unroll
    for (int i = 0; i < kEI; ++i) U[i] = 0ull;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        Bw[m] = 0ull;
        pre[m] = 0;
#pragma unroll
        for (int i = 0; i < kEI; ++i) {
            const unsigned long long b = S.bal[m][i];
            U[i] |= b;
            pre[m] += i < wave ? __popcll(b) : 0;
            Bw[m] = i == wave ? b : Bw[m];
        }
    }
    int ns = has_sh;
#pragma unroll
    for (int i = 0; i < kEI; ++i) ns += __popcll(U[i]);
    if (tid < E) {
        unsigned um = 0;
        float wm[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            um |= (unsigned)((Bw[m] >> lane) & 1ull) << m;
            wm[m] = wt[m * E + tid];
        }
        if (um) {
            int slot = has_sh;
            unsigned long long Uw = 0ull;
#pragma unroll
            for (int q = 0; q < kEI; ++q) {
                if (q < wave) slot += __popcll(U[q]);
                if (q == wave) Uw = U[q];
            }
            slot += lanes_below(Uw);
            S.se[slot] = tid;
            S.sm[slot] = um;
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                const bool on = (um >> m) & 1u;
                S.sw[slot][m] = on ? wm[m] : 0.0f;
                if (on) {
                    // expert tid's place in token m's list (ascending id); the shared
                    // expert's segments follow the K routed experts
                    const int pos = pre[m] + lanes_below(Bw[m]);
                    for (int sg = 0; sg < nsr; ++sg) S.tsub[m][pos * nsr + sg] = nsh + (slot - has_sh) * nsr + sg;
                }
            }
        }
    }
    if (tid < M) {
        for (int sg = 0; sg < nsh; ++sg) S.tsub[tid][K * nsr + sg] = sg;
        if (has_sh) S.sw[0][tid] = 1.0f;
    }
    if (tid == 0 && has_sh) {
        S.se[0] = E;
        S.sm[0] = (1u << M) - 1u;
    }
    __syncthreads();
    return __builtin_amdgcn_readfirstlane(ns);
}

// ----------------------------------------------------------------- units

// A unit's weights, 16-byte pieces (16 FP8 codes) per lane: gate/up units hold pieces
// j, j + 32, ... of the gate row in w[0..kPc) and of the up row in w[kPc..2kPc) (32
// lanes per row); down units hold pieces j, j + 8, ... of row c in w[0..kPc) and of row
// c + 32 in w[kPc..2kPc) (8 lanes per row pair). Pieces past the row are zero. sc holds
// the two rows' scales.
struct UnitBuf {
    uint4 w[2 * kPc];
    float sc[2];
};

enum { kGU = 0, kDN = 1, kCMB = 2 };

// Unit geometry per expert weight type: FP8 codes (16 to a 16-byte piece) or bf16 weights
// (8 to a piece). A bf16 unit has half the rows of an FP8 unit, so that both hold kPc
// pieces of each of two rows per lane.
template <bool BF>
struct Geo {
    static constexpr int EB = BF ? 2 : 1;      // bytes per weight
    static constexpr int CP = 16 / EB;         // columns per piece
    static constexpr int RG = BF ? 4 : 8;      // gate (and up) rows per gate/up unit
    static constexpr int LG = kWG / RG;        // lanes per gate/up row
    static constexpr int RD = BF ? 32 : 64;    // rows per down unit
    static constexpr int LD = 2 * kWG / RD;    // lanes per down row pair
    static_assert(LG * kPc * CP == kUS && LD * kPc * CP == kDS, "a unit row fills a padded LDS row");
};

struct UnitRef {
    int kind;
    int s;       // slot (gate/up, down)
    int row0;    // gate/up: the first of its rows
    int js;      // down: sub-slot
    int seg;     // down: column segment
    int cb;      // down: row block; combine: 64-row block
};

// The layer's unit list: the shared expert's gate/up units, its down units, the routed
// slots' gate/up units, their down units, then the combine units. The shared expert's
// units come first so that their place in the list does not depend on the routing.
struct UnitList {
    int sh_gu, sh_dn, r_gu, r_dn, U;   // ends of the five ranges
    int nsub;                           // sub-slots
};

template <bool BF>
__device__ __forceinline__ UnitList unit_list(AP a, int ns) {
    using g = Geo<BF>;
    UnitList L;
    const int has_sh = a->Ds > 0, nr = ns - has_sh, ndn = a->H / g::RD;
    L.sh_gu = has_sh ? a->Ds / g::RG : 0;
    L.sh_dn = L.sh_gu + (has_sh ? a->nseg_s * ndn : 0);
    L.r_gu = L.sh_dn + nr * (a->D / g::RG);
    L.r_dn = L.r_gu + nr * a->nseg_r * ndn;
    L.U = L.r_dn + a->ND;
    L.nsub = (has_sh ? a->nseg_s : 0) + nr * a->nseg_r;
    return L;
}

template <bool BF>
__device__ __forceinline__ UnitRef decode_unit(AP a, int q, const UnitList &L) {
    using g = Geo<BF>;
    UnitRef u;
    const int has_sh = a->Ds > 0, ndn = a->H / g::RD;
    u.s = u.row0 = u.js = u.seg = u.cb = 0;
    if (q < L.sh_gu) {
        u.kind = kGU;
        u.row0 = g::RG * q;
    } else if (q < L.sh_dn) {
        const int r = q - L.sh_gu;
        u.kind = kDN;
        u.js = u.seg = r / ndn;
        u.cb = r % ndn;
    } else if (q < L.r_gu) {
        const int r = q - L.sh_dn, DG = a->D / g::RG;
        u.kind = kGU;
        u.s = has_sh + r / DG;
        u.row0 = g::RG * (r % DG);
    } else if (q < L.r_dn) {
        const int r = q - L.r_gu, jr = r / ndn;
        u.kind = kDN;
        u.cb = r % ndn;
        u.js = (has_sh ? a->nseg_s : 0) + jr;
        u.s = has_sh + jr / a->nseg_r;
        u.seg = jr % a->nseg_r;
    } else {
        u.kind = kCMB;
        u.cb = q - L.r_dn;
    }
    return u;
}

// Request a unit's weights. Before the routing is known (pre_route) only the shared
// expert's units can be loaded.
template <bool BF>
__device__ __forceinline__ void load_unit(AP a, int l, const UnitRef &u, UnitBuf &b, bool pre_route) {
    using g = Geo<BF>;
    if (u.kind == kCMB) return;
    const WP wp = layer_w(a, l);
    const SlotLds &S = slots(a);
    // the unit's expert is the same for the whole workgroup
    const int e = __builtin_amdgcn_readfirstlane(pre_route ? a->E : S.se[u.s]), tid = ltid(), H = a->H;
    const bool shared = e == a->E;
    // Pieces past the end of a row re-read the row's last piece: they meet the zero
    // columns past the row in the LDS copy of u or h, and a single unconditional 16-byte
    // load per piece keeps the loads free of per-lane branches. bf16 weights carry no
    // scales (1).
    if (u.kind == kGU) {
        const int NP = H / g::CP, j = tid % g::LG, row = u.row0 + tid / g::LG;
        const size_t eoff = (size_t)e * a->D;
        const uint4 *gp = reinterpret_cast<const uint4 *>(
            (shared ? (const uint8_t *)wp->sh_gate_w : (const uint8_t *)wp->gate_w + eoff * H * g::EB) + (size_t)row * H * g::EB);
        const uint4 *vp = reinterpret_cast<const uint4 *>(
            (shared ? (const uint8_t *)wp->sh_up_w : (const uint8_t *)wp->up_w + eoff * H * g::EB) + (size_t)row * H * g::EB);
#pragma unroll
        for (int i = 0; i < kPc; ++i) b.w[i] = ld16nt(gp + min(j + g::LG * i, NP - 1));
#pragma unroll
        for (int i = 0; i < kPc; ++i) b.w[kPc + i] = ld16nt(vp + min(j + g::LG * i, NP - 1));
        b.sc[0] = BF ? 1.0f : *glb((shared ? wp->sh_gate_s : wp->gate_s + eoff) + row);
        b.sc[1] = BF ? 1.0f : *glb((shared ? wp->sh_up_s : wp->up_s + eoff) + row);
    } else {
        const int F = shared ? a->Ds : a->D, segF = F / (shared ? a->nseg_s : a->nseg_r), NP = segF / g::CP;
        const int j = tid % g::LD, c0 = u.cb * g::RD + tid / g::LD;
        const uint8_t *dp = (shared ? (const uint8_t *)wp->sh_down_w : (const uint8_t *)wp->down_w + (size_t)e * H * a->D * g::EB) +
                            ((size_t)c0 * F + u.seg * segF) * g::EB;
        const uint4 *d0 = reinterpret_cast<const uint4 *>(dp);
        const uint4 *d1 = reinterpret_cast<const uint4 *>(dp + (size_t)(g::RD / 2) * F * g::EB);
#pragma unroll
        for (int i = 0; i < kPc; ++i) b.w[i] = ld16nt(d0 + min(j + g::LD * i, NP - 1));
#pragma unroll
        for (int i = 0; i < kPc; ++i) b.w[kPc + i] = ld16nt(d1 + min(j + g::LD * i, NP - 1));
        const float *ds = shared ? wp->sh_down_s : wp->down_s + (size_t)e * H;
        b.sc[0] = BF ? 1.0f : *glb(ds + c0);
        b.sc[1] = BF ? 1.0f : *glb(ds + c0 + g::RD / 2);
    }
}

template <int MT>
__device__ __forceinline__ void slot_tokens(unsigned mask, int (&toks)[MT]) {
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        toks[t] = mask ? __ffs(mask) - 1 : 0;
        mask &= mask - 1u;
    }
}

// Gate/up unit: RG rows of the slot's gate and up matrices; lane group r (LG lanes)
// computes row row0 + r of both, CP columns of every LG * CP-column stretch per lane.
// Tokens are taken one at a time in a loop (FP8 codes are decoded again per token: one
// instruction per pair) so that the code does not grow with the token count.
template <int MT, bool BF>
__device__ __forceinline__ void run_gu(AP a, int l, const UnitRef &u, const UnitBuf &b, uint32_t tgt) {
    using g = Geo<BF>;
    const SlotLds &S = slots(a);
    const int tid = ltid(), j = tid % g::LG, row = u.row0 + tid / g::LG;
    const uint16_t *ul = ulds();
    unsigned mm = S.sm[u.s];
#pragma unroll 1
    while (mm) {
        const int m = __ffs(mm) - 1;
        mm &= mm - 1u;
        float ag = 0.0f, au = 0.0f;
        const uint16_t *um = ul + m * kUS + j * g::CP;
        if constexpr (BF) {
#pragma unroll
            for (int i = 0; i < kPc; ++i) {
                const uint4 gw = b.w[i], vw = b.w[kPc + i];
                const uint4 x0 = *reinterpret_cast<const uint4 *>(um + i * g::LG * g::CP);
                ag = dot2(as_bf2(gw.x), as_bf2(x0.x), ag);
                ag = dot2(as_bf2(gw.y), as_bf2(x0.y), ag);
                ag = dot2(as_bf2(gw.z), as_bf2(x0.z), ag);
                ag = dot2(as_bf2(gw.w), as_bf2(x0.w), ag);
                au = dot2(as_bf2(vw.x), as_bf2(x0.x), au);
                au = dot2(as_bf2(vw.y), as_bf2(x0.y), au);
                au = dot2(as_bf2(vw.z), as_bf2(x0.z), au);
                au = dot2(as_bf2(vw.w), as_bf2(x0.w), au);
            }
        } else {
            // the decode scale is opaque per token, so the decoded weights are not hoisted
            // out of the token loop (holding them would cost 88 registers and occupancy)
            float one = 1.0f;
            asm volatile("" : "+v"(one));
#pragma unroll
            for (int i = 0; i < kPc; ++i) {
                const uint4 gw = b.w[i], vw = b.w[kPc + i];
                const uint4 x0 = *reinterpret_cast<const uint4 *>(um + i * g::LG * g::CP);
                const uint4 x1 = *reinterpret_cast<const uint4 *>(um + i * g::LG * g::CP + 8);
                ag = dot2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(gw.x, one, false), as_bf2(x0.x), ag);
                ag = dot2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(gw.x, one, true), as_bf2(x0.y), ag);
                ag = dot2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(gw.y, one, false), as_bf2(x0.z), ag);
                ag = dot2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(gw.y, one, true), as_bf2(x0.w), ag);
                ag = dot2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(gw.z, one, false), as_bf2(x1.x), ag);
                ag = dot2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(gw.z, one, true), as_bf2(x1.y), ag);
                ag = dot2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(gw.w, one, false), as_bf2(x1.z), ag);
                ag = dot2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(gw.w, one, true), as_bf2(x1.w), ag);
                au = dot2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(vw.x, one, false), as_bf2(x0.x), au);
                au = dot2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(vw.x, one, true), as_bf2(x0.y), au);
                au = dot2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(vw.y, one, false), as_bf2(x0.z), au);
                au = dot2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(vw.y, one, true), as_bf2(x0.w), au);
                au = dot2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(vw.z, one, false), as_bf2(x1.x), au);
                au = dot2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(vw.z, one, true), as_bf2(x1.y), au);
                au = dot2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(vw.w, one, false), as_bf2(x1.z), au);
                au = dot2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(vw.w, one, true), as_bf2(x1.w), au);
            }
        }
        // a row's sum: over its half-wave (valid in lanes 16..31 of it) or its wave
        const float gs = BF ? wave_sum(ag) : half_sum(ag);
        const float us = BF ? wave_sum(au) : half_sum(au);
        if (j == (BF ? 0 : 16))
            st64(hact(a, l, u.s, m) + row, tagged(__float_as_uint(gelu_tanh(b.sc[0] * gs) * (b.sc[1] * us)), tgt));
    }
}

constexpr int kStage = 8;    // h words per thread per staging round of a down unit
constexpr int kCmbChunk = 12;   // sub-slot words per poll of a combine unit

// Down unit: rows c0 = RD cb + tid / LD and c0 + RD / 2 of the slot's down matrix over
// one column segment (LD lanes per row pair, CP columns of every LD * CP-column stretch
// per lane), for the slot's tokens, weighted by their combine weights.
template <int MT, bool BF>
__device__ __forceinline__ void run_dn(AP a, int l, const UnitRef &u, const UnitBuf &b, uint32_t tgt) {
    using g = Geo<BF>;
    const SlotLds &S = slots(a);
    const int e = S.se[u.s], tid = ltid(), j = tid % g::LD;
    const bool shared = e == a->E;
    const int F = shared ? a->Ds : a->D, segF = F / (shared ? a->nseg_s : a->nseg_r);
    const unsigned mask = S.sm[u.s];
    const int ntok = __popc(mask);
    int toks[MT];
    slot_tokens<MT>(mask, toks);
    // the slot's h for this segment, [ntok][kDS] in LDS (zeros past segF), polled until
    // current
    float *hs = reinterpret_cast<float *>(scratch(a));
    {
        const int np = ntok * segF;
#pragma unroll 1
        for (int k0 = 0; k0 * kWG < np; k0 += kStage) {
            float pv[kStage];
            Poll pl;
            bool ok;
            do {
                uint64_t v[kStage];
#pragma unroll
                for (int k = 0; k < kStage; ++k) {
                    const int i = tid + (k0 + k) * kWG;
                    if (i < np) {
                        int t = 0;
#pragma unroll
                        for (int tt = 1; tt < MT; ++tt) t += i >= tt * segF;
                        int m = toks[0];
#pragma unroll
                        for (int tt = 1; tt < MT; ++tt) m = t == tt ? toks[tt] : m;
                        v[k] = ld64(hact(a, l, u.s, m) + u.seg * segF + (i - t * segF));
                    }
                }
                ok = true;
#pragma unroll
                for (int k = 0; k < kStage; ++k) {
                    const int i = tid + (k0 + k) * kWG;
                    if (i < np) {
                        pv[k] = __uint_as_float((uint32_t)v[k]);
                        ok = ok && current(v[k], tgt);
                    }
                }
            } while (!pl.done(a, ok));
#pragma unroll
            for (int k = 0; k < kStage; ++k) {
                const int i = tid + (k0 + k) * kWG;
                if (i < np) {
                    int t = 0;
#pragma unroll
                    for (int tt = 1; tt < MT; ++tt) t += i >= tt * segF;
                    hs[t * kDS + (i - t * segF)] = pv[k];
                }
            }
        }
        if (segF < kDS) {
            const int pad = kDS - segF;
            for (int i = tid; i < ntok * pad; i += kWG) {
                const int t = i / pad;
                hs[t * kDS + segF + (i - t * pad)] = 0.0f;
            }
        }
    }
    __syncthreads();
    const float4 *hs4 = reinterpret_cast<const float4 *>(hs);
    const int c0 = u.cb * g::RD + tid / g::LD;
#pragma unroll 1
    for (int t = 0; t < ntok; ++t) {
        const int m = toks[0];
        float s0 = 0.0f, s1 = 0.0f;
        int zero = 0;   // opaque per token: the decoded weights stay inside the loop
        asm volatile("" : "+v"(zero));
#pragma unroll
        for (int i = 0; i < kPc; ++i) {
            // piece j + LD i of both rows: columns CP (j + LD i) .. + CP - 1 of the segment
            const float4 *hp = hs4 + (t * kDS + (j + g::LD * i) * g::CP) / 4;
            const uint32_t wv[4] = {b.w[i].x | zero, b.w[i].y | zero, b.w[i].z | zero, b.w[i].w | zero};
            const uint32_t vv[4] = {b.w[kPc + i].x | zero, b.w[kPc + i].y | zero, b.w[kPc + i].z | zero,
                                    b.w[kPc + i].w | zero};
            if constexpr (BF) {
                const float4 hq[2] = {hp[0], hp[1]};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float hx = q & 1 ? hq[q >> 1].z : hq[q >> 1].x, hy = q & 1 ? hq[q >> 1].w : hq[q >> 1].y;
                    s0 = fmaf(__uint_as_float(wv[q] << 16), hx, s0);
                    s0 = fmaf(__uint_as_float(wv[q] & 0xffff0000u), hy, s0);
                    s1 = fmaf(__uint_as_float(vv[q] << 16), hx, s1);
                    s1 = fmaf(__uint_as_float(vv[q] & 0xffff0000u), hy, s1);
                }
            } else {
                const float4 hq[4] = {hp[0], hp[1], hp[2], hp[3]};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const f32x2 p0 = fp8x2_to_f32<false>(wv[q]), p1 = fp8x2_to_f32<true>(wv[q]);
                    const f32x2 q0 = fp8x2_to_f32<false>(vv[q]), q1 = fp8x2_to_f32<true>(vv[q]);
                    s0 = fmaf(p0.x, hq[q].x, s0); s0 = fmaf(p0.y, hq[q].y, s0);
                    s0 = fmaf(p1.x, hq[q].z, s0); s0 = fmaf(p1.y, hq[q].w, s0);
                    s1 = fmaf(q0.x, hq[q].x, s1); s1 = fmaf(q0.y, hq[q].y, s1);
                    s1 = fmaf(q1.x, hq[q].z, s1); s1 = fmaf(q1.y, hq[q].w, s1);
                }
            }
        }
        // sums over the LD lanes of the row pair (8: two quads; 16: a DPP row)
        float v0 = quad_sum(s0);
        v0 += dpp<0x141>(v0);   // row_half_mirror: the two quads of each 8-lane group
        float v1 = quad_sum(s1);
        v1 += dpp<0x141>(v1);
        if constexpr (BF) {
            v0 += dpp<0x140>(v0);   // row_mirror: the two halves of the 16-lane row
            v1 += dpp<0x140>(v1);
        }
        if (j == 0) {
            const float cw = S.sw[u.s][m];
            uint64_t *yp = ypart(a, l, u.js, m);
            st64(yp + c0, tagged(__float_as_uint(cw * (b.sc[0] * v0)), tgt));
            st64(yp + c0 + g::RD / 2, tagged(__float_as_uint(cw * (b.sc[1] * v1)), tgt));
        }
        // the next token of the slot
#pragma unroll
        for (int q = 0; q + 1 < MT; ++q) toks[q] = toks[q + 1];
    }
    // hs is reused by the next down unit
    __syncthreads();
}

// Combine unit cb: y_l rows = bf16 of the token's sub-slots summed in order;
// h_{l+1} = bf16(h_l + noise_{l+1} + y_l) (no noise after the last layer). In pass p,
// thread t owns row 64 cb + (i & 63) of token i >> 6, i = 256 p + t; neighbouring
// lanes hold a row pair and trade values through DPP.
template <int MT>
__device__ __forceinline__ void run_cmb(AP a, int l, int cb, uint32_t tgt) {
    const SlotLds &S = slots(a);
    const int M = MT, H = a->H, tid = ltid();
    const int n = (a->Ds > 0 ? a->nseg_s : 0) + a->K * a->nseg_r;
    for (int p = 0; p * kWG < M * 64; ++p) {
        const int i = p * kWG + tid, m = i >> 6, c = cb * 64 + (i & 63);
        const bool act = m < M, odd = (i & 1) != 0;
        // the noise is requested before the polls, so that it arrives while they wait
        const uint16_t nz = act && l + 1 < a->L ? glb(a->noise)[((size_t)(l + 1) * M + m) * H + c] : (uint16_t)0;
        float s = 0.0f;
        uint32_t hp = 0;
        for (int k0 = 0; k0 < n; k0 += kCmbChunk) {
            // sub-slots k0 .. k0 + 11 (and, with the first chunk, the residual word)
            float sc = 0.0f;
            Poll pl;
            bool ok;
            do {
                uint64_t v[kCmbChunk], hv = 0;
#pragma unroll
                for (int k = 0; k < kCmbChunk; ++k)
                    if (act && k0 + k < n) v[k] = ld64(ypart(a, l, S.tsub[m][k0 + k], m) + c);
                if (act && l > 0 && k0 == 0) hv = ld64(hres(a, l, m) + c / 2);
                ok = true;
                sc = s;
#pragma unroll
                for (int k = 0; k < kCmbChunk; ++k) {
                    if (act && k0 + k < n) {
                        sc += __uint_as_float((uint32_t)v[k]);
                        ok = ok && current(v[k], tgt);
                    }
                }
                if (act && l > 0 && k0 == 0) {
                    hp = (uint32_t)hv;
                    ok = ok && current(hv, tgt);
                }
            } while (!pl.done(a, ok));
            s = sc;
        }
        if (act && l == 0 && !a->layer_mode) hp = h0_pair(a, m, c / 2);
        const uint16_t y = f2bf(s);
        float hv = bf2f(odd ? hp >> 16 : hp & 0xffffu);
        if (act && l + 1 < a->L) hv += bf2f(nz);
        const uint16_t hn = f2bf(hv + bf2f(y));
        // the pair partner's values (quad_perm [1,0,3,2])
        const uint32_t yo = dppu<0xB1>(y), ho = dppu<0xB1>(hn);
        if (act && !odd) {
            if (a->y) *glb(reinterpret_cast<uint32_t *>(a->y + (size_t)l * a->y_ls + (size_t)m * H + c)) = pack2(y, (uint16_t)yo);
            if (!a->layer_mode) st64(hres(a, l + 1, m) + c / 2, tagged(pack2(hn, (uint16_t)ho), tgt));
        }
    }
}

template <int MT, bool BF>
__device__ __forceinline__ void run_unit(AP a, int l, const UnitRef &u, const UnitBuf &b, uint32_t tgt) {
    if (u.kind == kGU) {
        run_gu<MT, BF>(a, l, u, b, tgt);
    } else if (u.kind == kDN) {
        run_dn<MT, BF>(a, l, u, b, tgt);
    } else {
        run_cmb<MT>(a, l, u.cb, tgt);
    }
}

// Unit workgroup w (0 <= w < GU), layer l: u_l, the routing, then its units w, w + GU,
// ..., two in flight with several tokens and one with one token (about 45 MB requested
// across the chip with two; a measured sweep of
// expert-shaped 45 KB reads on MI355X holds 6-6.7 TB/s at one or two units per
// workgroup, and deeper prefetch loses bandwidth once the units carry compute). A
// shared-expert unit's weights are requested before the routing is known.
template <int MT, bool BF>
__device__ __forceinline__ void expert_phase(AP a0, int l, int w, int GU, uint32_t tgt) {
    const AP a = uniform(a0);
    // the residual rows are polled with long sleeps in between: a unit workgroup needs u_l
    // only after the logits, which come a hop and a router GEMV after the rows, and every
    // unit workgroup polls meanwhile (64 measured faster than 1 at one and five tokens)
    layer_input<MT, 64>(a, l, tgt);
    // the shared expert's units sit at fixed places at the head of the list
    const UnitList L0 = unit_list<BF>(a, a->Ds > 0 ? 1 : 0);
    UnitBuf A;
    const bool early = w < L0.sh_dn;
    if (early) load_unit<BF>(a, l, decode_unit<BF>(a, w, L0), A, true);
    const int ns = route_phase<MT>(a, l, tgt, w == 0);
    const UnitList L = unit_list<BF>(a, ns);
    if (!early && w < L.U) load_unit<BF>(a, l, decode_unit<BF>(a, w, L), A, false);
    if constexpr (MT == 1) {
        // One token: one unit in flight per workgroup, requested as soon as the routing
        // is known (or the unit before it is done) and computed as soon as its weights
        // are in. A second unit in flight would hold the first unit's compute until the
        // second's loads had been accepted, which takes as long as the layer's weight
        // burst.
        for (int i = w; i < L.U; i += GU) {
            if (i != w) load_unit<BF>(a, l, decode_unit<BF>(a, i, L), A, false);
            run_unit<MT, BF>(a, l, decode_unit<BF>(a, i, L), A, tgt);
        }
        return;
    }
    UnitBuf B;
    if (w + GU < L.U) load_unit<BF>(a, l, decode_unit<BF>(a, w + GU, L), B, false);
    for (int i = w; i < L.U; i += 2 * GU) {
        run_unit<MT, BF>(a, l, decode_unit<BF>(a, i, L), A, tgt);
        if (i + 2 * GU < L.U) load_unit<BF>(a, l, decode_unit<BF>(a, i + 2 * GU, L), A, false);
        if (i + GU < L.U) {
            run_unit<MT, BF>(a, l, decode_unit<BF>(a, i + GU, L), B, tgt);
            if (i + 3 * GU < L.U) load_unit<BF>(a, l, decode_unit<BF>(a, i + 3 * GU, L), B, false);
        }
    }
}

// ------------------------------------------------------------------ lm_head

constexpr int kLmRows = 4;   // rows per lane (same column chunk)

struct LmBuf {
    uint4 q[kLmRows];
};

template <int MT>
struct LmAcc {
    float acc[kLmRows][MT];
    float sc[kLmRows];
    unsigned long long best[MT];
};

// Chunks per row of the lm_head: 16 lanes x 16 bytes, 256 FP8 columns or 128 bf16 columns
// (LBF: bf16 weights without scales).
template <bool LBF>
__device__ __forceinline__ int lm_chunks(AP a) { return LBF ? a->H / 128 : a->H / 256; }

// step st of this workgroup's row stream: 64-row unit u0 + st / NC, chunk st % NC
template <bool LBF>
__device__ __forceinline__ void lm_load(AP a, int u0, int nst, int st, LmBuf &b) {
    if (st < nst) {
        const int t = ltid(), NC = lm_chunks<LBF>(a), lane = t & 63, wave = t >> 6, EB = LBF ? 2 : 1;
        const int unit = u0 + st / NC, k = st % NC;
        const size_t row = (size_t)unit * 64 + wave * 16 + (lane >> 4) * kLmRows;
        const uint8_t *p = a->lm_w + row * a->H * EB + k * 256 + (lane & 15) * 16;
#pragma unroll
        for (int r = 0; r < kLmRows; ++r) b.q[r] = ld16nt(p + (size_t)r * a->H * EB);
    }
}

template <int MT, bool LBF>
__device__ __forceinline__ void lm_step(AP a, int u0, int nst, int st, const LmBuf &b, LmAcc<MT> &A) {
    if (st >= nst) return;
    const int tid = ltid(), NC = lm_chunks<LBF>(a), M = MT, lane = tid & 63, wave = tid >> 6, li = lane & 15;
    const int k = st % NC;
    const uint16_t *xl = ulds();
    if constexpr (LBF) {
        // bf16 weights: 8 columns per lane, one 16-byte activation piece per token
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            if (t < M) {
                const uint4 x0 = *reinterpret_cast<const uint4 *>(xl + t * kUS + k * 128 + li * 8);
#pragma unroll
                for (int r = 0; r < kLmRows; ++r) {
                    float v = A.acc[r][t];
                    v = dot2(as_bf2(b.q[r].x), as_bf2(x0.x), v);
                    v = dot2(as_bf2(b.q[r].y), as_bf2(x0.y), v);
                    v = dot2(as_bf2(b.q[r].z), as_bf2(x0.z), v);
                    A.acc[r][t] = dot2(as_bf2(b.q[r].w), as_bf2(x0.w), v);
                }
            }
        }
    } else if constexpr (MT == 1) {
        // one token: each row is decoded just before its dot product (fewer live registers)
        const uint4 *xs = reinterpret_cast<const uint4 *>(xl + k * 256 + li * 16);
        const uint4 x0 = xs[0], x1 = xs[1];
#pragma unroll
        for (int r = 0; r < kLmRows; ++r) {
            bf16x2 wv[8];
            decode16_bf16(b.q[r], wv);
            A.acc[r][0] = dot16(wv, x0, x1, A.acc[r][0]);
        }
    } else {
        bf16x2 wv[kLmRows][8];
#pragma unroll
        for (int r = 0; r < kLmRows; ++r) decode16_bf16(b.q[r], wv[r]);
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            if (t < M) {
                const uint4 *xs = reinterpret_cast<const uint4 *>(xl + t * kUS + k * 256 + li * 16);
                const uint4 x0 = xs[0], x1 = xs[1];
#pragma unroll
                for (int r = 0; r < kLmRows; ++r) A.acc[r][t] = dot16(wv[r], x0, x1, A.acc[r][t]);
            }
        }
    }
    if (k == NC - 1) {
        const int unit = u0 + st / NC;
        const int row = unit * 64 + wave * 16 + (lane >> 4) * kLmRows;
#pragma unroll
        for (int r = 0; r < kLmRows; ++r) {
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                if (t < M) {
                    const float lgv = A.sc[r] * row16_sum(A.acc[r][t]);
                    const unsigned long long key = ((unsigned long long)ordered(lgv) << 32) |
                                                   (unsigned long long)(0xffffffffu - (uint32_t)(row + r));
                    A.best[t] = key > A.best[t] ? key : A.best[t];
                }
                A.acc[r][t] = 0.0f;
            }
        }
        if (st + 1 < nst && !LBF) {   // the next unit's scales
#pragma unroll
            for (int r = 0; r < kLmRows; ++r) A.sc[r] = glb(a->lm_s)[row + 64 + r];
        }
    }
}

template <int MT, bool LBF>
__device__ __forceinline__ void lm_phase(AP a0, int w, int G, uint32_t tgt) {
    const AP a = uniform(a0);
    const int H = a->H, M = MT, NC = lm_chunks<LBF>(a), tid = ltid(), lane = tid & 63, wave = tid >> 6;
    const int u0 = (int)((long long)w * a->NLU / G), u1 = (int)((long long)(w + 1) * a->NLU / G);
    const int nst = (u1 - u0) * NC;
    LmBuf b0, b1, b2;
    lm_load<LBF>(a, u0, nst, 0, b0);
    lm_load<LBF>(a, u0, nst, 1, b1);
    lm_load<LBF>(a, u0, nst, 2, b2);
    LmAcc<MT> A;
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        A.best[t] = 0ull;
#pragma unroll
        for (int r = 0; r < kLmRows; ++r) A.acc[r][t] = 0.0f;
    }
#pragma unroll
    for (int r = 0; r < kLmRows; ++r) A.sc[r] = LBF ? 1.0f : 0.0f;
    if (nst > 0 && !LBF) {
        const int row = u0 * 64 + wave * 16 + (lane >> 4) * kLmRows;
#pragma unroll
        for (int r = 0; r < kLmRows; ++r) A.sc[r] = glb(a->lm_s)[row + r];
    }
    norm_to_lds<MT>(a, a->L, a->gains + (size_t)a->L * H, tgt);
    if (w == 0 && a->x_final) {
        const int r8 = H / 8;   // 16-byte pieces of a row
        for (int i = tid; i < M * r8; i += kWG) {
            const int m = i / r8, c = i - m * r8;
            { const uint4 v = reinterpret_cast<const uint4 *>(ulds() + m * kUS)[c];
              *(GAS u32x4 *)(a->x_final + (size_t)m * H + 8 * c) = u32x4{v.x, v.y, v.z, v.w}; }
        }
    }
    for (int st = 0; st < nst; st += 3) {
        lm_step<MT, LBF>(a, u0, nst, st, b0, A);
        lm_load<LBF>(a, u0, nst, st + 3, b0);
        lm_step<MT, LBF>(a, u0, nst, st + 1, b1, A);
        lm_load<LBF>(a, u0, nst, st + 4, b1);
        lm_step<MT, LBF>(a, u0, nst, st + 2, b2, A);
        lm_load<LBF>(a, u0, nst, st + 5, b2);
    }
    // the workgroup's best per token: 16 lane groups, then one key per token
    unsigned long long *gb = reinterpret_cast<unsigned long long *>(scratch(a));   // [16][MT]
    if ((lane & 15) == 0) {
#pragma unroll
        for (int t = 0; t < MT; ++t) gb[(wave * 4 + (lane >> 4)) * kMaxM + t] = A.best[t];
    }
    __syncthreads();
    if (tid < M) {
        unsigned long long bk = gb[tid];
        for (int k = 1; k < 16; ++k) bk = gb[k * kMaxM + tid] > bk ? gb[k * kMaxM + tid] : bk;
        st64(lmbest(a, w) + tid, bk);
    }
    publish(flags(a) + a->f_lm + w, tgt);
    if (w != 0) return;

    // workgroup 0: every workgroup's keys -> tokens, greedy acceptance, next epoch
    wait_flags(a, flags(a) + a->f_lm, G, tgt);
    unsigned long long kb[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) kb[t] = 0ull;
    for (int i0 = 0; i0 < G; i0 += kWG) {
        const int i = i0 + tid;
        if (i < G) {
            uint64_t v[MT];
#pragma unroll
            for (int t = 0; t < MT; ++t)
                if (t < M) v[t] = ld64(lmbest(a, i) + t);
#pragma unroll
            for (int t = 0; t < MT; ++t)
                if (t < M) kb[t] = v[t] > kb[t] ? v[t] : kb[t];
        }
    }
    __syncthreads();
    unsigned long long *wb = reinterpret_cast<unsigned long long *>(scratch(a));   // [4][MT]
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        if (t < M) {
            const unsigned long long v = wave_max_key(kb[t]);
            if (lane == 0) wb[wave * kMaxM + t] = v;
        }
    }
    __syncthreads();
    if (tid == 0) {
        int tok[MT];
        for (int t = 0; t < M; ++t) {
            unsigned long long key = wb[t];
            for (int q = 1; q < 4; ++q) key = wb[q * kMaxM + t] > key ? wb[q * kMaxM + t] : key;
            tok[t] = (int)(0xffffffffu - (uint32_t)(key & 0xffffffffull));
            glb(a->token)[t] = tok[t];
            if (a->max_logit) glb(a->max_logit)[t] = unordered((uint32_t)(key >> 32));
        }
        const int gamma = M - 1;
        int n = 0;
        while (n < gamma && glb(a->draft)[n] == tok[n]) ++n;
        for (int t = 0; t < M; ++t) glb(a->out_tokens)[t] = t <= n ? tok[t] : -1;
        *glb(a->accepted) = n;
        st32(flags(a) + a->f_epoch, tgt);   // every workgroup has read the epoch by now
    }
}

// Layer mode, the end of the call: workgroup 0 waits for every workgroup's flag (raised
// when it had read the epoch, at its start) and advances the epoch.
__device__ __forceinline__ void layer_end(AP a0, int w, int G, uint32_t tgt) {
    const AP a = uniform(a0);
    if (w != 0) return;
    wait_flags(a, flags(a) + a->f_lm, G, tgt);
    if (ltid() == 0) st32(flags(a) + a->f_epoch, tgt);
}

// ------------------------------------------------------------------- kernel

// Workgroups per compute unit: the register budget the kernel is compiled for, and the
// most the grid uses. The verify batches run two (two units in flight per workgroup).
// One token keeps one unit in flight and runs two workgroups per compute unit, compiled
// for a budget of three: every workgroup forms u_l and routes for itself, polling the
// residual rows and logits meanwhile, and on the Gemma-shaped stack fewer such
// workgroups measured faster (0.81 ms per step at two, 0.84 at three, 1.07 at five,
// 0.90 at one).
template <int MT>
constexpr int step_min_blocks() { return MT == 1 ? 3 : 2; }
template <int MT>
constexpr int step_max_blocks() { return MT == 1 ? 2 : 64; }
template <int MT, bool BF>
__global__ __launch_bounds__(256, step_min_blocks<MT>()) void k_step(StepArgs args) {
    (void)args;
    const AP base = (AP)__builtin_amdgcn_kernarg_segment_ptr();
    const int w = blockIdx.x, G = gridDim.x, GU = G - base->NR;
    const uint32_t tgt = __builtin_amdgcn_readfirstlane(ld32(flags(base) + base->f_epoch)) + 1u;
    // one-layer mode: the step counter may advance once every workgroup has read it, so the
    // flag workgroup 0 waits for at the end is raised here rather than after the work
    if (base->layer_mode) publish(flags(base) + base->f_lm + w, tgt);
    if (w >= GU) {
        // router workgroup: each layer's weights are requested as soon as the previous
        // layer's logits are out
        uint4 wq[kNC];
        if (base->layer_mode && !base->rt)
            router_load_hxe(base, w - GU, wq);
        else
            router_load(base, 0, w - GU, wq);
        for (int l = 0;; ++l) {
            AP a = base;
            asm volatile("" : "+s"(a));
            if (l >= a->L) break;
            router_phase<MT>(a, l, w - GU, wq, tgt);
            if (l + 1 < a->L) router_load(a, l + 1, w - GU, wq);
        }
    } else {
        for (int l = 0;; ++l) {
            // The argument pointer is made opaque each layer so that argument fields are
            // re-read by each phase instead of being held in registers across phases.
            AP a = base;
            asm volatile("" : "+s"(a));
            if (l >= a->L) break;
            expert_phase<MT, BF>(a, l, w, GU, tgt);
        }
    }
    AP a = base;
    asm volatile("" : "+s"(a));
    if (a->layer_mode)
        layer_end(a, w, G, tgt);
    else if (a->lm_bf)   // the lm_head's weight type picks one of two versions of the phase
        lm_phase<MT, true>(a, w, G, tgt);
    else
        lm_phase<MT, false>(a, w, G, tgt);
}

// Router weights [H][E] -> [E][H] (once, at prepare time); T is bf16 bits or FP8 codes.
template <class T>
__global__ void k_router_transpose(const T *__restrict__ src, T *__restrict__ dst, int H, int E) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (size_t)H * E) return;
    const int e = (int)(i / H), h = (int)(i % H);
    dst[i] = src[(size_t)h * E + e];
}

inline hipStream_t Sm(void *p) { return reinterpret_cast<hipStream_t>(p); }

// Every workgroup must be resident at once (units wait on other workgroups' units): the
// grid is the occupancy of the step kernel for M tokens times the compute units. With
// `coop` and outside stream capture the step is launched cooperatively, so the runtime
// starts it only with every workgroup resident and refuses a grid that cannot be
// (MOE_EUNSUPPORTED); it costs about 27 us per step on MI355X. A plain launch (and every
// captured step) relies on the caller not running other work on the device meanwhile;
// the bounded waits end a step that could not make progress (MOE_ETIMEOUT from
// moe_decode_step_status).
template <int MT, bool BF>
int launch_mt(const StepArgs &a, size_t lds, int NR, bool coop, void *stream) {
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_step<MT, BF>, kWG, lds) != hipSuccess || per_cu < 1)
        return MOE_ELAUNCH;
    const int grid = std::min(cus * std::min(per_cu, step_max_blocks<MT>()), kStepMaxGrid);
    if (grid <= NR) return MOE_EUNSUPPORTED;   // the last NR workgroups only route
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(Sm(stream), &cap) != hipSuccess) return MOE_ELAUNCH;
    if (!coop || cap != hipStreamCaptureStatusNone) {
        hipLaunchKernelGGL((k_step<MT, BF>), dim3(grid), dim3(kWG), lds, Sm(stream), a);
        return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ELAUNCH;
    }
    StepArgs arg = a;
    void *params[] = {&arg};
    const hipError_t e = hipLaunchCooperativeKernel(reinterpret_cast<const void *>(&k_step<MT, BF>), dim3(grid),
                                                    dim3(kWG), params, (unsigned)lds, Sm(stream));
    if (e == hipErrorCooperativeLaunchTooLarge) {
        (void)hipGetLastError();
        return MOE_EUNSUPPORTED;
    }
    return e == hipSuccess && hipGetLastError() == hipSuccess ? MOE_OK : MOE_ELAUNCH;
}

// One kernel per token count (token loops are unrolled exactly) and expert weight type.
template <bool BF>
int launch_m(int M, const StepArgs &a, size_t lds, int NR, bool coop, void *stream) {
    switch (M) {
    case 1: return launch_mt<1, BF>(a, lds, NR, coop, stream);
    case 2: return launch_mt<2, BF>(a, lds, NR, coop, stream);
    case 3: return launch_mt<3, BF>(a, lds, NR, coop, stream);
    case 4: return launch_mt<4, BF>(a, lds, NR, coop, stream);
    case 5: return launch_mt<5, BF>(a, lds, NR, coop, stream);
    case 6: return launch_mt<6, BF>(a, lds, NR, coop, stream);
    case 7: return launch_mt<7, BF>(a, lds, NR, coop, stream);
    case 8: return launch_mt<8, BF>(a, lds, NR, coop, stream);
    default: return MOE_EINVAL;
    }
}

// LDS of a launch for M tokens (every LDS array is indexed by the call's tokens, so a
// call with fewer tokens than the descriptor's maximum takes less LDS and can run more
// workgroups per compute unit).
size_t step_lds_bytes(const moe_step_desc &d, int M, int *l_scr, int *l_slot) {
    const int E = d.layer.num_experts;
    const size_t u = (size_t)M * kUS * 2;
    size_t scr = (size_t)M * kDS * 4;
    scr = std::max(scr, (size_t)M * E * 4);
    scr = std::max(scr, (size_t)16 * kMaxM * 8);
    scr = (scr + 15) & ~(size_t)15;
    *l_scr = (int)u;
    *l_slot = (int)(u + scr);
    return u + scr + ((sizeof(SlotLds) + 15) & ~(size_t)15);
}

}  // namespace

int step_prepare(const StepWs &W, const moe_layer_desc &ld, const moe_layer_weights *layers, char *ws) {
    if (hipMemset(ws, 0, W.total) != hipSuccess) return MOE_ELAUNCH;
    if (hipMemcpy(ws + W.table, layers, sizeof(moe_layer_weights) * W.L, hipMemcpyHostToDevice) != hipSuccess)
        return MOE_ELAUNCH;
    const int H = ld.hidden, E = ld.num_experts;
    const size_t n = (size_t)H * E;
    for (int l = 0; l < W.L; ++l) {
        if (ld.router_type & MOE_ROUTER_EXPERT_MAJOR) {   // already [E][H]: copied as it is
            if (hipMemcpy(ws + W.rt + (size_t)l * n * (ld.router_type & MOE_ROUTER_FP8 ? 1 : 2), layers[l].router_w,
                          n * (ld.router_type & MOE_ROUTER_FP8 ? 1 : 2), hipMemcpyDeviceToDevice) != hipSuccess)
                return MOE_ELAUNCH;
            continue;
        }
        if (ld.router_type & MOE_ROUTER_FP8)
            hipLaunchKernelGGL(k_router_transpose<uint8_t>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, nullptr,
                               static_cast<const uint8_t *>(layers[l].router_w),
                               reinterpret_cast<uint8_t *>(ws + W.rt) + (size_t)l * n, H, E);
        else
            hipLaunchKernelGGL(k_router_transpose<uint16_t>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, nullptr,
                               static_cast<const uint16_t *>(layers[l].router_w),
                               reinterpret_cast<uint16_t *>(ws + W.rt) + (size_t)l * n, H, E);
        if (hipGetLastError() != hipSuccess) return MOE_ELAUNCH;
    }
    return hipDeviceSynchronize() == hipSuccess ? MOE_OK : MOE_ELAUNCH;
}

// After a wait has given up, a workgroup that started after workgroup 0 advanced the
// epoch may have written hand-off words with the next step's tag (epoch + 1). The epoch
// is therefore advanced by two more, so that every word in the workspace is older than
// the next step's tag, and the flag is cleared. No step may be in flight.
int step_status(const StepWs &W, char *ws) {
    int err = 0;
    char *flag = ws + W.ctr + sizeof(int) * kCtrStride * kErrCtr;
    if (hipMemcpy(&err, flag, sizeof(int), hipMemcpyDeviceToHost) != hipSuccess) return MOE_ELAUNCH;
    if (!err) return MOE_OK;
    uint32_t epoch = 0;
    char *ep = ws + W.flags + sizeof(uint32_t) * (size_t)W.f_epoch;
    if (hipMemcpy(&epoch, ep, sizeof epoch, hipMemcpyDeviceToHost) != hipSuccess) return MOE_ELAUNCH;
    epoch += 2u;
    const int zero = 0;
    if (hipMemcpy(ep, &epoch, sizeof epoch, hipMemcpyHostToDevice) != hipSuccess ||
        hipMemcpy(flag, &zero, sizeof zero, hipMemcpyHostToDevice) != hipSuccess)
        return MOE_ELAUNCH;
    return MOE_ETIMEOUT;
}

int launch_layer_step(const moe_layer_desc &ld, const moe_layer_weights &w, int M, const uint16_t *x, uint16_t *y,
                      int32_t *topk_idx, float *topk_w, char *ws, void *stream) {
    (void)hipGetLastError();
    const moe_step_desc d = layer_step_desc(ld, M);
    const StepWs W = step_ws(d, false);
    StepArgs a{};
    a.layer_mode = 1;
    a.router_fp8 = ld.router_type & MOE_ROUTER_FP8 ? 1 : 0;
    a.rt = ld.router_type & MOE_ROUTER_EXPERT_MAJOR ? static_cast<const uint16_t *>(w.router_w) : nullptr;
    a.lw = w;
    a.x = x;
    a.y = y;
    a.y_ls = (size_t)M * ld.hidden;
    a.topk_idx = topk_idx;
    a.topk_w = topk_w;
    a.ws = ws;
    a.o_ctr = W.ctr;
    a.o_flags = W.flags;
    a.o_logits = W.logits;
    a.o_hres = W.hres;
    a.o_hact = W.hact;
    a.o_ypart = W.ypart;
    a.o_lmbest = W.lmbest;
    a.f_lm = W.f_lm;
    a.f_epoch = W.f_epoch;
    a.M = M;
    a.Mx = W.Mx;
    a.H = ld.hidden;
    a.E = ld.num_experts;
    a.K = ld.top_k;
    a.D = ld.expert_width;
    a.Ds = ld.shared_width;
    a.L = 1;
    a.V = 0;
    a.Sx = W.Sx;
    a.NR = W.NR;
    a.ND = W.ND;
    a.NSUBx = W.NSUBx;
    a.Fmax = W.F;
    a.nseg_r = W.nseg_r;
    a.nseg_s = W.nseg_s;
    a.NLU = 0;
    a.spin_limit = kDefaultSpin;
    // the router workgroups stage the whole [H][E] block of their experts in LDS at once
    const size_t tile = (size_t)(ld.hidden / 256) * 288 * (a.router_fp8 ? 8 : 16);
    const size_t lds = std::max(step_lds_bytes(d, M, &a.l_scr, &a.l_slot), tile);
    return ld.wtype == MOE_W_BF16 ? launch_m<true>(M, a, lds, W.NR, false, stream)
                                  : launch_m<false>(M, a, lds, W.NR, false, stream);
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
    a.rt = reinterpret_cast<const uint16_t *>(ws + W.rt);
    a.gains = gains;
    a.x = x;
    a.noise = noise;
    a.lm_w = lm_w;
    a.lm_s = lm_s;
    a.lm_bf = (d.flags & MOE_STEP_LM_BF16) ? 1 : 0;
    a.router_fp8 = d.layer.router_type & MOE_ROUTER_FP8 ? 1 : 0;
    a.draft = draft;
    a.token = token;
    a.max_logit = max_logit;
    a.accepted = accepted_len;
    a.out_tokens = out_tokens;
    a.y = y_layers;
    a.y_ls = (size_t)M * ld.hidden;
    a.topk_idx = topk_idx;
    a.topk_w = topk_w;
    a.x_final = x_final;
    a.ws = ws;
    a.o_ctr = W.ctr;
    a.o_flags = W.flags;
    a.o_logits = W.logits;
    a.o_hres = W.hres;
    a.o_hact = W.hact;
    a.o_ypart = W.ypart;
    a.o_lmbest = W.lmbest;
    a.f_lm = W.f_lm;
    a.f_epoch = W.f_epoch;
    a.M = M;
    a.Mx = W.Mx;
    a.H = ld.hidden;
    a.E = ld.num_experts;
    a.K = ld.top_k;
    a.D = ld.expert_width;
    a.Ds = ld.shared_width;
    a.L = d.num_layers;
    a.V = d.vocab;
    a.Sx = W.Sx;
    a.NR = W.NR;
    a.ND = W.ND;
    a.NSUBx = W.NSUBx;
    a.Fmax = W.F;
    a.nseg_r = W.nseg_r;
    a.nseg_s = W.nseg_s;
    a.NLU = d.vocab / 64;
    a.eps = d.eps;
    a.spin_limit = d.spin_limit ? d.spin_limit : kDefaultSpin;

    const size_t lds = step_lds_bytes(d, M, &a.l_scr, &a.l_slot);
    const bool coop = (d.flags & MOE_STEP_COOPERATIVE) != 0;
    return ld.wtype == MOE_W_BF16 ? launch_m<true>(M, a, lds, W.NR, coop, stream)
                                  : launch_m<false>(M, a, lds, W.NR, coop, stream);
}

}  // namespace moe
