// draft_fused.hip -- the MTP drafter's gamma drafts as one persistent gfx950 launch.
//
// Page "LLM decoding", "The one-line shape bug that disabled the model's own drafter" and
// "Lever 2: fewer passes (native MTP)": per draft the head projects [embedding(t) | g]
// down to its width, runs its body, normalises, takes the argmax over its own table and
// projects back up for the next draft's hidden state (the formulas are those of
// moe_draft_step). Run as a chain of launches, a draft is 27 small kernels that each move
// 3-8 MB in about 5 us: launch gaps, not bytes. Here kDraftPG workgroups (two per compute
// unit) stay resident for all gamma drafts, every matrix's rows spread over them with R
// rows per workgroup and 256 / R lanes per row:
//
//   pre     workgroups 0..D/Rp-1 hold their pre-projection rows in registers for the whole
//           call. Each reduces the previous draft's per-workgroup argmax keys to the token
//           itself (workgroup 0 also stores it), forms [e | g] in LDS and writes its rows
//           of z.
//   blocks  per block, every gate/up workgroup polls z, forms u = rmsnorm(z) in LDS and
//           writes its rows of h = gelu_tanh(gate u) * (up u); then the down workgroups
//           (fewer, with longer rows, so fewer read all of h) poll h and write z + down h.
//           A workgroup requests its next gate/up and down rows as soon as it has used the
//           current ones, so the weight stream runs under the waits.
//   final   every workgroup polls the last z and forms zf = rmsnorm(z) in LDS; the post
//           workgroups write g = post zf for the next draft; then every workgroup streams
//           an equal share of the table (its first three steps requested before the wait)
//           and writes its best (ordered logit, inverted row) key.
//
// Hand-off words are 64-bit: the value in the low half, the call's tag (epoch + 1) in the
// high half, written and read with relaxed agent-scope atomics (coherent across the XCDs'
// L2s). z, h, g and the keys have a slot per draft and stage, so each word is written once
// per call and a consumer polls until its tag is current. Every wait is on an earlier
// phase and every poll is bounded (a spin limit, then the error flag), so with every
// workgroup resident the call cannot deadlock, and it always ends. Workgroup 0 advances
// the epoch at the end, after reading every workgroup's last key (each written after that
// workgroup read the epoch).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "handoff.h"
#include "internal.h"

namespace moe {
namespace {

using namespace dev;

constexpr unsigned kDraftSpin = 1u << 18;   // default polls before a wait gives up
constexpr int kTabRows = 4;                 // table rows per lane (one 256-column chunk each)
// A gate/up-only workgroup requests its next block's rows this long (in 100 MHz ticks of
// the constant clock) after writing its h: by then the down workgroups' wait for h is
// over, so the 8 MB burst of gate/up rows does not queue ahead of those polls, and the
// rows still arrive before the next z does.
constexpr unsigned long long kPrefetchDelay = 260;

struct DfArgs {
    moe_draft_weights w;
    const int32_t *tok0;
    const uint16_t *hidden0;
    const uint8_t *emb_w;
    const float *emb_s;
    int32_t *drafts;
    char *ws;
    size_t o_ctr, o_epoch, o_z, o_h, o_g, o_k;
    int H, D, F, B, V, gamma;
    int lp, lgu, ld, lpo;   // lanes per row of the pre-projection, gate/up, down, post-projection
    float eps;
    unsigned spin_limit;
};

// The phase functions read the kernel arguments on demand through a pointer into the
// kernel-argument segment, made opaque to the optimiser at each phase so that argument
// fields are re-read (scalar loads) rather than held in registers across phases.
typedef const __attribute__((address_space(4))) DfArgs *DA;
__device__ __forceinline__ DA opaque(DA p) {
    asm volatile("" : "+s"(p));
    return p;
}

// LDS of a workgroup: the pre-projection's input [e | g] (bf16 pairs) or the blocks' inner
// vector h (fp32), z as read, u or zf (bf16 pairs), and a few reduction slots.
struct DfLds {
    uint32_t xh[8192];
    uint32_t z[512];
    uint32_t u[512];
    uint16_t stage[16];
    float red[4];
    unsigned long long keys[4];
};

// ------------------------------------------------------------ hand-off words

__device__ __forceinline__ uint64_t *zwords(DA a, int i, int s) {   // z of draft i, stage s
    return reinterpret_cast<uint64_t *>(a->ws + a->o_z) + ((size_t)i * (a->B + 1) + s) * (size_t)(a->D / 2);
}
__device__ __forceinline__ uint64_t *hwords(DA a, int i, int b) {   // h of draft i, block b
    return reinterpret_cast<uint64_t *>(a->ws + a->o_h) + ((size_t)i * a->B + b) * (size_t)a->F;
}
__device__ __forceinline__ uint64_t *gwords(DA a, int i) {   // g after draft i
    return reinterpret_cast<uint64_t *>(a->ws + a->o_g) + (size_t)i * (size_t)(a->H / 2);
}
__device__ __forceinline__ uint64_t *kwords(DA a, int i) {   // keys of draft i, two per workgroup
    return reinterpret_cast<uint64_t *>(a->ws + a->o_k) + (size_t)i * kDraftPG * 2;
}
__device__ __forceinline__ uint32_t *errflag(DA a) { return reinterpret_cast<uint32_t *>(a->ws + a->o_ctr); }
__device__ __forceinline__ uint32_t *epoch(DA a) { return reinterpret_cast<uint32_t *>(a->ws + a->o_epoch); }

// A wave's polling loop: done() is true once every lane's words are current, or once the
// spin limit is reached (which raises the error flag), or within 256 polls of any other
// wait having given up; otherwise it sleeps 64 cycles and the loop reloads.
// Sleep until `ticks` of the constant 100 MHz clock have passed since t0.
__device__ __forceinline__ void sleep_until(unsigned long long t0, unsigned long long ticks) {
    while (wall_clock64() - t0 < ticks) __builtin_amdgcn_s_sleep(2);
}

struct Spin {
    unsigned spins = 0;
    __device__ __forceinline__ bool done(DA a, bool ok) {
        if (__all(ok)) return true;
        if (++spins >= a->spin_limit) {
            if ((threadIdx.x & 63) == 0) st32(errflag(a), 1u);
            return true;
        }
        if ((spins & 255u) == 0u && __builtin_amdgcn_readfirstlane(ld32(errflag(a))) != 0u) return true;
        __builtin_amdgcn_s_sleep(1);
        return false;
    }
};

// Poll n tagged words until current and store their values to dst (LDS); NB words per
// thread per round (one memory latency a round). Ends with a barrier.
template <int NB>
__device__ __forceinline__ void poll_to_lds(DA a, const uint64_t *src, int n, uint32_t tag,
                                            uint32_t *dst) {
    const int tid = threadIdx.x;
    for (int i0 = 0; i0 < n; i0 += 256 * NB) {
        uint64_t v[NB];
        Spin sp;
        bool ok;
        do {
#pragma unroll
            for (int k = 0; k < NB; ++k) {
                const int i = i0 + tid + 256 * k;
                v[k] = i < n ? ld64(src + i) : tagged(0u, tag);
            }
            ok = true;
#pragma unroll
            for (int k = 0; k < NB; ++k) ok = ok && current(v[k], tag);
        } while (!sp.done(a, ok));
#pragma unroll
        for (int k = 0; k < NB; ++k) {
            const int i = i0 + tid + 256 * k;
            if (i < n) dst[i] = (uint32_t)v[k];
        }
    }
    __syncthreads();
}

// The R results of a workgroup's rows (lane li == 0 of each row's group holds its value)
// as R / 2 tagged bf16 pair words from dst.
__device__ __forceinline__ void publish_pairs(DfLds &s, uint16_t v, bool leader, int rloc, int R, uint64_t *dst,
                                              uint32_t tag) {
    if (leader) s.stage[rloc] = v;
    __syncthreads();
    const int t = threadIdx.x;
    if (t < R / 2) st64(dst + t, tagged(pack2(s.stage[2 * t], s.stage[2 * t + 1]), tag));
}

// ------------------------------------------------------------ register-held rows

// A lane's pieces of one row of an FP8 matrix with K codes per row: 16-byte pieces li,
// li + L, ... (clamped to the row's last piece; the dot products skip the clamped ones).
template <int MAXC>
struct Row {
    uint4 q[MAXC];
    __device__ __forceinline__ void load(const uint8_t *m, int row, int K, int L, int li) {
        const int nc = K >> 4;
        const uint8_t *p = m + (size_t)row * K;
#pragma unroll
        for (int k = 0; k < MAXC; ++k) q[k] = ld16nt(p + (size_t)min(k * L + li, nc - 1) * 16);
    }
    // sum of dec(q) x over the lane's pieces, x bf16 in LDS (two uint4 per piece)
    __device__ __forceinline__ float dot_bf16(const uint4 *xs, int K, int L, int li) const {
        const int nc = K >> 4;
        float acc = 0.0f;
#pragma unroll
        for (int k = 0; k < MAXC; ++k) {
            const int c = k * L + li;
            if (c < nc) {
                bf16x2 wv[8];
                decode16_bf16(q[k], wv);
                acc = dot16(wv, xs[2 * c], xs[2 * c + 1], acc);
            }
        }
        return acc;
    }
    // the same with an fp32 vector in LDS (four float4 per piece)
    __device__ __forceinline__ float dot_f32(const float4 *hs, int K, int L, int li) const {
        const int nc = K >> 4;
        float acc = 0.0f;
#pragma unroll
        for (int k = 0; k < MAXC; ++k) {
            const int c = k * L + li;
            if (c < nc) {
                const uint32_t qw[4] = {q[k].x, q[k].y, q[k].z, q[k].w};
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const f32x2 lo = fp8x2_to_f32<false>(qw[u]), hi = fp8x2_to_f32<true>(qw[u]);
                    const float4 hv = hs[4 * c + u];
                    acc = fmaf(lo.x, hv.x, acc);
                    acc = fmaf(lo.y, hv.y, acc);
                    acc = fmaf(hi.x, hv.z, acc);
                    acc = fmaf(hi.y, hv.w, acc);
                }
            }
        }
        return acc;
    }
};

// Sum over a row's L lanes (16..256, aligned groups), valid in every lane of the group.
// Groups of 128 and 256 lanes span waves and combine through LDS in a fixed order (with
// barriers: L is the same for the whole workgroup).
__device__ __forceinline__ float rows_sum(float v, int L, DfLds &s) {
    v = row16_sum(v);
    if (L >= 32) v += __shfl_xor(v, 16);
    if (L >= 64) v += __shfl_xor(v, 32);
    if (L <= 64) return v;
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) s.red[wave] = v;
    __syncthreads();
    const float r = L == 128 ? s.red[wave & ~1] + s.red[wave | 1] : (s.red[0] + s.red[1]) + (s.red[2] + s.red[3]);
    __syncthreads();
    return r;
}

// u = bf16(z r gain), r = 1 / sqrt(mean(z^2) + eps), over D values held as bf16 pairs in
// LDS (pair p by thread p mod 256; gv holds the gain pairs of those, requested before the
// caller's wait). The sum of squares goes per thread, over the wave and the four waves in
// a fixed order, so every workgroup forms the same u.
__device__ __forceinline__ void norm_pairs(DfLds &s, const uint32_t *zp, const uint32_t (&gv)[2], int D, float eps,
                                           uint32_t *up) {
    const int tid = threadIdx.x, np = D / 2;
    float ss = 0.0f;
    uint32_t zv[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int p = tid + 256 * k;
        zv[k] = p < np ? zp[p] : 0u;
        const float lo = bf2f(zv[k] & 0xffffu), hi = bf2f(zv[k] >> 16);
        ss = fmaf(lo, lo, ss);
        ss = fmaf(hi, hi, ss);
    }
    ss = wave_sum(ss);
    if ((tid & 63) == 0) s.red[tid >> 6] = ss;
    __syncthreads();
    const float r = rsqrtf(((s.red[0] + s.red[1]) + (s.red[2] + s.red[3])) / (float)D + eps);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int p = tid + 256 * k;
        if (p < np)
            up[p] = pack2(f2bf(bf2f(zv[k] & 0xffffu) * r * bf2f(gv[k] & 0xffffu)),
                          f2bf(bf2f(zv[k] >> 16) * r * bf2f(gv[k] >> 16)));
    }
    __syncthreads();
}

// gain pairs of norm b for the pairs tid, tid + 256
__device__ __forceinline__ void load_gains(DA a, int b, uint32_t (&gv)[2]) {
    const uint32_t *g = reinterpret_cast<const uint32_t *>(a->w.gains) + (size_t)b * (a->D / 2);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int p = threadIdx.x + 256 * k;
        gv[k] = p < a->D / 2 ? *glb(g + p) : 0u;
    }
}

// bf16 (round to nearest even) of a double that is the product of an fp32 and an FP8
// value (at most 28 significant bits, normal range): the mantissa is rounded at bit 45 in
// the integer bits, after which the value is exact in fp32.
__device__ __forceinline__ uint16_t d2bf(double d) {
    unsigned long long b = (unsigned long long)__double_as_longlong(d);
    b += ((b >> 45) & 1ull) + (1ull << 44) - 1ull;
    b &= ~((1ull << 45) - 1ull);
    return (uint16_t)(__float_as_uint((float)__longlong_as_double((long long)b)) >> 16);
}

// ------------------------------------------------------------ phases

// The token of draft i: the largest of the kDraftPG workgroups' keys (two words each),
// read by the whole workgroup; ties of the logit went to the lower row in each key.
__device__ __forceinline__ int draft_token(DA a, DfLds &s, int i, uint32_t tag) {
    a = opaque(a);
    const int tid = threadIdx.x, lane = tid & 63;
    const uint64_t *kw = kwords(a, i);
    uint64_t v[4];
    Spin sp;
    bool ok;
    do {
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            v[2 * k] = ld64(kw + 2 * (tid + 256 * k));
            v[2 * k + 1] = ld64(kw + 2 * (tid + 256 * k) + 1);
        }
        ok = current(v[0], tag) && current(v[1], tag) && current(v[2], tag) && current(v[3], tag);
    } while (!sp.done(a, ok));
    const uint64_t k0 = ((uint64_t)(uint32_t)v[0] << 32) | (uint32_t)v[1];
    const uint64_t k1 = ((uint64_t)(uint32_t)v[2] << 32) | (uint32_t)v[3];
    const uint64_t best = wave_max_key(k0 > k1 ? k0 : k1);
    if (lane == 0) s.keys[tid >> 6] = best;
    __syncthreads();
    unsigned long long b = s.keys[0];
#pragma unroll
    for (int q = 1; q < 4; ++q) b = s.keys[q] > b ? s.keys[q] : b;
    __syncthreads();
    return (int)(0xffffffffu - (uint32_t)b);
}

// z = bf16(pre_s (pre_w [e | g])) for this workgroup's rows, e = bf16(emb_s[t] dec(emb_w[t])).
__device__ __forceinline__ void pre_phase(DA a, DfLds &s, const Row<kDpPreC> &P, int i, int w,
                                          uint32_t tag) {
    a = opaque(a);
    const int tid = threadIdx.x, H = a->H, L = a->lp, R = 256 / L, li = tid & (L - 1), row = w * R + tid / L;
    const float sc = *glb(a->w.pre_s + row);
    int t;
    if (i == 0) {
        t = __builtin_amdgcn_readfirstlane(*glb(a->tok0));
    } else {
        t = draft_token(a, s, i - 1, tag);
        if (w == 0 && tid == 0) *glb(a->drafts + i - 1) = t;
    }
    t = t < 0 ? 0 : (t >= a->V ? a->V - 1 : t);
    // the embedding row: thread c < H / 16 holds codes 16 c .. 16 c + 15
    const bool emb = tid < H / 16;
    uint4 q = make_uint4(0u, 0u, 0u, 0u);
    if (emb) q = ld16(a->emb_w + (size_t)t * H + 16 * tid);
    const double st = (double)*glb(a->emb_s + t);
    uint4 *xs = reinterpret_cast<uint4 *>(s.xh);
    if (i == 0) {
        for (int j = tid; j < H / 8; j += 256) xs[H / 8 + j] = ld16(a->hidden0 + 8 * j);
    } else {
        poll_to_lds<8>(a, gwords(a, i - 1), H / 2, tag, s.xh + H / 2);
    }
    if (emb) {
        const uint32_t qw[4] = {q.x, q.y, q.z, q.w};
        uint32_t e[8];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const f32x2 lo = fp8x2_to_f32<false>(qw[u]), hi = fp8x2_to_f32<true>(qw[u]);
            e[2 * u] = pack2(d2bf(st * (double)lo.x), d2bf(st * (double)lo.y));
            e[2 * u + 1] = pack2(d2bf(st * (double)hi.x), d2bf(st * (double)hi.y));
        }
        xs[2 * tid] = make_uint4(e[0], e[1], e[2], e[3]);
        xs[2 * tid + 1] = make_uint4(e[4], e[5], e[6], e[7]);
    }
    __syncthreads();
    const float acc = rows_sum(P.dot_bf16(xs, 2 * H, L, li), L, s);
    publish_pairs(s, f2bf(sc * acc), li == 0, tid / L, R, zwords(a, i, 0) + w * R / 2, tag);
}

// Block b: u = rmsnorm(z), h = gelu_tanh(sg (G u)) * (su (U u)) for this workgroup's rows.
__device__ __forceinline__ void gu_phase(DA a, DfLds &s, const Row<kDpGuC> &G, const Row<kDpGuC> &U,
                                         int i, int b, int w, uint32_t tag) {
    a = opaque(a);
    const int tid = threadIdx.x, D = a->D, L = a->lgu, li = tid & (L - 1), row = w * (256 / L) + tid / L;
    const float sg = *glb(a->w.gate_s + (size_t)b * a->F + row), su = *glb(a->w.up_s + (size_t)b * a->F + row);
    uint32_t gv[2];
    load_gains(a, b, gv);
    poll_to_lds<2>(a, zwords(a, i, b), D / 2, tag, s.z);
    norm_pairs(s, s.z, gv, D, a->eps, s.u);
    const uint4 *us = reinterpret_cast<const uint4 *>(s.u);
    const float ag = rows_sum(G.dot_bf16(us, D, L, li), L, s);
    const float au = rows_sum(U.dot_bf16(us, D, L, li), L, s);
    if (li == 0) st64(hwords(a, i, b) + row, tagged(__float_as_uint(gelu_tanh(sg * ag) * (su * au)), tag));
}

// Block b: z = bf16(z + sd (Dn h)) for this workgroup's rows.
__device__ __forceinline__ void dn_phase(DA a, DfLds &s, const Row<kDpDnC> &Dn, int i, int b, int w,
                                         uint32_t tag) {
    a = opaque(a);
    const int tid = threadIdx.x, L = a->ld, R = 256 / L, li = tid & (L - 1), c = w * R + tid / L;
    const float sd = *glb(a->w.down_s + (size_t)b * a->D + c);
    // the row's residual, from the stage's z words: requested with the scale, before the
    // wait for h (it is current by then, as h depends on it), checked after it
    const uint64_t *zp = zwords(a, i, b) + c / 2;
    uint64_t zw = ld64(zp);
    poll_to_lds<16>(a, hwords(a, i, b), a->F, tag, s.xh);
    Spin sp;
    while (!sp.done(a, current(zw, tag))) zw = ld64(zp);
    const float zc = bf2f((c & 1) ? ((uint32_t)zw >> 16) : ((uint32_t)zw & 0xffffu));
    const float acc = rows_sum(Dn.dot_f32(reinterpret_cast<const float4 *>(s.xh), a->F, L, li), L, s);
    publish_pairs(s, f2bf(zc + sd * acc), li == 0, tid / L, R, zwords(a, i, b + 1) + w * R / 2, tag);
}

struct TabBuf {
    uint4 q[kTabRows];
};

// Step st of this workgroup's table stream: 64-row unit u0 + st / NC, 256-column chunk
// st % NC. Wave v reads rows 16 v .. 16 v + 15 of the unit, four per 16-lane group.
__device__ __forceinline__ void tab_load(DA a, int u0, int nst, int st, TabBuf &b) {
    if (st < nst) {
        const int t = threadIdx.x, NC = a->D >> 8, lane = t & 63, wave = t >> 6;
        const int unit = u0 + st / NC, k = st - (st / NC) * NC;
        const size_t row = (size_t)unit * 64 + wave * 16 + (lane >> 4) * kTabRows;
        const uint8_t *p = a->w.table_w + row * a->D + k * 256 + (lane & 15) * 16;
#pragma unroll
        for (int r = 0; r < kTabRows; ++r) b.q[r] = ld16nt(p + (size_t)r * a->D);
    }
}

struct TabAcc {
    float acc[kTabRows];
    float sc[kTabRows];
    unsigned long long best;
};

__device__ __forceinline__ void tab_step(DA a, const DfLds &s, int u0, int nst, int st, const TabBuf &b,
                                         TabAcc &A) {
    if (st >= nst) return;
    const int t = threadIdx.x, NC = a->D >> 8, lane = t & 63, wave = t >> 6, li = lane & 15;
    const int k = st - (st / NC) * NC;
    const uint4 *xs = reinterpret_cast<const uint4 *>(s.u) + k * 32 + li * 2;
    const uint4 x0 = xs[0], x1 = xs[1];
#pragma unroll
    for (int r = 0; r < kTabRows; ++r) {
        bf16x2 wv[8];
        decode16_bf16(b.q[r], wv);
        A.acc[r] = dot16(wv, x0, x1, A.acc[r]);
    }
    if (k == NC - 1) {
        const int row = (u0 + st / NC) * 64 + wave * 16 + (lane >> 4) * kTabRows;
#pragma unroll
        for (int r = 0; r < kTabRows; ++r) {
            const float lg = A.sc[r] * row16_sum(A.acc[r]);
            const unsigned long long key =
                ((unsigned long long)ordered(lg) << 32) | (unsigned long long)(0xffffffffu - (uint32_t)(row + r));
            A.best = key > A.best ? key : A.best;
            A.acc[r] = 0.0f;
        }
        if (st + 1 < nst) {   // the next unit's scales
#pragma unroll
            for (int r = 0; r < kTabRows; ++r) A.sc[r] = *glb(a->w.table_s + row + 64 + r);
        }
    }
}

// zf = rmsnorm(z_B); g = bf16(post_s (post_w zf)) for the next draft; this workgroup's
// share of the table argmax -> its key words.
__device__ __forceinline__ void final_phase(DA a, DfLds &s, const Row<kDpPoC> &PO, int i, int w,
                                            uint32_t tag) {
    a = opaque(a);
    const int tid = threadIdx.x, D = a->D, lane = tid & 63, wave = tid >> 6;
    const int NU = a->V / 64;
    const int u0 = (int)((long long)w * NU / kDraftPG), u1 = (int)((long long)(w + 1) * NU / kDraftPG);
    const int nst = (u1 - u0) * (D >> 8);
    TabBuf b0, b1, b2;
    tab_load(a, u0, nst, 0, b0);
    tab_load(a, u0, nst, 1, b1);
    tab_load(a, u0, nst, 2, b2);
    TabAcc A;
    A.best = 0ull;
#pragma unroll
    for (int r = 0; r < kTabRows; ++r) {
        A.acc[r] = 0.0f;
        A.sc[r] = 0.0f;
    }
    if (nst > 0) {
        const int row = u0 * 64 + wave * 16 + (lane >> 4) * kTabRows;
#pragma unroll
        for (int r = 0; r < kTabRows; ++r) A.sc[r] = *glb(a->w.table_s + row + r);
    }
    uint32_t gv[2];
    load_gains(a, a->B, gv);
    poll_to_lds<2>(a, zwords(a, i, a->B), D / 2, tag, s.z);
    norm_pairs(s, s.z, gv, D, a->eps, s.u);
    const int Lp = a->lpo, Rp = 256 / Lp;
    if (i + 1 < a->gamma && w < a->H / Rp) {
        const int li = tid & (Lp - 1), row = w * Rp + tid / Lp;
        const float sc = *glb(a->w.post_s + row);
        const float acc = rows_sum(PO.dot_bf16(reinterpret_cast<const uint4 *>(s.u), D, Lp, li), Lp, s);
        publish_pairs(s, f2bf(sc * acc), li == 0, tid / Lp, Rp, gwords(a, i) + w * Rp / 2, tag);
    }
    for (int st = 0; st < nst; st += 3) {
        tab_step(a, s, u0, nst, st, b0, A);
        tab_load(a, u0, nst, st + 3, b0);
        tab_step(a, s, u0, nst, st + 1, b1, A);
        tab_load(a, u0, nst, st + 4, b1);
        tab_step(a, s, u0, nst, st + 2, b2, A);
        tab_load(a, u0, nst, st + 5, b2);
    }
    const unsigned long long best = wave_max_key(A.best);
    if (lane == 0) s.keys[wave] = best;
    __syncthreads();
    if (tid == 0) {
        unsigned long long k = s.keys[0];
#pragma unroll
        for (int q = 1; q < 4; ++q) k = s.keys[q] > k ? s.keys[q] : k;
        st64(kwords(a, i) + 2 * w, tagged((uint32_t)(k >> 32), tag));
        st64(kwords(a, i) + 2 * w + 1, tagged((uint32_t)k, tag));
    }
    __syncthreads();
}

__global__ __launch_bounds__(256, 2) void k_draft_fused(DfArgs args) {
    (void)args;
    __shared__ DfLds s;
    const DA a = opaque((DA)__builtin_amdgcn_kernarg_segment_ptr());
    const int w = blockIdx.x, tid = threadIdx.x;
    const uint32_t tag = __builtin_amdgcn_readfirstlane(ld32(epoch(a))) + 1u;
    const int Lp = a->lp, Lg = a->lgu, Ld = a->ld, Lo = a->lpo;
    const int NP = a->D / (256 / Lp), NG = a->B > 0 ? a->F / (256 / Lg) : 0, ND = a->B > 0 ? a->D / (256 / Ld) : 0;
    const int NO = a->gamma > 1 ? a->H / (256 / Lo) : 0;
    const int rg = w * (256 / Lg) + tid / Lg, rd = w * (256 / Ld) + tid / Ld;
    // rows that stay the same for every draft and block: requested once
    Row<kDpPreC> P;
    Row<kDpPoC> PO;
    Row<kDpGuC> G, U;
    Row<kDpDnC> Dn;
    if (w < NP) P.load(a->w.pre_w, w * (256 / Lp) + tid / Lp, 2 * a->H, Lp, tid & (Lp - 1));
    if (w < NO) PO.load(a->w.post_w, w * (256 / Lo) + tid / Lo, a->D, Lo, tid & (Lo - 1));
    if (w < NG) {
        G.load(a->w.gate_w, rg, a->D, Lg, tid & (Lg - 1));
        U.load(a->w.up_w, rg, a->D, Lg, tid & (Lg - 1));
    }
    if (w < ND) Dn.load(a->w.down_w, rd, a->F, Ld, tid & (Ld - 1));
    for (int i = 0; i < a->gamma; ++i) {
        if (w < NP) pre_phase(a, s, P, i, w, tag);
        for (int b = 0; b < a->B; ++b) {
            // the rows used next: the following block's, or block 0's for the next draft
            const int nb = b + 1 < a->B ? b + 1 : 0;
            const bool more = b + 1 < a->B || i + 1 < a->gamma;
            // The next rows are requested where their burst does not queue ahead of a
            // critical poll (loads return in order, so a poll also waits for every load
            // issued before it): a gate/up-only workgroup waits kPrefetchDelay after its h;
            // a down workgroup requests its next gate/up rows before its wait for h and
            // this block's down rows after its gate/up (they arrive during that wait).
            if (w < NG) {
                gu_phase(a, s, G, U, i, b, w, tag);
                if (more) {
                    if (w >= ND) sleep_until(wall_clock64(), kPrefetchDelay);
                    G.load(a->w.gate_w, nb * a->F + rg, a->D, Lg, tid & (Lg - 1));
                    U.load(a->w.up_w, nb * a->F + rg, a->D, Lg, tid & (Lg - 1));
                }
            }
            if (w < ND && b > 0) Dn.load(a->w.down_w, b * a->D + rd, a->F, Ld, tid & (Ld - 1));
            if (w < ND) {
                dn_phase(a, s, Dn, i, b, w, tag);
                // block 0's down rows for the next draft
                if (more && nb == 0) Dn.load(a->w.down_w, rd, a->F, Ld, tid & (Ld - 1));
            }
        }
        final_phase(a, s, PO, i, w, tag);
    }
    if (w == 0) {
        const int t = draft_token(a, s, a->gamma - 1, tag);
        if (tid == 0) {
            *glb(a->drafts + a->gamma - 1) = t;
            st32(epoch(a), tag);   // every workgroup has read the epoch by now
        }
    }
}

inline hipStream_t S(void *p) { return reinterpret_cast<hipStream_t>(p); }

}  // namespace

int launch_draft_fused(const moe_draft_desc &d, const moe_draft_weights &w, int gamma, const int32_t *tok0,
                       const uint16_t *hidden0, const uint8_t *emb_w, const float *emb_s, int32_t *drafts,
                       char *ws, void *stream) {
    const DraftGeo g = draft_geo(d);
    if (!g.ok || (d.flags & MOE_DRAFT_CHAIN)) return MOE_EUNSUPPORTED;
    (void)hipGetLastError();
    // every workgroup must be resident at once (phases wait on other workgroups)
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_draft_fused, 256, 0) != hipSuccess)
        return MOE_ELAUNCH;
    if ((long long)cus * per_cu < kDraftPG) return MOE_EUNSUPPORTED;
    const DraftWs W = draft_ws(d);
    DfArgs a{};
    a.w = w;
    a.tok0 = tok0;
    a.hidden0 = hidden0;
    a.emb_w = emb_w;
    a.emb_s = emb_s;
    a.drafts = drafts;
    a.ws = ws;
    a.o_ctr = W.ctr;
    a.o_epoch = W.epoch;
    a.o_z = W.zw;
    a.o_h = W.hw;
    a.o_g = W.gw;
    a.o_k = W.kw;
    a.H = d.hidden;
    a.D = d.width;
    a.F = d.ffn;
    a.B = d.blocks;
    a.V = d.vocab;
    a.gamma = gamma;
    a.lp = g.lp;
    a.lgu = g.lgu;
    a.ld = g.ld;
    a.lpo = g.lpo;
    a.eps = d.eps;
    a.spin_limit = d.spin_limit ? d.spin_limit : kDraftSpin;
    hipLaunchKernelGGL(k_draft_fused, dim3(kDraftPG), dim3(256), 0, S(stream), a);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ELAUNCH;
}

// After a wait has given up, a workgroup that started after workgroup 0 advanced the epoch
// may have written hand-off words with the next call's tag; the epoch therefore moves on
// by two more, and the flag is cleared. No call may be in flight on the workspace.
int draft_status(const moe_draft_desc &d, char *ws) {
    if (!draft_geo(d).ok) return MOE_OK;
    const DraftWs W = draft_ws(d);
    uint32_t err = 0, ep = 0;
    if (hipMemcpy(&err, ws + W.ctr, sizeof err, hipMemcpyDeviceToHost) != hipSuccess) return MOE_ELAUNCH;
    if (!err) return MOE_OK;
    if (hipMemcpy(&ep, ws + W.epoch, sizeof ep, hipMemcpyDeviceToHost) != hipSuccess) return MOE_ELAUNCH;
    ep += 2u;
    const uint32_t zero = 0;
    if (hipMemcpy(ws + W.epoch, &ep, sizeof ep, hipMemcpyHostToDevice) != hipSuccess ||
        hipMemcpy(ws + W.ctr, &zero, sizeof zero, hipMemcpyHostToDevice) != hipSuccess)
        return MOE_ELAUNCH;
    return MOE_ETIMEOUT;
}

}  // namespace moe
