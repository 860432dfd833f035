// internal.h -- workspace layout and kernel launchers shared by api.cpp (host
// validation, no HIP headers) and kernels.hip (device code).
#pragma once
#include <stddef.h>
#include <algorithm>
#include <stdint.h>

#include "moe_decode.h"

namespace moe {

constexpr int kMaxM = 8;          // verify batch: gamma <= 7 drafts + 1
constexpr int kMaxTopK = 16;
constexpr int kMaxExperts = 256;
constexpr int kMaxSlots = kMaxM * kMaxTopK + 1;   // routed union bound plus the shared expert
constexpr int kMaxHidden = 4096;
constexpr int kMaxWidth = 4096;
constexpr int kRouterRows = 64;   // router rows per workgroup
constexpr int kLmRowsPerWG = 64;  // lm_head rows per workgroup iteration
constexpr int kLmMaxWG = 2048;    // lm_head grid cap

inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

inline int max_slots(int M, int K, int E, int Ds) {
    int r = M * K < E ? M * K : E;
    return r + (Ds > 0 ? 1 : 0);
}

// Workspace of one moe_decode_layer call, carved from one caller buffer.
struct LayerWs {
    size_t partial;      // fp32 [NB][M][E]      router partial logits per row block
    size_t n_slots;      // int32                number of expert slots (routed union + shared)
    size_t slot_expert;  // int32 [S]            expert id per slot (E = the shared expert)
    size_t slot_mask;    // uint32 [S]           bit m set: token m uses the slot
    size_t slot_w;       // fp32 [S][M]          combine weight of token m in slot s
    size_t h;            // fp32 [S][M][F]       gelu(gate) * up, per slot and token position
    size_t ypart;        // fp32 [S][M][H]       weighted down output per slot and token
    size_t total;
    int nb, S, F;
};

inline LayerWs layer_ws(const moe_layer_desc &d, int M) {
    LayerWs L{};
    const int H = d.hidden, E = d.num_experts;
    L.nb = (H + kRouterRows - 1) / kRouterRows;
    L.S = max_slots(M, d.top_k, E, d.shared_width);
    L.F = d.expert_width > d.shared_width ? d.expert_width : d.shared_width;
    size_t o = 0;
    L.partial = o;     o = align256(o + sizeof(float) * (size_t)L.nb * M * E);
    L.n_slots = o;     o = align256(o + sizeof(int32_t));
    L.slot_expert = o; o = align256(o + sizeof(int32_t) * (size_t)L.S);
    L.slot_mask = o;   o = align256(o + sizeof(uint32_t) * (size_t)L.S);
    L.slot_w = o;      o = align256(o + sizeof(float) * (size_t)L.S * M);
    L.h = o;           o = align256(o + sizeof(float) * (size_t)L.S * M * L.F);
    L.ypart = o;       o = align256(o + sizeof(float) * (size_t)L.S * M * H);
    L.total = o;
    return L;
}

inline int lm_grid(int V) {
    int blocks = V / kLmRowsPerWG;
    return blocks < kLmMaxWG ? blocks : kLmMaxWG;
}

// fp32 [grid][M] best logits, then (256-aligned) int32 [grid][M] their rows.
inline size_t lm_ws_bytes(int M, int V) {
    return align256((size_t)lm_grid(V) * M * sizeof(float)) +
           align256((size_t)lm_grid(V) * M * sizeof(int32_t));
}

// Workspace of lm_head_spec_sample for M tokens over V rows: the lm_head's per-workgroup
// bests (unused by the sampler, kept by the shared kernel), every logit, the per-chunk
// softmax states (maximum of logit / T and the sum of exp(logit / T - maximum) per
// 1024-entry chunk and row), the accepted count and the per-row log normalisers, the
// sampling workgroups' argmax keys.
constexpr int kSampleTok = 1024;   // vocabulary entries per sampling workgroup (4 per thread)
struct SampleWs {
    size_t best_v, best_i, logits, stats, acc, keys, total;
    int nwg, nsg;
};
inline SampleWs sample_ws(int M, int V) {
    SampleWs W{};
    W.nwg = lm_grid(V);
    W.nsg = (V + kSampleTok - 1) / kSampleTok;
    size_t o = 0;
    auto take = [&](size_t bytes) { size_t r = o; o = align256(o + bytes); return r; };
    W.best_v = take(4 * (size_t)W.nwg * M);
    W.best_i = take(4 * (size_t)W.nwg * M);
    W.logits = take(4 * (size_t)M * V);
    W.stats = take(8 * (size_t)W.nsg * M);       // float2 [nsg][M]
    W.acc = take(4 * (size_t)(1 + kMaxM));       // int n, then float logZ[M]
    W.keys = take(8 * 2 * (size_t)W.nsg);        // per sampling workgroup: residual key, target key
    W.total = o;
    return W;
}
constexpr int kSampleMaxVocab = 1 << 24;

// Workspace of moe_draft_step: the concatenated input, the head's vector and its norm,
// the next hidden state, the blocks' inner vector, the argmax's per-workgroup bests.
// Lanes per row (16, 32 or 64) for a drafter matrix of N rows (a multiple of 256) of K FP8
// codes, each lane reading at most maxch 16-byte pieces of a row: the fewest lanes that
// still give 256 workgroups of 256 threads, else the most workgroups; 0 when no split fits.
constexpr int kDraftMaxCh = 16;       // pre_projection, down, post-projection pieces per lane
constexpr int kDraftGateUpMaxCh = 8;  // gate and up pieces per lane (two rows per lane)
inline int draft_lpr(int N, int K, int maxch) {
    int best = 0;
    for (int lpr = 16; lpr <= 64; lpr *= 2) {
        if (K % (16 * lpr) || K / (16 * lpr) > maxch) continue;
        best = lpr;
        if ((long long)N * lpr / 256 >= 256) break;
    }
    return best;
}
inline bool draft_splits(const moe_draft_desc &d) {
    return draft_lpr(d.width, 2 * d.hidden, kDraftMaxCh) && draft_lpr(d.ffn, d.width, kDraftGateUpMaxCh) &&
           draft_lpr(d.width, d.ffn, kDraftMaxCh) && draft_lpr(d.hidden, d.width, kDraftMaxCh);
}

// The persistent drafter: all gamma drafts in one launch of kDraftPG workgroups of 256
// threads (two per compute unit), each matrix's rows spread over the workgroups with
// R rows per workgroup (a power of two) and L = 256 / R lanes per row; a lane holds at
// most the given number of 16-byte pieces of a row in registers.
constexpr int kDraftPG = 512;
constexpr int kDpPreC = 3, kDpGuC = 2, kDpDnC = 8, kDpPoC = 2;
constexpr int kDraftMaxGamma = kMaxM - 1;
struct DraftGeo {
    int lp, lgu, ld, lpo;   // lanes per row: pre-projection, gate/up, down, post-projection
    bool ok;                // the shape fits the persistent kernel
};
inline int pow2_at_least(int v) {
    int p = 1;
    while (p < v) p *= 2;
    return p;
}
inline DraftGeo draft_geo(const moe_draft_desc &d) {
    DraftGeo g{};
    const int H = d.hidden, D = d.width, F = d.ffn;
    if (D > 1024 || F > 8192 || H > 4096) return g;
    // rows per workgroup: at least rmin, and enough that N rows take at most kDraftPG
    auto lanes = [](int N, int rmin) {
        const int R = std::max(rmin, pow2_at_least((N + kDraftPG - 1) / kDraftPG));
        return R <= 256 ? 256 / R : 0;
    };
    auto pieces = [](int K, int L) { return (K / 16 + L - 1) / L; };
    g.lp = lanes(D, 2);                 // bf16 results go out in pairs
    g.lgu = lanes(F, 1);
    // down: the fewest workgroups whose rows still fit kDpDnC pieces a lane (fewer
    // workgroups poll the blocks' inner vector)
    const int ld_want = std::min(128, std::max(16, pow2_at_least(F / (16 * kDpDnC))));
    g.ld = std::min(lanes(D, 2), ld_want);
    g.lpo = lanes(H, 2);
    g.ok = g.lp && g.lgu && g.ld && g.lpo && pieces(2 * H, g.lp) <= kDpPreC && pieces(D, g.lgu) <= kDpGuC &&
           pieces(F, g.ld) <= kDpDnC && pieces(D, g.lpo) <= kDpPoC;
    return g;
}

struct DraftWs {
    size_t z, zf, g, h, lm;                 // the chain of launches
    size_t ctr, epoch, zw, hw, gw, kw;      // the persistent kernel (when draft_geo().ok)
    size_t total;
};
inline DraftWs draft_ws(const moe_draft_desc &d) {
    DraftWs W{};
    size_t o = 0;
    auto take = [&](size_t bytes) { size_t r = o; o = align256(o + bytes); return r; };
    W.z = take(2 * (size_t)d.width);
    W.zf = take(2 * (size_t)d.width);
    W.g = take(2 * (size_t)d.hidden);
    W.h = take(4 * (size_t)d.ffn);
    W.lm = take(lm_ws_bytes(1, d.vocab));
    if (draft_geo(d).ok) {
        const size_t G7 = kDraftMaxGamma;
        W.ctr = take(4);
        W.epoch = take(4);
        W.zw = take(8 * G7 * (size_t)(d.blocks + 1) * (size_t)(d.width / 2));
        W.hw = take(8 * G7 * (size_t)d.blocks * (size_t)d.ffn);
        W.gw = take(8 * G7 * (size_t)(d.hidden / 2));
        W.kw = take(8 * G7 * (size_t)kDraftPG * 2);
    }
    W.total = o;
    return W;
}

// ---------------------------------------------------------------- attention decode

// Layout of one layer's KV cache: values (bf16 or FP8 codes) [kv_heads][capacity][head_dim],
// then, for FP8, fp32 scales [kv_heads][capacity] at `scales`.
struct AttnCache {
    size_t scales, total;
};
inline AttnCache attn_cache(const moe_attn_desc &d) {
    AttnCache C{};
    const size_t n = (size_t)d.kv_heads * d.capacity * d.head_dim;
    if (d.kv_type == MOE_KV_FP8) {
        C.scales = align256(n);
        C.total = C.scales + 4 * (size_t)d.kv_heads * d.capacity;
    } else {
        C.scales = 0;
        C.total = 2 * n;
    }
    return C;
}

// The partial-softmax grid for M tokens at pos: G query heads per KV head, Q = G M queries
// per KV head in tiles of 16, 16-position chunks from lo0 (token 0's first visible position)
// to pos + M - 1, nwg stripes of chunks per (KV head, tile) so the grid stays <= 512
// workgroups and the records (one per query and stripe) <= 16 x 512. The matrix-core form
// (all of a KV head's queries in one workgroup) takes up to 32 x 512 records: a stripe per
// compute unit for 2 KV heads of 64 queries.
constexpr int kAttnMaxWG = 512;
constexpr int kAttnRecords = 32 * kAttnMaxWG;
struct AttnPlan {
    int G, Q, qsplit, lo0, nch, nwg;
};
inline AttnPlan attn_plan(const moe_attn_desc &d, int M, int pos) {
    AttnPlan P{};
    P.G = d.q_heads / d.kv_heads;
    P.Q = P.G * M;
    P.qsplit = (P.Q + 15) / 16;
    P.lo0 = d.window > 0 ? (pos - d.window + 1 > 0 ? pos - d.window + 1 : 0) : 0;
    P.nch = (pos + M - P.lo0 + 15) / 16;
    const int cap = kAttnMaxWG / (d.kv_heads * P.qsplit);
    P.nwg = P.nch < (cap > 1 ? cap : 1) ? P.nch : (cap > 1 ? cap : 1);
    return P;
}
struct AttnWs {
    size_t q, k, o, part, total;
};
inline AttnWs attn_ws(const moe_attn_desc &d, int max_M) {
    AttnWs W{};
    size_t o = 0;
    auto take = [&](size_t bytes) { size_t r = o; o = align256(o + bytes); return r; };
    const size_t NQ = (size_t)d.q_heads * d.head_dim, NK = (size_t)d.kv_heads * d.head_dim;
    W.q = take(2 * NQ * max_M);
    W.k = take(2 * NK * max_M);
    W.o = take(2 * NQ * max_M);
    W.part = take(4 * (size_t)kAttnRecords * (d.head_dim + 4));
    W.total = o;
    return W;
}

// Static scratch of lm_head_argmax_noalloc: the workspace of the largest call (M = 8,
// the full lm_head grid), 128 KiB.
constexpr size_t kLmNoallocScratch = 2 * (size_t)kLmMaxWG * kMaxM * 4;

// ---------------------------------------------------------------- fused step

constexpr int kMaxLayers = 64;
constexpr int kStepChunks = 11;       // the fused step's rows: 11 chunks (256 columns of H, 64 of a down row)
constexpr int kStepMaxHidden = kStepChunks * 256;   // 2816: a row of H per lane group, zero-padded
constexpr int kStepMaxWidth = kStepChunks * 64;     // 704: one 64-row down unit covers a whole routed row
constexpr int kStepMaxSharedSeg = 8;  // column segments of the shared expert's down rows
constexpr int kStepMaxGrid = 2048;    // persistent workgroups
constexpr int kCtrStride = 16;        // ints between counters (64 bytes)
constexpr unsigned kDefaultSpin = 1u << 18;   // about a quarter second of polling

// Column segments of a down row of width F: the fewest that divide the F / 64 chunks
// into at most kStepChunks chunks each.
inline int step_nseg(int F) {
    if (F <= 0) return 0;
    const int c = F / 64;
    for (int n = (c + kStepChunks - 1) / kStepChunks; n < c; ++n)
        if (c % n == 0) return n;
    return c;
}

struct StepWs {
    size_t table;        // moe_layer_weights [L]
    size_t rt;           // bf16 [L][E][H]: router weights re-laid out one expert per row
    size_t ctr;          // int [kCtrStride]: the error flag
    size_t flags;        // uint32: lm_head workgroup done [kStepMaxGrid], then the epoch
    // Hand-off words (uint64): the value in the low 32 bits, the step's tag in the high 32.
    size_t logits;       // [L][Mx][E] router logits (fp32)
    size_t hres;         // [L+1][Mx][H/2] residual stream entering each layer (2 x bf16); [0] unused
    size_t hact;         // [L][Sx][Mx][F] gelu(gate) * up per slot and token (fp32)
    size_t ypart;        // [L][NSUBx][Mx][H] weighted down output per sub-slot and token (fp32)
    size_t lmbest;       // uint64 [kStepMaxGrid][kMaxM] per-workgroup best (logit, row) keys
    size_t total;
    int L, Mx, Sx, NR, ND, UGx, NSUBx, F, segFmax, nseg_r, nseg_s;
    int f_lm, f_epoch, nflags;
};

// prepared: the fused step's layout (weight table and re-laid-out router weights first);
// otherwise moe_decode_layer's (neither region; the error flag and the flags come first, at
// offsets that do not depend on the token count).
inline StepWs step_ws(const moe_step_desc &d, bool prepared = true) {
    StepWs W{};
    const moe_layer_desc &ld = d.layer;
    const int H = ld.hidden, E = ld.num_experts, L = d.num_layers, Mx = d.max_tokens;
    const int D = ld.expert_width, Ds = ld.shared_width, has_sh = Ds > 0 ? 1 : 0;
    W.L = L;
    W.Mx = Mx;
    W.Sx = max_slots(Mx, ld.top_k, E, Ds);
    W.NR = (E + 7) / 8;
    W.ND = H / 64;
    W.nseg_r = step_nseg(D);
    W.nseg_s = step_nseg(Ds);
    W.UGx = (W.Sx - has_sh) * (D / 8) + Ds / 8;
    W.NSUBx = (W.Sx - has_sh) * W.nseg_r + W.nseg_s;
    W.F = D > Ds ? D : Ds;
    W.segFmax = D / W.nseg_r;
    if (Ds > 0 && Ds / W.nseg_s > W.segFmax) W.segFmax = Ds / W.nseg_s;
    W.f_lm = 0;
    W.f_epoch = kStepMaxGrid;
    W.nflags = W.f_epoch + 16;
    size_t o = 0;
    auto take = [&](size_t bytes) { size_t r = o; o = align256(o + bytes); return r; };
    W.table = take(prepared ? sizeof(moe_layer_weights) * (size_t)L : 0);
    W.rt = take(prepared ? 2 * (size_t)L * E * H : 0);
    W.ctr = take(sizeof(int) * (size_t)kCtrStride);
    W.flags = take(4 * (size_t)W.nflags);
    W.logits = take(8 * (size_t)L * Mx * E);
    W.hres = take(8 * (size_t)(L + 1) * Mx * (H / 2));
    W.hact = take(8 * (size_t)L * W.Sx * Mx * W.F);
    W.ypart = take(8 * (size_t)L * W.NSUBx * Mx * H);
    W.lmbest = take(8 * (size_t)kStepMaxGrid * kMaxM);
    W.total = o;
    return W;
}

// moe_decode_layer runs on the fused step's kernel (one layer, no lm_head) when the layer
// fits its unit geometry; wider layers take the separate per-layer kernels.
inline bool layer_fits_step(const moe_layer_desc &d) {
    return d.hidden <= kStepMaxHidden && d.expert_width <= kStepMaxWidth &&
           step_nseg(d.shared_width) <= kStepMaxSharedSeg;
}

inline moe_step_desc layer_step_desc(const moe_layer_desc &d, int M) {
    moe_step_desc s{};
    s.layer = d;
    s.num_layers = 1;
    s.vocab = 64;
    s.max_tokens = M;
    return s;
}

// Layout of moe_decode_layer's workspace on the fused kernel, for M tokens.
inline StepWs layer_step_ws(const moe_layer_desc &d, int M) { return step_ws(layer_step_desc(d, M), false); }

// Launchers (kernels.hip, step.hip). Arguments were validated by api.cpp. Each returns
// MOE_OK or MOE_ELAUNCH.
int launch_moe_layer(const moe_layer_desc &d, const moe_layer_weights &w, int M,
                     const uint16_t *x, uint16_t *y, int32_t *topk_idx, float *topk_w,
                     char *ws, const LayerWs &L, void *stream);
int launch_lm_head(int M, int H, int V, const uint16_t *x, const uint8_t *w, const float *s,
                   int32_t *token, float *max_logit, char *ws, void *stream);
int launch_lm_head_logits(int M, int H, int V, const uint16_t *x, const uint8_t *w, const float *s,
                          const SampleWs &L, char *ws, void *stream);
int launch_spec_sample(int M, int V, float inv_t, const int32_t *draft, const float *q, const float *u_acc,
                       uint64_t seed, uint64_t step, int32_t *accepted_len, int32_t *out_tokens,
                       const SampleWs &L, char *ws, void *stream);
int launch_lm_head_bf16(int M, int H, int V, const uint16_t *x, const uint16_t *w, int32_t *token, float *max_logit,
                        char *ws, void *stream);
int launch_draft_step(const moe_draft_desc &d, const moe_draft_weights &w, int gamma, const int32_t *tok0,
                      const uint16_t *hidden0, const uint8_t *emb_w, const float *emb_s, int32_t *drafts,
                      char *ws, void *stream);
// The persistent drafter (MOE_EUNSUPPORTED when the shape or the device does not fit it)
// and the status of its bounded waits.
int launch_draft_fused(const moe_draft_desc &d, const moe_draft_weights &w, int gamma, const int32_t *tok0,
                       const uint16_t *hidden0, const uint8_t *emb_w, const float *emb_s, int32_t *drafts,
                       char *ws, void *stream);
int draft_status(const moe_draft_desc &d, char *ws);
int launch_lm_head_noalloc(int M, int H, int V, const uint16_t *x, const uint8_t *w, const float *s,
                           int32_t *token, float *max_logit, void *stream);
int launch_spec_accept(int gamma, const int32_t *draft, const int32_t *target,
                       int32_t *accepted_len, int32_t *out_tokens, void *stream);
int launch_add_rmsnorm(int M, int H, const uint16_t *h_in, const uint16_t *a0, const uint16_t *a1,
                       const uint16_t *g, float eps, uint16_t *h_out, uint16_t *u, void *stream);
int launch_step(const moe_step_desc &d, const StepWs &W, int M, const uint16_t *gains,
                const uint8_t *lm_w, const float *lm_s, const uint16_t *x, const uint16_t *noise,
                const int32_t *draft, int32_t *token, float *max_logit, int32_t *accepted_len,
                int32_t *out_tokens, uint16_t *y_layers, int32_t *topk_idx, float *topk_w,
                uint16_t *x_final, char *ws, void *stream);
int launch_layer_step(const moe_layer_desc &d, const moe_layer_weights &w, int M, const uint16_t *x, uint16_t *y,
                      int32_t *topk_idx, float *topk_w, char *ws, void *stream);
int step_prepare(const StepWs &W, const moe_layer_desc &ld, const moe_layer_weights *layers, char *ws);
int step_status(const StepWs &W, char *ws);
int launch_fp8_decode(int n, const uint8_t *codes, float *via_bf16, float *via_f32, void *stream);
int launch_kv_write(const moe_attn_desc &d, int first_pos, int n, const uint16_t *k, char *cache, void *stream);
int launch_attn_decode(const moe_attn_desc &d, const moe_attn_weights &w, int M, int pos, const uint16_t *u,
                       char *cache, uint16_t *out, uint16_t *o_user, char *ws, void *stream);
int launch_read_probe(const void *src, size_t bytes, uint32_t *sink, void *stream);

}  // namespace moe
