// internal.h -- workspace layout and kernel launchers shared by api.cpp (host
// validation, no HIP headers) and kernels.hip (device code).
#pragma once
#include <stddef.h>
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

// ---------------------------------------------------------------- fused step

constexpr int kMaxLayers = 64;
constexpr int kStepMaxHidden = 3072;  // the fused step keeps 12 16-byte chunks of a row per lane
constexpr int kCtrStride = 16;        // ints between counters (64 bytes)
constexpr unsigned kDefaultSpin = 1u << 18;   // about a quarter second of polling
// counter slots: exit count, lm_head top-level count, error flag, lm_head group counts
constexpr int kLmGroups = 32;
constexpr int kExit = 0, kLmTop = 1, kError = 2, kLmSub = 3, kCtrFixed = kLmSub + kLmGroups;

struct StepWs {
    size_t table;        // moe_layer_weights [L]
    size_t ctr;          // int counters, kCtrStride apart
    size_t lmkey;        // uint64 [kLmGroups][kMaxM]: packed (logit, row) maxima per group
    size_t hres;         // bf16 [L+1][Mx][H] residual after each layer's add
    size_t u;            // bf16 [L][Mx][H] normalised layer inputs
    size_t sumsq;        // fp32 [L+1][ND][Mx] per row block sums of squares of hres
    size_t partial;      // fp32 [L][Mx][E][NB] router partial logits
    size_t nslots;       // int [L], kCtrStride apart
    size_t slot_expert;  // int [L][Sx]
    size_t slot_mask;    // uint32 [L][Sx]
    size_t slot_w;       // fp32 [L][Sx][Mx]
    size_t h;            // fp32 [L][Sx][Mx][F]
    size_t ypart;        // fp32 [L][Sx][Mx][H]
    size_t y;            // bf16 [L][Mx][H] (used when the caller passes no y_layers)
    size_t total;
    int L, Mx, Sx, NB, ND, F, nctr;
};

// Counters after the fixed ones (step.hip indexes them): router arrivals [L], routing
// published [L], layer output done [L], gate/up arrivals [L][Sx], down arrivals [L][ND].

inline StepWs step_ws(const moe_step_desc &d) {
    StepWs W{};
    const moe_layer_desc &ld = d.layer;
    const int H = ld.hidden, E = ld.num_experts, L = d.num_layers, Mx = d.max_tokens;
    W.L = L;
    W.Mx = Mx;
    W.Sx = max_slots(Mx, ld.top_k, E, ld.shared_width);
    W.NB = (H + kRouterRows - 1) / kRouterRows;
    W.ND = H / 64;
    W.F = ld.expert_width > ld.shared_width ? ld.expert_width : ld.shared_width;
    W.nctr = kCtrFixed + 3 * L + L * W.Sx + L * W.ND;
    size_t o = 0;
    auto take = [&](size_t bytes) { size_t r = o; o = align256(o + bytes); return r; };
    W.table = take(sizeof(moe_layer_weights) * (size_t)L);
    W.ctr = take(sizeof(int) * (size_t)kCtrStride * W.nctr);
    W.lmkey = take(8 * (size_t)kLmGroups * kMaxM);
    W.hres = take(2 * (size_t)(L + 1) * Mx * H);
    W.u = take(2 * (size_t)L * Mx * H);
    W.sumsq = take(4 * (size_t)(L + 1) * W.ND * Mx);
    W.partial = take(4 * (size_t)L * Mx * E * W.NB);
    W.nslots = take(sizeof(int) * (size_t)kCtrStride * L);
    W.slot_expert = take(4 * (size_t)L * W.Sx);
    W.slot_mask = take(4 * (size_t)L * W.Sx);
    W.slot_w = take(4 * (size_t)L * W.Sx * Mx);
    W.h = take(4 * (size_t)L * W.Sx * Mx * W.F);
    W.ypart = take(4 * (size_t)L * W.Sx * Mx * H);
    W.y = take(2 * (size_t)L * Mx * H);
    W.total = o;
    return W;
}

// Launchers (kernels.hip, step.hip). Arguments were validated by api.cpp. Each returns
// MOE_OK or MOE_ELAUNCH.
int launch_moe_layer(const moe_layer_desc &d, const moe_layer_weights &w, int M,
                     const uint16_t *x, uint16_t *y, int32_t *topk_idx, float *topk_w,
                     char *ws, const LayerWs &L, void *stream);
int launch_lm_head(int M, int H, int V, const uint16_t *x, const uint8_t *w, const float *s,
                   int32_t *token, float *max_logit, char *ws, void *stream);
int launch_spec_accept(int gamma, const int32_t *draft, const int32_t *target,
                       int32_t *accepted_len, int32_t *out_tokens, void *stream);
int launch_add_rmsnorm(int M, int H, const uint16_t *h_in, const uint16_t *a0, const uint16_t *a1,
                       const uint16_t *g, float eps, uint16_t *h_out, uint16_t *u, void *stream);
int launch_step(const moe_step_desc &d, const StepWs &W, int M, const uint16_t *gains,
                const uint8_t *lm_w, const float *lm_s, const uint16_t *x, const uint16_t *noise,
                const int32_t *draft, int32_t *token, float *max_logit, int32_t *accepted_len,
                int32_t *out_tokens, uint16_t *y_layers, int32_t *topk_idx, float *topk_w,
                uint16_t *x_final, char *ws, void *stream);
int step_prepare(const StepWs &W, const moe_layer_weights *layers, char *ws);
int step_status(const StepWs &W, char *ws);
int launch_fp8_decode(int n, const uint8_t *codes, float *via_bf16, float *via_f32, void *stream);

}  // namespace moe
