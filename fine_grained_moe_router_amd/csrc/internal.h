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

// Launchers (kernels.hip). Arguments were validated by api.cpp. Each returns
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
int launch_fp8_decode(int n, const uint8_t *codes, float *via_bf16, float *via_f32, void *stream);

}  // namespace moe
