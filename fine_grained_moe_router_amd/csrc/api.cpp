// api.cpp -- the C ABI: argument validation, workspace carving, and hand-off to
// the launchers in kernels.hip. Plain C++ with no HIP headers, so the validation
// can be built and exercised on a host without a GPU.
#include <limits.h>
#include <stdint.h>

#include "internal.h"

using namespace moe;

namespace {

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

int check_layer_desc(const moe_layer_desc *d) {
    if (!d) return MOE_EINVAL;
    if (d->hidden < 256 || d->hidden > kMaxHidden || d->hidden % 256) return MOE_EINVAL;
    if (d->num_experts < 2 || d->num_experts > kMaxExperts || d->num_experts % 2) return MOE_EINVAL;
    if (d->top_k < 1 || d->top_k > d->num_experts || d->top_k > kMaxTopK) return MOE_EINVAL;
    if (d->expert_width < 64 || d->expert_width > kMaxWidth || d->expert_width % 64) return MOE_EINVAL;
    if (d->shared_width < 0 || d->shared_width > kMaxWidth || d->shared_width % 64) return MOE_EINVAL;
    if (d->wtype != MOE_W_FP8_E4M3 && d->wtype != MOE_W_BF16) return MOE_EINVAL;
    const int rt = d->router_type & ~(int)MOE_ROUTER_EXPERT_MAJOR;
    if (rt != MOE_ROUTER_BF16 && rt != MOE_ROUTER_FP8) return MOE_EINVAL;
    return MOE_OK;
}

// A required device pointer: NULL -> EINVAL, misaligned -> EALIGN.
int need(const void *p) {
    if (!p) return MOE_EINVAL;
    return aligned16(p) ? MOE_OK : MOE_EALIGN;
}

#define CHECK(expr)                 \
    do {                            \
        int st_ = (expr);           \
        if (st_ != MOE_OK) return st_; \
    } while (0)

int check_weights(const moe_layer_desc *desc, const moe_layer_weights *w) {
    if (!w) return MOE_EINVAL;
    const bool fp8 = desc->wtype == MOE_W_FP8_E4M3;
    CHECK(need(w->router_w));
    if (desc->router_type & MOE_ROUTER_FP8) CHECK(need(w->router_s));
    if (w->router_bias && !aligned16(w->router_bias)) return MOE_EALIGN;
    CHECK(need(w->gate_w));
    CHECK(need(w->up_w));
    CHECK(need(w->down_w));
    if (fp8) {
        CHECK(need(w->gate_s));
        CHECK(need(w->up_s));
        CHECK(need(w->down_s));
    }
    if (desc->shared_width > 0) {
        CHECK(need(w->sh_gate_w));
        CHECK(need(w->sh_up_w));
        CHECK(need(w->sh_down_w));
        if (fp8) {
            CHECK(need(w->sh_gate_s));
            CHECK(need(w->sh_up_s));
            CHECK(need(w->sh_down_s));
        }
    }
    return MOE_OK;
}

int check_step_desc(const moe_step_desc *d) {
    if (!d) return MOE_EINVAL;
    CHECK(check_layer_desc(&d->layer));
    if (d->layer.hidden > kStepMaxHidden) return MOE_EINVAL;
    if (d->layer.expert_width > kStepMaxWidth) return MOE_EINVAL;
    if (step_nseg(d->layer.shared_width) > kStepMaxSharedSeg) return MOE_EINVAL;
    if (d->num_layers < 1 || d->num_layers > kMaxLayers) return MOE_EINVAL;
    if (d->vocab < 64 || d->vocab % 64 || d->vocab > (1 << 30)) return MOE_EINVAL;
    if (d->max_tokens < 1 || d->max_tokens > kMaxM) return MOE_EINVAL;
    if (!(d->eps >= 0.0f)) return MOE_EINVAL;
    if (d->flags & ~(MOE_STEP_COOPERATIVE | MOE_STEP_LM_BF16)) return MOE_EINVAL;
    return MOE_OK;
}

bool ws_ok(const void *ws, size_t bytes, size_t need_bytes) {
    return ws && !((uintptr_t)ws & 255u) && bytes >= need_bytes;
}

}  // namespace

extern "C" {

const char *moe_strerror(int status) {
    switch (status) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument (size out of range or required pointer NULL)";
    case MOE_EALIGN: return "pointer not 16-byte aligned";
    case MOE_EWORKSPACE: return "workspace missing or too small";
    case MOE_EUNSUPPORTED: return "unsupported configuration";
    case MOE_ELAUNCH: return "kernel launch failed";
    case MOE_ETIMEOUT: return "a device-side wait of the fused step gave up";
    default: return "unknown status";
    }
}

size_t moe_decode_layer_workspace(const moe_layer_desc *desc, int max_M) {
    if (check_layer_desc(desc) != MOE_OK || max_M < 1 || max_M > kMaxM) return 0;
    if (!layer_fits_step(*desc) && desc->router_type != MOE_ROUTER_BF16) return 0;
    return layer_fits_step(*desc) ? layer_step_ws(*desc, max_M).total : layer_ws(*desc, max_M).total;
}

int moe_decode_layer(const moe_layer_desc *desc, const moe_layer_weights *w, int M,
                     const uint16_t *x, uint16_t *y, int32_t *topk_idx, float *topk_w,
                     void *workspace, size_t workspace_bytes, void *stream) {
    CHECK(check_layer_desc(desc));
    if (!w || M < 1 || M > kMaxM) return MOE_EINVAL;
    CHECK(check_weights(desc, w));
    CHECK(need(x));
    CHECK(need(y));
    if (((uintptr_t)topk_idx | (uintptr_t)topk_w) & 3u) return MOE_EALIGN;
    if (layer_fits_step(*desc)) {
        if (!ws_ok(workspace, workspace_bytes, layer_step_ws(*desc, M).total)) return MOE_EWORKSPACE;
        return launch_layer_step(*desc, *w, M, x, y, topk_idx, topk_w, (char *)workspace, stream);
    }
    // the per-layer kernels read a bf16 router laid out [H][E]
    if (desc->router_type != MOE_ROUTER_BF16) return MOE_EUNSUPPORTED;
    const LayerWs L = layer_ws(*desc, M);
    if (!ws_ok(workspace, workspace_bytes, L.total)) return MOE_EWORKSPACE;
    return launch_moe_layer(*desc, *w, M, x, y, topk_idx, topk_w, (char *)workspace, L, stream);
}

int moe_decode_layer_status(const moe_layer_desc *desc, void *workspace) {
    CHECK(check_layer_desc(desc));
    if (!workspace || ((uintptr_t)workspace & 255u)) return MOE_EWORKSPACE;
    if (!layer_fits_step(*desc)) return MOE_OK;   // the per-layer kernels have no device-side waits
    return step_status(layer_step_ws(*desc, 1), (char *)workspace);
}

size_t lm_head_argmax_workspace(int max_M, int H, int V) {
    if (max_M < 1 || max_M > kMaxM || H < 256 || H > kMaxHidden || H % 256 || V < 64 ||
        V % 64 || V > (1 << 30))
        return 0;
    return lm_ws_bytes(max_M, V);
}

int lm_head_argmax(int M, int H, int V, const uint16_t *x, const uint8_t *w, const float *w_s,
                   int32_t *token, float *max_logit, void *workspace, size_t workspace_bytes,
                   void *stream) {
    if (M < 1 || M > kMaxM || H < 256 || H > kMaxHidden || H % 256 || V < 64 || V % 64 ||
        V > (1 << 30))
        return MOE_EINVAL;
    CHECK(need(x));
    CHECK(need(w));
    CHECK(need(w_s));
    CHECK(need(token));
    if (max_logit && !aligned16(max_logit)) return MOE_EALIGN;
    if (!workspace || ((uintptr_t)workspace & 255u) || workspace_bytes < lm_ws_bytes(M, V))
        return MOE_EWORKSPACE;
    return launch_lm_head(M, H, V, x, w, w_s, token, max_logit, (char *)workspace, stream);
}

int lm_head_argmax_bf16(int M, int H, int V, const uint16_t *x, const uint16_t *w, int32_t *token,
                        float *max_logit, void *workspace, size_t workspace_bytes, void *stream) {
    if (M < 1 || M > kMaxM || H < 256 || H > kMaxHidden || H % 256 || V < 64 || V % 64 ||
        V > (1 << 30))
        return MOE_EINVAL;
    CHECK(need(x));
    CHECK(need(w));
    CHECK(need(token));
    if (max_logit && !aligned16(max_logit)) return MOE_EALIGN;
    if (!workspace || ((uintptr_t)workspace & 255u) || workspace_bytes < lm_ws_bytes(M, V))
        return MOE_EWORKSPACE;
    return launch_lm_head_bf16(M, H, V, x, w, token, max_logit, (char *)workspace, stream);
}

size_t lm_head_spec_sample_workspace(int max_M, int H, int V) {
    if (max_M < 1 || max_M > kMaxM || H < 256 || H > kMaxHidden || H % 256 || V < 64 || V % 64 ||
        V > kSampleMaxVocab)
        return 0;
    return sample_ws(max_M, V).total;
}

int lm_head_spec_sample(int M, int H, int V, const uint16_t *x, const uint8_t *w, const float *w_s,
                        float temperature, const int32_t *draft, const float *q, const float *u_accept,
                        uint64_t seed, uint64_t step, int32_t *accepted_len, int32_t *out_tokens,
                        void *workspace, size_t workspace_bytes, void *stream) {
    if (M < 1 || M > kMaxM || H < 256 || H > kMaxHidden || H % 256 || V < 64 || V % 64 ||
        V > kSampleMaxVocab || !(temperature > 0.0f) || !(temperature < 1e30f))
        return MOE_EINVAL;
    CHECK(need(x));
    CHECK(need(w));
    CHECK(need(w_s));
    if (M > 1) {
        CHECK(need(q));
        if (!draft || !u_accept) return MOE_EINVAL;
    }
    if (!accepted_len || !out_tokens) return MOE_EINVAL;
    if (((uintptr_t)draft | (uintptr_t)u_accept | (uintptr_t)accepted_len | (uintptr_t)out_tokens) & 3u)
        return MOE_EALIGN;
    const SampleWs L = sample_ws(M, V);
    if (!ws_ok(workspace, workspace_bytes, L.total)) return MOE_EWORKSPACE;
    const float inv_t = 1.0f / temperature;
    CHECK(launch_lm_head_logits(M, H, V, x, w, w_s, L, (char *)workspace, stream));
    return launch_spec_sample(M, V, inv_t, draft, q, u_accept, seed, step, accepted_len, out_tokens, L,
                              (char *)workspace, stream);
}

int lm_head_argmax_noalloc(int M, int H, int V, const uint16_t *x, const uint8_t *w, const float *w_s,
                           int32_t *token, float *max_logit, void *stream) {
    if (M < 1 || M > kMaxM || H < 256 || H > kMaxHidden || H % 256 || V < 64 || V % 64 ||
        V > (1 << 30))
        return MOE_EINVAL;
    CHECK(need(x));
    CHECK(need(w));
    CHECK(need(w_s));
    CHECK(need(token));
    if (max_logit && !aligned16(max_logit)) return MOE_EALIGN;
    if (lm_ws_bytes(M, V) > kLmNoallocScratch) return MOE_EWORKSPACE;   // beyond the static scratch
    return launch_lm_head_noalloc(M, H, V, x, w, w_s, token, max_logit, stream);
}

int spec_accept(int num_draft, const int32_t *draft, const int32_t *target,
                int32_t *accepted_len, int32_t *out_tokens, void *stream) {
    if (num_draft < 0 || num_draft > kMaxM - 1) return MOE_EINVAL;
    if (num_draft > 0 && !draft) return MOE_EINVAL;
    if (!target || !accepted_len || !out_tokens) return MOE_EINVAL;
    if (((uintptr_t)draft | (uintptr_t)target | (uintptr_t)accepted_len |
         (uintptr_t)out_tokens) & 3u)
        return MOE_EALIGN;
    return launch_spec_accept(num_draft, draft, target, accepted_len, out_tokens, stream);
}

int moe_add_rmsnorm(int M, int H, const uint16_t *h_in, const uint16_t *add0,
                    const uint16_t *add1, const uint16_t *gain, float eps, uint16_t *h_out,
                    uint16_t *u_out, void *stream) {
    if (M < 1 || M > kMaxM || H < 256 || H > kMaxHidden || H % 256) return MOE_EINVAL;
    if (!(eps >= 0.0f)) return MOE_EINVAL;
    CHECK(need(h_in));
    CHECK(need(add0));
    if (add1 && !aligned16(add1)) return MOE_EALIGN;
    CHECK(need(gain));
    CHECK(need(h_out));
    CHECK(need(u_out));
    return launch_add_rmsnorm(M, H, h_in, add0, add1, gain, eps, h_out, u_out, stream);
}

size_t moe_decode_step_workspace(const moe_step_desc *desc) {
    if (check_step_desc(desc) != MOE_OK) return 0;
    return step_ws(*desc).total;
}

int moe_decode_step_prepare(const moe_step_desc *desc, const moe_layer_weights *layers,
                            void *workspace, size_t workspace_bytes) {
    CHECK(check_step_desc(desc));
    if (!layers) return MOE_EINVAL;
    for (int l = 0; l < desc->num_layers; ++l) CHECK(check_weights(&desc->layer, &layers[l]));
    const StepWs W = step_ws(*desc);
    if (!ws_ok(workspace, workspace_bytes, W.total)) return MOE_EWORKSPACE;
    return step_prepare(W, desc->layer, layers, (char *)workspace);
}

int moe_decode_step(const moe_step_desc *desc, int M, const uint16_t *gains,
                    const uint8_t *lm_w, const float *lm_s, const uint16_t *x,
                    const uint16_t *noise, const int32_t *draft, int32_t *token,
                    float *max_logit, int32_t *accepted_len, int32_t *out_tokens,
                    uint16_t *y_layers, int32_t *topk_idx, float *topk_w, uint16_t *x_final,
                    void *workspace, size_t workspace_bytes, void *stream) {
    CHECK(check_step_desc(desc));
    if (M < 1 || M > desc->max_tokens) return MOE_EINVAL;
    CHECK(need(gains));
    CHECK(need(lm_w));
    if (!(desc->flags & MOE_STEP_LM_BF16)) CHECK(need(lm_s));
    CHECK(need(x));
    CHECK(need(noise));
    if (M > 1 && !draft) return MOE_EINVAL;
    if (!token || !accepted_len || !out_tokens) return MOE_EINVAL;
    if (((uintptr_t)draft | (uintptr_t)token | (uintptr_t)accepted_len | (uintptr_t)out_tokens |
         (uintptr_t)max_logit | (uintptr_t)topk_idx | (uintptr_t)topk_w) & 3u)
        return MOE_EALIGN;
    if ((y_layers && !aligned16(y_layers)) || (x_final && !aligned16(x_final))) return MOE_EALIGN;
    const StepWs W = step_ws(*desc);
    if (!ws_ok(workspace, workspace_bytes, W.total)) return MOE_EWORKSPACE;
    return launch_step(*desc, W, M, gains, lm_w, lm_s, x, noise, draft, token, max_logit,
                       accepted_len, out_tokens, y_layers, topk_idx, topk_w, x_final,
                       (char *)workspace, stream);
}

int moe_decode_step_status(const moe_step_desc *desc, void *workspace) {
    CHECK(check_step_desc(desc));
    if (!workspace || ((uintptr_t)workspace & 255u)) return MOE_EWORKSPACE;
    return step_status(step_ws(*desc), (char *)workspace);
}

static int check_draft_desc(const moe_draft_desc *d) {
    if (!d) return MOE_EINVAL;
    if (d->hidden < 256 || d->hidden > kMaxHidden || d->hidden % 256) return MOE_EINVAL;
    if (d->width < 256 || d->width > 4096 || d->width % 256) return MOE_EINVAL;
    if (d->ffn < 256 || d->ffn > 16384 || d->ffn % 256) return MOE_EINVAL;
    if (d->blocks < 0 || d->blocks > 64) return MOE_EINVAL;
    if (d->vocab < 64 || d->vocab % 64 || d->vocab > (1 << 30)) return MOE_EINVAL;
    if (!(d->eps >= 0.0f)) return MOE_EINVAL;
    if (d->flags & ~MOE_DRAFT_CHAIN) return MOE_EINVAL;
    if (!draft_splits(*d)) return MOE_EINVAL;
    return MOE_OK;
}

size_t moe_draft_step_workspace(const moe_draft_desc *desc) {
    if (check_draft_desc(desc) != MOE_OK) return 0;
    return draft_ws(*desc).total;
}

int moe_draft_step(const moe_draft_desc *desc, const moe_draft_weights *w, int gamma, const int32_t *tok0,
                   const uint16_t *hidden0, const uint8_t *emb_w, const float *emb_s, int32_t *drafts,
                   void *workspace, size_t workspace_bytes, void *stream) {
    CHECK(check_draft_desc(desc));
    if (!w || gamma < 1 || gamma > kMaxM - 1) return MOE_EINVAL;
    CHECK(need(w->pre_w));
    CHECK(need(w->pre_s));
    if (desc->blocks > 0) {
        CHECK(need(w->gate_w));
        CHECK(need(w->gate_s));
        CHECK(need(w->up_w));
        CHECK(need(w->up_s));
        CHECK(need(w->down_w));
        CHECK(need(w->down_s));
    }
    CHECK(need(w->gains));
    CHECK(need(w->table_w));
    CHECK(need(w->table_s));
    CHECK(need(w->post_w));
    CHECK(need(w->post_s));
    CHECK(need(hidden0));
    CHECK(need(emb_w));
    CHECK(need(emb_s));
    if (!tok0 || !drafts) return MOE_EINVAL;
    if (((uintptr_t)tok0 | (uintptr_t)drafts) & 3u) return MOE_EALIGN;
    if (!ws_ok(workspace, workspace_bytes, draft_ws(*desc).total)) return MOE_EWORKSPACE;
    return launch_draft_step(*desc, *w, gamma, tok0, hidden0, emb_w, emb_s, drafts, (char *)workspace, stream);
}

int moe_draft_step_status(const moe_draft_desc *desc, void *workspace) {
    CHECK(check_draft_desc(desc));
    if (!workspace || ((uintptr_t)workspace & 255u)) return MOE_EWORKSPACE;
    return draft_status(*desc, (char *)workspace);
}

static int check_attn_desc(const moe_attn_desc *d) {
    if (!d) return MOE_EINVAL;
    if (d->hidden < 256 || d->hidden > kMaxHidden || d->hidden % 256) return MOE_EINVAL;
    if (d->q_heads < 1 || d->q_heads > 64 || d->kv_heads < 1 || d->kv_heads > 64) return MOE_EINVAL;
    if (d->q_heads % d->kv_heads || d->q_heads / d->kv_heads > 16) return MOE_EINVAL;
    if (d->head_dim != 128 && d->head_dim != 256 && d->head_dim != 512) return MOE_EINVAL;
    if (d->q_heads * d->head_dim > 16384) return MOE_EINVAL;
    if (d->window < 0 || d->window > (1 << 24) || d->capacity < 1 || d->capacity > (1 << 24))
        return MOE_EINVAL;
    if (d->window > 0 && d->capacity < d->window + kMaxM - 1) return MOE_EINVAL;
    if (d->kv_type != MOE_KV_BF16 && d->kv_type != MOE_KV_FP8) return MOE_EINVAL;
    return MOE_OK;
}

size_t moe_kv_cache_bytes(const moe_attn_desc *desc) {
    if (check_attn_desc(desc) != MOE_OK) return 0;
    return attn_cache(*desc).total;
}

int moe_kv_cache_write(const moe_attn_desc *desc, int first_pos, int n, const uint16_t *k, void *cache,
                       void *stream) {
    CHECK(check_attn_desc(desc));
    if (first_pos < 0 || n < 1 || n > (1 << 24) || first_pos > INT_MAX - n) return MOE_EINVAL;
    CHECK(need(k));
    CHECK(need(cache));
    if ((uintptr_t)cache & 255u) return MOE_EALIGN;
    return launch_kv_write(*desc, first_pos, n, k, (char *)cache, stream);
}

size_t moe_attn_decode_workspace(const moe_attn_desc *desc, int max_M) {
    if (check_attn_desc(desc) != MOE_OK || max_M < 1 || max_M > kMaxM) return 0;
    return attn_ws(*desc, max_M).total;
}

int moe_attn_decode(const moe_attn_desc *desc, const moe_attn_weights *w, int M, int pos, const uint16_t *u,
                    void *cache, uint16_t *out, uint16_t *o, void *workspace, size_t workspace_bytes,
                    void *stream) {
    CHECK(check_attn_desc(desc));
    if (!w || M < 1 || M > kMaxM || pos < 0 || pos > INT_MAX - M) return MOE_EINVAL;
    if (desc->window == 0 && pos + M > desc->capacity) return MOE_EINVAL;
    CHECK(need(w->q_w));
    CHECK(need(w->q_s));
    CHECK(need(w->k_w));
    CHECK(need(w->k_s));
    CHECK(need(w->o_w));
    CHECK(need(w->o_s));
    CHECK(need(u));
    CHECK(need(cache));
    CHECK(need(out));
    if ((uintptr_t)cache & 255u) return MOE_EALIGN;
    if (o && !aligned16(o)) return MOE_EALIGN;
    if (!ws_ok(workspace, workspace_bytes, attn_ws(*desc, M).total)) return MOE_EWORKSPACE;
    return launch_attn_decode(*desc, *w, M, pos, u, (char *)cache, out, o, (char *)workspace, stream);
}

int moe_fp8_decode(int n, const uint8_t *codes, float *out_via_bf16, float *out_via_f32,
                   void *stream) {
    if (n < 4 || n > (1 << 20) || n % 4) return MOE_EINVAL;
    CHECK(need(codes));
    CHECK(need(out_via_bf16));
    CHECK(need(out_via_f32));
    return launch_fp8_decode(n, codes, out_via_bf16, out_via_f32, stream);
}

int moe_hbm_read_probe(const void *src, size_t bytes, uint32_t *sink, void *stream) {
    if (bytes == 0 || bytes % 16) return MOE_EINVAL;
    CHECK(need(src));
    CHECK(need(sink));
    return launch_read_probe(src, bytes, sink, stream);
}

}  // extern "C"
