/*
 * moe_decode.h -- C ABI of the MI355X (gfx950) batch-1 fine-grained MoE decode step.
 *
 * One decode step of a Gemma-4-26B-A4B-shaped mixture-of-experts model at batch 1,
 * including the small verify batch of speculative decoding (M <= 8 tokens that
 * share one pass over the weights). Shapes and the structure of the step follow
 * the page "LLM decoding" (us-homepage.pages.dev/blog/llm-decoding):
 *   - "The exact architecture, and why it rules out 4-bit": each layer routes to
 *     the top 8 of 128 experts plus one always-on shared expert; expert width 704,
 *     hidden 2816; tied lm_head over a 262,144-token vocabulary.
 *   - "Where the 7.36 GB goes": per expert a gate, an up and a down matrix; a
 *     router; the lm_head read once per token.
 *   - "Lever 1: fewer bytes (FP8 weights)": weights stored in 8 bits and decoded
 *     to a wider type for the arithmetic.
 *   - "Lever 2: fewer passes (native MTP)": the target checks the drafted tokens
 *     in a single pass and keeps the ones it would have produced.
 *
 * Conventions for every entry point
 *   - Device pointers are owned by the caller; the library allocates nothing,
 *     never synchronises and keeps no global mutable state. Calls with distinct
 *     workspaces may run concurrently on different streams.
 *   - `stream` is a hipStream_t (NULL: the default stream). Work is enqueued
 *     asynchronously; calls are hipGraph-capturable (no memset nodes are used).
 *   - Matrices are row-major [rows][cols]. bf16 values are passed as their 16-bit
 *     patterns (uint16_t). FP8 values are OCP E4M3FN code bytes (bias 7, max 448,
 *     NaN = 0x7F/0xFF), each output row with one fp32 scale applied after its dot
 *     product: out[r] = scale[r] * sum_c decode(Q[r][c]) * x[c].
 *   - Arguments are validated on the host before anything is enqueued. A
 *     failure returns a negative moe_status and enqueues nothing; MOE_ELAUNCH
 *     means the runtime refused a launch (work already enqueued by the same call
 *     may have run). Faults inside kernels surface at the caller's next
 *     synchronisation.
 *   - Arithmetic: products of FP8/bf16 values are exact in fp32; sums are fp32.
 *     The router logits, the expert intermediates and the combine stay fp32;
 *     the only rounding to bf16 is that of each output tensor.
 */
#ifndef MOE_DECODE_H
#define MOE_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
    MOE_OK = 0,
    MOE_EINVAL = -1,        /* a size or count out of range, or a required pointer is NULL */
    MOE_EALIGN = -2,        /* a pointer is not 16-byte aligned                              */
    MOE_EWORKSPACE = -3,    /* workspace NULL or smaller than the *_workspace() size         */
    MOE_EUNSUPPORTED = -4,  /* a valid request the library does not implement               */
    MOE_ELAUNCH = -5,       /* the HIP runtime rejected a kernel launch                      */
    MOE_ETIMEOUT = -6       /* a device-side wait of moe_decode_step gave up                 */
} moe_status;

typedef enum moe_wtype {
    MOE_W_FP8_E4M3 = 0,     /* expert weights: FP8 E4M3FN codes + fp32 per-row scales        */
    MOE_W_BF16 = 1          /* expert weights: bf16, no scales                               */
} moe_wtype;

/* Router weights (page "LLM decoding", "Lever 1: fewer bytes" and "The ladder, every
 * rung": the precision of each matrix is a rung of its own). */
typedef enum moe_router_type {
    MOE_ROUTER_BF16 = 0,    /* router_w bf16 [H][E]                                          */
    MOE_ROUTER_FP8 = 1,     /* router_w FP8 E4M3FN codes [H][E], router_s fp32 [E] (one scale
                               per expert, applied to the finished logit)                     */
    MOE_ROUTER_EXPERT_MAJOR = 2  /* flag, OR-ed with either type: router_w laid out [E][H]
                               (row e = expert e's H weights) instead of [H][E]; the same
                               values give the same results bit for bit. moe_decode_layer's
                               one-launch form then reads each expert's row whole instead of
                               gathering it from [H][E] (about 5 us less per call at the
                               Gemma shape); the per-layer kernels do not take it          */
} moe_router_type;

/* Shape of one MoE layer.
 *   hidden        H: a multiple of 256, at most 4096            (Gemma-4-26B-A4B: 2816)
 *   num_experts   E: even, 2..256                                (128)
 *   top_k         K: 1..min(E, 16)                               (8)
 *   expert_width  D: a multiple of 64, 64..4096                  (704)
 *   shared_width  Ds: 0 (no shared expert) or a multiple of 64 up to 4096 (704; the
 *                 page's dense MLP is 2112 wide)
 *   wtype         a moe_wtype for the routed and shared expert matrices
 *   router_type   a moe_router_type (MOE_ROUTER_BF16 when zero-initialised), optionally OR-ed
 *                 with MOE_ROUTER_EXPERT_MAJOR; an FP8 or expert-major router runs on the
 *                 fused step and on moe_decode_layer's one-launch form only */
typedef struct moe_layer_desc {
    int hidden;
    int num_experts;
    int top_k;
    int expert_width;
    int shared_width;
    int wtype;
    int router_type;
} moe_layer_desc;

/* Weights of one MoE layer (device pointers, 16-byte aligned).
 *   router_w     [H][E] ([E][H] with MOE_ROUTER_EXPERT_MAJOR): bf16, or FP8 E4M3FN codes
 *                (MOE_ROUTER_FP8)
 *   router_bias  fp32 [E], added to the logits before the softmax; NULL for none
 *   gate_w, up_w [E][D][H]   down_w [E][H][D]   (FP8 codes or bf16 per wtype)
 *   gate_s, up_s fp32 [E][D] down_s fp32 [E][H] (FP8 only; ignored for bf16)
 *   sh_*         the shared expert: gate/up [Ds][H], down [H][Ds], scales [Ds],[Ds],[H];
 *                ignored when shared_width == 0
 *   router_s     fp32 [E], the FP8 router's per-expert scales (ignored for a bf16 router) */
typedef struct moe_layer_weights {
    const void *router_w;
    const float *router_bias;
    const void *gate_w;
    const void *up_w;
    const void *down_w;
    const float *gate_s;
    const float *up_s;
    const float *down_s;
    const void *sh_gate_w;
    const void *sh_up_w;
    const void *sh_down_w;
    const float *sh_gate_s;
    const float *sh_up_s;
    const float *sh_down_s;
    const float *router_s;
} moe_layer_weights;

/* Bytes of device workspace moe_decode_layer needs for up to max_M tokens
 * (0 if desc is invalid or max_M is outside 1..8). */
size_t moe_decode_layer_workspace(const moe_layer_desc *desc, int max_M);

/*
 * Synchronous: MOE_OK, or MOE_ETIMEOUT if a device-side wait of a moe_decode_layer call
 * on this workspace gave up since the last call (its results are then invalid); the
 * flag is cleared and the workspace made ready for the next call, as with
 * moe_decode_step_status. Call after the stream has been synchronised, with no call in
 * flight. Layers that take the separate per-layer kernels (see moe_decode_layer) have
 * no device-side waits and always return MOE_OK.
 */
int moe_decode_layer_status(const moe_layer_desc *desc, void *workspace);

/*
 * One MoE layer for M tokens (1 <= M <= 8; the batch-1 decode step is M = 1, the
 * speculative verify step with gamma drafts is M = gamma + 1). Page "LLM decoding":
 * "The exact architecture, and why it rules out 4-bit" (top 8 of 128 routed experts
 * plus one always-on shared expert, expert width 704, hidden 2816); "Where the
 * 7.36 GB goes" (a gate, an up and a down matrix per expert, and the router);
 * "Lever 1: fewer bytes (FP8 weights)" (8-bit weights, arithmetic in a wider type).
 * The gating (softmax over all experts, keep K, renormalise), the GELU-tanh gate and
 * the tie rule are readings the page leaves open.
 *   logits[m][e] = sum_c x[m][c] * router_w[c][e] (+ router_bias[e]); an FP8 router:
 *                  router_s[e] * sum_c x[m][c] * decode(router_w[c][e]) (+ router_bias[e])
 *   S_m          = the K experts with the largest logits (equal logits: lower id)
 *   w[m][e]      = softmax(logits[m])[e] / sum_{j in S_m} softmax(logits[m])[j]
 *   expert_e(v)  = down_e( gelu_tanh(gate_e v) * (up_e v) ),
 *                  gelu_tanh(z) = 0.5 z (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3)))
 *   y[m]         = sum_{e in S_m, ascending e} w[m][e] expert_e(x[m]) + shared(x[m])
 * The shared expert is always on with weight 1. Every selected expert's weights
 * are read once per call however many of the M tokens selected it. y[m] depends
 * only on x[m]: identical tokens give bit-identical rows, and a row does not
 * change with M or with the other tokens in the call.
 *   x          bf16 [M][H], the (already normalised) layer input
 *   y          bf16 [M][H], the MoE branch output (the residual is NOT added)
 *   topk_idx   int32 [M][K], S_m in ascending expert id, or NULL (4-byte aligned)
 *   topk_w     fp32 [M][K], the weights aligned with topk_idx, or NULL (4-byte aligned)
 *   workspace  at least moe_decode_layer_workspace(desc, M) bytes, 256-byte aligned,
 *              zero-filled before its first use and then left to the library (it keeps
 *              a step counter and tagged hand-off words between calls)
 * Layers with hidden <= 2816, expert_width <= 704 and a shared expert of at most eight
 * 704-column segments (the Gemma-4-26B-A4B layer among them) run as one launch of the
 * fused step's persistent kernel (see moe_decode_step: the same routing, units and
 * combine, so y is bit-identical to that step's layer output for the same input, and
 * the same co-residency requirement and bounded waits; see moe_decode_layer_status).
 * Wider layers run as five dependent kernels (router partials, top-K and union,
 * gate/up, down, combine) with no device-side waits.
 */
int moe_decode_layer(const moe_layer_desc *desc, const moe_layer_weights *w, int M,
                     const uint16_t *x, uint16_t *y, int32_t *topk_idx, float *topk_w,
                     void *workspace, size_t workspace_bytes, void *stream);

/* Bytes of workspace lm_head_argmax needs (0 for invalid sizes). */
size_t lm_head_argmax_workspace(int max_M, int H, int V);

/*
 * Tied lm_head GEMV and greedy argmax for M rows (page "LLM decoding", "Where the
 * 7.36 GB goes": the output projection read once per token over the whole vocabulary).
 *   logit[m][v] = w_s[v] * sum_c decode(w[v][c]) * x[m][c]
 *   token[m]    = argmax_v logit[m][v] (equal logits: lower v); max_logit[m] = that logit
 * The V x H matrix is streamed once per call for all M rows.
 *   M 1..8; H a multiple of 256 up to 4096; V a multiple of 64, 64..2^30
 *   x bf16 [M][H]; w FP8 codes [V][H]; w_s fp32 [V]; token int32 [M];
 *   max_logit fp32 [M] or NULL; workspace >= lm_head_argmax_workspace(M, H, V) bytes
 */
int lm_head_argmax(int M, int H, int V, const uint16_t *x, const uint8_t *w, const float *w_s,
                   int32_t *token, float *max_logit, void *workspace, size_t workspace_bytes,
                   void *stream);

/*
 * lm_head_argmax with bf16 weights (the precision ladder's BF16 rung; page "LLM decoding",
 * "Lever 1: fewer bytes" and "The ladder, every rung"): logit[m][v] = sum_c w[v][c] x[m][c],
 * no scales; otherwise as lm_head_argmax (same workspace size). w bf16 [V][H].
 */
int lm_head_argmax_bf16(int M, int H, int V, const uint16_t *x, const uint16_t *w, int32_t *token,
                        float *max_logit, void *workspace, size_t workspace_bytes, void *stream);

/* Bytes of workspace lm_head_spec_sample needs (0 for invalid sizes). */
size_t lm_head_spec_sample_workspace(int max_M, int H, int V);

/*
 * The verify step's lm_head with stochastic speculative acceptance at temperature T > 0
 * (page "LLM decoding", "What we learned, and where this goes": a drafted token is kept
 * only if it passes the exact distribution the target would have sampled from, so the
 * output is distributed as ordinary decoding; the temperature-0.7 column of the table
 * "The ladder, every rung"). The page does not spell out the procedure; the standard
 * speculative sampling rule is taken:
 *   logit[i][v] = w_s[v] * sum_c decode(w[v][c]) * x[i][c]     (as lm_head_argmax)
 *   p_i         = softmax(logit[i] / T), rows i = 0..gamma (gamma = M - 1)
 *   d_i (i = 1..gamma) is accepted iff u_accept[i-1] * q[i-1][d_i] < p_{i-1}(d_i),
 *                 i.e. with probability min(1, p/q); ids outside [0, V) are rejected;
 *                 n = the number of leading accepted drafts
 *   the last token t is drawn from r = max(0, p_n - q[n]) when n < gamma (the residual;
 *                 p_n itself if r is zero everywhere), else from r = p_gamma (the bonus),
 *                 by the Gumbel-max rule t = argmax_{v: r_v > 0} log r_v - log(-log U_v)
 *                 (equal values: lower v), with U_v = (W + 1/2) / 2^32 where W is word
 *                 v % 4 of Philox4x32-10 (Salmon et al., SC 2011) on the counter
 *                 (v / 4, n, step low, step high) under the key (seed low, seed high)
 *   accepted_len = n; out_tokens = d_1 .. d_n, t, then -1.
 * Given the same uniforms the result is a deterministic function of the inputs.
 *   M 1..8; H a multiple of 256 up to 4096; V a multiple of 64, 64..2^24; temperature > 0
 *   x bf16 [M][H]; w FP8 codes [V][H]; w_s fp32 [V]
 *   draft int32 [M-1]; q fp32 [M-1][V] (q[i-1] is the drafter's distribution that proposed
 *   d_i); u_accept fp32 [M-1] in [0, 1); draft, q and u_accept may be NULL when M == 1
 *   accepted_len int32 [1]; out_tokens int32 [M]
 *   workspace >= lm_head_spec_sample_workspace(M, H, V) bytes, 256-byte aligned
 */
int lm_head_spec_sample(int M, int H, int V, const uint16_t *x, const uint8_t *w, const float *w_s,
                        float temperature, const int32_t *draft, const float *q,
                        const float *u_accept, uint64_t seed, uint64_t step,
                        int32_t *accepted_len, int32_t *out_tokens, void *workspace,
                        size_t workspace_bytes, void *stream);

/*
 * lm_head_argmax for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same kernels and
 * results, with the scratch held in a static device array of the library instead of a
 * caller workspace. Arguments as lm_head_argmax (without the workspace).
 *   - The static scratch is 128 KiB per device, enough for every valid M and V; a call
 *     needing more returns MOE_EWORKSPACE. Each device keeps its copy until the process
 *     ends; its address is looked up on the first call on that device (with that device
 *     current), which is the only call that touches the HIP runtime beyond launching.
 *   - Allocates nothing (no hipMalloc, no allocating library routine).
 *   - Every call on a device shares that device's scratch, which keeps the last call's
 *     contents (every value read is written first by the same call): calls that
 *     overlap on one device, on different streams or from different threads, race.
 */
int lm_head_argmax_noalloc(int M, int H, int V, const uint16_t *x, const uint8_t *w,
                           const float *w_s, int32_t *token, float *max_logit, void *stream);

/*
 * Greedy speculative acceptance (page "LLM decoding", "Lever 2: fewer passes" and
 * "What we learned": a drafted token is kept only if it is the token the target
 * itself produces, so the output equals ordinary greedy decoding).
 *   draft   int32 [num_draft]      d_1..d_gamma (gamma = num_draft, 0..7)
 *   target  int32 [num_draft + 1]  t_0..t_gamma, the target's argmax at each verify row
 *   accepted_len int32 [1]: n = the largest j <= gamma with d_i == t_{i-1} for all i <= j
 *   out_tokens   int32 [num_draft + 1]: t_0..t_n (the n accepted drafts and the bonus
 *                token t_n), then -1
 * Draft ids outside the vocabulary simply never match. draft may be NULL when
 * num_draft == 0.
 */
int spec_accept(int num_draft, const int32_t *draft, const int32_t *target,
                int32_t *accepted_len, int32_t *out_tokens, void *stream);

/*
 * Residual add and RMSNorm between layers of the stacked step (attention is not
 * part of this step; a stacked workload adds noise in its place):
 *   h_out[m][c] = bf16(h_in[m][c] + add0[m][c] + add1[m][c])      (add1 may be NULL)
 *   u_out[m][c] = bf16(h_out[m][c] * rsqrt(mean_c h_out[m][c]^2 + eps) * gain[c])
 *   M 1..8; H a multiple of 256 up to 4096; all tensors bf16 [M][H] (gain [H]);
 *   h_out may equal h_in (in place); u_out must not alias the inputs.
 */
int moe_add_rmsnorm(int M, int H, const uint16_t *h_in, const uint16_t *add0,
                    const uint16_t *add1, const uint16_t *gain, float eps, uint16_t *h_out,
                    uint16_t *u_out, void *stream);

/*
 * Diagnostic: decode n FP8 E4M3FN codes with the two conversions the GEMV kernels
 * use (codes -> bf16 pairs for the bf16 dot products; codes -> fp32 pairs for the
 * fp32 FMAs) and write both as fp32. n a multiple of 4, 4..2^20; codes, out_via_bf16,
 * out_via_f32 16-byte aligned.
 */
int moe_fp8_decode(int n, const uint8_t *codes, float *out_via_bf16, float *out_via_f32,
                   void *stream);

/*
 * Diagnostic: the streaming-read rate a kernel of this library gets from HBM, the
 * practical ceiling to set beside the nominal 8 TB/s. Reads `bytes` bytes from src once,
 * with 16-byte loads carrying the nontemporal hint (as the library's weight streams do)
 * spread over MOE_PROBE_GRID workgroups of 256 threads, and folds them into one word per
 * workgroup (sink[w] = XOR of the 32-bit words workgroup w read), so that the loads are
 * kept. bytes a positive multiple of 16; src and sink 16-byte aligned; sink holds
 * MOE_PROBE_GRID words. Asynchronous on `stream`.
 */
#define MOE_PROBE_GRID 8192
int moe_hbm_read_probe(const void *src, size_t bytes, uint32_t *sink, void *stream);

/* ------------------------------------------------------------------------------
 * The whole stacked decode step in one launch.
 *
 * num_layers MoE layers, each preceded by a residual add and RMSNorm, then the
 * final norm, the tied lm_head with argmax and greedy acceptance:
 *   h_0 = bf16(x + noise_0),                  u_0 = rmsnorm(h_0; gain_0)
 *   y_l = moe_layer_l(u_l)                     (as moe_decode_layer)
 *   h_l = bf16(h_{l-1} + noise_l + y_{l-1}),   u_l = rmsnorm(h_l; gain_l)   (l >= 1)
 *   h_L = bf16(h_{L-1} + y_{L-1}),             x_f = rmsnorm(h_L; gain_L)
 *   token[m] = argmax_v logit(x_f[m])[v];      (n, out) = spec_accept(draft, token)
 * rmsnorm(h; g) = bf16(h * rsqrt(mean(h^2) + eps) * g). (Attention is not part of
 * this step; the stacked workload adds noise in its place.)
 *
 * The step runs as one kernel of persistent workgroups. Per layer, router workgroups
 * form the logits; every other workgroup selects the top K itself and takes its share
 * of the layer's units (8-row gate/up blocks, 64-row down blocks, 64-row combine
 * blocks) in a fixed order; then every workgroup streams a share of the lm_head.
 * Data passes between workgroups in tagged device-memory words, each polled until its
 * tag is the current step's. Every weight byte the step needs is read once. y_l[m] is
 * summed as in moe_decode_layer: token m's routed experts in ascending id, then the
 * shared expert (whose down rows are split into column segments when it is wider
 * than 704, each segment a separate term, in order). The shape must satisfy
 * hidden <= 2816 and expert_width <= 704 (one 704-column down row per unit); wider
 * layers are rejected with MOE_EINVAL.
 *
 * Co-residency: every workgroup of the step waits on other workgroups, so all of them
 * must be resident at once. The grid is sized to the kernel's occupancy on the device
 * (a grid that cannot fit returns MOE_EUNSUPPORTED). With MOE_STEP_COOPERATIVE in
 * flags, and outside stream capture, the step is launched cooperatively: the runtime
 * starts it only with every workgroup resident (about 27 us more per step on MI355X,
 * for callers that share the device with other work). Otherwise, and always inside
 * capture, it is a plain launch that relies on nothing else occupying the device. In
 * every case each device-side wait is bounded (spin_limit polls) and, once one gives
 * up, the others give up within a few hundred polls: a step that cannot make progress
 * ends quickly, its results invalid and the timeout recorded for
 * moe_decode_step_status; it never hangs and never reports wrong results as valid.
 * ---------------------------------------------------------------------------- */

typedef struct moe_step_desc {
    moe_layer_desc layer;   /* shape of every layer (wtype MOE_W_FP8_E4M3; hidden <= 2816)   */
    int num_layers;         /* L, 1..64                                                        */
    int vocab;              /* V, a multiple of 64, 64..2^30                                   */
    int max_tokens;         /* largest M the workspace serves, 1..8                            */
    float eps;              /* RMSNorm epsilon, >= 0                                           */
    unsigned spin_limit;    /* polls of a device-side wait before it gives up and flags a
                               timeout (0: a default of about a quarter second)                    */
    unsigned flags;         /* MOE_STEP_* bits                                                 */
} moe_step_desc;

#define MOE_STEP_COOPERATIVE 1u   /* launch cooperatively outside stream capture (see above) */
#define MOE_STEP_LM_BF16 2u       /* lm_w holds bf16 [V][H] weights without scales (lm_s unused,
                                     may be NULL): the precision ladder's BF16 lm_head */

/* Bytes of workspace for moe_decode_step (0 if desc is invalid). */
size_t moe_decode_step_workspace(const moe_step_desc *desc);

/*
 * Prepare a workspace for moe_decode_step (synchronous; not capturable). Validates
 * the L weight sets in `layers` (a HOST array of moe_layer_weights holding device
 * pointers, checked as in moe_decode_layer), zeroes the workspace and copies the
 * weight table into it. Call again if any weight pointer changes.
 */
int moe_decode_step_prepare(const moe_step_desc *desc, const moe_layer_weights *layers,
                            void *workspace, size_t workspace_bytes);

/*
 * One stacked decode step for M tokens (1 <= M <= desc->max_tokens), asynchronous on
 * `stream` and capturable. Concurrent steps must use distinct workspaces.
 *   gains      bf16 [L+1][H]            lm_w FP8 [V][H], lm_s fp32 [V] (MOE_STEP_LM_BF16: lm_w
 *                                       bf16 [V][H], lm_s unused)
 *   x          bf16 [M][H]              noise bf16 [L][M][H]
 *   draft      int32 [M-1] (NULL when M == 1)
 *   token      int32 [M]; max_logit fp32 [M] or NULL; accepted_len int32 [1];
 *   out_tokens int32 [M] (as spec_accept)
 *   y_layers   bf16 [L][M][H], every layer's MoE output y_l, or NULL
 *   topk_idx   int32 [L][M][K] or NULL; topk_w fp32 [L][M][K] or NULL
 *   x_final    bf16 [M][H], the lm_head input, or NULL
 */
int moe_decode_step(const moe_step_desc *desc, int M, const uint16_t *gains,
                    const uint8_t *lm_w, const float *lm_s, const uint16_t *x,
                    const uint16_t *noise, const int32_t *draft, int32_t *token,
                    float *max_logit, int32_t *accepted_len, int32_t *out_tokens,
                    uint16_t *y_layers, int32_t *topk_idx, float *topk_w, uint16_t *x_final,
                    void *workspace, size_t workspace_bytes, void *stream);

/*
 * Synchronous: MOE_OK, or MOE_ETIMEOUT if a device-side wait of a step run on this
 * workspace since the last call gave up (its results, and those of later steps up to
 * this call, are then invalid). After a timeout it clears the flag and moves the
 * workspace's step counter past every tag a hand-off word can hold, so the next step
 * runs normally. Call after the stream has been synchronised, with no step in flight.
 */
int moe_decode_step_status(const moe_step_desc *desc, void *workspace);

/* ------------------------------------------------------------------------------
 * The MTP drafter's step (page "LLM decoding", "The one-line shape bug that disabled the
 * model's own drafter": a pre_projection from 5632 = 2 x 2816 inputs, the target's
 * embedding of the token and a hidden state, down to the head's 1024-wide width, and the
 * head's own 1024-wide embedding table; "Lever 2: fewer passes": a 430M head proposes the
 * tokens the target verifies). The head's body is not on the page; the reading taken is a
 * stack of dense GELU-gated blocks at the head's width (pre-RMSNorm, residual), a final
 * RMSNorm, the head's own table for the draft's argmax, and a post-projection back to the
 * target's width for the next draft's hidden state. Per draft i = 1..gamma, from the
 * previous token t (t_0 = *tok0) and hidden state g (g_0 = hidden0):
 *   e   = bf16(emb_s[t] * decode(emb_w[t]))                 (the product exact, one rounding)
 *   z   = bf16(pre_w [e | g])                                [width] from [2 hidden]
 *   for b < blocks: u = rmsnorm(z; gains[b]), z = bf16(z + down_b(gelu_tanh(gate_b u) * up_b u))
 *   zf  = rmsnorm(z; gains[blocks]);  drafts[i-1] = argmax_v table_s[v] (table_w[v] . zf)
 *   g   = bf16(post_w zf)                                    [hidden], for the next draft
 * Every matrix is FP8 E4M3FN with per-row fp32 scales applied after the dot product; the
 * argmax breaks ties to the lower id. The drafted tokens stay on the device (each draft
 * reads the previous one from `drafts`), so the call is asynchronous and capturable.
 * ---------------------------------------------------------------------------- */
typedef struct moe_draft_desc {
    int hidden;   /* the target's width (2816): a multiple of 256, at most 4096            */
    int width;    /* the head's width (1024): a multiple of 256 up to 2048, or of 512 up
                     to 4096                                                              */
    int ffn;      /* the blocks' inner width: a multiple of 256 up to 4096, of 512 up to
                     8192, or of 1024 up to 16384                                         */
    int blocks;   /* 0..64                                                                  */
    int vocab;    /* a multiple of 64, 64..2^30                                             */
    float eps;    /* RMSNorm epsilon, >= 0                                                  */
    unsigned flags;       /* MOE_DRAFT_* bits (0 when zero-initialised)                     */
    unsigned spin_limit;  /* polls before a device-side wait of the one-launch form gives up
                             (0: the library's default, about a quarter second)             */
} moe_draft_desc;

#define MOE_DRAFT_CHAIN 1u   /* always run the chain of launches, never the one-launch form  */

typedef struct moe_draft_weights {     /* device pointers, 16-byte aligned                  */
    const uint8_t *pre_w;   const float *pre_s;    /* [width][2 hidden], [width]            */
    const uint8_t *gate_w;  const float *gate_s;   /* [blocks][ffn][width], [blocks][ffn]   */
    const uint8_t *up_w;    const float *up_s;     /* [blocks][ffn][width], [blocks][ffn]   */
    const uint8_t *down_w;  const float *down_s;   /* [blocks][width][ffn], [blocks][width] */
    const uint16_t *gains;                         /* bf16 [blocks + 1][width]              */
    const uint8_t *table_w; const float *table_s;  /* [vocab][width], [vocab]               */
    const uint8_t *post_w;  const float *post_s;   /* [hidden][width], [hidden]             */
} moe_draft_weights;

/* Bytes of workspace moe_draft_step needs (0 if desc is invalid). */
size_t moe_draft_step_workspace(const moe_draft_desc *desc);

/*
 * gamma drafts (1..7) of the head above. tok0 int32 [1] and hidden0 bf16 [hidden] are
 * device arrays (the target's last token and its hidden state); emb_w FP8 [vocab][hidden]
 * with emb_s fp32 [vocab] is the target's tied embedding table (the lm_head); drafts
 * int32 [gamma]. Asynchronous on `stream` and capturable. The workspace (at least
 * moe_draft_step_workspace(desc) bytes, 256-byte aligned) is zero-filled before its first
 * use and then left to the library: it keeps a call counter and tagged hand-off words
 * between calls, and concurrent calls must use distinct workspaces.
 * Heads with width <= 1024, ffn <= 8192 and pieces that fit its register budget (the
 * 430M head among them) run as ONE launch of 512 co-resident workgroups on a device that
 * holds them (two per compute unit on MI355X), unless MOE_DRAFT_CHAIN is set: the
 * workgroups pass z, the blocks' inner vectors, g and their argmax keys to one another
 * through tagged words in the workspace, with bounded waits (see moe_draft_step_status).
 * Like moe_decode_step, it relies on the caller not running other work on the device
 * meanwhile. Other heads, and other devices, run a short chain of launches per draft.
 * Both forms compute the formulas above; they may differ in the last bits of fp32 sums.
 */
int moe_draft_step(const moe_draft_desc *desc, const moe_draft_weights *w, int gamma,
                   const int32_t *tok0, const uint16_t *hidden0, const uint8_t *emb_w,
                   const float *emb_s, int32_t *drafts, void *workspace, size_t workspace_bytes,
                   void *stream);

/*
 * Synchronous: MOE_OK, or MOE_ETIMEOUT if a device-side wait of a one-launch drafter call
 * on this workspace gave up since the last status call (those calls' drafts are then
 * invalid). It then clears the flag and moves the workspace's call counter past every
 * tag a hand-off word can hold, so the next call runs normally. Call with no drafter call
 * in flight on the workspace.
 */
int moe_draft_step_status(const moe_draft_desc *desc, void *workspace);

/* ------------------------------------------------------------------------------
 * Attention decode with a KV cache (page "LLM decoding", "The exact architecture": 25
 * sliding-window layers and 5 global ones, grouped-query attention, a 256K context;
 * "Where the 7.36 GB goes": the q/k/o projections, about 966M parameters, 26.3 % of the
 * bytes, KV-cache reads not counted; "Lever 1" and "What we learned": an FP8 KV cache
 * halves the KV reads). The page names q, k and o projections and no v projection: the
 * reading taken is that the cached key is also the value, with 16 query heads of 256 and
 * 8 KV heads on sliding layers and 16 query heads of 512 and 2 KV heads on global ones,
 * which gives the page's 966,000,640 parameters exactly. No positional rotation is
 * applied (none is on the page; it would add arithmetic, not bytes), and the score scale
 * is 1/sqrt(head_dim). Per layer, for tokens m = 0..M-1 at positions pos + m:
 *   q_m  = bf16(q_s * (q_w u_m))                 [q_heads * head_dim]
 *   k_m  = bf16(k_s * (k_w u_m))                 [kv_heads * head_dim], appended to the cache
 *   for query head h (KV head g = h / (q_heads / kv_heads)), over the positions
 *   p in [lo_m, pos + m], lo_m = window ? max(0, pos + m - window + 1) : 0:
 *        s_p  = (q_m,h . K_g[p]) / sqrt(head_dim);  w = softmax(s)
 *        o_m,h = bf16(sum_p w_p K_g[p])          (the cached key is the value)
 *   out_m = bf16(o_s * (o_w o_m))                [hidden]
 * K_g[p] is the cached key as stored: bf16, or FP8 E4M3FN codes times a per-(position,
 * head) fp32 scale.
 * ---------------------------------------------------------------------------- */
enum {
    MOE_KV_BF16 = 0,   /* cache: bf16 [kv_heads][capacity][head_dim]                            */
    MOE_KV_FP8 = 1     /* cache: FP8 codes [kv_heads][capacity][head_dim], then fp32 scales
                          [kv_heads][capacity] at offset align256(kv_heads * capacity *
                          head_dim); a row's scale is max|k| / 448 (fp32) and its codes are
                          k / scale (fp32 division) rounded to nearest even, saturating at
                          448; an all-zero row has scale 0                                      */
};

typedef struct moe_attn_desc {
    int hidden;       /* model width (2816): a multiple of 256, at most 4096                    */
    int q_heads;      /* 1..64, a multiple of kv_heads                                          */
    int kv_heads;     /* 1..64; q_heads / kv_heads query heads share a KV head (at most 16)     */
    int head_dim;     /* 128, 256 or 512; q_heads * head_dim at most 16384                      */
    int window;       /* sliding window in positions (1024 on sliding layers), 0 for global;
                         at most 2^24                                                          */
    int capacity;     /* cache positions, 1..2^24; position p lives in slot p mod capacity. Sliding:
                         capacity >= window + 7 (the ring holds every token's window); global:
                         every call needs pos + M <= capacity                                  */
    int kv_type;      /* MOE_KV_BF16 or MOE_KV_FP8                                              */
} moe_attn_desc;

typedef struct moe_attn_weights {      /* device pointers, 16-byte aligned; FP8 E4M3FN codes
                                          with per-row fp32 scales                             */
    const uint8_t *q_w; const float *q_s;   /* [q_heads * head_dim][hidden], [q_heads * head_dim] */
    const uint8_t *k_w; const float *k_s;   /* [kv_heads * head_dim][hidden], [kv_heads * head_dim] */
    const uint8_t *o_w; const float *o_s;   /* [hidden][q_heads * head_dim], [hidden]            */
} moe_attn_weights;

/* Bytes of one layer's KV cache for desc (0 if desc is invalid). */
size_t moe_kv_cache_bytes(const moe_attn_desc *desc);

/*
 * Write keys of n positions first_pos .. first_pos + n - 1 into the cache (slot p mod
 * capacity), quantising to FP8 for MOE_KV_FP8 exactly as the decode call does for the keys
 * it appends. k bf16 [n][kv_heads][head_dim]; 1 <= n; first_pos >= 0. This is how a
 * context is placed in the cache (prefill itself is not part of this library).
 * Asynchronous on `stream`.
 */
int moe_kv_cache_write(const moe_attn_desc *desc, int first_pos, int n, const uint16_t *k, void *cache,
                       void *stream);

/* Bytes of workspace moe_attn_decode needs for up to max_M tokens (0 if invalid). */
size_t moe_attn_decode_workspace(const moe_attn_desc *desc, int max_M);

/*
 * One layer's attention for M tokens (1..8) at positions pos .. pos + M - 1 (the decode
 * step at M = 1, the speculative verify step at M = gamma + 1; each token attends to the
 * others before it), as defined above. Positions below pos must already be in the cache
 * (the last `window` of them on sliding layers); the call appends the M new keys.
 *   u      bf16 [M][hidden], the (already normalised) layer input
 *   cache  moe_kv_cache_bytes(desc) bytes, 256-byte aligned
 *   out    bf16 [M][hidden], the attention branch output (the residual is NOT added)
 *   o      bf16 [M][q_heads * head_dim], the heads' outputs before o_w, or NULL
 * Asynchronous on `stream`, four launches (q/k projection and append, per-chunk partial
 * softmax, combine, o projection); capturable.
 */
int moe_attn_decode(const moe_attn_desc *desc, const moe_attn_weights *w, int M, int pos, const uint16_t *u,
                    void *cache, uint16_t *out, uint16_t *o, void *workspace, size_t workspace_bytes,
                    void *stream);

/* A static string describing a moe_status value. */
const char *moe_strerror(int status);

#ifdef __cplusplus
}
#endif
#endif /* MOE_DECODE_H */
