// Host sanitizer driver for the C ABI's host code (test infrastructure): api.cpp is built
// with this file under AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_sanitizers.py, without the device code: the kernel launchers below are stubs
// that count their calls and check that the workspace layout the entry point hands them
// fits the workspace the caller passed. This program runs every entry point on valid
// arguments, on each kind of invalid argument, and on a seeded sweep of descriptor values
// from edge-case pools (negative, zero, off-by-one, power-of-two and INT_MAX sizes), so
// that an overflow in the size arithmetic, an out-of-bounds access or any undefined
// behaviour in the validation is reported. It also checks the contract between the
// workspace queries and the calls: a size the query returns is accepted (one byte less is
// MOE_EWORKSPACE) and reaches the launchers; a descriptor the query rejects is
// rejected by the call and launches nothing.
#include <climits>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <initializer_list>

#include "internal.h"
#include "moe_decode.h"

static int g_calls = 0;
static size_t g_ws_bytes = 0;   // the workspace size of the call in progress
static int failures = 0;
static long n_ok = 0, n_rejected = 0;   // calls that passed validation / were rejected
#define CHECK(c)                                                             \
    do {                                                                     \
        if (!(c)) {                                                          \
            std::fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); \
            ++failures;                                                      \
        }                                                                    \
    } while (0)

namespace moe {
static int hit(size_t need) {
    ++g_calls;
    CHECK(need <= g_ws_bytes);
    return MOE_OK;
}
int launch_moe_layer(const moe_layer_desc &, const moe_layer_weights &, int, const uint16_t *, uint16_t *,
                     int32_t *, float *, char *, const LayerWs &L, void *) { return hit(L.total); }
int launch_lm_head(int M, int, int V, const uint16_t *, const uint8_t *, const float *, int32_t *, float *, char *,
                   void *) { return hit(lm_ws_bytes(M, V)); }
int launch_lm_head_logits(int, int, int, const uint16_t *, const uint8_t *, const float *, const SampleWs &L, char *,
                          void *) { return hit(L.total); }
int launch_spec_sample(int, int, float, const int32_t *, const float *, const float *, uint64_t, uint64_t, int32_t *,
                       int32_t *, const SampleWs &L, char *, void *) { return hit(L.total); }
int launch_lm_head_bf16(int M, int, int V, const uint16_t *, const uint16_t *, int32_t *, float *, char *, void *) {
    return hit(lm_ws_bytes(M, V));
}
int launch_draft_step(const moe_draft_desc &d, const moe_draft_weights &, int, const int32_t *, const uint16_t *,
                      const uint8_t *, const float *, int32_t *, char *, void *) { return hit(draft_ws(d).total); }
int launch_lm_head_noalloc(int, int, int, const uint16_t *, const uint8_t *, const float *, int32_t *, float *,
                           void *) { return hit(0); }
int launch_spec_accept(int, const int32_t *, const int32_t *, int32_t *, int32_t *, void *) { return hit(0); }
int launch_add_rmsnorm(int, int, const uint16_t *, const uint16_t *, const uint16_t *, const uint16_t *, float,
                       uint16_t *, uint16_t *, void *) { return hit(0); }
int launch_step(const moe_step_desc &, const StepWs &W, int, const uint16_t *, const uint8_t *, const float *,
                const uint16_t *, const uint16_t *, const int32_t *, int32_t *, float *, int32_t *, int32_t *,
                uint16_t *, int32_t *, float *, uint16_t *, char *, void *) { return hit(W.total); }
int launch_layer_step(const moe_layer_desc &d, const moe_layer_weights &, int M, const uint16_t *, uint16_t *,
                      int32_t *, float *, char *, void *) { return hit(layer_step_ws(d, M).total); }
int step_prepare(const StepWs &W, const moe_layer_desc &, const moe_layer_weights *, char *) { return hit(W.total); }
int step_status(const StepWs &, char *) { return hit(0); }
int draft_status(const moe_draft_desc &, char *) { return hit(0); }
int launch_fp8_decode(int, const uint8_t *, float *, float *, void *) { return hit(0); }
int launch_read_probe(const void *, size_t, uint32_t *, void *) { return hit(0); }
int launch_kv_write(const moe_attn_desc &, int, int, const uint16_t *, char *, void *) { return hit(0); }
int launch_attn_decode(const moe_attn_desc &d, const moe_attn_weights &, int M, int, const uint16_t *, char *,
                       uint16_t *, uint16_t *, char *, void *) { return hit(attn_ws(d, M).total); }
}  // namespace moe

// Device pointers are never dereferenced by the host code: distinct fake aligned addresses.
static char *fake(int i) { return reinterpret_cast<char *>((uintptr_t)0x10000000u + (uintptr_t)i * 0x100000u); }

static uint64_t rs = 0x243F6A8885A308D3ull;
static uint32_t rnd() {
    rs ^= rs << 13;
    rs ^= rs >> 7;
    rs ^= rs << 17;
    return (uint32_t)(rs >> 11);
}
static const int kPool[] = {INT_MIN, -1, 0, 1, 2, 6, 7, 8, 9, 16, 63, 64, 65, 127, 128, 255, 256, 257, 512, 704, 705,
                            1024, 2048, 2112, 2304, 2816, 2817, 4096, 4097, 4352, 8192, 16384, 16385, 1 << 20,
                            1 << 24, (1 << 24) + 64, 1 << 30, (1 << 30) + 64, INT_MAX};
static int pick() {
    const int n = (int)(sizeof kPool / sizeof kPool[0]);
    return (rnd() & 3) ? kPool[rnd() % n] : (int)(rnd() % 5000) - 16;
}

static moe_layer_weights layer_w() {
    moe_layer_weights w;
    std::memset(&w, 0, sizeof w);
    const void **p = reinterpret_cast<const void **>(&w);
    for (size_t i = 0; i < sizeof w / sizeof(void *); ++i) p[i] = fake(1 + (int)i);
    w.router_bias = nullptr;
    return w;
}

// Call with `bytes` of workspace (the stubs check the layout against it) and expect `rc`; when ok, the call reached a launcher (the sampling call reaches two), else none.
#define EXPECT_CALL(expr, want) EXPECT_WS(g_ws_bytes, expr, want)
#define EXPECT_WS(bytes, expr, want)                      \
    do {                                                  \
        g_ws_bytes = (bytes);                             \
        g_calls = 0;                                      \
        const int rc_ = (expr);                           \
        CHECK(rc_ == (want));                             \
        if (rc_ == MOE_OK) CHECK(g_calls >= 1);           \
        ++(rc_ == MOE_OK ? n_ok : n_rejected);            \
        if (rc_ != MOE_OK) CHECK(g_calls == 0);           \
    } while (0)

static void layer_sweep(const moe_layer_desc &d, int M) {
    const moe_layer_weights w = layer_w();
    const size_t ws = moe_decode_layer_workspace(&d, M);
    char *x = fake(40), *y = fake(41), *WS = fake(42);
    if (ws) {
        g_ws_bytes = ws;
        EXPECT_CALL(moe_decode_layer(&d, &w, M, (uint16_t *)x, (uint16_t *)y, nullptr, nullptr, WS, ws, nullptr),
                    MOE_OK);
        EXPECT_WS(ws - 1, moe_decode_layer(&d, &w, M, (uint16_t *)x, (uint16_t *)y, nullptr, nullptr, WS, ws - 1,
                                           nullptr), MOE_EWORKSPACE);
        g_calls = 0;
        CHECK(moe_decode_layer_status(&d, WS) == MOE_OK);
    } else {
        g_ws_bytes = 0;
        g_calls = 0;
        const int rc = moe_decode_layer(&d, &w, M, (uint16_t *)x, (uint16_t *)y, nullptr, nullptr, WS,
                                        (size_t)1 << 40, nullptr);
        CHECK(rc != MOE_OK && g_calls == 0);
    }
}

static void lm_sweep(int M, int H, int V) {
    char *x = fake(50), *w = fake(51), *s = fake(52), *t = fake(53), *WS = fake(54);
    const size_t ws = lm_head_argmax_workspace(M, H, V);
    g_ws_bytes = ws;
    if (ws) {
        EXPECT_CALL(lm_head_argmax(M, H, V, (uint16_t *)x, (uint8_t *)w, (float *)s, (int32_t *)t, nullptr, WS, ws,
                                   nullptr), MOE_OK);
        EXPECT_WS(ws - 1, lm_head_argmax(M, H, V, (uint16_t *)x, (uint8_t *)w, (float *)s, (int32_t *)t, nullptr,
                                         WS, ws - 1, nullptr), MOE_EWORKSPACE);
        EXPECT_WS(ws, lm_head_argmax_bf16(M, H, V, (uint16_t *)x, (uint16_t *)w, (int32_t *)t, nullptr, WS, ws,
                                          nullptr), MOE_OK);
        EXPECT_WS(ws - 1, lm_head_argmax_bf16(M, H, V, (uint16_t *)x, (uint16_t *)w, (int32_t *)t, nullptr, WS,
                                              ws - 1, nullptr), MOE_EWORKSPACE);
        g_calls = 0;
        const int rc = lm_head_argmax_noalloc(M, H, V, (uint16_t *)x, (uint8_t *)w, (float *)s, (int32_t *)t, nullptr,
                                              nullptr);
        CHECK(rc == MOE_OK || rc == MOE_EWORKSPACE);
    } else {
        g_calls = 0;
        CHECK(lm_head_argmax(M, H, V, (uint16_t *)x, (uint8_t *)w, (float *)s, (int32_t *)t, nullptr, WS,
                             (size_t)1 << 40, nullptr) != MOE_OK);
        CHECK(lm_head_argmax_noalloc(M, H, V, (uint16_t *)x, (uint8_t *)w, (float *)s, (int32_t *)t, nullptr,
                                     nullptr) != MOE_OK);
        CHECK(g_calls == 0);
    }
    const size_t ss = lm_head_spec_sample_workspace(M, H, V);
    char *d = fake(55), *q = fake(56), *u = fake(57), *al = fake(58), *ot = fake(59);
    g_ws_bytes = ss;
    if (ss) {
        EXPECT_CALL(lm_head_spec_sample(M, H, V, (uint16_t *)x, (uint8_t *)w, (float *)s, 0.7f, (int32_t *)d,
                                        (float *)q, (float *)u, 1, 2, (int32_t *)al, (int32_t *)ot, WS, ss, nullptr),
                    MOE_OK);
        EXPECT_WS(ss - 1, lm_head_spec_sample(M, H, V, (uint16_t *)x, (uint8_t *)w, (float *)s, 0.7f, (int32_t *)d,
                                              (float *)q, (float *)u, 1, 2, (int32_t *)al, (int32_t *)ot, WS, ss - 1,
                                              nullptr), MOE_EWORKSPACE);
        EXPECT_CALL(lm_head_spec_sample(M, H, V, (uint16_t *)x, (uint8_t *)w, (float *)s, 0.0f, (int32_t *)d,
                                        (float *)q, (float *)u, 1, 2, (int32_t *)al, (int32_t *)ot, WS, ss, nullptr),
                    MOE_EINVAL);
    } else {
        g_calls = 0;
        CHECK(lm_head_spec_sample(M, H, V, (uint16_t *)x, (uint8_t *)w, (float *)s, 0.7f, (int32_t *)d, (float *)q,
                                  (float *)u, 1, 2, (int32_t *)al, (int32_t *)ot, WS, (size_t)1 << 40,
                                  nullptr) != MOE_OK && g_calls == 0);
    }
}

static void step_sweep(const moe_step_desc &sd, int M) {
    const size_t ws = moe_decode_step_workspace(&sd);
    char *WS = fake(60);
    static moe_layer_weights layers[70];
    for (auto &l : layers) l = layer_w();
    char *g = fake(61), *lw = fake(62), *ls = fake(63), *x = fake(64), *nz = fake(65), *dr = fake(66),
         *tk = fake(67), *al = fake(68), *ot = fake(69);
    if (ws) {
        g_ws_bytes = ws;
        EXPECT_CALL(moe_decode_step_prepare(&sd, layers, WS, ws), MOE_OK);
        EXPECT_WS(ws - 1, moe_decode_step_prepare(&sd, layers, WS, ws - 1), MOE_EWORKSPACE);
        const bool m_ok = M >= 1 && M <= sd.max_tokens;
        EXPECT_WS(ws, moe_decode_step(&sd, M, (uint16_t *)g, (uint8_t *)lw, (float *)ls, (uint16_t *)x, (uint16_t *)nz,
                                    M > 1 ? (int32_t *)dr : nullptr, (int32_t *)tk, nullptr, (int32_t *)al,
                                    (int32_t *)ot, nullptr, nullptr, nullptr, nullptr, WS, ws, nullptr),
                    m_ok ? MOE_OK : MOE_EINVAL);
        g_calls = 0;
        CHECK(moe_decode_step_status(&sd, WS) == MOE_OK);
    } else {
        g_ws_bytes = 0;
        g_calls = 0;
        CHECK(moe_decode_step_prepare(&sd, layers, WS, (size_t)1 << 40) != MOE_OK);
        CHECK(moe_decode_step(&sd, M, (uint16_t *)g, (uint8_t *)lw, (float *)ls, (uint16_t *)x, (uint16_t *)nz,
                              (int32_t *)dr, (int32_t *)tk, nullptr, (int32_t *)al, (int32_t *)ot, nullptr, nullptr,
                              nullptr, nullptr, WS, (size_t)1 << 40, nullptr) != MOE_OK);
        CHECK(g_calls == 0);
    }
}

static void draft_sweep(const moe_draft_desc &dd, int gamma) {
    moe_draft_weights w;
    const void **p = reinterpret_cast<const void **>(&w);
    for (size_t i = 0; i < sizeof w / sizeof(void *); ++i) p[i] = fake(80 + (int)i);
    const size_t ws = moe_draft_step_workspace(&dd);
    char *t = fake(95), *h = fake(96), *e = fake(97), *s = fake(98), *out = fake(99), *WS = fake(100);
    if (ws) {
        g_ws_bytes = ws;
        const bool g_ok = gamma >= 1 && gamma <= 7;
        EXPECT_CALL(moe_draft_step(&dd, &w, gamma, (int32_t *)t, (uint16_t *)h, (uint8_t *)e, (float *)s,
                                   (int32_t *)out, WS, ws, nullptr), g_ok ? MOE_OK : MOE_EINVAL);
        if (g_ok)
            EXPECT_WS(ws - 1, moe_draft_step(&dd, &w, gamma, (int32_t *)t, (uint16_t *)h, (uint8_t *)e, (float *)s,
                                             (int32_t *)out, WS, ws - 1, nullptr), MOE_EWORKSPACE);
        g_calls = 0;
        CHECK(moe_draft_step_status(&dd, WS) == MOE_OK && g_calls == 1);
        CHECK(moe_draft_step_status(&dd, nullptr) == MOE_EWORKSPACE && moe_draft_step_status(&dd, WS + 16) ==
              MOE_EWORKSPACE && g_calls == 1);
    } else {
        g_ws_bytes = 0;
        g_calls = 0;
        CHECK(moe_draft_step(&dd, &w, gamma, (int32_t *)t, (uint16_t *)h, (uint8_t *)e, (float *)s, (int32_t *)out,
                             WS, (size_t)1 << 40, nullptr) != MOE_OK && g_calls == 0);
        CHECK(moe_draft_step_status(&dd, WS) != MOE_OK && g_calls == 0);
    }
}

static void attn_sweep(const moe_attn_desc &ad, int M, int pos) {
    moe_attn_weights w;
    const void **p = reinterpret_cast<const void **>(&w);
    for (size_t i = 0; i < sizeof w / sizeof(void *); ++i) p[i] = fake(110 + (int)i);
    char *u = fake(120), *cache = fake(121), *out = fake(122), *WS = fake(123);
    const size_t cb = moe_kv_cache_bytes(&ad), ws = moe_attn_decode_workspace(&ad, M);
    if (cb) {
        CHECK(moe_attn_decode_workspace(&ad, 1) > 0);
        EXPECT_WS(0, moe_kv_cache_write(&ad, pos, 3, (uint16_t *)u, cache, nullptr),
                  (pos >= 0 && pos <= INT_MAX - 3) ? MOE_OK : MOE_EINVAL);
    } else {
        g_calls = 0;
        CHECK(moe_kv_cache_write(&ad, 0, 1, (uint16_t *)u, cache, nullptr) != MOE_OK && g_calls == 0);
    }
    if (ws) {
        const bool ok = pos >= 0 && (long long)pos + M <= INT_MAX &&
                        (ad.window > 0 || (long long)pos + M <= ad.capacity);
        EXPECT_WS(ws, moe_attn_decode(&ad, &w, M, pos, (uint16_t *)u, cache, (uint16_t *)out, nullptr, WS, ws, nullptr),
                  ok ? MOE_OK : MOE_EINVAL);
        if (ok)
            EXPECT_WS(ws - 1, moe_attn_decode(&ad, &w, M, pos, (uint16_t *)u, cache, (uint16_t *)out, nullptr, WS,
                                              ws - 1, nullptr), MOE_EWORKSPACE);
    } else {
        g_calls = 0;
        CHECK(moe_attn_decode(&ad, &w, M, pos, (uint16_t *)u, cache, (uint16_t *)out, nullptr, WS, (size_t)1 << 40,
                              nullptr) != MOE_OK && g_calls == 0);
    }
}

// The one-launch drafter's geometry against what its kernel assumes (kDraftPG workgroups of
// 256 threads; a matrix of N rows of K codes at L lanes per row, R = 256 / L rows per
// workgroup, lane li holding pieces li, li + L, ... clamped to the row's last): every
// workgroup count fits the grid, the rows split evenly, the pieces cover every 16-code
// chunk of a row, the matrices whose bf16 results go out in pairs have an even R of at
// most 16 (the kernel's staging), the vectors fit its LDS arrays (x or h: 8192 words; z and
// u: 512 pairs), and the hand-off words of every draft and stage fit their workspace
// regions. Shapes that fail any of these must run the chain instead (ok false).
static void draft_geo_check(const moe_draft_desc &d) {
    using namespace moe;
    const DraftGeo g = draft_geo(d);
    if (!g.ok) return;
    const int H = d.hidden, D = d.width, F = d.ffn, B = d.blocks;
    auto matrix = [&](int N, int K, int L, int maxc, bool pairs) {
        CHECK(L >= 16 && L <= 256 && (L & (L - 1)) == 0);
        const int R = 256 / L, nc = K / 16;
        CHECK(K % 16 == 0 && N % R == 0 && N / R <= kDraftPG);
        if (pairs) CHECK(R % 2 == 0 && R <= 16);
        CHECK((nc + L - 1) / L <= maxc);   // every chunk k L + li < nc is held by some piece
        return N / R;
    };
    matrix(D, 2 * H, g.lp, kDpPreC, true);
    matrix(H, D, g.lpo, kDpPoC, true);
    if (B > 0) {
        matrix(F, D, g.lgu, kDpGuC, false);
        matrix(D, F, g.ld, kDpDnC, true);
    }
    CHECK(H <= 4096 && F <= 8192 && D / 2 <= 512 && D % 256 == 0);   // LDS arrays, 256-column table chunks
    const DraftWs W = draft_ws(d);
    const size_t G7 = kDraftMaxGamma;
    CHECK(W.ctr < W.epoch && W.epoch < W.zw && W.zw <= W.hw && W.hw <= W.gw && W.gw < W.kw);
    CHECK(W.hw - W.zw >= 8 * G7 * (size_t)(B + 1) * (size_t)(D / 2));
    CHECK(W.gw - W.hw >= 8 * G7 * (size_t)B * (size_t)F);
    CHECK(W.kw - W.gw >= 8 * G7 * (size_t)(H / 2));
    CHECK(W.total - W.kw >= 8 * G7 * (size_t)kDraftPG * 2);
    // the table: 64-row units shared out, every unit's four-row lane groups inside the vocabulary
    const int NU = d.vocab / 64;
    long covered = 0;
    for (int w = 0; w < kDraftPG; ++w) {
        const int u0 = (int)((long long)w * NU / kDraftPG), u1 = (int)((long long)(w + 1) * NU / kDraftPG);
        CHECK(u0 <= u1 && u1 <= NU);
        covered += u1 - u0;
    }
    CHECK(covered == NU);
}

static void draft_geo_sweep() {
    long n_fused = 0;
    for (int H = 256; H <= 4096; H += 256)
        for (int D = 256; D <= 2048; D += 256)
            for (int F = 256; F <= 9216; F += 256)
                for (int B : {0, 1, 12}) {
                    const moe_draft_desc d = {H, D, F, B, 64 * (1 + (H + D + F) % 997), 1e-6f, 0u, 0u};
                    draft_geo_check(d);
                    n_fused += moe::draft_geo(d).ok;
                }
    // the 430M head takes the one-launch form
    const moe_draft_desc mtp = {2816, 1024, 4096, 12, 262144, 1e-6f, 0u, 0u};
    CHECK(moe::draft_geo(mtp).ok);
    CHECK(n_fused > 1000);
}

int main() {
    draft_geo_sweep();
    // known-good shapes
    const moe_layer_desc gemma = {2816, 128, 8, 704, 704, MOE_W_FP8_E4M3};
    for (int M = 0; M <= 9; ++M) layer_sweep(gemma, M);
    moe_layer_desc wide = gemma;
    wide.shared_width = 2112;
    layer_sweep(wide, 5);
    wide.expert_width = 1024;
    layer_sweep(wide, 5);   // beyond the fused geometry: the per-layer kernels
    for (int M = 0; M <= 9; ++M) lm_sweep(M, 2816, 262144);
    moe_step_desc sd;
    std::memset(&sd, 0, sizeof sd);
    sd.layer = gemma;
    sd.num_layers = 30;
    sd.vocab = 262144;
    sd.max_tokens = 8;
    sd.eps = 1e-6f;
    for (int M = 0; M <= 9; ++M) step_sweep(sd, M);
    const moe_draft_desc mtp = {2816, 1024, 4096, 12, 262144, 1e-6f, 0u, 0u};
    for (int g = 0; g <= 8; ++g) draft_sweep(mtp, g);
    moe_draft_desc mtp_chain = mtp;
    mtp_chain.flags = MOE_DRAFT_CHAIN;
    draft_sweep(mtp_chain, 4);
    const moe_attn_desc sliding = {2816, 16, 8, 256, 1024, 1032, MOE_KV_BF16};
    const moe_attn_desc global = {2816, 16, 2, 512, 0, 32768, MOE_KV_FP8};
    for (int M = 0; M <= 9; ++M) {
        attn_sweep(sliding, M, 5000);
        attn_sweep(global, M, 32760);
    }

    // pointer checks on one entry point each: NULL -> EINVAL, misaligned -> EALIGN
    {
        const moe_layer_weights w = layer_w();
        const size_t ws = moe_decode_layer_workspace(&gemma, 1);
        g_ws_bytes = ws;
        EXPECT_CALL(moe_decode_layer(&gemma, &w, 1, nullptr, (uint16_t *)fake(2), nullptr, nullptr, fake(3), ws,
                                     nullptr), MOE_EINVAL);
        EXPECT_CALL(moe_decode_layer(&gemma, &w, 1, (uint16_t *)(fake(1) + 2), (uint16_t *)fake(2), nullptr, nullptr,
                                     fake(3), ws, nullptr), MOE_EALIGN);
        EXPECT_CALL(moe_decode_layer(&gemma, nullptr, 1, (uint16_t *)fake(1), (uint16_t *)fake(2), nullptr, nullptr,
                                     fake(3), ws, nullptr), MOE_EINVAL);
        int32_t *dr = (int32_t *)fake(4), *tg = (int32_t *)fake(5), *al = (int32_t *)fake(6), *ot = (int32_t *)fake(7);
        for (int g = -2; g <= 9; ++g)
            EXPECT_CALL(spec_accept(g, dr, tg, al, ot, nullptr), (g >= 0 && g <= 7) ? MOE_OK : MOE_EINVAL);
        EXPECT_CALL(spec_accept(2, nullptr, tg, al, ot, nullptr), MOE_EINVAL);
        EXPECT_CALL(spec_accept(0, nullptr, tg, al, ot, nullptr), MOE_OK);
        for (int n : {-4, 0, 3, 4, 8, 1 << 20, (1 << 20) + 4})
            EXPECT_CALL(moe_fp8_decode(n, (uint8_t *)fake(1), (float *)fake(2), (float *)fake(3), nullptr),
                        (n >= 4 && n % 4 == 0 && n <= (1 << 20)) ? MOE_OK : MOE_EINVAL);
        for (size_t b : {(size_t)0, (size_t)15, (size_t)16, (size_t)1 << 32})
            EXPECT_CALL(moe_hbm_read_probe(fake(1), b, (uint32_t *)fake(2), nullptr),
                        (b && b % 16 == 0) ? MOE_OK : MOE_EINVAL);
        for (int M : {0, 1, 8, 9})
            for (int H : {0, 256, 2816, 2800, 4096, 4352})
                EXPECT_CALL(moe_add_rmsnorm(M, H, (uint16_t *)fake(1), (uint16_t *)fake(2), nullptr,
                                            (uint16_t *)fake(3), 1e-6f, (uint16_t *)fake(4), (uint16_t *)fake(5),
                                            nullptr),
                            (M >= 1 && M <= 8 && H >= 256 && H % 256 == 0 && H <= 4096) ? MOE_OK : MOE_EINVAL);
    }
    for (int s = -8; s <= 1; ++s) CHECK(moe_strerror(s) != nullptr && std::strlen(moe_strerror(s)) > 0);
    CHECK(moe_strerror(INT_MIN) != nullptr && moe_strerror(INT_MAX) != nullptr);

    // seeded sweep over edge-case descriptor values
    for (int it = 0; it < 20000; ++it) {
        moe_layer_desc d = {pick(), pick(), pick(), pick(), (rnd() & 1) ? pick() : 0, (int)(rnd() % 4) - 1};
        if (rnd() & 1) {   // near-valid: perturb one field of the Gemma layer
            d = gemma;
            int *f = reinterpret_cast<int *>(&d) + rnd() % 6;
            *f = pick();
        }
        layer_sweep(d, (int)(rnd() % 11) - 1);
        lm_sweep((int)(rnd() % 11) - 1, pick(), pick());
        moe_step_desc s = sd;
        s.layer = (rnd() & 1) ? d : gemma;
        switch (rnd() % 5) {
            case 0: s.num_layers = pick(); break;
            case 1: s.vocab = pick(); break;
            case 2: s.max_tokens = (int)(rnd() % 11) - 1; break;
            case 3: s.flags = rnd() % 8; break;
            default: s.eps = (rnd() & 1) ? -1.0f : 0.0f; break;
        }
        step_sweep(s, (int)(rnd() % 11) - 1);
        moe_draft_desc dd = mtp;
        int *f = reinterpret_cast<int *>(&dd) + rnd() % 5;
        *f = pick();
        if (rnd() % 8 == 0) dd = {pick(), pick(), pick(), pick(), pick(), 1e-6f, 0u, 0u};
        if (rnd() % 8 == 0) dd.flags = (unsigned)(rnd() % 4);   // bit 1 is not a flag
        dd.spin_limit = (unsigned)rnd();
        draft_sweep(dd, (int)(rnd() % 10) - 1);
        moe_attn_desc ad = (rnd() & 1) ? sliding : global;
        int *af = reinterpret_cast<int *>(&ad) + rnd() % 7;
        *af = (rnd() % 7 == 6) ? (int)(rnd() % 3) - 1 : pick();
        attn_sweep(ad, (int)(rnd() % 11) - 1, (rnd() & 1) ? pick() : (int)(rnd() % 40000));
    }
    if (failures) std::fprintf(stderr, "%d checks failed\n", failures);
    else std::printf("ABI sanitizer driver: ok (%ld accepted calls, %ld rejected)\n", n_ok, n_rejected);
    return failures ? 1 : 0;
}
