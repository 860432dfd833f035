/*
 * Host sanitizer driver for the oracle (test infrastructure): built together with
 * oracle/oracle.c under AddressSanitizer and UndefinedBehaviorSanitizer by
 * tests/test_sanitizers.py. Every buffer is its own heap block of exactly the size the
 * function's contract states, so a read or write past any extent, a use after free or
 * a leak is reported; the inputs cover the edge cases of each function (K == E, V == 1,
 * gamma == 0, M == 8, out-of-range draft ids, ties, NULL optional arguments). A few
 * invariants are checked as well; the exit status is nonzero if one fails.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double oracle_fp8_e4m3(uint8_t code);
double oracle_bf16(uint16_t bits);
uint16_t oracle_bf16_round(double v);
double oracle_gelu_tanh(double z);
void oracle_router(int M, int H, int E, int K, const uint16_t *u, const uint16_t *W, const float *bias,
                   double *logits, int32_t *idx, double *wts, double *gap);
void oracle_router_fp8(int M, int H, int E, int K, const uint16_t *u, const uint8_t *W8, const float *s,
                       const float *bias, double *logits, int32_t *idx, double *wts, double *gap);
void oracle_moe_layer(int M, int H, int E, int K, int D, int Ds, int wtype, const uint16_t *u,
                      const void *router_w, const float *router_s, const float *router_b, const void *G, const void *U,
                      const void *Dn, const float *gs, const float *us, const float *ds, const void *shG,
                      const void *shU, const void *shD, const float *shgs, const float *shus,
                      const float *shds, int32_t *idx, double *wts, double *gap, double *logits, double *y,
                      uint16_t *y_bf16);
void oracle_lm_head(int M, int H, int V, const uint16_t *x, const uint8_t *Q, const float *s, int32_t *tok,
                    double *max_logit, double *gap);
void oracle_lm_head_bf16(int M, int H, int V, const uint16_t *x, const uint16_t *W, int32_t *tok,
                         double *max_logit, double *gap);
void oracle_lm_head_rows(int M, int H, int nrows, const int32_t *rows, const uint16_t *x, const uint8_t *Q,
                         const float *s, double *out);
int oracle_spec_accept(int gamma, const int32_t *draft, const int32_t *target, int32_t *out);
void oracle_gemv_fp8(int N, int K, const uint8_t *Q, const float *s, const uint16_t *x, double *out);
void oracle_dense_mlp(int H, int F, const uint16_t *u, const uint8_t *G, const uint8_t *U, const uint8_t *Dn,
                      const float *sg, const float *su, const float *sd, double *o);
void oracle_bf16_round_n(int n, const double *v, uint16_t *out);
void oracle_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]);
double oracle_sample_uniform(uint64_t seed, uint64_t step, int row, int v);
void oracle_lm_head_logits(int M, int H, int V, const uint16_t *x, const uint8_t *Q, const float *s,
                           double *out);
int oracle_spec_sample(int M, int V, const double *logits, double T, const int32_t *draft, const float *q,
                       const float *u_acc, uint64_t seed, uint64_t step, int32_t *out, double *acc_margin,
                       double *samp_margin);
void oracle_add_rmsnorm(int M, int H, const uint16_t *h, const uint16_t *a0, const uint16_t *a1,
                        const uint16_t *g, double eps, uint16_t *h_out, uint16_t *u_out);
int oracle_num_threads(void);
void oracle_set_num_threads(int n);

static uint64_t rs = 0x9E3779B97F4A7C15ull;
static uint32_t rnd(void) {
    rs ^= rs << 13;
    rs ^= rs >> 7;
    rs ^= rs << 17;
    return (uint32_t)(rs >> 16);
}
static double unif(void) { return (rnd() + 0.5) / 4294967296.0; }
static double normal(double sd) { return sd * sqrt(-2.0 * log(unif())) * cos(6.283185307179586 * unif()); }

static int failures = 0;
#define CHECK(c)                                                        \
    do {                                                                \
        if (!(c)) {                                                     \
            fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); \
            ++failures;                                                 \
        }                                                               \
    } while (0)

/* exact-size blocks */
static void *blk(size_t n) {
    void *p = malloc(n ? n : 1);
    if (!p) abort();
    return p;
}
static uint16_t *bf16s(size_t n, double sd) {
    uint16_t *p = blk(n * 2);
    for (size_t i = 0; i < n; ++i) p[i] = oracle_bf16_round(normal(sd));
    return p;
}
static uint8_t *codes(size_t n) {
    uint8_t *p = blk(n);
    for (size_t i = 0; i < n; ++i) {
        uint8_t c = (uint8_t)rnd();
        p[i] = (c & 0x7f) == 0x7f ? (uint8_t)(c ^ 1u) : c; /* no NaN codes */
    }
    return p;
}
static float *scales(size_t n) {
    float *p = blk(n * 4);
    for (size_t i = 0; i < n; ++i) p[i] = (float)(1e-3 * (1.0 + unif()));
    return p;
}

static void scalars(void) {
    for (int c = 0; c < 256; ++c) {
        const double v = oracle_fp8_e4m3((uint8_t)c);
        CHECK(((c & 0x7f) == 0x7f) == (isnan(v) != 0));
    }
    const double sp[] = {0.0, -0.0, 1.0, -1.0, 1e-40, -1e-45, 3.4e38, 1e39, INFINITY, -INFINITY, NAN};
    for (size_t i = 0; i < sizeof sp / sizeof sp[0]; ++i) {
        const uint16_t b = oracle_bf16_round(sp[i]);
        if (!isnan(sp[i])) CHECK(!isnan(oracle_bf16(b)));
    }
    for (int i = 0; i < 65536; i += 7) (void)oracle_bf16((uint16_t)i);
    for (double z = -20.0; z <= 20.0; z += 0.37) CHECK(isfinite(oracle_gelu_tanh(z)));
    uint32_t ctr[4] = {0, 0, 0, 0}, key[2] = {0, 0}, out[4];
    oracle_philox4x32_10(ctr, key, out);
    for (int v = 0; v < 64; ++v) {
        const double u = oracle_sample_uniform(42, 7, v & 7, v);
        CHECK(u > 0.0 && u < 1.0);
    }
}

static void router(int M, int H, int E, int K, int with_bias) {
    uint16_t *u = bf16s((size_t)M * H, 1.0), *W = bf16s((size_t)H * E, 0.05);
    float *b = with_bias ? scales((size_t)E) : NULL;
    double *lg = blk(sizeof(double) * M * E), *w = blk(sizeof(double) * M * K), *gap = blk(sizeof(double) * M);
    int32_t *idx = blk(sizeof(int32_t) * M * K);
    oracle_router(M, H, E, K, u, W, b, lg, idx, w, gap);
    for (int m = 0; m < M; ++m) {
        double s = 0.0;
        for (int k = 0; k < K; ++k) {
            CHECK(idx[m * K + k] >= 0 && idx[m * K + k] < E);
            if (k) CHECK(idx[m * K + k] > idx[m * K + k - 1]);
            s += w[m * K + k];
        }
        CHECK(fabs(s - 1.0) < 1e-12);
        if (K == E) CHECK(isinf(gap[m]));
    }
    free(u); free(W); free(b); free(lg); free(w); free(gap); free(idx);
}

static void layer(int M, int H, int E, int K, int D, int Ds, int wtype) {
    const size_t esz = wtype == 0 ? 1 : 2;
    uint16_t *u = bf16s((size_t)M * H, 1.0), *R = bf16s((size_t)H * E, 0.05);
    void *G, *U, *Dn, *sG = NULL, *sU = NULL, *sD = NULL;
    if (wtype == 0) {
        G = codes((size_t)E * D * H); U = codes((size_t)E * D * H); Dn = codes((size_t)E * H * D);
        if (Ds) { sG = codes((size_t)Ds * H); sU = codes((size_t)Ds * H); sD = codes((size_t)H * Ds); }
    } else {
        G = bf16s((size_t)E * D * H, 0.02); U = bf16s((size_t)E * D * H, 0.02); Dn = bf16s((size_t)E * H * D, 0.02);
        if (Ds) { sG = bf16s((size_t)Ds * H, 0.02); sU = bf16s((size_t)Ds * H, 0.02); sD = bf16s((size_t)H * Ds, 0.02); }
    }
    (void)esz;
    float *gs = scales((size_t)E * D), *us = scales((size_t)E * D), *ds = scales((size_t)E * H);
    float *sgs = Ds ? scales((size_t)Ds) : NULL, *sus = Ds ? scales((size_t)Ds) : NULL, *sds = Ds ? scales((size_t)H) : NULL;
    int32_t *idx = blk(sizeof(int32_t) * M * K);
    double *w = blk(sizeof(double) * M * K), *gap = blk(sizeof(double) * M), *lg = blk(sizeof(double) * M * E);
    double *y = blk(sizeof(double) * M * H);
    uint16_t *yb = blk(2 * (size_t)M * H);
    oracle_moe_layer(M, H, E, K, D, Ds, wtype, u, R, NULL, NULL, G, U, Dn, gs, us, ds, sG, sU, sD, sgs, sus, sds, idx,
                     w, gap, lg, y, yb);
    /* the same layer with an FP8 router: codes [H][E] and per-expert scales */
    uint8_t *R8 = codes((size_t)H * E);
    float *rs = scales((size_t)E);
    oracle_moe_layer(M, H, E, K, D, Ds, wtype, u, R8, rs, NULL, G, U, Dn, gs, us, ds, sG, sU, sD, sgs, sus, sds, idx,
                     w, gap, lg, y, yb);
    free(R8);
    free(rs);
    for (int i = 0; i < M * H; ++i) CHECK(isfinite(y[i]));
    free(u); free(R); free(G); free(U); free(Dn); free(sG); free(sU); free(sD); free(gs); free(us); free(ds);
    free(sgs); free(sus); free(sds); free(idx); free(w); free(gap); free(lg); free(y); free(yb);
}

static void lm_heads(int M, int H, int V) {
    uint16_t *x = bf16s((size_t)M * H, 1.0), *Wb = bf16s((size_t)V * H, 0.02);
    uint8_t *Q = codes((size_t)V * H);
    float *s = scales((size_t)V);
    int32_t *tok = blk(sizeof(int32_t) * M);
    double *ml = blk(sizeof(double) * M), *gap = blk(sizeof(double) * M), *lg = blk(sizeof(double) * M * V);
    oracle_lm_head(M, H, V, x, Q, s, tok, ml, gap);
    for (int m = 0; m < M; ++m) {
        CHECK(tok[m] >= 0 && tok[m] < V);
        if (V == 1) CHECK(isinf(gap[m]));
    }
    oracle_lm_head_bf16(M, H, V, x, Wb, tok, ml, gap);
    oracle_lm_head_logits(M, H, V, x, Q, s, lg);
    const int nr = V < 3 ? V : 3;
    int32_t *rows = blk(sizeof(int32_t) * nr);
    for (int r = 0; r < nr; ++r) rows[r] = V - 1 - r;
    double *ro = blk(sizeof(double) * M * nr);
    oracle_lm_head_rows(M, H, nr, rows, x, Q, s, ro);
    for (int m = 0; m < M; ++m)
        for (int r = 0; r < nr; ++r) CHECK(ro[m * nr + r] == lg[(size_t)m * V + rows[r]]);
    free(x); free(Wb); free(Q); free(s); free(tok); free(ml); free(gap); free(lg); free(rows); free(ro);
}

static void accept(void) {
    for (int gamma = 0; gamma <= 7; ++gamma)
        for (int rep = 0; rep < 16; ++rep) {
            int32_t *d = gamma ? blk(sizeof(int32_t) * gamma) : NULL;
            int32_t *t = blk(sizeof(int32_t) * (gamma + 1)), *o = blk(sizeof(int32_t) * (gamma + 1));
            for (int i = 0; i <= gamma; ++i) t[i] = (int32_t)(rnd() % 4);
            for (int i = 0; i < gamma; ++i) d[i] = rep == 15 ? -5 : (int32_t)(rnd() % 4);
            const int n = oracle_spec_accept(gamma, d, t, o);
            CHECK(n >= 0 && n <= gamma && o[n] == t[n]);
            free(d); free(t); free(o);
        }
}

static void sample(int M, int V, double T) {
    double *lg = blk(sizeof(double) * M * V);
    for (int i = 0; i < M * V; ++i) lg[i] = normal(2.0);
    const int g = M - 1;
    int32_t *d = g ? blk(sizeof(int32_t) * g) : NULL;
    float *q = g ? blk(sizeof(float) * g * V) : NULL, *ua = g ? blk(sizeof(float) * g) : NULL;
    for (int i = 0; i < g; ++i) {
        d[i] = i == 2 ? V + 3 : (int32_t)(rnd() % V);   /* one id out of range */
        ua[i] = (float)unif();
        double z = 0.0;
        for (int v = 0; v < V; ++v) z += (q[(size_t)i * V + v] = (float)unif());
        for (int v = 0; v < V; ++v) q[(size_t)i * V + v] = (float)(q[(size_t)i * V + v] / z);
    }
    int32_t *o = blk(sizeof(int32_t) * M);
    double *am = g ? blk(sizeof(double) * g) : NULL, *sm = blk(sizeof(double));
    const int n = oracle_spec_sample(M, V, lg, T, d, q, ua, 1234, 5, o, am, sm);
    CHECK(n >= 0 && n <= g && o[n] >= 0 && o[n] < V);
    for (int i = n + 1; i < M; ++i) CHECK(o[i] == -1);
    free(lg); free(d); free(q); free(ua); free(o); free(am); free(sm);
}

static void dense(int H, int F) {
    uint16_t *u = bf16s((size_t)H, 1.0);
    uint8_t *G = codes((size_t)F * H), *U = codes((size_t)F * H), *Dn = codes((size_t)H * F);
    float *sg = scales((size_t)F), *su = scales((size_t)F), *sd = scales((size_t)H);
    double *o = blk(sizeof(double) * H), *g = blk(sizeof(double) * F);
    oracle_dense_mlp(H, F, u, G, U, Dn, sg, su, sd, o);
    oracle_gemv_fp8(F, H, G, sg, u, g);
    uint16_t *r = blk(2 * (size_t)F);
    oracle_bf16_round_n(F, g, r);
    free(u); free(G); free(U); free(Dn); free(sg); free(su); free(sd); free(o); free(g); free(r);
}

static void norms(int M, int H, int with_a1) {
    uint16_t *h = bf16s((size_t)M * H, 1.0), *a0 = bf16s((size_t)M * H, 0.1);
    uint16_t *a1 = with_a1 ? bf16s((size_t)M * H, 0.1) : NULL, *g = bf16s((size_t)H, 1.0);
    uint16_t *ho = blk(2 * (size_t)M * H), *uo = blk(2 * (size_t)M * H);
    oracle_add_rmsnorm(M, H, h, a0, a1, g, 1e-6, ho, uo);
    oracle_add_rmsnorm(M, H, h, a0, a1, g, 0.0, ho, uo);
    free(h); free(a0); free(a1); free(g); free(ho); free(uo);
}

int main(void) {
    oracle_set_num_threads(2);
    CHECK(oracle_num_threads() >= 1);
    scalars();
    router(1, 64, 16, 2, 0);
    router(5, 64, 16, 16, 1);   /* K == E */
    router(8, 32, 48, 6, 1);
    router(3, 16, 1, 1, 0);     /* a single expert */
    layer(1, 64, 8, 2, 16, 0, 0);
    layer(5, 64, 8, 2, 16, 32, 0);
    layer(8, 32, 6, 6, 8, 8, 1);   /* K == E, bf16 experts */
    lm_heads(1, 32, 1);            /* V == 1 */
    lm_heads(8, 64, 200);
    accept();
    sample(1, 7, 0.7);             /* gamma == 0: bonus draw only */
    sample(5, 64, 0.7);
    sample(8, 16, 2.0);
    dense(64, 96);
    norms(1, 64, 0);
    norms(8, 32, 1);
    if (failures) fprintf(stderr, "%d checks failed\n", failures);
    else printf("oracle sanitizer driver: ok\n");
    return failures ? 1 : 0;
}
