/*
 * oracle.c -- plain, slow, fp64 CPU reference of the batch-1 fine-grained MoE
 * decode step.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg load this library. The GPU library never includes, links or
 * calls it, and it shares no source with the GPU library.
 *
 * Every routine is the plain definition written out: straight loops, fp64
 * accumulation in index order, a library sort where a sort is a step. Values
 * enter in their storage formats (bf16 bits, OCP E4M3FN code bytes, fp32
 * scales) and are decoded here from the format definitions. The only roundings
 * to a narrow type are those where the boundary stores a bf16 tensor.
 *
 * Sources (web pages; quoted by address and section):
 *  [LLMD] "LLM decoding", us-homepage.pages.dev/blog/llm-decoding
 *    - "The exact architecture, and why it rules out 4-bit": top 8 of 128 routed
 *      experts plus one always-on shared expert; expert width 704, hidden 2816,
 *      tied 262,144-row lm_head.
 *    - "Where the 7.36 GB goes": gate, up and down matrices per expert; the
 *      router; the always-on shared MLP; the lm_head read once per token.
 *    - "Lever 1: fewer bytes (FP8 weights)": FP8 weight-only storage, each
 *      weight decoded to a wider type for the math.
 *    - "Lever 2: fewer passes (native MTP)" and "What we learned": the target
 *      verifies drafted tokens in one pass and keeps exactly the tokens it would
 *      have produced itself (greedy = exact token equality).
 *  Readings where the pages are silent (gating function, activation, tie
 *  breaks, scale placement, norm form) are listed next to each routine.
 *
 * Parity pins: each routine is checked by tests against closed forms, library
 * routines (torch FP8/bf16 conversion, numpy dense evaluation), brute force and
 * invariants. "Fidelity to the real Gemma-4 numerics" is parity unpinned: the
 * pages do not give the real router function, activation or norm.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------- formats */

/* OCP 8-bit floating point E4M3FN: 1 sign, 4 exponent bits (bias 7), 3 mantissa
 * bits; exponent 0 is subnormal (m/8 * 2^-6); 0x7F/0xFF are NaN; no infinity. */
double oracle_fp8_e4m3(uint8_t code)
{
    int sign = code >> 7;
    int e = (code >> 3) & 0xF;
    int m = code & 0x7;
    double v;
    if (e == 0xF && m == 0x7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m / 8.0, -6);
    else
        v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return sign ? -v : v;
}

/* bf16 is the top half of an IEEE binary32. */
double oracle_bf16(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Round a double to the nearest bf16 (ties to even), in one rounding.
 * bf16 keeps 8 significant bits and the binary32 exponent range; below 2^-126
 * the quantum stays 2^-133 (subnormals). */
uint16_t oracle_bf16_round(double v)
{
    if (isnan(v))
        return 0x7FC0;
    double a = fabs(v);
    double r;
    if (a == 0.0) {
        r = 0.0;
    } else {
        int k;
        frexp(a, &k);              /* a = f * 2^k, f in [0.5, 1): a in [2^(k-1), 2^k) */
        int ex = k - 1;            /* unbiased exponent of a */
        if (ex < -126)
            ex = -126;
        double q = ldexp(1.0, ex - 7);       /* spacing of bf16 values near a */
        r = nearbyint(a / q) * q;            /* default rounding mode: ties to even */
        if (r >= ldexp(1.0, 128))
            r = INFINITY;
    }
    float f = (float)(v < 0 ? -r : r);       /* exact: r is a bf16 value */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

/* GELU, tanh form: 0.5 z (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3))).
 * The pages do not name the expert activation; the tanh-approximated GELU gate
 * of the workload definition is used. */
double oracle_gelu_tanh(double z)
{
    const double c = sqrt(2.0 / M_PI);
    return 0.5 * z * (1.0 + tanh(c * (z + 0.044715 * z * z * z)));
}

/* The 256 values of oracle_fp8_e4m3, tabulated once so the matrix loops below do
 * not call ldexp per element (speed only; the values are those of the routine). */
static double fp8_tab[256];
static int fp8_tab_ready;

static void fp8_tab_init(void)
{
    if (fp8_tab_ready)
        return;
    for (int c = 0; c < 256; ++c)
        fp8_tab[c] = oracle_fp8_e4m3((uint8_t)c);
    fp8_tab_ready = 1;
}

static inline double fp8(uint8_t code) { return fp8_tab[code]; }

/* Decode element i of an expert weight matrix stored as FP8 codes (wtype 0) or
 * bf16 bits (wtype 1). */
static double wget(const void *w, int wtype, size_t i)
{
    if (wtype == 0)
        return fp8(((const uint8_t *)w)[i]);
    return oracle_bf16(((const uint16_t *)w)[i]);
}

/* ------------------------------------------------------------------ router */

typedef struct { double v; int i; } vi_t;

/* Larger logit first; equal logits: lower expert id first. */
static int by_logit_desc(const void *a, const void *b)
{
    const vi_t *x = a, *y = b;
    if (x->v > y->v) return -1;
    if (x->v < y->v) return 1;
    return (x->i > y->i) - (x->i < y->i);
}

static int int_asc(const void *a, const void *b)
{
    int x = *(const int *)a, y = *(const int *)b;
    return (x > y) - (x < y);
}

/*
 * Router GEMV, softmax, top-K, renormalise ([LLMD] "The exact architecture":
 * top 8 of 128 routed experts).
 *   logits[m][e] = sum_c u[m][c] * W[c][e] (+ bias[e])     W row-major [H][E]
 *   p = softmax(logits[m]) over all E experts
 *   S = the K largest logits (ties: lower expert id)        -- softmax is monotone
 *   w_k = p_k / sum_{j in S} p_j
 * Reading: the pages do not give the gating function; softmax over all experts,
 * keep K, renormalise over the K is taken. idx is written in ascending expert id
 * with wts aligned to it. gap[m] = K-th largest logit minus (K+1)-th (INFINITY when
 * K == E): the margin of the selection decision.
 */
/* Softmax, top-K and renormalisation of one token's logits l[0..E) (the selection of
 * oracle_router; shared by the bf16 and FP8 routers). */
static void router_select(int E, int K, const double *l, vi_t *order, int *sel, int32_t *idx, double *wts,
                          double *gap)
{
    double lmax = l[0];
    for (int e = 1; e < E; ++e)
        if (l[e] > lmax) lmax = l[e];
    double z = 0.0;
    for (int e = 0; e < E; ++e)
        z += exp(l[e] - lmax);
    for (int e = 0; e < E; ++e) {
        order[e].v = l[e];
        order[e].i = e;
    }
    qsort(order, (size_t)E, sizeof(vi_t), by_logit_desc);
    for (int k = 0; k < K; ++k)
        sel[k] = order[k].i;
    *gap = (K < E) ? order[K - 1].v - order[K].v : INFINITY;
    qsort(sel, (size_t)K, sizeof(int), int_asc);
    double ps = 0.0;
    for (int k = 0; k < K; ++k)
        ps += exp(l[sel[k]] - lmax) / z;
    for (int k = 0; k < K; ++k) {
        idx[k] = sel[k];
        wts[k] = (exp(l[sel[k]] - lmax) / z) / ps;
    }
}

void oracle_router(int M, int H, int E, int K, const uint16_t *u, const uint16_t *W,
                   const float *bias, double *logits, int32_t *idx, double *wts,
                   double *gap)
{
    vi_t *order = malloc(sizeof(vi_t) * (size_t)E);
    int *sel = malloc(sizeof(int) * (size_t)K);
    for (int m = 0; m < M; ++m) {
        double *l = logits + (size_t)m * E;
        for (int e = 0; e < E; ++e) {
            double acc = 0.0;
            for (int c = 0; c < H; ++c)
                acc += oracle_bf16(u[(size_t)m * H + c]) * oracle_bf16(W[(size_t)c * E + e]);
            if (bias)
                acc += (double)bias[e];
            l[e] = acc;
        }
        router_select(E, K, l, order, sel, idx + (size_t)m * K, wts + (size_t)m * K, gap + m);
    }
    free(order);
    free(sel);
}

/*
 * The FP8 router (the precision ladder's FP8 router rung: [LLMD] "Lever 1: fewer bytes" and
 * "The ladder, every rung"): W8 holds E4M3FN codes [H][E] and s one fp32 scale per expert,
 * applied after the dot product as for the experts' rows:
 *   logits[m][e] = s[e] * sum_c u[m][c] * decode(W8[c][e]) (+ bias[e])
 * then the selection of oracle_router.
 */
void oracle_router_fp8(int M, int H, int E, int K, const uint16_t *u, const uint8_t *W8, const float *s,
                       const float *bias, double *logits, int32_t *idx, double *wts, double *gap)
{
    vi_t *order = malloc(sizeof(vi_t) * (size_t)E);
    int *sel = malloc(sizeof(int) * (size_t)K);
    fp8_tab_init();
    for (int m = 0; m < M; ++m) {
        double *l = logits + (size_t)m * E;
        for (int e = 0; e < E; ++e) {
            double acc = 0.0;
            for (int c = 0; c < H; ++c)
                acc += oracle_bf16(u[(size_t)m * H + c]) * fp8(W8[(size_t)c * E + e]);
            acc *= (double)s[e];
            if (bias)
                acc += (double)bias[e];
            l[e] = acc;
        }
        router_select(E, K, l, order, sel, idx + (size_t)m * K, wts + (size_t)m * K, gap + m);
    }
    free(order);
    free(sel);
}

/* ------------------------------------------------------------- expert FFN */

/*
 * One expert applied to one token ([LLMD] "Where the 7.36 GB goes": gate, up and
 * down matrices per expert; "Lever 1": weights decoded to a wider type, scale per
 * output channel applied after the dot product):
 *   a_j = sg[j] * sum_c G[j][c] u[c]     G row-major [F][H]
 *   b_j = su[j] * sum_c U[j][c] u[c]     U row-major [F][H]
 *   h_j = gelu_tanh(a_j) * b_j
 *   o_c = sd[c] * sum_j Dn[c][j] h_j     Dn row-major [H][F]
 * Scales are NULL for bf16 weights (factor 1).
 */
static void expert_apply(int H, int F, int wtype, const uint16_t *u,
                         const void *G, const void *U, const void *Dn,
                         const float *sg, const float *su, const float *sd,
                         double *hbuf, double *o)
{
    int j, c;
#pragma omp parallel for schedule(static)
    for (j = 0; j < F; ++j) {
        double a = 0.0, b = 0.0;
        for (int cc = 0; cc < H; ++cc) {
            double x = oracle_bf16(u[cc]);
            a += wget(G, wtype, (size_t)j * H + cc) * x;
            b += wget(U, wtype, (size_t)j * H + cc) * x;
        }
        if (sg) a *= (double)sg[j];
        if (su) b *= (double)su[j];
        hbuf[j] = oracle_gelu_tanh(a) * b;
    }
#pragma omp parallel for schedule(static)
    for (c = 0; c < H; ++c) {
        double acc = 0.0;
        for (int jj = 0; jj < F; ++jj)
            acc += wget(Dn, wtype, (size_t)c * F + jj) * hbuf[jj];
        if (sd) acc *= (double)sd[c];
        o[c] = acc;
    }
}

/*
 * One MoE layer for M tokens: router (above), then for each token
 *   y[m] = sum_{e in S_m, ascending e} w_{m,e} * expert_e(u[m]) + shared(u[m])
 * The shared expert is always on with weight 1 ([LLMD] "The exact architecture":
 * one always-on shared expert); it is not renormalised with the routed experts.
 * y is returned in fp64 and rounded once to bf16 (y_bf16), the boundary's type.
 * Expert weights: G, U [E][D][H], Dn [E][H][D]; shared [Ds][H], [Ds][H], [H][Ds]
 * (Ds == 0: no shared expert). router_w is bf16 [H][E], or FP8 codes [H][E] when
 * router_s (fp32 [E]) is given (oracle_router_fp8).
 */
void oracle_moe_layer(int M, int H, int E, int K, int D, int Ds, int wtype,
                      const uint16_t *u, const void *router_w, const float *router_s, const float *router_b,
                      const void *G, const void *U, const void *Dn,
                      const float *gs, const float *us, const float *ds,
                      const void *shG, const void *shU, const void *shD,
                      const float *shgs, const float *shus, const float *shds,
                      int32_t *idx, double *wts, double *gap, double *logits,
                      double *y, uint16_t *y_bf16)
{
    size_t esz = wtype == 0 ? 1 : 2;
    int F = D > Ds ? D : Ds;
    double *hbuf = malloc(sizeof(double) * (size_t)(F > 0 ? F : 1));
    double *o = malloc(sizeof(double) * (size_t)H);
    fp8_tab_init();
    if (router_s)
        oracle_router_fp8(M, H, E, K, u, (const uint8_t *)router_w, router_s, router_b, logits, idx, wts, gap);
    else
        oracle_router(M, H, E, K, u, (const uint16_t *)router_w, router_b, logits, idx, wts, gap);
    for (int m = 0; m < M; ++m) {
        const uint16_t *um = u + (size_t)m * H;
        double *ym = y + (size_t)m * H;
        for (int c = 0; c < H; ++c)
            ym[c] = 0.0;
        for (int k = 0; k < K; ++k) {
            int e = idx[(size_t)m * K + k];
            double w = wts[(size_t)m * K + k];
            size_t off = (size_t)e * D * H;
            expert_apply(H, D, wtype, um,
                         (const char *)G + off * esz, (const char *)U + off * esz,
                         (const char *)Dn + off * esz,
                         gs ? gs + (size_t)e * D : NULL, us ? us + (size_t)e * D : NULL,
                         ds ? ds + (size_t)e * H : NULL, hbuf, o);
            for (int c = 0; c < H; ++c)
                ym[c] += w * o[c];
        }
        if (Ds > 0) {
            expert_apply(H, Ds, wtype, um, shG, shU, shD, shgs, shus, shds, hbuf, o);
            for (int c = 0; c < H; ++c)
                ym[c] += o[c];
        }
        for (int c = 0; c < H; ++c)
            y_bf16[(size_t)m * H + c] = oracle_bf16_round(ym[c]);
    }
    free(hbuf);
    free(o);
}

/* ----------------------------------------------------------------- lm_head */

/*
 * Tied lm_head GEMV and greedy argmax ([LLMD] "Where the 7.36 GB goes": the
 * 2816 x 262,144 output projection read once per token to produce logits over the
 * whole vocabulary; the greedy (temperature 0) decoding of the measurements):
 *   logit[m][v] = s[v] * sum_c Q[v][c] x[m][c]        Q row-major [V][H] FP8
 *   tok[m] = argmax_v logit[m][v], ties: lower v
 * max_logit[m] = logit at tok; gap[m] = best minus second best (INFINITY if V == 1).
 */
void oracle_lm_head(int M, int H, int V, const uint16_t *x, const uint8_t *Q,
                    const float *s, int32_t *tok, double *max_logit, double *gap)
{
    double *lg = malloc(sizeof(double) * (size_t)V);
    fp8_tab_init();
    for (int m = 0; m < M; ++m) {
        const uint16_t *xm = x + (size_t)m * H;
        int v;
#pragma omp parallel for schedule(static)
        for (v = 0; v < V; ++v) {
            double acc = 0.0;
            for (int c = 0; c < H; ++c)
                acc += fp8(Q[(size_t)v * H + c]) * oracle_bf16(xm[c]);
            lg[v] = (double)s[v] * acc;
        }
        int best = 0;
        for (int vv = 1; vv < V; ++vv)
            if (lg[vv] > lg[best])
                best = vv;
        double second = -INFINITY;
        for (int vv = 0; vv < V; ++vv)
            if (vv != best && lg[vv] > second)
                second = lg[vv];
        tok[m] = best;
        max_logit[m] = lg[best];
        gap[m] = V > 1 ? lg[best] - second : INFINITY;
    }
    free(lg);
}

/*
 * The tied lm_head with bf16 weights (the precision ladder's BF16 rung, [LLMD] "Lever 1:
 * fewer bytes" and the table "The ladder, every rung": the same projection before FP8
 * quantisation), no scales:
 *   logit[m][v] = sum_c W[v][c] x[m][c]           W row-major [V][H] bf16
 *   tok[m] = argmax_v logit[m][v], ties: lower v; max_logit, gap as oracle_lm_head.
 */
void oracle_lm_head_bf16(int M, int H, int V, const uint16_t *x, const uint16_t *W, int32_t *tok,
                         double *max_logit, double *gap)
{
    double *lg = malloc(sizeof(double) * (size_t)V);
    for (int m = 0; m < M; ++m) {
        const uint16_t *xm = x + (size_t)m * H;
        int v;
#pragma omp parallel for schedule(static)
        for (v = 0; v < V; ++v) {
            double acc = 0.0;
            for (int c = 0; c < H; ++c)
                acc += oracle_bf16(W[(size_t)v * H + c]) * oracle_bf16(xm[c]);
            lg[v] = acc;
        }
        int best = 0;
        for (int vv = 1; vv < V; ++vv)
            if (lg[vv] > lg[best])
                best = vv;
        double second = -INFINITY;
        for (int vv = 0; vv < V; ++vv)
            if (vv != best && lg[vv] > second)
                second = lg[vv];
        tok[m] = best;
        max_logit[m] = lg[best];
        gap[m] = V > 1 ? lg[best] - second : INFINITY;
    }
    free(lg);
}

/* Logits of selected rows only: out[m][r] = s[rows[r]] * sum_c Q[rows[r]][c] x[m][c]. */
void oracle_lm_head_rows(int M, int H, int nrows, const int32_t *rows, const uint16_t *x,
                         const uint8_t *Q, const float *s, double *out)
{
    fp8_tab_init();
    for (int m = 0; m < M; ++m)
        for (int r = 0; r < nrows; ++r) {
            size_t v = (size_t)rows[r];
            double acc = 0.0;
            for (int c = 0; c < H; ++c)
                acc += fp8(Q[v * H + c]) * oracle_bf16(x[(size_t)m * H + c]);
            out[(size_t)m * nrows + r] = (double)s[v] * acc;
        }
}

/* --------------------------------------------------------- spec acceptance */

/*
 * Greedy speculative acceptance ([LLMD] "Lever 2: fewer passes": the target checks
 * the drafted tokens in one pass and keeps the ones it would have produced;
 * "What we learned": the output equals ordinary decoding).
 * draft[0..gamma-1] = d_1..d_gamma; target[0..gamma] = t_0..t_gamma, where t_i is
 * the target's token after the prefix extended by d_1..d_i.
 *   n = the largest j <= gamma with d_i == t_{i-1} for every i <= j
 *   out[0..n] = t_0..t_n (n accepted drafts, then the bonus token t_n); out[i > n] = -1
 * Returns n.
 */
int oracle_spec_accept(int gamma, const int32_t *draft, const int32_t *target, int32_t *out)
{
    int n = 0;
    while (n < gamma && draft[n] == target[n])
        ++n;
    for (int i = 0; i <= gamma; ++i)
        out[i] = i <= n ? target[i] : -1;
    return n;
}

/* ------------------------------------------------------------ drafter step */

/*
 * A dense FP8 matrix-vector product with per-row scales (the drafter's projections):
 *   out[n] = s[n] * sum_c Q[n][c] x[c]        Q row-major [N][K] FP8, x bf16 [K]
 */
void oracle_gemv_fp8(int N, int K, const uint8_t *Q, const float *s, const uint16_t *x, double *out)
{
    int n;
    fp8_tab_init();
#pragma omp parallel for schedule(static)
    for (n = 0; n < N; ++n) {
        double acc = 0.0;
        for (int c = 0; c < K; ++c)
            acc += fp8(Q[(size_t)n * K + c]) * oracle_bf16(x[c]);
        out[n] = (double)s[n] * acc;
    }
}

/* A dense GELU-gated MLP on one bf16 vector (the drafter's blocks): the expert routine
 * above with FP8 weights, o = down(gelu_tanh(gate u) * (up u)), fp64. */
void oracle_dense_mlp(int H, int F, const uint16_t *u, const uint8_t *G, const uint8_t *U, const uint8_t *Dn,
                      const float *sg, const float *su, const float *sd, double *o)
{
    double *hbuf = malloc(sizeof(double) * (size_t)F);
    fp8_tab_init();
    expert_apply(H, F, 0, u, G, U, Dn, sg, su, sd, hbuf, o);
    free(hbuf);
}

/* Round n doubles to bf16 (oracle_bf16_round element by element). */
void oracle_bf16_round_n(int n, const double *v, uint16_t *out)
{
    for (int i = 0; i < n; ++i)
        out[i] = oracle_bf16_round(v[i]);
}

/* --------------------------------------------- stochastic speculative acceptance */

/*
 * Philox4x32-10, the counter-based generator of Salmon, Moraes, Dror and Shaw,
 * "Parallel random numbers: as easy as 1, 2, 3" (SC 2011): ten rounds of two 32x32->64
 * multiplications on a 4-word counter, with a 2-word key bumped by the Weyl constants
 * between rounds. out = Philox(ctr, key).
 */
void oracle_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4])
{
    const uint64_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
    const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
    uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int r = 0; r < 10; ++r) {
        uint64_t p0 = M0 * (uint64_t)c0, p1 = M1 * (uint64_t)c2;
        uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        uint32_t n0 = hi1 ^ c1 ^ k0, n1 = lo1, n2 = hi0 ^ c3 ^ k1, n3 = lo0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
        k0 += W0;
        k1 += W1;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* The uniform draw for vocabulary entry v of target row `row` in decode step `step`
 * under `seed`: Philox4x32-10 with key (seed low, seed high) on the counter
 * (v / 4, row, step low, step high), word v % 4, mapped to (x + 1/2) / 2^32, so in (0, 1). */
double oracle_sample_uniform(uint64_t seed, uint64_t step, int row, int v)
{
    const uint32_t ctr[4] = {(uint32_t)v >> 2, (uint32_t)row, (uint32_t)step, (uint32_t)(step >> 32)};
    const uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t out[4];
    oracle_philox4x32_10(ctr, key, out);
    return ((double)out[v & 3] + 0.5) / 4294967296.0;
}

/* Full logits of the tied lm_head: out[m][v] = s[v] * sum_c Q[v][c] x[m][c] (fp64). */
void oracle_lm_head_logits(int M, int H, int V, const uint16_t *x, const uint8_t *Q, const float *s,
                           double *out)
{
    fp8_tab_init();
    for (int m = 0; m < M; ++m) {
        const uint16_t *xm = x + (size_t)m * H;
        int v;
#pragma omp parallel for schedule(static)
        for (v = 0; v < V; ++v) {
            double acc = 0.0;
            for (int c = 0; c < H; ++c)
                acc += fp8(Q[(size_t)v * H + c]) * oracle_bf16(xm[c]);
            out[(size_t)m * V + v] = (double)s[v] * acc;
        }
    }
}

/*
 * Stochastic speculative acceptance ([LLMD] "What we learned, and where this goes": a
 * drafted token is kept only if it passes the exact distribution the target would have
 * sampled from, and a rejected one falls back to a real model step, so the output is
 * distributed as ordinary decoding; the temperature-0.7 column of "The ladder, every
 * rung"). The page does not spell the procedure out; the standard speculative sampling
 * rule is taken:
 *   p_i = softmax(logits[i] / T) for target rows i = 0..gamma (row i: the token after
 *         the prefix and d_1..d_i); q_i = q + (i - 1) V, the drafter's distribution that
 *         proposed d_i (i = 1..gamma)
 *   d_i is accepted iff u_i * q_i(d_i) < p_{i-1}(d_i) (probability min(1, p/q));
 *         ids outside [0, V) are rejected; n = the number of leading accepted drafts
 *   the last token is drawn from r = max(0, p_n - q_{n+1}) if n < gamma (the residual),
 *         else from r = p_gamma (the bonus token), by the Gumbel-max rule:
 *         t = argmax over {v : r_v > 0} of log r_v - log(-log U_v), U_v =
 *         oracle_sample_uniform(seed, step, n, v); equal values: lower v. (If r is zero
 *         everywhere, p_n is used.)
 *   out = d_1 .. d_n, t, then -1; returns n.
 * Margins of the decisions (for parity against a float32 implementation), fp64:
 *   acc_margin[i-1] = |log(u_i q_i(d_i)) - log p_{i-1}(d_i)| for the decided drafts
 *   (INFINITY where it was not reached or the id is out of range);
 *   *samp_margin = best minus second-best perturbed value, less a bound on how far a
 *   float32 evaluation can move each of the two (cancellation in p - q:
 *   2^-20 (p_v + q_v) / r_v + 1e-5 per value).
 */
int oracle_spec_sample(int M, int V, const double *logits, double T, const int32_t *draft,
                       const float *q, const float *u_acc, uint64_t seed, uint64_t step,
                       int32_t *out, double *acc_margin, double *samp_margin)
{
    const int gamma = M - 1;
    double *logz = malloc(sizeof(double) * (size_t)M);
    for (int i = 0; i < M; ++i) {
        const double *l = logits + (size_t)i * V;
        double mx = -INFINITY;
        for (int v = 0; v < V; ++v)
            if (l[v] / T > mx) mx = l[v] / T;
        double z = 0.0;
        for (int v = 0; v < V; ++v)
            z += exp(l[v] / T - mx);
        logz[i] = mx + log(z);
    }
    for (int i = 0; i < gamma; ++i)
        acc_margin[i] = INFINITY;
    int n = 0;
    while (n < gamma) {
        const int d = draft[n];
        if (d < 0 || d >= V)
            break;
        const double lp = logits[(size_t)n * V + d] / T - logz[n];
        const double qd = (double)q[(size_t)n * V + d];
        const double lq = log((double)u_acc[n] * qd);
        acc_margin[n] = fabs(lq - lp);
        if (!(lq < lp))
            break;
        ++n;
    }
    const double *l = logits + (size_t)n * V;
    const float *qr = n < gamma ? q + (size_t)n * V : NULL;
    int any = 0;
    if (qr)
        for (int v = 0; v < V && !any; ++v)
            any = exp(l[v] / T - logz[n]) > (double)qr[v];
    if (!any)
        qr = NULL;
    double best = -INFINITY, second = -INFINITY, best_err = 0.0, second_err = 0.0;
    int tb = -1;
    for (int v = 0; v < V; ++v) {
        const double p = exp(l[v] / T - logz[n]);
        const double qv = qr ? (double)qr[v] : 0.0;
        const double r = p - qv;
        if (!(r > 0.0))
            continue;
        const double g = -log(-log(oracle_sample_uniform(seed, step, n, v)));
        const double val = log(r) + g;
        const double err = ldexp(p + qv, -20) / r + 1e-5;
        if (val > best) {
            second = best;
            second_err = best_err;
            best = val;
            best_err = err;
            tb = v;
        } else if (val > second) {
            second = val;
            second_err = err;
        }
    }
    *samp_margin = second == -INFINITY ? INFINITY : (best - second) - best_err - second_err;
    for (int i = 0; i < M; ++i)
        out[i] = i < n ? draft[i] : (i == n ? tb : -1);
    free(logz);
    return n;
}

/* --------------------------------------------------------- attention decode */

/*
 * E4M3FN code of an fp32 value, the FP8 KV cache's quantiser ([LLMD] "Lever 1" and "What
 * we learned": an FP8 KV cache halves the KV reads): the nearest representable value, ties
 * to the even mantissa, magnitudes from 448 up saturating to 448 (0x7E), NaN to 0x7F.
 * Written from the format: below 2^-6 the values are m 2^-9 (m = 0..7); above, 2^E (1 +
 * m/8) with E = -6..8 and m = 0..7 except m = 7 at E = 8. Both scalings are exact powers of
 * two and the rounding is the default round-to-nearest-even, so the result is a function
 * of the fp32 input alone.
 */
static uint8_t fp8_code_rne(float v)
{
    if (v != v)
        return 0x7F;
    const uint8_t sign = signbit(v) ? 0x80 : 0x00;
    const float a = fabsf(v);
    if (a >= 448.0f)
        return sign | 0x7E;
    if (a < 0.015625f) {
        const int m = (int)nearbyintf(a * 512.0f);
        return sign | (uint8_t)m;             /* m == 8 is 0x08: the smallest normal, 2^-6 */
    }
    int e;
    (void)frexpf(a, &e);                      /* a = f 2^e, f in [0.5, 1) */
    int E = e - 1;
    int r = (int)nearbyintf(ldexpf(a, 3 - E));  /* in [8, 16] */
    if (r == 16) {
        r = 8;
        E += 1;
    }
    if (E > 8 || (E == 8 && r > 14))
        return sign | 0x7E;
    return sign | (uint8_t)(((E + 7) << 3) | (r - 8));
}

uint8_t oracle_fp8_from_f32(float v) { return fp8_code_rne(v); }

/*
 * One row of the FP8 KV cache (one position of one KV head): scale = max_i |x_i| / 448 in
 * fp32, code_i = fp8_code_rne(x_i / scale) with an fp32 division; a row of zeros has scale
 * 0 and codes 0. The decoded value is decode(code) * scale.
 */
void oracle_fp8_quant_row(int n, const uint16_t *x, uint8_t *codes, float *scale)
{
    float amax = 0.0f;
    for (int i = 0; i < n; ++i)
        amax = fmaxf(amax, fabsf((float)oracle_bf16(x[i])));
    const float s = amax / 448.0f;
    *scale = s;
    for (int i = 0; i < n; ++i)
        codes[i] = s > 0.0f ? fp8_code_rne((float)oracle_bf16(x[i]) / s) : 0;
}

/*
 * One attention layer of the decode step for M tokens at positions pos .. pos + M - 1
 * ([LLMD] "The exact architecture": sliding-window and global layers, grouped-query
 * attention; "Where the 7.36 GB goes": q, k and o projections, no v projection). Readings:
 * the cached key is also the value; no positional rotation; scores scaled by
 * 1/sqrt(dh); the vectors between stages are bf16 as elsewhere in the step.
 *   q[m]   = bf16(qs * (Q_q u[m]))   [nq dh]        k[m] = bf16(ks * (Q_k u[m]))   [nkv dh]
 *   the new key of head g at position pos + m: k[m][g dh ..] (bf16 cache) or its FP8 row
 *   (oracle_fp8_quant_row) decoded (FP8 cache)
 *   head h uses KV head g = h / (nq / nkv); token m sees positions p in [lo, pos + m],
 *   lo = window > 0 ? max(0, pos + m - window + 1) : 0:
 *     s_p = (q[m][h] . K_g[p]) / sqrt(dh), w = softmax(s), o[m][h] = sum_p w_p K_g[p]
 *   o_bf16 = bf16(o); out[m] = os * (Q_o o_bf16[m]); out_bf16 = bf16(out)
 * hist holds the decoded cached keys of positions h0 .. pos - 1, [nkv][pos - h0][dh]; every
 * position a token sees below pos must be >= h0. Outputs: q_bf, k_bf (the projections),
 * k_codes [M][nkv][dh] and k_scales [M][nkv] (FP8 cache only; may be NULL otherwise), o and
 * o_bf [M][nq dh], out and out_bf [M][H]. Returns 0, or -1 if a needed position is below h0.
 */
int oracle_attn_decode(int M, int H, int nq, int nkv, int dh, int window, int pos, int kv_fp8,
                       const uint16_t *u, const uint8_t *qw, const float *qs, const uint8_t *kw,
                       const float *ks, const uint8_t *ow, const float *os, int h0, const double *hist,
                       uint16_t *q_bf, uint16_t *k_bf, uint8_t *k_codes, float *k_scales, double *o,
                       uint16_t *o_bf, double *out, uint16_t *out_bf)
{
    const int NQ = nq * dh, NK = nkv * dh, G = nq / nkv;
    fp8_tab_init();
    for (int m = 0; m < M; ++m) {
        const uint16_t *um = u + (size_t)m * H;
        int r;
#pragma omp parallel for schedule(static)
        for (r = 0; r < NQ + NK; ++r) {
            const uint8_t *row = r < NQ ? qw + (size_t)r * H : kw + (size_t)(r - NQ) * H;
            double acc = 0.0;
            for (int c = 0; c < H; ++c)
                acc += fp8(row[c]) * oracle_bf16(um[c]);
            if (r < NQ)
                q_bf[(size_t)m * NQ + r] = oracle_bf16_round((double)qs[r] * acc);
            else
                k_bf[(size_t)m * NK + (r - NQ)] = oracle_bf16_round((double)ks[r - NQ] * acc);
        }
    }
    /* the new keys as the cache holds them, decoded: [M][nkv][dh] */
    double *newk = malloc(sizeof(double) * (size_t)M * NK);
    for (int m = 0; m < M; ++m)
        for (int g = 0; g < nkv; ++g) {
            const uint16_t *kr = k_bf + (size_t)m * NK + (size_t)g * dh;
            double *dst = newk + (size_t)m * NK + (size_t)g * dh;
            if (kv_fp8) {
                uint8_t *cd = k_codes + (size_t)m * NK + (size_t)g * dh;
                float *sc = k_scales + (size_t)m * nkv + g;
                oracle_fp8_quant_row(dh, kr, cd, sc);
                for (int d = 0; d < dh; ++d)
                    dst[d] = fp8(cd[d]) * (double)*sc;
            } else {
                for (int d = 0; d < dh; ++d)
                    dst[d] = oracle_bf16(kr[d]);
            }
        }
    const int span = pos + M;
    double *sc = malloc(sizeof(double) * (size_t)span);
    int bad = 0;
    const double inv_sqrt = 1.0 / sqrt((double)dh);
    for (int m = 0; m < M && !bad; ++m)
        for (int h = 0; h < nq && !bad; ++h) {
            const int g = h / G, pm = pos + m;
            const int lo = window > 0 ? (pm - window + 1 > 0 ? pm - window + 1 : 0) : 0;
            if (lo < pos && lo < h0) {
                bad = 1;
                break;
            }
            const uint16_t *qh = q_bf + (size_t)m * NQ + (size_t)h * dh;
            double mx = -INFINITY;
            for (int p = lo; p <= pm; ++p) {
                const double *key = p < pos ? hist + ((size_t)g * (pos - h0) + (p - h0)) * dh
                                            : newk + (size_t)(p - pos) * NK + (size_t)g * dh;
                double acc = 0.0;
                for (int d = 0; d < dh; ++d)
                    acc += oracle_bf16(qh[d]) * key[d];
                sc[p] = acc * inv_sqrt;
                if (sc[p] > mx)
                    mx = sc[p];
            }
            double z = 0.0;
            for (int p = lo; p <= pm; ++p) {
                sc[p] = exp(sc[p] - mx);
                z += sc[p];
            }
            double *oh = o + (size_t)m * NQ + (size_t)h * dh;
            for (int d = 0; d < dh; ++d)
                oh[d] = 0.0;
            for (int p = lo; p <= pm; ++p) {
                const double *key = p < pos ? hist + ((size_t)g * (pos - h0) + (p - h0)) * dh
                                            : newk + (size_t)(p - pos) * NK + (size_t)g * dh;
                const double wgt = sc[p] / z;
                for (int d = 0; d < dh; ++d)
                    oh[d] += wgt * key[d];
            }
            for (int d = 0; d < dh; ++d)
                o_bf[(size_t)m * NQ + (size_t)h * dh + d] = oracle_bf16_round(oh[d]);
        }
    free(sc);
    free(newk);
    if (bad)
        return -1;
    for (int m = 0; m < M; ++m) {
        const uint16_t *om = o_bf + (size_t)m * NQ;
        int c;
#pragma omp parallel for schedule(static)
        for (c = 0; c < H; ++c) {
            double acc = 0.0;
            for (int i = 0; i < NQ; ++i)
                acc += fp8(ow[(size_t)c * NQ + i]) * oracle_bf16(om[i]);
            out[(size_t)m * H + c] = (double)os[c] * acc;
            out_bf[(size_t)m * H + c] = oracle_bf16_round(out[(size_t)m * H + c]);
        }
    }
    return 0;
}

/* ----------------------------------------------------------- residual norm */

/*
 * Residual add and RMSNorm between MoE layers (the pages omit attention; the
 * stacked workload replaces it by a residual add of noise):
 *   h'[c] = bf16(h[c] + a0[c] + a1[c])              a1 may be NULL
 *   r     = 1 / sqrt(mean_c h'[c]^2 + eps)
 *   u[c]  = bf16(h'[c] * r * g[c])
 * Reading: the gain multiplies directly (not 1 + g); one rounding of the sum.
 */
void oracle_add_rmsnorm(int M, int H, const uint16_t *h, const uint16_t *a0,
                        const uint16_t *a1, const uint16_t *g, double eps,
                        uint16_t *h_out, uint16_t *u_out)
{
    for (int m = 0; m < M; ++m) {
        size_t o = (size_t)m * H;
        double ss = 0.0;
        for (int c = 0; c < H; ++c) {
            double v = oracle_bf16(h[o + c]) + oracle_bf16(a0[o + c]);
            if (a1)
                v += oracle_bf16(a1[o + c]);
            h_out[o + c] = oracle_bf16_round(v);
            double hv = oracle_bf16(h_out[o + c]);
            ss += hv * hv;
        }
        double r = 1.0 / sqrt(ss / (double)H + eps);
        for (int c = 0; c < H; ++c)
            u_out[o + c] = oracle_bf16_round(oracle_bf16(h_out[o + c]) * r * oracle_bf16(g[c]));
    }
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads the parallel loops above use from now on (for timing the oracle). */
void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    omp_set_num_threads(n > 0 ? n : 1);
#else
    (void)n;
#endif
}
