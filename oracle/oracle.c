/*
 * CPU oracle for the routed MoE layer with decoupled top-k1/k2 weights.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no source,
 * header, table or constant with the GPU library: every constant below is
 * derived here, from the mathematics, at first use.
 *
 * Sources (the pages this follows):
 *  [P1] "Paper of the Week #3 - Half the FLOPs Is Not Half the Time"
 *       (sotaaz.com), section "The Receipt", Eq. 2, and section
 *       "Ship It - Code of the Week" (the router method).
 *  [P4] "Channel Selection for Mixture-of-Experts Decoding Needs No
 *       Calibration Data" (paperlayer.ai), section 2 "Background": a routed
 *       expert is a gated MLP; a channel owns one gate row, one up row and one
 *       down column.
 *
 * Precision.  The route (softmax, top-k, Eq. 2) is computed in fp32 because
 * the P1 router method computes the probabilities with dtype=float and forms
 * the weights from them; the steps the pages leave open (exp, sum order,
 * tie-break) follow the readings listed in the docstring of oracle/__init__.py and
 * below.  Everything the pages do not fix (router logits, expert matmuls,
 * silu, combine) is accumulated in fp64 and rounded to fp32 once at the end.
 *
 * Build: gcc -O2 -ffp-contract=off -fopenmp -shared -fPIC (no fast-math).
 * Parity of this file is pinned by tests/test_oracle_pins.py.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_ABI 1

enum { OR_F32 = 0, OR_BF16 = 1 };
enum { OR_OK = 0, OR_EINVAL = 1, OR_ENONFINITE = 2, OR_ENOMEM = 3 };

int oracle_abi_version(void) { return ORACLE_ABI; }

/* ------------------------------------------------------------------ */
/* bfloat16: the upper 16 bits of an IEEE binary32.  Upcast is exact.  */
/* ------------------------------------------------------------------ */
static float bf16_to_f32(uint16_t b)
{
    uint32_t u = ((uint32_t)b) << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

static uint32_t f32_bits(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    return u;
}

static float bits_f32(uint32_t u)
{
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* element i of a tensor stored as fp32 or bf16, upcast exactly */
static double load_elem(const void *base, int dtype, int64_t i)
{
    if (dtype == OR_BF16)
        return (double)bf16_to_f32(((const uint16_t *)base)[i]);
    return (double)((const float *)base)[i];
}

/* ------------------------------------------------------------------ */
/* exp for d <= 0, written from Cody & Waite's argument reduction      */
/* (Cody & Waite, "Software Manual for the Elementary Functions",      */
/* 1980): e^d = 2^n * e^r with n = rint(d / ln2) and r = d - n*ln2,    */
/* where ln2 is split in a high part with trailing zero bits and a low */
/* correction.  e^r is the degree-7 Taylor polynomial, by Horner.      */
/* The pages only say softmax in fp32; this exact recipe is the        */
/* reading that makes the route reproducible bit for bit.             */
/* ------------------------------------------------------------------ */
static int   g_consts_ready = 0;
static float g_log2e, g_ln2_hi, g_ln2_lo, g_inv_fact[8];

static void derive_exp_constants(void)
{
    if (g_consts_ready)
        return;
    /* log2(e) = 1/ln(2), rounded to the nearest float */
    g_log2e = (float)(1.0 / M_LN2);
    /* ln 2 rounded to float, then its 8 lowest significand bits cleared:
     * 16 significant bits remain, so n * ln2_hi is exact for |n| < 2^8. */
    g_ln2_hi = bits_f32(f32_bits((float)M_LN2) & 0xFFFFFF00u);
    /* the remainder ln2 - ln2_hi, rounded to float */
    g_ln2_lo = (float)(M_LN2 - (double)g_ln2_hi);
    /* Taylor coefficients 1/k!, k = 0..7, each rounded to float */
    double f = 1.0;
    for (int k = 0; k < 8; ++k) {
        if (k > 0)
            f *= (double)k;
        g_inv_fact[k] = (float)(1.0 / f);
    }
    g_consts_ready = 1;
}

float oracle_exp_spec(float d)
{
    derive_exp_constants();
    if (d < -80.0f)
        return 0.0f; /* below e^-80 every probability is treated as 0 */
    float t = d * g_log2e;
    float n = rintf(t); /* round half to even (default rounding mode) */
    float r = fmaf(-n, g_ln2_hi, d);
    r = fmaf(-n, g_ln2_lo, r);
    float q = g_inv_fact[7];
    for (int k = 6; k >= 0; --k)
        q = fmaf(q, r, g_inv_fact[k]);
    return ldexpf(q, (int)n);
}

void oracle_exp_spec_n(const float *d, float *out, int64_t n)
{
    derive_exp_constants();
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_exp_spec(d[i]);
}

/* ------------------------------------------------------------------ */
/* Pairwise sum of v[0..n), zero-padded to the next power of two P:    */
/* S(v[0..P)) = S(v[0..P/2)) + S(v[P/2..P)), S of one element = itself. */
/* ------------------------------------------------------------------ */
static float pairwise_sum(const float *v, int64_t lo, int64_t len, int64_t n)
{
    if (len == 1)
        return lo < n ? v[lo] : 0.0f;
    int64_t half = len / 2;
    float a = pairwise_sum(v, lo, half, n);
    float b = pairwise_sum(v, lo + half, half, n);
    return a + b;
}

static int64_t next_pow2(int64_t n)
{
    int64_t p = 1;
    while (p < n)
        p *= 2;
    return p;
}

/* Softmax of one row of E logits, fp32 (P1, Code of the Week: probabilities
 * from softmax with dtype=float).  Returns OR_ENONFINITE on a non-finite
 * logit, which the reading treats as a violated precondition. */
static int softmax_row(const float *l, int32_t E, float *p)
{
    float m = l[0];
    for (int32_t e = 0; e < E; ++e) {
        if (!isfinite(l[e]))
            return OR_ENONFINITE;
        if (l[e] > m)
            m = l[e];
    }
    for (int32_t e = 0; e < E; ++e)
        p[e] = oracle_exp_spec(l[e] - m);
    float S = pairwise_sum(p, 0, next_pow2(E), E);
    for (int32_t e = 0; e < E; ++e)
        p[e] = p[e] / S;
    return OR_OK;
}

int oracle_softmax(const float *logits, int64_t T, int32_t E, float *probs)
{
    if (T < 0 || E < 1)
        return OR_EINVAL;
    derive_exp_constants();
    for (int64_t t = 0; t < T; ++t) {
        int rc = softmax_row(logits + t * E, E, probs + t * E);
        if (rc != OR_OK)
            return rc;
    }
    return OR_OK;
}

/* ------------------------------------------------------------------ */
/* Route of one token (P1 Code of the Week; P1 The Receipt, Eq. 2):    */
/*  rank experts by probability, highest first, the lower index first  */
/*  on equal probability; keep the first min(k2, E) of them; the first */
/*  k1 are activated.  If k2 >= E the weights are the probabilities    */
/*  themselves (no renormalisation); otherwise each activated weight  */
/*  is its probability divided by the sum of the kept min(k2,E)        */
/*  probabilities, summed in rank order.                               */
/* ------------------------------------------------------------------ */
static int route_row(const float *l, int32_t E, int32_t k1, int32_t k2,
                     int32_t *ids, float *w, float *p, int32_t *rank_id,
                     unsigned char *taken)
{
    int rc = softmax_row(l, E, p);
    if (rc != OR_OK)
        return rc;
    int32_t K2 = k2 < E ? k2 : E;
    memset(taken, 0, (size_t)E);
    /* K2 rounds of "pick the best expert not yet picked" */
    for (int32_t r = 0; r < K2; ++r) {
        int32_t best = -1;
        for (int32_t e = 0; e < E; ++e) {
            if (taken[e])
                continue;
            if (best < 0 || p[e] > p[best])
                best = e; /* strict '>' keeps the lower index on ties */
        }
        taken[best] = 1;
        rank_id[r] = best;
    }
    if (k2 >= E) {
        for (int32_t r = 0; r < k1; ++r) {
            ids[r] = rank_id[r];
            w[r] = p[rank_id[r]];
        }
    } else {
        float M = 0.0f;
        for (int32_t r = 0; r < K2; ++r)
            M = M + p[rank_id[r]];
        for (int32_t r = 0; r < k1; ++r) {
            ids[r] = rank_id[r];
            w[r] = p[rank_id[r]] / M;
        }
    }
    return OR_OK;
}

int oracle_route(const float *logits, int64_t T, int32_t E, int32_t k1,
                 int32_t k2, int32_t *ids, float *w)
{
    if (T < 0 || E < 1 || k1 < 1 || k1 > E || k2 < k1)
        return OR_EINVAL;
    derive_exp_constants();
    float *p = (float *)malloc(sizeof(float) * (size_t)E);
    int32_t *rank_id = (int32_t *)malloc(sizeof(int32_t) * (size_t)E);
    unsigned char *taken = (unsigned char *)malloc((size_t)E);
    if (!p || !rank_id || !taken) {
        free(p); free(rank_id); free(taken);
        return OR_ENOMEM;
    }
    int rc = OR_OK;
    for (int64_t t = 0; t < T && rc == OR_OK; ++t)
        rc = route_row(logits + t * E, E, k1, k2, ids + t * k1, w + t * k1,
                       p, rank_id, taken);
    free(p); free(rank_id); free(taken);
    return rc;
}

/* ------------------------------------------------------------------ */
/* Router logits (P1 Code of the Week: a linear layer over the hidden  */
/* state): l[t,e] = sum_h x[t,h] * Wr[e,h] (+ br[e]); fp64 sum, one    */
/* rounding to fp32.                                                   */
/* ------------------------------------------------------------------ */
int oracle_logits(const void *x, int act, int64_t T, int32_t H,
                  const float *Wr, const float *br, int32_t E, float *logits,
                  int nthreads)
{
    if (T < 0 || H < 1 || E < 1 || (act != OR_F32 && act != OR_BF16))
        return OR_EINVAL;
#ifdef _OPENMP
    if (nthreads < 1)
        nthreads = 1;
#pragma omp parallel for num_threads(nthreads) schedule(dynamic, 1)
#endif
    for (int64_t t = 0; t < T; ++t) {
        for (int32_t e = 0; e < E; ++e) {
            double s = 0.0;
            for (int32_t h = 0; h < H; ++h)
                s += load_elem(x, act, t * H + h) * (double)Wr[(int64_t)e * H + h];
            if (br)
                s += (double)br[e];
            logits[t * E + e] = (float)s;
        }
    }
    return OR_OK;
}

/* ------------------------------------------------------------------ */
/* Routed experts and combine.  Expert e is a gated MLP (P4 section 2): */
/* channel c owns gate row Wg[e,c,:], up row Wu[e,c,:] and down column  */
/* Wd[e,:,c]; with silu on the gate (the SwiGLU reading),               */
/*   a_c = silu(Wg[e,c,:].x) * (Wu[e,c,:].x),  z_h = sum_c Wd[e,h,c] a_c */
/* and the layer output is the weighted sum of the activated experts    */
/* (P1 The Receipt: the weights of Eq. 2 scale the expert branch):     */
/*   y = sum_{r<k1} w_r * z^(r), in rank order.                         */
/* ids index the E experts present in Wg/Wu/Wd (a caller may pass only  */
/* the activated experts, with ids remapped).  fp64 throughout.         */
/* ------------------------------------------------------------------ */
static double silu(double z) { return z / (1.0 + exp(-z)); }

int oracle_experts(const void *x, int act, int64_t T, int32_t H,
                   const void *Wg, const void *Wu, const void *Wd, int wt,
                   int32_t E, int32_t I, int32_t k1, const int32_t *ids,
                   const float *w, float *y, int nthreads)
{
    if (T < 0 || H < 1 || I < 1 || E < 1 || k1 < 1 ||
        (act != OR_F32 && act != OR_BF16) || (wt != OR_F32 && wt != OR_BF16))
        return OR_EINVAL;
    for (int64_t i = 0; i < T * k1; ++i)
        if (ids[i] < 0 || ids[i] >= E)
            return OR_EINVAL;
    int bad = 0;
#ifdef _OPENMP
    if (nthreads < 1)
        nthreads = 1;
#pragma omp parallel for num_threads(nthreads) schedule(dynamic, 1)
#endif
    for (int64_t t = 0; t < T; ++t) {
        double *xv = (double *)malloc(sizeof(double) * (size_t)H);
        double *a = (double *)malloc(sizeof(double) * (size_t)I);
        double *acc = (double *)malloc(sizeof(double) * (size_t)H);
        if (!xv || !a || !acc) {
            free(xv); free(a); free(acc);
#ifdef _OPENMP
#pragma omp atomic write
#endif
            bad = 1;
            continue;
        }
        for (int32_t h = 0; h < H; ++h) {
            xv[h] = load_elem(x, act, t * H + h);
            acc[h] = 0.0;
        }
        for (int32_t r = 0; r < k1; ++r) {
            int64_t e = ids[t * k1 + r];
            for (int32_t c = 0; c < I; ++c) {
                int64_t row = (e * I + c) * (int64_t)H;
                double g = 0.0, u = 0.0;
                for (int32_t h = 0; h < H; ++h) {
                    g += load_elem(Wg, wt, row + h) * xv[h];
                    u += load_elem(Wu, wt, row + h) * xv[h];
                }
                a[c] = silu(g) * u;
            }
            double wr = (double)w[t * k1 + r];
            for (int32_t h = 0; h < H; ++h) {
                int64_t row = (e * H + h) * (int64_t)I;
                double z = 0.0;
                for (int32_t c = 0; c < I; ++c)
                    z += load_elem(Wd, wt, row + c) * a[c];
                acc[h] += wr * z;
            }
        }
        for (int32_t h = 0; h < H; ++h)
            y[t * H + h] = (float)acc[h];
        free(xv); free(a); free(acc);
    }
    return bad ? OR_ENOMEM : OR_OK;
}

/* The whole layer: logits, route, experts, combine. */
int oracle_forward(const void *x, int act, int64_t T, int32_t H,
                   const float *Wr, const float *br, int32_t E,
                   const void *Wg, const void *Wu, const void *Wd, int wt,
                   int32_t I, int32_t k1, int32_t k2, float *y,
                   float *logits, int32_t *ids, float *w, int nthreads)
{
    int rc = oracle_logits(x, act, T, H, Wr, br, E, logits, nthreads);
    if (rc != OR_OK)
        return rc;
    rc = oracle_route(logits, T, E, k1, k2, ids, w);
    if (rc != OR_OK)
        return rc;
    return oracle_experts(x, act, T, H, Wg, Wu, Wd, wt, E, I, k1, ids, w, y,
                          nthreads);
}

/* ================================================================== */
/* The bf16 router of the P1 router method as it runs on a bf16 model */
/* (P1 Code of the Week): the linear layer is computed in the model's */
/* dtype, so the logits are bf16; the softmax upcasts them to fp32    */
/* (dtype=float); the returned weights are cast back to the logits'   */
/* dtype.  Readings: the bf16 logit is the exact dot product rounded  */
/* once to bf16 (round to nearest, ties to even, the usual cast); the */
/* cast of the weights rounds the fp32 Eq. 2 weight the same way; the */
/* experts are then scaled by that bf16 weight.                       */
/* ================================================================== */

/* d rounded to the nearest bfloat16 value, ties to even.  bf16 keeps 8
 * significant bits, so d = m * 2^q with m an integer of at most 8 bits and
 * q = exponent(d) - 8; below the smallest normal (2^-126) the spacing stays
 * 2^-133.  nearbyint rounds in the default mode: to nearest, ties to even. */
static float round_bf16(double d)
{
    if (d == 0.0 || !isfinite(d))
        return (float)d;
    int ex;
    (void)frexp(d, &ex); /* |d| = f * 2^ex with f in [0.5, 1) */
    int q = ex - 8;
    if (q < -133)
        q = -133;
    double m = nearbyint(ldexp(d, -q));
    return (float)ldexp(m, q);
}

void oracle_round_bf16_n(const double *in, float *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = round_bf16(in[i]);
}

/* bf16 logits: l[t,e] = bf16(sum_h x[t,h] * Wr[e,h]), the products of bf16
 * values exact in fp64, the sum in fp64, one rounding to bf16. */
int oracle_logits_bf16(const uint16_t *x, int64_t T, int32_t H,
                       const uint16_t *Wr, int32_t E, float *logits,
                       int nthreads)
{
    if (T < 0 || H < 1 || E < 1)
        return OR_EINVAL;
#ifdef _OPENMP
    if (nthreads < 1)
        nthreads = 1;
#pragma omp parallel for num_threads(nthreads) schedule(dynamic, 1)
#endif
    for (int64_t t = 0; t < T; ++t) {
        for (int32_t e = 0; e < E; ++e) {
            double s = 0.0;
            for (int32_t h = 0; h < H; ++h)
                s += (double)bf16_to_f32(x[t * H + h]) *
                     (double)bf16_to_f32(Wr[(int64_t)e * H + h]);
            logits[t * E + e] = round_bf16(s);
        }
    }
    return OR_OK;
}

/* The route of oracle_route, then each weight cast to bf16. */
int oracle_route_bf16w(const float *logits, int64_t T, int32_t E, int32_t k1,
                       int32_t k2, int32_t *ids, float *w)
{
    int rc = oracle_route(logits, T, E, k1, k2, ids, w);
    if (rc != OR_OK)
        return rc;
    for (int64_t i = 0; i < T * k1; ++i)
        w[i] = round_bf16((double)w[i]);
    return OR_OK;
}

/* The whole layer with the bf16 router: bf16 x, Wr and expert weights. */
int oracle_forward_bf16_router(const uint16_t *x, int64_t T, int32_t H,
                               const uint16_t *Wr, int32_t E,
                               const uint16_t *Wg, const uint16_t *Wu,
                               const uint16_t *Wd, int32_t I, int32_t k1,
                               int32_t k2, float *y, float *logits,
                               int32_t *ids, float *w, int nthreads)
{
    int rc = oracle_logits_bf16(x, T, H, Wr, E, logits, nthreads);
    if (rc != OR_OK)
        return rc;
    rc = oracle_route_bf16w(logits, T, E, k1, k2, ids, w);
    if (rc != OR_OK)
        return rc;
    return oracle_experts(x, OR_BF16, T, H, Wg, Wu, Wd, OR_BF16, E, I, k1, ids,
                          w, y, nthreads);
}

/* ================================================================== */
/* Shared expert ("Channel Selection for Mixture-of-Experts Decoding  */
/* Needs No Calibration Data", appendix B "Experimental setup": shared */
/* experts always run in full, beside the routed ones).  The pages do  */
/* not give its gating; the reading taken: the shared expert is a     */
/* gated MLP like a routed one, with Is channels, added to the routed */
/* sum with the factor g = sigmoid(x . sg) when a gate vector sg is   */
/* given and g = 1 without one:                                       */
/*   y = sum_r w_r E_{id_r}(x) + g * Sd (silu(Sg x) * (Su x)).         */
/* fp64 throughout, rounded once to fp32.                             */
/* ================================================================== */
int oracle_shared(const void *x, int act, int64_t T, int32_t H,
                  const void *Sg, const void *Su, const void *Sd, int wt,
                  int32_t Is, const float *sg, float *ys, int nthreads)
{
    if (T < 0 || H < 1 || Is < 1 || (act != OR_F32 && act != OR_BF16) ||
        (wt != OR_F32 && wt != OR_BF16))
        return OR_EINVAL;
    int bad = 0;
#ifdef _OPENMP
    if (nthreads < 1)
        nthreads = 1;
#pragma omp parallel for num_threads(nthreads) schedule(dynamic, 1)
#endif
    for (int64_t t = 0; t < T; ++t) {
        double *xv = (double *)malloc(sizeof(double) * (size_t)H);
        double *a = (double *)malloc(sizeof(double) * (size_t)Is);
        if (!xv || !a) {
            free(xv); free(a);
#ifdef _OPENMP
#pragma omp atomic write
#endif
            bad = 1;
            continue;
        }
        for (int32_t h = 0; h < H; ++h)
            xv[h] = load_elem(x, act, t * H + h);
        double g = 1.0;
        if (sg) {
            double z = 0.0;
            for (int32_t h = 0; h < H; ++h)
                z += xv[h] * (double)sg[h];
            g = 1.0 / (1.0 + exp(-z));
        }
        for (int32_t c = 0; c < Is; ++c) {
            int64_t row = (int64_t)c * H;
            double gg = 0.0, u = 0.0;
            for (int32_t h = 0; h < H; ++h) {
                gg += load_elem(Sg, wt, row + h) * xv[h];
                u += load_elem(Su, wt, row + h) * xv[h];
            }
            a[c] = silu(gg) * u;
        }
        for (int32_t h = 0; h < H; ++h) {
            int64_t row = (int64_t)h * Is;
            double z = 0.0;
            for (int32_t c = 0; c < Is; ++c)
                z += load_elem(Sd, wt, row + c) * a[c];
            ys[t * H + h] = (float)(g * z);
        }
        free(xv); free(a);
    }
    return bad ? OR_ENOMEM : OR_OK;
}

/* ================================================================== */
/* Channel top-k inside the activated experts ("Channel Selection for */
/* Mixture-of-Experts Decoding Needs No Calibration Data", section 5.2 */
/* "output-scaled score"; section 2: a channel owns one gate row, one  */
/* up row and one down column).  For a token routed to experts e_r    */
/* with weights w_r, channel (r, c) has                                */
/*   a = silu(Wg[e_r,c,:] . x) * (Wu[e_r,c,:] . x),                    */
/*   score = w_r * ||Wd[e_r,:,c]||_2 * |a|,                             */
/* an estimate of its output contribution in output units, so channels */
/* of different experts compare; the keep highest scores over the     */
/* token's k1*I channels are kept (exact top-k; reading: equal scores */
/* go to the lower flat index r*I + c), and                            */
/*   y = sum over kept (r, c), in flat-index order, of w_r a Wd[e_r,:,c]. */
/* fp64 throughout; scores rounded once to fp32.                       */
/* ================================================================== */

/* dn[e, c] = ||Wd[e, :, c]||_2 */
int oracle_down_column_norms(const void *Wd, int wt, int32_t E, int32_t H,
                             int32_t I, float *dn)
{
    if (E < 1 || H < 1 || I < 1 || (wt != OR_F32 && wt != OR_BF16))
        return OR_EINVAL;
    for (int64_t e = 0; e < E; ++e)
        for (int32_t c = 0; c < I; ++c) {
            double s = 0.0;
            for (int32_t h = 0; h < H; ++h) {
                double v = load_elem(Wd, wt, (e * H + h) * (int64_t)I + c);
                s += v * v;
            }
            dn[e * I + c] = (float)sqrt(s);
        }
    return OR_OK;
}

/* scores [T, k1*I] of the channels of each token's activated experts */
int oracle_channel_scores(const void *x, int act, int64_t T, int32_t H,
                          const void *Wg, const void *Wu, int wt, int32_t E,
                          int32_t I, int32_t k1, const int32_t *ids,
                          const float *w, const float *dn, float *scores)
{
    if (T < 0 || H < 1 || I < 1 || E < 1 || k1 < 1)
        return OR_EINVAL;
    for (int64_t t = 0; t < T; ++t)
        for (int32_t r = 0; r < k1; ++r) {
            int64_t e = ids[t * k1 + r];
            if (e < 0 || e >= E)
                return OR_EINVAL;
            for (int32_t c = 0; c < I; ++c) {
                int64_t row = (e * I + c) * (int64_t)H;
                double g = 0.0, u = 0.0;
                for (int32_t h = 0; h < H; ++h) {
                    double xv = load_elem(x, act, t * H + h);
                    g += load_elem(Wg, wt, row + h) * xv;
                    u += load_elem(Wu, wt, row + h) * xv;
                }
                double a = silu(g) * u;
                scores[(t * k1 + r) * (int64_t)I + c] =
                    (float)((double)w[t * k1 + r] * (double)dn[e * I + c] * fabs(a));
            }
        }
    return OR_OK;
}

/* kept[t, j] = 1 for the keep highest scores of row t (n = k1*I scores),
 * equal scores to the lower j; keep rounds of "take the best not taken". */
int oracle_channel_select(const float *scores, int64_t T, int32_t n, int32_t keep,
                          unsigned char *kept)
{
    if (T < 0 || n < 1 || keep < 0 || keep > n)
        return OR_EINVAL;
    for (int64_t t = 0; t < T; ++t) {
        const float *s = scores + t * n;
        unsigned char *k = kept + t * n;
        memset(k, 0, (size_t)n);
        for (int32_t q = 0; q < keep; ++q) {
            int32_t best = -1;
            for (int32_t j = 0; j < n; ++j) {
                if (k[j])
                    continue;
                if (best < 0 || s[j] > s[best])
                    best = j; /* strict '>' keeps the lower index on ties */
            }
            k[best] = 1;
        }
    }
    return OR_OK;
}

/* y [T, H] from the kept channels only (flat-index order). */
int oracle_experts_kept(const void *x, int act, int64_t T, int32_t H,
                        const void *Wg, const void *Wu, const void *Wd, int wt,
                        int32_t E, int32_t I, int32_t k1, const int32_t *ids,
                        const float *w, const unsigned char *kept, float *y)
{
    if (T < 0 || H < 1 || I < 1 || E < 1 || k1 < 1)
        return OR_EINVAL;
    double *acc = (double *)malloc(sizeof(double) * (size_t)H);
    if (!acc)
        return OR_ENOMEM;
    for (int64_t t = 0; t < T; ++t) {
        for (int32_t h = 0; h < H; ++h)
            acc[h] = 0.0;
        for (int32_t r = 0; r < k1; ++r) {
            int64_t e = ids[t * k1 + r];
            if (e < 0 || e >= E) {
                free(acc);
                return OR_EINVAL;
            }
            for (int32_t c = 0; c < I; ++c) {
                if (!kept[(t * k1 + r) * (int64_t)I + c])
                    continue;
                int64_t row = (e * I + c) * (int64_t)H;
                double g = 0.0, u = 0.0;
                for (int32_t h = 0; h < H; ++h) {
                    double xv = load_elem(x, act, t * H + h);
                    g += load_elem(Wg, wt, row + h) * xv;
                    u += load_elem(Wu, wt, row + h) * xv;
                }
                double a = silu(g) * u * (double)w[t * k1 + r];
                for (int32_t h = 0; h < H; ++h)
                    acc[h] += load_elem(Wd, wt, (e * H + h) * (int64_t)I + c) * a;
            }
        }
        for (int32_t h = 0; h < H; ++h)
            y[t * H + h] = (float)acc[h];
    }
    free(acc);
    return OR_OK;
}
