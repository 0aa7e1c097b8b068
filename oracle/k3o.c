/*
 * k3o.c -- CPU oracle for the routed-expert MXFP4 path.
 *
 * TEST INFRASTRUCTURE. Only tests/, __graft_entry__.smoke() and bench.py's
 * cpu_baseline leg may load this library. The GPU library never links it,
 * shares no source, header, table or constant generator with it, and the
 * product path never falls back to it.
 *
 * Plain, slow, obviously correct: every value is computed from its definition
 * in double precision (or in the precision the method itself fixes), one output
 * at a time, in the order stated next to each function. OpenMP spreads whole
 * outputs over threads; each output is still summed by one thread in one fixed
 * order, so the bits do not depend on the thread count ("kimi-k3-in-c: 2.78
 * trillion parameters, one CPU, 8 GB of RAM", section "A floating-point
 * contract, not a convention"). Built with -ffp-contract=off for the same
 * reason ("kimi-k3-in-c" README, section "The codebase").
 *
 * Sources (pages, with their sections):
 *   [KIC-README]  "kimi-k3-in-c" README (spark.entire.vc tools page)
 *   [KIC-ARTICLE] "kimi-k3-in-c: 2.78 trillion parameters, one CPU, 8 GB of RAM"
 *   [COLIBRI-K3]  "Kimi K3 engine (c/kimi_k3.c)" (colibri docs)
 *
 * Parity status of each function is stated in its comment; every function is
 * pinned by tests/test_oracle_*.py except where a comment says "parity
 * unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define K3O_GROUP 32

#ifdef _OPENMP
#include <omp.h>
#endif

/* Threads an OpenMP region of the oracle uses (1 without OpenMP). */
int k3o_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Set the threads of the calling thread's later OpenMP regions (n >= 1).
 * The results do not depend on it: each output is summed by one thread. */
void k3o_set_threads(int n)
{
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* ------------------------------------------------------------------------ */
/* Format tables, built from the bit-field definitions (never copied).        */
/* ------------------------------------------------------------------------ */

static double e2m1_val[16];   /* code -> value                              */
static int e2m1_dbl[16];      /* code -> 2*value, an integer in [-12, 12]   */
static double e8m0_val[256];  /* byte -> 2^(byte-127); [255] unused (skip)  */
static int tables_ready;

/* E2M1 (OCP microscaling element type): bit 3 = sign, bits 2..1 = exponent
 * (bias 1), bit 0 = mantissa; exponent 0 is subnormal (0 or 0.5).
 * [COLIBRI-K3] "Weights": e2m1 nibbles, bit 3 = sign; [KIC-ARTICLE]
 * "Reduction one": a 4-bit code indexing a 16-entry table. */
static double e2m1_from_bits(unsigned c)
{
    const unsigned sign = (c >> 3) & 1u, ex = (c >> 1) & 3u, man = c & 1u;
    double mag;
    if (ex == 0)
        mag = 0.5 * (double)man;
    else
        mag = ldexp(1.0 + 0.5 * (double)man, (int)ex - 1);
    return sign ? -mag : mag;
}

__attribute__((constructor)) static void init_tables(void)
{
    if (tables_ready)
        return;
    for (unsigned c = 0; c < 16; ++c) {
        e2m1_val[c] = e2m1_from_bits(c);
        e2m1_dbl[c] = (int)lrint(2.0 * e2m1_val[c]);
    }
    /* ue8m0: w = v * 2^(s-127) ([COLIBRI-K3] "Weights"); 255 is the NaN
     * encoding, which the pages' kernel skips ([KIC-ARTICLE] "Reduction one"). */
    for (int s = 0; s < 255; ++s)
        e8m0_val[s] = ldexp(1.0, s - 127);
    e8m0_val[255] = NAN;
    tables_ready = 1;
}

double k3o_e2m1(int code)
{
    init_tables();
    return e2m1_val[code & 15];
}

int k3o_e2m1_doubled(int code)
{
    init_tables();
    return e2m1_dbl[code & 15];
}

double k3o_e8m0(int s)
{
    init_tables();
    return e8m0_val[s & 255];
}

/* Nibble j of a packed row: the low nibble of byte j/2 is the even column, the
 * high nibble the odd one ([COLIBRI-K3] "Weights"). */
static inline unsigned nibble(const uint8_t *row, int j)
{
    const uint8_t b = row[j >> 1];
    return (j & 1) ? (unsigned)(b >> 4) : (unsigned)(b & 15u);
}

/* Sizes of one MXFP4 matrix [rows x in]: in/2 bytes of nibbles and in/32
 * scale bytes per row ([KIC-README] "The problem: a model that does not fit":
 * 0.5 byte per nibble plus 1/32 byte of shared scale). */
int64_t k3o_mxfp4_bytes(int64_t rows, int64_t in)
{
    return rows * (in / 2) + rows * (in / K3O_GROUP);
}

/* ------------------------------------------------------------------------ */
/* EXACT product on the packed layout.                                        */
/* ------------------------------------------------------------------------ */

/* The EXACT product of one packed row with x, in two passes:
 *   1. gsum[g] = the dot product of group g's 32 decoded weights (e2m1 values,
 *      exact in double) with x's 32 entries, products and additions in double,
 *      columns in increasing order (the pages give one double accumulator per
 *      group: [KIC-ARTICLE] "Reduction one");
 *   2. y = sum over the groups in increasing order of 2^(s_g-127) * gsum[g],
 *      leaving out every group whose scale byte is 255 (the format's NaN code,
 *      which the pages' kernel treats as a group of zeros, same section).
 * The normaliser sum_j |w_j||x_j| of the tolerance is formed the same way. */
static double mxfp4_row_exact(const uint8_t *row, const uint8_t *srow, const float *x,
                              int ngrp, double *gsum, double *gabs, double *nrm)
{
    for (int g = 0; g < ngrp; ++g) {
        double d = 0.0, a = 0.0;
        for (int c = 0; c < K3O_GROUP; ++c) {
            const int j = g * K3O_GROUP + c;
            const double w = e2m1_val[nibble(row, j)];
            const double xv = (double)x[j];
            d += w * xv;
            a += fabs(w) * fabs(xv);
        }
        gsum[g] = d;
        gabs[g] = a;
    }
    double y = 0.0, n = 0.0;
    for (int g = 0; g < ngrp; ++g) {
        const uint8_t code = srow[g];
        if (code == 255)
            continue;
        y += e8m0_val[code] * gsum[g];
        n += e8m0_val[code] * gabs[g];
    }
    *nrm = n;
    return y;
}

/* y[r] = the EXACT product of row r (mxfp4_row_exact), rounded to float once.
 * Optional: y64 = the double result before rounding; nrm = sum_j |w_rj||x_j|
 * (the normaliser of the tolerance). Returns 0, or -1 on bad arguments. */
int k3o_mxfp4_gemv(float *y, double *y64, double *nrm, const float *x,
                   const uint8_t *packed, const uint8_t *scales,
                   int in, int rows, int group)
{
    init_tables();
    if (group != K3O_GROUP || in <= 0 || in % K3O_GROUP || rows < 0)
        return -1;
    const int ngrp = in / K3O_GROUP;
#pragma omp parallel
    {
        double *gsum = malloc(sizeof(double) * (size_t)ngrp);
        double *gabs = malloc(sizeof(double) * (size_t)ngrp);
#pragma omp for schedule(static)
        for (int r = 0; r < rows; ++r) {
            double n;
            const double v = mxfp4_row_exact(packed + (size_t)r * (size_t)(in / 2),
                                             scales + (size_t)r * (size_t)ngrp, x, ngrp,
                                             gsum, gabs, &n);
            y[r] = (float)v;
            if (y64)
                y64[r] = v;
            if (nrm)
                nrm[r] = n;
        }
        free(gsum);
        free(gabs);
    }
    return 0;
}

/* Dequantise to a dense double matrix W[rows][in]: W = e2m1 * 2^(s-127), and
 * 0 for a skipped group. This is the "dequantise-then-multiply" form the pages
 * compare the kernel against ([KIC-ARTICLE] "A floating-point contract"). */
int k3o_mxfp4_dequant(double *W, const uint8_t *packed, const uint8_t *scales,
                      int in, int rows, int group)
{
    init_tables();
    if (group != K3O_GROUP || in <= 0 || in % K3O_GROUP || rows < 0)
        return -1;
    const int ngrp = in / K3O_GROUP;
    for (int r = 0; r < rows; ++r) {
        const uint8_t *pr = packed + (size_t)r * (size_t)(in / 2);
        for (int j = 0; j < in; ++j) {
            const uint8_t sb = scales[(size_t)r * ngrp + j / K3O_GROUP];
            W[(size_t)r * in + j] = (sb == 255) ? 0.0 : e2m1_val[nibble(pr, j)] * e8m0_val[sb];
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Dense products in the pages' fixed order.                                  */
/* ------------------------------------------------------------------------ */

/* bfloat16 bits -> float: the 16 bits are the high half of a float32, so the
 * widening is exact. */
static inline double bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Dense dot products, the plain definition: every product w_i * x_i is formed
 * in double (exact for fp32 and bf16 operands: at most 24 + 24 significant
 * bits), and the products are added into one double in increasing i. The
 * pages fix an order per output so that results do not depend on threads
 * ([KIC-ARTICLE] "A floating-point contract, not a convention"); this oracle's
 * order is plain index order. Optional *absdot = sum_i |w_i||x_i|. */
static double dot_f32_in_order(const float *w, const float *x, int n)
{
    double s = 0.0;
    for (int i = 0; i < n; ++i)
        s += (double)x[i] * (double)w[i];
    return s;
}

static double dot_bf16_in_order(const uint16_t *w, const float *x, int n, double *absdot)
{
    double s = 0.0, a = 0.0;
    for (int i = 0; i < n; ++i) {
        const double wi = bf16_to_double(w[i]);
        s += (double)x[i] * wi;
        a += fabs((double)x[i]) * fabs(wi);
    }
    if (absdot)
        *absdot = a;
    return s;
}

/* y[o] = sum_i W[o][i] x[i] for fp32 W, in index order. */
int k3o_matmul_f32(double *y, const float *x, const float *W, int in, int out)
{
    if (in <= 0 || out < 0)
        return -1;
#pragma omp parallel for schedule(static)
    for (int o = 0; o < out; ++o)
        y[o] = dot_f32_in_order(W + (size_t)o * in, x, in);
    return 0;
}

/* Same for bf16 W; optional nrm[o] = sum_i |W_oi||x_i|. */
int k3o_matmul_bf16(double *y, double *nrm, const float *x, const uint16_t *W, int in, int out)
{
    if (in <= 0 || out < 0)
        return -1;
#pragma omp parallel for schedule(static)
    for (int o = 0; o < out; ++o)
        y[o] = dot_bf16_in_order(W + (size_t)o * in, x, in, nrm ? &nrm[o] : NULL);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* SiTU-GLU.                                                                  */
/* ------------------------------------------------------------------------ */

/* h = b1*tanh(g/b1) * sigmoid(g) * b2*tanh(u/b2), sigmoid(z) = 1/(1+e^-z);
 * b1 = 4, b2 = 25 for the checkpoint ([COLIBRI-K3] "Architecture notes",
 * Stable LatentMoE; [KIC-README] config struct, situ_b1/situ_b2). g is the
 * w1 (gate) product, u the w3 (up) product: which of w1/w3 is the gate is not
 * stated on the pages (reading: w1 = gate, w3 = up; parity unpinned by the
 * pages for that assignment). */
double k3o_situ(double g, double u, double b1, double b2)
{
    const double sig = 1.0 / (1.0 + exp(-g));
    return b1 * tanh(g / b1) * sig * b2 * tanh(u / b2);
}

/* Elementwise h[i] = SiTU(g[i], u[i]) with b1 = 4, b2 = 25, each value
 * computed in double and rounded to float once. */
int k3o_situ_vec(float *h, const float *g, const float *u, int n)
{
    if (n < 0)
        return -1;
    for (int i = 0; i < n; ++i)
        h[i] = (float)k3o_situ((double)g[i], (double)u[i], 4.0, 25.0);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* IDOT: int8 activations against doubled e2m1 values.                        */
/* ------------------------------------------------------------------------ */

/* Per row of x and per group of 32: amax = max|x_j|; s = amax/127 (float);
 * q_j = rint(x_j / s) clamped to [-127, 127] (float division, rounding half
 * to even); amax == 0 gives s = 0 and q = 0. All steps in float, as the GPU
 * takes them ([COLIBRI-K3] "Streaming design", K3_IDOT: per-32-group int8
 * activations; the scale and rounding rule are the workload's). */
int k3o_quant_i8_groups(int8_t *q, float *s, const float *x, int n_rows, int in)
{
    if (in <= 0 || in % K3O_GROUP || n_rows < 0)
        return -1;
    const int ngrp = in / K3O_GROUP;
#pragma omp parallel for schedule(static)
    for (int t = 0; t < n_rows; ++t) {
        for (int g = 0; g < ngrp; ++g) {
            const float *xg = x + (size_t)t * in + (size_t)g * K3O_GROUP;
            int8_t *qg = q + (size_t)t * in + (size_t)g * K3O_GROUP;
            float amax = 0.0f;
            for (int j = 0; j < K3O_GROUP; ++j) {
                const float a = fabsf(xg[j]);
                if (a > amax)
                    amax = a;
            }
            if (amax == 0.0f) {
                s[(size_t)t * ngrp + g] = 0.0f;
                memset(qg, 0, K3O_GROUP);
                continue;
            }
            const float sc = amax / 127.0f;
            s[(size_t)t * ngrp + g] = sc;
            for (int j = 0; j < K3O_GROUP; ++j) {
                float r = rintf(xg[j] / sc);
                if (r > 127.0f)
                    r = 127.0f;
                if (r < -127.0f)
                    r = -127.0f;
                qg[j] = (int8_t)r;
            }
        }
    }
    return 0;
}

/* I[t][r][g] = sum_{j in g} q_tj * (2*e2m1(n_rj)), an exact int32: the doubled
 * e2m1 values are integers in [-12, 12] ([COLIBRI-K3] "Streaming design"). */
int k3o_idot_groupsums(int32_t *I, const int8_t *q, const uint8_t *packed,
                       int in, int rows, int n_tokens)
{
    init_tables();
    if (in <= 0 || in % K3O_GROUP || rows < 0 || n_tokens < 0)
        return -1;
    const int ngrp = in / K3O_GROUP;
#pragma omp parallel for schedule(static)
    for (int t = 0; t < n_tokens; ++t)
        for (int r = 0; r < rows; ++r) {
            const uint8_t *pr = packed + (size_t)r * (size_t)(in / 2);
            const int8_t *qt = q + (size_t)t * in;
            for (int g = 0; g < ngrp; ++g) {
                int32_t acc = 0;
                for (int j = g * K3O_GROUP; j < (g + 1) * K3O_GROUP; ++j)
                    acc += (int32_t)qt[j] * (int32_t)e2m1_dbl[nibble(pr, j)];
                I[((size_t)t * rows + r) * ngrp + g] = acc;
            }
        }
    return 0;
}

/* y[r] = sum over groups with s_rg != 255 of I_rg * s_x[g] * 2^(s_rg-128),
 * in double, rounded to float. 2^(s-128) = 2^(s-127)/2 undoes the doubling.
 * nrm[r] = sum_g 2^(s_rg-128) * s_x[g] * sum_j |d_rj||q_j|. One token. */
int k3o_mxfp4_gemv_idot(float *y, double *y64, double *nrm, const int8_t *q, const float *sx,
                        const uint8_t *packed, const uint8_t *scales, int in, int rows)
{
    init_tables();
    if (in <= 0 || in % K3O_GROUP || rows < 0)
        return -1;
    const int ngrp = in / K3O_GROUP;
#pragma omp parallel for schedule(static)
    for (int r = 0; r < rows; ++r) {
        const uint8_t *pr = packed + (size_t)r * (size_t)(in / 2);
        const uint8_t *sr = scales + (size_t)r * (size_t)ngrp;
        double acc = 0.0, n = 0.0;
        for (int g = 0; g < ngrp; ++g) {
            const uint8_t sb = sr[g];
            if (sb == 255)
                continue;
            int32_t I = 0;
            int64_t In = 0;
            for (int j = g * K3O_GROUP; j < (g + 1) * K3O_GROUP; ++j) {
                const int d = e2m1_dbl[nibble(pr, j)];
                I += (int32_t)q[j] * d;
                In += (int64_t)abs((int)q[j]) * abs(d);
            }
            const double sc = (double)sx[g] * ldexp(1.0, (int)sb - 128);
            acc += (double)I * sc;
            n += (double)In * sc;
        }
        y[r] = (float)acc;
        if (y64)
            y64[r] = acc;
        if (nrm)
            nrm[r] = n;
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Expert GLU and the MoE layer.                                              */
/* ------------------------------------------------------------------------ */

typedef struct {
    const uint8_t *w1p, *w1s, *w3p, *w3s, *w2p, *w2s;
} k3o_expert;

enum { K3O_EXACT = 0, K3O_IDOT = 1 };

/* One expert on one token, every stage rounded to float as the API's tensors
 * are: g = w1 x, u = w3 x; h = SiTU(g, u); y = w2 h ([COLIBRI-K3]
 * "Architecture notes": experts are GLUs, inter 3072, in the latent space).
 * IDOT quantises x before w1/w3 and h before w2. Optional outputs g, u, h. */
static void expert_one(float *y, float *g, float *u, float *h, const float *x,
                       const k3o_expert *e, int latent, int inter, int mode,
                       double b1, double b2, int8_t *qbuf, float *sbuf)
{
    if (mode == K3O_EXACT) {
        k3o_mxfp4_gemv(g, NULL, NULL, x, e->w1p, e->w1s, latent, inter, K3O_GROUP);
        k3o_mxfp4_gemv(u, NULL, NULL, x, e->w3p, e->w3s, latent, inter, K3O_GROUP);
    } else {
        k3o_quant_i8_groups(qbuf, sbuf, x, 1, latent);
        k3o_mxfp4_gemv_idot(g, NULL, NULL, qbuf, sbuf, e->w1p, e->w1s, latent, inter);
        k3o_mxfp4_gemv_idot(u, NULL, NULL, qbuf, sbuf, e->w3p, e->w3s, latent, inter);
    }
    for (int r = 0; r < inter; ++r)
        h[r] = (float)k3o_situ((double)g[r], (double)u[r], b1, b2);
    if (mode == K3O_EXACT) {
        k3o_mxfp4_gemv(y, NULL, NULL, h, e->w2p, e->w2s, inter, latent, K3O_GROUP);
    } else {
        k3o_quant_i8_groups(qbuf, sbuf, h, 1, inter);
        k3o_mxfp4_gemv_idot(y, NULL, NULL, qbuf, sbuf, e->w2p, e->w2s, inter, latent);
    }
}

/* Public single-expert GLU. y [latent]; g, u, h [inter] may be NULL. */
int k3o_expert_glu(float *y, float *g, float *u, float *h, const float *x,
                   const uint8_t *w1p, const uint8_t *w1s, const uint8_t *w3p,
                   const uint8_t *w3s, const uint8_t *w2p, const uint8_t *w2s,
                   int latent, int inter, int mode)
{
    init_tables();
    if (latent <= 0 || inter <= 0 || latent % K3O_GROUP || inter % K3O_GROUP)
        return -1;
    if (mode != K3O_EXACT && mode != K3O_IDOT)
        return -1;
    const k3o_expert e = {w1p, w1s, w3p, w3s, w2p, w2s};
    const int mx = latent > inter ? latent : inter;
    float *gb = g ? g : malloc(sizeof(float) * inter);
    float *ub = u ? u : malloc(sizeof(float) * inter);
    float *hb = h ? h : malloc(sizeof(float) * inter);
    int8_t *qb = malloc((size_t)mx);
    float *sb = malloc(sizeof(float) * (size_t)(mx / K3O_GROUP));
    expert_one(y, gb, ub, hb, x, &e, latent, inter, mode, 4.0, 25.0, qb, sb);
    if (!g) free(gb);
    if (!u) free(ub);
    if (!h) free(hb);
    free(qb);
    free(sb);
    return 0;
}

/* Routing, step 1: logits[t][e] = sum_i W[e][i] x[t][i] in double, added in
 * index order. fp32 x fp32 products are exact in double, so only the
 * additions round. */
int k3o_route_logits(double *logits, const float *x, const float *W, int n_tokens, int in, int n_experts)
{
    if (in <= 0 || n_tokens < 0 || n_experts <= 0)
        return -1;
#pragma omp parallel for schedule(static) collapse(2)
    for (int t = 0; t < n_tokens; ++t)
        for (int e = 0; e < n_experts; ++e)
            logits[(size_t)t * n_experts + e] = dot_f32_in_order(W + (size_t)e * in, x + (size_t)t * in, in);
    return 0;
}

/* Routing, step 2 (Stable LatentMoE, [COLIBRI-K3] "Architecture notes";
 * [KIC-README] "Three invariants", invariant 3):
 *   score_e = sigmoid(logit_e) in double; biased_e = score_e + bias_e;
 *   select the top_k experts by biased score, larger first, equal scores going
 *   to the lower expert id; weight_k = score_k / sum of the selected scores
 *   (the bias steers selection only), rounded to float.
 * Optional out: biased[t][k] (double) of the selected experts. */
int k3o_route_select(int32_t *idx, float *wts, double *biased, const double *logits,
                     const float *bias, int n_tokens, int n_experts, int top_k)
{
    if (n_tokens < 0 || n_experts <= 0 || top_k < 1 || top_k > n_experts)
        return -1;
#pragma omp parallel for schedule(static)
    for (int t = 0; t < n_tokens; ++t) {
        double *sc = malloc(sizeof(double) * (size_t)n_experts);
        double *b = malloc(sizeof(double) * (size_t)n_experts);
        char *taken = calloc((size_t)n_experts, 1);
        for (int e = 0; e < n_experts; ++e) {
            sc[e] = 1.0 / (1.0 + exp(-logits[(size_t)t * n_experts + e]));
            b[e] = sc[e] + (double)bias[e];
        }
        double sum = 0.0;
        for (int k = 0; k < top_k; ++k) {
            int best = -1;
            for (int e = 0; e < n_experts; ++e) {
                if (taken[e])
                    continue;
                if (best < 0 || b[e] > b[best])
                    best = e; /* strict '>': an equal score keeps the lower id */
            }
            taken[best] = 1;
            idx[(size_t)t * top_k + k] = best;
            if (biased)
                biased[(size_t)t * top_k + k] = b[best];
            sum += sc[best];
        }
        for (int k = 0; k < top_k; ++k)
            wts[(size_t)t * top_k + k] = (float)(sc[idx[(size_t)t * top_k + k]] / sum);
        free(sc);
        free(b);
        free(taken);
    }
    return 0;
}

/* K3_TOPP on the output of k3o_route_select ([COLIBRI-K3] "Streaming design",
 * and its table of environment variables: keep the routed experts up to a
 * cumulative weight p, drop the low-weight tail of the top-k, renormalise;
 * p = 0 is off). The pages leave the order and the boundary open; this
 * library's reading:
 *   - the weights are the renormalised raw scores w_k = sc_k / sum, sum over
 *     the selected experts in selection order (double, as k3o_route_select);
 *   - the selected experts are taken largest weight first, equal weights in
 *     selection order;
 *   - an expert is kept when the weight taken before it (summed in that
 *     order, double) is still below p: the expert that reaches p is kept;
 *   - a dropped entry becomes idx -1, wts 0, in place (route order kept);
 *     kept entries get wts sc_k / (sum of the kept sc, selection order).
 * p <= 0 leaves the routing as it is. In place on idx and wts; the raw
 * scores are recomputed from the logits as k3o_route_select computes them. */
int k3o_route_topp(int32_t *idx, float *wts, const double *logits, int n_tokens, int n_experts,
                   int top_k, double p)
{
    if (n_tokens < 0 || n_experts <= 0 || top_k < 1 || top_k > n_experts || !(p >= 0.0))
        return -1;
    if (p == 0.0)
        return 0;
    for (int t = 0; t < n_tokens; ++t) {
        int32_t *id = idx + (size_t)t * top_k;
        float *w = wts + (size_t)t * top_k;
        double sc[64];
        int order[64];
        char keep[64];
        if (top_k > 64)
            return -1;
        double sum = 0.0;
        for (int k = 0; k < top_k; ++k) {
            if (id[k] < 0 || id[k] >= n_experts)
                return -1;
            sc[k] = 1.0 / (1.0 + exp(-logits[(size_t)t * n_experts + id[k]]));
            sum += sc[k];
            order[k] = k;
        }
        /* insertion sort by weight, largest first; equal weights keep
         * selection order (a later entry moves only past a smaller weight) */
        for (int a = 1; a < top_k; ++a) {
            const int o = order[a];
            int b = a;
            while (b > 0 && sc[order[b - 1]] / sum < sc[o] / sum) {
                order[b] = order[b - 1];
                --b;
            }
            order[b] = o;
        }
        double before = 0.0;
        for (int r = 0; r < top_k; ++r) {
            keep[order[r]] = before < p;
            before += sc[order[r]] / sum;
        }
        double kept = 0.0;
        for (int k = 0; k < top_k; ++k)
            if (keep[k])
                kept += sc[k];
        for (int k = 0; k < top_k; ++k) {
            if (keep[k]) {
                w[k] = (float)(sc[k] / kept);
            } else {
                id[k] = -1;
                w[k] = 0.0f;
            }
        }
    }
    return 0;
}

/* The MoE layer for given routing: y[t] = sum_k w[t][k] * E_{idx[t][k]}(x_t),
 * each expert output rounded to float, the weighted sum in double over k in
 * route order, rounded to float ([COLIBRI-K3] "Architecture notes": weights
 * are the renormalised raw scores; routed_scale 1.0 in [KIC-README]'s config).
 * The experts are passed as six pointer arrays indexed by expert id (entries
 * that no token selects may be NULL). An entry with idx -1 is a pair that
 * K3_TOPP dropped: it adds nothing (its ypair and hpair rows are zero).
 * Optional per-pair outputs ypair[t][k][latent] and hpair[t][k][inter]. */
int k3o_moe_layer(float *y, float *ypair, float *hpair, const float *x,
                  const int32_t *idx, const float *wts,
                  const uint8_t *const *w1p, const uint8_t *const *w1s,
                  const uint8_t *const *w3p, const uint8_t *const *w3s,
                  const uint8_t *const *w2p, const uint8_t *const *w2s,
                  int n_experts, int n_tokens, int top_k, int latent, int inter, int mode)
{
    init_tables();
    if (n_tokens < 0 || top_k < 1 || latent <= 0 || inter <= 0 ||
        latent % K3O_GROUP || inter % K3O_GROUP || (mode != K3O_EXACT && mode != K3O_IDOT))
        return -1;
    for (int i = 0; i < n_tokens * top_k; ++i) {
        const int e = idx[i];
        if (e == -1)
            continue;
        if (e < 0 || e >= n_experts || !w1p[e] || !w1s[e] || !w3p[e] || !w3s[e] || !w2p[e] || !w2s[e])
            return -2;
    }
    const int mx = latent > inter ? latent : inter;
    const int P = n_tokens * top_k;
    float *ye_all = malloc(sizeof(float) * (size_t)P * latent);
    float *h_all = malloc(sizeof(float) * (size_t)P * inter);
    /* pairs are independent; each is computed by one thread (inner gemvs then
     * run single-threaded inside the parallel region) */
#pragma omp parallel for schedule(dynamic, 1)
    for (int p = 0; p < P; ++p) {
        const int e = idx[p];
        const int t = p / top_k;
        if (e == -1) {
            memset(ye_all + (size_t)p * latent, 0, sizeof(float) * latent);
            memset(h_all + (size_t)p * inter, 0, sizeof(float) * inter);
            continue;
        }
        const k3o_expert ex = {w1p[e], w1s[e], w3p[e], w3s[e], w2p[e], w2s[e]};
        float *g = malloc(sizeof(float) * inter);
        float *u = malloc(sizeof(float) * inter);
        int8_t *qb = malloc((size_t)mx);
        float *sb = malloc(sizeof(float) * (size_t)(mx / K3O_GROUP));
        expert_one(ye_all + (size_t)p * latent, g, u, h_all + (size_t)p * inter,
                   x + (size_t)t * latent, &ex, latent, inter, mode, 4.0, 25.0, qb, sb);
        free(g);
        free(u);
        free(qb);
        free(sb);
    }
    for (int t = 0; t < n_tokens; ++t)
        for (int i = 0; i < latent; ++i) {
            double acc = 0.0;
            for (int k = 0; k < top_k; ++k)
                if (idx[(size_t)t * top_k + k] != -1)
                    acc += (double)wts[(size_t)t * top_k + k] *
                           (double)ye_all[((size_t)t * top_k + k) * latent + i];
            y[(size_t)t * latent + i] = (float)acc;
        }
    if (ypair)
        memcpy(ypair, ye_all, sizeof(float) * (size_t)P * latent);
    if (hpair)
        memcpy(hpair, h_all, sizeof(float) * (size_t)P * inter);
    free(ye_all);
    free(h_all);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* The LatentMoE block ([COLIBRI-K3] "Architecture notes", Stable LatentMoE;  */
/* [KIC-README] config: rms_eps 1e-5, latent_norm on the aggregate,           */
/* n_shared 2 added unweighted).                                              */
/* ------------------------------------------------------------------------ */

/* RMSNorm of one vector: n_i = a_i / sqrt(mean(a^2) + eps) * gamma_i, in
 * double, rounded to float. */
int k3o_rmsnorm(float *n, const float *a, const float *gamma, int len, double eps)
{
    if (len <= 0)
        return -1;
    double ss = 0.0;
    for (int i = 0; i < len; ++i)
        ss += (double)a[i] * (double)a[i];
    const double rms = sqrt(ss / (double)len + eps);
    for (int i = 0; i < len; ++i)
        n[i] = (float)((double)a[i] / rms * (double)gamma[i]);
    return 0;
}

/* out[t] = W_up * RMSNorm(layer(W_down x_t)) * gamma
 *        + sum_s W2_s * SiTU(W1_s x_t, W3_s x_t),
 * with routing computed on x_t (the router is [n_experts x hidden]).
 * Every inter-stage tensor (lat, agg, n, the shared g/u/h) is rounded to
 * float; the three addends of out are added in double. Optional stage
 * outputs: lat [T][latent], agg [T][latent], nrm_out [T][latent], idx/wts
 * [T][top_k], and onorm[t][i] = the tolerance normaliser of out (sum of
 * |W||a| over the three addends' last products). The w_up/W2 products'
 * normalisers include |W_up||n| and |W2_s||h_s|. */
int k3o_latent_block(float *out, float *lat, float *agg, float *nrm_out, double *onorm,
                     int32_t *idx, float *wts, const float *x,
                     const float *w_router, const float *bias,
                     const uint16_t *w_down, const uint16_t *w_up, const float *gamma,
                     const uint16_t *const *sh_w1, const uint16_t *const *sh_w3,
                     const uint16_t *const *sh_w2, int n_shared,
                     const uint8_t *const *w1p, const uint8_t *const *w1s,
                     const uint8_t *const *w3p, const uint8_t *const *w3s,
                     const uint8_t *const *w2p, const uint8_t *const *w2s,
                     int n_experts, int n_tokens, int top_k, int hidden, int latent,
                     int inter, int sh_inter, int mode, double eps)
{
    if (n_tokens < 0 || hidden <= 0 || latent <= 0 || sh_inter <= 0 || n_shared < 0)
        return -1;
    const size_t T = (size_t)n_tokens;
    double *logits = malloc(sizeof(double) * T * n_experts);
    float *latb = malloc(sizeof(float) * T * latent);
    float *aggb = malloc(sizeof(float) * T * latent);
    float *nb = malloc(sizeof(float) * T * latent);
    int32_t *ib = malloc(sizeof(int32_t) * T * top_k);
    float *wb = malloc(sizeof(float) * T * top_k);
    double *tmp = malloc(sizeof(double) * (size_t)(hidden > sh_inter ? hidden : sh_inter));
    double *tn = malloc(sizeof(double) * (size_t)(hidden > sh_inter ? hidden : sh_inter));
    double *acc = malloc(sizeof(double) * (size_t)hidden);
    double *accn = malloc(sizeof(double) * (size_t)hidden);
    float *gs = malloc(sizeof(float) * (size_t)sh_inter);
    float *us = malloc(sizeof(float) * (size_t)sh_inter);
    float *hs = malloc(sizeof(float) * (size_t)sh_inter);
    int rc = 0;

    rc |= k3o_route_logits(logits, x, w_router, n_tokens, hidden, n_experts);
    rc |= k3o_route_select(ib, wb, NULL, logits, bias, n_tokens, n_experts, top_k);
    for (size_t t = 0; t < T && !rc; ++t) {
        rc |= k3o_matmul_bf16(tmp, NULL, x + t * hidden, w_down, hidden, latent);
        for (int i = 0; i < latent; ++i)
            latb[t * latent + i] = (float)tmp[i];
    }
    if (!rc)
        rc |= k3o_moe_layer(aggb, NULL, NULL, latb, ib, wb, w1p, w1s, w3p, w3s, w2p, w2s,
                            n_experts, n_tokens, top_k, latent, inter, mode);
    for (size_t t = 0; t < T && !rc; ++t) {
        rc |= k3o_rmsnorm(nb + t * latent, aggb + t * latent, gamma, latent, eps);
        rc |= k3o_matmul_bf16(acc, accn, nb + t * latent, w_up, latent, hidden);
        for (int s = 0; s < n_shared; ++s) {
            k3o_matmul_bf16(tmp, NULL, x + t * hidden, sh_w1[s], hidden, sh_inter);
            for (int r = 0; r < sh_inter; ++r)
                gs[r] = (float)tmp[r];
            k3o_matmul_bf16(tmp, NULL, x + t * hidden, sh_w3[s], hidden, sh_inter);
            for (int r = 0; r < sh_inter; ++r)
                us[r] = (float)tmp[r];
            for (int r = 0; r < sh_inter; ++r)
                hs[r] = (float)k3o_situ((double)gs[r], (double)us[r], 4.0, 25.0);
            k3o_matmul_bf16(tmp, tn, hs, sh_w2[s], sh_inter, hidden);
            for (int i = 0; i < hidden; ++i) {
                acc[i] += tmp[i];
                accn[i] += tn[i];
            }
        }
        for (int i = 0; i < hidden; ++i) {
            out[t * hidden + i] = (float)acc[i];
            if (onorm)
                onorm[t * hidden + i] = accn[i];
        }
    }
    if (lat)
        memcpy(lat, latb, sizeof(float) * T * latent);
    if (agg)
        memcpy(agg, aggb, sizeof(float) * T * latent);
    if (nrm_out)
        memcpy(nrm_out, nb, sizeof(float) * T * latent);
    if (idx)
        memcpy(idx, ib, sizeof(int32_t) * T * top_k);
    if (wts)
        memcpy(wts, wb, sizeof(float) * T * top_k);
    free(logits); free(latb); free(aggb); free(nb); free(ib); free(wb);
    free(tmp); free(tn); free(acc); free(accn); free(gs); free(us); free(hs);
    return rc ? -1 : 0;
}
