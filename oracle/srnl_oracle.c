/*
 * srnl_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, single-threaded, double-precision CPU reference for the
 * forward pass of the stabilised SRNL operator over a 2-D feature grid with
 * four routes, row/column-aligned chunks and learned channel-scale fusion.
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * may load it. It shares no code, header, table or constant with the HIP
 * library; the two meet only in the tests, on the same seeded input bytes.
 *
 * Sources (web pages about VisionHOPE; cited by title and section):
 *   [README]   "VisionHOPE" README of github.com/PSRben/VisionHOPE:
 *              sections "Overview", "SRNL and VisionHOPE operator",
 *              "Fast inference".
 *   [OVERVIEW] "VisionHOPE Model Overview: Architecture, Benchmarks, and
 *              Practical Limits": sections "How VisionHOPE's Five Memories
 *              Work", "Four-Directional Scanning and Spatial Chunking",
 *              "Why the Stability Controls Matter".
 *   [SUMMARY]  "VisionHOPE: Visual Backbones as Self-Modifying Learning
 *              Systems" (arXiv 2609.33325 summary): the paragraphs on the
 *              write rule, on stabilisation, and on 2-D maps.
 *
 * The pages print no equation; every step below restates their prose, and
 * where they leave a detail open the plainest consistent reading is taken
 * (each is marked READING and listed in the design notes):
 *
 *   memories      per route and head: content, key and value matrices
 *                 M_c, M_k, M_v (d x d) and learning-rate / retention
 *                 vectors m_eta, m_alpha (length d); all five move on every
 *                 token [README Overview; SUMMARY write rule; OVERVIEW five
 *                 memories]. Stored as 3d+2 rows of length d.
 *   fresh start   every call starts from the given initial states [README
 *                 SRNL and VisionHOPE operator; OVERVIEW five memories].
 *   generation    at each chunk boundary the boundary states produce every
 *                 token's key, value, step size and retention [SUMMARY 2-D
 *                 maps; OVERVIEW scanning and chunking]:
 *                   k = B_k x, v = B_v x,
 *                   eta = sigmoid(b_eta . x),
 *                   alpha = alpha_max * sigmoid(b_alpha . x)   (READING)
 *   key norm      stabilised L2 normalisation k^ = k / sqrt(|k|^2 + eps)
 *                 [SUMMARY stabilisation]                      (READING)
 *   soft cap      e = k^ - v (key-value discrepancy), g = |e| |k^|,
 *                 eta' = (1-alpha) tanh(eta g / (1-alpha)) / g, so that
 *                 eta' g < 1 - alpha [SUMMARY stabilisation; OVERVIEW
 *                 stability controls]                          (READING)
 *   clamp         eta'' = min(eta', 2 alpha / |k^|^2), which makes the
 *                 retained transition alpha I - eta'' k^ k^T have spectral
 *                 norm <= alpha [SUMMARY stabilisation; OVERVIEW stability
 *                 controls]                                    (READING)
 *   write rule    retained Delta Gradient Descent [SUMMARY write rule]:
 *                 each memory maps the shared value through its own
 *                 boundary state (private target B v), takes the L2 loss
 *                 at the current key, 1/2 |M k^ - B v|^2, whose gradient at
 *                 the boundary is B (k^ - v) k^T = (B e) k^T; with the
 *                 residual correction against what the working memory
 *                 returns at the key, M k^ k^T, and retention alpha:
 *                   M <- alpha M - eta'' (M k^ + B e) k^T       (READING)
 *                 applied row by row to all 3d+2 rows, in token order
 *                 inside a chunk.
 *   readout       y_t = M_c q_t after token t's write; q = x unless given
 *                 [README SRNL and VisionHOPE operator]        (READING)
 *   routes        forward / reverse row-major, forward / reverse
 *                 column-major, each with its own states; chunk length W on
 *                 row routes and H on column routes unless overridden; the
 *                 last chunk may be short [OVERVIEW scanning and chunking;
 *                 SUMMARY 2-D maps; README chunk_size].
 *   fusion        outputs restored to their grid positions and combined
 *                 with learned per-channel scales, summed over the active
 *                 routes in ascending route order [OVERVIEW scanning and
 *                 chunking; SUMMARY 2-D maps]                  (READING)
 *
 * Variants (ablations named on the pages): hard injection clamp
 * min(eta, (1-alpha)/g) instead of the soft cap, no cap, no spectral
 * clamp, and frozen key/value and dynamics memories [SUMMARY ablation
 * paragraph]; fixed retention alpha = alpha_max and readout before the
 * write (alternative readings). With the memories frozen only the content
 * memory M_c is written; M_k, M_v, m_eta and m_alpha keep their initial
 * values for the whole scan, so every chunk generates from them.  (READING)
 *
 * Precision. The reference is this file built as is: every state, product
 * and sum in IEEE double. Built with -DSRNL_ORACLE_REAL=float, the same
 * steps keep their states, products and sums in IEEE single precision
 * (inputs rounded to float when read, libm results rounded to float). That
 * second build is no reference: the tests use it only to measure how far any
 * evaluation in fp32 can drift from the double result on a given chunk of
 * a given input (the conditioning of that chunk).
 */
#include <math.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>

#include "srnl_oracle.h"

#ifndef SRNL_ORACLE_REAL
#define SRNL_ORACLE_REAL double
#endif
typedef SRNL_ORACLE_REAL real;

/* Route traversal: token t of route r visits grid cell (i, j). */
void srnl_oracle_route_index(int r, int H, int W, long t, int *i, int *j)
{
    long N = (long)H * W;
    long s = (r == 1 || r == 3) ? (N - 1 - t) : t; /* reverse routes */
    if (r == 0 || r == 1) {                         /* row-major */
        *i = (int)(s / W);
        *j = (int)(s % W);
    } else {                                        /* column-major */
        *i = (int)(s % H);
        *j = (int)(s / H);
    }
}

/* Chunk length of route r: a full row (W) or a full column (H) unless a
 * positive override is given. */
int srnl_oracle_chunk_len(int r, int H, int W, int chunk_row, int chunk_col)
{
    if (r == 0 || r == 1)
        return chunk_row > 0 ? chunk_row : W;
    return chunk_col > 0 ? chunk_col : H;
}

static real sigmoid(real z) { return (real)1 / ((real)1 + (real)exp(-z)); }

static real dot(const real *a, const real *b, int n)
{
    real s = 0;
    for (int j = 0; j < n; ++j)
        s += a[j] * b[j];
    return s;
}

/* Per-token quantities produced from the boundary states. */
typedef struct {
    real *khat;   /* d */
    real *e;      /* d: khat - v */
    real *w;      /* 3d+2: boundary rows applied to e */
    real alpha, eta, eta1, eta2, g, nkh;
} token_gen;

/* Boundary generation for one token (any order inside a chunk). `bnd` holds
 * the 3d+2 boundary rows: rows [0,d) M_c, [d,2d) M_k, [2d,3d) M_v, 3d m_eta,
 * 3d+1 m_alpha. */
static void generate(const real *bnd, int d, const real *xt,
                     const srnl_oracle_opts *o, token_gen *g, real *scratch)
{
    const real *Bk = bnd + (size_t)d * d;
    const real *Bv = bnd + (size_t)2 * d * d;
    const real *beta = bnd + (size_t)3 * d * d;
    const real *balpha = beta + d;
    real *k = scratch, *v = scratch + d;
    int rows = 3 * d + 2;
    const real alpha_max = (real)o->alpha_max, eps = (real)o->eps;

    for (int i = 0; i < d; ++i) {
        k[i] = dot(Bk + (size_t)i * d, xt, d);   /* key memory generates k */
        v[i] = dot(Bv + (size_t)i * d, xt, d);   /* value memory generates v */
    }
    g->eta = sigmoid(dot(beta, xt, d));          /* learning-rate memory */
    g->alpha = o->fixed_alpha ? alpha_max
                              : alpha_max * sigmoid(dot(balpha, xt, d));

    real nk2 = dot(k, k, d);
    real inv = (real)1 / (real)sqrt(nk2 + eps);  /* stabilised L2 norm */
    for (int i = 0; i < d; ++i)
        g->khat[i] = k[i] * inv;
    for (int i = 0; i < d; ++i)
        g->e[i] = g->khat[i] - v[i];             /* key-value discrepancy */

    real nkh2 = dot(g->khat, g->khat, d);
    g->nkh = (real)sqrt(nkh2);
    g->g = (real)sqrt(dot(g->e, g->e, d)) * g->nkh;

    /* injection cap: keep eta' * g inside the margin 1 - alpha */
    real m = (real)1 - g->alpha;
    if (o->cap_mode == SRNL_ORACLE_CAP_SOFT) {
        g->eta1 = (g->g > 0) ? m * (real)tanh(g->eta * g->g / m) / g->g : g->eta;
    } else if (o->cap_mode == SRNL_ORACLE_CAP_HARD) {
        g->eta1 = (g->g > 0 && m / g->g < g->eta) ? m / g->g : g->eta;
    } else {
        g->eta1 = g->eta;
    }
    /* spectral clamp: |alpha - eta'' |k^|^2| <= alpha */
    g->eta2 = g->eta1;
    if (o->clamp && nkh2 > 0) {
        real cap = (real)2 * g->alpha / nkh2;
        if (cap < g->eta2)
            g->eta2 = cap;
    }
    /* L2 learning signal of every memory at the boundary: B e */
    for (int r = 0; r < rows; ++r)
        g->w[r] = dot(bnd + (size_t)r * d, g->e, d);
}

/* One retained-DGD step on the working rows: all 3d+2, or only the d rows
 * of M_c when the other memories are frozen. */
static void write_token(real *mem, int d, const token_gen *g, int freeze_kv)
{
    int rows = freeze_kv ? d : 3 * d + 2;
    for (int r = 0; r < rows; ++r) {
        real *m = mem + (size_t)r * d;
        real s = dot(m, g->khat, d) + g->w[r];    /* M k^ + B e */
        for (int j = 0; j < d; ++j)
            m[j] = g->alpha * m[j] - g->eta2 * s * g->khat[j];
    }
}

static double frob(const real *a, int n)
{
    double s = 0.0;
    for (int j = 0; j < n; ++j)
        s += (double)a[j] * a[j];
    return sqrt(s);
}

/* d consecutive input values, rounded to the working precision */
static void read_row(real *dst, const double *src, int d)
{
    for (int a = 0; a < d; ++a)
        dst[a] = (real)src[a];
}

int srnl_oracle_scan(const double *x, const double *q, int B, int H, int W,
                     int C, int heads, int d, unsigned route_mask,
                     const double *states, const srnl_oracle_opts *o,
                     double *y, double *trace)
{
    if (B < 1 || H < 1 || W < 1 || d < 1 || heads < 1 || C != heads * d ||
        route_mask < 1 || route_mask > 15 || !(o->alpha_max > 0.0) ||
        !(o->alpha_max < 1.0) || !(o->eps > 0.0) || o->chunk_row < 0 ||
        o->chunk_col < 0)
        return -1;

    const long N = (long)H * W;
    const int rows = 3 * d + 2;
    const size_t ssz = (size_t)rows * d;
    real *mem = malloc(ssz * sizeof(real));
    real *bnd = malloc(ssz * sizeof(real));
    real *scratch = malloc(2 * (size_t)d * sizeof(real));
    real *xt = malloc((size_t)d * sizeof(real));
    real *qt = malloc((size_t)d * sizeof(real));
    int Lmax = W > H ? W : H;
    if (o->chunk_row > Lmax) Lmax = o->chunk_row;
    if (o->chunk_col > Lmax) Lmax = o->chunk_col;
    if (Lmax > N) Lmax = (int)N;
    real *genbuf = malloc((size_t)Lmax * (2 * d + rows) * sizeof(real));
    token_gen *gen = malloc((size_t)Lmax * sizeof(token_gen));
    if (!mem || !bnd || !scratch || !xt || !qt || !genbuf || !gen) {
        free(mem); free(bnd); free(scratch); free(xt); free(qt);
        free(genbuf); free(gen);
        return -2;
    }
    for (int t = 0; t < Lmax; ++t) {
        real *base = genbuf + (size_t)t * (2 * d + rows);
        gen[t].khat = base;
        gen[t].e = base + d;
        gen[t].w = base + 2 * d;
    }

    int slot = 0;
    for (int r = 0; r < 4; ++r) {
        if (!(route_mask & (1u << r)))
            continue;
        const int L = srnl_oracle_chunk_len(r, H, W, o->chunk_row, o->chunk_col);
        for (int b = 0; b < B; ++b) {
            for (int h = 0; h < heads; ++h) {
                /* a fresh trajectory from this route's learned states */
                read_row(mem, states + ((size_t)r * heads + h) * ssz, (int)ssz);
                for (long c0 = 0; c0 < N; c0 += L) {
                    long nc = (N - c0 < L) ? (N - c0) : L;
                    memcpy(bnd, mem, ssz * sizeof(real)); /* boundary */
                    for (long u = 0; u < nc; ++u) {
                        int i, j;
                        srnl_oracle_route_index(r, H, W, c0 + u, &i, &j);
                        read_row(xt, x + (((size_t)b * H + i) * W + j) * C + (size_t)h * d, d);
                        generate(bnd, d, xt, o, &gen[u], scratch);
                    }
                    for (long u = 0; u < nc; ++u) {
                        long t = c0 + u;
                        int i, j;
                        srnl_oracle_route_index(r, H, W, t, &i, &j);
                        const double *src = q ? q : x;
                        read_row(qt, src + (((size_t)b * H + i) * W + j) * C + (size_t)h * d, d);
                        double *yt = y + (((size_t)slot * B + b) * N + t) * C + (size_t)h * d;
                        if (o->readout_before)
                            for (int a = 0; a < d; ++a)
                                yt[a] = dot(mem + (size_t)a * d, qt, d);
                        write_token(mem, d, &gen[u], o->freeze_kv);
                        if (!o->readout_before)
                            for (int a = 0; a < d; ++a)
                                yt[a] = dot(mem + (size_t)a * d, qt, d);
                        if (trace) {
                            double *tr = trace + ((((size_t)slot * B + b) * heads + h) * N + t) * SRNL_ORACLE_TRACE_W;
                            const size_t off[5] = {0, (size_t)d * d, (size_t)2 * d * d,
                                                   (size_t)3 * d * d, (size_t)3 * d * d + d};
                            const int len[5] = {d * d, d * d, d * d, d, d};
                            for (int m = 0; m < 5; ++m) {
                                tr[m] = frob(mem + off[m], len[m]);
                                tr[5 + m] = frob(bnd + off[m], len[m]);
                            }
                            const token_gen *g = &gen[u];
                            tr[10] = g->alpha;
                            tr[11] = g->eta;
                            tr[12] = g->eta1;
                            tr[13] = g->eta2;
                            tr[14] = g->g;
                            tr[15] = g->nkh;
                            tr[16] = fabs((double)(g->alpha - g->eta2 * g->nkh * g->nkh));
                            tr[17] = (double)u;
                        }
                    }
                }
            }
        }
        ++slot;
    }
    free(mem); free(bnd); free(scratch); free(xt); free(qt);
    free(genbuf); free(gen);
    return 0;
}

int srnl_oracle_fuse(const double *y, int B, int H, int W, int C,
                     unsigned route_mask, const double *scales, double *out)
{
    if (B < 1 || H < 1 || W < 1 || C < 1 || route_mask < 1 || route_mask > 15)
        return -1;
    const long N = (long)H * W;
    memset(out, 0, (size_t)B * N * C * sizeof(double));
    int slot = 0;
    for (int r = 0; r < 4; ++r) {           /* ascending route order */
        if (!(route_mask & (1u << r)))
            continue;
        for (int b = 0; b < B; ++b)
            for (long t = 0; t < N; ++t) {
                int i, j;
                srnl_oracle_route_index(r, H, W, t, &i, &j); /* restore */
                const double *yt = y + (((size_t)slot * B + b) * N + t) * C;
                double *o = out + (((size_t)b * H + i) * W + j) * C;
                for (int c = 0; c < C; ++c)
                    o[c] += scales[(size_t)r * C + c] * yt[c];
            }
        ++slot;
    }
    return 0;
}
