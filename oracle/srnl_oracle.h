/*
 * srnl_oracle.h -- TEST INFRASTRUCTURE ONLY: the double-precision CPU
 * reference of the four-route SRNL forward pass (see srnl_oracle.c for the
 * sources it follows). Not part of the HIP library; shares nothing with it.
 */
#ifndef SRNL_ORACLE_H
#define SRNL_ORACLE_H

#ifdef __cplusplus
extern "C" {
#endif

enum { SRNL_ORACLE_CAP_SOFT = 0, SRNL_ORACLE_CAP_HARD = 1, SRNL_ORACLE_CAP_OFF = 2 };

/* Diagnostics per (route slot, b, head, token), when a trace buffer is given:
 * [0..4] Frobenius norms of M_c, M_k, M_v, m_eta, m_alpha after the write;
 * [5..9] the same for the chunk's boundary snapshot;
 * [10] alpha, [11] eta, [12] eta after the cap, [13] eta after the clamp,
 * [14] g = |e| |k^|, [15] |k^|, [16] |alpha - eta'' |k^|^2|,
 * [17] position of the token inside its chunk. */
#define SRNL_ORACLE_TRACE_W 18

typedef struct {
    double alpha_max;   /* retention ceiling, in (0, 1) */
    double eps;         /* key-normalisation stabiliser, > 0 */
    int chunk_row;      /* 0: W on row routes, else the override */
    int chunk_col;      /* 0: H on column routes, else the override */
    int cap_mode;       /* SRNL_ORACLE_CAP_* */
    int clamp;          /* 1: spectral clamp on */
    int fixed_alpha;    /* 1: alpha = alpha_max */
    int readout_before; /* 1: y_t read before token t's write */
    int freeze_kv;      /* 1: only M_c is written; M_k, M_v, m_eta, m_alpha stay */
} srnl_oracle_opts;

void srnl_oracle_route_index(int r, int H, int W, long t, int *i, int *j);
int srnl_oracle_chunk_len(int r, int H, int W, int chunk_row, int chunk_col);

/* x, q: [B,H,W,C] (q may be NULL: q = x). states: [4][heads][3d^2+2d] rows
 * M_c, M_k, M_v (row-major d x d), m_eta, m_alpha. y: [R][B][H*W][C] in
 * traversal order, R = active routes ascending. trace: NULL or
 * [R][B][heads][H*W][SRNL_ORACLE_TRACE_W]. Returns 0, -1 (bad argument) or
 * -2 (out of memory). */
int srnl_oracle_scan(const double *x, const double *q, int B, int H, int W,
                     int C, int heads, int d, unsigned route_mask,
                     const double *states, const srnl_oracle_opts *opts,
                     double *y, double *trace);

/* out[b,i,j,c] = sum over active routes r (ascending) of
 * scales[r][c] * y[slot(r)][b][t][c] with route r's token t at (i, j). */
int srnl_oracle_fuse(const double *y, int B, int H, int W, int C,
                     unsigned route_mask, const double *scales, double *out);

#ifdef __cplusplus
}
#endif
#endif
