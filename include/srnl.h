/*
 * srnl.h -- C ABI of libsrnl.so: the forward pass of the stabilised SRNL
 * operator over a 2-D feature grid (four routes, row/column-aligned chunks,
 * learned channel-scale fusion) on AMD Instinct MI355X (gfx950), with its
 * backward pass, the standalone 1-D operator and one residual block around
 * the operator.
 *
 * Sources, cited by page title and section:
 *   [README]   "VisionHOPE" README (github.com/PSRben/VisionHOPE), sections
 *              "Overview", "SRNL and VisionHOPE operator", "Fast inference".
 *   [OVERVIEW] "VisionHOPE Model Overview: Architecture, Benchmarks, and
 *              Practical Limits", sections "How VisionHOPE's Five Memories
 *              Work", "Four-Directional Scanning and Spatial Chunking", "Why
 *              the Stability Controls Matter", "Fast Inference, Mixed
 *              Precision, and Evaluation", "Practical Limitations and Common
 *              Pitfalls".
 *   [SUMMARY]  "VisionHOPE: Visual Backbones as Self-Modifying Learning
 *              Systems" (arXiv 2609.33325 summary), paragraphs on the write
 *              rule, on stabilisation, on 2-D maps and on the ablations.
 *
 * Conventions for every entry point:
 *   - Tensors are device pointers (HBM) unless a comment says "host". The
 *     caller allocates and owns every buffer; the library never allocates
 *     or frees, keeps no state between calls, and does not wait for the
 *     stream (except under SRNL_FLAG_CHECK_FINITE).
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream)
 *     and runs asynchronously: a return of SRNL_OK means the arguments were
 *     valid and the kernels were launched.
 *   - Grids are NHWC: x[b][i][j][c], c fastest. Head h owns channels
 *     [h*d, (h+1)*d) [README SRNL and VisionHOPE operator].
 *   - Errors are returned as srnl_status; nothing throws across the ABI.
 *     srnl_last_error() gives a thread-local human-readable detail.
 *   - Empty grids (B, H or W equal to 0) are valid and launch nothing.
 *   - Tensor pointers must be 16-byte aligned (the kernels move 16-byte
 *     vectors); a misaligned one is SRNL_ERR_PTR. srnl_route_gather is the
 *     exception: it accepts any element-aligned view.
 */
#ifndef SRNL_H
#define SRNL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SRNL_OK = 0,
    SRNL_ERR_ARG = -1,       /* a size, mask, head_dim or scalar is invalid */
    SRNL_ERR_DTYPE = -2,     /* unknown dtype */
    SRNL_ERR_PTR = -3,       /* NULL, or not device memory where required */
    SRNL_ERR_WORKSPACE = -4, /* workspace missing or smaller than required */
    SRNL_ERR_HIP = -5,       /* a HIP runtime call or launch failed */
    SRNL_ERR_NONFINITE = -6  /* SRNL_FLAG_CHECK_FINITE found NaN or Inf (outputs are written) */
} srnl_status;

typedef enum { SRNL_F32 = 0, SRNL_BF16 = 1 } srnl_dtype;

/* Routes, in the order the pages list them [OVERVIEW Four-Directional
 * Scanning and Spatial Chunking]: bit 0 forward row-major, bit 1 reverse
 * row-major, bit 2 forward column-major, bit 3 reverse column-major. A
 * reverse route visits the whole sequence of its forward route backwards. */
#define SRNL_ROUTE_ROW      1u
#define SRNL_ROUTE_ROW_REV  2u
#define SRNL_ROUTE_COL      4u
#define SRNL_ROUTE_COL_REV  8u
#define SRNL_ROUTES_ALL     15u

/* Variant flags for srnl_params.flags. 0 is the operator as described:
 * soft injection cap, spectral clamp, retention from the retention memory,
 * readout after each token's write. The others are the ablations named in
 * [SUMMARY ablation paragraph] and alternative readings. */
#define SRNL_FLAG_HARD_CAP     0x1u  /* hard injection clamp min(eta, (1-alpha)/g) */
#define SRNL_FLAG_NO_CAP       0x2u  /* no injection cap */
#define SRNL_FLAG_NO_CLAMP     0x4u  /* no spectral clamp */
#define SRNL_FLAG_FIXED_ALPHA  0x8u  /* alpha = alpha_max for every token */
#define SRNL_FLAG_READ_BEFORE  0x10u /* y_t read before token t's write */
#define SRNL_FLAG_FREEZE_KV    0x20u /* only M_c is written; M_k, M_v, m_eta, m_alpha keep
                                        their initial values (frozen key/value and dynamics) */
/* Count NaN and Inf in x, q and the outputs of srnl_scan_fwd / srnl_scan_1d
 * and report them through the status (SRNL_ERR_NONFINITE). The count needs
 * a workspace of srnl_scan_workspace_bytes, and the call then waits for its
 * stream to finish. Other entry points ignore the flag. */
#define SRNL_FLAG_CHECK_FINITE 0x40u
/* Keep the forward's record for the backward pass (training). srnl_scan_fwd
 * (srnl_scan_1d) also writes, into params->workspace, the per-chain record
 * that the windowed backward reads (each chunk's boundary rows and closing
 * Q, and each 16-token window's opening Q, u rows and transition scalars);
 * srnl_scan_bwd (srnl_scan_1d_bwd) called with the same arguments, flags and
 * workspace then reads that record instead of recomputing it. Applies where
 * the windowed backward does: d = 32 with the readout after the write;
 * elsewhere, and in the other entry points, the flag changes nothing. The
 * record takes srnl_scan_workspace_bytes (srnl_scan_1d_workspace_bytes). */
#define SRNL_FLAG_RECORD 0x80u

/* Floats of initial state per (route, head): 3d^2 + 2d. */
#define SRNL_STATE_FLOATS(d) (3 * (d) * (d) + 2 * (d))

typedef struct {
    /* Learned initial states [README SRNL and VisionHOPE operator; OVERVIEW
     * How VisionHOPE's Five Memories Work], fp32, device,
     * [4 routes][heads][3d^2+2d]: M_c, M_k, M_v (row-major d x d), then
     * m_eta, m_alpha (length d). All four routes' slots are present even if
     * route_mask leaves some out. Every call starts from these states: each
     * forward pass begins a new sequence. */
    const float *states;
    /* Queries, same shape and dtype as x, or NULL for q = x [README SRNL and
     * VisionHOPE operator]. */
    const void *q;
    srnl_dtype in_dtype;  /* dtype of x and q; state and arithmetic are fp32 */
    float alpha_max;      /* retention ceiling, in (0, 1); alpha = alpha_max * sigmoid(m_alpha . x) */
    float eps;            /* > 0; key normalisation k / sqrt(|k|^2 + eps) */
    int chunk_row;        /* 0: chunk = W on row routes; > 0: that length (last chunk may be short) */
    int chunk_col;        /* 0: chunk = H on column routes; > 0: that length */
    unsigned flags;       /* SRNL_FLAG_* */
    void *stream;         /* hipStream_t */
    /* Device workspace for srnl_scan_fwd (srnl_scan_1d), at least
     * srnl_scan_workspace_bytes(...) (srnl_scan_1d_workspace_bytes(...))
     * bytes (that is 0, and this may be NULL, unless SRNL_FLAG_CHECK_FINITE or
     * SRNL_FLAG_RECORD is set), 16-byte aligned; caller-owned. With
     * SRNL_FLAG_RECORD it starts with the forward record, which srnl_scan_bwd
     * (srnl_scan_1d_bwd) reads from here; otherwise scratch. */
    void *workspace;
    size_t workspace_bytes;
} srnl_params;

/*
 * srnl_scan_fwd -- the SRNL scan along the active routes.
 *
 * Computes, for every active route r, batch b and head h, independently
 * [OVERVIEW Four-Directional Scanning and Spatial Chunking; SUMMARY 2-D
 * maps]: tokens are visited in route order; at each chunk boundary the
 * boundary states generate every token's key k = B_k x, value v = B_v x,
 * step size eta = sigmoid(b_eta . x) and retention alpha = alpha_max *
 * sigmoid(b_alpha . x); keys are normalised k^ = k / sqrt(|k|^2 + eps); the
 * step is soft-capped with the key-value discrepancy e = k^ - v and margin
 * 1 - alpha, then clamped to 2 alpha / |k^|^2 so the retained transition
 * stays within alpha [SUMMARY stabilisation; OVERVIEW Why the Stability
 * Controls Matter]; inside the chunk the five working memories update in
 * token order by retained delta gradient descent, M <- alpha M - eta''
 * (M k^ + B e) k^T [SUMMARY write rule]; the readout is y_t = M_c q_t after
 * the write.
 *
 *   x     [B][H][W][C], in_dtype, device. C must equal heads * d.
 *   d     head dim, one of 4, 8, 16, 32, 64 [README SRNL and VisionHOPE
 *         operator].
 *   route_mask  1..15 (SRNL_ROUTE_*).
 *   out   [R][B][H*W][C] fp32, device, R = popcount(route_mask): slot s
 *         holds the s-th active route (ascending bit order), tokens in
 *         that route's traversal order. Fully overwritten.
 * Errors: SRNL_ERR_ARG (C != heads*d, d not allowed, mask out of range,
 * negative sizes, alpha_max not in (0,1), eps <= 0, negative chunk,
 * sizes whose element counts overflow), SRNL_ERR_DTYPE, SRNL_ERR_PTR
 * (x, out or params->states NULL or not device memory; q not device
 * memory), SRNL_ERR_HIP; with SRNL_FLAG_CHECK_FINITE also SRNL_ERR_WORKSPACE
 * (workspace NULL or too small) and SRNL_ERR_NONFINITE (the detail string
 * gives the counts of non-finite inputs and outputs).
 */
srnl_status srnl_scan_fwd(const void *x, int B, int H, int W, int C, int heads,
                          int d, unsigned route_mask, const srnl_params *params,
                          float *out);

/*
 * srnl_scan_workspace_bytes -- device workspace srnl_scan_fwd needs in
 * params->workspace for these sizes and params: the forward record under
 * SRNL_FLAG_RECORD (where it applies), then 256 bytes for two counters
 * (non-finite input and output values) under SRNL_FLAG_CHECK_FINITE; 0
 * without either flag, for an empty grid or for invalid arguments.
 */
size_t srnl_scan_workspace_bytes(int B, int H, int W, int C, int heads, int d,
                                 unsigned route_mask, const srnl_params *params);

/*
 * srnl_scan_1d -- standalone 1-D SRNL [README SRNL and VisionHOPE operator]:
 * a sequence of N tokens scanned once, in token order, with the same write
 * rule, stabilisation and readout as srnl_scan_fwd. A new sequence starts at
 * every call. The default chunk is 64 tokens; a positive
 * params->chunk_row overrides it, and the last chunk may be short
 * [README SRNL and VisionHOPE operator]. params->chunk_col is ignored.
 *
 *   x      [B][N][C], in_dtype, device. C must equal heads * d.
 *   params->states  [heads][3d^2+2d] fp32, device (one block: the 1-D
 *          operator has a single direction).
 *   params->q       [B][N][C] in in_dtype, or NULL for q = x; separate
 *          queries must have the dtype of x [README Fast inference].
 *   out    [B][N][C] fp32, device. Fully overwritten.
 * Equal to srnl_scan_fwd on the 1 x N grid with route_mask = 1 and
 * chunk_row = the chunk above. Errors: as srnl_scan_fwd.
 */
srnl_status srnl_scan_1d(const void *x, int B, int N, int C, int heads, int d,
                         const srnl_params *params, float *out);

/*
 * srnl_scan_1d_workspace_bytes -- params->workspace srnl_scan_1d needs (the
 * record under SRNL_FLAG_RECORD, the counters under SRNL_FLAG_CHECK_FINITE),
 * with the 1-D chunk default applied: srnl_scan_workspace_bytes of the 1 x N
 * grid, route SRNL_ROUTE_ROW, chunk_row 64 when params->chunk_row is 0.
 * 0 for NULL params, an empty sequence or invalid arguments.
 */
size_t srnl_scan_1d_workspace_bytes(int B, int N, int C, int heads, int d,
                                    const srnl_params *params);

/*
 * srnl_fuse -- restore and fuse [OVERVIEW Four-Directional Scanning and
 * Spatial Chunking; SUMMARY 2-D maps]: each route's outputs go back to
 * their grid cells and are combined with learned per-channel scales,
 *   out[b][i][j][c] = sum over active r, ascending, of
 *                     scales[r][c] * y[slot(r)][b][t_r(i,j)][c]
 * where t_r(i,j) is the step at which route r visits cell (i, j).
 *
 *   y_routes  [R][B][H*W][C] fp32 as written by srnl_scan_fwd.
 *   scales    [4][C] fp32 (rows of inactive routes are ignored).
 *   out       [B][H][W][C] in out_dtype (bf16: round to nearest even).
 * Errors: SRNL_ERR_ARG, SRNL_ERR_DTYPE, SRNL_ERR_PTR, SRNL_ERR_HIP.
 */
srnl_status srnl_fuse(const float *y_routes, int B, int H, int W, int C,
                      unsigned route_mask, const float *scales,
                      srnl_dtype out_dtype, void *out, void *stream);

/*
 * Backward pass [README SRNL and VisionHOPE operator: the operator supports
 * training with autograd]. The gradients are those of the forward pass
 * above, in the same readings and variants (params are the forward's).
 *
 * srnl_scan_bwd_workspace_bytes -- bytes of device workspace srnl_scan_bwd
 * needs for these sizes (0 for an empty grid).
 *
 * srnl_scan_bwd -- given dy = dL/dy for the scan outputs, computes
 *   dx      [B][H][W][C] fp32 = dL/dx (overwritten; includes the query
 *           path when params->q is NULL, i.e. q = x);
 *   dq      [B][H][W][C] fp32 = dL/dq when params->q is not NULL
 *           (overwritten), else unused and may be NULL;
 *   dstates [4][heads][3d^2+2d] fp32 = dL/d(initial states), summed over
 *           the batch (overwritten; zero for inactive routes).
 *   dy      [R][B][H*W][C] fp32 in the layout srnl_scan_fwd writes.
 * At d = 32 with the readout after the write, a recording forward writes,
 * per chain, every chunk's boundary and closing state and every 16-token
 * window's opening state, update rows, transition scalars and window tables
 * into the workspace; the adjoint then walks the chunks and windows backwards, 16
 * tokens at a time. With SRNL_FLAG_RECORD the record comes instead from
 * params->workspace, written by srnl_scan_fwd with the same arguments and
 * params, and the workspace here holds only the rest (smaller
 * srnl_scan_bwd_workspace_bytes). Otherwise each chain re-runs the forward to record the
 * boundary of every chunk, then walks the chunks backwards, re-running each
 * chunk to record the working state after every token, and walks the tokens
 * backwards. Sums run in a fixed order (bitwise reproducible).
 * The workspace is caller-owned device memory of at least
 * srnl_scan_bwd_workspace_bytes(...) bytes; its contents are scratch.
 * Errors: as srnl_scan_fwd, plus SRNL_ERR_WORKSPACE, and SRNL_ERR_PTR for
 * missing dy, dx, dstates or (with separate queries) dq.
 */
size_t srnl_scan_bwd_workspace_bytes(int B, int H, int W, int C, int heads, int d,
                                     unsigned route_mask, const srnl_params *params);
srnl_status srnl_scan_bwd(const void *x, int B, int H, int W, int C, int heads, int d,
                          unsigned route_mask, const srnl_params *params,
                          const float *dy, void *workspace, size_t workspace_bytes,
                          float *dx, float *dq, float *dstates);

/*
 * srnl_scan_1d_bwd_workspace_bytes / srnl_scan_1d_bwd -- backward of
 * srnl_scan_1d [README SRNL and VisionHOPE operator: training with
 * autograd], with its 64-token chunk default (params->chunk_row 0): the
 * same as srnl_scan_bwd on the 1 x N grid with route_mask SRNL_ROUTE_ROW,
 * except for the layout of the state gradient.
 *   x, dx, dy  [B][N][C] (x in in_dtype; dx and dy fp32);
 *   dq         [B][N][C] fp32 when params->q is not NULL, else unused;
 *   dstates    [heads][3d^2+2d] fp32, the layout of the 1-D states
 *              (overwritten).
 * Under SRNL_FLAG_RECORD the record comes from params->workspace as written
 * by srnl_scan_1d with the same arguments and params.
 * Errors: as srnl_scan_bwd; SRNL_ERR_PTR for NULL params.
 */
size_t srnl_scan_1d_bwd_workspace_bytes(int B, int N, int C, int heads, int d,
                                        const srnl_params *params);
srnl_status srnl_scan_1d_bwd(const void *x, int B, int N, int C, int heads, int d,
                             const srnl_params *params, const float *dy, void *workspace,
                             size_t workspace_bytes, float *dx, float *dq, float *dstates);

/*
 * srnl_fuse_bwd_workspace_bytes / srnl_fuse_bwd -- backward of srnl_fuse:
 *   dy_routes[slot(r)][b][t][c] = scales[r][c] * dout[b][i][j][c] with
 *     (i, j) the cell route r visits at step t  (overwritten);
 *   dscales[r][c] = sum over b, t of y_routes[slot(r)][b][t][c] *
 *     dout[b][i][j][c]  (overwritten; zero rows for inactive routes).
 *   dout [B][H][W][C] fp32; y_routes, dy_routes [R][B][H*W][C] fp32;
 *   scales, dscales [4][C] fp32. Sums run in a fixed order (bitwise
 *   reproducible). Errors: SRNL_ERR_ARG, SRNL_ERR_PTR, SRNL_ERR_WORKSPACE,
 *   SRNL_ERR_HIP.
 */
size_t srnl_fuse_bwd_workspace_bytes(int B, int H, int W, int C, unsigned route_mask);
srnl_status srnl_fuse_bwd(const float *dout, const float *y_routes, int B, int H, int W,
                          int C, unsigned route_mask, const float *scales,
                          float *dy_routes, float *dscales, void *workspace,
                          size_t workspace_bytes, void *stream);

/*
 * srnl_scan_fuse_bwd_workspace_bytes / srnl_scan_fuse_bwd -- backward of the
 * whole operator, srnl_fuse after srnl_scan_fwd [README SRNL and VisionHOPE
 * operator: training with autograd; OVERVIEW Four-Directional Scanning and
 * Spatial Chunking: the routes' outputs fused with learned per-channel
 * scales], in one call: the results of srnl_fuse_bwd followed by
 * srnl_scan_bwd on its dy_routes, without dy_routes in memory where the
 * windowed d = 32 adjoint runs (d = 32, readout after the write): that
 * adjoint reads dout at the cells each route visits and multiplies by the
 * route's scales as it reads them (the same fp32 products, so dx, dq and
 * dstates are bitwise those of the two calls). Elsewhere dy_routes are
 * written to the workspace and the two calls' kernels run in turn.
 *   x, params   as srnl_scan_bwd (the forward's);
 *   y_routes    [R][B][H*W][C] fp32, the forward's route outputs;
 *   scales      [4][C] fp32, the fusion's scales;
 *   dout        [B][H][W][C] fp32 = dL/d(fused output);
 *   dx, dq, dstates  as srnl_scan_bwd (overwritten);
 *   dscales     [4][C] fp32 as srnl_fuse_bwd (overwritten).
 * All on params->stream. The workspace is caller-owned device memory of at
 * least srnl_scan_fuse_bwd_workspace_bytes(...) bytes (0 for an empty grid
 * or invalid arguments), 16-byte aligned; its contents are scratch. Sums run
 * in a fixed order (bitwise reproducible). Errors: as srnl_scan_bwd and
 * srnl_fuse_bwd (C <= 1024).
 */
size_t srnl_scan_fuse_bwd_workspace_bytes(int B, int H, int W, int C, int heads, int d,
                                          unsigned route_mask, const srnl_params *params);
srnl_status srnl_scan_fuse_bwd(const void *x, int B, int H, int W, int C, int heads, int d,
                               unsigned route_mask, const srnl_params *params,
                               const float *y_routes, const float *scales, const float *dout,
                               void *workspace, size_t workspace_bytes, float *dx, float *dq,
                               float *dstates, float *dscales);

/*
 * srnl_fuse_bwd_noalloc -- srnl_fuse_bwd for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving or training
 * loops, harnesses that forbid hipMalloc). It takes no workspace: the
 * partial sums go to a device array owned by the library, one per GPU, of
 * SRNL_FUSE_BWD_SCRATCH_BYTES, held until the process ends. The call
 * allocates nothing; its first call on a device looks up that device's
 * array. Results are bitwise those of srnl_fuse_bwd (same kernels, same
 * order). Calls that overlap on one GPU (other streams, other threads)
 * share the array and race: the caller serialises them. Errors: as
 * srnl_fuse_bwd; SRNL_ERR_WORKSPACE when the partial sums, R x
 * ceil(B*H*W / 256) x C x 4 bytes (srnl_fuse_bwd_workspace_bytes), exceed
 * SRNL_FUSE_BWD_SCRATCH_BYTES, e.g. B*H*W > 2,097,152 at four routes and
 * C = 64.
 */
#define SRNL_FUSE_BWD_SCRATCH_BYTES (8u << 20)
srnl_status srnl_fuse_bwd_noalloc(const float *dout, const float *y_routes, int B, int H,
                                  int W, int C, unsigned route_mask, const float *scales,
                                  float *dy_routes, float *dscales, void *stream);

/*
 * srnl_block_fwd -- one residual block around the operator [SUMMARY
 * paragraph on 2-D maps: a two-branch residual of a depthwise convolution
 * and SRNL, then a feed-forward network; OVERVIEW Four-Directional Scanning
 * and Spatial Chunking: one shared query projection supplies the readout
 * queries of every route, and the residual blocks hold projections,
 * normalisation, a depthwise convolution and a feed-forward network]:
 *   u   = LN1(x)                         per-token layer norm over C
 *   q   = u wq^T                         shared query projection, no bias
 *   s   = srnl_fuse(srnl_scan_fwd(u; q), scales)
 *   h   = x + DWConv3x3(u) + s           zero padding, with bias
 *   out = h + w2 GELU(w1 LN2(h) + b1) + b2   exact (erf) GELU
 * LN(z) = (z - mean) / sqrt(var + ln_eps) * gain + bias, biased variance.
 *   x, out  [B][H][W][C] in params->in_dtype (bf16 out is rounded to
 *           nearest even); the operator runs on u and q in fp32 with every
 *           other field of params (states, alpha_max, eps, chunks, flags,
 *           stream); params->q must be NULL.
 *   C in {32, 64, 128, 192, 256, 512} (512: the hierarchical model's last
 *   stage); ffn_hidden F a positive multiple of 32.
 *   wq, w1, w2 are bf16 words; the products are formed exactly from them
 *   and fp32 activations, accumulated in fp32.
 *   workspace: caller-owned device memory of srnl_block_workspace_bytes
 *   (u, q, s and the route outputs, and at C = 512 also h, all fp32).
 * Every pointer must be device memory, 16-byte aligned. Errors:
 * SRNL_ERR_ARG, SRNL_ERR_DTYPE, SRNL_ERR_PTR, SRNL_ERR_WORKSPACE,
 * SRNL_ERR_HIP.
 */
typedef struct {
    const float *ln1_w, *ln1_b;      /* [C] gain and bias of LN1 */
    const uint16_t *wq;              /* [C][C] bf16 */
    const float *dw_w, *dw_b;        /* [C][3][3] taps (row offset, column offset), [C] */
    const float *ln2_w, *ln2_b;      /* [C] */
    const uint16_t *w1;              /* [F][C] bf16 */
    const float *b1;                 /* [F] */
    const uint16_t *w2;              /* [C][F] bf16 */
    const float *b2;                 /* [C] */
    const float *scales;             /* [4][C] route fusion scales (as srnl_fuse) */
    int ffn_hidden;                  /* F */
    float ln_eps;                    /* > 0 */
} srnl_block_weights;

size_t srnl_block_workspace_bytes(int B, int H, int W, int C, unsigned route_mask);
srnl_status srnl_block_fwd(const void *x, int B, int H, int W, int C, int heads, int d,
                           unsigned route_mask, const srnl_params *params,
                           const srnl_block_weights *weights, void *workspace,
                           size_t workspace_bytes, void *out);

/*
 * srnl_route_gather -- the route traversal as a standalone copy [OVERVIEW
 * Four-Directional Scanning and Spatial Chunking]:
 *   out[slot(r)][b][t][c] = x[b][i][j][c],  (i, j) = route r's t-th cell.
 * srnl_scan_fwd performs the same gather inside its load stage; this entry
 * point exposes it for callers (and for bit-exact checks).
 *   x    [B][H][W][C] in dtype;  out  [R][B][H*W][C] in dtype.
 * Errors: SRNL_ERR_ARG, SRNL_ERR_DTYPE, SRNL_ERR_PTR, SRNL_ERR_HIP.
 */
srnl_status srnl_route_gather(const void *x, int B, int H, int W, int C,
                              unsigned route_mask, srnl_dtype dtype, void *out,
                              void *stream);

/*
 * srnl_init_states -- fill the learned-initial-state buffer [README SRNL
 * and VisionHOPE operator; OVERVIEW How VisionHOPE's Five Memories Work]
 * with std * N(0,1) entries, deterministically from `seed`:
 *   states  [4][heads][3d^2+2d] fp32, device.
 * Entry n is normal n of stream 2 of the counter-based generator
 * Philox4x32-10 (Salmon et al., SC'11) keyed by seed: block k uses counter
 * (k mod 2^32, k div 2^32, 2, 0x53524E4C); its words a0..a3 give
 * u(a) = (a + 0.5) 2^-32 and, by Box-Muller in double precision, normals
 * 4k..4k+3 = r0 cos t0, r0 sin t0, r1 cos t1, r1 sin t1 with
 * r = sqrt(-2 ln u(a0 or a2)), t = 2 pi u(a1 or a3).
 * Errors: SRNL_ERR_ARG (heads < 1, d not allowed, std < 0 or not finite),
 * SRNL_ERR_PTR, SRNL_ERR_HIP.
 */
srnl_status srnl_init_states(float *states, int heads, int d,
                             unsigned long long seed, float std, void *stream);

/* Host helpers (no device work). */

/* Cell (i, j) visited at step t of route r (0..3) on an H x W grid; host. */
void srnl_route_index(int r, int H, int W, long t, int *i, int *j);
/* Chunk length route r uses: W or H unless the override is > 0; host. */
int srnl_chunk_len(int r, int H, int W, int chunk_row, int chunk_col);
const char *srnl_status_string(srnl_status s);
/* Detail of the last error on the calling thread ("" if none). */
const char *srnl_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* SRNL_H */
