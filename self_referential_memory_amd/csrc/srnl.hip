// srnl.hip -- libsrnl.so: HIP kernels for gfx950 and the C ABI of
// include/srnl.h (forward pass of the stabilised SRNL operator over a 2-D
// grid: four routes, row/column-aligned chunks, channel-scale fusion).
//
// Sources, cited by page title and section:
//   [README]   "VisionHOPE" README: "SRNL and VisionHOPE operator",
//              "Fast inference".
//   [OVERVIEW] "VisionHOPE Model Overview: Architecture, Benchmarks, and
//              Practical Limits": "How VisionHOPE's Five Memories Work",
//              "Four-Directional Scanning and Spatial Chunking", "Why the
//              Stability Controls Matter".
//   [SUMMARY]  "VisionHOPE: Visual Backbones as Self-Modifying Learning
//              Systems": paragraphs on the write rule, stabilisation, 2-D
//              maps.
//
// Kernel map:
//   scan_mfma_kernel (d = 32, 64) and scan_simple_kernel (d = 4, 8, 16):
//                  one workgroup per chain (route, batch, head). Per chunk:
//                  gathers the chunk's tokens along the route (the route
//                  gather fused into the load), generates every token's key,
//                  value, step and retention from the boundary states,
//                  normalises keys, applies the soft cap and spectral clamp,
//                  runs the token-order update, reads out, and refreshes the
//                  boundary. The five memories are carried in "Q-form": inside
//                  a chunk every memory equals its boundary value times one
//                  shared d x d matrix Q (Q = I at the boundary), because the
//                  write rule M <- alpha M - eta'' (M k^ + B e) k^T keeps
//                  M = B Q with Q <- alpha Q - eta'' (Q k^ + e) k^T. This is
//                  the reading of the fast-inference recurrence [README Fast
//                  inference; OVERVIEW scanning and chunking: readouts and
//                  update quantities come from the boundary memories, token
//                  contributions accumulate in order, memories refresh at the
//                  chunk boundary]. Readout y_t = B_c (Q_t q_t); refresh
//                  M = B Q_L.
//   fuse_kernel    restore each route's outputs to grid order and combine
//                  them with per-channel scales.
//   gather_kernel  the route traversal as a standalone copy.
//   init_kernel    Philox4x32-10 + Box-Muller initial states.
#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <string>
#include <type_traits>

#include "srnl.h"

namespace {

thread_local std::string g_last_error;

srnl_status fail(srnl_status s, const std::string &msg)
{
    g_last_error = msg;
    return s;
}

// ------------------------------------------------------------ device helpers

__device__ __forceinline__ float bf16_to_f32(uint16_t w)
{
    return __uint_as_float(static_cast<uint32_t>(w) << 16);
}

__device__ __forceinline__ uint16_t f32_to_bf16(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu))
        return static_cast<uint16_t>((u >> 16) | 0x40u);   // quiet NaN
    u += 0x7FFFu + ((u >> 16) & 1u);                        // nearest, ties even
    return static_cast<uint16_t>(u >> 16);
}

template <typename T> __device__ __forceinline__ float load_in(const T *p, size_t i);
template <> __device__ __forceinline__ float load_in<float>(const float *p, size_t i) { return p[i]; }
template <> __device__ __forceinline__ float load_in<uint16_t>(const uint16_t *p, size_t i)
{
    return bf16_to_f32(p[i]);
}

// Cell (i, j) that route r visits at step t [OVERVIEW Four-Directional
// Scanning and Spatial Chunking]: routes 0/1 row-major forward/reverse,
// 2/3 column-major forward/reverse; reverse = whole sequence backwards.
__device__ __forceinline__ void route_cell(int r, int H, int W, long long N,
                                           long long t, int &i, int &j)
{
    long long s = (r & 1) ? (N - 1 - t) : t;
    if (r < 2) {
        i = static_cast<int>(s / W);
        j = static_cast<int>(s - static_cast<long long>(i) * W);
    } else {
        j = static_cast<int>(s / H);
        i = static_cast<int>(s - static_cast<long long>(j) * H);
    }
}

// Step at which route r visits cell (i, j): the inverse of route_cell.
__device__ __forceinline__ long long route_step(int r, int H, int W, long long N,
                                                int i, int j)
{
    long long s = (r < 2) ? static_cast<long long>(i) * W + j
                          : static_cast<long long>(j) * H + i;
    return (r & 1) ? (N - 1 - s) : s;
}

__device__ __forceinline__ int nth_route(unsigned mask, int slot)
{
    for (int r = 0; r < 4; ++r)
        if (mask & (1u << r)) {
            if (slot == 0)
                return r;
            --slot;
        }
    return 0;
}

// Sum over the 4 lanes of an aligned quad; every lane gets the total.
__device__ __forceinline__ float quad_sum(float v)
{
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false)); // xor 1
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false)); // xor 2
    return v;
}

// 1 / (1 + e^-z) as the reciprocal of 1 + 2^(-z log2 e) (v_exp_f32,
// v_rcp_f32): within 4 + 2|z| ulp, the |z| part from rounding the argument
__device__ __forceinline__ float sigmoidf(float z)
{
    return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(z * -1.4426950408889634f));
}

// tanh(u) for u >= 0, branch-free: below 0.3 the odd Taylor polynomial
// through u^13 (the first term left out is under 1e-10 of the value there),
// above it (1 - e) / (1 + e) with e = exp(-2u), where 1 - e >= 0.45 and so
// loses nothing to cancellation; within 6 ulp with an exact exp2.
__device__ __forceinline__ float tanh_pos(float u)
{
    const float u2 = u * u;
    float p = 21844.0f / 6081075.0f;
    p = fmaf(p, u2, -1382.0f / 155925.0f);
    p = fmaf(p, u2, 62.0f / 2835.0f);
    p = fmaf(p, u2, -17.0f / 315.0f);
    p = fmaf(p, u2, 2.0f / 15.0f);
    p = fmaf(p, u2, -1.0f / 3.0f);
    const float ts = fmaf(u * u2, p, u);
    const float e = __builtin_amdgcn_exp2f(u * -2.8853900817779268f);   // exp(-2u)
    const float tl = (1.0f - e) * __builtin_amdgcn_rcpf(1.0f + e);
    return u < 0.3f ? ts : tl;
}

// Workgroups are dispatched round-robin over the 8 XCDs (blockIdx % 8 picks
// the XCD); give each XCD a contiguous range of chains so that chains that
// read the same pixels (same batch item, other heads / routes) share that
// XCD's L2. nblocks is a multiple of 8.
__device__ __forceinline__ int xcd_remap(int bid, int nblocks)
{
    int per = nblocks >> 3;
    return (bid & 7) * per + (bid >> 3);
}

// ------------------------------------------------------------ scan kernel, d <= 16
//
// Plain VALU version for the small head dims: every contraction is a loop
// over LDS, one output per thread.

template <int D> struct ScanCfg {
    static constexpr int NT = (4 * D < 64) ? 64 : 4 * D;  // threads per workgroup
    static constexpr int TB = 32;                          // tokens per sub-block
    static constexpr int ROWS = 3 * D + 2;                 // rows of the five memories
    static constexpr int LDP = D + 1;                      // padded LDS row stride
    static constexpr int CPL = D / 4;                      // Q columns per lane
    static constexpr int NREF = (ROWS * D + NT - 1) / NT;  // refresh outputs per thread
};

enum : unsigned {
    F_HARD_CAP = 0x1u, F_NO_CAP = 0x2u, F_NO_CLAMP = 0x4u, F_FIXED_ALPHA = 0x8u,
    F_READ_BEFORE = 0x10u, F_FREEZE_KV = 0x20u, F_CHECK_FINITE = 0x40u,
    F_RECORD = 0x80u
};

template <int D, typename InT>
__global__ __launch_bounds__(ScanCfg<D>::NT) void scan_simple_kernel(
    const InT *__restrict__ x, const InT *__restrict__ q,
    const float *__restrict__ states, float *__restrict__ out, int B, int H,
    int W, int C, int heads, unsigned route_mask, int R, float alpha_max,
    float eps, int chunk_row, int chunk_col, unsigned flags, int nchains)
{
    using Cfg = ScanCfg<D>;
    constexpr int NT = Cfg::NT, TB = Cfg::TB, ROWS = Cfg::ROWS, LDP = Cfg::LDP,
                  CPL = Cfg::CPL, NREF = Cfg::NREF;

    __shared__ float Bs[ROWS * LDP];   // boundary states (rows of M_c, M_k, M_v, m_eta, m_alpha)
    __shared__ float Xs[TB * LDP];     // chunk tokens x_t
    __shared__ float Qx[TB * LDP];     // separate queries q_t (when given)
    __shared__ float Ks[TB * LDP];     // k, then k^
    __shared__ float Es[TB * LDP];     // v, then e = k^ - v
    __shared__ float Zs[TB * LDP];     // z_t = Q_t q_t
    __shared__ float Sa[TB];           // pre-activation, then alpha_t
    __shared__ float Se[TB];           // pre-activation, then eta''_t
    __shared__ float Qm[D * LDP];      // Q at the chunk end

    const int chain = xcd_remap(blockIdx.x, gridDim.x);
    if (chain >= nchains)
        return;
    const int slot = chain % R;
    const int bh = chain / R;
    const int h = bh % heads;
    const int b = bh / heads;
    const int r = nth_route(route_mask, slot);
    const long long N = static_cast<long long>(H) * W;
    long long L = (r < 2) ? (chunk_row > 0 ? chunk_row : W)
                          : (chunk_col > 0 ? chunk_col : H);
    if (L > N)
        L = N;

    const int tid = threadIdx.x;
    const float *st = states + (static_cast<size_t>(r) * heads + h) * (ROWS * D);
    for (int idx = tid; idx < ROWS * D; idx += NT)
        Bs[(idx / D) * LDP + idx % D] = st[idx];

    // token-loop layout: row `qrow` of Q, columns [part*CPL, part*CPL+CPL)
    const int qrow = tid >> 2;
    const int part = tid & 3;
    const bool qactive = qrow < D;
    float P[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c)
        P[c] = (part * CPL + c == qrow) ? 1.0f : 0.0f;

    const float *qtile = q ? Qx : Xs;
    const size_t out_base = static_cast<size_t>(slot) * B + b;

    for (long long c0 = 0; c0 < N; c0 += L) {
        const long long cend = (c0 + L < N) ? c0 + L : N;
        __syncthreads();   // boundary rows in Bs are complete
        for (long long s0 = c0; s0 < cend; s0 += TB) {
            const int nt = static_cast<int>((cend - s0 < TB) ? cend - s0 : TB);

            // (1) gather this sub-block's tokens along the route
            for (int idx = tid; idx < nt * D; idx += NT) {
                const int u = idx / D, c = idx % D;
                int i, j;
                route_cell(r, H, W, N, s0 + u, i, j);
                const size_t off = ((static_cast<size_t>(b) * H + i) * W + j) * C +
                                   static_cast<size_t>(h) * D + c;
                Xs[u * LDP + c] = load_in(x, off);
                if (q)
                    Qx[u * LDP + c] = load_in(q, off);
            }
            __syncthreads();

            // (2) boundary generation: k = B_k x, v = B_v x, b_eta . x, b_alpha . x
            for (int idx = tid; idx < nt * (2 * D + 2); idx += NT) {
                const int u = idx / (2 * D + 2), o = idx % (2 * D + 2);
                const float *brow = Bs + (D + o) * LDP;
                const float *xu = Xs + u * LDP;
                float acc = 0.0f;
#pragma unroll 8
                for (int jj = 0; jj < D; ++jj)
                    acc = fmaf(brow[jj], xu[jj], acc);
                if (o < D)
                    Ks[u * LDP + o] = acc;
                else if (o < 2 * D)
                    Es[u * LDP + (o - D)] = acc;
                else if (o == 2 * D)
                    Se[u] = acc;
                else
                    Sa[u] = acc;
            }
            __syncthreads();

            // (3) per-token transition scalars: key normalisation, soft cap,
            //     spectral clamp [SUMMARY stabilisation]
            for (int u = tid; u < nt; u += NT) {
                float *k = Ks + u * LDP;
                float *e = Es + u * LDP;
                float nk2 = 0.0f;
                for (int jj = 0; jj < D; ++jj)
                    nk2 = fmaf(k[jj], k[jj], nk2);
                const float inv = 1.0f / sqrtf(nk2 + eps);
                float nkh2 = 0.0f, ne2 = 0.0f;
                for (int jj = 0; jj < D; ++jj) {
                    const float kh = k[jj] * inv;
                    const float ev = kh - e[jj];
                    k[jj] = kh;
                    e[jj] = ev;
                    nkh2 = fmaf(kh, kh, nkh2);
                    ne2 = fmaf(ev, ev, ne2);
                }
                const float eta = sigmoidf(Se[u]);
                const float alpha = (flags & F_FIXED_ALPHA) ? alpha_max
                                                            : alpha_max * sigmoidf(Sa[u]);
                const float g = sqrtf(ne2) * sqrtf(nkh2);
                const float m = 1.0f - alpha;
                float eta1 = eta;
                if (flags & F_NO_CAP) {
                    eta1 = eta;
                } else if (flags & F_HARD_CAP) {
                    if (g > 0.0f && m < eta * g)
                        eta1 = m / g;
                } else if (g > 0.0f) {
                    const float uu = eta * g / m;
                    eta1 = (uu < 1e-3f) ? eta * (1.0f - uu * uu * (1.0f / 3.0f))
                                        : m * tanh_pos(uu) / g;
                }
                float eta2 = eta1;
                if (!(flags & F_NO_CLAMP) && nkh2 > 0.0f) {
                    const float cap = 2.0f * alpha / nkh2;
                    if (cap < eta2)
                        eta2 = cap;
                }
                Sa[u] = alpha;
                Se[u] = eta2;
            }
            __syncthreads();

            // (4) token-order update in Q-form and z_t = Q_t q_t
            if (qactive) {
                const bool before = (flags & F_READ_BEFORE) != 0;
                for (int u = 0; u < nt; ++u) {
                    const float *kh = Ks + u * LDP + part * CPL;
                    const float *qq = qtile + u * LDP + part * CPL;
                    float kv[CPL];
#pragma unroll
                    for (int c = 0; c < CPL; ++c)
                        kv[c] = kh[c];
                    if (before) {
                        float z = 0.0f;
#pragma unroll
                        for (int c = 0; c < CPL; ++c)
                            z = fmaf(P[c], qq[c], z);
                        z = quad_sum(z);
                        if (part == 0)
                            Zs[u * LDP + qrow] = z;
                    }
                    float dot = 0.0f;
#pragma unroll
                    for (int c = 0; c < CPL; ++c)
                        dot = fmaf(P[c], kv[c], dot);
                    dot = quad_sum(dot);
                    const float alpha = Sa[u];
                    const float s = Se[u] * (dot + Es[u * LDP + qrow]);
#pragma unroll
                    for (int c = 0; c < CPL; ++c)
                        P[c] = fmaf(-s, kv[c], alpha * P[c]);
                    if (!before) {
                        float z = 0.0f;
#pragma unroll
                        for (int c = 0; c < CPL; ++c)
                            z = fmaf(P[c], qq[c], z);
                        z = quad_sum(z);
                        if (part == 0)
                            Zs[u * LDP + qrow] = z;
                    }
                }
            }
            __syncthreads();

            // (5) readout y_t = B_c z_t, written in traversal order
            for (int idx = tid; idx < nt * D; idx += NT) {
                const int u = idx / D, i = idx % D;
                const float *bc = Bs + i * LDP;
                const float *z = Zs + u * LDP;
                float acc = 0.0f;
#pragma unroll 8
                for (int jj = 0; jj < D; ++jj)
                    acc = fmaf(bc[jj], z[jj], acc);
                out[(out_base * N + s0 + u) * C + static_cast<size_t>(h) * D + i] = acc;
            }
            __syncthreads();
        }

        // (6) boundary refresh M = B Q_L for the next chunk
        if (cend < N) {
            if (qactive) {
#pragma unroll
                for (int c = 0; c < CPL; ++c)
                    Qm[qrow * LDP + part * CPL + c] = P[c];
            }
            __syncthreads();
            // frozen key/value and dynamics memories: only M_c is refreshed
            const int nref = (flags & F_FREEZE_KV) ? D * D : ROWS * D;
            float acc[NREF];
#pragma unroll
            for (int k = 0; k < NREF; ++k) {
                const int idx = tid + k * NT;
                float a = 0.0f;
                if (idx < nref) {
                    const int rr = idx / D, jj = idx % D;
                    const float *brow = Bs + rr * LDP;
#pragma unroll 8
                    for (int kk = 0; kk < D; ++kk)
                        a = fmaf(brow[kk], Qm[kk * LDP + jj], a);
                }
                acc[k] = a;
            }
            __syncthreads();
#pragma unroll
            for (int k = 0; k < NREF; ++k) {
                const int idx = tid + k * NT;
                if (idx < nref)
                    Bs[(idx / D) * LDP + idx % D] = acc[k];
            }
#pragma unroll
            for (int c = 0; c < CPL; ++c)
                P[c] = (part * CPL + c == qrow) ? 1.0f : 0.0f;
        }
    }
}

// ------------------------------------------------------------ scan kernel, d = 32, 64
//
// One workgroup of NW waves per chain; T tokens per sub-block (a chunk is
// processed in sub-blocks of at most T tokens: generation inside a chunk reads
// only the fixed boundary states, so it may be split), and each sub-block in
// windows of 16 tokens.
//
//   load      tokens of the next sub-block are prefetched into registers
//             (16-byte loads along the route) while the current one computes
//   generate  [k | v] = X [B_k; B_v]^T on MFMA (v_mfma_f32_16x16x4f32)
//   epilogue  NT/T lanes per token: |k|^2, b_eta . x, b_alpha . x, k^, e, the
//             soft cap and the spectral clamp (DPP group reductions)
//   windows   one wave per 16-token window: key/key and query/key Gram
//             matrices on MFMA, retention products, and the window's
//             triangular system (below)
//   update    the token-order update of a window as dense products on MFMA;
//             the rows of Q are independent, so wave w owns rows
//             16w .. 16w+15 of Q (held transposed, in MFMA accumulators) and
//             the waves never exchange data inside a sub-block
//   readout   Y = Z B_c^T on MFMA, z_t = Q_t q_t
//   refresh   B <- B Q_L on MFMA (the two vector memories on VALU)
//
// Windowed form of the update. Write the update of one token as
// Q_t = alpha_t Q_{t-1} + u_t k^_t^T with u_t = -eta''_t (Q_{t-1} k^_t + e_t).
// Over a window that starts from Q_0, with local products
// G_t = alpha_0 ... alpha_t (G_{-1} = 1) and R[t][s] = alpha_{s+1} ... alpha_t
// (R[t][t] = 1):
//   Q_t = G_t Q_0 + sum_{s<=t} R[t][s] u_s k^_s^T,
// so the u_s solve the unit lower-triangular system
//   u_t + sum_{s<t} L[t][s] u_s = -eta''_t (G_{t-1} Q_0 k^_t + e_t),
//   L[t][s] = eta''_t R[t-1][s] (k^_s . k^_t),
// i.e. U = T' (A + E) with T' = (I + L)^-1 diag(-eta''), A[t] = G_{t-1} Q_0 k^_t.
// Then z_t = Q_t q_t = G_t Q_0 q_t + sum_{s<=t} R[t][s] (k^_s . q_t) u_s and
// Q_16 = G_15 Q_0 + sum_s R[15][s] u_s k^_s^T. Every product is exact
// algebra of the token-order recurrence; only the summation order differs.
// Ratios of retention products are never formed (R is built from products of
// the alphas themselves), so tiny retentions need no rescaling. Padding
// tokens of a short window carry alpha = 1, eta'' = 0, k^ = e = q = 0 and
// change nothing.
//
// MFMA 16x16x4 f32 operand layout (lane l, lm = l % 16, lk = l / 16):
// A[lm][k], B[k][lm], D[4 lk + r][lm] in accumulator register r. Over the four
// instructions r = 0..3 of one 16-wide block of the reduction index, lane l
// supplies reduction index 4 lk + r, so an accumulator tile can serve directly
// as the B operand of a product that contracts over its row index, and a lane's
// A or B operands from a [row][reduction] array are one 16-byte read.
// [token][channel] arrays have row stride d + 4 floats, [channel][token]
// arrays T + 4, the per-window 16 x 16 tables 20: 16-byte aligned rows whose
// 16-byte reads by 8 consecutive lanes hit distinct banks.

typedef float v4f __attribute__((ext_vector_type(4)));

__device__ __forceinline__ v4f mfma4(float a, float b, v4f c)
{
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// bf16 operands of v_mfma_f32_16x16x32_bf16: 8 per lane. Lane l supplies
// reduction indices k = 8 (l / 16) + e, e = 0..7, for both operands.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Eight floats that are exactly representable in bf16, packed as bf16.
__device__ __forceinline__ bf16x8 pack_bf16_exact(const float (&v)[8])
{
    u32x4 w;
#pragma unroll
    for (int k = 0; k < 4; ++k)
        w[k] = (__float_as_uint(v[2 * k]) >> 16) | (__float_as_uint(v[2 * k + 1]) & 0xFFFF0000u);
    return __builtin_bit_cast(bf16x8, w);
}

// Exact split of eight floats into three bf16 parts, v = hi + mid + lo:
// truncation to bf16 keeps the leading 8 significant bits, so three parts
// hold all 24 bits of an fp32 significand (each residual is exact in fp32).
__device__ __forceinline__ void split3_bf16(const float (&v)[8], bf16x8 &hi, bf16x8 &mid, bf16x8 &lo)
{
    u32x4 wh, wm, wl;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        uint32_t h[2], m[2], l[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const float x = v[2 * k + e];
            h[e] = __float_as_uint(x) & 0xFFFF0000u;
            const float r = x - __uint_as_float(h[e]);
            m[e] = __float_as_uint(r) & 0xFFFF0000u;
            const float r2 = r - __uint_as_float(m[e]);
            l[e] = __float_as_uint(r2) & 0xFFFF0000u;
        }
        wh[k] = (h[0] >> 16) | h[1];
        wm[k] = (m[0] >> 16) | m[1];
        wl[k] = (l[0] >> 16) | l[1];
    }
    hi = __builtin_bit_cast(bf16x8, wh);
    mid = __builtin_bit_cast(bf16x8, wm);
    lo = __builtin_bit_cast(bf16x8, wl);
}

// c += A B over one 16-wide block of the reduction index (4 instructions)
__device__ __forceinline__ v4f mfma16(const float4 &a, const float4 &b, v4f c)
{
    c = mfma4(a.x, b.x, c);
    c = mfma4(a.y, b.y, c);
    c = mfma4(a.z, b.z, c);
    c = mfma4(a.w, b.w, c);
    return c;
}
__device__ __forceinline__ v4f mfma16(const float4 &a, const v4f &b, v4f c)
{
    c = mfma4(a.x, b[0], c);
    c = mfma4(a.y, b[1], c);
    c = mfma4(a.z, b[2], c);
    c = mfma4(a.w, b[3], c);
    return c;
}

template <int D, int NW_, int T, bool HAS_Q, bool DEF = false> struct MCfg {
    static constexpr int NW = NW_;                 // waves per chain
    static constexpr int NT = NW * 64;             // threads
    static constexpr int ROWS = 3 * D + 2;
    // [row][channel] arrays: at d = 32 with sub-blocks of 64 or 128 tokens,
    // unpadded rows whose 16-byte blocks are XOR-swizzled by the row
    // (swz_row); else rows padded by 4 floats (for the two-wave sub-blocks
    // the swizzle's address arithmetic costs more than the conflicts it saves)
    static constexpr bool SWZ = D == 32 && T >= 64;
    static constexpr int LDP = SWZ ? D : D + 4;    // [row][channel] row stride
    static constexpr int KS = D / 4;               // MFMA K-steps over d
    static constexpr int NTC = D / 16;             // 16-wide column tiles of d
    static constexpr int NWIN = T / 16;            // windows per sub-block
    static constexpr int EPL = NT / T;             // epilogue lanes per token
    static constexpr int ECPL = D / EPL;           // channels per epilogue lane
    // token columns of the e rows: the sub-block's, at least 32, except that
    // the 16-token sub-block at d = 32 keeps 16 (which brings its LDS
    // footprint under a sixth of the CU's: six chains a CU)
    static constexpr int TE = (D == 32 && T == 16) ? 16 : (T > 32 ? T : 32);
    static constexpr int ETS = TE + 4;             // [channel][token] row stride
    static constexpr int WS = 20;                  // row stride of the per-window L tables
    // row stride of the per-window N tables: as WS, except with separate
    // queries in the long sub-blocks at d = 32, where unpadded rows let the T'
    // tables share the v rows and keep the footprint within half a CU's LDS
    // (two chains per CU) at the cost of 2-way conflicts on one read per window
    static constexpr int NS = (HAS_Q && SWZ) ? 16 : WS;
    static constexpr int JS = (NW >= 2 * NTC) ? 2 : 1;   // waves sharing 16 rows of Q
    static constexpr int NJ = NTC / JS;            // 16-column tiles of Q per wave
    static constexpr int CW = NTC * JS;            // waves in the token-order update
    static_assert(T % 16 == 0 && T <= 128, "sub-block of whole windows");
    static_assert(EPL * T == NT && EPL >= 2 && EPL <= 16 && ECPL % 4 == 0, "epilogue lanes");
    static_assert(NW >= NTC, "one wave per 16 rows of Q");
    static_assert(NTC % JS == 0 && CW <= NW, "column split over whole tiles");
    static_assert(NT >= 4 * D, "vector-memory refresh: at least two lanes per output");

    // LDS pool (floats). Arrays that are dead in a phase lend their space:
    // the k rows (dead after the epilogue, until the update writes z) hold
    // the windows' L tables; the v rows (dead after the epilogue) hold the
    // N tables, the T' tables when they fit too, and at a chunk end Q_L^T
    // when it fits.
    static constexpr int SZ_TOK = T * LDP;
    static constexpr int SZ_LC = NWIN * 16 * WS;
    static constexpr int SZ_NN = NWIN * 16 * NS;
    static constexpr int SZ_TP = NWIN * 256;
    static constexpr int SZ_QT = D * LDP;
    static_assert(SZ_LC <= SZ_TOK && SZ_NN <= SZ_TOK, "window tables fit");
    static constexpr bool TP_IN_ES = SZ_NN + SZ_TP <= SZ_TOK;
    // Window-local tables: with the long sub-blocks at d = 32 each wave's
    // epilogue covers exactly the 16 tokens of the window whose tables the
    // same wave builds (EPL = 4, one window per wave), so no block barrier
    // is needed between the two phases if every window's tables live in
    // that window's own dead k and v rows (16 rows of LDP floats): L in its
    // k rows, N (and T', when it shares the v rows) in its v rows.
    static constexpr bool WL = SWZ && EPL == 4 && NWIN == NW;
    static constexpr int WSTR_L = WL ? 16 * LDP : 16 * WS;   // L table stride per window
    static constexpr int WSTR_N = WL ? 16 * LDP : 16 * NS;   // N table stride per window
    static_assert(!WL || (16 * WS <= 16 * LDP && 16 * NS + (TP_IN_ES ? 256 : 0) <= 16 * LDP),
                  "window tables fit the window's rows");
    // (with DEF, the deferred refresh of M_c, Q_L^T keeps an array of its
    // own: it is read again in the next sub-block's table phase)
    static constexpr bool QT_IN_ES = !DEF && SZ_QT <= SZ_TOK;
    // else, when it fits, over the x, k/z, v and k^ rows (contiguous), which
    // are dead at a chunk end once the readout has read the z rows
    static constexpr bool QT_IN_TOK = !DEF && !QT_IN_ES && SZ_QT <= 4 * SZ_TOK;
    static constexpr int O_BS = 0;
    static constexpr int O_XS = O_BS + ROWS * LDP;
    static constexpr int O_KZ = O_XS + SZ_TOK;
    static constexpr int O_ES = O_KZ + SZ_TOK;
    static constexpr int O_KH = O_ES + SZ_TOK;
    static constexpr int O_ET = O_KH + SZ_TOK;
    static constexpr int O_AL = O_ET + D * ETS;
    static constexpr int O_EH = O_AL + T;
    static constexpr int O_GA = O_EH + T;
    static constexpr int O_GZ = O_GA + T;
    static constexpr int O_RB = O_GZ + T;
    static constexpr int O_WG = O_RB + T;
    static constexpr int O_PI = O_WG + (NWIN + 3) / 4 * 4;
    static constexpr int O_XB = O_PI + T;
    static constexpr int SZ_XB = (JS == 2) ? 2 * NTC * 512 : 0;
    static constexpr int O_KZ2 = O_XB + SZ_XB;
    static constexpr int O_QV = O_KZ2 + ((JS == 2) ? SZ_TOK : 0);
    static constexpr int O_TPX = O_QV + (HAS_Q ? SZ_TOK : 0);     // T' tables, if not in v rows
    static constexpr int O_TP = TP_IN_ES ? O_ES + (WL ? 16 * NS : SZ_NN) : O_TPX;
    static constexpr int WSTR_T = (TP_IN_ES && WL) ? 16 * LDP : 256;   // T' table stride per window
    static constexpr int O_QTX = O_TPX + (TP_IN_ES ? 0 : SZ_TP);  // Q_L^T, if on its own
    static constexpr int O_QT = QT_IN_ES ? O_ES : QT_IN_TOK ? O_XS : O_QTX;
    static constexpr int POOL = O_QTX + ((QT_IN_ES || QT_IN_TOK) ? 0 : SZ_QT);
};

// Index of T'[s][t] in a window's 16 x 16 table: rows of 16 floats, the four
// 16-byte groups of a row rotated by (s >> 1) & 3 so that the 16-byte reads
// of 8 consecutive rows hit distinct banks.
__device__ __forceinline__ int tp_index(int s, int t)
{
    return s * 16 + ((((t >> 2) ^ (s >> 1)) & 3) << 2) + (t & 3);
}

// Swizzle of the 16-byte blocks of row `row` in the unpadded [row][channel]
// arrays of the scan kernel's long sub-blocks at d = 32: block b of the row
// is stored at block b ^ swz_row(row).
// Chosen with a model of the LDS banks (128-bit reads: 64 banks, 16 lanes a
// cycle, a half-wave's quads split by the parity of the quad index; 128-bit
// writes: 32 banks, 8 consecutive lanes; 32-bit accesses: 32 banks, 32
// lanes) so that every row access of the scan kernel is free of bank
// conflicts: 16 lanes on 16 rows at one column block, 16 rows at two column
// blocks, 4 or 8 lanes per row on consecutive blocks, and 32-bit column
// accesses of 4 rows x 16 channels.
__device__ __forceinline__ int swz_row(int row)
{
    // [0, 4, 6, 2][(row >> 2) & 3] | (bit 0 ^ bit 1 of row)
    return ((0x2640 >> (((row >> 2) & 3) << 2)) & 0xF) | ((row ^ (row >> 1)) & 1);
}

// 16-byte vector of input elements
template <typename InT> struct InVec { static constexpr int VE = 16 / sizeof(InT); };

__device__ __forceinline__ void unpack(const uint4 &w, float (&f)[4], const float *)
{
    f[0] = __uint_as_float(w.x);
    f[1] = __uint_as_float(w.y);
    f[2] = __uint_as_float(w.z);
    f[3] = __uint_as_float(w.w);
}
__device__ __forceinline__ void unpack(const uint4 &w, float (&f)[8], const uint16_t *)
{
    const uint32_t a[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        f[2 * k] = __uint_as_float(a[k] << 16);
        f[2 * k + 1] = __uint_as_float(a[k] & 0xFFFF0000u);
    }
}

// Sum over an aligned group of G lanes (G = 2, 4 or 8) with DPP adds.
template <int G> __device__ __forceinline__ float group_sum(float v)
{
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, true)); // xor 1
    if (G >= 4)
        v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, true)); // xor 2
    if (G >= 8)   // row_half_mirror: lane i <- lane 7-i within each group of 8
        v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, true));
    if (G >= 16)  // row_mirror: lane i <- lane 15-i within each row of 16
        v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, true));
    return v;
}

// 32-bit form of route_cell (the host guarantees H * W < 2^31).
__device__ __forceinline__ void route_cell32(int r, int H, int W, int N, int t, int &i, int &j)
{
    const unsigned s = static_cast<unsigned>((r & 1) ? (N - 1 - t) : t);
    if (r < 2) {
        i = static_cast<int>(s / static_cast<unsigned>(W));
        j = static_cast<int>(s - static_cast<unsigned>(i) * W);
    } else {
        j = static_cast<int>(s / static_cast<unsigned>(H));
        i = static_cast<int>(s - static_cast<unsigned>(j) * H);
    }
}

// n consecutive floats from LDS (16-byte aligned) into registers
template <int n> __device__ __forceinline__ void lds_load(const float *p, float (&r)[n])
{
    static_assert(n % 4 == 0, "");
#pragma unroll
    for (int k = 0; k < n / 4; ++k) {
        const float4 v = reinterpret_cast<const float4 *>(p)[k];
        r[4 * k] = v.x;
        r[4 * k + 1] = v.y;
        r[4 * k + 2] = v.z;
        r[4 * k + 3] = v.w;
    }
}

__device__ __forceinline__ float4 ld4(const float *p) { return *reinterpret_cast<const float4 *>(p); }
__device__ __forceinline__ void st4(float *p, float a, float b, float c, float d)
{
    *reinterpret_cast<float4 *>(p) = make_float4(a, b, c, d);
}

// Order this wave's LDS writes before its later LDS reads by other lanes of
// the same wave (LDS operations of one wave complete in issue order).
__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Value of the lane N places lower in the same 16-lane row; 1 where that
// lane lies outside the row (DPP row_shr with the old value kept).
template <int N> __device__ __forceinline__ float row_shr_fill1(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(1.0f), __float_as_int(v),
                                                      0x110 + N, 0xF, 0xF, false));
}

// Value of lane `src` (0..3) of each aligned quad, in every lane of the quad.
__device__ __forceinline__ float quad_bcast(float v, int src)
{
    const int ctrl = src * 0x55;   // quad_perm [src, src, src, src]
    switch (ctrl) {
    case 0x00: return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x00, 0xF, 0xF, false));
    case 0x55: return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x55, 0xF, 0xF, false));
    case 0xAA: return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xAA, 0xF, 0xF, false));
    default: return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xFF, 0xF, 0xF, false));
    }
}

// Per-chain record of the forward that the windowed backward reads (SAVE):
// every chunk's boundary rows and closing Q_L, and every 16-token window's
// opening Q_0 (neither at d = 64, see SaveLayout), its u_t rows, its tokens'
// transition scalars and its window tables (windows counted from each chunk
// start). Scalars of a token, 16 floats: 1/sqrt(|k|^2 + eps), |k^|^2, |e|^2,
// g, eta, alpha, 1 - alpha, u = eta g / (1 - alpha), eta', eta'', the branch
// bits (SCB_*), and the five coefficients of the backward through these
// scalars (written with them). Window tables (TW_* offsets, TW floats): the
// k^ and e rows [16][D] (zero on padding tokens), the Grams k^_s . k^_t and
// q_t . k^_s and R[t][s] (masked: 1 on the diagonal, 0 above), each [t][s],
// T = (I + L)^-1 transposed ([s][t]), R[t-1][s] (k^_s . k^_t) (s < t) and
// R[t][s] (q_t . k^_s) (s <= t), each [t][s], then G_t, G_{t-1} and R[15][s].
// Chains are chain_floats apart; inside a chain the layout depends on the
// route's chunk count nch and window slots per chunk nwc.
struct FwdSave {
    float *base = nullptr;
    long long chain_floats = 0;
};
// At d = 64 the record serves chunks of one window only: every window opens
// its chunk (Q_0 = I) and the forward refreshes the boundary without forming
// Q_L, so the record holds no Q_0 or Q_L there (the backward rebuilds Q_L
// from the window's u and k^ rows).
template <int D> struct SaveLayout {
    static constexpr long long BR = (3LL * D + 2) * D;   // boundary rows
    static constexpr bool QREC = D != 64;                // Q_0 and Q_L recorded
    static constexpr long long QD = QREC ? D * D : 0;
    static constexpr int TW_KH = 0, TW_E = 16 * D, TW_KK = 32 * D, TW_QK = TW_KK + 256,
                         TW_R = TW_QK + 256, TW_T = TW_R + 256, TW_LF = TW_T + 256,
                         TW_NF = TW_LF + 256, TW_G = TW_NF + 256, TW_GP = TW_G + 16,
                         TW_PI = TW_GP + 16, TW = TW_PI + 16 + 16;
    long long nch, nwc;
    __host__ __device__ long long o_bnd(long long c) const { return c * BR; }
    __host__ __device__ long long o_ql(long long c) const { return nch * BR + c * QD; }
    __host__ __device__ long long o_q0(long long c, long long w) const {
        return nch * (BR + QD) + (c * nwc + w) * QD;
    }
    __host__ __device__ long long o_u(long long c, long long w) const {
        return nch * (BR + QD) + nch * nwc * QD + (c * nwc + w) * 16 * D;
    }
    __host__ __device__ long long o_sc(long long c, long long w) const {
        return nch * (BR + QD) + nch * nwc * (QD + 16 * D) + (c * nwc + w) * 256;
    }
    __host__ __device__ long long o_tab(long long c, long long w) const {
        return nch * (BR + QD) + nch * nwc * (QD + 16 * D + 256) + (c * nwc + w) * TW;
    }
    __host__ __device__ long long floats() const {
        return nch * (BR + QD + nwc * (QD + 16 * D + 256 + TW));
    }
};
// branch bits of a recorded token: soft-cap series, hard cap taken, clamp taken
constexpr int SCB_SERIES = 1, SCB_HARD = 2, SCB_CLAMP = 4;

// Phase clocks (a separate build with -DSRNL_PHASE_CLOCKS=1, never the
// library itself): wave 0 of every scan block reads the shader clock right
// after each phase's closing barrier and accumulates the cycles per phase in
// srnl_phase_buf[block][0 .. kPhaseSlots - 3], then the count of sub-blocks
// (windows in the backward) [kPhaseSlots - 2] and the whole block's cycles
// [kPhaseSlots - 1]; srnl_phase_clocks copies them out. The forward scan's
// phases: load, generation, epilogue, window tables, update, readout,
// refresh. The windowed backward's: chunk start (loads), commit, generation,
// transition scalars, forward tables, backward tables, the Gin recurrence,
// the per-token gradients in three parts (products; row dots and tables;
// dalpha, z, dq, dk), scalar chain, generation backward, chunk start
// (refresh terms).
#ifndef SRNL_PHASE_CLOCKS
#define SRNL_PHASE_CLOCKS 0
#endif
#if SRNL_PHASE_CLOCKS
constexpr int kPhaseBlocks = 16384, kPhaseSlots = 15;
__device__ unsigned long long srnl_phase_buf[kPhaseBlocks * kPhaseSlots];
// (the per-phase sums live in LDS, ph_lds, added to by lane 0 of wave 0
// without waiting for a return, so the stamps cost the instrumented kernel
// no registers beyond the last clock reading)
#define SRNL_PHASE(k)                                                                \
    do {                                                                             \
        if (wave == 0) {                                                             \
            const unsigned long long t_ = clock64();                                 \
            if (lane == 0)                                                           \
                atomicAdd(&ph_lds[k], static_cast<unsigned>(t_ - ph_t));             \
            ph_t = t_;                                                               \
        }                                                                            \
    } while (0)
#else
#define SRNL_PHASE(k) ((void)0)
#endif

template <int D, int NW, int T, bool BEFORE, bool HAS_Q, typename InT, bool SAVE = false,
          bool OUT = !SAVE>
__global__ __launch_bounds__(NW * 64, (D == 32 && T == 16 && !SAVE && !HAS_Q) ? 3 : 1) void scan_mfma_kernel(
    const InT *__restrict__ x, const InT *__restrict__ q,
    const float *__restrict__ states, float *__restrict__ out, int B, int H,
    int W, int C, int heads, unsigned route_mask, int R, float alpha_max,
    float eps, int chunk_row, int chunk_col, unsigned flags, int nchains, FwdSave sv)
{
    // The refresh of M_c (the readout memory) is deferred to the next
    // sub-block's table phase in the long sub-blocks at d = 32: the next
    // chunk's generation and epilogue read only M_k, M_v and the vector
    // memories, and its readout, the first reader of M_c, comes after its
    // update. The chunk end then refreshes 8 of the 12 tiles.
    static constexpr bool DEFER_MC = D == 32 && T >= 64 && !SAVE && OUT && !HAS_Q;
    using Cfg = MCfg<D, NW, T, HAS_Q, DEFER_MC>;
    constexpr int NT = Cfg::NT, ROWS = Cfg::ROWS, LDP = Cfg::LDP, KS = Cfg::KS,
                  NTC = Cfg::NTC, ETS = Cfg::ETS, WS = Cfg::WS, NS = Cfg::NS, JS = Cfg::JS, NJ = Cfg::NJ,
                  CW = Cfg::CW, NWIN = Cfg::NWIN;
    constexpr int VE = InVec<InT>::VE;
    constexpr int SEGS = D / VE;                       // 16-byte segments per token
    constexpr int NPF = (T * SEGS + NT - 1) / NT;      // prefetch registers per thread
    constexpr int RT = (3 * D / 16) * NTC;             // refresh tiles (matrix memories)

    __shared__ __align__(16) float pool[Cfg::POOL];
    float *const Bs = pool + Cfg::O_BS;    // boundary rows M_c, M_k, M_v, m_eta, m_alpha
    float *const Xs = pool + Cfg::O_XS;    // x_t rows
    float *const KZ = pool + Cfg::O_KZ;    // k rows (generation), then z_t rows (readout)
    float *const Lc = pool + Cfg::O_KZ;    // per window L [t][s] (window tables)
    float *const Es = pool + Cfg::O_ES;    // v rows (generation)
    float *const Nn = pool + Cfg::O_ES;    // per window N [t][s] (window tables, update)
    float *const Tp = pool + Cfg::O_TP;    // per window T', tp_index layout
    float *const KHa = pool + Cfg::O_KH;   // k^_t rows
    float *const Et = pool + Cfg::O_ET;    // e = k^ - v, [channel][token]
    float *const AL = pool + Cfg::O_AL;    // alpha_t (1 on padding tokens)
    float *const EH = pool + Cfg::O_EH;    // eta''_t (0 on padding tokens)
    float *const GA = pool + Cfg::O_GA;    // G_{t-1}
    float *const GZ = pool + Cfg::O_GZ;    // readout scale: G_t (G_{t-1} when reading before the write)
    float *const RB = pool + Cfg::O_RB;    // R[15][t] of the token's window
    float *const WG = pool + Cfg::O_WG;    // G_15 per window
    float *const PI = pool + Cfg::O_PI;    // G_t (window tables)
    float *const XB = pool + Cfg::O_XB;    // partial products exchanged between column halves
    float *const KZ2 = pool + Cfg::O_KZ2;  // second partial sum of the z_t rows (JS = 2)
    float *const QVa = pool + Cfg::O_QV;   // separate query rows q_t (HAS_Q)
    float *const Qt = pool + Cfg::O_QT;    // Q_L^T at a chunk end
    const float *const QR = HAS_Q ? QVa : Xs;   // query rows
    // Offset of element (row, c) of a [row][channel] array (x, k/z, v, k^,
    // query and boundary rows, Q_L^T); c % 4 is kept, so aligned groups of 4
    // channels stay contiguous.
    auto ix = [](int row, int c) {
        return row * LDP + (Cfg::SWZ ? (c ^ (swz_row(row) << 2)) : c);
    };
    // n consecutive channels c0.. (c0 % 4 == 0) of one row into registers
    auto ldrow = [&](const float *base, int row, int c0, auto &r) {
        constexpr int n = sizeof(r) / sizeof(float);
        static_assert(n % 4 == 0, "whole 16-byte blocks");
#pragma unroll
        for (int k = 0; k < n / 4; ++k) {
            const float4 v = ld4(base + ix(row, c0 + 4 * k));
            r[4 * k] = v.x;
            r[4 * k + 1] = v.y;
            r[4 * k + 2] = v.z;
            r[4 * k + 3] = v.w;
        }
    };
    // Token column of e in its [channel][token] layout, XOR-swizzled by the
    // epilogue lane that stores the channel: those lanes each store ECPL
    // consecutive channels of one token, and unswizzled the lanes of a
    // half-wave would share LDS banks. The XOR is a multiple of 4 below TE,
    // so aligned groups of 4 tokens stay contiguous and in the row.
    constexpr int EPL = Cfg::EPL, ECPL = Cfg::ECPL, TE = Cfg::TE;
    constexpr int ET_SW = (32 / EPL < 4) ? 4 : 32 / EPL;
    auto et_col = [](int row, int u) {
        if constexpr (TE == 16)   // (by groups of 8 channels: no bank shared by the storing lanes)
            return u ^ (((row / 8) & 3) << 2);
        else
            return u ^ ((((row / ECPL) & (EPL - 1)) * ET_SW) & (TE - 4));
    };

    const int chain = xcd_remap(blockIdx.x, gridDim.x);
    if (chain >= nchains)
        return;
    const int slot = chain % R;
    const int bh = chain / R;
    const int h = bh % heads;
    const int b = bh / heads;
    const int r = nth_route(route_mask, slot);
    const int N = H * W;
    int L = (r < 2) ? (chunk_row > 0 ? chunk_row : W) : (chunk_col > 0 ? chunk_col : H);
    if (L > N)
        L = N;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int lm = lane & 15, lk = lane >> 4;        // MFMA operand row / k block

    const float *st = states + (static_cast<size_t>(r) * heads + h) * (ROWS * D);
    for (int idx = tid; idx < ROWS * D; idx += NT)
        Bs[ix(idx / D, idx % D)] = st[idx];

    const size_t xbase = static_cast<size_t>(b) * N * C + static_cast<size_t>(h) * D;
    uint4 pre[NPF], preq[NPF];
    auto issue_loads = [&](int s, int n) {
#pragma unroll
        for (int k = 0; k < NPF; ++k) {
            const int seg = tid + k * NT;
            if (seg < n * SEGS) {
                const int u = seg / SEGS, sg = seg % SEGS;
                int i, j;
                route_cell32(r, H, W, N, s + u, i, j);
                const size_t off = xbase + static_cast<size_t>(i * W + j) * C + sg * VE;
                pre[k] = *reinterpret_cast<const uint4 *>(x + off);
                if (HAS_Q)
                    preq[k] = *reinterpret_cast<const uint4 *>(q + off);
            }
        }
    };

    // Q^T of this wave's block of Q (wave < CW, it = wave % NTC, jg = wave / NTC):
    // tile jl holds Q^T[16 jt + 4 lk + i][16 it + lm] in register i, with
    // jt = jg NJ + jl. Q = I at a boundary.
    v4f qacc[NJ];
    auto reset_q = [&]() {
        const int it = wave % NTC, jg = wave / NTC;
#pragma unroll
        for (int jl = 0; jl < NJ; ++jl)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                qacc[jl][i] = (16 * (jg * NJ + jl) + 4 * lk + i == 16 * it + lm) ? 1.0f : 0.0f;
    };
    reset_q();
    // Q_L^T into LDS for the boundary refresh (waves < CW)
    auto stage_qt = [&]() {
        const int it = wave % NTC, jg = wave / NTC;
#pragma unroll
        for (int jl = 0; jl < NJ; ++jl)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                Qt[ix(16 * (jg * NJ + jl) + 4 * lk + i, 16 * it + lm)] = qacc[jl][i];
    };
    // With two waves per 16 rows of Q, every window ends in a block barrier
    // after the window's table reads, so Q_L^T can be staged at the end of the
    // update, over the tables, when it does not cover rows the readout reads.
    constexpr bool QT_EARLY = JS == 2 && !Cfg::QT_IN_TOK;
    // Single-window chunks at d = 64 (16-token sub-blocks: every sub-block
    // a whole chunk of at most 16 tokens, opening from Q_0 = I): the refresh
    // takes B Q_L = G_15 B + (B U^T) diag(R[15]) K^ without forming Q_L, half
    // the products of B Q_L. (At d = 32 the two forms take the same products,
    // and the Q-form measured faster.)
    constexpr bool DIRECT = D == 64 && T == 16;
    static_assert(!DIRECT || (NWIN == 1 && JS == 1 && CW == NW), "direct refresh layout");
    static_assert(!SAVE || SaveLayout<D>::QREC != DIRECT, "the record keeps Q_0 and Q_L unless direct");

    const size_t out_row0 = (static_cast<size_t>(slot) * B + b) * N;

    int c0 = 0;
    int cend = L;
    int s0 = 0;
    int nt = (T < cend) ? T : cend;
    issue_loads(s0, nt);

    float *const svc = SAVE ? sv.base + static_cast<long long>(chain) * sv.chain_floats : nullptr;
#if SRNL_PHASE_CLOCKS
    __shared__ unsigned ph_lds[16];
    if (tid < 16)
        ph_lds[tid] = 0u;
    unsigned long long ph_n = 0, ph_t = clock64();
    const unsigned long long ph_t0 = ph_t;
#endif
    const SaveLayout<D> sl{(N + L - 1) / L, (L + 15) / 16};
    bool mc_pending = false;   // M_c still waits for the last chunk's Q_L (DEFER_MC)
    // The direct refresh of a single-window chunk (DIRECT):
    //   B' = G_15 B + P diag(R[15]) K^,  P = B U^T  [row][token],
    // with U staged over the query rows by the update. P is formed per
    // 16-row tile as P^T (the product's output is then the next product's
    // second operand as it stands), and B'^T tiles come out with four
    // consecutive channels of one row per lane. Each wave owns whole row tiles
    // of B. The first part reads only B_c, U and k^, so it runs beside the
    // readout; the vector rows' dots cross waves through the v rows (dead
    // after the update). The second part writes B' after a barrier.
    constexpr int RTM_D = 3 * D / 16, RTD_D = (RTM_D + NW - 1) / NW;
    float *const PV = Es;
    auto direct_products = [&](v4f (&pt)[RTD_D]) {
        if constexpr (DIRECT) {
#pragma unroll
            for (int w = 0; w < RTD_D; ++w) {
                const int tm = wave + NW * w;
                v4f acc = {0.f, 0.f, 0.f, 0.f};
                if (tm < RTM_D) {
#pragma unroll
                    for (int kb = 0; kb < NTC; ++kb)
                        acc = mfma16(ld4(Xs + ix(lm, 16 * kb + 4 * lk)),
                                     ld4(Bs + ix(16 * tm + lm, 16 * kb + 4 * lk)), acc);
                }
                pt[w] = acc;
            }
            // vector rows: p_v[s] = b_v . u_s, LPD lanes per dot
            constexpr int LPD = NT / 32, CPL = D / LPD;
            static_assert(LPD == 4 || LPD == 8, "a power-of-two group of lanes per dot");
            static_assert(CPL % 4 == 0 && NT == 4 * D, "whole 16-byte blocks; two lanes per output");
            const int o = tid / LPD, part = tid % LPD, v = o >> 4, sx = o & 15;
            float acc = 0.f;
#pragma unroll
            for (int k = 0; k < CPL / 4; ++k) {
                const int c = part * CPL + 4 * k;
                const float4 uu = ld4(Xs + ix(sx, c));
                const float4 bb = ld4(Bs + ix(3 * D + v, c));
                acc = fmaf(uu.x, bb.x, acc);
                acc = fmaf(uu.y, bb.y, acc);
                acc = fmaf(uu.z, bb.z, acc);
                acc = fmaf(uu.w, bb.w, acc);
            }
            acc = group_sum<LPD>(acc);
            if (part == 0)
                PV[o] = acc;
        }
    };
    auto direct_store = [&](const v4f (&pt)[RTD_D], bool frz) {
        if constexpr (DIRECT) {
            __syncthreads();   // the readout is done with B_c; the vector-row dots are in
            const float g15 = WG[0];
            const float4 rb = ld4(RB + 4 * lk);
#pragma unroll
            for (int tn = 0; tn < NTC; ++tn) {
                const int cc = 16 * tn + lm;
                const float4 ka = make_float4(rb.x * KHa[ix(4 * lk, cc)], rb.y * KHa[ix(4 * lk + 1, cc)],
                                              rb.z * KHa[ix(4 * lk + 2, cc)], rb.w * KHa[ix(4 * lk + 3, cc)]);
#pragma unroll
                for (int w = 0; w < RTD_D; ++w) {
                    const int tm = wave + NW * w;
                    if (tm >= RTM_D || (frz && tm >= NTC))
                        continue;
                    float *bp = Bs + ix(16 * tm + lm, 16 * tn + 4 * lk);
                    const float4 b0 = ld4(bp);
                    v4f acc = {g15 * b0.x, g15 * b0.y, g15 * b0.z, g15 * b0.w};
                    acc = mfma16(ka, make_float4(pt[w][0], pt[w][1], pt[w][2], pt[w][3]), acc);
                    st4(bp, acc[0], acc[1], acc[2], acc[3]);
                }
            }
            // vector rows: b_v' = G_15 b_v + sum_s p_v[s] R[15][s] k^_s, two
            // lanes per element
            if (!frz) {
                const int o = tid >> 1, part = tid & 1, v = o / D, cc = o % D;
                float acc = 0.f;
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const int sx = 8 * part + k;
                    acc = fmaf(PV[16 * v + sx] * RB[sx], KHa[ix(sx, cc)], acc);
                }
                acc = group_sum<2>(acc);
                if (part == 0)
                    Bs[ix(3 * D + v, cc)] = fmaf(g15, Bs[ix(3 * D + v, cc)], acc);
            }
        }
    };
    // Readout Y^T = B_c Z^T of token tile tm, channel tile tn: each lane ends
    // with four consecutive channels of one token (a 16-byte store).
    auto readout_tile = [&](int tm, int tn) {
        float a[KS];
        ldrow(KZ, tm * 16 + lm, lk * KS, a);
        if (JS == 2) {
            float a2[KS];
            ldrow(KZ2, tm * 16 + lm, lk * KS, a2);
#pragma unroll
            for (int s = 0; s < KS; ++s)
                a[s] += a2[s];
        }
        const int u0 = tm * 16 + lm;
        float br[KS];
        ldrow(Bs, tn * 16 + lm, lk * KS, br);
        v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s)
            acc = mfma4(br[s], a[s], acc);
        if (u0 < nt) {
            float *orow = out + (out_row0 + s0 + u0) * C + static_cast<size_t>(h) * D + 4 * lk;
            *reinterpret_cast<float4 *>(orow + tn * 16) = make_float4(acc[0], acc[1], acc[2], acc[3]);
        }
    };
    while (true) {
        __syncthreads();   // previous sub-block is done with every token array; Bs is current
        if constexpr (SAVE) {
            if (s0 == c0) {   // a chunk's boundary rows
                float *dst = svc + sl.o_bnd(c0 / L);
                for (int idx = tid; idx < ROWS * D; idx += NT)
                    dst[idx] = Bs[ix(idx / D, idx % D)];
            }
        }

        // (1) store the prefetched tokens (zero rows past nt)
#pragma unroll
        for (int k = 0; k < NPF; ++k) {
            const int seg = tid + k * NT;
            if (seg < T * SEGS) {
                const int u = seg / SEGS, sg = seg % SEGS;
                float f[VE], fq[VE];
                if (seg < nt * SEGS) {
                    unpack(pre[k], f, static_cast<const InT *>(nullptr));
                    if (HAS_Q)
                        unpack(preq[k], fq, static_cast<const InT *>(nullptr));
                } else {
#pragma unroll
                    for (int e = 0; e < VE; ++e)
                        f[e] = fq[e] = 0.0f;
                }
#pragma unroll
                for (int e = 0; e < VE / 4; ++e) {
                    st4(Xs + ix(u, sg * VE + 4 * e), f[4 * e], f[4 * e + 1], f[4 * e + 2], f[4 * e + 3]);
                    if (HAS_Q)
                        st4(QVa + ix(u, sg * VE + 4 * e), fq[4 * e], fq[4 * e + 1], fq[4 * e + 2],
                            fq[4 * e + 3]);
                }
            }
        }
        // position of the next sub-block; prefetch it
        const int s1 = s0 + nt;
        const bool chunk_end = (s1 == cend);
        int c1 = c0, cend1 = cend;
        if (chunk_end) {
            c1 = cend;
            cend1 = (c1 < N - L) ? c1 + L : N;
        }
        const int nt1 = (s1 < N) ? ((T < cend1 - s1) ? T : cend1 - s1) : 0;
        if (nt1 > 0)
            issue_loads(s1, nt1);
        __syncthreads();
        SRNL_PHASE(0);

        const int nwin = (nt + 15) >> 4;   // 16-token windows (= token tiles)

        // (2) boundary generation on MFMA: [k | v] = X [B_k; B_v]^T; wave w
        //     produces the 16-wide output tiles tn = w, w + NW, ... With bf16
        //     input, x is exact in bf16 and each boundary row is split exactly
        //     into three bf16 parts, so three bf16 products (16x16x32) per
        //     32-wide block give the fp32 result at a third of the cost of the
        //     fp32 instruction.
        //     With at least two waves per output tile (the eight-wave
        //     sub-blocks) the token tiles of a tile are dealt out between them.
        constexpr int GT = 2 * NTC;                        // output tiles
        constexpr int GS = (NW >= 2 * GT) ? NW / GT : 1;   // waves per output tile
        constexpr int NTM = NWIN / GS;                     // token tiles per wave
        static_assert(NWIN % GS == 0, "token tiles deal out evenly");
        const int tm_ph = (GS > 1) ? wave / GT : 0;        // this wave's token tiles tm_ph + GS k
        for (int tn = (GS > 1) ? wave % GT : wave; tn < GT; tn += (GS > 1) ? GT : NW) {
            float *dst = (tn < NTC) ? KZ : Es;
            // the transposed product [k | v]^T = [B_k; B_v] X^T leaves four
            // consecutive output channels oc0.. of one token in each lane
            const int oc0 = (tn % NTC) * 16 + 4 * lk;
            const int brow = D + tn * 16 + lm;   // boundary row of this lane
            if constexpr (std::is_same<InT, uint16_t>::value) {
                constexpr int KB = D / 32;
                bf16x8 bh[KB], bm[KB], bl[KB];
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) {
                    float bv[8];
                    ldrow(Bs, brow, 32 * kb + 8 * lk, bv);
                    split3_bf16(bv, bh[kb], bm[kb], bl[kb]);
                }
                // this wave's token tiles of the sub-block (rows past nt are zero)
                bf16x8 xa[NTM][KB];
#pragma unroll
                for (int k = 0; k < NTM; ++k)
#pragma unroll
                    for (int kb = 0; kb < KB; ++kb) {
                        float xv[8];
                        ldrow(Xs, (tm_ph + GS * k) * 16 + lm, 32 * kb + 8 * lk, xv);
                        xa[k][kb] = pack_bf16_exact(xv);
                    }
#pragma unroll
                for (int k = 0; k < NTM; ++k) {
                    const int tm = tm_ph + GS * k;
                    v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kb = 0; kb < KB; ++kb) {
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bl[kb], xa[k][kb], acc, 0, 0, 0);
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bm[kb], xa[k][kb], acc, 0, 0, 0);
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bh[kb], xa[k][kb], acc, 0, 0, 0);
                    }
                    st4(dst + ix(tm * 16 + lm, oc0), acc[0], acc[1], acc[2], acc[3]);
                }
            } else {
                float bg[KS];
                ldrow(Bs, brow, lk * KS, bg);
#pragma unroll
                for (int k = 0; k < NTM; ++k) {
                    const int tm = tm_ph + GS * k;
                    float a[KS];
                    ldrow(Xs, tm * 16 + lm, lk * KS, a);
                    v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int s = 0; s < KS; ++s)
                        acc = mfma4(bg[s], a[s], acc);
                    st4(dst + ix(tm * 16 + lm, oc0), acc[0], acc[1], acc[2], acc[3]);
                }
            }
        }
        __syncthreads();
        SRNL_PHASE(1);

        // (3) transition scalars, EPL lanes per token [SUMMARY stabilisation]:
        //     k^ = k / sqrt(|k|^2 + eps), e = k^ - v, eta = sigmoid(b_eta . x),
        //     alpha = alpha_max sigmoid(b_alpha . x), soft cap, spectral clamp.
        {
            const int u = tid / EPL, ep = tid % EPL;
            const int c0e = ep * ECPL;
            if (u < nt) {
                float kk[ECPL], vv[ECPL], xv[ECPL], be[ECPL], ba[ECPL];
                ldrow(KZ, u, c0e, kk);
                ldrow(Es, u, c0e, vv);
                ldrow(Xs, u, c0e, xv);
                ldrow(Bs, 3 * D, c0e, be);
                ldrow(Bs, 3 * D + 1, c0e, ba);
                float nk2 = 0.f, er = 0.f, ar = 0.f;
#pragma unroll
                for (int c = 0; c < ECPL; ++c) {
                    nk2 = fmaf(kk[c], kk[c], nk2);
                    er = fmaf(be[c], xv[c], er);
                    ar = fmaf(ba[c], xv[c], ar);
                }
                nk2 = group_sum<EPL>(nk2);
                er = group_sum<EPL>(er);
                ar = group_sum<EPL>(ar);
                const float inv = __builtin_amdgcn_rsqf(nk2 + eps);
                float nkh2 = 0.f, ne2 = 0.f;
                float khv[ECPL], evv[ECPL];
#pragma unroll
                for (int c = 0; c < ECPL; ++c) {
                    khv[c] = kk[c] * inv;
                    evv[c] = khv[c] - vv[c];
                    nkh2 = fmaf(khv[c], khv[c], nkh2);
                    ne2 = fmaf(evv[c], evv[c], ne2);
                }
#pragma unroll
                for (int c4 = 0; c4 < ECPL / 4; ++c4)
                    st4(KHa + ix(u, c0e + 4 * c4), khv[4 * c4], khv[4 * c4 + 1], khv[4 * c4 + 2],
                        khv[4 * c4 + 3]);
#pragma unroll
                for (int c = 0; c < ECPL; ++c)
                    Et[(c0e + c) * ETS + et_col(c0e + c, u)] = evv[c];
                nkh2 = group_sum<EPL>(nkh2);
                ne2 = group_sum<EPL>(ne2);
                const float eta = sigmoidf(er);
                const float alpha = (flags & F_FIXED_ALPHA) ? alpha_max
                                                            : alpha_max * sigmoidf(ar);
                const float g = __builtin_amdgcn_sqrtf(ne2 * nkh2);
                const float m = 1.0f - alpha;
                float eta1 = eta, uu = 0.f;
                int bits = 0;
                if (flags & F_NO_CAP) {
                    eta1 = eta;
                } else if (flags & F_HARD_CAP) {
                    if (g > 0.0f && m < eta * g) {
                        eta1 = m * __builtin_amdgcn_rcpf(g);
                        bits |= SCB_HARD;
                    }
                } else if (g > 0.0f) {
                    uu = eta * g * __builtin_amdgcn_rcpf(m);
                    const bool series = uu < 1e-3f;
                    eta1 = series ? eta * (1.0f - uu * uu * (1.0f / 3.0f))
                                  : m * tanh_pos(uu) * __builtin_amdgcn_rcpf(g);
                    if (series)
                        bits |= SCB_SERIES;
                }
                float eta2 = eta1;
                if (!(flags & F_NO_CLAMP) && nkh2 > 0.0f) {
                    const float cap = 2.0f * alpha * __builtin_amdgcn_rcpf(nkh2);
                    if (cap < eta2) {
                        eta2 = cap;
                        bits |= SCB_CLAMP;
                    }
                }
                if (ep == 0) {
                    AL[u] = alpha;
                    EH[u] = eta2;
                }
                if constexpr (SAVE) {
                    float *tw = svc + sl.o_tab(c0 / L, (s0 - c0) / 16 + u / 16) + (u % 16) * D + c0e;
#pragma unroll
                    for (int c4 = 0; c4 < ECPL / 4; ++c4) {
                        st4(tw + SaveLayout<D>::TW_KH + 4 * c4, khv[4 * c4], khv[4 * c4 + 1],
                            khv[4 * c4 + 2], khv[4 * c4 + 3]);
                        st4(tw + SaveLayout<D>::TW_E + 4 * c4, evv[4 * c4], evv[4 * c4 + 1],
                            evv[4 * c4 + 2], evv[4 * c4 + 3]);
                    }
                    if (ep == 0) {
                        // The backward through these scalars is linear in
                        // dL/deta'' and dL/dalpha; its five coefficients:
                        //   dL/d(eta pre-activation)   = c0 dL/deta''
                        //   dL/d(alpha pre-activation) = c1 dL/dalpha + c2 dL/deta''
                        //   dL/d|e|^2 = c3 dL/deta'',  dL/d|k^|^2 = c4 dL/deta''
                        const bool clamp_on = (bits & SCB_CLAMP) != 0;
                        const float p1 = clamp_on ? 0.f : 1.f;   // deta1 per deta''
                        float ke = 0.f, km = 0.f, kg = 0.f;      // d eta, d m, d g per deta1
                        if (flags & F_NO_CAP) {
                            ke = 1.f;
                        } else if (flags & F_HARD_CAP) {
                            if (bits & SCB_HARD) {
                                km = 1.0f / g;
                                kg = -m / (g * g);
                            } else {
                                ke = 1.f;
                            }
                        } else if (g > 0.0f) {
                            float kuu;
                            if (bits & SCB_SERIES) {
                                ke = 1.0f - uu * uu * (1.0f / 3.0f);
                                kuu = eta * (-2.0f * uu * (1.0f / 3.0f));
                            } else {
                                const float th = tanh_pos(uu);
                                km = th / g;
                                kuu = m * (1.0f - th * th) / g;
                                kg = -m * th / (g * g);
                            }
                            ke += kuu * g / m;
                            kg += kuu * eta / m;
                            km -= kuu * eta * g / (m * m);
                        } else {
                            ke = 1.f;
                        }
                        const float ga = (flags & F_FIXED_ALPHA) ? 0.f : alpha * (1.0f - alpha / alpha_max);
                        const float cf0 = p1 * ke * eta * (1.0f - eta);
                        const float cf2 = ga * ((clamp_on ? 2.0f / nkh2 : 0.f) - p1 * km);
                        float cf3 = 0.f, cf4 = 0.f;
                        if (g > 0.0f) {
                            cf3 = p1 * kg * g / (2.0f * ne2);
                            cf4 = p1 * kg * g / (2.0f * nkh2);
                        }
                        if (clamp_on)
                            cf4 -= 2.0f * alpha / (nkh2 * nkh2);
                        float4 *ds = reinterpret_cast<float4 *>(
                            svc + sl.o_sc(c0 / L, (s0 - c0) / 16 + u / 16) + (u % 16) * 16);
                        ds[0] = make_float4(inv, nkh2, ne2, g);
                        ds[1] = make_float4(eta, alpha, m, uu);
                        ds[2] = make_float4(eta1, eta2, __int_as_float(bits), cf0);
                        ds[3] = make_float4(ga, cf2, cf3, cf4);
                    }
                }
            } else {
                // padding token: leaves Q unchanged
#pragma unroll
                for (int c4 = 0; c4 < ECPL / 4; ++c4)
                    st4(KHa + ix(u, c0e + 4 * c4), 0.f, 0.f, 0.f, 0.f);
                if constexpr (SAVE) {
                    // (only inside the sub-block's windows: past them lie the
                    // next chunk's slots)
                    if (u / 16 < nwin) {
                        float *tw = svc + sl.o_tab(c0 / L, (s0 - c0) / 16 + u / 16) + (u % 16) * D + c0e;
#pragma unroll
                        for (int c4 = 0; c4 < ECPL / 4; ++c4) {
                            st4(tw + SaveLayout<D>::TW_KH + 4 * c4, 0.f, 0.f, 0.f, 0.f);
                            st4(tw + SaveLayout<D>::TW_E + 4 * c4, 0.f, 0.f, 0.f, 0.f);
                        }
                    }
                }
#pragma unroll
                for (int c = 0; c < ECPL; ++c)
                    Et[(c0e + c) * ETS + et_col(c0e + c, u)] = 0.f;
                if (ep == 0) {
                    AL[u] = 1.0f;
                    EH[u] = 0.0f;
                }
            }
        }
        if constexpr (Cfg::WL)
            wave_lds_sync();   // this wave's epilogue is its window's only input
        else
            __syncthreads();
        SRNL_PHASE(2);

        // deferred M_c refresh, products: wave w < NTC^2 takes tile (w / NTC,
        // w % NTC) of M_c Q_L into registers; stored after this phase's
        // closing barrier (every wave has read M_c by then)
        v4f mc_acc = {0.f, 0.f, 0.f, 0.f};
        const bool do_mc = DEFER_MC && mc_pending && wave < NTC * NTC;
        if constexpr (DEFER_MC) {
            if (do_mc) {
                float a[KS], bq[KS];
                ldrow(Bs, (wave / NTC) * 16 + lm, lk * KS, a);
                ldrow(Qt, (wave % NTC) * 16 + lm, lk * KS, bq);
#pragma unroll
                for (int s = 0; s < KS; ++s)
                    mc_acc = mfma4(bq[s], a[s], mc_acc);
            }
        }
        // (4) window tables, wave w for windows w, w + NW, ... (window-local
        //     token indices t, s in 0..15; lane holds s = 4 lk + i, t = lm)
        for (int win = wave; win < nwin; win += NW) {
            const int tb = 16 * win;
            // Gram matrices on MFMA: gkk[i] = k^_s . k^_t, gqk[i] = k^_s . q_t
            v4f gkk = {0.f, 0.f, 0.f, 0.f}, gqk = {0.f, 0.f, 0.f, 0.f};
            if constexpr (std::is_same<InT, uint16_t>::value && !HAS_Q) {
                // the query rows are the bf16 input (exact in bf16): k^ split
                // exactly into three bf16 parts gives k^ . q from three bf16
                // products per 32 channels and k^ . k^ from all nine part
                // products; every product is exact and the sums are fp32, as
                // in the fp32 instruction (smallest parts first)
#pragma unroll
                for (int kb = 0; kb < D / 32; ++kb) {
                    float kf[8], xf[8];
                    ldrow(KHa, tb + lm, 32 * kb + 8 * lk, kf);
                    ldrow(QR, tb + lm, 32 * kb + 8 * lk, xf);
                    bf16x8 kh, km, kl;
                    split3_bf16(kf, kh, km, kl);
                    const bf16x8 xb = pack_bf16_exact(xf);
                    gqk = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kl, xb, gqk, 0, 0, 0);
                    gkk = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kl, kl, gkk, 0, 0, 0);
                    gqk = __builtin_amdgcn_mfma_f32_16x16x32_bf16(km, xb, gqk, 0, 0, 0);
                    gkk = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kl, km, gkk, 0, 0, 0);
                    gqk = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kh, xb, gqk, 0, 0, 0);
                    gkk = __builtin_amdgcn_mfma_f32_16x16x32_bf16(km, kl, gkk, 0, 0, 0);
                    gkk = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kl, kh, gkk, 0, 0, 0);
                    gkk = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kh, kl, gkk, 0, 0, 0);
                    gkk = __builtin_amdgcn_mfma_f32_16x16x32_bf16(km, km, gkk, 0, 0, 0);
                    gkk = __builtin_amdgcn_mfma_f32_16x16x32_bf16(km, kh, gkk, 0, 0, 0);
                    gkk = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kh, km, gkk, 0, 0, 0);
                    gkk = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kh, kh, gkk, 0, 0, 0);
                }
            } else {
#pragma unroll
                for (int jt = 0; jt < NTC; ++jt) {
                    const float4 kv = ld4(KHa + ix(tb + lm, 16 * jt + 4 * lk));
                    const float4 qv = ld4(QR + ix(tb + lm, 16 * jt + 4 * lk));
                    gkk = mfma16(kv, kv, gkk);
                    gqk = mfma16(kv, qv, gqk);
                }
            }
            const int t = lm;
            const float at = AL[tb + t], et = EH[tb + t];
            // prefix products pi = G_t over the window (each 16-lane row holds
            // the whole window; DPP row shifts with 1 shifted in)
            float pi = at;
            pi *= row_shr_fill1<1>(pi);
            pi *= row_shr_fill1<2>(pi);
            pi *= row_shr_fill1<4>(pi);
            pi *= row_shr_fill1<8>(pi);
            const float gprev = row_shr_fill1<1>(pi);   // G_{t-1}
            const float gtot = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pi), 15));
            // P[i] = R[t-1][s], Rr[i] = R[t][s] for s = 4 lk + i < t
            float P[4], Rr[4];
            if (gtot >= 0x1p-100f) {
                // every prefix product is >= 2^-100: ratios are safe
                if (lk == 0)
                    PI[tb + t] = pi;
                wave_lds_sync();
                const float4 ps = ld4(PI + tb + 4 * lk);
                const float q4[4] = {__builtin_amdgcn_rcpf(ps.x), __builtin_amdgcn_rcpf(ps.y),
                                     __builtin_amdgcn_rcpf(ps.z), __builtin_amdgcn_rcpf(ps.w)};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    P[i] = gprev * q4[i];
                    Rr[i] = pi * q4[i];
                }
            } else {
                // direct products (a prefix product underflows): p3 = product of
                // alpha_j over 4 lk + 4 <= j < t
                float av[16];
                lds_load(AL + tb, av);
                float p3 = 1.0f;
                const int sb = 4 * lk + 4;
#pragma unroll
                for (int j = 4; j < 15; ++j)
                    p3 *= (j >= sb && j < t) ? av[j] : 1.0f;
                const float4 as4 = ld4(AL + tb + 4 * lk);
                P[3] = p3;
                P[2] = P[3] * ((4 * lk + 3 < t) ? as4.w : 1.0f);
                P[1] = P[2] * ((4 * lk + 2 < t) ? as4.z : 1.0f);
                P[0] = P[1] * ((4 * lk + 1 < t) ? as4.y : 1.0f);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    Rr[i] = P[i] * at;
            }
            float Nr[4], Lr[4];
            float *lc = Lc + win * Cfg::WSTR_L;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int s = 4 * lk + i;
                const bool lt = s < t;
                Rr[i] = lt ? Rr[i] : (s == t ? 1.0f : 0.0f);
                Lr[i] = lt ? et * P[i] * gkk[i] : 0.0f;
                Nr[i] = BEFORE ? (lt ? P[i] * gqk[i] : 0.0f) : Rr[i] * gqk[i];
            }
            st4(lc + t * WS + 4 * lk, Lr[0], Lr[1], Lr[2], Lr[3]);
            st4(Nn + win * Cfg::WSTR_N + t * NS + 4 * lk, Nr[0], Nr[1], Nr[2], Nr[3]);
            if constexpr (SAVE) {
                using SL = SaveLayout<D>;
                float *tw = svc + sl.o_tab(c0 / L, (s0 - c0) / 16 + win) + t * 16 + 4 * lk;
                st4(tw + SL::TW_KK, gkk[0], gkk[1], gkk[2], gkk[3]);
                st4(tw + SL::TW_QK, gqk[0], gqk[1], gqk[2], gqk[3]);
                st4(tw + SL::TW_R, Rr[0], Rr[1], Rr[2], Rr[3]);
                float lf[4];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    lf[i] = (4 * lk + i < t) ? P[i] * gkk[i] : 0.0f;
                st4(tw + SL::TW_LF, lf[0], lf[1], lf[2], lf[3]);
                st4(tw + SL::TW_NF, Nr[0], Nr[1], Nr[2], Nr[3]);
                float *tg = svc + sl.o_tab(c0 / L, (s0 - c0) / 16 + win);
                if (lk == 0) {
                    tg[SL::TW_G + t] = pi;
                    tg[SL::TW_GP + t] = gprev;
                }
                if (t == 15)
                    st4(tg + SL::TW_PI + 4 * lk, Rr[0], Rr[1], Rr[2], Rr[3]);
            }
            if (t == 15)
                st4(RB + tb + 4 * lk, Rr[0], Rr[1], Rr[2], Rr[3]);
            if (lk == 0) {
                GA[tb + t] = gprev;
                GZ[tb + t] = BEFORE ? gprev : pi;
                if (t == 15)
                    WG[win] = pi;
            }
            wave_lds_sync();

            // T = (I + L)^-1 by block forward substitution over 4 x 4 blocks:
            // lane 4 c + g holds rows 4 g .. 4 g + 3 of column c of T. For each
            // block b in turn, the lanes of block b finish their four rows, the
            // quad broadcasts them (DPP), and the lanes of later blocks fold
            // them into their partial sums. Then T'[s][c] = -eta''_c T[s][c].
            {
                const int c = lane >> 2, g = lane & 3;
                float lrow[4][16];   // L[4 g + i][m]
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    lds_load(lc + (4 * g + i) * WS, lrow[i]);
                float acc[4], xf[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    acc[i] = (4 * g + i == c) ? 1.0f : 0.0f;
                    xf[i] = 0.0f;
                }
                auto block = [&](auto bbc) {
                    constexpr int bb = decltype(bbc)::value;
                    // rows of block bb (final in the lanes with g == bb)
                    float xs[4];
                    xs[0] = acc[0];
                    xs[1] = fmaf(-lrow[1][4 * bb], xs[0], acc[1]);
                    xs[2] = fmaf(-lrow[2][4 * bb + 1], xs[1], fmaf(-lrow[2][4 * bb], xs[0], acc[2]));
                    xs[3] = fmaf(-lrow[3][4 * bb + 2], xs[2],
                                 fmaf(-lrow[3][4 * bb + 1], xs[1], fmaf(-lrow[3][4 * bb], xs[0], acc[3])));
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        xf[i] = (g == bb) ? xs[i] : xf[i];
                    if constexpr (bb < 3) {
                        float xb[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            xb[i] = quad_bcast(xs[i], bb);
#pragma unroll
                        for (int i = 0; i < 4; ++i)
#pragma unroll
                            for (int j = 0; j < 4; ++j)
                                acc[i] = fmaf(-lrow[i][4 * bb + j], xb[j], acc[i]);
                    }
                };
                block(std::integral_constant<int, 0>());
                block(std::integral_constant<int, 1>());
                if (nt - tb > 8) {
                    block(std::integral_constant<int, 2>());
                    block(std::integral_constant<int, 3>());
                } else {
                    // tokens 8 .. 15 of the window are padding: their rows of L
                    // are zero, so rows 8 .. 15 of T are those of I, which is
                    // what the lanes of blocks 2 and 3 hold in acc (the same
                    // values the two skipped steps would leave there)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        xf[i] = (g >= 2) ? acc[i] : xf[i];
                }
                if constexpr (SAVE)   // T transposed: [c][4 g + i]
                    st4(svc + sl.o_tab(c0 / L, (s0 - c0) / 16 + win) + SaveLayout<D>::TW_T + c * 16 + 4 * g,
                        xf[0], xf[1], xf[2], xf[3]);
                const float ec = -EH[tb + c];
                float *tp = Tp + win * Cfg::WSTR_T;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    tp[tp_index(4 * g + i, c)] = ec * xf[i];
            }
        }
        __syncthreads();
        if constexpr (DEFER_MC) {
            if (do_mc)   // transposed product: four consecutive channels of one row
                st4(Bs + ix((wave / NTC) * 16 + lm, (wave % NTC) * 16 + 4 * lk), mc_acc[0], mc_acc[1],
                    mc_acc[2], mc_acc[3]);
            mc_pending = false;
        }
        SRNL_PHASE(3);

        // (5) token-order update, window by window, on MFMA. Wave w owns rows
        //     16 it .. 16 it + 15 of Q (it = w % NTC) and, when two waves share
        //     those rows (JS = 2), the columns of its half jg = w / NTC of Q.
        //     Per window:
        //       A   = diag(G_{t-1}) K^ Q_0^T + E           [t][i]
        //       U   = T' A                                 [s][i]
        //       Z   = diag(G_t) Qrows Q_0^T + N U          [t][i]  -> z_t rows
        //       Q^T = G_15 Q_0^T + K^^T diag(R[15]) U      [j][i]
        //     With JS = 2 the contraction over j in A is completed by
        //     exchanging the halves through LDS (double-buffered by window
        //     parity: one barrier per window); Z is left as two partial sums
        //     (each wave also takes half of the N U terms) that the readout adds.
        const bool first_sub = (s0 == c0);   // this sub-block opens its chunk
        if (wave < CW) {
            // the window chain is the chunk's critical path: with the long
            // sub-blocks (two chains a CU) its waves issue ahead of the
            // other chain's
            if constexpr (T >= 64)
                __builtin_amdgcn_s_setprio(2);
            const int it = wave % NTC, jg = wave / NTC;
            float4 kv[NJ], qv[NJ];
            auto load_rows = [&](int tb) {
#pragma unroll
                for (int jl = 0; jl < NJ; ++jl) {
                    const int jt = jg * NJ + jl;
                    kv[jl] = ld4(KHa + ix(tb + lm, 16 * jt + 4 * lk));
                    qv[jl] = ld4(QR + ix(tb + lm, 16 * jt + 4 * lk));
                }
            };
            if (nwin > 0)
                load_rows(0);
            auto save_q = [&](float *dst) {   // this wave's tiles of Q, row-major
#pragma unroll
                for (int jl = 0; jl < NJ; ++jl)
                    *reinterpret_cast<float4 *>(dst + (16 * it + lm) * D + 16 * (jg * NJ + jl) + 4 * lk) =
                        make_float4(qacc[jl][0], qacc[jl][1], qacc[jl][2], qacc[jl][3]);
            };
            for (int win = 0; win < nwin; ++win) {
                const int tb = 16 * win;
                if constexpr (SAVE && !DIRECT)
                    save_q(svc + sl.o_q0(c0 / L, (s0 - c0) / 16 + win));
                v4f A = {0.f, 0.f, 0.f, 0.f}, Z = {0.f, 0.f, 0.f, 0.f};
                // a chunk's first window opens from Q_0 = I: A is then the
                // window's k^ rows (already complete, no exchange) and the z
                // partial its q rows, in the column part that holds this
                // wave's rows (the products give the same values exactly)
                const bool q_id = first_sub && win == 0;
                // (without outputs, the record-only forward forms no z rows)
                if (q_id) {
                    const bool own = (it / NJ == jg);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        A[i] = KHa[ix(tb + 4 * lk + i, 16 * it + lm)];
                        if constexpr (OUT)
                            Z[i] = own ? QR[ix(tb + 4 * lk + i, 16 * it + lm)] : 0.f;
                    }
                } else {
#pragma unroll
                    for (int jl = 0; jl < NJ; ++jl) {
                        A = mfma16(kv[jl], qacc[jl], A);
                        if constexpr (OUT)
                            Z = mfma16(qv[jl], qacc[jl], Z);
                    }
                }
                const float4 ga = ld4(GA + tb + 4 * lk);
                const float4 gz = ld4(GZ + tb + 4 * lk);
                const float4 rb = ld4(RB + tb + 4 * lk);
                const float4 ee = ld4(Et + (16 * it + lm) * ETS + et_col(16 * it + lm, tb + 4 * lk));
                const float4 tpv = ld4(Tp + win * Cfg::WSTR_T + tp_index(lm, 4 * lk));
                const float4 nnv = ld4(Nn + win * Cfg::WSTR_N + lm * NS + 4 * lk);
                const float wg = WG[win];
                // K^^T operand of the Q update with diag(R[15]) folded in
                // (off the window's dependency chain, unlike scaling U)
                float4 kt[NJ];
#pragma unroll
                for (int jl = 0; jl < NJ; ++jl) {
                    const int jt = jg * NJ + jl;
                    kt[jl] = make_float4(KHa[ix(tb + 4 * lk, 16 * jt + lm)] * rb.x,
                                         KHa[ix(tb + 4 * lk + 1, 16 * jt + lm)] * rb.y,
                                         KHa[ix(tb + 4 * lk + 2, 16 * jt + lm)] * rb.z,
                                         KHa[ix(tb + 4 * lk + 3, 16 * jt + lm)] * rb.w);
                }
                if (JS == 2 && !q_id) {
                    float *xb = XB + ((win & 1) * NTC + it) * 512 + 4 * lane;
                    st4(xb + 256 * jg, A[0], A[1], A[2], A[3]);
                    __syncthreads();
                    const float4 pa = ld4(xb + 256 * (1 - jg));
                    A[0] += pa.x;
                    A[1] += pa.y;
                    A[2] += pa.z;
                    A[3] += pa.w;
                }
                A[0] = fmaf(ga.x, A[0], ee.x);
                A[1] = fmaf(ga.y, A[1], ee.y);
                A[2] = fmaf(ga.z, A[2], ee.z);
                A[3] = fmaf(ga.w, A[3], ee.w);
                v4f U = {0.f, 0.f, 0.f, 0.f};
                U = mfma16(tpv, A, U);
                if constexpr (SAVE) {   // u_t rows of the window (both column halves hold them)
                    if (jg == 0) {
                        float *du = svc + sl.o_u(c0 / L, (s0 - c0) / 16 + win);
#pragma unroll
                        for (int rr = 0; rr < 4; ++rr)
                            du[(4 * lk + rr) * D + 16 * it + lm] = U[rr];
                    }
                }
                if constexpr (OUT) {
                    Z[0] *= gz.x;
                    Z[1] *= gz.y;
                    Z[2] *= gz.z;
                    Z[3] *= gz.w;
                    if (JS == 1) {
                        Z = mfma16(nnv, U, Z);
                    } else if (jg == 0) {
                        Z = mfma4(nnv.x, U[0], Z);
                        Z = mfma4(nnv.y, U[1], Z);
                    } else {
                        Z = mfma4(nnv.z, U[2], Z);
                        Z = mfma4(nnv.w, U[3], Z);
                    }
                }
                if constexpr (DIRECT) {
                    // the u rows, [token][channel], over the query rows: this
                    // lane has read its own elements of those (the z
                    // partial above) and no other wave reads them
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr)
                        Xs[ix(4 * lk + rr, 16 * it + lm)] = U[rr];
                }
                if constexpr (!DIRECT) {
#pragma unroll
                    for (int jl = 0; jl < NJ; ++jl) {
                        qacc[jl] *= wg;
                        qacc[jl] = mfma16(kt[jl], U, qacc[jl]);
                    }
                }
                if (win + 1 < nwin)
                    load_rows(tb + 16);
                if constexpr (OUT) {
                    float *zd = (JS == 2 && jg == 1) ? KZ2 : KZ;
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        zd[ix(tb + 4 * lk + i, 16 * it + lm)] = Z[i];
                }
            }
            if constexpr (T >= 64)
                __builtin_amdgcn_s_setprio(0);
            if constexpr (QT_EARLY) {
                if (chunk_end && cend < N)
                    stage_qt();
            }
            if constexpr (SAVE && !DIRECT) {
                if (chunk_end)
                    save_q(svc + sl.o_ql(c0 / L));
            }
        } else if constexpr (JS == 2) {
            // the update's per-window block barrier, for the waves outside it
            // (their MFMA work here would share the update waves' pipes and
            // lengthen the window chain)
            for (int win = first_sub ? 1 : 0; win < nwin; ++win)
                __syncthreads();
        }
        __syncthreads();
        SRNL_PHASE(4);
        if constexpr (!QT_EARLY && !Cfg::QT_IN_TOK) {
            if (chunk_end && cend < N) {
                if (wave < CW)
                    stage_qt();
                __syncthreads();
            }
        }

        // (6) readout on MFMA: Y^T = B_c Z^T, so that each lane holds four
        //     consecutive channels of one token (16-byte stores). With more
        //     waves than 16-wide channel tiles, wave w takes the token tiles
        //     tm = w, w + NW, ... and writes whole output rows of its head;
        //     otherwise wave w takes the channel tiles tn = w, w + NW, ... for
        //     every token tile.
        if constexpr (OUT) {
            constexpr bool BY_TOKENS = NW > NTC;
            if constexpr (BY_TOKENS) {
                // a token tile's z rows once for all its channel tiles, and
                // every operand read before the first product
                for (int tm = wave; tm < nwin; tm += NW) {
                    float a[KS], a2[KS], br[NTC][KS];
                    ldrow(KZ, tm * 16 + lm, lk * KS, a);
                    if (JS == 2)
                        ldrow(KZ2, tm * 16 + lm, lk * KS, a2);
#pragma unroll
                    for (int tn = 0; tn < NTC; ++tn)
                        ldrow(Bs, tn * 16 + lm, lk * KS, br[tn]);
#pragma unroll
                    for (int s = 0; s < KS; ++s) {
                        asm volatile("" ::"v"(a[s]));
                        if (JS == 2)
                            asm volatile("" ::"v"(a2[s]));
#pragma unroll
                        for (int tn = 0; tn < NTC; ++tn)
                            asm volatile("" ::"v"(br[tn][s]));
                    }
                    if (JS == 2) {
#pragma unroll
                        for (int s = 0; s < KS; ++s)
                            a[s] += a2[s];
                    }
                    const int u0 = tm * 16 + lm;
#pragma unroll
                    for (int tn = 0; tn < NTC; ++tn) {
                        v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int s = 0; s < KS; ++s)
                            acc = mfma4(br[tn][s], a[s], acc);
                        if (u0 < nt) {
                            float *orow = out + (out_row0 + s0 + u0) * C + static_cast<size_t>(h) * D + 4 * lk;
                            *reinterpret_cast<float4 *>(orow + tn * 16) =
                                make_float4(acc[0], acc[1], acc[2], acc[3]);
                        }
                    }
                }
            } else {
                for (int tn = wave; tn < NTC; tn += NW)
                    for (int tm = 0; tm < nwin; ++tm)
                        readout_tile(tm, tn);
            }
        }
        v4f pt_d[RTD_D];
        if constexpr (DIRECT) {
            if (chunk_end && cend < N)
                direct_products(pt_d);
        }

        SRNL_PHASE(5);
        if (chunk_end) {
            if (cend < N) {
                // (7) refresh the boundary: B <- B Q_L (tiles split over the
                //     waves). Q_L^T is staged already unless it covers the z
                //     rows, which the readout above had to finish with first.
                // frozen key/value and dynamics memories: only the M_c
                // tiles (rows < D) and no vector memory are stored back
                const bool frz = (flags & F_FREEZE_KV) != 0;
                if constexpr (DIRECT) {
                    direct_store(pt_d, frz);
                } else {
                    if constexpr (Cfg::QT_IN_TOK) {
                        __syncthreads();
                        if (wave < CW)
                            stage_qt();
                        __syncthreads();
                    }
                    // (with DEFER_MC the M_c tiles wait for the next sub-block)
                    constexpr int T0 = DEFER_MC ? NTC * NTC : 0;   // first tile refreshed here
                    constexpr int RTH = RT - T0, RTWH = (RTH + NW - 1) / NW;
                    v4f racc[RTWH];
#pragma unroll
                    for (int w = 0; w < RTWH; ++w) {
                        const int tile = T0 + wave + w * NW;
                        if (RTH % NW != 0 && tile >= RT)
                            break;
                        const int tm = tile / NTC, tn = tile % NTC;
                        float a[KS], bq[KS];
                        ldrow(Bs, tm * 16 + lm, lk * KS, a);
                        ldrow(Qt, tn * 16 + lm, lk * KS, bq);
                        v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int s = 0; s < KS; ++s)
                            acc = mfma4(a[s], bq[s], acc);
                        racc[w] = acc;
                    }
                    // vector memories: two lanes per output element, each over
                    // half of the reduction index, summed by DPP (the same order
                    // in every sub-block configuration)
                    constexpr int VG = 2;
                    float vacc = 0.f;
                    const int vo = tid / VG, vpart = tid % VG;
                    const int vv = vo / D, vj = vo % D;
                    if (tid < 2 * D * VG && !frz) {
#pragma unroll
                        for (int k = 0; k < D / (4 * VG); ++k) {
                            const int c = 4 * (vpart * (D / (4 * VG)) + k);
                            const float4 bb = ld4(Bs + ix(3 * D + vv, c));
                            const float4 qq = ld4(Qt + ix(vj, c));
                            vacc = fmaf(bb.x, qq.x, vacc);
                            vacc = fmaf(bb.y, qq.y, vacc);
                            vacc = fmaf(bb.z, qq.z, vacc);
                            vacc = fmaf(bb.w, qq.w, vacc);
                        }
                        vacc = group_sum<VG>(vacc);
                    }
                    __syncthreads();
#pragma unroll
                    for (int w = 0; w < RTWH; ++w) {
                        const int tile = T0 + wave + w * NW;
                        if (RTH % NW != 0 && tile >= RT)
                            break;
                        const int tm = tile / NTC, tn = tile % NTC;
#pragma unroll
                        for (int rr = 0; rr < 4; ++rr)
                            if (!frz || tm < NTC)
                                Bs[ix(tm * 16 + 4 * lk + rr, tn * 16 + lm)] = racc[w][rr];
                    }
                    if (tid < 2 * D * VG && vpart == 0 && !frz)
                        Bs[ix(3 * D + vv, vj)] = vacc;
                    if constexpr (DEFER_MC)
                        mc_pending = true;
                }
            }
            reset_q();
        }
        SRNL_PHASE(6);
#if SRNL_PHASE_CLOCKS
        ph_n += 1;
#endif
        if (s1 >= N)
            break;
        s0 = s1;
        c0 = c1;
        cend = cend1;
        nt = nt1;
    }
#if SRNL_PHASE_CLOCKS
    if (wave == 0 && lane == 0 && blockIdx.x < kPhaseBlocks) {
        unsigned long long *o = srnl_phase_buf + blockIdx.x * kPhaseSlots;
        for (int k = 0; k < kPhaseSlots - 2; ++k)
            o[k] = (k < 7) ? ph_lds[k] : 0;
        o[kPhaseSlots - 2] = ph_n;
        o[kPhaseSlots - 1] = clock64() - ph_t0;
    }
#endif
}

// ------------------------------------------------------------ finite check

// NaN or Inf: the exponent field is all ones
__device__ __forceinline__ unsigned nonfinite(float v) { return (__float_as_uint(v) & 0x7F800000u) == 0x7F800000u; }
__device__ __forceinline__ unsigned nonfinite(uint16_t v) { return (v & 0x7F80u) == 0x7F80u; }

// counters[0..1] = 0, enqueued on the stream like the counting kernels
__global__ void zero_counters_kernel(unsigned *__restrict__ counters)
{
    if (threadIdx.x < 2)
        counters[threadIdx.x] = 0u;
}

// *counter += number of NaN or Inf among v[0 .. n)
template <typename T>
__global__ __launch_bounds__(256) void nonfinite_kernel(const T *__restrict__ v, long long n,
                                                        unsigned *__restrict__ counter)
{
    __shared__ unsigned part[4];
    unsigned c = 0;
    for (long long i = blockIdx.x * 256LL + threadIdx.x; i < n; i += static_cast<long long>(gridDim.x) * 256)
        c += nonfinite(v[i]);
    for (int off = 32; off > 0; off >>= 1)
        c += __shfl_xor(c, off);
    if ((threadIdx.x & 63) == 0)
        part[threadIdx.x >> 6] = c;
    __syncthreads();
    if (threadIdx.x == 0) {
        const unsigned t = part[0] + part[1] + part[2] + part[3];
        if (t)
            atomicAdd(counter, t);
    }
}

// ------------------------------------------------------------ fuse kernel

__device__ __forceinline__ void store4(float *o, float4 a) { *reinterpret_cast<float4 *>(o) = a; }
__device__ __forceinline__ void store4(uint16_t *o, float4 a)
{
    uint2 w;
    w.x = static_cast<uint32_t>(f32_to_bf16(a.x)) | (static_cast<uint32_t>(f32_to_bf16(a.y)) << 16);
    w.y = static_cast<uint32_t>(f32_to_bf16(a.z)) | (static_cast<uint32_t>(f32_to_bf16(a.w)) << 16);
    *reinterpret_cast<uint2 *>(o) = w;
}

// Block shape of the restore/fuse and gather kernels: threadIdx.x walks the
// 16-byte (or narrower) channel vectors of one token, threadIdx.y the cells,
// so a token's index math is done once per thread with one 32-bit division
// at most, and a wave moves whole rows of consecutive tokens.
struct PlaneShape {
    int cv = 1, ty = 1;  // vectors per token, tokens per block
};

PlaneShape plane_shape(int vectors_per_token)
{
    PlaneShape s;
    s.cv = vectors_per_token < 256 ? vectors_per_token : 256;
    s.ty = 256 / s.cv;
    return s;
}

// One thread per 4 channels of one grid cell of batch item b = blockIdx.y
// (grid-strided); routes summed in ascending order [OVERVIEW scanning and
// chunking; SUMMARY 2-D maps].
template <typename OutT>
__global__ __launch_bounds__(256) void fuse_kernel(const float *__restrict__ y,
                                                   const float *__restrict__ scales,
                                                   OutT *__restrict__ out, int B, int H,
                                                   int W, int C, unsigned mask)
{
    const int N = H * W;
    const int C4 = C >> 2;
    const int pix = blockIdx.x * blockDim.y + threadIdx.y;
    if (pix >= N)
        return;
    const int i = static_cast<int>(static_cast<unsigned>(pix) / static_cast<unsigned>(W));
    const int j = pix - i * W;
    int ts[4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
        ts[r] = static_cast<int>(route_step(r, H, W, N, i, j));
    for (int b = blockIdx.y; b < B; b += gridDim.y) {
        for (int cv = threadIdx.x; cv < C4; cv += blockDim.x) {
            float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
            int slot = 0;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if (!(mask & (1u << r)))
                    continue;
                const float4 yv = *reinterpret_cast<const float4 *>(
                    y + ((static_cast<long long>(slot) * B + b) * N + ts[r]) * C + cv * 4);
                const float4 s = *reinterpret_cast<const float4 *>(scales + r * C + cv * 4);
                acc.x = fmaf(s.x, yv.x, acc.x);
                acc.y = fmaf(s.y, yv.y, acc.y);
                acc.z = fmaf(s.z, yv.z, acc.z);
                acc.w = fmaf(s.w, yv.w, acc.w);
                ++slot;
            }
            store4(out + (static_cast<long long>(b) * N + pix) * C + cv * 4, acc);
        }
    }
}

// ------------------------------------------------------------ gather kernel

// out[slot][b][t_r(i, j)][:] = x[b][i][j][:] for every active route r, with
// t_r the step at which route r visits cell (i, j): each token row of x is
// read once and written to every route slot, moved as V vectors. Cell
// pix = blockIdx.x * blockDim.y + threadIdx.y in grid order, batch item
// b = blockIdx.y (grid-strided).
template <typename V>
__global__ __launch_bounds__(256) void gather_kernel(const char *__restrict__ x,
                                                     char *__restrict__ out, int B, int H,
                                                     int W, int row_bytes, unsigned mask)
{
    const int N = H * W;
    const int pix = blockIdx.x * blockDim.y + threadIdx.y;
    if (pix >= N)
        return;
    const int i = static_cast<int>(static_cast<unsigned>(pix) / static_cast<unsigned>(W));
    const int j = pix - i * W;
    int ts[4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
        ts[r] = static_cast<int>(route_step(r, H, W, N, i, j));
    const int nv = row_bytes / static_cast<int>(sizeof(V));
    for (int b = blockIdx.y; b < B; b += gridDim.y) {
        const V *src = reinterpret_cast<const V *>(
            x + (static_cast<long long>(b) * N + pix) * row_bytes);
        for (int cv = threadIdx.x; cv < nv; cv += blockDim.x) {
            const V val = src[cv];
            int slot = 0;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if (!(mask & (1u << r)))
                    continue;
                V *dst = reinterpret_cast<V *>(
                    out + ((static_cast<long long>(slot) * B + b) * N + ts[r]) * row_bytes);
                dst[cv] = val;
                ++slot;
            }
        }
    }
}

// ------------------------------------------------------------ state init

// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11).
__device__ __forceinline__ void philox4x32_10(uint32_t c[4], uint32_t k0, uint32_t k1)
{
#pragma unroll
    for (int rnd = 0; rnd < 10; ++rnd) {
        const uint32_t hi0 = __umulhi(0xD2511F53u, c[0]), lo0 = 0xD2511F53u * c[0];
        const uint32_t hi1 = __umulhi(0xCD9E8D57u, c[2]), lo1 = 0xCD9E8D57u * c[2];
        const uint32_t n0 = hi1 ^ c[1] ^ k0;
        const uint32_t n2 = hi0 ^ c[3] ^ k1;
        c[0] = n0;
        c[1] = lo1;
        c[2] = n2;
        c[3] = lo0;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
}

__global__ __launch_bounds__(256) void init_kernel(float *__restrict__ st, long long n,
                                                   unsigned long long seed, float stdv)
{
    const long long nb = (n + 3) / 4;
    const double s = static_cast<double>(stdv);
    for (long long k = blockIdx.x * static_cast<long long>(blockDim.x) + threadIdx.x; k < nb;
         k += static_cast<long long>(gridDim.x) * blockDim.x) {
        uint32_t c[4] = {static_cast<uint32_t>(k), static_cast<uint32_t>(k >> 32), 2u,
                         0x53524E4Cu};
        philox4x32_10(c, static_cast<uint32_t>(seed), static_cast<uint32_t>(seed >> 32));
        double u[4];
#pragma unroll
        for (int a = 0; a < 4; ++a)
            u[a] = (static_cast<double>(c[a]) + 0.5) * 2.3283064365386963e-10;  // 2^-32
        const double r0 = sqrt(-2.0 * log(u[0])), t0 = 6.283185307179586 * u[1];
        const double r1 = sqrt(-2.0 * log(u[2])), t1 = 6.283185307179586 * u[3];
        const double z[4] = {r0 * cos(t0), r0 * sin(t0), r1 * cos(t1), r1 * sin(t1)};
#pragma unroll
        for (int a = 0; a < 4; ++a)
            if (4 * k + a < n)
                st[4 * k + a] = static_cast<float>(s * z[a]);
    }
}

// ------------------------------------------------------------ backward pass

#include "srnl_bwd.inc"
#include "srnl_bwd_wy.inc"
#include "srnl_bwd_wy64.inc"

// ------------------------------------------------------------ host side

bool valid_d(int d) { return d == 4 || d == 8 || d == 16 || d == 32 || d == 64; }

int popcount4(unsigned m)
{
    int n = 0;
    for (int r = 0; r < 4; ++r)
        n += (m >> r) & 1u;
    return n;
}

// true if p is device (or managed) memory visible to HIP
bool is_device_ptr(const void *p)
{
    if (!p)
        return false;
    hipPointerAttribute_t a;
    hipError_t e = hipPointerGetAttributes(&a, p);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return false;
    }
    return a.type == hipMemoryTypeDevice || a.type == hipMemoryTypeManaged;
}

// element count a*b*c*d*e, or -1 on overflow past 2^62
long long checked_count(std::initializer_list<long long> dims)
{
    __int128 n = 1;
    for (long long v : dims) {
        n *= v;
        if (n > (static_cast<__int128>(1) << 62))
            return -1;
    }
    return static_cast<long long>(n);
}

srnl_status launch_check(const char *what)
{
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return fail(SRNL_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
    return SRNL_OK;
}

int grid_for(long long work, int block)
{
    long long g = (work + block - 1) / block;
    if (g > 65536LL * 8)
        g = 65536LL * 8;
    return static_cast<int>(g < 1 ? 1 : g);
}

// Sub-block length T (tokens) of the MFMA scan kernel, from the longest
// chunk of the active routes: a chunk no longer than 16 or 32 tokens takes a
// sub-block of that length, whose smaller LDS footprint fits more chains on a
// CU. Longer chunks take 64 tokens at d = 32 (32 at d = 64); at d = 32, when
// there are no more chains than CUs, 128 tokens on 8 waves, which halves the
// per-token latency of every phase but the token-order update. Waves per
// chain NW: 2 for d = 32 at T <= 32, 8 at T = 128, else 4.
template <int D> struct MfmaTMax { static constexpr int value = (D == 32) ? 64 : 32; };
template <int D, int T> struct MfmaNW {
    static constexpr int value = (D == 32 && T <= 32) ? 2 : (T == 128) ? 8 : 4;
};
constexpr int kFewChains = 256;   // one chain per CU at most

int longest_chunk(int H, int W, unsigned mask, int chunk_row, int chunk_col)
{
    const long long N = static_cast<long long>(H) * W;
    long long L = 0;
    for (int r = 0; r < 4; ++r) {
        if (!(mask & (1u << r)))
            continue;
        long long l = (r < 2) ? (chunk_row > 0 ? chunk_row : W) : (chunk_col > 0 ? chunk_col : H);
        if (l > N)
            l = N;
        if (l > L)
            L = l;
    }
    return static_cast<int>(L);
}

// With SAVE the kernel writes the record FwdSave sv for the windowed
// backward (readout after the write only), and the route outputs too with OUT.
template <int D, int T, typename InT, bool SAVE = false, bool OUT = !SAVE>
void launch_scan_mfma(const void *x, const srnl_params *p, int B, int H, int W, int C,
                      int heads, unsigned mask, int R, int nchains, int nblocks, float *out,
                      FwdSave sv = FwdSave())
{
    constexpr int NW = MfmaNW<D, T>::value;
    hipStream_t st = static_cast<hipStream_t>(p->stream);
    const bool before = (p->flags & F_READ_BEFORE) != 0, has_q = p->q != nullptr;
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, dim3(nblocks), dim3(NW * 64), 0, st,
                           static_cast<const InT *>(x), static_cast<const InT *>(p->q),
                           p->states, out, B, H, W, C, heads, mask, R, p->alpha_max, p->eps,
                           p->chunk_row, p->chunk_col, p->flags, nchains, sv);
    };
    if constexpr (SAVE) {
        has_q ? go(scan_mfma_kernel<D, NW, T, false, true, InT, true, OUT>)
              : go(scan_mfma_kernel<D, NW, T, false, false, InT, true, OUT>);
    } else if (before) {
        has_q ? go(scan_mfma_kernel<D, NW, T, true, true, InT>)
              : go(scan_mfma_kernel<D, NW, T, true, false, InT>);
    } else {
        has_q ? go(scan_mfma_kernel<D, NW, T, false, true, InT>)
              : go(scan_mfma_kernel<D, NW, T, false, false, InT>);
    }
}

template <int D, typename InT>
srnl_status launch_scan(const void *x, const srnl_params *p, int B, int H, int W, int C,
                        int heads, unsigned mask, float *out)
{
    const int R = popcount4(mask);
    const long long nchains = static_cast<long long>(R) * B * heads;
    if (nchains > INT_MAX - 8)
        return fail(SRNL_ERR_ARG, "too many chains (routes * B * heads)");
    const int nblocks = static_cast<int>((nchains + 7) / 8 * 8);
    const int nc = static_cast<int>(nchains);
    if constexpr (D >= 32) {
        const int L = longest_chunk(H, W, mask, p->chunk_row, p->chunk_col);
        if (L <= 16)
            launch_scan_mfma<D, 16, InT>(x, p, B, H, W, C, heads, mask, R, nc, nblocks, out);
        else if (L <= 32 || MfmaTMax<D>::value == 32)
            launch_scan_mfma<D, 32, InT>(x, p, B, H, W, C, heads, mask, R, nc, nblocks, out);
        else if (D == 32 && L > 64 && nc <= kFewChains)
            launch_scan_mfma<D, (D == 32 ? 128 : 32), InT>(x, p, B, H, W, C, heads, mask, R, nc,
                                                           nblocks, out);
        else
            launch_scan_mfma<D, MfmaTMax<D>::value, InT>(x, p, B, H, W, C, heads, mask, R, nc,
                                                         nblocks, out);
        return launch_check("scan_mfma_kernel");
    } else {
        hipStream_t st = static_cast<hipStream_t>(p->stream);
        hipLaunchKernelGGL((scan_simple_kernel<D, InT>), dim3(nblocks), dim3(ScanCfg<D>::NT), 0,
                           st, static_cast<const InT *>(x), static_cast<const InT *>(p->q),
                           p->states, out, B, H, W, C, heads, mask, R, p->alpha_max, p->eps,
                           p->chunk_row, p->chunk_col, p->flags, nc);
        return launch_check("scan_simple_kernel");
    }
}

// The recording forward (readout after the write; d = 32, or d = 64 with
// chunks of at most 16 tokens): the record sv of every chain for the
// windowed backward, and the route outputs when out is not NULL. The
// sub-block follows the longest chunk.
template <int D, typename InT>
srnl_status launch_record_fwd(const void *x, const srnl_params *p, int B, int H, int W, int C,
                              int heads, unsigned mask, float *out, const FwdSave &sv)
{
    const int R = popcount4(mask);
    const long long nchains = static_cast<long long>(R) * B * heads;
    if (nchains > INT_MAX - 8)
        return fail(SRNL_ERR_ARG, "too many chains (routes * B * heads)");
    const int nc = static_cast<int>(nchains);
    const int nblocks = (nc + 7) / 8 * 8;
    const int L = longest_chunk(H, W, mask, p->chunk_row, p->chunk_col);
    auto go = [&](auto t, auto o) {
        constexpr int T = decltype(t)::value;
        constexpr bool O = decltype(o)::value;
        launch_scan_mfma<D, T, InT, true, O>(x, p, B, H, W, C, heads, mask, R, nc, nblocks, out, sv);
    };
    auto pick = [&](auto o) {
        if constexpr (D == 64) {   // chunks of at most 16 tokens only
            go(std::integral_constant<int, 16>(), o);
        } else {
            if (L <= 16)
                go(std::integral_constant<int, 16>(), o);
            else if (L <= 32)
                go(std::integral_constant<int, 32>(), o);
            else
                go(std::integral_constant<int, 64>(), o);
        }
    };
    if (out)
        pick(std::true_type());
    else
        pick(std::false_type());
    return launch_check("scan_mfma_kernel (forward record)");
}

template <typename InT>
srnl_status dispatch_scan(int d, const void *x, const srnl_params *p, int B, int H, int W,
                          int C, int heads, unsigned mask, float *out)
{
    switch (d) {
    case 4: return launch_scan<4, InT>(x, p, B, H, W, C, heads, mask, out);
    case 8: return launch_scan<8, InT>(x, p, B, H, W, C, heads, mask, out);
    case 16: return launch_scan<16, InT>(x, p, B, H, W, C, heads, mask, out);
    case 32: return launch_scan<32, InT>(x, p, B, H, W, C, heads, mask, out);
    case 64: return launch_scan<64, InT>(x, p, B, H, W, C, heads, mask, out);
    }
    return fail(SRNL_ERR_ARG, "head dim must be 4, 8, 16, 32 or 64");
}

srnl_status check_grid(int B, int H, int W, int C, unsigned mask, long long *n_out)
{
    if (B < 0 || H < 0 || W < 0)
        return fail(SRNL_ERR_ARG, "B, H and W must be >= 0");
    if (C < 4 || (C & 3))
        return fail(SRNL_ERR_ARG, "C must be a positive multiple of 4");
    if (mask < 1u || mask > 15u)
        return fail(SRNL_ERR_ARG, "route_mask must be in 1..15");
    const long long n = checked_count({popcount4(mask), B, H, W, C});
    if (n < 0 || static_cast<long long>(H) * W > INT_MAX)
        return fail(SRNL_ERR_ARG, "grid too large");
    *n_out = n;
    return SRNL_OK;
}

// Workspace layout of srnl_scan_bwd (floats, 64-float aligned parts):
// per-chain scratch, per-route dx partials, per-route dq partials, per-chain
// initial-state gradients.
struct BwdLayout {
    long long chain_floats = 0, chains = 0, o_dx = 0, o_dq = 0, o_st = 0, total = -1;
    bool record_given = false;   // the forward record comes in params->workspace
};   // total < 0: the sizes overflow

long long align64(long long n) { return (n + 63) / 64 * 64; }

// The windowed backward (readout after the write; d = 32, or d = 64 when no
// active route's chunk is longer than one 16-token window) reads a record of
// the forward instead of re-running it token by token.
bool bwd_windowed(int d, const srnl_params *p, int H, int W, unsigned mask)
{
    if (p->flags & F_READ_BEFORE)
        return false;
    return d == 32 || (d == 64 && longest_chunk(H, W, mask, p->chunk_row, p->chunk_col) <= 16);
}

// Floats of one chain's forward record for nch chunks of nwc window slots.
long long record_floats(int d, long long nch, long long nwc)
{
    return d == 64 ? SaveLayout<64>{nch, nwc}.floats() : SaveLayout<32>{nch, nwc}.floats();
}

// Floats of one chain's forward record (the longest over the active routes),
// 64-float aligned.
long long record_chain_floats(int d, int H, int W, unsigned mask, const srnl_params *p)
{
    const long long N = static_cast<long long>(H) * W;
    long long m = 0;
    for (int r = 0; r < 4; ++r) {
        if (!(mask & (1u << r)))
            continue;
        long long L = (r < 2) ? (p->chunk_row > 0 ? p->chunk_row : W)
                              : (p->chunk_col > 0 ? p->chunk_col : H);
        if (L > N)
            L = N;
        if (L < 1)
            L = 1;
        const long long f = record_floats(d, (N + L - 1) / L, (L + 15) / 16);
        if (f > m)
            m = f;
    }
    return align64(m);
}

// Bytes of the record SRNL_FLAG_RECORD asks for (0 where the windowed
// backward does not apply), 256-byte aligned; -1 past 2^62 bytes.
long long record_bytes(int B, int H, int W, int heads, int d, unsigned mask, const srnl_params *p)
{
    if (!(p->flags & F_RECORD) || !bwd_windowed(d, p, H, W, mask))
        return 0;
    const long long chains = static_cast<long long>(popcount4(mask)) * B * heads;
    long long f = 0;
    if (__builtin_mul_overflow(chains, record_chain_floats(d, H, W, mask, p), &f) ||
        f > (1LL << 60) - 64)
        return -1;
    return (f * 4 + 255) / 256 * 256;
}

BwdLayout bwd_layout(int B, int H, int W, int C, int heads, int d, unsigned mask,
                     const srnl_params *p)
{
    BwdLayout l;
    const bool wy = bwd_windowed(d, p, H, W, mask);
    const int R = popcount4(mask);
    const long long N = static_cast<long long>(H) * W;
    const long long rows = 3LL * d + 2;
    for (int r = 0; r < 4; ++r) {
        if (!(mask & (1u << r)))
            continue;
        long long L = (r < 2) ? (p->chunk_row > 0 ? p->chunk_row : W)
                              : (p->chunk_col > 0 ? p->chunk_col : H);
        if (L > N)
            L = N;
        if (L < 1)
            L = 1;
        const long long nch = (N + L - 1) / L;
        const long long f = wy ? record_floats(d, nch, (L + 15) / 16)
                               : nch * rows * d + L * d * d + rows * d;
        if (f > l.chain_floats)
            l.chain_floats = f;
    }
    l.chain_floats = align64(l.chain_floats);
    l.chains = static_cast<long long>(R) * B * heads;
    l.record_given = wy && (p->flags & F_RECORD);
    const long long part = align64(static_cast<long long>(R) * B * N * C);
    long long rec = 0;
    if (!l.record_given && __builtin_mul_overflow(l.chains, l.chain_floats, &rec))
        return l;
    l.o_dx = rec;
    l.o_dq = l.o_dx + part;
    l.o_st = l.o_dq + (p->q ? part : 0);
    const long long t = l.o_st + align64(l.chains * rows * d);
    if (rec > (1LL << 60) || t > (1LL << 60))
        return l;
    l.total = t;
    return l;
}

// The fusion backward's part of the operator's one-call backward, run after
// the windowed adjoint (its partial sums in one launch with the dx sum, then
// the scales' gradient): dout [B][H][W][C], the route outputs y, the scales,
// nfb partial-sum blocks of rb grid cells in part, dscales.
struct FuseTail {
    const float *dout, *y, *scales;
    float *part, *dscales;
    long long rb, nfb;
};

template <int D, typename InT>
srnl_status launch_scan_bwd(const void *x, const srnl_params *p, int B, int H, int W, int C,
                            int heads, unsigned mask, const float *dy, float *ws,
                            const BwdLayout &l, float *dx, float *dq, float *dstates, int nr_out,
                            const float *ysc, const FuseTail *ft)
{
    const int R = popcount4(mask);
    const int nchains = static_cast<int>(l.chains);
    hipStream_t st = static_cast<hipStream_t>(p->stream);
    float *dxr = ws + l.o_dx, *dqr = p->q ? ws + l.o_dq : nullptr, *dstp = ws + l.o_st;
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, dim3(nchains), dim3(BwdCfg<D>::NT), 0, st,
                           static_cast<const InT *>(x), static_cast<const InT *>(p->q), p->states,
                           dy, ws, l.chain_floats, B, H, W, C, heads, mask, R, p->alpha_max, p->eps,
                           p->chunk_row, p->chunk_col, p->flags, nchains, dxr, dqr, dstp);
    };
    srnl_status s;
    if constexpr (D == 32 || D == 64) {
        if (bwd_windowed(D, p, H, W, mask)) {
            // the forward record (from the caller's forward, or recorded
            // here), then the windowed backward
            const int nblocks = (nchains + 7) / 8 * 8;
            const FwdSave sv{l.record_given ? static_cast<float *>(p->workspace) : ws,
                             l.chain_floats};
            if (!l.record_given) {
                s = launch_record_fwd<D, InT>(x, p, B, H, W, C, heads, mask, nullptr, sv);
                if (s != SRNL_OK)
                    return s;
            }
            auto gw = [&](auto kern, int nt) {
                hipLaunchKernelGGL(kern, dim3(nblocks), dim3(nt), 0, st,
                                   static_cast<const InT *>(x), static_cast<const InT *>(p->q), dy,
                                   sv, B, H, W, C, heads, mask, R, p->alpha_max, p->eps,
                                   p->chunk_row, p->chunk_col, p->flags, nchains, dxr, dqr, dstp);
            };
            if constexpr (D == 32) {
                // ysc: dy is the fused output's gradient, scaled per route here
                auto g32 = [&](auto kern) {
                    hipLaunchKernelGGL(kern, dim3(nblocks), dim3(wyb::NT), 0, st,
                                       static_cast<const InT *>(x), static_cast<const InT *>(p->q), dy,
                                       ysc, sv, B, H, W, C, heads, mask, R, p->alpha_max, p->eps,
                                       p->chunk_row, p->chunk_col, p->flags, nchains, dxr, dqr, dstp);
                };
                if (p->q)
                    ysc ? g32(scan_bwd_wy_kernel<true, InT, true>) : g32(scan_bwd_wy_kernel<true, InT>);
                else
                    ysc ? g32(scan_bwd_wy_kernel<false, InT, true>) : g32(scan_bwd_wy_kernel<false, InT>);
                s = launch_check("scan_bwd_wy_kernel");
            } else {
                if (p->q)
                    gw(scan_bwd_wy64_kernel<true, InT>, wy1::NT);
                else
                    gw(scan_bwd_wy64_kernel<false, InT>, wy1::NT);
                s = launch_check("scan_bwd_wy64_kernel");
            }
        } else {
            // the sequential adjoint: reading before the write, or (d = 64)
            // chunks longer than one window
            if constexpr (D == 64) {
                if (p->flags & F_READ_BEFORE)
                    go(scan_bwd_kernel<D, true, InT>);
                else
                    go(scan_bwd_kernel<D, false, InT>);
            } else {
                go(scan_bwd_kernel<D, true, InT>);
            }
            s = launch_check("scan_bwd_kernel");
        }
    } else {
        if (p->flags & F_READ_BEFORE)
            go(scan_bwd_kernel<D, true, InT>);
        else
            go(scan_bwd_kernel<D, false, InT>);
        s = launch_check("scan_bwd_kernel");
    }
    if (s != SRNL_OK)
        return s;
    const long long n = static_cast<long long>(B) * H * W * C;
    if (ft && !p->q && nr_out == 4) {
        // the fusion partial sums, the dx sum and the state gradient in one
        // launch, then the scales' gradient
        const int sz = 3 * D * D + 2 * D;
        const long long nsum = grid_for(n / 4, 256);
        const long long nst = (4LL * heads * sz + 63) / 64;
        hipLaunchKernelGGL(bwd_tail_kernel, dim3(static_cast<unsigned>(ft->nfb + nsum + nst)), dim3(256), 0,
                           st, ft->dout, ft->y, ft->scales, ft->part, B, H, W, C, mask, ft->rb, ft->nfb,
                           dxr, dx, R, n, nsum, dstp, dstates, heads, sz);
        hipLaunchKernelGGL(fuse_bwd_scales_kernel, dim3(grid_for(4LL * C * 64, 256)), dim3(256), 0, st,
                           ft->part, ft->dscales, C, mask, static_cast<int>(ft->nfb));
        return launch_check("scan_fuse_bwd tail");
    }
    if (ft) {
        // with separate queries: the dq sum too, as its own launch
        const long long nsum = grid_for(n / 4, 256);
        hipLaunchKernelGGL(bwd_tail_kernel, dim3(static_cast<unsigned>(ft->nfb + nsum)), dim3(256), 0, st,
                           ft->dout, ft->y, ft->scales, ft->part, B, H, W, C, mask, ft->rb, ft->nfb,
                           dxr, dx, R, n, nsum, nullptr, nullptr, heads, 0);
        hipLaunchKernelGGL(fuse_bwd_scales_kernel, dim3(grid_for(4LL * C * 64, 256)), dim3(256), 0, st,
                           ft->part, ft->dscales, C, mask, static_cast<int>(ft->nfb));
    } else {
        hipLaunchKernelGGL(sum_slots_kernel, dim3(grid_for(n / 4, 256)), dim3(256), 0, st, dxr, dx, R, n);
    }
    if (p->q)
        hipLaunchKernelGGL(sum_slots_kernel, dim3(grid_for(n / 4, 256)), dim3(256), 0, st, dqr, dq, R, n);
    const int sz = 3 * D * D + 2 * D;
    const long long nst = static_cast<long long>(nr_out) * heads * sz;
    hipLaunchKernelGGL(states_grad_kernel, dim3(static_cast<unsigned>((nst + 63) / 64)), dim3(256), 0, st,
                       dstp, dstates, B, heads, R, mask, sz, nr_out);
    return launch_check("scan_bwd reductions");
}

template <typename InT>
srnl_status dispatch_scan_bwd(int d, const void *x, const srnl_params *p, int B, int H, int W,
                              int C, int heads, unsigned mask, const float *dy, float *ws,
                              const BwdLayout &l, float *dx, float *dq, float *dstates, int nr_out,
                              const float *ysc, const FuseTail *ft)
{
    switch (d) {
    case 4: return launch_scan_bwd<4, InT>(x, p, B, H, W, C, heads, mask, dy, ws, l, dx, dq, dstates, nr_out, ysc, ft);
    case 8: return launch_scan_bwd<8, InT>(x, p, B, H, W, C, heads, mask, dy, ws, l, dx, dq, dstates, nr_out, ysc, ft);
    case 16: return launch_scan_bwd<16, InT>(x, p, B, H, W, C, heads, mask, dy, ws, l, dx, dq, dstates, nr_out, ysc, ft);
    case 32: return launch_scan_bwd<32, InT>(x, p, B, H, W, C, heads, mask, dy, ws, l, dx, dq, dstates, nr_out, ysc, ft);
    case 64: return launch_scan_bwd<64, InT>(x, p, B, H, W, C, heads, mask, dy, ws, l, dx, dq, dstates, nr_out, ysc, ft);
    }
    return fail(SRNL_ERR_ARG, "head dim must be 4, 8, 16, 32 or 64");
}

constexpr long long kFuseBwdRows = 256;    // grid cells per partial-sum block of srnl_fuse_bwd

long long fuse_bwd_blocks(int B, int H, int W)
{
    const long long rows = static_cast<long long>(B) * H * W;
    return (rows + kFuseBwdRows - 1) / kFuseBwdRows;
}

// validation shared by the forward and the backward scan
srnl_status check_scan_args(int B, int H, int W, int C, int heads, int d, unsigned route_mask,
                            const srnl_params *p, long long *n)
{
    if (!p)
        return fail(SRNL_ERR_PTR, "params is NULL");
    if (!valid_d(d))
        return fail(SRNL_ERR_ARG, "head dim must be 4, 8, 16, 32 or 64");
    if (heads < 1 || C != heads * d)
        return fail(SRNL_ERR_ARG, "C must equal heads * d with heads >= 1");
    srnl_status s = check_grid(B, H, W, C, route_mask, n);
    if (s != SRNL_OK)
        return s;
    if (!(p->alpha_max > 0.0f && p->alpha_max < 1.0f))
        return fail(SRNL_ERR_ARG, "alpha_max must lie in (0, 1)");
    if (!(p->eps > 0.0f) || !std::isfinite(p->eps))
        return fail(SRNL_ERR_ARG, "eps must be positive and finite");
    if (p->chunk_row < 0 || p->chunk_col < 0)
        return fail(SRNL_ERR_ARG, "chunk lengths must be >= 0");
    if (p->flags & ~0xFFu)
        return fail(SRNL_ERR_ARG, "unknown flag bits");
    if (p->in_dtype != SRNL_F32 && p->in_dtype != SRNL_BF16)
        return fail(SRNL_ERR_DTYPE, "in_dtype must be SRNL_F32 or SRNL_BF16");
    return SRNL_OK;
}

#include "srnl_block.inc"

// Workspace of srnl_block_fwd (floats, 64-float aligned parts): u, q and the
// fused operator output s ([B][H][W][C] each), then the route outputs
// [R][B][H*W][C].
// Block workspace (floats, 64-float aligned parts): u, q, the fused operator
// output s, the route outputs y, and for the wide kernels (C > 256) h.
struct BlockLayout {
    long long plane = 0, o_q = 0, o_s = 0, o_y = 0, o_h = 0, total = 0;
};
BlockLayout block_layout(int B, int H, int W, int C, unsigned mask)
{
    BlockLayout l;
    l.plane = align64(static_cast<long long>(B) * H * W * C);
    l.o_q = l.plane;
    l.o_s = 2 * l.plane;
    l.o_y = 3 * l.plane;
    l.o_h = l.o_y + align64(static_cast<long long>(popcount4(mask)) * B * H * W * C);
    l.total = l.o_h + (C > 256 ? l.plane : 0);
    return l;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// workspace of srnl_scan_fwd with SRNL_FLAG_CHECK_FINITE: two counters
constexpr size_t kScanCheckBytes = 256;

// Scratch of srnl_fuse_bwd_noalloc: the per-block partial sums of the scale
// gradient live in this library-owned device array (one copy per GPU, held
// until the process ends) instead of a caller's workspace. Every call
// overwrites the part it uses before reading it, so nothing needs clearing;
// calls that overlap on one GPU share the array and race. In host code the
// array's name is a stand-in, not a device address: host code uses only the
// address looked up once per device by fuse_bwd_scratch.
constexpr size_t kFuseBwdScratchBytes = SRNL_FUSE_BWD_SCRATCH_BYTES;
static __device__ __align__(256) float scratch[kFuseBwdScratchBytes / sizeof(float)];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// Device address of this GPU's scratch array, for the device that runs
// `stream` (the current device for the null stream): looked up with that
// device current on the first call there, then kept.
srnl_status fuse_bwd_scratch(hipStream_t stream, float **out)
{
    int cur = 0, dev = 0;
    if (hipGetDevice(&cur) != hipSuccess) {
        (void)hipGetLastError();
        return fail(SRNL_ERR_HIP, "hipGetDevice failed");
    }
    dev = cur;
    if (stream && hipStreamGetDevice(stream, &dev) != hipSuccess) {
        (void)hipGetLastError();
        return fail(SRNL_ERR_HIP, "hipStreamGetDevice failed");
    }
    if (dev < 0 || dev >= kMaxDevices)
        return fail(SRNL_ERR_ARG, "device index out of range for the scratch table");
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        if (dev != cur && hipSetDevice(dev) != hipSuccess) {
            (void)hipGetLastError();
            return fail(SRNL_ERR_HIP, "hipSetDevice failed");
        }
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (dev != cur)
            (void)hipSetDevice(cur);
        if (e != hipSuccess || !p) {
            (void)hipGetLastError();
            return fail(SRNL_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") +
                                          hipGetErrorString(e));
        }
        g_scratch_ptr[dev] = p;
    }
    *out = static_cast<float *>(g_scratch_ptr[dev]);
    return SRNL_OK;
}

// params of srnl_scan_1d's scan: the 1 x N grid's row route, 64-token
// chunks unless chunk_row overrides them
srnl_params params_1d(const srnl_params *p)
{
    srnl_params q = *p;
    if (q.chunk_row == 0)
        q.chunk_row = 64;   // the 1-D default chunk
    q.chunk_col = 0;
    return q;
}

}  // namespace

// ------------------------------------------------------------ C ABI

extern "C" {

const char *srnl_status_string(srnl_status s)
{
    switch (s) {
    case SRNL_OK: return "ok";
    case SRNL_ERR_ARG: return "invalid argument";
    case SRNL_ERR_DTYPE: return "invalid dtype";
    case SRNL_ERR_PTR: return "invalid pointer";
    case SRNL_ERR_WORKSPACE: return "workspace too small";
    case SRNL_ERR_HIP: return "HIP error";
    case SRNL_ERR_NONFINITE: return "non-finite values";
    }
    return "unknown status";
}

const char *srnl_last_error(void) { return g_last_error.c_str(); }

void srnl_route_index(int r, int H, int W, long t, int *i, int *j)
{
    const long long N = static_cast<long long>(H) * W;
    const long long s = (r & 1) ? (N - 1 - t) : t;
    if (r < 2) {
        *i = static_cast<int>(s / W);
        *j = static_cast<int>(s % W);
    } else {
        *i = static_cast<int>(s % H);
        *j = static_cast<int>(s / H);
    }
}

int srnl_chunk_len(int r, int H, int W, int chunk_row, int chunk_col)
{
    if (r < 2)
        return chunk_row > 0 ? chunk_row : W;
    return chunk_col > 0 ? chunk_col : H;
}

srnl_status srnl_scan_fwd(const void *x, int B, int H, int W, int C, int heads, int d,
                          unsigned route_mask, const srnl_params *p, float *out)
{
    g_last_error.clear();
    if (!p)
        return fail(SRNL_ERR_PTR, "params is NULL");
    if (!valid_d(d))
        return fail(SRNL_ERR_ARG, "head dim must be 4, 8, 16, 32 or 64");
    if (heads < 1 || C != heads * d)
        return fail(SRNL_ERR_ARG, "C must equal heads * d with heads >= 1");
    long long n = 0;
    srnl_status s = check_grid(B, H, W, C, route_mask, &n);
    if (s != SRNL_OK)
        return s;
    if (!(p->alpha_max > 0.0f && p->alpha_max < 1.0f))
        return fail(SRNL_ERR_ARG, "alpha_max must lie in (0, 1)");
    if (!(p->eps > 0.0f) || !std::isfinite(p->eps))
        return fail(SRNL_ERR_ARG, "eps must be positive and finite");
    if (p->chunk_row < 0 || p->chunk_col < 0)
        return fail(SRNL_ERR_ARG, "chunk lengths must be >= 0");
    if (p->flags & ~0xFFu)
        return fail(SRNL_ERR_ARG, "unknown flag bits");
    if (p->in_dtype != SRNL_F32 && p->in_dtype != SRNL_BF16)
        return fail(SRNL_ERR_DTYPE, "in_dtype must be SRNL_F32 or SRNL_BF16");
    if (n == 0)
        return SRNL_OK;   // empty grid
    const long long rec = record_bytes(B, H, W, heads, d, route_mask, p);
    if (rec < 0)
        return fail(SRNL_ERR_ARG, "grid too large for SRNL_FLAG_RECORD");
    if (!is_device_ptr(x) || !is_device_ptr(out) || !is_device_ptr(p->states))
        return fail(SRNL_ERR_PTR, "x, out and states must be device memory");
    if (p->q && !is_device_ptr(p->q))
        return fail(SRNL_ERR_PTR, "q must be device memory");
    if (!aligned16(x) || !aligned16(out) || !aligned16(p->states) || (p->q && !aligned16(p->q)))
        return fail(SRNL_ERR_PTR, "x, q, out and states must be 16-byte aligned");
    const bool check = (p->flags & F_CHECK_FINITE) != 0;
    // workspace: the forward record (SRNL_FLAG_RECORD), then the counters
    const size_t need = static_cast<size_t>(rec) + (check ? kScanCheckBytes : 0);
    unsigned *counters = nullptr;
    if (need > 0) {
        if (!p->workspace || p->workspace_bytes < need)
            return fail(SRNL_ERR_WORKSPACE, "params->workspace smaller than srnl_scan_workspace_bytes");
        if (!is_device_ptr(p->workspace) || !aligned16(p->workspace))
            return fail(SRNL_ERR_PTR, "params->workspace must be 16-byte aligned device memory");
        if (check)
            counters = reinterpret_cast<unsigned *>(static_cast<char *>(p->workspace) + rec);
    }
    hipStream_t st = static_cast<hipStream_t>(p->stream);
    const long long nx = static_cast<long long>(B) * H * W * C;
    if (check) {
        hipLaunchKernelGGL(zero_counters_kernel, dim3(1), dim3(64), 0, st, counters);
        if (p->in_dtype == SRNL_F32) {
            hipLaunchKernelGGL(nonfinite_kernel<float>, dim3(grid_for(nx, 256)), dim3(256), 0, st,
                               static_cast<const float *>(x), nx, counters);
            if (p->q)
                hipLaunchKernelGGL(nonfinite_kernel<float>, dim3(grid_for(nx, 256)), dim3(256), 0, st,
                                   static_cast<const float *>(p->q), nx, counters);
        } else {
            hipLaunchKernelGGL(nonfinite_kernel<uint16_t>, dim3(grid_for(nx, 256)), dim3(256), 0, st,
                               static_cast<const uint16_t *>(x), nx, counters);
            if (p->q)
                hipLaunchKernelGGL(nonfinite_kernel<uint16_t>, dim3(grid_for(nx, 256)), dim3(256), 0,
                                   st, static_cast<const uint16_t *>(p->q), nx, counters);
        }
        s = launch_check("nonfinite_kernel (inputs)");
        if (s != SRNL_OK)
            return s;
    }
    if (rec > 0) {
        const FwdSave sv{static_cast<float *>(p->workspace), record_chain_floats(d, H, W, route_mask, p)};
        if (d == 64)
            s = (p->in_dtype == SRNL_F32)
                    ? launch_record_fwd<64, float>(x, p, B, H, W, C, heads, route_mask, out, sv)
                    : launch_record_fwd<64, uint16_t>(x, p, B, H, W, C, heads, route_mask, out, sv);
        else
            s = (p->in_dtype == SRNL_F32)
                    ? launch_record_fwd<32, float>(x, p, B, H, W, C, heads, route_mask, out, sv)
                    : launch_record_fwd<32, uint16_t>(x, p, B, H, W, C, heads, route_mask, out, sv);
    } else {
        s = (p->in_dtype == SRNL_F32)
                ? dispatch_scan<float>(d, x, p, B, H, W, C, heads, route_mask, out)
                : dispatch_scan<uint16_t>(d, x, p, B, H, W, C, heads, route_mask, out);
    }
    if (s != SRNL_OK || !check)
        return s;
    hipLaunchKernelGGL(nonfinite_kernel<float>, dim3(grid_for(n, 256)), dim3(256), 0, st, out, n,
                       counters + 1);
    s = launch_check("nonfinite_kernel (outputs)");
    if (s != SRNL_OK)
        return s;
    unsigned host[2] = {0u, 0u};
    if (hipMemcpyAsync(host, counters, sizeof(host), hipMemcpyDeviceToHost, st) != hipSuccess ||
        hipStreamSynchronize(st) != hipSuccess)
        return fail(SRNL_ERR_HIP, std::string("reading the finite-check counters: ") +
                                      hipGetErrorString(hipGetLastError()));
    if (host[0] || host[1])
        return fail(SRNL_ERR_NONFINITE, std::to_string(host[0]) + " non-finite input values, " +
                                            std::to_string(host[1]) + " non-finite outputs");
    return SRNL_OK;
}

size_t srnl_scan_workspace_bytes(int B, int H, int W, int C, int heads, int d,
                                 unsigned route_mask, const srnl_params *p)
{
    long long n = 0;
    if (!p || !valid_d(d) || heads < 1 || C != heads * d ||
        check_grid(B, H, W, C, route_mask, &n) != SRNL_OK || n == 0)
        return 0;
    const long long rec = record_bytes(B, H, W, heads, d, route_mask, p);
    if (rec < 0)
        return 0;
    return static_cast<size_t>(rec) + ((p->flags & F_CHECK_FINITE) ? kScanCheckBytes : 0);
}

srnl_status srnl_scan_1d(const void *x, int B, int N, int C, int heads, int d,
                         const srnl_params *p, float *out)
{
    g_last_error.clear();
    if (!p)
        return fail(SRNL_ERR_PTR, "params is NULL");
    const srnl_params q = params_1d(p);
    return srnl_scan_fwd(x, B, 1, N, C, heads, d, SRNL_ROUTE_ROW, &q, out);
}

srnl_status srnl_fuse(const float *y, int B, int H, int W, int C, unsigned route_mask,
                      const float *scales, srnl_dtype out_dtype, void *out, void *stream)
{
    g_last_error.clear();
    long long n = 0;
    srnl_status s = check_grid(B, H, W, C, route_mask, &n);
    if (s != SRNL_OK)
        return s;
    if (out_dtype != SRNL_F32 && out_dtype != SRNL_BF16)
        return fail(SRNL_ERR_DTYPE, "out_dtype must be SRNL_F32 or SRNL_BF16");
    if (n == 0)
        return SRNL_OK;
    if (!is_device_ptr(y) || !is_device_ptr(scales) || !is_device_ptr(out))
        return fail(SRNL_ERR_PTR, "y_routes, scales and out must be device memory");
    if (!aligned16(y) || !aligned16(scales) || !aligned16(out))
        return fail(SRNL_ERR_PTR, "y_routes, scales and out must be 16-byte aligned");
    const PlaneShape ps = plane_shape(C / 4);
    const dim3 grid((H * W + ps.ty - 1) / ps.ty, B < 65535 ? B : 65535), block(ps.cv, ps.ty);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (out_dtype == SRNL_F32)
        hipLaunchKernelGGL(fuse_kernel<float>, grid, block, 0, st, y, scales,
                           static_cast<float *>(out), B, H, W, C, route_mask);
    else
        hipLaunchKernelGGL(fuse_kernel<uint16_t>, grid, block, 0, st, y, scales,
                           static_cast<uint16_t *>(out), B, H, W, C, route_mask);
    return launch_check("fuse_kernel");
}

size_t srnl_scan_bwd_workspace_bytes(int B, int H, int W, int C, int heads, int d,
                                     unsigned route_mask, const srnl_params *p)
{
    long long n = 0;
    if (check_scan_args(B, H, W, C, heads, d, route_mask, p, &n) != SRNL_OK || n == 0)
        return 0;
    const long long t = bwd_layout(B, H, W, C, heads, d, route_mask, p).total;
    return t < 0 ? 0 : static_cast<size_t>(t) * sizeof(float);
}

}   // extern "C"

namespace {
// srnl_scan_bwd, with the state gradients written for route slots
// 0 .. nr_out - 1 (4 for the 2-D operator, 1 for the 1-D one). With ysc
// (the windowed d = 32 adjoint only), dy is the fused output's gradient
// [B][H][W][C] and each route's dy is formed from it with the scales ysc;
// ft (with ysc): the fusion backward's partial sums and scales' gradient
// run after the adjoint.
srnl_status scan_bwd_impl(const void *x, int B, int H, int W, int C, int heads, int d,
                          unsigned route_mask, const srnl_params *p, const float *dy,
                          void *workspace, size_t workspace_bytes, float *dx, float *dq,
                          float *dstates, int nr_out, const float *ysc = nullptr,
                          const FuseTail *ft = nullptr)
{
    long long n = 0;
    srnl_status s = check_scan_args(B, H, W, C, heads, d, route_mask, p, &n);
    if (s != SRNL_OK)
        return s;
    if (n == 0)
        return SRNL_OK;   // empty grid
    const BwdLayout l = bwd_layout(B, H, W, C, heads, d, route_mask, p);
    if (l.total < 0)
        return fail(SRNL_ERR_ARG, "grid too large for srnl_scan_bwd's workspace");
    if (!workspace || workspace_bytes < static_cast<size_t>(l.total) * sizeof(float))
        return fail(SRNL_ERR_WORKSPACE, "workspace smaller than srnl_scan_bwd_workspace_bytes");
    if (!is_device_ptr(x) || !is_device_ptr(p->states) || !is_device_ptr(dy) ||
        !is_device_ptr(dx) || !is_device_ptr(dstates) || !is_device_ptr(workspace))
        return fail(SRNL_ERR_PTR, "x, states, dy, dx, dstates and workspace must be device memory");
    if (p->q && (!is_device_ptr(p->q) || !is_device_ptr(dq)))
        return fail(SRNL_ERR_PTR, "with separate queries, q and dq must be device memory");
    if (!aligned16(x) || !aligned16(p->states) || !aligned16(dy) || !aligned16(dx) ||
        !aligned16(dstates) || !aligned16(workspace) || (p->q && (!aligned16(p->q) || !aligned16(dq))))
        return fail(SRNL_ERR_PTR, "x, q, states, dy, dx, dq, dstates and workspace must be 16-byte aligned");
    if (l.chains > INT_MAX)
        return fail(SRNL_ERR_ARG, "too many chains (routes * B * heads)");
    if (l.record_given) {
        const long long rec = record_bytes(B, H, W, heads, d, route_mask, p);
        if (rec < 0)
            return fail(SRNL_ERR_ARG, "grid too large for SRNL_FLAG_RECORD");
        if (!p->workspace || p->workspace_bytes < static_cast<size_t>(rec))
            return fail(SRNL_ERR_WORKSPACE, "SRNL_FLAG_RECORD: params->workspace must hold the forward record");
        if (!is_device_ptr(p->workspace) || !aligned16(p->workspace))
            return fail(SRNL_ERR_PTR, "params->workspace must be 16-byte aligned device memory");
    }
    float *ws = static_cast<float *>(workspace);
    if (p->in_dtype == SRNL_F32)
        return dispatch_scan_bwd<float>(d, x, p, B, H, W, C, heads, route_mask, dy, ws, l, dx, dq,
                                        dstates, nr_out, ysc, ft);
    return dispatch_scan_bwd<uint16_t>(d, x, p, B, H, W, C, heads, route_mask, dy, ws, l, dx, dq,
                                       dstates, nr_out, ysc, ft);
}

}   // namespace

extern "C" {

srnl_status srnl_scan_bwd(const void *x, int B, int H, int W, int C, int heads, int d,
                          unsigned route_mask, const srnl_params *p, const float *dy,
                          void *workspace, size_t workspace_bytes, float *dx, float *dq,
                          float *dstates)
{
    g_last_error.clear();
    return scan_bwd_impl(x, B, H, W, C, heads, d, route_mask, p, dy, workspace, workspace_bytes,
                         dx, dq, dstates, 4);
}

size_t srnl_scan_1d_workspace_bytes(int B, int N, int C, int heads, int d, const srnl_params *p)
{
    if (!p)
        return 0;
    const srnl_params q = params_1d(p);
    return srnl_scan_workspace_bytes(B, 1, N, C, heads, d, SRNL_ROUTE_ROW, &q);
}

size_t srnl_scan_1d_bwd_workspace_bytes(int B, int N, int C, int heads, int d,
                                        const srnl_params *p)
{
    if (!p)
        return 0;
    const srnl_params q = params_1d(p);
    return srnl_scan_bwd_workspace_bytes(B, 1, N, C, heads, d, SRNL_ROUTE_ROW, &q);
}

srnl_status srnl_scan_1d_bwd(const void *x, int B, int N, int C, int heads, int d,
                             const srnl_params *p, const float *dy, void *workspace,
                             size_t workspace_bytes, float *dx, float *dq, float *dstates)
{
    g_last_error.clear();
    if (!p)
        return fail(SRNL_ERR_PTR, "params is NULL");
    const srnl_params q = params_1d(p);
    return scan_bwd_impl(x, B, 1, N, C, heads, d, SRNL_ROUTE_ROW, &q, dy, workspace,
                         workspace_bytes, dx, dq, dstates, 1);
}

size_t srnl_fuse_bwd_workspace_bytes(int B, int H, int W, int C, unsigned route_mask)
{
    long long n = 0;
    if (check_grid(B, H, W, C, route_mask, &n) != SRNL_OK || n == 0)
        return 0;
    return static_cast<size_t>(popcount4(route_mask) * fuse_bwd_blocks(B, H, W) * C) * sizeof(float);
}

}   // extern "C"

namespace {
// srnl_fuse_bwd with its partial sums in `workspace`, or (noalloc) in the
// library's scratch array of this GPU
// (check_only: the checks alone, no launch, and dyr may be NULL, for the
// one-call backward whose adjoint forms the route gradients itself)
srnl_status fuse_bwd_impl(const float *dout, const float *y, int B, int H, int W, int C,
                          unsigned route_mask, const float *scales, float *dyr, float *dscales,
                          void *workspace, size_t workspace_bytes, void *stream, bool noalloc,
                          bool check_only = false)
{
    long long n = 0;
    srnl_status s = check_grid(B, H, W, C, route_mask, &n);
    if (s != SRNL_OK)
        return s;
    if (C > 1024)
        return fail(SRNL_ERR_ARG, "srnl_fuse_bwd supports C <= 1024");
    if (n == 0)
        return SRNL_OK;
    const int R = popcount4(route_mask);
    const long long nblk = fuse_bwd_blocks(B, H, W);
    const size_t need = static_cast<size_t>(R * nblk * C) * sizeof(float);
    if (noalloc) {
        if (need > kFuseBwdScratchBytes)
            return fail(SRNL_ERR_WORKSPACE,
                        "srnl_fuse_bwd_noalloc: the partial sums need " + std::to_string(need) +
                        " bytes, more than the library's scratch of " +
                        std::to_string(kFuseBwdScratchBytes) + " bytes (use srnl_fuse_bwd)");
    } else if (!workspace || workspace_bytes < need) {
        return fail(SRNL_ERR_WORKSPACE, "workspace smaller than srnl_fuse_bwd_workspace_bytes");
    }
    if (nblk > 65535LL * 16)
        return fail(SRNL_ERR_ARG, "grid too large for srnl_fuse_bwd");
    const bool skip_dyr = check_only && dyr == nullptr;
    if (!is_device_ptr(dout) || !is_device_ptr(y) || !is_device_ptr(scales) ||
        (!skip_dyr && !is_device_ptr(dyr)) || !is_device_ptr(dscales) ||
        (!noalloc && !is_device_ptr(workspace)))
        return fail(SRNL_ERR_PTR, "dout, y_routes, scales, dy_routes, dscales and workspace must be device memory");
    if (!aligned16(dout) || !aligned16(y) || !aligned16(scales) || (!skip_dyr && !aligned16(dyr)) ||
        !aligned16(dscales) || (!noalloc && !aligned16(workspace)))
        return fail(SRNL_ERR_PTR, "dout, y_routes, scales, dy_routes, dscales and workspace must be 16-byte aligned");
    if (check_only)
        return SRNL_OK;
    hipStream_t st = static_cast<hipStream_t>(stream);
    float *part = static_cast<float *>(workspace);
    if (noalloc) {
        s = fuse_bwd_scratch(st, &part);
        if (s != SRNL_OK)
            return s;
    }
    hipLaunchKernelGGL(fuse_bwd_kernel, dim3(static_cast<unsigned>(nblk)), dim3(256), 0, st, dout, y,
                       scales, dyr, part, B, H, W, C, route_mask, kFuseBwdRows);
    s = launch_check("fuse_bwd_kernel");
    if (s != SRNL_OK)
        return s;
    hipLaunchKernelGGL(fuse_bwd_scales_kernel, dim3(grid_for(4LL * C * 64, 256)), dim3(256), 0, st, part,
                       dscales, C, route_mask, static_cast<int>(nblk));
    return launch_check("fuse_bwd_scales_kernel");
}
}   // namespace

extern "C" {

srnl_status srnl_fuse_bwd(const float *dout, const float *y, int B, int H, int W, int C,
                          unsigned route_mask, const float *scales, float *dyr, float *dscales,
                          void *workspace, size_t workspace_bytes, void *stream)
{
    g_last_error.clear();
    return fuse_bwd_impl(dout, y, B, H, W, C, route_mask, scales, dyr, dscales, workspace,
                         workspace_bytes, stream, false);
}

srnl_status srnl_fuse_bwd_noalloc(const float *dout, const float *y, int B, int H, int W, int C,
                                  unsigned route_mask, const float *scales, float *dyr,
                                  float *dscales, void *stream)
{
    g_last_error.clear();
    return fuse_bwd_impl(dout, y, B, H, W, C, route_mask, scales, dyr, dscales, nullptr, 0,
                         stream, true);
}

}   // extern "C"

namespace {
// Workspace of srnl_scan_fuse_bwd in floats: the scan backward's, the fusion
// backward's partial sums, and (where the adjoint cannot form each route's
// dy itself) the route gradients; -1 if too large or invalid.
struct OpBwdLayout {
    bool direct = false;     // windowed d = 32 adjoint reads dout and the scales
    long long scan = 0, part = 0, dyr = 0, total = -1;
};

long long round64(long long v) { return (v + 63) / 64 * 64; }

OpBwdLayout op_bwd_layout(int B, int H, int W, int C, int heads, int d, unsigned mask,
                          const srnl_params *p)
{
    OpBwdLayout o;
    const BwdLayout l = bwd_layout(B, H, W, C, heads, d, mask, p);
    if (l.total < 0)
        return o;
    o.direct = d == 32 && bwd_windowed(d, p, H, W, mask);
    o.scan = round64(l.total);
    o.part = round64(static_cast<long long>(popcount4(mask)) * fuse_bwd_blocks(B, H, W) * C);
    o.dyr = o.direct ? 0 : round64(static_cast<long long>(popcount4(mask)) * B * H * W * C);
    o.total = o.scan + o.part + o.dyr;
    return o;
}
}   // namespace

extern "C" {

size_t srnl_scan_fuse_bwd_workspace_bytes(int B, int H, int W, int C, int heads, int d,
                                          unsigned route_mask, const srnl_params *p)
{
    long long n = 0;
    if (check_scan_args(B, H, W, C, heads, d, route_mask, p, &n) != SRNL_OK || n == 0 || C > 1024)
        return 0;
    const OpBwdLayout o = op_bwd_layout(B, H, W, C, heads, d, route_mask, p);
    return o.total < 0 ? 0 : static_cast<size_t>(o.total) * sizeof(float);
}

srnl_status srnl_scan_fuse_bwd(const void *x, int B, int H, int W, int C, int heads, int d,
                               unsigned route_mask, const srnl_params *p, const float *y_routes,
                               const float *scales, const float *dout, void *workspace,
                               size_t workspace_bytes, float *dx, float *dq, float *dstates,
                               float *dscales)
{
    g_last_error.clear();
    long long n = 0;
    srnl_status s = check_scan_args(B, H, W, C, heads, d, route_mask, p, &n);
    if (s != SRNL_OK)
        return s;
    if (n == 0)
        return SRNL_OK;   // empty grid
    if (C > 1024)
        return fail(SRNL_ERR_ARG, "srnl_scan_fuse_bwd supports C <= 1024");
    const OpBwdLayout o = op_bwd_layout(B, H, W, C, heads, d, route_mask, p);
    if (o.total < 0)
        return fail(SRNL_ERR_ARG, "grid too large for srnl_scan_fuse_bwd's workspace");
    if (!workspace || workspace_bytes < static_cast<size_t>(o.total) * sizeof(float))
        return fail(SRNL_ERR_WORKSPACE, "workspace smaller than srnl_scan_fuse_bwd_workspace_bytes");
    float *ws = static_cast<float *>(workspace);
    float *part = ws + o.scan, *dyr = o.direct ? nullptr : part + o.part;
    // direct: the checks here, the fusion backward's kernels after the adjoint
    s = fuse_bwd_impl(dout, y_routes, B, H, W, C, route_mask, scales, dyr, dscales, part,
                      static_cast<size_t>(o.part) * sizeof(float), p->stream, false, o.direct);
    if (s != SRNL_OK)
        return s;
    if (o.direct) {
        const FuseTail ft{dout, y_routes, scales, part, dscales, kFuseBwdRows, fuse_bwd_blocks(B, H, W)};
        return scan_bwd_impl(x, B, H, W, C, heads, d, route_mask, p, dout, ws,
                             static_cast<size_t>(o.scan) * sizeof(float), dx, dq, dstates, 4, scales,
                             &ft);
    }
    return scan_bwd_impl(x, B, H, W, C, heads, d, route_mask, p, dyr, ws,
                         static_cast<size_t>(o.scan) * sizeof(float), dx, dq, dstates, 4);
}

size_t srnl_block_workspace_bytes(int B, int H, int W, int C, unsigned route_mask)
{
    long long n = 0;
    if (check_grid(B, H, W, C, route_mask, &n) != SRNL_OK || n == 0)
        return 0;
    return static_cast<size_t>(block_layout(B, H, W, C, route_mask).total) * sizeof(float);
}

srnl_status srnl_block_fwd(const void *x, int B, int H, int W, int C, int heads, int d,
                           unsigned route_mask, const srnl_params *p,
                           const srnl_block_weights *w, void *workspace, size_t workspace_bytes,
                           void *out)
{
    g_last_error.clear();
    long long n = 0;
    srnl_status s = check_scan_args(B, H, W, C, heads, d, route_mask, p, &n);
    if (s != SRNL_OK)
        return s;
    if (!w)
        return fail(SRNL_ERR_PTR, "block weights are NULL");
    if (p->q)
        return fail(SRNL_ERR_ARG, "the block forms its own queries: params->q must be NULL");
    if (C != 32 && C != 64 && C != 128 && C != 192 && C != 256 && C != 512)
        return fail(SRNL_ERR_ARG, "block channels must be 32, 64, 128, 192, 256 or 512");
    if (w->ffn_hidden < 32 || w->ffn_hidden % 32 != 0 || w->ffn_hidden > (1 << 16))
        return fail(SRNL_ERR_ARG, "ffn_hidden must be a positive multiple of 32, at most 65536");
    if (!(w->ln_eps > 0.0f) || !std::isfinite(w->ln_eps))
        return fail(SRNL_ERR_ARG, "ln_eps must be positive and finite");
    if (n == 0)
        return SRNL_OK;
    const BlockLayout l = block_layout(B, H, W, C, route_mask);
    if (!workspace || workspace_bytes < static_cast<size_t>(l.total) * sizeof(float))
        return fail(SRNL_ERR_WORKSPACE, "workspace smaller than srnl_block_workspace_bytes");
    const void *ptrs[] = {x, out, workspace, p->states, w->ln1_w, w->ln1_b, w->wq, w->dw_w,
                          w->dw_b, w->ln2_w, w->ln2_b, w->w1, w->b1, w->w2, w->b2, w->scales};
    for (const void *q : ptrs)
        if (!is_device_ptr(q))
            return fail(SRNL_ERR_PTR, "x, out, workspace, states and every block weight must be device memory");
    for (const void *q : ptrs)
        if (!aligned16(q))
            return fail(SRNL_ERR_PTR, "x, out, workspace, states and every block weight must be 16-byte aligned");
    const long long ntok = static_cast<long long>(B) * H * W;
    float *u = static_cast<float *>(workspace), *q = u + l.o_q, *sf = u + l.o_s, *y = u + l.o_y,
          *hb = u + l.o_h;
    hipStream_t st = static_cast<hipStream_t>(p->stream);
    const bool bf = p->in_dtype == SRNL_BF16;
    s = bf ? dispatch_block_kernels<uint16_t>(C, x, ntok, H, W, w, u, q, nullptr, hb, nullptr, st, true)
           : dispatch_block_kernels<float>(C, x, ntok, H, W, w, u, q, nullptr, hb, nullptr, st, true);
    if (s != SRNL_OK)
        return s;
    srnl_params ps = *p;   // the operator reads u (fp32) with queries q
    ps.q = q;
    ps.in_dtype = SRNL_F32;
    s = dispatch_scan<float>(d, u, &ps, B, H, W, C, heads, route_mask, y);
    if (s != SRNL_OK)
        return s;
    s = srnl_fuse(y, B, H, W, C, route_mask, w->scales, SRNL_F32, sf, p->stream);
    if (s != SRNL_OK)
        return s;
    return bf ? dispatch_block_kernels<uint16_t>(C, x, ntok, H, W, w, u, q, sf, hb, out, st, false)
              : dispatch_block_kernels<float>(C, x, ntok, H, W, w, u, q, sf, hb, out, st, false);
}

srnl_status srnl_route_gather(const void *x, int B, int H, int W, int C, unsigned route_mask,
                              srnl_dtype dtype, void *out, void *stream)
{
    g_last_error.clear();
    long long n = 0;
    srnl_status s = check_grid(B, H, W, C, route_mask, &n);
    if (s != SRNL_OK)
        return s;
    if (dtype != SRNL_F32 && dtype != SRNL_BF16)
        return fail(SRNL_ERR_DTYPE, "dtype must be SRNL_F32 or SRNL_BF16");
    if (n == 0)
        return SRNL_OK;
    if (!is_device_ptr(x) || !is_device_ptr(out))
        return fail(SRNL_ERR_PTR, "x and out must be device memory");
    const int row_bytes = C * (dtype == SRNL_F32 ? 4 : 2);
    const uintptr_t align = reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(out) |
                            static_cast<uintptr_t>(row_bytes);
    const int vb = (align % 16 == 0) ? 16 : (align % 8 == 0) ? 8 : (align % 4 == 0) ? 4 : 2;
    const PlaneShape ps = plane_shape(row_bytes / vb);
    const dim3 grid((H * W + ps.ty - 1) / ps.ty, B < 65535 ? B : 65535), block(ps.cv, ps.ty);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const char *xs = static_cast<const char *>(x);
    char *os = static_cast<char *>(out);
    if (vb == 16)
        hipLaunchKernelGGL(gather_kernel<uint4>, grid, block, 0, st, xs, os, B, H, W, row_bytes,
                           route_mask);
    else if (vb == 8)
        hipLaunchKernelGGL(gather_kernel<uint2>, grid, block, 0, st, xs, os, B, H, W, row_bytes,
                           route_mask);
    else if (vb == 4)
        hipLaunchKernelGGL(gather_kernel<uint32_t>, grid, block, 0, st, xs, os, B, H, W,
                           row_bytes, route_mask);
    else
        hipLaunchKernelGGL(gather_kernel<uint16_t>, grid, block, 0, st, xs, os, B, H, W,
                           row_bytes, route_mask);
    return launch_check("gather_kernel");
}

srnl_status srnl_init_states(float *states, int heads, int d, unsigned long long seed,
                             float stdv, void *stream)
{
    g_last_error.clear();
    if (heads < 1 || !valid_d(d))
        return fail(SRNL_ERR_ARG, "heads must be >= 1 and d one of 4, 8, 16, 32, 64");
    if (!(stdv >= 0.0f) || !std::isfinite(stdv))
        return fail(SRNL_ERR_ARG, "std must be finite and >= 0");
    if (!is_device_ptr(states))
        return fail(SRNL_ERR_PTR, "states must be device memory");
    const long long n = 4LL * heads * SRNL_STATE_FLOATS(static_cast<long long>(d));
    const int grid = grid_for((n + 3) / 4, 256);
    hipLaunchKernelGGL(init_kernel, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                       states, n, seed, stdv);
    return launch_check("init_kernel");
}

}  // extern "C"

#if SRNL_PHASE_CLOCKS
// Phase-clock build only: the first n counters of srnl_phase_buf
// (kPhaseSlots per block of the last instrumented launch) into host memory.
// Returns a hipError_t.
extern "C" int srnl_phase_clocks(unsigned long long *host, size_t n)
{
    return static_cast<int>(hipMemcpyFromSymbol(host, HIP_SYMBOL(srnl_phase_buf),
                                                n * sizeof(unsigned long long)));
}
#endif
