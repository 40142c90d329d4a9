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
#include <string>

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

__device__ __forceinline__ float sigmoidf(float z) { return 1.0f / (1.0f + expf(-z)); }

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
    F_READ_BEFORE = 0x10u
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
                                        : m * tanhf(uu) / g;
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
            float acc[NREF];
#pragma unroll
            for (int k = 0; k < NREF; ++k) {
                const int idx = tid + k * NT;
                float a = 0.0f;
                if (idx < ROWS * D) {
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
                if (idx < ROWS * D)
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
// One workgroup of 4d threads per chain; T tokens per sub-block (a chunk is
// processed in sub-blocks of at most T tokens: generation inside a chunk
// reads only the fixed boundary states, so it may be split).
//
//   load      tokens of the next sub-block are prefetched into registers
//             (16-byte loads along the route) while the current one computes
//   generate  [k | v] = X B_[k|v]^T on MFMA (v_mfma_f32_16x16x4f32)
//   epilogue  4 lanes per token: |k|^2, b_eta . x, b_alpha . x, k^, e, the
//             soft cap and the spectral clamp (quad DPP reductions)
//   update    4 lanes per row of Q = cq * P, d/4 columns per lane; the
//             retention factors accumulate in the scalar cq so the write is
//             one FMA per element: P <- P - (eta''/cq') (cq P k^ + e) k^T
//   readout   Y = Z B_c^T on MFMA, z_t = Q_t q_t
//   refresh   B <- B Q_L on MFMA (the two vector memories on VALU)
//
// MFMA 16x16x4 f32 operand layout (lane l): A[l%16][l/16], B[l/16][l%16],
// D[4(l/16)+r][l%16] in accumulator register r. Every operand is read from
// an LDS array stored [m or n][k] with row stride d+2, which puts the 64
// lanes of one read on distinct banks.

typedef float v4f __attribute__((ext_vector_type(4)));

template <int D, int T> struct MCfg {
    static constexpr int NT = 4 * D;               // threads: 4 lanes per row of Q
    static constexpr int NW = NT / 64;             // waves
    static constexpr int ROWS = 3 * D + 2;
    static constexpr int LDP = D + 2;              // operand row stride
    static constexpr int CPL = D / 4;              // Q columns per lane
    static constexpr int KS = D / 4;               // MFMA K-steps over d
    static constexpr int RT = (3 * D / 16) * (D / 16);  // refresh tiles (matrix rows)
    static constexpr int RTW = RT / NW;            // refresh tiles per wave
    static_assert(RT % NW == 0, "refresh tiles must split evenly over waves");
    static_assert(T % 16 == 0, "T must be a multiple of 16");
};

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

constexpr float kTinyScale = 8.673617379884035e-19f;   // 2^-60

template <int D, int T, typename InT>
__global__ __launch_bounds__(4 * D) void scan_mfma_kernel(
    const InT *__restrict__ x, const InT *__restrict__ q,
    const float *__restrict__ states, float *__restrict__ out, int B, int H,
    int W, int C, int heads, unsigned route_mask, int R, float alpha_max,
    float eps, int chunk_row, int chunk_col, unsigned flags, int nchains)
{
    using Cfg = MCfg<D, T>;
    constexpr int NT = Cfg::NT, NW = Cfg::NW, ROWS = Cfg::ROWS, LDP = Cfg::LDP,
                  CPL = Cfg::CPL, KS = Cfg::KS, RTW = Cfg::RTW;
    constexpr int VE = InVec<InT>::VE;
    constexpr int SEGS = D / VE;                       // 16-byte segments per token
    constexpr int NPF = (T * SEGS + NT - 1) / NT;      // prefetch registers per thread

    __shared__ __align__(16) float Bs[ROWS * LDP];     // boundary rows M_c, M_k, M_v, m_eta, m_alpha
    __shared__ __align__(16) float Xs[T * LDP];        // x_t (MFMA operand)
    __shared__ __align__(16) float QVa[T * D];         // q_t (token loop)
    __shared__ __align__(16) float KZ[T * LDP];        // k (generation), then z_t (readout)
    __shared__ __align__(16) float Es[T * LDP];        // v, then e = k^ - v
    __shared__ __align__(16) float KHa[T * D];         // k^ (token loop)
    __shared__ __align__(16) float2 Sae[T];            // (alpha_t, eta''_t)
    __shared__ __align__(16) float Qt[D * LDP];        // Q_L^T at the chunk end

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
    const int lane = tid & 63, wave = tid >> 6;
    const int lm = lane & 15, lk = lane >> 4;        // MFMA operand row / k slot
    const int row = tid >> 2, part = tid & 3;         // token-loop row of Q and column part

    const float *st = states + (static_cast<size_t>(r) * heads + h) * (ROWS * D);
    for (int idx = tid; idx < ROWS * D; idx += NT)
        Bs[(idx / D) * LDP + idx % D] = st[idx];

    const size_t xbase = static_cast<size_t>(b) * H * W * C + static_cast<size_t>(h) * D;
    uint4 pre[NPF], preq[NPF];
    auto issue_loads = [&](long long s, int n) {
#pragma unroll
        for (int k = 0; k < NPF; ++k) {
            const int seg = tid + k * NT;
            if (seg < n * SEGS) {
                const int u = seg / SEGS, sg = seg % SEGS;
                int i, j;
                route_cell(r, H, W, N, s + u, i, j);
                const size_t off = xbase + (static_cast<size_t>(i) * W + j) * C + sg * VE;
                pre[k] = *reinterpret_cast<const uint4 *>(x + off);
                if (q)
                    preq[k] = *reinterpret_cast<const uint4 *>(q + off);
            }
        }
    };

    float P[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c)
        P[c] = (part * CPL + c == row) ? 1.0f : 0.0f;
    float cq = 1.0f;

    const size_t out_base = static_cast<size_t>(slot) * B + b;
    const bool before = (flags & F_READ_BEFORE) != 0;

    long long c0 = 0;
    long long cend = (L < N) ? L : N;
    long long s0 = 0;
    int nt = static_cast<int>((T < cend) ? T : cend);
    issue_loads(s0, nt);

    while (true) {
        __syncthreads();   // previous sub-block is done with Xs, QVa, KZ; Bs is current

        // (1) store the prefetched tokens; zero the padding rows
#pragma unroll
        for (int k = 0; k < NPF; ++k) {
            const int seg = tid + k * NT;
            if (seg < T * SEGS) {
                const int u = seg / SEGS, sg = seg % SEGS;
                float f[VE], fq[VE];
                if (seg < nt * SEGS) {
                    unpack(pre[k], f, static_cast<const InT *>(nullptr));
                    if (q)
                        unpack(preq[k], fq, static_cast<const InT *>(nullptr));
                } else {
#pragma unroll
                    for (int e = 0; e < VE; ++e)
                        f[e] = fq[e] = 0.0f;
                }
#pragma unroll
                for (int e = 0; e < VE; ++e) {
                    Xs[u * LDP + sg * VE + e] = f[e];
                    QVa[u * D + sg * VE + e] = q ? fq[e] : f[e];
                }
            }
        }
        // position of the next sub-block; prefetch it
        const long long s1 = s0 + nt;
        const bool chunk_end = (s1 == cend);
        long long c1 = c0, cend1 = cend;
        if (chunk_end) {
            c1 = cend;
            cend1 = (c1 + L < N) ? c1 + L : N;
        }
        const int nt1 = (s1 < N) ? static_cast<int>((T < cend1 - s1) ? T : cend1 - s1) : 0;
        if (nt1 > 0)
            issue_loads(s1, nt1);
        __syncthreads();

        const int ntm = (nt + 15) >> 4;   // token tiles

        // (2) boundary generation on MFMA: [k | v] = X [B_k; B_v]^T
        {
            constexpr int NTN = 2 * D / 16;
            for (int tile = wave; tile < ntm * NTN; tile += NW) {
                const int tm = tile / NTN, tn = tile % NTN;
                const float *pa = Xs + (tm * 16 + lm) * LDP + lk;
                const float *pb = Bs + (D + tn * 16 + lm) * LDP + lk;
                v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < KS; ++s)
                    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(pa[4 * s], pb[4 * s], acc, 0, 0, 0);
                float *dst = (tn * 16 < D) ? KZ : Es;
                const int oc = (tn * 16) % D + lm;
#pragma unroll
                for (int rr = 0; rr < 4; ++rr)
                    dst[(tm * 16 + 4 * lk + rr) * LDP + oc] = acc[rr];
            }
        }
        __syncthreads();

        // (3) transition scalars, 4 lanes per token [SUMMARY stabilisation]
        {
            const int eu = tid >> 2, ep = tid & 3;
            for (int ub = 0; ub < nt; ub += NT / 4) {
                const int u = ub + eu;
                if (u < nt) {
                    float kk[CPL], vv[CPL];
                    float nk2 = 0.f, er = 0.f, ar = 0.f;
#pragma unroll
                    for (int c = 0; c < CPL; ++c) {
                        const int jj = ep * CPL + c;
                        kk[c] = KZ[u * LDP + jj];
                        vv[c] = Es[u * LDP + jj];
                        const float xv = Xs[u * LDP + jj];
                        nk2 = fmaf(kk[c], kk[c], nk2);
                        er = fmaf(Bs[3 * D * LDP + jj], xv, er);
                        ar = fmaf(Bs[(3 * D + 1) * LDP + jj], xv, ar);
                    }
                    nk2 = quad_sum(nk2);
                    er = quad_sum(er);
                    ar = quad_sum(ar);
                    const float inv = 1.0f / sqrtf(nk2 + eps);
                    float nkh2 = 0.f, ne2 = 0.f;
#pragma unroll
                    for (int c = 0; c < CPL; ++c) {
                        const int jj = ep * CPL + c;
                        const float kh = kk[c] * inv;
                        const float ev = kh - vv[c];
                        KHa[u * D + jj] = kh;
                        Es[u * LDP + jj] = ev;
                        nkh2 = fmaf(kh, kh, nkh2);
                        ne2 = fmaf(ev, ev, ne2);
                    }
                    nkh2 = quad_sum(nkh2);
                    ne2 = quad_sum(ne2);
                    const float eta = sigmoidf(er);
                    const float alpha = (flags & F_FIXED_ALPHA) ? alpha_max
                                                                : alpha_max * sigmoidf(ar);
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
                                            : m * tanhf(uu) / g;
                    }
                    float eta2 = eta1;
                    if (!(flags & F_NO_CLAMP) && nkh2 > 0.0f) {
                        const float cap = 2.0f * alpha / nkh2;
                        if (cap < eta2)
                            eta2 = cap;
                    }
                    if (ep == 0)
                        Sae[u] = make_float2(alpha, eta2);
                }
            }
        }
        __syncthreads();

        // (4) token-order update, Q = cq * P
        for (int u = 0; u < nt; ++u) {
            float kv[CPL], qv[CPL];
            const float4 *kp = reinterpret_cast<const float4 *>(KHa + u * D + part * CPL);
            const float4 *qp = reinterpret_cast<const float4 *>(QVa + u * D + part * CPL);
#pragma unroll
            for (int c4 = 0; c4 < CPL / 4; ++c4) {
                const float4 a = kp[c4], bq = qp[c4];
                kv[4 * c4] = a.x; kv[4 * c4 + 1] = a.y; kv[4 * c4 + 2] = a.z; kv[4 * c4 + 3] = a.w;
                qv[4 * c4] = bq.x; qv[4 * c4 + 1] = bq.y; qv[4 * c4 + 2] = bq.z; qv[4 * c4 + 3] = bq.w;
            }
            const float ee = Es[u * LDP + row];
            const float2 ae = Sae[u];
            float zb = 0.f;
            if (before) {
                float z0 = 0.f, z1 = 0.f;
#pragma unroll
                for (int c = 0; c < CPL; c += 2) {
                    z0 = fmaf(P[c], qv[c], z0);
                    z1 = fmaf(P[c + 1], qv[c + 1], z1);
                }
                zb = cq * quad_sum(z0 + z1);
            }
            float d0 = 0.f, d1 = 0.f;
#pragma unroll
            for (int c = 0; c < CPL; c += 2) {
                d0 = fmaf(P[c], kv[c], d0);
                d1 = fmaf(P[c + 1], kv[c + 1], d1);
            }
            const float sc = fmaf(cq, quad_sum(d0 + d1), ee);   // (Q k^ + e)_row
            const float cn = cq * ae.x;
            if (cn >= kTinyScale) {
                const float coef = ae.y / cn * sc;
#pragma unroll
                for (int c = 0; c < CPL; ++c)
                    P[c] = fmaf(-coef, kv[c], P[c]);
                cq = cn;
            } else {   // fold the scale back into P before it underflows
                const float s = ae.y * sc;
#pragma unroll
                for (int c = 0; c < CPL; ++c)
                    P[c] = fmaf(-s, kv[c], cn * P[c]);
                cq = 1.0f;
            }
            float z;
            if (before) {
                z = zb;
            } else {
                float z0 = 0.f, z1 = 0.f;
#pragma unroll
                for (int c = 0; c < CPL; c += 2) {
                    z0 = fmaf(P[c], qv[c], z0);
                    z1 = fmaf(P[c + 1], qv[c + 1], z1);
                }
                z = cq * quad_sum(z0 + z1);
            }
            if (part == 0)
                KZ[u * LDP + row] = z;
        }
        __syncthreads();

        // (5) readout on MFMA: y_t = B_c z_t
        {
            constexpr int NTN = D / 16;
            for (int tile = wave; tile < ntm * NTN; tile += NW) {
                const int tm = tile / NTN, tn = tile % NTN;
                const float *pa = KZ + (tm * 16 + lm) * LDP + lk;
                const float *pb = Bs + (tn * 16 + lm) * LDP + lk;
                v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < KS; ++s)
                    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(pa[4 * s], pb[4 * s], acc, 0, 0, 0);
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const int u = tm * 16 + 4 * lk + rr;
                    if (u < nt)
                        out[(out_base * N + s0 + u) * C + static_cast<size_t>(h) * D + tn * 16 + lm] =
                            acc[rr];
                }
            }
        }

        if (chunk_end) {
            if (cend < N) {
                // (6) refresh the boundary: B <- B Q_L
#pragma unroll
                for (int c = 0; c < CPL; ++c)
                    Qt[(part * CPL + c) * LDP + row] = cq * P[c];
                __syncthreads();
                v4f racc[RTW];
#pragma unroll
                for (int w = 0; w < RTW; ++w) {
                    const int tile = wave + w * NW;
                    const int tm = tile / (D / 16), tn = tile % (D / 16);
                    const float *pa = Bs + (tm * 16 + lm) * LDP + lk;
                    const float *pb = Qt + (tn * 16 + lm) * LDP + lk;
                    v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int s = 0; s < KS; ++s)
                        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(pa[4 * s], pb[4 * s], acc, 0, 0, 0);
                    racc[w] = acc;
                }
                float vacc = 0.f;
                const int vv = tid / D, vj = tid % D;
                if (tid < 2 * D) {
#pragma unroll 8
                    for (int k = 0; k < D; ++k)
                        vacc = fmaf(Bs[(3 * D + vv) * LDP + k], Qt[vj * LDP + k], vacc);
                }
                __syncthreads();
#pragma unroll
                for (int w = 0; w < RTW; ++w) {
                    const int tile = wave + w * NW;
                    const int tm = tile / (D / 16), tn = tile % (D / 16);
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr)
                        Bs[(tm * 16 + 4 * lk + rr) * LDP + tn * 16 + lm] = racc[w][rr];
                }
                if (tid < 2 * D)
                    Bs[(3 * D + vv) * LDP + vj] = vacc;
            }
#pragma unroll
            for (int c = 0; c < CPL; ++c)
                P[c] = (part * CPL + c == row) ? 1.0f : 0.0f;
            cq = 1.0f;
        }
        if (s1 >= N)
            break;
        s0 = s1;
        c0 = c1;
        cend = cend1;
        nt = nt1;
    }
}

// ------------------------------------------------------------ fuse kernel

struct bf16x4 { uint16_t v[4]; };

__device__ __forceinline__ void store4(float *o, float4 a) { *reinterpret_cast<float4 *>(o) = a; }
__device__ __forceinline__ void store4(uint16_t *o, float4 a)
{
    uint2 w;
    w.x = static_cast<uint32_t>(f32_to_bf16(a.x)) | (static_cast<uint32_t>(f32_to_bf16(a.y)) << 16);
    w.y = static_cast<uint32_t>(f32_to_bf16(a.z)) | (static_cast<uint32_t>(f32_to_bf16(a.w)) << 16);
    *reinterpret_cast<uint2 *>(o) = w;
}

// One thread per 4 channels of one grid cell; routes summed in ascending
// order [OVERVIEW scanning and chunking; SUMMARY 2-D maps].
template <typename OutT>
__global__ __launch_bounds__(256) void fuse_kernel(const float *__restrict__ y,
                                                   const float *__restrict__ scales,
                                                   OutT *__restrict__ out, int B, int H,
                                                   int W, int C, unsigned mask,
                                                   long long nvec)
{
    const long long N = static_cast<long long>(H) * W;
    const int C4 = C >> 2;
    for (long long v = blockIdx.x * static_cast<long long>(blockDim.x) + threadIdx.x; v < nvec;
         v += static_cast<long long>(gridDim.x) * blockDim.x) {
        const int cv = static_cast<int>(v % C4);
        const long long pix = v / C4;
        const long long b = pix / N;
        const long long cell = pix - b * N;
        const int i = static_cast<int>(cell / W);
        const int j = static_cast<int>(cell - static_cast<long long>(i) * W);
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        int slot = 0;
        for (int r = 0; r < 4; ++r) {
            if (!(mask & (1u << r)))
                continue;
            const long long t = route_step(r, H, W, N, i, j);
            const float4 yv = *reinterpret_cast<const float4 *>(
                y + ((static_cast<long long>(slot) * B + b) * N + t) * C + cv * 4);
            const float4 s = *reinterpret_cast<const float4 *>(scales + r * C + cv * 4);
            acc.x = fmaf(s.x, yv.x, acc.x);
            acc.y = fmaf(s.y, yv.y, acc.y);
            acc.z = fmaf(s.z, yv.z, acc.z);
            acc.w = fmaf(s.w, yv.w, acc.w);
            ++slot;
        }
        store4(out + pix * C + cv * 4, acc);
    }
}

// ------------------------------------------------------------ gather kernel

template <typename T> struct Vec4;
template <> struct Vec4<float> { using type = float4; };
template <> struct Vec4<uint16_t> { using type = uint2; };

template <typename T>
__global__ __launch_bounds__(256) void gather_kernel(const T *__restrict__ x,
                                                     T *__restrict__ out, int B, int H,
                                                     int W, int C, unsigned mask, int R,
                                                     long long nvec)
{
    using V = typename Vec4<T>::type;
    const long long N = static_cast<long long>(H) * W;
    const int C4 = C >> 2;
    for (long long v = blockIdx.x * static_cast<long long>(blockDim.x) + threadIdx.x; v < nvec;
         v += static_cast<long long>(gridDim.x) * blockDim.x) {
        const int cv = static_cast<int>(v % C4);
        long long rest = v / C4;
        const long long t = rest % N;
        rest /= N;
        const long long b = rest % B;
        const int slot = static_cast<int>(rest / B);
        const int r = nth_route(mask, slot);
        int i, j;
        route_cell(r, H, W, N, t, i, j);
        const V val = *reinterpret_cast<const V *>(
            x + ((b * H + i) * static_cast<long long>(W) + j) * C + cv * 4);
        *reinterpret_cast<V *>(out + ((static_cast<long long>(slot) * B + b) * N + t) * C +
                               cv * 4) = val;
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

// tokens per sub-block of the MFMA scan kernel
template <int D> struct MfmaT { static constexpr int value = (D == 32) ? 64 : 32; };

template <int D, typename InT>
srnl_status launch_scan(const void *x, const srnl_params *p, int B, int H, int W, int C,
                        int heads, unsigned mask, float *out)
{
    const int R = popcount4(mask);
    const long long nchains = static_cast<long long>(R) * B * heads;
    if (nchains > INT_MAX - 8)
        return fail(SRNL_ERR_ARG, "too many chains (routes * B * heads)");
    const int nblocks = static_cast<int>((nchains + 7) / 8 * 8);
    hipStream_t st = static_cast<hipStream_t>(p->stream);
    if constexpr (D >= 32) {
        constexpr int T = MfmaT<D>::value;
        hipLaunchKernelGGL((scan_mfma_kernel<D, T, InT>), dim3(nblocks), dim3(4 * D), 0, st,
                           static_cast<const InT *>(x), static_cast<const InT *>(p->q),
                           p->states, out, B, H, W, C, heads, mask, R, p->alpha_max, p->eps,
                           p->chunk_row, p->chunk_col, p->flags, static_cast<int>(nchains));
        return launch_check("scan_mfma_kernel");
    } else {
        hipLaunchKernelGGL((scan_simple_kernel<D, InT>), dim3(nblocks), dim3(ScanCfg<D>::NT), 0,
                           st, static_cast<const InT *>(x), static_cast<const InT *>(p->q),
                           p->states, out, B, H, W, C, heads, mask, R, p->alpha_max, p->eps,
                           p->chunk_row, p->chunk_col, p->flags, static_cast<int>(nchains));
        return launch_check("scan_simple_kernel");
    }
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
    case SRNL_ERR_HIP: return "HIP error";
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
    if (p->flags & ~0x1Fu)
        return fail(SRNL_ERR_ARG, "unknown flag bits");
    if (p->in_dtype != SRNL_F32 && p->in_dtype != SRNL_BF16)
        return fail(SRNL_ERR_DTYPE, "in_dtype must be SRNL_F32 or SRNL_BF16");
    if (n == 0)
        return SRNL_OK;   // empty grid
    if (!is_device_ptr(x) || !is_device_ptr(out) || !is_device_ptr(p->states))
        return fail(SRNL_ERR_PTR, "x, out and states must be device memory");
    if (p->q && !is_device_ptr(p->q))
        return fail(SRNL_ERR_PTR, "q must be device memory");
    if (p->in_dtype == SRNL_F32)
        return dispatch_scan<float>(d, x, p, B, H, W, C, heads, route_mask, out);
    return dispatch_scan<uint16_t>(d, x, p, B, H, W, C, heads, route_mask, out);
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
    const long long nvec = static_cast<long long>(B) * H * W * (C / 4);
    const int grid = grid_for(nvec, 256);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (out_dtype == SRNL_F32)
        hipLaunchKernelGGL(fuse_kernel<float>, dim3(grid), dim3(256), 0, st, y, scales,
                           static_cast<float *>(out), B, H, W, C, route_mask, nvec);
    else
        hipLaunchKernelGGL(fuse_kernel<uint16_t>, dim3(grid), dim3(256), 0, st, y, scales,
                           static_cast<uint16_t *>(out), B, H, W, C, route_mask, nvec);
    return launch_check("fuse_kernel");
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
    const int R = popcount4(route_mask);
    const long long nvec = n / 4;
    const int grid = grid_for(nvec, 256);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (dtype == SRNL_F32)
        hipLaunchKernelGGL(gather_kernel<float>, dim3(grid), dim3(256), 0, st,
                           static_cast<const float *>(x), static_cast<float *>(out), B, H, W,
                           C, route_mask, R, nvec);
    else
        hipLaunchKernelGGL(gather_kernel<uint16_t>, dim3(grid), dim3(256), 0, st,
                           static_cast<const uint16_t *>(x), static_cast<uint16_t *>(out), B,
                           H, W, C, route_mask, R, nvec);
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
