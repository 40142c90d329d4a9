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
// One workgroup of LPR*d threads per chain (LPR lanes per row of Q: 8 for
// d = 32, so that a chain spans four waves and each SIMD holds two waves,
// which a single wave's VALU issue rate needs; 4 for d = 64); T tokens per
// sub-block (a chunk is
// processed in sub-blocks of at most T tokens: generation inside a chunk
// reads only the fixed boundary states, so it may be split).
//
//   load      tokens of the next sub-block are prefetched into registers
//             (16-byte loads along the route) while the current one computes
//   generate  [k | v] = X [B_k; B_v]^T on MFMA (v_mfma_f32_16x16x4f32)
//   epilogue  NT/T lanes per token: |k|^2, b_eta . x, b_alpha . x, k^, e, the
//             soft cap, the spectral clamp, and the key Gram scalar
//             k^_{t-1} . k^_t (DPP group reductions)
//   scales    one wave forms the running retention products c_t of the
//             sub-block (prefix product over its tokens)
//   update    LPR lanes per row of Q = c P, d/LPR columns per lane (below)
//   readout   Y = Z B_c^T on MFMA, z_t = Q_t q_t
//   refresh   B <- B Q_L on MFMA (the two vector memories on VALU)
//
// MFMA 16x16x4 f32 operand layout (lane l): A[l%16][k], B[k][l%16] with the
// k index of instruction s taken as (l/16) * d/4 + s (any bijection onto the
// reduction index gives the same sum), so each lane's operands for one tile
// are d/4 consecutive floats, read with ds_read_b128; D[4(l/16)+r][l%16] in
// accumulator register r. Operand arrays are stored [m or n][k] with row
// stride d+4 floats (16-byte aligned rows, distinct banks per 8-lane phase).

typedef float v4f __attribute__((ext_vector_type(4)));

template <int D, int LPR, int T> struct MCfg {
    static constexpr int NT = LPR * D;             // threads: LPR lanes per row of Q
    static constexpr int NW = NT / 64;             // waves
    static constexpr int ROWS = 3 * D + 2;
    static constexpr int LDP = D + 4;              // operand row stride
    static constexpr int CPL = D / LPR;            // Q columns per lane
    static constexpr int KS = D / 4;               // MFMA K-steps over d
    static constexpr int TP = T + 2;               // token rows incl. two prefetch pad rows
    static constexpr int NTC = D / 16;             // 16-wide column tiles of d
    static_assert(T % 16 == 0, "T must be a multiple of 16");
    static_assert(T <= 64, "one wave scans the sub-block's retention products");
    static_assert(CPL % 4 == 0, "lanes hold whole float4s of a row");
    static_assert(NW % NTC == 0 || NTC % NW == 0, "tile split over waves");
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

// Sum over an aligned quad with DPP adds (fused v_add_f32_dpp).
__device__ __forceinline__ float quad_sum_dpp(float v)
{
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, true));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, true));
    return v;
}

// Sum over an aligned group of G lanes (G = 2, 4 or 8) with DPP adds.
template <int G> __device__ __forceinline__ float group_sum(float v)
{
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, true)); // xor 1
    if (G >= 4)
        v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, true)); // xor 2
    if (G >= 8)   // row_half_mirror: lane i <- lane 7-i within each group of 8
        v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, true));
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

// Per-token operands of the token loop for one lane: its CPL columns of k^
// and q, e at its row, and the token's scalars.
template <int CPL> struct TokOps {
    float k[CPL];
    float q[CPL];
    float e;
    float4 s;
};

template <int D, int LPR, int T, bool BEFORE, typename InT>
__global__ __launch_bounds__(LPR * D) void scan_mfma_kernel(
    const InT *__restrict__ x, const InT *__restrict__ q,
    const float *__restrict__ states, float *__restrict__ out, int B, int H,
    int W, int C, int heads, unsigned route_mask, int R, float alpha_max,
    float eps, int chunk_row, int chunk_col, unsigned flags, int nchains)
{
    using Cfg = MCfg<D, LPR, T>;
    constexpr int NT = Cfg::NT, NW = Cfg::NW, ROWS = Cfg::ROWS, LDP = Cfg::LDP,
                  CPL = Cfg::CPL, KS = Cfg::KS, TP = Cfg::TP, NTC = Cfg::NTC;
    constexpr int VE = InVec<InT>::VE;
    constexpr int SEGS = D / VE;                       // 16-byte segments per token
    constexpr int NPF = (T * SEGS + NT - 1) / NT;      // prefetch registers per thread
    constexpr int RT = (3 * D / 16) * NTC;             // refresh tiles (matrix memories)
    static_assert(RT % NW == 0, "refresh tiles split evenly over waves");
    constexpr int RTW = RT / NW;                       // refresh tiles per wave

    __shared__ __align__(16) float Bs[ROWS * LDP];     // boundary rows M_c, M_k, M_v, m_eta, m_alpha
    __shared__ __align__(16) float Xs[T * LDP];        // x_t (MFMA operand)
    __shared__ __align__(16) float KZ[T * LDP];        // k (generation), then z_t (readout)
    __shared__ __align__(16) float Es[TP * LDP];       // v, then e = k^ - v
    __shared__ __align__(16) float QVa[TP * D];        // q_t (token loop)
    __shared__ __align__(16) float KHa[TP * D];        // k^_t (token loop)
    __shared__ __align__(16) float4 Sx[TP];            // alpha_t, eta''_t, k^_{t-1} . k^_t, -
    __shared__ __align__(16) float4 Sy[TP];            // c_{t-1}, eta''_t / c_t, c_t, k^_{t-1} . k^_t
    __shared__ __align__(16) float Qt[D * LDP];        // Q_L^T at the chunk end
    __shared__ int s_fast;

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
    const int row = tid / LPR, part = tid % LPR;      // token-loop row of Q and column part

    const float *st = states + (static_cast<size_t>(r) * heads + h) * (ROWS * D);
    for (int idx = tid; idx < ROWS * D; idx += NT)
        Bs[(idx / D) * LDP + idx % D] = st[idx];
    // the two pad rows are read (never used) by the prefetch of the last tokens
    for (int idx = tid; idx < 2 * LDP; idx += NT)
        Es[T * LDP + idx] = 0.f;
    for (int idx = tid; idx < 2 * D; idx += NT) {
        QVa[T * D + idx] = 0.f;
        KHa[T * D + idx] = 0.f;
    }
    if (tid < 2) {
        Sx[T + tid] = make_float4(0.f, 0.f, 0.f, 0.f);
        Sy[T + tid] = make_float4(0.f, 0.f, 0.f, 0.f);
    }

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

    const size_t out_row0 = (static_cast<size_t>(slot) * B + b) * N;

    int c0 = 0;
    int cend = L;
    int s0 = 0;
    int nt = (T < cend) ? T : cend;
    issue_loads(s0, nt);

    while (true) {
        __syncthreads();   // previous sub-block is done with Xs, QVa, KZ; Bs is current

        // (1) store the prefetched tokens (zero rows past nt)
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
                float4 *xd = reinterpret_cast<float4 *>(Xs + u * LDP + sg * VE);
                float4 *qd = reinterpret_cast<float4 *>(QVa + u * D + sg * VE);
#pragma unroll
                for (int e = 0; e < VE / 4; ++e) {
                    xd[e] = make_float4(f[4 * e], f[4 * e + 1], f[4 * e + 2], f[4 * e + 3]);
                    qd[e] = q ? make_float4(fq[4 * e], fq[4 * e + 1], fq[4 * e + 2], fq[4 * e + 3])
                              : make_float4(f[4 * e], f[4 * e + 1], f[4 * e + 2], f[4 * e + 3]);
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

        const int ntm = (nt + 15) >> 4;   // token tiles

        // (2) boundary generation on MFMA: [k | v] = X [B_k; B_v]^T; wave w
        //     produces the 16-wide output tiles tn = w, w + NW, ...
        {
            for (int tn = wave; tn < 2 * NTC; tn += NW) {
                float bg[KS];
                lds_load(Bs + (D + tn * 16 + lm) * LDP + lk * KS, bg);
                float *dst = (tn < NTC) ? KZ : Es;
                const int oc = (tn % NTC) * 16 + lm;
                for (int tm = 0; tm < ntm; ++tm) {
                    float a[KS];
                    lds_load(Xs + (tm * 16 + lm) * LDP + lk * KS, a);
                    v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int s = 0; s < KS; ++s)
                        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], bg[s], acc, 0, 0, 0);
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr)
                        dst[(tm * 16 + 4 * lk + rr) * LDP + oc] = acc[rr];
                }
            }
        }
        __syncthreads();

        // (3) transition scalars, EPL lanes per token [SUMMARY stabilisation];
        //     also the key Gram scalar k^_{t-1} . k^_t used by the token loop
        {
            constexpr int EPL = NT / T;
            constexpr int ECPL = D / EPL;
            static_assert(EPL * T == NT && (EPL == 2 || EPL == 4 || EPL == 8), "epilogue lanes");
            const int u = tid / EPL, ep = tid % EPL;
            if (u < nt) {
                const int up = (u > 0) ? u - 1 : 0;
                float kk[ECPL], vv[ECPL], xv[ECPL], kp[ECPL], be[ECPL], ba[ECPL];
                lds_load(KZ + u * LDP + ep * ECPL, kk);
                lds_load(Es + u * LDP + ep * ECPL, vv);
                lds_load(Xs + u * LDP + ep * ECPL, xv);
                lds_load(KZ + up * LDP + ep * ECPL, kp);
                lds_load(Bs + 3 * D * LDP + ep * ECPL, be);
                lds_load(Bs + (3 * D + 1) * LDP + ep * ECPL, ba);
                float nk2 = 0.f, er = 0.f, ar = 0.f, np2 = 0.f, kdot = 0.f;
#pragma unroll
                for (int c = 0; c < ECPL; ++c) {
                    nk2 = fmaf(kk[c], kk[c], nk2);
                    np2 = fmaf(kp[c], kp[c], np2);
                    kdot = fmaf(kp[c], kk[c], kdot);
                    er = fmaf(be[c], xv[c], er);
                    ar = fmaf(ba[c], xv[c], ar);
                }
                nk2 = group_sum<EPL>(nk2);
                np2 = group_sum<EPL>(np2);
                kdot = group_sum<EPL>(kdot);
                er = group_sum<EPL>(er);
                ar = group_sum<EPL>(ar);
                const float inv = __builtin_amdgcn_rsqf(nk2 + eps);
                const float gram = kdot * inv * __builtin_amdgcn_rsqf(np2 + eps);
                float nkh2 = 0.f, ne2 = 0.f;
                float khv[ECPL], evv[ECPL];
#pragma unroll
                for (int c = 0; c < ECPL; ++c) {
                    khv[c] = kk[c] * inv;
                    evv[c] = khv[c] - vv[c];
                    nkh2 = fmaf(khv[c], khv[c], nkh2);
                    ne2 = fmaf(evv[c], evv[c], ne2);
                }
                float4 *kd = reinterpret_cast<float4 *>(KHa + u * D + ep * ECPL);
                float4 *ed = reinterpret_cast<float4 *>(Es + u * LDP + ep * ECPL);
#pragma unroll
                for (int c4 = 0; c4 < ECPL / 4; ++c4) {
                    kd[c4] = make_float4(khv[4 * c4], khv[4 * c4 + 1], khv[4 * c4 + 2], khv[4 * c4 + 3]);
                    ed[c4] = make_float4(evv[4 * c4], evv[4 * c4 + 1], evv[4 * c4 + 2], evv[4 * c4 + 3]);
                }
                nkh2 = group_sum<EPL>(nkh2);
                ne2 = group_sum<EPL>(ne2);
                const float eta = sigmoidf(er);
                const float alpha = (flags & F_FIXED_ALPHA) ? alpha_max
                                                            : alpha_max * sigmoidf(ar);
                const float g = sqrtf(ne2 * nkh2);
                const float m = 1.0f - alpha;
                float eta1 = eta;
                if (flags & F_NO_CAP) {
                    eta1 = eta;
                } else if (flags & F_HARD_CAP) {
                    if (g > 0.0f && m < eta * g)
                        eta1 = m * __builtin_amdgcn_rcpf(g);
                } else if (g > 0.0f) {
                    const float uu = eta * g * __builtin_amdgcn_rcpf(m);
                    eta1 = (uu < 1e-3f) ? eta * (1.0f - uu * uu * (1.0f / 3.0f))
                                        : m * tanhf(uu) * __builtin_amdgcn_rcpf(g);
                }
                float eta2 = eta1;
                if (!(flags & F_NO_CLAMP) && nkh2 > 0.0f) {
                    const float cap = 2.0f * alpha * __builtin_amdgcn_rcpf(nkh2);
                    if (cap < eta2)
                        eta2 = cap;
                }
                if (ep == 0)
                    Sx[u] = make_float4(alpha, eta2, gram, 0.f);
            }
        }
        __syncthreads();

        // (3b) running retention products of the sub-block (wave 0, lane = token):
        //      c_t = alpha_0 ... alpha_t, with the sub-block starting at scale 1.
        //      If c stays above 2^-60 the token loop takes the fast form.
        if (wave == 0) {
            const float4 sx = Sx[(lane < nt) ? lane : 0];
            float cprod = (lane < nt) ? sx.x : 1.0f;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float o = __shfl_up(cprod, off);
                if (lane >= off)
                    cprod *= o;
            }
            float cprev = __shfl_up(cprod, 1);
            if (lane == 0)
                cprev = 1.0f;
            const float clast = __shfl(cprod, nt - 1);
            if (lane < nt)
                Sy[lane] = make_float4(cprev, sx.y * __builtin_amdgcn_rcpf(cprod), cprod, sx.z);
            if (lane == 0)
                s_fast = clast >= kTinyScale;
        }
        __syncthreads();

        // (4) token-order update, LPR lanes per row of Q = cq P, CPL columns per
        //     lane. Per token t, for this lane's row:
        //       sc = (Q_{t-1} k^_t + e_t)_row,   w = (eta''_t / c_t) sc,
        //       P_t = P_{t-1} - w k^_t^T         (Q_t = alpha_t Q_{t-1} - eta''_t sc k^_t^T)
        //     The next token's dot needs no fresh reduction on the critical
        //     path: P_t . k^_{t+1} = pre - w G_{t,t+1}, with pre = P_{t-1} . k^_{t+1}
        //     reduced one token earlier and G from the epilogue. Operands are
        //     prefetched two tokens ahead (three rotating register buffers).
        //     Fast form: the sub-block starts at scale 1 and uses the
        //     precomputed c_t. General form (a running product would fall
        //     below 2^-60): the scale is tracked token by token and folded
        //     into P before it underflows.
        {
            auto run = [&](auto fast_tag) {
                constexpr bool FAST = decltype(fast_tag)::value;
                if (FAST) {
#pragma unroll
                    for (int c = 0; c < CPL; ++c)
                        P[c] *= cq;
                    cq = 1.0f;
                }
                auto load_tok = [&](int u, TokOps<CPL> &o) {
                    lds_load(KHa + u * D + part * CPL, o.k);
                    lds_load(QVa + u * D + part * CPL, o.q);
                    o.e = Es[u * LDP + row];
                    o.s = FAST ? Sy[u] : Sx[u];
                };
                TokOps<CPL> t0, t1, t2;
                load_tok(0, t0);
                load_tok(1, t1);
                float dk = 0.f;
#pragma unroll
                for (int c = 0; c < CPL; ++c)
                    dk = fmaf(P[c], t0.k[c], dk);
                dk = group_sum<LPR>(dk);
                auto step = [&](int u, TokOps<CPL> &cur, TokOps<CPL> &nxt, TokOps<CPL> &nn) {
                    load_tok(u + 2, nn);
                    float p = 0.f, zb = 0.f;
#pragma unroll
                    for (int c = 0; c < CPL; ++c) {
                        p = fmaf(P[c], nxt.k[c], p);
                        if (BEFORE)
                            zb = fmaf(P[c], cur.q[c], zb);
                    }
                    const float pre = group_sum<LPR>(p);
                    float z = 0.f, w, fold = 1.0f, gnext;
                    if (FAST) {
                        const float sc = fmaf(cur.s.x, dk, cur.e);
                        w = cur.s.y * sc;
                        if (BEFORE)
                            z = cur.s.x * group_sum<LPR>(zb);
                        gnext = nxt.s.w;
                    } else {
                        const float sc = fmaf(cq, dk, cur.e);
                        const float cn = cq * cur.s.x;
                        const bool small = cn < kTinyScale;
                        const float cqn = small ? 1.0f : cn;
                        fold = small ? cn : 1.0f;
                        w = cur.s.y * __builtin_amdgcn_rcpf(cqn) * sc;
                        if (BEFORE)
                            z = cq * group_sum<LPR>(zb);
                        if (small) {
#pragma unroll
                            for (int c = 0; c < CPL; ++c)
                                P[c] *= cn;
                        }
                        cq = cqn;
                        gnext = nxt.s.z;
                    }
#pragma unroll
                    for (int c = 0; c < CPL; ++c)
                        P[c] = fmaf(-w, cur.k[c], P[c]);
                    if (!BEFORE) {
                        float zz = 0.f;
#pragma unroll
                        for (int c = 0; c < CPL; ++c)
                            zz = fmaf(P[c], cur.q[c], zz);
                        z = (FAST ? cur.s.z : cq) * group_sum<LPR>(zz);
                    }
                    KZ[u * LDP + row] = z;   // the LPR lanes of the row store the same value
                    dk = fmaf(-w, gnext, fold * pre);
                };
                int u = 0;
                for (; u + 2 < nt; u += 3) {
                    step(u, t0, t1, t2);
                    step(u + 1, t1, t2, t0);
                    step(u + 2, t2, t0, t1);
                }
                if (u < nt)
                    step(u, t0, t1, t2);
                if (u + 1 < nt)
                    step(u + 1, t1, t2, t0);
                if (FAST)
                    cq = Sy[nt - 1].z;
            };
            if (s_fast)
                run(std::true_type{});
            else
                run(std::false_type{});
        }
        __syncthreads();

        // (5) readout on MFMA: y_t = B_c z_t. With more waves than 16-wide
        //     channel tiles, wave w takes the token tiles tm = w, w + NW, ... and
        //     writes whole output rows of its head; otherwise wave w takes the
        //     channel tiles tn = w, w + NW, ... for every token tile.
        {
            constexpr bool BY_TOKENS = NW > NTC;
            const int tn0 = BY_TOKENS ? 0 : wave, tns = BY_TOKENS ? 1 : NW;
            const int tm0 = BY_TOKENS ? wave : 0, tms = BY_TOKENS ? NW : 1;
            for (int tm = tm0; tm < ntm; tm += tms) {
                float a[KS];
                lds_load(KZ + (tm * 16 + lm) * LDP + lk * KS, a);
                for (int tn = tn0; tn < NTC; tn += tns) {
                    float br[KS];
                    lds_load(Bs + (tn * 16 + lm) * LDP + lk * KS, br);
                    v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int s = 0; s < KS; ++s)
                        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], br[s], acc, 0, 0, 0);
                    float *orow = out + (out_row0 + s0) * C + static_cast<size_t>(h) * D + tn * 16 + lm;
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) {
                        const int u0 = tm * 16 + 4 * lk + rr;
                        if (u0 < nt)
                            orow[static_cast<size_t>(u0) * C] = acc[rr];
                    }
                }
            }
        }

        if (chunk_end) {
            if (cend < N) {
                // (6) refresh the boundary: B <- B Q_L (tiles split over the waves)
#pragma unroll
                for (int c = 0; c < CPL; ++c)
                    Qt[(part * CPL + c) * LDP + row] = cq * P[c];
                __syncthreads();
                v4f racc[RTW];
#pragma unroll
                for (int w = 0; w < RTW; ++w) {
                    const int tile = wave + w * NW;
                    const int tm = tile / NTC, tn = tile % NTC;
                    float a[KS], bq[KS];
                    lds_load(Bs + (tm * 16 + lm) * LDP + lk * KS, a);
                    lds_load(Qt + (tn * 16 + lm) * LDP + lk * KS, bq);
                    v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int s = 0; s < KS; ++s)
                        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], bq[s], acc, 0, 0, 0);
                    racc[w] = acc;
                }
                float vacc = 0.f;
                const int vv = tid / D, vj = tid % D;
                if (tid < 2 * D) {
                    const float4 *br4 = reinterpret_cast<const float4 *>(Bs + (3 * D + vv) * LDP);
                    const float4 *q4 = reinterpret_cast<const float4 *>(Qt + vj * LDP);
#pragma unroll
                    for (int k = 0; k < D / 4; ++k) {
                        const float4 bb = br4[k], qq = q4[k];
                        vacc = fmaf(bb.x, qq.x, vacc);
                        vacc = fmaf(bb.y, qq.y, vacc);
                        vacc = fmaf(bb.z, qq.z, vacc);
                        vacc = fmaf(bb.w, qq.w, vacc);
                    }
                }
                __syncthreads();
#pragma unroll
                for (int w = 0; w < RTW; ++w) {
                    const int tile = wave + w * NW;
                    const int tm = tile / NTC, tn = tile % NTC;
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

// tokens per sub-block and lanes per row of Q of the MFMA scan kernel
template <int D> struct MfmaT { static constexpr int value = (D == 32) ? 64 : 32; };
template <int D> struct MfmaLPR { static constexpr int value = (D == 32) ? 8 : 4; };

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
        constexpr int LPR = MfmaLPR<D>::value;
        if (p->flags & F_READ_BEFORE)
            hipLaunchKernelGGL((scan_mfma_kernel<D, LPR, T, true, InT>), dim3(nblocks), dim3(LPR * D), 0,
                               st, static_cast<const InT *>(x), static_cast<const InT *>(p->q),
                               p->states, out, B, H, W, C, heads, mask, R, p->alpha_max, p->eps,
                               p->chunk_row, p->chunk_col, p->flags, static_cast<int>(nchains));
        else
            hipLaunchKernelGGL((scan_mfma_kernel<D, LPR, T, false, InT>), dim3(nblocks), dim3(LPR * D), 0,
                               st, static_cast<const InT *>(x), static_cast<const InT *>(p->q),
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
