// Eigenvalues of a large dense symmetric matrix on gfx950: two-stage reduction
// to tridiagonal form, then bisection on Sturm counts.
//
// This is the single eigendecomposition of an aggregated covariance (Swift-SVD
// page, sections 2 and 7) and the O(d^3) step the "Random matrix theory
// spectral methods" page (section 6.1) names as the cost for large d.
//
// Stage 1, dense -> band (bandwidth NB = 32).  For each panel of NB columns
//   the m x NB block below the band is QR-factored, Q = I - V T V^T, and the
//   trailing matrix gets A <- Q^T A Q in the two-sided form
//     X = A (V T),  M = T^T V^T X,  Z = X - V M / 2,  A <- A - V Z^T - Z V^T
//   with the products A (V T) (symmetric, lower-stored) and V Z^T + Z V^T
//   (lower triangle only) on MFMA.  A panel that fits in LDS is factored by one
//   workgroup; a taller one by TSQR: local Householder QRs of row blocks, a QR
//   of the stacked R factors, the explicit orthonormal factor Q1, and
//   Householder vectors reconstructed from Q1 by an unpivoted LU of Q1 - S
//   (S = diag(+-1)), which gives V = [Y1; Y2], T = -U S Y1^{-T}, R_panel = S R.
// Stage 2, band -> tridiagonal (bulge chasing).  Sweep s annihilates column s
//   below the subdiagonal with a Householder reflector on rows s+1..s+NB, and
//   chases the fill down the band one NB-block at a time: task k of sweep s
//   applies the previous reflector from the right to the off-diagonal block,
//   builds a reflector from its first column, applies it from the left and to
//   the diagonal block from both sides.  Task (s, k) may run once task
//   (s-1, k+1) is done, so the tasks (s, t - 2s) of one time step t are
//   independent.  A group of G consecutive sweeps runs in one workgroup, one
//   wave per sweep, a time step at a time, with their rows in an LDS ring and
//   each task's block in the wave's registers; a loader wave and a storer wave
//   move band rows between the ring and global memory; consecutive groups are
//   ordered by a row watermark (rows below it are final and stored back), with
//   a bounded wait.  The grid is persistent and about as large as the number
//   of groups that can be active at once: each workgroup runs every
//   gridDim.x-th group, so the waiting groups hold no CUs.  Each reflector's tau is 2 / v^T v of the v it is applied with, so
//   every reflection is orthogonal to rounding.
// Stage 3, eigenvalues of the tridiagonal: 16-section on the Sturm count
//   (number of negative pivots of LDL^T(T - xI)), 16 lanes per eigenvalue, from
//   the Gershgorin interval; results in descending order.  An fp32 matrix is
//   counted in fp32 (backward stable: exact for a matrix within a few ulps of T
//   entry by entry), an fp64 one in fp64.
#include <float.h>

#include <algorithm>
#include <mutex>
#include <type_traits>

#include "common.h"
#include "internal.h"

namespace {

constexpr int NB = 32;       // bandwidth of stage 1 / block size of stage 2
constexpr int LDP = NB + 1;  // LDS row stride of panel blocks

template <typename T> struct Cfg;
template <> struct Cfg<float> {
    static constexpr int RB = 1024;  // panel rows held in LDS by one workgroup
};
template <> struct Cfg<double> {
    static constexpr int RB = 512;
};

__device__ __forceinline__ int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

template <typename T>
__device__ T block_sum256(T x, T *red)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
    const int tid = threadIdx.x;
    __syncthreads();
    if ((tid & 63) == 0) red[tid >> 6] = x;
    __syncthreads();
    T s = red[0] + red[1] + red[2] + red[3];
    __syncthreads();
    return s;
}

// Register-resident Householder QR of a rows x NB block (rows <= NT) by NT
// threads, one row per thread, all NB columns in registers; the column loop is
// expanded at compile time (static_for) so every register index is static.
// Per column k:
//   * every thread forms tau_k and v_k[k] = 1, v_k[r] = x_r / v0 from sigma =
//     sum_{r > k} x_r^2 and x_k (published in LDS by the previous column's update);
//   * the dot products d_c = v_k^T P[:, c] of all NB columns come from one
//     butterfly reduce-scatter across the wave (31 lane exchanges leave the sum
//     of column c in lane c) and a sum across the waves in LDS; d_c for c > k
//     gives the update P[:, c] -= tau v d_c, and d_c = v_c^T v_k for c < k gives
//     column k of T: T[0:k, k] = -tau_k T[0:k, 0:k] d[0:k];
//   * the update leaves sigma and x of column k + 1 for the next column.
// On exit R is in the upper triangle of the block, v_k below the diagonal of
// column k, tau in tau[], T (NB x NB, upper, H_0 ... H_{kr-1} = I - V T V^T) in Tl.
template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F &&f)
{
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<I + 1, N>(f);
    }
}

template <typename T, int NT>
struct RegQr {
    static constexpr int NW = NT / 64;
    T red[NW][NB];   // per-wave column sums
    T dvec[NW][NB];  // d_c of the current column (one copy per wave)
    T sig[NW];      // per-wave partial sigma of the next column
    T x0;           // P[k][k] of the next column
    T tau[NB];
    T Tl[NB * NB];
};


// butterfly reduce-scatter within each half-wave: lane ci (0..31) returns the
// sum over the half of q[ci >> 1].  Level by level the partner differs in bit
// 4 (row swap), 3 (row mirror), 2 (half-row mirror), 1 and 0 (quad permutes)
// of the lane index and shares the higher bits, and each lane keeps the half
// of its values selected by that bit.
template <typename T>
__device__ __forceinline__ T reduce_scatter16(const T (&q)[16], int ci)
{
    T y8[8], y4[4], y2[2];
    const bool b3 = ci & 8, b2 = ci & 4, b1 = ci & 2;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        T a = q[m], b = q[m + 8];
        rowswap16(a, b);
        y8[m] = a + b;
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) y4[m] = (b3 ? y8[m + 4] : y8[m]) + dpp<0x140>(b3 ? y8[m] : y8[m + 4]);
#pragma unroll
    for (int m = 0; m < 2; ++m) y2[m] = (b2 ? y4[m + 2] : y4[m]) + dpp<0x141>(b2 ? y4[m] : y4[m + 2]);
    const T y1 = (b1 ? y2[1] : y2[0]) + dpp<0x4E>(b1 ? y2[0] : y2[1]);
    return y1 + dpp<0xB1>(y1);
}

// 1/x: hardware reciprocal with one Newton step in fp32 (within an ulp or so),
// a correctly rounded division in fp64
__device__ __forceinline__ float recip(float x)
{
    const float r = __builtin_amdgcn_rcpf(x);
    return r * (2.f - x * r);
}
__device__ __forceinline__ double recip(double x) { return 1.0 / x; }



// sum over the wave
template <typename T>
__device__ __forceinline__ T wave_sum64(T x)
{
    return pair32_sum(half_sum(x));
}

// butterfly reduce-scatter: returns, in every lane, the sum over the wave of
// x[lane % 32].  Level by level the partner differs in bit 4 (row swap), 3
// (row mirror), 2 (half-row mirror), 1 and 0 (quad permutes) of the lane index
// and shares the higher bits; the two half-waves are added at the end.
template <typename T>
__device__ __forceinline__ T reduce_scatter32(const T (&x)[NB], int lane)
{
    T y16[16], y8[8], y4[4], y2[2];
    const bool b3 = lane & 8, b2 = lane & 4, b1 = lane & 2, b0 = lane & 1;
#pragma unroll
    for (int m = 0; m < 16; ++m) {
        T a = x[m], b = x[m + 16];
        rowswap16(a, b);
        y16[m] = a + b;
    }
#pragma unroll
    for (int m = 0; m < 8; ++m) y8[m] = (b3 ? y16[m + 8] : y16[m]) + dpp<0x140>(b3 ? y16[m] : y16[m + 8]);
#pragma unroll
    for (int m = 0; m < 4; ++m) y4[m] = (b2 ? y8[m + 4] : y8[m]) + dpp<0x141>(b2 ? y8[m] : y8[m + 4]);
#pragma unroll
    for (int m = 0; m < 2; ++m) y2[m] = (b1 ? y4[m + 2] : y4[m]) + dpp<0x4E>(b1 ? y4[m] : y4[m + 2]);
    const T y1 = (b0 ? y2[1] : y2[0]) + dpp<0xB1>(b0 ? y2[0] : y2[1]);
    return pair32_sum(y1);
}

template <typename T, int NT>
__device__ __forceinline__ void reg_qr(T (&p)[NB], int rows, int kr, RegQr<T, NT> &S)
{
    constexpr int NW = NT / 64;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const bool live = tid < rows;
    for (int q = tid; q < NB * NB; q += NT) S.Tl[q] = 0;
    {
        T part = (tid > 0 && live) ? p[0] * p[0] : (T)0;
        part = wave_sum64(part);
        if (lane == 0) S.sig[wv] = part;
        if (tid == 0) S.x0 = p[0];
    }
    __syncthreads();
    static_for<0, NB>([&](auto KC) {
        constexpr int k = decltype(KC)::value;
        if (k < kr) {
            T sigma = 0;
#pragma unroll
            for (int w = 0; w < NW; ++w) sigma += S.sig[w];
            const T x0 = S.x0;
            T t = 0, scale = 0, mu = 0;
            if (sigma > 0) {
                mu = sqrt(x0 * x0 + sigma);
                const T v0 = x0 <= 0 ? x0 - mu : -sigma / (x0 + mu);
                t = 2 * v0 * v0 / (sigma + v0 * v0);
                scale = 1 / v0;
            }
            const T v = live ? (tid > k ? scale * p[k] : (tid == k ? (T)1 : (T)0)) : (T)0;
            if (t != 0) {
                // d_c = sum_i v_i P[i][c]: for c > k the update of column c, for c < k
                // (where P holds the earlier Householder vectors below the diagonal)
                // the inner products that form the new column of T
                T x[NB];
#pragma unroll
                for (int c = 0; c < NB; ++c) x[c] = v * p[c];
                const T dsum = reduce_scatter32<T>(x, lane);
                if (lane < NB) S.red[wv][lane] = dsum;
            }
            __syncthreads();  // the partial sums are complete; sig and x0 of column k have been read
            if (t != 0) {
                // every wave forms its own copy of d
                if (lane < NB) {
                    T acc = 0;
#pragma unroll
                    for (int w = 0; w < NW; ++w) acc += S.red[w][lane];
                    S.dvec[wv][lane] = acc;
                }
                wave_sync();
                const T *dv = S.dvec[wv];
                const T tv = t * v;
#pragma unroll
                for (int c = k + 1; c < NB; ++c) p[c] -= tv * dv[c];
                if (tid == k) p[k] = mu;
                if (tid > k) p[k] = v;
                // T[i][k] = -t sum_{i <= j < k} T[i][j] d_j: thread (i, j mod 8), 8-lane sum
                if (k > 0 && tid < 8 * NB) {
                    const int i = tid >> 3, jg = tid & 7;
                    T acc = 0;
#pragma unroll
                    for (int j = jg; j < k; j += 8)
                        if (j >= i) acc += S.Tl[i * NB + j] * dv[j];
                    acc += dpp<0xB1>(acc);
                    acc += dpp<0x4E>(acc);
                    acc += dpp<0x141>(acc);
                    if (jg == 0 && i < k) S.Tl[i * NB + k] = -t * acc;
                }
            }
            if (tid == k) S.Tl[k * NB + k] = t;
            if (tid == 0) S.tau[k] = t;
            if constexpr (k + 1 < NB) {
                T part = (tid > k + 1 && live) ? p[k + 1] * p[k + 1] : (T)0;
                part = wave_sum64(part);
                if (lane == 0) S.sig[wv] = part;
                if (tid == k + 1) S.x0 = p[k + 1];
                __syncthreads();
            }
        }
    });
    for (int k = kr + tid; k < NB; k += NT) S.tau[k] = 0;
    __syncthreads();
}

// ---- direct panel: m <= 256 rows, one workgroup
template <typename T>
__global__ __launch_bounds__(256) void k_panel_direct(T *__restrict__ Pg, int64_t lda, int m, T *__restrict__ V,
                                                      T *__restrict__ Tm)
{
    __shared__ RegQr<T, 256> S;
    const int tid = threadIdx.x;
    T p[NB];
#pragma unroll
    for (int c = 0; c < NB; ++c) p[c] = tid < m ? Pg[(int64_t)tid * lda + c] : (T)0;
    const int kr = min(m - 1, NB);
    reg_qr<T, 256>(p, m, kr, S);
    if (tid < m) {
#pragma unroll
        for (int c = 0; c < NB; ++c) {
            if (tid <= c) Pg[(int64_t)tid * lda + c] = p[c];
            T v = 0;
            if (c < kr) v = tid == c ? (T)1 : (tid > c ? p[c] : (T)0);
            V[(int64_t)tid * NB + c] = v;
        }
    }
    for (int q = tid; q < NB * NB; q += 256) Tm[q] = S.Tl[q];
}

// ---- TSQR, step 1: local QR of row block b (rows [b*per, min(m, (b+1)*per)), per <= NT)
template <typename T, int NT>
__global__ __launch_bounds__(NT) void k_tsqr_local(const T *__restrict__ Pg, int64_t lda, int m, int per,
                                                   T *__restrict__ Vloc, T *__restrict__ Tloc, T *__restrict__ Rstack,
                                                   const int *__restrict__ gate)
{
    if (gate != nullptr && *gate != 1) return;  // runs only for a panel whose CholeskyQR broke down (state 1)
    __shared__ RegQr<T, NT> S;
    const int tid = threadIdx.x;
    const int b = blockIdx.x;
    const int r0 = b * per;
    const int rows = min(per, m - r0);
    T p[NB];
#pragma unroll
    for (int c = 0; c < NB; ++c) p[c] = tid < rows ? Pg[(int64_t)(r0 + tid) * lda + c] : (T)0;
    reg_qr<T, NT>(p, rows, NB, S);
    if (tid < rows) {
#pragma unroll
        for (int c = 0; c < NB; ++c) {
            Vloc[(int64_t)(r0 + tid) * NB + c] = tid == c ? (T)1 : (tid > c ? p[c] : (T)0);
            if (tid < NB) Rstack[(int64_t)b * NB * NB + tid * NB + c] = tid <= c ? p[c] : (T)0;
        }
    }
    for (int q = tid; q < NB * NB; q += NT) Tloc[(int64_t)b * NB * NB + q] = S.Tl[q];
}

// ---- TSQR, steps 1 and 2 in fp32: NW waves with four rows per lane (up to
// 256 NW rows); wave w, lane l holds rows 256 w + l, + 64, + 128, + 192, so
// row k < NB is slot 0 of wave 0's lane k.  The same Householder steps as
// reg_qr: one wave needs no workgroup barrier (its sums are butterflies inside
// the wave); with more, each column takes two (partial sigma, partial d).  As
// the QR of the stacked R factors (one block, Kt not null) it also writes
// K = T V[0:NB]^T, from which Q_top [I; 0] = [I; 0] - V K.
template <typename T, int NW>
__global__ __launch_bounds__(64 * NW) void k_tsqr_wave(const T *__restrict__ Pg, int64_t lda, int m, int per,
                                                       T *__restrict__ Vloc, T *__restrict__ Tloc,
                                                       T *__restrict__ Rstack, T *__restrict__ Kt,
                                                       const int *__restrict__ gate)
{
    if (gate != nullptr && *gate != 1) return;  // runs only for a panel whose CholeskyQR broke down (state 1)
    static_assert(std::is_same<T, float>::value, "rows of 32 fp32 columns in registers");
    constexpr int RPL = 4;
    __shared__ __attribute__((aligned(16))) T red[NW][NB];  // per-wave column sums
    __shared__ T sig[2][NW], x0s[2];                         // per-wave partial sigma, P[k][k] (two buffers)
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int b = blockIdx.x;
    const int r0 = b * per;
    const int rows = min(per, m - r0);
    const int rb = wv * 64 * RPL + lane;  // row of slot 0
    T p[RPL][NB];
#pragma unroll
    for (int q = 0; q < RPL; ++q) {
        const int r = rb + q * 64;
#pragma unroll
        for (int c = 0; c < NB; ++c) p[q][c] = r < rows ? Pg[(int64_t)(r0 + r) * lda + c] : (T)0;
    }
    T Tr[NB];  // wave 0, lane i < NB: row i of T (upper triangular)
#pragma unroll
    for (int c = 0; c < NB; ++c) Tr[c] = 0;
    static_for<0, NB>([&](auto KC) {
        constexpr int k = decltype(KC)::value;
        T part = 0;
#pragma unroll
        for (int q = 0; q < RPL; ++q) part += rb + q * 64 > k ? p[q][k] * p[q][k] : (T)0;
        part = wave_sum64(part);
        T sigma, x0;
        if constexpr (NW == 1) {
            sigma = part;
            x0 = readlane_t(p[0][k], k);
        } else {
            if (lane == 0) sig[k & 1][wv] = part;
            if (tid == k) x0s[k & 1] = p[0][k];
            __syncthreads();
            sigma = 0;
#pragma unroll
            for (int w = 0; w < NW; ++w) sigma += sig[k & 1][w];
            x0 = x0s[k & 1];
        }
        T t = 0, scale = 0, mu = 0;
        if (sigma > 0) {
            mu = sqrt(x0 * x0 + sigma);
            const T v0 = x0 <= 0 ? x0 - mu : -sigma / (x0 + mu);
            t = 2 * v0 * v0 / (sigma + v0 * v0);
            scale = 1 / v0;
        }
        T v[RPL];
#pragma unroll
        for (int q = 0; q < RPL; ++q) {
            const int r = rb + q * 64;
            v[q] = r > k ? scale * p[q][k] : (r == k ? (T)1 : (T)0);
        }
        if (t != 0) {  // the same in every wave
            // d_c = sum_r v_r P[r][c]: for c > k the update of column c, for c < k
            // the inner products with the earlier Householder vectors (T's column)
            T x[NB];
#pragma unroll
            for (int c = 0; c < NB; ++c) {
                T a = 0;
#pragma unroll
                for (int q = 0; q < RPL; ++q) a += v[q] * p[q][c];
                x[c] = a;
            }
            const T dsum = reduce_scatter32<T>(x, lane);
            if constexpr (NW == 1) {
                wave_sync();
                red[0][lane & (NB - 1)] = dsum;
                wave_sync();
            } else {
                if (lane < NB) red[wv][lane] = dsum;
                __syncthreads();
            }
            T d[NB];
#pragma unroll
            for (int c4 = 0; c4 < NB / 4; ++c4) {
                float4 q4 = reinterpret_cast<const float4 *>(red[0])[c4];
#pragma unroll
                for (int w = 1; w < NW; ++w) {
                    const float4 o = reinterpret_cast<const float4 *>(red[w])[c4];
                    q4.x += o.x;
                    q4.y += o.y;
                    q4.z += o.z;
                    q4.w += o.w;
                }
                d[4 * c4] = q4.x;
                d[4 * c4 + 1] = q4.y;
                d[4 * c4 + 2] = q4.z;
                d[4 * c4 + 3] = q4.w;
            }
#pragma unroll
            for (int q = 0; q < RPL; ++q) {
                const T tv = t * v[q];
#pragma unroll
                for (int c = k + 1; c < NB; ++c) p[q][c] -= tv * d[c];
            }
            // T[i][k] = -t sum_{i <= j < k} T[i][j] d_j (T[i][j] = 0 for j < i)
            T acc = 0;
#pragma unroll
            for (int j = 0; j < k; ++j) acc += Tr[j] * d[j];
            Tr[k] = lane < k ? -t * acc : (T)0;
#pragma unroll
            for (int q = 0; q < RPL; ++q) {
                const int r = rb + q * 64;
                if (r == k) p[q][k] = mu;
                if (r > k) p[q][k] = v[q];
            }
        }
        if (lane == k) Tr[k] = t;
    });
#pragma unroll
    for (int q = 0; q < RPL; ++q) {
        const int r = rb + q * 64;
        if (r < rows) {
#pragma unroll
            for (int c = 0; c < NB; ++c) {
                Vloc[(int64_t)(r0 + r) * NB + c] = r == c ? (T)1 : (r > c ? p[q][c] : (T)0);
                if (r < NB) Rstack[(int64_t)b * NB * NB + r * NB + c] = r <= c ? p[q][c] : (T)0;
            }
        }
    }
    if (wv != 0) return;
    if (lane < NB) {
#pragma unroll
        for (int c = 0; c < NB; ++c) Tloc[(int64_t)b * NB * NB + lane * NB + c] = Tr[c];
    }
    if (Kt != nullptr) {
        // K[j][c] = sum_{j <= l <= c} T[j][l] V[c][l] (upper triangular): lane
        // (j, c parity); V's top rows as LDS broadcasts, T's row j from lane j
        constexpr int LV = NB + 4;
        __shared__ __attribute__((aligned(16))) T Vs[NB * LV];
        if (lane < NB) {
#pragma unroll
            for (int c = 0; c < NB; ++c) Vs[lane * LV + c] = lane == c ? (T)1 : (lane > c ? p[0][c] : (T)0);
        }
        T tj[NB];
#pragma unroll
        for (int l = 0; l < NB; ++l) {
            T a = Tr[l], c2 = Tr[l];
            halfswap32(a, c2);
            tj[l] = (lane & 32) ? a : Tr[l];
        }
        wave_sync();
        const int j = lane & 31, h = lane >> 5;
#pragma unroll
        for (int c = 0; c < NB; ++c) {
            if ((c & 1) != h) continue;
            T acc = 0;
#pragma unroll
            for (int l = 0; l <= c; ++l) acc += tj[l] * Vs[c * LV + l];
            Kt[j * NB + c] = acc;
        }
    }
}

// ---- TSQR, step 2: QR of the stacked R factors; Rf, V_top and K = T V_top[0:NB]^T
// (Q_top [I; 0] = [I; 0] - V_top K)
template <typename T, int NT>
__global__ __launch_bounds__(NT) void k_tsqr_top(const T *__restrict__ Rstack, int nblk, T *__restrict__ Rf,
                                                 T *__restrict__ Vtop, T *__restrict__ Kt,
                                                 const int *__restrict__ gate)
{
    if (gate != nullptr && *gate != 1) return;  // runs only for a panel whose CholeskyQR broke down (state 1)
    __shared__ RegQr<T, NT> S;
    __shared__ T Vt[NB * LDP];
    const int tid = threadIdx.x;
    const int rows = nblk * NB;
    T p[NB];
#pragma unroll
    for (int c = 0; c < NB; ++c) p[c] = tid < rows ? Rstack[(int64_t)tid * NB + c] : (T)0;
    reg_qr<T, NT>(p, rows, NB, S);
    if (tid < NB) {
#pragma unroll
        for (int c = 0; c < NB; ++c) {
            Vt[tid * LDP + c] = tid == c ? (T)1 : (tid > c ? p[c] : (T)0);
            Rf[tid * NB + c] = tid <= c ? p[c] : (T)0;
        }
    }
    __syncthreads();
    // K = T V_top[0:NB]^T
    for (int q = tid; q < NB * NB; q += NT) {
        const int j = q / NB, c = q % NB;
        T acc = 0;
        for (int l = j; l <= c; ++l) acc += S.Tl[j * NB + l] * Vt[c * LDP + l];
        Kt[q] = acc;
    }
    if (tid < rows) {
#pragma unroll
        for (int c = 0; c < NB; ++c) Vtop[(int64_t)tid * NB + c] = tid == c ? (T)1 : (tid > c ? p[c] : (T)0);
    }
}

// ---- TSQR, step 3: Q1 rows of block b = [Qt_b; 0] - V_b (T_b V_b[0:NB]^T Qt_b),
// with Qt_b = [I; 0]_b - V_top,b K_top, rows b NB .. b NB + NB of Q_top [I; 0]
template <typename T>
__global__ __launch_bounds__(256) void k_tsqr_q1(const T *__restrict__ Vloc, const T *__restrict__ Tloc,
                                                 const T *__restrict__ Vtop, const T *__restrict__ Ktop, int m,
                                                 int per, T *__restrict__ Q1, const int *__restrict__ gate)
{
    if (gate != nullptr && *gate != 1) return;  // runs only for a panel whose CholeskyQR broke down (state 1)
    constexpr int L = NB + 1;  // padded rows: a lane per row reads without bank conflicts
    __shared__ T Vt[NB * L], Tb[NB * L], Qb[NB * L], Y[NB * L], K[NB * L];
    const int tid = threadIdx.x;
    const int b = blockIdx.y;
    const int r0 = b * per;
    const int rows = min(per, m - r0);
    for (int p = tid; p < NB * NB; p += 256) {
        const int q = (p / NB) * L + p % NB;
        Vt[q] = Vloc[(int64_t)(r0 + p / NB) * NB + p % NB];
        Tb[q] = Tloc[(int64_t)b * NB * NB + p];
        Y[q] = Vtop[(int64_t)b * NB * NB + p];
        K[q] = Ktop[p];
    }
    __syncthreads();
    if constexpr (sizeof(T) == 4) {
        // three 32 x 32 x 32 products on MFMA by wave 0:
        //   Qb = [I; 0]_b - Y K,  Y = V_b[0:NB]^T Qb,  K = T_b Y
        // (lane l supplies A[l % 32][k + l / 32] and B[k + l / 32][l % 32]; the
        // result element e of lane l is row 8 (e / 4) + 4 (l / 32) + e % 4, column l % 32)
        if (tid < 64) {
            const int lane = tid, cl = lane & 31, hl = lane >> 5;
            auto product = [&](const T *Am, bool a_rows, const T *Bm) {
                f32x16_t acc = {};
#pragma unroll
                for (int kk = 0; kk < NB; kk += 2) {
                    // a_rows: A[i][k] stored at Am[i][k]; else stored transposed, Am[k][i]
                    const float a = a_rows ? Am[cl * L + kk + hl] : Am[(kk + hl) * L + cl];
                    const float bv = Bm[(kk + hl) * L + cl];
                    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a, bv, acc, 0, 0, 0);
                }
                return acc;
            };
            auto row_of = [&](int e) { return (e >> 2) * 8 + hl * 4 + (e & 3); };
            f32x16_t acc = product(Y, true, K);
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int r = row_of(e);
                Qb[r * L + cl] = (b * NB + r == cl ? 1.f : 0.f) - acc[e];
            }
            wave_sync();
            acc = product(Vt, false, Qb);  // V_b^T: A[j][l] = Vt[l][j]
            wave_sync();
#pragma unroll
            for (int e = 0; e < 16; ++e) Y[row_of(e) * L + cl] = acc[e];
            wave_sync();
            acc = product(Tb, true, Y);
            wave_sync();
#pragma unroll
            for (int e = 0; e < 16; ++e) K[row_of(e) * L + cl] = acc[e];
        }
    } else {
        for (int p = tid; p < NB * NB; p += 256) {
            const int i = p / NB, c = p % NB;
            T s = b * NB + i == c ? (T)1 : (T)0;
            for (int j = 0; j < NB; ++j) s -= Y[i * L + j] * K[j * L + c];
            Qb[i * L + c] = s;
        }
        __syncthreads();
        // Y = V_b[0:NB]^T Qt_b ; K = T_b Y
        T yv[NB * NB / 256];
        for (int p = tid, u = 0; p < NB * NB; p += 256, ++u) {
            const int jj = p / NB, c = p % NB;
            T s = 0;
            for (int l = jj; l < NB; ++l) s += Vt[l * L + jj] * Qb[l * L + c];
            yv[u] = s;
        }
        __syncthreads();
        for (int p = tid, u = 0; p < NB * NB; p += 256, ++u) Y[(p / NB) * L + p % NB] = yv[u];
        __syncthreads();
        for (int p = tid; p < NB * NB; p += 256) {
            const int jj = p / NB, c = p % NB;
            T s = 0;
            for (int l = jj; l < NB; ++l) s += Tb[jj * L + l] * Y[l * L + c];
            K[jj * L + c] = s;
        }
    }
    __syncthreads();
    const int i = blockIdx.x * 8 + (tid >> 5);  // row within the block
    const int c = tid & 31;
    if (i < rows) {
        T s = i < NB ? Qb[i * L + c] : (T)0;
        const T *vr = Vloc + (int64_t)(r0 + i) * NB;
        T vrow[NB];
#pragma unroll
        for (int jj = 0; jj < NB; ++jj) vrow[jj] = vr[jj];
#pragma unroll
        for (int jj = 0; jj < NB; ++jj) s -= vrow[jj] * K[jj * L + c];
        Q1[(int64_t)(r0 + i) * NB + c] = s;
    }
}

// ---- Panel QR by CholeskyQR2 in fp64: G = P^T P (partial Grams of CQ_ROWS-row
// blocks, summed by one workgroup), R = chol(G), Q = P R^{-1}, and the same
// once more on Q; the product of the two R factors is the panel's R and the
// second Q its orthonormal factor Q1 (Yamamoto, Nakatsukasa, Yanagisawa and
// Fukaya's CholeskyQR2).  All of it is parallel over the panel's rows, where
// Householder QR of the same panel runs NB dependent column steps.  With the
// Gram in fp64 the first pass leaves Q orthogonal to ~cond(P)^2 eps64 and the
// second to working precision, for cond(P) up to ~1e6: a pivot below CQ_TOL
// times its column's squared norm (or a zero or non-finite one) sets the
// panel's flag, and the TSQR kernels, which run only when it is set, factor the
// panel instead.
constexpr int CQ_ROWS = 256;     // rows per Gram workgroup (two LDS chunks of 128)
constexpr int CQ_AROWS = 32;     // rows per workgroup of Q = P R^{-1}
constexpr double CQ_TOL = 1e-12;

// States of a panel's CholeskyQR (one int in the workspace).
enum : int {
    CQ_DONE1 = 0,   // one pass was enough: Q1 and Rf written by the first pass
    CQ_BROKE = 1,   // a pivot failed: TSQR factors the panel
    CQ_NEED2 = 2,   // the first pass's Q (fp64) goes through a second pass
    CQ_DONE2 = 3,   // the second pass succeeded
};
// One pass leaves Q orthogonal to ~cond(P)^2 eps64: below fp32 rounding while
// cond_F(R) = |R|_F |R^{-1}|_F stays under this (fp32 panels only).
constexpr double CQ_ONE_PASS_COND = 2000.0;

// The partial Grams of P's CQ_ROWS-row blocks (the second pass only in state CQ_NEED2).
template <typename Tin>
__global__ __launch_bounds__(256) void k_cqr_gram(const Tin *__restrict__ P, int64_t ldp, int m,
                                                  double *__restrict__ Gpart, const int *__restrict__ flag)
{
    if (flag != nullptr && *flag != CQ_NEED2) return;
    constexpr int LS = NB + 2;  // 16-byte aligned rows
    constexpr int CH = 128;     // rows per LDS chunk
    constexpr int PER = CH * NB / 256;
    __shared__ __attribute__((aligned(16))) double S[CH * LS];
    const int tid = threadIdx.x;
    // four row groups of 32 rows per chunk; in each, thread t owns the 4 x 4
    // tile (t / 8, t % 8) of the 32 x 32 Gram
    const int g = tid >> 6, t = tid & 63, i0 = 4 * (t >> 3), j0 = 4 * (t & 7);
    double acc[4][4] = {};
#pragma unroll 1
    for (int ch = 0; ch < CQ_ROWS / CH; ++ch) {
        const int64_t r0 = (int64_t)blockIdx.x * CQ_ROWS + ch * CH;
        // every load of the chunk in flight before the first LDS store
        Tin v[PER];
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            const int p = tid + 256 * q, r = p / NB, c = p % NB;
            v[q] = r0 + r < m ? P[(r0 + r) * ldp + c] : (Tin)0;
        }
        if (ch > 0) __syncthreads();  // the previous chunk is consumed
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            const int p = tid + 256 * q;
            S[(p / NB) * LS + p % NB] = (double)v[q];
        }
        __syncthreads();
#pragma unroll 2
        for (int r = g * 32; r < g * 32 + 32; ++r) {
            const double2 a01 = *(const double2 *)&S[r * LS + i0], a23 = *(const double2 *)&S[r * LS + i0 + 2];
            const double2 b01 = *(const double2 *)&S[r * LS + j0], b23 = *(const double2 *)&S[r * LS + j0 + 2];
            const double a[4] = {a01.x, a01.y, a23.x, a23.y}, bb[4] = {b01.x, b01.y, b23.x, b23.y};
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int w = 0; w < 4; ++w) acc[u][w] = fma(a[u], bb[w], acc[u][w]);
        }
    }
    __syncthreads();
    double *red = S;  // 4 x NB x NB partial sums (4096 doubles <= CH * LS)
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int w = 0; w < 4; ++w) red[g * NB * NB + (i0 + u) * NB + j0 + w] = acc[u][w];
    __syncthreads();
    for (int p = tid; p < NB * NB; p += 256)
        Gpart[(int64_t)blockIdx.x * NB * NB + p] = (red[p] + red[NB * NB + p]) + (red[2 * NB * NB + p] + red[3 * NB * NB + p]);
}

// G = the sum of nblk partial Grams; R (upper, G = R^T R) and R^{-1} together
// by Gauss-Jordan elimination on [G | I] without pivoting (G is symmetric
// positive definite): after it the left half is U = D L^T and the right half
// L^{-1} (G = L D L^T, L unit lower), so R = D^{-1/2} U and R^{-1} =
// L^{-T} D^{-1/2}.  Four waves sum the partial Grams (four entries a thread);
// the 32 elimination steps run in one wave without a barrier: lane l holds
// column l of the 32 x 64 system in registers, and step k takes its pivot and
// multipliers from lane k's column by readlane.  A 256-thread workgroup also
// starts on a CU that other kernels' workgroups partly hold, where the
// former 1024-thread one (one barrier per column) waited for a free CU.
// First pass (second == false): R into R1 and R^{-1} into Rinv; the state
// becomes CQ_BROKE on a failed pivot, else CQ_DONE1 (with Rf = R) when T is
// fp32 and cond_F(R) is below CQ_ONE_PASS_COND, else CQ_NEED2.  Second pass
// (only in state CQ_NEED2): Rf = R R1 and R^{-1} into Rinv, state CQ_DONE2, or
// CQ_BROKE on a failed pivot.
constexpr int CH_T = 256;  // threads of k_cqr_chol
template <typename T>
__global__ __launch_bounds__(CH_T) void k_cqr_chol(const double *__restrict__ Gpart, int nblk, bool second,
                                                   double *__restrict__ R1, double *__restrict__ Rinv,
                                                   T *__restrict__ Rf, int *__restrict__ flag)
{
    if (second && *flag != CQ_NEED2) return;
    constexpr int L2 = 2 * NB + 1;
    constexpr int EPT = NB * NB / CH_T;  // entries per thread
    __shared__ double A[NB * L2], diag0[NB], rs[NB], nr[CH_T / 64], ni[CH_T / 64];
    __shared__ int bad;
    const int tid = threadIdx.x;
    // the sum over the partial Grams: eight independent chains of loads per entry
#pragma unroll
    for (int q = 0; q < EPT; ++q) {
        const int p = tid + CH_T * q;
        double s8[8] = {};
        int b = 0;
        for (; b + 8 <= nblk; b += 8) {
#pragma unroll
            for (int u = 0; u < 8; ++u) s8[u] += Gpart[(int64_t)(b + u) * NB * NB + p];
        }
        for (int u = 0; b + u < nblk; ++u) s8[u] += Gpart[(int64_t)(b + u) * NB * NB + p];
        const double sum = ((s8[0] + s8[1]) + (s8[2] + s8[3])) + ((s8[4] + s8[5]) + (s8[6] + s8[7]));
        const int i = p / NB, j = p % NB;
        A[i * L2 + j] = sum;
        A[i * L2 + NB + j] = i == j ? 1.0 : 0.0;
        if (i == j) diag0[i] = sum;
    }
    __syncthreads();
    if (tid < 64) {
        const int l = tid;  // column l of [G | I]
        double a[NB];
#pragma unroll
        for (int i = 0; i < NB; ++i) a[i] = A[i * L2 + l];
        int failed = 0;
#pragma unroll
        for (int k = 0; k < NB; ++k) {
            const double piv = readlane_t(a[k], k);  // uniform: every lane takes the same branch
            if (!(piv > CQ_TOL * diag0[k] && piv <= DBL_MAX)) {
                failed = 1;
                break;
            }
            const double inv = 1.0 / piv;
#pragma unroll
            for (int i = k + 1; i < NB; ++i) {
                const double mi = readlane_t(a[i], k) * inv;
                const double upd = a[i] - mi * a[k];
                a[i] = l > k ? upd : a[i];
            }
        }
#pragma unroll
        for (int i = 0; i < NB; ++i) A[i * L2 + l] = a[i];
        if (l == 0) bad = failed;
    }
    __syncthreads();
    if (bad) {
        if (tid == 0) *flag = CQ_BROKE;
        return;
    }
    if (tid < NB) rs[tid] = 1.0 / sqrt(A[tid * L2 + tid]);
    __syncthreads();
    double r[EPT];
    double sr = 0.0, si = 0.0;
#pragma unroll
    for (int q = 0; q < EPT; ++q) {
        const int p = tid + CH_T * q, i = p / NB, j = p % NB;
        r[q] = j >= i ? A[i * L2 + j] * rs[i] : 0.0;                 // R = D^{-1/2} U
        const double ri = j >= i ? A[j * L2 + NB + i] * rs[j] : 0.0;  // R^{-1} = L^{-T} D^{-1/2}
        Rinv[p] = ri;
        sr += r[q] * r[q];
        si += ri * ri;
    }
    if (second) {
#pragma unroll
        for (int q = 0; q < EPT; ++q) {
            const int p = tid + CH_T * q, i = p / NB, j = p % NB;
            double x = 0.0;  // Rf = R R1
            for (int l = i; l <= j; ++l) x += A[i * L2 + l] * rs[i] * R1[l * NB + j];
            Rf[p] = (T)x;
        }
        if (tid == 0) *flag = CQ_DONE2;
        return;
    }
#pragma unroll
    for (int q = 0; q < EPT; ++q) R1[tid + CH_T * q] = r[q];
    // cond_F(R): wave sums, then the waves' partials
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        sr += __shfl_xor(sr, o);
        si += __shfl_xor(si, o);
    }
    if ((tid & 63) == 0) {
        nr[tid >> 6] = sr;
        ni[tid >> 6] = si;
    }
    __syncthreads();
    double tr = 0.0, ti = 0.0;
    for (int w = 0; w < CH_T / 64; ++w) {
        tr += nr[w];
        ti += ni[w];
    }
    const bool one = sizeof(T) == 4 && sqrt(tr * ti) < CQ_ONE_PASS_COND;
    if (one) {
#pragma unroll
        for (int q = 0; q < EPT; ++q) Rf[tid + CH_T * q] = (T)r[q];
    }
    if (tid == 0) *flag = one ? CQ_DONE1 : CQ_NEED2;
}

// First pass of Q = P R^{-1} (CQ_AROWS rows per workgroup; thread (r, c) forms
// entry c of row r from the row in LDS and column c of R^{-1}): into Q1 (T) in
// state CQ_DONE1, into Qd (fp64) in state CQ_NEED2, nothing otherwise.  Second
// pass (Qd -> Q1): only in state CQ_DONE2.
template <typename Tin, typename T>
__global__ __launch_bounds__(256) void k_cqr_apply(const Tin *__restrict__ P, int64_t ldp, int m,
                                                   const double *__restrict__ Rinv, bool second,
                                                   T *__restrict__ Q1, double *__restrict__ Qd,
                                                   const int *__restrict__ flag)
{
    const int st = *flag;
    if (second ? st != CQ_DONE2 : (st != CQ_DONE1 && st != CQ_NEED2)) return;
    constexpr int L = NB + 1;
    __shared__ double Ri[NB * L], Ps[CQ_AROWS * L];
    const int tid = threadIdx.x, c = tid & 31, rr = tid >> 5;
    const int64_t r0 = (int64_t)blockIdx.x * CQ_AROWS;
    for (int p = tid; p < NB * NB; p += 256) Ri[(p / NB) * L + p % NB] = Rinv[p];
    for (int p = tid; p < CQ_AROWS * NB; p += 256) {
        const int64_t r = r0 + p / NB;
        Ps[(p / NB) * L + p % NB] = r < m ? (double)P[r * ldp + p % NB] : 0.0;
    }
    __syncthreads();
    const bool to_q1 = second || st == CQ_DONE1;
#pragma unroll
    for (int q = 0; q < CQ_AROWS / 8; ++q) {
        const int lr = rr + 8 * q;
        const int64_t r = r0 + lr;
        double x = 0.0;
        for (int i = 0; i <= c; ++i) x = fma(Ps[lr * L + i], Ri[i * L + c], x);
        if (r < m) {
            if (to_q1)
                Q1[r * NB + c] = (T)x;
            else
                Qd[r * NB + c] = x;
        }
    }
}

// ---- TSQR, step 4: Householder reconstruction from Q1's top block
template <typename T>
__global__ __launch_bounds__(64) void k_tsqr_recon(const T *__restrict__ Q1, const T *__restrict__ Rf,
                                                   T *__restrict__ Pg, int64_t lda, T *__restrict__ V,
                                                   T *__restrict__ Ug, T *__restrict__ Tm)
{
    // one wave; lane i (and i + 32) holds row i of Q1 - S in registers, and the
    // pivot rows reach the other lanes as scalars (readlane)
    const int lane = threadIdx.x;
    const int i = lane & 31;
    T m[NB], rf[NB];  // row i of Q1 and of the stacked R, both loaded up front:
                      // a load under the store loop's branch would wait for
                      // every store before it
#pragma unroll
    for (int j = 0; j < NB; ++j) m[j] = Q1[i * NB + j];
#pragma unroll
    for (int j = 0; j < NB; ++j) rf[j] = Rf[i * NB + j];
    T si = 0;  // S[i]
    T sv[NB];  // S, the same in every lane
    static_for<0, NB>([&](auto KC) {
        constexpr int k = decltype(KC)::value;
        const T mk = readlane_t(m[k], k);
        const T s = mk >= 0 ? (T)-1 : (T)1;
        sv[k] = s;
        if (i == k) si = s;
        const T piv = mk - s;
        if (i == k) m[k] = piv;
        T rowk[NB];
#pragma unroll
        for (int j = k + 1; j < NB; ++j) rowk[j] = readlane_t(m[j], k);
        const T rp = recip(piv);  // |piv| >= 1
        if (i > k) {
            const T l = m[k] * rp;
            m[k] = l;
#pragma unroll
            for (int j = k + 1; j < NB; ++j) m[j] -= l * rowk[j];
        }
    });
    // T = -(U S) Y1^{-T}: row i solves z Y1^T = -(U S)[i] by forward substitution,
    // with Y1 unit lower (the multipliers below the diagonal).  Y1 goes through
    // LDS once and its rows are read back as broadcasts.
    constexpr int LY = NB + 4;
    __shared__ __attribute__((aligned(16))) T Y1s[NB * LY];
    if (lane < NB) {
#pragma unroll
        for (int j = 0; j < NB; ++j) Y1s[i * LY + j] = j < i ? m[j] : (T)0;
    }
    wave_sync();
    T z[NB];
    static_for<0, NB>([&](auto JC) {
        constexpr int j = decltype(JC)::value;
        T b = j >= i ? -m[j] * sv[j] : (T)0;
#pragma unroll
        for (int l = 0; l < j; ++l) b -= Y1s[j * LY + l] * z[l];
        asm volatile("" : "+v"(b));  // computed here, not sunk into the stores below
        z[j] = b;
    });
    if (lane < NB) {
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            Tm[i * NB + j] = z[j];
            Ug[i * NB + j] = j >= i ? m[j] : (T)0;
            V[i * NB + j] = i == j ? (T)1 : (i > j ? m[j] : (T)0);
            if (i <= j) Pg[i * lda + j] = si * rf[j];  // R_panel = S R
        }
    }
}

// ---- V rows r_q1.. = Q1 rows U^{-1} (TSQR step 5; rows below r_q1 are already
// in V), then W = V T.  32 lanes per row (lane c owns column c), two rows per
// wave: the forward substitution and the product walk j = 0..31, y_j reaching
// every lane of its row by readlane (lane j, or j + 32 for the upper row), so
// a panel of m rows runs m / 2 waves instead of m / 64.
constexpr int VW_T = 256;
constexpr int VW_R = VW_T / NB;  // rows per workgroup

template <typename T>
__global__ __launch_bounds__(VW_T) void k_vw(const T *__restrict__ Q1, const T *__restrict__ Ug,
                                             const T *__restrict__ Tm, int m, int r_q1, T *__restrict__ V,
                                             T *__restrict__ W)
{
    __shared__ T U[NB * LDP], Ts[NB * LDP];
    const int tid = threadIdx.x;
    for (int p = tid; p < NB * NB; p += VW_T) {
        U[(p / NB) * LDP + p % NB] = r_q1 < m ? Ug[p] : (T)0;
        Ts[(p / NB) * LDP + p % NB] = Tm[p];
    }
    __syncthreads();
    const int c = tid & 31, hi = (tid >> 5) & 1;
    const int64_t r = (int64_t)blockIdx.x * VW_R + (tid >> 5);
    const bool ok = r < m;
    const int64_t rc = ok ? r : m - 1;  // rows past m repeat row m - 1 and store nothing
    T tcol[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) tcol[j] = Ts[j * LDP + c];
    T yc;
    // r_q1 is m (every row, the repeated ones too, takes the first side) or NB,
    // which is even: the two rows of a wave, 2w and 2w + 1, take the same side
    if (rc < r_q1) {
        yc = V[rc * NB + c];
    } else {
        T ucol[NB], udg[NB];
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            ucol[j] = U[j * LDP + c];
            udg[j] = U[j * LDP + j];
        }
        T sc = Q1[rc * NB + c];
        yc = 0;
        static_for<0, NB>([&](auto JC) {
            constexpr int j = decltype(JC)::value;
            const T lo = readlane_t(sc, j), up = readlane_t(sc, j + 32);
            const T yj = (hi ? up : lo) / udg[j];
            if (c == j) yc = yj;
            if (c > j) sc -= yj * ucol[j];
        });
        if (ok) V[r * NB + c] = yc;
    }
    T wc = 0;
    static_for<0, NB>([&](auto JC) {
        constexpr int j = decltype(JC)::value;
        const T lo = readlane_t(yc, j), up = readlane_t(yc, j + 32);
        if (j <= c) wc += (hi ? up : lo) * tcol[j];  // T is upper triangular
    });
    if (ok) W[r * NB + c] = wc;
}

// ---- X partials = A22[rows, jrange] W[jrange]  (A22 lower-stored symmetric)
constexpr int SY_RB = 128;  // rows per workgroup
constexpr int SY_JB = 64;   // columns per K-step

template <typename T>
__global__ __launch_bounds__(256) void k_symm(const T *__restrict__ A, int64_t lda, int m, const T *__restrict__ W,
                                              T *__restrict__ Xpart, int chunk)
{
    __shared__ T As[SY_RB * (SY_JB + 1)];
    __shared__ T Ws[SY_JB * (NB + 1)];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int i0 = blockIdx.x * SY_RB;
    const int jlo = blockIdx.y * chunk, jhi = min(m, jlo + chunk);
    constexpr int NA = SY_RB * SY_JB / 256, NWL = SY_JB * NB / 256;
    T ra[NA], rw[NWL];
    // the A tile (rows i0.., columns j0..) of the lower-stored symmetric matrix,
    // loaded into registers (all loads in flight together)
    auto gload = [&](int j0) {
        const bool lowerTile = j0 + SY_JB - 1 <= i0;
        const bool upperTile = i0 + SY_RB - 1 < j0;
        if (lowerTile) {
#pragma unroll
            for (int q = 0; q < NA; ++q) {
                const int idx = tid + 256 * q, r = idx / SY_JB, c = idx % SY_JB;
                const int i = i0 + r, j = j0 + c;
                ra[q] = (i < m && j < jhi) ? A[(int64_t)i * lda + j] : (T)0;
            }
        } else if (upperTile) {
#pragma unroll
            for (int q = 0; q < NA; ++q) {
                const int idx = tid + 256 * q, c = idx / SY_RB, r = idx % SY_RB;
                const int i = i0 + r, j = j0 + c;
                ra[q] = (i < m && j < jhi) ? A[(int64_t)j * lda + i] : (T)0;
            }
        } else {
#pragma unroll
            for (int q = 0; q < NA; ++q) {
                const int idx = tid + 256 * q, r = idx / SY_JB, c = idx % SY_JB;
                const int i = i0 + r, j = j0 + c;
                T v = 0;
                if (i < m && j < jhi) v = i >= j ? A[(int64_t)i * lda + j] : A[(int64_t)j * lda + i];
                ra[q] = v;
            }
        }
#pragma unroll
        for (int q = 0; q < NWL; ++q) {
            const int idx = tid + 256 * q, r = idx / NB, c = idx % NB;
            const int j = j0 + r;
            rw[q] = j < jhi ? W[(int64_t)j * NB + c] : (T)0;
        }
    };
    auto lstore = [&](int j0) {
        const bool upperTile = i0 + SY_RB - 1 < j0;
        if (upperTile) {
#pragma unroll
            for (int q = 0; q < NA; ++q) {
                const int idx = tid + 256 * q, c = idx / SY_RB, r = idx % SY_RB;
                As[r * (SY_JB + 1) + c] = ra[q];
            }
        } else {
#pragma unroll
            for (int q = 0; q < NA; ++q) {
                const int idx = tid + 256 * q, r = idx / SY_JB, c = idx % SY_JB;
                As[r * (SY_JB + 1) + c] = ra[q];
            }
        }
#pragma unroll
        for (int q = 0; q < NWL; ++q) {
            const int idx = tid + 256 * q, r = idx / NB, c = idx % NB;
            Ws[r * (NB + 1) + c] = rw[q];
        }
    };
    f32x16_t acc32 = {};
    f64x4_t acc64[4] = {};
    if (jlo < jhi) {
        gload(jlo);
        lstore(jlo);
    }
    __syncthreads();
    for (int j0 = jlo; j0 < jhi; j0 += SY_JB) {
        const bool more = j0 + SY_JB < jhi;
        if (more) gload(j0 + SY_JB);
        if constexpr (sizeof(T) == 4) {
#pragma unroll 4
            for (int kk = 0; kk < SY_JB; kk += 2) {
                const float a = As[(wave * 32 + (lane & 31)) * (SY_JB + 1) + kk + (lane >> 5)];
                const float b = Ws[(kk + (lane >> 5)) * (NB + 1) + (lane & 31)];
                acc32 = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc32, 0, 0, 0);
            }
        } else {
#pragma unroll 2
            for (int kk = 0; kk < SY_JB; kk += 4) {
                double a[2], b[2];
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    a[q] = As[(wave * 32 + q * 16 + (lane & 15)) * (SY_JB + 1) + kk + (lane >> 4)];
                    b[q] = Ws[(kk + (lane >> 4)) * (NB + 1) + q * 16 + (lane & 15)];
                }
#pragma unroll
                for (int qa = 0; qa < 2; ++qa)
#pragma unroll
                    for (int qb = 0; qb < 2; ++qb)
                        acc64[qa * 2 + qb] =
                            __builtin_amdgcn_mfma_f64_16x16x4f64(a[qa], b[qb], acc64[qa * 2 + qb], 0, 0, 0);
            }
        }
        __syncthreads();
        if (more) lstore(j0 + SY_JB);
        __syncthreads();
    }
    T *Xp = Xpart + (int64_t)blockIdx.y * m * NB;
    if constexpr (sizeof(T) == 4) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int r = i0 + wave * 32 + (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3);
            if (r < m) Xp[(int64_t)r * NB + (lane & 31)] = acc32[e];
        }
    } else {
#pragma unroll
        for (int qa = 0; qa < 2; ++qa)
#pragma unroll
            for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = i0 + wave * 32 + qa * 16 + (lane >> 4) + 4 * e;
                    if (r < m) Xp[(int64_t)r * NB + qb * 16 + (lane & 15)] = acc64[qa * 2 + qb][e];
                }
    }
}

// ---- the same partial products in fp32 with 16-byte loads.  Tiles of A wholly
// below the diagonal are read row by row (float4 along j) into a row-major LDS
// tile; tiles wholly above it come from the stored lower triangle as rows j of
// A (float4 along i) and stay k-major in LDS (no transpose); the few tiles that
// cross the diagonal are read element by element into the row-major form.  W
// stays row-major.  The two k-slots of a lane's MFMAs walk columns h * 32 + q
// (h = lane / 32, q = 0..31; the sum over k is the same in any order), so on a
// row-major tile one ds_read_b128 gives the A operands of four
// v_mfma_f32_32x32x2f32; the other operands are 32-bit reads of 32 consecutive
// words per half-wave, and rows h * 32 + q of the k-major tile and of W are
// skewed so that the two halves fall on opposite banks.  One LDS buffer and
// one register stage: the loads of K-step k + 1 are in flight during step k's
// MFMAs; 43 KB of LDS and fewer than 168 VGPRs let three workgroups share a CU
// and cover each other's waits.
constexpr int SQ_LD = SY_JB + 4;   // row-major A tile: stride 68 floats (16-byte rows, b128 reads)
constexpr int SQ_LT = SY_RB + 4;   // k-major A tile: stride 132 floats, rows >= 32 skewed by 32 words
constexpr int SQ_LW = NB + 1;      // W: stride 33 floats (the halves 32 rows apart differ by 32 banks)

__device__ __forceinline__ int sq_trow(int k) { return k * SQ_LT + (k >= 32 ? 32 : 0); }

__global__ __launch_bounds__(256) void k_symm_f32(const float *__restrict__ A, int64_t lda, int m,
                                                  const float *__restrict__ W, float *__restrict__ Xpart, int chunk)
{
    static_assert(SY_JB * SQ_LT + 32 <= SY_RB * SQ_LD, "the k-major tile fits the row-major one's space");
    __shared__ __attribute__((aligned(16))) float As[SY_RB * SQ_LD];
    __shared__ float Ws[SY_JB * SQ_LW];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int i0 = blockIdx.x * SY_RB;
    const int jlo = blockIdx.y * chunk, jhi = min(m, jlo + chunk);
    const int64_t end = (int64_t)(m - 1) * lda + m;  // one past A22[m-1][m-1], in elements
    float4 ra[8], rw[2];
    // tile kind of the K-step at column j0: 0 below the diagonal, 1 above, 2 crossing
    auto kind = [&](int j0) __attribute__((always_inline)) {
        return j0 + SY_JB - 1 <= i0 ? 0 : (i0 + SY_RB - 1 < j0 ? 1 : 2);
    };
    auto rsrc = [&](int64_t corner) __attribute__((always_inline)) {
        const int64_t span = (end - corner) * 4;
        return __builtin_amdgcn_make_buffer_rsrc((void *)(A + corner), 0,
                                                 (int)(span < 0x7FFFFFF0 ? (span > 0 ? span : 0) : 0x7FFFFFF0),
                                                 0x00020000);
    };
    auto gload = [&](float4 (&va)[8], float4 (&vw)[2], int j0) __attribute__((always_inline)) {
        const int kd = kind(j0);
        if (kd == 0) {  // rows i0 + r, columns j0 + c4 .. + 3; columns past jhi masked on store
            const __amdgpu_buffer_rsrc_t rs = rsrc((int64_t)i0 * lda + j0);
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int idx = tid + 256 * q, r = idx >> 4, c4 = (idx & 15) * 4;
                va[q] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(
                                                       rs, (int)(((int64_t)r * lda + c4) * 4), 0, 0));
            }
        } else if (kd == 1) {  // stored rows j0 + jr, columns i0 + i4 .. + 3
            const __amdgpu_buffer_rsrc_t rs = rsrc((int64_t)j0 * lda + i0);
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int idx = tid + 256 * q, jr = idx >> 5, i4 = (idx & 31) * 4;
                va[q] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(
                                                       rs, (int)(((int64_t)jr * lda + i4) * 4), 0, 0));
            }
        } else {  // crossing the diagonal: element by element from the lower triangle
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int idx = tid + 256 * q, r = idx >> 4, c4 = (idx & 15) * 4;
                const int i = i0 + r;
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int j = j0 + c4 + e;
                    v[e] = i < m && j < jhi ? (i >= j ? A[(int64_t)i * lda + j] : A[(int64_t)j * lda + i]) : 0.f;
                }
                va[q] = make_float4(v[0], v[1], v[2], v[3]);
            }
        }
#pragma unroll
        for (int q = 0; q < 2; ++q) {  // W rows j0 + k (k < 64), columns c4 .. + 3
            const int idx = tid + 256 * q, k = idx >> 3, c4 = (idx & 7) * 4;
            const int j = min(j0 + k, m - 1);  // clamped (a row past jhi is masked on store)
            vw[q] = *reinterpret_cast<const float4 *>(W + (int64_t)j * NB + c4);
        }
    };
    auto lstore = [&](const float4 (&va)[8], const float4 (&vw)[2], int j0) __attribute__((always_inline)) {
        if (kind(j0) == 1) {  // k-major: row jr holds column j0 + jr of the tile (rows past jhi zero)
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int idx = tid + 256 * q, jr = idx >> 5, i4 = (idx & 31) * 4;
                const bool ok = j0 + jr < jhi;
                *reinterpret_cast<float4 *>(&As[sq_trow(jr) + i4]) = ok ? va[q] : make_float4(0.f, 0.f, 0.f, 0.f);
            }
        } else {
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int idx = tid + 256 * q, r = idx >> 4, c4 = (idx & 15) * 4;
                const int j = j0 + c4;
                float4 v = va[q];
                v.x = j < jhi ? v.x : 0.f;
                v.y = j + 1 < jhi ? v.y : 0.f;
                v.z = j + 2 < jhi ? v.z : 0.f;
                v.w = j + 3 < jhi ? v.w : 0.f;
                *reinterpret_cast<float4 *>(&As[r * SQ_LD + c4]) = v;
            }
        }
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int idx = tid + 256 * q, k = idx >> 3, c4 = (idx & 7) * 4;
            const bool ok = j0 + k < jhi;
            float *wr = &Ws[k * SQ_LW + c4];
            wr[0] = ok ? vw[q].x : 0.f;
            wr[1] = ok ? vw[q].y : 0.f;
            wr[2] = ok ? vw[q].z : 0.f;
            wr[3] = ok ? vw[q].w : 0.f;
        }
    };
    f32x16_t acc = {};
    const int h = lane >> 5, c = lane & 31;
    const float *fa = &As[(wave * 32 + c) * SQ_LD + h * 32];  // row-major: row wave*32 + c, columns h*32..
    const float *ft = &As[sq_trow(h * 32) + wave * 32 + c];  // k-major: rows h*32.., column wave*32 + c
    const float *fw = &Ws[(h * 32) * SQ_LW + c];               // W rows h*32.., column c
    if (jlo < jhi) {
        gload(ra, rw, jlo);
        lstore(ra, rw, jlo);
    }
    __syncthreads();
    for (int jc = jlo; jc < jhi; jc += SY_JB) {
        const bool more = jc + SY_JB < jhi;
        if (more) gload(ra, rw, jc + SY_JB);  // in flight during this step's MFMAs
        if (kind(jc) == 1) {
#pragma unroll
            for (int q = 0; q < 32; ++q)
                acc = __builtin_amdgcn_mfma_f32_32x32x2f32(ft[q * SQ_LT], fw[q * SQ_LW], acc, 0, 0, 0);
        } else {
#pragma unroll
            for (int q4 = 0; q4 < 8; ++q4) {
                const float4 a4 = *reinterpret_cast<const float4 *>(fa + q4 * 4);
                acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a4.x, fw[(q4 * 4 + 0) * SQ_LW], acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a4.y, fw[(q4 * 4 + 1) * SQ_LW], acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a4.z, fw[(q4 * 4 + 2) * SQ_LW], acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a4.w, fw[(q4 * 4 + 3) * SQ_LW], acc, 0, 0, 0);
            }
        }
        __syncthreads();
        if (more) lstore(ra, rw, jc + SY_JB);
        __syncthreads();
    }
    float *Xp = Xpart + (int64_t)blockIdx.y * m * NB;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const int r = i0 + wave * 32 + (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3);
        if (r < m) Xp[(int64_t)r * NB + (lane & 31)] = acc[e];
    }
}

// ---- X = sum of partials; Ppart[blk] = V_blk^T X_blk (XR-row blocks)
constexpr int XR = 128;

template <typename T>
__global__ __launch_bounds__(256) void k_xreduce(const T *__restrict__ Xpart, int ks, int m, const T *__restrict__ V,
                                                 T *__restrict__ X, T *__restrict__ Ppart)
{
    __shared__ T Xs[XR * (NB + 1)];
    __shared__ T Vs[XR * NB];
    __shared__ T red[8][NB * NB];
    const int tid = threadIdx.x;
    const int r0 = blockIdx.x * XR;
    const int rows = min(XR, m - r0);
    constexpr int PER = XR * NB / 256;
    T acc[PER], vv[PER];
#pragma unroll
    for (int q = 0; q < PER; ++q) {
        acc[q] = 0;
        const int idx = tid + 256 * q;
        vv[q] = idx / NB < rows ? V[(int64_t)r0 * NB + idx] : (T)0;
    }
    // four partitions per round, every load unconditional (partition and row
    // clamped, the value masked): one round trip per four partitions instead
    // of one per partition
    for (int p = 0; p < ks; p += 4) {
        T part[4][PER];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const T *src = Xpart + (int64_t)min(p + u, ks - 1) * m * NB + (int64_t)r0 * NB;
#pragma unroll
            for (int q = 0; q < PER; ++q) {
                const int idx = tid + 256 * q;
                part[u][q] = src[idx / NB < rows ? idx : (rows - 1) * NB + idx % NB];
            }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int q = 0; q < PER; ++q) {
                const int idx = tid + 256 * q;
                acc[q] += (p + u < ks && idx / NB < rows) ? part[u][q] : (T)0;
            }
    }
#pragma unroll
    for (int q = 0; q < PER; ++q) {
        const int idx = tid + 256 * q, r = idx / NB, c = idx % NB;
        if (r < rows) X[(int64_t)r0 * NB + idx] = acc[q];
        Xs[r * (NB + 1) + c] = acc[q];
        Vs[idx] = vv[q];
    }
    __syncthreads();
    // thread (c, g): P[j][c] over rows r = g, g + 8, ... for every j
    const int c = tid & 31, g = tid >> 5;
    T pj[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) pj[j] = 0;
    for (int r = g; r < XR; r += 8) {
        const T xc = Xs[r * (NB + 1) + c];
#pragma unroll
        for (int j = 0; j < NB; ++j) pj[j] += Vs[r * NB + j] * xc;
    }
#pragma unroll
    for (int j = 0; j < NB; ++j) red[g][j * NB + c] = pj[j];
    __syncthreads();
    for (int q = tid; q < NB * NB; q += 256) {
        T sum = 0;
#pragma unroll
        for (int gg = 0; gg < 8; ++gg) sum += red[gg][q];
        Ppart[(int64_t)blockIdx.x * NB * NB + q] = sum;
    }
}

// ---- M = T^T sum(Ppart) (every workgroup forms its own copy), then Z = X - V M / 2
// in place in X for the workgroup's rows
constexpr int MZ_BLOCKS = 64;

template <typename T>
__global__ __launch_bounds__(256) void k_mz(const T *__restrict__ Ppart, int nblk, const T *__restrict__ Tm,
                                            T *__restrict__ X, const T *__restrict__ V, int m)
{
    __shared__ T P[NB * LDP], Ts[NB * LDP], Ms[NB * NB];
    const int tid = threadIdx.x;
    constexpr int PER = NB * NB / 256;
    T acc[PER];
#pragma unroll
    for (int q = 0; q < PER; ++q) acc[q] = 0;
    // 16 partial blocks per round, every load unconditional (block index
    // clamped, the value masked) so that a round is one round trip
    for (int b0 = 0; b0 < nblk; b0 += 16) {
        T part[16][PER];
#pragma unroll
        for (int u = 0; u < 16; ++u)
#pragma unroll
            for (int q = 0; q < PER; ++q)
                part[u][q] = Ppart[(int64_t)min(b0 + u, nblk - 1) * NB * NB + tid + 256 * q];
#pragma unroll
        for (int u = 0; u < 16; ++u)
#pragma unroll
            for (int q = 0; q < PER; ++q) acc[q] += b0 + u < nblk ? part[u][q] : (T)0;
    }
#pragma unroll
    for (int q = 0; q < PER; ++q) {
        const int p = tid + 256 * q;
        P[(p / NB) * LDP + p % NB] = acc[q];
        Ts[(p / NB) * LDP + p % NB] = Tm[p];
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < PER; ++q) {
        const int p = tid + 256 * q;
        const int i = p / NB, c = p % NB;
        T s = 0;
#pragma unroll
        for (int l = 0; l < NB; ++l)
            if (l <= i) s += Ts[l * LDP + i] * P[l * LDP + c];  // T^T is lower
        Ms[p] = s;
    }
    __syncthreads();
    // rows in batches of four, their loads in flight together
    const int c = tid & 31;
    const int64_t stride = (int64_t)gridDim.x * 8;
    for (int64_t r0 = (int64_t)blockIdx.x * 8 + (tid >> 5); r0 < m; r0 += 4 * stride) {
        T vrow[4][NB], x[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t r = r0 + u * stride;
            const int64_t rc = r < m ? r : m - 1;  // clamped: unconditional loads (the
                                                   // values of a row past m are never stored)
#pragma unroll
            for (int j = 0; j < NB; ++j) vrow[u][j] = V[rc * NB + j];
            x[u] = X[rc * NB + c];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t r = r0 + u * stride;
            T s = 0;
#pragma unroll
            for (int j = 0; j < NB; ++j) s += vrow[u][j] * Ms[j * NB + c];
            if (r < m) X[r * NB + c] = x[u] - (T)0.5 * s;
        }
    }
}

// ---- the same update on the first NB columns of A22 only (every row i >= j):
// the block column of the next panel, updated before that panel is factored.
// SC_ROWS rows per workgroup, four threads per row, eight columns each.
constexpr int SC_ROWS = 64;

template <typename T>
__global__ __launch_bounds__(256) void k_syr2k_cols(T *__restrict__ A, int64_t lda, int m, const T *__restrict__ V,
                                                    const T *__restrict__ Z)
{
    __shared__ T Vj[NB * LDP], Zj[NB * LDP];
    const int tid = threadIdx.x;
    for (int q = tid; q < NB * NB; q += 256) {
        const int r = q / NB, c = q % NB;
        const bool ok = r < m;
        Vj[r * LDP + c] = ok ? V[q] : (T)0;
        Zj[r * LDP + c] = ok ? Z[q] : (T)0;
    }
    __syncthreads();
    const int i = blockIdx.x * SC_ROWS + (tid >> 2), cg = (tid & 3) * 8;
    const int ic = min(i, m - 1);  // clamped: unconditional loads, nothing stored past m
    T vi[NB], zi[NB];
#pragma unroll
    for (int k = 0; k < NB; ++k) {
        vi[k] = V[(int64_t)ic * NB + k];
        zi[k] = Z[(int64_t)ic * NB + k];
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const int j = cg + c;
        T sum = 0;
#pragma unroll
        for (int k = 0; k < NB; ++k) sum += vi[k] * Zj[j * LDP + k] + zi[k] * Vj[j * LDP + k];
        if (i < m && i >= j) A[(int64_t)i * lda + j] -= sum;
    }
}

// ---- A22 -= V Z^T + Z V^T on lower 128 x 128 tiles
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
constexpr int S2_T = 128;
constexpr int S2_K = 2 * NB;

template <typename T>
__global__ __launch_bounds__(256, sizeof(T) == 4 ? 2 : 1) void k_syr2k(T *__restrict__ A, int64_t lda, int m, const T *__restrict__ V,
                                               const T *__restrict__ Z)
{
    __shared__ T Ls[S2_T * (S2_K + 1)];
    __shared__ T Rs[S2_T * (S2_K + 1)];
    int ti, tj;
    tri_tile(xcd_remap(blockIdx.x, gridDim.x), ti, tj);
    const int i0 = ti * S2_T, j0 = tj * S2_T;
    const bool diag = ti == tj;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const bool live = !(diag && wm == 0 && wn == 1);  // the strictly upper quadrant of a diagonal tile
    if constexpr (sizeof(T) == 4) {
        // The tile through a buffer resource that starts at A[i0][j0] and ends
        // after A[m-1][m-1]: rows past m read as zero and take no stores, and a
        // masked element gets an offset past every resource.  Offsets inside
        // the tile are 32-bit (lda < 2^22), one VGPR per element instead of a
        // 64-bit address, so two workgroups fit a CU.
        const int64_t corner = (int64_t)i0 * lda + j0;
        const int64_t span = ((int64_t)(m - 1) * lda + (m - 1) - corner + 1) * 4;  // > 0: the tile starts above m
        const int64_t extent = ((int64_t)(S2_T - 1) * lda + S2_T) * 4;               // the whole tile, < 2^31
        const __amdgpu_buffer_rsrc_t rs =
            __builtin_amdgcn_make_buffer_rsrc(A + corner, 0, (int)(span < extent ? span : extent), 0x00020000);
        // Off the diagonal the product is formed transposed (the MFMA takes R
        // as its first operand), so a lane holds one tile row and 4 x 4
        // consecutive columns: its old values come and go as 16-byte accesses
        // (row wm*64 + qa*32 + lane%32, columns wn*64 + qb*32 + 8 jb + 4 (lane/32)
        // .. + 3).  A diagonal tile keeps the untransposed layout (a lane holds
        // one column, 16 rows) and masks the part above the diagonal element
        // by element.
        const int rT = wm * 64 + (lane & 31), cT = wn * 64 + 4 * (lane >> 5);
        auto voff = [&](int qa, int qb, int jb) {
            return (uint32_t)((rT + qa * 32) * (int)lda + cT + qb * 32 + 8 * jb) * 4u;
        };
        const int rl = wm * 64 + (lane >> 5) * 4, cl = wn * 64 + (lane & 31);  // diagonal: lane's first row and column
        const uint32_t vbase = (uint32_t)(rl * (int)lda + cl) * 4u;
        // element (qa, qb, e): row rl + qa*32 + (e>>2)*8 + (e&3), column cl + qb*32
        auto eoff = [&](int qa, int qb, int e) {
            const int dr = qa * 32 + (e >> 2) * 8 + (e & 3);
            const bool ok = rl + dr >= cl + qb * 32;
            return ok ? vbase + (uint32_t)(dr * (int)lda + qb * 32) * 4u : 0x80000000u;
        };
        // L = [V | Z] rows i0.., R = [Z | V] rows j0.. (16-byte loads, rows
        // clamped to m - 1 and masked after, so all stay in flight together)
        constexpr int SQ = S2_T * NB / (4 * 256);
        {
            float4 v_i[SQ], z_i[SQ], v_j[SQ], z_j[SQ];
#pragma unroll
            for (int q = 0; q < SQ; ++q) {
                const int idx = tid + 256 * q, r = idx >> 3, c4 = (idx & 7) * 4;
                const int64_t ic = min(i0 + r, m - 1), jc = min(j0 + r, m - 1);
                v_i[q] = *reinterpret_cast<const float4 *>(V + ic * NB + c4);
                z_i[q] = *reinterpret_cast<const float4 *>(Z + ic * NB + c4);
                v_j[q] = *reinterpret_cast<const float4 *>(V + jc * NB + c4);
                z_j[q] = *reinterpret_cast<const float4 *>(Z + jc * NB + c4);
            }
#pragma unroll
            for (int q = 0; q < SQ; ++q) {
                const int idx = tid + 256 * q, r = idx >> 3, c4 = (idx & 7) * 4;
                const bool iok = i0 + r < m, jok = j0 + r < m;
                const float vi[4] = {v_i[q].x, v_i[q].y, v_i[q].z, v_i[q].w};
                const float zi[4] = {z_i[q].x, z_i[q].y, z_i[q].z, z_i[q].w};
                const float vj[4] = {v_j[q].x, v_j[q].y, v_j[q].z, v_j[q].w};
                const float zj[4] = {z_j[q].x, z_j[q].y, z_j[q].z, z_j[q].w};
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    Ls[r * (S2_K + 1) + c4 + u] = iok ? vi[u] : 0.f;
                    Ls[r * (S2_K + 1) + NB + c4 + u] = iok ? zi[u] : 0.f;
                    Rs[r * (S2_K + 1) + c4 + u] = jok ? zj[u] : 0.f;
                    Rs[r * (S2_K + 1) + NB + c4 + u] = jok ? vj[u] : 0.f;
                }
            }
        }
        __syncthreads();
        if (!live) return;
        // the old values are requested after the staging and are in flight
        // while the MFMAs run
        f32x16_t acc[2][2] = {};
        if (!diag) {
            float4 oldv[2][2][4];
#pragma unroll
            for (int qa = 0; qa < 2; ++qa)
#pragma unroll
                for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                    for (int jb = 0; jb < 4; ++jb)
                        oldv[qa][qb][jb] = __builtin_bit_cast(
                            float4, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)voff(qa, qb, jb), 0, 0));
#pragma unroll 4
            for (int kk = 0; kk < S2_K; kk += 2) {
                float a[2], b[2];
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    a[q] = Ls[(wm * 64 + q * 32 + (lane & 31)) * (S2_K + 1) + kk + (lane >> 5)];
                    b[q] = Rs[(wn * 64 + q * 32 + (lane & 31)) * (S2_K + 1) + kk + (lane >> 5)];
                }
#pragma unroll
                for (int qa = 0; qa < 2; ++qa)
#pragma unroll
                    for (int qb = 0; qb < 2; ++qb)
                        acc[qa][qb] = __builtin_amdgcn_mfma_f32_32x32x2f32(b[qb], a[qa], acc[qa][qb], 0, 0, 0);
            }
#pragma unroll
            for (int qa = 0; qa < 2; ++qa)
#pragma unroll
                for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                    for (int jb = 0; jb < 4; ++jb) {
                        const float4 o = oldv[qa][qb][jb];
                        const float4 nv = make_float4(o.x - acc[qa][qb][4 * jb], o.y - acc[qa][qb][4 * jb + 1],
                                                      o.z - acc[qa][qb][4 * jb + 2], o.w - acc[qa][qb][4 * jb + 3]);
                        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, nv), rs,
                                                               (int)voff(qa, qb, jb), 0, 0);
                    }
        } else {
            float old[2][2][16];  // masked-off elements (the dead quadrant included) read as zero
#pragma unroll
            for (int qa = 0; qa < 2; ++qa)
#pragma unroll
                for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                    for (int e = 0; e < 16; ++e)
                        old[qa][qb][e] = __builtin_bit_cast(
                            float, __builtin_amdgcn_raw_buffer_load_b32(rs, (int)eoff(qa, qb, e), 0, 0));
#pragma unroll 4
            for (int kk = 0; kk < S2_K; kk += 2) {
                float a[2], b[2];
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    a[q] = Ls[(wm * 64 + q * 32 + (lane & 31)) * (S2_K + 1) + kk + (lane >> 5)];
                    b[q] = Rs[(wn * 64 + q * 32 + (lane & 31)) * (S2_K + 1) + kk + (lane >> 5)];
                }
#pragma unroll
                for (int qa = 0; qa < 2; ++qa)
#pragma unroll
                    for (int qb = 0; qb < 2; ++qb)
                        acc[qa][qb] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[qa], b[qb], acc[qa][qb], 0, 0, 0);
            }
#pragma unroll
            for (int qa = 0; qa < 2; ++qa)
#pragma unroll
                for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                    for (int e = 0; e < 16; ++e)
                        __builtin_amdgcn_raw_buffer_store_b32(
                            __builtin_bit_cast(uint32_t, old[qa][qb][e] - acc[qa][qb][e]), rs, (int)eoff(qa, qb, e),
                            0, 0);
        }
    } else {
        // L = [V | Z] rows i0.., R = [Z | V] rows j0..
#pragma unroll
        for (int q = 0; q < S2_T * NB / 256; ++q) {
            const int idx = tid + 256 * q, r = idx / NB, c = idx % NB;
            const int i = i0 + r, j = j0 + r;
            // rows clamped to m - 1 and masked: unconditional loads stay in flight
            // together (a load under a branch would wait for all before it)
            const int64_t ic = min(i, m - 1), jc = min(j, m - 1);
            const T v_i = V[ic * NB + c], z_i = Z[ic * NB + c], v_j = V[jc * NB + c], z_j = Z[jc * NB + c];
            const T vi = i < m ? v_i : (T)0, zi = i < m ? z_i : (T)0;
            const T vj = j < m ? v_j : (T)0, zj = j < m ? z_j : (T)0;
            Ls[r * (S2_K + 1) + c] = vi;
            Ls[r * (S2_K + 1) + NB + c] = zi;
            Rs[r * (S2_K + 1) + c] = zj;
            Rs[r * (S2_K + 1) + NB + c] = vj;
        }
        __syncthreads();
        if (!live) return;
        f64x4_t acc[4][4] = {};
        for (int kk = 0; kk < S2_K; kk += 4) {
            double a[4], b[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                a[q] = Ls[(wm * 64 + q * 16 + (lane & 15)) * (S2_K + 1) + kk + (lane >> 4)];
                b[q] = Rs[(wn * 64 + q * 16 + (lane & 15)) * (S2_K + 1) + kk + (lane >> 4)];
            }
#pragma unroll
            for (int qa = 0; qa < 4; ++qa)
#pragma unroll
                for (int qb = 0; qb < 4; ++qb)
                    acc[qa][qb] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[qa], b[qb], acc[qa][qb], 0, 0, 0);
        }
        // every old value is loaded before the first store
        double old[4][4][4];
#pragma unroll
        for (int qa = 0; qa < 4; ++qa)
#pragma unroll
            for (int qb = 0; qb < 4; ++qb) {
                const int j = j0 + wn * 64 + qb * 16 + (lane & 15);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int i = i0 + wm * 64 + qa * 16 + (lane >> 4) + 4 * e;
                    old[qa][qb][e] = i < m && j < m && i >= j ? A[(int64_t)i * lda + j] : 0.0;
                }
            }
#pragma unroll
        for (int qa = 0; qa < 4; ++qa)
#pragma unroll
            for (int qb = 0; qb < 4; ++qb) {
                const int j = j0 + wn * 64 + qb * 16 + (lane & 15);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int i = i0 + wm * 64 + qa * 16 + (lane >> 4) + 4 * e;
                    if (i < m && j < m && i >= j) A[(int64_t)i * lda + j] = old[qa][qb][e] - acc[qa][qb][e];
                }
            }
    }
}

// ---------------------------------------------------------------- stage 2

constexpr int BW = 2 * NB;  // band storage: band[c * BW + (r - c)] = A[r][c], 0 <= r - c < BW

// Reflector (s, k) of the bulge chase (sweep s, task k) is kept, when the
// eigenvectors are wanted, at index refl_index(n, s) + k: sweeps in order, each
// with its (n - 2 - s) / NB + 1 tasks, RFL entries each (v, then tau).
constexpr int RFL = NB + 1;
__host__ __device__ inline int64_t refl_g(int64_t x)  // sum of u / NB over 0 <= u <= x
{
    const int64_t q = x / NB, r = x % NB;
    return NB * q * (q - 1) / 2 + q * (r + 1);
}
__host__ __device__ inline int64_t refl_index(int64_t n, int64_t s)
{
    const int64_t N = n - 2;
    return s + refl_g(N) - refl_g(N - s);
}

template <typename T>
__global__ __launch_bounds__(256) void k_band_copy(const T *__restrict__ A, int64_t lda, int64_t n,
                                                   T *__restrict__ band, int32_t *__restrict__ prog)
{
    // row-major band: band[r * BW + j] = A[r][r - j], 0 <= j < BW (zero beyond the
    // stage-1 bandwidth; the extra columns hold the bulges of stage 2)
    const int64_t idx = blockIdx.x * 256 + threadIdx.x;
    if (idx < n * BW) {
        const int64_t r = idx / BW, j = idx % BW;
        T v = 0;
        if (j <= NB && r - j >= 0) v = A[r * lda + (r - j)];
        band[idx] = v;
    }
    if (idx <= n) prog[idx] = 0;  // per-group row watermarks; prog[n] is the error flag
}

__device__ __forceinline__ int ntasks_of(int64_t s, int64_t n) { return (int)((n - 2 - s) / NB) + 1; }


// Band rows are exchanged between workgroups on different XCDs.  Every such
// access is a relaxed agent-scope atomic (a load or store that is coherent
// across the device by itself), so no cache-wide writeback or invalidation is
// needed; a group's row stores are complete (s_waitcnt) before its watermark is
// published, and the next group loads rows only after it has seen it.  Waits
// are bounded: on time-out the error flag is set and every workgroup leaves.
template <typename T>
__device__ __forceinline__ T cload(const T *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ void cstore(T *p, T v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}


// One group of G consecutive sweeps s0 .. s0+G-1 at a time per workgroup: G
// compute waves, a loader wave and a storer wave.  At time step t compute wave i runs
// task (s0 + i, t - 2 (s0 + i)); the tasks of one time step touch disjoint rows
// and depend only on tasks of earlier steps ("(s, k) after (s - 1, k + 1)"), so
// the G waves run them side by side.  The rows of the group stay in an LDS ring
// (row r at slot (r - s0 - 1) mod CAPR, its band entries A[r][r - j] contiguous).
//  * loader: the lead sweep s0 needs NB new rows per step.  The rows for step
//    t + 1 are loaded at step t, as soon as the previous group's watermark has
//    passed them, and written into the ring before the step ends, so no
//    compute wave waits on a load.
//  * storer: the rows no future task of the group touches (below the
//    watermark) are stored at the step after their release, and once the
//    stores are complete, in the same step, the watermark is published for
//    the next group.
// Band rows move between the ring and global memory as buffer loads and
// stores (one instruction per row, row offsets in the instruction; rows past
// the end of the band read as zero) with the same cache policy as cload/cstore.
template <typename T>
__device__ __forceinline__ T band_load(__amdgpu_buffer_rsrc_t rs, int voff, int soff)
{
    if constexpr (sizeof(T) == 4)
        return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b32(rs, voff, soff, 16));
    else
        return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b64(rs, voff, soff, 16));
}
template <typename T>
__device__ __forceinline__ void band_store(__amdgpu_buffer_rsrc_t rs, T x, int voff, int soff)
{
    if constexpr (sizeof(T) == 4)
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, x), rs, voff, soff, 16);
    else
    {
        typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, x), rs, voff, soff, 16);
    }
}

// Bulge-task reductions on the 8 x 8 lane grid (lane = 8 I + J):
// sum8 adds over the 8 lanes of a row group (J = 0..7: lane xor 1, xor 2, then
// the half-row mirror, which pairs the two quads of the group); sum_cols adds
// over the 8 lanes of a column group (I = 0..7: lane xor 8 by a row rotation of
// 8, then xor 16 and xor 32 by the row swaps).  Every lane ends with the sum.
template <typename T>
__device__ __forceinline__ T sum8(T x)
{
    x += dpp<0xB1>(x);
    x += dpp<0x4E>(x);
    x += dpp<0x141>(x);
    return x;
}
template <typename T>
__device__ __forceinline__ T sum_cols(T x)
{
    x += dpp<0x128>(x);
    T a = x, b = x;
    rowswap16(a, b);
    x = a + b;
    a = x;
    b = x;
    halfswap32(a, b);
    return a + b;
}

template <typename T, int G, int CAPR>
__global__ __launch_bounds__(64 * (G + 2)) void k_bulge(T *__restrict__ band, int64_t n, int32_t *__restrict__ wm,
                                                        uint64_t spin_ticks, T *__restrict__ refl)
{
    constexpr int LA = 2;  // the ring holds the lead's chunks up to the next step's (LA - 1 ahead)
    static_assert(CAPR % NB == 0 && (LA + 2 * G - 1) * NB <= CAPR, "ring too small");
    constexpr int LDW = BW + 7;  // 71 = 8 (mod 32) - 1: row-group lanes land on distinct banks
    constexpr int RB = BW * sizeof(T);  // bytes per band row
    constexpr int QI = 4096 / RB;       // rows reachable from one base through the instruction offset
    __shared__ T WRbuf[NB + CAPR * LDW + 64];
    T *const WR = WRbuf + NB;  // NB guard entries before the first ring row
    constexpr int SINK = CAPR * LDW;  // 64 entries after the ring: target of masked-off stores
    __shared__ T vsw[G][NB];
    __shared__ T w2s[G][NB];
    __shared__ int abort_flag[2];  // set at step t in entry t & 1, read by every wave after that step
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: sweep, task and row counts stay scalar
    const int I = lane >> 3, J = lane & 7;  // compute waves: row group and column group of the lane
    const int nn = (int)n;
    const int nsw = nn - 2;
    int32_t *err = wm + n;
    const int ngroups = (nsw + G - 1) / G;
    // a persistent grid: workgroup b runs groups b, b + gridDim.x, ... in turn
    // (each group's lifetime is far shorter than gridDim.x group start offsets,
    // so the next group of a workgroup is due only after its previous one ends)
    int g = blockIdx.x, s0 = 0, Ge = 0, ntl = 0;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(band, 0, nn * RB, 0x00020000);
    // ring slot of row r, counted from the group's first row so that the lead's
    // NB-row chunks never wrap
    auto slot = [&](int r) { return (r - s0 - 1) % CAPR; };
    auto ntasks = [&](int s) { return (nn - 2 - s) / NB + 1; };
    // a task (s, k) reads and writes only rows s + 1 + k NB .. s + (k + 1) NB
    auto minrow = [&](int s, int k) { return k <= 0 ? s + 1 : s + 1 + k * NB; };
    auto lastrow = [&](int s, int k) { return min(s + (k + 1) * NB, nn - 1); };
    // rows loaded into the ring once the lead's task k has been fetched
    auto loaded_to = [&](int k) { return k < 0 ? s0 + 1 : lastrow(s0, min(k, ntl - 1)) + 1; };

    // the loader's wait for the previous group; sets abort_flag[par] on time-out
    auto wait_rows = [&](int r1, int par) {
        int ok = 1;
        if (g > 0 && lane == 0) {
            if (cload(wm + g - 1) <= r1) {
                const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
                while (cload(wm + g - 1) <= r1) {
                    if (cload(err) != 0 || __builtin_amdgcn_s_memrealtime() - t0 > spin_ticks) {
                        ok = 0;
                        break;
                    }
                    __builtin_amdgcn_s_sleep(1);
                }
            }
            if (!ok) {
                cstore(err, 1);
                abort_flag[par] = 1;
            }
        }
        return __builtin_amdgcn_readfirstlane(ok);
    };
    // the NB rows lo .. lo+NB-1 of a lead chunk (rows past the end read as zero)
    auto load_chunk = [&](int lo, T (&buf)[NB]) {
#pragma unroll
        for (int q = 0; q < NB; ++q)
            buf[q] = band_load<T>(rs, lane * (int)sizeof(T) + (q % QI) * RB, (lo + q / QI * QI) * RB);
    };
    auto write_chunk = [&](int lo, const T (&buf)[NB]) {
        T *p = WR + slot(lo) * LDW + lane;
#pragma unroll
        for (int q = 0; q < NB; ++q) p[q * LDW] = buf[q];
    };

    // stores rows r0 .. r1-1 from the ring to the band
    auto store_rows = [&](int r0, int r1) {
        for (int r = r0; r < r1; r += NB) {
            const int m = min(NB, r1 - r);
            const int sb = slot(r);
            T tmp[NB];
            if (sb + NB <= CAPR) {  // the rows are consecutive in the ring
                const T *p = WR + sb * LDW + lane;
#pragma unroll
                for (int q = 0; q < NB; ++q) tmp[q] = p[q * LDW];
            } else {
#pragma unroll
                for (int q = 0; q < NB; ++q) tmp[q] = WR[(sb + q < CAPR ? sb + q : sb + q - CAPR) * LDW + lane];
            }
            if (m == NB) {
#pragma unroll
                for (int q = 0; q < NB; ++q)
                    band_store<T>(rs, tmp[q], lane * (int)sizeof(T) + (q % QI) * RB, (r + q / QI * QI) * RB);
            } else {
#pragma unroll
                for (int q = 0; q < NB; ++q)
                    if (q < m) band_store<T>(rs, tmp[q], lane * (int)sizeof(T), (r + q) * RB);
            }
        }
    };

    for (; g < ngroups; g += gridDim.x) {
    s0 = g * G;
    Ge = min(G, nsw - s0);
    ntl = ntasks(s0);  // tasks of the lead sweep
    if (tid < 2) abort_flag[tid] = 0;
    __syncthreads();
    // ---- prologue: the lead's first chunk
    if (wv == G) {
        for (int k = 0; k < LA - 1 && k < ntl; ++k) {
            const int lo = loaded_to(k - 1), hi = loaded_to(k);
            if (!wait_rows(hi - 1, 0)) break;
            T tmp[NB];
            load_chunk(lo, tmp);
            write_chunk(lo, tmp);
        }
    }
    __syncthreads();
    if (abort_flag[0]) return;

    int wst = s0 + 1;  // rows below wst have been handed to the storer
    int wmk = s0 + 1;  // rows below wmk are released
    int wpoll = 0;       // loader: the previous group's watermark as last requested
    T taup = 0;          // compute wave: tau of the previous reflector of its sweep
    T vpk[4] = {0, 0, 0, 0};  // compute wave: that reflector at columns J + 8b
    // the group's last sweep ends last: its last task is the group's last step
    const int t_end = 2 * (s0 + Ge - 1) + ntasks(s0 + Ge - 1);
    for (int t = 2 * s0; t < t_end; ++t) {
        const int k0 = t - 2 * s0;
        if (wv == G) {
            // the lead's chunk for the next step.  The previous group's watermark
            // was requested behind the last step's row loads, so it has usually
            // arrived: if it already covers the chunk the rows are loaded at
            // once (watermarks only grow, so an older value is a safe bound),
            // else the loader waits as at the start.
            const int kn = k0 + LA - 1;
            if (kn < ntl) {
                const int lo = loaded_to(kn - 1), hi = loaded_to(kn);
                const int seen = g > 0 ? __builtin_amdgcn_readfirstlane(wpoll) : nn;
                if (seen > hi - 1 || wait_rows(hi - 1, t & 1)) {
                    T ld[NB];
                    load_chunk(lo, ld);
                    if (g > 0) wpoll = cload(wm + g - 1);  // for the next step, in flight behind the rows
                    write_chunk(lo, ld);
                }
            }
        } else if (wv == G + 1) {
            // store the rows released at the previous step and publish their
            // watermark once the stores are complete
            if (wmk > wst) {
                store_rows(wst, wmk);
                __builtin_amdgcn_s_waitcnt(0);
                if (lane == 0) cstore(wm + g, (int32_t)wmk);
            }
        } else {
            const int s = s0 + wv;
            const int k = t - 2 * s;
            if (wv < Ge && k >= 0 && k < ntasks(s)) {
                // Lane (I, J) = (lane / 8, lane % 8) holds rows I + 8a and columns
                // J + 8b (a, b = 0..3) of the task's two blocks: O = A[r0.., c0 ..
                // c0 + NB) (k > 0) and the whole symmetric diagonal block D =
                // A[r0.., r0..] (entries above its diagonal read from their lower
                // mirror).  Sums along a row reduce over the 8 lanes of a row group
                // (three DPP adds), sums down a column over the 8 lanes of a column
                // group (a DPP row rotation and the two row swaps).  With the ring
                // stride LDW = 8 (mod 32) - 1 every one of these block accesses
                // hits distinct banks (or the same word, for the two copies of a
                // diagonal-block entry).
                const int r0 = s + 1 + k * NB;
                const int L = lastrow(s, k) - r0 + 1;
                const int sl0 = slot(r0);
                int rbI[4], rbJ[4];  // ring offsets of rows r0 + I + 8a and r0 + J + 8a
                bool rv[4], cv[4];   // row I + 8a, column J + 8a inside the task
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    int x = sl0 + I + 8 * a;
                    x -= x >= CAPR ? CAPR : 0;
                    rbI[a] = x * LDW;
                    int y = sl0 + J + 8 * a;
                    y -= y >= CAPR ? CAPR : 0;
                    rbJ[a] = y * LDW;
                    rv[a] = I + 8 * a < L;
                    cv[a] = J + 8 * a < L;
                }
                T *v = vsw[wv];
                T o[4][4], dd[4][4], vp[4];
#pragma unroll
                for (int a = 0; a < 4; ++a) {
#pragma unroll
                    for (int b = 0; b < 4; ++b) {
                        o[a][b] = WR[rbI[a] + NB + I - J + 8 * (a - b)];
                        if (a > b)
                            dd[a][b] = WR[rbI[a] + I - J + 8 * (a - b)];
                        else if (a < b)
                            dd[a][b] = WR[rbJ[b] + J - I + 8 * (b - a)];
                        else
                            dd[a][b] = WR[I >= J ? rbI[a] + I - J : rbJ[a] + J - I];
                    }
                    vp[a] = vpk[a];  // the previous task's reflector at column J + 8a
                }
                const bool full = L == NB;  // every row of the task inside the band (all but a sweep's last task)
                if (!full) {
#pragma unroll
                    for (int a = 0; a < 4; ++a)
#pragma unroll
                        for (int b = 0; b < 4; ++b) {
                            dd[a][b] = rv[a] && cv[b] ? dd[a][b] : (T)0;
                            o[a][b] = rv[a] ? o[a][b] : (T)0;
                        }
                }
                T x[4];  // the column the reflector annihilates (rows I + 8a; lanes J == 0 for k > 0)
                if (k == 0) {
#pragma unroll
                    for (int a = 0; a < 4; ++a) x[a] = rv[a] ? WR[rbI[a] + I + 8 * a + 1] : (T)0;  // column s
                } else {
                    // right: O <- O (I - taup vp vp^T)
                    if (taup != 0) {
#pragma unroll
                        for (int a = 0; a < 4; ++a) {
                            const T u = taup * sum8((o[a][0] * vp[0] + o[a][1] * vp[1]) + (o[a][2] * vp[2] + o[a][3] * vp[3]));
#pragma unroll
                            for (int b = 0; b < 4; ++b) o[a][b] -= u * vp[b];
                        }
                    }
#pragma unroll
                    for (int a = 0; a < 4; ++a) x[a] = o[a][0];  // column c0
                }
                // reflector (I - tau v v^T) x = mu e_0, v_0 = 1
                T sp = (I > 0 ? x[0] * x[0] : (T)0) + x[1] * x[1] + (x[2] * x[2] + x[3] * x[3]);
                const T sigma = readlane0(sum_cols(sp));  // lane 0 sums column group J = 0
                const T x0 = readlane0(x[0]);
                T tau_k = 0, mu = 0;
                T vr[4] = {0, 0, 0, 0};  // v at rows I + 8a (lanes J == 0 until exchanged)
                if (sigma > 0) {
                    mu = sqrt(x0 * x0 + sigma);
                    // v_0 and 1/v_0 need not be exact: tau below is computed from the
                    // v actually stored, so H stays orthogonal, and the column that H
                    // annihilates is set to mu e_0 explicitly
                    const T v0 = x0 <= 0 ? x0 - mu : -sigma * recip(x0 + mu);
                    const T iv0 = recip(v0);
#pragma unroll
                    for (int a = 0; a < 4; ++a) vr[a] = x[a] * iv0;
                    if (I == 0) vr[0] = 1;
                    // tau = 2 / v^T v with v^T v = 1 + sigma iv0^2, the same iv0 that
                    // scales v: I - tau v v^T is orthogonal up to the rounding of the
                    // entries (a tau from v0 alone, whose reciprocal is rounded
                    // differently from iv0, drifts the trace over many applications)
                    tau_k = (T)2 / ((T)1 + sigma * iv0 * iv0);
                }
                wave_sync();
                if (J == 0) {
#pragma unroll
                    for (int a = 0; a < 4; ++a) v[I + 8 * a] = vr[a];
                    if (refl != nullptr) {  // kept for the eigenvectors (rows past the band end: v = 0)
                        T *rp = refl + (refl_index(n, s) + k) * RFL;
#pragma unroll
                        for (int a = 0; a < 4; ++a) rp[I + 8 * a] = vr[a];
                        if (I == 0) rp[NB] = tau_k;
                    }
                }
                wave_sync();
                T vc[4];
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    vr[a] = v[I + 8 * a];
                    vc[a] = v[J + 8 * a];
                }
                if (tau_k != 0) {
                    if (k > 0) {
                        // left: O <- (I - tau v v^T) O, then the annihilated column is mu e_0
#pragma unroll
                        for (int b = 0; b < 4; ++b) {
                            const T wb = tau_k * sum_cols((vr[0] * o[0][b] + vr[1] * o[1][b]) + (vr[2] * o[2][b] + vr[3] * o[3][b]));
#pragma unroll
                            for (int a = 0; a < 4; ++a) o[a][b] -= vr[a] * wb;
                        }
                        if (J == 0) {
#pragma unroll
                            for (int a = 0; a < 4; ++a) o[a][0] = 0;
                            if (I == 0) o[0][0] = mu;
                        }
                    }
                    // two-sided on D: p = tau D v, w = p - (tau/2)(p^T v) v, D -= v w^T + w v^T
                    T p[4];
#pragma unroll
                    for (int a = 0; a < 4; ++a)
                        p[a] = tau_k * sum8((dd[a][0] * vc[0] + dd[a][1] * vc[1]) + (dd[a][2] * vc[2] + dd[a][3] * vc[3]));
                    const T pv = sum_cols((p[0] * vr[0] + p[1] * vr[1]) + (p[2] * vr[2] + p[3] * vr[3]));
                    T w2[4];
#pragma unroll
                    for (int a = 0; a < 4; ++a) w2[a] = p[a] - (T)0.5 * tau_k * pv * vr[a];
                    if (J == 0) {
#pragma unroll
                        for (int a = 0; a < 4; ++a) w2s[wv][I + 8 * a] = w2[a];
                    }
                    wave_sync();
                    T wc[4];
#pragma unroll
                    for (int b = 0; b < 4; ++b) wc[b] = w2s[wv][J + 8 * b];
#pragma unroll
                    for (int a = 0; a < 4; ++a)
#pragma unroll
                        for (int b = 0; b < 4; ++b) dd[a][b] -= vr[a] * wc[b] + w2[a] * vc[b];
                }
                // stores: masked-off entries go to the sink, so they need no branches
                if (k == 0) {
                    if (tau_k != 0 && J == 0) {
#pragma unroll
                        for (int a = 0; a < 4; ++a)
                            WR[rv[a] ? rbI[a] + I + 8 * a + 1 : SINK + lane] = (I == 0 && a == 0) ? mu : (T)0;
                    }
                } else if (full) {
#pragma unroll
                    for (int a = 0; a < 4; ++a)
#pragma unroll
                        for (int b = 0; b < 4; ++b) WR[rbI[a] + NB + I - J + 8 * (a - b)] = o[a][b];
                } else {
#pragma unroll
                    for (int a = 0; a < 4; ++a)
#pragma unroll
                        for (int b = 0; b < 4; ++b) WR[rv[a] ? rbI[a] + NB + I - J + 8 * (a - b) : SINK + lane] = o[a][b];
                }
                if (tau_k != 0) {
                    // the lower triangle: entries with a > b, and a == b where I >= J
                    if (full) {
#pragma unroll
                        for (int a = 0; a < 4; ++a) {
#pragma unroll
                            for (int b = 0; b < a; ++b) WR[rbI[a] + I - J + 8 * (a - b)] = dd[a][b];
                            WR[I >= J ? rbI[a] + I - J : SINK + lane] = dd[a][a];
                        }
                    } else {
#pragma unroll
                        for (int a = 0; a < 4; ++a) {
#pragma unroll
                            for (int b = 0; b < a; ++b) WR[rv[a] ? rbI[a] + I - J + 8 * (a - b) : SINK + lane] = dd[a][b];
                            WR[rv[a] && I >= J ? rbI[a] + I - J : SINK + lane] = dd[a][a];
                        }
                    }
                }
                taup = tau_k;
#pragma unroll
                for (int b = 0; b < 4; ++b) vpk[b] = vc[b];
            }
        }
        // a wait that timed out at the previous step set its entry before that
        // step's barrier; every wave reads it here (it is not written again
        // before the next barrier) and all leave at the same step, the read
        // completing with the task's own LDS stores
        if (abort_flag[(t - 1) & 1]) return;
        __syncthreads();
        // ---- uniform bookkeeping: the storer has taken [wst, wmk); rows below the
        // first row of every remaining task, and already in the ring, are released.
        // At step t + 1 sweep s0 + i is at task x - 2 i (x = t + 1 - 2 s0): the
        // first sweep that has not started (i >= x / 2) starts at its row s0 + i + 1,
        // and the started ones are further down (at least NB rows per task), so
        // that row is the minimum; once all have started, the last sweep's task is.
        wst = max(wst, wmk);
        {
            const int x = t + 1 - 2 * s0;
            const int iu = (x + 1) >> 1;
            const int nt = iu < Ge ? s0 + iu + 1 : minrow(s0 + Ge - 1, x - 2 * (Ge - 1));
            const int nwm = min(loaded_to(k0 + LA - 1), nt);
            if (nwm > wmk) wmk = nwm;
        }
    }
    // ---- epilogue: store what is left and publish the end
    if (wv == G + 1) {
        __builtin_amdgcn_s_waitcnt(0);
        store_rows(wst, nn);
        __builtin_amdgcn_s_waitcnt(0);
        if (lane == 0) cstore(wm + g, (int32_t)nn);
    }
    __syncthreads();  // the ring and the flags are reused by the workgroup's next group
    }
}

// ---------------------------------------------------------------- stage 3

template <typename T>
__global__ __launch_bounds__(256) void k_tridiag_prep(const T *__restrict__ band, int64_t n, double *__restrict__ dd,
                                                      double *__restrict__ ee2, double *__restrict__ bounds,
                                                      float2 *__restrict__ de32)
{
    __shared__ double rlo[256], rhi[256], remax[256];
    const int tid = threadIdx.x;
    double lo = INFINITY, hi = -INFINITY, em = 0.0;
    for (int64_t i = tid; i < n; i += 256) {
        const double d = (double)band[i * BW];                         // A[i][i]
        const double e = i + 1 < n ? (double)band[(i + 1) * BW + 1] : 0.0;  // A[i+1][i]
        const double ep = i > 0 ? (double)band[i * BW + 1] : 0.0;           // A[i][i-1]
        dd[i] = d;
        ee2[i] = e * e;
        if (de32 != nullptr) de32[i] = make_float2((float)d, (float)(ep * ep));  // (d_i, e_{i-1}^2)
        const double r = fabs(e) + fabs(ep);
        lo = fmin(lo, d - r);
        hi = fmax(hi, d + r);
        em = fmax(em, e * e);
    }
    rlo[tid] = lo;
    rhi[tid] = hi;
    remax[tid] = em;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
        if (tid < o) {
            rlo[tid] = fmin(rlo[tid], rlo[tid + o]);
            rhi[tid] = fmax(rhi[tid], rhi[tid + o]);
            remax[tid] = fmax(remax[tid], remax[tid + o]);
        }
        __syncthreads();
    }
    if (tid == 0) {
        const double span = rhi[0] - rlo[0];
        const double pad = 1e-12 * span + 1e-300;
        bounds[0] = rlo[0] - pad;
        bounds[1] = rhi[0] + pad;
        bounds[2] = fmax(1.0, remax[0]) * 1e-300;  // pivmin
        bounds[3] = fmax(1.0, remax[0]) * 1.1754943508222875e-38;  // pivmin of the fp32 recurrence
    }
}

// Sturm count (number of negative pivots of T - x I) in fp64.  1 / q by the
// hardware reciprocal and two Newton steps (relative error a few ulps: the
// count is exact for a matrix whose e_{i-1}^2 differ by a few ulps, within
// the bisection's own tolerance); rows in chunks of 8, the chunk's loads
// issued before its recurrence.
__device__ __forceinline__ double recip64(double q)
{
    double r = __builtin_amdgcn_rcp(q);
    r = fma(r, fma(-q, r, 1.0), r);
    return fma(r, fma(-q, r, 1.0), r);
}
__device__ __forceinline__ int sturm_below(const double *__restrict__ dd, const double *__restrict__ ee2, int64_t n,
                                           double x, double pivmin)
{
    int cnt = 0;
    double q = dd[0] - x;
    if (fabs(q) < pivmin) q = -pivmin;
    cnt += q < 0.0;
    int64_t i = 1;
    for (; i + 8 <= n; i += 8) {
        double d8[8], e8[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            d8[u] = dd[i + u];
            e8[u] = ee2[i + u - 1];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            q = (d8[u] - x) - e8[u] * recip64(q);
            if (fabs(q) < pivmin) q = -pivmin;
            cnt += q < 0.0;
        }
    }
    for (; i < n; ++i) {
        q = (dd[i] - x) - ee2[i - 1] * recip64(q);
        if (fabs(q) < pivmin) q = -pivmin;
        cnt += q < 0.0;
    }
    return cnt;
}

// 4 eigenvalues per 64-lane workgroup, 16 lanes (15 interior points + 1) each
// A multisection grid shared by all eigenvalues of a tridiagonal: the Sturm
// counts at SG_P points evenly inside the starting interval (one lane per
// point), so that each eigenvalue's search starts from the grid cell that
// holds it, about three rounds of 17-section later than from the whole
// interval, for the cost of SG_P counts instead of 16 n.
constexpr int SG_P = 4096;      // grid points (16^3: a three-level 16-way search)
constexpr int SG_MIN_N = 2048;  // below this the grid costs more than it saves

// The grid of the fp64 search (k_sturm_grid_f32 below is the fp32 one).
__global__ __launch_bounds__(64) void k_sturm_grid(const double *__restrict__ dd, const double *__restrict__ ee2,
                                                   int64_t n, const double *__restrict__ bounds,
                                                   double *__restrict__ gx, int *__restrict__ gc)
{
    const double a = bounds[0], b = bounds[1], pivmin = bounds[2];
    const int p = blockIdx.x * 64 + threadIdx.x;
    const double x = a + (b - a) * (double)(p + 1) / (double)(SG_P + 1);
    gx[p] = x;
    gc[p] = sturm_below(dd, ee2, n, x, pivmin);
}

template <typename T>
__global__ __launch_bounds__(64) void k_bisect(const double *__restrict__ dd, const double *__restrict__ ee2,
                                               int64_t n, const double *__restrict__ bounds, double rel_tol,
                                               const double *__restrict__ gx, const int *__restrict__ gc,
                                               T *__restrict__ w)
{
    const int lane = threadIdx.x;
    const int g = lane >> 4, j = lane & 15;
    const int64_t kidx = blockIdx.x * 4 + g;  // descending index
    const bool live = kidx < n;
    const int64_t target = n - 1 - (live ? kidx : 0);  // ascending index
    double a = bounds[0], b = bounds[1];
    const double pivmin = bounds[2];
    if (gc != nullptr) {  // the starting cell from the shared grid, as in the fp32 search
        const unsigned long long gmask = 0xFFFFull << (16 * g);
        int base = 0;
#pragma unroll
        for (int sp = SG_P / 16; sp >= 1; sp /= 16) {
            const int pj = base + (j + 1) * sp - 1;
            const bool le = pj < SG_P && gc[min(pj, SG_P - 1)] <= target;
            base += (int)__popcll(__ballot(le) & gmask) * sp;
        }
        if (base > 0 && gc[base - 1] <= target) a = fmax(a, gx[base - 1]);
        if (base < SG_P && gc[base] > target) b = fmin(b, gx[base]);
    }
    for (int it = 0; it < 40; ++it) {
        const double width = b - a;
        const bool done = width <= rel_tol * fmax(fabs(a), fabs(b)) + 4.0 * pivmin;
        // groups finish independently; all lanes keep the loop uniform
        double x = a + width * (double)(j + 1) / 17.0;
        int cnt = (live && !done) ? sturm_below(dd, ee2, n, x, pivmin) : 0;
        // new a = largest x_j with count <= target, new b = smallest x_j with count > target
        const bool le = cnt <= target;
        double na = le ? x : -INFINITY;
        double nb = le ? INFINITY : x;
#pragma unroll
        for (int o = 8; o > 0; o >>= 1) {
            na = fmax(na, __shfl_xor(na, o, 16));
            nb = fmin(nb, __shfl_xor(nb, o, 16));
        }
        if (!done) {
            if (na > a) a = na;
            if (nb < b) b = nb;
        }
        const int all_done = __all(done || !live);
        if (all_done) break;
    }
    if (live && j == 0) w[kidx] = (T)(0.5 * (a + b));
}

// Sturm count in fp32 for an fp32 matrix: q_i = (d_i - x) - e_{i-1}^2 / q_{i-1}
// with the hardware reciprocal.  Each step perturbs d_i and e_{i-1}^2 by a few
// ulps relative, so the count is exact for a matrix within a few ulps of T
// entry by entry, and the eigenvalues found are within a small multiple of
// eps ||T|| (Kahan's and Demmel's error analysis of the bisection count).  The
// (d_i, e_{i-1}^2) pairs are the same for every lane and are read as scalars.
__device__ __forceinline__ int sturm_below_f32(const float2 *__restrict__ de, int n, float x, float pivmin)
{
    int cnt = 0;
    float q = 1.f;  // e_{-1}^2 = 0
    int i = 0;
    for (; i + 8 <= n; i += 8) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const float2 p = de[i + u];
            q = (p.x - x) - p.y * __builtin_amdgcn_rcpf(q);
            q = fabsf(q) < pivmin ? -pivmin : q;
            cnt += q < 0.f;
        }
    }
    for (; i < n; ++i) {
        const float2 p = de[i];
        q = (p.x - x) - p.y * __builtin_amdgcn_rcpf(q);
        q = fabsf(q) < pivmin ? -pivmin : q;
        cnt += q < 0.f;
    }
    return cnt;
}

// fp32 multisection: 4 eigenvalues per wave, 16 lanes (15 interior points + 1)
// each, down to 2 ulps of |lambda| or 1/16 ulp of ||T||, below the accuracy of
// the count itself
// The starting interval of every fp32 eigenvalue: the fp64 Gershgorin bounds,
// rounded outwards with a few ulps of slack, and the absolute tolerance.
struct BisectStartF32 {
    float a, b, pivmin, atol;
};
__device__ __forceinline__ BisectStartF32 bisect_start_f32(const double *__restrict__ bounds)
{
    float a = (float)bounds[0], b = (float)bounds[1];
    const float span = fmaxf(fabsf(a), fabsf(b));
    a -= 4.f * 1.1920929e-7f * span;
    b += 4.f * 1.1920929e-7f * span;
    return {a, b, (float)bounds[3], 0.0625f * 1.1920929e-7f * span};
}

// The grid of the fp32 search (the multisection grid above, in fp32 from the
// same starting interval as k_bisect_f32).
__global__ __launch_bounds__(64) void k_sturm_grid_f32(const float2 *__restrict__ de, int n,
                                                       const double *__restrict__ bounds, float *__restrict__ gx,
                                                       int *__restrict__ gc)
{
    const BisectStartF32 st = bisect_start_f32(bounds);
    const int p = blockIdx.x * 64 + threadIdx.x;
    const float x = st.a + (st.b - st.a) * ((float)(p + 1) * (1.f / (float)(SG_P + 1)));
    gx[p] = x;
    gc[p] = sturm_below_f32(de, n, x, st.pivmin);
}

__global__ __launch_bounds__(64) void k_bisect_f32(const float2 *__restrict__ de, int n,
                                                   const double *__restrict__ bounds, const float *__restrict__ gx,
                                                   const int *__restrict__ gc, float *__restrict__ w)
{
    const int lane = threadIdx.x;
    const int g = lane >> 4, j = lane & 15;
    const int kidx = blockIdx.x * 4 + g;  // descending index
    const bool live = kidx < n;
    const int target = n - 1 - (live ? kidx : 0);  // ascending index
    const BisectStartF32 st = bisect_start_f32(bounds);
    float a = st.a, b = st.b;
    const float pivmin = st.pivmin, atol = st.atol;
    if (gc != nullptr) {
        // the number of grid points whose count is <= target (the counts grow
        // with x): a 16-way search in three levels, the 16 lanes of a group
        // probing one level's 16 points and counting the hits in their ballot
        const unsigned long long gmask = 0xFFFFull << (16 * g);
        int base = 0;
#pragma unroll
        for (int sp = SG_P / 16; sp >= 1; sp /= 16) {
            const int pj = base + (j + 1) * sp - 1;
            const bool le = pj < SG_P && gc[min(pj, SG_P - 1)] <= target;
            base += (int)__popcll(__ballot(le) & gmask) * sp;
        }
        // the cell's ends bound the search only where their own counts confirm
        // it: count(a) <= target < count(b)
        if (base > 0 && gc[base - 1] <= target) a = fmaxf(a, gx[base - 1]);
        if (base < SG_P && gc[base] > target) b = fminf(b, gx[base]);
    }
    for (int it = 0; it < 40; ++it) {
        const float width = b - a;
        const bool done = width <= fmaxf(atol, 2.f * 1.1920929e-7f * fmaxf(fabsf(a), fabsf(b)));
        const float x = a + width * (float)(j + 1) * (1.f / 17.f);
        const int cnt = (live && !done) ? sturm_below_f32(de, n, x, pivmin) : 0;
        // new a = largest x_j with count <= target, new b = smallest x_j with count > target
        const bool le = cnt <= target;
        float na = le ? x : -INFINITY;
        float nb = le ? INFINITY : x;
        na = fmaxf(na, dpp<0xB1>(na));
        nb = fminf(nb, dpp<0xB1>(nb));
        na = fmaxf(na, dpp<0x4E>(na));
        nb = fminf(nb, dpp<0x4E>(nb));
        na = fmaxf(na, dpp<0x141>(na));
        nb = fminf(nb, dpp<0x141>(nb));
        na = fmaxf(na, dpp<0x140>(na));
        nb = fminf(nb, dpp<0x140>(nb));
        if (!done) {
            if (na > a) a = na;
            if (nb < b) b = nb;
        }
        if (__all(done || !live)) break;
    }
    if (live && j == 0) w[kidx] = 0.5f * (a + b);
}

__global__ void k_info(const int32_t *__restrict__ err, int32_t *__restrict__ info)
{
    if (threadIdx.x == 0) info[0] = err[0] != 0 ? 1 : 0;
}

// ---------------------------------------------------------------- eigenvectors
// The eigenvectors of the k largest eigenvalues, in three steps after stage 3:
//  * inverse iteration on the tridiagonal T (fp64, one thread per eigenvalue):
//    three solves of (T - lambda I) z = x by Gaussian elimination with row
//    interchanges, factored and forward-eliminated in one pass (U's three
//    diagonals and the eliminated right-hand side are kept per row), then back
//    substitution; lambda from fp64 bisection.  Eigenvalues closer than
//    1e-9 ||T|| form a cluster whose vectors one thread computes in order,
//    each orthogonalised against the cluster's earlier ones after every solve
//    (inverse iteration alone leaves them parallel).
//  * the bulge chase's reflectors in reverse order: T = H_M ... H_1 B H_1 ... H_M,
//    so an eigenvector of the band B is H_1 ... H_M y.  A workgroup keeps two
//    columns of Z in LDS and applies every reflector to both (half-wave dot
//    products).
//  * the stage-1 panels in reverse order: A = Q_1 ... Q_P B Q_P^T ... Q_1^T,
//    Q_p = I - V_p T_p V_p^T, so x = Q_1 (... (Q_P y)): per panel W = V^T Z,
//    W <- T W, Z -= V W on 32-column blocks of Z.
// V_p is kept in the strictly lower part of A's panel (below the band, free
// once the panel is factored), T_p in the workspace.

// keep panel p: V (m x NB, unit lower, contiguous) into the strictly lower part
// of the panel block P of A, T into Tk
template <typename T>
__global__ __launch_bounds__(256) void k_keep_panel(const T *__restrict__ V, const T *__restrict__ Tm, int m,
                                                    T *__restrict__ P, int64_t lda, T *__restrict__ Tk)
{
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (blockIdx.x == 0)
        for (int q = threadIdx.x; q < NB * NB; q += 256) Tk[q] = Tm[q];
    const int64_t i = idx / NB;
    const int j = (int)(idx % NB);
    if (i < m && i > j) P[i * lda + j] = V[i * NB + j];
}

// a value in [-1, 1) from (i, c): the start vector of inverse iteration
__device__ __forceinline__ double start_entry(int64_t i, int64_t c)
{
    uint64_t x = (uint64_t)i * 0x9E3779B97F4A7C15ull ^ ((uint64_t)c + 0x632BE59BD9B4E019ull) * 0xBF58476D1CE4E5B9ull;
    x ^= x >> 31;
    x *= 0x94D049BB133111EBull;
    x ^= x >> 29;
    return (double)(x >> 11) * (2.0 / 9007199254740992.0) - 1.0;
}

// Unreduced blocks of the tridiagonal: row i lies in rows blo[i] .. bhi[i] - 1,
// a block ending after row i when |e_i| <= thr ||T|| (zeroing such an e_i moves
// no eigenvalue by more than thr ||T||, the size of the rounding the reduction
// leaves in T).  Vectors of different blocks are orthogonal by their supports.
// One workgroup, n <= VS_ROWS; prefix max / suffix min scans in LDS.
constexpr int VS_ROWS = 8192;
static_assert(VS_ROWS >= EIGVEC_MAX_N, "one workgroup splits every row");
template <typename T>
__global__ __launch_bounds__(1024) void k_vsplit(const T *__restrict__ band, int64_t n,
                                                 const double *__restrict__ bounds, double thr,
                                                 int32_t *__restrict__ blo, int32_t *__restrict__ bhi)
{
    constexpr int R = VS_ROWS / 1024;
    __shared__ int32_t sa[VS_ROWS], sb[VS_ROWS];
    const int tid = threadIdx.x;
    const double cut = thr * fmax(fabs(bounds[0]), fabs(bounds[1]));
    auto brk = [&](int64_t i) {  // a block starts at row i
        return i == 0 || fabs((double)band[i * BW + 1]) <= cut;  // e_{i-1} = A[i][i-1]
    };
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int i = tid * R + r;
        sa[i] = i < n && brk(i) ? i : 0;
        sb[i] = i + 1 < n ? (brk(i + 1) ? i + 1 : (int32_t)n) : (int32_t)n;
    }
    __syncthreads();
    for (int o = 1; o < VS_ROWS; o <<= 1) {
        int32_t ta[R], tb[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int i = tid * R + r;
            ta[r] = i >= o ? max(sa[i], sa[i - o]) : sa[i];
            tb[r] = i + o < VS_ROWS ? min(sb[i], sb[i + o]) : sb[i];
        }
        __syncthreads();
#pragma unroll
        for (int r = 0; r < R; ++r) {
            sa[tid * R + r] = ta[r];
            sb[tid * R + r] = tb[r];
        }
        __syncthreads();
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int i = tid * R + r;
        if (i < n) {
            blo[i] = sa[i];
            bhi[i] = sb[i];
        }
    }
}

// mu[i] = the (i - blo[i])-th largest eigenvalue of row i's block, by the same
// 16-point multisection as the whole-matrix bisection, to 2 eps ||T||
__global__ __launch_bounds__(64) void k_vbisect(const double *__restrict__ dd, const double *__restrict__ ee2,
                                                int64_t n, const double *__restrict__ bounds,
                                                const int32_t *__restrict__ blo, const int32_t *__restrict__ bhi,
                                                double *__restrict__ mu)
{
    const int lane = threadIdx.x;
    const int g = lane >> 4, j = lane & 15;
    const int64_t i = blockIdx.x * 4 + g;
    const bool live = i < n;
    const int64_t lo = live ? blo[i] : 0, hi = live ? bhi[i] : 1;
    const int64_t target = hi - 1 - (live ? i : 0);  // ascending index within the block
    double a = bounds[0], b = bounds[1];
    const double pivmin = bounds[2];
    const double tol = 2.0 * DBL_EPSILON * fmax(fabs(a), fabs(b)) + 4.0 * pivmin;
    for (int it = 0; it < 40; ++it) {
        const double width = b - a;
        const bool done = width <= tol;
        const double x = a + width * (double)(j + 1) / 17.0;
        const int cnt = (live && !done) ? sturm_below(dd + lo, ee2 + lo, hi - lo, x, pivmin) : 0;
        const bool le = cnt <= target;
        double na = le ? x : -INFINITY;
        double nb = le ? INFINITY : x;
#pragma unroll
        for (int o = 8; o > 0; o >>= 1) {
            na = fmax(na, __shfl_xor(na, o, 16));
            nb = fmin(nb, __shfl_xor(nb, o, 16));
        }
        if (!done) {
            if (na > a) a = na;
            if (nb < b) b = nb;
        }
        if (__all(done || !live)) break;
    }
    if (live && j == 0) mu[i] = 0.5 * (a + b);
}

// rank[i] = position of mu[i] in the descending order of all blocks' values
// (ties by row, a NaN after every number), so that column rank[i] of Z belongs
// to w[rank[i]] and the ranks are a permutation whatever the values
__global__ __launch_bounds__(256) void k_vrank(const double *__restrict__ mu, int64_t n, int32_t *__restrict__ rank)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    const double x = mu[i];
    const bool xn = isnan(x);
    int64_t r = 0;
    for (int64_t j = 0; j < n; ++j) {
        const double y = mu[j];
        const bool yn = isnan(y);
        const bool before = xn ? (!yn || j < i) : (!yn && (y > x || (y == x && j < i)));
        r += before;
    }
    rank[i] = (int32_t)r;
}

// Z <- 0 on [n][k] (the rows outside a vector's block stay zero)
template <typename T>
__global__ __launch_bounds__(256) void k_zfill(T *__restrict__ Z, int64_t n, int64_t k, int64_t ldz)
{
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx < n * k) Z[(idx / k) * ldz + idx % k] = (T)0;
}

// Inverse iteration, one thread per row i of the tridiagonal whose eigenvalue
// mu[i] ranks below k: three steps of (T_b - mu I) y <- y on row i's block T_b,
// each a partial-pivoting LU solve (a factor and the right-hand side's
// elimination in one forward pass, then back substitution), the iterate
// normalised.  Eigenvalues of one block closer than 1e-9 ||T|| form a cluster,
// whose first row computes all its vectors in turn, each orthogonalised
// against the earlier ones (modified Gram-Schmidt) after every step.  The
// iteration runs on T / ||T||; pivots are floored at eps, and divide by way
// of their reciprocal (hardware estimate and two Newton steps, a few ulps).
// Passes over the block: the start vector is generated inside the first forward pass, the
// back substitution accumulates max |y| and |y|^2, and the normalisation is
// applied inside the next pass (or the final store); rows move in chunks of
// IV_CH, loads of a chunk issued before its arithmetic.  Scratch: 4 arrays of
// [n][k] doubles, entry q of the thread's slot (its rank) at q * k + slot.
constexpr int IV_CH = 8;
template <typename T>
__global__ __launch_bounds__(64) void k_invit(const T *__restrict__ band, int64_t n,
                                              const double *__restrict__ bounds, const int32_t *__restrict__ blo,
                                              const int32_t *__restrict__ bhi, const double *__restrict__ mu,
                                              const int32_t *__restrict__ rank, int64_t k, double *__restrict__ scr,
                                              T *__restrict__ Z, int64_t ldz)
{
    const int64_t i = (int64_t)blockIdx.x * 64 + threadIdx.x;
    if (i >= n) return;
    const int64_t slot = rank[i];
    if (slot >= k) return;
    const int64_t lo = blo[i], hi = bhi[i], m = hi - lo;
    const double norm = fmax(fabs(bounds[0]), fabs(bounds[1]));
    const double ortol = 1e-9 * norm;
    if (i > lo && mu[i - 1] - mu[i] < ortol) return;  // inside a cluster: its first row does it
    const double si = norm > 0.0 ? 1.0 / norm : 1.0;
    const double tiny = DBL_EPSILON;
    const int64_t nk = n * k;
    double *u0 = scr + slot, *u1 = scr + nk + slot, *u2 = scr + 2 * nk + slot, *y = scr + 3 * nk + slot;
    const T *dg = band + lo * BW;  // d_q = dg[q BW], e_q = dg[(q + 1) BW + 1]
    auto D = [&](int64_t q) { return (double)dg[q * BW] * si; };
    auto E = [&](int64_t q) { return q + 1 < m ? (double)dg[(q + 1) * BW + 1] * si : 0.0; };
    auto floor_piv = [&](double x) { return fabs(x) < tiny ? (x < 0.0 ? -tiny : tiny) : x; };
    for (int64_t c = i;; ++c) {
        const int64_t rc = rank[c];
        const double sh = mu[c] * si;
        double scale = 1.0;  // y holds the iterate times 1 / scale
        bool fresh = true;   // the right-hand side is the start vector (not in y)
        int64_t seed = rc;
        for (int it = 0; it < 3; ++it) {
            // ---- forward: rows (cd, cu, 0 | cr) and (dl, nd, ndu | nr), the larger
            // of cd, dl pivots
            double cd = D(0) - sh, cu = E(0), cr = fresh ? start_entry(0, seed) : y[0] * scale;
            for (int64_t q0 = 0; q0 + 1 < m; q0 += IV_CH) {
                const int cnt = (int)min<int64_t>(IV_CH, m - 1 - q0);
                double ee[IV_CH + 1], dd[IV_CH], rr[IV_CH];
#pragma unroll
                for (int j = 0; j <= IV_CH; ++j) ee[j] = j <= cnt ? E(q0 + j) : 0.0;
#pragma unroll
                for (int j = 0; j < IV_CH; ++j) {
                    const int64_t q = q0 + j + 1;
                    dd[j] = j < cnt ? D(q) - sh : 0.0;
                    rr[j] = j < cnt ? (fresh ? start_entry(q, seed) : y[q * k] * scale) : 0.0;
                }
#pragma unroll
                for (int j = 0; j < IV_CH; ++j) {
                    if (j < cnt) {
                        const int64_t q = q0 + j;
                        const double dl = ee[j], nd = dd[j], ndu = ee[j + 1], nr = rr[j];
                        const bool sw = !(fabs(cd) >= fabs(dl));
                        const double p0 = sw ? dl : floor_piv(cd);
                        const double p1 = sw ? nd : cu, p2 = sw ? ndu : 0.0, pr = sw ? nr : cr;
                        const double f = (sw ? cd : dl) * recip64(p0);
                        u0[q * k] = p0;
                        u1[q * k] = p1;
                        u2[q * k] = p2;
                        y[q * k] = pr;
                        cd = (sw ? cu : nd) - f * p1;
                        cu = (sw ? 0.0 : ndu) - f * p2;
                        cr = (sw ? cr : nr) - f * pr;
                    }
                }
            }
            u0[(m - 1) * k] = floor_piv(cd);
            y[(m - 1) * k] = cr;
            // ---- back substitution, in place, with max |y| and |y|^2
            double z1 = 0.0, z2 = 0.0, amax = 0.0, ss = 0.0;
            for (int64_t qe = m; qe > 0; qe -= IV_CH) {
                const int cnt = (int)min<int64_t>(IV_CH, qe);
                double a0[IV_CH], a1[IV_CH], a2[IV_CH], yy[IV_CH];
#pragma unroll
                for (int j = 0; j < IV_CH; ++j) {
                    const int64_t q = qe - 1 - j;
                    const bool ok = j < cnt;
                    a0[j] = ok ? u0[q * k] : 1.0;
                    a1[j] = ok ? u1[q * k] : 0.0;
                    a2[j] = ok ? u2[q * k] : 0.0;
                    yy[j] = ok ? y[q * k] : 0.0;
                }
                double ra[IV_CH];  // the pivots' reciprocals, off the recurrence
#pragma unroll
                for (int j = 0; j < IV_CH; ++j) ra[j] = recip64(a0[j]);
#pragma unroll
                for (int j = 0; j < IV_CH; ++j) {
                    if (j < cnt) {
                        const double zq = (yy[j] - a1[j] * z1 - a2[j] * z2) * ra[j];
                        yy[j] = zq;
                        z2 = z1;
                        z1 = zq;
                        amax = fmax(amax, fabs(zq));
                        ss += zq * zq;
                    }
                }
#pragma unroll
                for (int j = 0; j < IV_CH; ++j)
                    if (j < cnt) y[(qe - 1 - j) * k] = yy[j];
            }
            fresh = false;
            if (!(amax <= DBL_MAX) || !(amax > 0.0) || ss != ss) {
                // overflow, a NaN or a zero solve: start again from another vector
                seed = rc + 7919 * (it + 1);
                ss = 0.0;
                for (int64_t q = 0; q < m; ++q) {
                    const double x = start_entry(q, seed);
                    y[q * k] = x;
                    ss += x * x;
                }
            } else if (!(ss <= DBL_MAX) || !(ss > 0.0)) {
                // |y|^2 out of range: scale by the largest entry first
                const double ia = 1.0 / amax;
                ss = 0.0;
                for (int64_t q = 0; q < m; ++q) {
                    const double x = y[q * k] * ia;
                    y[q * k] = x;
                    ss += x * x;
                }
            }
            scale = 1.0 / sqrt(ss);
            if (c > i) {
                // a later member of a cluster: normalise, then against the cluster's
                // earlier vectors (already in Z), then normalise again
                for (int64_t q = 0; q < m; ++q) y[q * k] *= scale;
                for (int64_t p = i; p < c; ++p) {
                    const T *zp = Z + lo * ldz + rank[p];
                    double dp = 0.0;
                    for (int64_t q = 0; q < m; ++q) dp += y[q * k] * (double)zp[q * ldz];
                    for (int64_t q = 0; q < m; ++q) y[q * k] -= dp * (double)zp[q * ldz];
                }
                double s2 = 0.0;
                for (int64_t q = 0; q < m; ++q) s2 += y[q * k] * y[q * k];
                scale = s2 > 0.0 ? 1.0 / sqrt(s2) : 0.0;
            }
        }
        for (int64_t q = 0; q < m; ++q) Z[(lo + q) * ldz + rc] = (T)(y[q * k] * scale);
        if (!(c + 1 < hi && mu[c] - mu[c + 1] < ortol && rank[c + 1] < k)) break;
    }
}

// Z <- H_1 ... H_M Z for the kept bulge reflectors.  Reflector (s, k) acts on
// rows s + 1 + 32 k .. s + 32 + 32 k; two reflectors that share a row must be
// applied last-created first, and (s, k) shares rows only with (s - d, k + j)
// for 32 (j - 1) < d < 32 (j + 1), j >= 0.  So the order "k ascending, s
// descending within k" is valid: pass k slides a 32-row window up one row per
// reflector.  Lane = column of Z (64 per workgroup), the window in registers
// (row r in slot r mod 32, bodies of 32 steps aligned so the slots are
// compile-time), no cross-lane work.  The WV waves of a workgroup run passes
// k = w, w + WV, ... as a pipeline: pass k takes each row after pass k - 1 has
// released it (a row leaves a window at its bottom); rows move through Z
// itself (coherent loads and stores, as in the bulge chase), progress through
// one LDS counter per wave (pass k at PS k + (BASE - lowest step done)).  A
// pass runs virtual steps above its first reflector and below s = 0 (no
// reflector) so that its rows enter and leave at the same pace.  Waits are
// bounded: on time-out the error flag is set and the workgroup leaves.
constexpr int BTB_PS = 16384;  // progress stride per pass (> steps per pass)
template <typename T>
struct BtBulgeCfg {
    static constexpr int WV = sizeof(T) == 4 ? 8 : 4;  // passes in flight per workgroup
};
template <typename T>
__global__ __launch_bounds__(64 * BtBulgeCfg<T>::WV) void k_bt_bulge(const T *__restrict__ refl, int64_t n,
                                                                     int64_t k, T *__restrict__ Z, int64_t ldz,
                                                                     uint64_t spin_ticks, int32_t *__restrict__ err)
{
    constexpr int WV = BtBulgeCfg<T>::WV;
    constexpr int PER = (NB * RFL + 63) / 64;  // reflector entries per lane per body
    constexpr uint32_t OOB = 0x7FFFFFFFu;      // a row offset past every record
    __shared__ int32_t prog[WV];
    __shared__ int32_t quit;
    __shared__ T rs[WV][NB * RFL];  // the body's 32 reflectors, per wave
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t col = (int64_t)blockIdx.x * 64 + lane;
    const int nn = (int)n;
    const int nsw = nn - 2;
    const int KK = nsw / NB;        // passes 0 .. KK
    const int BASE = nn + 2 * NB;   // BASE - s > 0 for every step s >= -32
    // Z and the reflectors through buffer resources with 32-bit offsets (the
    // caller guarantees (n + 64) ldz sizeof(T) < 2^31): a row past n, or a
    // column past k (offset 2^31), is out of range, so its load reads 0 and its
    // store is dropped; Z moves with the coherent policy of the bulge chase
    const uint32_t ldzb = (uint32_t)ldz * (uint32_t)sizeof(T);
    const __amdgpu_buffer_rsrc_t rz = __builtin_amdgcn_make_buffer_rsrc(Z, 0, (int)(ldzb * (uint32_t)nn), 0x00020000);
    const int nrefl = refl_index(n, nsw);
    const __amdgpu_buffer_rsrc_t rr =
        __builtin_amdgcn_make_buffer_rsrc((void *)refl, 0, (int)((uint32_t)nrefl * RFL * sizeof(T)), 0x00020000);
    const uint32_t vcol = col < k ? (uint32_t)col * (uint32_t)sizeof(T) : 0x80000000u;
    if (threadIdx.x < WV) prog[threadIdx.x] = (int32_t)threadIdx.x * BTB_PS;
    if (threadIdx.x == 0) quit = 0;
    __syncthreads();
    T *rw = rs[wv];
    // the 32 reflectors of body sb (steps s = sb - u) of pass kk: lane-strided
    // loads of their (v, tau) records (0 for steps without a reflector)
    auto fetch = [&](int kk, int sb, int shi, T (&pre)[PER]) {
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int e = lane + 64 * j;
            const int u = e / RFL, q = e % RFL;
            const int sr = sb - u;
            const bool ok = e < NB * RFL && sr >= 0 && sr <= shi;
            const uint32_t off = ok ? ((uint32_t)(refl_index(n, sr) + kk) * RFL + q) * (uint32_t)sizeof(T) : OOB;
            pre[j] = band_load<T>(rr, (int)off, 0);
        }
    };
    auto park = [&](const T (&pre)[PER]) {
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int e = lane + 64 * j;
            if (e < NB * RFL) rw[e] = pre[j];
        }
    };
    for (int kk = wv; kk <= KK; kk += WV) {
        const int shi = kk == 0 ? nsw - 1 : nsw - NB * kk;  // the pass's first reflector
        const int rlo = 1 + NB * kk;                        // rows the pass touches: rlo .. n - 1
        // bodies start at sb with sb + 1 = 0 mod 32, the first at or above shi + 31
        const int sb0 = ((shi + 31 + 1 + NB - 1) / NB) * NB - 1;
        const int pneed_base = (kk - 1) * BTB_PS + BASE;  // + (-(s_done)) of pass kk - 1
        T z[NB];
#pragma unroll
        for (int q = 0; q < NB; ++q) z[q] = (T)0;
        T pre[PER];
        fetch(kk, sb0, shi, pre);
        for (int sb = sb0; sb >= -NB; sb -= NB) {
            // rows entering at steps u = 0..31: r = sb + 1 - u + 32 kk.  Pass kk - 1
            // stores the bottom row s + 32 kk of its step s at its next step, so
            // once it has published steps down to s_d, rows >= s_d + 1 + 32 kk
            // are in Z.
            const int top = sb + 1 + NB * kk;  // row entering at u = 0
            const int rmin = max(top - (NB - 1), rlo), rmax = min(top, nn - 1);
            if (kk > 0 && rmin <= rmax) {
                const int s_need = rmin - 1 - NB * kk;
                const int32_t need = pneed_base - s_need;
                const int pw = (wv + WV - 1) % WV;
                if (__hip_atomic_load(&prog[pw], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) < need) {
                    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
                    while (__hip_atomic_load(&prog[pw], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) < need) {
                        if (__hip_atomic_load(&quit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) != 0 ||
                            __builtin_amdgcn_s_memrealtime() - t0 > spin_ticks) {
                            __hip_atomic_store(&quit, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                            if (lane == 0) cstore(err, 1);
                            return;
                        }
                        __builtin_amdgcn_s_sleep(1);
                    }
                }
            }
            // row offsets: rows below the pass's range map past every record
            // (rows past n are past it anyway)
            auto roff = [&](int r) { return r >= rlo ? (uint32_t)r * ldzb : OOB; };
            T ent[NB];
#pragma unroll
            for (int u = 0; u < NB; ++u) ent[u] = band_load<T>(rz, (int)(vcol + roff(top - u)), 0);
            wave_sync();
            park(pre);
            wave_sync();
            if (sb - NB >= -NB) fetch(kk, sb - NB, shi, pre);  // the next body's reflectors, in flight
#pragma unroll
            for (int u = 0; u < NB; ++u) {
                // release the bottom row of the previous step (slot of the entering row)
                const int slot = (NB - u) & (NB - 1);
                band_store<T>(rz, z[slot], (int)(vcol + roff(top - u + NB)), 0);
                z[slot] = ent[u];
                const T tau = rw[u * RFL + NB];
                if (tau != (T)0) {  // uniform: one reflector per step
                    T d0 = 0, d1 = 0, d2 = 0, d3 = 0;
#pragma unroll
                    for (int q = 0; q < NB; q += 4) {
                        d0 += rw[u * RFL + q] * z[(q - u) & (NB - 1)];
                        d1 += rw[u * RFL + q + 1] * z[(q + 1 - u) & (NB - 1)];
                        d2 += rw[u * RFL + q + 2] * z[(q + 2 - u) & (NB - 1)];
                        d3 += rw[u * RFL + q + 3] * z[(q + 3 - u) & (NB - 1)];
                    }
                    const T td = tau * ((d0 + d1) + (d2 + d3));
#pragma unroll
                    for (int q = 0; q < NB; ++q) z[(q - u) & (NB - 1)] -= td * rw[u * RFL + q];
                }
            }
            // publish: this body's rows are stored, steps down to sb - 31 done
            __builtin_amdgcn_s_waitcnt(0);
            if (lane == 0)
                __hip_atomic_store(&prog[wv], kk * BTB_PS + BASE - (sb - (NB - 1)), __ATOMIC_RELEASE,
                                   __HIP_MEMORY_SCOPE_WORKGROUP);
        }
    }
}

// Z[r0:, :] <- (I - V T V^T) Z[r0:, :] for a kept panel (V in A's panel
// block P: m rows, unit lower with the strict part stored; T in Tk, as the
// reduction applied it), in three kernels over the whole grid:
//   Wp[c] = V[rows of chunk c]^T Z[rows of chunk c]   (BTP_RC-row chunks)
//   Y = T sum_c Wp[c]
//   Z -= V Y                                           (64 x 64 tiles)
constexpr int BTP_RC = 128;  // rows per partial
template <typename T>
__device__ __forceinline__ T panel_v(const T *__restrict__ P, int64_t lda, int64_t i, int a)
{
    return i == a ? (T)1 : (i > a ? P[i * lda + a] : (T)0);
}

template <typename T>
__global__ __launch_bounds__(256) void k_btp_w(const T *__restrict__ P, int64_t lda, int m,
                                               const T *__restrict__ Zr, int64_t ldz, int64_t k,
                                               T *__restrict__ Wp)
{
    constexpr int LV = NB + 1, LZ = 64 + 4;
    __shared__ T Vs[BTP_RC * LV], Zs[BTP_RC * LZ];
    const int tid = threadIdx.x;
    const int64_t cb = (int64_t)blockIdx.x * 64;
    const int64_t r0 = (int64_t)blockIdx.y * BTP_RC;
    for (int p = tid; p < BTP_RC * NB; p += 256) {
        const int rr = p / NB, a = p % NB;
        const int64_t i = r0 + rr;
        Vs[rr * LV + a] = i < m ? panel_v(P, lda, i, a) : (T)0;
    }
    for (int p = tid; p < BTP_RC * 64; p += 256) {
        const int rr = p / 64, c = p % 64;
        const int64_t i = r0 + rr;
        Zs[rr * LZ + c] = i < m && cb + c < k ? Zr[i * ldz + cb + c] : (T)0;
    }
    __syncthreads();
    const int a = tid / 8, c8 = (tid % 8) * 8;
    T acc[8] = {};
    for (int rr = 0; rr < BTP_RC; ++rr) {
        const T va = Vs[rr * LV + a];
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] += va * Zs[rr * LZ + c8 + j];
    }
    T *out = Wp + ((int64_t)blockIdx.y * NB + a) * k + cb + c8;
#pragma unroll
    for (int j = 0; j < 8; ++j)
        if (cb + c8 + j < k) out[j] = acc[j];
}

template <typename T>
__global__ __launch_bounds__(256) void k_btp_y(const T *__restrict__ Wp, int nch, const T *__restrict__ Tk,
                                               int64_t k, T *__restrict__ Y)
{
    constexpr int L = 64 + 4;
    __shared__ T Ts[NB * (NB + 1)], Ws[NB * L];
    const int tid = threadIdx.x;
    for (int p = tid; p < NB * NB; p += 256) Ts[(p / NB) * (NB + 1) + p % NB] = Tk[p];
    const int64_t cb = (int64_t)blockIdx.x * 64;
    const int a = tid / 8, c8 = (tid % 8) * 8;
    // W[a][c8 .. c8 + 7] = sum over the row chunks
    T w[8] = {};
#pragma unroll 2
    for (int ch = 0; ch < nch; ++ch) {
        const T *src = Wp + ((int64_t)ch * NB + a) * k + cb + c8;
#pragma unroll
        for (int j = 0; j < 8; ++j) w[j] += cb + c8 + j < k ? src[j] : (T)0;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) Ws[a * L + c8 + j] = w[j];
    __syncthreads();
    T y[8] = {};
#pragma unroll 4
    for (int l = 0; l < NB; ++l) {
        const T t = Ts[a * (NB + 1) + l];
#pragma unroll
        for (int j = 0; j < 8; ++j) y[j] += t * Ws[l * L + c8 + j];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j)
        if (cb + c8 + j < k) Y[(int64_t)a * k + cb + c8 + j] = y[j];
}

template <typename T>
__global__ __launch_bounds__(256) void k_btp_u(const T *__restrict__ P, int64_t lda, int m,
                                               const T *__restrict__ Y, int64_t k, T *__restrict__ Zr,
                                               int64_t ldz)
{
    constexpr int LV = NB + 1, LY = 64 + 4;
    __shared__ T Vs[64 * LV], Ys[NB * LY];
    const int tid = threadIdx.x;
    const int64_t r0 = (int64_t)blockIdx.x * 64, cb = (int64_t)blockIdx.y * 64;
    for (int p = tid; p < 64 * NB; p += 256) {
        const int rr = p / NB, a = p % NB;
        const int64_t i = r0 + rr;
        Vs[rr * LV + a] = i < m ? panel_v(P, lda, i, a) : (T)0;
    }
    for (int p = tid; p < NB * 64; p += 256) {
        const int a = p / 64, c = p % 64;
        Ys[a * LY + c] = cb + c < k ? Y[(int64_t)a * k + cb + c] : (T)0;
    }
    __syncthreads();
    const int tr = (tid / 16) * 4, tc = (tid % 16) * 4;
    T acc[4][4] = {};
#pragma unroll 8
    for (int a = 0; a < NB; ++a) {
        T v[4], y[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = Vs[(tr + i) * LV + a];
#pragma unroll
        for (int j = 0; j < 4; ++j) y[j] = Ys[a * LY + tc + j];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] += v[i] * y[j];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t r = r0 + tr + i;
        if (r >= m) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (cb + tc + j < k) Zr[r * ldz + cb + tc + j] -= acc[i][j];
    }
}

// ---------------------------------------------------------------- host side

inline int64_t cdiv_h(int64_t a, int64_t b) { return (a + b - 1) / b; }

struct Ws {
    size_t off = 0;
    char *base = nullptr;
    template <typename U>
    U *take(size_t count)
    {
        U *p = (U *)(base + off);
        off += (count * sizeof(U) + 255) / 256 * 256;
        return p;
    }
};

template <typename T>
struct Bufs {
    T *band, *V, *V2, *W, *X, *Xpart, *Q1, *Vloc, *Tloc, *Rstack, *Rf, *Vtop, *Ttop, *Ktop, *U, *Tm, *Ppart;
    int32_t *prog, *cqf;
    double *dd, *ee2, *bounds, *Qd, *Gp, *R1, *Rinv;
    float2 *de32;
    float *sgx;    // multisection grid of the eigenvalue search: points (fp32
    double *sgxd;  // or fp64) and their Sturm counts
    int32_t *sgc;
};

constexpr int KS_MAX = 16;

template <typename T>
size_t layout(int64_t n, char *base, Bufs<T> &b)
{
    Ws ws;
    ws.base = base;
    b.band = ws.take<T>((size_t)n * BW);
    b.prog = ws.take<int32_t>((size_t)n + 1);
    b.V = ws.take<T>((size_t)n * NB);
    b.V2 = ws.take<T>((size_t)n * NB);
    b.W = ws.take<T>((size_t)n * NB);
    b.X = ws.take<T>((size_t)n * NB);
    b.Xpart = ws.take<T>((size_t)KS_MAX * n * NB);
    b.Q1 = ws.take<T>((size_t)n * NB);
    b.Vloc = ws.take<T>((size_t)n * NB);
    b.Tloc = ws.take<T>((size_t)32 * NB * NB);
    b.Rstack = ws.take<T>((size_t)32 * NB * NB);
    b.Rf = ws.take<T>((size_t)NB * NB);
    b.Vtop = ws.take<T>((size_t)32 * NB * NB);
    b.Ttop = ws.take<T>((size_t)NB * NB);
    b.Ktop = ws.take<T>((size_t)NB * NB);
    b.U = ws.take<T>((size_t)NB * NB);
    b.Tm = ws.take<T>((size_t)NB * NB);
    b.Ppart = ws.take<T>((size_t)cdiv_h(n, XR) * NB * NB);
    b.dd = ws.take<double>((size_t)n);
    b.ee2 = ws.take<double>((size_t)n);
    b.bounds = ws.take<double>(4);
    b.de32 = ws.take<float2>((size_t)n);
    b.sgx = ws.take<float>((size_t)SG_P);
    b.sgxd = ws.take<double>((size_t)SG_P);
    b.sgc = ws.take<int32_t>((size_t)SG_P);
    b.Qd = ws.take<double>((size_t)n * NB);
    b.Gp = ws.take<double>((size_t)cdiv_h(n, CQ_ROWS) * NB * NB);
    b.R1 = ws.take<double>((size_t)NB * NB);
    b.Rinv = ws.take<double>((size_t)NB * NB);
    b.cqf = ws.take<int32_t>(1);
    return ws.off;
}

// Trailing sizes from which the next panel is factored beside the trailing
// update: below it the update is shorter than the extra block-column kernel
// and the two stream handoffs cost (measured at n = 4096: 39.2 -> 41.8 ms with
// the look-ahead on every panel).
constexpr int64_t LOOKAHEAD_MIN = 6144;

// The helper stream of stage 1 (one per caller stream and device, default
// priority, created on first use) and the two events that order it with the
// caller's stream.  Solves on different caller streams get different helpers,
// so their panel factorisations overlap instead of queueing on one stream.
struct Aux {
    hipStream_t key = nullptr;  // the caller's stream
    int dev = -1;
    hipStream_t s = nullptr;    // nullptr: free slot
    hipEvent_t fork = nullptr, join = nullptr;
    std::mutex mu;
};
constexpr int AUX_SLOTS = 64;
Aux aux_tab[AUX_SLOTS];
std::mutex aux_init_mu;

hipError_t aux_for(hipStream_t st, Aux **out)
{
    hipDevice_t dev = 0;
    hipError_t e = hipStreamGetDevice(st, &dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> g(aux_init_mu);
    Aux *fallback = nullptr;
    for (Aux &a : aux_tab) {
        if (a.s != nullptr && a.dev == dev) {
            if (a.key == st) {
                *out = &a;
                return hipSuccess;
            }
            if (fallback == nullptr) fallback = &a;
        }
    }
    Aux *slot = nullptr;
    for (Aux &a : aux_tab)
        if (a.s == nullptr) {
            slot = &a;
            break;
        }
    if (slot == nullptr) {  // table full: share a helper of this device (its calls then queue on it)
        if (fallback == nullptr) return hipErrorOutOfMemory;
        *out = fallback;
        return hipSuccess;
    }
    int cur = 0;
    if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    hipStream_t s = nullptr;
    hipEvent_t f = nullptr, j = nullptr;
    e = hipStreamCreateWithFlags(&s, hipStreamNonBlocking);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&f, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&j, hipEventDisableTiming);
    if (cur != dev) {
        hipError_t e2 = hipSetDevice(cur);
        if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    slot->key = st;
    slot->dev = dev;
    slot->fork = f;
    slot->join = j;
    slot->s = s;
    *out = slot;
    return hipSuccess;
}

#define LAUNCH_OK()                                     \
    do {                                                \
        hipError_t e_ = hipGetLastError();              \
        if (e_ != hipSuccess) return e_;                \
    } while (0)

// What the eigenvector path adds to a solve: the k columns of Z (n x k,
// row-major, column j for the j-th largest eigenvalue) and the workspace it
// keeps the reduction in.
template <typename T>
struct VecReq {
    T *Z;
    int64_t ldz, k;
    T *refl, *keepT;          // bulge reflectors (refl_index layout), panel T factors
    int32_t *blo, *bhi, *rk;  // each row's block of the tridiagonal, the rank of its eigenvalue
    double *mu, *scr;         // per-block eigenvalues (fp64), inverse-iteration scratch
    T *wp, *yb;               // panel back-transformation: partial V^T Z per row chunk, Y = T V^T Z
};

template <typename T>
hipError_t run(hipStream_t st, T *A, int64_t n, int64_t lda, T *w, void *ws, int32_t *info,
               const VecReq<T> *vec = nullptr)
{
    Bufs<T> b;
    layout<T>(n, (char *)ws, b);
    constexpr int RB = Cfg<T>::RB;
    constexpr int TOP_BLOCKS = RB / NB;  // stacked R rows (<= 1024 f32, 512 f64) fit one workgroup's registers
    constexpr int DIRECT_ROWS = 256;
    static_assert(DIRECT_ROWS <= RB, "direct panel must fit");
    // ---- stage 1: dense -> band
    // For trailing sizes of at least LOOKAHEAD_MIN, panel p's trailing update is
    // split: the next panel's block column (NB columns, all rows) first, then
    // the rest of the trailing matrix; the next panel is factored on a helper
    // stream while the main stream runs that rest, and the main stream waits
    // for it before the next SYMM.  The two touch disjoint parts of A; V
    // alternates between two buffers (the running SYR2K reads panel p's V
    // while panel p + 1's is written).  Smaller panels run in order.
    Aux *aux = nullptr;
    hipError_t ae = aux_for(st, &aux);
    if (ae != hipSuccess) return ae;
    std::lock_guard<std::mutex> aux_lock(aux->mu);  // one call at a time on the helper stream and its events
    T *Vbuf[2] = {b.V, b.V2};
    // factorisation of the panel at column c0 on stream s: V (into Vout), T, W = V T, R into A
    auto factor = [&](hipStream_t s, int64_t c0, T *Vout) -> hipError_t {
        const int64_t r0 = c0 + NB;
        const int64_t m = n - r0;
        T *P = A + r0 * lda + c0;
        KTimer kt_panel(s, SPEC_KT_PANEL);
            if (m <= DIRECT_ROWS) {
                hipLaunchKernelGGL(k_panel_direct<T>, dim3(1), dim3(256), 0, s, P, lda, (int)m, Vout, b.Tm);
                LAUNCH_OK();
            } else {
                // CholeskyQR2 into Q1 and Rf; the TSQR below runs only if it breaks down
                const int ng = (int)cdiv_h(m, CQ_ROWS), na = (int)cdiv_h(m, CQ_AROWS);
                hipLaunchKernelGGL(k_cqr_gram<T>, dim3(ng), dim3(256), 0, s, (const T *)P, lda, (int)m, b.Gp,
                                   (const int *)nullptr);
                LAUNCH_OK();
                hipLaunchKernelGGL(k_cqr_chol<T>, dim3(1), dim3(CH_T), 0, s, b.Gp, ng, false, b.R1, b.Rinv, b.Rf,
                                   b.cqf);
                LAUNCH_OK();
                hipLaunchKernelGGL((k_cqr_apply<T, T>), dim3(na), dim3(256), 0, s, (const T *)P, lda, (int)m,
                                   b.Rinv, false, b.Q1, b.Qd, b.cqf);
                LAUNCH_OK();
                hipLaunchKernelGGL(k_cqr_gram<double>, dim3(ng), dim3(256), 0, s, (const double *)b.Qd, (int64_t)NB,
                                   (int)m, b.Gp, b.cqf);
                LAUNCH_OK();
                hipLaunchKernelGGL(k_cqr_chol<T>, dim3(1), dim3(CH_T), 0, s, b.Gp, ng, true, b.R1, b.Rinv, b.Rf,
                                   b.cqf);
                LAUNCH_OK();
                hipLaunchKernelGGL((k_cqr_apply<double, T>), dim3(na), dim3(256), 0, s, (const double *)b.Qd,
                                   (int64_t)NB, (int)m, b.Rinv, true, b.Q1, b.Qd, b.cqf);
                LAUNCH_OK();
                // row blocks of about 256 rows, at most TOP_BLOCKS of them (the stacked R
                // factors of all blocks are factored by one workgroup)
                const int nblk = (int)std::min<int64_t>(TOP_BLOCKS, cdiv_h(m, 256));
                const int per = (int)cdiv_h(m, nblk);
                const int rows_top = nblk * NB;
                // fp32: QRs with four rows per lane (one wave up to 256 rows, two up to 512,
                // four up to 1024); fp64: one row per thread
                if constexpr (std::is_same<T, float>::value) {
                    if (per <= 256)
                        hipLaunchKernelGGL((k_tsqr_wave<T, 1>), dim3(nblk), dim3(64), 0, s, P, lda, (int)m, per, b.Vloc,
                                           b.Tloc, b.Rstack, (T *)nullptr, (const int *)b.cqf);
                    else if (per <= 512)
                        hipLaunchKernelGGL((k_tsqr_wave<T, 2>), dim3(nblk), dim3(128), 0, s, P, lda, (int)m, per,
                                           b.Vloc, b.Tloc, b.Rstack, (T *)nullptr, (const int *)b.cqf);
                    else
                        hipLaunchKernelGGL((k_tsqr_wave<T, 4>), dim3(nblk), dim3(256), 0, s, P, lda, (int)m, per,
                                           b.Vloc, b.Tloc, b.Rstack, (T *)nullptr, (const int *)b.cqf);
                    LAUNCH_OK();
                    if (rows_top <= 256)
                        hipLaunchKernelGGL((k_tsqr_wave<T, 1>), dim3(1), dim3(64), 0, s, b.Rstack, (int64_t)NB, rows_top,
                                           rows_top, b.Vtop, b.Ttop, b.Rf, b.Ktop, (const int *)b.cqf);
                    else if (rows_top <= 512)
                        hipLaunchKernelGGL((k_tsqr_wave<T, 2>), dim3(1), dim3(128), 0, s, b.Rstack, (int64_t)NB,
                                           rows_top, rows_top, b.Vtop, b.Ttop, b.Rf, b.Ktop, (const int *)b.cqf);
                    else
                        hipLaunchKernelGGL((k_tsqr_wave<T, 4>), dim3(1), dim3(256), 0, s, b.Rstack, (int64_t)NB,
                                           rows_top, rows_top, b.Vtop, b.Ttop, b.Rf, b.Ktop, (const int *)b.cqf);
                    LAUNCH_OK();
                } else {
                    if (per <= 256)
                        hipLaunchKernelGGL((k_tsqr_local<T, 256>), dim3(nblk), dim3(256), 0, s, P, lda, (int)m, per,
                                           b.Vloc, b.Tloc, b.Rstack, (const int *)b.cqf);
                    else if (per <= 512)
                        hipLaunchKernelGGL((k_tsqr_local<T, 512>), dim3(nblk), dim3(512), 0, s, P, lda, (int)m, per,
                                           b.Vloc, b.Tloc, b.Rstack, (const int *)b.cqf);
                    else
                        hipLaunchKernelGGL((k_tsqr_local<T, 1024>), dim3(nblk), dim3(1024), 0, s, P, lda, (int)m, per,
                                           b.Vloc, b.Tloc, b.Rstack, (const int *)b.cqf);
                    LAUNCH_OK();
                    if (rows_top <= 256)
                        hipLaunchKernelGGL((k_tsqr_top<T, 256>), dim3(1), dim3(256), 0, s, b.Rstack, nblk, b.Rf, b.Vtop,
                                           b.Ktop, (const int *)b.cqf);
                    else if (rows_top <= 512)
                        hipLaunchKernelGGL((k_tsqr_top<T, 512>), dim3(1), dim3(512), 0, s, b.Rstack, nblk, b.Rf, b.Vtop,
                                           b.Ktop, (const int *)b.cqf);
                    else
                        hipLaunchKernelGGL((k_tsqr_top<T, 1024>), dim3(1), dim3(1024), 0, s, b.Rstack, nblk, b.Rf,
                                           b.Vtop, b.Ktop, (const int *)b.cqf);
                    LAUNCH_OK();
                }
                hipLaunchKernelGGL(k_tsqr_q1<T>, dim3((unsigned)cdiv_h(per, 8), nblk), dim3(256), 0, s, b.Vloc, b.Tloc,
                                   b.Vtop, b.Ktop, (int)m, per, b.Q1, (const int *)b.cqf);
                LAUNCH_OK();
                hipLaunchKernelGGL(k_tsqr_recon<T>, dim3(1), dim3(64), 0, s, b.Q1, b.Rf, P, lda, Vout, b.U, b.Tm);
                LAUNCH_OK();
            }
            // V rows below the reconstructed top block (TSQR), then W = V T
            hipLaunchKernelGGL(k_vw<T>, dim3((unsigned)cdiv_h(m, VW_R)), dim3(VW_T), 0, s, b.Q1, b.U, b.Tm, (int)m,
                               m <= DIRECT_ROWS ? (int)m : NB, Vout, b.W);
            LAUNCH_OK();
            if (vec != nullptr) {  // the panel's V below the band and its T, for the eigenvectors
                hipLaunchKernelGGL(k_keep_panel<T>, dim3((unsigned)cdiv_h(m * NB, 256)), dim3(256), 0, s, Vout, b.Tm,
                                   (int)m, P, lda, vec->keepT + (c0 / NB) * NB * NB);
                LAUNCH_OK();
            }
        return hipSuccess;
    };
    if (n - NB >= 2) {
        hipError_t e = factor(st, 0, Vbuf[0]);
        if (e != hipSuccess) return e;
    }
    for (int64_t c0 = 0;; c0 += NB) {
        const int64_t r0 = c0 + NB;
        const int64_t m = n - r0;
        if (m < 2) break;
        T *A22 = A + r0 * lda + r0;
        T *Vc = Vbuf[(c0 / NB) & 1];
        const int nrb = (int)cdiv_h(m, SY_RB);
        // column chunks per row block: fp32, about three workgroups per CU (the
        // kernel's occupancy) without a partial round; fp64, about 512 workgroups
        // and at most 8 chunks
        int ks = std::is_same<T, float>::value ? (int)std::min<int64_t>(KS_MAX, std::max<int64_t>(1, 768 / nrb))
                                               : (int)std::min<int64_t>(8, std::max<int64_t>(1, cdiv_h(512, nrb)));
        int chunk = (int)(cdiv_h(cdiv_h(m, ks), SY_JB) * SY_JB);
        ks = (int)cdiv_h(m, chunk);
        {
            KTimer kt(st, SPEC_KT_SYMM);
            if constexpr (std::is_same<T, float>::value)
                hipLaunchKernelGGL(k_symm_f32, dim3(nrb, ks), dim3(256), 0, st, A22, lda, (int)m, b.W, b.Xpart,
                                   chunk);
            else
                hipLaunchKernelGGL(k_symm<T>, dim3(nrb, ks), dim3(256), 0, st, A22, lda, (int)m, b.W, b.Xpart,
                                   chunk);
        }
        LAUNCH_OK();
        const int nxb = (int)cdiv_h(m, XR);
        {
            KTimer kt(st, SPEC_KT_PANEL);
            hipLaunchKernelGGL(k_xreduce<T>, dim3(nxb), dim3(256), 0, st, b.Xpart, ks, (int)m, Vc, b.X, b.Ppart);
            hipLaunchKernelGGL(k_mz<T>, dim3((unsigned)std::min<int64_t>(MZ_BLOCKS, cdiv_h(m, 8))), dim3(256), 0, st,
                               b.Ppart, nxb, b.Tm, b.X, Vc, (int)m);
        }
        LAUNCH_OK();
        if (m - NB >= LOOKAHEAD_MIN) {
            // the next panel's block column, then its factorisation beside the rest
            {
                KTimer kt(st, SPEC_KT_SYR2K);
                hipLaunchKernelGGL(k_syr2k_cols<T>, dim3((unsigned)cdiv_h(m, SC_ROWS)), dim3(256), 0, st, A22, lda,
                                   (int)m, Vc, b.X);
            }
            LAUNCH_OK();
            if ((ae = hipEventRecord(aux->fork, st)) != hipSuccess) return ae;
            if ((ae = hipStreamWaitEvent(aux->s, aux->fork, 0)) != hipSuccess) return ae;
            if ((ae = factor(aux->s, c0 + NB, Vbuf[(c0 / NB + 1) & 1])) != hipSuccess) return ae;
            if ((ae = hipEventRecord(aux->join, aux->s)) != hipSuccess) return ae;
            const int64_t mr = m - NB;
            const int64_t nt = cdiv_h(mr, S2_T);
            {
                KTimer kt(st, SPEC_KT_SYR2K);
                hipLaunchKernelGGL(k_syr2k<T>, dim3((unsigned)(nt * (nt + 1) / 2)), dim3(256), 0, st,
                                   A22 + NB * lda + NB, lda, (int)mr, Vc + NB * NB, b.X + NB * NB);
            }
            LAUNCH_OK();
            if ((ae = hipStreamWaitEvent(st, aux->join, 0)) != hipSuccess) return ae;
        } else {
            const int64_t nt = cdiv_h(m, S2_T);
            {
                KTimer kt(st, SPEC_KT_SYR2K);
                hipLaunchKernelGGL(k_syr2k<T>, dim3((unsigned)(nt * (nt + 1) / 2)), dim3(256), 0, st, A22, lda,
                                   (int)m, Vc, b.X);
            }
            LAUNCH_OK();
            if (m - NB >= 2) {  // the next panel in order on the caller's stream
                hipError_t e = factor(st, c0 + NB, Vbuf[(c0 / NB + 1) & 1]);
                if (e != hipSuccess) return e;
            }
        }
    }
    // ---- stage 2: band -> tridiagonal
    hipLaunchKernelGGL(k_band_copy<T>, dim3((unsigned)cdiv_h(n * BW + 1, 256)), dim3(256), 0, st, A, lda, n, b.band,
                       b.prog);
    LAUNCH_OK();
    if (n >= 3) {
        // G sweeps per workgroup (one wave each); the LDS ring holds >= (2G + 1) NB rows
        constexpr int G = sizeof(T) == 4 ? 4 : 3;
        constexpr int CAPR = sizeof(T) == 4 ? 288 : 256;
        const int64_t nsw = n - 2;
        const int64_t ngroups = cdiv_h(nsw, G);
        // about n / (2 G NB) groups are active at once (a group lives for the
        // ~n / NB steps of its lead sweep, groups start 2 G steps apart): a
        // persistent grid of that many plus a margin keeps the other CUs free
        const int64_t nwg = std::min<int64_t>(ngroups, n / (2 * G * NB) * 5 / 4 + 16);
        const uint64_t spin_ticks = 100000000ull * 10;  // 10 s at the 100 MHz real-time counter
        {
            KTimer kt(st, SPEC_KT_BULGE);
            hipLaunchKernelGGL((k_bulge<T, G, CAPR>), dim3((unsigned)nwg), dim3(64 * (G + 2)), 0, st, b.band, n,
                               b.prog, spin_ticks, vec != nullptr ? vec->refl : (T *)nullptr);
        }
        LAUNCH_OK();
    }
    // ---- stage 3: eigenvalues of the tridiagonal
    {
    KTimer kt_s3(st, SPEC_KT_TRIDIAG);
    hipLaunchKernelGGL(k_tridiag_prep<T>, dim3(1), dim3(256), 0, st, b.band, n, b.dd, b.ee2, b.bounds,
                       sizeof(T) == 4 ? b.de32 : nullptr);
    LAUNCH_OK();
    if constexpr (sizeof(T) == 4) {
        const bool grid = n >= SG_MIN_N;
        if (grid) {
            hipLaunchKernelGGL(k_sturm_grid_f32, dim3(SG_P / 64), dim3(64), 0, st, b.de32, (int)n, b.bounds, b.sgx,
                               b.sgc);
            LAUNCH_OK();
        }
        hipLaunchKernelGGL(k_bisect_f32, dim3((unsigned)cdiv_h(n, 4)), dim3(64), 0, st, b.de32, (int)n, b.bounds,
                           grid ? b.sgx : nullptr, grid ? b.sgc : nullptr, w);
    } else {
        const bool grid = n >= SG_MIN_N;
        if (grid) {
            hipLaunchKernelGGL(k_sturm_grid, dim3(SG_P / 64), dim3(64), 0, st, b.dd, b.ee2, n, b.bounds, b.sgxd,
                               b.sgc);
            LAUNCH_OK();
        }
        hipLaunchKernelGGL(k_bisect<T>, dim3((unsigned)cdiv_h(n, 4)), dim3(64), 0, st, b.dd, b.ee2, n, b.bounds,
                           4e-16, grid ? b.sgxd : nullptr, grid ? b.sgc : nullptr, w);
    }
    }
    LAUNCH_OK();
    if (vec != nullptr) {
        // ---- eigenvectors: the tridiagonal's blocks and their fp64 eigenvalues,
        // inverse iteration, then back through the bulge reflectors and the panels
        const double thr = sizeof(T) == 4 ? (double)FLT_EPSILON : DBL_EPSILON;
        hipLaunchKernelGGL(k_vsplit<T>, dim3(1), dim3(1024), 0, st, b.band, n, b.bounds, thr, vec->blo, vec->bhi);
        LAUNCH_OK();
        hipLaunchKernelGGL(k_vbisect, dim3((unsigned)cdiv_h(n, 4)), dim3(64), 0, st, b.dd, b.ee2, n, b.bounds,
                           vec->blo, vec->bhi, vec->mu);
        LAUNCH_OK();
        hipLaunchKernelGGL(k_vrank, dim3((unsigned)cdiv_h(n, 256)), dim3(256), 0, st, vec->mu, n, vec->rk);
        LAUNCH_OK();
        hipLaunchKernelGGL(k_zfill<T>, dim3((unsigned)cdiv_h(n * vec->k, 256)), dim3(256), 0, st, vec->Z, n, vec->k,
                           vec->ldz);
        LAUNCH_OK();
        hipLaunchKernelGGL(k_invit<T>, dim3((unsigned)cdiv_h(n, 64)), dim3(64), 0, st, b.band, n, b.bounds, vec->blo,
                           vec->bhi, vec->mu, vec->rk, vec->k, vec->scr, vec->Z, vec->ldz);
        LAUNCH_OK();
        if (n >= 3) {
            const uint64_t spin_ticks = 100000000ull * 10;  // 10 s at the 100 MHz real-time counter
            hipLaunchKernelGGL(k_bt_bulge<T>, dim3((unsigned)cdiv_h(vec->k, 64)), dim3(64 * BtBulgeCfg<T>::WV), 0,
                               st, vec->refl, n, vec->k, vec->Z, vec->ldz, spin_ticks, b.prog + n);
            LAUNCH_OK();
        }
        for (int64_t c0 = std::max<int64_t>(0, n - NB - 2) / NB * NB; c0 >= 0; c0 -= NB) {
            const int64_t r0 = c0 + NB, m = n - r0;
            if (m < 2) continue;
            const T *Pp = A + r0 * lda + c0;
            T *Zr = vec->Z + r0 * vec->ldz;
            const int nch = (int)cdiv_h(m, BTP_RC);
            const unsigned ncb = (unsigned)cdiv_h(vec->k, 64);
            hipLaunchKernelGGL(k_btp_w<T>, dim3(ncb, (unsigned)nch), dim3(256), 0, st, Pp, lda, (int)m,
                               (const T *)Zr, vec->ldz, vec->k, vec->wp);
            LAUNCH_OK();
            hipLaunchKernelGGL(k_btp_y<T>, dim3(ncb), dim3(256), 0, st,
                               (const T *)vec->wp, nch, (const T *)(vec->keepT + (c0 / NB) * NB * NB), vec->k,
                               vec->yb);
            LAUNCH_OK();
            hipLaunchKernelGGL(k_btp_u<T>, dim3((unsigned)cdiv_h(m, 64), ncb), dim3(256), 0, st, Pp, lda, (int)m,
                               (const T *)vec->yb, vec->k, Zr, vec->ldz);
            LAUNCH_OK();
        }
    }
    if (info != nullptr) {
        hipLaunchKernelGGL(k_info, dim3(1), dim3(64), 0, st, b.prog + n, info);
        LAUNCH_OK();
    }
    return hipSuccess;
}

// ---- sum of the XR-row partial products: B = sum_blk Ppart[blk] (NB x NB)
__global__ __launch_bounds__(256) void k_psum(const float *__restrict__ Ppart, int nblk, float *__restrict__ B)
{
    const int q = blockIdx.x * 256 + threadIdx.x;  // grid NB * NB / 256
    float acc = 0.f;
#pragma unroll 8
    for (int b = 0; b < nblk; ++b) acc += Ppart[(int64_t)b * NB * NB + q];
    B[q] = acc;
}

// ---- eigenvectors of the small Rayleigh quotient B = sum of the nblk partial
// blocks Ppart (NB x NB, symmetrised) by parallel Jacobi: in step r of a sweep
// the indices are paired by the round-robin tournament (31 with r, and i with
// (2r - i) mod 31), which covers every pair once in NB - 1 steps, and the 16
// disjoint rotations of a step are applied together as B <- J^T B J,
// V <- V J.  Each rotation zeroes its b_pq with tan from tau = (b_qq - b_pp) /
// (2 b_pq); a pair is left alone when |b_pq| <= max(2e-6 sqrt(|b_pp b_qq|),
// 1e-7 max|b_ij|) (2e-6 ~ NB times the f32 unit roundoff, the level at which
// rounding keeps re-creating off-diagonal mass), a step with no rotation is
// skipped, and the sweeps stop when none rotates (at most 30).
// J has two non-zeros per column: column j of B J is al_j col_j + be_j
// col_partner(j), so every new element is a 4-term sum of the old B (double
// buffered in LDS).  Output: w descending and U with column r the vector of w[r].
__global__ __launch_bounds__(256) void k_ritz_jacobi(const float *__restrict__ Ppart, int nblk, float *__restrict__ w,
                                                     float *__restrict__ U, int32_t *__restrict__ info)
{
    constexpr int L = NB + 1, EPT = NB * NB / 256;
    __shared__ float Bs[2][NB * L], Vs[2][NB * L];
    __shared__ float4 cf[4][NB];  // per wave, per index: (al, be, new diagonal, 1 if its pair rotates)
    __shared__ float red[8];
    const int tid = threadIdx.x;
    float bmax = 0.f;
    {
        float acc[EPT];
#pragma unroll
        for (int k = 0; k < EPT; ++k) acc[k] = 0.f;
        for (int b = 0; b < nblk; ++b) {
#pragma unroll
            for (int k = 0; k < EPT; ++k) acc[k] += Ppart[(int64_t)b * NB * NB + tid + 256 * k];
        }
#pragma unroll
        for (int k = 0; k < EPT; ++k) {
            const int e = tid + 256 * k, r = e / NB, c = e % NB;
            Bs[1][r * L + c] = acc[k];
            Vs[0][r * L + c] = r == c ? 1.f : 0.f;
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < EPT; ++k) {
            const int e = tid + 256 * k, r = e / NB, c = e % NB;
            const float v = 0.5f * (Bs[1][r * L + c] + Bs[1][c * L + r]);
            Bs[0][r * L + c] = v;
            bmax = fmaxf(bmax, fabsf(v));
        }
        for (int o = 32; o > 0; o >>= 1) bmax = fmaxf(bmax, __shfl_xor(bmax, o));
        if ((tid & 63) == 0) red[tid >> 6] = bmax;
        __syncthreads();
        bmax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    }
    // a NaN or Inf in B (fmaxf skips NaN, so test every entry): no rotation is
    // meaningful; every output is written as NaN and info says why
    int bad = 0;
#pragma unroll
    for (int k = 0; k < EPT; ++k) bad |= !isfinite(Bs[0][((tid + 256 * k) / NB) * L + (tid + 256 * k) % NB]);
    bad = __syncthreads_or(bad);
    if (bad) {
        if (tid < NB) {
            w[tid] = __builtin_nanf("");
            for (int k = 0; k < NB; ++k) U[k * NB + tid] = __builtin_nanf("");
        }
        if (tid == 0 && info != nullptr) *info = 1;
        return;
    }
    const float floor_abs = 1e-7f * bmax;
    int cur = 0;
    int converged = 0;
    const int wv = tid >> 6, lane = tid & 63;
    for (int sweep = 0; sweep < 30; ++sweep) {
        int any = 0;
        for (int r = 0; r < NB - 1; ++r) {
            auto partner = [r](int i) { return i == NB - 1 ? r : (i == r ? NB - 1 : (2 * r - i + 2 * (NB - 1)) % (NB - 1)); };
            // Every wave computes the step's rotations itself (lanes 0-31, one
            // index each) into its own slot: all waves read the same B, so their
            // coefficients and their skip decision agree, and one workgroup
            // barrier per step (after the update) is enough.
            int on = 0;
            if (lane < NB) {  // the rotation of index lane's pair (both members compute it alike)
                const int i = lane, j = partner(i), p = min(i, j), q = max(i, j);
                const float *B = Bs[cur];
                const float apq = B[p * L + q], app = B[p * L + p], aqq = B[q * L + q];
                float a = 1.f, bb = 0.f, d = B[i * L + i];
                if (fabsf(apq) > fmaxf(2e-6f * sqrtf(fabsf(app * aqq)), floor_abs)) {
                    // hardware reciprocal and reciprocal square root (about 1 ulp):
                    // c^2 + s^2 = 1 to a few ulp, which is all the rotation needs
                    const float tau = (aqq - app) * __builtin_amdgcn_rcpf(2.f * apq);
                    const float at = fabsf(tau);
                    const float t = copysignf(at > 1e18f ? __builtin_amdgcn_rcpf(2.f * at)
                                                         : __builtin_amdgcn_rcpf(at + __builtin_amdgcn_sqrtf(1.f + tau * tau)),
                                              tau);
                    const float c = __builtin_amdgcn_rsqf(1.f + t * t), sn = t * c;
                    a = c;
                    bb = i == p ? -sn : sn;
                    d = i == p ? app - t * apq : aqq + t * apq;
                    on = 1;
                }
                cf[wv][i] = make_float4(a, bb, d, on ? 1.f : 0.f);
            }
            const bool step_on = __ballot(on) != 0;  // the same in every wave
            if (!step_on) continue;                  // B unchanged: nothing to order
            any = 1;
            wave_sync();  // this wave's coefficients are in LDS
            const float *B = Bs[cur];
            const float *V = Vs[cur];
            float *Bn = Bs[cur ^ 1];
            float *Vn = Vs[cur ^ 1];
            const int j = tid % NB, pj = partner(j);  // the same column in every k
            const float4 cj = cf[wv][j];
#pragma unroll
            for (int k = 0; k < EPT; ++k) {
                const int i = tid / NB + (256 / NB) * k, pi = partner(i);
                const float4 ci = cf[wv][i];
                const float b00 = B[i * L + j], b01 = B[i * L + pj], b10 = B[pi * L + j], b11 = B[pi * L + pj];
                const float v0 = V[i * L + j], v1 = V[i * L + pj];
                float v = ci.x * (cj.x * b00 + cj.y * b01) + ci.y * (cj.x * b10 + cj.y * b11);
                v = (pi == j && ci.w != 0.f) ? 0.f : v;  // the rotated pair's b_pq
                v = i == j ? ci.z : v;
                Bn[i * L + j] = v;
                Vn[i * L + j] = cj.x * v0 + cj.y * v1;
            }
            cur ^= 1;
            __syncthreads();  // the new B and V are complete; the old ones are no longer read
        }
        if (!any) {  // the same in every wave
            converged = 1;
            break;
        }
    }
    // rank of eigenvalue i among the diagonal: descending, ties by index, a NaN
    // (from rounding overflow) after every number, so the ranks are a permutation
    // and every slot of w and U is written
    if (tid < NB) {
        const int i = tid;
        const float li = Bs[cur][i * L + i];
        int r = 0;
        for (int j = 0; j < NB; ++j) {
            const float lj = Bs[cur][j * L + j];
            const bool ni = isnan(li), nj = isnan(lj);
            const bool before = (ni || nj) ? (ni && (!nj || j < i)) : (lj > li || (lj == li && j < i));
            r += before ? 1 : 0;
        }
        w[r] = li;
        for (int k = 0; k < NB; ++k) U[k * NB + r] = Vs[cur][k * L + i];
    }
    if (tid == 0 && info != nullptr) *info = converged ? 0 : 2;
}

// ---- P = Q1 U (m x NB): the Ritz vectors
__global__ __launch_bounds__(256) void k_ritz_vectors(const float *__restrict__ Q, int m, const float *__restrict__ U,
                                                      float *__restrict__ P, int64_t ldp)
{
    __shared__ float Us[NB * NB];
    const int tid = threadIdx.x;
    for (int q = tid; q < NB * NB; q += 256) Us[q] = U[q];
    __syncthreads();
    const int64_t r = (int64_t)blockIdx.x * 8 + (tid >> 5);
    const int c = tid & 31;
    if (r >= m) return;
    float qrow[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) qrow[j] = Q[r * NB + j];
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < NB; ++j) acc += qrow[j] * Us[j * NB + c];
    P[r * ldp + c] = acc;
}

// Leading eigenvalues by random projection ("Random matrix theory spectral
// methods" page, section 3.2): Y = A Omega, Q = orth(Y), q times Q = orth(A Q),
// then the NB Ritz values eig(Q^T A Q), descending.  The products are the
// reduction's SYMM (lower-stored A, split over column chunks) and partial sums;
// orth is the TSQR of the reduction with its explicit Q1; Q^T A Q is the sum of
// the per-block products Q_blk^T (A Q)_blk; its eigenvalues come from the
// batched small solver.  A is read, not written.
hipError_t run_topk(hipStream_t st, const float *A, int64_t n, int64_t lda, const float *Omega, int q, float *w,
                    float *P, int64_t ldp, void *ws, int32_t *info)
{
    Bufs<float> b;
    layout<float>(n, (char *)ws, b);
    const int m = (int)n;
    constexpr int TOP_BLOCKS = Cfg<float>::RB / NB;
    auto symm = [&](const float *Wm) -> hipError_t {
        const int nrb = (int)cdiv_h(m, SY_RB);
        int ks = (int)std::min<int64_t>(KS_MAX, std::max<int64_t>(1, cdiv_h(512, nrb)));
        const int chunk = (int)(cdiv_h(cdiv_h(m, ks), SY_JB) * SY_JB);
        ks = (int)cdiv_h(m, chunk);
        hipLaunchKernelGGL(k_symm_f32, dim3(nrb, ks), dim3(256), 0, st, A, lda, m, Wm, b.Xpart, chunk);
        LAUNCH_OK();
        const int nxb = (int)cdiv_h(m, XR);
        hipLaunchKernelGGL(k_xreduce<float>, dim3(nxb), dim3(256), 0, st, b.Xpart, ks, m, Wm, b.X, b.Ppart);
        return hipGetLastError();
    };
    auto orth = [&]() -> hipError_t {  // Q1 = the first NB columns of the Q of X = QR
        const int nblk = (int)std::min<int64_t>(TOP_BLOCKS, cdiv_h(m, 256));
        const int per = (int)cdiv_h(m, nblk);
        const int rows_top = nblk * NB;
        if (per <= 256)
            hipLaunchKernelGGL((k_tsqr_wave<float, 1>), dim3(nblk), dim3(64), 0, st, b.X, (int64_t)NB, m, per,
                               b.Vloc, b.Tloc, b.Rstack, (float *)nullptr, (const int *)nullptr);
        else if (per <= 512)
            hipLaunchKernelGGL((k_tsqr_wave<float, 2>), dim3(nblk), dim3(128), 0, st, b.X, (int64_t)NB, m, per,
                               b.Vloc, b.Tloc, b.Rstack, (float *)nullptr, (const int *)nullptr);
        else
            hipLaunchKernelGGL((k_tsqr_wave<float, 4>), dim3(nblk), dim3(256), 0, st, b.X, (int64_t)NB, m, per,
                               b.Vloc, b.Tloc, b.Rstack, (float *)nullptr, (const int *)nullptr);
        LAUNCH_OK();
        if (rows_top <= 256)
            hipLaunchKernelGGL((k_tsqr_wave<float, 1>), dim3(1), dim3(64), 0, st, b.Rstack, (int64_t)NB, rows_top,
                               rows_top, b.Vtop, b.Ttop, b.Rf, b.Ktop, (const int *)nullptr);
        else if (rows_top <= 512)
            hipLaunchKernelGGL((k_tsqr_wave<float, 2>), dim3(1), dim3(128), 0, st, b.Rstack, (int64_t)NB, rows_top,
                               rows_top, b.Vtop, b.Ttop, b.Rf, b.Ktop, (const int *)nullptr);
        else
            hipLaunchKernelGGL((k_tsqr_wave<float, 4>), dim3(1), dim3(256), 0, st, b.Rstack, (int64_t)NB, rows_top,
                               rows_top, b.Vtop, b.Ttop, b.Rf, b.Ktop, (const int *)nullptr);
        LAUNCH_OK();
        hipLaunchKernelGGL(k_tsqr_q1<float>, dim3((unsigned)cdiv_h(per, 8), nblk), dim3(256), 0, st, b.Vloc, b.Tloc,
                           b.Vtop, b.Ktop, m, per, b.Q1, (const int *)nullptr);
        return hipGetLastError();
    };
    hipError_t e;
    if ((e = symm(Omega)) != hipSuccess) return e;
    if ((e = orth()) != hipSuccess) return e;
    for (int it = 0; it < q; ++it) {
        if ((e = symm(b.Q1)) != hipSuccess) return e;
        if ((e = orth()) != hipSuccess) return e;
    }
    if ((e = symm(b.Q1)) != hipSuccess) return e;  // X = A Q and the blocks of Q^T X
    if (P != nullptr) {  // Ritz values and vectors: Jacobi on B, then P = Q U
        hipLaunchKernelGGL(k_ritz_jacobi, dim3(1), dim3(256), 0, st, b.Ppart, (int)cdiv_h(m, XR), w, b.Tm, info);
        LAUNCH_OK();
        hipLaunchKernelGGL(k_ritz_vectors, dim3((unsigned)cdiv_h(m, 8)), dim3(256), 0, st, b.Q1, m, b.Tm, P, ldp);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(k_psum, dim3(NB * NB / 256), dim3(256), 0, st, b.Ppart, (int)cdiv_h(m, XR), b.U);
    LAUNCH_OK();
    spec_batch_src src;
    src.kind = SPEC_SRC_DENSE;
    src.a = b.U;
    src.lda = NB;
    src.stride_a = NB * NB;
    src.streams = 0;
    src.T = 0;
    src.stride = 1;
    src.scale = 1.f;
    return launch_eigvalsh_batched(st, &src, 1, NB, w, nullptr);
}

}  // namespace

size_t eig_large_workspace_bytes(int64_t n, int t)
{
    if (t == SPEC_F32) {
        Bufs<float> b;
        return layout<float>(n, nullptr, b);
    }
    Bufs<double> b;
    return layout<double>(n, nullptr, b);
}

namespace {

// the eigenvector path's workspace after the solver's own: reflectors, panel
// T factors, the tridiagonal's blocks, eigenvalues and ranks, inverse-iteration
// scratch (4 n k doubles), the panel back-transformation's partials
template <typename T>
size_t vec_layout(int64_t n, int64_t k, char *base, VecReq<T> &v)
{
    Ws ws;
    ws.base = base;
    const int64_t nrefl = n >= 3 ? refl_index(n, n - 2) : 0;
    v.refl = ws.take<T>((size_t)std::max<int64_t>(1, nrefl) * RFL);
    v.keepT = ws.take<T>((size_t)(n / NB + 1) * NB * NB);
    v.blo = ws.take<int32_t>((size_t)n);
    v.bhi = ws.take<int32_t>((size_t)n);
    v.rk = ws.take<int32_t>((size_t)n);
    v.mu = ws.take<double>((size_t)n);
    v.scr = ws.take<double>((size_t)4 * n * k);
    v.wp = ws.take<T>((size_t)(n / BTP_RC + 1) * NB * k);
    v.yb = ws.take<T>((size_t)NB * k);
    return ws.off;
}

}  // namespace

size_t eigh_large_workspace_bytes(int64_t n, int t, int64_t k)
{
    const size_t base = (eig_large_workspace_bytes(n, t) + 255) / 256 * 256;
    if (t == SPEC_F32) {
        VecReq<float> v;
        return base + vec_layout<float>(n, k, nullptr, v);
    }
    VecReq<double> v;
    return base + vec_layout<double>(n, k, nullptr, v);
}

hipError_t launch_eigh_large(hipStream_t stream, void *A, int t, int64_t n, int64_t lda, void *w, void *Z,
                             int64_t ldz, int64_t k, void *ws, int32_t *info)
{
    const size_t base = (eig_large_workspace_bytes(n, t) + 255) / 256 * 256;
    char *extra = (char *)ws + base;
    if (t == SPEC_F32) {
        VecReq<float> v;
        vec_layout<float>(n, k, extra, v);
        v.Z = (float *)Z;
        v.ldz = ldz;
        v.k = k;
        return run<float>(stream, (float *)A, n, lda, (float *)w, ws, info, &v);
    }
    VecReq<double> v;
    vec_layout<double>(n, k, extra, v);
    v.Z = (double *)Z;
    v.ldz = ldz;
    v.k = k;
    return run<double>(stream, (double *)A, n, lda, (double *)w, ws, info, &v);
}

hipError_t launch_eig_large(hipStream_t stream, void *A, int t, int64_t n, int64_t lda, void *w, void *ws,
                            int32_t *info)
{
    if (t == SPEC_F32) return run<float>(stream, (float *)A, n, lda, (float *)w, ws, info);
    return run<double>(stream, (double *)A, n, lda, (double *)w, ws, info);
}

hipError_t launch_topk_ritz(hipStream_t stream, const float *A, int64_t n, int64_t lda, const float *Omega, int q,
                            float *w, float *P, int64_t ldp, void *ws, int32_t *info)
{
    return run_topk(stream, A, n, lda, Omega, q, w, P, ldp, ws, info);
}
