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
//   independent.  A workgroup runs G consecutive sweeps, one wave each, a time
//   step at a time, with their rows in an LDS ring and each task's block in
//   the wave's registers; a loader wave and a storer wave move band rows
//   between the ring and global memory; consecutive groups are ordered by a
//   row watermark (rows below it are final and stored back), with a bounded
//   wait.  Each reflector's tau is 2 / v^T v of the v it is applied with, so
//   every reflection is orthogonal to rounding.
// Stage 3, eigenvalues of the tridiagonal: 16-section on the Sturm count
//   (number of negative pivots of LDL^T(T - xI)), 16 lanes per eigenvalue, from
//   the Gershgorin interval; results in descending order.  An fp32 matrix is
//   counted in fp32 (backward stable: exact for a matrix within a few ulps of T
//   entry by entry), an fp64 one in fp64.
#include <float.h>

#include <algorithm>
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
                                                   T *__restrict__ Vloc, T *__restrict__ Tloc, T *__restrict__ Rstack)
{
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
                                                       T *__restrict__ Rstack, T *__restrict__ Kt)
{
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
                                                 T *__restrict__ Vtop, T *__restrict__ Kt)
{
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
                                                 int per, T *__restrict__ Q1)
{
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

// ---- A22 -= V Z^T + Z V^T on lower 128 x 128 tiles
constexpr int S2_T = 128;
constexpr int S2_K = 2 * NB;

template <typename T>
__global__ __launch_bounds__(256) void k_syr2k(T *__restrict__ A, int64_t lda, int m, const T *__restrict__ V,
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
        const int rl = wm * 64 + (lane >> 5) * 4, cl = wn * 64 + (lane & 31);  // lane's first row and column
        const uint32_t vbase = (uint32_t)(rl * (int)lda + cl) * 4u;
        // element (qa, qb, e): row rl + qa*32 + (e>>2)*8 + (e&3), column cl + qb*32
        auto eoff = [&](int qa, int qb, int e) {
            const int dr = qa * 32 + (e >> 2) * 8 + (e & 3);
            const bool ok = !diag || rl + dr >= cl + qb * 32;
            return ok ? vbase + (uint32_t)(dr * (int)lda + qb * 32) * 4u : 0x80000000u;
        };
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
        // the old values are requested after the staging (memory counters
        // retire in issue order, so earlier they would hold up the LDS stores)
        // and are in flight while the MFMAs run
        float old[2][2][16];
#pragma unroll
        for (int qa = 0; qa < 2; ++qa)
#pragma unroll
            for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    old[qa][qb][e] =
                        __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, (int)eoff(qa, qb, e), 0, 0));
        f32x16_t acc[2][2] = {};
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
                        __builtin_bit_cast(uint32_t, old[qa][qb][e] - acc[qa][qb][e]), rs, (int)eoff(qa, qb, e), 0, 0);
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


// One workgroup per group of G consecutive sweeps s0 .. s0+G-1: G compute
// waves, a loader wave and a storer wave.  At time step t compute wave i runs
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

template <typename T, int G, int CAPR>
__global__ __launch_bounds__(64 * (G + 2)) void k_bulge(T *__restrict__ band, int64_t n, int32_t *__restrict__ wm,
                                                        uint64_t spin_ticks)
{
    constexpr int LA = 2;  // the ring holds the lead's chunks up to the next step's (LA - 1 ahead)
    static_assert(CAPR % NB == 0 && (LA + 2 * G - 1) * NB <= CAPR, "ring too small");
    constexpr int LDW = BW + 1;
    constexpr int RB = BW * sizeof(T);  // bytes per band row
    constexpr int QI = 4096 / RB;       // rows reachable from one base through the instruction offset
    __shared__ T WRbuf[NB + CAPR * LDW + 64];
    T *const WR = WRbuf + NB;  // NB guard entries before the first ring row
    constexpr int SINK = CAPR * LDW;  // 64 entries after the ring: target of masked-off stores
    __shared__ T vsw[G][NB];
    __shared__ T red[G][NB];
    __shared__ T w2s[G][NB];
    __shared__ int abort_flag[2];  // set at step t in entry t & 1, read by every wave after that step
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int ci = lane & 31, h = lane >> 5;
    const int nn = (int)n;
    const int nsw = nn - 2;
    int32_t *err = wm + n;
    const int g = blockIdx.x;
    const int s0 = g * G;
    const int Ge = min(G, nsw - s0);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(band, 0, nn * RB, 0x00020000);
    // ring slot of row r, counted from the group's first row so that the lead's
    // NB-row chunks never wrap
    auto slot = [&](int r) { return (r - s0 - 1) % CAPR; };
    auto ntasks = [&](int s) { return (nn - 2 - s) / NB + 1; };
    // a task (s, k) reads and writes only rows s + 1 + k NB .. s + (k + 1) NB
    auto minrow = [&](int s, int k) { return k <= 0 ? s + 1 : s + 1 + k * NB; };
    auto lastrow = [&](int s, int k) { return min(s + (k + 1) * NB, nn - 1); };
    const int ntl = ntasks(s0);  // tasks of the lead sweep
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
    T taup = 0;          // compute wave: tau of the previous reflector of its sweep
    int ab = 0;          // abort flag of the previous step
    // the group's last sweep ends last: its last task is the group's last step
    const int t_end = 2 * (s0 + Ge - 1) + ntasks(s0 + Ge - 1);
    for (int t = 2 * s0; t < t_end; ++t) {
        const int k0 = t - 2 * s0;
        if (wv == G) {
            // the lead's chunk for the next step
            const int kn = k0 + LA - 1;
            if (kn < ntl) {
                const int lo = loaded_to(kn - 1), hi = loaded_to(kn);
                if (wait_rows(hi - 1, t & 1)) {
                    T ld[NB];
                    load_chunk(lo, ld);
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
                // Lane (ci, h) holds row r0 + ci of the task's block in registers: the
                // columns h*16 .. h*16+15 of O = A[r0.., c0 .. c0+NB) (k > 0) and of the
                // lower triangle of the diagonal block D = A[r0.., r0..].  All of it lies
                // in the lane's own ring row at fixed offsets, so the loads issue back to
                // back; entries outside the task are masked after loading (the guard
                // before the ring keeps every offset inside the array).
                const int r0 = s + 1 + k * NB;
                const int L = lastrow(s, k) - r0 + 1;
                const bool rowok = ci < L;
                const int rb = slot(r0 + ci) * LDW;  // ring slot of row r0 + ci
                const int e = rowok ? ci - h * 16 : -1;          // D column c of this lane is in the lower triangle iff c <= e
                T *v = vsw[wv];
                T o[16], dd[16], vp[16];
#pragma unroll
                for (int c = 0; c < 16; ++c) {
                    dd[c] = WR[rb + ci - h * 16 - c];
                    o[c] = WR[rb + NB + ci - h * 16 - c];
                    vp[c] = v[h * 16 + c];  // the previous task's reflector
                }
                const T xs = WR[rb + ci + 1];  // column s
                const T dg = rowok ? WR[rb] : (T)0;
#pragma unroll
                for (int c = 0; c < 16; ++c) dd[c] = c <= e ? dd[c] : (T)0;
                if (L < NB) {
#pragma unroll
                    for (int c = 0; c < 16; ++c) o[c] = rowok ? o[c] : (T)0;
                }
                T x;
                if (k == 0) {
                    x = rowok ? xs : (T)0;
                } else {
                    // right: O <- O (I - taup vp vp^T)
                    if (taup != 0) {
                        T u = 0;
#pragma unroll
                        for (int c = 0; c < 16; ++c) u += o[c] * vp[c];
                        u = taup * pair32_sum(u);
#pragma unroll
                        for (int c = 0; c < 16; ++c) o[c] -= u * vp[c];
                    }
                    x = from_lower_half(o[0]);  // column c0, held by the lanes of half 0
                }
                // reflector (I - tau v v^T) x = mu e_0, v_0 = 1
                const T sigma = half_sum(ci >= 1 ? x * x : (T)0);
                const T x0 = readlane0(x);
                T tau_k = 0, mu = 0, vi = 0;
                if (sigma > 0) {
                    mu = sqrt(x0 * x0 + sigma);
                    // v_0 and 1/v_0 need not be exact: tau below is computed from the
                    // v actually stored, so H stays orthogonal, and the column that H
                    // annihilates is set to mu e_0 explicitly
                    const T v0 = x0 <= 0 ? x0 - mu : -sigma * recip(x0 + mu);
                    const T iv0 = recip(v0);
                    vi = ci == 0 ? (T)1 : x * iv0;
                    // tau = 2 / v^T v with v^T v = 1 + sigma iv0^2, the same iv0 that
                    // scales v: I - tau v v^T is orthogonal up to the rounding of the
                    // entries (a tau from v0 alone, whose reciprocal is rounded
                    // differently from iv0, drifts the trace over many applications)
                    tau_k = (T)2 / ((T)1 + sigma * iv0 * iv0);
                }
                wave_sync();
                if (h == 0) v[ci] = vi;
                if (tau_k != 0) {
                    // column sums, reduced over the 32 rows of each half (lane ci ends
                    // with column h*16 + ci/2): w = O^T v and the part of D v that
                    // comes from the upper triangle, sum_{j >= i} D[j][i] v_j
                    T q[16];
                    if (k > 0) {
#pragma unroll
                        for (int c = 0; c < 16; ++c) q[c] = vi * o[c];
                        const T wj = reduce_scatter16(q, ci);
                        if ((ci & 1) == 0) red[wv][h * 16 + (ci >> 1)] = wj;
                    }
#pragma unroll
                    for (int c = 0; c < 16; ++c) q[c] = vi * dd[c];
                    const T pj = reduce_scatter16(q, ci);
                    if ((ci & 1) == 0) w2s[wv][h * 16 + (ci >> 1)] = pj;
                }
                wave_sync();
                T vr[16];
#pragma unroll
                for (int c = 0; c < 16; ++c) vr[c] = v[h * 16 + c];
                if (tau_k != 0) {
                    const T pcol = w2s[wv][ci];
                    if (k > 0) {
                        const T tv = tau_k * vi;
#pragma unroll
                        for (int c = 0; c < 16; ++c) o[c] -= tv * red[wv][h * 16 + c];
                        if (h == 0) o[0] = ci == 0 ? mu : (T)0;
                    }
                    // two-sided on D: p = tau D v, w = p - (tau/2)(p^T v) v, D -= v w^T + w v^T
                    T pp = 0;
#pragma unroll
                    for (int c = 0; c < 16; ++c) pp += dd[c] * vr[c];
                    pp = tau_k * (pair32_sum(pp) + pcol - dg * vi);
                    const T pv = half_sum(pp * vi);
                    const T w2 = pp - (T)0.5 * tau_k * pv * vi;
                    wave_sync();
                    if (h == 0) w2s[wv][ci] = w2;
                    wave_sync();
#pragma unroll
                    for (int c = 0; c < 16; ++c) dd[c] -= vi * w2s[wv][h * 16 + c] + w2 * vr[c];
                }
                if (rowok) {
                    if (k == 0) {
                        if (tau_k != 0) WR[rb + ci + 1] = ci == 0 ? mu : (T)0;
                    } else {
#pragma unroll
                        for (int c = 0; c < 16; ++c) WR[rb + NB + ci - h * 16 - c] = o[c];
                    }
                }
                if (tau_k != 0) {
                    // entries above the block's diagonal go to the sink, so the 16
                    // stores need no branches
#pragma unroll
                    for (int c = 0; c < 16; ++c) WR[c <= e ? rb + ci - h * 16 - c : SINK + lane] = dd[c];
                }
                taup = tau_k;
            }
        }
        if (ab) return;  // every wave leaves at the same step
        __syncthreads();
        ab = abort_flag[t & 1];  // not written again before the next barrier
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

__device__ __forceinline__ int sturm_below(const double *__restrict__ dd, const double *__restrict__ ee2, int64_t n,
                                           double x, double pivmin)
{
    int cnt = 0;
    double q = dd[0] - x;
    if (fabs(q) < pivmin) q = -pivmin;
    cnt += q < 0.0;
    for (int64_t i = 1; i < n; ++i) {
        q = (dd[i] - x) - ee2[i - 1] / q;
        if (fabs(q) < pivmin) q = -pivmin;
        cnt += q < 0.0;
    }
    return cnt;
}

// 4 eigenvalues per 64-lane workgroup, 16 lanes (15 interior points + 1) each
template <typename T>
__global__ __launch_bounds__(64) void k_bisect(const double *__restrict__ dd, const double *__restrict__ ee2,
                                               int64_t n, const double *__restrict__ bounds, double rel_tol,
                                               T *__restrict__ w)
{
    const int lane = threadIdx.x;
    const int g = lane >> 4, j = lane & 15;
    const int64_t kidx = blockIdx.x * 4 + g;  // descending index
    const bool live = kidx < n;
    const int64_t target = n - 1 - (live ? kidx : 0);  // ascending index
    double a = bounds[0], b = bounds[1];
    const double pivmin = bounds[2];
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
__global__ __launch_bounds__(64) void k_bisect_f32(const float2 *__restrict__ de, int n,
                                                   const double *__restrict__ bounds, float *__restrict__ w)
{
    const int lane = threadIdx.x;
    const int g = lane >> 4, j = lane & 15;
    const int kidx = blockIdx.x * 4 + g;  // descending index
    const bool live = kidx < n;
    const int target = n - 1 - (live ? kidx : 0);  // ascending index
    // the fp64 Gershgorin bounds, rounded outwards, with a few ulps of slack
    float a = (float)bounds[0], b = (float)bounds[1];
    const float span = fmaxf(fabsf(a), fabsf(b));
    a -= 4.f * 1.1920929e-7f * span;
    b += 4.f * 1.1920929e-7f * span;
    const float pivmin = (float)bounds[3];
    const float atol = 0.0625f * 1.1920929e-7f * span;
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
    T *band, *V, *W, *X, *Xpart, *Q1, *Vloc, *Tloc, *Rstack, *Rf, *Vtop, *Ttop, *Ktop, *U, *Tm, *Ppart;
    int32_t *prog;
    double *dd, *ee2, *bounds;
    float2 *de32;
};

constexpr int KS_MAX = 8;

template <typename T>
size_t layout(int64_t n, char *base, Bufs<T> &b)
{
    Ws ws;
    ws.base = base;
    b.band = ws.take<T>((size_t)n * BW);
    b.prog = ws.take<int32_t>((size_t)n + 1);
    b.V = ws.take<T>((size_t)n * NB);
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
    return ws.off;
}

#define LAUNCH_OK()                                     \
    do {                                                \
        hipError_t e_ = hipGetLastError();              \
        if (e_ != hipSuccess) return e_;                \
    } while (0)

template <typename T>
hipError_t run(hipStream_t st, T *A, int64_t n, int64_t lda, T *w, void *ws, int32_t *info)
{
    Bufs<T> b;
    layout<T>(n, (char *)ws, b);
    constexpr int RB = Cfg<T>::RB;
    constexpr int TOP_BLOCKS = RB / NB;  // stacked R rows (<= 1024 f32, 512 f64) fit one workgroup's registers
    constexpr int DIRECT_ROWS = 256;
    static_assert(DIRECT_ROWS <= RB, "direct panel must fit");
    // ---- stage 1: dense -> band
    for (int64_t c0 = 0;; c0 += NB) {
        const int64_t r0 = c0 + NB;
        const int64_t m = n - r0;
        if (m < 2) break;
        T *P = A + r0 * lda + c0;
        T *A22 = A + r0 * lda + r0;
        if (m <= DIRECT_ROWS) {
            hipLaunchKernelGGL(k_panel_direct<T>, dim3(1), dim3(256), 0, st, P, lda, (int)m, b.V, b.Tm);
            LAUNCH_OK();
        } else {
            // row blocks of about 256 rows, at most TOP_BLOCKS of them (the stacked R
            // factors of all blocks are factored by one workgroup)
            const int nblk = (int)std::min<int64_t>(TOP_BLOCKS, cdiv_h(m, 256));
            const int per = (int)cdiv_h(m, nblk);
            const int rows_top = nblk * NB;
            // fp32: QRs with four rows per lane (one wave up to 256 rows, two up to 512,
            // four up to 1024); fp64: one row per thread
            if constexpr (std::is_same<T, float>::value) {
                if (per <= 256)
                    hipLaunchKernelGGL((k_tsqr_wave<T, 1>), dim3(nblk), dim3(64), 0, st, P, lda, (int)m, per, b.Vloc,
                                       b.Tloc, b.Rstack, (T *)nullptr);
                else if (per <= 512)
                    hipLaunchKernelGGL((k_tsqr_wave<T, 2>), dim3(nblk), dim3(128), 0, st, P, lda, (int)m, per,
                                       b.Vloc, b.Tloc, b.Rstack, (T *)nullptr);
                else
                    hipLaunchKernelGGL((k_tsqr_wave<T, 4>), dim3(nblk), dim3(256), 0, st, P, lda, (int)m, per,
                                       b.Vloc, b.Tloc, b.Rstack, (T *)nullptr);
                LAUNCH_OK();
                if (rows_top <= 256)
                    hipLaunchKernelGGL((k_tsqr_wave<T, 1>), dim3(1), dim3(64), 0, st, b.Rstack, (int64_t)NB, rows_top,
                                       rows_top, b.Vtop, b.Ttop, b.Rf, b.Ktop);
                else if (rows_top <= 512)
                    hipLaunchKernelGGL((k_tsqr_wave<T, 2>), dim3(1), dim3(128), 0, st, b.Rstack, (int64_t)NB,
                                       rows_top, rows_top, b.Vtop, b.Ttop, b.Rf, b.Ktop);
                else
                    hipLaunchKernelGGL((k_tsqr_wave<T, 4>), dim3(1), dim3(256), 0, st, b.Rstack, (int64_t)NB,
                                       rows_top, rows_top, b.Vtop, b.Ttop, b.Rf, b.Ktop);
                LAUNCH_OK();
            } else {
                if (per <= 256)
                    hipLaunchKernelGGL((k_tsqr_local<T, 256>), dim3(nblk), dim3(256), 0, st, P, lda, (int)m, per,
                                       b.Vloc, b.Tloc, b.Rstack);
                else if (per <= 512)
                    hipLaunchKernelGGL((k_tsqr_local<T, 512>), dim3(nblk), dim3(512), 0, st, P, lda, (int)m, per,
                                       b.Vloc, b.Tloc, b.Rstack);
                else
                    hipLaunchKernelGGL((k_tsqr_local<T, 1024>), dim3(nblk), dim3(1024), 0, st, P, lda, (int)m, per,
                                       b.Vloc, b.Tloc, b.Rstack);
                LAUNCH_OK();
                if (rows_top <= 256)
                    hipLaunchKernelGGL((k_tsqr_top<T, 256>), dim3(1), dim3(256), 0, st, b.Rstack, nblk, b.Rf, b.Vtop,
                                       b.Ktop);
                else if (rows_top <= 512)
                    hipLaunchKernelGGL((k_tsqr_top<T, 512>), dim3(1), dim3(512), 0, st, b.Rstack, nblk, b.Rf, b.Vtop,
                                       b.Ktop);
                else
                    hipLaunchKernelGGL((k_tsqr_top<T, 1024>), dim3(1), dim3(1024), 0, st, b.Rstack, nblk, b.Rf,
                                       b.Vtop, b.Ktop);
                LAUNCH_OK();
            }
            hipLaunchKernelGGL(k_tsqr_q1<T>, dim3((unsigned)cdiv_h(per, 8), nblk), dim3(256), 0, st, b.Vloc, b.Tloc,
                               b.Vtop, b.Ktop, (int)m, per, b.Q1);
            LAUNCH_OK();
            hipLaunchKernelGGL(k_tsqr_recon<T>, dim3(1), dim3(64), 0, st, b.Q1, b.Rf, P, lda, b.V, b.U, b.Tm);
            LAUNCH_OK();
        }
        // V rows below the reconstructed top block (TSQR), then W = V T
        hipLaunchKernelGGL(k_vw<T>, dim3((unsigned)cdiv_h(m, VW_R)), dim3(VW_T), 0, st, b.Q1, b.U, b.Tm, (int)m,
                           m <= DIRECT_ROWS ? (int)m : NB, b.V, b.W);
        LAUNCH_OK();
        const int nrb = (int)cdiv_h(m, SY_RB);
        int ks = (int)std::min<int64_t>(KS_MAX, std::max<int64_t>(1, cdiv_h(512, nrb)));
        int chunk = (int)(cdiv_h(cdiv_h(m, ks), SY_JB) * SY_JB);
        ks = (int)cdiv_h(m, chunk);
        hipLaunchKernelGGL(k_symm<T>, dim3(nrb, ks), dim3(256), 0, st, A22, lda, (int)m, b.W, b.Xpart, chunk);
        LAUNCH_OK();
        const int nxb = (int)cdiv_h(m, XR);
        hipLaunchKernelGGL(k_xreduce<T>, dim3(nxb), dim3(256), 0, st, b.Xpart, ks, (int)m, b.V, b.X, b.Ppart);
        LAUNCH_OK();
        hipLaunchKernelGGL(k_mz<T>, dim3((unsigned)std::min<int64_t>(MZ_BLOCKS, cdiv_h(m, 8))), dim3(256), 0, st,
                           b.Ppart, nxb, b.Tm, b.X, b.V, (int)m);
        LAUNCH_OK();
        const int64_t nt = cdiv_h(m, S2_T);
        hipLaunchKernelGGL(k_syr2k<T>, dim3((unsigned)(nt * (nt + 1) / 2)), dim3(256), 0, st, A22, lda, (int)m, b.V,
                           b.X);
        LAUNCH_OK();
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
        const uint64_t spin_ticks = 100000000ull * 10;  // 10 s at the 100 MHz real-time counter
        hipLaunchKernelGGL((k_bulge<T, G, CAPR>), dim3((unsigned)ngroups), dim3(64 * (G + 2)), 0, st, b.band, n,
                           b.prog, spin_ticks);
        LAUNCH_OK();
    }
    // ---- stage 3: eigenvalues of the tridiagonal
    hipLaunchKernelGGL(k_tridiag_prep<T>, dim3(1), dim3(256), 0, st, b.band, n, b.dd, b.ee2, b.bounds,
                       sizeof(T) == 4 ? b.de32 : nullptr);
    LAUNCH_OK();
    if constexpr (sizeof(T) == 4) {
        hipLaunchKernelGGL(k_bisect_f32, dim3((unsigned)cdiv_h(n, 4)), dim3(64), 0, st, b.de32, (int)n, b.bounds, w);
    } else {
        hipLaunchKernelGGL(k_bisect<T>, dim3((unsigned)cdiv_h(n, 4)), dim3(64), 0, st, b.dd, b.ee2, n, b.bounds,
                           4e-16, w);
    }
    LAUNCH_OK();
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
                                                     float *__restrict__ U)
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
    const float floor_abs = 1e-7f * bmax;
    int cur = 0;
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
        if (!any) break;  // the same in every wave
    }
    // rank of eigenvalue i among the diagonal (descending, ties by index)
    if (tid < NB) {
        const int i = tid;
        const float li = Bs[cur][i * L + i];
        int r = 0;
        for (int j = 0; j < NB; ++j) {
            const float lj = Bs[cur][j * L + j];
            r += (lj > li || (lj == li && j < i)) ? 1 : 0;
        }
        w[r] = li;
        for (int k = 0; k < NB; ++k) U[k * NB + r] = Vs[cur][k * L + i];
    }
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
                    float *P, int64_t ldp, void *ws)
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
        hipLaunchKernelGGL(k_symm<float>, dim3(nrb, ks), dim3(256), 0, st, A, lda, m, Wm, b.Xpart, chunk);
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
                               b.Vloc, b.Tloc, b.Rstack, (float *)nullptr);
        else if (per <= 512)
            hipLaunchKernelGGL((k_tsqr_wave<float, 2>), dim3(nblk), dim3(128), 0, st, b.X, (int64_t)NB, m, per,
                               b.Vloc, b.Tloc, b.Rstack, (float *)nullptr);
        else
            hipLaunchKernelGGL((k_tsqr_wave<float, 4>), dim3(nblk), dim3(256), 0, st, b.X, (int64_t)NB, m, per,
                               b.Vloc, b.Tloc, b.Rstack, (float *)nullptr);
        LAUNCH_OK();
        if (rows_top <= 256)
            hipLaunchKernelGGL((k_tsqr_wave<float, 1>), dim3(1), dim3(64), 0, st, b.Rstack, (int64_t)NB, rows_top,
                               rows_top, b.Vtop, b.Ttop, b.Rf, b.Ktop);
        else if (rows_top <= 512)
            hipLaunchKernelGGL((k_tsqr_wave<float, 2>), dim3(1), dim3(128), 0, st, b.Rstack, (int64_t)NB, rows_top,
                               rows_top, b.Vtop, b.Ttop, b.Rf, b.Ktop);
        else
            hipLaunchKernelGGL((k_tsqr_wave<float, 4>), dim3(1), dim3(256), 0, st, b.Rstack, (int64_t)NB, rows_top,
                               rows_top, b.Vtop, b.Ttop, b.Rf, b.Ktop);
        LAUNCH_OK();
        hipLaunchKernelGGL(k_tsqr_q1<float>, dim3((unsigned)cdiv_h(per, 8), nblk), dim3(256), 0, st, b.Vloc, b.Tloc,
                           b.Vtop, b.Ktop, m, per, b.Q1);
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
        hipLaunchKernelGGL(k_ritz_jacobi, dim3(1), dim3(256), 0, st, b.Ppart, (int)cdiv_h(m, XR), w, b.Tm);
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

hipError_t launch_eig_large(hipStream_t stream, void *A, int t, int64_t n, int64_t lda, void *w, void *ws,
                            int32_t *info)
{
    if (t == SPEC_F32) return run<float>(stream, (float *)A, n, lda, (float *)w, ws, info);
    return run<double>(stream, (double *)A, n, lda, (double *)w, ws, info);
}

hipError_t launch_topk_ritz(hipStream_t stream, const float *A, int64_t n, int64_t lda, const float *Omega, int q,
                            float *w, float *P, int64_t ldp, void *ws)
{
    return run_topk(stream, A, n, lda, Omega, q, w, P, ldp, ws);
}
