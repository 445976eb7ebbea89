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
//   step at a time, with their rows in an LDS ring; consecutive groups are
//   ordered by a row watermark (rows below it are final and stored back),
//   with a bounded wait.
// Stage 3, eigenvalues of the tridiagonal: 16-section on the Sturm count
//   (number of negative pivots of LDL^T(T - xI)) in fp64, 16 lanes per
//   eigenvalue, from the Gershgorin interval; results in descending order.
#include <float.h>

#include <algorithm>

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

// Householder QR of the rows x NB matrix P (LDS, stride LDP) by 256 threads:
// kr reflectors H_k = I - tau_k v_k v_k^T (v_k[k] = 1 implicit, v_k below the
// diagonal of column k), R in the upper triangle, and T (NB x NB, upper) of the
// forward product H_0 ... H_{kr-1} = I - V T V^T in Tl.
// Per column k, thread (c, g) = (tid % 32, tid / 32) covers rows k+1+g, +8, ...:
//   pass 1 forms the dot products d_c = v_k^T P[k:, c] for every column c, which
//     gives w_c (c > k) for the update and G[c][k] = v_c^T v_k (c < k) for T;
//   pass 2 updates the columns c > k, writes v_k, accumulates the squared norm
//     of column k+1 below its diagonal (the next reflector's sigma) and forms
//     T[0:k, k] = -tau_k T[0:k, 0:k] G[0:k, k].
// v_k is produced on the fly as scale * x in pass 1 and stored in pass 2.
template <typename T>
__device__ void lds_qr_larft(T *P, int rows, int kr, T *tau, T *Tl, T *red)
{
    const int tid = threadIdx.x;
    const int c = tid & 31, g = tid >> 5;
    T *dots = red;         // 8 x 32 partial dot products
    T *sig = red + 256;    // 8 partial sums of squares (next column)
    T *bc = red + 264;     // broadcast: [0] scale, [1] tau
    T *gk = red + 272;     // G[0:k, k] of the previous step
    for (int p = tid; p < NB * NB; p += 256) Tl[p] = 0;
    // sigma of column 0
    if (c == 0) {
        T s = 0;
        for (int i = 1 + g; i < rows; i += 8) s += P[i * LDP] * P[i * LDP];
        sig[g] = s;
    }
    __syncthreads();
    // T[0:k, k] = -tau_k T[0:k, 0:k] G[0:k, k], from the G column published by step k
    auto t_column = [&](int k) {
        if (tid < k) {
            T acc = 0;
            for (int j = tid; j < k; ++j) acc += Tl[tid * NB + j] * gk[j];
            Tl[tid * NB + k] = -tau[k] * acc;
        }
        if (tid == 0) Tl[k * NB + k] = tau[k];
    };
    for (int k = 0; k < kr; ++k) {
        if (k > 0) t_column(k - 1);
        if (tid == 0) {
            T sigma = 0;
#pragma unroll
            for (int q = 0; q < 8; ++q) sigma += sig[q];
            const T x0 = P[k * LDP + k];
            T t = 0, scale = 0;
            if (sigma > 0) {
                const T mu = sqrt(x0 * x0 + sigma);
                const T v0 = x0 <= 0 ? x0 - mu : -sigma / (x0 + mu);
                t = 2 * v0 * v0 / (sigma + v0 * v0);
                scale = 1 / v0;
                P[k * LDP + k] = mu;  // R_kk; column k, row k is not read by pass 1 below
            }
            tau[k] = t;
            bc[0] = scale;
            bc[1] = t;
        }
        __syncthreads();
        const T scale = bc[0], t = bc[1];
        // pass 1: d_c = P[k][c] (v_k[k] = 1; for c == k the row-k value is R_kk, unused)
        //             + sum_{i > k} scale * P[i][k] * P[i][c]
        T d0 = 0, d1 = 0;
        int i = k + 1 + g;
        for (; i + 8 < rows; i += 16) {
            d0 += P[i * LDP + k] * P[i * LDP + c];
            d1 += P[(i + 8) * LDP + k] * P[(i + 8) * LDP + c];
        }
        if (i < rows) d0 += P[i * LDP + k] * P[i * LDP + c];
        dots[g * 32 + c] = (d0 + d1) * scale;
        __syncthreads();
        T dc = P[k * LDP + c];
#pragma unroll
        for (int q = 0; q < 8; ++q) dc += dots[q * 32 + c];
        // pass 2
        if (t != 0 && c > k) {
            const T wc = t * dc;
            if (g == 0) P[k * LDP + c] -= wc;
            T s2 = 0;
            for (int r = k + 1 + g; r < rows; r += 8) {
                const T nv = P[r * LDP + c] - wc * scale * P[r * LDP + k];
                P[r * LDP + c] = nv;
                if (c == k + 1 && r > k + 1) s2 += nv * nv;
            }
            if (c == k + 1) sig[g] = s2;
        } else if (t == 0 && c == k + 1) {
            T s2 = 0;
            for (int r = k + 2 + g; r < rows; r += 8) s2 += P[r * LDP + c] * P[r * LDP + c];
            sig[g] = s2;
        }
        if (c == k && t != 0)
            for (int r = k + 1 + g; r < rows; r += 8) P[r * LDP + k] *= scale;
        if (g == 0 && c < k) gk[c] = dc;  // G[c][k] = v_c^T v_k
        __syncthreads();
    }
    if (kr > 0) t_column(kr - 1);
    for (int k = kr + tid; k < NB; k += 256) tau[k] = 0;
    __syncthreads();
}

// LDS budget of the QR kernels: panel rows x LDP + tau + T + reduction scratch
template <typename T>
struct QrLds {
    T P[Cfg<T>::RB * LDP];
    T tau[NB];
    T Tl[NB * NB];
    T red[272 + NB];
};

// ---- direct panel: m <= RB rows, one workgroup
template <typename T>
__global__ __launch_bounds__(256) void k_panel_direct(T *__restrict__ Pg, int64_t lda, int m, T *__restrict__ V,
                                                      T *__restrict__ Tm)
{
    __shared__ QrLds<T> L;
    const int tid = threadIdx.x;
    for (int idx = tid; idx < m * NB; idx += 256) {
        const int i = idx / NB, c = idx % NB;
        L.P[i * LDP + c] = Pg[i * lda + c];
    }
    __syncthreads();
    const int kr = min(m - 1, NB);
    lds_qr_larft<T>(L.P, m, kr, L.tau, L.Tl, L.red);
    for (int idx = tid; idx < m * NB; idx += 256) {
        const int i = idx / NB, c = idx % NB;
        if (i <= c) Pg[i * lda + c] = L.P[i * LDP + c];
        T v = 0;
        if (c < kr) v = i == c ? (T)1 : (i > c ? L.P[i * LDP + c] : (T)0);
        V[(int64_t)i * NB + c] = v;
    }
    for (int p = tid; p < NB * NB; p += 256) Tm[p] = L.Tl[p];
}

// ---- TSQR, step 1: local QR of row block b (rows [b*per, min(m, (b+1)*per)))
template <typename T>
__global__ __launch_bounds__(256) void k_tsqr_local(const T *__restrict__ Pg, int64_t lda, int m, int per,
                                                    T *__restrict__ Vloc, T *__restrict__ Tloc,
                                                    T *__restrict__ Rstack)
{
    __shared__ QrLds<T> L;
    const int tid = threadIdx.x;
    const int b = blockIdx.x;
    const int r0 = b * per;
    const int rows = min(per, m - r0);
    for (int idx = tid; idx < rows * NB; idx += 256) {
        const int i = idx / NB, c = idx % NB;
        L.P[i * LDP + c] = Pg[(int64_t)(r0 + i) * lda + c];
    }
    __syncthreads();
    lds_qr_larft<T>(L.P, rows, NB, L.tau, L.Tl, L.red);
    for (int idx = tid; idx < rows * NB; idx += 256) {
        const int i = idx / NB, c = idx % NB;
        Vloc[(int64_t)(r0 + i) * NB + c] = i == c ? (T)1 : (i > c ? L.P[i * LDP + c] : (T)0);
    }
    for (int p = tid; p < NB * NB; p += 256) {
        const int i = p / NB, c = p % NB;
        Rstack[(int64_t)b * NB * NB + p] = i <= c ? L.P[i * LDP + c] : (T)0;
        Tloc[(int64_t)b * NB * NB + p] = L.Tl[p];
    }
}

// ---- TSQR, step 2: QR of the stacked R factors; Rf and Qt = Q_top [I; 0]
template <typename T>
__global__ __launch_bounds__(256) void k_tsqr_top(const T *__restrict__ Rstack, int nblk, T *__restrict__ Rf,
                                                  T *__restrict__ Qt)
{
    __shared__ QrLds<T> L;
    __shared__ T K[NB * NB];
    const int tid = threadIdx.x;
    const int rows = nblk * NB;
    for (int idx = tid; idx < rows * NB; idx += 256) L.P[(idx / NB) * LDP + idx % NB] = Rstack[idx];
    __syncthreads();
    lds_qr_larft<T>(L.P, rows, NB, L.tau, L.Tl, L.red);
    // K = T V_top[0:NB]^T  (NB x NB); V_top[0:NB] is unit lower triangular
    for (int p = tid; p < NB * NB; p += 256) {
        const int j = p / NB, c = p % NB;  // K[j][c] = sum_l T[j][l] V[c][l]
        T s = 0;
        for (int l = j; l < NB; ++l) {
            const T vcl = c == l ? (T)1 : (c > l ? L.P[c * LDP + l] : (T)0);
            s += L.Tl[j * NB + l] * vcl;
        }
        K[p] = s;
    }
    for (int p = tid; p < NB * NB; p += 256) {
        const int i = p / NB, c = p % NB;
        Rf[p] = i <= c ? L.P[i * LDP + c] : (T)0;
    }
    __syncthreads();
    // Qt[r][c] = [r == c] - sum_j V[r][j] K[j][c]
    for (int idx = tid; idx < rows * NB; idx += 256) {
        const int r = idx / NB, c = idx % NB;
        T s = r == c ? (T)1 : (T)0;
        for (int j = 0; j < NB; ++j) {
            const T vrj = r == j ? (T)1 : (r > j ? L.P[r * LDP + j] : (T)0);
            s -= vrj * K[j * NB + c];
        }
        Qt[idx] = s;
    }
}

// ---- TSQR, step 3: Q1 rows of block b = [Qt_b; 0] - V_b (T_b V_b[0:NB]^T Qt_b)
template <typename T>
__global__ __launch_bounds__(256) void k_tsqr_q1(const T *__restrict__ Vloc, const T *__restrict__ Tloc,
                                                 const T *__restrict__ Qt, int m, int per, T *__restrict__ Q1)
{
    __shared__ T Vt[NB * NB], Tb[NB * NB], Qb[NB * NB], Y[NB * NB], K[NB * NB];
    const int tid = threadIdx.x;
    const int b = blockIdx.y;
    const int r0 = b * per;
    const int rows = min(per, m - r0);
    for (int p = tid; p < NB * NB; p += 256) {
        Vt[p] = Vloc[(int64_t)(r0 + p / NB) * NB + p % NB];
        Tb[p] = Tloc[(int64_t)b * NB * NB + p];
        Qb[p] = Qt[(int64_t)b * NB * NB + p];
    }
    __syncthreads();
    // Y = V_b[0:NB]^T Qt_b ; K = T_b Y
    for (int p = tid; p < NB * NB; p += 256) {
        const int j = p / NB, c = p % NB;
        T s = 0;
        for (int l = j; l < NB; ++l) s += Vt[l * NB + j] * Qb[l * NB + c];
        Y[p] = s;
    }
    __syncthreads();
    for (int p = tid; p < NB * NB; p += 256) {
        const int j = p / NB, c = p % NB;
        T s = 0;
        for (int l = j; l < NB; ++l) s += Tb[j * NB + l] * Y[l * NB + c];
        K[p] = s;
    }
    __syncthreads();
    const int i = blockIdx.x * 8 + (tid >> 5);  // row within the block
    const int c = tid & 31;
    if (i < rows) {
        T s = i < NB ? Qb[i * NB + c] : (T)0;
        const T *vr = Vloc + (int64_t)(r0 + i) * NB;
        for (int j = 0; j < NB; ++j) s -= vr[j] * K[j * NB + c];
        Q1[(int64_t)(r0 + i) * NB + c] = s;
    }
}

// ---- TSQR, step 4: Householder reconstruction from Q1's top block
template <typename T>
__global__ __launch_bounds__(256) void k_tsqr_recon(const T *__restrict__ Q1, const T *__restrict__ Rf,
                                                    T *__restrict__ Pg, int64_t lda, T *__restrict__ V,
                                                    T *__restrict__ Ug, T *__restrict__ Tm)
{
    __shared__ T M[NB * LDP];
    __shared__ T S[NB];
    const int tid = threadIdx.x;
    for (int p = tid; p < NB * NB; p += 256) M[(p / NB) * LDP + p % NB] = Q1[p];
    __syncthreads();
    for (int k = 0; k < NB; ++k) {
        if (tid == 0) {
            const T s = M[k * LDP + k] >= 0 ? (T)-1 : (T)1;
            S[k] = s;
            M[k * LDP + k] -= s;
        }
        __syncthreads();
        const T piv = M[k * LDP + k];
        for (int i = k + 1 + tid; i < NB; i += 256) M[i * LDP + k] /= piv;
        __syncthreads();
        for (int p = tid; p < NB * NB; p += 256) {
            const int i = p / NB, j = p % NB;
            if (i > k && j > k) M[i * LDP + j] -= M[i * LDP + k] * M[k * LDP + j];
        }
        __syncthreads();
    }
    // T = -(U S) Y1^{-T}: row i solves z Y1^T = -(U S)[i], by forward substitution
    if (tid < NB) {
        const int i = tid;
        T z[NB];
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            T b = j >= i ? -M[i * LDP + j] * S[j] : (T)0;
            for (int l = 0; l < j; ++l) b -= M[j * LDP + l] * z[l];
            z[j] = b;
        }
#pragma unroll
        for (int j = 0; j < NB; ++j) Tm[i * NB + j] = z[j];
    }
    for (int p = tid; p < NB * NB; p += 256) {
        const int i = p / NB, j = p % NB;
        Ug[p] = j >= i ? M[i * LDP + j] : (T)0;
        V[p] = i == j ? (T)1 : (i > j ? M[i * LDP + j] : (T)0);
        if (i <= j) Pg[i * lda + j] = S[i] * Rf[p];  // R_panel = S R
    }
}

// ---- TSQR, step 5: V rows NB.. = Q1 rows U^{-1}
template <typename T>
__global__ __launch_bounds__(256) void k_tsqr_y2(const T *__restrict__ Q1, const T *__restrict__ Ug, int m,
                                                 T *__restrict__ V)
{
    __shared__ T U[NB * LDP];
    const int tid = threadIdx.x;
    for (int p = tid; p < NB * NB; p += 256) U[(p / NB) * LDP + p % NB] = Ug[p];
    __syncthreads();
    const int64_t r = NB + blockIdx.x * 256 + tid;
    if (r >= m) return;
    T q[NB], y[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) q[j] = Q1[r * NB + j];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
        T s = q[j];
#pragma unroll
        for (int l = 0; l < j; ++l) s -= y[l] * U[l * LDP + j];
        y[j] = s / U[j * LDP + j];
    }
#pragma unroll
    for (int j = 0; j < NB; ++j) V[r * NB + j] = y[j];
}

// ---- W = V T (m x NB)
template <typename T>
__global__ __launch_bounds__(256) void k_make_w(const T *__restrict__ V, const T *__restrict__ Tm, int m,
                                                T *__restrict__ W)
{
    __shared__ T Ts[NB * NB];
    const int tid = threadIdx.x;
    for (int p = tid; p < NB * NB; p += 256) Ts[p] = Tm[p];
    __syncthreads();
    const int64_t r = blockIdx.x * 8 + (tid >> 5);
    const int c = tid & 31;
    if (r >= m) return;
    T s = 0;
    for (int j = 0; j <= c; ++j) s += V[r * NB + j] * Ts[j * NB + c];
    W[r * NB + c] = s;
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
    constexpr int NACC = sizeof(T) == 4 ? 1 : 4;
    f32x16_t acc32 = {};
    f64x4_t acc64[4] = {};
    for (int j0 = jlo; j0 < jhi; j0 += SY_JB) {
        const bool lowerTile = j0 + SY_JB - 1 <= i0;
        const bool upperTile = i0 + SY_RB - 1 < j0;
        if (lowerTile) {
            for (int idx = tid; idx < SY_RB * SY_JB; idx += 256) {
                const int r = idx / SY_JB, c = idx % SY_JB;
                const int i = i0 + r, j = j0 + c;
                As[r * (SY_JB + 1) + c] = (i < m && j < jhi) ? A[(int64_t)i * lda + j] : (T)0;
            }
        } else if (upperTile) {
            for (int idx = tid; idx < SY_RB * SY_JB; idx += 256) {
                const int c = idx / SY_RB, r = idx % SY_RB;
                const int i = i0 + r, j = j0 + c;
                As[r * (SY_JB + 1) + c] = (i < m && j < jhi) ? A[(int64_t)j * lda + i] : (T)0;
            }
        } else {
            for (int idx = tid; idx < SY_RB * SY_JB; idx += 256) {
                const int r = idx / SY_JB, c = idx % SY_JB;
                const int i = i0 + r, j = j0 + c;
                T v = 0;
                if (i < m && j < jhi) v = i >= j ? A[(int64_t)i * lda + j] : A[(int64_t)j * lda + i];
                As[r * (SY_JB + 1) + c] = v;
            }
        }
        for (int idx = tid; idx < SY_JB * NB; idx += 256) {
            const int r = idx / NB, c = idx % NB;
            const int j = j0 + r;
            Ws[r * (NB + 1) + c] = j < jhi ? W[(int64_t)j * NB + c] : (T)0;
        }
        __syncthreads();
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
    }
    T *Xp = Xpart + (int64_t)blockIdx.y * m * NB;
    (void)NACC;
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

// ---- X = sum of partials; Ppart[blk] = V_blk^T X_blk
template <typename T>
__global__ __launch_bounds__(256) void k_xreduce(const T *__restrict__ Xpart, int ks, int m, const T *__restrict__ V,
                                                 T *__restrict__ X, T *__restrict__ Ppart)
{
    __shared__ T Xs[256 * NB];
    __shared__ T Vs[256 * NB];
    const int tid = threadIdx.x;
    const int r0 = blockIdx.x * 256;
    const int rows = min(256, m - r0);
    for (int idx = tid; idx < rows * NB; idx += 256) {
        const int64_t g = (int64_t)r0 * NB + idx;
        T s = 0;
        for (int q = 0; q < ks; ++q) s += Xpart[(int64_t)q * m * NB + g];
        X[g] = s;
        Xs[idx] = s;
        Vs[idx] = V[g];
    }
    __syncthreads();
    for (int p = tid; p < NB * NB; p += 256) {
        const int j = p / NB, c = p % NB;
        T s = 0;
        for (int r = 0; r < rows; ++r) s += Vs[r * NB + j] * Xs[r * NB + c];
        Ppart[(int64_t)blockIdx.x * NB * NB + p] = s;
    }
}

// ---- M = T^T sum(Ppart)
template <typename T>
__global__ __launch_bounds__(256) void k_mfin(const T *__restrict__ Ppart, int nblk, const T *__restrict__ Tm,
                                              T *__restrict__ Mm)
{
    __shared__ T P[NB * NB];
    const int tid = threadIdx.x;
    for (int p = tid; p < NB * NB; p += 256) {
        T s = 0;
        for (int b = 0; b < nblk; ++b) s += Ppart[(int64_t)b * NB * NB + p];
        P[p] = s;
    }
    __syncthreads();
    for (int p = tid; p < NB * NB; p += 256) {
        const int i = p / NB, c = p % NB;
        T s = 0;
        for (int l = 0; l <= i; ++l) s += Tm[l * NB + i] * P[l * NB + c];  // T^T is lower
        Mm[p] = s;
    }
}

// ---- Z = X - V M / 2  (in place in X)
template <typename T>
__global__ __launch_bounds__(256) void k_zform(T *__restrict__ X, const T *__restrict__ V, const T *__restrict__ Mm,
                                               int m)
{
    __shared__ T Ms[NB * NB];
    const int tid = threadIdx.x;
    for (int p = tid; p < NB * NB; p += 256) Ms[p] = Mm[p];
    __syncthreads();
    const int64_t r = blockIdx.x * 8 + (tid >> 5);
    const int c = tid & 31;
    if (r >= m) return;
    T s = 0;
    for (int j = 0; j < NB; ++j) s += V[r * NB + j] * Ms[j * NB + c];
    X[r * NB + c] -= (T)0.5 * s;
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
    // L = [V | Z] rows i0.., R = [Z | V] rows j0..
    for (int idx = tid; idx < S2_T * NB; idx += 256) {
        const int r = idx / NB, c = idx % NB;
        const int i = i0 + r, j = j0 + r;
        const T vi = i < m ? V[(int64_t)i * NB + c] : (T)0, zi = i < m ? Z[(int64_t)i * NB + c] : (T)0;
        const T vj = j < m ? V[(int64_t)j * NB + c] : (T)0, zj = j < m ? Z[(int64_t)j * NB + c] : (T)0;
        Ls[r * (S2_K + 1) + c] = vi;
        Ls[r * (S2_K + 1) + NB + c] = zi;
        Rs[r * (S2_K + 1) + c] = zj;
        Rs[r * (S2_K + 1) + NB + c] = vj;
    }
    __syncthreads();
    const int wm = wave >> 1, wn = wave & 1;
    if (diag && wm == 0 && wn == 1) return;
    if constexpr (sizeof(T) == 4) {
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
            for (int qb = 0; qb < 2; ++qb) {
                const int j = j0 + wn * 64 + qb * 32 + (lane & 31);
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int i = i0 + wm * 64 + qa * 32 + (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3);
                    if (i < m && j < m && i >= j) A[(int64_t)i * lda + j] -= acc[qa][qb][e];
                }
            }
    } else {
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
#pragma unroll
        for (int qa = 0; qa < 4; ++qa)
#pragma unroll
            for (int qb = 0; qb < 4; ++qb) {
                const int j = j0 + wn * 64 + qb * 16 + (lane & 15);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int i = i0 + wm * 64 + qa * 16 + (lane >> 4) + 4 * e;
                    if (i < m && j < m && i >= j) A[(int64_t)i * lda + j] -= acc[qa][qb][e];
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

template <typename T>
__device__ __forceinline__ T wave_sum(T x)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
    return x;
}

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

// Orders LDS traffic between the lanes of one wave (a wave's LDS operations
// complete in program order; this keeps the compiler from moving them).
__device__ __forceinline__ void wave_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// One workgroup of G waves per group of G consecutive sweeps s0 .. s0+G-1.
// At time step t wave i runs task (s0 + i, t - 2 (s0 + i)): the tasks of one
// time step touch disjoint rows and depend only on tasks of earlier steps
// ("(s, k) after (s - 1, k + 1)"), so the G waves run them side by side.  The
// rows of the group stay in an LDS ring (row r at slot r & (CAPR - 1), its band
// entries A[r][r - j] contiguous).  The lead sweep s0 loads each row once, after
// the previous group's watermark has passed it; after every time step the rows
// no future task of the group touches are stored back and the group's
// watermark moves.
template <typename T, int G, int CAPR>
__global__ __launch_bounds__(64 * G) void k_bulge(T *__restrict__ band, int64_t n, int32_t *__restrict__ wm,
                                                  uint64_t spin_ticks)
{
    static_assert((CAPR & (CAPR - 1)) == 0 && 2 * G * NB + NB <= CAPR, "ring too small");
    constexpr int LDW = BW + 1;
    __shared__ T WR[CAPR * LDW];
    __shared__ T vsw[G][NB];
    __shared__ T red[G][NB];
    __shared__ int go;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int ci = lane & 31, h = lane >> 5;
    const int nn = (int)n;
    const int nsw = nn - 2;
    int32_t *err = wm + n;
    const int g = blockIdx.x;
    const int s0 = g * G;
    const int Ge = min(G, nsw - s0);
    auto E = [&](int r, int c) -> T & { return WR[(r & (CAPR - 1)) * LDW + (r - c)]; };
    auto ntasks = [&](int s) { return (nn - 2 - s) / NB + 1; };
    // a task (s, k) reads and writes only rows s + 1 + k NB .. s + (k + 1) NB
    auto minrow = [&](int s, int k) { return k <= 0 ? s + 1 : s + 1 + k * NB; };

    int lw = s0 + 1;   // rows [s0 + 1, lw) are in the ring
    int wmk = s0 + 1;  // rows [s0 + 1, wmk) have been stored back
    T taup = 0;        // this wave's previous reflector (v in vsw[wv])
    for (int t = 2 * s0;; ++t) {
        // ---- the lead sweep's rows, once the previous group has released them
        const int k0 = t - 2 * s0;
        if (k0 < ntasks(s0)) {
            const int r1 = min(s0 + (k0 + 1) * NB, nn - 1);
            if (r1 >= lw) {
                if (g > 0) {
                    if (tid == 0) {
                        int ok = 1;
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
                        if (!ok) cstore(err, 1);
                        go = ok;
                    }
                    __syncthreads();
                    if (!go) return;
                }
                if (r1 + 1 - wmk > CAPR) {  // cannot happen: the ring holds (2G + 1) NB rows
                    if (tid == 0) cstore(err, 2);
                    return;
                }
                const int cnt = r1 + 1 - lw;  // <= NB
                if (wv == 0) {
                    T tmp[NB];
#pragma unroll
                    for (int q = 0; q < NB; ++q) tmp[q] = q < cnt ? cload(band + (int64_t)(lw + q) * BW + lane) : (T)0;
#pragma unroll
                    for (int q = 0; q < NB; ++q)
                        if (q < cnt) E(lw + q, lw + q - lane) = tmp[q];
                }
                lw = r1 + 1;
                __syncthreads();
            }
        }
        // ---- this wave's task
        const int s = s0 + wv;
        const int k = t - 2 * s;
        if (wv < Ge && k >= 0 && k < ntasks(s)) {
            const int r0 = s + 1 + k * NB;
            const int r1 = min(s + (k + 1) * NB, nn - 1);
            const int L = r1 - r0 + 1;
            T *v = vsw[wv];
            T tau_k = 0, mu = 0;
            if (k == 0) {
                const T x = lane < L ? E(r0 + lane, s) : (T)0;
                const T sigma = wave_sum(lane >= 1 && lane < L ? x * x : (T)0);
                const T x0 = __shfl(x, 0, 64);
                T vi = 0;
                if (sigma > 0) {
                    mu = sqrt(x0 * x0 + sigma);
                    const T v0 = x0 <= 0 ? x0 - mu : -sigma / (x0 + mu);
                    tau_k = 2 * v0 * v0 / (sigma + v0 * v0);
                    vi = lane == 0 ? (T)1 : x / v0;
                    if (lane < L) E(r0 + lane, s) = lane == 0 ? mu : (T)0;
                }
                if (lane < NB) v[lane] = vi;
            } else {
                const int c0 = r0 - NB;
                // right: O <- O (I - taup vp vp^T), O = A[r0.., c0..c0+NB)
                if (taup != 0) {
                    T u = 0;
                    if (ci < L)
#pragma unroll
                        for (int c = 0; c < 16; ++c) u += E(r0 + ci, c0 + h * 16 + c) * v[h * 16 + c];
                    u += __shfl_xor(u, 32, 64);
                    if (ci < L)
#pragma unroll
                        for (int c = 0; c < 16; ++c) E(r0 + ci, c0 + h * 16 + c) -= taup * u * v[h * 16 + c];
                    wave_sync();
                }
                // reflector from column c0
                const T x = lane < L ? E(r0 + lane, c0) : (T)0;
                const T sigma = wave_sum(lane >= 1 && lane < L ? x * x : (T)0);
                const T x0 = __shfl(x, 0, 64);
                T vi = 0;
                if (sigma > 0) {
                    mu = sqrt(x0 * x0 + sigma);
                    const T v0 = x0 <= 0 ? x0 - mu : -sigma / (x0 + mu);
                    tau_k = 2 * v0 * v0 / (sigma + v0 * v0);
                    vi = lane == 0 ? (T)1 : x / v0;
                }
                wave_sync();
                if (lane < NB) v[lane] = lane < L ? vi : (T)0;
                wave_sync();
                if (tau_k != 0) {
                    // left: O <- (I - tau v v^T) O; column c0 becomes mu e_0
                    T w = 0;
                    for (int r = h; r < L; r += 2) w += v[r] * E(r0 + r, c0 + ci);
                    w += __shfl_xor(w, 32, 64);
                    for (int r = h; r < L; r += 2) E(r0 + r, c0 + ci) -= tau_k * v[r] * w;
                    wave_sync();
                    if (lane < L) E(r0 + lane, c0) = lane == 0 ? mu : (T)0;
                }
            }
            wave_sync();
            if (tau_k != 0) {
                // two-sided on the diagonal block A[r0..r1, r0..r1] (lower part stored)
                T p = 0;
                if (ci < L)
                    for (int j = h * 16; j < min(L, h * 16 + 16); ++j)
                        p += (j <= ci ? E(r0 + ci, r0 + j) : E(r0 + j, r0 + ci)) * v[j];
                p += __shfl_xor(p, 32, 64);
                p *= tau_k;
                const T vci = ci < L ? v[ci] : (T)0;
                const T pv = wave_sum(h == 0 ? p * vci : (T)0);
                if (h == 0) red[wv][ci] = ci < L ? p - (T)0.5 * tau_k * pv * vci : (T)0;
                wave_sync();
                for (int r = h; r < L; r += 2)
                    if (ci <= r) E(r0 + r, r0 + ci) -= v[r] * red[wv][ci] + red[wv][r] * v[ci];
            }
            taup = tau_k;
        }
        __syncthreads();
        // ---- rows below the first row of every remaining task are final
        int nwm = lw;
        bool more = false;
        for (int i = 0; i < Ge; ++i) {
            const int kk = t + 1 - 2 * (s0 + i);
            if (kk < ntasks(s0 + i)) {
                nwm = min(nwm, minrow(s0 + i, kk));
                more = true;
            }
        }
        if (!more) break;
        if (nwm > wmk) {
            if (wv == 0) {
                for (int r = wmk; r < nwm; ++r) cstore(band + (int64_t)r * BW + lane, E(r, r - lane));
                __builtin_amdgcn_s_waitcnt(0);
                wave_sync();
                if (lane == 0) cstore(wm + g, (int32_t)nwm);
            }
            wmk = nwm;
        }
    }
    if (wv == 0) {
        for (int r = wmk; r < lw; ++r) cstore(band + (int64_t)r * BW + lane, E(r, r - lane));
        __builtin_amdgcn_s_waitcnt(0);
        wave_sync();
        if (lane == 0) cstore(wm + g, (int32_t)nn);
    }
}

// ---------------------------------------------------------------- stage 3

template <typename T>
__global__ __launch_bounds__(256) void k_tridiag_prep(const T *__restrict__ band, int64_t n, double *__restrict__ dd,
                                                      double *__restrict__ ee2, double *__restrict__ bounds)
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
    T *band, *V, *W, *X, *Xpart, *Q1, *Vloc, *Tloc, *Rstack, *Rf, *Qt, *U, *Tm, *Mm, *Ppart;
    int32_t *prog;
    double *dd, *ee2, *bounds;
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
    b.Qt = ws.take<T>((size_t)32 * NB * NB);
    b.U = ws.take<T>((size_t)NB * NB);
    b.Tm = ws.take<T>((size_t)NB * NB);
    b.Mm = ws.take<T>((size_t)NB * NB);
    b.Ppart = ws.take<T>((size_t)cdiv_h(n, 256) * NB * NB);
    b.dd = ws.take<double>((size_t)n);
    b.ee2 = ws.take<double>((size_t)n);
    b.bounds = ws.take<double>(4);
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
    constexpr int TOP_BLOCKS = RB / NB;  // stacked R rows fit the LDS panel
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
            hipLaunchKernelGGL(k_tsqr_local<T>, dim3(nblk), dim3(256), 0, st, P, lda, (int)m, per, b.Vloc, b.Tloc,
                               b.Rstack);
            LAUNCH_OK();
            hipLaunchKernelGGL(k_tsqr_top<T>, dim3(1), dim3(256), 0, st, b.Rstack, nblk, b.Rf, b.Qt);
            LAUNCH_OK();
            hipLaunchKernelGGL(k_tsqr_q1<T>, dim3((unsigned)cdiv_h(per, 8), nblk), dim3(256), 0, st, b.Vloc, b.Tloc,
                               b.Qt, (int)m, per, b.Q1);
            LAUNCH_OK();
            hipLaunchKernelGGL(k_tsqr_recon<T>, dim3(1), dim3(256), 0, st, b.Q1, b.Rf, P, lda, b.V, b.U, b.Tm);
            LAUNCH_OK();
            hipLaunchKernelGGL(k_tsqr_y2<T>, dim3((unsigned)cdiv_h(m - NB, 256)), dim3(256), 0, st, b.Q1, b.U,
                               (int)m, b.V);
            LAUNCH_OK();
        }
        hipLaunchKernelGGL(k_make_w<T>, dim3((unsigned)cdiv_h(m, 8)), dim3(256), 0, st, b.V, b.Tm, (int)m, b.W);
        LAUNCH_OK();
        const int nrb = (int)cdiv_h(m, SY_RB);
        int ks = (int)std::min<int64_t>(KS_MAX, std::max<int64_t>(1, cdiv_h(512, nrb)));
        int chunk = (int)(cdiv_h(cdiv_h(m, ks), SY_JB) * SY_JB);
        ks = (int)cdiv_h(m, chunk);
        hipLaunchKernelGGL(k_symm<T>, dim3(nrb, ks), dim3(256), 0, st, A22, lda, (int)m, b.W, b.Xpart, chunk);
        LAUNCH_OK();
        const int nxb = (int)cdiv_h(m, 256);
        hipLaunchKernelGGL(k_xreduce<T>, dim3(nxb), dim3(256), 0, st, b.Xpart, ks, (int)m, b.V, b.X, b.Ppart);
        LAUNCH_OK();
        hipLaunchKernelGGL(k_mfin<T>, dim3(1), dim3(256), 0, st, b.Ppart, nxb, b.Tm, b.Mm);
        LAUNCH_OK();
        hipLaunchKernelGGL(k_zform<T>, dim3((unsigned)cdiv_h(m, 8)), dim3(256), 0, st, b.X, b.V, b.Mm, (int)m);
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
        constexpr int CAPR = sizeof(T) == 4 ? 512 : 256;
        const int64_t nsw = n - 2;
        const int64_t ngroups = cdiv_h(nsw, G);
        const uint64_t spin_ticks = 100000000ull * 10;  // 10 s at the 100 MHz real-time counter
        hipLaunchKernelGGL((k_bulge<T, G, CAPR>), dim3((unsigned)ngroups), dim3(64 * G), 0, st, b.band, n, b.prog,
                           spin_ticks);
        LAUNCH_OK();
    }
    // ---- stage 3: eigenvalues of the tridiagonal
    hipLaunchKernelGGL(k_tridiag_prep<T>, dim3(1), dim3(256), 0, st, b.band, n, b.dd, b.ee2, b.bounds);
    LAUNCH_OK();
    const double rel_tol = sizeof(T) == 4 ? 1e-9 : 4e-16;
    hipLaunchKernelGGL(k_bisect<T>, dim3((unsigned)cdiv_h(n, 4)), dim3(64), 0, st, b.dd, b.ee2, n, b.bounds, rel_tol,
                       w);
    LAUNCH_OK();
    if (info != nullptr) {
        hipLaunchKernelGGL(k_info, dim3(1), dim3(64), 0, st, b.prog + n, info);
        LAUNCH_OK();
    }
    return hipSuccess;
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
