// Screen of the swap candidates of the S3 page (section 3.1): for the left
// singular vectors u_i and right singular vectors v_j of the tail (i, j in
// [i0, i0 + t), the page's last 10 %), |u_i^T v_j|, and the pairs that lie in
// one head's index range (i / head_dim == j / head_dim) with |u_i^T v_j| < eps
// (the page keeps them below 0.015).  The page approximates this with PCA and
// an ANN index; here it is exact: the t x t product U_tail^T V_tail is a dense
// contraction over the N rows, on fp64 MFMA (v_mfma_f64_16x16x4f64) with the
// f32 or f64 inputs widened exactly, so every comparison with eps is taken in
// fp64.
//
// k_tail_dots: one workgroup per 32 x 32 output tile, four waves of 16 x 16;
//   64 rows of U and V per step through LDS.
// k_keep_count: the number of kept pairs (one workgroup, a reduction).
#include "common.h"
#include "internal.h"

namespace {

constexpr int TS = 32;  // output tile edge
constexpr int TK = 64;  // rows per step

template <typename T>
__global__ __launch_bounds__(256) void k_tail_dots(const T *__restrict__ U, int64_t ldu, const T *__restrict__ V,
                                                   int64_t ldv, int64_t n, int64_t i0, int t, int64_t head_dim,
                                                   double eps, double *__restrict__ absdot, int64_t ldo,
                                                   uint8_t *__restrict__ keep, int64_t ldk)
{
    __shared__ double Us[TK][TS + 1], Vs[TK][TS + 1];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int a0 = blockIdx.y * TS, b0 = blockIdx.x * TS;
    const int bi = wave >> 1, bj = wave & 1;
    f64x4_t acc = {0.0, 0.0, 0.0, 0.0};
    for (int64_t k0 = 0; k0 < n; k0 += TK) {
        // 64 rows x 32 columns of each factor: 8 elements per thread, the 32
        // columns of a row contiguous in memory
#pragma unroll
        for (int q = 0; q < TK * TS / 256; ++q) {
            const int idx = tid + 256 * q, kr = idx / TS, c = idx % TS;
            const int64_t k = k0 + kr;
            const bool rowok = k < n;
            Us[kr][c] = rowok && a0 + c < t ? (double)U[k * ldu + i0 + a0 + c] : 0.0;
            Vs[kr][c] = rowok && b0 + c < t ? (double)V[k * ldv + i0 + b0 + c] : 0.0;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < TK; kk += 4) {
            const double a = Us[kk + (lane >> 4)][bi * 16 + (lane & 15)];
            const double b = Vs[kk + (lane >> 4)][bj * 16 + (lane & 15)];
            acc = __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, acc, 0, 0, 0);
        }
        __syncthreads();
    }
    // result layout: lane l holds column l % 16, rows l / 16 + 4 e
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int a = a0 + bi * 16 + (lane >> 4) + 4 * e, b = b0 + bj * 16 + (lane & 15);
        if (a < t && b < t) {
            const double v = fabs(acc[e]);
            if (absdot != nullptr) absdot[(int64_t)a * ldo + b] = v;
            const bool same = (i0 + a) / head_dim == (i0 + b) / head_dim;
            keep[(int64_t)a * ldk + b] = same && v < eps ? 1 : 0;
        }
    }
}

__global__ __launch_bounds__(256) void k_keep_count(const uint8_t *__restrict__ keep, int64_t ldk, int t,
                                                    int64_t *__restrict__ count)
{
    __shared__ int64_t part[4];
    int64_t s = 0;
    for (int64_t q = threadIdx.x; q < (int64_t)t * t; q += 256) s += keep[(q / t) * ldk + q % t];
    for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = s;
    __syncthreads();
    if (threadIdx.x == 0) *count = part[0] + part[1] + part[2] + part[3];
}

}  // namespace

hipError_t launch_tail_pair_screen(hipStream_t stream, const void *U, const void *V, int dt, int64_t n, int64_t ldu,
                                   int64_t ldv, int64_t i0, int64_t t, int64_t head_dim, double eps, double *absdot,
                                   int64_t ldo, uint8_t *keep, int64_t ldk, int64_t *count)
{
    const unsigned nt = (unsigned)((t + TS - 1) / TS);
    if (dt == SPEC_F32)
        hipLaunchKernelGGL(k_tail_dots<float>, dim3(nt, nt), dim3(256), 0, stream, (const float *)U, ldu,
                           (const float *)V, ldv, n, i0, (int)t, head_dim, eps, absdot, ldo, keep, ldk);
    else
        hipLaunchKernelGGL(k_tail_dots<double>, dim3(nt, nt), dim3(256), 0, stream, (const double *)U, ldu,
                           (const double *)V, ldv, n, i0, (int)t, head_dim, eps, absdot, ldo, keep, ldk);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || count == nullptr) return e;
    hipLaunchKernelGGL(k_keep_count, dim3(1), dim3(256), 0, stream, keep, ldk, (int)t, count);
    return hipGetLastError();
}
