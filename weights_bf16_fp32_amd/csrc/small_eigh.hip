// Eigenpairs of a batch of small symmetric matrices (the sliding-window
// covariances of "Random matrix theory spectral methods", section 3.1: the
// window decomposition gives the eigenvalues and the eigenvectors) by parallel
// cyclic Jacobi with the rotations accumulated into V.
//
// One wave per matrix, padded to 32 x 32 with zeros (the padding never couples
// to the matrix: its off-diagonal entries stay exactly zero, so no rotation
// touches it, and it is left out of the ranking).  B and V live in LDS,
// double-buffered.  Step r of a sweep pairs the indices by the round-robin
// tournament (31 with r, i with (2r - i) mod 31), which meets every pair once
// in 31 steps; the 16 disjoint rotations of a step are applied together as
// B <- J^T B J, V <- V J, every new entry a 4-term sum of the old B.  Each
// rotation zeroes its b_pq with tan theta from tau = (b_qq - b_pp) / (2 b_pq)
// (the smaller root); a pair is left alone when
// |b_pq| <= max(2e-6 sqrt(|b_pp b_qq|), 1e-7 max|b_ij|), the level at which
// fp32 rounding keeps re-creating off-diagonal mass, and the sweeps stop when
// no pair rotates (at most 30).

#include <hip/hip_runtime.h>

#include "common.h"
#include "internal.h"

namespace {

constexpr int JN = 32;            // padded order
constexpr int JL = JN + 1;        // LDS row stride
constexpr int JEPT = JN * JN / 64;  // entries per lane

__device__ __forceinline__ int jpartner(int r, int i)
{
    return i == JN - 1 ? r : (i == r ? JN - 1 : (2 * r - i + 2 * (JN - 1)) % (JN - 1));
}

__global__ __launch_bounds__(64) void small_eigh_jacobi(spec_batch_src src, int64_t batch, int n,
                                                        float *__restrict__ w, float *__restrict__ V,
                                                        int32_t *__restrict__ info)
{
    __shared__ float Bs[2][JN * JL], Vs[2][JN * JL];
    __shared__ float4 cf[JN];  // per index: (c or s factor of its own column, of its partner's, new diagonal, rotates)
    const int64_t b = blockIdx.x;
    const int lane = threadIdx.x;
    // ---- the matrix (lower triangle of the source, mirrored), zero-padded
    float bmax = 0.f;
    bool fin = true;
    const int64_t W = src.kind == SPEC_SRC_BAND ? (src.T - n) / src.stride + 1 : 1;
    const float *base;
    if (src.kind == SPEC_SRC_DENSE) {
        base = src.a + b * src.stride_a;
    } else {
        const int64_t s = b / W, win = b % W;
        base = src.a + (s * src.T + win * src.stride) * n;  // step t of the window: base + t n
    }
#pragma unroll
    for (int k = 0; k < JEPT; ++k) {
        const int e = lane + 64 * k, r = e / JN, c = e % JN;
        float x = 0.f;
        if (r < n && c < n) {
            const int hi = max(r, c), lo = min(r, c);
            x = src.kind == SPEC_SRC_DENSE ? base[(int64_t)hi * src.lda + lo] : src.scale * base[(int64_t)hi * n + (hi - lo)];
        }
        Bs[0][r * JL + c] = x;
        Vs[0][r * JL + c] = r == c ? 1.f : 0.f;
        fin = fin && isfinite(x);
        bmax = fmaxf(bmax, fabsf(x));
    }
    float *wb = w + b * n;
    float *Vb = V + b * n * n;
    if (!__all(fin)) {  // no rotation is meaningful: every output is NaN
        const float qnan = __int_as_float(0x7fc00000);
        if (lane < n) wb[lane] = qnan;
        for (int e = lane; e < n * n; e += 64) Vb[e] = qnan;
        if (info != nullptr && lane == 0) info[b] = -1;
        return;
    }
    for (int o = 32; o > 0; o >>= 1) bmax = fmaxf(bmax, __shfl_xor(bmax, o));
    const float floor_abs = 1e-7f * bmax;
    wave_sync();
    int cur = 0, sweeps = 0;
    bool converged = false;
    for (int sweep = 0; sweep < 30 && !converged; ++sweep) {
        bool any = false;
        for (int r = 0; r < JN - 1; ++r) {
            int on = 0;
            if (lane < JN) {  // the rotation of index lane's pair (both members compute it alike)
                const int i = lane, j = jpartner(r, i), p = min(i, j), q = max(i, j);
                const float *B = Bs[cur];
                const float apq = B[p * JL + q], app = B[p * JL + p], aqq = B[q * JL + q];
                float a = 1.f, bb = 0.f, d = B[i * JL + i];
                if (fabsf(apq) > fmaxf(2e-6f * sqrtf(fabsf(app * aqq)), floor_abs)) {
                    const float tau = (aqq - app) / (2.f * apq);
                    const float at = fabsf(tau);
                    const float t = copysignf(at > 1e18f ? 0.5f / at : 1.f / (at + sqrtf(1.f + tau * tau)), tau);
                    const float c = 1.f / sqrtf(1.f + t * t), sn = t * c;
                    a = c;
                    bb = i == p ? -sn : sn;
                    d = i == p ? app - t * apq : aqq + t * apq;
                    on = 1;
                }
                cf[i] = make_float4(a, bb, d, on ? 1.f : 0.f);
            }
            if (__ballot(on) == 0) continue;  // B unchanged
            any = true;
            wave_sync();
            const float *B = Bs[cur];
            const float *Vo = Vs[cur];
            float *Bn = Bs[cur ^ 1];
            float *Vn = Vs[cur ^ 1];
            const int j = lane % JN, pj = jpartner(r, j);  // the same column for every k
            const float4 cj = cf[j];
#pragma unroll
            for (int k = 0; k < JEPT; ++k) {
                const int i = lane / JN + 2 * k, pi = jpartner(r, i);
                const float4 ci = cf[i];
                const float b00 = B[i * JL + j], b01 = B[i * JL + pj], b10 = B[pi * JL + j], b11 = B[pi * JL + pj];
                const float v0 = Vo[i * JL + j], v1 = Vo[i * JL + pj];
                float v = ci.x * (cj.x * b00 + cj.y * b01) + ci.y * (cj.x * b10 + cj.y * b11);
                v = (pi == j && ci.w != 0.f) ? 0.f : v;  // the rotated pair's b_pq
                v = i == j ? ci.z : v;
                Bn[i * JL + j] = v;
                Vn[i * JL + j] = cj.x * v0 + cj.y * v1;
            }
            cur ^= 1;
            wave_sync();
        }
        ++sweeps;
        converged = !any;
    }
    // rank of eigenvalue i < n among the first n diagonal entries: descending,
    // ties by index, a NaN (from overflow in the rotations) after every number,
    // so the ranks are a permutation and every output slot is written
    if (lane < n) {
        const int i = lane;
        const float li = Bs[cur][i * JL + i];
        int r = 0;
        for (int j = 0; j < n; ++j) {
            const float lj = Bs[cur][j * JL + j];
            const bool ni = isnan(li), nj = isnan(lj);
            const bool before = (ni || nj) ? (ni && (!nj || j < i)) : (lj > li || (lj == li && j < i));
            r += before ? 1 : 0;
        }
        wb[r] = li;
        for (int k = 0; k < n; ++k) Vb[k * n + r] = Vs[cur][k * JL + i];
    }
    if (info != nullptr && lane == 0) info[b] = converged ? sweeps : -2;
}

}  // namespace

hipError_t launch_eigh_batched(hipStream_t stream, const spec_batch_src *src, int64_t batch, int n, float *w, float *V,
                               int32_t *info)
{
    if (batch == 0) return hipSuccess;
    hipLaunchKernelGGL(small_eigh_jacobi, dim3((unsigned)batch), dim3(64), 0, stream, *src, batch, n, w, V, info);
    return hipGetLastError();
}
