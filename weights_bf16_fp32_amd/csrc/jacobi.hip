// Batched eigenvalues of small symmetric matrices (n <= 64) by parallel cyclic
// Jacobi, one 64-lane wave per matrix, the matrix resident in LDS.
//
// The pages take the spectrum of each EigenTrack window with a library
// eigvalsh and flip it to descending order ("Random matrix theory spectral
// methods" page, section 3.2 code).  Here each window's 30 x 30 Gram is
// diagonalised in place:
//   - round-robin ("circle") ordering: n' = n rounded up to even, n'/2 disjoint
//     pivot pairs per step, n' - 1 steps per sweep, so every pair (p, q) is
//     visited once per sweep and all rotations of a step commute;
//   - lanes 0 .. n'/2 - 1 compute the step's rotations from a_pp, a_qq, a_pq
//     (t = sign(tau) / (|tau| + sqrt(1 + tau^2)), tau = (a_qq - a_pp) / (2 a_pq));
//   - the update A <- J^T A J is applied by 2 x 2 blocks {p_K, q_K} x {p_L, q_L}
//     (K <= L), each block read and written by one lane, its mirror image
//     written by the same lane, so a step has no cross-lane hazard;
//   - a pair is rotated only if |a_pq| > eps_f32 sqrt(|a_pp a_qq|); the solve
//     stops after a sweep that rotates nothing (or max_sweeps);
//   - the diagonal is sorted descending with a 64-lane bitonic network.
#include <float.h>

#include "common.h"
#include "internal.h"

namespace {

constexpr int JB_MAXN = 64;
constexpr int JB_LD = JB_MAXN + 1;

// position of index slot i in round r of the circle method for n' players:
// slot 0 is fixed, the others rotate by r
__device__ __forceinline__ int circle_member(int slot, int r, int np)
{
    return slot == 0 ? 0 : 1 + (slot - 1 + r) % (np - 1);
}

__device__ __forceinline__ float wave_bcast_sort_desc(float x, int lane)
{
    // bitonic sort of 64 values across the wave, descending
#pragma unroll
    for (int k = 2; k <= 64; k <<= 1) {
#pragma unroll
        for (int j = k >> 1; j > 0; j >>= 1) {
            float y = __shfl_xor(x, j, 64);
            const bool up = ((lane & k) == 0);  // this block sorts descending if up
            const bool lower = (lane & j) == 0;
            // descending order in `up` blocks: lower lane keeps the max
            float mx = fmaxf(x, y), mn = fminf(x, y);
            x = (up == lower) ? mx : mn;
        }
    }
    return x;
}

__global__ __launch_bounds__(64) void jacobi_batched(spec_batch_src src, int64_t batch, int n, float *__restrict__ w,
                                                     int max_sweeps, int32_t *__restrict__ info)
{
    __shared__ float A[JB_MAXN * JB_LD];
    __shared__ float cs_c[JB_MAXN / 2], cs_s[JB_MAXN / 2], cs_t[JB_MAXN / 2];
    __shared__ int pp[JB_MAXN / 2], qq[JB_MAXN / 2];

    const int64_t b = blockIdx.x;
    const int lane = threadIdx.x;
    const int np = (n + 1) & ~1;
    const int m = np / 2;

    // ---- load the lower triangle and mirror it
    if (src.kind == SPEC_SRC_DENSE) {
        const float *a = src.a + b * src.stride_a;
        for (int idx = lane; idx < n * n; idx += 64) {
            int i = idx / n, j = idx % n;
            if (i >= j) {
                float v = a[i * src.lda + j];
                A[i * JB_LD + j] = v;
                A[j * JB_LD + i] = v;
            }
        }
    } else {
        const int64_t W = (src.T - n) / src.stride + 1;
        const int64_t s = b / W, win = b % W;
        const float *band = src.a + s * src.T * n;
        const int64_t t0 = win * src.stride;
        for (int idx = lane; idx < n * n; idx += 64) {
            int i = idx / n, j = idx % n;
            if (i >= j) {
                float v = src.scale * band[(t0 + i) * n + (i - j)];
                A[i * JB_LD + j] = v;
                A[j * JB_LD + i] = v;
            }
        }
    }
    if (np != n) {  // dummy index n: an isolated zero row and column
        for (int j = lane; j <= n; j += 64) {
            A[n * JB_LD + j] = 0.f;
            A[j * JB_LD + n] = 0.f;
        }
    }
    __syncthreads();

    const int nblk = m * (m + 1) / 2;
    int sweeps = 0;
    bool converged = false;
    for (; sweeps < max_sweeps; ++sweeps) {
        int rotated = 0;
        for (int r = 0; r < np - 1; ++r) {
            if (lane < m) {
                int p = circle_member(lane, r, np);
                int q = circle_member(np - 1 - lane, r, np);
                if (p > q) { int tmp = p; p = q; q = tmp; }
                float c = 1.f, s = 0.f, t = 0.f;
                if (q < n) {
                    const float apq = A[p * JB_LD + q];
                    const float app = A[p * JB_LD + p], aqq = A[q * JB_LD + q];
                    const float thr = FLT_EPSILON * sqrtf(fabsf(app)) * sqrtf(fabsf(aqq));
                    if (fabsf(apq) > thr && fabsf(apq) > FLT_MIN) {
                        const float tau = (aqq - app) / (2.f * apq);
                        if (fabsf(tau) < 1e18f)
                            t = copysignf(1.f, tau) / (fabsf(tau) + sqrtf(1.f + tau * tau));
                        else
                            t = 0.5f / tau;
                        c = 1.f / sqrtf(1.f + t * t);
                        s = t * c;
                        rotated = 1;
                    }
                }
                pp[lane] = p;
                qq[lane] = q;
                cs_c[lane] = c;
                cs_s[lane] = s;
                cs_t[lane] = t;
            }
            __syncthreads();
            for (int blk = lane; blk < nblk; blk += 64) {
                // blk -> (K, L) with K <= L
                int L = (int)((sqrtf(8.f * blk + 1.f) - 1.f) * 0.5f);
                while ((L + 1) * (L + 2) / 2 <= blk) ++L;
                while (L * (L + 1) / 2 > blk) --L;
                const int K = blk - L * (L + 1) / 2;
                const int pK = pp[K], qK = qq[K], pL = pp[L], qL = qq[L];
                const float cK = cs_c[K], sK = cs_s[K], cL = cs_c[L], sL = cs_s[L];
                if (K == L) {
                    if (sK != 0.f) {
                        const float apq = A[pK * JB_LD + qK];
                        const float tK = cs_t[K];
                        A[pK * JB_LD + pK] -= tK * apq;
                        A[qK * JB_LD + qK] += tK * apq;
                        A[pK * JB_LD + qK] = 0.f;
                        A[qK * JB_LD + pK] = 0.f;
                    }
                } else if (sK != 0.f || sL != 0.f) {
                    const float a00 = A[pK * JB_LD + pL], a01 = A[pK * JB_LD + qL];
                    const float a10 = A[qK * JB_LD + pL], a11 = A[qK * JB_LD + qL];
                    // right: columns (pL, qL) by J_L = [[c, s], [-s, c]]
                    const float r00 = cL * a00 - sL * a01, r01 = sL * a00 + cL * a01;
                    const float r10 = cL * a10 - sL * a11, r11 = sL * a10 + cL * a11;
                    // left: rows (pK, qK) by J_K^T
                    const float b00 = cK * r00 - sK * r10, b01 = cK * r01 - sK * r11;
                    const float b10 = sK * r00 + cK * r10, b11 = sK * r01 + cK * r11;
                    A[pK * JB_LD + pL] = b00;
                    A[pK * JB_LD + qL] = b01;
                    A[qK * JB_LD + pL] = b10;
                    A[qK * JB_LD + qL] = b11;
                    A[pL * JB_LD + pK] = b00;
                    A[qL * JB_LD + pK] = b01;
                    A[pL * JB_LD + qK] = b10;
                    A[qL * JB_LD + qK] = b11;
                }
            }
            __syncthreads();
        }
        rotated = __any(rotated);
        if (!rotated) {
            converged = true;
            break;
        }
    }
    float x = (lane < n) ? A[lane * JB_LD + lane] : -INFINITY;
    if (x != x) x = INFINITY;  // a NaN sorts first as +inf so the descriptors flag it
    x = wave_bcast_sort_desc(x, lane);
    if (lane < n) w[b * n + lane] = x;
    if (info != nullptr && lane == 0) info[b] = converged ? sweeps : -1;
}

}  // namespace

hipError_t launch_jacobi_batched(hipStream_t stream, const spec_batch_src *src, int64_t batch, int n, float *w,
                                 int max_sweeps, int32_t *info)
{
    if (batch == 0) return hipSuccess;
    hipLaunchKernelGGL(jacobi_batched, dim3((unsigned)batch), dim3(64), 0, stream, *src, batch, n, w, max_sweeps,
                       info);
    return hipGetLastError();
}
