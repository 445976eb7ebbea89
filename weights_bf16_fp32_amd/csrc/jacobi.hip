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
//   - the matrix is stored as packed 2 x 2 blocks of position pairs (only
//     blocks K <= L), and the indices are renumbered every step so that the
//     step's pivot pairs are always positions (2k, 2k+1): a rotation then acts
//     inside blocks, and each rotated block is written straight to the
//     positions its entries take in the next step (a second LDS buffer);
//   - lanes 0 .. n'/2 - 1 compute the step's rotations from a_pp, a_qq, a_pq
//     (t = sign(tau) / (|tau| + sqrt(1 + tau^2)), tau = (a_qq - a_pp) / (2 a_pq));
//     every other lane reads one block (16 bytes), applies J_K^T (.) J_L and
//     writes four entries, so a step has no cross-lane hazard;
//   - a pair is rotated only if |a_pq| > eps_f32 sqrt(|a_pp a_qq|); the solve
//     stops after a sweep that rotates nothing (or max_sweeps);
//   - the diagonal is sorted descending with a 64-lane bitonic network.
#include <float.h>

#include "common.h"
#include "internal.h"

namespace {

constexpr int JB_MAXN = 64;

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

// Pair-block index of the packed symmetric storage: block (K, L), K <= L, holds
// rows 2K, 2K+1 x columns 2L, 2L+1 as (a00, a01, a10, a11); a diagonal block
// keeps its off-diagonal entry in a01 only.
__device__ __forceinline__ int bidx(int K, int L) { return L * (L + 1) / 2 + K; }

// Circle-method positions: position 2k holds slot k, position 2k+1 holds slot
// np-1-k, so the step's pairs are (slot k, slot np-1-k).  From one step to the
// next every index moves from slot s to slot s-1 (slot 1 to slot np-1, slot 0
// stays), i.e. position x moves to npos(x).
__device__ __forceinline__ int slot_of(int pos, int np) { return (pos & 1) ? np - 1 - (pos >> 1) : (pos >> 1); }
__device__ __forceinline__ int pos_of(int s, int np) { return s < np / 2 ? 2 * s : 2 * (np - 1 - s) + 1; }
__device__ __forceinline__ int npos(int x, int np)
{
    const int s = slot_of(x, np);
    const int ps = s == 0 ? 0 : (s == 1 ? np - 1 : s - 1);
    return pos_of(ps, np);
}

// destination (block * 4 + component) of element (x, y) in the next step
__device__ __forceinline__ int dest(int x, int y)
{
    if ((x >> 1) > (y >> 1)) {
        const int t = x;
        x = y;
        y = t;
    }
    int comp = ((x & 1) << 1) | (y & 1);
    if ((x >> 1) == (y >> 1) && comp == 2) comp = 1;
    return bidx(x >> 1, y >> 1) * 4 + comp;
}

template <int NBL>
__global__ __launch_bounds__(64) void jacobi_batched(spec_batch_src src, int64_t batch, int n, float *__restrict__ w,
                                                     int max_sweeps, int32_t *__restrict__ info)
{
    constexpr int MAXB = (JB_MAXN / 2) * (JB_MAXN / 2 + 1) / 2;
    __shared__ float4 Bk[2][MAXB > 64 * NBL ? 64 * NBL : MAXB];
    __shared__ float4 rot[JB_MAXN / 2];

    const int64_t b = blockIdx.x;
    const int lane = threadIdx.x;
    const int np = (n + 1) & ~1;
    const int m = np / 2;
    const int nblk = m * (m + 1) / 2;

    // ---- the lane's blocks, their (K, L) and the destinations of their entries
    int KK[NBL], LL[NBL], dst[NBL][4];
#pragma unroll
    for (int j = 0; j < NBL; ++j) {
        const int blk = lane + 64 * j;
        int L = 0;
        while ((L + 1) * (L + 2) / 2 <= blk) ++L;
        KK[j] = blk - L * (L + 1) / 2;
        LL[j] = L;
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int c = 0; c < 2; ++c)
                dst[j][a * 2 + c] = dest(npos(2 * KK[j] + a, np), npos(2 * LL[j] + c, np));
    }

    // ---- load: position p holds original index slot_of(p)
    auto value = [&](int i, int j) -> float {
        if (i >= n || j >= n) return 0.f;  // the dummy index of odd n
        if (src.kind == SPEC_SRC_DENSE) {
            const int r = max(i, j), c = min(i, j);
            return src.a[b * src.stride_a + (int64_t)r * src.lda + c];
        }
        const int64_t W = (src.T - n) / src.stride + 1;
        const int64_t s = b / W, win = b % W;
        return src.scale * src.a[s * src.T * n + (win * src.stride + max(i, j)) * n + abs(i - j)];
    };
#pragma unroll
    for (int j = 0; j < NBL; ++j) {
        const int blk = lane + 64 * j;
        if (blk < nblk) {
            const int r0 = slot_of(2 * KK[j], np), r1 = slot_of(2 * KK[j] + 1, np);
            const int c0 = slot_of(2 * LL[j], np), c1 = slot_of(2 * LL[j] + 1, np);
            const float a01 = value(r0, c1);
            Bk[0][blk] = make_float4(value(r0, c0), a01, KK[j] == LL[j] ? a01 : value(r1, c0), value(r1, c1));
        }
    }
    __syncthreads();

    int cur = 0;
    int sweeps = 0;
    bool converged = false;
    for (; sweeps < max_sweeps; ++sweeps) {
        int rotated = 0;
        for (int step = 0; step < np - 1; ++step) {
            if (lane < m) {
                const float4 d = Bk[cur][bidx(lane, lane)];
                const float app = d.x, apq = d.y, aqq = d.w;
                float c = 1.f, s = 0.f, t = 0.f;
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
                rot[lane] = make_float4(c, s, t, 0.f);
            }
            __syncthreads();
            float *nx = reinterpret_cast<float *>(Bk[cur ^ 1]);
#pragma unroll
            for (int j = 0; j < NBL; ++j) {
                const int blk = lane + 64 * j;
                if (blk < nblk) {
                    const float4 a = Bk[cur][blk];
                    const float4 rK = rot[KK[j]];
                    if (KK[j] == LL[j]) {
                        if (rK.y != 0.f) {
                            nx[dst[j][0]] = a.x - rK.z * a.y;
                            nx[dst[j][3]] = a.w + rK.z * a.y;
                            nx[dst[j][1]] = 0.f;
                        } else {
                            nx[dst[j][0]] = a.x;
                            nx[dst[j][3]] = a.w;
                            nx[dst[j][1]] = a.y;
                        }
                    } else {
                        const float4 rL = rot[LL[j]];
                        const float cK = rK.x, sK = rK.y, cL = rL.x, sL = rL.y;
                        // right: columns by J_L = [[c, s], [-s, c]]; left: rows by J_K^T
                        const float r00 = cL * a.x - sL * a.y, r01 = sL * a.x + cL * a.y;
                        const float r10 = cL * a.z - sL * a.w, r11 = sL * a.z + cL * a.w;
                        nx[dst[j][0]] = cK * r00 - sK * r10;
                        nx[dst[j][1]] = cK * r01 - sK * r11;
                        nx[dst[j][2]] = sK * r00 + cK * r10;
                        nx[dst[j][3]] = sK * r01 + cK * r11;
                    }
                }
            }
            __syncthreads();
            cur ^= 1;
        }
        rotated = __any(rotated);
        if (!rotated) {
            converged = true;
            break;
        }
    }
    // after whole sweeps every index is back at its starting position
    float x = -INFINITY;
    if (lane < np && slot_of(lane, np) < n) {
        const float4 d = Bk[cur][bidx(lane >> 1, lane >> 1)];
        x = (lane & 1) ? d.w : d.x;
        if (x != x) x = INFINITY;  // a NaN sorts first as +inf so the descriptors flag it
    }
    x = wave_bcast_sort_desc(x, lane);
    if (lane < n) w[b * n + lane] = x;
    if (info != nullptr && lane == 0) info[b] = converged ? sweeps : -1;
}

}  // namespace

hipError_t launch_jacobi_batched(hipStream_t stream, const spec_batch_src *src, int64_t batch, int n, float *w,
                                 int max_sweeps, int32_t *info)
{
    if (batch == 0) return hipSuccess;
    if (n <= 32)
        hipLaunchKernelGGL(jacobi_batched<3>, dim3((unsigned)batch), dim3(64), 0, stream, *src, batch, n, w,
                           max_sweeps, info);
    else
        hipLaunchKernelGGL(jacobi_batched<9>, dim3((unsigned)batch), dim3(64), 0, stream, *src, batch, n, w,
                           max_sweeps, info);
    return hipGetLastError();
}
