// Projection compression of a square weight onto a signal-subspace basis
// ("Random matrix theory spectral methods" page, section 4.1: with
// P = [u_1 .. u_k] in R^{d x k}, the d x d layer weight W becomes
// W' = P^T W P in R^{k x k}), on gfx950.
//
//   k_wp_part    X_c = W[:, chunk c] P[chunk c, :] for 256-column chunks of W:
//                f32 MFMA 32x32x2 (bf16 weights widen exactly), 4 waves x 32 rows
//                per workgroup; the P chunk is staged transposed in LDS so a
//                lane takes its 8 consecutive k-values with two 16-byte reads.
//   k_wp_reduce  X = sum_c X_c (written when asked: the right factor W P) and the
//                partial P[rows]^T X[rows] of 32 rows.
//   k_wp_gsum    W' = the sum of the partials.
// The k columns are padded to 32 with zeros (P's columns k..31 read as 0).
#include <hip/hip_runtime.h>

#include "common.h"
#include "internal.h"

namespace {

constexpr int KP = 32;          // padded basis width
constexpr int JC = 256;         // columns of W per chunk (a multiple of 16)
constexpr int RB = 128;         // rows of W per workgroup (4 waves x 32)
constexpr int RR = 32;          // rows per workgroup of the reduction
constexpr int PL = JC + 4;      // padded LDS row of the transposed P chunk

int64_t cdiv_h(int64_t a, int64_t b) { return (a + b - 1) / b; }

// 8 consecutive weights of a row as raw registers (zero past column d), widened
// to f32 only when used, so that a whole chunk's loads are issued at once.
struct RawBF16 {
    uint4 u;
};
struct RawF32 {
    float4 a, b;
};
template <typename T>
struct RawOf;
template <>
struct RawOf<uint16_t> {
    using type = RawBF16;
};
template <>
struct RawOf<float> {
    using type = RawF32;
};

template <bool FULL>
SPEC_DEVICE RawBF16 load_raw(const uint16_t *__restrict__ row, int64_t j, int64_t d)
{
    RawBF16 r;
    if (FULL) {
        r.u = *reinterpret_cast<const uint4 *>(row + j);
    } else {
        uint32_t w[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const uint32_t lo = j + 2 * t < d ? row[j + 2 * t] : 0u;
            const uint32_t hi = j + 2 * t + 1 < d ? row[j + 2 * t + 1] : 0u;
            w[t] = lo | (hi << 16);
        }
        r.u = make_uint4(w[0], w[1], w[2], w[3]);
    }
    return r;
}
template <bool FULL>
SPEC_DEVICE RawF32 load_raw(const float *__restrict__ row, int64_t j, int64_t d)
{
    RawF32 r;
    if (FULL) {
        r.a = *reinterpret_cast<const float4 *>(row + j);
        r.b = *reinterpret_cast<const float4 *>(row + j + 4);
    } else {
        float v[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) v[t] = j + t < d ? row[j + t] : 0.f;
        r.a = make_float4(v[0], v[1], v[2], v[3]);
        r.b = make_float4(v[4], v[5], v[6], v[7]);
    }
    return r;
}
SPEC_DEVICE void widen(const RawBF16 &r, float (&v)[8])
{
    v[0] = bf16_lo(r.u.x), v[1] = bf16_hi(r.u.x), v[2] = bf16_lo(r.u.y), v[3] = bf16_hi(r.u.y);
    v[4] = bf16_lo(r.u.z), v[5] = bf16_hi(r.u.z), v[6] = bf16_lo(r.u.w), v[7] = bf16_hi(r.u.w);
}
SPEC_DEVICE void widen(const RawF32 &r, float (&v)[8])
{
    v[0] = r.a.x, v[1] = r.a.y, v[2] = r.a.z, v[3] = r.a.w, v[4] = r.b.x, v[5] = r.b.y, v[6] = r.b.z, v[7] = r.b.w;
}

// One 32-row tile of X_c for this lane's wave: W loads, basis chunk to LDS,
// then the MFMAs group by group.  FULL: the chunk lies inside the matrix.
template <typename T, bool FULL>
SPEC_DEVICE f32x16_t wp_chunk(const T *__restrict__ wr, int64_t jb, int64_t d, int h, int c,
                              const float (&pst)[KP * JC / 256], float *Pt)
{
    constexpr int NG = JC / 16;  // 16-column groups per chunk
    const int tid = threadIdx.x;
    typename RawOf<T>::type raw[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) raw[g] = load_raw<FULL>(wr, jb + 16 * g + 8 * h, d);
#pragma unroll
    for (int i = 0; i < KP * JC / 256; ++i) {
        const int q = tid + 256 * i, j = q / KP, cc = q % KP;
        Pt[cc * PL + j] = pst[i];
    }
    __syncthreads();
    f32x16_t acc;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = 0.f;
#pragma unroll
    for (int g = 0; g < NG; ++g) {
        float wv8[8];
        widen(raw[g], wv8);
        const float *pt = &Pt[c * PL + 16 * g + 8 * h];  // 16 g + 8 h + 7 < JC
        const float4 p0 = *reinterpret_cast<const float4 *>(pt);
        const float4 p1 = *reinterpret_cast<const float4 *>(pt + 4);
        const float pv[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
#pragma unroll
        for (int t = 0; t < 8; ++t) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(wv8[t], pv[t], acc, 0, 0, 0);
    }
    return acc;
}

// grid (cdiv(d, RB), cdiv(d, JC)), 256 threads.  Xpart[c][r][0..31].
template <typename T>
__global__ __launch_bounds__(256) void k_wp_part(const T *__restrict__ W, int64_t ldw, int64_t d,
                                                 const float *__restrict__ P, int64_t ldp, int k,
                                                 float *__restrict__ Xpart)
{
    __shared__ __align__(16) float Pt[KP * PL];  // Pt[c][j - j_begin]
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int64_t jb = (int64_t)blockIdx.y * JC;
    const int jn = (int)min<int64_t>(JC, d - jb);
    const int64_t row = (int64_t)blockIdx.x * RB + wv * 32 + (lane & 31);
    const int h = lane >> 5, c = lane & 31;
    // rows past d read row d - 1 (valid memory); their outputs are never stored
    const T *wr = W + min<int64_t>(row, d - 1) * ldw;
    // Load order matters: memory counters retire in issue order, so the basis
    // chunk is loaded first (the LDS stores wait for it alone), then this
    // lane's 8 columns of every group of W, whose MFMAs each wait only for
    // their own group while the later groups are still in flight.  The full
    // and the ragged chunk run separate straight-line bodies: a loaded value
    // merged across a branch would make every load wait for the previous one.
    constexpr int PPT = KP * JC / 256;  // basis values per thread
    float pst[PPT];
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
        const int q = tid + 256 * i, j = q / KP, cc = q % KP;  // coalesced over cc
        pst[i] = (j < jn && cc < k) ? P[(jb + j) * ldp + cc] : 0.f;
    }
    const f32x16_t acc = jn == JC ? wp_chunk<T, true>(wr, jb, d, h, c, pst, Pt)
                                  : wp_chunk<T, false>(wr, jb, d, h, c, pst, Pt);
    float *xp = Xpart + (int64_t)blockIdx.y * d * KP;
    const int64_t r0 = (int64_t)blockIdx.x * RB + wv * 32;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const int64_t r = r0 + 8 * (e / 4) + 4 * h + (e % 4);
        if (r < d) xp[r * KP + c] = acc[e];
    }
}

// grid cdiv(d, RR), 256 threads: X rows of this block summed over the chunks,
// then Gpart[block][a][b] = sum_r P[r][a] X[r][b].
__global__ __launch_bounds__(256) void k_wp_reduce(const float *__restrict__ Xpart, int nchunk, int64_t d,
                                                   const float *__restrict__ P, int64_t ldp, int k,
                                                   float *__restrict__ X, int64_t ldx, float *__restrict__ Gpart)
{
    __shared__ float Xs[RR * (KP + 1)], Ps[RR * (KP + 1)];
    const int tid = threadIdx.x;
    const int64_t r0 = (int64_t)blockIdx.x * RR;
    for (int q = tid; q < RR * KP; q += 256) {
        const int rr = q / KP, c = q % KP;
        const int64_t r = r0 + rr;
        float x = 0.f, p = 0.f;
        if (r < d) {
#pragma unroll 16
            for (int ch = 0; ch < nchunk; ++ch) x += Xpart[((int64_t)ch * d + r) * KP + c];
            if (c < k) {
                p = P[r * ldp + c];
                if (X != nullptr) X[r * ldx + c] = x;
            }
        }
        Xs[rr * (KP + 1) + c] = x;
        Ps[rr * (KP + 1) + c] = p;
    }
    __syncthreads();
    for (int q = tid; q < KP * KP; q += 256) {
        const int a = q / KP, b = q % KP;
        float g = 0.f;
#pragma unroll 8
        for (int rr = 0; rr < RR; ++rr) g += Ps[rr * (KP + 1) + a] * Xs[rr * (KP + 1) + b];
        Gpart[(int64_t)blockIdx.x * KP * KP + q] = g;
    }
}

// grid KP * KP / 16, 256 threads: 16 outputs per workgroup, each summed by 16
// threads over interleaved partials, then combined in LDS
__global__ __launch_bounds__(256) void k_wp_gsum(const float *__restrict__ Gpart, int nblk, int k,
                                                 float *__restrict__ Wp, int64_t ldo)
{
    __shared__ float part[16][17];
    const int o = threadIdx.x & 15, sl = threadIdx.x >> 4;
    const int q = blockIdx.x * 16 + o, a = q / KP, b = q % KP;
    float g = 0.f;
#pragma unroll 8
    for (int i = sl; i < nblk; i += 16) g += Gpart[(int64_t)i * KP * KP + q];
    part[sl][o] = g;
    __syncthreads();
    if (threadIdx.x < 16) {
        float t = 0.f;
        for (int i = 0; i < 16; ++i) t += part[i][o];
        if (a < k && b < k) Wp[a * ldo + b] = t;
    }
}

}  // namespace

size_t project_weight_workspace_bytes(int64_t d)
{
    const size_t xpart = (size_t)cdiv_h(d, JC) * (size_t)d * KP * sizeof(float);
    const size_t gpart = (size_t)cdiv_h(d, RR) * KP * KP * sizeof(float);
    return ((xpart + 255) / 256) * 256 + gpart;
}

hipError_t launch_project_weight(hipStream_t stream, const void *W, int wt, int64_t d, int64_t ldw, const float *P,
                                 int64_t ldp, int k, float *Wp, int64_t ldo, float *X, int64_t ldx, void *ws)
{
    const int nchunk = (int)cdiv_h(d, JC), nrb = (int)cdiv_h(d, RB), nrr = (int)cdiv_h(d, RR);
    float *Xpart = (float *)ws;
    float *Gpart = (float *)((char *)ws + (((size_t)nchunk * (size_t)d * KP * sizeof(float) + 255) / 256) * 256);
    const dim3 g1((unsigned)nrb, (unsigned)nchunk);
    if (wt == SPEC_BF16)
        hipLaunchKernelGGL(k_wp_part<uint16_t>, g1, dim3(256), 0, stream, (const uint16_t *)W, ldw, d, P, ldp, k,
                           Xpart);
    else
        hipLaunchKernelGGL(k_wp_part<float>, g1, dim3(256), 0, stream, (const float *)W, ldw, d, P, ldp, k, Xpart);
    SPEC_LAUNCH_CHECK();
    hipLaunchKernelGGL(k_wp_reduce, dim3((unsigned)nrr), dim3(256), 0, stream, Xpart, nchunk, d, P, ldp, k, X, ldx,
                       Gpart);
    SPEC_LAUNCH_CHECK();
    hipLaunchKernelGGL(k_wp_gsum, dim3(KP * KP / 16), dim3(256), 0, stream, Gpart, nrr, k, Wp, ldo);
    return hipGetLastError();
}
