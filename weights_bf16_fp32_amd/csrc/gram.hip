// Sliding-window Gram of EigenTrack activations ("Random matrix theory spectral
// methods" page, section 3.1: the window H = [h_{t-N+1} .. h_t]^T of the last N
// decode steps and its covariance (1/N) H^T H).  For N << d the N x N Gram
// (1/N) H H^T has the same nonzero spectrum, and every window's Gram is a
// submatrix of the banded product <h_t, h_{t-j}>, 0 <= j < N, so the band is
// all that is computed: each activation row is read once per call instead of
// once per window containing it.
//
// gram_band_mfma (bf16, d % 8 == 0): one workgroup per (stream, block of 128
//   steps).  It stages rows [t0 - 32 (NCT - 1), t0 + 128) of the stream, 64
//   features at a time, in LDS (double-buffered, natural row-major layout: the
//   contraction runs along the features, which the MFMA wants contiguous per
//   lane).  Wave w owns the 32 steps of row tile t0 + 32 w and multiplies it
//   with itself and with the NCT - 1 preceding row tiles on
//   v_mfma_f32_32x32x16_bf16.  Only |i - j| < N of the product is stored.
// gram_band_generic: any dtype or d, VALU dot products (tests, odd shapes).
// gram_dense: scale * H_w H_w^T for each window, both triangles (small cases).
#include "common.h"
#include "internal.h"

namespace {

constexpr int GB_RB = 128;     // steps per workgroup
constexpr int GB_BK = 64;      // features per K-step
constexpr int GB_ROW = 72;     // uint16 per LDS row (64 + 8 pad)

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

template <int NCT>
__global__ __launch_bounds__(256) void gram_band_mfma(const uint16_t *__restrict__ H, int64_t streams, int64_t T,
                                                      int64_t d, int64_t ld_t, int64_t ld_s, int N,
                                                      float *__restrict__ out)
{
    constexpr int ROWS = GB_RB + 32 * (NCT - 1);  // staged rows
    __shared__ __attribute__((aligned(16))) uint16_t lds[2][ROWS * GB_ROW];

    const int64_t nrb = (T + GB_RB - 1) / GB_RB;
    const int64_t logical = xcd_remap(blockIdx.x, gridDim.x);
    const int64_t s = logical / nrb;
    const int64_t t0 = (logical % nrb) * GB_RB;
    const int64_t r_lo = t0 - 32 * (NCT - 1);
    const uint16_t *Hs = H + s * ld_s;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // loader: 8 threads per row (8 features each), 32 rows per pass
    constexpr int PASSES = (ROWS + 31) / 32;
    const int lr = tid >> 3, lc = (tid & 7) * 8;
    u32x4_t v[PASSES];
    auto gload = [&](int64_t k0) {
#pragma unroll
        for (int p = 0; p < PASSES; ++p) {
            const int r = p * 32 + lr;
            const int64_t t = r_lo + r;
            if (r < ROWS && t >= 0 && t < T && k0 + lc < d)
                v[p] = *reinterpret_cast<const u32x4_t *>(Hs + t * ld_t + k0 + lc);
            else
                v[p] = u32x4_t{0u, 0u, 0u, 0u};
        }
    };
    auto lstore = [&](int stage) {
#pragma unroll
        for (int p = 0; p < PASSES; ++p) {
            const int r = p * 32 + lr;
            if (r < ROWS) *reinterpret_cast<u32x4_t *>(&lds[stage][r * GB_ROW + lc]) = v[p];
        }
    };

    f32x16_t acc[NCT];
#pragma unroll
    for (int c = 0; c < NCT; ++c)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[c][e] = 0.f;

    // the wave's own row tile sits at staged row 32 (NCT - 1) + 32 wave
    const int own = 32 * (NCT - 1) + 32 * wave;
    const bool wave_live = t0 + 32 * wave < T;

    gload(0);
    lstore(0);
    __syncthreads();
    int cur = 0;
    for (int64_t k0 = 0; k0 < d; k0 += GB_BK) {
        const bool more = k0 + GB_BK < d;
        if (more) gload(k0 + GB_BK);
        if (wave_live) {
            const uint16_t *L = lds[cur];
#pragma unroll
            for (int kk = 0; kk < GB_BK / 16; ++kk) {
                const int koff = kk * 16 + (lane >> 5) * 8;
                bf16x8_t fr[NCT];
#pragma unroll
                for (int c = 0; c < NCT; ++c)
                    fr[c] = *reinterpret_cast<const bf16x8_t *>(L + (own - 32 * c + (lane & 31)) * GB_ROW + koff);
                // c = 0: the tile with itself; c > 0: with the tile 32 c steps earlier
#pragma unroll
                for (int c = 0; c < NCT; ++c)
                    acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[0], fr[c], acc[c], 0, 0, 0);
            }
        }
        if (more) lstore(cur ^ 1);
        __syncthreads();
        cur ^= 1;
    }
    if (!wave_live) return;
    float *outs = out + s * T * N;
    const int col = lane & 31;
#pragma unroll
    for (int c = 0; c < NCT; ++c)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int row = (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3);
            const int lag = row - col + 32 * c;  // (t0 + 32 w + row) - (t0 + 32 w - 32 c + col)
            const int64_t t = t0 + 32 * wave + row;
            if (lag >= 0 && lag < N && t < T) outs[t * N + lag] = acc[c][e];
        }
}

template <typename TIn>
__device__ __forceinline__ float ld_in(const TIn *p);
template <>
__device__ __forceinline__ float ld_in<float>(const float *p) { return *p; }
template <>
__device__ __forceinline__ float ld_in<uint16_t>(const uint16_t *p) { return bf16_to_f32(*p); }

// one workgroup per (stream, 32 steps); rows [t0 - 63, t0 + 32) staged 64 features at a time
template <typename TIn>
__global__ __launch_bounds__(256) void gram_band_generic(const TIn *__restrict__ H, int64_t streams, int64_t T,
                                                         int64_t d, int64_t ld_t, int64_t ld_s, int N,
                                                         float *__restrict__ out)
{
    __shared__ float rows[96][65];
    const int64_t nrb = (T + 31) / 32;
    const int64_t s = blockIdx.x / nrb;
    const int64_t t0 = (blockIdx.x % nrb) * 32;
    const int64_t r_lo = t0 - 64;
    const TIn *Hs = H + s * ld_s;
    // each thread owns up to 8 (t, lag) pairs of the 32 x N block
    float acc[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] = 0.f;
    for (int64_t k0 = 0; k0 < d; k0 += 64) {
        for (int idx = threadIdx.x; idx < 96 * 64; idx += 256) {
            int r = idx / 64, c = idx % 64;
            int64_t t = r_lo + r;
            rows[r][c] = (t >= 0 && t < T && k0 + c < d) ? ld_in<TIn>(Hs + t * ld_t + k0 + c) : 0.f;
        }
        __syncthreads();
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            int pair = threadIdx.x + 256 * q;
            if (pair < 32 * N) {
                int i = pair / N, lag = pair % N;
                float a = 0.f;
                for (int c = 0; c < 64; ++c) a += rows[64 + i][c] * rows[64 + i - lag][c];
                acc[q] += a;
            }
        }
        __syncthreads();
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        int pair = threadIdx.x + 256 * q;
        if (pair < 32 * N) {
            int i = pair / N, lag = pair % N;
            int64_t t = t0 + i;
            if (t < T) out[(s * T + t) * N + lag] = acc[q];
        }
    }
}

// one workgroup per (stream, window): scale * H_w H_w^T
template <typename TIn>
__global__ __launch_bounds__(256) void gram_dense(const TIn *__restrict__ H, int64_t streams, int64_t T, int64_t d,
                                                  int64_t ld_t, int64_t ld_s, int N, int stride, float scale,
                                                  float *__restrict__ out)
{
    __shared__ float rows[64][65];
    const int64_t W = (T - N) / stride + 1;
    const int64_t s = blockIdx.x / W, w = blockIdx.x % W;
    const TIn *Hw = H + s * ld_s + (w * stride) * ld_t;
    float acc[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) acc[q] = 0.f;
    for (int64_t k0 = 0; k0 < d; k0 += 64) {
        for (int idx = threadIdx.x; idx < N * 64; idx += 256) {
            int r = idx / 64, c = idx % 64;
            rows[r][c] = (k0 + c < d) ? ld_in<TIn>(Hw + r * ld_t + k0 + c) : 0.f;
        }
        __syncthreads();
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            int pair = threadIdx.x + 256 * q;
            if (pair < N * N) {
                int i = pair / N, j = pair % N;
                float a = 0.f;
                for (int c = 0; c < 64; ++c) a += rows[i][c] * rows[j][c];
                acc[q] += a;
            }
        }
        __syncthreads();
    }
    float *o = out + (s * W + w) * N * N;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        int pair = threadIdx.x + 256 * q;
        if (pair < N * N) o[pair] = scale * acc[q];
    }
}

}  // namespace

hipError_t launch_gram_band(hipStream_t stream, const void *H, int ht, int64_t streams, int64_t T, int64_t d,
                            int64_t ld_t, int64_t ld_s, int N, float *out)
{
    const bool aligned = ht == SPEC_BF16 && d % 8 == 0 && ld_t % 8 == 0 && ld_s % 8 == 0 && ((uintptr_t)H % 16) == 0;
    if (aligned) {
        const int64_t grid = streams * ((T + GB_RB - 1) / GB_RB);
        const uint16_t *h = (const uint16_t *)H;
        if (N <= 1)
            hipLaunchKernelGGL(gram_band_mfma<1>, dim3((unsigned)grid), dim3(256), 0, stream, h, streams, T, d, ld_t,
                               ld_s, N, out);
        else if (N <= 33)
            hipLaunchKernelGGL(gram_band_mfma<2>, dim3((unsigned)grid), dim3(256), 0, stream, h, streams, T, d, ld_t,
                               ld_s, N, out);
        else
            hipLaunchKernelGGL(gram_band_mfma<3>, dim3((unsigned)grid), dim3(256), 0, stream, h, streams, T, d, ld_t,
                               ld_s, N, out);
    } else {
        const int64_t grid = streams * ((T + 31) / 32);
        if (ht == SPEC_BF16)
            hipLaunchKernelGGL(gram_band_generic<uint16_t>, dim3((unsigned)grid), dim3(256), 0, stream,
                               (const uint16_t *)H, streams, T, d, ld_t, ld_s, N, out);
        else
            hipLaunchKernelGGL(gram_band_generic<float>, dim3((unsigned)grid), dim3(256), 0, stream, (const float *)H,
                               streams, T, d, ld_t, ld_s, N, out);
    }
    return hipGetLastError();
}

hipError_t launch_gram_dense(hipStream_t stream, const void *H, int ht, int64_t streams, int64_t T, int64_t d,
                             int64_t ld_t, int64_t ld_s, int N, int stride, float scale, float *out)
{
    const int64_t W = (T - N) / stride + 1;
    const int64_t grid = streams * W;
    if (ht == SPEC_BF16)
        hipLaunchKernelGGL(gram_dense<uint16_t>, dim3((unsigned)grid), dim3(256), 0, stream, (const uint16_t *)H,
                           streams, T, d, ld_t, ld_s, N, stride, scale, out);
    else
        hipLaunchKernelGGL(gram_dense<float>, dim3((unsigned)grid), dim3(256), 0, stream, (const float *)H, streams, T,
                           d, ld_t, ld_s, N, stride, scale, out);
    return hipGetLastError();
}
