// Spectral descriptors of sorted spectra, fp64 arithmetic.
//
// Descriptors of the "Random matrix theory spectral methods" page: spectral
// entropy H, leading-eigenvalue mass m1, eigengap g_k = lambda_k / lambda_{k+1}
// and the deviation from the Marchenko-Pastur law (section 2.3), the MP edge
// lambda_plus = sigma^2 (1 + sqrt c)^2 (section 2.1) and the count of
// eigenvalues beyond it (spiked model, section 2.2); the effective rank of the
// Swift-SVD page (section 3) as exp(H); the S3 page's long-tail test (top 20 %
// share, tail level; section 1) and its count of near-zero singular values
// (section 2).
//
// mp_table: Q_i = F^{-1}((i + 1/2) / r) of the MP law with sigma^2 = 1 and
//   ratio c <= 1, one thread per level.  With lambda = m - h cos(phi)
//   (m = 1 + c, h = 2 sqrt c) the distribution function has the closed form
//     F(phi) = [ sin(phi) / sqrt(c) + (1 + c) phi / (2c)
//                - ((1 - c) / c) atan(kappa tan(phi / 2)) ] / pi,
//   kappa = (1 + sqrt c) / (1 - sqrt c)   (the antiderivative of
//   h^2 sin^2(phi) / (2 pi c lambda(phi))), inverted by bisection on phi.
//   MP(sigma^2, c) is MP(1, c) scaled by sigma^2.
// descriptors: one 64-lane wave per spectrum; every sum is an fp64 wave
//   reduction.
#include <float.h>

#include <algorithm>
#include <mutex>

#include "common.h"
#include "internal.h"

namespace {

__global__ void mp_table(double c, int64_t r, double *__restrict__ q)
{
    const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    if (i >= r) return;
    const double u = ((double)i + 0.5) / (double)r;
    double a = 0.0, b = M_PI;
    for (int it = 0; it < 64; ++it) {
        const double mid = 0.5 * (a + b);
        if (mp_cdf_phi(mid, c) < u)
            a = mid;
        else
            b = mid;
    }
    const double phi = 0.5 * (a + b);
    const double sc = sqrt(c);
    const double lminus = (1.0 - sc) * (1.0 - sc);
    const double s = sin(0.5 * phi);
    q[i] = lminus + 4.0 * sc * s * s;  // = m - h cos(phi)
}

// sums over the wave, in every lane: DPP and row swaps, no LDS round trips;
// counts (< 2^53) go through fp64 exactly
__device__ __forceinline__ double wsum(double x) { return pair32_sum(half_sum(x)); }

__device__ __forceinline__ int64_t wsum_i(int64_t x) { return (int64_t)pair32_sum(half_sum((double)x)); }

// the descriptors of spectrum b, by one wave
template <typename T>
__device__ __forceinline__ void desc_one(const T *__restrict__ w, int64_t b, int64_t r, int64_t ldw,
                                         const spec_desc_params &p, const double *__restrict__ qtab,
                                         spec_desc *__restrict__ out)
{
    const int lane = threadIdx.x & 63;
    const T *wb = w + b * ldw;
    auto lam = [&](int64_t i) -> double {
        double v = (double)wb[i];
        return v > 0.0 ? v : (v == v ? 0.0 : v);  // clamp round-off, keep NaN
    };

    // pass 1: S, positives, non-finite, top-k sums
    const int64_t kt = (int64_t)floor(p.top_frac * (double)r);
    double S = 0.0, Ssig = 0.0, Stop = 0.0, Stop_sig = 0.0;
    int64_t rpos = 0, bad = 0;
    for (int64_t i = lane; i < r; i += 64) {
        const double v = lam(i);
        if (!isfinite(v)) {
            ++bad;
            continue;
        }
        const double sg = sqrt(v);
        S += v;
        Ssig += sg;
        if (v > 0.0) ++rpos;
        if (i < kt) {
            Stop += v;
            Stop_sig += sg;
        }
    }
    S = wsum(S);
    Ssig = wsum(Ssig);
    Stop = wsum(Stop);
    Stop_sig = wsum(Stop_sig);
    rpos = wsum_i(rpos);
    bad = wsum_i(bad);

    const double l0 = lam(0);
    const double l1 = r > 1 ? lam(1) : 0.0;
    double sigma2;
    if (p.sigma2_mode == SPEC_SIGMA2_MEDIAN)
        sigma2 = 0.5 * (lam((r - 1) / 2) + lam(r / 2));
    else if (p.sigma2_mode == SPEC_SIGMA2_MEAN)
        sigma2 = S / (double)p.p_dim;
    else
        sigma2 = p.sigma2;
    const double c = (double)p.p_dim / (double)p.n_samples;
    const double lplus = sigma2 * (1.0 + sqrt(c)) * (1.0 + sqrt(c));
    const double sig1 = sqrt(l0);
    const double small_thr = p.small_rel * sig1;

    // pass 2: entropy, counts, W1
    const bool companion = p.p_dim > p.n_samples;
    const double mu_scale = companion ? (double)p.n_samples / (double)p.p_dim : 1.0;
    double Hs = 0.0, w1 = 0.0;
    int64_t above = 0, small = 0;
    for (int64_t i = lane; i < r; i += 64) {
        const double v = lam(i);
        if (!isfinite(v)) continue;
        if (S > 0.0) {
            const double pi = v / S;
            if (pi > 0.0) Hs -= pi * log(pi);
        }
        if (v > lplus) ++above;
        if (sqrt(v) < small_thr) ++small;
        // ascending rank of lambda_i is r - 1 - i
        w1 += fabs(mu_scale * v - sigma2 * qtab[r - 1 - i]);
    }
    Hs = wsum(Hs);
    w1 = wsum(w1);
    above = wsum_i(above);
    small = wsum_i(small);

    if (lane == 0) {
        spec_desc d;
        const double nan = __builtin_nan("");
        int64_t flags = 0;
        if (bad) flags |= SPEC_FLAG_NONFINITE;
        if (!(S > 0.0)) flags |= SPEC_FLAG_S_ZERO;
        d.S = S;
        d.H = S > 0.0 ? Hs : nan;
        d.erank = S > 0.0 ? exp(Hs) : nan;
        d.m1 = S > 0.0 ? l0 / S : nan;
        const int64_t k = p.k;
        if (k < r && lam(k) > 0.0) {
            d.gk = lam(k - 1) / lam(k);
        } else {
            d.gk = nan;
            flags |= SPEC_FLAG_GK_UNDEF;
        }
        d.g1 = (r > 1 && l1 > 0.0) ? l0 / l1 : nan;
        d.sigma2 = sigma2;
        d.lambda_plus = lplus;
        d.mp_w1 = sigma2 > 0.0 ? w1 / (double)r : nan;
        d.top_energy = S > 0.0 ? Stop / S : nan;
        d.top_sigma_share = Ssig > 0.0 ? Stop_sig / Ssig : nan;
        int64_t th = (int64_t)floor(p.tail_frac * (double)r);
        if (th > r - 1) th = r - 1;
        d.tail_head = sqrt(lam(th));
        d.tail_min = sqrt(lam(r - 1));
        d.sigma1 = sig1;
        d.n_above = above;
        d.n_small = small;
        d.r_pos = rpos;
        d.flags = flags;
        out[b] = d;
    }
}

// four waves per workgroup, each taking spectra b = 4 g + wave, + 4 G, ...: a
// workgroup per short spectrum would be limited by the dispatch rate
constexpr int DW = 4;

template <typename T>
__global__ __launch_bounds__(64 * DW) void descriptors_kernel(const T *__restrict__ w, int64_t batch, int64_t r,
                                                              int64_t ldw, spec_desc_params p,
                                                              const double *__restrict__ qtab,
                                                              spec_desc *__restrict__ out)
{
    for (int64_t b = (int64_t)blockIdx.x * DW + (threadIdx.x >> 6); b < batch; b += (int64_t)gridDim.x * DW)
        desc_one<T>(w, b, r, ldw, p, qtab, out);
}

// The MP quantile table of spec_descriptors_static: one per GPU, in the
// library's own device memory, for callers that cannot allocate a workspace.
// Every call on a GPU rewrites it before reading it; calls that overlap on one
// GPU race on it.
static __device__ __align__(256) double scratch[DESC_SCRATCH_MAX_R];

constexpr int MAX_DEVICES = 64;
std::mutex scratch_mu;
double *scratch_ptr[MAX_DEVICES];  // device address of `scratch` on each GPU, once looked up

// the address of `scratch` on the device `stream` belongs to: looked up once per
// device with that device current (the host-side name is only a stand-in)
hipError_t scratch_on(hipStream_t stream, double **out)
{
    hipDevice_t dev = 0;
    hipError_t e = hipStreamGetDevice(stream, &dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> g(scratch_mu);
    if (scratch_ptr[dev] == nullptr) {
        int cur = 0;
        if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) {
            hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess) e = e2;
        }
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        scratch_ptr[dev] = (double *)p;
    }
    *out = scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace

size_t descriptors_workspace_bytes(int64_t r) { return (size_t)((r + 31) / 32 * 32) * sizeof(double); }

hipError_t launch_mp_table(hipStream_t stream, const spec_desc_params *p, int64_t r, void *ws)
{
    const double c = p->p_dim <= p->n_samples ? (double)p->p_dim / (double)p->n_samples
                                               : (double)p->n_samples / (double)p->p_dim;
    hipLaunchKernelGGL(mp_table, dim3((unsigned)((r + 255) / 256)), dim3(256), 0, stream, c, r, (double *)ws);
    return hipGetLastError();
}

hipError_t launch_descriptors(hipStream_t stream, const void *w, int wt, int64_t batch, int64_t r, int64_t ldw,
                              const spec_desc_params *p, spec_desc *out, void *ws)
{
    double *q = (double *)ws;
    hipError_t e = launch_mp_table(stream, p, r, ws);
    if (e != hipSuccess) return e;
    if (batch == 0) return hipSuccess;
    const unsigned grid = (unsigned)std::min<int64_t>((batch + DW - 1) / DW, 8192);
    KTimer kt(stream, SPEC_KT_DESC);
    if (wt == SPEC_F32)
        hipLaunchKernelGGL(descriptors_kernel<float>, dim3(grid), dim3(64 * DW), 0, stream, (const float *)w,
                           batch, r, ldw, *p, q, out);
    else
        hipLaunchKernelGGL(descriptors_kernel<double>, dim3(grid), dim3(64 * DW), 0, stream, (const double *)w,
                           batch, r, ldw, *p, q, out);
    return hipGetLastError();
}

hipError_t launch_descriptors_static(hipStream_t stream, const void *w, int wt, int64_t batch, int64_t r, int64_t ldw,
                                     const spec_desc_params *p, spec_desc *out)
{
    if (r > DESC_SCRATCH_MAX_R) return hipErrorInvalidValue;
    double *q = nullptr;
    hipError_t e = scratch_on(stream, &q);
    if (e != hipSuccess) return e;
    return launch_descriptors(stream, w, wt, batch, r, ldw, p, out, q);
}
