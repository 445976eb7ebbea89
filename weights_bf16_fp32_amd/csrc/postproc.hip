// Post-processing of spectra and descriptor series, fp64 arithmetic.
//
// desc_smooth: exponential smoothing of each descriptor time series ("Random
//   matrix theory spectral methods" page, section 3.2): y_0 = x_0,
//   y_t = alpha x_t + (1 - alpha) y_{t-1} along the window index of one stream.
//   One workgroup per stream, one thread per fp64 field; a non-finite value
//   leaves the state unchanged (and the record gets SPEC_FLAG_HELD), and the
//   output is NaN until the first finite value.  Counts are copied.
// spectrum_robust: one 64-lane wave per spectrum (sorted descending), four
//   waves per workgroup:
//   * the median (the two middle values of the sorted spectrum) and the
//     winsorised estimate sum(clip(lambda, lambda_(q+1) from below, lambda_(q+1)
//     from above)) / p of sigma^2 (section 4.2: median rather than mean,
//     winsorised extremes);
//   * the MAD, median |lambda - median|: the deviations of the values above and
//     below the median are two sorted sequences, so their order statistics come
//     from a binary search over the split between the two, no sort; and the
//     count of deviations beyond mad_k * 1.4826 * MAD (section 4.2, MAD anomaly
//     detection);
//   * mean and spread of ln lambda over the positive values (section 3.2, log
//     transform);
//   * the KL divergence of the spectrum's histogram over B equal-width bins of
//     the MP support [lambda_-, lambda_+] (outside values counted in the end
//     bins) from the MP bin masses (section 2.3).  The bin edges sit at angles
//     phi_b = acos(1 - 2b/B) whatever sigma^2 is, so q_b = F(phi_{b+1}) -
//     F(phi_b) with the closed-form F of the MP law; counts go through LDS.
#include <float.h>

#include "common.h"
#include "internal.h"

namespace {

constexpr int NSMOOTH = 14;  // the fp64 fields of spec_desc, in declaration order

__global__ __launch_bounds__(64) void desc_smooth_kernel(const spec_desc *__restrict__ in, int64_t W, double alpha,
                                                         spec_desc *__restrict__ out)
{
    const int64_t s = blockIdx.x;
    const int f = threadIdx.x;
    const spec_desc *src = in + s * W;
    spec_desc *dst = out + s * W;
    if (f < NSMOOTH) {
        // the recursion is serial; the loads of 16 steps are issued together
        constexpr int U = 16;
        double state = __builtin_nan("");
        bool have = false;
        for (int64_t t0 = 0; t0 < W; t0 += U) {
            double v[U];
#pragma unroll
            for (int u = 0; u < U; ++u)
                v[u] = t0 + u < W ? reinterpret_cast<const double *>(src + t0 + u)[f] : 0.0;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (t0 + u < W) {
                    if (isfinite(v[u])) {
                        state = have ? alpha * v[u] + (1.0 - alpha) * state : v[u];
                        have = true;
                    }
                    reinterpret_cast<double *>(dst + t0 + u)[f] = state;
                }
            }
        }
    }
    // counts and flags, every record independent: all 64 threads
    for (int64_t t = f; t < W; t += 64) {
        const double *d = reinterpret_cast<const double *>(src + t);
        bool held = false;
#pragma unroll
        for (int g = 0; g < NSMOOTH; ++g) held = held || !isfinite(d[g]);
        dst[t].n_above = src[t].n_above;
        dst[t].n_small = src[t].n_small;
        dst[t].r_pos = src[t].r_pos;
        dst[t].flags = src[t].flags | (held ? SPEC_FLAG_HELD : 0);
    }
}

// sums over the wave, in every lane: DPP and row swaps, no LDS round trips;
// counts (< 2^53) go through fp64 exactly
__device__ __forceinline__ double wsum(double x) { return pair32_sum(half_sum(x)); }

__device__ __forceinline__ int64_t wsum_i(int64_t x) { return (int64_t)pair32_sum(half_sum((double)x)); }

constexpr int RS = 1024;  // spectra up to this length are staged in LDS
constexpr int RW = 4;     // waves (spectra in flight) per workgroup

// the statistics of spectrum b, by one wave with its own LDS slices
template <typename T>
__device__ __forceinline__ void robust_one(const T *__restrict__ w, int64_t b, int64_t r, int64_t ldw,
                                           const spec_robust_params &p, spec_robust *__restrict__ out,
                                           int *__restrict__ cnt, double *__restrict__ ls)
{
    const int lane = threadIdx.x & 63;
    const T *wb = w + b * ldw;
    const bool staged = r <= RS;
    wave_sync();  // the previous spectrum's reads of the slices are done
    if (staged)
        for (int64_t i = lane; i < r; i += 64) ls[i] = (double)wb[i];
    cnt[lane] = 0;
    wave_sync();
    auto lam = [&](int64_t i) -> double {
        const double v = staged ? ls[i] : (double)wb[i];
        return v > 0.0 ? v : (v == v ? 0.0 : v);  // clamp round-off, keep NaN
    };

    // median of the sorted spectrum
    const double med = 0.5 * (lam((r - 1) / 2) + lam(r / 2));
    // winsorising bounds: the (q+1)-th largest and smallest values
    int64_t q = (int64_t)floor(p.winsor_frac * (double)r);
    if (q > (r - 1) / 2) q = (r - 1) / 2;
    const double whi = lam(q), wlo = lam(r - 1 - q);

    // pass 1: sums, counts, non-finite values, the split at the median
    double S = 0.0, Sw = 0.0, Slog = 0.0;
    int64_t npos = 0, nbad = 0, nup = 0;
    for (int64_t i = lane; i < r; i += 64) {
        const double v = lam(i);
        if (!isfinite(v)) {
            ++nbad;
            continue;
        }
        S += v;
        Sw += fmin(fmax(v, wlo), whi);
        if (v > 0.0) {
            ++npos;
            Slog += log(v);
        }
        if (v >= med) ++nup;
    }
    S = wsum(S);
    Sw = wsum(Sw);
    Slog = wsum(Slog);
    npos = wsum_i(npos);
    nbad = wsum_i(nbad);
    nup = wsum_i(nup);
    const double nan = __builtin_nan("");
    const double log_mean = npos > 0 ? Slog / (double)npos : nan;
    const double s2w = Sw / (double)p.p_dim;

    // MAD: the k-th smallest deviation.  U[j] = lambda_(nup-1-j) - med and
    // L[j] = med - lambda_(nup+j) are ascending; the k+1 smallest of both take
    // some i from U and k+1-i from L.
    const int64_t nu = nup, nl = r - nup;
    auto U = [&](int64_t j) { return lam(nu - 1 - j) - med; };
    auto L = [&](int64_t j) { return med - lam(nu + j); };
    auto kth = [&](int64_t k) {
        int64_t lo = k + 1 - nl > 0 ? k + 1 - nl : 0, hi = k + 1 < nu ? k + 1 : nu;
        while (lo < hi) {
            const int64_t i = (lo + hi) / 2, j = k + 1 - i;
            if (U(i) < L(j - 1))
                lo = i + 1;
            else
                hi = i;
        }
        const int64_t i = lo, j = k + 1 - lo;
        const double a = i > 0 ? U(i - 1) : -DBL_MAX, c = j > 0 ? L(j - 1) : -DBL_MAX;
        return a > c ? a : c;
    };
    double mad = 0.0;
    if (nbad == 0) mad = (r & 1) ? kth((r - 1) / 2) : 0.5 * (kth(r / 2 - 1) + kth(r / 2));
    const double thr = p.mad_k * 1.4826 * mad;

    // sigma^2 of the MP reference and the histogram
    double s2;
    if (p.sigma2_mode == SPEC_SIGMA2_MEDIAN)
        s2 = med;
    else if (p.sigma2_mode == SPEC_SIGMA2_MEAN)
        s2 = S / (double)p.p_dim;
    else if (p.sigma2_mode == SPEC_SIGMA2_WINSOR)
        s2 = s2w;
    else
        s2 = p.sigma2;
    const bool companion = p.p_dim > p.n_samples;
    const double mu_scale = companion ? (double)p.n_samples / (double)p.p_dim : 1.0;
    const double cc = companion ? (double)p.n_samples / (double)p.p_dim : (double)p.p_dim / (double)p.n_samples;
    const double sc = sqrt(cc);
    const double lm = s2 * ((1.0 - sc) * (1.0 - sc)), lp = s2 * ((1.0 + sc) * (1.0 + sc));
    const int B = p.bins;
    const bool kl_ok = s2 > 0.0 && nbad == 0;

    // pass 2: log spread, MAD outliers, histogram
    double Vlog = 0.0;
    int64_t nmad = 0;
    for (int64_t i = lane; i < r; i += 64) {
        const double v = lam(i);
        if (!isfinite(v)) continue;
        if (v > 0.0) {
            const double dl = log(v) - log_mean;
            Vlog += dl * dl;
        }
        if (fabs(v - med) > thr) ++nmad;
        if (kl_ok) {
            const double x = mu_scale * v;
            const double t = floor((x - lm) / (lp - lm) * (double)B);  // clamped before the conversion
            const int bi = t < 0.0 ? 0 : (t > (double)(B - 1) ? B - 1 : (int)t);
            atomicAdd(&cnt[bi], 1);
        }
    }
    Vlog = wsum(Vlog);
    nmad = wsum_i(nmad);
    wave_sync();
    double kl = 0.0;
    if (kl_ok && lane < B) {
        const double Fa = lane == 0 ? 0.0 : mp_cdf_phi(acos(1.0 - 2.0 * lane / (double)B), cc);
        const double Fb = lane == B - 1 ? 1.0 : mp_cdf_phi(acos(1.0 - 2.0 * (lane + 1) / (double)B), cc);
        const double pb = (double)cnt[lane] / (double)r;
        if (pb > 0.0) kl = pb * log(pb / (Fb - Fa));
    }
    kl = wsum(kl);

    if (lane == 0) {
        spec_robust o;
        int64_t flags = 0;
        if (nbad) flags |= SPEC_FLAG_NONFINITE;
        if (npos == 0) flags |= SPEC_FLAG_S_ZERO;
        // a non-finite value leaves the order statistics, the sums and every
        // estimate of sigma^2 undefined; the log statistics use the finite values
        o.median = nbad ? nan : med;
        o.sigma2_winsor = nbad ? nan : s2w;
        o.mad = nbad ? nan : mad;
        o.log_mean = log_mean;
        o.log_std = npos > 0 ? sqrt(Vlog / (double)npos) : nan;
        o.sigma2 = nbad && p.sigma2_mode != SPEC_SIGMA2_GIVEN ? nan : s2;
        o.kl_mp = kl_ok ? kl : nan;
        o.n_mad = nmad;
        o.flags = flags;
        out[b] = o;
    }
}

template <typename T>
__global__ __launch_bounds__(64 * RW) void robust_kernel(const T *__restrict__ w, int64_t batch, int64_t r,
                                                         int64_t ldw, spec_robust_params p,
                                                         spec_robust *__restrict__ out)
{
    __shared__ int cnt[RW][64];
    __shared__ double ls[RW][RS];
    const int wv = threadIdx.x >> 6;
    for (int64_t b = (int64_t)blockIdx.x * RW + wv; b < batch; b += (int64_t)gridDim.x * RW)
        robust_one<T>(w, b, r, ldw, p, out, cnt[wv], ls[wv]);
}

}  // namespace

hipError_t launch_desc_smooth(hipStream_t stream, const spec_desc *in, int64_t streams, int64_t W, double alpha,
                              spec_desc *out)
{
    if (streams == 0) return hipSuccess;
    hipLaunchKernelGGL(desc_smooth_kernel, dim3((unsigned)streams), dim3(64), 0, stream, in, W, alpha, out);
    return hipGetLastError();
}

hipError_t launch_spectrum_robust(hipStream_t stream, const void *w, int wt, int64_t batch, int64_t r, int64_t ldw,
                                  const spec_robust_params *p, spec_robust *out)
{
    if (batch == 0) return hipSuccess;
    const unsigned grid = (unsigned)((batch + RW - 1) / RW < 8192 ? (batch + RW - 1) / RW : 8192);
    if (wt == SPEC_F32)
        hipLaunchKernelGGL(robust_kernel<float>, dim3(grid), dim3(64 * RW), 0, stream, (const float *)w, batch, r,
                           ldw, *p, out);
    else
        hipLaunchKernelGGL(robust_kernel<double>, dim3(grid), dim3(64 * RW), 0, stream, (const double *)w, batch, r,
                           ldw, *p, out);
    return hipGetLastError();
}
