// Batched eigenvalues of small symmetric matrices (n <= 64), one 64-lane wave
// per matrix: Householder reduction to tridiagonal form with the matrix in
// registers, then bisection on Sturm counts.
//
// The pages take the spectrum of each EigenTrack window with a library
// eigvalsh and flip it to descending order ("Random matrix theory spectral
// methods" page, section 3.2 code); here each window's N x N Gram is reduced
// directly:
//   - lane i holds row i of the matrix (both triangles).  Step k builds the
//     reflector that zeroes column k below the subdiagonal from the lanes'
//     column-k entries (one wave reduction for the norm), forms p = tau A v
//     and w = p - (tau/2)(p^T v) v with v and w broadcast through LDS, and
//     applies A <- A - v w^T - w v^T to the trailing rows.  tau = 2 / v^T v
//     of the v actually used, so every reflection is orthogonal to rounding.
//   - the diagonal d and subdiagonal e of T = Q^T A Q end up the same in every
//     lane; eigenvalue l (descending) is found by lanes l and l + 32 together
//     (n <= 32): each counts the eigenvalues below one of two interior points
//     of the current interval (Sturm count: negative pivots of LDL^T(T - xI),
//     in fp32 with the hardware reciprocal), the pair exchange counts with a
//     half-wave swap and keep the third that holds eigenvalue l.  For
//     32 < n <= 64 every lane bisects its own eigenvalue.  The output is in
//     descending order by construction.
//   - Accuracy: the reduction is backward stable, and the fp32 count is exact
//     for a tridiagonal within a few ulps of T entry by entry (Kahan's and
//     Demmel's analysis of the bisection count), so the eigenvalues are within
//     a small multiple of eps_f32 ||A||.  Intervals stop at 2 ulps of |lambda|
//     or eps_f32 ||T|| (the default absolute tolerance of LAPACK's bisection),
//     below the error the fp32 reduction already carries.
#include <float.h>

#include "common.h"
#include "internal.h"

namespace {

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F &&f)
{
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<I + 1, N>(f);
    }
}

__device__ __forceinline__ float wave_total(float x) { return pair32_sum(half_sum(x)); }

// the same int in the partner lane (lane ^ 32)
__device__ __forceinline__ int partner32(int x)
{
    float a = __int_as_float(x), b = a;
    halfswap32(a, b);
    // a: lanes 32..63 got lane - 32; b: lanes 0..31 got lane + 32
    return __float_as_int((threadIdx.x & 32) ? a : b);
}

template <int NM>
__global__ __launch_bounds__(64) void small_eig_batched(spec_batch_src src, int64_t batch, int n,
                                                        float *__restrict__ w, int32_t *__restrict__ info)
{
    __shared__ __attribute__((aligned(16))) float vs[NM];
    __shared__ __attribute__((aligned(16))) float wsh[NM];
    const int64_t b = blockIdx.x;
    const int lane = threadIdx.x;
    const int i = lane;  // row of this lane; rows >= n are zero
    const bool rowok = i < n;

    // ---- row i, A[i][j] for every j (the source's lower triangle, mirrored)
    float a[NM];
    if (src.kind == SPEC_SRC_DENSE) {
        const float *base = src.a + b * src.stride_a;
#pragma unroll
        for (int j = 0; j < NM; ++j)
            a[j] = rowok && j < n ? base[(int64_t)max(i, j) * src.lda + min(i, j)] : 0.f;
    } else {
        const int64_t W = (src.T - n) / src.stride + 1;
        const int64_t s = b / W, win = b % W;
        const float *base = src.a + (s * src.T + win * src.stride) * n;  // step t of the window: base + t n
#pragma unroll
        for (int j = 0; j < NM; ++j)
            a[j] = rowok && j < n ? src.scale * base[(int64_t)max(i, j) * n + abs(i - j)] : 0.f;
    }
    bool fin = true;
#pragma unroll
    for (int j = 0; j < NM; ++j) fin = fin && isfinite(a[j]);
    if (!__all(fin)) {
        if (lane < n) w[b * n + lane] = __int_as_float(0x7fc00000);
        if (info != nullptr && lane == 0) info[b] = -1;
        return;
    }

    // ---- Householder tridiagonalisation; e[k] = T[k+1][k], the same in every lane
    float e[NM];
    static_for<0, NM - 2>([&](auto KC) {
        constexpr int k = decltype(KC)::value;
        if (k < n - 2) {
            const float x = a[k];  // A[i][k]
            const float sig = wave_total(i > k + 1 ? x * x : 0.f);
            const float x0 = readlane_t(x, k + 1);
            float tau = 0.f, mu = x0, vi = 0.f;
            if (sig > 0.f) {
                mu = sqrtf(x0 * x0 + sig);
                const float v0 = x0 <= 0.f ? x0 - mu : -sig / (x0 + mu);
                vi = i == k + 1 ? 1.f : (i > k + 1 ? x / v0 : 0.f);
                tau = 2.f / (1.f + wave_total(i > k + 1 ? vi * vi : 0.f));
            }
            e[k] = mu;
            if (tau != 0.f) {
                wave_sync();
                if (lane < NM) vs[lane] = vi;
                wave_sync();
                float p = 0.f;
#pragma unroll
                for (int j = k + 1; j < NM; ++j) p += a[j] * vs[j];
                p *= tau;
                const float pv = wave_total(i > k ? p * vi : 0.f);
                const float wi = p - 0.5f * tau * pv * vi;
                if (lane < NM) wsh[lane] = wi;
                wave_sync();
                if (i > k) {
#pragma unroll
                    for (int j = k + 1; j < NM; ++j) a[j] -= vi * wsh[j] + wi * vs[j];
                }
            }
        }
    });
    // diagonal, last subdiagonal entry, squares; rows past n are padded so that
    // they never count (d = FLT_MAX, e = 0)
    float d[NM], e2[NM];
    static_for<0, NM>([&](auto KC) {
        constexpr int k = decltype(KC)::value;
        d[k] = k < n ? readlane_t(a[k], k) : FLT_MAX;
        if constexpr (k + 1 < NM) {
            if (k == n - 2) e[k] = readlane_t(a[k], k + 1);
            e2[k] = k + 1 < n ? e[k] * e[k] : 0.f;
        }
    });
    // Gershgorin interval and pivot guard
    float lo = FLT_MAX, hi = -FLT_MAX, emax = 0.f;
    static_for<0, NM>([&](auto KC) {
        constexpr int k = decltype(KC)::value;
        if (k < n) {
            float r = 0.f;
            if constexpr (k > 0) r += fabsf(e[k - 1]);
            if constexpr (k + 1 < NM) {
                if (k + 1 < n) {
                    r += fabsf(e[k]);
                    emax = fmaxf(emax, e2[k]);
                }
            }
            lo = fminf(lo, d[k] - r);
            hi = fmaxf(hi, d[k] + r);
        }
    });
    const float span = fmaxf(fabsf(lo), fabsf(hi));
    lo -= 4.f * FLT_EPSILON * span;
    hi += 4.f * FLT_EPSILON * span;
    const float pivmin = FLT_MIN * fmaxf(1.f, emax);
    const float atol = FLT_EPSILON * span;

    auto below = [&](float x) {
        int cnt = 0;
        float q = 1.f;
#pragma unroll
        for (int k = 0; k < NM; ++k) {
            q = (d[k] - x) - (k > 0 ? e2[k - 1] : 0.f) * __builtin_amdgcn_rcpf(q);
            q = fabsf(q) < pivmin ? -pivmin : q;
            cnt += q < 0.f;
        }
        return cnt;
    };

    // ---- eigenvalue l (descending), i.e. ascending index n - 1 - l
    constexpr bool PAIR = NM <= 32;
    const int l = PAIR ? (lane & 31) : lane;
    const int target = n - 1 - min(l, n - 1);
    float lo_l = lo, hi_l = hi;
    int it = 0;
    for (; it < 64; ++it) {
        const float width = hi_l - lo_l;
        const bool done = width <= fmaxf(atol, 2.f * FLT_EPSILON * fmaxf(fabsf(lo_l), fabsf(hi_l)));
        if (__all(done || l >= n)) break;
        if constexpr (PAIR) {
            const float x1 = lo_l + width * (1.f / 3.f), x2 = lo_l + width * (2.f / 3.f);
            const int cnt = below((lane & 32) ? x2 : x1);
            const int other = partner32(cnt);
            const int c1 = (lane & 32) ? other : cnt, c2 = (lane & 32) ? cnt : other;
            if (!done) {
                if (c1 > target) {
                    hi_l = x1;
                } else if (c2 > target) {
                    lo_l = x1;
                    hi_l = x2;
                } else {
                    lo_l = x2;
                }
            }
        } else {
            const float x = lo_l + 0.5f * width;
            const int cnt = below(x);
            if (!done) {
                if (cnt > target)
                    hi_l = x;
                else
                    lo_l = x;
            }
        }
    }
    if ((!PAIR || lane < 32) && l < n) w[b * n + l] = 0.5f * (lo_l + hi_l);
    if (info != nullptr && lane == 0) info[b] = it;
}

// The descriptors of one spectrum held by a half-wave (lane i of the half has
// the i-th largest value lam, i < r), as spec_descriptors computes them from
// memory: the same formulas, fp64, half-wave sums; written by lane 0 of the
// half.  lamsh is a per-half LDS row of the clamped values.
__device__ __forceinline__ double hsum(double x) { return half_sum(x); }

__device__ void desc_half(float lamf, int i, int r, const spec_desc_params &p, const double *__restrict__ qtab,
                          double *__restrict__ lamsh, spec_desc *__restrict__ out, bool live)
{
    const bool in = i < r;
    double v = (double)lamf;
    v = v > 0.0 ? v : (v == v ? 0.0 : v);  // clamp round-off, keep NaN
    v = in ? v : 0.0;
    wave_sync();
    lamsh[i] = v;
    wave_sync();
    auto lam = [&](int k) { return lamsh[k]; };
    const int kt = (int)floor(p.top_frac * (double)r);
    const bool fin = isfinite(v);
    const double vf = fin ? v : 0.0, sg = sqrt(vf);
    const double S = hsum(in && fin ? vf : 0.0);
    const double Ssig = hsum(in && fin ? sg : 0.0);
    const double Stop = hsum(in && fin && i < kt ? vf : 0.0);
    const double Stop_sig = hsum(in && fin && i < kt ? sg : 0.0);
    const double rpos = hsum(in && fin && vf > 0.0 ? 1.0 : 0.0);
    const double bad = hsum(in && !fin ? 1.0 : 0.0);
    const double l0 = lam(0), l1 = r > 1 ? lam(1) : 0.0;
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
    const bool companion = p.p_dim > p.n_samples;
    const double mu_scale = companion ? (double)p.n_samples / (double)p.p_dim : 1.0;
    double hs = 0.0;
    if (in && fin && S > 0.0) {
        const double pi = vf / S;
        if (pi > 0.0) hs = -pi * log(pi);
    }
    const double Hs = hsum(hs);
    const double w1 = hsum(in && fin ? fabs(mu_scale * vf - sigma2 * qtab[in ? r - 1 - i : 0]) : 0.0);
    const double above = hsum(in && fin && vf > lplus ? 1.0 : 0.0);
    const double small = hsum(in && fin && sg < small_thr ? 1.0 : 0.0);
    if (i == 0 && live) {
        spec_desc d;
        const double nan = __builtin_nan("");
        int64_t flags = 0;
        if (bad > 0.0) flags |= SPEC_FLAG_NONFINITE;
        if (!(S > 0.0)) flags |= SPEC_FLAG_S_ZERO;
        d.S = S;
        d.H = S > 0.0 ? Hs : nan;
        d.erank = S > 0.0 ? exp(Hs) : nan;
        d.m1 = S > 0.0 ? l0 / S : nan;
        const int k = (int)p.k;
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
        int th = (int)floor(p.tail_frac * (double)r);
        if (th > r - 1) th = r - 1;
        d.tail_head = sqrt(lam(th));
        d.tail_min = sqrt(lam(r - 1));
        d.sigma1 = sig1;
        d.n_above = (int64_t)above;
        d.n_small = (int64_t)small;
        d.r_pos = (int64_t)rpos;
        d.flags = flags;
        *out = d;
    }
}

// Two matrices per wave for n <= 32: half h = lane / 32 takes matrix 2 g + h
// and lane i = lane % 32 its row i.  Every sum is a half-wave butterfly, the
// broadcasts go through per-half LDS rows, and each lane finds its own
// eigenvalue.  The reduction is that of small_eig_batched, value for value.
template <int NM, bool DESC>
__global__ __launch_bounds__(64) void small_eig_pair(spec_batch_src src, int64_t batch, int n,
                                                     float *__restrict__ w, int32_t *__restrict__ info,
                                                     spec_desc_params dp, const double *__restrict__ qtab,
                                                     spec_desc *__restrict__ dout)
{
    static_assert(NM <= 32, "a half-wave per matrix");
    __shared__ __attribute__((aligned(16))) float vs[2][32];
    __shared__ __attribute__((aligned(16))) float wsh[2][32];
    __shared__ __attribute__((aligned(16))) float dsh[2][33];
    __shared__ int cnt[2][64];
    __shared__ double lamsh[2][32];
    const int lane = threadIdx.x, h = lane >> 5, i = lane & 31;
    const int64_t b = 2 * (int64_t)blockIdx.x + h;
    const bool live = b < batch;
    const bool rowok = live && i < n;

    // Every load is unconditional, at indices clamped into the matrix (row and
    // column n - 1 at most), and masked afterwards: a load under a branch
    // would wait for the one before it.
    float a[NM];
    const int ic = min(i, n - 1);
    if (src.kind == SPEC_SRC_DENSE) {
        const float *base = src.a + (live ? b : 0) * src.stride_a;
#pragma unroll
        for (int j = 0; j < NM; ++j) {
            const int jc = min(j, n - 1);
            const float v = base[(int64_t)max(ic, jc) * src.lda + min(ic, jc)];
            a[j] = rowok && j < n ? v : 0.f;
        }
    } else {
        const int64_t W = (src.T - n) / src.stride + 1;
        const int64_t bb = live ? b : 0;
        const int64_t s = bb / W, win = bb % W;
        const float *base = src.a + (s * src.T + win * src.stride) * n;
#pragma unroll
        for (int j = 0; j < NM; ++j) {
            const int jc = min(j, n - 1);
            const float v = base[(int64_t)max(ic, jc) * n + abs(ic - jc)];
            a[j] = rowok && j < n ? src.scale * v : 0.f;
        }
    }
    bool fin = true;
#pragma unroll
    for (int j = 0; j < NM; ++j) fin = fin && isfinite(a[j]);
    const uint64_t badm = __ballot(!fin);
    const bool bad = (h ? (badm >> 32) : (badm & 0xffffffffull)) != 0;
    if (bad) {  // this half reports NaN; its lanes go on with zeros
#pragma unroll
        for (int j = 0; j < NM; ++j) a[j] = 0.f;
    }

    // ---- Householder tridiagonalisation, the two halves side by side
    float e[NM];
    static_for<0, NM - 2>([&](auto KC) {
        constexpr int k = decltype(KC)::value;
        if (k < n - 2) {
            const float x = a[k];  // A[i][k]
            const float sig = half_sum(i > k + 1 ? x * x : 0.f);
            const float x0 = half_sum(i == k + 1 ? x : 0.f);
            const bool go = sig > 0.f;
            const float mu = go ? sqrtf(x0 * x0 + sig) : x0;
            const float v0 = go ? (x0 <= 0.f ? x0 - mu : -sig / (x0 + mu)) : 1.f;
            const float vi = go ? (i == k + 1 ? 1.f : (i > k + 1 ? x / v0 : 0.f)) : 0.f;
            const float vv = half_sum(i > k + 1 ? vi * vi : 0.f);
            const float tau = go ? 2.f / (1.f + vv) : 0.f;
            e[k] = mu;
            wave_sync();
            vs[h][i] = vi;
            wave_sync();
            float p = 0.f;
#pragma unroll
            for (int j = k + 1; j < NM; ++j) p += a[j] * vs[h][j];
            p *= tau;
            const float pv = half_sum(i > k ? p * vi : 0.f);
            const float wi = p - 0.5f * tau * pv * vi;
            wsh[h][i] = wi;
            wave_sync();
            if (i > k) {
#pragma unroll
                for (int j = k + 1; j < NM; ++j) a[j] -= vi * wsh[h][j] + wi * vs[h][j];
            }
        }
    });
    // the diagonal and the last subdiagonal entry through LDS
    {
        float diag = 0.f;
#pragma unroll
        for (int j = 0; j < NM; ++j) diag = i == j ? a[j] : diag;
        float last = 0.f;
#pragma unroll
        for (int j = 0; j < NM; ++j) last = j == n - 2 ? a[j] : last;
        wave_sync();
        dsh[h][i] = diag;
        if (n >= 2 && i == n - 1) dsh[h][32] = last;
        wave_sync();
    }
    float d[NM], e2[NM];
    const float elast = n >= 2 ? dsh[h][32] : 0.f;
#pragma unroll
    for (int k = 0; k < NM; ++k) {
        d[k] = k < n ? dsh[h][k] : FLT_MAX;
        if (k + 1 < NM) {
            if (k == n - 2) e[k] = elast;
            e2[k] = k + 1 < n ? e[k] * e[k] : 0.f;
        }
    }
    // Gershgorin interval and pivot guard
    float lo = FLT_MAX, hi = -FLT_MAX, emax = 0.f;
#pragma unroll
    for (int k = 0; k < NM; ++k) {
        if (k < n) {
            float r = 0.f;
            if (k > 0) r += fabsf(e[k - 1]);
            if (k + 1 < NM && k + 1 < n) {
                r += fabsf(e[k]);
                emax = fmaxf(emax, e2[k]);
            }
            lo = fminf(lo, d[k] - r);
            hi = fmaxf(hi, d[k] + r);
        }
    }
    const float span = fmaxf(fabsf(lo), fabsf(hi));
    lo -= 4.f * FLT_EPSILON * span;
    hi += 4.f * FLT_EPSILON * span;
    const float pivmin = FLT_MIN * fmaxf(1.f, emax);
    const float atol = FLT_EPSILON * span;

    // the Sturm count below x
    auto count1 = [&](float x) __attribute__((always_inline)) {
        int c = 0;
        float q = 1.f;
#pragma unroll
        for (int k = 0; k < NM; ++k) {
            q = (d[k] - x) - (k > 0 ? e2[k - 1] : 0.f) * __builtin_amdgcn_rcpf(q);
            q = fabsf(q) < pivmin ? -pivmin : q;
            c += q < 0.f;
        }
        return c;
    };
    // the Sturm counts below two points in one pass (two independent recurrences)
    auto count2 = [&](float x1, float x2, int &c1, int &c2) __attribute__((always_inline)) {
        c1 = 0;
        c2 = 0;
        float q1 = 1.f, q2 = 1.f;
#pragma unroll
        for (int k = 0; k < NM; ++k) {
            const float ek = k > 0 ? e2[k - 1] : 0.f;
            q1 = (d[k] - x1) - ek * __builtin_amdgcn_rcpf(q1);
            q2 = (d[k] - x2) - ek * __builtin_amdgcn_rcpf(q2);
            q1 = fabsf(q1) < pivmin ? -pivmin : q1;
            q2 = fabsf(q2) < pivmin ? -pivmin : q2;
            c1 += q1 < 0.f;
            c2 += q2 < 0.f;
        }
    };
    // ---- eigenvalue l = i (descending), ascending index n - 1 - l.  First a
    // multisection shared by the half: its 32 lanes count below the 64 points
    // lo + (q + 1) (hi - lo) / 65, and each lane takes the cell whose points
    // bracket its eigenvalue (a binary search over the counts, which do not
    // decrease); then bisection, one count per lane and step: the kernel is
    // bound by VALU issue, and a halving costs half a trisection's two counts
    // for 1 bit against log2(3) bits.
    const int l = i;
    const int target = n - 1 - min(l, n - 1);
    float lo_l = lo, hi_l = hi;
    {
        const float step = (hi - lo) * (1.f / 65.f);
        int ca, cb;
        count2(lo + (float)(2 * i + 1) * step, lo + (float)(2 * i + 2) * step, ca, cb);
        wave_sync();
        cnt[h][2 * i] = ca;
        cnt[h][2 * i + 1] = cb;
        wave_sync();
        // the first point q with cnt[q] > target (64 if none): 65 answers, so
        // seven halvings of [a0, a1), each only while the range is not empty
        int a0 = 0, a1 = 64;
#pragma unroll
        for (int s = 0; s < 7; ++s) {
            if (a0 < a1) {
                const int mid = (a0 + a1) >> 1;  // < 64
                const bool le = cnt[h][mid] <= target;
                a0 = le ? mid + 1 : a0;
                a1 = le ? a1 : mid;
            }
        }
        lo_l = a0 == 0 ? lo : lo + (float)a0 * step;
        hi_l = a0 == 64 ? hi : lo + (float)(a0 + 1) * step;
    }
    int it = 1;
    for (; it < 64; ++it) {
        const float width = hi_l - lo_l;
        const bool done = width <= fmaxf(atol, 2.f * FLT_EPSILON * fmaxf(fabsf(lo_l), fabsf(hi_l)));
        if (__all(done || l >= n || !live)) break;
        const float x = lo_l + 0.5f * width;
        const int c = count1(x);
        if (!done) {
            if (c > target)
                hi_l = x;
            else
                lo_l = x;
        }
    }
    const float lam_l = bad ? __int_as_float(0x7fc00000) : 0.5f * (lo_l + hi_l);
    if (w != nullptr && live && l < n) w[b * n + l] = lam_l;
    if (live && info != nullptr && i == 0) info[b] = bad ? -1 : it;
    if constexpr (DESC) desc_half(lam_l, i, n, dp, qtab, lamsh[h], dout + (live ? b : 0), live);
}

}  // namespace

hipError_t launch_eigvalsh_batched(hipStream_t stream, const spec_batch_src *src, int64_t batch, int n, float *w,
                                   int32_t *info)
{
    if (batch == 0) return hipSuccess;
    const spec_desc_params none{};
    if (n == 30)  // the EigenTrack window: no padding rows in the Sturm counts
        hipLaunchKernelGGL((small_eig_pair<30, false>), dim3((unsigned)((batch + 1) / 2)), dim3(64), 0, stream, *src,
                           batch, n, w, info, none, (const double *)nullptr, (spec_desc *)nullptr);
    else if (n <= 32)
        hipLaunchKernelGGL((small_eig_pair<32, false>), dim3((unsigned)((batch + 1) / 2)), dim3(64), 0, stream, *src,
                           batch, n, w, info, none, (const double *)nullptr, (spec_desc *)nullptr);
    else
        hipLaunchKernelGGL(small_eig_batched<64>, dim3((unsigned)batch), dim3(64), 0, stream, *src, batch, n, w, info);
    return hipGetLastError();
}

hipError_t launch_eigvalsh_batched_desc(hipStream_t stream, const spec_batch_src *src, int64_t batch, int n, float *w,
                                        int32_t *info, const spec_desc_params *p, spec_desc *out, void *ws)
{
    hipError_t e = launch_mp_table(stream, p, n, ws);
    if (e != hipSuccess || batch == 0) return e;
    if (n == 30)
        hipLaunchKernelGGL((small_eig_pair<30, true>), dim3((unsigned)((batch + 1) / 2)), dim3(64), 0, stream, *src,
                           batch, n, w, info, *p, (const double *)ws, out);
    else
        hipLaunchKernelGGL((small_eig_pair<32, true>), dim3((unsigned)((batch + 1) / 2)), dim3(64), 0, stream, *src,
                           batch, n, w, info, *p, (const double *)ws, out);
    return hipGetLastError();
}
