// Sliding-window spectra by rank-one down- and up-dates of the window Gram, fp64.
//
// The "Random matrix theory spectral methods" page (section 3.2) names
// incremental updates of the window decomposition, instead of a fresh
// decomposition per step, as the way to cut EigenTrack's cost.  Here a chain of
// consecutive windows of one stream keeps the eigenpairs (lam, Y) of the window
// Gram K = Y diag(lam) Y^T (rows of Y = window rows, oldest first) and moves
// them from window to window:
//   - delete the oldest row: the eigenvalues of K[1:, 1:] are the roots of the
//     secular equation sum_i y_i^2 / (lam_i - x) = 0 (y = row 0 of Y), one
//     between each pair of consecutive lam; the eigenvector of root mu is
//     (Y (diag(lam) - mu)^{-1} y)[1:], normalised;
//   - append the new step: in the basis diag(Y, 1) the bordered matrix
//     [[K', g], [g^T, gamma]] is an arrowhead with c = Y^T g, whose eigenvalues
//     are the roots of x - gamma + sum_i c_i^2 / (lam_i - x) = 0 (one below,
//     one between each pair, one above the lam), with eigenvectors
//     diag(Y, 1) [c / (lam - x); -1], normalised.
// Poles with a negligible weight (|y_i| or |c_i| below 8 eps times the scale)
// or within 8 eps ||K|| of the next pole are deflated first (a Givens rotation
// moves the weight of the pair onto one of them); the deflated eigenvalues keep
// their eigenvectors.  Each root is found by a safeguarded iteration in the
// distance tau from its nearer pole: the parts of the secular function left and
// right of the root are each matched, in value and slope, by a constant plus
// one pole term at the interval's end (Bunch, Nielsen and Sorensen's rational
// model), the model's root is the next iterate, and a bisection step replaces
// it whenever it leaves the sign bracket.  The weights are then recomputed from
// the roots (Gu and Eisenstat's formula), so the new eigenvectors are
// orthogonal to working precision whatever the roots' errors.
//
// Chains start from an empty window (N appends) every `restart` windows, which
// bounds the round-off a chain accumulates and gives the launch its
// parallelism.  Two chains per wave (half-waves of 32 lanes) for N <= 32, one
// per wave up to N = 64; lane i solves root i and builds eigenvector column i
// from the chain's Y in LDS.
#include <float.h>

#include "common.h"
#include "internal.h"

namespace {

constexpr double EPS = DBL_EPSILON;
constexpr int MAXIT = 40;
constexpr double PAD_POLE = 1e300;  // padding pole, zero weight

template <int G>
struct alignas(16) Chain {
    double Y[G][G + 2];  // Y[c][r]: column c (eigenvector of lam[c]), window row r
    double lam[G];       // ascending
    double2 pw[G];       // compacted poles {p, weight}; the weight becomes y-hat / c-hat
    double2 root[G];     // {origin pole, tau}: root = origin + tau
    double vec[G];       // y = row 0 of Y, or c = Y^T g; rotated by the deflation
    double aux[G];       // appended row g, then the root values
    double dval[G];      // deflated eigenvalues
    int idx[G];          // column of compacted pole i; bit 8 set for a negative y_i / c_i
    int didx[G];         // column of deflated eigenvalue e
    int dflag[G];
};

template <int G>
SPEC_DEVICE double gsum(double x)
{
    if constexpr (G == 32)
        return half_sum(x);
    else
        return pair32_sum(half_sum(x));
}

// the ballot of this lane's group (bit i = lane i of the group)
template <int G>
SPEC_DEVICE uint64_t gballot(bool p)
{
    const uint64_t m = __ballot(p);
    if constexpr (G == 32)
        return (threadIdx.x & 32) ? (m >> 32) : (m & 0xffffffffull);
    else
        return m;
}

template <int G>
SPEC_DEVICE int gmax(int v)
{
#pragma unroll
    for (int o = 1; o < G; o <<= 1) v = max(v, __shfl_xor(v, o));
    return v;
}

// 1/t to working precision: the hardware estimate and two Newton steps
SPEC_DEVICE double rcp64(double t)
{
    double r = __builtin_amdgcn_rcp(t);
    double e = fma(-t, r, 1.0);
    r = fma(r, e, r);
    e = fma(-t, r, 1.0);
    return fma(r, e, r);
}

// Root j of g(x) = rho (x - gamma) + sum_{i<m} w_i / (p_i - x) over the
// compacted poles pw[0..m) (ascending, w_i > 0); g increases between poles.
// rho = 0 (deletion): root j lies in (p_j, p_{j+1}).  rho = 1 (arrowhead):
// root j lies in (p_{j-1}, p_j), with p_{-1} = -inf and p_m = +inf bounded by
// min(p_0, gamma) - |c| and max(p_{m-1}, gamma) + |c| (sw = |c|^2).
// Returns the root as org + tau, org a pole next to the root (gamma when m = 0).
template <int G>
SPEC_DEVICE void secular_root(const double2 *pw, int m, double rho, double gamma, double sw, int j, bool act,
                              double &org, double &tau, int &its)
{
    const int ia = rho == 0.0 ? j : j - 1, ib = ia + 1;
    const bool ha = act && ia >= 0, hb = act && ib < m;
    const double pa = pw[min(max(ia, 0), G - 1)].x, pb = pw[min(ib, G - 1)].x;
    bool done = !act;
    bool oleft = true;
    double tlo = 0.0, thi = 0.0;
    org = 0.0;
    its = 0;
    if (ha && hb) {
        // the side of the midpoint the root is on picks the origin pole
        const double mid = 0.5 * (pa + pb);
        double g = rho * (mid - gamma);
        for (int i = 0; i < m; ++i) {
            const double2 q = pw[i];
            g += q.y * rcp64(q.x - mid);
        }
        oleft = g >= 0.0;
        org = oleft ? pa : pb;
        tlo = oleft ? 0.0 : mid - pb;
        thi = oleft ? mid - pa : 0.0;
    } else if (hb) {  // below every pole
        oleft = false;
        org = pb;
        tlo = fmin(fmin(pw[0].x, gamma) - sqrt(sw) - pb, -(fabs(pb) * EPS + DBL_MIN));
        thi = 0.0;
    } else if (ha) {  // above every pole
        org = pa;
        tlo = 0.0;
        thi = fmax(fmax(pw[m - 1].x, gamma) + sqrt(sw) - pa, fabs(pa) * EPS + DBL_MIN);
    } else {
        org = gamma;  // no poles left: the root is gamma itself
        done = true;
    }
    const double da = pa - org, db = pb - org;
    tau = 0.5 * (tlo + thi);
    for (int it = 0; it < MAXIT; ++it) {
        if (__ballot(!done) == 0) break;
        // psi: the poles left of the root (negative terms), phi: the rest
        double psi = 0.0, dpsi = 0.0, gt = 0.0, dgt = 0.0;
        for (int i = 0; i < m; ++i) {
            const double2 q = pw[i];
            const double r = rcp64((q.x - org) - tau);
            const double term = q.y * r, d = term * r;
            const bool left = i <= ia;
            psi += left ? term : 0.0;
            dpsi += left ? d : 0.0;
            gt += term;
            dgt += d;
        }
        if (done) continue;
        ++its;
        const double phi = (gt - psi) + rho * ((org + tau) - gamma), dphi = (dgt - dpsi) + rho;
        const double g = psi + phi;
        // rounding bound of g: the terms' magnitudes and the error of tau itself
        const double err = 8.0 * EPS * ((gt - 2.0 * psi) + rho * (fabs(org + tau) + fabs(gamma)) +
                                        fabs(tau) * (dpsi + dphi));
        if (g < 0.0)
            tlo = tau;
        else
            thi = tau;
        if (fabs(g) <= err || thi - tlo <= 2.0 * EPS * fmax(fabs(tlo), fabs(thi))) {
            done = true;
            continue;
        }
        double x = __builtin_nan("");
        if (ha && hb) {
            const double B1 = dpsi * (da - tau) * (da - tau), A1 = psi - dpsi * (da - tau);
            const double B2 = dphi * (db - tau) * (db - tau), A2 = phi - dphi * (db - tau);
            const double C = A1 + A2, D = db - da;
            if (oleft) {  // u = -x in (-D, 0): C u^2 + (C D + B1 + B2) u + B1 D = 0
                const double beta = C * D + B1 + B2;
                const double sq = sqrt(fmax(beta * beta - 4.0 * C * B1 * D, 0.0));
                x = beta > 0.0 ? 2.0 * B1 * D / (beta + sq) : -(sq - beta) / (2.0 * C);
            } else {  // v = -x in (0, D): C v^2 + (B1 + B2 - C D) v - B2 D = 0
                const double beta = B1 + B2 - C * D;
                const double sq = sqrt(fmax(beta * beta + 4.0 * C * B2 * D, 0.0));
                x = -(beta > 0.0 ? 2.0 * B2 * D / (beta + sq) : (sq - beta) / (2.0 * C));
            }
        } else if (hb) {  // A2 + B2 / (-x) = 0
            const double B2 = dphi * tau * tau, A2 = phi + dphi * tau;
            if (A2 < 0.0) x = B2 / A2;
        } else {  // A1 + B1 / u + (org - u - gamma) = 0 with u = -x < 0
            const double B1 = dpsi * tau * tau, A1 = psi + dpsi * tau;
            const double E = A1 + rho * (org - gamma);
            const double sq = sqrt(E * E + 4.0 * rho * B1);
            const double u = E > 0.0 ? -2.0 * B1 / (E + sq) : (E - sq) / (2.0 * rho);
            x = -u;
        }
        if (!(x > tlo && x < thi)) x = 0.5 * (tlo + thi);
        if (fabs(x - tau) <= EPS * fabs(tau)) done = true;
        tau = x;
    }
}

// Deflation of close poles: scanning the poles in order, a pole within tol of
// the previous undeflated one gets the pair's weight by a Givens rotation of
// the two columns (rows [0, rows)), and the previous one is deflated.
template <int G>
SPEC_DEVICE void rotate_close(Chain<G> &c, int k, int rows, double tol, int li)
{
    int prev = -1;
    for (int i = 0; i < k; ++i) {
        if (c.dflag[i]) continue;
        if (prev >= 0 && c.lam[i] - c.lam[prev] <= tol) {
            const double a = c.vec[prev], b = c.vec[i];
            const double r = sqrt(a * a + b * b);
            const double cs = b / r, sn = a / r;
            if (li < rows) {
                const double yp = c.Y[prev][li], yi = c.Y[i][li];
                c.Y[prev][li] = cs * yp - sn * yi;
                c.Y[i][li] = sn * yp + cs * yi;
            }
            wave_sync();
            if (li == 0) {
                c.vec[prev] = 0.0;
                c.vec[i] = r;
                c.dflag[prev] = 1;
            }
            wave_sync();
        }
        prev = i;
    }
}

// Flags in c.dflag (lanes < k, set by the caller) and c.vec hold the weights:
// the close-pole deflation, then the undeflated poles compacted into c.pw
// ({lam, vec^2}, padded) and c.idx, the deflated ones into c.dval / c.didx.
// Returns m, the number of undeflated poles.
template <int G>
SPEC_DEVICE int compact(Chain<G> &c, int k, double tol, int li)
{
    const bool close = li + 1 < k && c.lam[li + 1] - c.lam[li] <= tol;
    wave_sync();
    if (gballot<G>(close)) rotate_close<G>(c, k, k, tol, li);
    wave_sync();
    const bool in = li < k;
    const double v = c.vec[li];
    const bool nd = in && !c.dflag[li];
    const uint64_t msk = gballot<G>(nd);
    const int m = __popcll(msk), pos = __popcll(msk & ((1ull << li) - 1));
    const double lv = c.lam[li];
    wave_sync();
    if (nd) {
        c.pw[pos] = make_double2(lv, v * v);
        c.idx[pos] = li | (v < 0.0 ? 0x100 : 0);
    } else if (in) {
        c.dval[li - pos] = lv;
        c.didx[li - pos] = li;
    }
    if (li >= m) c.pw[li] = make_double2(PAD_POLE, 0.0);
    wave_sync();
    return m;
}

// Eigenvector columns and ranks after the roots: lanes [0, nroots) build the
// column of their root from the compacted poles (weights in pw[].y) and Y;
// lanes [nroots, nroots + kd) copy a deflated column.  `shift` drops row 0
// (deletion); `lastrow` >= 0 sets that row to -1 (roots) or 0 (deflated) for
// the arrowhead.  The new columns replace Y in ascending order of their values.
template <int G>
SPEC_DEVICE void rebuild_columns(Chain<G> &c, int m, int nroots, int kd, bool shift, int lastrow, int li)
{
    double acc[G];
#pragma unroll
    for (int r = 0; r < G; ++r) acc[r] = 0.0;
    double val = 0.0;
    int rank = 0;
    const bool isroot = li < nroots, isdefl = !isroot && li < nroots + kd;
    if (isroot) {
        const double2 rt = c.root[li];
        double nrm = lastrow >= 0 ? 1.0 : 0.0;
        for (int i = 0; i < m; ++i) {
            const double2 q = c.pw[i];
            const double z = q.y / ((q.x - rt.x) - rt.y);
            nrm += z * z;
            const double *col = c.Y[c.idx[i] & 0xff];
#pragma unroll
            for (int r = 0; r < G; r += 2) {
                const double2 y2 = *(const double2 *)(col + r);
                acc[r] = fma(y2.x, z, acc[r]);
                acc[r + 1] = fma(y2.y, z, acc[r + 1]);
            }
        }
        const double s = 1.0 / sqrt(nrm);
#pragma unroll
        for (int r = 0; r < G; ++r) acc[r] = r == lastrow ? -s : acc[r] * s;
        val = rt.x + rt.y;
        int cnt = 0;
        for (int e = 0; e < kd; ++e) cnt += c.dval[e] < val;
        rank = li + cnt;
    } else if (isdefl) {
        const int e = li - nroots;
        const double *col = c.Y[c.didx[e]];
#pragma unroll
        for (int r = 0; r < G; r += 2) {
            const double2 y2 = *(const double2 *)(col + r);
            acc[r] = y2.x;
            acc[r + 1] = y2.y;
        }
#pragma unroll
        for (int r = 0; r < G; ++r) acc[r] = r == lastrow ? 0.0 : acc[r];
        val = c.dval[e];
        int cnt = 0;
        for (int j = 0; j < nroots; ++j) cnt += c.aux[j] <= val;
        rank = e + cnt;
    }
    wave_sync();  // every read of the old columns is done
    if (isroot || isdefl) {
        double *dst = c.Y[rank];
        if (shift) {
#pragma unroll
            for (int r = 0; r + 1 < G; ++r) dst[r] = acc[r + 1];
        } else {
#pragma unroll
            for (int r = 0; r < G; r += 2) *(double2 *)(dst + r) = make_double2(acc[r], acc[r + 1]);
        }
        c.lam[rank] = val;
    }
    wave_sync();
}

// Drop window row 0 from the decomposition of size k (k >= 1).  Returns the
// largest iteration count of the group's roots.
template <int G>
SPEC_DEVICE int delete_oldest(Chain<G> &c, int k, int li)
{
    const bool in = li < k;
    const double y = in ? c.Y[li][0] : 0.0;
    const double lmax = fmax(fabs(c.lam[0]), fabs(c.lam[k - 1]));
    wave_sync();
    c.vec[li] = y;
    c.dflag[li] = in && fabs(y) <= 8.0 * EPS;
    wave_sync();
    const int m = compact<G>(c, k, 8.0 * EPS * lmax, li);
    const int nroots = m - 1, kd = k - m;
    double org, tau;
    int its;
    secular_root<G>(c.pw, m, 0.0, 0.0, 0.0, li, li < nroots, org, tau, its);
    if (li < nroots) {
        c.root[li] = make_double2(org, tau);
        c.aux[li] = org + tau;
    }
    wave_sync();
    // y-hat_i^2 = prod_l (mu_l - p_i) / prod_{j != i} (p_j - p_i), each root
    // paired with the pole on its far side from p_i (positive ratios)
    double yh = 0.0;
    if (li < m) {
        const double pi = c.pw[li].x;
        double prod = 1.0, num = 1.0, den = 1.0;
        for (int l = 0; l < nroots; ++l) {
            const double2 rt = c.root[l];
            num *= (rt.x - pi) + rt.y;
            den *= c.pw[l < li ? l : l + 1].x - pi;
            if ((l & 3) == 3) {
                prod *= num / den;
                num = den = 1.0;
            }
        }
        prod *= num / den;
        const double s = sqrt(fmax(prod, 0.0));
        yh = (c.idx[li] & 0x100) ? -s : s;
    }
    wave_sync();
    if (li < m) c.pw[li].y = yh;
    wave_sync();
    rebuild_columns<G>(c, m, nroots, kd, true, -1, li);
    return gmax<G>(its);
}

// Append window row k (the step with band row `row`: row[j] = <h_t, h_{t-j}>)
// to the decomposition of size k (k < G).  Returns the largest iteration count,
// or -1 (nothing changed) if the row holds a non-finite value.
template <int G>
SPEC_DEVICE int append_step(Chain<G> &c, int k, int li, const float *row, double scale)
{
    const bool in = li < k;
    const float graw = in ? row[k - li] : 0.f;  // window row li is step t - (k - li)
    const float graw0 = row[0];
    if (gballot<G>(!(isfinite(graw) && isfinite(graw0)))) return -1;
    const double gamma = scale * (double)graw0;
    wave_sync();
    c.aux[li] = scale * (double)graw;
    wave_sync();
    double ci = 0.0;
    if (in) {
        const double *col = c.Y[li];
        for (int r = 0; r < k; ++r) ci = fma(col[r], c.aux[r], ci);
    }
    const double nc2 = gsum<G>(ci * ci);
    const double lmax = k > 0 ? fmax(fabs(c.lam[0]), fabs(c.lam[k - 1])) : 0.0;
    const double tol = 8.0 * EPS * fmax(fmax(lmax, fabs(gamma)), sqrt(nc2));
    wave_sync();
    c.vec[li] = ci;
    c.dflag[li] = in && fabs(ci) <= tol;
    wave_sync();
    const int m = compact<G>(c, k, tol, li);
    const int nroots = m + 1, kd = k - m;
    const double sw = gsum<G>(li < m ? c.pw[li].y : 0.0);
    double org, tau;
    int its;
    secular_root<G>(c.pw, m, 1.0, gamma, sw, li, li < nroots, org, tau, its);
    wave_sync();
    if (li < nroots) {
        c.root[li] = make_double2(org, tau);
        c.aux[li] = org + tau;
    }
    wave_sync();
    // c-hat_i^2 = -prod_j (p_i - nu_j) / prod_{l != i} (p_i - p_l): the two
    // roots around p_i unpaired, the others paired with the pole beyond them
    double ch = 0.0;
    if (li < m) {
        const double pi = c.pw[li].x;
        auto pm = [&](int j) __attribute__((always_inline)) {
            const double2 rt = c.root[j];
            return (pi - rt.x) - rt.y;
        };
        double prod = pm(li) * -pm(li + 1), num = 1.0, den = 1.0;
        int cnt = 0;
        for (int j = 0; j <= m; ++j) {
            if (j == li || j == li + 1) continue;
            num *= pm(j);
            den *= pi - c.pw[j < li ? j : j - 1].x;
            if ((++cnt & 3) == 0) {
                prod *= num / den;
                num = den = 1.0;
            }
        }
        prod *= num / den;
        const double s = sqrt(fmax(prod, 0.0));
        ch = (c.idx[li] & 0x100) ? -s : s;
    }
    wave_sync();
    if (li < m) c.pw[li].y = ch;
    wave_sync();
    rebuild_columns<G>(c, m, nroots, kd, false, k, li);
    return gmax<G>(its);
}

template <int G>
__global__ __launch_bounds__(64) void sliding_eig(const float *__restrict__ band, int64_t T, int N, int stride,
                                                  double scale, int64_t W, int64_t R, int64_t nchains,
                                                  float *__restrict__ w, int32_t *__restrict__ info)
{
    constexpr int CH = 64 / G;
    __shared__ Chain<G> chains[CH];
    const int h = threadIdx.x / G, li = threadIdx.x % G;
    Chain<G> &c = chains[h];
    const int64_t ch = (int64_t)blockIdx.x * CH + h;
    const int64_t cps = (W + R - 1) / R;
    const int64_t s = ch / cps, w0 = (ch % cps) * R;
    const int nw = ch < nchains ? (int)min<int64_t>(R, W - w0) : 0;
    const float *bs = band + (ch < nchains ? s : 0) * T * N;
    int k = 0;
    int64_t first = 0, bad = -1;
    bool valid = false;
    for (int wi = 0;; ++wi) {
        const bool live = wi < nw;
        if (__ballot(live) == 0) break;
        if (!live) continue;
        const int64_t tf = (w0 + wi) * stride;  // first step of window w0 + wi
        const bool inbad = bad >= tf;
        int its = 0;
        if (!inbad) {
            if (!valid || tf - first >= k) {  // start over from an empty window
                k = 0;
                first = tf;
                valid = true;
            }
            for (; first < tf; ++first) {
                its = max(its, delete_oldest<G>(c, k, li));
                --k;
            }
            for (; k < N;) {
                const int r = append_step<G>(c, k, li, bs + (first + k) * N, scale);
                if (r < 0) {  // a non-finite value: the windows holding this step get NaN
                    bad = first + k;
                    valid = false;
                    k = 0;
                    break;
                }
                its = max(its, r);
                ++k;
            }
        }
        const bool ok = valid && !inbad;
        const int64_t wg = s * W + w0 + wi;
        if (li < N) w[wg * N + li] = ok ? (float)c.lam[N - 1 - li] : __builtin_nanf("");
        if (info != nullptr && li == 0) info[wg] = ok ? its : -1;
    }
}

}  // namespace

hipError_t launch_eigvalsh_sliding(hipStream_t stream, const spec_batch_src *src, int n, int restart, float *w,
                                   int32_t *info)
{
    const int64_t W = (src->T - n) / src->stride + 1;
    const int64_t chains = src->streams * ((W + restart - 1) / restart);
    if (chains == 0) return hipSuccess;
    if (n <= 32)
        hipLaunchKernelGGL(sliding_eig<32>, dim3((unsigned)((chains + 1) / 2)), dim3(64), 0, stream, src->a, src->T, n,
                           src->stride, (double)src->scale, W, (int64_t)restart, chains, w, info);
    else
        hipLaunchKernelGGL(sliding_eig<64>, dim3((unsigned)chains), dim3(64), 0, stream, src->a, src->T, n,
                           src->stride, (double)src->scale, W, (int64_t)restart, chains, w, info);
    return hipGetLastError();
}
