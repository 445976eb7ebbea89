// C ABI of the spectral library: argument validation and dispatch to the
// gfx950 kernels.  Every check runs on the host before anything is enqueued;
// nothing here allocates device memory or synchronises.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "internal.h"

namespace {

inline bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

inline int from_hip(hipError_t e) { return e == hipSuccess ? SPEC_OK : SPEC_EHIP; }

inline size_t elt_size(int t) { return t == SPEC_BF16 ? 2 : (t == SPEC_F32 ? 4 : 8); }

// the descriptor parameters for spectra of r values
int check_desc_params(int64_t r, const spec_desc_params *p)
{
    if (p == nullptr || r < 2) return SPEC_EINVAL;
    if (p->k < 1 || p->k >= r || p->n_samples < 1 || p->p_dim < 1) return SPEC_EINVAL;
    if (!(p->top_frac >= 0.0 && p->top_frac <= 1.0) || !(p->tail_frac >= 0.0 && p->tail_frac <= 1.0) ||
        !(p->small_rel >= 0.0))
        return SPEC_EINVAL;
    if (p->sigma2_mode < SPEC_SIGMA2_GIVEN || p->sigma2_mode > SPEC_SIGMA2_MEAN) return SPEC_EINVAL;
    if (p->sigma2_mode == SPEC_SIGMA2_GIVEN && !(p->sigma2 > 0.0 && isfinite(p->sigma2))) return SPEC_EINVAL;
    return SPEC_OK;
}

// the checks spec_descriptors and spec_descriptors_static share
int check_descriptors(const void *w, int wt, int64_t batch, int64_t r, int64_t ldw, const spec_desc_params *p,
                      spec_desc *out)
{
    if (w == nullptr || p == nullptr || out == nullptr) return SPEC_EINVAL;
    if (wt != SPEC_F32 && wt != SPEC_F64) return SPEC_EUNSUPPORTED;
    if (batch < 0 || batch > ((int64_t)1 << 31) - 1 || r < 2 || ldw < r) return SPEC_EINVAL;
    if (p->k < 1 || p->k >= r || p->n_samples < 1 || p->p_dim < 1) return SPEC_EINVAL;
    if (!(p->top_frac >= 0.0 && p->top_frac <= 1.0) || !(p->tail_frac >= 0.0 && p->tail_frac <= 1.0) ||
        !(p->small_rel >= 0.0))
        return SPEC_EINVAL;
    if (p->sigma2_mode < SPEC_SIGMA2_GIVEN || p->sigma2_mode > SPEC_SIGMA2_MEAN) return SPEC_EINVAL;
    if (p->sigma2_mode == SPEC_SIGMA2_GIVEN && !(p->sigma2 > 0.0 && isfinite(p->sigma2))) return SPEC_EINVAL;
    if (!aligned(w, elt_size(wt)) || !aligned(out, 8)) return SPEC_EINVAL;
    return SPEC_OK;
}

}  // namespace

extern "C" {

const char *spec_strerror(int status)
{
    switch (status) {
    case SPEC_OK: return "success";
    case SPEC_EINVAL: return "invalid argument (pointer, size, stride or parameter)";
    case SPEC_EUNSUPPORTED: return "unsupported dtype combination or size";
    case SPEC_EWORKSPACE: return "workspace missing or too small";
    case SPEC_EHIP: return "HIP runtime error while enqueueing a kernel";
    default: return "unknown status";
    }
}

const char *spec_version(void) { return "0.1.0"; }

int spec_cov_accumulate(void *stream, const void *X, int xt, int64_t n, int64_t d, int64_t ldx, void *C, int ct,
                        int64_t ldc, double alpha, double beta)
{
    if (C == nullptr || (X == nullptr && n > 0)) return SPEC_EINVAL;
    if (n < 0 || d < 1 || ldc < d || (n > 0 && ldx < d)) return SPEC_EINVAL;
    if (!isfinite(alpha) || !isfinite(beta)) return SPEC_EINVAL;
    const bool pair_ok = (xt == SPEC_BF16 && ct == SPEC_F32) || (xt == SPEC_F32 && ct == SPEC_F32) ||
                         (xt == SPEC_F32 && ct == SPEC_F64);
    if (!pair_ok) return SPEC_EUNSUPPORTED;
    if (!aligned(C, elt_size(ct)) || (X != nullptr && !aligned(X, elt_size(xt)))) return SPEC_EINVAL;
    if (d > (int64_t)1 << 20 || n > ((int64_t)1 << 40)) return SPEC_EUNSUPPORTED;
    KTimer kt((hipStream_t)stream, SPEC_KT_SYRK);
    return from_hip(launch_syrk((hipStream_t)stream, X, xt, n, d, ldx, C, ct, ldc, alpha, beta));
}

int spec_gram_window(void *stream, const void *H, int ht, int64_t streams, int64_t T, int64_t d, int64_t ld_t,
                     int64_t ld_s, int N, int stride, double scale, int layout, float *out)
{
    if (H == nullptr || out == nullptr) return SPEC_EINVAL;
    if (ht != SPEC_BF16 && ht != SPEC_F32) return SPEC_EUNSUPPORTED;
    if (streams < 1 || T < 1 || d < 1 || N < 1 || N > 64 || N > T || stride < 1) return SPEC_EINVAL;
    if (ld_t < d || ld_s < T * ld_t) return SPEC_EINVAL;
    if (!aligned(H, elt_size(ht)) || !aligned(out, 4)) return SPEC_EINVAL;
    if (!isfinite(scale)) return SPEC_EINVAL;
    KTimer kt((hipStream_t)stream, SPEC_KT_GRAM);
    if (layout == SPEC_GRAM_BAND)
        return from_hip(launch_gram_band((hipStream_t)stream, H, ht, streams, T, d, ld_t, ld_s, N, out));
    if (layout == SPEC_GRAM_DENSE) {
        if (streams * ((T - N) / stride + 1) > ((int64_t)1 << 31) - 1) return SPEC_EUNSUPPORTED;
        return from_hip(
            launch_gram_dense((hipStream_t)stream, H, ht, streams, T, d, ld_t, ld_s, N, stride, (float)scale, out));
    }
    return SPEC_EINVAL;
}

// the batch source of the small solvers: its kind, strides and batch count
static int check_batch_src(const spec_batch_src *src, int64_t batch, int n)
{
    if (src == nullptr || src->a == nullptr) return SPEC_EINVAL;
    if (batch < 0 || batch > ((int64_t)1 << 31) - 1) return SPEC_EINVAL;
    if (!aligned(src->a, 4)) return SPEC_EINVAL;
    if (src->kind == SPEC_SRC_DENSE) {
        if (src->lda < n || src->stride_a < (int64_t)n * src->lda) return SPEC_EINVAL;
    } else if (src->kind == SPEC_SRC_BAND) {
        if (src->streams < 1 || src->T < n || src->stride < 1 || !isfinite(src->scale)) return SPEC_EINVAL;
        const int64_t W = (src->T - n) / src->stride + 1;
        if (batch != src->streams * W) return SPEC_EINVAL;
    } else {
        return SPEC_EINVAL;
    }
    return SPEC_OK;
}

int spec_eigvalsh_batched(void *stream, const spec_batch_src *src, int64_t batch, int n, float *w, int32_t *info)
{
    if (src == nullptr || w == nullptr || src->a == nullptr) return SPEC_EINVAL;
    if (n < 1 || n > 64) return n > 64 ? SPEC_EUNSUPPORTED : SPEC_EINVAL;
    if (!aligned(w, 4) || (info != nullptr && !aligned(info, 4))) return SPEC_EINVAL;
    const int st = check_batch_src(src, batch, n);
    if (st != SPEC_OK) return st;
    KTimer kt((hipStream_t)stream, SPEC_KT_SMALL_EIG);
    return from_hip(launch_eigvalsh_batched((hipStream_t)stream, src, batch, n, w, info));
}

int spec_eigh_batched(void *stream, const spec_batch_src *src, int64_t batch, int n, float *w, float *V,
                      int32_t *info)
{
    if (src == nullptr || w == nullptr || V == nullptr || src->a == nullptr) return SPEC_EINVAL;
    if (n < 1 || n > 32) return n > 32 ? SPEC_EUNSUPPORTED : SPEC_EINVAL;
    if (!aligned(w, 4) || !aligned(V, 4) || (info != nullptr && !aligned(info, 4))) return SPEC_EINVAL;
    const int st = check_batch_src(src, batch, n);
    if (st != SPEC_OK) return st;
    return from_hip(launch_eigh_batched((hipStream_t)stream, src, batch, n, w, V, info));
}

int spec_eigvalsh_sliding(void *stream, const spec_batch_src *src, int64_t batch, int n, int restart, float *w,
                          int32_t *info)
{
    if (src == nullptr || w == nullptr || src->a == nullptr || src->kind != SPEC_SRC_BAND) return SPEC_EINVAL;
    if (n < 1 || n > 64) return n > 64 ? SPEC_EUNSUPPORTED : SPEC_EINVAL;
    if (batch < 0 || batch > ((int64_t)1 << 31) - 1 || restart < 1) return SPEC_EINVAL;
    if (!aligned(w, 4) || !aligned(src->a, 4) || (info != nullptr && !aligned(info, 4))) return SPEC_EINVAL;
    if (src->streams < 1 || src->T < n || src->stride < 1 || !isfinite(src->scale)) return SPEC_EINVAL;
    const int64_t W = (src->T - n) / src->stride + 1;
    if (batch != src->streams * W) return SPEC_EINVAL;
    return from_hip(launch_eigvalsh_sliding((hipStream_t)stream, src, n, restart, w, info));
}

int spec_eigvalsh_batched_desc(void *stream, const spec_batch_src *src, int64_t batch, int n, float *w, int32_t *info,
                               const spec_desc_params *p, spec_desc *out, void *ws, size_t ws_bytes)
{
    if (src == nullptr || src->a == nullptr || out == nullptr) return SPEC_EINVAL;
    if (n < 2 || n > 32) return n > 32 ? SPEC_EUNSUPPORTED : SPEC_EINVAL;
    if (batch < 0 || batch > ((int64_t)1 << 31) - 1) return SPEC_EINVAL;
    const int st = check_desc_params(n, p);
    if (st != SPEC_OK) return st;
    if ((w != nullptr && !aligned(w, 4)) || !aligned(src->a, 4) || (info != nullptr && !aligned(info, 4)) ||
        !aligned(out, 8))
        return SPEC_EINVAL;
    if (src->kind == SPEC_SRC_DENSE) {
        if (src->lda < n || src->stride_a < (int64_t)n * src->lda) return SPEC_EINVAL;
    } else if (src->kind == SPEC_SRC_BAND) {
        if (src->streams < 1 || src->T < n || src->stride < 1 || !isfinite(src->scale)) return SPEC_EINVAL;
        const int64_t W = (src->T - n) / src->stride + 1;
        if (batch != src->streams * W) return SPEC_EINVAL;
    } else {
        return SPEC_EINVAL;
    }
    if (ws == nullptr || ws_bytes < descriptors_workspace_bytes(n)) return SPEC_EWORKSPACE;
    if (!aligned(ws, 256)) return SPEC_EINVAL;
    KTimer kt((hipStream_t)stream, SPEC_KT_SMALL_EIG);
    return from_hip(launch_eigvalsh_batched_desc((hipStream_t)stream, src, batch, n, w, info, p, out, ws));
}

int spec_eigvalsh_large_workspace(int64_t n, int t, size_t *bytes)
{
    if (bytes == nullptr || n < 1) return SPEC_EINVAL;
    if (t != SPEC_F32 && t != SPEC_F64) return SPEC_EUNSUPPORTED;
    if ((t == SPEC_F32 && n > 32768) || (t == SPEC_F64 && n > 8192)) return SPEC_EUNSUPPORTED;
    *bytes = eig_large_workspace_bytes(n, t);
    return SPEC_OK;
}

int spec_eigvalsh_large(void *stream, void *A, int t, int64_t n, int64_t lda, void *w, void *ws, size_t ws_bytes,
                        int32_t *info)
{
    size_t need = 0;
    int st = spec_eigvalsh_large_workspace(n, t, &need);
    if (st != SPEC_OK) return st;
    if (A == nullptr || w == nullptr || lda < n || lda >= ((int64_t)1 << 22)) return SPEC_EINVAL;
    if (!aligned(A, 16) || !aligned(w, elt_size(t)) || (info != nullptr && !aligned(info, 4))) return SPEC_EINVAL;
    if (ws == nullptr || ws_bytes < need) return SPEC_EWORKSPACE;
    if (!aligned(ws, 256)) return SPEC_EINVAL;
    return from_hip(launch_eig_large((hipStream_t)stream, A, t, n, lda, w, ws, info));
}

int spec_eigh_large_workspace(int64_t n, int t, int64_t k, size_t *bytes)
{
    if (bytes == nullptr || n < 1 || k < 1 || k > n) return SPEC_EINVAL;
    if (t != SPEC_F32 && t != SPEC_F64) return SPEC_EUNSUPPORTED;
    if (n > EIGVEC_MAX_N) return SPEC_EUNSUPPORTED;
    *bytes = eigh_large_workspace_bytes(n, t, k);
    return SPEC_OK;
}

int spec_eigh_large(void *stream, void *A, int t, int64_t n, int64_t lda, void *w, void *Z, int64_t ldz, int64_t k,
                    void *ws, size_t ws_bytes, int32_t *info)
{
    size_t need = 0;
    int st = spec_eigh_large_workspace(n, t, k, &need);
    if (st != SPEC_OK) return st;
    if (A == nullptr || w == nullptr || Z == nullptr || lda < n || lda >= ((int64_t)1 << 22) || ldz < k)
        return SPEC_EINVAL;
    if (!aligned(A, 16) || !aligned(w, elt_size(t)) || !aligned(Z, elt_size(t)) ||
        (info != nullptr && !aligned(info, 4)))
        return SPEC_EINVAL;
    // Z is addressed with 32-bit byte offsets (rows up to n + 128 reached)
    if ((n + 128) * ldz * (int64_t)elt_size(t) >= ((int64_t)1 << 31)) return SPEC_EUNSUPPORTED;
    if (ws == nullptr || ws_bytes < need) return SPEC_EWORKSPACE;
    if (!aligned(ws, 256)) return SPEC_EINVAL;
    return from_hip(launch_eigh_large((hipStream_t)stream, A, t, n, lda, w, Z, ldz, k, ws, info));
}

int spec_descriptors_workspace(int64_t r, size_t *bytes)
{
    if (bytes == nullptr || r < 1) return SPEC_EINVAL;
    *bytes = descriptors_workspace_bytes(r);
    return SPEC_OK;
}

int spec_descriptors_static(void *stream, const void *w, int wt, int64_t batch, int64_t r, int64_t ldw,
                            const spec_desc_params *p, spec_desc *out)
{
    const int st = check_descriptors(w, wt, batch, r, ldw, p, out);
    if (st != SPEC_OK) return st;
    if (r > DESC_SCRATCH_MAX_R) return SPEC_EUNSUPPORTED;
    return from_hip(launch_descriptors_static((hipStream_t)stream, w, wt, batch, r, ldw, p, out));
}

int spec_descriptors(void *stream, const void *w, int wt, int64_t batch, int64_t r, int64_t ldw,
                     const spec_desc_params *p, spec_desc *out, void *ws, size_t ws_bytes)
{
    const int st = check_descriptors(w, wt, batch, r, ldw, p, out);
    if (st != SPEC_OK) return st;
    if (ws == nullptr || ws_bytes < descriptors_workspace_bytes(r)) return SPEC_EWORKSPACE;
    if (!aligned(ws, 256)) return SPEC_EINVAL;
    return from_hip(launch_descriptors((hipStream_t)stream, w, wt, batch, r, ldw, p, out, ws));
}

int spec_eigvalsh_topk(void *stream, const void *A, int t, int64_t n, int64_t lda, const void *Omega, int q, void *w,
                       void *ws, size_t ws_bytes)
{
    if (t != SPEC_F32) return SPEC_EUNSUPPORTED;
    if (A == nullptr || Omega == nullptr || w == nullptr) return SPEC_EINVAL;
    if (n < 64 || n > 32768 || lda < n || lda >= ((int64_t)1 << 22) || q < 0 || q > 16) return SPEC_EINVAL;
    if (!aligned(A, 16) || !aligned(Omega, 16) || !aligned(w, 4)) return SPEC_EINVAL;
    if (ws == nullptr || ws_bytes < eig_large_workspace_bytes(n, SPEC_F32)) return SPEC_EWORKSPACE;
    if (!aligned(ws, 256)) return SPEC_EINVAL;
    return from_hip(launch_topk_ritz((hipStream_t)stream, (const float *)A, n, lda, (const float *)Omega, q,
                                     (float *)w, nullptr, 0, ws, nullptr));
}

int spec_eigvecs_topk(void *stream, const void *A, int t, int64_t n, int64_t lda, const void *Omega, int q, void *w,
                      void *P, int64_t ldp, void *ws, size_t ws_bytes, int32_t *info)
{
    if (t != SPEC_F32) return SPEC_EUNSUPPORTED;
    if (A == nullptr || Omega == nullptr || w == nullptr || P == nullptr) return SPEC_EINVAL;
    if (n < 64 || n > 32768 || lda < n || lda >= ((int64_t)1 << 22) || q < 0 || q > 16) return SPEC_EINVAL;
    if (ldp < 32 || ldp >= ((int64_t)1 << 22)) return SPEC_EINVAL;
    if (!aligned(A, 16) || !aligned(Omega, 16) || !aligned(w, 4) || !aligned(P, 4)) return SPEC_EINVAL;
    if (info != nullptr && !aligned(info, 4)) return SPEC_EINVAL;
    if (ws == nullptr || ws_bytes < eig_large_workspace_bytes(n, SPEC_F32)) return SPEC_EWORKSPACE;
    if (!aligned(ws, 256)) return SPEC_EINVAL;
    return from_hip(launch_topk_ritz((hipStream_t)stream, (const float *)A, n, lda, (const float *)Omega, q,
                                     (float *)w, (float *)P, ldp, ws, info));
}

int spec_desc_smooth(void *stream, const spec_desc *in, int64_t streams, int64_t W, double alpha, spec_desc *out)
{
    if (in == nullptr || out == nullptr || streams < 0 || streams > ((int64_t)1 << 31) - 1 || W < 1) return SPEC_EINVAL;
    if (!(alpha > 0.0 && alpha <= 1.0)) return SPEC_EINVAL;
    if (!aligned(in, 8) || !aligned(out, 8)) return SPEC_EINVAL;
    const char *a = (const char *)in, *b = (const char *)out;
    const size_t bytes = (size_t)streams * (size_t)W * sizeof(spec_desc);
    if (a < b + bytes && b < a + bytes) return SPEC_EINVAL;  // overlapping
    return from_hip(launch_desc_smooth((hipStream_t)stream, in, streams, W, alpha, out));
}

int spec_spectrum_robust(void *stream, const void *w, int wt, int64_t batch, int64_t r, int64_t ldw,
                         const spec_robust_params *p, spec_robust *out)
{
    if (w == nullptr || p == nullptr || out == nullptr) return SPEC_EINVAL;
    if (wt != SPEC_F32 && wt != SPEC_F64) return SPEC_EUNSUPPORTED;
    if (batch < 0 || batch > ((int64_t)1 << 31) - 1 || r < 2 || ldw < r) return SPEC_EINVAL;
    if (p->bins < 1 || p->bins > 64 || p->n_samples < 1 || p->p_dim < 1) return SPEC_EINVAL;
    if (!(p->winsor_frac >= 0.0 && p->winsor_frac <= 0.5) || !(p->mad_k > 0.0 && isfinite(p->mad_k)))
        return SPEC_EINVAL;
    if (p->sigma2_mode < SPEC_SIGMA2_GIVEN || p->sigma2_mode > SPEC_SIGMA2_WINSOR) return SPEC_EINVAL;
    if (p->sigma2_mode == SPEC_SIGMA2_GIVEN && !(p->sigma2 > 0.0 && isfinite(p->sigma2))) return SPEC_EINVAL;
    if (!aligned(w, elt_size(wt)) || !aligned(out, 8)) return SPEC_EINVAL;
    return from_hip(launch_spectrum_robust((hipStream_t)stream, w, wt, batch, r, ldw, p, out));
}

int spec_project_weight_workspace(int64_t d, size_t *bytes)
{
    if (bytes == nullptr || d < 1 || d > 65536) return SPEC_EINVAL;
    *bytes = project_weight_workspace_bytes(d);
    return SPEC_OK;
}

int spec_project_weight(void *stream, const void *W, int wt, int64_t d, int64_t ldw, const void *P, int64_t ldp, int k,
                        void *Wp, int64_t ldo, void *X, int64_t ldx, void *ws, size_t ws_bytes)
{
    if (wt != SPEC_BF16 && wt != SPEC_F32) return SPEC_EUNSUPPORTED;
    if (W == nullptr || P == nullptr || Wp == nullptr) return SPEC_EINVAL;
    if (d < 1 || d > 65536 || k < 1 || k > 32 || k > d) return SPEC_EINVAL;
    if (ldw < d || ldp < k || ldo < k || (X != nullptr && ldx < k)) return SPEC_EINVAL;
    const int64_t vec = wt == SPEC_BF16 ? 8 : 4;  // 16-byte rows
    if (!aligned(W, 16) || ldw % vec != 0) return SPEC_EINVAL;
    if (!aligned(P, 4) || !aligned(Wp, 4) || (X != nullptr && !aligned(X, 4))) return SPEC_EINVAL;
    if (ws == nullptr || ws_bytes < project_weight_workspace_bytes(d)) return SPEC_EWORKSPACE;
    if (!aligned(ws, 256)) return SPEC_EINVAL;
    return from_hip(launch_project_weight((hipStream_t)stream, W, wt, d, ldw, (const float *)P, ldp, k, (float *)Wp,
                                          ldo, (float *)X, ldx, ws));
}

int spec_tail_pair_screen(void *stream, const void *U, const void *V, int dt, int64_t n, int64_t ldu, int64_t ldv,
                          int64_t i0, int64_t t, int64_t head_dim, double eps, double *absdot, int64_t ldo,
                          uint8_t *keep, int64_t ldk, int64_t *count)
{
    if (dt != SPEC_F32 && dt != SPEC_F64) return SPEC_EUNSUPPORTED;
    if (U == nullptr || V == nullptr || keep == nullptr) return SPEC_EINVAL;
    if (n < 1 || i0 < 0 || t < 1 || t > 65535 || head_dim < 1 || !(eps > 0.0 && isfinite(eps))) return SPEC_EINVAL;
    if (i0 + t > ldu || i0 + t > ldv || ldk < t || (absdot != nullptr && ldo < t)) return SPEC_EINVAL;
    if (!aligned(U, elt_size(dt)) || !aligned(V, elt_size(dt))) return SPEC_EINVAL;
    if ((absdot != nullptr && !aligned(absdot, 8)) || (count != nullptr && !aligned(count, 8))) return SPEC_EINVAL;
    return from_hip(launch_tail_pair_screen((hipStream_t)stream, U, V, dt, n, ldu, ldv, i0, t, head_dim, eps, absdot,
                                            ldo, keep, ldk, count));
}

}  // extern "C"
