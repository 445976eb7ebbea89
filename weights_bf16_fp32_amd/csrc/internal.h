// Host-side launchers of the gfx950 kernels, called by the C ABI layer after
// argument validation.  Each enqueues on `stream` and returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/spec.h"

hipError_t launch_syrk(hipStream_t stream, const void *X, int xt, int64_t n, int64_t d, int64_t ldx, void *C, int ct,
                       int64_t ldc, double alpha, double beta);

hipError_t launch_gram_band(hipStream_t stream, const void *H, int ht, int64_t streams, int64_t T, int64_t d,
                            int64_t ld_t, int64_t ld_s, int N, float *out);

hipError_t launch_gram_dense(hipStream_t stream, const void *H, int ht, int64_t streams, int64_t T, int64_t d,
                             int64_t ld_t, int64_t ld_s, int N, int stride, float scale, float *out);

hipError_t launch_eigvalsh_batched(hipStream_t stream, const spec_batch_src *src, int64_t batch, int n, float *w,
                                   int32_t *info);
hipError_t launch_eigh_batched(hipStream_t stream, const spec_batch_src *src, int64_t batch, int n, float *w, float *V,
                               int32_t *info);

hipError_t launch_eigvalsh_sliding(hipStream_t stream, const spec_batch_src *src, int n, int restart, float *w,
                                   int32_t *info);

size_t eig_large_workspace_bytes(int64_t n, int t);

// the eigenvector path: eig_large's workspace followed by its own
size_t eigh_large_workspace_bytes(int64_t n, int t, int64_t k);

hipError_t launch_eigh_large(hipStream_t stream, void *A, int t, int64_t n, int64_t lda, void *w, void *Z,
                             int64_t ldz, int64_t k, void *ws, int32_t *info);

// largest n of the eigenvector path (its back-transformation keeps columns in LDS)
constexpr int64_t EIGVEC_MAX_N = 8192;

hipError_t launch_eig_large(hipStream_t stream, void *A, int t, int64_t n, int64_t lda, void *w, void *ws,
                            int32_t *info);

size_t descriptors_workspace_bytes(int64_t r);

// the MP quantile table of r levels for the aspect ratio of p, into ws
hipError_t launch_mp_table(hipStream_t stream, const spec_desc_params *p, int64_t r, void *ws);

hipError_t launch_eigvalsh_batched_desc(hipStream_t stream, const spec_batch_src *src, int64_t batch, int n, float *w,
                                        int32_t *info, const spec_desc_params *p, spec_desc *out, void *ws);

// spectra lengths the library-held MP table of spec_descriptors_static covers
constexpr int64_t DESC_SCRATCH_MAX_R = 32768;

hipError_t launch_descriptors_static(hipStream_t stream, const void *w, int wt, int64_t batch, int64_t r, int64_t ldw,
                                     const spec_desc_params *p, spec_desc *out);

hipError_t launch_descriptors(hipStream_t stream, const void *w, int wt, int64_t batch, int64_t r, int64_t ldw,
                              const spec_desc_params *p, spec_desc *out, void *ws);

hipError_t launch_desc_smooth(hipStream_t stream, const spec_desc *in, int64_t streams, int64_t W, double alpha,
                              spec_desc *out);

hipError_t launch_spectrum_robust(hipStream_t stream, const void *w, int wt, int64_t batch, int64_t r, int64_t ldw,
                                  const spec_robust_params *p, spec_robust *out);

hipError_t launch_topk_ritz(hipStream_t stream, const float *A, int64_t n, int64_t lda, const float *Omega, int q,
                            float *w, float *P, int64_t ldp, void *ws, int32_t *info);

hipError_t launch_tail_pair_screen(hipStream_t stream, const void *U, const void *V, int dt, int64_t n, int64_t ldu,
                                   int64_t ldv, int64_t i0, int64_t t, int64_t head_dim, double eps, double *absdot,
                                   int64_t ldo, uint8_t *keep, int64_t ldk, int64_t *count);

size_t project_weight_workspace_bytes(int64_t d);

hipError_t launch_project_weight(hipStream_t stream, const void *W, int wt, int64_t d, int64_t ldw, const float *P,
                                 int64_t ldp, int k, float *Wp, int64_t ldo, float *X, int64_t ldx, void *ws);

// Kernel timing brackets (timing.cpp): ktimer_begin returns a slot (or -1 when
// the kernel is not being timed); ktimer_end records the matching end event.
int ktimer_begin(hipStream_t stream, int id);
void ktimer_end(hipStream_t stream, int slot);

struct KTimer {
    hipStream_t s;
    int slot;
    KTimer(hipStream_t stream, int id) : s(stream), slot(ktimer_begin(stream, id)) {}
    ~KTimer() { ktimer_end(s, slot); }
};
