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

size_t eig_large_workspace_bytes(int64_t n, int t);

hipError_t launch_eig_large(hipStream_t stream, void *A, int t, int64_t n, int64_t lda, void *w, void *ws,
                            int32_t *info);

size_t descriptors_workspace_bytes(int64_t r);

hipError_t launch_descriptors(hipStream_t stream, const void *w, int wt, int64_t batch, int64_t r, int64_t ldw,
                              const spec_desc_params *p, spec_desc *out, void *ws);

hipError_t launch_desc_smooth(hipStream_t stream, const spec_desc *in, int64_t streams, int64_t W, double alpha,
                              spec_desc *out);

hipError_t launch_spectrum_robust(hipStream_t stream, const void *w, int wt, int64_t batch, int64_t r, int64_t ldw,
                                  const spec_robust_params *p, spec_robust *out);

hipError_t launch_topk_ritz(hipStream_t stream, const float *A, int64_t n, int64_t lda, const float *Omega, int q,
                            float *w, float *P, int64_t ldp, void *ws);

size_t project_weight_workspace_bytes(int64_t d);

hipError_t launch_project_weight(hipStream_t stream, const void *W, int wt, int64_t d, int64_t ldw, const float *P,
                                 int64_t ldp, int k, float *Wp, int64_t ldo, float *X, int64_t ldx, void *ws);
