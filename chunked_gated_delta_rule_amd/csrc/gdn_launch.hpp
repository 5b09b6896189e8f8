// Host-side launchers of the gfx950 GDN kernels (internal to the library).
// Each enqueues work on `stream` and returns the launch status; none
// allocates or synchronises. Shapes have already been validated by the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

hipError_t launch_chunk_index(const int32_t *cu_seqlens, int32_t n_max, int32_t nt_max,
                              int32_t *table, hipStream_t stream);

hipError_t launch_front(const void *qkv, const void *conv_w, int32_t d_conv,
                        const int32_t *cu_seqlens, int32_t n_max, int32_t t_max, int32_t h,
                        int32_t hv, float *q, float *k, float *v, hipStream_t stream);

hipError_t launch_intra(bool f32_in, const void *k, const void *v, const float *g,
                        const float *beta, const int32_t *cu_seqlens, const int32_t *table,
                        int32_t nt_max, int32_t h, int32_t hv, int32_t t_max, void *w, float *u,
                        hipStream_t stream);

hipError_t launch_inter(bool f32_in, const void *q, const void *k, const void *w, const float *u,
                        const float *g, const float *h0, const int32_t *cu_seqlens,
                        int32_t n_max, int32_t h, int32_t hv, int32_t t_max, float scale,
                        float *o, float *hT, hipStream_t stream);

}  // namespace gdn
