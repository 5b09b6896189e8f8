// Conv + SiLU + L2-norm front: turns the packed pre-conv q|k|v channels (bf16)
// into the fp32 q, k, v of the chunk forward.
//
//  * Causal depthwise conv, tap d_conv-1 is the current token, zero history at
//    each sequence start, no bias (llama.cpp PR 399, "How (exactness)").
//  * SiLU y = x / (1 + e^-x) on every channel (hardware exp2 and reciprocal).
//  * Each q and k head (128 channels) is scaled by 1 / sqrt(sum y^2 + 1e-6)
//    with the whole row kept in registers (AMX page, section 7).
//
// Thread layout: a thread owns 8 consecutive channels (one 16-byte load per
// tap); 16 threads cover one 128-channel head, so the head's sum of squares is
// a 16-lane butterfly inside the wave. A work-group covers 2048 channels of
// kTokens consecutive tokens. HBM-bound: bf16 rows are read once from HBM (the
// d_conv-1 re-reads hit cache) and fp32 rows written once.
#include "gdn_common.hpp"
#include "gdn_launch.hpp"

namespace gdn {

namespace {

constexpr int kTokens = 16;
constexpr int kMaxTaps = 8;

__global__ __launch_bounds__(kThreads) void front_kernel(
    const uint16_t *__restrict__ qkv, const uint16_t *__restrict__ conv_w, int d_conv,
    const int32_t *__restrict__ cu, int n_max, int t_max, int h, int hv,
    float *__restrict__ q, float *__restrict__ k, float *__restrict__ v) {
  const int channels = (2 * h + hv) * kD;
  const int c0 = (blockIdx.x * kThreads + threadIdx.x) * 8;
  const bool active = c0 < channels;  // inactive lanes still join the butterfly
  const int t_begin = blockIdx.y * kTokens;
  const int t_total = cu_at(cu, n_max, t_max);
  if (t_begin >= t_total) return;

  float wt[8][kMaxTaps];
  if (active) {
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
      for (int j = 0; j < kMaxTaps; ++j)
        wt[c][j] = j < d_conv ? bf16_bits_to_float(conv_w[(int64_t)(c0 + c) * d_conv + j]) : 0.f;
  }
  // sequence containing t_begin: last s with cu[s] <= t_begin (and cu[s+1] > t_begin)
  int lo = 0, hi = n_max;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu_at(cu, mid, t_max) <= t_begin) lo = mid; else hi = mid;
  }
  int s = lo;
  const bool is_qk = c0 < 2 * h * kD;
  const int t_end = min(t_begin + kTokens, t_total);
  for (int t = t_begin; t < t_end; ++t) {
    while (s + 1 < n_max && cu_at(cu, s + 1, t_max) <= t) ++s;
    const int bos = min(cu_at(cu, s, t_max), t);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (active) {
#pragma unroll
      for (int j = 0; j < kMaxTaps; ++j) {
        const int src = t - (d_conv - 1) + j;
        if (j >= d_conv || src < bos) continue;
        const u32x4 raw = *reinterpret_cast<const u32x4 *>(qkv + (int64_t)src * channels + c0);
        float x[8];
        unpack8(raw, x);
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[c] = fmaf(x[c], wt[c][j], acc[c]);
      }
    }
    float y[8];
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      y[c] = silu(acc[c]);
      ss = fmaf(y[c], y[c], ss);
    }
    // 16 consecutive lanes hold one head (heads start on 128-channel boundaries)
    ss = sum16(ss);
    if (!active) continue;
    float *dst;
    if (c0 < h * kD) {
      dst = q + (int64_t)t * h * kD + c0;
    } else if (is_qk) {
      dst = k + (int64_t)t * h * kD + (c0 - h * kD);
    } else {
      dst = v + (int64_t)t * hv * kD + (c0 - 2 * h * kD);
    }
    if (is_qk) {
      const float r = 1.f / sqrtf(ss + 1e-6f);
#pragma unroll
      for (int c = 0; c < 8; ++c) y[c] *= r;
    }
    reinterpret_cast<f32x4 *>(dst)[0] = f32x4{y[0], y[1], y[2], y[3]};
    reinterpret_cast<f32x4 *>(dst)[1] = f32x4{y[4], y[5], y[6], y[7]};
  }
}

}  // namespace

hipError_t launch_front(const void *qkv, const void *conv_w, int32_t d_conv,
                        const int32_t *cu_seqlens, int32_t n_max, int32_t t_max, int32_t h,
                        int32_t hv, float *q, float *k, float *v, hipStream_t stream,
                        KernelEvents ev) {
  if (d_conv < 1 || d_conv > kMaxTaps) return hipErrorInvalidValue;
  const int channels = (2 * h + hv) * kD;
  const dim3 grid((channels / 8 + kThreads - 1) / kThreads, (t_max + kTokens - 1) / kTokens);
  if (grid.y == 0) return hipSuccess;
  hipExtLaunchKernelGGL(front_kernel, grid, dim3(kThreads), 0, stream, ev.start, ev.stop, 0,
                        static_cast<const uint16_t *>(qkv), static_cast<const uint16_t *>(conv_w),
                        d_conv, cu_seqlens, n_max, t_max, h, hv, q, k, v);
  return hipGetLastError();
}

}  // namespace gdn
