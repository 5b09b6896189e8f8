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
// row); 16 threads cover one 128-channel head, so the head's sum of squares is
// a 16-lane butterfly inside the wave. A work-group covers 2048 channels of
// kTokens consecutive tokens and walks them in order, keeping the last
// kTaps - 1 rows in registers: each token loads one new row, requested one
// token ahead. The tap count is a template parameter (the window is a register
// array and needs constant indices). Taps are accumulated oldest first with
// rows before the sequence start skipped, the order the front fused into
// stage 1 uses, so both produce the same bits. HBM-bound: bf16 rows are read
// once (plus a kTaps - 1 row halo per work-group) and fp32 rows written once.
#include "gdn_common.hpp"
#include "gdn_launch.hpp"

namespace gdn {

namespace {

constexpr int kTokens = 64;
constexpr int kMaxTaps = 8;

template <int kTaps>
__global__ __launch_bounds__(kThreads) void front_kernel(
    const uint16_t *__restrict__ qkv, const uint16_t *__restrict__ conv_w,
    const int32_t *__restrict__ cu, int n_max, int t_max, int h, int hv,
    float *__restrict__ q, float *__restrict__ k, float *__restrict__ v) {
  const int channels = (2 * h + hv) * kD;
  // flat work-group number -> (channel block, token block), channels fastest
  const int cblocks = (channels / 8 + kThreads - 1) / kThreads;
  const int wg = flat_block();
  const int c0 = (wg % cblocks * kThreads + threadIdx.x) * 8;
  const bool active = c0 < channels;  // inactive lanes still join the butterfly
  const int t_begin = wg / cblocks * kTokens;
  const int t_total = cu_at(cu, n_max, t_max);
  if (t_begin >= t_total) return;
  const int t_end = min(t_begin + kTokens, t_total);

  float wt[8][kTaps];
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int j = 0; j < kTaps; ++j)
      wt[c][j] = active ? bf16_bits_to_float(conv_w[(int64_t)(c0 + c) * kTaps + j]) : 0.f;
  auto row = [&](int r) __attribute__((always_inline)) {
    return active ? *reinterpret_cast<const u32x4 *>(qkv + (int64_t)r * channels + c0)
                  : u32x4{0u, 0u, 0u, 0u};
  };
  // sequence containing t_begin: last s with cu[s] <= t_begin (and cu[s+1] > t_begin)
  int lo = 0, hi = n_max;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu_at(cu, mid, t_max) <= t_begin) lo = mid; else hi = mid;
  }
  int s = lo;
  const bool is_qk = c0 < 2 * h * kD;
  // win[j] holds row t - (kTaps - 1) + j (raw bf16); rows before 0 are never used
  u32x4 win[kTaps];
#pragma unroll
  for (int j = 0; j < kTaps - 1; ++j) {
    const int r = t_begin - (kTaps - 1) + j;
    win[j] = r >= 0 ? row(r) : u32x4{0u, 0u, 0u, 0u};
  }
  win[kTaps - 1] = row(t_begin);
  for (int t = t_begin; t < t_end; ++t) {
    const u32x4 next = t + 1 < t_end ? row(t + 1) : u32x4{0u, 0u, 0u, 0u};
    while (s + 1 < n_max && cu_at(cu, s + 1, t_max) <= t) ++s;
    const int bos = min(cu_at(cu, s, t_max), t);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < kTaps; ++j) {
      if (t - (kTaps - 1) + j < bos) continue;  // before the sequence start (same for all lanes)
      float x[8];
      unpack8(win[j], x);
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[c] = fmaf(x[c], wt[c][j], acc[c]);
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
#pragma unroll
    for (int j = 0; j < kTaps - 1; ++j) win[j] = win[j + 1];
    win[kTaps - 1] = next;
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
  const int64_t cblocks = (channels / 8 + kThreads - 1) / kThreads;
  const int64_t tblocks = (static_cast<int64_t>(t_max) + kTokens - 1) / kTokens;
  if (tblocks == 0) return hipSuccess;
  dim3 grid;
  if (!flat_grid(cblocks * tblocks, kThreads, grid)) return hipErrorInvalidValue;
  const uint16_t *x = static_cast<const uint16_t *>(qkv);
  const uint16_t *w = static_cast<const uint16_t *>(conv_w);
#define GDN_LAUNCH_FRONT(TAPS)                                                                   \
  hipExtLaunchKernelGGL(front_kernel<TAPS>, grid, dim3(kThreads), 0, stream, ev.start, ev.stop, \
                        0, x, w, cu_seqlens, n_max, t_max, h, hv, q, k, v)
  switch (d_conv) {
    case 1: GDN_LAUNCH_FRONT(1); break;
    case 2: GDN_LAUNCH_FRONT(2); break;
    case 3: GDN_LAUNCH_FRONT(3); break;
    case 4: GDN_LAUNCH_FRONT(4); break;
    case 5: GDN_LAUNCH_FRONT(5); break;
    case 6: GDN_LAUNCH_FRONT(6); break;
    case 7: GDN_LAUNCH_FRONT(7); break;
    default: GDN_LAUNCH_FRONT(8); break;
  }
#undef GDN_LAUNCH_FRONT
  return hipGetLastError();
}

}  // namespace gdn
