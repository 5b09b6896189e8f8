// Token-serial recurrent kernel: decode and speculative verify.
//
// "Chunking Qwen3.5's gated DeltaNet ..." (Alloy page), section "What is the
// gated delta rule in Qwen3.5?": per token t the state S (Dk x Dv) is decayed
// by e^{g_t}, corrected by beta_t (v_t - S^T k_t), written back as
// S += k_t d^T, and the output o_t = scale S^T q_t is read after the write.
// Section "How does decode run a sequential update on a GPU?" of the same page
// parallelises one token's update over the state, which stays on chip between
// the tokens of a call; section "Why keep the serial kernel at all?" is why a
// verify batch (1 to 16 draft tokens, llama.cpp PR 399, "What") runs the same
// token-serial fp32 arithmetic as decode instead of the chunked form, whose
// triangular inverse reorders it.
//
// gfx950 mapping: one 256-thread work-group per (sequence, value head) holds
// the whole 128 x 128 fp32 state in registers, 64 values per thread, and walks
// the sequence's tokens in order. States are value-major (St[v][d] = S[d][v],
// as h0 / hT). Thread (rg, ds) = (tid / 8, tid % 8) owns rows v = 4 rg .. 4 rg
// + 3 and columns d = 32 j + 4 ds .. 32 j + 4 ds + 3 (j < 4), so the eight
// threads of a row group are eight consecutive lanes of one wave: the two sums
// over d of each token (S^T k before the write, S^T q after it) finish with
// three DPP steps and no LDS or barrier. The state is read from h0 and written
// to hT once, each 16-byte access instruction covering whole 128-byte lines
// (eight lanes per line), with non-temporal loads and stores: the state is
// streamed through once, so it is not kept in the caches. The next token's
// k, q, v, g and beta are requested while the current one is processed (one
// buffer range per token row, empty past the sequence, so that request reads
// zeros).
#include "gdn_common.hpp"
#include "gdn_launch.hpp"

namespace gdn {

namespace {

constexpr int kRecThreads = 256;

template <int kCtrl>
__device__ __forceinline__ float dpp_take(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), kCtrl,
                                                                0xf, 0xf, true));
}

// Sum over the eight lanes 8 j .. 8 j + 7 (every one of them gets it): the two
// quad swaps leave each lane its quad's sum, the half-row mirror pairs lane i
// with lane 7 - i of the other quad. Floating-point addition commutes, so all
// eight lanes hold the same bits.
__device__ __forceinline__ float sum8(float x) {
  x += dpp_take<0xB1>(x);   // quad_perm [1, 0, 3, 2]
  x += dpp_take<0x4E>(x);   // quad_perm [2, 3, 0, 1]
  x += dpp_take<0x141>(x);  // row_half_mirror
  return x;
}

// Four consecutive elements of a row as floats.
template <bool kF32In>
__device__ __forceinline__ void load4(rsrc_t r, uint32_t off, float (&x)[4]) {
  if constexpr (kF32In) {
    const u32x4 w = buf_load16(r, off);
#pragma unroll
    for (int c = 0; c < 4; ++c) x[c] = __uint_as_float(w[c]);
  } else {
    const u32x2 w = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      x[2 * c] = __uint_as_float(w[c] << 16);
      x[2 * c + 1] = __uint_as_float(w[c] & 0xffff0000u);
    }
  }
}

// Elements 32 j + d4 .. 32 j + d4 + 3 (j < 4) of a row (bf16 or fp32) as
// floats x[4 j + c].
template <bool kF32In>
__device__ __forceinline__ void load16(rsrc_t r, int d4, float (&x)[16]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float y[4];
    load4<kF32In>(r, (32 * j + d4) * (kF32In ? 4 : 2), y);
#pragma unroll
    for (int c = 0; c < 4; ++c) x[4 * j + c] = y[c];
  }
}

template <bool kF32In>
__global__ __launch_bounds__(kRecThreads) void recurrent_kernel(
    const void *__restrict__ qin, const void *__restrict__ kin, const void *__restrict__ vin,
    const float *__restrict__ g, const float *__restrict__ beta, const float *__restrict__ h0,
    const int32_t *__restrict__ cu, float *__restrict__ o, float *__restrict__ hT, int n_max, int H,
    int Hv, int t_max, float scale) {
  constexpr int kEl = kF32In ? 4 : 2;
  const int s = flat_block() / Hv, hv = flat_block() % Hv;
  if (s >= n_max) return;  // past the grid's count (last row)
  const int h = hv / (Hv / H);
  const int tid = threadIdx.x;
  const int v0 = 4 * (tid >> 3), d4 = 4 * (tid & 7);
  const int bos = cu_at(cu, s, t_max), eos = cu_end(cu, s, bos, t_max);
  const int n = eos - bos;

  // token i's row of q, k (key head h) or v (value head hv) as a buffer range;
  // a request for a token past the sequence (i >= n) reads zeros
  const char *qb = static_cast<const char *>(qin) + ((int64_t)bos * H + h) * kD * kEl;
  const char *kb = static_cast<const char *>(kin) + ((int64_t)bos * H + h) * kD * kEl;
  const char *vb = static_cast<const char *>(vin) + ((int64_t)bos * Hv + hv) * kD * kEl;
  const int64_t qk_row = (int64_t)H * kD * kEl, v_row = (int64_t)Hv * kD * kEl;
  auto row = [&](const char *base, int64_t stride, int i) __attribute__((always_inline)) {
    return make_rsrc(base + i * stride, i < n ? kD * kEl : 0u);
  };
  // g and beta of token i (clamped to the last token: read, never used, past it)
  auto gate = [&](const float *p, int i) __attribute__((always_inline)) {
    return p[(int64_t)(bos + min(i, n - 1)) * Hv + hv];
  };

  // state rows v0 .. v0 + 3, columns 32 j + d4 .. 32 j + d4 + 3
  f32x4 St[4][4];
  const int64_t sb = ((int64_t)s * Hv + hv) * kD * kD;
  if (h0) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        St[i][j] = __builtin_nontemporal_load(
            reinterpret_cast<const f32x4 *>(h0 + sb + (v0 + i) * kD + 32 * j + d4));
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) St[i][j] = zero4();
  }

  float kx[16], qx[16], vx[4], gx = 0.f, bx = 0.f;
  if (n > 0) {
    load16<kF32In>(row(kb, qk_row, 0), d4, kx);
    load16<kF32In>(row(qb, qk_row, 0), d4, qx);
    load4<kF32In>(row(vb, v_row, 0), v0 * kEl, vx);
    gx = gate(g, 0);
    bx = gate(beta, 0);
  }
  for (int i = 0; i < n; ++i) {
    const int t = bos + i;
    const float gt = gx, bt = bx;
    const float kc[16] = {kx[0], kx[1], kx[2], kx[3], kx[4], kx[5], kx[6], kx[7],
                          kx[8], kx[9], kx[10], kx[11], kx[12], kx[13], kx[14], kx[15]};
    const float qc[16] = {qx[0], qx[1], qx[2], qx[3], qx[4], qx[5], qx[6], qx[7],
                          qx[8], qx[9], qx[10], qx[11], qx[12], qx[13], qx[14], qx[15]};
    const float vc[4] = {vx[0], vx[1], vx[2], vx[3]};
    // the next token's operands (zeros past the end)
    load16<kF32In>(row(kb, qk_row, i + 1), d4, kx);
    load16<kF32In>(row(qb, qk_row, i + 1), d4, qx);
    load4<kF32In>(row(vb, v_row, i + 1), v0 * kEl, vx);
    gx = gate(g, i + 1);
    bx = gate(beta, i + 1);

    const float e = fast_exp2(gt * kLog2e);
    // S^T k on the state before this token (the decay is applied to the sum)
    float dk[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float a = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int c = 0; c < 4; ++c) a = fmaf(St[r][j][c], kc[4 * j + c], a);
      dk[r] = sum8(a);
    }
    // S = e^g S + k (beta (v - e^g S^T k))^T, then S^T q
    float dq[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float dlt = bt * (vc[r] - e * dk[r]);
      float a = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          St[r][j][c] = fmaf(kc[4 * j + c], dlt, e * St[r][j][c]);
          a = fmaf(St[r][j][c], qc[4 * j + c], a);
        }
      dq[r] = sum8(a);
    }
    if ((tid & 7) == 0)
      *reinterpret_cast<f32x4 *>(o + ((int64_t)t * Hv + hv) * kD + v0) =
          f32x4{scale * dq[0], scale * dq[1], scale * dq[2], scale * dq[3]};
  }
  if (hT) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        __builtin_nontemporal_store(St[i][j],
                                    reinterpret_cast<f32x4 *>(hT + sb + (v0 + i) * kD + 32 * j + d4));
  }
}

}  // namespace

hipError_t launch_recurrent(bool f32_in, const void *q, const void *k, const void *v,
                            const float *g, const float *beta, const float *h0,
                            const int32_t *cu_seqlens, int32_t n_max, int32_t t_max, int32_t h,
                            int32_t hv, float scale, float *o, float *hT, hipStream_t stream,
                            KernelEvents ev) {
  const int64_t blocks = static_cast<int64_t>(n_max) * hv;
  if (blocks <= 0) return hipSuccess;
  dim3 grid;
  if (!flat_grid(blocks, kRecThreads, grid)) return hipErrorInvalidValue;
  if (f32_in)
    hipExtLaunchKernelGGL((recurrent_kernel<true>), grid, dim3(kRecThreads), 0, stream, ev.start,
                          ev.stop, 0, q, k, v, g, beta, h0, cu_seqlens, o, hT, n_max, h, hv, t_max, scale);
  else
    hipExtLaunchKernelGGL((recurrent_kernel<false>), grid, dim3(kRecThreads), 0, stream, ev.start,
                          ev.stop, 0, q, k, v, g, beta, h0, cu_seqlens, o, hT, n_max, h, hv, t_max, scale);
  return hipGetLastError();
}

}  // namespace gdn
