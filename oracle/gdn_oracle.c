/*
 * fp64 CPU oracle for the gated delta rule (GDN) prefill forward.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path links, loads or calls
 * this file; only the tests, the smoke check and the benchmark's CPU-baseline
 * leg do. It shares no code, header or constant with the HIP library.
 *
 * What it computes, token by token, in double precision:
 *
 *   "Chunking Qwen3.5's gated DeltaNet ... on Apple Silicon", section
 *   "What is the gated delta rule in Qwen3.5?": each head keeps a state S with
 *   one row per key dimension and one column per value dimension (128 x 128,
 *   fp32 in the model). Per token the layer (1) decays the state, (2) forms a
 *   correction from what the decayed state predicts for the token's key,
 *   (3) writes the correction back, and (4) reads the output from the updated
 *   state. The equation itself did not survive the page extraction; the four
 *   steps are written out here in the order the prose gives them:
 *
 *     S  <- exp(g_t) * S                       decay
 *     d  <- beta_t * (v_t - S^T k_t)           correction from the prediction
 *     S  <- S + k_t d^T                        write back
 *     o_t = scale * S^T q_t                    read after the write
 *
 *   The decay-before-correction order is the one the chunked formulas of
 *   "Optimizing GDN Chunk Prefill on Intel AMX CPU", section 4, imply (their
 *   w carries exp(g), the cumulative decay up to and including the token).
 *
 * Layouts (all row-major, packed varlen batch with B = 1 as in section 9 of the
 * AMX page):
 *   q, k   [T, H,  Dk]      v, o  [T, Hv, Dv]      g, beta [T, Hv]
 *   h0, hT [N, Hv, Dv, Dk]  (value-major "VK" state, AMX page section 9)
 *   cu_seqlens [N + 1], int32, non-decreasing, cu[0] = 0.
 * Value head hv reads key head hv / (Hv / H) (AMX page section 4, GQA groups).
 *
 * The conv + SiLU + L2-norm front follows the llama.cpp PR 399 page, section
 * "How (exactness)" (conv sum over d_conv taps with the current token last, no
 * bias) and the AMX page, section 7 (1 / sqrt(sum of squares + eps)).
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Number of OpenMP threads the oracle's parallel loops use. */
int gdn_oracle_threads(void) { return omp_get_max_threads(); }

/* Sets the number of OpenMP threads of later calls (n >= 1). */
void gdn_oracle_set_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }

/* Token recurrence over every (sequence, value head) lane. h0 may be NULL
 * (zero initial state); hT may be NULL. Lanes are independent, so they run in
 * parallel under OpenMP; each lane's arithmetic order is fixed. */
void gdn_oracle_recurrent(const double *q, const double *k, const double *v,
                          const double *g, const double *beta,
                          const double *h0, const int32_t *cu_seqlens,
                          int32_t n_seqs, int32_t H, int32_t Hv, int32_t Dk,
                          int32_t Dv, double scale, double *o, double *hT) {
  const int32_t HG = Hv / H;
  const int64_t lanes = (int64_t)n_seqs * Hv;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t lane = 0; lane < lanes; ++lane) {
    const int32_t s = (int32_t)(lane / Hv);
    const int32_t hv = (int32_t)(lane % Hv);
    const int32_t h = hv / HG;
    double *S = (double *)calloc((size_t)Dk * Dv, sizeof(double)); /* [Dk][Dv] */
    double *d = (double *)malloc((size_t)Dv * sizeof(double));
    if (h0) {
      const double *src = h0 + ((int64_t)s * Hv + hv) * Dv * Dk;
      for (int32_t j = 0; j < Dv; ++j)
        for (int32_t i = 0; i < Dk; ++i) S[(int64_t)i * Dv + j] = src[(int64_t)j * Dk + i];
    }
    for (int32_t t = cu_seqlens[s]; t < cu_seqlens[s + 1]; ++t) {
      const double *kt = k + ((int64_t)t * H + h) * Dk;
      const double *qt = q + ((int64_t)t * H + h) * Dk;
      const double *vt = v + ((int64_t)t * Hv + hv) * Dv;
      const double a = exp(g[(int64_t)t * Hv + hv]);
      const double b = beta[(int64_t)t * Hv + hv];
      for (int64_t e = 0; e < (int64_t)Dk * Dv; ++e) S[e] *= a;
      for (int32_t j = 0; j < Dv; ++j) d[j] = 0.0;
      for (int32_t i = 0; i < Dk; ++i)
        for (int32_t j = 0; j < Dv; ++j) d[j] += S[(int64_t)i * Dv + j] * kt[i];
      for (int32_t j = 0; j < Dv; ++j) d[j] = b * (vt[j] - d[j]);
      for (int32_t i = 0; i < Dk; ++i)
        for (int32_t j = 0; j < Dv; ++j) S[(int64_t)i * Dv + j] += kt[i] * d[j];
      double *ot = o + ((int64_t)t * Hv + hv) * Dv;
      for (int32_t j = 0; j < Dv; ++j) ot[j] = 0.0;
      for (int32_t i = 0; i < Dk; ++i)
        for (int32_t j = 0; j < Dv; ++j) ot[j] += S[(int64_t)i * Dv + j] * qt[i];
      for (int32_t j = 0; j < Dv; ++j) ot[j] *= scale;
    }
    if (hT) {
      double *dst = hT + ((int64_t)s * Hv + hv) * Dv * Dk;
      for (int32_t j = 0; j < Dv; ++j)
        for (int32_t i = 0; i < Dk; ++i) dst[(int64_t)j * Dk + i] = S[(int64_t)i * Dv + j];
    }
    free(d);
    free(S);
  }
}

/* Causal depthwise conv (d_conv taps, tap d_conv-1 is the current token, zero
 * history at each sequence start, no bias), then SiLU on every channel, then
 * the L2 norm of each q and k head. Channel order of x and of the output
 * buffers: q (H*Dk) | k (H*Dk) | v (Hv*Dv), head-major within each part.
 *   x [T, C]  conv_w [C, d_conv]  ->  y [T, C] (q/k heads normalised). */
void gdn_oracle_front(const double *x, const double *conv_w, int32_t d_conv,
                      const int32_t *cu_seqlens, int32_t n_seqs, int32_t H,
                      int32_t Hv, int32_t Dk, int32_t Dv, double eps, double *y) {
  const int64_t C = (int64_t)2 * H * Dk + (int64_t)Hv * Dv;
  const int64_t T = cu_seqlens[n_seqs];
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    int32_t s = 0;
    while (cu_seqlens[s + 1] <= t) ++s;
    const int64_t bos = cu_seqlens[s];
    for (int64_t c = 0; c < C; ++c) {
      double acc = 0.0;
      for (int32_t j = 0; j < d_conv; ++j) {
        const int64_t src = t - (d_conv - 1) + j;
        if (src >= bos) acc += x[src * C + c] * conv_w[c * d_conv + j];
      }
      y[t * C + c] = acc / (1.0 + exp(-acc));
    }
    for (int32_t head = 0; head < 2 * H; ++head) {
      double *row = y + t * C + (int64_t)head * Dk;
      double ss = 0.0;
      for (int32_t i = 0; i < Dk; ++i) ss += row[i] * row[i];
      const double r = 1.0 / sqrt(ss + eps);
      for (int32_t i = 0; i < Dk; ++i) row[i] *= r;
    }
  }
}
