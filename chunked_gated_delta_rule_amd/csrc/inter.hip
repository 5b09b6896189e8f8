// Stage 2 of the chunked forward: the inter-chunk kernel.
//
// "Optimizing GDN Chunk Prefill on Intel AMX CPU", section 5: per sequence and
// value head the chunks are walked in order with the fp32 state updated in
// place; per chunk (gamma the chunk-local cumulative g, Gamma its masked decay
// matrix, S the Dk x Dv state):
//
//   v'  = u - w S
//   o   = scale * ( diag(e^gamma) q S + tril(q k^T * Gamma) v' )   (diagonal kept)
//   S   = e^{gamma_last} S + (diag(e^{gamma_last - gamma}) k)^T v'
//
// The value columns of S are independent, so the state is blocked over Dv
// (Alloy page, "How do you parallelize a recurrence for prefill?": the state
// tile is blocked along the value dimension to fit on chip). One 256-thread
// work-group owns a 128 x 16 column block of S for one (sequence, value head)
// for the whole sequence:
//   * S lives in MFMA accumulators (fp32, 8 floats per lane) and, for use as
//     an MFMA operand, as a hi/lo bf16 pair in LDS;
//   * every product runs on v_mfma_f32_16x16x32_bf16; the fp32 operands S, P,
//     v' and the decayed v' enter as hi + lo bf16 pairs (two or three terms);
//   * the next chunk's q, k, w, u, g are loaded into registers while the
//     current chunk computes, then written to LDS (k both row-major and
//     transposed, since k is contracted over Dk in q k^T and over tokens in
//     the state update).
// Work-group numbering is XCD-aware: all value-column blocks of all value
// heads that share a key head (16 work-groups at Hv = 2 H) get the same
// blockIdx modulo 8, so they run on one XCD and their shared q, k, w reads
// hit that XCD's L2.
#include "gdn_common.hpp"
#include "gdn_launch.hpp"

namespace gdn {

namespace {

constexpr int kBV = 16;               // value columns per work-group
constexpr int kNVT = kD / kBV;        // value-column blocks per head
constexpr int kLdRow = kD + 8;        // [64][136] bf16 row-major tiles
constexpr int kLdCol = kC + 8;        // [128][72] bf16 transposed k; [64][72] P
constexpr int kLdS = kD + 8;          // S^T hi/lo [16][136]
constexpr int kLdV = kC + 8;          // v'^T hi/lo [16][72]
constexpr int kXcds = 8;

template <bool kF32In>
struct InterSmem {
  static constexpr int kT = kF32In ? 2 : 1;
  static constexpr int kQ = kT * 64 * kLdRow * 2;
  static constexpr int kKr = kT * 64 * kLdRow * 2;
  static constexpr int kKc = kT * 128 * kLdCol * 2;
  static constexpr int kW = 64 * kLdRow * 2;
  static constexpr int kS = 2 * kBV * kLdS * 2;
  static constexpr int kP = 2 * 64 * kLdCol * 2;
  static constexpr int kDl = 2 * kBV * kLdV * 2;
  static constexpr int kBytes = kQ + kKr + kKc + kW + kS + kP + 2 * kDl + 64 * 4;
  static_assert(kBytes <= 160 * 1024, "LDS budget");
};

// One chunk's inputs as held in registers between the global load and the
// LDS store. A thread owns 4 rows x 8 columns of each 64 x 128 tile.
template <bool kF32In>
struct ChunkRegs {
  u32x4 qh[4], ql[4], kh[4], kl[4], w[4];
  float u[4];
  float g;
};

__device__ __forceinline__ uint16_t half_of(const u32x4 &w, int i) {
  return static_cast<uint16_t>((w[i >> 1] >> (16 * (i & 1))) & 0xffffu);
}

template <bool kF32In>
__device__ __forceinline__ void load_tile(const void *base, int64_t row_stride, int row0, int valid,
                                          int col, u32x4 (&hi)[4], u32x4 (&lo)[4]) {
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const int r = row0 + rr;
    hi[rr] = u32x4{0u, 0u, 0u, 0u};
    lo[rr] = u32x4{0u, 0u, 0u, 0u};
    if (r < valid) {
      if constexpr (kF32In) {
        const float *p = static_cast<const float *>(base) + (int64_t)r * row_stride + col;
        const f32x4 a = reinterpret_cast<const f32x4 *>(p)[0];
        const f32x4 b = reinterpret_cast<const f32x4 *>(p)[1];
        const float x[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          __bf16 h0, l0, h1, l1;
          split_bf16(x[2 * i], h0, l0);
          split_bf16(x[2 * i + 1], h1, l1);
          hi[rr][i] = pack2(h0, h1);
          lo[rr][i] = pack2(l0, l1);
        }
      } else {
        hi[rr] = *reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(base) +
                                                  (int64_t)r * row_stride + col);
      }
    }
  }
}

__device__ __forceinline__ void store_col4x8(__bf16 *dst, int row0, int col, const u32x4 (&v)[4]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t a = half_of(v[0], i) | (static_cast<uint32_t>(half_of(v[1], i)) << 16);
    const uint32_t b = half_of(v[2], i) | (static_cast<uint32_t>(half_of(v[3], i)) << 16);
    *reinterpret_cast<u32x2 *>(dst + (col + i) * kLdCol + row0) = u32x2{a, b};
  }
}

// Split four fp32 values (consecutive along the LDS row) into hi/lo bf16.
__device__ __forceinline__ void store_split4(__bf16 *hi, __bf16 *lo, const float (&x)[4]) {
  __bf16 h[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) split_bf16(x[i], h[i], l[i]);
  *reinterpret_cast<u32x2 *>(hi) = u32x2{pack2(h[0], h[1]), pack2(h[2], h[3])};
  *reinterpret_cast<u32x2 *>(lo) = u32x2{pack2(l[0], l[1]), pack2(l[2], l[3])};
}

template <bool kF32In>
__global__ __launch_bounds__(kThreads, 1) void inter_kernel(
    const void *__restrict__ qin, const void *__restrict__ kin, const __bf16 *__restrict__ win,
    const float *__restrict__ uin, const float *__restrict__ g, const float *__restrict__ h0,
    const int32_t *__restrict__ cu, float *__restrict__ o, float *__restrict__ hT, int n_max,
    int H, int Hv, int t_max, float scale) {
  using Smem = InterSmem<kF32In>;
  __shared__ __attribute__((aligned(16))) unsigned char smem[Smem::kBytes];
  unsigned char *p = smem;
  __bf16 *qrow = reinterpret_cast<__bf16 *>(p); p += Smem::kQ;
  __bf16 *krow = reinterpret_cast<__bf16 *>(p); p += Smem::kKr;
  __bf16 *kcol = reinterpret_cast<__bf16 *>(p); p += Smem::kKc;
  __bf16 *wrow = reinterpret_cast<__bf16 *>(p); p += Smem::kW;
  __bf16 *s_hi = reinterpret_cast<__bf16 *>(p);
  __bf16 *s_lo = s_hi + kBV * kLdS; p += Smem::kS;
  __bf16 *p_hi = reinterpret_cast<__bf16 *>(p);
  __bf16 *p_lo = p_hi + 64 * kLdCol; p += Smem::kP;
  __bf16 *dl_hi = reinterpret_cast<__bf16 *>(p);
  __bf16 *dl_lo = dl_hi + kBV * kLdV; p += Smem::kDl;
  __bf16 *dp_hi = reinterpret_cast<__bf16 *>(p);
  __bf16 *dp_lo = dp_hi + kBV * kLdV; p += Smem::kDl;
  float *gam = reinterpret_cast<float *>(p);

  // ---- XCD-aware work-group -> (sequence, value head, column block) -------
  const int HG = Hv / H;
  const int members = HG * kNVT;
  const int xcd = blockIdx.x % kXcds;
  const int slot = blockIdx.x / kXcds;
  const int group = (slot / members) * kXcds + xcd;  // (sequence, key head)
  const int member = slot % members;
  if (group >= n_max * H) return;
  const int s = group / H;
  const int h = group % H;
  const int hv = h * HG + member / kNVT;
  const int vt = member % kNVT;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int lrow = 4 * (tid >> 4);
  const int lcol = 8 * (tid & 15);
  const int vcol = kBV * vt + (lane & 15);  // this lane's value column in C layouts
  const int quad = 4 * (lane >> 4);

  const int bos = cu[s];
  const int eos = cu[s + 1];
  const int nchunks = (eos - bos + kC - 1) / kC;
  const size_t elt = kF32In ? 4 : 2;

  // ---- initial state: S[d][v] for d = 32 wv + 16 b + quad + i ---------------
  f32x4 sacc[2];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int d = 32 * wv + 16 * b + quad;
    sacc[b] = h0 ? *reinterpret_cast<const f32x4 *>(h0 + (((int64_t)s * Hv + hv) * kD + vcol) * kD + d)
                 : zero4();
  }
  if (nchunks == 0) {
    if (hT) {
#pragma unroll
      for (int b = 0; b < 2; ++b)
        *reinterpret_cast<f32x4 *>(hT + (((int64_t)s * Hv + hv) * kD + vcol) * kD + 32 * wv + 16 * b + quad) = sacc[b];
    }
    return;
  }
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const float x[4] = {sacc[b][0], sacc[b][1], sacc[b][2], sacc[b][3]};
    const int d = 32 * wv + 16 * b + quad;
    store_split4(s_hi + (lane & 15) * kLdS + d, s_lo + (lane & 15) * kLdS + d, x);
  }

  ChunkRegs<kF32In> nx;
  auto fetch = [&](int c) {
    const int t0 = bos + c * kC;
    const int L = min(kC, eos - t0);
    load_tile<kF32In>(static_cast<const char *>(qin) + ((int64_t)t0 * H + h) * kD * elt,
                      (int64_t)H * kD, lrow, L, lcol, nx.qh, nx.ql);
    load_tile<kF32In>(static_cast<const char *>(kin) + ((int64_t)t0 * H + h) * kD * elt,
                      (int64_t)H * kD, lrow, L, lcol, nx.kh, nx.kl);
    u32x4 dummy[4];
    load_tile<false>(win + ((int64_t)hv * t_max + t0) * kD, kD, lrow, L, lcol, nx.w, dummy);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * wv + quad + i;
      nx.u[i] = r < L ? uin[((int64_t)hv * t_max + t0 + r) * kD + vcol] : 0.f;
    }
    nx.g = (wv == 0 && lane < L) ? g[(int64_t)(t0 + lane) * Hv + hv] : 0.f;
  };
  fetch(0);

  for (int c = 0; c < nchunks; ++c) {
    const int t0 = bos + c * kC;
    const int L = min(kC, eos - t0);
    // ---- stage the prefetched chunk into LDS -------------------------------
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      *reinterpret_cast<u32x4 *>(qrow + (lrow + rr) * kLdRow + lcol) = nx.qh[rr];
      *reinterpret_cast<u32x4 *>(krow + (lrow + rr) * kLdRow + lcol) = nx.kh[rr];
      *reinterpret_cast<u32x4 *>(wrow + (lrow + rr) * kLdRow + lcol) = nx.w[rr];
      if constexpr (kF32In) {
        *reinterpret_cast<u32x4 *>(qrow + 64 * kLdRow + (lrow + rr) * kLdRow + lcol) = nx.ql[rr];
        *reinterpret_cast<u32x4 *>(krow + 64 * kLdRow + (lrow + rr) * kLdRow + lcol) = nx.kl[rr];
      }
    }
    store_col4x8(kcol, lrow, lcol, nx.kh);
    if constexpr (kF32In) store_col4x8(kcol + 128 * kLdCol, lrow, lcol, nx.kl);
    if (wv == 0) gam[lane] = wave_inclusive_scan(nx.g, lane);
    float ucur[4] = {nx.u[0], nx.u[1], nx.u[2], nx.u[3]};
    if (c + 1 < nchunks) fetch(c + 1);
    __syncthreads();

    // ---- X = w S and Y = q S for rows 16 wv .. 16 wv + 15 ---------------------
    f32x4 X = zero4(), Y = zero4();
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8 sh = frag_rows(s_hi, kLdS, 0, 32 * ks, lane);
      const bf16x8 sl = frag_rows(s_lo, kLdS, 0, 32 * ks, lane);
      const bf16x8 aw = frag_rows(wrow, kLdRow, 16 * wv, 32 * ks, lane);
      const bf16x8 aq = frag_rows(qrow, kLdRow, 16 * wv, 32 * ks, lane);
      X = mfma(aw, sh, X);
      X = mfma(aw, sl, X);
      Y = mfma(aq, sh, Y);
      Y = mfma(aq, sl, Y);
      if constexpr (kF32In) Y = mfma(frag_rows(qrow + 64 * kLdRow, kLdRow, 16 * wv, 32 * ks, lane), sh, Y);
    }
    // ---- v' and decayed v' (rows r = 16 wv + quad + i, column lane & 15) ------
    const float glast = gam[63];
    {
      float dl[4], dp[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * wv + quad + i;
        dl[i] = ucur[i] - X[i];
        dp[i] = dl[i] * expf(glast - gam[r]);
      }
      const int at = (lane & 15) * kLdV + 16 * wv + quad;
      store_split4(dl_hi + at, dl_lo + at, dl);
      store_split4(dp_hi + at, dp_lo + at, dp);
    }
    // ---- P = tril(q k^T * Gamma) for row block wv, computed as P^T blocks ------
    // P^T block (jb, wv): lane holds P[t = 16 wv + (lane & 15)][j = 16 jb + quad + i]
    for (int jb = 0; jb < 4; ++jb) {
      const int t = 16 * wv + (lane & 15);
      const int j0 = 16 * jb + quad;
      float pv[4] = {0.f, 0.f, 0.f, 0.f};
      if (jb <= wv) {
        f32x4 acc = zero4();
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const bf16x8 ak = frag_rows(krow, kLdRow, 16 * jb, 32 * ks, lane);
          const bf16x8 bq = frag_rows(qrow, kLdRow, 16 * wv, 32 * ks, lane);
          acc = mfma(ak, bq, acc);
          if constexpr (kF32In) {
            acc = mfma(frag_rows(krow + 64 * kLdRow, kLdRow, 16 * jb, 32 * ks, lane), bq, acc);
            acc = mfma(ak, frag_rows(qrow + 64 * kLdRow, kLdRow, 16 * wv, 32 * ks, lane), acc);
          }
        }
        const float gt = gam[t];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = j0 + i;
          pv[i] = j <= t ? acc[i] * expf(gt - gam[j]) : 0.f;
        }
      }
      if (jb <= wv || jb == (wv | 1)) store_split4(p_hi + t * kLdCol + j0, p_lo + t * kLdCol + j0, pv);
    }
    __syncthreads();

    // ---- o rows 16 wv .. : scale (e^gamma Y + P v') ----------------------------
    {
      f32x4 oacc = zero4();
      const int nks = (wv >> 1) + 1;
      for (int ks = 0; ks < nks; ++ks) {
        const bf16x8 ph = frag_rows(p_hi, kLdCol, 16 * wv, 32 * ks, lane);
        const bf16x8 pl = frag_rows(p_lo, kLdCol, 16 * wv, 32 * ks, lane);
        const bf16x8 dh = frag_rows(dl_hi, kLdV, 0, 32 * ks, lane);
        const bf16x8 dlo = frag_rows(dl_lo, kLdV, 0, 32 * ks, lane);
        oacc = mfma(ph, dh, oacc);
        oacc = mfma(ph, dlo, oacc);
        oacc = mfma(pl, dh, oacc);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * wv + quad + i;
        if (r < L) {
          const float val = scale * (expf(gam[r]) * Y[i] + oacc[i]);
          o[((int64_t)(t0 + r) * Hv + hv) * kD + vcol] = val;
        }
      }
    }
    // ---- S = e^{gamma_last} S + k^T v'_decayed ----------------------------------
    {
      const float decay = expf(glast);
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        f32x4 acc = sacc[b] * decay;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const bf16x8 ak = frag_rows(kcol, kLdCol, 32 * wv + 16 * b, 32 * ks, lane);
          const bf16x8 dh = frag_rows(dp_hi, kLdV, 0, 32 * ks, lane);
          const bf16x8 dlo = frag_rows(dp_lo, kLdV, 0, 32 * ks, lane);
          acc = mfma(ak, dh, acc);
          acc = mfma(ak, dlo, acc);
          if constexpr (kF32In)
            acc = mfma(frag_rows(kcol + 128 * kLdCol, kLdCol, 32 * wv + 16 * b, 32 * ks, lane), dh, acc);
        }
        sacc[b] = acc;
      }
    }
    __syncthreads();
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const float x[4] = {sacc[b][0], sacc[b][1], sacc[b][2], sacc[b][3]};
      const int d = 32 * wv + 16 * b + quad;
      store_split4(s_hi + (lane & 15) * kLdS + d, s_lo + (lane & 15) * kLdS + d, x);
    }
  }
  if (hT) {
#pragma unroll
    for (int b = 0; b < 2; ++b)
      *reinterpret_cast<f32x4 *>(hT + (((int64_t)s * Hv + hv) * kD + vcol) * kD + 32 * wv + 16 * b + quad) = sacc[b];
  }
}

}  // namespace

hipError_t launch_inter(bool f32_in, const void *q, const void *k, const void *w, const float *u,
                        const float *g, const float *h0, const int32_t *cu_seqlens,
                        int32_t n_max, int32_t h, int32_t hv, int32_t t_max, float scale,
                        float *o, float *hT, hipStream_t stream) {
  const int members = (hv / h) * kNVT;
  const int groups = n_max * h;
  const int rounds = (groups + kXcds - 1) / kXcds;
  const dim3 grid(rounds * kXcds * members);
  if (f32_in) {
    hipLaunchKernelGGL(inter_kernel<true>, grid, dim3(kThreads), 0, stream, q, k,
                       static_cast<const __bf16 *>(w), u, g, h0, cu_seqlens, o, hT, n_max, h,
                       hv, t_max, scale);
  } else {
    hipLaunchKernelGGL(inter_kernel<false>, grid, dim3(kThreads), 0, stream, q, k,
                       static_cast<const __bf16 *>(w), u, g, h0, cu_seqlens, o, hT, n_max, h,
                       hv, t_max, scale);
  }
  return hipGetLastError();
}

}  // namespace gdn
