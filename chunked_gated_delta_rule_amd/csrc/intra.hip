// Stage 1 of the chunked forward: the intra-chunk kernel over [chunks, key heads].
//
// "Optimizing GDN Chunk Prefill on Intel AMX CPU", section 4: for one chunk and
// one key head h, attn = K K^T is formed once; then for each value head of the
// GQA group the beta/decay-masked strictly lower matrix is solved and w, u are
// recomputed, without the solve ever leaving the chip. Written out (gamma is
// the chunk-local inclusive cumsum of g, section 3; Gamma[r, i] =
// exp(gamma_r - gamma_i) for i <= r):
//
//   A = strict_lower(diag(beta) (K K^T * Gamma)),   T = (I + A)^-1 (fp32)
//   w = T diag(beta e^gamma) K,    u = T diag(beta) V
//
// Everything the inter-chunk stage needs that does not depend on the state is
// produced here, where the work is parallel over chunks, and written in the
// exact MFMA fragment order the inter stage reads (each fragment one 1 KB
// block, 16 bytes per lane), so that stage only streams blocks:
//   w16   fp16 [hv, t, 128]     -w, d permuted inside each 32-column block
//   q16   fp16 [t, h, 128]      q rounded to fp16, same d permutation
//   kimg  bf16 per (h, chunk)   K^T fragments for the state update (hi[, lo])
//   uimg  fp32 per (hv, chunk)  u fragments, one 1 KB block per 16 x 16 tile
//   pimg  bf16 per (hv, chunk)  P = scale * tril(q k^T * Gamma) as hi + lo
//   gimg  fp32 per (hv, chunk)  e^{gamma_last - gamma}, scale e^gamma, e^{gamma_last}
// P is the intra-chunk attention term of the output (AMX page, section 5); it
// shares the masked decay factors with A. Per-chunk blocks are addressed by
// the slot floor(t0 / 64) + n of chunk start t0 in sequence n, which is
// distinct for every chunk of a batch and below cdiv(t_max, 64) + n_max - 1.
//
// The exponent is always a masked difference gamma_r - gamma_i <= 0, never
// e^gamma_r * e^-gamma_i, which would overflow under strong decay. Only lower
// 16x16 blocks are computed (AMX page, section 8: triangular work stays
// triangular).
//
// gfx950 mapping: one 256-thread work-group per (chunk, h), four wave64s.
//  * K K^T and K q^T on v_mfma_f32_16x16x32_bf16 (lower 16x16 blocks, kept in
//    registers across the value heads). fp32 inputs are split x = hi + lo into
//    two bf16 terms and the products take three MFMA terms.
//  * The solve runs in fp32 in LDS: the four diagonal 16x16 blocks by column
//    forward substitution, then the off-diagonal blocks in three wavefront
//    steps T_ij = -T_ii (sum_k A_ik T_kj).
//  * w and u are MFMA products of the transposed K (V) tile with the scaled
//    T; the scaled T is split into hi + lo bf16 so w/u carry ~16 bits of T.
//  * A tile of K (V) is read once from HBM and written to LDS both row-major
//    (for K K^T) and transposed (for the products that contract over tokens).
// Rows of a partial last chunk are zero-filled, so they add nothing; w and q16
// are written for valid rows only, the per-chunk blocks in full (zeros past
// the end).
#include "gdn_common.hpp"
#include "gdn_launch.hpp"

namespace gdn {

namespace {

constexpr int kLdRow = kD + 8;   // bf16 row-major tile [64][136]
constexpr int kLdCol = kC + 8;   // bf16 transposed tile [128][72]
constexpr int kLdA = kC + 8;     // fp32 A [64][72] (also hosts the split T)
constexpr int kLdT = kC + 4;     // fp32 T [64][68]
constexpr int kLdX = 16 + 4;     // fp32 per-wave 16x16 scratch

template <bool kF32In>
struct IntraSmem {
  static constexpr int kTerms = kF32In ? 2 : 1;
  // region 1: K row-major (hi[, lo]) while K K^T runs, then V transposed (hi[, lo])
  static constexpr int kR1 = kTerms * 128 * kLdCol * 2;
  // region 2: K transposed (hi[, lo])
  static constexpr int kR2 = kTerms * 128 * kLdCol * 2;
  // region 3: A (fp32) during the solve, then T-scaled hi/lo (bf16)
  static constexpr int kR3 = 64 * kLdA * 4;
  static constexpr int kR4 = 64 * kLdT * 4;
  static constexpr int kR5 = 4 * 16 * kLdX * 4;
  static constexpr int kBytes = kR1 + kR2 + kR3 + kR4 + kR5 + 3 * 64 * 4;
  static_assert(kTerms * 64 * kLdRow * 2 <= kR1, "row tile must fit region 1");
};

// Load 4 rows x 8 columns of a [rows, heads, 128] tile starting at token row
// `row0` (rows >= valid are zero) as bf16 hi (and lo for fp32 input).
template <bool kF32In>
__device__ __forceinline__ void load_rows4x8(const void *base, int64_t row_stride, int row0,
                                             int valid, int col, u32x4 (&hi)[4], u32x4 (&lo)[4]) {
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const int r = row0 + rr;
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
        const uint16_t *p = static_cast<const uint16_t *>(base) + (int64_t)r * row_stride + col;
        hi[rr] = *reinterpret_cast<const u32x4 *>(p);
        lo[rr] = u32x4{0u, 0u, 0u, 0u};
      }
    } else {
      hi[rr] = u32x4{0u, 0u, 0u, 0u};
      lo[rr] = u32x4{0u, 0u, 0u, 0u};
    }
  }
}

__device__ __forceinline__ uint16_t half_of(const u32x4 &w, int i) {
  return static_cast<uint16_t>((w[i >> 1] >> (16 * (i & 1))) & 0xffffu);
}

// Write a thread's 4x8 block transposed: dst[col + i][row0 .. row0 + 3].
__device__ __forceinline__ void store_col4x8(__bf16 *dst, int row0, int col, const u32x4 (&v)[4]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t a = half_of(v[0], i) | (static_cast<uint32_t>(half_of(v[1], i)) << 16);
    const uint32_t b = half_of(v[2], i) | (static_cast<uint32_t>(half_of(v[3], i)) << 16);
    *reinterpret_cast<u32x2 *>(dst + (col + i) * kLdCol + row0) = u32x2{a, b};
  }
}

// P pairs (q, R): token block q (32 tokens) of column tile R (16 outputs);
// each pair is two 16x16 tiles of P^T, (2q, R) and (2q + 1, R).
__device__ __forceinline__ int pair_q(int pi) { return pi == 3 || pi == 5 ? 1 : 0; }
__device__ __forceinline__ int pair_r(int pi) { return pi < 2 ? pi : 2 + ((pi - 2) >> 1); }

template <bool kF32In>
__global__ __launch_bounds__(kThreads, kF32In ? 1 : 2) void intra_kernel(
    const void *__restrict__ qin, const void *__restrict__ kin, const void *__restrict__ vin,
    const float *__restrict__ g, const float *__restrict__ beta, const int32_t *__restrict__ cu,
    const int32_t *__restrict__ table, StageBuffers out, int H, int Hv, int t_max, int nt,
    float scale) {
  using Smem = IntraSmem<kF32In>;
  __shared__ __attribute__((aligned(16))) unsigned char smem[Smem::kBytes];
  __bf16 *r1 = reinterpret_cast<__bf16 *>(smem);
  __bf16 *kcol = reinterpret_cast<__bf16 *>(smem + Smem::kR1);
  float *amat = reinterpret_cast<float *>(smem + Smem::kR1 + Smem::kR2);
  __bf16 *ts_hi = reinterpret_cast<__bf16 *>(amat);
  __bf16 *ts_lo = ts_hi + 64 * kLdCol;
  __bf16 *rq = ts_hi;  // q row-major (hi[, lo]) while the products with K run: regions 3-4
  float *tmat = reinterpret_cast<float *>(smem + Smem::kR1 + Smem::kR2 + Smem::kR3);
  float *xs = reinterpret_cast<float *>(smem + Smem::kR1 + Smem::kR2 + Smem::kR3 + Smem::kR4);
  float *gam = xs + 4 * 16 * kLdX;
  float *bet = gam + 64;
  float *scl = bet + 64;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int2 ent = reinterpret_cast<const int2 *>(table)[blockIdx.x];
  if (ent.x < 0) return;  // sentinel slot
  const int h = blockIdx.y;
  const int HG = Hv / H;
  const int bos = cu[ent.x];
  const int t0 = bos + ent.y * kC;
  const int L = min(kC, cu[ent.x + 1] - t0);
  const int slot = (t0 >> 6) + ent.x;
  constexpr int kNK = kF32In ? 32 : 16;

  // ---- K tile -> LDS (row-major in region 1, transposed in region 2) ------
  const int lrow = 4 * (tid >> 4);  // this thread's 4 rows and 8 columns
  const int lcol = 8 * (tid & 15);
  {
    u32x4 khi[4], klo[4];
    load_rows4x8<kF32In>(static_cast<const char *>(kin) +
                             ((int64_t)t0 * H + h) * kD * (kF32In ? 4 : 2),
                         (int64_t)H * kD, lrow, L, lcol, khi, klo);
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      *reinterpret_cast<u32x4 *>(r1 + (lrow + rr) * kLdRow + lcol) = khi[rr];
      if constexpr (kF32In)
        *reinterpret_cast<u32x4 *>(r1 + 64 * kLdRow + (lrow + rr) * kLdRow + lcol) = klo[rr];
    }
    store_col4x8(kcol, lrow, lcol, khi);
    if constexpr (kF32In) store_col4x8(kcol + 128 * kLdCol, lrow, lcol, klo);
  }
  // ---- q tile -> LDS row-major, and the fp16 copy q16 ---------------------
  {
    u32x4 qhi[4], qlo[4];
    load_rows4x8<kF32In>(static_cast<const char *>(qin) +
                             ((int64_t)t0 * H + h) * kD * (kF32In ? 4 : 2),
                         (int64_t)H * kD, lrow, L, lcol, qhi, qlo);
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      *reinterpret_cast<u32x4 *>(rq + (lrow + rr) * kLdRow + lcol) = qhi[rr];
      if constexpr (kF32In)
        *reinterpret_cast<u32x4 *>(rq + 64 * kLdRow + (lrow + rr) * kLdRow + lcol) = qlo[rr];
      if (lrow + rr < L) {
        float f[8], fl[8];
        unpack8(qhi[rr], f);
        unpack8(qlo[rr], fl);
        uint32_t hh[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) hh[i] = pack_f16(f[2 * i] + fl[2 * i], f[2 * i + 1] + fl[2 * i + 1]);
        _Float16 *dst = out.q16 + ((int64_t)(t0 + lrow + rr) * H + h) * kD + 32 * (lcol >> 5);
        const int m = (lcol & 31) >> 2;  // first group of four columns
        *reinterpret_cast<u32x2 *>(dst + perm4(m)) = u32x2{hh[0], hh[1]};
        *reinterpret_cast<u32x2 *>(dst + perm4(m + 1)) = u32x2{hh[2], hh[3]};
      }
    }
  }
  __syncthreads();

  // ---- K^T fragments for the state update: fragment (tau, q), lane (g, c)
  // holds K[32 q + 4 g + j][16 tau + c] for j < 4 and K[32 q + 16 + 4 g + j - 4][..]
  // for j >= 4 (the token order of the inter stage's delta fragments).
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int item = tid + kThreads * m;
    const int f = item >> 6, l = item & 63;
    const int tau = f >> 1, qq = f & 1;
    const int off = (16 * tau + (l & 15)) * kLdCol + 32 * qq + 4 * (l >> 4);
    __bf16 *dst = out.kimg + ((((int64_t)h * nt + slot) * kNK + f) * 64 + l) * 8;
    const u32x2 a = *reinterpret_cast<const u32x2 *>(kcol + off);
    const u32x2 b = *reinterpret_cast<const u32x2 *>(kcol + off + 16);
    *reinterpret_cast<u32x4 *>(dst) = u32x4{a[0], a[1], b[0], b[1]};
    if constexpr (kF32In) {
      const u32x2 al = *reinterpret_cast<const u32x2 *>(kcol + 128 * kLdCol + off);
      const u32x2 bl = *reinterpret_cast<const u32x2 *>(kcol + 128 * kLdCol + off + 16);
      *reinterpret_cast<u32x4 *>(dst + 16 * 64 * 8) = u32x4{al[0], al[1], bl[0], bl[1]};
    }
  }

  // ---- G = K K^T, lower 16x16 blocks, kept in registers ---------------------
  // block b = 0..9 in the order (0,0)(1,0)(1,1)(2,0)(2,1)(2,2)(3,0)(3,1)(3,2)(3,3);
  // wave wv owns blocks b = wv, wv + 4, wv + 8.
  f32x4 gacc[3];
  int gbi[3], gbj[3];
  const int nblk = wv < 2 ? 3 : 2;
#pragma unroll
  for (int n = 0; n < 3; ++n) {
    const int b = wv + 4 * n;
    const int bi = b < 1 ? 0 : b < 3 ? 1 : b < 6 ? 2 : 3;
    const int bj = b - (bi * (bi + 1)) / 2;
    gbi[n] = bi;
    gbj[n] = bj;
    f32x4 acc = zero4();
    if (n < nblk) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 a = frag_rows(r1, kLdRow, 16 * bi, 32 * ks, lane);
        const bf16x8 bb = frag_rows(r1, kLdRow, 16 * bj, 32 * ks, lane);
        acc = mfma(a, bb, acc);
        if constexpr (kF32In) {
          const __bf16 *rlo = r1 + 64 * kLdRow;
          acc = mfma(frag_rows(rlo, kLdRow, 16 * bi, 32 * ks, lane), bb, acc);
          acc = mfma(a, frag_rows(rlo, kLdRow, 16 * bj, 32 * ks, lane), acc);
        }
      }
    }
    gacc[n] = acc;
  }

  // ---- P^T tiles = K q^T for this wave's pairs (unmasked, unscaled) ---------
  // waves 0 and 1 own pairs {0, 1} and {2, 3}; waves 2 and 3 own pair 4 and 5.
  const int npair = wv < 2 ? 2 : 1;
  const int pair0 = wv < 2 ? 2 * wv : wv + 2;
  f32x4 pacc[4];
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const int pi = pair0 + (n >> 1);
    const int tj = 2 * pair_q(pi) + (n & 1), tr = pair_r(pi);
    f32x4 acc = zero4();
    if ((n >> 1) < npair && tj <= tr) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 a = frag_rows(r1, kLdRow, 16 * tj, 32 * ks, lane);
        const bf16x8 bb = frag_rows(rq, kLdRow, 16 * tr, 32 * ks, lane);
        acc = mfma(a, bb, acc);
        if constexpr (kF32In) {
          acc = mfma(frag_rows(r1 + 64 * kLdRow, kLdRow, 16 * tj, 32 * ks, lane), bb, acc);
          acc = mfma(a, frag_rows(rq + 64 * kLdRow, kLdRow, 16 * tr, 32 * ks, lane), acc);
        }
      }
    }
    pacc[n] = acc;
  }
  __syncthreads();  // regions 1, 3 and 4 are free from here on

  for (int gi = 0; gi < HG; ++gi) {
    const int hv = h * HG + gi;
    // V tile prefetch (stored after A is formed)
    u32x4 vhi[4], vlo[4];
    load_rows4x8<kF32In>(static_cast<const char *>(vin) +
                             ((int64_t)t0 * Hv + hv) * kD * (kF32In ? 4 : 2),
                         (int64_t)Hv * kD, lrow, L, lcol, vhi, vlo);
    if (wv == 0) {
      const bool ok = lane < L;
      const float gv = ok ? g[(int64_t)(t0 + lane) * Hv + hv] : 0.f;
      const float bv = ok ? beta[(int64_t)(t0 + lane) * Hv + hv] : 0.f;
      const float gc = wave_inclusive_scan(gv, lane);
      gam[lane] = gc;
      bet[lane] = bv;
      const float gl = __shfl(gc, L - 1, 64);  // gamma of the last valid token
      float *gd = out.gimg + ((int64_t)hv * nt + slot) * kGateStride;
      gd[lane] = ok ? expf(gl - gc) : 0.f;
      gd[64 + lane] = ok ? scale * expf(gc) : 0.f;
      gd[128 + lane] = lane == 0 ? expf(gl) : 0.f;
    }
    __syncthreads();

    // ---- P = scale * tril(q k^T * Gamma), this wave's pairs, as hi + lo bf16
    // pair lane (g, c): tile (2q, R) rows 4 g + i then tile (2q + 1, R).
#pragma unroll
    for (int n2 = 0; n2 < 2; ++n2) {
      if (n2 < npair) {
        const int pi = pair0 + n2;
        const int r = 16 * pair_r(pi) + (lane & 15);
        float x[8];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int j = 32 * pair_q(pi) + 16 * hf + 4 * (lane >> 4) + i;
            x[4 * hf + i] = (j <= r && r < L) ? scale * pacc[2 * n2 + hf][i] * expf(gam[r] - gam[j]) : 0.f;
          }
        }
        u32x4 hi, lo;
        split8_words(x, hi, lo);
        __bf16 *dst = out.pimg + ((((int64_t)hv * nt + slot) * 6 + pi) * 2 * 64 + lane) * 8;
        *reinterpret_cast<u32x4 *>(dst) = hi;
        *reinterpret_cast<u32x4 *>(dst + 64 * 8) = lo;
      }
    }

    // ---- A = strict_lower(beta_r G e^{gamma_r - gamma_j}) -> LDS ----------
#pragma unroll
    for (int n = 0; n < 3; ++n) {
      if (n < nblk) {
        const int j = 16 * gbj[n] + (lane & 15);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * gbi[n] + 4 * (lane >> 4) + i;
          const float a = j < r ? bet[r] * gacc[n][i] * expf(gam[r] - gam[j]) : 0.f;
          amat[r * kLdA + j] = a;
        }
      }
    }
    store_col4x8(r1, lrow, lcol, vhi);
    if constexpr (kF32In) store_col4x8(r1 + 128 * kLdCol, lrow, lcol, vlo);
    __syncthreads();

    // ---- solve: diagonal blocks by column forward substitution ------------
    if (lane < 16) {
      const int c = lane;
      const float *ab = amat + (16 * wv) * kLdA + 16 * wv;
      float tc[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = 0.f;
#pragma unroll
        for (int i = 0; i < r; ++i) x = fmaf(ab[r * kLdA + i], tc[i], x);
        tc[r] = r == c ? 1.f : (r < c ? 0.f : -x);
        tmat[(16 * wv + r) * kLdT + 16 * wv + c] = tc[r];
      }
    } else if (lane < 32 && (wv == 0 || wv == 2)) {
      // zero the upper blocks (0,1) and (2,3): the w/u products read them
      const int c = 16 * (wv + 1) + lane - 16;
#pragma unroll
      for (int r = 0; r < 16; ++r) tmat[(16 * wv + r) * kLdT + c] = 0.f;
    }
    __syncthreads();
    // ---- solve: off-diagonal blocks, one block diagonal per step ----------
    {
      const int r = lane >> 2;
      const int cq = 4 * (lane & 3);
      float *xw = xs + wv * 16 * kLdX;
      for (int d = 1; d < 4; ++d) {
        const bool act = wv < 4 - d;
        const int bi = wv + d, bj = wv;
        if (act) {
          f32x4 x = zero4();
          for (int kb = bj; kb < bi; ++kb) {
            const float *arow = amat + (16 * bi + r) * kLdA + 16 * kb;
            const float *tcol = tmat + (16 * kb) * kLdT + 16 * bj + cq;
#pragma unroll
            for (int m = 0; m < 16; ++m) {
              const float a = arow[m];
              const f32x4 t = *reinterpret_cast<const f32x4 *>(tcol + m * kLdT);
              x += a * t;
            }
          }
          *reinterpret_cast<f32x4 *>(xw + r * kLdX + cq) = x;
        }
        __syncthreads();
        if (act) {
          f32x4 y = zero4();
          const float *trow = tmat + (16 * bi + r) * kLdT + 16 * bi;
#pragma unroll
          for (int m = 0; m < 16; ++m) y += trow[m] * *reinterpret_cast<const f32x4 *>(xw + m * kLdX + cq);
          *reinterpret_cast<f32x4 *>(tmat + (16 * bi + r) * kLdT + 16 * bj + cq) = -y;
        }
        __syncthreads();
      }
    }

    // ---- w then u: scaled T split to hi/lo bf16, MFMA with K^T / V^T -------
    for (int pass = 0; pass < 2; ++pass) {
      if (tid < 64) scl[tid] = pass == 0 ? bet[tid] * expf(gam[tid]) : bet[tid];
      __syncthreads();
      {
        const int r = tid >> 2;
        const int c0 = 16 * (tid & 3);
#pragma unroll
        for (int cc = 0; cc < 16; cc += 2) {
          const int c = c0 + cc;
          const float x0 = c <= r ? tmat[r * kLdT + c] * scl[c] : 0.f;
          const float x1 = c + 1 <= r ? tmat[r * kLdT + c + 1] * scl[c + 1] : 0.f;
          __bf16 h0, l0, h1, l1;
          split_bf16(x0, h0, l0);
          split_bf16(x1, h1, l1);
          *reinterpret_cast<uint32_t *>(ts_hi + r * kLdCol + c) = pack2(h0, h1);
          *reinterpret_cast<uint32_t *>(ts_lo + r * kLdCol + c) = pack2(l0, l1);
        }
      }
      __syncthreads();
      const __bf16 *src = pass == 0 ? kcol : r1;  // K^T or V^T, [128][72]
      // tiles (d-block db, token block rb): w as W^T = K^T (T s)^T (lane holds
      // four d of one token), u as U = (T s) V (lane holds four tokens of one d)
#pragma unroll
      for (int db2 = 0; db2 < 2; ++db2) {
        const int db = 2 * wv + db2;
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
          f32x4 acc = zero4();
          const int nks = (rb >> 1) + 1;
          for (int ks = 0; ks < nks; ++ks) {
            const bf16x8 a = frag_rows(src, kLdCol, 16 * db, 32 * ks, lane);
            const bf16x8 bh = frag_rows(ts_hi, kLdCol, 16 * rb, 32 * ks, lane);
            const bf16x8 bl = frag_rows(ts_lo, kLdCol, 16 * rb, 32 * ks, lane);
            if (pass == 0) {
              acc = mfma(a, bh, acc);
              acc = mfma(a, bl, acc);
              if constexpr (kF32In)
                acc = mfma(frag_rows(src + 128 * kLdCol, kLdCol, 16 * db, 32 * ks, lane), bh, acc);
            } else {
              acc = mfma(bh, a, acc);
              acc = mfma(bl, a, acc);
              if constexpr (kF32In)
                acc = mfma(bh, frag_rows(src + 128 * kLdCol, kLdCol, 16 * db, 32 * ks, lane), acc);
            }
          }
          if (pass == 0) {
            // lane holds w[r = 16 rb + (lane & 15)][d = 16 db + 4 (lane >> 4) + i]
            const int r = 16 * rb + (lane & 15);
            if (r < L) {
              _Float16 *dst = out.w16 + ((int64_t)hv * t_max + t0 + r) * kD + 32 * (db >> 1) +
                              perm4(4 * (db & 1) + (lane >> 4));
              *reinterpret_cast<u32x2 *>(dst) =
                  u32x2{pack_f16(-acc[0], -acc[1]), pack_f16(-acc[2], -acc[3])};
            }
          } else {
            // lane holds u[r = 16 rb + 4 (lane >> 4) + i][d = 16 db + (lane & 15)]
            float *dst = out.uimg + (((((int64_t)hv * nt + slot) * 8 + db) * 4 + rb) * 64 + lane) * 4;
            *reinterpret_cast<f32x4 *>(dst) = acc;
          }
        }
      }
      __syncthreads();
    }
  }
}

}  // namespace

hipError_t launch_intra(bool f32_in, const void *q, const void *k, const void *v, const float *g,
                        const float *beta, const int32_t *cu_seqlens, const int32_t *table,
                        int32_t nt_max, int32_t h, int32_t hv, int32_t t_max, float scale,
                        const StageBuffers &out, hipStream_t stream) {
  if (nt_max <= 0) return hipSuccess;
  const dim3 grid(nt_max, h);
  if (f32_in) {
    hipLaunchKernelGGL(intra_kernel<true>, grid, dim3(kThreads), 0, stream, q, k, v, g, beta,
                       cu_seqlens, table, out, h, hv, t_max, nt_max, scale);
  } else {
    hipLaunchKernelGGL(intra_kernel<false>, grid, dim3(kThreads), 0, stream, q, k, v, g, beta,
                       cu_seqlens, table, out, h, hv, t_max, nt_max, scale);
  }
  return hipGetLastError();
}

}  // namespace gdn
