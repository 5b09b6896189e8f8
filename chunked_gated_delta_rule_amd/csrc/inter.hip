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
// for the whole sequence; wave wv owns token rows 16 wv .. 16 wv + 15 of the
// chunk and state rows 32 wv .. 32 wv + 31.
//
// Per chunk there are two phases separated by a barrier, and a barrier ends
// the chunk:
//   phase 1: X = w S and Y = q S (w, q fragments straight from HBM/L2 into
//            registers, S as hi/lo bf16 from LDS); this wave's row block of
//            P = tril(q k^T * Gamma), kept in registers; v' = u - X and the
//            decayed v' go to LDS as hi/lo bf16.
//   phase 2: o = scale (e^gamma Y + P v') and S = e^{gamma_last} S + k^T v'_dec
//            (k transposed from LDS); S goes back to LDS as hi/lo bf16; the
//            next chunk's k tile and gates are staged.
// The next chunk's inputs are loaded at the start of phase 1 (buffer loads;
// rows past the sequence end read as zero) so their latency hides behind a
// whole chunk of work. Every product runs on v_mfma_f32_16x16x32_bf16; the
// fp32 operands S, P, v' and the decayed v' enter as hi + lo bf16 pairs.
//
// P stays in registers: the MFMA result layout of a P^T block gives each lane
// one row t and four consecutive columns j, so two P^T blocks form the lane's
// eight contraction slots of a P v' product. v' is stored with the matching
// permutation of j, so its fragment is still one 16-byte LDS read.
//
// Work-group numbering is XCD-aware: all value-column blocks of all value
// heads that share a key head (16 work-groups at Hv = 2 H) get the same
// blockIdx modulo 8, so they run on one XCD and share q, k, w through its L2.
// Gates enter the exponentials as log2-scaled cumulative sums, and every
// exponent is a difference that is <= 0 (masked before the exponential).
#include "gdn_common.hpp"
#include "gdn_launch.hpp"

namespace gdn {

namespace {

constexpr int kBV = 16;          // value columns per work-group
constexpr int kNVT = kD / kBV;   // value-column blocks per head
constexpr int kLdRow = kD + 8;   // k row-major [64][136] bf16
constexpr int kLdCol = kC + 8;   // k transposed [128][72] bf16, 16-byte groups swizzled
constexpr int kLdS = kD + 8;     // S^T hi/lo [16][136]
constexpr int kLdV = kC + 8;     // v'^T hi/lo [16][72]
constexpr int kXcds = 8;

template <bool kF32In>
struct InterSmem {
  static constexpr int kT = kF32In ? 2 : 1;
  static constexpr int kKr = kT * 64 * kLdRow * 2;
  static constexpr int kKc = kT * 128 * kLdCol * 2;
  static constexpr int kS = 2 * kBV * kLdS * 2;
  static constexpr int kDl = 2 * kBV * kLdV * 2;
  static constexpr int kBytes = kKr + kKc + kS + 2 * kDl + 2 * 64 * 4;
  static_assert(kBytes <= 160 * 1024, "LDS budget");
};

// Element (d, j) of the transposed k tile. The eight 16-byte groups of a row
// are XOR-swizzled by d / 16 so that the transposing stores (one d per lane,
// four consecutive j) and the fragment reads (16 consecutive d, eight j) are
// both free of bank conflicts.
__device__ __forceinline__ int kcol_at(int d, int j) {
  return d * kLdCol + ((((j >> 3) ^ (d >> 4)) & 7) << 3) + (j & 7);
}

__device__ __forceinline__ uint16_t half_of(const u32x4 &w, int i) {
  return static_cast<uint16_t>((w[i >> 1] >> (16 * (i & 1))) & 0xffffu);
}

// Eight fp32 (two 16-byte words) -> eight bf16 hi and eight bf16 lo.
__device__ __forceinline__ void split8(const u32x4 &a, const u32x4 &b, u32x4 &hi, u32x4 &lo) {
  uint32_t h[4], l[4];
  split2(__uint_as_float(a[0]), __uint_as_float(a[1]), h[0], l[0]);
  split2(__uint_as_float(a[2]), __uint_as_float(a[3]), h[1], l[1]);
  split2(__uint_as_float(b[0]), __uint_as_float(b[1]), h[2], l[2]);
  split2(__uint_as_float(b[2]), __uint_as_float(b[3]), h[3], l[3]);
  hi = u32x4{h[0], h[1], h[2], h[3]};
  lo = u32x4{l[0], l[1], l[2], l[3]};
}

// One chunk's per-wave MFMA operands, as loaded from memory.
template <bool kF32In>
struct ChunkFrags {
  static constexpr int kN = kF32In ? 8 : 4;
  u32x4 q[kN];  // q rows 16 wv + (lane & 15); k-step kk in q[kk] (fp32: q[2kk], q[2kk+1])
  u32x4 w[4];   // w rows 16 wv + (lane & 15), bf16
  float u[4];   // u rows 16 wv + quad + i, column vcol
};

// This thread's 4 x 8 block of the chunk's k tile, and (wave 0) its gate.
template <bool kF32In>
struct ChunkK {
  static constexpr int kN = kF32In ? 8 : 4;
  u32x4 v[kN];
  float g;
};

template <bool kF32In>
__global__ __launch_bounds__(kThreads, 1) void inter_kernel(
    const void *__restrict__ qin, const void *__restrict__ kin, const __bf16 *__restrict__ win,
    const float *__restrict__ uin, const float *__restrict__ g, const float *__restrict__ h0,
    const int32_t *__restrict__ cu, float *__restrict__ o, float *__restrict__ hT, int n_max,
    int H, int Hv, int t_max, float scale) {
  using Smem = InterSmem<kF32In>;
  constexpr int kElt = kF32In ? 4 : 2;
  __shared__ __attribute__((aligned(16))) unsigned char smem[Smem::kBytes];
  unsigned char *p = smem;
  __bf16 *krow = reinterpret_cast<__bf16 *>(p); p += Smem::kKr;
  __bf16 *kcol = reinterpret_cast<__bf16 *>(p); p += Smem::kKc;
  __bf16 *s_hi = reinterpret_cast<__bf16 *>(p);
  __bf16 *s_lo = s_hi + kBV * kLdS; p += Smem::kS;
  __bf16 *dl_hi = reinterpret_cast<__bf16 *>(p);
  __bf16 *dl_lo = dl_hi + kBV * kLdV; p += Smem::kDl;
  __bf16 *dp_hi = reinterpret_cast<__bf16 *>(p);
  __bf16 *dp_lo = dp_hi + kBV * kLdV; p += Smem::kDl;
  float *gam2 = reinterpret_cast<float *>(p);  // [2][64], log2-scaled cumulative gates

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
  const int l16 = lane & 15;
  const int quad = 4 * (lane >> 4);
  const int lrow = 4 * (tid >> 4);  // k staging: rows lrow .. lrow + 3
  const int lcol = 8 * (tid & 15);  //            columns lcol .. lcol + 7
  const int vcol = kBV * vt + l16;  // this lane's value column in result layouts

  const int bos = cu[s];
  const int eos = cu[s + 1];
  const int nchunks = (eos - bos + kC - 1) / kC;
  const uint32_t rs_qk = static_cast<uint32_t>(H) * kD * kElt;  // bytes per q/k token row
  const uint32_t rs_o = static_cast<uint32_t>(Hv) * kD * 4;     // bytes per o token row
  float *hT_lane = hT ? hT + (((int64_t)s * Hv + hv) * kD + vcol) * kD : nullptr;

  // ---- initial state: S[d][v] for d = 32 wv + 16 b + quad + i ---------------
  f32x4 sacc[2];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int d = 32 * wv + 16 * b + quad;
    sacc[b] = h0 ? *reinterpret_cast<const f32x4 *>(h0 + (((int64_t)s * Hv + hv) * kD + vcol) * kD + d)
                 : zero4();
  }
  if (nchunks == 0) {
    if (hT_lane) {
#pragma unroll
      for (int b = 0; b < 2; ++b)
        *reinterpret_cast<f32x4 *>(hT_lane + 32 * wv + 16 * b + quad) = sacc[b];
    }
    return;
  }

  auto store_state = [&]() {
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const float x[4] = {sacc[b][0], sacc[b][1], sacc[b][2], sacc[b][3]};
      u32x2 hi, lo;
      split_pack4(x, hi, lo);
      const int d = 32 * wv + 16 * b + quad;
      *reinterpret_cast<u32x2 *>(s_hi + l16 * kLdS + d) = hi;
      *reinterpret_cast<u32x2 *>(s_lo + l16 * kLdS + d) = lo;
    }
  };

  auto load_chunk = [&](int c, ChunkFrags<kF32In> &f, ChunkK<kF32In> &kr) {
    const int t0 = bos + c * kC;
    const uint32_t L = static_cast<uint32_t>(min(kC, eos - t0));
    const char *qb = static_cast<const char *>(qin) + ((int64_t)t0 * H + h) * kD * kElt;
    const char *kb = static_cast<const char *>(kin) + ((int64_t)t0 * H + h) * kD * kElt;
    const rsrc_t rq = make_rsrc(qb, L * rs_qk);
    const rsrc_t rk = make_rsrc(kb, L * rs_qk);
    const rsrc_t rw = make_rsrc(win + ((int64_t)hv * t_max + t0) * kD, L * kD * 2);
    const rsrc_t ru = make_rsrc(uin + ((int64_t)hv * t_max + t0) * kD, L * kD * 4);
    const rsrc_t rg = make_rsrc(g + (int64_t)t0 * Hv + hv, L * Hv * 4);
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const uint32_t off = (lrow + rr) * rs_qk + lcol * kElt;
      if constexpr (kF32In) {
        kr.v[2 * rr] = buf_load16(rk, off);
        kr.v[2 * rr + 1] = buf_load16(rk, off + 16);
      } else {
        kr.v[rr] = buf_load16(rk, off);
      }
    }
    kr.g = wv == 0 ? buf_load_f32(rg, lane * Hv * 4) : 0.f;
    const uint32_t qrow = (16 * wv + l16) * rs_qk;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int col = 32 * kk + 8 * (lane >> 4);
      if constexpr (kF32In) {
        f.q[2 * kk] = buf_load16(rq, qrow + col * 4);
        f.q[2 * kk + 1] = buf_load16(rq, qrow + col * 4 + 16);
      } else {
        f.q[kk] = buf_load16(rq, qrow + col * 2);
      }
      f.w[kk] = buf_load16(rw, (16 * wv + l16) * kD * 2 + col * 2);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) f.u[i] = buf_load_f32(ru, ((16 * wv + quad + i) * kD + vcol) * 4);
  };

  auto k_rows = [&](const ChunkK<kF32In> &kr, u32x4 (&hi)[4], u32x4 (&lo)[4]) {
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      if constexpr (kF32In) {
        split8(kr.v[2 * rr], kr.v[2 * rr + 1], hi[rr], lo[rr]);
      } else {
        hi[rr] = kr.v[rr];
        lo[rr] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };

  auto stage_krow = [&](const ChunkK<kF32In> &kr) {
    u32x4 hi[4], lo[4];
    k_rows(kr, hi, lo);
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      *reinterpret_cast<u32x4 *>(krow + (lrow + rr) * kLdRow + lcol) = hi[rr];
      if constexpr (kF32In)
        *reinterpret_cast<u32x4 *>(krow + 64 * kLdRow + (lrow + rr) * kLdRow + lcol) = lo[rr];
    }
  };

  auto stage_kcol = [&](const ChunkK<kF32In> &kr) {
    u32x4 hi[4], lo[4];
    k_rows(kr, hi, lo);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int at = kcol_at(lcol + i, lrow);
      const uint32_t a = half_of(hi[0], i) | (static_cast<uint32_t>(half_of(hi[1], i)) << 16);
      const uint32_t b = half_of(hi[2], i) | (static_cast<uint32_t>(half_of(hi[3], i)) << 16);
      *reinterpret_cast<u32x2 *>(kcol + at) = u32x2{a, b};
      if constexpr (kF32In) {
        const uint32_t c2 = half_of(lo[0], i) | (static_cast<uint32_t>(half_of(lo[1], i)) << 16);
        const uint32_t d2 = half_of(lo[2], i) | (static_cast<uint32_t>(half_of(lo[3], i)) << 16);
        *reinterpret_cast<u32x2 *>(kcol + 128 * kLdCol + at) = u32x2{c2, d2};
      }
    }
  };

  auto stage_gates = [&](const ChunkK<kF32In> &kr, int buf) {
    if (wv == 0) gam2[buf * 64 + lane] = wave_inclusive_scan(kr.g, lane) * kLog2e;
  };

  // One chunk: `cur` holds its fragments, the next chunk is loaded into `nxt`.
  ChunkK<kF32In> kr;
  auto chunk = [&](int c, ChunkFrags<kF32In> &cur, ChunkFrags<kF32In> &nxt) {
    const int t0 = bos + c * kC;
    const int L = min(kC, eos - t0);
    const float *gm = gam2 + (c & 1) * 64;
    stage_kcol(kr);
    const bool more = c + 1 < nchunks;
    if (more) load_chunk(c + 1, nxt, kr);

    // ---- phase 1: X = w S, Y = q S ------------------------------------------
    bf16x8 qh[4], ql[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      if constexpr (kF32In) {
        u32x4 hi, lo;
        split8(cur.q[2 * kk], cur.q[2 * kk + 1], hi, lo);
        qh[kk] = as_bf16x8(hi);
        ql[kk] = as_bf16x8(lo);
      } else {
        qh[kk] = as_bf16x8(cur.q[kk]);
      }
    }
    f32x4 xh = zero4(), xl = zero4(), yh = zero4(), yl = zero4();
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const bf16x8 sh = frag_rows(s_hi, kLdS, 0, 32 * kk, lane);
      const bf16x8 sl = frag_rows(s_lo, kLdS, 0, 32 * kk, lane);
      const bf16x8 aw = as_bf16x8(cur.w[kk]);
      xh = mfma(aw, sh, xh);
      xl = mfma(aw, sl, xl);
      yh = mfma(qh[kk], sh, yh);
      yl = mfma(qh[kk], sl, yl);
      if constexpr (kF32In) yl = mfma(ql[kk], sh, yl);
    }
    // ---- this wave's row block of P, as P^T blocks (jb, wv) in registers ------
    // lane holds P[t = 16 wv + l16][j = 16 jb + quad + i]
    u32x2 ph[4], pl[4];
    const int t = 16 * wv + l16;
    const float gt = gm[t];
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) {
      ph[jb] = u32x2{0u, 0u};
      pl[jb] = u32x2{0u, 0u};
      if (jb <= wv) {
        f32x4 acc = zero4();
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const bf16x8 ak = frag_rows(krow, kLdRow, 16 * jb, 32 * kk, lane);
          acc = mfma(ak, qh[kk], acc);
          if constexpr (kF32In) {
            acc = mfma(frag_rows(krow + 64 * kLdRow, kLdRow, 16 * jb, 32 * kk, lane), qh[kk], acc);
            acc = mfma(ak, ql[kk], acc);
          }
        }
        float pv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = 16 * jb + quad + i;
          const float e = fast_exp2(gt - gm[j]);  // only used where j <= t
          pv[i] = j <= t ? acc[i] * e : 0.f;
        }
        split_pack4(pv, ph[jb], pl[jb]);
      }
    }
    // ---- v' and decayed v' ---------------------------------------------------
    const float gl = gm[63];
    f32x4 X = xh + xl;
    {
      float dl[4], dp[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * wv + quad + i;
        dl[i] = cur.u[i] - X[i];
        dp[i] = dl[i] * fast_exp2(gl - gm[r]);
      }
      u32x2 hi, lo;
      split_pack4(dl, hi, lo);
      const int perm = 32 * (wv >> 1) + 2 * quad + 4 * (wv & 1);  // see the P v' product
      *reinterpret_cast<u32x2 *>(dl_hi + l16 * kLdV + perm) = hi;
      *reinterpret_cast<u32x2 *>(dl_lo + l16 * kLdV + perm) = lo;
      split_pack4(dp, hi, lo);
      *reinterpret_cast<u32x2 *>(dp_hi + l16 * kLdV + 16 * wv + quad) = hi;
      *reinterpret_cast<u32x2 *>(dp_lo + l16 * kLdV + 16 * wv + quad) = lo;
    }
    __syncthreads();

    // ---- phase 2: o = scale (e^gamma Y + P v') --------------------------------
    {
      f32x4 oacc = zero4();
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        if (kk <= (wv >> 1)) {
          const bf16x8 pa = __builtin_bit_cast(
              bf16x8, u32x4{ph[2 * kk][0], ph[2 * kk][1], ph[2 * kk + 1][0], ph[2 * kk + 1][1]});
          const bf16x8 pb = __builtin_bit_cast(
              bf16x8, u32x4{pl[2 * kk][0], pl[2 * kk][1], pl[2 * kk + 1][0], pl[2 * kk + 1][1]});
          const bf16x8 dh = frag_rows(dl_hi, kLdV, 0, 32 * kk, lane);
          const bf16x8 dlo = frag_rows(dl_lo, kLdV, 0, 32 * kk, lane);
          oacc = mfma(pa, dh, oacc);
          oacc = mfma(pa, dlo, oacc);
          oacc = mfma(pb, dh, oacc);
        }
      }
      const f32x4 Y = yh + yl;
      const rsrc_t ro = make_rsrc(o + ((int64_t)t0 * Hv + hv) * kD, L * rs_o);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * wv + quad + i;
        const float val = scale * (fast_exp2(gm[r]) * Y[i] + oacc[i]);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(val), ro, r * rs_o + vcol * 4, 0, 0);
      }
    }
    // ---- S = e^{gamma_last} S + k^T v'_dec -------------------------------------
    {
      const float decay = fast_exp2(gl);
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int d = 32 * wv + 16 * b + l16;
        f32x4 ah = sacc[b] * decay, al = zero4();
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const int at = kcol_at(d, 32 * kk + 8 * (lane >> 4));
          const bf16x8 ak = lds_frag(kcol + at);
          const bf16x8 bh = frag_rows(dp_hi, kLdV, 0, 32 * kk, lane);
          const bf16x8 bl = frag_rows(dp_lo, kLdV, 0, 32 * kk, lane);
          ah = mfma(ak, bh, ah);
          al = mfma(ak, bl, al);
          if constexpr (kF32In) al = mfma(lds_frag(kcol + 128 * kLdCol + at), bh, al);
        }
        sacc[b] = ah + al;
      }
    }
    store_state();
    if (more) {
      stage_krow(kr);
      stage_gates(kr, (c + 1) & 1);
    }
    __syncthreads();
  };

  ChunkFrags<kF32In> fa, fb;
  load_chunk(0, fa, kr);
  stage_krow(kr);
  stage_gates(kr, 0);
  store_state();
  __syncthreads();
  for (int c = 0;;) {
    chunk(c, fa, fb);
    if (++c >= nchunks) break;
    chunk(c, fb, fa);
    if (++c >= nchunks) break;
  }

  if (hT_lane) {
#pragma unroll
    for (int b = 0; b < 2; ++b)
      *reinterpret_cast<f32x4 *>(hT_lane + 32 * wv + 16 * b + quad) = sacc[b];
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
