// Stage 2 of the chunked forward: the inter-chunk kernel.
//
// "Optimizing GDN Chunk Prefill on Intel AMX CPU", section 5: per sequence and
// value head the chunks are walked in order with the fp32 state updated in
// place; per chunk (gamma the chunk-local cumulative g, Gamma its masked decay
// matrix, S the Dk x Dv state):
//
//   v'  = u - w S
//   o   = scale * ( diag(e^gamma) q S + tril(q k^T * Gamma) v' )   (diagonal kept)
//   S   = e^{gamma_last} S + k^T diag(e^{gamma_last - gamma}) v'
//
// The value columns of S are independent, so the state is blocked over Dv
// (Alloy page, "How do you parallelize a recurrence for prefill?": the state
// tile is blocked along the value dimension to fit on chip). Here one wave64
// owns a 128 x 16 column slice of S for the whole sequence and keeps it in
// registers, as eight 16 x 16 MFMA accumulators. Every product of the chunk
// step is arranged so that its operands come either from those accumulators
// directly or from fragments the intra stage stored in MFMA order:
//
//   v'      = u + (-w) S          A = -w fragment, B = S (fp16)      C = v' tiles
//   o^T     = S^T q^T             A = S (fp16),   B = q16 fragment   C = o^T tiles
//   o^T    += v'^T P^T            A = v' (hi+lo), B = P fragment (hi+lo)
//   S       = e^{gamma_last} S + K^T v'_dec    A = K^T fragment, B = v'_dec (hi+lo)
//
// A 16x16 accumulator gives lane (g, c) = (l >> 4, l & 15) rows 4g .. 4g + 3 of
// column c; two accumulators stacked along the contraction give a lane exactly
// the eight contraction values of an A (row c) or B (column c) fragment, with
// the contraction order {4g + i, 16 + 4g + i}. The intra stage writes w, q16,
// K^T and P in that order, so no value ever moves between lanes or through
// LDS inside the recurrence, and the chunk step itself has no barrier.
//
// Each slice is worked by two waves of one work-group, on different SIMDs:
//   chain wave : S -> fp16, v' = u + (-w) S, the decayed v' as hi + lo and the
//                state update -- the work that lies on the chunk-to-chunk
//                dependence chain;
//   helper wave: y = S^T q^T, v' as hi + lo, P v' and the output, one chunk
//                behind, from S (fp16) and v' that the chain wave leaves in a
//                double-buffered LDS exchange (8 KB per chunk).
// One barrier per chunk hands a chunk from the chain wave to the helper. A
// single wave issues its MFMA and VALU work one after the other, so splitting
// the chunk step over two SIMDs shortens the chain itself.
// Every operand fragment is one coalesced 16-byte-per-lane load straight into
// registers (rows past the sequence end read as zero). Each fragment array is
// refilled with the next chunk's fragments as soon as the current chunk's
// product has consumed it, so every load has about one chunk step of latency
// to land, and no wave blocks on issue.
//
// Work-group numbering is XCD-aware: all work-groups of the value heads that
// share a key head get the same blockIdx modulo 8, so they run on one XCD and
// share q16 and K^T through its L2.
#include "gdn_common.hpp"
#include "gdn_launch.hpp"

namespace gdn {

namespace {

constexpr int kXcds = 8;
constexpr int kSlices = kD / 16;  // 16-column value slices per head

// Fragments of one chunk (16 bytes per lane each):
//   w    (token tile R, d block p)   [4 R + p]   A of (-w) S        chain wave
//   K^T  (d tile tau, token block q) [2 tau + q] (+16: lo term)     chain wave
//   q16  (token tile R, d block p)   [4 R + p]   B of S^T q^T       helper wave
//   P    pair pi, term t (hi, lo)    [2 pi + t]  B of v'^T P^T      helper wave
template <bool kF32In>
struct ChainOps {
  static constexpr int kNK = kF32In ? 32 : 16;
  f16x8 w[16];
  bf16x8 k[kNK];
  f32x4 u[4];     // u tile R: rows 16 R + 4 g + i, value column v0 + c
  f32x4 dec[4];   // e^{gamma_last - gamma} of those rows
  float el;       // e^{gamma_last}
};
struct HelperOps {
  f16x8 q[16];
  bf16x8 p[12];
  float exs[4];   // scale * e^{gamma_r}, r = 16 R + c
};

__device__ __forceinline__ u32x4 ld16(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
}

// Two stacked accumulators -> bf16 hi + lo fragments.
__device__ __forceinline__ void split8(const f32x4 &a, const f32x4 &b, bf16x8 &hi, bf16x8 &lo) {
  const float x[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  u32x4 h, l;
  split8_words(x, h, l);
  hi = __builtin_bit_cast(bf16x8, h);
  lo = __builtin_bit_cast(bf16x8, l);
}

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// Raw buffer descriptor words (same fields as make_rsrc) for the store below.
__device__ __forceinline__ i32x4 rsrc_words(const void *base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return i32x4{static_cast<int32_t>(a & 0xffffffffu), static_cast<int32_t>((a >> 32) & 0xffffu),
               static_cast<int32_t>(bytes), 0x00020000};
}

// 16-byte buffer store issued as inline assembly. The compiler then never
// sees a store among the outstanding vector-memory operations, so its waits
// for the prefetched fragments stay counts of loads (loads return in order)
// instead of draining every load at each store. Out-of-range lanes are
// dropped like any buffer store; the leading s_nop covers a scalar operand
// written just before.
__device__ __forceinline__ void store16(const i32x4 &r, uint32_t voff, uint32_t soff, const f32x4 &v) {
  asm volatile("s_nop 4\n\tbuffer_store_dwordx4 %0, %1, %2, %3 offen"
               :
               : "v"(v), "v"(voff), "s"(r), "s"(soff)
               : "memory");
}

// Work-group barrier for the LDS hand-off: waits for this wave's LDS
// operations only (a plain __syncthreads would also drain the prefetched
// global loads).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Two stacked accumulators as one fp16 fragment (round to nearest even).
__device__ __forceinline__ f16x8 to_f16x8(const f32x4 &a, const f32x4 &b) {
  const u32x4 w{pack_f16(a[0], a[1]), pack_f16(a[2], a[3]), pack_f16(b[0], b[1]),
                pack_f16(b[2], b[3])};
  return __builtin_bit_cast(f16x8, w);
}

template <bool kF32In>
__global__ __launch_bounds__(128) void inter_kernel(StageBuffers in, const float *__restrict__ h0,
                                                   const int32_t *__restrict__ cu,
                                                   float *__restrict__ o, float *__restrict__ hT,
                                                   int n_max, int H, int Hv, int t_max, int nt) {
  constexpr int kNK = ChainOps<kF32In>::kNK;
  // chunk hand-off, two buffers x {S as fp16: 4 fragments, v': 4 tiles} x 1 KB
  __shared__ __attribute__((aligned(16))) u32x4 xch[2][8][64];

  // ---- XCD-aware work-group -> (sequence, value head, slice) --------------
  const int HG = Hv / H;
  const int members = HG * kSlices;
  const int xcd = blockIdx.x % kXcds;
  const int wslot = blockIdx.x / kXcds;
  const int group = (wslot / members) * kXcds + xcd;  // (sequence, key head)
  const int member = wslot % members;
  if (group >= n_max * H) return;
  const int s = group / H;
  const int h = group % H;
  const int hv = h * HG + member / kSlices;
  const int slice = member % kSlices;
  const int v0 = 16 * slice;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  const int lane = threadIdx.x & 63;
  const int c16 = lane & 15;
  const int g4 = 4 * (lane >> 4);

  const int bos = cu[s];
  const int eos = cu[s + 1];
  const int nc = (eos - bos + kC - 1) / kC;

  const uint32_t vo_f = static_cast<uint32_t>(lane) * 16;  // 1 KB fragment blocks

  if (wave == 0) {
    // =========================== chain wave ================================
    const uint32_t vo_w = static_cast<uint32_t>(c16 * kD + 2 * g4) * 2;  // w16 rows
    struct Rsrc { rsrc_t w, k, u, g; };
    auto rsrc_of = [&](int c) __attribute__((always_inline)) {
      const int t0 = bos + kC * c;
      const int slot = (t0 >> 6) + s;
      const bool ok = c < nc;
      const uint32_t lc = ok ? static_cast<uint32_t>(min(kC, eos - t0)) : 0u;
      Rsrc r;
      r.w = make_rsrc(in.w16 + ((int64_t)hv * t_max + t0) * kD, lc * kD * 2);
      r.k = make_rsrc(in.kimg + ((int64_t)h * nt + slot) * kNK * 512, ok ? kNK * 1024 : 0);
      r.u = make_rsrc(in.uimg + (((int64_t)hv * nt + slot) * kSlices + slice) * 4 * 256, ok ? 4096 : 0);
      r.g = make_rsrc(in.gimg + ((int64_t)hv * nt + slot) * kGateStride, ok ? kGateStride * 4 : 0);
      return r;
    };
    ChainOps<kF32In> x;
    auto load_w = [&](const Rsrc &r) __attribute__((always_inline)) {
#pragma unroll
      for (int f = 0; f < 16; ++f)
        x.w[f] = __builtin_bit_cast(f16x8, ld16(r.w, vo_w, (f >> 2) * 16 * kD * 2 + (f & 3) * 64));
    };
    auto load_k = [&](const Rsrc &r) __attribute__((always_inline)) {
#pragma unroll
      for (int f = 0; f < kNK; ++f) x.k[f] = __builtin_bit_cast(bf16x8, ld16(r.k, vo_f, f * 1024));
    };
    auto load_u = [&](const Rsrc &r) __attribute__((always_inline)) {
#pragma unroll
      for (int R = 0; R < 4; ++R) {
        x.u[R] = __builtin_bit_cast(f32x4, ld16(r.u, vo_f, R * 1024));
        x.dec[R] = __builtin_bit_cast(f32x4, ld16(r.g, 4 * g4, R * 64));
      }
      x.el = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r.g, 0, 512, 0));
    };

    // state slice: S[tau] holds S[d = 16 tau + 4g + i][v0 + c]
    f32x4 S[8];
    const int64_t sbase = (((int64_t)s * Hv + hv) * kD + v0 + c16) * kD + g4;
#pragma unroll
    for (int tau = 0; tau < 8; ++tau)
      S[tau] = h0 ? *reinterpret_cast<const f32x4 *>(h0 + sbase + 16 * tau) : zero4();

    {  // chunk 0's operands, in the loop's order
      const Rsrc r = rsrc_of(0);
      __builtin_amdgcn_sched_barrier(0);
      load_w(r);
      __builtin_amdgcn_sched_barrier(0);
      load_u(r);
      __builtin_amdgcn_sched_barrier(0);
      load_k(r);
      __builtin_amdgcn_sched_barrier(0);
    }
    for (int c = 0; c < nc; ++c) {
      const Rsrc rn = rsrc_of(c + 1);
      u32x4 *xb = &xch[c & 1][0][lane];
      f16x8 s16[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        s16[p] = to_f16x8(S[2 * p], S[2 * p + 1]);
        xb[64 * p] = __builtin_bit_cast(u32x4, s16[p]);
      }
      // v' = u + (-w) S
      f32x4 v[4] = {x.u[0], x.u[1], x.u[2], x.u[3]};
#pragma unroll
      for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int R = 0; R < 4; ++R) v[R] = mfma(x.w[4 * R + p], s16[p], v[R]);
#pragma unroll
      for (int tau = 0; tau < 8; ++tau) S[tau] = S[tau] * x.el;
      __builtin_amdgcn_sched_barrier(0);
      load_w(rn);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int R = 0; R < 4; ++R) xb[64 * (4 + R)] = __builtin_bit_cast(u32x4, v[R]);
      lds_barrier();  // chunk c's S (fp16) and v' are ready for the helper
      // S += K^T (e^{gamma_last - gamma} v')
      bf16x8 eh[2], elo[2];
      split8(v[0] * x.dec[0], v[1] * x.dec[1], eh[0], elo[0]);
      split8(v[2] * x.dec[2], v[3] * x.dec[3], eh[1], elo[1]);
      __builtin_amdgcn_sched_barrier(0);
      load_u(rn);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int tau = 0; tau < 8; ++tau) {
          S[tau] = mfma(x.k[2 * tau + q], eh[q], S[tau]);
          S[tau] = mfma(x.k[2 * tau + q], elo[q], S[tau]);
          if constexpr (kF32In) S[tau] = mfma(x.k[16 + 2 * tau + q], eh[q], S[tau]);
        }
      __builtin_amdgcn_sched_barrier(0);
      load_k(rn);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (hT) {
#pragma unroll
      for (int tau = 0; tau < 8; ++tau) *reinterpret_cast<f32x4 *>(hT + sbase + 16 * tau) = S[tau];
    }
  } else {
    // =========================== helper wave ===============================
    const uint32_t vo_q = static_cast<uint32_t>(c16 * H * kD + 2 * g4) * 2;  // q16 rows
    const uint32_t vo_o = static_cast<uint32_t>(c16 * Hv * kD + g4) * 4;     // o rows
    const uint32_t row_q = static_cast<uint32_t>(16 * H * kD * 2);           // 16 q16 rows
    const uint32_t row_o = static_cast<uint32_t>(16 * Hv * kD * 4);          // 16 o rows
    struct Rsrc { rsrc_t q, p, g; };
    auto rsrc_of = [&](int c) __attribute__((always_inline)) {
      const int t0 = bos + kC * c;
      const int slot = (t0 >> 6) + s;
      const bool ok = c < nc;
      const uint32_t lc = ok ? static_cast<uint32_t>(min(kC, eos - t0)) : 0u;
      Rsrc r;
      r.q = make_rsrc(in.q16 + ((int64_t)t0 * H + h) * kD, lc * H * kD * 2);
      r.p = make_rsrc(in.pimg + ((int64_t)hv * nt + slot) * 12 * 512, ok ? 12 * 1024 : 0);
      r.g = make_rsrc(in.gimg + ((int64_t)hv * nt + slot) * kGateStride, ok ? kGateStride * 4 : 0);
      return r;
    };
    HelperOps y;
    auto load_q = [&](const Rsrc &r) __attribute__((always_inline)) {
#pragma unroll
      for (int f = 0; f < 16; ++f)
        y.q[f] = __builtin_bit_cast(f16x8, ld16(r.q, vo_q, (f >> 2) * row_q + (f & 3) * 64));
    };
    auto load_p = [&](const Rsrc &r) __attribute__((always_inline)) {
#pragma unroll
      for (int f = 0; f < 12; ++f) y.p[f] = __builtin_bit_cast(bf16x8, ld16(r.p, vo_f, f * 1024));
#pragma unroll
      for (int R = 0; R < 4; ++R)
        y.exs[R] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r.g, 4 * c16, 256 + R * 64, 0));
    };
    {
      const Rsrc r = rsrc_of(0);
      __builtin_amdgcn_sched_barrier(0);
      load_q(r);
      __builtin_amdgcn_sched_barrier(0);
      load_p(r);
      __builtin_amdgcn_sched_barrier(0);
    }
    for (int c = 0; c < nc; ++c) {
      const Rsrc rn = rsrc_of(c + 1);
      lds_barrier();  // chunk c handed over
      const u32x4 *xb = &xch[c & 1][0][lane];
      f16x8 s16[4];
      f32x4 v[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) s16[p] = __builtin_bit_cast(f16x8, xb[64 * p]);
#pragma unroll
      for (int R = 0; R < 4; ++R) v[R] = __builtin_bit_cast(f32x4, xb[64 * (4 + R)]);
      // y^T = S^T q^T while v' is split into hi + lo
      f32x4 ya[4] = {zero4(), zero4(), zero4(), zero4()};
#pragma unroll
      for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int R = 0; R < 4; ++R) ya[R] = mfma(s16[p], y.q[4 * R + p], ya[R]);
      bf16x8 dh[2], dl[2];
      split8(v[0], v[1], dh[0], dl[0]);
      split8(v[2], v[3], dh[1], dl[1]);
      __builtin_amdgcn_sched_barrier(0);
      load_q(rn);
      __builtin_amdgcn_sched_barrier(0);
      // o^T = v'^T P^T + scale e^gamma y^T
      f32x4 pa[4] = {zero4(), zero4(), zero4(), zero4()};
#pragma unroll
      for (int R = 0; R < 4; ++R) {
#pragma unroll
        for (int q = 0; q <= (R >> 1); ++q) {
          const int pi = R < 2 ? R : 2 * R - 2 + q;
          pa[R] = mfma(dh[q], y.p[2 * pi], pa[R]);
          pa[R] = mfma(dl[q], y.p[2 * pi], pa[R]);
          pa[R] = mfma(dh[q], y.p[2 * pi + 1], pa[R]);
        }
      }
      const float exs[4] = {y.exs[0], y.exs[1], y.exs[2], y.exs[3]};
      __builtin_amdgcn_sched_barrier(0);
      load_p(rn);
      __builtin_amdgcn_sched_barrier(0);
      const int t0 = bos + kC * c;
      const uint32_t lc = static_cast<uint32_t>(min(kC, eos - t0));
      const i32x4 ro = rsrc_words(o + ((int64_t)t0 * Hv + hv) * kD + v0, lc * Hv * kD * 4);
#pragma unroll
      for (int R = 0; R < 4; ++R) store16(ro, vo_o, R * row_o, pa[R] + exs[R] * ya[R]);
    }
  }
}

template <bool kF32In>
hipError_t launch_waves(const StageBuffers &in, const float *h0, const int32_t *cu, int32_t n_max,
                        int32_t h, int32_t hv, int32_t t_max, int32_t nt, float *o, float *hT,
                        hipStream_t stream, KernelEvents ev) {
  const int members = (hv / h) * kSlices;
  const int groups = n_max * h;
  const int rounds = (groups + kXcds - 1) / kXcds;
  const dim3 grid(rounds * kXcds * members);
  hipExtLaunchKernelGGL((inter_kernel<kF32In>), grid, dim3(128), 0, stream, ev.start, ev.stop, 0,
                        in, h0, cu, o, hT, n_max, h, hv, t_max, nt);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_inter(bool f32_in, const StageBuffers &in, const float *h0,
                        const int32_t *cu_seqlens, int32_t n_max, int32_t h, int32_t hv,
                        int32_t t_max, int32_t nt_max, float *o, float *hT, hipStream_t stream,
                        KernelEvents ev) {
  return f32_in
             ? launch_waves<true>(in, h0, cu_seqlens, n_max, h, hv, t_max, nt_max, o, hT, stream, ev)
             : launch_waves<false>(in, h0, cu_seqlens, n_max, h, hv, t_max, nt_max, o, hT, stream, ev);
}

}  // namespace gdn
