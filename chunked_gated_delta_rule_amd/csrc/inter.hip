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
//   v'      = u + w (-S)          A = w fragment, B = -S (fp16)      C = v' tiles
//   o^T     = -(-S)^T q^T         A = -S (fp16),  B = q16 fragment   C = o^T tiles
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
// Every operand fragment is one coalesced 16-byte-per-lane load straight into
// registers (rows past the sequence end read as zero); nothing goes through
// LDS. Each fragment array is refilled with the next chunk's fragments as soon
// as the current chunk's product has consumed it, so every load has about one
// chunk step of latency to land, and the wave never blocks on issue. A
// work-group is a single wave: waves never wait for each other.
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
//   w    (token tile R, d block p)   [4 R + p]   A of w S
//   q16  (token tile R, d block p)   [4 R + p]   B of S^T q^T
//   P    pair pi, term t (hi, lo)    [2 pi + t]  B of v'^T P^T
//   K^T  (d tile tau, token block q) [2 tau + q] (+16: lo term)  A of K^T v'
template <bool kF32In>
struct Chunk {
  static constexpr int kNK = kF32In ? 32 : 16;
  f16x8 w[16];
  f16x8 q[16];
  bf16x8 p[12];
  bf16x8 k[kNK];
  f32x4 u[4];     // u tile R: rows 16 R + 4 g + i, value column v0 + c
  f32x4 dec[4];   // e^{gamma_last - gamma} of those rows
  float exs[4];   // scale * e^{gamma_r}, r = 16 R + c
  float el;       // e^{gamma_last}
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

// -S of two stacked accumulators as one fp16 fragment (round to nearest even).
__device__ __forceinline__ f16x8 neg_f16(const f32x4 &a, const f32x4 &b) {
  const u32x4 w{pack_f16(-a[0], -a[1]), pack_f16(-a[2], -a[3]), pack_f16(-b[0], -b[1]),
                pack_f16(-b[2], -b[3])};
  return __builtin_bit_cast(f16x8, w);
}

template <bool kF32In>
__global__ __launch_bounds__(64) void inter_kernel(StageBuffers in, const float *__restrict__ h0,
                                                  const int32_t *__restrict__ cu,
                                                  float *__restrict__ o, float *__restrict__ hT,
                                                  int n_max, int H, int Hv, int t_max, int nt) {
  using CK = Chunk<kF32In>;
  constexpr int kNK = CK::kNK;

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

  const int lane = threadIdx.x & 63;
  const int c16 = lane & 15;
  const int g4 = 4 * (lane >> 4);

  const int bos = cu[s];
  const int eos = cu[s + 1];
  const int nc = (eos - bos + kC - 1) / kC;

  // lane parts of the buffer offsets (chunk parts go into the descriptors)
  const uint32_t vo_w = static_cast<uint32_t>(c16 * kD + 2 * g4) * 2;      // w16 rows
  const uint32_t vo_q = static_cast<uint32_t>(c16 * H * kD + 2 * g4) * 2;  // q16 rows
  const uint32_t vo_f = static_cast<uint32_t>(lane) * 16;                  // 1 KB blocks
  const uint32_t vo_o = static_cast<uint32_t>(c16 * Hv * kD + g4) * 4;     // o rows
  const uint32_t row_q = static_cast<uint32_t>(16 * H * kD * 2);           // 16 q16 rows
  const uint32_t row_o = static_cast<uint32_t>(16 * Hv * kD * 4);          // 16 o rows

  // descriptors of chunk c (zero-length past the last chunk: loads read 0)
  struct Rsrc { rsrc_t w, q, p, k, u, g; };
  auto rsrc_of = [&](int c) __attribute__((always_inline)) {
    const int t0 = bos + kC * c;
    const int slot = (t0 >> 6) + s;
    const bool ok = c < nc;
    const uint32_t lc = ok ? static_cast<uint32_t>(min(kC, eos - t0)) : 0u;
    Rsrc r;
    r.w = make_rsrc(in.w16 + ((int64_t)hv * t_max + t0) * kD, lc * kD * 2);
    r.q = make_rsrc(in.q16 + ((int64_t)t0 * H + h) * kD, lc * H * kD * 2);
    r.p = make_rsrc(in.pimg + ((int64_t)hv * nt + slot) * 12 * 512, ok ? 12 * 1024 : 0);
    r.k = make_rsrc(in.kimg + ((int64_t)h * nt + slot) * kNK * 512, ok ? kNK * 1024 : 0);
    r.u = make_rsrc(in.uimg + (((int64_t)hv * nt + slot) * kSlices + slice) * 4 * 256, ok ? 4096 : 0);
    r.g = make_rsrc(in.gimg + ((int64_t)hv * nt + slot) * kGateStride, ok ? kGateStride * 4 : 0);
    return r;
  };
  auto load_w = [&](CK &x, const Rsrc &r) __attribute__((always_inline)) {
#pragma unroll
    for (int f = 0; f < 16; ++f)
      x.w[f] = __builtin_bit_cast(f16x8, ld16(r.w, vo_w, (f >> 2) * 16 * kD * 2 + (f & 3) * 64));
  };
  auto load_q = [&](CK &x, const Rsrc &r) __attribute__((always_inline)) {
#pragma unroll
    for (int f = 0; f < 16; ++f)
      x.q[f] = __builtin_bit_cast(f16x8, ld16(r.q, vo_q, (f >> 2) * row_q + (f & 3) * 64));
  };
  auto load_p = [&](CK &x, const Rsrc &r) __attribute__((always_inline)) {
#pragma unroll
    for (int f = 0; f < 12; ++f) x.p[f] = __builtin_bit_cast(bf16x8, ld16(r.p, vo_f, f * 1024));
  };
  auto load_k = [&](CK &x, const Rsrc &r) __attribute__((always_inline)) {
#pragma unroll
    for (int f = 0; f < kNK; ++f) x.k[f] = __builtin_bit_cast(bf16x8, ld16(r.k, vo_f, f * 1024));
  };
  auto load_gates = [&](CK &x, const Rsrc &r) __attribute__((always_inline)) {
#pragma unroll
    for (int R = 0; R < 4; ++R) {
      x.u[R] = __builtin_bit_cast(f32x4, ld16(r.u, vo_f, R * 1024));
      x.dec[R] = __builtin_bit_cast(f32x4, ld16(r.g, 4 * g4, R * 64));
      x.exs[R] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r.g, 4 * c16, 256 + R * 64, 0));
    }
    x.el = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r.g, 0, 512, 0));
  };

  // ---- state slice: S[tau] holds S[d = 16 tau + 4g + i][v0 + c] ---------------
  f32x4 S[8];
  {
    const int64_t base = (((int64_t)s * Hv + hv) * kD + v0 + c16) * kD + g4;
#pragma unroll
    for (int tau = 0; tau < 8; ++tau)
      S[tau] = h0 ? *reinterpret_cast<const f32x4 *>(h0 + base + 16 * tau) : zero4();
  }

  // Chunk 0's fragments, issued in the loop's order (the compiler's waits at
  // the loop head assume the same order on entry and on the back edge).
  CK x;
  {
    const Rsrc r = rsrc_of(0);
    __builtin_amdgcn_sched_barrier(0);
    load_w(x, r);
    __builtin_amdgcn_sched_barrier(0);
    load_q(x, r);
    __builtin_amdgcn_sched_barrier(0);
    load_gates(x, r);
    __builtin_amdgcn_sched_barrier(0);
    load_p(x, r);
    __builtin_amdgcn_sched_barrier(0);
    load_k(x, r);
    __builtin_amdgcn_sched_barrier(0);
  }
  for (int c = 0; c < nc; ++c) {
    const Rsrc rn = rsrc_of(c + 1);

    // v' = u + w (-S); then the next chunk's w
    f16x8 sn[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) sn[p] = neg_f16(S[2 * p], S[2 * p + 1]);
    f32x4 v[4] = {x.u[0], x.u[1], x.u[2], x.u[3]};
#pragma unroll
    for (int p = 0; p < 4; ++p)
#pragma unroll
      for (int R = 0; R < 4; ++R) v[R] = mfma(x.w[4 * R + p], sn[p], v[R]);
    __builtin_amdgcn_sched_barrier(0);
    load_w(x, rn);
    __builtin_amdgcn_sched_barrier(0);

    // y^T = (-S)^T q^T; then the next chunk's q16
    f32x4 ya[4] = {zero4(), zero4(), zero4(), zero4()};
#pragma unroll
    for (int p = 0; p < 4; ++p)
#pragma unroll
      for (int R = 0; R < 4; ++R) ya[R] = mfma(sn[p], x.q[4 * R + p], ya[R]);
    __builtin_amdgcn_sched_barrier(0);
    load_q(x, rn);
    __builtin_amdgcn_sched_barrier(0);

    // v' and the decayed v' as hi + lo; pa^T = v'^T P^T
    bf16x8 dh[2], dl[2], eh[2], elo[2];
    split8(v[0], v[1], dh[0], dl[0]);
    split8(v[2], v[3], dh[1], dl[1]);
    split8(v[0] * x.dec[0], v[1] * x.dec[1], eh[0], elo[0]);
    split8(v[2] * x.dec[2], v[3] * x.dec[3], eh[1], elo[1]);
    float exs[4] = {x.exs[0], x.exs[1], x.exs[2], x.exs[3]};
    const float el = x.el;
    __builtin_amdgcn_sched_barrier(0);
    load_gates(x, rn);
    __builtin_amdgcn_sched_barrier(0);
    f32x4 pa[4] = {zero4(), zero4(), zero4(), zero4()};
#pragma unroll
    for (int R = 0; R < 4; ++R) {
#pragma unroll
      for (int q = 0; q <= (R >> 1); ++q) {
        const int pi = R < 2 ? R : 2 * R - 2 + q;
        pa[R] = mfma(dh[q], x.p[2 * pi], pa[R]);
        pa[R] = mfma(dl[q], x.p[2 * pi], pa[R]);
        pa[R] = mfma(dh[q], x.p[2 * pi + 1], pa[R]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    load_p(x, rn);
    {
      // o^T = scale e^gamma S^T q^T + v'^T P^T
      const int t0 = bos + kC * c;
      const uint32_t lc = static_cast<uint32_t>(min(kC, eos - t0));
      const i32x4 ro = rsrc_words(o + ((int64_t)t0 * Hv + hv) * kD + v0, lc * Hv * kD * 4);
#pragma unroll
      for (int R = 0; R < 4; ++R) store16(ro, vo_o, R * row_o, pa[R] - exs[R] * ya[R]);
    }
    __builtin_amdgcn_sched_barrier(0);

    // S = e^{gamma_last} S + K^T (e^{gamma_last - gamma} v'); then the next K^T
#pragma unroll
    for (int tau = 0; tau < 8; ++tau) S[tau] = S[tau] * el;
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int tau = 0; tau < 8; ++tau) {
        S[tau] = mfma(x.k[2 * tau + q], eh[q], S[tau]);
        S[tau] = mfma(x.k[2 * tau + q], elo[q], S[tau]);
        if constexpr (kF32In) S[tau] = mfma(x.k[16 + 2 * tau + q], eh[q], S[tau]);
      }
    __builtin_amdgcn_sched_barrier(0);
    load_k(x, rn);
    __builtin_amdgcn_sched_barrier(0);
  }

  if (hT) {
    const int64_t base = (((int64_t)s * Hv + hv) * kD + v0 + c16) * kD + g4;
#pragma unroll
    for (int tau = 0; tau < 8; ++tau) *reinterpret_cast<f32x4 *>(hT + base + 16 * tau) = S[tau];
  }
}

template <bool kF32In>
hipError_t launch_waves(const StageBuffers &in, const float *h0, const int32_t *cu, int32_t n_max,
                        int32_t h, int32_t hv, int32_t t_max, int32_t nt, float *o, float *hT,
                        hipStream_t stream) {
  const int members = (hv / h) * kSlices;
  const int groups = n_max * h;
  const int rounds = (groups + kXcds - 1) / kXcds;
  const dim3 grid(rounds * kXcds * members);
  hipLaunchKernelGGL((inter_kernel<kF32In>), grid, dim3(64), 0, stream, in, h0, cu, o, hT, n_max,
                     h, hv, t_max, nt);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_inter(bool f32_in, const StageBuffers &in, const float *h0,
                        const int32_t *cu_seqlens, int32_t n_max, int32_t h, int32_t hv,
                        int32_t t_max, int32_t nt_max, float *o, float *hT, hipStream_t stream) {
  return f32_in ? launch_waves<true>(in, h0, cu_seqlens, n_max, h, hv, t_max, nt_max, o, hT, stream)
                : launch_waves<false>(in, h0, cu_seqlens, n_max, h, hv, t_max, nt_max, o, hT, stream);
}

}  // namespace gdn
