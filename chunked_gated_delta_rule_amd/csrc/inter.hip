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
// tile is blocked along the value dimension to fit on chip). One work-group of
// four wave64s owns a 128 x 16 column slice of S for the whole sequence. Every
// product of the chunk step is arranged so that its operands come either from
// MFMA accumulators directly or from fragments the intra stage stored in MFMA
// order:
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
// K^T and P in that order, so no value moves between lanes inside a product.
//
// The four waves run on the four SIMDs of one CU:
//   chain waves 0 and 1: wave X keeps key rows 64 X .. 64 X + 63 of the slice
//       in registers (four 16 x 16 fp32 accumulators). Per chunk it forms its
//       partial (-w) S over those rows (wave 0 starts from u), publishes the
//       partial and its fp16 rows of S in LDS, and after the chunk's barrier
//       adds the other wave's partial to get v', then applies the state update
//       to its own rows. The chunk-to-chunk chain therefore runs half the
//       products of the step on each of two SIMDs.
//   helper waves 2 and 3: after the barrier, helper Y reads S (fp16) and both
//       partials of the chunk and writes output rows 32 Y .. 32 Y + 31:
//       y = S^T q^T and o = P v' + scale e^gamma y.
// One barrier per chunk; the exchange is double-buffered (12 KB per chunk),
// so the chain waves run ahead while the helpers finish the previous chunk.
// Every operand fragment is one 1 KB block (16 bytes per lane) loaded straight
// into registers; past the last chunk the buffer range is empty and loads
// return zero. Fragments are prefetched two chunks ahead.
// Between them the four waves load each operand once per chunk.
//
// Work-group numbering is XCD-aware: all work-groups of the value heads that
// share a key head get the same blockIdx modulo 8, so they run on one XCD and
// share q16 and K^T through its L2.
#include <type_traits>
#include <utility>

#include "gdn_common.hpp"
#include "gdn_launch.hpp"

namespace gdn {

namespace {

constexpr int kXcds = 8;
constexpr int kSlices = kD / 16;  // 16-column value slices per head
constexpr int kDepthSingle = 2;  // prefetch depth with one work-group per CU
constexpr int kL2Lead = 2;       // chunks between the L2 warm-up and the operand loads

// The L2 warm-up wave is a fifth wave of the work-group; fp32 input at depth 2
// needs more than the 256 VGPRs a SIMD with two waves of it could give, and
// runs without it.
template <bool kF32In, int kDepth>
constexpr bool kWarmWave = !(kF32In && kDepth == 2);
template <bool kF32In, int kDepth>
constexpr int kInterThreads = kWarmWave<kF32In, kDepth> ? 320 : 256;

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

// Chunk hand-off buffer: [2 buffers][12 fragments][64 lanes] x 16 bytes.
//   fragments 0..3 : S as fp16, contraction block p (key rows 32 p ..)
//   fragments 4..7 : chain wave 0's partial v' (u + (-w) S over rows 0..63), tile R
//   fragments 8..11: chain wave 1's partial (-w) S over rows 64..127, tile R
constexpr int kXchFrags = 12;

struct Lane {
  int s, h, hv, v0, lane, c16, g4, bos, eos, nc, H, Hv, t_max, nt;
};

// Per-chunk slot of a sequence's chunk c (chunks of one batch never share one).
__device__ __forceinline__ int slot_of(const Lane &L, int c) { return ((L.bos + kC * c) >> 6) + L.s; }

// Both kinds of wave keep kDepth sets of operand fragments (set B serves
// chunks c with c % kDepth == B) and walk the chunks in groups of kDepth: each
// array of the current set is refilled with chunk c + kDepth's fragments as
// soon as chunk c has consumed it, so every load has about kDepth chunk steps
// to arrive. With one work-group per CU (single-sequence prefill) the load
// latency of a busy CU needs kDepth = 2; when the grid has more work-groups
// than CUs, kDepth = 1 keeps two work-groups resident per CU instead and
// their interleaving hides the latency. The sets are plain register arrays
// indexed by a compile-time set number, and every value is consumed before
// its refill is issued, so each refill lands in the registers it replaces and
// the compiler's load counting never has to drain.
template <int B>
using SetIndex = std::integral_constant<int, B>;

// f(SetIndex<0>{}), f(SetIndex<1>{}), ..., f(SetIndex<kDepth - 1>{}) in order.
template <int kDepth, typename F, int... B>
__device__ __forceinline__ void for_sets_impl(F &&f, std::integer_sequence<int, B...>) {
  (f(SetIndex<B>{}), ...);
}
template <int kDepth, typename F>
__device__ __forceinline__ void for_sets(F &&f) {
  for_sets_impl<kDepth>(f, std::make_integer_sequence<int, kDepth>{});
}

template <bool kF32In, int kDepth, int X>
__device__ __forceinline__ void chain_wave(const Lane &L, const StageBuffers &in,
                                           const float *__restrict__ h0, float *__restrict__ hT,
                                           u32x4 (*xch)[kXchFrags][64]) {
  constexpr int kNKw = kF32In ? 16 : 8;  // K^T fragments this wave uses per chunk
  const uint32_t vo_f = static_cast<uint32_t>(L.lane) * 16;  // 1 KB fragment blocks
  const int slice = L.v0 / 16;
  struct Rsrc { rsrc_t w, k, u, g; };
  auto rsrc_of = [&](int c) __attribute__((always_inline)) {
    const int slot = slot_of(L, c);
    const bool ok = c < L.nc;
    Rsrc r;
    r.w = make_rsrc(in.w16 + ((int64_t)L.hv * L.nt + slot) * 16 * 512, ok ? 16 * 1024 : 0);
    r.k = make_rsrc(in.kimg + ((int64_t)L.h * L.nt + slot) * (kF32In ? 32 : 16) * 512,
                    ok ? (kF32In ? 32 : 16) * 1024 : 0);
    r.u = make_rsrc(in.uimg + (((int64_t)L.hv * L.nt + slot) * kSlices + slice) * 4 * 256,
                    ok && X == 0 ? 4096 : 0);
    r.g = make_rsrc(in.gimg + ((int64_t)L.hv * L.nt + slot) * kGateStride, ok ? kGateStride * 4 : 0);
    return r;
  };
  f16x8 w[kDepth][8];       // (-w) fragment (token tile R, key block 2 X + pl) at [2 R + pl]
  bf16x8 k[kDepth][kNKw];   // K^T fragment (key tile 4 X + tl, token block q) at [2 tl + q] (+8: lo)
  f32x4 u[kDepth][4];       // wave 0: u tile R, rows 16 R + 4 g + i, value column v0 + c
  f32x4 dec[kDepth][4];     // e^{gamma_last - gamma} of those rows
  float el[kDepth];         // e^{gamma_last}
  auto load_w = [&](auto Bc, const Rsrc &r) __attribute__((always_inline)) {
    constexpr int B = decltype(Bc)::value;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      w[B][i] = __builtin_bit_cast(f16x8, ld16(r.w, vo_f, (4 * (i >> 1) + 2 * X + (i & 1)) * 1024));
  };
  auto load_k = [&](auto Bc, const Rsrc &r) __attribute__((always_inline)) {
    constexpr int B = decltype(Bc)::value;
#pragma unroll
    for (int i = 0; i < 8; ++i) k[B][i] = __builtin_bit_cast(bf16x8, ld16(r.k, vo_f, (8 * X + i) * 1024));
    if constexpr (kF32In) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        k[B][8 + i] = __builtin_bit_cast(bf16x8, ld16(r.k, vo_f, (16 + 8 * X + i) * 1024));
    }
  };
  auto load_u = [&](auto Bc, const Rsrc &r) __attribute__((always_inline)) {
    constexpr int B = decltype(Bc)::value;
#pragma unroll
    for (int R = 0; R < 4; ++R) {
      if constexpr (X == 0) u[B][R] = __builtin_bit_cast(f32x4, ld16(r.u, vo_f, R * 1024));
      dec[B][R] = __builtin_bit_cast(f32x4, ld16(r.g, 4 * L.g4, R * 64));
    }
    el[B] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r.g, 0, 512, 0));
  };
  auto load_all = [&](auto Bc, const Rsrc &r) __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    load_w(Bc, r);
    __builtin_amdgcn_sched_barrier(0);
    load_u(Bc, r);
    __builtin_amdgcn_sched_barrier(0);
    load_k(Bc, r);
    __builtin_amdgcn_sched_barrier(0);
  };

  // state rows: S[tl] holds S[d = 64 X + 16 tl + 4 g + i][v0 + c]
  f32x4 S[4];
  const int64_t sbase = (((int64_t)L.s * L.Hv + L.hv) * kD + L.v0 + L.c16) * kD + 64 * X + L.g4;
#pragma unroll
  for (int tl = 0; tl < 4; ++tl)
    S[tl] = h0 ? *reinterpret_cast<const f32x4 *>(h0 + sbase + 16 * tl) : zero4();

  // One chunk step on set B, which is refilled with chunk c + kDepth. A step
  // past the last chunk (c >= nc) runs on zero fragments with a decay of 1
  // and leaves S unchanged.
  auto step = [&](const int c, auto Bc) __attribute__((always_inline)) {
    constexpr int B = decltype(Bc)::value;
    const Rsrc rn = rsrc_of(c + kDepth);
    const float e_last = c < L.nc ? el[B] : 1.f;
    u32x4 *xb = &xch[c & 1][0][L.lane];
    f16x8 s16[2];
#pragma unroll
    for (int pl = 0; pl < 2; ++pl) {
      s16[pl] = to_f16x8(S[2 * pl], S[2 * pl + 1]);
      xb[64 * (2 * X + pl)] = __builtin_bit_cast(u32x4, s16[pl]);
    }
    // partial v' over this wave's key rows (wave 0 starts from u)
    f32x4 pv[4];
#pragma unroll
    for (int R = 0; R < 4; ++R) pv[R] = X == 0 ? u[B][R] : zero4();
#pragma unroll
    for (int pl = 0; pl < 2; ++pl)
#pragma unroll
      for (int R = 0; R < 4; ++R) pv[R] = mfma(w[B][2 * R + pl], s16[pl], pv[R]);
#pragma unroll
    for (int R = 0; R < 4; ++R) xb[64 * (4 + 4 * X + R)] = __builtin_bit_cast(u32x4, pv[R]);
#pragma unroll
    for (int tl = 0; tl < 4; ++tl) S[tl] = S[tl] * e_last;
    __builtin_amdgcn_sched_barrier(0);
    load_w(Bc, rn);
    __builtin_amdgcn_sched_barrier(0);
    lds_barrier();  // chunk c's S (fp16) and both partials are published
    f32x4 v[4];
#pragma unroll
    for (int R = 0; R < 4; ++R) {
      const f32x4 other = __builtin_bit_cast(f32x4, xb[64 * (4 + 4 * (1 - X) + R)]);
      v[R] = X == 0 ? pv[R] + other : other + pv[R];  // both waves: partial0 + partial1
    }
    // S += K^T (e^{gamma_last - gamma} v')
    bf16x8 eh[2], elo[2];
    split8(v[0] * dec[B][0], v[1] * dec[B][1], eh[0], elo[0]);
    split8(v[2] * dec[B][2], v[3] * dec[B][3], eh[1], elo[1]);
    __builtin_amdgcn_sched_barrier(0);
    load_u(Bc, rn);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
#pragma unroll
      for (int tl = 0; tl < 4; ++tl) S[tl] = mfma(k[B][2 * tl + q], eh[q], S[tl]);
#pragma unroll
      for (int tl = 0; tl < 4; ++tl) S[tl] = mfma(k[B][2 * tl + q], elo[q], S[tl]);
      if constexpr (kF32In) {
#pragma unroll
        for (int tl = 0; tl < 4; ++tl) S[tl] = mfma(k[B][8 + 2 * tl + q], eh[q], S[tl]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    load_k(Bc, rn);
    __builtin_amdgcn_sched_barrier(0);
  };

  for_sets<kDepth>([&](auto Bc) __attribute__((always_inline)) {
    load_all(Bc, rsrc_of(decltype(Bc)::value));
  });
  for (int c = 0; c < L.nc; c += kDepth)  // a step past the last chunk changes nothing
    for_sets<kDepth>([&](auto Bc) __attribute__((always_inline)) {
      step(c + decltype(Bc)::value, Bc);
    });
  if (hT) {
#pragma unroll
    for (int tl = 0; tl < 4; ++tl) *reinterpret_cast<f32x4 *>(hT + sbase + 16 * tl) = S[tl];
  }
}

// Helper wave Y: output token tiles R = 2 Y, 2 Y + 1 (rows 32 Y .. 32 Y + 31).
template <int kDepth, int Y>
__device__ __forceinline__ void helper_wave(const Lane &L, const StageBuffers &in,
                                            float *__restrict__ o, u32x4 (*xch)[kXchFrags][64]) {
  constexpr int kNQ = Y + 1;                 // token blocks of v' this wave contracts over
  constexpr int kPairs = Y == 0 ? 2 : 4;     // P pairs of its tiles
  constexpr int kPair0 = Y == 0 ? 0 : 2;
  const uint32_t vo_o = static_cast<uint32_t>(L.c16 * L.Hv * kD + L.g4) * 4;     // o rows
  const uint32_t vo_f = static_cast<uint32_t>(L.lane) * 16;
  const uint32_t row_o = static_cast<uint32_t>(16 * L.Hv * kD * 4);             // 16 o rows
  struct Rsrc { rsrc_t q, p, g; };
  auto rsrc_of = [&](int c) __attribute__((always_inline)) {
    const int slot = slot_of(L, c);
    const bool ok = c < L.nc;
    Rsrc r;
    r.q = make_rsrc(in.q16 + ((int64_t)L.h * L.nt + slot) * 16 * 512, ok ? 16 * 1024 : 0);
    r.p = make_rsrc(in.pimg + ((int64_t)L.hv * L.nt + slot) * 12 * 512, ok ? 12 * 1024 : 0);
    r.g = make_rsrc(in.gimg + ((int64_t)L.hv * L.nt + slot) * kGateStride, ok ? kGateStride * 4 : 0);
    return r;
  };
  f16x8 qf[kDepth][8];            // q16 fragment (token tile 2 Y + Rl, key block p) at [4 Rl + p]
  bf16x8 pf[kDepth][2 * kPairs];  // P pair kPair0 + n, term t at [2 n + t]
  u32x2 exs[kDepth];              // scale * e^{gamma_r} (fp32 bits), r = 16 (2 Y + Rl) + c
  auto load_q = [&](auto Bc, const Rsrc &r) __attribute__((always_inline)) {
    constexpr int B = decltype(Bc)::value;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      qf[B][i] = __builtin_bit_cast(f16x8, ld16(r.q, vo_f, (4 * (2 * Y + (i >> 2)) + (i & 3)) * 1024));
  };
  auto load_p = [&](auto Bc, const Rsrc &r) __attribute__((always_inline)) {
    constexpr int B = decltype(Bc)::value;
#pragma unroll
    for (int i = 0; i < 2 * kPairs; ++i)
      pf[B][i] = __builtin_bit_cast(bf16x8, ld16(r.p, vo_f, (2 * kPair0 + i) * 1024));
    exs[B] = __builtin_amdgcn_raw_buffer_load_b64(r.g, 16 * L.c16 + 8 * Y, 256, 0);
  };
  auto load_all = [&](auto Bc, const Rsrc &r) __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    load_q(Bc, r);
    __builtin_amdgcn_sched_barrier(0);
    load_p(Bc, r);
    __builtin_amdgcn_sched_barrier(0);
  };
  auto step = [&](const int c, auto Bc) __attribute__((always_inline)) {
    constexpr int B = decltype(Bc)::value;
    const Rsrc rn = rsrc_of(c + kDepth);
    lds_barrier();  // chunk c handed over
    const u32x4 *xb = &xch[c & 1][0][L.lane];
    f16x8 s16[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) s16[p] = __builtin_bit_cast(f16x8, xb[64 * p]);
    f32x4 v[2 * kNQ];
#pragma unroll
    for (int R = 0; R < 2 * kNQ; ++R)
      v[R] = __builtin_bit_cast(f32x4, xb[64 * (4 + R)]) + __builtin_bit_cast(f32x4, xb[64 * (8 + R)]);
    // y^T = S^T q^T for this wave's two token tiles
    f32x4 ya[2] = {zero4(), zero4()};
#pragma unroll
    for (int p = 0; p < 4; ++p)
#pragma unroll
      for (int Rl = 0; Rl < 2; ++Rl) ya[Rl] = mfma(s16[p], qf[B][4 * Rl + p], ya[Rl]);
    bf16x8 dh[kNQ], dl[kNQ];
#pragma unroll
    for (int q = 0; q < kNQ; ++q) split8(v[2 * q], v[2 * q + 1], dh[q], dl[q]);
    __builtin_amdgcn_sched_barrier(0);
    load_q(Bc, rn);
    __builtin_amdgcn_sched_barrier(0);
    // o^T = v'^T P^T + scale e^gamma y^T
    f32x4 pa[2] = {zero4(), zero4()};
#pragma unroll
    for (int Rl = 0; Rl < 2; ++Rl) {
      const int R = 2 * Y + Rl;
#pragma unroll
      for (int q = 0; q <= (R >> 1); ++q) {
        const int n = (R < 2 ? R : 2 * R - 2 + q) - kPair0;
        pa[Rl] = mfma(dh[q], pf[B][2 * n], pa[Rl]);
        pa[Rl] = mfma(dl[q], pf[B][2 * n], pa[Rl]);
        pa[Rl] = mfma(dh[q], pf[B][2 * n + 1], pa[Rl]);
      }
    }
    const int t0 = L.bos + kC * c;
    const uint32_t lc = c < L.nc ? static_cast<uint32_t>(min(kC, L.eos - t0)) : 0u;  // past the end: no store
    const i32x4 ro = rsrc_words(o + ((int64_t)t0 * L.Hv + L.hv) * kD + L.v0, lc * L.Hv * kD * 4);
#pragma unroll
    for (int Rl = 0; Rl < 2; ++Rl)
      store16(ro, vo_o, (2 * Y + Rl) * row_o, pa[Rl] + __uint_as_float(exs[B][Rl]) * ya[Rl]);
    __builtin_amdgcn_sched_barrier(0);
    load_p(Bc, rn);
    __builtin_amdgcn_sched_barrier(0);
  };

  for_sets<kDepth>([&](auto Bc) __attribute__((always_inline)) {
    load_all(Bc, rsrc_of(decltype(Bc)::value));
  });
  for (int c = 0; c < L.nc; c += kDepth)  // a step past the last chunk changes nothing
    for_sets<kDepth>([&](auto Bc) __attribute__((always_inline)) {
      step(c + decltype(Bc)::value, Bc);
    });
}

// L2 warm-up wave. The work-groups of one key head (and of one value head)
// read the same per-chunk blocks, at nearly the same time, from one XCD's L2;
// their first requests for a chunk would all wait on the same misses to the
// last-level cache or HBM. Per chunk step this wave requests, one 128-byte
// line per lane, this work-group's share of the lines of chunk c + kDepth +
// kL2Lead: 1/members of the key head's K^T and q16 blocks, 1/8 of the value
// head's w16, P and gate blocks, and its own u slice. The loads go to LDS
// (LDS-DMA: no register is written) and are never read, so nothing waits on
// them until the wave ends. Requests past the last chunk repeat its lines.
template <bool kF32In, int kDepth>
__device__ __forceinline__ void l2_warm_wave(const Lane &L, const StageBuffers &in, int member,
                                             int members, uint32_t *sink) {
  constexpr int kKLines = (kF32In ? 32 : 16) * 8;
  constexpr int kHLines = kKLines + 128;             // K^T image, q16
  constexpr int kWLines = 128, kPLines = 96;
  constexpr int kVLines = kWLines + kPLines + kGateStride * 4 / 128;  // w16, P, gates
  constexpr int kULines = 32;
  static_assert(kGateStride * 4 % 128 == 0, "gate block is whole lines");
  if (L.nc == 0) return;
  const int slice = L.v0 / 16;
  const int nh = (kHLines + members - 1) / members;
  const int nv = (kVLines + kSlices - 1) / kSlices;
  auto issue = [&](int c) __attribute__((always_inline)) {
    const int slot = slot_of(L, min(c, L.nc - 1));
    const uint64_t kb = reinterpret_cast<uint64_t>(in.kimg + ((int64_t)L.h * L.nt + slot) * kKLines * 64);
    const uint64_t qb = reinterpret_cast<uint64_t>(in.q16 + ((int64_t)L.h * L.nt + slot) * 16 * 512);
    const uint64_t wb = reinterpret_cast<uint64_t>(in.w16 + ((int64_t)L.hv * L.nt + slot) * 16 * 512);
    const uint64_t pb = reinterpret_cast<uint64_t>(in.pimg + ((int64_t)L.hv * L.nt + slot) * 12 * 512);
    const uint64_t gb = reinterpret_cast<uint64_t>(in.gimg + ((int64_t)L.hv * L.nt + slot) * kGateStride);
    const uint64_t ub = reinterpret_cast<uint64_t>(
        in.uimg + (((int64_t)L.hv * L.nt + slot) * kSlices + slice) * 4 * 256);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int j = L.lane + 64 * i;
      const int lh = min(member * nh + j, kHLines - 1);
      const int lv = min(slice * nv + (j - nh), kVLines - 1);
      const int lu = min(j - nh - nv, kULines - 1);
      const uint64_t ah = lh < kKLines ? kb + 128u * lh : qb + 128u * (lh - kKLines);
      const uint64_t av = lv < kWLines ? wb + 128u * lv
                          : lv < kWLines + kPLines ? pb + 128u * (lv - kWLines)
                                                   : gb + 128u * (lv - kWLines - kPLines);
      const uint64_t a = j < nh ? ah : j < nh + nv ? av : ub + 128u * max(lu, 0);
      __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void *)a,
                                       (__attribute__((address_space(3))) void *)sink, 4, 0, 0);
    }
  };
  for (int c = kDepth; c < kDepth + kL2Lead; ++c) issue(c);
  for (int c = 0; c < L.nc; c += kDepth)
    for_sets<kDepth>([&](auto Bc) __attribute__((always_inline)) {
      issue(c + decltype(Bc)::value + kDepth + kL2Lead);
      lds_barrier();
    });
  // the LDS-DMA writes must land before the work-group's LDS is released
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

template <bool kF32In, int kDepth>
__global__ __launch_bounds__((kInterThreads<kF32In, kDepth>)) void inter_kernel(StageBuffers in, const float *__restrict__ h0,
                                                              const int32_t *__restrict__ cu,
                                                              float *__restrict__ o, float *__restrict__ hT,
                                                              int n_max, int H, int Hv, int t_max, int nt) {
  __shared__ __attribute__((aligned(16))) u32x4 xch[2][kXchFrags][64];
  __shared__ uint32_t l2_sink[64];

  // ---- XCD-aware work-group -> (sequence, value head, slice) --------------
  const int HG = Hv / H;
  const int members = HG * kSlices;
  const int xcd = blockIdx.x % kXcds;
  const int wslot = blockIdx.x / kXcds;
  const int group = (wslot / members) * kXcds + xcd;  // (sequence, key head)
  const int member = wslot % members;
  if (group >= n_max * H) return;
  Lane L;
  L.s = group / H;
  L.h = group % H;
  L.hv = L.h * HG + member / kSlices;
  L.v0 = 16 * (member % kSlices);
  L.lane = threadIdx.x & 63;
  L.c16 = L.lane & 15;
  L.g4 = 4 * (L.lane >> 4);
  L.bos = cu[L.s];
  L.eos = cu[L.s + 1];
  L.nc = (L.eos - L.bos + kC - 1) / kC;
  L.H = H;
  L.Hv = Hv;
  L.t_max = t_max;
  L.nt = nt;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (wave == 0)
    chain_wave<kF32In, kDepth, 0>(L, in, h0, hT, xch);
  else if (wave == 1)
    chain_wave<kF32In, kDepth, 1>(L, in, h0, hT, xch);
  else if (wave == 2)
    helper_wave<kDepth, 0>(L, in, o, xch);
  else if (wave == 3)
    helper_wave<kDepth, 1>(L, in, o, xch);
  else if constexpr (kWarmWave<kF32In, kDepth>)
    l2_warm_wave<kF32In, kDepth>(L, in, member, members, l2_sink);
}

// Compute units of the current device (queried once per device).
int cu_count() {
  static int counts[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (counts[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    counts[dev] = n;
  }
  return counts[dev];
}

template <bool kF32In>
hipError_t launch_waves(const StageBuffers &in, const float *h0, const int32_t *cu, int32_t n_max,
                        int32_t h, int32_t hv, int32_t t_max, int32_t nt, float *o, float *hT,
                        hipStream_t stream, KernelEvents ev) {
  const int members = (hv / h) * kSlices;
  const int groups = n_max * h;
  const int rounds = (groups + kXcds - 1) / kXcds;
  const dim3 grid(rounds * kXcds * members);
  if (static_cast<int>(grid.x) <= cu_count())
    hipExtLaunchKernelGGL((inter_kernel<kF32In, kDepthSingle>), grid,
                          dim3(kInterThreads<kF32In, kDepthSingle>), 0, stream, ev.start,
                          ev.stop, 0, in, h0, cu, o, hT, n_max, h, hv, t_max, nt);
  else
    hipExtLaunchKernelGGL((inter_kernel<kF32In, 1>), grid, dim3(kInterThreads<kF32In, 1>), 0, stream, ev.start,
                          ev.stop, 0, in, h0, cu, o, hT, n_max, h, hv, t_max, nt);
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
