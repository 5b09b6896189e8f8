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
// four wave64s owns a 128 x 16 column slice of S (one column tile), or a
// 128 x 32 or 128 x 64 slice (two or four tiles), for the whole sequence. Every
// product of the chunk step is arranged so that its operands come either from
// MFMA accumulators directly or from fragments the intra stage stored in MFMA
// order:
//
//   v'      = u + (-w) S          A = -w fragment, B = S (fp16)      C = v' tiles
//   o^T     = S^T q^T             A = S (fp16),   B = q16 fragment   C = o^T tiles
//   o^T    += v'^T P^T            A = v' (fp16 hi+lo), B = P fragment (fp16)
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
// One barrier per chunk; the exchange is double-buffered (12 KB per chunk and
// column tile), so the chain waves run ahead while the helpers finish the
// previous chunk. Every operand fragment is one block loaded straight into
// registers, 16 bytes per lane (u: four 24-bit floats in 12; the two
// half-zero pairs of P: 8); past the last chunk the buffer range is empty and
// loads return zero. Between them the four waves load each operand once per
// chunk.
//
// A segmented walk (a later segment of a long sequence, carrying the state
// from zero and the homogeneous state from the identity) adds a second pair
// of chain waves for the homogeneous state. It runs one chunk behind and
// takes w, K^T and the gate factors from LDS copies the first pair leaves,
// so the work-group still loads each operand once; the helper waves write
// both states' outputs.
//
// Three launch shapes (the caller's choice, or automatic by grid size and
// tokens per sequence). When the grid of one-tile work-groups fits the device
// (one per CU), fragments are prefetched two chunks ahead and a fifth wave
// warms the L2. Larger grids use two or four column tiles per work-group: w,
// K^T, q16 and P are then loaded once for all its columns (for two tiles 64 KB
// per chunk instead of 2 x 61 KB), every product is done once per tile in the
// same order as for one tile (so the results are bitwise those of the
// one-tile shape), and fragments are prefetched one chunk ahead. Two-tile
// work-groups stay resident two per CU, which hides the start and end of
// short walks; four-tile ones run one per CU and load least per column, which
// pays on long walks.
//
// Work-group numbering is XCD-aware: all work-groups of the value heads that
// share a key head get the same blockIdx modulo 8, so they run on one XCD and
// share q16 and K^T through its L2. Sequences are numbered by the rank stage 1
// gives them (longest first) when it ranks the batch, so the longest walks
// start first. o rows of the one-tile, one-piece walk are stored streaming
// (non-temporal).
#include <atomic>
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
// runs without it. Work-groups of two column tiles (kNV = 2) run two per CU
// with four waves each, within 256 VGPRs, and have no warm-up wave either;
// four tiles (kNV = 4) run one per CU with four waves of up to 512 registers.
template <bool kF32In, int kDepth, int kS, int kNV>
constexpr bool kWarmWave = kNV == 1 && !(kF32In && kDepth == 2) && (kS == 1 || kDepth == 1);
constexpr int kDepthSeg = 1;  // prefetch depth of the two-state walk (keeps the warm-up wave;
                              // depth 2 measured the same)

// Segments of a sequence of nc chunks walked in P parts at once. Segment 0
// (from h0, one state) takes the first nc - (P - 1) y chunks; each later
// segment carries two states (a chunk step about 1.25 times as long, and
// rows for the fix-up) and takes y = floor(4 nc / (4 P + 1)) chunks, so
// segment 0 gets about 1.25 times as many (T = 32768, H = Hv = 16, two
// parts: ratios 1, 1.25 and 1.5 gave stage 2 484, 438 and 444 us).
__host__ __device__ constexpr int seg_len(int nc, int parts) { return nc * 4 / (4 * parts + 1); }
// first chunk of segment r (r = parts: the end of the sequence)
__host__ __device__ constexpr int seg_begin(int nc, int parts, int r) {
  return r == 0 ? 0 : nc - (parts - r) * seg_len(nc, parts);
}
// The two-state walk carries each state on its own pair of chain waves.
template <bool kF32In, int kDepth, int kS, int kNV>
constexpr int kInterThreads = 64 * (2 * kS + 2 + (kWarmWave<kF32In, kDepth, kS, kNV> ? 1 : 0));
// waves per SIMD the register allocation must leave room for
template <int kNV>
constexpr int kInterWavesPerSimd = kNV == 2 ? 2 : 1;

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

// Two stacked accumulators -> fp16 hi + lo fragments (x = hi + lo to about
// 22 significant bits; hi rounded to nearest even).
__device__ __forceinline__ void split8_f16(const f32x4 &a, const f32x4 &b, f16x8 &hi, f16x8 &lo) {
  const float x[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  f16x8 h, l;
#pragma unroll
  for (int i = 0; i < 8; i += 2) {
    const f16x2 p = __builtin_convertvector(f32x2{x[i], x[i + 1]}, f16x2);
    const f32x2 back = __builtin_convertvector(p, f32x2);
    const f16x2 r = __builtin_convertvector(f32x2{x[i] - back[0], x[i + 1] - back[1]}, f16x2);
    h[i] = p[0];
    h[i + 1] = p[1];
    l[i] = r[0];
    l[i + 1] = r[1];
  }
  hi = h;
  lo = l;
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
// written just before. kStream marks the store non-temporal (streamed through
// the caches), for output that nothing reads back soon.
template <bool kStream>
__device__ __forceinline__ void store16(const i32x4 &r, uint32_t voff, uint32_t soff, const f32x4 &v) {
  if constexpr (kStream)
    asm volatile("s_nop 4\n\tbuffer_store_dwordx4 %0, %1, %2, %3 offen nt"
                 :
                 : "v"(v), "v"(voff), "s"(r), "s"(soff)
                 : "memory");
  else
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

// What one work-group walks: chunks [c0, c1) of its sequence, carrying kS
// states of its column slice. State 0 takes u and starts from init0
// (value-major [dv][dk] states of this head, or zero when null); state 1,
// when carried, takes no u and starts from the identity (the homogeneous
// part of the recurrence). out[st]: where state st's output rows go; fin[st]:
// where its final slice goes (state 0 value-major like hT, state 1 key-major
// [dk][dv]); a null pointer is not written.
struct Walk {
  int c0, c1;
  const float *init0;
  float *out[2];
  float *fin[2];
  bool two;  // state 1 is carried (a later segment of a segmented walk)
};

// LDS copies the zero-start state's chain waves leave for the identity-start
// state's in a two-state walk: w and K^T fragments of two chunks (by chunk
// parity) and e^{gamma_last} of three (chunk modulo 3, like the gate factors).
template <bool kF32In>
struct HomShare {
  u32x4 (*w)[16][64];
  u32x4 (*k)[kF32In ? 32 : 16][64];
  float *el;
};

// Chain wave X of the zero-start state (the one that takes u). In a two-state
// walk (kS = 2) it also leaves each chunk's w and K^T fragments, gate factors
// and e^{gamma_last} in LDS for the identity-start state's chain waves, which
// run a chunk behind, and takes one step more than the chunks.
template <bool kF32In, int kDepth, int X, int kS, int kNV, bool kGq>
__device__ __forceinline__ void chain_wave(const Lane &L, const Walk &W, const StageBuffers &in,
                                           u32x4 (*xch)[kXchFrags * kS * kNV][64],
                                           float (*decx)[kGq ? kNV : 1][64],
                                           const HomShare<kF32In> &sh) {
  static_assert(kS == 1 || kNV == 1, "the two-state walk covers one column tile");
  constexpr int kNKw = kF32In ? 16 : 8;  // K^T fragments this wave uses per chunk
  constexpr int kNW = kGq ? kNV : 1;     // value heads whose w, u and gates are loaded
  // distance between tile ct's rows of a state (the next value head, or the
  // next 16 columns of one)
  constexpr int64_t kCtState = kGq ? kD * kD : 16 * kD;
  const uint32_t vo_f = static_cast<uint32_t>(L.lane) * 16;  // 1 KB fragment blocks
  const int slice = L.v0 / 16;
  struct Rsrc { rsrc_t w[kNW], k, u[kNW], g[kNW]; };
  auto rsrc_of = [&](int c) __attribute__((always_inline)) {
    const int slot = slot_of(L, c);
    const bool ok = c < W.c1;
    Rsrc r;
#pragma unroll
    for (int j = 0; j < kNW; ++j) {
      const int64_t hvj = L.hv + j;
      r.w[j] = make_rsrc(in.w16 + (hvj * L.nt + slot) * 16 * 512, ok ? 16 * 1024 : 0);
      r.u[j] = make_rsrc(in.uimg + ((hvj * L.nt + slot) * kSlices + slice) * 4 * 64 * 3,
                         ok && X == 0 ? 3072 * (kNV / kNW) : 0);
      r.g[j] = make_rsrc(in.gimg + (hvj * L.nt + slot) * kGateStride, ok ? kGateStride * 4 : 0);
    }
    r.k = make_rsrc(in.kimg + ((int64_t)L.h * L.nt + slot) * (kF32In ? 32 : 16) * 512,
                    ok ? (kF32In ? 32 : 16) * 1024 : 0);
    return r;
  };
  f16x8 w[kDepth][kNW][8];  // (-w) fragment (token tile R, key block 2 X + pl) at [2 R + pl]
  bf16x8 k[kDepth][kNKw];   // K^T fragment (key tile 4 X + tl, token block q) at [2 tl + q] (+8: lo)
  u32x3 u[kDepth][kNV][4];  // wave 0: u tile R (24-bit), rows 16 R + 4 g + i, of tile ct
  float dec[kDepth][kNW];   // e^{gamma_last - gamma} of token L.lane (shared through LDS)
  float el[kDepth][kNW];    // e^{gamma_last}
  auto load_w = [&](auto Bc, const Rsrc &r) __attribute__((always_inline)) {
    constexpr int B = decltype(Bc)::value;
#pragma unroll
    for (int j = 0; j < kNW; ++j)
#pragma unroll
      for (int i = 0; i < 8; ++i)
        w[B][j][i] =
            __builtin_bit_cast(f16x8, ld16(r.w[j], vo_f, (4 * (i >> 1) + 2 * X + (i & 1)) * 1024));
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
    if constexpr (X == 0) {
#pragma unroll
      for (int ct = 0; ct < kNV; ++ct)
#pragma unroll
        for (int R = 0; R < 4; ++R)
          u[B][ct][R] = __builtin_amdgcn_raw_buffer_load_b96(r.u[kGq ? ct : 0], L.lane * 12,
                                                             (kGq ? R : 4 * ct + R) * 768, 0);
    }
#pragma unroll
    for (int j = 0; j < kNW; ++j) {
      dec[B][j] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r.g[j], 4 * L.lane, 0, 0));
      el[B][j] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r.g[j], 0, 512, 0));
    }
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

  // state rows: S[st][ct][tl] holds S[d = 64 X + 16 tl + 4 g + i][v0 + 16 ct + c]
  // state rows: S[ct][tl] holds S[d = 64 X + 16 tl + 4 g + i][v0 + 16 ct + c]
  f32x4 S[kNV][4];
  const int64_t sbase = (((int64_t)L.s * L.Hv + L.hv) * kD + L.v0 + L.c16) * kD + 64 * X + L.g4;
#pragma unroll
  for (int ct = 0; ct < kNV; ++ct)
#pragma unroll
    for (int tl = 0; tl < 4; ++tl)
      S[ct][tl] = W.init0 ? *reinterpret_cast<const f32x4 *>(W.init0 + sbase + ct * kCtState + 16 * tl)
                          : zero4();

  // One chunk step on set B, which is refilled with chunk c + kDepth. A step
  // past the last chunk (c >= c1) runs on zero fragments with a decay of 1
  // and leaves the states unchanged.
  auto step = [&](const int c, auto Bc) __attribute__((always_inline)) {
    constexpr int B = decltype(Bc)::value;
    const Rsrc rn = rsrc_of(c + kDepth);
    float e_last[kNW];
#pragma unroll
    for (int j = 0; j < kNW; ++j) e_last[j] = c < W.c1 ? el[B][j] : 1.f;
    u32x4 *xb = &xch[c & 1][0][L.lane];
    const int ds = kS == 2 ? c % 3 : c & 1;  // gate-factor buffer of chunk c
    f32x4 pv[kNV][4];
#pragma unroll
    for (int ct = 0; ct < kNV; ++ct) {
      const int wj = kGq ? ct : 0;
      u32x4 *xs = xb + 64 * kXchFrags * ct;
      f16x8 s16[2];
#pragma unroll
      for (int pl = 0; pl < 2; ++pl) {
        s16[pl] = to_f16x8(S[ct][2 * pl], S[ct][2 * pl + 1]);
        xs[64 * (2 * X + pl)] = __builtin_bit_cast(u32x4, s16[pl]);
      }
      // partial v' over this wave's key rows (wave 0 starts from u)
#pragma unroll
      for (int R = 0; R < 4; ++R) pv[ct][R] = X == 0 ? unpack_f24x4(u[B][ct][R]) : zero4();
#pragma unroll
      for (int pl = 0; pl < 2; ++pl)
#pragma unroll
        for (int R = 0; R < 4; ++R) pv[ct][R] = mfma(w[B][wj][2 * R + pl], s16[pl], pv[ct][R]);
#pragma unroll
      for (int R = 0; R < 4; ++R) xs[64 * (4 + 4 * X + R)] = __builtin_bit_cast(u32x4, pv[ct][R]);
#pragma unroll
      for (int tl = 0; tl < 4; ++tl) S[ct][tl] = S[ct][tl] * e_last[wj];
    }
    if constexpr (X == 0) {
#pragma unroll
      for (int j = 0; j < kNW; ++j) decx[ds][j][L.lane] = dec[B][j];  // token L.lane's factor
      if constexpr (kS == 2) {
        if (L.lane == 0) sh.el[ds] = el[B][0];
      }
    }
    if constexpr (kS == 2) {
      if (W.two) {
#pragma unroll
        for (int i = 0; i < 8; ++i) sh.w[c & 1][8 * X + i][L.lane] = __builtin_bit_cast(u32x4, w[B][0][i]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    load_w(Bc, rn);
    __builtin_amdgcn_sched_barrier(0);
    lds_barrier();  // chunk c's states (fp16) and all partials are published
    __builtin_amdgcn_sched_barrier(0);
    load_u(Bc, rn);
    __builtin_amdgcn_sched_barrier(0);
    // S += K^T (e^{gamma_last - gamma} v'): rows 16 R + 4 g + i of this lane
    // take their factors from the chunk's gate factors that wave 0 put in LDS
    // before the barrier (one broadcast 16-byte read per token tile)
    f32x4 dr[kNW][4];
#pragma unroll
    for (int j = 0; j < kNW; ++j)
#pragma unroll
      for (int R = 0; R < 4; ++R)
        dr[j][R] = *reinterpret_cast<const f32x4 *>(&decx[ds][j][16 * R + L.g4]);
    // per token block q: form dec v' of its two token tiles, then apply them
    // (the per-accumulator order of the products is q = 0 then q = 1)
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      bf16x8 eh[kNV], elo[kNV];
#pragma unroll
      for (int ct = 0; ct < kNV; ++ct) {
        const int wj = kGq ? ct : 0;
        const u32x4 *xs = xb + 64 * kXchFrags * ct;
        f32x4 v[2];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const int R = 2 * q + h2;
          const f32x4 other = __builtin_bit_cast(f32x4, xs[64 * (4 + 4 * (1 - X) + R)]);
          // both waves: partial0 + partial1
          v[h2] = X == 0 ? pv[ct][R] + other : other + pv[ct][R];
        }
        split8(v[0] * dr[wj][2 * q], v[1] * dr[wj][2 * q + 1], eh[ct], elo[ct]);
      }
#pragma unroll
      for (int ct = 0; ct < kNV; ++ct) {
#pragma unroll
        for (int tl = 0; tl < 4; ++tl) S[ct][tl] = mfma(k[B][2 * tl + q], eh[ct], S[ct][tl]);
#pragma unroll
        for (int tl = 0; tl < 4; ++tl) S[ct][tl] = mfma(k[B][2 * tl + q], elo[ct], S[ct][tl]);
        if constexpr (kF32In) {
#pragma unroll
          for (int tl = 0; tl < 4; ++tl) S[ct][tl] = mfma(k[B][8 + 2 * tl + q], eh[ct], S[ct][tl]);
        }
      }
    }
    if constexpr (kS == 2) {
      if (W.two) {
#pragma unroll
        for (int i = 0; i < kNKw; ++i) sh.k[c & 1][kNKw * X + i][L.lane] = __builtin_bit_cast(u32x4, k[B][i]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    load_k(Bc, rn);
    __builtin_amdgcn_sched_barrier(0);
  };

  for_sets<kDepth>([&](auto Bc) __attribute__((always_inline)) {
    load_all(Bc, rsrc_of(W.c0 + decltype(Bc)::value));
  });
  if constexpr (kS == 2) {
    // one step past the last chunk (it changes nothing here) closes the
    // lagging chain's last chunk
    const int c_end = W.c1 + (W.two ? 1 : 0);
    for (int c = W.c0; c < c_end; c += kDepth)
      for_sets<kDepth>([&](auto Bc) __attribute__((always_inline)) {
        step(c + decltype(Bc)::value, Bc);
      });
  } else {
    for (int c = W.c0; c < W.c1; c += kDepth)  // a step past the last chunk changes nothing
      for_sets<kDepth>([&](auto Bc) __attribute__((always_inline)) {
        step(c + decltype(Bc)::value, Bc);
      });
  }
  if (W.fin[0]) {
#pragma unroll
    for (int ct = 0; ct < kNV; ++ct)
#pragma unroll
      for (int tl = 0; tl < 4; ++tl)
        *reinterpret_cast<f32x4 *>(W.fin[0] + sbase + ct * kCtState + 16 * tl) = S[ct][tl];
  }
}

// Chain wave X of the identity-start (homogeneous) state of a later segment.
// It runs one chunk behind the zero-start state's chain waves and takes w,
// K^T, the gate factors and e^{gamma_last} of each chunk from the LDS copies
// they leave, so the work-group loads every operand once. Per step c it forms
// chunk c - 1's partial (-w) Phi over its key rows before the step's barrier
// and applies chunk c - 1's update after it; the exchange is that of the
// one-state chain (its own double-buffered block).
template <bool kF32In, int X>
__device__ __forceinline__ void hom_chain_wave(const Lane &L, const Walk &W,
                                               u32x4 (*xch)[kXchFrags * 2][64],
                                               float (*decx)[1][64], const HomShare<kF32In> &sh) {
  constexpr int kNKw = kF32In ? 16 : 8;
  if (!W.two) {  // segment 0 carries no homogeneous state: keep the barrier count
    for (int c = W.c0; c < W.c1; ++c) lds_barrier();
    return;
  }
  // rows d = 64 X + 16 tl + 4 g + i of the identity's columns v0 + c
  f32x4 S[4];
#pragma unroll
  for (int tl = 0; tl < 4; ++tl)
#pragma unroll
    for (int i = 0; i < 4; ++i) S[tl][i] = 64 * X + 16 * tl + L.g4 + i == L.v0 + L.c16 ? 1.f : 0.f;
  for (int c = W.c0; c <= W.c1; ++c) {
    const int p = c - 1;  // the chunk of this step
    const bool live = p >= W.c0;
    u32x4 *xs = &xch[p & 1][kXchFrags][L.lane];
    f32x4 pv[4];
    if (live) {
      f16x8 s16[2];
#pragma unroll
      for (int pl = 0; pl < 2; ++pl) {
        s16[pl] = to_f16x8(S[2 * pl], S[2 * pl + 1]);
        xs[64 * (2 * X + pl)] = __builtin_bit_cast(u32x4, s16[pl]);
      }
      const u32x4 *wf = &sh.w[p & 1][8 * X][L.lane];
#pragma unroll
      for (int R = 0; R < 4; ++R) pv[R] = zero4();
#pragma unroll
      for (int pl = 0; pl < 2; ++pl)
#pragma unroll
        for (int R = 0; R < 4; ++R)
          pv[R] = mfma(__builtin_bit_cast(f16x8, wf[64 * (2 * R + pl)]), s16[pl], pv[R]);
#pragma unroll
      for (int R = 0; R < 4; ++R) xs[64 * (4 + 4 * X + R)] = __builtin_bit_cast(u32x4, pv[R]);
      const float e_last = sh.el[p % 3];
#pragma unroll
      for (int tl = 0; tl < 4; ++tl) S[tl] = S[tl] * e_last;
    }
    lds_barrier();  // chunk p's Phi rows (fp16) and partials are published
    if (live) {
      f32x4 dr[4];
#pragma unroll
      for (int R = 0; R < 4; ++R) dr[R] = *reinterpret_cast<const f32x4 *>(&decx[p % 3][0][16 * R + L.g4]);
      const u32x4 *kf = &sh.k[p & 1][kNKw * X][L.lane];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        f32x4 v[2];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const int R = 2 * q + h2;
          const f32x4 other = __builtin_bit_cast(f32x4, xs[64 * (4 + 4 * (1 - X) + R)]);
          v[h2] = X == 0 ? pv[R] + other : other + pv[R];
        }
        bf16x8 eh, elo;
        split8(v[0] * dr[2 * q], v[1] * dr[2 * q + 1], eh, elo);
#pragma unroll
        for (int tl = 0; tl < 4; ++tl)
          S[tl] = mfma(__builtin_bit_cast(bf16x8, kf[64 * (2 * tl + q)]), eh, S[tl]);
#pragma unroll
        for (int tl = 0; tl < 4; ++tl)
          S[tl] = mfma(__builtin_bit_cast(bf16x8, kf[64 * (2 * tl + q)]), elo, S[tl]);
        if constexpr (kF32In) {
#pragma unroll
          for (int tl = 0; tl < 4; ++tl)
            S[tl] = mfma(__builtin_bit_cast(bf16x8, kf[64 * (8 + 2 * tl + q)]), eh, S[tl]);
        }
      }
    }
  }
  if (W.fin[1]) {
    // key-major: row d = 64 X + 16 tl + 4 g + i, column v0 + c
    float *f = W.fin[1] + ((int64_t)L.s * L.Hv + L.hv) * kD * kD + L.v0 + L.c16;
#pragma unroll
    for (int tl = 0; tl < 4; ++tl)
#pragma unroll
      for (int i = 0; i < 4; ++i) f[(64 * X + 16 * tl + L.g4 + i) * kD] = S[tl][i];
  }
}

// Helper wave Y: output token tiles R = 2 Y, 2 Y + 1 (rows 32 Y .. 32 Y + 31)
// of every carried state. In a two-state walk step c writes chunk c of the
// zero-start state and chunk c - 1 of the identity-start one (its chain runs a
// chunk behind), with that chunk's q16, P and gate fragments kept from the
// step before.
template <int kDepth, int Y, int kS, int kNV, bool kGq>
__device__ __forceinline__ void helper_wave(const Lane &L, const Walk &W, const StageBuffers &in,
                                            u32x4 (*xch)[kXchFrags * kS * kNV][64]) {
  constexpr int kNQ = Y + 1;                 // token blocks of v' this wave contracts over
  constexpr int kNW = kGq ? kNV : 1;         // value heads whose P and gates are loaded
  constexpr int kCtO = kGq ? kD : 16;        // o columns between tile ct and ct + 1
  // o rows stream past the caches in the one-tile, one-piece walk: at one
  // work-group per CU, o's dirty lines otherwise displace what the next
  // kernels read (T = 4096: the following stage 1 ran 53 -> 44 us). Not in a
  // segmented walk (the fix-up reads o back) nor with two tiles (each store
  // covers half a 128-byte line, which then went out as partial writes).
  constexpr bool kStreamO = kS == 1 && kNV == 1;
  constexpr int kPairs = Y == 0 ? 2 : 4;     // P pairs of its tiles
  constexpr int kPair0 = Y == 0 ? 0 : 2;
  const uint32_t vo_o = static_cast<uint32_t>(L.c16 * L.Hv * kD + L.g4) * 4;     // o rows
  const uint32_t vo_f = static_cast<uint32_t>(L.lane) * 16;
  const uint32_t row_o = static_cast<uint32_t>(16 * L.Hv * kD * 4);             // 16 o rows
  struct Rsrc { rsrc_t q, p[kNW], g[kNW]; };
  auto rsrc_of = [&](int c) __attribute__((always_inline)) {
    const int slot = slot_of(L, c);
    const bool ok = c < W.c1;
    Rsrc r;
    r.q = make_rsrc(in.q16 + ((int64_t)L.h * L.nt + slot) * 16 * 512, ok ? 16 * 1024 : 0);
#pragma unroll
    for (int j = 0; j < kNW; ++j) {
      const int64_t hvj = L.hv + j;
      r.p[j] = make_rsrc(reinterpret_cast<const char *>(in.pimg) + (hvj * L.nt + slot) * kPBytes,
                         ok ? kPBytes : 0);
      r.g[j] = make_rsrc(in.gimg + (hvj * L.nt + slot) * kGateStride, ok ? kGateStride * 4 : 0);
    }
    return r;
  };
  f16x8 qf[kDepth][8];            // q16 fragment (token tile 2 Y + Rl, key block p) at [4 Rl + p]
  f16x8 pf[kDepth][kNW][kPairs];  // P pair kPair0 + n at [n]
  u32x2 exs[kDepth][kNW];         // scale * e^{gamma_r} (fp32 bits), r = 16 (2 Y + Rl) + c
  f16x8 qpv[8], ppv[kPairs];      // two states: the previous chunk's q16 and P fragments
  u32x2 epv;                      // and gate factors
  auto load_q = [&](auto Bc, const Rsrc &r) __attribute__((always_inline)) {
    constexpr int B = decltype(Bc)::value;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      qf[B][i] = __builtin_bit_cast(f16x8, ld16(r.q, vo_f, (4 * (2 * Y + (i >> 2)) + (i & 3)) * 1024));
  };
  auto load_p = [&](auto Bc, const Rsrc &r) __attribute__((always_inline)) {
    constexpr int B = decltype(Bc)::value;
#pragma unroll
    for (int j = 0; j < kNW; ++j) {
#pragma unroll
      for (int i = 0; i < kPairs; ++i) {
        const int pi = kPair0 + i, off = p_offset(pi);
        if (p_half(pi)) {  // the upper half of the lane's slots is zero
          const u32x2 h = __builtin_amdgcn_raw_buffer_load_b64(r.p[j], L.lane * 8, off, 0);
          pf[B][j][i] = __builtin_bit_cast(f16x8, u32x4{h[0], h[1], 0u, 0u});
        } else {
          pf[B][j][i] = __builtin_bit_cast(f16x8, ld16(r.p[j], vo_f, off));
        }
      }
      exs[B][j] = __builtin_amdgcn_raw_buffer_load_b64(r.g[j], 16 * L.c16 + 8 * Y, 256, 0);
    }
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
    f32x4 ya[kS][kNV][2];
    f16x8 dh[kS][kNV][kNQ], dl[kS][kNV][kNQ];
#pragma unroll
    for (int st = 0; st < kS; ++st)
#pragma unroll
      for (int ct = 0; ct < kNV; ++ct) {
        if (st == 1 && !W.two) continue;  // segment 0 carries state 0 only
        const int cs = st == 0 ? c : c - 1;  // the chunk of state st written this step
        const u32x4 *xs = &xch[cs & 1][0][L.lane] + 64 * kXchFrags * (kNV * st + ct);
        f16x8 s16[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) s16[p] = __builtin_bit_cast(f16x8, xs[64 * p]);
        f32x4 v[2 * kNQ];
#pragma unroll
        for (int R = 0; R < 2 * kNQ; ++R)
          v[R] = __builtin_bit_cast(f32x4, xs[64 * (4 + R)]) +
                 __builtin_bit_cast(f32x4, xs[64 * (8 + R)]);
        // y^T = S^T q^T for this wave's two token tiles
        ya[st][ct][0] = zero4();
        ya[st][ct][1] = zero4();
#pragma unroll
        for (int p = 0; p < 4; ++p)
#pragma unroll
          for (int Rl = 0; Rl < 2; ++Rl)
            ya[st][ct][Rl] = mfma(s16[p], st == 0 ? qf[B][4 * Rl + p] : qpv[4 * Rl + p], ya[st][ct][Rl]);
#pragma unroll
        for (int q = 0; q < kNQ; ++q) split8_f16(v[2 * q], v[2 * q + 1], dh[st][ct][q], dl[st][ct][q]);
      }
    if constexpr (kS == 2) {
      if (W.two) {
#pragma unroll
        for (int i = 0; i < 8; ++i) qpv[i] = qf[B][i];
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    load_q(Bc, rn);
    __builtin_amdgcn_sched_barrier(0);
    // o^T = v'^T P^T + scale e^gamma y^T
    const int t0c = L.bos + kC * c;
    const uint32_t lcc = c < W.c1 ? static_cast<uint32_t>(min(kC, L.eos - t0c)) : 0u;  // past the end: no store
#pragma unroll
    for (int st = 0; st < kS; ++st)
#pragma unroll
      for (int ct = 0; ct < kNV; ++ct) {
        if (st == 1 && !W.two) continue;  // segment 0 carries state 0 only
        int t0 = t0c;
        uint32_t lc = lcc;
        if constexpr (kS == 2) {
          if (st == 1) {  // chunk c - 1: no store before the segment's start
            t0 = t0c - kC;
            lc = c - 1 >= W.c0 && c - 1 < W.c1 ? static_cast<uint32_t>(min(kC, L.eos - t0)) : 0u;
          }
        }
        const int wj = kGq ? ct : 0;
        f32x4 pa[2] = {zero4(), zero4()};
#pragma unroll
        for (int Rl = 0; Rl < 2; ++Rl) {
          const int R = 2 * Y + Rl;
#pragma unroll
          for (int q = 0; q <= (R >> 1); ++q) {
            const int n = (R < 2 ? R : 2 * R - 2 + q) - kPair0;
            const f16x8 pn = st == 0 ? pf[B][wj][n] : ppv[n];
            pa[Rl] = mfma(dh[st][ct][q], pn, pa[Rl]);
            pa[Rl] = mfma(dl[st][ct][q], pn, pa[Rl]);
          }
        }
        // a state without an output destination gets an empty store range
        const uintptr_t ob = reinterpret_cast<uintptr_t>(W.out[st]) +
                             (((uintptr_t)t0 * L.Hv + L.hv) * kD + L.v0 + kCtO * ct) * 4;
        const i32x4 ro = rsrc_words(reinterpret_cast<const void *>(ob),
                                    W.out[st] ? lc * L.Hv * kD * 4 : 0u);
#pragma unroll
        for (int Rl = 0; Rl < 2; ++Rl)
          store16<kStreamO>(ro, vo_o, (2 * Y + Rl) * row_o,
                            pa[Rl] + __uint_as_float(st == 0 ? exs[B][wj][Rl] : epv[Rl]) * ya[st][ct][Rl]);
      }
    if constexpr (kS == 2) {
      if (W.two) {
#pragma unroll
        for (int i = 0; i < kPairs; ++i) ppv[i] = pf[B][0][i];
        epv = exs[B][0];
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    load_p(Bc, rn);
    __builtin_amdgcn_sched_barrier(0);
  };

  for_sets<kDepth>([&](auto Bc) __attribute__((always_inline)) {
    load_all(Bc, rsrc_of(W.c0 + decltype(Bc)::value));
  });
  if constexpr (kS == 2) {
    const int c_end = W.c1 + (W.two ? 1 : 0);  // the lagging state's last chunk
    for (int c = W.c0; c < c_end; c += kDepth)
      for_sets<kDepth>([&](auto Bc) __attribute__((always_inline)) {
        step(c + decltype(Bc)::value, Bc);
      });
  } else {
    for (int c = W.c0; c < W.c1; c += kDepth)  // a step past the last chunk changes nothing
      for_sets<kDepth>([&](auto Bc) __attribute__((always_inline)) {
        step(c + decltype(Bc)::value, Bc);
      });
  }
}

// L2 warm-up wave. The work-groups of one key head (and of one value head)
// read the same per-chunk blocks, at nearly the same time, from one XCD's L2;
// their first requests for a chunk would all wait on the same misses to the
// last-level cache or HBM. Per chunk step this wave requests, one 128-byte
// line per lane, this work-group's share of the lines of chunk c + kDepth +
// kL2Lead: 1/members of the key head's K^T and q16 blocks and, when
// warm_values is set, 1/8 of the value head's w16, P and gate blocks and its
// own u slice. The host sets warm_values when the intermediates outgrow the
// last-level cache (they then come from HBM); when they fit, the second
// request per lane cost more than it saved (T = 4096: stage 2 52.3 us with
// the key head's lines only, 54.7 us with both). The loads go to LDS
// (LDS-DMA: no register is written) and are never read, so nothing waits on
// them until the wave ends. Requests past the last chunk repeat its lines.
template <bool kF32In, int kDepth, bool kTwo>
__device__ __forceinline__ void l2_warm_wave(const Lane &L, const Walk &W, const StageBuffers &in,
                                             int member, int members, uint32_t *sink,
                                             bool warm_values) {
  constexpr int kKLines = (kF32In ? 32 : 16) * 8;
  constexpr int kHLines = kKLines + 128;             // K^T image, q16
  constexpr int kWLines = 128, kPLines = kPBytes / 128;
  constexpr int kVLines = kWLines + kPLines + kGateStride * 4 / 128;  // w16, P, gates
  constexpr int kULines = 24;  // one slice of u: 4 tiles x 768 bytes
  static_assert(kGateStride * 4 % 128 == 0, "gate block is whole lines");
  if (W.c1 <= W.c0) {  // nothing to warm; the other waves' barriers still count this wave
    if constexpr (kTwo) {
      if (W.two) lds_barrier();  // the lagging chain's closing step
    }
    return;
  }
  const int slice = L.v0 / 16;
  const int nh = (kHLines + members - 1) / members;
  const int nv = (kVLines + kSlices - 1) / kSlices;
  auto issue = [&](int c) __attribute__((always_inline)) {
    const int slot = slot_of(L, min(c, W.c1 - 1));
    const uint64_t kb = reinterpret_cast<uint64_t>(in.kimg + ((int64_t)L.h * L.nt + slot) * kKLines * 64);
    const uint64_t qb = reinterpret_cast<uint64_t>(in.q16 + ((int64_t)L.h * L.nt + slot) * 16 * 512);
    const uint64_t wb = reinterpret_cast<uint64_t>(in.w16 + ((int64_t)L.hv * L.nt + slot) * 16 * 512);
    const uint64_t pb = reinterpret_cast<uint64_t>(reinterpret_cast<const char *>(in.pimg) +
                                                   ((int64_t)L.hv * L.nt + slot) * kPBytes);
    const uint64_t gb = reinterpret_cast<uint64_t>(in.gimg + ((int64_t)L.hv * L.nt + slot) * kGateStride);
    const uint64_t ub = reinterpret_cast<uint64_t>(
        in.uimg + (((int64_t)L.hv * L.nt + slot) * kSlices + slice) * 4 * 64 * 3);
    if (!warm_values) {  // the key head's lines only: one request per lane
      const int lh = min(member * nh + min(L.lane, nh - 1), kHLines - 1);
      const uint64_t a = lh < kKLines ? kb + 128u * lh : qb + 128u * (lh - kKLines);
      __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void *)a,
                                       (__attribute__((address_space(3))) void *)sink, 4, 0, 0);
      return;
    }
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
  for (int c = W.c0 + kDepth; c < W.c0 + kDepth + kL2Lead; ++c) issue(c);
  for (int c = W.c0; c < W.c1; c += kDepth)
    for_sets<kDepth>([&](auto Bc) __attribute__((always_inline)) {
      issue(c + decltype(Bc)::value + kDepth + kL2Lead);
      lds_barrier();
    });
  if constexpr (kTwo) {
    if (W.two) lds_barrier();  // a two-state walk's extra step (nothing left to warm)
  }
  // the LDS-DMA writes must land before the work-group's LDS is released
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// With kS = 1 every work-group walks its whole sequence. With kS = 2 the grid
// is seg.parts times the one-walk grid: copy 0 walks segment 0 of each
// sequence from h0 (its final slice goes to seg.sa), copy r >= 1 walks
// segment r carrying the zero-start state (outputs into o, final slice to
// seg.z's array r - 1) and the identity-start homogeneous state (outputs to
// seg.oh, final slice to seg.phi's array r - 1); the fix-up kernels then
// combine them.
template <bool kF32In, int kDepth, int kS, int kNV, bool kGq>
__global__ __launch_bounds__((kInterThreads<kF32In, kDepth, kS, kNV>),
                             kInterWavesPerSimd<kNV>) void inter_kernel(
    StageBuffers in, const float *__restrict__ h0, const int32_t *__restrict__ cu,
    float *__restrict__ o, float *__restrict__ hT, int n_max, int H, int Hv, int t_max, int nt,
    SegScratch seg, bool warm_values) {
  __shared__ __attribute__((aligned(16))) u32x4 xch[2][kXchFrags * kS * kNV][64];
  __shared__ uint32_t l2_sink[64];
  // per chunk (double-buffered) the gate factors e^{gamma_last - gamma} by token
  // (three buffers with two states: the lagging chain reads chunk c - 1's
  // while chunk c + 1's are written)
  __shared__ __attribute__((aligned(16))) float decx[kS == 2 ? 3 : 2][kGq ? kNV : 1][64];
  // two states: the LDS copies for the identity-start state's chain
  __shared__ __attribute__((aligned(16))) u32x4 hom_w[kS == 2 ? 2 : 1][16][64];
  __shared__ __attribute__((aligned(16))) u32x4 hom_k[kS == 2 ? 2 : 1][kF32In ? 32 : 16][64];
  __shared__ float hom_el[kS == 2 ? 3 : 1];

  // ---- XCD-aware work-group -> (sequence, value head, slice) --------------
  // kGq: the kNV tiles are one 16-column slice of kNV consecutive value heads
  // of the key head; otherwise kNV consecutive slices of one value head
  constexpr int kWgSlices = kGq ? kSlices : kSlices / kNV;  // work-groups per value-head set
  const int HG = Hv / H;
  const int members = (kGq ? HG / kNV : HG) * kWgSlices;
  const int one_walk = (n_max * H + kXcds - 1) / kXcds * kXcds * members;
  const int wg = flat_block();
  const int role = kS == 2 ? wg / one_walk : 0;  // the segment walked
  if (role >= seg.parts) return;
  const int b = wg - role * one_walk;
  const int xcd = b % kXcds;
  const int wslot = b / kXcds;
  const int group = (wslot / members) * kXcds + xcd;  // (rank of the sequence, key head)
  const int member = wslot % members;
  if (group >= n_max * H) return;
  Lane L;
  // the sequence of that rank when stage 1 ranked them (longest walks first)
  L.s = in.order ? in.order[group / H] : group / H;
  if (L.s < 0 || L.s >= n_max) return;
  L.h = group % H;
  L.hv = L.h * HG + (member / kWgSlices) * (kGq ? kNV : 1);
  L.v0 = 16 * (kGq ? 1 : kNV) * (member % kWgSlices);
  L.lane = threadIdx.x & 63;
  L.c16 = L.lane & 15;
  L.g4 = 4 * (L.lane >> 4);
  L.bos = cu_at(cu, L.s, t_max);
  L.eos = cu_end(cu, L.s, L.bos, t_max);
  L.nc = (L.eos - L.bos + kC - 1) / kC;
  L.H = H;
  L.Hv = Hv;
  L.t_max = t_max;
  L.nt = nt;
  Walk W;
  if (kS == 1) {
    W = Walk{0, L.nc, h0, {o, nullptr}, {hT, nullptr}, false};
  } else {
    const int c0 = seg_begin(L.nc, seg.parts, role);
    const int c1 = seg_begin(L.nc, seg.parts, role + 1);
    const int64_t at = static_cast<int64_t>(role - 1) * seg.state_elems;
    W = role == 0 ? Walk{0, c1, h0, {o, nullptr}, {seg.sa, nullptr}, false}
                  : Walk{c0, c1, nullptr, {o, seg.oh}, {seg.z + at, seg.phi + at}, true};
  }
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const HomShare<kF32In> sh{hom_w, hom_k, hom_el};
  if constexpr (kS == 2) {
    // waves 0, 1: the identity-start state, a chunk behind; 2, 3: the
    // zero-start state; 4, 5: both states' outputs; 6: L2 warm-up
    if (wave == 0)
      hom_chain_wave<kF32In, 0>(L, W, xch, decx, sh);
    else if (wave == 1)
      hom_chain_wave<kF32In, 1>(L, W, xch, decx, sh);
    else if (wave == 2)
      chain_wave<kF32In, kDepth, 0, kS, kNV, kGq>(L, W, in, xch, decx, sh);
    else if (wave == 3)
      chain_wave<kF32In, kDepth, 1, kS, kNV, kGq>(L, W, in, xch, decx, sh);
    else if (wave == 4)
      helper_wave<kDepth, 0, kS, kNV, kGq>(L, W, in, xch);
    else if (wave == 5)
      helper_wave<kDepth, 1, kS, kNV, kGq>(L, W, in, xch);
    else if constexpr (kWarmWave<kF32In, kDepth, kS, kNV>)
      l2_warm_wave<kF32In, kDepth, true>(L, W, in, member, members, l2_sink, warm_values);
  } else {
    if (wave == 0)
      chain_wave<kF32In, kDepth, 0, kS, kNV, kGq>(L, W, in, xch, decx, sh);
    else if (wave == 1)
      chain_wave<kF32In, kDepth, 1, kS, kNV, kGq>(L, W, in, xch, decx, sh);
    else if (wave == 2)
      helper_wave<kDepth, 0, kS, kNV, kGq>(L, W, in, xch);
    else if (wave == 3)
      helper_wave<kDepth, 1, kS, kNV, kGq>(L, W, in, xch);
    else if constexpr (kWarmWave<kF32In, kDepth, kS, kNV>)
      l2_warm_wave<kF32In, kDepth, false>(L, W, in, member, members, l2_sink, warm_values);
  }
}

// ---- segment fix-up ----------------------------------------------------------
// The recurrence is affine in the state a segment starts from: with S_{k-1}
// the state before segment k >= 1, segment k's true final state is
// S_k = Z_k + Phi_k S_{k-1} and its true output rows are o_zero + o_hom
// S_{k-1} (Z, o_zero: the walk from zero with u; Phi, o_hom: the walk from
// the identity without u). In the stored layouts (value-major St[v][d]; Phi
// key-major) both updates are C = A B^T products:
//   o rows:  C[v][t] = sum_j S_t[v][j] o_hom[t][j],    o[t][v] += C[v][t]
//   state:   C[d][v] = sum_j Phi[d][j] S_t[v][j],      S'_t[v][d] = Z_t[v][d] + C[d][v]
// One 256-thread work-group computes one 128 x 128 C (128 output rows of a
// (sequence, value head), or a state) on v_mfma_f32_16x16x32_bf16, both fp32
// operands split into bf16 hi + lo and three product terms; A is staged in
// LDS, each wave owns 32 columns of C, and the wave's B^T rows and the output
// tile are requested before A is staged. With two parts one launch does the
// rows and the final state (S_1 from S_0); with more, one launch per state
// S_1, ..., S_{P-1} in order (S_k over Z_k in place, the last into hT), then
// one for the rows of every later segment.
constexpr int kFixThreads = 256;
constexpr int kLdFix = kD + 8;

// dst[n][16 mt + 4 g + i] = base[n][..] + C: rows n < rows of B^T (row
// stride bt_row bytes) and of base / dst (base_row bytes); A is 128 x 128
// value-major or key-major as above (row stride 128 floats).
// With kBtLds, B^T is a 128 x 128 fp32 block in LDS (row stride kLdS) instead
// of global memory; with kOutLds the result rows are also written to `sout`
// in LDS (same layout), where the next product of a chain reads them.
constexpr int kLdS = kD + 4;
template <bool kBtLds = false, bool kOutLds = false>
__device__ __forceinline__ void fix_block(const float *A, const float *Bt, uint32_t bt_row,
                                          const float *base, float *dst, uint32_t base_row,
                                          int rows, __bf16 *ahi, __bf16 *alo,
                                          float *sout = nullptr) {
  const rsrc_t rb = make_rsrc(kBtLds ? nullptr : Bt, kBtLds ? 0u : static_cast<uint32_t>(rows) * bt_row);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int g = lane >> 4, c = lane & 15;
  // requests first: this wave's B^T rows (32 wv + 16 nt + c, all k) and the
  // output tile the products are added to, so they arrive while A is staged
  u32x4 braw[4][2][2];  // [ks][nt][half]
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      if constexpr (kBtLds) {
        const float *r = Bt + (32 * wv + 16 * nt + c) * kLdS + 32 * ks + 8 * g;
        braw[ks][nt][0] = *reinterpret_cast<const u32x4 *>(r);
        braw[ks][nt][1] = *reinterpret_cast<const u32x4 *>(r + 4);
      } else {
        const uint32_t off = (32 * wv + 16 * nt + c) * bt_row + (32 * ks + 8 * g) * 4;
        braw[ks][nt][0] = __builtin_amdgcn_raw_buffer_load_b128(rb, off, 0, 0);
        braw[ks][nt][1] = __builtin_amdgcn_raw_buffer_load_b128(rb, off + 16, 0, 0);
      }
    }
  // C tile (mt, nt) element i: row 16 mt + 4 g + i, column n = 32 wv + 16 nt + c
  // (rows past the sequence read as zero and are not written)
  const rsrc_t rc = make_rsrc(base, static_cast<uint32_t>(rows) * base_row);
  f32x4 add[8][2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
      add[mt][nt] = __builtin_bit_cast(
          f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                     rc, (32 * wv + 16 * nt + c) * base_row + (16 * mt + 4 * g) * 4, 0, 0));
  {  // A (128 x 128 fp32) -> LDS as bf16 hi / lo rows
    const int r = tid >> 1, c0 = 64 * (tid & 1);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const f32x4 x0 = *reinterpret_cast<const f32x4 *>(A + r * kD + c0 + 8 * q);
      const f32x4 x1 = *reinterpret_cast<const f32x4 *>(A + r * kD + c0 + 8 * q + 4);
      const float x[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
      u32x4 h, l;
      split8_words(x, h, l);
      *reinterpret_cast<u32x4 *>(ahi + r * kLdFix + c0 + 8 * q) = h;
      *reinterpret_cast<u32x4 *>(alo + r * kLdFix + c0 + 8 * q) = l;
    }
  }
  __syncthreads();
  f32x4 acc[8][2];
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) acc[mt][0] = acc[mt][1] = zero4();
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    bf16x8 bh[2], bl[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const u32x4 w0 = braw[ks][nt][0], w1 = braw[ks][nt][1];
      const float x[8] = {__uint_as_float(w0[0]), __uint_as_float(w0[1]), __uint_as_float(w0[2]),
                          __uint_as_float(w0[3]), __uint_as_float(w1[0]), __uint_as_float(w1[1]),
                          __uint_as_float(w1[2]), __uint_as_float(w1[3])};
      u32x4 h, l;
      split8_words(x, h, l);
      bh[nt] = __builtin_bit_cast(bf16x8, h);
      bl[nt] = __builtin_bit_cast(bf16x8, l);
    }
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      const int off = (16 * mt + c) * kLdFix + 32 * ks + 8 * g;
      const bf16x8 ah = *reinterpret_cast<const bf16x8 *>(ahi + off);
      const bf16x8 al = *reinterpret_cast<const bf16x8 *>(alo + off);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        acc[mt][nt] = mfma(ah, bh[nt], acc[mt][nt]);
        acc[mt][nt] = mfma(ah, bl[nt], acc[mt][nt]);
        acc[mt][nt] = mfma(al, bh[nt], acc[mt][nt]);
      }
    }
  }
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int n = 32 * wv + 16 * nt + c;
    if (n < rows) {
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) {
        const f32x4 r = add[mt][nt] + acc[mt][nt];
        *reinterpret_cast<f32x4 *>(dst + (int64_t)n * (base_row / 4) + 16 * mt + 4 * g) = r;
        if constexpr (kOutLds) *reinterpret_cast<f32x4 *>(sout + n * kLdS + 16 * mt + 4 * g) = r;
      }
    }
  }
}

// Row blocks of 128 outputs of segments 1 .. P - 1 (nbo per segment), and
// with two parts also the final state S_1 (one more block per pair).
__global__ __launch_bounds__(kFixThreads) void segfix_kernel(const int32_t *__restrict__ cu,
                                                             float *__restrict__ o,
                                                             float *__restrict__ hT, SegScratch seg,
                                                             int n_max, int Hv, int t_max, int nbo) {
  __shared__ __attribute__((aligned(16))) __bf16 ahi[kD * kLdFix];
  __shared__ __attribute__((aligned(16))) __bf16 alo[kD * kLdFix];
  const int parts = seg.parts;
  // (at least one work-group per pair: with a capacity too short for the
  // later segments there are no row blocks, and the launch does nothing)
  const int per = max(1, (parts - 1) * nbo + (parts == 2 ? 1 : 0));
  const int pair = flat_block() / per, r = flat_block() % per;
  const int s = pair / Hv, hv = pair % Hv;
  if (s >= n_max) return;
  const int64_t st = ((int64_t)s * Hv + hv) * kD * kD;
  // one block, so that its code is inlined once
  const float *A, *Bt, *base;
  float *dst;
  uint32_t bt_row, base_row;
  int rows;
  if (parts == 2 && r == nbo) {  // S_1 = Z_1 + Phi_1 S_0, the final state
    if (hT == nullptr) return;
    A = seg.phi + st;
    Bt = seg.sa + st;
    base = seg.z + st;
    dst = hT + st;
    bt_row = base_row = kD * 4;
    rows = kD;
  } else {
    if (nbo == 0) return;
    const int bos = cu_at(cu, s, t_max), eos = cu_end(cu, s, bos, t_max);
    const int nc = (eos - bos + kC - 1) / kC;
    const int k = 1 + r / nbo, blk = r % nbo;  // segment, 128-row block of it
    const int t_begin = bos + kC * (seg_begin(nc, parts, k) + 2 * blk);
    const int t_end = min(eos, bos + kC * seg_begin(nc, parts, k + 1));
    if (t_begin >= t_end) return;
    A = k == 1 ? seg.sa + st : seg.z + (k - 2) * seg.state_elems + st;  // S_{k-1}
    const int64_t row0 = ((int64_t)t_begin * Hv + hv) * kD;
    Bt = seg.oh + row0;
    base = o + row0;
    dst = o + row0;
    bt_row = base_row = static_cast<uint32_t>(Hv) * kD * 4;
    rows = min(2 * kC, t_end - t_begin);
  }
  fix_block(A, Bt, bt_row, base, dst, base_row, rows, ahi, alo);
}

// States S_1 .. S_{P-1} of a walk in more than two parts, in order, by one
// work-group per (sequence, value head): S_k = Z_k + Phi_k S_{k-1}, over Z_k
// in place, or into hT for the last (left out when hT is null: the row fix-up
// needs S_1 .. S_{P-2} only). Each S_k also stays in LDS as the operand of the
// next product, so the chain needs no round trip through global memory and
// one launch.
__global__ __launch_bounds__(kFixThreads) void segchain_kernel(float *__restrict__ hT,
                                                               SegScratch seg, int n_max, int Hv) {
  __shared__ __attribute__((aligned(16))) __bf16 ahi[kD * kLdFix];
  __shared__ __attribute__((aligned(16))) __bf16 alo[kD * kLdFix];
  __shared__ __attribute__((aligned(16))) float sprev[kD * kLdS];
  const int pair = flat_block();
  if (pair >= n_max * Hv) return;
  const int64_t st = static_cast<int64_t>(pair) * kD * kD;
  const int64_t E = seg.state_elems;
  const int last = hT ? seg.parts - 1 : seg.parts - 2;
  for (int k = 1; k <= last; ++k) {
    float *z = seg.z + (k - 1) * E + st;
    float *dst = k == seg.parts - 1 ? hT + st : z;
    if (k == 1)
      fix_block<false, true>(seg.phi + st, seg.sa + st, kD * 4, z, dst, kD * 4, kD, ahi, alo, sprev);
    else
      fix_block<true, true>(seg.phi + (k - 1) * E + st, sprev, 0, z, dst, kD * 4, kD, ahi, alo, sprev);
    __syncthreads();  // S_k complete in LDS; A's staging space free again
  }
}

// Row blocks of 128 outputs per later segment: a segment has at most
// seg_len(nc, parts) chunks, nc = ceil(t_max / 64) at most.
int fix_row_blocks(int32_t t_max, int parts) {
  const int nc = (t_max + kC - 1) / kC;
  return (seg_len(nc, parts) + 1) / 2;
}

// Work-groups of the row fix-up launch (at least one per pair).
int64_t fix_grid(int32_t n_max, int32_t hv, int32_t t_max, int parts) {
  const int64_t per =
      (parts - 1) * static_cast<int64_t>(fix_row_blocks(t_max, parts)) + (parts == 2 ? 1 : 0);
  return static_cast<int64_t>(n_max) * hv * std::max<int64_t>(1, per);
}

template <bool kF32In, int kDepth, int kS, int kNV = 1, bool kGq = false>
hipError_t launch_walk(const StageBuffers &in, const float *h0, const int32_t *cu, int32_t n_max,
                       int32_t h, int32_t hv, int32_t t_max, int32_t nt, float *o, float *hT,
                       const SegScratch &seg, hipStream_t stream, hipEvent_t start,
                       hipEvent_t stop) {
  const int64_t members = kGq ? (hv / h / kNV) * kSlices : (hv / h) * (kSlices / kNV);
  const int64_t rounds = (static_cast<int64_t>(n_max) * h + kXcds - 1) / kXcds;
  constexpr int kThr = kInterThreads<kF32In, kDepth, kS, kNV>;
  dim3 grid;
  if (!flat_grid((kS == 2 ? seg.parts : 1) * rounds * kXcds * members, kThr, grid))
    return hipErrorInvalidValue;
  // warm the value heads' lines too when the intermediates come from HBM
  const bool warm_values = stage2_operand_bytes(nt, h, hv, kF32In) > kLlcResident;
  hipExtLaunchKernelGGL((inter_kernel<kF32In, kDepth, kS, kNV, kGq>), grid, dim3(kThr), 0, stream,
                        start, stop, 0, in, h0, cu, o, hT, n_max, h, hv, t_max, nt, seg,
                        warm_values);
  return hipGetLastError();
}

template <bool kF32In>
hipError_t launch_waves(const StageBuffers &in, const float *h0, const int32_t *cu, int32_t n_max,
                        int32_t h, int32_t hv, int32_t t_max, int32_t nt, float *o, float *hT,
                        hipStream_t stream, KernelEvents ev, int segments, int tiles, int share,
                        const SegScratch &seg) {
  // the GQA-shared shape (one slice of `share` value heads per work-group);
  // the host admits it only for the one-piece, one-tile walk
  if (share == 4)
    return launch_walk<kF32In, 1, 1, 4, true>(in, h0, cu, n_max, h, hv, t_max, nt, o, hT, seg,
                                              stream, ev.start, ev.stop);
  if (share == 2)
    return launch_walk<kF32In, 1, 1, 2, true>(in, h0, cu, n_max, h, hv, t_max, nt, o, hT, seg,
                                              stream, ev.start, ev.stop);
  if (segments < 2) {
    if (tiles == 4)
      return launch_walk<kF32In, 1, 1, 4>(in, h0, cu, n_max, h, hv, t_max, nt, o, hT, seg, stream,
                                          ev.start, ev.stop);
    if (tiles == 2)
      return launch_walk<kF32In, 1, 1, 2>(in, h0, cu, n_max, h, hv, t_max, nt, o, hT, seg, stream,
                                          ev.start, ev.stop);
    return launch_walk<kF32In, kDepthSingle, 1>(in, h0, cu, n_max, h, hv, t_max, nt, o, hT, seg,
                                                stream, ev.start, ev.stop);
  }
  // the fix-up grids were checked on the host before anything was queued
  const int parts = seg.parts;
  if (parts != segments || parts > 4) return hipErrorInvalidValue;
  const int nbo = fix_row_blocks(t_max, parts);
  dim3 grid, sgrid;
  if (!flat_grid(fix_grid(n_max, hv, t_max, parts), kFixThreads, grid) ||
      !flat_grid(static_cast<int64_t>(n_max) * hv, kFixThreads, sgrid))
    return hipErrorInvalidValue;
  const hipError_t e = launch_walk<kF32In, kDepthSeg, 2>(in, h0, cu, n_max, h, hv, t_max, nt, o,
                                                         hT, seg, stream, ev.start, nullptr);
  if (e != hipSuccess) return e;
  if (parts > 2) {  // S_1 .. S_{P-1} in order
    hipLaunchKernelGGL(segchain_kernel, sgrid, dim3(kFixThreads), 0, stream, hT, seg, n_max, hv);
    const hipError_t es = hipGetLastError();
    if (es != hipSuccess) return es;
  }
  hipExtLaunchKernelGGL(segfix_kernel, grid, dim3(kFixThreads), 0,
                        stream, nullptr, ev.stop, 0, cu, o, hT, seg, n_max, hv, t_max, nbo);
  return hipGetLastError();
}

}  // namespace

// Compute units of the current device (queried once per device; the cache
// is atomic, so concurrent callers at worst query the device twice).
int cu_count() {
  static std::atomic<int> counts[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = counts[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    counts[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

bool inter_grids_fit(int32_t n_max, int32_t h, int32_t hv, int32_t t_max, int segments, int tiles,
                     int share) {
  const int64_t members = (hv / h / share) * (kSlices / (segments >= 2 ? 1 : tiles));
  const int64_t rounds = (static_cast<int64_t>(n_max) * h + kXcds - 1) / kXcds;
  dim3 grid;
  const int threads = segments >= 2 ? kInterThreads<false, kDepthSeg, 2, 1> : 320;
  if (!flat_grid((segments >= 2 ? segments : 1) * rounds * kXcds * members, threads, grid))
    return false;
  if (segments < 2) return true;
  return flat_grid(fix_grid(n_max, hv, t_max, segments), kFixThreads, grid) &&
         flat_grid(static_cast<int64_t>(n_max) * hv, kFixThreads, grid);
}

int inter_one_walk_grid(int32_t n_max, int32_t h, int32_t hv) {
  const int64_t rounds = (static_cast<int64_t>(n_max) * h + kXcds - 1) / kXcds;
  const int64_t g = rounds * kXcds * (hv / h) * kSlices;
  return g > 0x3fffffff ? 0x3fffffff : static_cast<int>(g);
}

hipError_t launch_inter(bool f32_in, const StageBuffers &in, const float *h0,
                        const int32_t *cu_seqlens, int32_t n_max, int32_t h, int32_t hv,
                        int32_t t_max, int32_t nt_max, float *o, float *hT, hipStream_t stream,
                        KernelEvents ev, int segments, int tiles, int share, SegScratch seg) {
  return f32_in ? launch_waves<true>(in, h0, cu_seqlens, n_max, h, hv, t_max, nt_max, o, hT, stream,
                                     ev, segments, tiles, share, seg)
                : launch_waves<false>(in, h0, cu_seqlens, n_max, h, hv, t_max, nt_max, o, hT,
                                      stream, ev, segments, tiles, share, seg);
}

}  // namespace gdn
