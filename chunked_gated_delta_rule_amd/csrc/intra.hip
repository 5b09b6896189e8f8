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
// block, 16 bytes per lane; u's 768 bytes), so that stage only streams blocks:
//   w16   fp16 per (hv, chunk)  -w fragments (A operand of (-w) S)
//   q16   fp16 per (h, chunk)   q rounded to fp16 (B operand of S^T q^T)
//   kimg  bf16 per (h, chunk)   K^T fragments for the state update (hi[, lo])
//   uimg  f24 per (hv, chunk)   u fragments rounded to 24-bit floats (fp32's top
//                               three bytes), one 768-byte block per 16 x 16 tile
//   pimg  fp16 per (hv, chunk)  P = scale * tril(q k^T * Gamma), the two
//                               half-zero pairs packed to 8 bytes per lane
//   gimg  fp32 per (hv, chunk)  e^{gamma_last - gamma}, scale e^gamma (ordered
//                               [c][R] for r = 16 R + c), e^{gamma_last}
// P is the intra-chunk attention term of the output (AMX page, section 5); it
// shares the masked decay factors with A. Per-chunk blocks are addressed by
// the slot floor(t0 / 64) + n of chunk start t0 in sequence n, which is
// distinct for every chunk of a batch and below cdiv(t_max, 64) + n_max - 1.
//
// The exponent is always a masked difference gamma_r - gamma_i <= 0, never
// e^gamma_r * e^-gamma_i, which would overflow under strong decay; it is taken
// as exp2 of log2-scaled cumulative gates. Only lower 16x16 blocks are
// computed (AMX page, section 8: triangular work stays triangular).
//
// gfx950 mapping: one 256-thread work-group per (chunk, h), four wave64s.
//  * Every global operand of the work-group (K, q, and V, g, beta of the
//    first value head) is requested at entry; V, g, beta of the next value
//    head are requested while the current one is processed.
//  * K K^T and K q^T on v_mfma_f32_16x16x32_bf16 (lower 16x16 blocks, kept in
//    registers across the value heads). fp32 inputs are split x = hi + lo into
//    two bf16 terms and the products take three MFMA terms.
//  * Each wave scans the chunk's gates itself (one token per lane) and keeps
//    its own copy in LDS, so the gates need no work-group barrier.
//  * The solve runs in fp32: the four diagonal 16x16 blocks by column forward
//    substitution (four lanes per column, quad reductions), then the
//    off-diagonal blocks in two doubling levels on v_mfma_f32_16x16x4_f32
//    (T_10 = -T_11 A_10 T_00 and T_32 likewise, then the lower-left 32x32
//    block = -T_BB A_BA T_AA).
//  * w and u are MFMA products of the transposed K (V) tile with the scaled
//    T. The six nonzero 16x32 pieces of T diag(beta e^gamma) and T diag(beta)
//    are scaled and split into hi + lo bf16 once each, into LDS in fragment
//    order, and every wave reads them for its own d-blocks.
// Rows of a partial last chunk are zero-filled, so they add nothing; every
// per-chunk block is written in full (zeros past the end).
#include "gdn.h"
#include "gdn_common.hpp"
#include "gdn_launch.hpp"

namespace gdn {

static_assert(kFusedIndexMaxSeqs == GDN_FUSED_INDEX_MAX_SEQS, "fused index bound");

namespace {

// stage-1 work-group orders (see intra_kernel)
constexpr int kSlotFastest = 0, kHeadFastest = 1, kHeadFastestReversed = 2;

constexpr int kLdRow = kD + 8;   // bf16 row-major tile [64][136]
constexpr int kLdAT = kC + 4;    // fp32 A, then T in place [64][68]
constexpr int kLdX = 16 + 4;     // fp32 per-wave 16x16 scratch

// LDS of one work-group (bf16 input: 77 KB, two work-groups per CU; fp32
// input: 111 KB):
//   K rows   [terms][64][136] bf16   for K K^T, K q^T, the K^T fragments and w
//   A / T    [64][68] fp32           A, solved into T in place
//   V rows   [terms][64][136] bf16   for u; the solve's per-wave scratch lives
//                                    here until V is stored after the solve
//   gates    per wave: log2-scaled gamma and beta (64 floats each)
//   T s      six 4 KB items: hi / lo bf16 fragments of T diag(beta e^gamma)
//            and T diag(beta) for the w / u products
// During set-up the q rows occupy the A / T region (and V's for fp32 input).
template <bool kF32In>
struct IntraSmem {
  static constexpr int kTerms = kF32In ? 2 : 1;
  static constexpr int kTile = 64 * kLdRow * 2;
  static constexpr int kOffK = 0;
  static constexpr int kOffAT = kOffK + kTerms * kTile;
  static constexpr int kOffV = kOffAT + 64 * kLdAT * 4;
  static constexpr int kOffGates = kOffV + kTerms * kTile;
  static constexpr int kOffTS = kOffGates + 4 * 2 * 64 * 4;
  static constexpr int kBytes = kOffTS + 6 * 4 * 64 * 16;
  static_assert(64 * kLdAT * 4 == kTile, "q rows must fit the A / T region (and V's)");
  static_assert(4 * 16 * kLdX * 4 <= kTile, "solve scratch must fit the V region");
};

// x of the lane that quad permutation kCtrl (DPP quad_perm) selects.
template <int kCtrl>
__device__ __forceinline__ float quad_swap(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), kCtrl,
                                                                0xf, 0xf, true));
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Transposed read of a row-major bf16 tile in LDS (ds_read_b64_tr_b16): within
// each 16-lane group, lane s supplies the 8-byte chunk M[row + (s >> 2)][col +
// 4 (s & 3) ..], and lane j receives element j of columns col .. col + 15 from
// rows row .. row + 3, i.e. lane j holds M[row + i][col + j], i = 0..3.
__device__ __forceinline__ bf16x4 tr4(const __bf16 *base, int ld, int row, int col, int lane) {
  const int s = lane & 15;
  const __bf16 *p = base + (row + (s >> 2)) * ld + col + 4 * (s & 3);
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4 *)(const_cast<__bf16 *>(p)));
  return __builtin_bit_cast(bf16x4, v);
}

// MFMA operand from a row-major tile M[k][n] (k the contraction): lane (g, n)
// holds M[rowA + i][col + n] (i < 4) then M[rowB + i][col + n], where rowA and
// rowB may depend on the lane group g.
__device__ __forceinline__ bf16x8 frag_tr2(const __bf16 *base, int ld, int rowA, int rowB, int col,
                                           int lane) {
  const bf16x4 a = tr4(base, ld, rowA, col, lane);
  const bf16x4 b = tr4(base, ld, rowB, col, lane);
  return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// The same with eight consecutive contraction rows per group: lane (g, n)
// holds M[row0 + 8 g + e][col + n], e < 8 (the k order of frag_rows).
__device__ __forceinline__ bf16x8 frag_tr(const __bf16 *base, int ld, int row0, int col, int lane) {
  const int r = row0 + 8 * (lane >> 4);
  return frag_tr2(base, ld, r, r + 4, col, lane);
}

// A tile of a [rows, heads, 128] tensor: rows t0 .. t0 + L - 1 of one head,
// as a buffer range that ends after row L - 1, so rows past the chunk read as
// zero with no branch (row stride `heads` x 128 elements).
template <bool kF32In>
struct Tile {
  rsrc_t r;
  uint32_t row_bytes;
};

template <bool kF32In>
__device__ __forceinline__ Tile<kF32In> tile_of(const void *base, int t0, int heads, int head,
                                                int L) {
  constexpr int kEl = kF32In ? 4 : 2;
  const uint32_t row_bytes = static_cast<uint32_t>(heads) * kD * kEl;
  const char *p = static_cast<const char *>(base) + ((int64_t)t0 * heads + head) * kD * kEl;
  return Tile<kF32In>{make_rsrc(p, static_cast<uint32_t>(L) * row_bytes), row_bytes};
}

// Raw 16-byte words of 4 rows x 8 columns of a tile starting at row `row0`
// (fp32 input: two words per row).
template <bool kF32In>
struct Raw4x8 {
  u32x4 w[4][kF32In ? 2 : 1];
};

template <bool kF32In>
__device__ __forceinline__ Raw4x8<kF32In> load_raw4x8(const Tile<kF32In> &t, int row0, int col) {
  constexpr int kEl = kF32In ? 4 : 2;
  Raw4x8<kF32In> x;
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const uint32_t off = (row0 + rr) * t.row_bytes + col * kEl;
    x.w[rr][0] = buf_load16(t.r, off);
    if constexpr (kF32In) x.w[rr][1] = buf_load16(t.r, off + 16);
  }
  return x;
}

// The raw words as bf16 hi (and lo for fp32 input, x = hi + lo).
template <bool kF32In>
__device__ __forceinline__ void to_terms(const Raw4x8<kF32In> &x, u32x4 (&hi)[4], u32x4 (&lo)[4]) {
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    if constexpr (kF32In) {
      const f32x4 a = __builtin_bit_cast(f32x4, x.w[rr][0]);
      const f32x4 b = __builtin_bit_cast(f32x4, x.w[rr][1]);
      const float v[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
      split8_words(v, hi[rr], lo[rr]);
    } else {
      hi[rr] = x.w[rr][0];
      lo[rr] = u32x4{0u, 0u, 0u, 0u};
    }
  }
}

// ---- fused front: 4 rows x 8 channels of q, k or v computed from the
// pre-conv bf16 channels (rows t0 + row0 - 3 .. t0 + row0 + 3 and the 8
// channels' taps), with the same arithmetic, in the same order, as the
// standalone front kernel: conv taps accumulated oldest first by fmaf, SiLU
// x / (1 + e^-x) by the shared silu(), and for q and k the 16-lane sum of
// squares of the head and x / sqrt(sum + 1e-6).
struct ConvRaw {
  u32x4 x[7];  // source rows t0 + row0 - 3 + i (zero before the sequence start)
  u32x4 w[4];  // conv weights of the 8 channels, [channel][tap], up to 4 taps
};

// tb: first row the buffer range starts at (max(bos, t0 - (d_conv - 1)));
// rows_end: one past the last row that may be read.
__device__ __forceinline__ ConvRaw load_conv(const ConvIn &ci, int channels, int ch0, int t0,
                                             int rows_end, int tb, int row0, int col) {
  ConvRaw r;
  const rsrc_t x = make_rsrc(ci.qkv + (int64_t)tb * channels + ch0,
                             static_cast<uint32_t>(rows_end - tb) * channels * 2);
#pragma unroll
  for (int i = 0; i < 7; ++i) {
    const int rel = t0 + row0 - 3 + i - tb;  // negative: before the range, reads zero
    r.x[i] = buf_load16(x, static_cast<uint32_t>(rel * channels * 2 + col * 2));
  }
  const rsrc_t w = make_rsrc(ci.conv_w, static_cast<uint32_t>(channels) * ci.d_conv * 2);
  const uint32_t wo = static_cast<uint32_t>(ch0 + col) * ci.d_conv * 2;
#pragma unroll
  for (int i = 0; i < 4; ++i) r.w[i] = i < ci.d_conv ? buf_load16(w, wo + 16 * i) : u32x4{0u, 0u, 0u, 0u};
  return r;
}

// Rows rr < valid of the thread's 4 x 8 block as fp32, split into bf16 hi + lo
// (rows >= valid are zero, as rows past a sequence are for stored inputs).
// kTaps = d_conv, a template parameter so that every register index is fixed.
template <int kTaps, bool kHalf>
__device__ __forceinline__ void conv_terms(const ConvRaw &r, bool l2, int valid,
                                           u32x4 (&hi)[4], u32x4 (&lo)[4]) {
  float x[7][8];
#pragma unroll
  for (int i = 0; i < 7; ++i) unpack8(r.x[i], x[i]);
  float wf[32];
#pragma unroll
  for (int i = 0; i < 4; ++i) unpack8(r.w[i], wf + 8 * i);
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    float y[8];
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      float acc = 0.f;
#pragma unroll
      for (int j = 0; j < kTaps; ++j) acc = fmaf(x[rr + j + 4 - kTaps][c], wf[c * kTaps + j], acc);
      y[c] = silu(acc);
      ss = fmaf(y[c], y[c], ss);
    }
    if (l2) {
      ss = sum16(ss);
      const float inv = 1.f / sqrtf(ss + 1e-6f);
#pragma unroll
      for (int c = 0; c < 8; ++c) y[c] *= inv;
    }
    if (rr >= valid) {
#pragma unroll
      for (int c = 0; c < 8; ++c) y[c] = 0.f;
    }
    if constexpr (kHalf) {  // rounded to fp16 (nearest even), one term
      hi[rr] = u32x4{pack_f16(y[0], y[1]), pack_f16(y[2], y[3]), pack_f16(y[4], y[5]),
                     pack_f16(y[6], y[7])};
      lo[rr] = u32x4{0u, 0u, 0u, 0u};
    } else {
      split8_words(y, hi[rr], lo[rr]);
    }
  }
}

// MFMA on two 16-bit operand fragments held as raw bits: bf16, or fp16 when
// kHalf (fp16 inputs).
template <bool kHalf>
__device__ __forceinline__ f32x4 mma(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
  if constexpr (kHalf)
    return mfma(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c);
  else
    return mfma(a, b, c);
}

// fp16 bits -> float.
__device__ __forceinline__ float f16_bits_to_float(uint32_t bits16) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits16)));
}

// Eight fp32 values split into fp16 hi and lo words (x = hi + lo to about 22
// significant bits; hi rounded to nearest even).
__device__ __forceinline__ void split8_words_f16(const float (&x)[8], u32x4 &hi, u32x4 &lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h[i] = pack_f16(x[2 * i], x[2 * i + 1]);
    l[i] = pack_f16(x[2 * i] - f16_bits_to_float(h[i] & 0xffffu),
                    x[2 * i + 1] - f16_bits_to_float(h[i] >> 16));
  }
  hi = u32x4{h[0], h[1], h[2], h[3]};
  lo = u32x4{l[0], l[1], l[2], l[3]};
}

// P pairs (q, R): token block q (32 tokens) of column tile R (16 outputs);
// each pair is two 16x16 tiles of P^T, (2q, R) and (2q + 1, R).
__device__ __forceinline__ int pair_q(int pi) { return pi == 3 || pi == 5 ? 1 : 0; }
__device__ __forceinline__ int pair_r(int pi) { return pi < 2 ? pi : 2 + ((pi - 2) >> 1); }

// acc += X Y for 16 x 16 fp32 blocks in LDS (row strides ldx, ldy) on the
// fp32 MFMA. Step s contracts k = 4 (lane >> 4) + s: lane l holds X row
// (l & 15) and Y column (l & 15), so one 16-byte read gives its X values for
// all four steps. Result: lane (g, c) holds rows 4 g .. 4 g + 3 of column c.
__device__ __forceinline__ f32x4 mm16(const float *x, int ldx, const float *y, int ldy, int lane,
                                      f32x4 acc) {
  const int r = lane & 15, g = lane >> 4;
  const f32x4 xa = *reinterpret_cast<const f32x4 *>(x + r * ldx + 4 * g);
#pragma unroll
  for (int s = 0; s < 4; ++s)
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(xa[s], y[(4 * g + s) * ldy + r], acc, 0, 0, 0);
  return acc;
}

// Store an accumulator (lane (g, c): rows 4 g + i of column c) to a 16 x 16
// fp32 block in LDS, multiplied by `sign`.
__device__ __forceinline__ void put16(float *dst, int ld, const f32x4 &acc, float sign, int lane) {
  const int c = lane & 15, g = lane >> 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) dst[(4 * g + i) * ld + c] = sign * acc[i];
}

// Orders this wave's LDS writes before its own later LDS reads by other lanes
// (a wave's LDS operations complete in order; this keeps the compiler from
// moving the reads up).
__device__ __forceinline__ void wave_lds_sync() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

// Stage 2 walks every chunk of a sequence in order, so with many sequences
// the longest walks should start first (the longest-processing-time rule:
// the work-groups of the last sequences to start then finish with the rest
// instead of after them). One work-group of stage 1 ranks the n <= kThreads
// sequences by chunk count, longest first and ties by index, so the ranks
// are a permutation: thread t compares its sequence with all n (their chunk
// counts staged in LDS, read as broadcasts) and writes order[rank] = t.
// The caller's LDS must be free (no other wave still reading it).
__device__ __forceinline__ void write_walk_order(const int32_t *__restrict__ cu, int n, int t_max,
                                                 int32_t *__restrict__ order, int *ncs) {
  const int t = threadIdx.x;
  int mine = 0;
  if (t < n) {
    mine = seq_chunks(cu, t, t_max);
    ncs[t] = mine;
  }
  __syncthreads();
  if (t < n) {
    int rank = 0;
    for (int s = 0; s < n; ++s) {
      const int x = ncs[s];
      rank += (x > mine || (x == mine && s < t)) ? 1 : 0;
    }
    order[rank] = t;
  }
}

// kTaps: 0 reads q, k, v; 1..4 computes them from the pre-conv channels with a
// kTaps-tap conv (the fused front). kHalf: q, k, v are fp16 (read as fp16, or
// from the fused front rounded to fp16); the row tiles and their MFMAs are then
// fp16 instead of bf16, the T s items are split into fp16 hi + lo, and the K^T
// image is written as exact bf16 hi + lo terms (the layout of fp32 input).
template <bool kF32In, int kTaps, bool kHalf = false>
__global__ __launch_bounds__(kThreads, kF32In ? 1 : 2) void intra_kernel(
    const void *__restrict__ qin, const void *__restrict__ kin, const void *__restrict__ vin,
    const float *__restrict__ g, const float *__restrict__ beta, const int32_t *__restrict__ cu,
    const int32_t *__restrict__ table, int32_t *__restrict__ table_out, int n_max,
    StageBuffers out, int H, int Hv, int t_max, int nt, float scale, ConvIn ci,
    int order) {
  constexpr bool kConv = kTaps > 0;
  static_assert(!kConv || kF32In || kHalf, "the fused front produces fp32 or fp16 q, k, v");
  static_assert(!(kF32In && kHalf), "one input kind");
  using Smem = IntraSmem<kF32In>;
  __shared__ __attribute__((aligned(16))) unsigned char smem[Smem::kBytes];
  __bf16 *rk = reinterpret_cast<__bf16 *>(smem + Smem::kOffK);    // K rows (hi[, lo])
  float *at = reinterpret_cast<float *>(smem + Smem::kOffAT);      // A, then T in place
  __bf16 *rv = reinterpret_cast<__bf16 *>(smem + Smem::kOffV);    // V rows (hi[, lo])
  float *xs = reinterpret_cast<float *>(smem + Smem::kOffV);      // solve scratch (in V's place)
  u32x4 *ts = reinterpret_cast<u32x4 *>(smem + Smem::kOffTS);     // T s items (hi / lo)
  __bf16 *rq = reinterpret_cast<__bf16 *>(smem + Smem::kOffAT);   // q rows during set-up

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  float *gsh = reinterpret_cast<float *>(smem + Smem::kOffGates) + wv * 2 * 64;  // this wave's gates
  float *bsh = gsh + 64;
  // work-group -> (item = table slot, key head), in one of three orders:
  //   kSlotFastest: one sequence whose stage-2 operands stay in the
  //     last-level cache; keeps the work-groups in flight spread over the
  //     whole sequence;
  //   kHeadFastest: batches; the dispatch reaches the sentinel slots past the
  //     batch's last chunk only at the end (a varlen batch of 32 sequences has
  //     more sentinel slots than chunks);
  //   kHeadFastestReversed: one sequence whose stage-2 operands outgrow the
  //     last-level cache; the last chunks come first, so the intermediates
  //     stage 2 reads first are the last written and still in that cache.
  // a one-dimensional grid of nt * H work-groups (for batches it measured
  // faster than a two-dimensional (H, nt) grid in the same order)
  const int wg = flat_block();
  if (wg >= nt * H) return;  // past the grid's count (last row)
  int item, h;
  if (order == kSlotFastest) {
    item = wg % nt;
    h = wg / nt;
  } else {
    item = order == kHeadFastest ? wg / H : nt - 1 - wg / H;
    h = wg % H;
  }
  // this work-group's chunk: from the caller's table, or located from
  // cu_seqlens here (every wave computes it; the key-head-0 work-groups also
  // fill the workspace copy of the table)
  int2 ent;
  if (table) {
    ent = reinterpret_cast<const int2 *>(table)[item];
    // an entry naming no sequence, or a chunk that starts past its sequence's
    // end, is treated as a sentinel (checked below, after the bounds)
    if (ent.x < 0 || ent.x >= n_max || ent.y < 0 || ent.y > t_max / kC) ent = make_int2(-1, -1);
  } else {
    ent = locate_chunk(cu, n_max, t_max, item, lane);
    ent.x = __builtin_amdgcn_readfirstlane(ent.x);  // the same in every lane
    ent.y = __builtin_amdgcn_readfirstlane(ent.y);
    if (h == 0 && tid == 0) reinterpret_cast<int2 *>(table_out)[item] = ent;
  }
  // the work-group of slot 0, key head 0 ranks the sequences for stage 2,
  // after its own chunk (its LDS is then free) or here if it has none
  const bool ranks = out.order && wg == 0;
  const int bos = ent.x < 0 ? 0 : cu_at(cu, ent.x, t_max);
  const int t0 = bos + max(ent.y, 0) * kC;
  const int L = ent.x < 0 ? 0 : min(kC, cu_end(cu, ent.x, bos, t_max) - t0);
  if (L <= 0) {  // sentinel slot
    if (ranks) write_walk_order(cu, n_max, t_max, out.order, reinterpret_cast<int *>(smem));
    return;
  }
  const int HG = Hv / H;
  const int slot = (t0 >> 6) + ent.x;
  constexpr int kNK = kF32In || kHalf ? 32 : 16;

  const int lrow = 4 * (tid >> 4);  // this thread's 4 rows and 8 columns of a tile
  const int lcol = 8 * (tid & 15);

  // ---- requests: K, q, then V / g / beta of the first value head (buffer
  // loads, rows past the chunk read as zero); with the fused front, the
  // pre-conv rows of those heads' channels and their conv weights ----------
  const int channels = (2 * H + Hv) * kD;
  const int tb = max(bos, t0 - (ci.d_conv - 1));  // first pre-conv row of the halo
  auto load_tile = [&](const void *base, int heads, int head, int ch0, int rows)
      __attribute__((always_inline)) {
    if constexpr (kConv)
      return load_conv(ci, channels, ch0, t0, t0 + rows, tb, lrow, lcol);
    else
      return load_raw4x8(tile_of<kF32In>(base, t0, heads, head, rows), lrow, lcol);
  };
  auto tile_terms = [&](const auto &raw, bool l2, u32x4 (&hi)[4], u32x4 (&lo)[4])
      __attribute__((always_inline)) {
    if constexpr (kConv)
      conv_terms<kTaps, kHalf>(raw, l2, L - lrow, hi, lo);
    else
      to_terms(raw, hi, lo);
  };
  // a 4 x 8 block of a row-major tile (hi[, lo]) into LDS
  auto put_rows = [&](__bf16 *dst, const u32x4 (&hi)[4], const u32x4 (&lo)[4])
      __attribute__((always_inline)) {
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      *reinterpret_cast<u32x4 *>(dst + (lrow + rr) * kLdRow + lcol) = hi[rr];
      if constexpr (kF32In)
        *reinterpret_cast<u32x4 *>(dst + 64 * kLdRow + (lrow + rr) * kLdRow + lcol) = lo[rr];
    }
  };
  const auto kraw = load_tile(kin, H, h, (H + h) * kD, L);
  const auto qraw = load_tile(qin, H, h, h * kD, L);
  auto vraw = load_tile(vin, Hv, h * HG, (2 * H + h * HG) * kD, L);
  const bool tok_ok = lane < L;
  const uint32_t gate_bytes = static_cast<uint32_t>(L) * Hv * 4;
  auto load_gate = [&](const float *p, int hv) __attribute__((always_inline)) {
    return buf_load_f32(make_rsrc(p + (int64_t)t0 * Hv + hv, gate_bytes), lane * Hv * 4);
  };
  float g_next = load_gate(g, h * HG);
  float b_next = load_gate(beta, h * HG);
  {
    u32x4 hi[4], lo[4];
    tile_terms(kraw, true, hi, lo);
    put_rows(rk, hi, lo);
    tile_terms(qraw, true, hi, lo);
    put_rows(rq, hi, lo);
  }
  __syncthreads();

  // ---- K^T fragments for the state update, read transposed from the K
  // rows: fragment (tau, q), lane (g, c) holds K[32 q + 4 g + j][16 tau + c]
  // for j < 4 and K[32 q + 16 + 4 g + j - 4][..] for j >= 4 (the token order of
  // the inter stage's delta fragments).
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int f = wv + 4 * m;  // fragment 0..15 = 2 tau + q
    const int tau = f >> 1, qq = f & 1;
    const int g4 = 4 * (lane >> 4);
    __bf16 *dst = out.kimg + ((((int64_t)h * nt + slot) * kNK + f) * 64 + lane) * 8;
    const bf16x8 kt = frag_tr2(rk, kLdRow, 32 * qq + g4, 32 * qq + 16 + g4, 16 * tau, lane);
    if constexpr (kHalf) {  // fp16 values as exact bf16 hi + lo terms
      const u32x4 bits = __builtin_bit_cast(u32x4, kt);
      float x[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[2 * i] = f16_bits_to_float(bits[i] & 0xffffu);
        x[2 * i + 1] = f16_bits_to_float(bits[i] >> 16);
      }
      u32x4 hi, lo;
      split8_words(x, hi, lo);
      *reinterpret_cast<u32x4 *>(dst) = hi;
      *reinterpret_cast<u32x4 *>(dst + 16 * 64 * 8) = lo;
    } else {
      *reinterpret_cast<bf16x8 *>(dst) = kt;
    }
    if constexpr (kF32In)
      *reinterpret_cast<bf16x8 *>(dst + 16 * 64 * 8) =
          frag_tr2(rk + 64 * kLdRow, kLdRow, 32 * qq + g4, 32 * qq + 16 + g4, 16 * tau, lane);
  }

  // ---- q16 fragments for y = S^T q^T: fragment (R, p), lane (g, c) holds
  // q[16 R + c][32 p + 4 g + j] for j < 4 and q[16 R + c][32 p + 16 + 4 g + j - 4]
  // for j >= 4, rounded to fp16 once (from hi + lo for fp32 input).
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int item = tid + kThreads * m;
    const int f = item >> 6, l = item & 63;
    const int off = (16 * (f >> 2) + (l & 15)) * kLdRow + 32 * (f & 3) + 4 * (l >> 4);
    float x[8];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const u32x2 a = *reinterpret_cast<const u32x2 *>(rq + off + 16 * half);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        if constexpr (kHalf) {
          x[4 * half + 2 * i] = f16_bits_to_float(a[i] & 0xffffu);
          x[4 * half + 2 * i + 1] = f16_bits_to_float(a[i] >> 16);
        } else {
          x[4 * half + 2 * i] = __uint_as_float(a[i] << 16);
          x[4 * half + 2 * i + 1] = __uint_as_float(a[i] & 0xffff0000u);
        }
      }
      if constexpr (kF32In) {
        const u32x2 b = *reinterpret_cast<const u32x2 *>(rq + 64 * kLdRow + off + 16 * half);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          x[4 * half + 2 * i] += __uint_as_float(b[i] << 16);
          x[4 * half + 2 * i + 1] += __uint_as_float(b[i] & 0xffff0000u);
        }
      }
    }
    _Float16 *dst = out.q16 + ((((int64_t)h * nt + slot) * 16 + f) * 64 + l) * 8;
    *reinterpret_cast<u32x4 *>(dst) = u32x4{pack_f16(x[0], x[1]), pack_f16(x[2], x[3]),
                                            pack_f16(x[4], x[5]), pack_f16(x[6], x[7])};
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
        const bf16x8 a = frag_rows(rk, kLdRow, 16 * bi, 32 * ks, lane);
        const bf16x8 bb = frag_rows(rk, kLdRow, 16 * bj, 32 * ks, lane);
        acc = mma<kHalf>(a, bb, acc);
        if constexpr (kF32In) {
          const __bf16 *rlo = rk + 64 * kLdRow;
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
        const bf16x8 a = frag_rows(rk, kLdRow, 16 * tj, 32 * ks, lane);
        const bf16x8 bb = frag_rows(rq, kLdRow, 16 * tr, 32 * ks, lane);
        acc = mma<kHalf>(a, bb, acc);
        if constexpr (kF32In) {
          acc = mfma(frag_rows(rk + 64 * kLdRow, kLdRow, 16 * tj, 32 * ks, lane), bb, acc);
          acc = mfma(a, frag_rows(rq + 64 * kLdRow, kLdRow, 16 * tr, 32 * ks, lane), acc);
        }
      }
    }
    pacc[n] = acc;
  }
  __syncthreads();  // the q rows (in the A / T and V regions) are dead from here on

  // T's upper blocks (0,1) and (2,3) are read as zeros by the w/u products;
  // neither A nor T is ever written there.
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int e = tid + kThreads * m;  // 0..511
    const int blk = e >> 8, r = (e >> 4) & 15, c = e & 15;
    at[(32 * blk + r) * kLdAT + 32 * blk + 16 + c] = 0.f;
  }

  for (int gi = 0; gi < HG; ++gi) {
    const int hv = h * HG + gi;
    // The lane index as the lane-dependent conditions of this loop (token
    // validity, the causal masks of P and A, the solve's row and column
    // tests) see it. The opaque copy keeps their compares inside the loop:
    // hoisted out of it, the lane masks (64-bit scalar values each) outgrew
    // the scalar registers and were spilled to vector-register lanes.
    int ml = lane;
    asm volatile("" : "+v"(ml));
    // ---- this value head's operands, next value head's requests (a request
    // past the group reads an empty range) ----------------------------------
    u32x4 vh[4], vl[4];
    tile_terms(vraw, false, vh, vl);
    const float gv = g_next, bv = b_next;
    {
      const int nx = gi + 1 < HG ? hv + 1 : hv;
      const int Ln = gi + 1 < HG ? L : 0;
      vraw = load_tile(vin, Hv, nx, (2 * H + nx) * kD, Ln);
      const uint32_t gb = static_cast<uint32_t>(Ln) * Hv * 4;
      g_next = buf_load_f32(make_rsrc(g + (int64_t)t0 * Hv + nx, gb), lane * Hv * 4);
      b_next = buf_load_f32(make_rsrc(beta + (int64_t)t0 * Hv + nx, gb), lane * Hv * 4);
    }

    // ---- gates: each wave scans its own copy (lane = token) ---------------
    const float gam2 = wave_inclusive_scan(gv * kLog2e, lane);  // log2-scaled gamma
    const float gl2 = __shfl(gam2, L - 1, 64);                   // last valid token
    const float eg = fast_exp2(gam2);
    gsh[lane] = gam2;
    bsh[lane] = bv;
    if (wv == 0) {
      float *gd = out.gimg + ((int64_t)hv * nt + slot) * kGateStride;
      gd[lane] = ml < L ? fast_exp2(gl2 - gam2) : 0.f;
      gd[64 + 4 * (lane & 15) + (lane >> 4)] = ml < L ? scale * eg : 0.f;  // [c][R], r = 16 R + c
      gd[128 + lane] = ml == 0 ? fast_exp2(gl2) : 0.f;
    }
    wave_lds_sync();

    // ---- P = scale * tril(q k^T * Gamma), this wave's pairs, as fp16
    // pair lane (g, c): tile (2q, R) rows 4 g + i then tile (2q + 1, R).
#pragma unroll
    for (int n2 = 0; n2 < 2; ++n2) {
      if (n2 < npair) {
        const int pi = pair0 + n2;
        const int r = 16 * pair_r(pi) + (ml & 15);
        const float gr = gsh[r];
        float x[8];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const int j0 = 32 * pair_q(pi) + 16 * hf + 4 * (ml >> 4);
          const f32x4 gj = *reinterpret_cast<const f32x4 *>(gsh + j0);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int j = j0 + i;
            x[4 * hf + i] = (j <= r && r < L) ? scale * pacc[2 * n2 + hf][i] * fast_exp2(gr - gj[i]) : 0.f;
          }
        }
        char *dst = reinterpret_cast<char *>(out.pimg) + ((int64_t)hv * nt + slot) * kPBytes +
                    p_offset(pi);
        if (p_half(pi)) {  // x[4..7] are above the diagonal: only the first 8 bytes
          *reinterpret_cast<u32x2 *>(dst + lane * 8) = u32x2{pack_f16(x[0], x[1]), pack_f16(x[2], x[3])};
        } else {
          *reinterpret_cast<u32x4 *>(dst + lane * 16) =
              u32x4{pack_f16(x[0], x[1]), pack_f16(x[2], x[3]), pack_f16(x[4], x[5]), pack_f16(x[6], x[7])};
        }
      }
    }

    // ---- A = strict_lower(beta_r G e^{gamma_r - gamma_j}) -> LDS ----------
#pragma unroll
    for (int n = 0; n < 3; ++n) {
      if (n < nblk) {
        const int j = 16 * gbj[n] + (ml & 15);
        const int r0 = 16 * gbi[n] + 4 * (ml >> 4);
        const float gj = gsh[j];
        const f32x4 gr = *reinterpret_cast<const f32x4 *>(gsh + r0);
        const f32x4 br = *reinterpret_cast<const f32x4 *>(bsh + r0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = r0 + i;
          at[r * kLdAT + j] = j < r ? br[i] * gacc[n][i] * fast_exp2(gr[i] - gj) : 0.f;
        }
      }
    }
    __syncthreads();

    // ---- solve 1: diagonal blocks by column forward substitution, in place
    // (T[r][c] = delta_rc - sum_{i < r} A[r][i] T[i][c]). Four lanes per
    // column: lane (c, q) = (lane >> 2, lane & 3) keeps T[4 q .. 4 q + 3][c]
    // and forms that quarter of each row's sum; a quad reduction completes
    // it. A is strictly lower and unknown T entries are still zero, so the
    // quarters need no mask. The whole block is read before T is written.
    {
      const int c = ml >> 2, q = ml & 3;
      float *ab = at + (16 * wv) * kLdAT + 16 * wv;
      f32x4 arow[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) arow[r] = *reinterpret_cast<const f32x4 *>(ab + r * kLdAT + 4 * q);
      f32x4 t = zero4();
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float part = fmaf(arow[r][0], t[0], arow[r][1] * t[1]) + fmaf(arow[r][2], t[2], arow[r][3] * t[3]);
        part += quad_swap<0xB1>(part);  // lanes 4c + {1, 0, 3, 2}
        part += quad_swap<0x4E>(part);  // lanes 4c + {2, 3, 0, 1}
        const float val = r == c ? 1.f : (r < c ? 0.f : -part);
        t[r & 3] = q == (r >> 2) ? val : t[r & 3];
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) ab[(4 * q + j) * kLdAT + c] = t[j];
    }
    __syncthreads();
    // ---- solve 2: T_10 = -T_11 (A_10 T_00), T_32 = -T_33 (A_32 T_22) -------
    float *xw = xs + wv * 16 * kLdX;
    if (wv < 2) {
      const int b = 2 * wv;  // diagonal pair (b, b + 1)
      float *blk = at + (16 * (b + 1)) * kLdAT + 16 * b;  // A_10 -> T_10 (A_32 -> T_32)
      const float *t_bb = at + (16 * b) * kLdAT + 16 * b;
      const float *t_nn = at + (16 * (b + 1)) * kLdAT + 16 * (b + 1);
      put16(xw, kLdX, mm16(blk, kLdAT, t_bb, kLdAT, lane, zero4()), 1.f, lane);
      wave_lds_sync();
      put16(blk, kLdAT, mm16(t_nn, kLdAT, xw, kLdX, lane, zero4()), -1.f, lane);
    }
    __syncthreads();
    // ---- solve 3: lower-left 32x32 block, X = A_BA T_AA ... ----------------
    const int bi = 2 + (wv >> 1), bj = wv & 1;
    {
      const float *a_i0 = at + (16 * bi) * kLdAT;
      const float *a_i1 = a_i0 + 16;
      f32x4 x = zero4();
      if (bj == 0) {
        x = mm16(a_i0, kLdAT, at, kLdAT, lane, x);                        // A_i0 T_00
        x = mm16(a_i1, kLdAT, at + 16 * kLdAT, kLdAT, lane, x);           // A_i1 T_10
      } else {
        x = mm16(a_i1, kLdAT, at + 16 * kLdAT + 16, kLdAT, lane, x);      // A_i1 T_11
      }
      put16(xw, kLdX, x, 1.f, lane);
    }
    __syncthreads();
    // ---- ... then T_BA = -T_BB X, over A_BA ----------------------------------
    {
      const float *t22 = at + 32 * kLdAT + 32;
      const float *t32 = at + 48 * kLdAT + 32;
      const float *t33 = at + 48 * kLdAT + 48;
      f32x4 y;
      if (bi == 2) {
        y = mm16(t22, kLdAT, xw, kLdX, lane, zero4());
      } else {
        y = mm16(t32, kLdAT, xs + (wv - 2) * 16 * kLdX, kLdX, lane, zero4());
        y = mm16(t33, kLdAT, xw, kLdX, lane, y);
      }
      put16(at + (16 * bi) * kLdAT + 16 * bj, kLdAT, y, -1.f, lane);
    }
    __syncthreads();  // T complete; the solve scratch (V's region) is free

    // ---- T diag(beta e^gamma) and T diag(beta), split hi + lo, once per
    // nonzero (token block rb, contraction block ks) of T: item it in the
    // order (0,0)(1,0)(2,0)(2,1)(3,0)(3,1); lane (g, c) holds row 16 rb + c,
    // columns j = 32 ks + 8 g .. + 7 (an A fragment of U = (T s) V and a B
    // fragment of W^T = K^T (T s)^T alike).
    for (int it = wv; it < 6; it += 4) {
      const int rb = it < 2 ? it : 1 + (it >> 1), ks = it < 2 ? 0 : (it & 1);
      const int j0 = 32 * ks + 8 * (lane >> 4);
      const float *trow = at + (16 * rb + (lane & 15)) * kLdAT + j0;
      const f32x4 t_a = *reinterpret_cast<const f32x4 *>(trow);
      const f32x4 t_b = *reinterpret_cast<const f32x4 *>(trow + 4);
      const f32x4 g_a = *reinterpret_cast<const f32x4 *>(gsh + j0);
      const f32x4 g_b = *reinterpret_cast<const f32x4 *>(gsh + j0 + 4);
      const f32x4 b_a = *reinterpret_cast<const f32x4 *>(bsh + j0);
      const f32x4 b_b = *reinterpret_cast<const f32x4 *>(bsh + j0 + 4);
      float xw8[8], xu8[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        xu8[i] = t_a[i] * b_a[i];
        xu8[4 + i] = t_b[i] * b_b[i];
        xw8[i] = xu8[i] * fast_exp2(g_a[i]);
        xw8[4 + i] = xu8[4 + i] * fast_exp2(g_b[i]);
      }
      u32x4 *d = ts + it * 4 * 64 + lane;
      if constexpr (kHalf) {
        split8_words_f16(xw8, d[0], d[64]);
        split8_words_f16(xu8, d[128], d[192]);
      } else {
        split8_words(xw8, d[0], d[64]);
        split8_words(xu8, d[128], d[192]);
      }
    }
    put_rows(rv, vh, vl);
    __syncthreads();

    // ---- w and u in one pass: the T s items against K^T / V^T read
    // transposed from the row tiles. Tiles (d-block db, token block rb): w as
    // W^T = K^T (T s)^T (lane holds four d of one token), u as U = (T s) V
    // (lane holds four tokens of one d).
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      f32x4 wacc[2] = {zero4(), zero4()}, uacc[2] = {zero4(), zero4()};
#pragma unroll
      for (int ks = 0; ks <= (rb >> 1); ++ks) {
        const u32x4 *item = ts + (rb < 2 ? rb : 2 * rb - 2 + ks) * 4 * 64 + lane;
        const u32x4 wh = item[0], wl = item[64], uh = item[128], ul = item[192];
#pragma unroll
        for (int db2 = 0; db2 < 2; ++db2) {
          const int db = 2 * wv + db2;
          const bf16x8 ka = frag_tr(rk, kLdRow, 32 * ks, 16 * db, lane);
          const bf16x8 vb = frag_tr(rv, kLdRow, 32 * ks, 16 * db, lane);
          f32x4 aw = wacc[db2], au = uacc[db2];
          aw = mma<kHalf>(ka, as_bf16x8(wh), aw);
          aw = mma<kHalf>(ka, as_bf16x8(wl), aw);
          au = mma<kHalf>(as_bf16x8(uh), vb, au);
          au = mma<kHalf>(as_bf16x8(ul), vb, au);
          if constexpr (kF32In) {
            aw = mfma(frag_tr(rk + 64 * kLdRow, kLdRow, 32 * ks, 16 * db, lane), as_bf16x8(wh), aw);
            au = mfma(as_bf16x8(uh), frag_tr(rv + 64 * kLdRow, kLdRow, 32 * ks, 16 * db, lane), au);
          }
          wacc[db2] = aw;
          uacc[db2] = au;
        }
      }
      {
        // -w fragment (rb, p = wv): lane (g, c) holds w[r = 16 rb + c][d] for
        // d = 32 wv + 4 g + i (tile db = 2 wv) and 32 wv + 16 + 4 g + i (db = 2 wv + 1)
        const f32x4 a0 = wacc[0], a1 = wacc[1];
        _Float16 *dst = out.w16 + ((((int64_t)hv * nt + slot) * 16 + 4 * rb + wv) * 64 + lane) * 8;
        *reinterpret_cast<u32x4 *>(dst) = u32x4{pack_f16(-a0[0], -a0[1]), pack_f16(-a0[2], -a0[3]),
                                                pack_f16(-a1[0], -a1[1]), pack_f16(-a1[2], -a1[3])};
      }
#pragma unroll
      for (int db2 = 0; db2 < 2; ++db2) {
        const int db = 2 * wv + db2;
        // u: lane holds u[r = 16 rb + 4 (lane >> 4) + i][d = 16 db + (lane & 15)],
        // stored as four 24-bit floats in 12 bytes
        uint32_t *dst = out.uimg + (((((int64_t)hv * nt + slot) * 8 + db) * 4 + rb) * 64 + lane) * 3;
        *reinterpret_cast<u32x3_a4 *>(dst) = pack_f24x4(uacc[db2]);
      }
    }
    __syncthreads();  // A / T, V and the gate copies are rewritten next
  }
  if (ranks) write_walk_order(cu, n_max, t_max, out.order, reinterpret_cast<int *>(smem));
}

}  // namespace

hipError_t launch_intra(InKind in_kind, const void *q, const void *k, const void *v,
                        const float *g, const float *beta, const int32_t *cu_seqlens,
                        const int32_t *table, int32_t *table_out, int32_t n_max, int32_t nt_max,
                        int32_t h, int32_t hv, int32_t t_max, float scale,
                        const StageBuffers &out, hipStream_t stream, KernelEvents ev, ConvIn conv) {
  if (!table && (n_max > kFusedIndexMaxSeqs || !table_out)) return hipErrorInvalidValue;
  if (out.order && n_max > kThreads) return hipErrorInvalidValue;  // one thread per sequence
  if (conv.qkv && (in_kind == InKind::kBf16 || !conv.conv_w || conv.d_conv < 1 || conv.d_conv > 4))
    return hipErrorInvalidValue;
  if (nt_max <= 0) return hipSuccess;
  // work-group order (see the kernel)
  const int order = n_max > 1 ? kHeadFastest
                    : stage2_operand_bytes(nt_max, h, hv, in_kind != InKind::kBf16) > kLlcResident
                        ? kHeadFastestReversed
                        : kSlotFastest;
  dim3 grid;
  if (!flat_grid(static_cast<int64_t>(nt_max) * h, kThreads, grid)) return hipErrorInvalidValue;
#define GDN_LAUNCH_INTRA(F32, TAPS, HALF)                                                       \
  hipExtLaunchKernelGGL((intra_kernel<F32, TAPS, HALF>), grid, dim3(kThreads), 0, stream,       \
                        ev.start, ev.stop, 0, q, k, v, g, beta, cu_seqlens, table, table_out,   \
                        n_max, out, h, hv, t_max, nt_max, scale, conv, order)
  if (conv.qkv && in_kind == InKind::kF16) {
    switch (conv.d_conv) {
      case 1: GDN_LAUNCH_INTRA(false, 1, true); break;
      case 2: GDN_LAUNCH_INTRA(false, 2, true); break;
      case 3: GDN_LAUNCH_INTRA(false, 3, true); break;
      default: GDN_LAUNCH_INTRA(false, 4, true); break;
    }
  } else if (conv.qkv) {
    switch (conv.d_conv) {
      case 1: GDN_LAUNCH_INTRA(true, 1, false); break;
      case 2: GDN_LAUNCH_INTRA(true, 2, false); break;
      case 3: GDN_LAUNCH_INTRA(true, 3, false); break;
      default: GDN_LAUNCH_INTRA(true, 4, false); break;
    }
  } else if (in_kind == InKind::kF32) {
    GDN_LAUNCH_INTRA(true, 0, false);
  } else if (in_kind == InKind::kF16) {
    GDN_LAUNCH_INTRA(false, 0, true);
  } else {
    GDN_LAUNCH_INTRA(false, 0, false);
  }
#undef GDN_LAUNCH_INTRA
  return hipGetLastError();
}

}  // namespace gdn
