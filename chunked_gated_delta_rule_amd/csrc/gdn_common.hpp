// Device-side building blocks shared by the gfx950 GDN kernels: vector types,
// bf16 rounding and hi/lo splitting, the 16x16x32 bf16 MFMA, and fragment
// loads from LDS.
//
// MFMA fragment convention (v_mfma_f32_16x16x32_bf16, one wave64):
//   A (16 x 32): lane l holds row (l & 15), eight consecutive k starting at
//                8 * (l >> 4);
//   B (32 x 16): lane l holds column (l & 15), the same eight k;
//   C (16 x 16): lane l holds column (l & 15), rows 4 * (l >> 4) + i, i < 4.
// Which physical k each lane slot feeds does not change the result as long as
// A and B use the same assignment, which the loaders below guarantee. So an
// operand whose contraction index is contiguous in LDS is read with one
// 16-byte load per fragment.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kD = 128;       // Dk = Dv
constexpr int kC = 64;        // chunk length
constexpr int kThreads = 256; // four wave64s per work-group

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// fp16 operands: the state S enters w S and q S as a single fp16 term (11
// significant bits; its products carry the fp32 state to well below the
// method's tolerance), with w stored in fp16 and q converted exactly.
__device__ __forceinline__ f32x4 mfma(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Two fp32 -> packed fp16 pair (round to nearest even).
__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
  typedef float f32x2_ __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_{a, b}, f16x2));
}

// Round to nearest even (hardware conversion on gfx950).
__device__ __forceinline__ __bf16 to_bf16(float x) { return static_cast<__bf16>(x); }
__device__ __forceinline__ float from_bf16(__bf16 x) { return static_cast<float>(x); }

// x = hi + lo with hi = bf16(x), lo = bf16(x - hi): 16 significant bits.
__device__ __forceinline__ void split_bf16(float x, __bf16 &hi, __bf16 &lo) {
  hi = to_bf16(x);
  lo = to_bf16(x - from_bf16(hi));
}

__device__ __forceinline__ bf16x8 lds_frag(const __bf16 *p) {
  return *reinterpret_cast<const bf16x8 *>(p);
}

// A fragment of a row-major LDS matrix (row stride ld elements), rows
// [r0, r0 + 16), contraction columns [k0, k0 + 32).
__device__ __forceinline__ bf16x8 frag_rows(const __bf16 *base, int ld, int r0, int k0, int lane) {
  return lds_frag(base + (r0 + (lane & 15)) * ld + k0 + 8 * (lane >> 4));
}

__device__ __forceinline__ float bf16_bits_to_float(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Unpack 8 bf16 held in a 16-byte word into floats.
__device__ __forceinline__ void unpack8(const u32x4 &w, float *f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

__device__ __forceinline__ uint32_t pack2(__bf16 a, __bf16 b) {
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, a)) |
         (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, b)) << 16);
}

// Raw buffer access: a descriptor over [base, base + bytes) whose out-of-range
// reads return zero, which masks the rows past a sequence's end without
// branches (gfx9 buffer resource, word 3 = 0x00020000).
typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, bytes, 0x00020000);
}

__device__ __forceinline__ u32x4 buf_load16(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

__device__ __forceinline__ float buf_load_f32(rsrc_t r, uint32_t off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4 &v) { return __builtin_bit_cast(bf16x8, v); }

// 24-bit float: the upper three bytes of an fp32 (sign, 8-bit exponent, 15
// mantissa bits). It keeps fp32's range with a relative step of 2^-16. Four
// of them pack into three words: value i takes bytes 3 i .. 3 i + 2 (little
// endian).
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
// the same three words at 4-byte alignment (a lane's 12 bytes in a block)
typedef uint32_t u32x3_a4 __attribute__((ext_vector_type(3), aligned(4)));

// x rounded to nearest with 16 significant bits by Veltkamp's split (Dekker,
// "A floating-point technique for extending the available precision", 1971):
// with c = (2^8 + 1) x, hi = c - (c - x) has its low 8 mantissa bits zero, so
// bytes 1..3 of its word are the 24-bit value. A NaN stays a NaN; an infinity
// or |x| above about 1.3e36 (where c overflows) becomes a NaN. Each step is
// written as an FMA with an exact product (by 1, or plus 0), i.e. one rounding
// each: left as a product and differences, contraction would fuse c - x into
// fma(x, 257, -x) and return x unrounded.
__device__ __forceinline__ uint32_t round_f24_word(float x) {
  const float c = __builtin_fmaf(x, 257.f, 0.f);   // RN(257 x)
  const float d = __builtin_fmaf(-1.f, x, c);      // RN(c - x)
  return __float_as_uint(__builtin_fmaf(-1.f, d, c));  // RN(c - d)
}

__device__ __forceinline__ u32x3 pack_f24x4(const f32x4 &v) {
  const uint32_t a = round_f24_word(v[0]), b = round_f24_word(v[1]), c = round_f24_word(v[2]),
                 d = round_f24_word(v[3]);
  // v_perm_b32 (hi, lo, sel): result byte i is byte sel_i of lo (sel_i < 4) or
  // byte sel_i - 4 of hi (4..7)
  return u32x3{__builtin_amdgcn_perm(b, a, 0x05030201u), __builtin_amdgcn_perm(c, b, 0x06050302u),
               __builtin_amdgcn_perm(d, c, 0x07060503u)};
}

__device__ __forceinline__ f32x4 unpack_f24x4(const u32x3 &w) {
  // selector 0x0c gives a zero byte (the dropped low byte)
  return f32x4{__uint_as_float(__builtin_amdgcn_perm(0u, w[0], 0x0201000cu)),
               __uint_as_float(__builtin_amdgcn_perm(w[1], w[0], 0x0504030cu)),
               __uint_as_float(__builtin_amdgcn_perm(w[2], w[1], 0x0403020cu)),
               __uint_as_float(__builtin_amdgcn_perm(0u, w[2], 0x0302010cu))};
}

// 2^x on the hardware transcendental unit (v_exp_f32); used with exponents
// that are differences of log2-scaled cumulative gates, always <= 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

constexpr float kLog2e = 1.4426950408889634f;

// SiLU x / (1 + e^-x) as x * rcp(1 + 2^(-x log2 e)) on the hardware exp2 and
// reciprocal (about one ulp each); the front kernel and the front fused into
// stage 1 both use this, so they produce the same bits.
__device__ __forceinline__ float silu(float x) {
  return x * __builtin_amdgcn_rcpf(1.f + fast_exp2(-x * kLog2e));
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two fp32 -> packed bf16 hi pair and packed bf16 lo pair (x = hi + lo), using
// one packed conversion per pair.
__device__ __forceinline__ void split2(float x0, float x1, uint32_t &hi, uint32_t &lo) {
  const bf16x2 h = __builtin_convertvector(f32x2{x0, x1}, bf16x2);
  hi = __builtin_bit_cast(uint32_t, h);
  const float r0 = x0 - __uint_as_float(hi << 16);
  const float r1 = x1 - __uint_as_float(hi & 0xffff0000u);
  lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{r0, r1}, bf16x2));
}

// Split eight fp32 values into packed bf16 hi and lo words (x = hi + lo).
__device__ __forceinline__ void split8_words(const float (&x)[8], u32x4 &hi, u32x4 &lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) split2(x[2 * i], x[2 * i + 1], h[i], l[i]);
  hi = u32x4{h[0], h[1], h[2], h[3]};
  lo = u32x4{l[0], l[1], l[2], l[3]};
}

// Split four fp32 values into hi/lo bf16, packed as {01, 23} pairs.
__device__ __forceinline__ void split_pack4(const float (&x)[4], u32x2 &hi, u32x2 &lo) {
  uint32_t h0, l0, h1, l1;
  split2(x[0], x[1], h0, l0);
  split2(x[2], x[3], h1, l1);
  hi = u32x2{h0, h1};
  lo = u32x2{l0, l1};
}


// Floats per (value head, chunk) in the gate block: e^{gamma_last - gamma_t}
// [64], scale * e^{gamma_t} [64] ordered [c][R] for token t = 16 R + c,
// e^{gamma_last} and zero padding [64].
constexpr int kGateStride = 192;

// The value DPP control kCtrl moves into each lane of the rows in kRowMask (0
// in the other rows, and where the source lane is outside the row).
template <int kCtrl, int kRowMask>
__device__ __forceinline__ float dpp_in(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kCtrl,
                                                               kRowMask, 0xf, true));
}

// Sum over each aligned group of 16 lanes, left in every lane of the group:
// pairs, quads (quad_perm), halves (row_half_mirror pairs lane i with 7 - i)
// and rows (row_mirror pairs i with 15 - i). Addition commutes, so all 16
// lanes hold the same bits. The front kernel and the fused front use it for
// the per-head sum of squares.
__device__ __forceinline__ float sum16(float x) {
  x += dpp_in<0xB1, 0xf>(x);   // quad_perm [1, 0, 3, 2]
  x += dpp_in<0x4E, 0xf>(x);   // quad_perm [2, 3, 0, 1]
  x += dpp_in<0x141, 0xf>(x);  // row_half_mirror
  x += dpp_in<0x140, 0xf>(x);  // row_mirror
  return x;
}

// Inclusive prefix sum over the 64 lanes of a wave: within each row of 16
// lanes x[i] += x[i - 1], x[i - 2], x[i - 4], x[i - 8] (row_shr), then rows 1
// and 3 add lane 15 of the row before (row_bcast:15) and rows 2 and 3 add
// lane 31 (row_bcast:31). All on DPP: no LDS round trip.
__device__ __forceinline__ float wave_inclusive_scan(float x, int /*lane*/) {
  x += dpp_in<0x111, 0xf>(x);  // row_shr:1
  x += dpp_in<0x112, 0xf>(x);  // row_shr:2
  x += dpp_in<0x114, 0xf>(x);  // row_shr:4
  x += dpp_in<0x118, 0xf>(x);  // row_shr:8
  x += dpp_in<0x142, 0xa>(x);  // row_bcast:15 into rows 1, 3
  x += dpp_in<0x143, 0xc>(x);  // row_bcast:31 into rows 2, 3
  return x;
}

// Inclusive prefix sum of integers over the 64 lanes of a wave.
__device__ __forceinline__ int wave_inclusive_scan_int(int x, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  return x;
}

// Entry s of cu_seqlens as every kernel reads it: clamped to [0, t_max]. A
// valid cu_seqlens (cu[0] = 0, non-decreasing, cu[n_max] <= t_max) is a
// documented precondition and passes unchanged; with an invalid one the
// results are unspecified, but every row a kernel touches stays inside the
// caller's [t_max, ...] buffers.
__device__ __forceinline__ int cu_at(const int32_t *__restrict__ cu, int s, int t_max) {
  return min(max(cu[s], 0), t_max);
}
// End of sequence s given its (clamped) start: never before it.
__device__ __forceinline__ int cu_end(const int32_t *__restrict__ cu, int s, int bos, int t_max) {
  return max(cu_at(cu, s + 1, t_max), bos);
}
// Chunks of sequence s.
__device__ __forceinline__ int seq_chunks(const int32_t *__restrict__ cu, int s, int t_max) {
  const int bos = cu_at(cu, s, t_max);
  return (cu_end(cu, s, bos, t_max) - bos + kC - 1) / kC;
}

// Batches of at most this many sequences let stage 1 locate its chunk from
// cu_seqlens itself (one pass of 64-lane scans per wave).
constexpr int kFusedIndexMaxSeqs = 256;

// Entry `slot` of the chunk-index table, computed by one wave from cu_seqlens
// (n_max <= kFusedIndexMaxSeqs): (sequence, chunk within the sequence) of the
// slot-th chunk of the batch in (sequence, chunk) order, or (-1, -1) past the
// last chunk. Empty sequences own no chunk. Same definition as the table
// kernel's searchsorted fill.
__device__ __forceinline__ int2 locate_chunk(const int32_t *__restrict__ cu, int n_max, int t_max,
                                             int slot, int lane) {
  constexpr int kBlocks = kFusedIndexMaxSeqs / 64;
  int nc[kBlocks];
#pragma unroll
  for (int b = 0; b < kBlocks; ++b) {  // all loads first: one round trip
    const int s = 64 * b + lane;
    nc[b] = s < n_max ? seq_chunks(cu, s, t_max) : 0;
  }
  int base = 0;  // chunks of the sequences before this block
#pragma unroll
  for (int b = 0; b < kBlocks; ++b) {
    if (64 * b >= n_max) break;
    const int incl = wave_inclusive_scan_int(nc[b], lane);
    const int excl = base + incl - nc[b];
    const unsigned long long hit = __ballot(nc[b] > 0 && excl <= slot && slot < excl + nc[b]);
    if (hit) {
      const int src = __ffsll(static_cast<long long>(hit)) - 1;
      return make_int2(64 * b + src, slot - __shfl(excl, src, 64));
    }
    base += __shfl(incl, 63, 64);
  }
  return make_int2(-1, -1);
}

// Flat work-group number of a grid made by flat_grid (rows of gridDim.x);
// numbers past the requested count occur in the last row only.
__device__ __forceinline__ int flat_block() {
  return static_cast<int>(blockIdx.x + gridDim.x * blockIdx.y);
}

}  // namespace gdn
