// Host-side launchers of the gfx950 GDN kernels (internal to the library).
// Each enqueues work on `stream` and returns the launch status; none
// allocates or synchronises. Shapes have already been validated by the C ABI.
// Every launcher takes an optional pair of caller-created HIP events that the
// dispatch itself records at its start and end (hipExtLaunchKernel), for
// kernel timing without extra packets between launches.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

// P = scale * tril(q k^T * Gamma) per (value head, chunk): six pairs of
// 16 x 16 tiles of P^T, each a 16 x 32 MFMA fragment of fp16 values. In pairs
// 0 and 3 (output tiles 0 and 2, against the token block that starts with
// their own tile) the second half of every lane's contraction slots lies
// above the diagonal and is always zero, so those pairs keep 8 bytes per lane
// (512-byte blocks) and the others 16 (1 KB).
constexpr int kPBytes = 5 * 1024;
__host__ __device__ constexpr bool p_half(int pi) { return pi == 0 || pi == 3; }
__host__ __device__ constexpr int p_term_bytes(int pi) { return p_half(pi) ? 512 : 1024; }
// byte offset of pair pi's block
__host__ __device__ constexpr int p_offset(int pi) {
  return pi == 0 ? 0 : pi == 1 ? 512 : pi == 2 ? 1536 : pi == 3 ? 2560 : pi == 4 ? 3072 : 4096;
}
static_assert(p_offset(5) + p_term_bytes(5) == kPBytes, "P block layout");

// Intermediates written by the intra stage and read by the inter stage (all
// device memory inside the caller's workspace; layouts in intra.hip).
struct StageBuffers {
  _Float16 *w16;  // [hv, nt_max, 16 fragments, 64 lanes, 8]
  _Float16 *q16;  // [h, nt_max, 16 fragments, 64 lanes, 8]
  __bf16 *kimg;   // [h, nt_max, 16 or 32 fragments, 64 lanes, 8]
  uint32_t *uimg; // [hv, nt_max, 8, 4, 64 lanes, 3 words]: four 24-bit floats per lane
  _Float16 *pimg; // [hv, nt_max, 5 KB]: P fragments (fp16)
  float *gimg;    // [hv, nt_max, 192]
  // [n_max]: sequence indices ranked by chunk count, longest first (ties by
  // index), written by stage 1 and read by stage 2 to start the longest walks
  // first; null when the batch is not ranked (one sequence, or more than
  // kThreads sequences)
  int32_t *order;
};

// Pre-conv input of the fused front: stage 1 computes q, k, v itself from the
// packed bf16 channels q | k | v (conv + SiLU, and the L2 norm of q and k).
struct ConvIn {
  const uint16_t *qkv = nullptr;     // [t_max, (2 h + hv) * 128] bf16
  const uint16_t *conv_w = nullptr;  // [(2 h + hv) * 128, d_conv] bf16
  int d_conv = 0;                    // 1..4
};

// Start / end events recorded by one dispatch (both may be null).
// Grid of `blocks` work-groups of `threads` threads, numbered flat (see
// flat_block): the dispatch packet takes each grid dimension in work-items as
// a 32-bit number, so one row holds at most 2^31 - 1 work-items (a multiple of
// 64 work-groups, which keeps work-group i on XCD i mod 8) and larger grids
// take further rows (at most 65535). Returns false when that is not enough.
inline bool flat_grid(int64_t blocks, int threads, dim3 &grid) {
  const int64_t row = (0x7fffffffLL / threads) / 64 * 64;
  const int64_t x = blocks < row ? blocks : row;
  const int64_t y = x > 0 ? (blocks + x - 1) / x : 0;
  // every flat number, the last row's surplus included, must fit an int
  if (blocks < 0 || x * y > 0x7fffffffLL || y > 65535) return false;
  grid = dim3(static_cast<uint32_t>(x), static_cast<uint32_t>(y));
  return true;
}

struct KernelEvents {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};

hipError_t launch_chunk_index(const int32_t *cu_seqlens, int32_t n_max, int32_t nt_max,
                              int32_t t_max, int32_t *table, hipStream_t stream,
                              KernelEvents ev = {});

hipError_t launch_front(const void *qkv, const void *conv_w, int32_t d_conv,
                        const int32_t *cu_seqlens, int32_t n_max, int32_t t_max, int32_t h,
                        int32_t hv, float *q, float *k, float *v, hipStream_t stream,
                        KernelEvents ev = {});

// How stage 1 takes q, k, v: bf16 (one bf16 term), fp32 (split into bf16
// hi + lo, three-term products) or fp16 (one fp16 term). fp32 and fp16 both
// write the K^T image as bf16 hi + lo terms, so stage 2 reads them alike.
enum class InKind { kBf16 = 0, kF32 = 1, kF16 = 2 };

// table: the chunk-index table, or null to have each work-group locate its
// chunk from cu_seqlens (n_max <= kFusedIndexMaxSeqs) and write the table into
// table_out. With conv.qkv set, q, k, v are ignored and computed from the
// pre-conv channels, kept in fp32 (in_kind kF32) or rounded to fp16 (kF16).
hipError_t launch_intra(InKind in_kind, const void *q, const void *k, const void *v,
                        const float *g, const float *beta, const int32_t *cu_seqlens,
                        const int32_t *table, int32_t *table_out, int32_t n_max, int32_t nt_max,
                        int32_t h, int32_t hv, int32_t t_max, float scale,
                        const StageBuffers &out, hipStream_t stream, KernelEvents ev = {},
                        ConvIn conv = {});

hipError_t launch_recurrent(bool f32_in, const void *q, const void *k, const void *v,
                            const float *g, const float *beta, const float *h0,
                            const int32_t *cu_seqlens, int32_t n_max, int32_t t_max, int32_t h,
                            int32_t hv, float scale, float *o, float *hT, hipStream_t stream,
                            KernelEvents ev = {});

// Bytes of the stage-1 intermediates stage 2 reads, nt chunk slots (K^T as
// hi + lo when split_k). Above kLlcResident (the last-level cache is 256 MB
// and also holds the inputs and o) they come back from HBM.
inline int64_t stage2_operand_bytes(int64_t nt, int64_t h, int64_t hv, bool split_k) {
  const int64_t per_chunk = hv * (16 * 1024 + 128 * 64 * 3 + kPBytes + 192 * 4) +
                            h * ((split_k ? 32 : 16) * 1024 + 16 * 1024);
  return nt * per_chunk;
}
constexpr int64_t kLlcResident = 160ll << 20;

// Scratch of the segmented stage-2 walk (P = parts segments): sa, segment
// 0's final state; z and phi, the P - 1 later segments' final zero-start
// states (value-major [dv][dk] per (sequence, value head)) and homogeneous
// states (key-major [dk][dv]), one array of state_elems floats each,
// consecutive; oh, the homogeneous output rows [t_max, hv, dv] of every later
// segment's tokens.
struct SegScratch {
  float *sa = nullptr, *z = nullptr, *phi = nullptr, *oh = nullptr;
  int64_t state_elems = 0;
  int parts = 1;
};

// Compute units of the current device (queried once per device).
int cu_count();

// Whether every grid stage 2 launches for this shape (the walk, and with two
// segments the fix-up) fits flat_grid; checked on the host before any launch.
bool inter_grids_fit(int32_t n_max, int32_t h, int32_t hv, int32_t t_max, int segments, int tiles,
                     int share);

// Work-groups of the one-walk stage-2 grid (one per (sequence, value head,
// 16-column slice), rounded to whole XCD rounds).
int inter_one_walk_grid(int32_t n_max, int32_t h, int32_t hv);

// segments: 1 walks each sequence in one piece; 2 to 4 walk that many
// segments of it at once (all but the first carrying the zero-start and the
// homogeneous state) and then combine them with fix-up kernels, using `seg`. tiles: 16-column slices of
// one value head per work-group (1, 2, 4). share: 2 or 4 selects the
// GQA-shared shape instead (one 16-column slice of `share` value heads of a
// key head per work-group; one-piece walk only).
hipError_t launch_inter(bool f32_in, const StageBuffers &in, const float *h0,
                        const int32_t *cu_seqlens, int32_t n_max, int32_t h, int32_t hv,
                        int32_t t_max, int32_t nt_max, float *o, float *hT, hipStream_t stream,
                        KernelEvents ev = {}, int segments = 1, int tiles = 1, int share = 1,
                        SegScratch seg = {});

}  // namespace gdn
