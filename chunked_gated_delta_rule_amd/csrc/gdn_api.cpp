// C ABI of the gfx950 GDN chunk-prefill library (declared in include/gdn.h).
//
// Every entry point validates all of its arguments on the host first and
// returns a status without touching the GPU when a check fails; only then does
// it enqueue kernels on the caller's stream. Nothing here allocates, frees or
// synchronises, so a call can be captured into a HIP graph.
#include "gdn.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "gdn_launch.hpp"

namespace {

constexpr int kD = 128;
constexpr int kChunk = 64;
constexpr int kMaxHeads = 4096;
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

gdn_status check_config(const gdn_config *cfg) {
  if (!cfg) return GDN_ERR_INVALID_ARG;
  if (cfg->t_max < 0 || cfg->n_max < 1 || cfg->h < 1 || cfg->hv < 1) return GDN_ERR_INVALID_ARG;
  if (cfg->qkv_dtype != GDN_BF16 && cfg->qkv_dtype != GDN_F32 && cfg->qkv_dtype != GDN_F16)
    return GDN_ERR_INVALID_ARG;
  if (cfg->o_dtype != GDN_BF16 && cfg->o_dtype != GDN_F32) return GDN_ERR_INVALID_ARG;
  if (std::isnan(cfg->scale) || std::isinf(cfg->scale)) return GDN_ERR_INVALID_ARG;
  if (cfg->segments < 0 || cfg->segments > 4) return GDN_ERR_INVALID_ARG;
  if (cfg->tiles != 0 && cfg->tiles != 1 && cfg->tiles != 2 && cfg->tiles != 4)
    return GDN_ERR_INVALID_ARG;
  if (cfg->gqa_share != 0 && cfg->gqa_share != 1 && cfg->gqa_share != 2 && cfg->gqa_share != 4)
    return GDN_ERR_INVALID_ARG;
  if (cfg->dk != kD || cfg->dv != kD || cfg->chunk != kChunk) return GDN_ERR_UNSUPPORTED;
  if (cfg->hv % cfg->h != 0) return GDN_ERR_UNSUPPORTED;
  if (cfg->gqa_share > 1 && ((cfg->hv / cfg->h) % cfg->gqa_share != 0 || cfg->segments >= 2 ||
                             cfg->tiles > 1))
    return GDN_ERR_UNSUPPORTED;
  if (cfg->o_dtype != GDN_F32) return GDN_ERR_UNSUPPORTED;
  if (cfg->t_max > GDN_T_MAX_LIMIT || cfg->n_max > GDN_N_MAX_LIMIT || cfg->hv > kMaxHeads)
    return GDN_ERR_CAPACITY;
  return GDN_OK;
}

int32_t nt_max_of(const gdn_config *cfg) {
  return static_cast<int32_t>((static_cast<int64_t>(cfg->t_max) + kChunk - 1) / kChunk +
                              cfg->n_max - 1);
}

// Stage-2 segments of a (validated) config: automatic = when t_max allows long
// sequences, the most segments (up to 4) whose walks together still fit the
// device at one work-group per CU (segments beyond that measured slower).
int segments_of(const gdn_config *cfg) {
  if (cfg->segments != 0) return cfg->segments;
  if (cfg->gqa_share > 1) return 1;
  if (cfg->t_max < GDN_SEGMENT_MIN_TOKENS) return 1;
  const int64_t one = gdn::inter_one_walk_grid(cfg->n_max, cfg->h, cfg->hv);
  int parts = 1;
  for (int p = 2; p <= 4; ++p)
    if (p * one <= gdn::cu_count()) parts = p;
  return parts;
}

// 16-column tiles per work-group of the one-piece stage-2 walk (validated
// config).
int tiles_of(const gdn_config *cfg) {
  if (cfg->tiles != 0) return cfg->tiles;
  if (cfg->gqa_share > 1) return 1;
  const int64_t one = gdn::inter_one_walk_grid(cfg->n_max, cfg->h, cfg->hv);
  const int64_t cus = gdn::cu_count();
  if (one <= cus) return 1;
  if (one > 2 * cus &&
      static_cast<int64_t>(cfg->t_max) >= static_cast<int64_t>(cfg->n_max) * GDN_FOUR_TILE_MIN_TOKENS)
    return 4;
  return 2;
}

// Value heads per GQA-shared stage-2 work-group (validated config; 1 = the
// column-tile shapes).
int share_of(const gdn_config *cfg) { return cfg->gqa_share > 1 ? cfg->gqa_share : 1; }

// Whether stage 1 ranks the sequences for stage 2 (longest walks first): with
// more than one sequence, up to one per stage-1 thread.
bool ranks_sequences(const gdn_config *cfg) {
  return cfg->n_max >= 2 && cfg->n_max <= GDN_FUSED_INDEX_MAX_SEQS;
}

gdn_workspace_layout_t layout_of(const gdn_config *cfg) {
  const size_t t = static_cast<size_t>(cfg->t_max), nt = static_cast<size_t>(nt_max_of(cfg));
  const size_t h = static_cast<size_t>(cfg->h), hv = static_cast<size_t>(cfg->hv);
  const size_t nk = cfg->qkv_dtype == GDN_BF16 ? 16 : 32;  // K^T terms (hi[, lo])
  gdn_workspace_layout_t l;
  size_t at = 0;
  auto take = [&](size_t bytes) { const size_t here = at; at += align_up(bytes); return here; };
  l.w16 = take(hv * nt * 16 * 1024);
  l.q16 = take(h * nt * 16 * 1024);
  l.kimg = take(h * nt * nk * 1024);
  l.uimg = take(hv * nt * kD * kChunk * 3);  // 24-bit u
  l.pimg = take(hv * nt * gdn::kPBytes);
  l.gimg = take(hv * nt * 192 * 4);
  l.table = take(nt * 2 * 4);
  l.order = take(ranks_sequences(cfg) ? static_cast<size_t>(cfg->n_max) * 4 : 0);
  const int parts = segments_of(cfg);
  if (parts >= 2) {
    const size_t state = static_cast<size_t>(cfg->n_max) * hv * kD * kD * 4;
    l.seg_sa = take(state);
    l.seg_z = take((parts - 1) * state);
    l.seg_phi = take((parts - 1) * state);
    l.seg_oh = take(t * hv * kD * 4);
  } else {
    l.seg_sa = l.seg_z = l.seg_phi = l.seg_oh = at;
  }
  l.total = at;
  return l;
}

gdn::SegScratch seg_scratch(const gdn_config *cfg, const gdn_workspace_layout_t &l,
                            const void *workspace) {
  char *ws = static_cast<char *>(const_cast<void *>(workspace));
  gdn::SegScratch g;
  g.sa = reinterpret_cast<float *>(ws + l.seg_sa);
  g.z = reinterpret_cast<float *>(ws + l.seg_z);
  g.phi = reinterpret_cast<float *>(ws + l.seg_phi);
  g.oh = reinterpret_cast<float *>(ws + l.seg_oh);
  g.state_elems = static_cast<int64_t>(cfg->n_max) * cfg->hv * kD * kD;
  g.parts = segments_of(cfg);
  return g;
}

gdn::StageBuffers stage_buffers(const gdn_config *cfg, const gdn_workspace_layout_t &l,
                                const void *workspace) {
  char *ws = static_cast<char *>(const_cast<void *>(workspace));
  gdn::StageBuffers b;
  b.w16 = reinterpret_cast<_Float16 *>(ws + l.w16);
  b.q16 = reinterpret_cast<_Float16 *>(ws + l.q16);
  b.kimg = reinterpret_cast<__bf16 *>(ws + l.kimg);
  b.uimg = reinterpret_cast<uint32_t *>(ws + l.uimg);
  b.pimg = reinterpret_cast<_Float16 *>(ws + l.pimg);
  b.gimg = reinterpret_cast<float *>(ws + l.gimg);
  // stage 1 writes the ranking; with t_max == 0 it does not run, so stage 2
  // must not read the (unwritten) table
  b.order = ranks_sequences(cfg) && cfg->t_max > 0 ? reinterpret_cast<int32_t *>(ws + l.order)
                                                   : nullptr;
  return b;
}

// Workspace present, large enough and 256-byte aligned.
gdn_status check_workspace(const gdn_workspace_layout_t &l, const void *ws, size_t ws_bytes) {
  if (!ws || ws_bytes < l.total) return GDN_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(ws) % kAlign) return GDN_ERR_WORKSPACE;
  return GDN_OK;
}

float scale_of(const gdn_config *cfg) {
  return cfg->scale > 0.f ? cfg->scale : 1.0f / std::sqrt(static_cast<float>(cfg->dk));
}

gdn_status from_hip(hipError_t e) { return e == hipSuccess ? GDN_OK : GDN_ERR_HIP; }

// How stage 1 takes q, k, v; stage 2 reads bf16 input's intermediates in one
// layout and fp32 / fp16 input's (K^T as bf16 hi + lo) in the other.
gdn::InKind in_kind(const gdn_config *cfg) {
  return cfg->qkv_dtype == GDN_F32 ? gdn::InKind::kF32
         : cfg->qkv_dtype == GDN_F16 ? gdn::InKind::kF16
                                     : gdn::InKind::kBf16;
}
bool split_k(const gdn_config *cfg) { return cfg->qkv_dtype != GDN_BF16; }

// Every stage-2 grid of a (validated) config fits one launch; checked before
// anything is queued, so a config past the limits returns without side effects.
gdn_status check_inter_grids(const gdn_config *cfg) {
  return gdn::inter_grids_fit(cfg->n_max, cfg->h, cfg->hv, cfg->t_max, segments_of(cfg),
                              tiles_of(cfg), share_of(cfg))
             ? GDN_OK
             : GDN_ERR_CAPACITY;
}

hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

// Shared bodies of the plain and the timed entry points.
gdn_status front_impl(const gdn_config *cfg, const void *qkv, const void *conv_w, int32_t d_conv,
                      const int32_t *cu_seqlens, float *q, float *k, float *v, void *stream,
                      gdn::KernelEvents ev) {
  const gdn_status st = check_config(cfg);
  if (st != GDN_OK) return st;
  if (!qkv || !conv_w || !cu_seqlens || !q || !k || !v) return GDN_ERR_INVALID_ARG;
  if (!aligned16(qkv) || !aligned16(q) || !aligned16(k) || !aligned16(v) ||
      (reinterpret_cast<uintptr_t>(conv_w) & 1u) || (reinterpret_cast<uintptr_t>(cu_seqlens) & 3u))
    return GDN_ERR_INVALID_ARG;
  if (d_conv < 1 || d_conv > 8) return GDN_ERR_UNSUPPORTED;
  return from_hip(gdn::launch_front(qkv, conv_w, d_conv, cu_seqlens, cfg->n_max, cfg->t_max,
                                    cfg->h, cfg->hv, q, k, v, as_stream(stream), ev));
}

gdn_status chunk_fwd_impl(const gdn_config *cfg, const void *q, const void *k, const void *v,
                          const float *g, const float *beta, const float *h0,
                          const int32_t *cu_seqlens, const int32_t *chunk_indices, void *o,
                          float *hT, void *workspace, size_t ws_bytes, void *stream,
                          const gdn::KernelEvents (&ev)[3], const gdn::ConvIn &conv = {}) {
  const gdn_status st = check_config(cfg);
  if (st != GDN_OK) return st;
  if (conv.qkv) {  // fused front: q, k, v come from the pre-conv channels
    if (!conv.conv_w) return GDN_ERR_INVALID_ARG;
    if (!aligned16(conv.qkv) || (reinterpret_cast<uintptr_t>(conv.conv_w) & 1u))
      return GDN_ERR_INVALID_ARG;
    if (conv.d_conv < 1 || conv.d_conv > 4 || cfg->qkv_dtype == GDN_BF16) return GDN_ERR_UNSUPPORTED;
    q = k = v = conv.qkv;
  }
  if (!q || !k || !v || !g || !beta || !cu_seqlens || !o) return GDN_ERR_INVALID_ARG;
  const gdn_workspace_layout_t l = layout_of(cfg);
  const gdn_status ws = check_workspace(l, workspace, ws_bytes);
  if (ws != GDN_OK) return ws;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
      (h0 && !aligned16(h0)) || (hT && !aligned16(hT)) ||
      (chunk_indices && !aligned16(chunk_indices)) || (reinterpret_cast<uintptr_t>(g) & 3u) ||
      (reinterpret_cast<uintptr_t>(beta) & 3u) || (reinterpret_cast<uintptr_t>(cu_seqlens) & 3u))
    return GDN_ERR_INVALID_ARG;
  const gdn_status grids = check_inter_grids(cfg);
  if (grids != GDN_OK) return grids;
  hipStream_t s = as_stream(stream);
  int32_t *ws_table = reinterpret_cast<int32_t *>(static_cast<char *>(workspace) + l.table);
  if (!chunk_indices && cfg->n_max > GDN_FUSED_INDEX_MAX_SEQS) {
    const hipError_t e =
        gdn::launch_chunk_index(cu_seqlens, cfg->n_max, nt_max_of(cfg), cfg->t_max, ws_table, s,
                                ev[0]);
    if (e != hipSuccess) return GDN_ERR_HIP;
    chunk_indices = ws_table;
  }
  const gdn::StageBuffers b = stage_buffers(cfg, l, workspace);
  if (cfg->t_max > 0) {
    // without a table, stage 1 locates its chunks and fills ws_table itself
    const hipError_t e = gdn::launch_intra(in_kind(cfg), q, k, v, g, beta, cu_seqlens,
                                           chunk_indices, ws_table, cfg->n_max, nt_max_of(cfg),
                                           cfg->h, cfg->hv, cfg->t_max, scale_of(cfg), b, s, ev[1],
                                           conv);
    if (e != hipSuccess) return GDN_ERR_HIP;
  }
  return from_hip(gdn::launch_inter(split_k(cfg), b, h0, cu_seqlens, cfg->n_max,
                                    cfg->h, cfg->hv, cfg->t_max, nt_max_of(cfg),
                                    static_cast<float *>(o), hT, s, ev[2], segments_of(cfg),
                                    tiles_of(cfg), share_of(cfg), seg_scratch(cfg, l, workspace)));
}

gdn_status recurrent_impl(const gdn_config *cfg, const void *q, const void *k, const void *v,
                          const float *g, const float *beta, const float *h0,
                          const int32_t *cu_seqlens, void *o, float *hT, void *stream,
                          gdn::KernelEvents ev) {
  const gdn_status st = check_config(cfg);
  if (st != GDN_OK) return st;
  if (!q || !k || !v || !g || !beta || !cu_seqlens || !o) return GDN_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
      (h0 && !aligned16(h0)) || (hT && !aligned16(hT)) || (reinterpret_cast<uintptr_t>(g) & 3u) ||
      (reinterpret_cast<uintptr_t>(beta) & 3u) || (reinterpret_cast<uintptr_t>(cu_seqlens) & 3u))
    return GDN_ERR_INVALID_ARG;
  if (cfg->qkv_dtype == GDN_F16) return GDN_ERR_UNSUPPORTED;
  return from_hip(gdn::launch_recurrent(cfg->qkv_dtype == GDN_F32, q, k, v, g, beta, h0,
                                        cu_seqlens, cfg->n_max, cfg->t_max, cfg->h, cfg->hv,
                                        scale_of(cfg),
                                        static_cast<float *>(o), hT, as_stream(stream), ev));
}

}  // namespace

extern "C" {

int64_t gdn_nt_max(int32_t t_max, int32_t n_max, int32_t chunk) {
  if (t_max < 0 || n_max < 1 || chunk < 1) return -1;
  return (static_cast<int64_t>(t_max) + chunk - 1) / chunk + n_max - 1;
}

gdn_status gdn_workspace_layout(const gdn_config *cfg, gdn_workspace_layout_t *layout) {
  const gdn_status st = check_config(cfg);
  if (st != GDN_OK) return st;
  if (!layout) return GDN_ERR_INVALID_ARG;
  *layout = layout_of(cfg);
  return GDN_OK;
}

gdn_status gdn_workspace_size(const gdn_config *cfg, size_t *bytes) {
  const gdn_status st = check_config(cfg);
  if (st != GDN_OK) return st;
  if (!bytes) return GDN_ERR_INVALID_ARG;
  *bytes = layout_of(cfg).total;
  return GDN_OK;
}

gdn_status gdn_build_chunk_indices(const gdn_config *cfg, const int32_t *cu_seqlens,
                                   int32_t *chunk_indices, void *stream) {
  const gdn_status st = check_config(cfg);
  if (st != GDN_OK) return st;
  if (!cu_seqlens || !chunk_indices || !aligned16(chunk_indices) ||
      (reinterpret_cast<uintptr_t>(cu_seqlens) & 3u))
    return GDN_ERR_INVALID_ARG;
  return from_hip(gdn::launch_chunk_index(cu_seqlens, cfg->n_max, nt_max_of(cfg), cfg->t_max,
                                          chunk_indices,
                                          as_stream(stream)));
}

gdn_status gdn_front_conv_silu_l2(const gdn_config *cfg, const void *qkv, const void *conv_w,
                                  int32_t d_conv, const int32_t *cu_seqlens, float *q, float *k,
                                  float *v, void *stream) {
  return front_impl(cfg, qkv, conv_w, d_conv, cu_seqlens, q, k, v, stream, {});
}

gdn_status gdn_front_conv_silu_l2_timed(const gdn_config *cfg, const void *qkv,
                                        const void *conv_w, int32_t d_conv,
                                        const int32_t *cu_seqlens, float *q, float *k, float *v,
                                        void *stream, void *ev_start, void *ev_stop) {
  if (!ev_start || !ev_stop) return GDN_ERR_INVALID_ARG;
  return front_impl(cfg, qkv, conv_w, d_conv, cu_seqlens, q, k, v, stream,
                    {static_cast<hipEvent_t>(ev_start), static_cast<hipEvent_t>(ev_stop)});
}

gdn_status gdn_chunk_fwd_intra(const gdn_config *cfg, const void *q, const void *k, const void *v,
                               const float *g, const float *beta, const int32_t *cu_seqlens,
                               const int32_t *chunk_indices, void *workspace, size_t ws_bytes,
                               void *stream) {
  const gdn_status st = check_config(cfg);
  if (st != GDN_OK) return st;
  if (!q || !k || !v || !g || !beta || !cu_seqlens || !chunk_indices) return GDN_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(chunk_indices) ||
      (reinterpret_cast<uintptr_t>(g) & 3u) || (reinterpret_cast<uintptr_t>(beta) & 3u) ||
      (reinterpret_cast<uintptr_t>(cu_seqlens) & 3u))
    return GDN_ERR_INVALID_ARG;
  const gdn_workspace_layout_t l = layout_of(cfg);
  const gdn_status ws = check_workspace(l, workspace, ws_bytes);
  if (ws != GDN_OK) return ws;
  if (cfg->t_max == 0) return GDN_OK;
  return from_hip(gdn::launch_intra(in_kind(cfg), q, k, v, g, beta, cu_seqlens,
                                    chunk_indices, nullptr, cfg->n_max, nt_max_of(cfg), cfg->h,
                                    cfg->hv, cfg->t_max, scale_of(cfg), stage_buffers(cfg, l, workspace),
                                    as_stream(stream)));
}

gdn_status gdn_chunk_fwd_inter(const gdn_config *cfg, const float *h0, const int32_t *cu_seqlens,
                               const void *workspace, size_t ws_bytes, void *o, float *hT,
                               void *stream) {
  const gdn_status st = check_config(cfg);
  if (st != GDN_OK) return st;
  if (!cu_seqlens || !o) return GDN_ERR_INVALID_ARG;
  if (!aligned16(o) || (h0 && !aligned16(h0)) || (hT && !aligned16(hT)) ||
      (reinterpret_cast<uintptr_t>(cu_seqlens) & 3u))
    return GDN_ERR_INVALID_ARG;
  const gdn_workspace_layout_t l = layout_of(cfg);
  const gdn_status ws = check_workspace(l, workspace, ws_bytes);
  if (ws != GDN_OK) return ws;
  const gdn_status grids = check_inter_grids(cfg);
  if (grids != GDN_OK) return grids;
  return from_hip(gdn::launch_inter(split_k(cfg), stage_buffers(cfg, l, workspace), h0,
                                    cu_seqlens, cfg->n_max, cfg->h, cfg->hv, cfg->t_max,
                                    nt_max_of(cfg), static_cast<float *>(o), hT, as_stream(stream),
                                    {}, segments_of(cfg), tiles_of(cfg), share_of(cfg),
                                    seg_scratch(cfg, l, workspace)));
}

gdn_status gdn_chunk_fwd(const gdn_config *cfg, const void *q, const void *k, const void *v,
                         const float *g, const float *beta, const float *h0,
                         const int32_t *cu_seqlens, const int32_t *chunk_indices, void *o,
                         float *hT, void *workspace, size_t ws_bytes, void *stream) {
  const gdn::KernelEvents none[3] = {};
  return chunk_fwd_impl(cfg, q, k, v, g, beta, h0, cu_seqlens, chunk_indices, o, hT, workspace,
                        ws_bytes, stream, none);
}

gdn_status gdn_chunk_fwd_timed(const gdn_config *cfg, const void *q, const void *k, const void *v,
                               const float *g, const float *beta, const float *h0,
                               const int32_t *cu_seqlens, const int32_t *chunk_indices, void *o,
                               float *hT, void *workspace, size_t ws_bytes, void *stream,
                               void *const *events) {
  if (!events) return GDN_ERR_INVALID_ARG;
  for (int i = 0; i < 6; ++i)
    if (!events[i]) return GDN_ERR_INVALID_ARG;
  gdn::KernelEvents ev[3];
  for (int i = 0; i < 3; ++i)
    ev[i] = {static_cast<hipEvent_t>(events[2 * i]), static_cast<hipEvent_t>(events[2 * i + 1])};
  return chunk_fwd_impl(cfg, q, k, v, g, beta, h0, cu_seqlens, chunk_indices, o, hT, workspace,
                        ws_bytes, stream, ev);
}

gdn_status gdn_chunk_fwd_conv(const gdn_config *cfg, const void *qkv, const void *conv_w,
                              int32_t d_conv, const float *g, const float *beta, const float *h0,
                              const int32_t *cu_seqlens, const int32_t *chunk_indices, void *o,
                              float *hT, void *workspace, size_t ws_bytes, void *stream) {
  if (!qkv) return GDN_ERR_INVALID_ARG;
  const gdn::KernelEvents none[3] = {};
  gdn::ConvIn conv;
  conv.qkv = static_cast<const uint16_t *>(qkv);
  conv.conv_w = static_cast<const uint16_t *>(conv_w);
  conv.d_conv = d_conv;
  return chunk_fwd_impl(cfg, nullptr, nullptr, nullptr, g, beta, h0, cu_seqlens, chunk_indices, o,
                        hT, workspace, ws_bytes, stream, none, conv);
}

gdn_status gdn_chunk_fwd_conv_timed(const gdn_config *cfg, const void *qkv, const void *conv_w,
                                    int32_t d_conv, const float *g, const float *beta,
                                    const float *h0, const int32_t *cu_seqlens,
                                    const int32_t *chunk_indices, void *o, float *hT,
                                    void *workspace, size_t ws_bytes, void *stream,
                                    void *const *events) {
  if (!qkv || !events) return GDN_ERR_INVALID_ARG;
  for (int i = 0; i < 6; ++i)
    if (!events[i]) return GDN_ERR_INVALID_ARG;
  gdn::KernelEvents ev[3];
  for (int i = 0; i < 3; ++i)
    ev[i] = {static_cast<hipEvent_t>(events[2 * i]), static_cast<hipEvent_t>(events[2 * i + 1])};
  gdn::ConvIn conv;
  conv.qkv = static_cast<const uint16_t *>(qkv);
  conv.conv_w = static_cast<const uint16_t *>(conv_w);
  conv.d_conv = d_conv;
  return chunk_fwd_impl(cfg, nullptr, nullptr, nullptr, g, beta, h0, cu_seqlens, chunk_indices, o,
                        hT, workspace, ws_bytes, stream, ev, conv);
}

gdn_status gdn_recurrent_fwd(const gdn_config *cfg, const void *q, const void *k, const void *v,
                             const float *g, const float *beta, const float *h0,
                             const int32_t *cu_seqlens, void *o, float *hT, void *stream) {
  return recurrent_impl(cfg, q, k, v, g, beta, h0, cu_seqlens, o, hT, stream, {});
}

gdn_status gdn_recurrent_fwd_timed(const gdn_config *cfg, const void *q, const void *k,
                                   const void *v, const float *g, const float *beta,
                                   const float *h0, const int32_t *cu_seqlens, void *o, float *hT,
                                   void *stream, void *ev_start, void *ev_stop) {
  if (!ev_start || !ev_stop) return GDN_ERR_INVALID_ARG;
  return recurrent_impl(cfg, q, k, v, g, beta, h0, cu_seqlens, o, hT, stream,
                        {static_cast<hipEvent_t>(ev_start), static_cast<hipEvent_t>(ev_stop)});
}

const char *gdn_status_str(gdn_status status) {
  switch (status) {
    case GDN_OK: return "GDN_OK";
    case GDN_ERR_INVALID_ARG: return "GDN_ERR_INVALID_ARG";
    case GDN_ERR_UNSUPPORTED: return "GDN_ERR_UNSUPPORTED";
    case GDN_ERR_CAPACITY: return "GDN_ERR_CAPACITY";
    case GDN_ERR_WORKSPACE: return "GDN_ERR_WORKSPACE";
    case GDN_ERR_HIP: return "GDN_ERR_HIP";
  }
  return "GDN_ERR_UNKNOWN";
}

}  // extern "C"
