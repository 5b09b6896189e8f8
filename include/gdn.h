/*
 * gdn.h -- C ABI of the MI355X (gfx950) chunked gated-delta-rule prefill forward.
 *
 * The operation (gated delta rule, per sequence s and value head hv, state S of
 * Dk x Dv = 128 x 128 fp32; Alloy page "Chunking Qwen3.5's gated DeltaNet ...",
 * section "What is the gated delta rule in Qwen3.5?"): for each token t the
 * state is decayed by exp(g[t,hv]), corrected by beta[t,hv] * (v_t - S^T k_t),
 * written back as S += k_t d^T, and the output is o_t = scale * S^T q_t, read
 * after the write. It is evaluated in chunks of 64 tokens in two stages whose
 * parallel domains differ ("Optimizing GDN Chunk Prefill on Intel AMX CPU",
 * sections 1 and 3): an intra-chunk stage over [chunks, key heads] producing
 * w and u, and an inter-chunk stage over [sequences, value heads] carrying S.
 *
 * Conventions shared by every entry point
 *  - Pointers marked (device) are device memory owned by the caller. The
 *    library never allocates, never frees, never synchronises, and launches
 *    only on `stream` (a hipStream_t passed as void*, NULL = null stream), so
 *    every call can be captured into a HIP graph.
 *  - Inputs are read-only. Layouts are row-major, packed varlen with batch 1
 *    (AMX page, section 9): token rows [t_max, ...].
 *  - cu_seqlens (device, int32, n_max + 1 entries): cu[0] = 0, non-decreasing,
 *    cu[n_max] <= t_max; unused tail sequences are zero-length (FLA issue 1155,
 *    "Core design"). It is a precondition: it is never read on the host. The
 *    kernels clamp every entry they read to [0, t_max] and never let a
 *    sequence end before it starts, so a malformed cu_seqlens gives
 *    unspecified results but no access outside the buffers that cfg sizes.
 *    Likewise a caller's chunk table entry that names no sequence (< 0 or
 *    >= n_max) or no chunk of its sequence is treated as a sentinel.
 *  - GQA: value head hv reads key/query head hv / (hv_count / h_count) (AMX
 *    page, section 4).
 *  - States h0 / hT: [n_max, hv, dv, dk] fp32, value-major (AMX page, s. 9).
 *  - Errors: every argument and capacity is checked on the host before any
 *    HIP call; a failed check returns a status and touches nothing. A launch
 *    failure returns GDN_ERR_HIP. No call ever aborts the process.
 *  - Magnitudes (chunked forward): stage 2 hands the state S to its w S and
 *    S^T q products, w, the masked intra-chunk attention P and the corrected
 *    values v' to their products as fp16 (fp16 q, k, v and the solve's T s
 *    items too, with fp16 input). fp16's range ends at 65504, so the results
 *    hold the method's tolerance while every entry of S, w, v' (about v's
 *    size) and T s stays below that. With unit-norm keys (the method's L2
 *    normalisation) and beta <= 1, |S| stayed below 0.7 max|v| + max|h0| in
 *    every workload tried; v and h0 scaled by 2^-8 .. 2^12 (max |v| about
 *    1.9e4, with and without decay) meet the tolerance in the GPU tests.
 *    Larger magnitudes overflow to infinity, and a non-finite output is the
 *    sign; the token-serial kernel computes in fp32 throughout.
 *  - Thread safety: the only state the library keeps is a per-device cache of
 *    the compute-unit count (atomic; read by the automatic launch-shape
 *    choices). Concurrent calls on different streams are safe when their
 *    output and workspace buffers are disjoint.
 */
#ifndef GDN_H_
#define GDN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GDN_OK = 0,
  GDN_ERR_INVALID_ARG = 1, /* null pointer, negative size, bad enum */
  GDN_ERR_UNSUPPORTED = 2, /* dk/dv != 128, chunk != 64, hv % h != 0, dtype */
  GDN_ERR_CAPACITY = 3,    /* t_max / n_max beyond what the kernels index */
  GDN_ERR_WORKSPACE = 4,   /* workspace too small or misaligned */
  GDN_ERR_HIP = 5          /* a kernel launch failed */
} gdn_status;

/* Element types. GDN_F16 is accepted for q, k, v by the chunked forward
 * (gdn_chunk_fwd and its stages) and selects fp16 intermediates for the fused
 * front (gdn_chunk_fwd_conv); the token-serial kernel takes bf16 or fp32. */
typedef enum { GDN_BF16 = 0, GDN_F32 = 1, GDN_F16 = 2 } gdn_dtype;

typedef struct {
  int32_t t_max;       /* token capacity (rows of q, k, v, g, beta, o) */
  int32_t n_max;       /* sequence capacity (cu_seqlens has n_max + 1 entries) */
  int32_t h;           /* key / query heads */
  int32_t hv;          /* value heads, a multiple of h */
  int32_t dk, dv;      /* head dims; must both be 128 */
  int32_t chunk;       /* chunk length; must be 64 */
  gdn_dtype qkv_dtype; /* dtype of q, k, v: GDN_BF16, GDN_F32 or GDN_F16 */
  gdn_dtype o_dtype;   /* dtype of o: GDN_F32 (the only one supported) */
  float scale;         /* output scale; <= 0 selects 1 / sqrt(dk) */
  int32_t segments;    /* stage-2 walk of each sequence: 1 = one piece; P = 2, 3
                          or 4 = P segments at once (of a sequence of nc chunks,
                          every later segment y = floor(4 nc / (4P + 1)) chunks,
                          walked from zero and from the identity; the first
                          segment the rest, from the initial state), then fix-ups
                          that chain the segments' states and correct their
                          outputs (the recurrence is affine in the starting
                          state); 0 = automatic: when t_max >=
                          GDN_SEGMENT_MIN_TOKENS, the largest P <= 4 for which P
                          times the one-piece stage-2 grid fits the current
                          device's compute units (1 if none) */
  int32_t tiles;       /* 16-column tiles of the state per stage-2 work-group in the
                          one-piece walk: 1, 2 or 4 (the results are bitwise the same);
                          0 = automatic: 1 when the one-tile grid fits the device, 4
                          when it is more than 2x the device and t_max >= n_max *
                          GDN_FOUR_TILE_MIN_TOKENS (long sequences), else 2. The
                          segmented walk always uses 1. */
  int32_t gqa_share;   /* GQA-shared stage 2 ("Optimizing GDN Chunk Prefill on
                          Intel AMX CPU", sections 3 and 5: the inter stage run
                          over key heads, reusing the key head's operands across
                          its value heads): 2 or 4 = each stage-2 work-group
                          carries one 16-column slice of that many value heads
                          of one key head and loads the key head's K^T and q
                          fragments once for all of them; it must divide hv / h,
                          and needs segments <= 1 and tiles <= 1 (automatic
                          segments and tiles then resolve to 1). 0 or 1 = the
                          column-tile shapes above. Results are bitwise those of
                          tiles = 1. Never chosen automatically: at equal
                          registers per work-group, two or four column tiles of
                          one value head load fewer bytes per column. */
} gdn_config;

/* Token capacity per sequence from which the automatic choice considers
 * four-tile stage-2 work-groups (one per CU: fewer loads per column, but the
 * start and end of each walk are not hidden behind another work-group). */
#define GDN_FOUR_TILE_MIN_TOKENS 384

/* Token capacity from which the automatic choice considers segments. */
#define GDN_SEGMENT_MIN_TOKENS 2048

/* Largest valid gdn_config.t_max / n_max. Each kernel takes at most
 * 2^31 - 1 work-groups per launch. Within these limits only the output fix-up
 * of a segmented walk can need more: about n_max * hv * t_max / 320
 * work-groups with two segments (/ 224 with three, / 192 with four), so with
 * segments >= 2 and n_max * hv * t_max above about 2^38.6 (four segments) to
 * 2^39.3 (two) the forward returns
 * GDN_ERR_CAPACITY. That check runs on the host before anything is queued,
 * like every other check. The automatic choice takes segments only for grids
 * that fit the device several times over, far inside that bound. */
#define GDN_T_MAX_LIMIT (1 << 24)
#define GDN_N_MAX_LIMIT 16384

/* gdn_chunk_fwd without a caller table: up to this many sequences (n_max),
 * each stage-1 work-group locates its chunk from cu_seqlens itself and the
 * table is filled in the workspace by stage 1; beyond it a table kernel runs
 * first. Either way the workspace table ends up as gdn_build_chunk_indices
 * would write it. */
#define GDN_FUSED_INDEX_MAX_SEQS 256

/* Static bound on the number of chunks of any batch of at most t_max tokens in
 * at most n_max sequences: cdiv(t_max, chunk) + n_max - 1 (FLA issue 1155,
 * "Core design"). Returns -1 if an argument is not positive (t_max may be 0). */
int64_t gdn_nt_max(int32_t t_max, int32_t n_max, int32_t chunk);

/* Byte offsets of the intermediates inside a workspace, each 256-byte aligned.
 * The intra stage writes them and the inter stage reads them; their layouts
 * are an internal contract between the two stages (MFMA fragment order: a
 * fragment is 64 lanes x 16 bytes, lane (g, c) = (l / 16, l % 16)), but they
 * are documented so that they can be inspected:
 *   w16   fp16 [hv, nt_max, 16, 64, 8]: -w (AMX page, section 4, negated);
 *         fragment 4 R + p, lane (g, c) holds row 16 R + c, columns
 *         32 p + 4 g + j (j < 4) and 32 p + 16 + 4 g + j - 4 (j >= 4)
 *   q16   fp16 [h, nt_max, 16, 64, 8]: q rounded to fp16, same fragments
 *   kimg  bf16 [h, nt_max, 16 (32 for fp32 or fp16 input), 64, 8]: K^T
 *         fragments (bf16 input: the values; otherwise exact hi + lo terms)
 *   uimg  u32 [hv, nt_max, dv / 16, 4, 64, 3]: u (AMX page, section 4), one
 *         16 x 16 tile per 768-byte block; each lane's four values are 24-bit
 *         floats (the upper three bytes of fp32, rounded to nearest even),
 *         value i in bytes 3 i .. 3 i + 2 of the lane's 12
 *   pimg  fp16 [hv, nt_max, 5 KB]: scale * tril(q k^T * Gamma) as six 16 x 32
 *         fragments; pairs 0 and 3 keep the 8 bytes per lane below the
 *         diagonal (512-byte blocks), the others 16 (1 KB); block offsets
 *         0, 512, 1536, 2560, 3072, 4096
 *   gimg  fp32 [hv, nt_max, 192]: per token e^{gamma_last - gamma} [64],
 *         scale * e^gamma [64] with token 16 R + c at 4 c + R, then
 *         e^{gamma_last}
 *   table int32 [nt_max, 2]: the chunk-index table
 *   order int32 [n_max] when 2 <= n_max <= GDN_FUSED_INDEX_MAX_SEQS, else
 *         empty: the sequence indices ranked by chunk count, longest first
 *         (ties by index). Stage 1 writes it and stage 2 starts the walks in
 *         that order, so that the longest sequences do not start last.
 *   seg_sa fp32 [n_max, hv, dv, dk]: with P >= 2 segments, the state after
 *         the first segment
 *   seg_z fp32 [P - 1][n_max, hv, dv, dk]: each later segment's end state
 *         from zero (then, for all but the last, its true end state)
 *   seg_phi fp32 [P - 1][n_max, hv, dk, dk]: each later segment's
 *         homogeneous end state (the product of its chunk transitions),
 *         key-major
 *   seg_oh fp32 [t_max, hv, dv]: the later segments' homogeneous output rows
 * Per-chunk blocks are indexed by slot floor(t0 / 64) + n for a chunk starting
 * at token t0 of sequence n (distinct per chunk, < nt_max). With automatic
 * segments the size depends on the current device (its compute units). */
typedef struct {
  size_t w16, q16, kimg, uimg, pimg, gimg, table, order;
  size_t seg_sa, seg_z, seg_phi, seg_oh; /* segment scratch (equal to total when the
                                            config resolves to one segment) */
  size_t total; /* bytes of workspace gdn_chunk_fwd needs */
} gdn_workspace_layout_t;

/* Fills *layout for `cfg`; returns a validation status. */
gdn_status gdn_workspace_layout(const gdn_config *cfg, gdn_workspace_layout_t *layout);

/* Bytes of workspace gdn_chunk_fwd needs for `cfg` (layout.total). Writes
 * *bytes; returns a validation status. The size depends on the capacities
 * (t_max, n_max) only, never on a batch's lengths, so one buffer sized once
 * serves every batch of a static shape (FLA issue 1155, "Core design": static
 * buffers sized from the maxima, owned by the caller). */
gdn_status gdn_workspace_size(const gdn_config *cfg, size_t *bytes);

/* Chunk-index table built on the device (FLA issue 1155, "Core design": a
 * searchsorted fill of a fixed [NT_max, 2] buffer, sentinel in unused slots).
 *   cu_seqlens    (device) int32 [n_max + 1]
 *   chunk_indices (device) int32 [nt_max, 2], written: slot j < total chunks
 *                 holds (sequence id, chunk number within the sequence), in
 *                 (sequence, chunk) order; every other slot holds (-1, -1).
 * One work-group; reads cu_seqlens on the device only. */
gdn_status gdn_build_chunk_indices(const gdn_config *cfg, const int32_t *cu_seqlens,
                                   int32_t *chunk_indices, void *stream);

/* Causal depthwise conv + SiLU + per-head L2 norm of q and k, producing the
 * fp32 q, k, v that the chunk forward consumes (llama.cpp PR 399, "How
 * (exactness)": sum over d_conv taps with the current token last, no bias;
 * AMX page, section 7: x / sqrt(sum x^2 + eps), eps = 1e-6).
 *   qkv    (device) bf16 [t_max, 2*h*dk + hv*dv], channels q | k | v, head-major
 *   conv_w (device) bf16 [2*h*dk + hv*dv, d_conv], 1 <= d_conv <= 8
 *   q, k   (device) fp32 [t_max, h, dk]   v (device) fp32 [t_max, hv, dv]
 * History before each sequence start is zero. Rows past cu[n_max] are not
 * written. cfg->qkv_dtype is ignored (the front always reads bf16). */
gdn_status gdn_front_conv_silu_l2(const gdn_config *cfg, const void *qkv, const void *conv_w,
                                  int32_t d_conv, const int32_t *cu_seqlens, float *q, float *k,
                                  float *v, void *stream);

/* Intra-chunk stage over [nt_max, h] (AMX page, section 4): per chunk and key
 * head, K K^T and K q^T once; per value head of the group the beta/decay-masked
 * strictly lower A, T = (I + A)^-1 kept on chip, w = T diag(beta e^gamma) K and
 * u = T diag(beta) V, gamma the chunk-local cumulative g (section 3), and the
 * masked intra-chunk attention P = scale * tril(q k^T * Gamma) of section 5.
 *   q, k (device) [t_max, h, dk]; v (device) [t_max, hv, dv]; dtype qkv_dtype
 *   g, beta (device) fp32 [t_max, hv]
 *   chunk_indices (device) int32 [nt_max, 2] as built by gdn_build_chunk_indices
 *   workspace (device) >= gdn_workspace_size bytes, 256-byte aligned: all the
 *     intermediates of gdn_workspace_layout except the table are written
 *     (token rows of w16 / q16 for valid tokens only).
 * q16 is q rounded to fp16 (exact for bf16 inputs of magnitude >= 2^-14). */
gdn_status gdn_chunk_fwd_intra(const gdn_config *cfg, const void *q, const void *k, const void *v,
                               const float *g, const float *beta, const int32_t *cu_seqlens,
                               const int32_t *chunk_indices, void *workspace, size_t ws_bytes,
                               void *stream);

/* Inter-chunk stage over [n_max, hv, dv / 16] (AMX page, section 5), or with
 * P segments over P times that grid plus fix-ups (cfg->segments): chunks in
 * order with S on chip: v' = u - w S; o = scale (diag(e^gamma) q S +
 * tril(q k^T * Gamma) v'); S = e^{gamma_last} S + (diag(e^{gamma_last - gamma}) k)^T v',
 * Gamma[r, i] = exp(gamma_r - gamma_i) for i <= r (diagonal kept). Reads only
 * the intermediates gdn_chunk_fwd_intra wrote into `workspace` for the same
 * cfg and cu_seqlens.
 *   h0 (device, nullable = zero state) fp32 [n_max, hv, dv, dk];
 *   o  (device) fp32 [t_max, hv, dv]: valid rows written, others untouched;
 *   hT (device, nullable) fp32 [n_max, hv, dv, dk]; hT may alias h0 exactly.
 * A zero-length sequence writes hT = h0 (or zeros when h0 is null). */
gdn_status gdn_chunk_fwd_inter(const gdn_config *cfg, const float *h0, const int32_t *cu_seqlens,
                               const void *workspace, size_t ws_bytes, void *o, float *hT,
                               void *stream);

/* Whole forward: [chunk table if chunk_indices is NULL and n_max >
 * GDN_FUSED_INDEX_MAX_SEQS] -> intra -> inter, all on `stream`, no host
 * synchronisation. This is the AMX page's section 3 wrapper (q, k, v, g,
 * beta, an optional initial state and cu_seqlens in; o and the final state
 * out), with FLA issue 1155's capture rules ("Core design": an optional
 * caller-built chunk table, caller-owned static workspace, no host read of
 * cu_seqlens). Arguments as above; workspace (device) of at least
 * gdn_workspace_size bytes, 256-byte aligned, holds the intermediates and the
 * table between the stages (when chunk_indices is NULL the table is built in
 * it, by the table kernel or by stage 1) and may be reused once the stream
 * passes the call. */
gdn_status gdn_chunk_fwd(const gdn_config *cfg, const void *q, const void *k, const void *v,
                         const float *g, const float *beta, const float *h0,
                         const int32_t *cu_seqlens, const int32_t *chunk_indices, void *o,
                         float *hT, void *workspace, size_t ws_bytes, void *stream);

/* Bytes of the library's fixed device scratch used by gdn_chunk_fwd_noalloc
 * (256 MiB; one copy per GPU the library runs that call on, held until the
 * process ends). */
#define GDN_NOALLOC_SCRATCH_BYTES (256 << 20)

/* gdn_chunk_fwd without a caller workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, hosts
 * that forbid allocation after start-up). The intermediates go to a fixed
 * device array inside the library, GDN_NOALLOC_SCRATCH_BYTES per device,
 * whose address is looked up once per device on the first call with that
 * device current. The call allocates nothing and frees nothing.
 *   Arguments, layouts and results as gdn_chunk_fwd (workspace omitted).
 *   Returns GDN_ERR_WORKSPACE when gdn_workspace_size(cfg) exceeds
 *   GDN_NOALLOC_SCRATCH_BYTES (for example T = 4096 tokens at h = 16, hv = 32
 *   needs about 134 MiB; about 7,800 tokens fit at those head counts), before
 *   anything is queued.
 * All calls on one device share its array: calls that overlap in time on one
 * device (different streams, or threads enqueueing concurrently) race, and
 * the caller must order them. Nothing in the array has to start at zero. */
gdn_status gdn_chunk_fwd_noalloc(const gdn_config *cfg, const void *q, const void *k,
                                 const void *v, const float *g, const float *beta,
                                 const float *h0, const int32_t *cu_seqlens,
                                 const int32_t *chunk_indices, void *o, float *hT, void *stream);

/* Whole forward with the front fused into the intra stage (the "next" step
 * after gdn_front_conv_silu_l2 + gdn_chunk_fwd): each stage-1 work-group
 * computes its chunk's q, k (conv, SiLU, per-head L2 norm) and v (conv,
 * SiLU) itself from the pre-conv channels, reading a (d_conv - 1)-token halo
 * before the chunk (zero before each sequence start), with the same fp32
 * arithmetic as gdn_front_conv_silu_l2 (llama.cpp PR 399, "How (exactness)";
 * AMX page, section 7). The q, k, v never reach HBM.
 *   qkv    (device) bf16 [t_max, 2*h*dk + hv*dv], channels q | k | v, head-major
 *   conv_w (device) bf16 [2*h*dk + hv*dv, d_conv], 1 <= d_conv <= 4
 *   cfg->qkv_dtype selects the precision the front's q, k, v enter the chunk
 *   forward in: GDN_F32 keeps them in fp32, and the result equals
 *   gdn_front_conv_silu_l2 followed by gdn_chunk_fwd (GDN_F32) on its
 *   outputs; GDN_F16 rounds them to fp16 (nearest even), and the result
 *   equals gdn_front_conv_silu_l2, its outputs rounded to fp16, then
 *   gdn_chunk_fwd (GDN_F16). fp16 runs stage 1 at twice the occupancy with
 *   one-term products; the rounding adds about 3e-4 of max |o| to the error.
 *   The workspace is sized with the same cfg; other arguments as gdn_chunk_fwd. */
gdn_status gdn_chunk_fwd_conv(const gdn_config *cfg, const void *qkv, const void *conv_w,
                              int32_t d_conv, const float *g, const float *beta, const float *h0,
                              const int32_t *cu_seqlens, const int32_t *chunk_indices, void *o,
                              float *hT, void *workspace, size_t ws_bytes, void *stream);

/* Token-serial recurrent forward, for decode and speculative verify (1 to 16
 * tokens per sequence is its purpose; any length is computed). Each sequence's
 * tokens are applied one at a time in fp32, in the order of the Alloy page's
 * section "What is the gated delta rule in Qwen3.5?": S <- e^{g_t} S,
 * d = beta_t (v_t - S^T k_t), S <- S + k_t d^T, o_t = scale S^T q_t. The state
 * stays on chip between tokens (section "How does decode run a sequential
 * update on a GPU?"), and a verify batch reproduces decode's arithmetic
 * token by token (section "Why keep the serial kernel at all?"; llama.cpp PR
 * 399, "What": verify widths of 1 to 16 tokens). No workspace.
 *   q, k (device) [t_max, h, dk]; v (device) [t_max, hv, dv]; dtype qkv_dtype
 *   g, beta (device) fp32 [t_max, hv]
 *   h0 (device, nullable = zero state) fp32 [n_max, hv, dv, dk]
 *   o  (device) fp32 [t_max, hv, dv]: valid rows written, others untouched
 *   hT (device, nullable) fp32 [n_max, hv, dv, dk]; hT may alias h0 exactly.
 * cfg->chunk must be valid (64) but is not used. A zero-length sequence writes
 * hT = h0 (or zeros when h0 is null). */
gdn_status gdn_recurrent_fwd(const gdn_config *cfg, const void *q, const void *k, const void *v,
                             const float *g, const float *beta, const float *h0,
                             const int32_t *cu_seqlens, void *o, float *hT, void *stream);

/* Timed variants, for measurement. They behave exactly like the entry point
 * they extend, and in addition each kernel they launch records a pair of HIP
 * events at its own start and end (the dispatch itself records them, so no
 * packet is added between launches and the elapsed time between a pair is
 * the kernel's execution time).
 *   events (host array of 6 hipEvent_t passed as void*, each created by the
 *          caller): [0], [1] around the chunk table kernel (recorded only when
 *          that kernel runs: chunk_indices NULL and n_max >
 *          GDN_FUSED_INDEX_MAX_SEQS), [2], [3] around the intra stage, [4],
 *          [5] around the inter stage.
 *   ev_start, ev_stop: around the front kernel (the recurrent kernel).
 * A NULL event returns GDN_ERR_INVALID_ARG before any launch. */
gdn_status gdn_chunk_fwd_timed(const gdn_config *cfg, const void *q, const void *k, const void *v,
                               const float *g, const float *beta, const float *h0,
                               const int32_t *cu_seqlens, const int32_t *chunk_indices, void *o,
                               float *hT, void *workspace, size_t ws_bytes, void *stream,
                               void *const *events);
gdn_status gdn_front_conv_silu_l2_timed(const gdn_config *cfg, const void *qkv,
                                        const void *conv_w, int32_t d_conv,
                                        const int32_t *cu_seqlens, float *q, float *k, float *v,
                                        void *stream, void *ev_start, void *ev_stop);
gdn_status gdn_chunk_fwd_conv_timed(const gdn_config *cfg, const void *qkv, const void *conv_w,
                                    int32_t d_conv, const float *g, const float *beta,
                                    const float *h0, const int32_t *cu_seqlens,
                                    const int32_t *chunk_indices, void *o, float *hT,
                                    void *workspace, size_t ws_bytes, void *stream,
                                    void *const *events);

gdn_status gdn_recurrent_fwd_timed(const gdn_config *cfg, const void *q, const void *k,
                                   const void *v, const float *g, const float *beta,
                                   const float *h0, const int32_t *cu_seqlens, void *o, float *hT,
                                   void *stream, void *ev_start, void *ev_stop);

/* Static string for a status code (never NULL). */
const char *gdn_status_str(gdn_status status);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H_ */
