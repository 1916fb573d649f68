/*
 * vmla.h -- C ABI of libvmla.so: latent-KV chunk attention for streaming video
 * diffusion on AMD Instinct MI355X (gfx950).
 *
 * What the library computes is the self-attention layer of VideoMLA ("VideoMLA:
 * Low-Rank Latent KV Cache for Minute-Scale Autoregressive Video Diffusion",
 * sections 3.1-3.3 and appendices C.1, D.1, D.4): every cached token keeps one
 * head-shared content latent c (d_c scalars) and one head-shared decoupled
 * 3D-RoPE key k_r (d_rope scalars) in a sliding window of latent frames, and a
 * chunk of query frames attends to that window plus itself.  Queries are
 * absorbed into latent space through W_UK and outputs are lifted through W_UV
 * (the Multi-Head Latent Attention rearrangement the paper builds on), so the
 * per-head keys and values are never materialised.
 *
 * Conventions shared by every entry point
 *   - All device memory (weights, cache, workspace, x, out) is owned by the
 *     caller.  The library borrows the pointers; it never allocates, frees or
 *     copies device memory on the host's behalf.  Weights, cache and workspace
 *     must stay valid, unmoved and (for weights) unchanged for the life of a ctx.
 *   - Every device pointer must be 16-byte aligned.
 *   - Element type of all tensors is the config's dtype (bf16 or f32), row-major.
 *     Weights use the torch.nn.Linear layout [out_features, in_features].
 *   - Calls enqueue work on the given HIP stream and return without waiting.
 *     All argument checks happen before anything is enqueued; on a non-zero
 *     status nothing was enqueued and the ctx is unchanged.  Launch failures are
 *     reported as VMLA_ERR_HIP (from hipGetLastError after the launch).
 *   - A ctx is not thread-safe; all calls on one ctx must be issued in one stream
 *     order.  No exception crosses the ABI.
 */
#ifndef VMLA_H
#define VMLA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define VMLA_API __attribute__((visibility("default")))

/* status codes */
enum {
  VMLA_OK = 0,
  VMLA_ERR_NULL = 1,        /* a required pointer argument is NULL */
  VMLA_ERR_CONFIG = 2,      /* config fields out of range or inconsistent */
  VMLA_ERR_UNSUPPORTED = 3, /* valid config, but no kernel built for (dtype, d_c, d_rope) */
  VMLA_ERR_ALIGN = 4,       /* a device pointer is not 16-byte aligned */
  VMLA_ERR_STATE = 5,       /* call not valid in the ctx's current state */
  VMLA_ERR_ARG = 6,         /* another argument out of range */
  VMLA_ERR_HIP = 7,         /* the HIP runtime reported an error for a launch */
  VMLA_ERR_SCRATCH = 8      /* per-call buffers larger than VMLA_SCRATCH_BYTES (vmla_attend_noalloc) */
};

enum { VMLA_DTYPE_BF16 = 0, VMLA_DTYPE_F32 = 1 };

/*
 * Layer geometry.  Names follow the paper's notation (section 3; section 4.1
 * gives the Wan-1.3B values: hidden 1536, 12 heads, d_nope 96 + d_rope 32,
 * d_c 192, d_q 768; appendix D.1: 30x52 grid, 3-frame chunks, 21-frame window).
 *   head dim d_h = d_nope + d_rope; softmax scale 1/sqrt(d_h).
 *   rope_pairs_t/h/w: complex pairs of the decoupled key per axis, in the
 *     order t, h, w; 2*(t+h+w) must equal d_rope (section 3.2, 4.1).
 *   tokens per frame T = grid_h*grid_w; token s sits at row s/grid_w,
 *     column s%grid_w.  Chunk = chunk_frames frames = C*T query tokens.
 *   batch: independent streams advanced in lockstep (one frame counter).
 *   attn_workgroups: persistent attention workgroups (0 = 256, one per MI355X
 *     compute unit); it sizes part of the workspace.
 *   sink_frames: S >= 0 pinned sink frames (appendix D.4: the long-horizon cache
 *     keeps one sink latent frame ahead of a six-frame window).  The first S
 *     frames appended stay in slots 0..S-1; later frames slide through the
 *     window_frames FIFO slots.  The visible cache is sink frames [0, min(n, S))
 *     plus window frames [max(S, n - window_frames), n).
 *   rope_at_use: 0 rotates the decoupled key with its absolute frame index when
 *     it is appended; 1 stores it un-rotated and rotates every visible key, and
 *     the chunk's keys and queries, with local temporal coordinates: a frame's
 *     index in [sink frames, window frames, chunk frames] (appendix D.5
 *     re-indexing).  Without sinks both give the same scores (rotary relative
 *     invariance); sink_frames > 0 requires rope_at_use = 1.
 * Constraints (else VMLA_ERR_CONFIG): all sizes > 0 (sink_frames >= 0);
 *   1 <= chunk_frames <= window_frames; d_nope, d_rope, d_c, d_v, d_q and hidden
 *   multiples of 8; rope_theta > 0; rope_at_use in {0, 1}; batch <= 65,535 and
 *   batch * chunk_frames * grid_h * grid_w <= 64 * 65,535 query tokens per call
 *   (launch-grid limits).
 * Built kernels (else VMLA_ERR_UNSUPPORTED): (dtype, d_c, d_rope) in
 *   {(f32, 24, 8), (bf16, 24, 8), (bf16, 96, 32), (bf16, 192, 32), (bf16, 448, 32)}.
 */
typedef struct vmla_config {
  int32_t batch;
  int32_t hidden;
  int32_t n_heads;
  int32_t d_nope;
  int32_t d_rope;
  int32_t d_v;
  int32_t d_c;
  int32_t d_q;
  int32_t rope_pairs_t, rope_pairs_h, rope_pairs_w;
  float rope_theta;
  int32_t grid_h, grid_w;
  int32_t window_frames;
  int32_t chunk_frames;
  int32_t dtype;
  int32_t attn_workgroups;
  int32_t sink_frames;
  int32_t rope_at_use;
} vmla_config;

/*
 * Device pointers to one layer's weights (Linear layout, config dtype).
 *   w_dkv [d_c, hidden]       content latent c = W_DKV x          (section 3.1)
 *   w_kr  [d_rope, hidden]    decoupled key k^ = W_KR x, rotated by 3D-RoPE (3.2)
 *   w_dq  [d_q, hidden]       query latent c^Q = W_DQ x            (section 4.1)
 *   w_uq  [n_heads*(d_nope+d_rope), d_q]  per head [q_nope ; q_rope]
 *   w_uk  [n_heads, d_nope, d_c]  per-head content-key lift k_nope = W_UK^h c (3.3)
 *   w_uv  [n_heads, d_v, d_c]     per-head value lift v = W_UV^h c           (3.3)
 *   w_o   [hidden, n_heads*d_v]   output projection
 */
typedef struct vmla_weights {
  const void *w_dkv, *w_kr, *w_dq, *w_uq, *w_uk, *w_uv, *w_o;
} vmla_weights;

typedef struct vmla_ctx vmla_ctx; /* opaque; holds host-side metadata only */

/* Bytes of the ring cache: batch * (sink_frames + window_frames) * T *
 * (d_c + d_rope) elements.  Row (slot*T + s) of stream b holds [c (d_c) | k_r
 * (d_rope)] of token s of the frame in that slot -- the per-token latent entry
 * of paper section 3.1 (content latent plus the head-shared decoupled key of
 * section 3.2; 224 scalars at the Wan-1.3B widths) -- k_r rotated with the
 * absolute frame index (rope_at_use = 0) or un-rotated (rope_at_use = 1, the
 * form appendix D.5 caches).  Frame f lives in slot f if f < S, else in slot
 * S + (f - S) % window_frames (the sink-plus-FIFO window of appendix D.4).
 * Occupied slots are always 0..(visible frames - 1).  Returns 0 for an invalid
 * config. */
VMLA_API size_t vmla_cache_bytes(const vmla_config* cfg);

/* Bytes of device memory a ctx needs beside the cache: a persistent part
 * written by vmla_prepare (the range flag, the cosine and sine of the 3D-RoPE
 * row and column angles -- d_rope/2 x max(grid_h, grid_w) pairs of fp32 --
 * and the weights in the activation type, below) and the per-call buffers of vmla_attend (chunk latents,
 * the activation-type copy of x and the cosine and sine of the chunk tokens' rotary angles (16-bit
 * storage), absorbed queries, latent outputs, per-head outputs, partial softmax states,
 * key tiles; vmla_prepare also uses them as scratch).  Returns 0 for an
 * invalid config.
 *
 * Operand types.  x, out, the cache and the caller's weights have the config's
 * dtype.  What the layer computes between x and out (absorbed queries,
 * attention outputs, per-head outputs) is held in the activation type: fp16
 * for bf16 storage (same 16 bits, 11 significant bits instead of 8, same MFMA
 * rate on gfx950), fp32 for fp32 storage; so are the weights vmla_prepare
 * writes, the copy of x the chunk GEMM of an attend stages, and the fp16 key
 * tiles the attention kernel reads the cached rows from.  bf16 values within
 * fp16's normal range (2^-14 .. 65504 in magnitude) convert exactly; smaller
 * ones become fp16 subnormals (absolute error below 2^-25).  A finite value
 * beyond +-65504 is saturated to +-65504 -- the result then differs from
 * full-range arithmetic -- and sets bit 0 of the ctx's range flag
 * (vmla_range_flags).  NaN and infinite values pass through unchanged. */
VMLA_API size_t vmla_workspace_bytes(const vmla_config* cfg);

/* Create a ctx over caller-owned memory.  cache: vmla_cache_bytes(cfg) bytes;
 * its contents are not read until frames are appended (unused slots may hold
 * anything).  workspace: vmla_workspace_bytes(cfg) bytes.  rope_freqs: host
 * array of d_rope/2 floats giving omega per complex pair (axis order t, h, w),
 * copied at create; NULL selects theta^(-2i/(2p_a)), i = 0..p_a-1, per axis.
 * A non-finite entry -> VMLA_ERR_ARG.  Makes no HIP call.  On success *out is
 * a new ctx with 0 frames appended, not yet prepared. */
VMLA_API int vmla_create(const vmla_config* cfg, const vmla_weights* w, void* cache,
                         void* workspace, const float* rope_freqs, vmla_ctx** out);

/* Enqueue the one-time set-up of a ctx: clear its range flag, tabulate the
 * rotary row and column angles, and write, into the persistent part of the
 * workspace, these weights in the activation type:
 *   [W_DKV; W_KR];
 *   absorbed query weight, per head h, the [d_c + d_rope, hidden] block
 *     qscale * [W_UK^h^T W_UQ^h,nope ; W_UQ^h,rope] W_DQ  (qscale = log2(e)/sqrt(d_h)),
 *   so one GEMM over x gives the chunk's cache rows together with the
 *   absorbed query q~_h = W_UK^h^T q^nope_h and the un-rotated q^R_h of the
 *   MLA absorption (paper section 3.3; c^Q = W_DQ x only ever feeds W_UQ, so
 *   W_DQ is taken into the product, with one rounding of it);
 *   qscale * W_UQ W_DQ (the per-head queries of the expanded path), W_UV, W_O.
 * The products are summed in fp32 and rounded once; the per-call part of the
 * workspace holds the fp32 intermediate.
 * Must follow vmla_create before any vmla_attend*, vmla_expand or
 * vmla_range_flags on the ctx (else those return VMLA_ERR_STATE); appends and
 * vmla_compress do not need it.  Since it copies the weights, the caller's
 * weights must not change afterwards (call it again if they do). */
VMLA_API int vmla_prepare(vmla_ctx* ctx, hipStream_t stream);

/* Read and clear the ctx's range flag: waits for `stream`, stores the flag in
 * *flags (bit 0 set: since vmla_prepare or the last read, some fp16 operand
 * copy -- a cached or chunk latent element, a hidden-state element of x, an
 * absorbed query, a per-head output, an expanded key or value, a prepared
 * weight -- had a finite value
 * beyond +-65504 and was saturated), then enqueues the clear on `stream`. */
VMLA_API int vmla_range_flags(vmla_ctx* ctx, uint32_t* flags, hipStream_t stream);

/* Append one chunk: x is [batch, chunk_frames*T, hidden].  Computes the cache
 * rows [c | k_r] of frames f = n..n+C-1 (n = frames appended so far): c = W_DKV
 * x, k_r = W_KR x rotated by 3D-RoPE at the absolute frame index (un-rotated
 * with rope_at_use), rounded to the storage type, and writes frame f into slot
 * f if f < S, else slot S + (f - S) % window_frames, evicting the frame that
 * held it (oldest first; paper sections 3.1-3.2, appendix D.4).  Then n += C
 * on the host. */
VMLA_API int vmla_compress_append(vmla_ctx* ctx, const void* x, hipStream_t stream);

/* Attend one chunk: x is [batch, C*T, hidden], out is [batch, C*T, hidden].
 * Every query token of frames n..n+C-1 attends, in every head, to all visible
 * cached frames (sinks [0, min(n, S)) and the window [max(S, n-W), n)) and all
 * tokens of the chunk itself (chunk-causal, appendix D.4), followed by W_UV and
 * W_O (paper section 3.3, absorbed form).  Leaves the cache and n unchanged:
 * the frozen-cache denoising steps of a rollout call this repeatedly, then
 * append the final step's x.  Needs vmla_prepare.  With bf16 storage every
 * product runs on fp16 operands: x as the chunk GEMM stages it, fp16 copies of
 * the visible cached rows (each saturating beyond +-65504, see the operand
 * types above), the fp16 absorbed queries and the prepared fp16 weights. */
VMLA_API int vmla_attend(vmla_ctx* ctx, const void* x, void* out, hipStream_t stream);

/* Same as vmla_attend, and additionally records attn_start and attn_stop at
 * the start and the end of the latent-attention kernel (the call's dominant
 * kernel; the events are attached to its dispatch, so timing adds no gap to
 * the stream), so a caller can time that kernel with hipEventElapsedTime.
 * Both events must be created by the caller (hipEventCreate); NULL ->
 * VMLA_ERR_NULL. */
VMLA_API int vmla_attend_profiled(vmla_ctx* ctx, const void* x, void* out, hipEvent_t attn_start,
                                  hipEvent_t attn_stop, hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): vmla_attend
 * with the per-call buffers (chunk latents, absorbed queries, latent and
 * per-head outputs, partial softmax states, key tiles) taken from a scratch
 * array inside the library instead of the ctx's workspace.  The array holds
 * VMLA_SCRATCH_BYTES (128 MiB) on every GPU the library runs on, from when its
 * code is loaded there until the process ends -- enough for one Wan-1.3B layer
 * call (4,680 query tokens against 37,440 keys needs ~112 MiB).  The ctx must
 * be prepared; only the persistent part of its workspace (prepared weights,
 * range flag) is read.  Same inputs, outputs and results as vmla_attend.
 * Allocates nothing and needs no free call.  Errors: VMLA_ERR_SCRATCH if the
 * ctx's per-call buffers exceed VMLA_SCRATCH_BYTES (larger batch or chunk),
 * else as vmla_attend.  Every call on one GPU uses the same array and leaves it
 * holding that call's buffers; nothing is assumed about its contents at entry.
 * Calls that overlap on one GPU (several streams or host threads at once) race
 * on it: issue them in one stream order. */
#define VMLA_SCRATCH_BYTES ((size_t)128 << 20)
VMLA_API int vmla_attend_noalloc(vmla_ctx* ctx, const void* x, void* out, hipStream_t stream);

/* Test hook: compute the cache rows [c | RoPE(k^)] of x ([batch, C*T, hidden])
 * as frames frame0..frame0+C-1 into latents_out ([batch, C*T, d_c+d_rope]) --
 * the row vmla_compress_append writes (paper sections 3.1-3.2), always rotated,
 * at the absolute coordinate frame0 + i -- without touching the cache or n.
 * frame0 >= 0 else VMLA_ERR_ARG. */
VMLA_API int vmla_compress(vmla_ctx* ctx, const void* x, int64_t frame0, void* latents_out,
                           hipStream_t stream);

/* Host metadata of the sliding window (appendix D.4: sink frames ahead of a
 * FIFO window with oldest-frame eviction): frames appended n, the first window
 * frame min(n, max(S, n-W)) (= max(0, n-W) without sinks), and the number of
 * visible cached frames min(n, S) + max(0, min(n - S, W)).  Any output pointer
 * may be NULL. */
VMLA_API int vmla_cache_state(const vmla_ctx* ctx, int64_t* frames_appended,
                              int64_t* first_valid_frame, int32_t* n_valid_frames);

/* Forget all appended frames (n = 0).  Cache bytes are left as they are. */
VMLA_API int vmla_reset(vmla_ctx* ctx);

/* Free a ctx (host memory only).  NULL is ignored. */
VMLA_API void vmla_destroy(vmla_ctx* ctx);

/*
 * Block-causal clip (the training-time form of the layer, appendix D.4): all
 * window_frames frames of one clip attend at once, tokens of chunk q (frames
 * [q*C, (q+1)*C)) seeing every token of chunks 0..q; the ring cache is neither
 * read nor written and the frame counter is unchanged.  Temporal coordinates
 * are the clip's frame indices 0..window_frames-1.  Key tiles above the block
 * diagonal are skipped.
 * vmla_clip_workspace_bytes: bytes of the caller-owned clip workspace (the
 *   per-call buffers of vmla_attend sized for window_frames*T query tokens; the
 *   prepared weights and the range flag stay in the ctx's workspace);
 *   0 if the config is invalid or batch * window_frames * T exceeds 64 * 65,535
 *   (launch-grid limit; vmla_attend_clip then returns VMLA_ERR_CONFIG).
 * vmla_attend_clip: x and out are [batch, window_frames*T, hidden]; same rules
 *   as vmla_attend, including vmla_prepare (a window_frames not divisible by
 *   chunk_frames gives a shorter last block).
 */
VMLA_API size_t vmla_clip_workspace_bytes(const vmla_config* cfg);
VMLA_API int vmla_attend_clip(vmla_ctx* ctx, const void* x, void* clip_workspace, void* out,
                              hipStream_t stream);
/* vmla_attend_clip plus caller-made events taking the start and end time of the
 * attention kernel (NULL -> VMLA_ERR_NULL). */
VMLA_API int vmla_attend_clip_profiled(vmla_ctx* ctx, const void* x, void* clip_workspace, void* out,
                                       hipEvent_t attn_start, hipEvent_t attn_stop, hipStream_t stream);

/*
 * Expanded (non-absorbed) latent path (paper section 3.3: the cached latents
 * are up-projected to per-head keys and values, which are then attended like a
 * dense layer).  Same result as vmla_attend up to rounding; for the
 * frozen-cache denoising steps of a chunk (appendix D.5) the window is
 * up-projected once and reused by every step.  Built for bf16 with
 * d_nope + d_rope = d_v = 128 (else VMLA_ERR_UNSUPPORTED).
 *
 * vmla_expanded_bytes: size of the caller-owned `expanded` buffer (per-head
 *   keys and values of the window in the dense cache layout, see
 *   vmla_dense_*, plus the chunk's keys/values, queries, outputs and partial
 *   states: ~260 MB at the Wan-1.3B layer).  0 if unsupported or invalid.
 * vmla_expand: per stream, head h and valid ring key j,
 *   K_h[j] = [W_UK^h c_j ; k_r_j] and V_h[j] = W_UV^h c_j into `expanded` (fp16,
 *   saturating as above), from the ring as it stands (n frames).  Leaves the
 *   cache and n unchanged.  Needs vmla_prepare.
 * vmla_attend_expanded: attend one chunk (x, out as vmla_attend) with fp16 per-head
 *   queries [q_nope ; RoPE(q_rope)] against the expanded window and the
 *   chunk's own up-projected keys/values, then W_O.  `expanded` must be the
 *   buffer of the last vmla_expand, made after the last append (else
 *   VMLA_ERR_STATE; vmla_reset forgets it).
 * vmla_attend_expanded_profiled: same, with caller-made events taking the
 *   attention kernel's start and end time (NULL -> VMLA_ERR_NULL).
 */
VMLA_API size_t vmla_expanded_bytes(const vmla_config* cfg);
VMLA_API int vmla_expand(vmla_ctx* ctx, void* expanded, hipStream_t stream);
VMLA_API int vmla_attend_expanded(vmla_ctx* ctx, const void* expanded, const void* x, void* out,
                                  hipStream_t stream);
VMLA_API int vmla_attend_expanded_profiled(vmla_ctx* ctx, const void* expanded, const void* x, void* out,
                                           hipEvent_t attn_start, hipEvent_t attn_stop, hipStream_t stream);

/*
 * Dense per-head baseline (paper section 1 and appendix C.1: the layer VideoMLA
 * replaces, whose cache holds every head's key and value, n_heads*2*d_h scalars
 * per token, 16-bit).  Same chunk-causal window, ring eviction and 3D-RoPE as
 * the latent layer; per head h and token x:
 *   q_h = RoPE(W_Q^h x), k_h = RoPE(W_K^h x) (all d_h channels rotated, pairs
 *   (2p, 2p+1), axis order t, h, w), v_h = W_V^h x,
 *   o_h = softmax(q_h k_h^T / sqrt(d_h)) v_h, out = W_O [o_1; ...; o_H].
 * It takes the same vmla_config, read this way: d_rope = d_h (the rotated
 * per-head width; rope_pairs_* split its d_h/2 pairs), d_v = value width, and
 * d_nope = d_c = d_q = 0 (else VMLA_ERR_CONFIG).  Built kernels (else
 * VMLA_ERR_UNSUPPORTED): bf16 with d_rope = d_v = 128, sink_frames = 0 and
 * rope_at_use = 0.
 *
 * Weights (Linear layout, bf16):
 *   w_q, w_k [n_heads*d_rope, hidden]; w_v [n_heads*d_v, hidden];
 *   w_o [hidden, n_heads*d_v].
 *
 * Cache layout (vmla_dense_cache_bytes), P = window_frames*T rounded up to a
 * multiple of 128:
 *   keys   [batch][n_heads][P][d_rope] fp16, rotated with the absolute frame index;
 *   values [batch][n_heads][d_v][P] fp16, transposed: the value of ring key j
 *          (frame f in slot f % window_frames, key j = slot*T + s) sits in
 *          column j with bits 2 and 3 of j swapped; columns past the valid
 *          keys (up to the next multiple of 128) are kept at zero by the library.
 * Keys and values are stored as fp16 (the cache size equals a bf16 one), so
 * both products run on fp16 operands with the fp16 queries; conversions
 * saturate beyond +-65504 and set the dense ctx's range flag.  The attention
 * output is fp16 and W_O runs on the fp16 copy vmla_dense_prepare writes.
 */
typedef struct vmla_dense_weights {
  const void *w_q, *w_k, *w_v, *w_o;
} vmla_dense_weights;

typedef struct vmla_dense_ctx vmla_dense_ctx; /* opaque; host-side metadata only */

/* Bytes of the dense ring cache (layout above); 0 for an invalid config. */
VMLA_API size_t vmla_dense_cache_bytes(const vmla_config* cfg);

/* Bytes of scratch device memory a dense ctx needs (rotated queries, the
 * chunk's keys and values, attention output, partial softmax states). */
VMLA_API size_t vmla_dense_workspace_bytes(const vmla_config* cfg);

/* Create a dense ctx over caller-owned memory; same rules as vmla_create
 * (rope_freqs: d_rope/2 floats or NULL for theta^(-2i/(2p_a)) per axis). */
VMLA_API int vmla_dense_create(const vmla_config* cfg, const vmla_dense_weights* w, void* cache,
                               void* workspace, const float* rope_freqs, vmla_dense_ctx** out);

/* One-time set-up of a dense ctx: clear its range flag and write the fp16 copy
 * of W_O into the workspace.  Required before vmla_dense_append,
 * vmla_dense_attend* and vmla_dense_range_flags (else VMLA_ERR_STATE). */
VMLA_API int vmla_dense_prepare(vmla_dense_ctx* ctx, hipStream_t stream);

/* As vmla_range_flags, for a dense ctx (bit 0: a key, value, query or W_O
 * element was saturated to +-65504). */
VMLA_API int vmla_dense_range_flags(vmla_dense_ctx* ctx, uint32_t* flags, hipStream_t stream);

/* Append one chunk (x [batch, C*T, hidden]): keys and values of frames
 * n..n+C-1 into their ring slots, evicting the oldest frames; n += C. */
VMLA_API int vmla_dense_append(vmla_dense_ctx* ctx, const void* x, hipStream_t stream);

/* Attend one chunk (x, out [batch, C*T, hidden]) against the cached frames
 * [max(0, n-W), n) and the chunk itself; the cache and n are unchanged. */
VMLA_API int vmla_dense_attend(vmla_dense_ctx* ctx, const void* x, void* out, hipStream_t stream);

/* vmla_dense_attend plus caller-made events taking the start and end time of
 * the attention kernel (NULL -> VMLA_ERR_NULL). */
VMLA_API int vmla_dense_attend_profiled(vmla_dense_ctx* ctx, const void* x, void* out,
                                        hipEvent_t attn_start, hipEvent_t attn_stop, hipStream_t stream);

/* As vmla_cache_state / vmla_reset / vmla_destroy, for a dense ctx. */
VMLA_API int vmla_dense_cache_state(const vmla_dense_ctx* ctx, int64_t* frames_appended,
                                    int64_t* first_valid_frame, int32_t* n_valid_frames);
VMLA_API int vmla_dense_reset(vmla_dense_ctx* ctx);
VMLA_API void vmla_dense_destroy(vmla_dense_ctx* ctx);

/* Static description of a status code. */
VMLA_API const char* vmla_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif /* VMLA_H */
