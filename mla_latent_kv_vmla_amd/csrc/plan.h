// Internal interface between the host runtime (vmla_host.cpp) and the kernel
// pipelines (pipeline.hip, dense.hip, expanded.hip, attention.hip).  Host-only types; no HIP
// kernels.
#pragma once
#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace vmla {

enum class DType : int { BF16 = 0, F32 = 1 };

// Rows per attention workgroup used to size the partial-state workspace
// (the largest row block any built attention kernel uses).
constexpr int kAttnMaxRows = 256;
constexpr int kMaxRopePairs = 64;
// Key-tile size of the dense attention kernel; the dense ring and the chunk's
// staged keys are padded to a multiple of it.
constexpr int kDenseKeyTile = 128;

// Everything one layer call needs: geometry, borrowed device pointers and the
// workspace carve-up.  Filled by the host runtime; read by the pipelines.
//
// Operand types.  The ring cache, x and out have the storage type (bf16 or
// fp32).  Everything the layer computes between them -- absorbed queries,
// attention outputs, per-head outputs -- and the weights of the GEMMs that
// produce them have the activation type: fp16 for bf16 storage (11 significant
// bits where bf16 keeps 8, at the same MFMA rate), fp32 for fp32 storage.  Those
// weights are converted (and, for the queries, derived) once per ctx by
// run_prepare into the persistent part of the workspace.  The query weights
// take W_DQ in: c^Q = W_DQ x only ever feeds W_UQ, so the product of the two
// (and of W_UK, for the absorbed form) is applied to x directly, one GEMM and
// one rounding where the pages' order has two.
struct Plan {
  DType dtype;
  int B, d, nh, d_nope, dr, dv, dc, dq, D, dh;  // D = dc + dr, dh = d_nope + dr
  int Tpf, grid_w, W, C, Nq;                    // tokens/frame, window and chunk frames
  int S, rope_at_use;                           // sink frames; rotate k_r at use (local coordinates)
  int causal_tokens;  // > 0: a whole clip of Nq tokens, block-causal in blocks of this many tokens
  int pairs_t, pairs_h, pairs_w;
  float freq[kMaxRopePairs];
  float qscale;  // log2(e) / sqrt(dh): softmax scale folded into the query weights
  int G;         // persistent attention workgroups
  const void *w_dkv, *w_kr, *w_dq, *w_uq, *w_uk, *w_uv, *w_o;
  void* cache;   // [B][(S+W)*Tpf][D]
  // persistent workspace (written by run_prepare)
  uint32_t* flags;  // bit 0: an fp16 operand copy saturated (see kF16Max)
  float* rope_tab;  // [pairs][rope_tab_stride][2] cos and sin of the row and column angles
  void *wlat;    // [D][d]        [W_DKV; W_KR]
  void *wqa;     // [nh][D][d]    absorbed query weight: per head qscale*[W_UK^h^T W_UQ^h,nope ; W_UQ^h,rope] W_DQ
  void *wuq;     // [nh*dh][d]    qscale * W_UQ W_DQ (per-head queries of the expanded path)
  void *wuv;     // [nh][dv][dc]  W_UV
  void *wo;      // [d][nh*dv]    W_O
  // per-call workspace
  void *stage;   // [B][Nq][D]            chunk latents (rotated), storage type
  void *xa;      // [B][Nq][d]            x in the activation type (bf16 storage; fp32 reads x itself)
  void *ctab;    // [Nq][dr/2][2]         cos and sin of the chunk tokens' rotary angles (bf16 storage)
  void *qt;      // [B][Nq][nh][D]        absorbed query [W_UK^T q_nope | q_rope] * qscale
  void *olat;    // [B][Nq][nh][dc]       attention output in latent space
  void *o;       // [B][Nq][nh*dv]        per-head outputs after W_UV (same bytes as qt)
  float *part_o; // [2G][kAttnMaxRows][dc] normalised partial outputs (activation type)
  float *part_ml;// [2G][kAttnMaxRows][2]  running max (log2 domain) and sum
  void *vtiles;  // pre-pass tiles of the visible keys (per call): fp16 key tiles for bf16, value images for fp32
  void *assembled;  // rope_at_use with fp32 storage: the visible cache rows with k_r rotated at local coordinates
  void *prep;    // run_prepare's fp32 scratch (the per-call region's start; no call is in flight then)
};

// Visible cached frames after n appends: sinks [0, min(n, S)) + window [max(S, n-W), n).
inline int64_t cached_frames(const Plan& p, int64_t n) {
  const int64_t sink = n < p.S ? n : p.S;
  const int64_t win = n - p.S < p.W ? n - p.S : p.W;
  return sink + (win > 0 ? win : 0);
}

// Byte offsets of the workspace regions.  The persistent part (flags and
// prepared weights) sits at the start of a ctx's workspace; the per-call part
// follows it there, or fills a clip workspace of its own.
struct WorkspaceLayout {
  size_t flags, rope_tab, wlat, wqa, wuq, wuv, wo, persistent;        // from the workspace start
  size_t stage, xa, ctab, qt, olat, o, part_o, part_ml, vtiles, assembled, per_call;  // from the per-call start
  size_t prep;  // run_prepare's scratch: the first prep_bytes of the per-call part (per_call >= it)
  size_t total;  // persistent + per_call
};

WorkspaceLayout workspace_layout(const Plan& p);
// Positions per pair of the rotary table (grid_h or grid_w, whichever is larger).
inline int rope_tab_stride(int Tpf, int grid_w) { return Tpf / grid_w > grid_w ? Tpf / grid_w : grid_w; }
inline size_t rope_tab_bytes(int pairs, int Tpf, int grid_w) {
  return (size_t)pairs * rope_tab_stride(Tpf, grid_w) * 2 * sizeof(float);
}
// Fill a rotary table (pairs p >= pairs_t; the t-axis entries stay unused).
hipError_t run_rope_table(float* tab, int pairs, int pairs_t, int pairs_h, int Tpf, int grid_w, const float* freq,
                          hipStream_t s);
// Bytes of one element of the activation type (fp16 for bf16 storage).
inline size_t act_bytes(DType t) { return t == DType::F32 ? 4 : 2; }

// Kernel pipelines.  Each returns hipSuccess or the first launch error.
// prepare: clear the range flag and write the persistent weights (wlat, wqa,
// wuq, wuv, wo), using p.prep (prep_bytes(p)) as scratch.
hipError_t run_prepare(const Plan& p, hipStream_t s);
// Scratch bytes run_prepare needs: the absorbed query weight before W_DQ is
// taken in, [nh*D][dq] fp32.
inline size_t prep_bytes(const Plan& p) { return (size_t)p.nh * p.D * p.dq * sizeof(float); }
// Zero one flag word (a kernel, so the clear can sit in a captured graph).
hipError_t run_clear_flags(uint32_t* flags, hipStream_t s);
// compress: rows [c | RoPE(k^)] of x for frames frame0.. into dst; ring != 0
// writes the frame's ring slot row (slot*Tpf + s; sinks pinned) of each
// stream's cache, else row t of dst.  k^ is rotated with frame index frame0 + i
// unless the rows go to the ring of a rope_at_use layer (stored un-rotated).
hipError_t run_compress(const Plan& p, const void* x, int64_t frame0, void* dst, bool ring,
                        hipStream_t s);
// The chunk's cache rows (frames frame0.., into p.stage) and its queries from
// one GEMM over x with the prepared [W_DKV; W_KR] and query weight, the queries
// rotated at the chunk's frames frame0..:
//   Absorbed: p.wqa -> p.qt [B*Nq][nh*D] (latent attention);
//   PerHead:  p.wuq -> q [B][nh][Nq][dh], fp16 (the expanded path's dense attention).
enum class QueryForm { Absorbed, PerHead };
hipError_t run_chunk_rows_and_queries(const Plan& p, const void* x, int64_t frame0, QueryForm form, void* q,
                                      hipStream_t s);
// rope_at_use with fp32 storage: the visible cache rows after n appends, k^
// rotated with each frame's local coordinate, into p.assembled.  (With bf16
// storage the rotation happens where the rows are converted: the attention
// key-tile pre-pass and the expansion epilogue.)
hipError_t run_assemble(const Plan& p, int64_t n, hipStream_t s);
// attend: full chunk attention against the ring holding n frames.
hipError_t run_attend(const Plan& p, int64_t n, const void* x, void* out, hipStream_t s,
                      hipEvent_t attn_start = nullptr, hipEvent_t attn_stop = nullptr);

// Latent attention kernels (attention.hip): keys = n_ring cache rows, then the
// chunk's staged rows.  Returns hipErrorInvalidValue for an unbuilt shape.
struct AttnCall {
  DType dtype;
  int dc, dr;
  uint32_t* range_flag;  // raised when the fp16 key-tile pre-pass saturates a cached element
  const void* qt;
  const void* cache;
  const void* stage;
  void* out;
  float* part_o;
  float* part_ml;
  void* vtiles;
  hipEvent_t ev_start, ev_stop;       // optional: recorded around the attention kernel itself
  long cache_bstride, stage_bstride;  // elements
  int B, R, n_ring, n_stage;
  int G;
  int causal_tokens;  // > 0: block-causal over the staged keys only (n_ring = 0), blocks of this many tokens
  // rot_ring (bf16 storage, rope_at_use): the ring rows hold k^ un-rotated and the
  // key-tile pre-pass turns them at their local coordinate (rot_n frames appended,
  // rot_S sinks, rot_W window frames), with this rotary table
  int rot_ring, rot_S, rot_W;
  int64_t rot_n;
  int pairs_t, pairs_h, grid_w, tokens_per_frame;
  float freq[kMaxRopePairs];
  const float* rope_tab;
};
hipError_t run_latent_attention(const AttnCall& a, hipStream_t s);
bool latent_attention_supported(DType dt, int dc, int dr);
// Workspace bytes of the attention pre-pass tiles (fp16 key tiles for bf16,
// transposed value images for fp32) for up to max_ring_keys ring keys plus
// stage_keys chunk keys.
size_t latent_prepass_bytes(DType dt, int dc, int dr, int B, int max_ring_keys, int stage_keys);

// ---------------------------------------------------------------- dense baseline
// Per-head keys and values (the dense layer of the paper's section 1 and
// appendix C.1).  Per (stream b, head h):
//   keys   [P][dh] fp16, rotated by 3D-RoPE on all dh channels;
//   values [dv][P] fp16, transposed, key j at column perm16(j) (bits 2 and 3
//          of j swapped), zero at every column past the valid keys up to P;
// P = ring_stride (ring: W*T keys, frame f in slots (f % W)*T..) or
// stage_stride (the chunk's own C*T keys), both multiples of kDenseKeyTile.
struct DensePlan {
  int B, d, nh, dh, dv;
  int Tpf, grid_w, W, C, Nq;
  int pairs_t, pairs_h, pairs_w;
  float freq[kMaxRopePairs];
  float qscale;  // log2(e) / sqrt(dh)
  int G;
  int ring_stride, stage_stride;
  const void *w_q, *w_k, *w_v, *w_o;
  void *kring, *vring;  // cache
  // persistent workspace (run_dense_prepare)
  uint32_t* flags;  // bit 0: an fp16 operand copy saturated
  float* rope_tab;  // rotary table of the row and column axes (see Rope)
  void* wo;         // [d][nh*dv] fp16 W_O
  // per-call workspace
  void *q;       // [B][nh][Nq][dh]  rotated, scaled queries (fp16)
  void *kstage;  // [B][nh][stage_stride][dh]
  void *vstage;  // [B][nh][dv][stage_stride]
  void *o;       // [B][Nq][nh*dv]  attention output
  float *part_o, *part_ml;
};

struct DenseLayout {
  size_t kring, vring, cache_total;                                  // cache
  size_t flags, rope_tab, wo, q, kstage, vstage, o, part_o, part_ml, ws_total;  // workspace
};
// with_persistent = false (the expanded path's buffer, which takes the flag
// and W_O of its latent ctx): flags and wo are left out (offsets 0, size 0).
DenseLayout dense_layout(const DensePlan& p, bool with_persistent = true);

// prepare: clear the range flag and write the fp16 W_O.
hipError_t run_dense_prepare(const DensePlan& p, hipStream_t s);

// append: K/V of the chunk (frames n..n+C-1) into ring slots.
hipError_t run_dense_append(const DensePlan& p, int64_t n, const void* x, hipStream_t s);
// attend: chunk attention against the ring holding n frames, then W_O.
hipError_t run_dense_attend(const DensePlan& p, int64_t n, const void* x, void* out, hipStream_t s,
                            hipEvent_t attn_start = nullptr, hipEvent_t attn_stop = nullptr);

struct DenseAttnCall {
  int dh, dv;  // keys, queries and values fp16
  const void* q;
  const void *kring, *vring, *kstage, *vstage;
  void* out;  // [B][Nq][H][dv]
  float* part_o;
  float* part_ml;
  hipEvent_t ev_start, ev_stop;
  int B, H, Nq, n_ring, ring_stride, stage_stride;
  int G;
};
hipError_t run_dense_attention(const DenseAttnCall& a, hipStream_t s);
bool dense_attention_supported(DType dt, int dh, int dv);
// Zero the value columns of keys [c0, c1) (key order as stored: bits 2 and 3
// swapped) in `rows` transposed value rows of stride P (dense.hip).
void zero_value_columns_async(void* v, long rows, long P, int c0, int c1, hipStream_t s);

// ---------------------------------------------------------------- expanded latent path
// The latent layer computed without absorption: the window's latent rows are
// up-projected once to per-head keys [W_UK^h c | k_r] and values W_UV^h c in the
// dense layout (DensePlan regions of an "expanded" buffer), then attended with
// the dense kernel.  ex.* regions live in the expanded buffer; p supplies the
// latent geometry, weights, ring cache and the latent workspace (stage, c^Q).
struct ExpandedLayout {
  DenseLayout dense;  // kring/vring then q/kstage/vstage/o/part_o/part_ml
  size_t wext;        // [nh][dh][d_c + d_r] bf16: per head [W_UK^h | 0 ; 0 | I]
  size_t total;
};
ExpandedLayout expanded_layout(const Plan& p, DensePlan& ex);
hipError_t run_expand(const Plan& p, const DensePlan& ex, void* wext, int64_t n, hipStream_t s);
hipError_t run_attend_expanded(const Plan& p, const DensePlan& ex, const void* wext, int64_t n, const void* x,
                               void* out, hipStream_t s, hipEvent_t attn_start = nullptr,
                               hipEvent_t attn_stop = nullptr);
bool expanded_supported(const Plan& p);

}  // namespace vmla
