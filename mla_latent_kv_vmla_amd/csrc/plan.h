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
struct Plan {
  DType dtype;
  int B, d, nh, d_nope, dr, dv, dc, dq, D, dh;  // D = dc + dr, dh = d_nope + dr
  int Tpf, grid_w, W, C, Nq;                    // tokens/frame, window and chunk frames
  int S, rope_at_use;                           // sink frames; rotate k_r at use (local coordinates)
  int causal_tokens;  // > 0: a whole clip of Nq tokens, block-causal in blocks of this many tokens
  int pairs_t, pairs_h, pairs_w;
  float freq[kMaxRopePairs];
  float qscale;  // log2(e) / sqrt(dh): softmax scale folded into the absorbed query
  int G;         // persistent attention workgroups
  const void *w_dkv, *w_kr, *w_dq, *w_uq, *w_uk, *w_uv, *w_o;
  void* cache;   // [B][W*Tpf][D]
  // workspace regions
  void *stage;   // [B][Nq][D]            chunk latents (rotated)
  void *cq;      // [B][Nq][dq]           query latent
  void *qnope;   // [B][Nq][nh][d_nope]   content part of the per-head query
  void *qt;      // [B][Nq][nh][D]        absorbed query [W_UK^T q_nope | q_rope] * qscale
  void *olat;    // [B][Nq][nh][dc]       attention output in latent space
  void *o;       // [B][Nq][nh*dv]        per-head outputs after W_UV
  float *part_o; // [2G][kAttnMaxRows][dc] normalised partial outputs (fp16 for 16-bit storage, else fp32)
  float *part_ml;// [2G][kAttnMaxRows][2]  running max (log2 domain) and sum
  void *vtiles;  // pre-pass tiles of the visible keys (per call): fp16 key tiles for bf16, value images for fp32
  void *assembled;  // rope_at_use: the visible cache rows with k_r rotated at local coordinates
};

// Visible cached frames after n appends: sinks [0, min(n, S)) + window [max(S, n-W), n).
inline int64_t cached_frames(const Plan& p, int64_t n) {
  const int64_t sink = n < p.S ? n : p.S;
  const int64_t win = n - p.S < p.W ? n - p.S : p.W;
  return sink + (win > 0 ? win : 0);
}

struct WorkspaceLayout {
  size_t stage, cq, qnope, qt, olat, o, part_o, part_ml, vtiles, assembled, total;
};

WorkspaceLayout workspace_layout(const Plan& p);

// Kernel pipelines.  Each returns hipSuccess or the first launch error.
// compress: rows [c | RoPE(k^)] of x for frames frame0.. into dst; ring != 0
// writes the frame's ring slot row (slot*Tpf + s; sinks pinned) of each
// stream's cache, else row t of dst.  k^ is rotated with frame index frame0 + i
// unless the rows go to the ring of a rope_at_use layer (stored un-rotated).
hipError_t run_compress(const Plan& p, const void* x, int64_t frame0, void* dst, bool ring,
                        hipStream_t s);
// rope_at_use: the visible cache rows after n appends, k^ rotated with each
// frame's local coordinate, into p.assembled.
hipError_t run_assemble(const Plan& p, int64_t n, hipStream_t s);
// attend: full chunk attention against the ring holding n frames.
hipError_t run_attend(const Plan& p, int64_t n, const void* x, void* out, hipStream_t s,
                      hipEvent_t attn_start = nullptr, hipEvent_t attn_stop = nullptr);

// Latent attention kernels (attention.hip): keys = n_ring cache rows, then the
// chunk's staged rows.  Returns hipErrorInvalidValue for an unbuilt shape.
struct AttnCall {
  DType dtype;
  int dc, dr;
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
//   keys   [P][dh] bf16, rotated by 3D-RoPE on all dh channels;
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
  // workspace regions
  void *q;       // [B][nh][Nq][dh]  rotated, scaled queries
  void *kstage;  // [B][nh][stage_stride][dh]
  void *vstage;  // [B][nh][dv][stage_stride]
  void *o;       // [B][Nq][nh*dv]  attention output
  float *part_o, *part_ml;
};

struct DenseLayout {
  size_t kring, vring, cache_total;                         // cache
  size_t q, kstage, vstage, o, part_o, part_ml, ws_total;   // workspace
};
DenseLayout dense_layout(const DensePlan& p);

// append: K/V of the chunk (frames n..n+C-1) into ring slots.
hipError_t run_dense_append(const DensePlan& p, int64_t n, const void* x, hipStream_t s);
// attend: chunk attention against the ring holding n frames, then W_O.
hipError_t run_dense_attend(const DensePlan& p, int64_t n, const void* x, void* out, hipStream_t s,
                            hipEvent_t attn_start = nullptr, hipEvent_t attn_stop = nullptr);

struct DenseAttnCall {
  int dh, dv;
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
