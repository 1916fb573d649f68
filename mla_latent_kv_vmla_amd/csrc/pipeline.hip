// Launch sequences of the two library calls and the GEMM epilogues they use.
//
//   compress (VideoMLA paper, sections 3.1-3.2): one GEMM x . [W_DKV; W_KR]^T whose
//     epilogue rotates the decoupled key channels by 3D-RoPE at the absolute
//     frame (ring rows with rope_at_use stay un-rotated), rounds to the storage
//     type and scatters each token's row to its ring slot (slot * T + s; frames
//     f < S take sink slot f, later ones slot S + (f - S) % W) or to a linear
//     buffer.
//   attend: compress the chunk into staging; with rope_at_use, rotate the
//     visible ring rows at their window-local coordinates into the workspace
//     (assemble_window); c^Q = W_DQ x; q = W_UQ c^Q with the
//     rotary channels turned and scaled straight into the absorbed query;
//     absorbed query q~_h = W_UK^h^T q_nope_h (per-head GEMM on MFMA);
//     latent attention (attention.hip); o_h = W_UV^h o~_h; out = W_O o.
#include "gemm.h"
#include "plan.h"

namespace vmla {

static Rope make_rope(const Plan& p) {
  Rope r;
  r.pairs_t = p.pairs_t;
  r.pairs_h = p.pairs_h;
  r.grid_w = p.grid_w;
  r.tokens_per_frame = p.Tpf;
  for (int i = 0; i < kMaxRopePairs; ++i) r.freq[i] = p.freq[i];
  return r;
}

// Latent cache rows: features [0, dc) are c, [dc, dc+dr) the decoupled key,
// rotated with the token's (frame, row, column) unless `rotate` is 0.  Token m
// is chunk token m % Nq of stream m / Nq, frame frame0 + t / T; in the ring,
// frame f < S sits in sink slot f, later frames in slot S + (f - S) % W.
template <typename T> struct EpiLatent {
  T* dst;
  long bstride;   // elements per stream in dst
  int64_t frame0;
  int Nq, W, S, dc, D;
  int ring, rotate;
  Rope rope;
  __device__ void operator()(int, int m, int n, const float* v) const {
    const int b = m / Nq, t = m % Nq;
    const int64_t frame = frame0 + t / rope.tokens_per_frame;
    const int s = t % rope.tokens_per_frame;
    const int64_t slot = frame < S ? frame : S + (frame - S) % W;
    const long row = ring ? (long)slot * rope.tokens_per_frame + s : (long)t;
    float a0 = v[0], a1 = v[1], a2 = v[2], a3 = v[3];
    if (n >= dc && rotate) {
      const int pair = (n - dc) >> 1;
      rope.rotate2(pair, frame, s, a0, a1);
      rope.rotate2(pair + 1, frame, s, a2, a3);
    }
    store4(dst + b * bstride + row * D + n, a0, a1, a2, a3);
  }
};

// q = W_UQ c^Q, per head [q_nope (d_nope) ; q_rope (dr)].  q_nope goes to its
// own buffer; q_rope is rotated, scaled by qscale and written into the rotary
// part of the absorbed query row.
template <typename T> struct EpiQuery {
  T* qnope;  // [M][nh][d_nope]
  T* qt;     // [M][nh][D]
  int Nq, nh, d_nope, dh, dc, D;
  float qscale;
  Rope rope;
  __device__ void operator()(int, int m, int n, const float* v) const {
    const int h = n / dh, j = n % dh;
    if (j < d_nope) {
      store4(qnope + ((long)m * nh + h) * d_nope + j, v[0], v[1], v[2], v[3]);
      return;
    }
    const int t = m % Nq;
    const int64_t frame = frame0 + t / rope.tokens_per_frame;
    const int s = t % rope.tokens_per_frame;
    const int pair = (j - d_nope) >> 1;
    float a0 = v[0], a1 = v[1], a2 = v[2], a3 = v[3];
    rope.rotate2(pair, frame, s, a0, a1);
    rope.rotate2(pair + 1, frame, s, a2, a3);
    store4(qt + ((long)m * nh + h) * D + dc + (j - d_nope), a0 * qscale, a1 * qscale, a2 * qscale,
           a3 * qscale);
  }
  int64_t frame0;
};

// Absorbed content query: q~[m][h][n] = qscale * (q_nope_h W_UK^h)[n]
template <typename T> struct EpiAbsorb {
  T* qt;
  int nh, D;
  float qscale;
  __device__ void operator()(int z, int m, int n, const float* v) const {
    store4(qt + ((long)m * nh + z) * D + n, v[0] * qscale, v[1] * qscale, v[2] * qscale, v[3] * qscale);
  }
};

template <typename T>
static GemmOps<T> ops(const void* w, long ldw, long wz, const void* x, long ldx, long xz, int N, int M, int K) {
  GemmOps<T> o;
  o.w = o.w2 = static_cast<const T*>(w);
  o.ldw = ldw;
  o.wz = wz;
  o.x = static_cast<const T*>(x);
  o.ldx = ldx;
  o.xz = xz;
  o.N = N;
  o.M = M;
  o.K = K;
  o.n_split = N;
  return o;
}

template <typename T>
static void compress_t(const Plan& p, const void* x, int64_t frame0, void* dst, bool ring, hipStream_t s) {
  const int M = p.B * p.Nq;
  GemmOps<T> op = ops<T>(p.w_dkv, p.d, 0, x, p.d, 0, p.D, M, p.d);
  op.w2 = static_cast<const T*>(p.w_kr);
  op.n_split = p.dc;
  EpiLatent<T> e;
  e.dst = static_cast<T*>(dst);
  e.bstride = ring ? (long)(p.S + p.W) * p.Tpf * p.D : (long)p.Nq * p.D;
  e.frame0 = frame0;
  e.Nq = p.Nq;
  e.W = p.W;
  e.S = p.S;
  e.dc = p.dc;
  e.D = p.D;
  e.ring = ring ? 1 : 0;
  e.rotate = ring && p.rope_at_use ? 0 : 1;
  e.rope = make_rope(p);
  gemm<T, false>(op, 1, e, s);
}

// rope_at_use: visible cache row r of stream b (slot r / T, token r % T) with
// k^ rotated at its frame's local coordinate: sink slot i holds frame i at
// coordinate i; window slot S + j holds the window frame f with (f - S) % W == j,
// at coordinate (sinks) + (f - first window frame).
template <typename T>
__global__ __launch_bounds__(256) void assemble_window(const T* cache, T* out, long rows, long bstride, int64_t n,
                                                       int S, int W, int dc, int D, Rope rope) {
  const int dr = D - dc, pairs = dr / 2;
  const int64_t n_sink = n < S ? n : S;
  const int64_t w0 = n - W > S ? n - W : S;  // first window frame
  const int b = blockIdx.y;
  const T* src = cache + (long)b * bstride;
  T* dst = out + (long)b * bstride;
  const int per_row = dc + pairs;  // c elements copied, then one work item per rotary pair
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < rows * per_row; i += (long)gridDim.x * 256) {
    const long r = i / per_row;
    const int e = (int)(i % per_row);
    if (e < dc) {
      dst[r * D + e] = src[r * D + e];
      continue;
    }
    const int pair = e - dc;
    const int slot = (int)(r / rope.tokens_per_frame), s = (int)(r % rope.tokens_per_frame);
    int64_t tau;
    if (slot < S) {
      tau = slot;
    } else {
      const int64_t f = w0 + (((int64_t)(slot - S) - (w0 - S)) % W + W) % W;
      tau = n_sink + (f - w0);
    }
    float a = (float)src[r * D + dc + 2 * pair], bb = (float)src[r * D + dc + 2 * pair + 1];
    rope.rotate2(pair, tau, s, a, bb);
    dst[r * D + dc + 2 * pair] = (T)a;
    dst[r * D + dc + 2 * pair + 1] = (T)bb;
  }
}

template <typename T>
static void assemble_t(const Plan& p, int64_t n, hipStream_t s) {
  const long rows = cached_frames(p, n) * p.Tpf;
  if (rows == 0) return;
  const long work = rows * (p.dc + p.dr / 2);
  const int gx = (int)((work + 255) / 256 < 2048 ? (work + 255) / 256 : 2048);
  assemble_window<T><<<dim3(gx, p.B), 256, 0, s>>>(static_cast<const T*>(p.cache), static_cast<T*>(p.assembled),
                                                    rows, (long)(p.S + p.W) * p.Tpf * p.D, n, p.S, p.W, p.dc, p.D,
                                                    make_rope(p));
}

hipError_t run_assemble(const Plan& p, int64_t n, hipStream_t s) {
  if (p.dtype == DType::F32) assemble_t<float>(p, n, s);
  else assemble_t<bf16>(p, n, s);
  return hipGetLastError();
}

template <typename T>
static hipError_t attend_t(const Plan& p, int64_t n, const void* x, void* out, hipStream_t s, hipEvent_t ev0,
                           hipEvent_t ev1) {
  const int M = p.B * p.Nq;
  // temporal coordinate of the chunk's first frame: absolute, or local (after the visible cached frames)
  const int64_t tq = p.rope_at_use ? cached_frames(p, n) : n;
  compress_t<T>(p, x, tq, p.stage, false, s);
  if (p.rope_at_use) assemble_t<T>(p, n, s);
  {  // c^Q = W_DQ x
    EpiStore<T> e{static_cast<T*>(p.cq), p.dq, 0};
    gemm<T, false>(ops<T>(p.w_dq, p.d, 0, x, p.d, 0, p.dq, M, p.d), 1, e, s);
  }
  {  // q = W_UQ c^Q -> q_nope, rotated/scaled q_rope into the absorbed query
    EpiQuery<T> e;
    e.qnope = static_cast<T*>(p.qnope);
    e.qt = static_cast<T*>(p.qt);
    e.Nq = p.Nq;
    e.nh = p.nh;
    e.d_nope = p.d_nope;
    e.dh = p.dh;
    e.dc = p.dc;
    e.D = p.D;
    e.qscale = p.qscale;
    e.rope = make_rope(p);
    e.frame0 = tq;
    gemm<T, false>(ops<T>(p.w_uq, p.dq, 0, p.cq, p.dq, 0, p.nh * p.dh, M, p.dq), 1, e, s);
  }
  if (p.d_nope > 0) {  // q~_h = W_UK^h^T q_nope_h for every head (z = head)
    EpiAbsorb<T> e{static_cast<T*>(p.qt), p.nh, p.D, p.qscale};
    gemm<T, true>(ops<T>(p.w_uk, p.dc, (long)p.d_nope * p.dc, p.qnope, (long)p.nh * p.d_nope, p.d_nope,
                         p.dc, M, p.d_nope),
                  p.nh, e, s);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  {
    AttnCall a;
    a.dtype = p.dtype;
    a.dc = p.dc;
    a.dr = p.dr;
    a.qt = p.qt;
    a.cache = p.rope_at_use ? p.assembled : p.cache;
    a.stage = p.stage;
    a.out = p.olat;
    a.part_o = p.part_o;
    a.part_ml = p.part_ml;
    a.vtiles = p.vtiles;
    a.cache_bstride = (long)(p.S + p.W) * p.Tpf * p.D;
    a.stage_bstride = (long)p.Nq * p.D;
    a.B = p.B;
    a.R = p.Nq * p.nh;
    a.n_ring = (int)(cached_frames(p, n) * p.Tpf);
    a.n_stage = p.Nq;
    a.G = p.G;
    a.ev_start = ev0;
    a.ev_stop = ev1;
    a.causal_tokens = p.causal_tokens;
    err = run_latent_attention(a, s);
    if (err != hipSuccess) return err;
  }
  {  // o_h = W_UV^h o~_h (z = head)
    EpiStore<T> e{static_cast<T*>(p.o), (long)p.nh * p.dv, p.dv};
    gemm<T, false>(ops<T>(p.w_uv, p.dc, (long)p.dv * p.dc, p.olat, (long)p.nh * p.dc, p.dc, p.dv, M, p.dc),
                   p.nh, e, s);
  }
  {  // out = W_O o
    EpiStore<T> e{static_cast<T*>(out), p.d, 0};
    gemm<T, false>(ops<T>(p.w_o, (long)p.nh * p.dv, 0, p.o, (long)p.nh * p.dv, 0, p.d, M, p.nh * p.dv), 1, e,
                   s);
  }
  return hipGetLastError();
}

hipError_t run_compress(const Plan& p, const void* x, int64_t frame0, void* dst, bool ring, hipStream_t s) {
  if (p.dtype == DType::F32)
    compress_t<float>(p, x, frame0, dst, ring, s);
  else
    compress_t<bf16>(p, x, frame0, dst, ring, s);
  return hipGetLastError();
}

hipError_t run_attend(const Plan& p, int64_t n, const void* x, void* out, hipStream_t s, hipEvent_t ev0,
                      hipEvent_t ev1) {
  if (p.dtype == DType::F32) return attend_t<float>(p, n, x, out, s, ev0, ev1);
  return attend_t<bf16>(p, n, x, out, s, ev0, ev1);
}

}  // namespace vmla
