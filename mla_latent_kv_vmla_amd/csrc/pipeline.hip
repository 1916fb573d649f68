// Launch sequences of the two library calls and the GEMM epilogues they use.
//
//   prepare (once per ctx): the concatenation [W_DKV; W_KR; W_DQ] (storage
//     type), and the weights the activation-type GEMMs consume, in that type
//     (fp16 for bf16 storage): the absorbed query weight
//     qscale * [W_UK^h^T W_UQ^h,nope ; W_UQ^h,rope] per head (the MLA
//     absorption, VideoMLA paper section 3.3, taken into the weight so one GEMM
//     yields the absorbed query), qscale * W_UQ, W_UV and W_O.
//   compress (VideoMLA paper, sections 3.1-3.2): one GEMM x . [W_DKV; W_KR]^T whose
//     epilogue rotates the decoupled key channels by 3D-RoPE at the absolute
//     frame (ring rows with rope_at_use stay un-rotated), rounds to the storage
//     type and scatters each token's row to its ring slot (slot * T + s; frames
//     f < S take sink slot f, later ones slot S + (f - S) % W) or to a linear
//     buffer.
//   attend: the chunk's cache rows into staging and c^Q = W_DQ x (one GEMM over
//     x with the prepared [W_DKV; W_KR; W_DQ]); with rope_at_use and fp32
//     storage, rotate the visible ring rows at their window-local coordinates
//     into the workspace (assemble_window; with bf16 storage the attention
//     pre-pass rotates them); absorbed query = prepared weight . c^Q
//     with the rotary channels turned in the epilogue; latent attention
//     (attention.hip); o_h = W_UV^h o~_h; out = W_O o.  Everything between x
//     and out is held in the activation type.
#include <type_traits>

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

// Absorbed query straight from c^Q through the prepared weight: feature n of
// token m is channel j = n % D of head n / D; channels [0, dc) are the content
// part qscale * W_UK^h^T q_nope, channels [dc, D) the rotary part qscale * q_rope,
// turned here at the token's (frame, row, column).
template <typename A> struct EpiQueryAbs {
  A* qt;  // [M][nh*D]
  int Nq, N, dc, D;
  int64_t frame0;
  Rope rope;
  uint32_t* flag;
  __device__ void operator()(int, int m, int n, const float* v) const {
    const int j = n % D;
    float a0 = v[0], a1 = v[1], a2 = v[2], a3 = v[3];
    if (j >= dc) {
      const int t = m % Nq;
      const int64_t frame = frame0 + t / rope.tokens_per_frame;
      const int s = t % rope.tokens_per_frame;
      const int pair = (j - dc) >> 1;
      rope.rotate2(pair, frame, s, a0, a1);
      rope.rotate2(pair + 1, frame, s, a2, a3);
    }
    store4(qt + (long)m * N + n, a0, a1, a2, a3, flag);
  }
};

// One GEMM over the chunk's hidden states with the prepared weight [W_DKV; W_KR;
// W_DQ]: features [0, D) are the chunk's cache rows (EpiLatent to the staging
// buffer), features [D, D + d_q) are c^Q (activation type).  The row features
// accumulate in the same k order as in a compress alone, so the staged rows
// are the ones an append of the same x would write.
template <typename T, typename A> struct EpiLatentCq {
  EpiLatent<T> lat;
  A* cq;
  int dq;
  uint32_t* flag;
  __device__ void operator()(int z, int m, int n, const float* v) const {
    if (n < lat.D) lat(z, m, n, v);
    else store4(cq + (long)m * dq + (n - lat.D), v[0], v[1], v[2], v[3], flag);
  }
};

// ---------------------------------------------------------------- prepare
// Absorbed query weight, head h = row / D, channel j = row % D, column k:
//   j <  dc: qscale * sum_i W_UK^h[i][j] * W_UQ[h*dh + i][k]   (i < d_nope)
//   j >= dc: qscale * W_UQ[h*dh + d_nope + (j - dc)][k]
// One thread per element, fp32 sums of the stored weights, one rounding.
template <typename T, typename A>
__global__ __launch_bounds__(256) void derive_query_weight(A* wqa, const T* w_uq, const T* w_uk, int nh, int d_nope,
                                                           int dr, int dc, int dq, float qscale, uint32_t* flag) {
  const int D = dc + dr, dh = d_nope + dr;
  const long total = (long)nh * D * dq;
  bool over = false;
  for (long e = (long)blockIdx.x * 256 + threadIdx.x; e < total; e += (long)gridDim.x * 256) {
    const int k = (int)(e % dq);
    const long row = e / dq;
    const int j = (int)(row % D), h = (int)(row / D);
    float acc;
    if (j < dc) {
      acc = 0.f;
      for (int i = 0; i < d_nope; ++i)
        acc += (float)w_uk[((long)h * d_nope + i) * dc + j] * (float)w_uq[((long)h * dh + i) * dq + k];
    } else {
      acc = (float)w_uq[((long)h * dh + d_nope + (j - dc)) * dq + k];
    }
    acc *= qscale;
    if constexpr (sizeof(A) == 2) wqa[e] = to_f16_sat(acc, over);
    else wqa[e] = acc;
  }
  raise_range_flag(over, flag);
}

// dst[i] = scale * src[i] in the activation type.
template <typename T, typename A>
__global__ __launch_bounds__(256) void convert_weight(A* dst, const T* src, long n, float scale, uint32_t* flag) {
  bool over = false;
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long)gridDim.x * 256) {
    const float v = (float)src[i] * scale;
    if constexpr (sizeof(A) == 2) dst[i] = to_f16_sat(v, over);
    else dst[i] = v;
  }
  raise_range_flag(over, flag);
}

// Plain copy of n elements (16-byte vectors; n a multiple of 16 B / sizeof(T)).
template <typename T>
__global__ __launch_bounds__(256) void copy_rows(T* dst, const T* src, long n) {
  const long nv = n * (long)sizeof(T) / 16;
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < nv; i += (long)gridDim.x * 256)
    reinterpret_cast<u32x4*>(dst)[i] = reinterpret_cast<const u32x4*>(src)[i];
}

__global__ void clear_flags(uint32_t* flags) { *flags = 0u; }

hipError_t run_clear_flags(uint32_t* flags, hipStream_t s) {
  clear_flags<<<1, 1, 0, s>>>(flags);
  return hipGetLastError();
}

static int grid_for(long n) { return (int)((n + 255) / 256 < 2048 ? (n + 255) / 256 : 2048); }

template <typename T, typename A>
static void prepare_t(const Plan& p, hipStream_t s) {
  clear_flags<<<1, 1, 0, s>>>(p.flags);
  {  // [W_DKV; W_KR; W_DQ], storage type, rows of `hidden`
    T* wx = static_cast<T*>(p.wx);
    const long a = (long)p.dc * p.d, b = (long)p.dr * p.d, c = (long)p.dq * p.d;
    copy_rows<T><<<grid_for(a * (long)sizeof(T) / 16), 256, 0, s>>>(wx, static_cast<const T*>(p.w_dkv), a);
    copy_rows<T><<<grid_for(b * (long)sizeof(T) / 16), 256, 0, s>>>(wx + a, static_cast<const T*>(p.w_kr), b);
    copy_rows<T><<<grid_for(c * (long)sizeof(T) / 16), 256, 0, s>>>(wx + a + b, static_cast<const T*>(p.w_dq), c);
  }
  const long nqa = (long)p.nh * p.D * p.dq;
  derive_query_weight<T, A><<<grid_for(nqa), 256, 0, s>>>(static_cast<A*>(p.wqa), static_cast<const T*>(p.w_uq),
                                                          static_cast<const T*>(p.w_uk), p.nh, p.d_nope, p.dr, p.dc,
                                                          p.dq, p.qscale, p.flags);
  const long nuq = (long)p.nh * p.dh * p.dq, nuv = (long)p.nh * p.dv * p.dc, no = (long)p.d * p.nh * p.dv;
  convert_weight<T, A><<<grid_for(nuq), 256, 0, s>>>(static_cast<A*>(p.wuq), static_cast<const T*>(p.w_uq), nuq,
                                                     p.qscale, p.flags);
  convert_weight<T, A><<<grid_for(nuv), 256, 0, s>>>(static_cast<A*>(p.wuv), static_cast<const T*>(p.w_uv), nuv,
                                                     1.f, p.flags);
  convert_weight<T, A><<<grid_for(no), 256, 0, s>>>(static_cast<A*>(p.wo), static_cast<const T*>(p.w_o), no, 1.f,
                                                    p.flags);
}

hipError_t run_prepare(const Plan& p, hipStream_t s) {
  if (p.dtype == DType::F32) prepare_t<float, float>(p, s);
  else prepare_t<bf16, f16>(p, s);
  return hipGetLastError();
}

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
static EpiLatent<T> latent_epilogue(const Plan& p, int64_t frame0, void* dst, bool ring) {
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
  return e;
}

template <typename T>
static void compress_t(const Plan& p, const void* x, int64_t frame0, void* dst, bool ring, hipStream_t s) {
  const int M = p.B * p.Nq;
  GemmOps<T> op = ops<T>(p.w_dkv, p.d, 0, x, p.d, 0, p.D, M, p.d);
  op.w2 = static_cast<const T*>(p.w_kr);
  op.n_split = p.dc;
  gemm<T, false>(op, 1, latent_epilogue<T>(p, frame0, dst, ring), s);
}

// The chunk's cache rows (rotated at frame frame0.., into p.stage) and c^Q
// (into p.cq), one GEMM with the prepared [W_DKV; W_KR; W_DQ].
template <typename T>
static void chunk_rows_and_cq_t(const Plan& p, const void* x, int64_t frame0, hipStream_t s) {
  using A = typename std::conditional<sizeof(T) == 2, f16, float>::type;
  const int M = p.B * p.Nq;
  EpiLatentCq<T, A> e{latent_epilogue<T>(p, frame0, p.stage, false), static_cast<A*>(p.cq), p.dq, p.flags};
  gemm<T, false>(ops<T>(p.wx, p.d, 0, x, p.d, 0, p.D + p.dq, M, p.d), 1, e, s);
}

hipError_t run_chunk_rows_and_cq(const Plan& p, const void* x, int64_t frame0, hipStream_t s) {
  if (p.dtype == DType::F32) chunk_rows_and_cq_t<float>(p, x, frame0, s);
  else chunk_rows_and_cq_t<bf16>(p, x, frame0, s);
  return hipGetLastError();
}

// rope_at_use: visible cache row r of stream b (slot r / T, token r % T) with
// k^ rotated at its frame's local coordinate: sink slot i holds frame i at
// coordinate i; window slot S + j holds the window frame f with (f - S) % W == j,
// at coordinate (sinks) + (f - first window frame).
template <typename T>
__global__ __launch_bounds__(256) void assemble_window(const T* cache, T* out, long rows, long bstride, int64_t n,
                                                       int S, int W, int dc, int D, Rope rope) {
  const int dr = D - dc, pairs = dr / 2;
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
    const int64_t tau = local_frame(slot, n, S, W);
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

// Activation type of a storage type: fp16 for bf16, fp32 for fp32.
template <typename T> using Act = typename std::conditional<sizeof(T) == 2, f16, float>::type;

template <typename T>
static hipError_t attend_t(const Plan& p, int64_t n, const void* x, void* out, hipStream_t s, hipEvent_t ev0,
                           hipEvent_t ev1) {
  using A = Act<T>;
  const int M = p.B * p.Nq;
  // temporal coordinate of the chunk's first frame: absolute, or local (after the visible cached frames)
  const int64_t tq = p.rope_at_use ? cached_frames(p, n) : n;
  chunk_rows_and_cq_t<T>(p, x, tq, s);  // the chunk's cache rows and c^Q = W_DQ x, one GEMM
  // rotation at use: fp32 storage rotates the visible rows into a copy; bf16
  // storage lets the attention pre-pass turn them as it converts them to fp16
  const bool rot_in_prepass = p.rope_at_use && sizeof(T) == 2;
  if (p.rope_at_use && !rot_in_prepass) assemble_t<T>(p, n, s);
  {  // absorbed query [qscale W_UK^T q_nope | RoPE(qscale q_rope)] per head, one GEMM from c^Q
    EpiQueryAbs<A> e;
    e.qt = static_cast<A*>(p.qt);
    e.Nq = p.Nq;
    e.N = p.nh * p.D;
    e.dc = p.dc;
    e.D = p.D;
    e.frame0 = tq;
    e.rope = make_rope(p);
    e.flag = p.flags;
    gemm<A, false>(ops<A>(p.wqa, p.dq, 0, p.cq, p.dq, 0, p.nh * p.D, M, p.dq), 1, e, s);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  {
    AttnCall a;
    a.dtype = p.dtype;
    a.dc = p.dc;
    a.dr = p.dr;
    a.range_flag = p.flags;
    a.qt = p.qt;
    a.cache = p.rope_at_use && !rot_in_prepass ? p.assembled : p.cache;
    a.rot_ring = rot_in_prepass ? 1 : 0;
    a.rot_S = p.S;
    a.rot_W = p.W;
    a.rot_n = n;
    a.pairs_t = p.pairs_t;
    a.pairs_h = p.pairs_h;
    a.grid_w = p.grid_w;
    a.tokens_per_frame = p.Tpf;
    for (int i = 0; i < kMaxRopePairs; ++i) a.freq[i] = p.freq[i];
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
    EpiStore<A> e{static_cast<A*>(p.o), (long)p.nh * p.dv, p.dv, p.flags};
    gemm<A, false>(ops<A>(p.wuv, p.dc, (long)p.dv * p.dc, p.olat, (long)p.nh * p.dc, p.dc, p.dv, M, p.dc), p.nh,
                   e, s);
  }
  {  // out = W_O o (storage type)
    EpiStore<T> e{static_cast<T*>(out), p.d, 0};
    gemm<A, false>(ops<A>(p.wo, (long)p.nh * p.dv, 0, p.o, (long)p.nh * p.dv, 0, p.d, M, p.nh * p.dv), 1, e, s);
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
