// Launch sequences of the two library calls and the GEMM epilogues they use.
//
//   prepare (once per ctx): the weights of the activation-type GEMMs, in that
//     type (fp16 for bf16 storage): [W_DKV; W_KR]; the absorbed query weight
//     qscale * [W_UK^h^T W_UQ^h,nope ; W_UQ^h,rope] W_DQ per head (the MLA
//     absorption, VideoMLA paper section 3.3, taken into the weight, and the
//     query down-projection with it, so one GEMM over x yields the absorbed
//     query); qscale * W_UQ W_DQ; W_UV and W_O.
//   compress (VideoMLA paper, sections 3.1-3.2): one GEMM x . [W_DKV; W_KR]^T whose
//     epilogue rotates the decoupled key channels by 3D-RoPE at the absolute
//     frame (ring rows with rope_at_use stay un-rotated), rounds to the storage
//     type and scatters each token's row to its ring slot (slot * T + s; frames
//     f < S take sink slot f, later ones slot S + (f - S) % W) or to a linear
//     buffer.
//   attend: the chunk's cache rows into staging and the absorbed query, one GEMM
//     over x with the prepared [W_DKV; W_KR] and query weight, the query's rotary
//     channels turned in the epilogue; with rope_at_use and fp32 storage, rotate
//     the visible ring rows at their window-local coordinates into the workspace
//     (assemble_window; with bf16 storage the attention pre-pass rotates them);
//     latent attention (attention.hip); o_h = W_UV^h o~_h; out = W_O o.
//     Everything between x and out is held in the activation type.
#include <type_traits>

#include "gemm.h"
#include "plan.h"

namespace vmla {

static Rope make_rope(const Plan& p) {
  Rope r;
  r.set(p.pairs_t, p.pairs_h, p.grid_w, p.Tpf, p.freq, kMaxRopePairs, p.rope_tab, rope_tab_stride(p.Tpf, p.grid_w));
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
  int W, S, dc, D;
  int ring, rotate;
  // ring slot of chunk frame i: i + wrel < 0 -> sink slot frame0 + i, else
  // S + ((i + wrel) mod W); wrel = (frame0 - S) mod W when frame0 >= S, else
  // frame0 - S (negative), so i + wrel < W + C <= 2W (no 64-bit modulo per token)
  int wrel;
  FastDiv nq;     // chunk tokens per stream
  Rope rope;
  // the chunk tokens' cos and sin per pair of pairs ([t][pair / 2], chunk_rope
  // layout), or null: then computed here
  const float4* ctab = nullptr;
  int hp = 0;     // pairs of pairs per token in ctab
  // features n..n+3 of token m after the rotation of the decoupled key channels
  __device__ void values(int m, int n, const float* v, float* a) const {
    a[0] = v[0], a[1] = v[1], a[2] = v[2], a[3] = v[3];
    if (n >= dc && rotate) {
      const int t = (int)nq.mod(m);
      const int pair = (n - dc) >> 1;
      if (ctab) {
        const float4 c = ctab[t * hp + (pair >> 1)];
        Rope::turn(c.x, c.y, a[0], a[1]);
        Rope::turn(c.z, c.w, a[2], a[3]);
      } else {
        const int64_t frame = frame0 + (int)rope.tpf.div(t);
        const int s = (int)rope.tpf.mod(t);
        rope.template rotate2<true>(pair, frame, s, a[0], a[1]);
        rope.template rotate2<true>(pair + 1, frame, s, a[2], a[3]);
      }
    }
  }
  __device__ T* row(int, int m, int n) const {
    const int b = (int)nq.div(m), t = m - b * (int)nq.d;
    long r = t;
    if (ring) {
      const int i = (int)rope.tpf.div(t), s = t - i * rope.tokens_per_frame;
      const int rel = i + wrel;
      const long slot = rel < 0 ? (long)(frame0 + i) : (long)S + (rel >= W ? rel - W : rel);
      r = slot * rope.tokens_per_frame + s;
    }
    return dst + b * bstride + r * D + n;
  }
  __device__ void operator()(int z, int m, int n, const float* v) const {
    float a[4];
    values(m, n, v, a);
    store4(row(z, m, n), a[0], a[1], a[2], a[3]);
  }
  static constexpr bool kRows = sizeof(T) == 2;
  __device__ u32x2 pack(int, int m, int n, const float* v, bool& over) const {
    float a[4];
    values(m, n, v, a);
    if constexpr (sizeof(T) == 2) return pack4<T>(a[0], a[1], a[2], a[3], over);
    else return u32x2{0u, 0u};
  }
  __device__ void raise(bool) const {}
  bool rows_aligned() const { return (uintptr_t)dst % 16 == 0 && D % 8 == 0 && bstride % 8 == 0; }
};

// Absorbed query straight from c^Q through the prepared weight: feature n of
// token m is channel j = n % D of head n / D; channels [0, dc) are the content
// part qscale * W_UK^h^T q_nope, channels [dc, D) the rotary part qscale * q_rope,
// turned here at the token's (frame, row, column).
template <typename A> struct EpiQueryAbs {
  A* qt;  // [M][nh*D]
  int N, dc;
  FastDiv nq, dd;  // chunk tokens per stream; D = dc + dr features per head
  int64_t frame0;
  Rope rope;
  uint32_t* flag;
  const float4* ctab = nullptr;  // as in EpiLatent
  int hp = 0;
  __device__ void values(int m, int n, const float* v, float* a) const {
    const int j = (int)dd.mod(n);
    a[0] = v[0], a[1] = v[1], a[2] = v[2], a[3] = v[3];
    if (j >= dc) {
      const int t = (int)nq.mod(m);
      const int pair = (j - dc) >> 1;
      if (ctab) {
        const float4 c = ctab[t * hp + (pair >> 1)];
        Rope::turn(c.x, c.y, a[0], a[1]);
        Rope::turn(c.z, c.w, a[2], a[3]);
      } else {
        const int64_t frame = frame0 + (int)rope.tpf.div(t);
        const int s = (int)rope.tpf.mod(t);
        rope.template rotate2<true>(pair, frame, s, a[0], a[1]);
        rope.template rotate2<true>(pair + 1, frame, s, a[2], a[3]);
      }
    }
  }
  __device__ A* row(int, int m, int n) const { return qt + (long)m * N + n; }
  __device__ void operator()(int z, int m, int n, const float* v) const {
    float a[4];
    values(m, n, v, a);
    store4(row(z, m, n), a[0], a[1], a[2], a[3], flag);
  }
  static constexpr bool kRows = sizeof(A) == 2;
  __device__ u32x2 pack(int, int m, int n, const float* v, bool& over) const {
    float a[4];
    values(m, n, v, a);
    if constexpr (sizeof(A) == 2) return pack4<A>(a[0], a[1], a[2], a[3], over);
    else return u32x2{0u, 0u};
  }
  __device__ void raise(bool over) const { raise_range_flag(over, flag); }
  bool rows_aligned() const { return (uintptr_t)qt % 16 == 0 && N % 8 == 0; }
};

// Per-head query of the non-absorbed form, [q_nope | RoPE(q_rope)] * qscale:
// feature n of token m is channel j = n % dh of head n / dh, written to the dense
// query layout [B][nh][Nq][dh].
struct EpiQueryHead {
  f16* q;
  int nh, dh, d_nope;
  FastDiv nq, hd;  // chunk tokens per stream; dh features per head
  int64_t frame0;
  Rope rope;
  uint32_t* flag;
  const float4* ctab = nullptr;  // as in EpiLatent
  int hp = 0;
  __device__ void values(int m, int n, const float* v, float* a) const {
    const int t = (int)nq.mod(m), j = (int)hd.mod(n);
    a[0] = v[0], a[1] = v[1], a[2] = v[2], a[3] = v[3];
    if (j >= d_nope) {
      const int pair = (j - d_nope) >> 1;
      if (ctab) {
        const float4 c = ctab[t * hp + (pair >> 1)];
        Rope::turn(c.x, c.y, a[0], a[1]);
        Rope::turn(c.z, c.w, a[2], a[3]);
      } else {
        const int64_t frame = frame0 + (int)rope.tpf.div(t);
        const int s = (int)rope.tpf.mod(t);
        rope.template rotate2<true>(pair, frame, s, a[0], a[1]);
        rope.template rotate2<true>(pair + 1, frame, s, a[2], a[3]);
      }
    }
  }
  __device__ f16* row(int, int m, int n) const {
    const int b = (int)nq.div(m), t = m - b * (int)nq.d, h = (int)hd.div(n), j = n - h * dh;
    return q + (((long)b * nh + h) * (int)nq.d + t) * dh + j;
  }
  __device__ void operator()(int z, int m, int n, const float* v) const {
    float a[4];
    values(m, n, v, a);
    store4(row(z, m, n), a[0], a[1], a[2], a[3], flag);
  }
  static constexpr bool kRows = true;
  __device__ u32x2 pack(int, int m, int n, const float* v, bool& over) const {
    float a[4];
    values(m, n, v, a);
    return pack4<f16>(a[0], a[1], a[2], a[3], over);
  }
  __device__ void raise(bool over) const { raise_range_flag(over, flag); }
  bool rows_aligned() const { return (uintptr_t)q % 16 == 0 && dh % 8 == 0; }
};

// One GEMM over the chunk's hidden states: features [0, D) are the chunk's cache
// rows (EpiLatent to the staging buffer), features [D, ...) the queries (Q, with
// the feature index rebased to 0).
template <typename T, class Q> struct EpiRowsAndQuery {
  EpiLatent<T> lat;
  Q q;
  __device__ void operator()(int z, int m, int n, const float* v) const {
    if (n < lat.D) lat(z, m, n, v);
    else q(z, m, n - lat.D, v);
  }
  static constexpr bool kRows = EpiLatent<T>::kRows && Q::kRows;
  __device__ u32x2 pack(int z, int m, int n, const float* v, bool& over) const {
    return n < lat.D ? lat.pack(z, m, n, v, over) : q.pack(z, m, n - lat.D, v, over);
  }
  __device__ void* row(int z, int m, int n) const {
    return n < lat.D ? (void*)lat.row(z, m, n) : (void*)q.row(z, m, n - lat.D);
  }
  __device__ void raise(bool over) const { q.raise(over); }
  // a 16-B chunk of features never straddles the two parts
  bool rows_aligned() const { return lat.D % 8 == 0 && lat.rows_aligned() && q.rows_aligned(); }
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

// out[r][k] = scale * sum_l a[r][l] * b[l][k]: a [R][L], b [L][K] row-major,
// fp32 products and sums, one rounding to the output type (saturating for
// fp16).  Plain LDS-tiled fp32 FMA (64x64 outputs per workgroup, 4x4 per
// thread, 16 l per step); it runs once per ctx.
template <typename TA, typename TB, typename O>
__global__ __launch_bounds__(256) void fold_weight(O* out, const TA* a, const TB* b, int R, int L, int K, float scale,
                                                   uint32_t* flag) {
  __shared__ float As[16][64 + 1];  // [l][r]
  __shared__ float Bs[16][64];      // [l][k]
  const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
  const int r0 = blockIdx.y * 64, k0 = blockIdx.x * 64;
  float acc[4][4] = {};
  for (int l0 = 0; l0 < L; l0 += 16) {
    for (int i = threadIdx.x; i < 16 * 64; i += 256) {
      const int ra = i / 16, la = i % 16, lb = i / 64, kb = i % 64;
      As[la][ra] = r0 + ra < R && l0 + la < L ? (float)a[(long)(r0 + ra) * L + l0 + la] : 0.f;
      Bs[lb][kb] = l0 + lb < L && k0 + kb < K ? (float)b[(long)(l0 + lb) * K + k0 + kb] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int l = 0; l < 16; ++l) {
      float av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = As[l][ty + 16 * i];
#pragma unroll
      for (int j = 0; j < 4; ++j) bv[j] = Bs[l][tx + 16 * j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(av[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }
  bool over = false;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = r0 + ty + 16 * i, k = k0 + tx + 16 * j;
      if (r >= R || k >= K) continue;
      const float v = acc[i][j] * scale;
      if constexpr (sizeof(O) == 2) out[(long)r * K + k] = to_f16_sat(v, over);
      else out[(long)r * K + k] = v;
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

// Rotary table: cos and sin of pos * freq[p] for every pair p of the row
// (pos < grid_h) and column (pos < grid_w) axes, the same sincosf of the same
// float argument as Rope::rotate2's direct evaluation.
__global__ __launch_bounds__(256) void rope_table(float* tab, int pairs, int pairs_t, int pairs_h, int grid_h,
                                                  int grid_w, int stride, Rope r) {
  for (int i = blockIdx.x * 256 + threadIdx.x; i < pairs * stride; i += gridDim.x * 256) {
    const int p = i / stride, pos = i % stride;
    if (p < pairs_t) continue;
    const int lim = p < pairs_t + pairs_h ? grid_h : grid_w;
    float sn = 0.f, cs = 1.f;
    if (pos < lim) sincosf((float)pos * r.freq[p], &sn, &cs);
    tab[2 * i] = cs;
    tab[2 * i + 1] = sn;
  }
}

hipError_t run_rope_table(float* tab, int pairs, int pairs_t, int pairs_h, int Tpf, int grid_w, const float* freq,
                          hipStream_t s) {
  Rope r;
  r.set(pairs_t, pairs_h, grid_w, Tpf, freq, kMaxRopePairs, nullptr, 0);
  const int stride = rope_tab_stride(Tpf, grid_w), n = pairs * stride;
  rope_table<<<(n + 255) / 256, 256, 0, s>>>(tab, pairs, pairs_t, pairs_h, Tpf / grid_w, grid_w, stride, r);
  return hipGetLastError();
}

hipError_t run_clear_flags(uint32_t* flags, hipStream_t s) {
  clear_flags<<<1, 1, 0, s>>>(flags);
  return hipGetLastError();
}

static int grid_for(long n) { return (int)((n + 255) / 256 < 2048 ? (n + 255) / 256 : 2048); }

template <typename TA, typename TB, typename O>
static void fold(O* out, const TA* a, const TB* b, int R, int L, int K, float scale, uint32_t* flag, hipStream_t s) {
  fold_weight<TA, TB, O><<<dim3((K + 63) / 64, (R + 63) / 64), 256, 0, s>>>(out, a, b, R, L, K, scale, flag);
}

template <typename T, typename A>
static void prepare_t(const Plan& p, hipStream_t s) {
  clear_flags<<<1, 1, 0, s>>>(p.flags);
  (void)run_rope_table(p.rope_tab, p.dr / 2, p.pairs_t, p.pairs_h, p.Tpf, p.grid_w, p.freq, s);  // errors: hipGetLastError below
  {  // [W_DKV; W_KR], rows of `hidden`
    A* wl = static_cast<A*>(p.wlat);
    const long a = (long)p.dc * p.d, b = (long)p.dr * p.d;
    convert_weight<T, A><<<grid_for(a), 256, 0, s>>>(wl, static_cast<const T*>(p.w_dkv), a, 1.f, p.flags);
    convert_weight<T, A><<<grid_for(b), 256, 0, s>>>(wl + a, static_cast<const T*>(p.w_kr), b, 1.f, p.flags);
  }
  // absorbed query weight over c^Q in fp32 (scratch), then W_DQ taken in
  float* wq32 = static_cast<float*>(p.prep);
  const long nqa = (long)p.nh * p.D * p.dq;
  derive_query_weight<T, float><<<grid_for(nqa), 256, 0, s>>>(wq32, static_cast<const T*>(p.w_uq),
                                                              static_cast<const T*>(p.w_uk), p.nh, p.d_nope, p.dr,
                                                              p.dc, p.dq, p.qscale, p.flags);
  const T* w_dq = static_cast<const T*>(p.w_dq);
  fold<float, T, A>(static_cast<A*>(p.wqa), wq32, w_dq, p.nh * p.D, p.dq, p.d, 1.f, p.flags, s);
  fold<T, T, A>(static_cast<A*>(p.wuq), static_cast<const T*>(p.w_uq), w_dq, p.nh * p.dh, p.dq, p.d, p.qscale,
                p.flags, s);
  const long nuv = (long)p.nh * p.dv * p.dc, no = (long)p.d * p.nh * p.dv;
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
  e.nq = FastDiv((uint32_t)p.Nq);
  e.W = p.W;
  e.S = p.S;
  e.wrel = frame0 >= p.S ? (int)((frame0 - p.S) % p.W) : (int)(frame0 - p.S);
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

// Activation type of a storage type: fp16 for bf16, fp32 for fp32.
template <typename T> using Act = typename std::conditional<sizeof(T) == 2, f16, float>::type;

// x (bf16) to the activation type, 8 elements per thread and step
// (bf16x8_to_f16x8: exact in fp16's normal range, saturating and flagging
// beyond it); n8 = elements / 8.  Then the chunk's rotary table: for chunk
// token t (frame frame0 + t / T) and pairs 2k, 2k+1, ctab[t][k] = (cos, sin,
// cos, sin) as Rope::angle gives them, so that the GEMM epilogues turn with the
// same values they would compute themselves (nq tokens, hp pairs of pairs).
__global__ __launch_bounds__(256) void convert_x(u32x4* dst, const u32x4* src, long n8, uint32_t* flag, float4* ctab,
                                                 int nq, int hp, int64_t frame0, Rope rope) {
  bool over = false;
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n8; i += (long)gridDim.x * 256)
    dst[i] = bf16x8_to_f16x8(src[i], over);
  raise_range_flag(over, flag);
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < (long)nq * hp; i += (long)gridDim.x * 256) {
    const int t = (int)(i / hp), k = (int)(i % hp);
    const int64_t frame = frame0 + (int)rope.tpf.div(t);
    const int s = (int)rope.tpf.mod(t);
    float4 c;
    rope.angle(2 * k, frame, s, c.x, c.y);
    rope.angle(2 * k + 1, frame, s, c.z, c.w);
    ctab[i] = c;
  }
}

// The chunk's cache rows (rotated at frames frame0.., into p.stage) and its
// queries, one GEMM over x in the activation type with the prepared [W_DKV;
// W_KR] and query weight.  The row features are the fp32 sums of the same
// products as in a compress of x (bf16 -> fp16 is exact in fp16's normal
// range), so the staged rows are, up to the order of the sums, the ones an
// append of the same x writes.
template <typename T, class Q>
static void rows_and_queries_t(const Plan& p, const void* x, int64_t frame0, const void* wq, int nq, const Q& q,
                               hipStream_t s) {
  using A = Act<T>;
  const int M = p.B * p.Nq;
  const void* xa = x;
  EpiRowsAndQuery<T, Q> e{latent_epilogue<T>(p, frame0, p.stage, false), q};
  if constexpr (!std::is_same<T, A>::value) {
    const long n8 = (long)M * p.d / 8;  // hidden is a multiple of 8 (config check)
    // the rotary table when each 4-feature group holds two whole pairs
    const bool tab = p.dc % 4 == 0 && p.dr % 4 == 0 && p.d_nope % 4 == 0;
    const int hp = tab ? p.dr / 4 : 0;
    convert_x<<<grid_for(n8), 256, 0, s>>>(static_cast<u32x4*>(p.xa), static_cast<const u32x4*>(x), n8, p.flags,
                                           static_cast<float4*>(p.ctab), p.Nq, hp, frame0, make_rope(p));
    xa = p.xa;
    if (tab) {
      e.lat.ctab = e.q.ctab = static_cast<const float4*>(p.ctab);
      e.lat.hp = e.q.hp = hp;
    }
  }
  GemmOps<A> op = ops<A>(p.wlat, p.d, 0, xa, p.d, 0, p.D + nq, M, p.d);
  op.w2 = static_cast<const A*>(wq);
  op.n_split = p.D;
  gemm<A, false>(op, 1, e, s);
}

template <typename T>
static void chunk_rows_and_queries_t(const Plan& p, const void* x, int64_t frame0, QueryForm form, void* qdst,
                                     hipStream_t s) {
  using A = Act<T>;
  if (form == QueryForm::Absorbed) {
    EpiQueryAbs<A> e;
    e.qt = static_cast<A*>(qdst);
    e.nq = FastDiv((uint32_t)p.Nq);
    e.dd = FastDiv((uint32_t)p.D);
    e.N = p.nh * p.D;
    e.dc = p.dc;
    e.frame0 = frame0;
    e.rope = make_rope(p);
    e.flag = p.flags;
    rows_and_queries_t<T>(p, x, frame0, p.wqa, p.nh * p.D, e, s);
  } else if constexpr (sizeof(T) == 2) {
    EpiQueryHead e;
    e.q = static_cast<f16*>(qdst);
    e.nq = FastDiv((uint32_t)p.Nq);
    e.hd = FastDiv((uint32_t)p.dh);
    e.nh = p.nh;
    e.dh = p.dh;
    e.d_nope = p.d_nope;
    e.frame0 = frame0;
    e.rope = make_rope(p);
    e.flag = p.flags;
    rows_and_queries_t<T>(p, x, frame0, p.wuq, p.nh * p.dh, e, s);
  }
}

hipError_t run_chunk_rows_and_queries(const Plan& p, const void* x, int64_t frame0, QueryForm form, void* q,
                                      hipStream_t s) {
  if (p.dtype == DType::F32) {
    if (form != QueryForm::Absorbed) return hipErrorInvalidValue;  // the expanded path is bf16 only
    chunk_rows_and_queries_t<float>(p, x, frame0, form, q, s);
  } else {
    chunk_rows_and_queries_t<bf16>(p, x, frame0, form, q, s);
  }
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

template <typename T>
static hipError_t attend_t(const Plan& p, int64_t n, const void* x, void* out, hipStream_t s, hipEvent_t ev0,
                           hipEvent_t ev1) {
  using A = Act<T>;
  const int M = p.B * p.Nq;
  // temporal coordinate of the chunk's first frame: absolute, or local (after the visible cached frames)
  const int64_t tq = p.rope_at_use ? cached_frames(p, n) : n;
  // the chunk's cache rows and the absorbed query [qscale W_UK^T q_nope | RoPE(qscale q_rope)], one GEMM over x
  chunk_rows_and_queries_t<T>(p, x, tq, QueryForm::Absorbed, p.qt, s);
  // rotation at use: fp32 storage rotates the visible rows into a copy; bf16
  // storage lets the attention pre-pass turn them as it converts them to fp16
  const bool rot_in_prepass = p.rope_at_use && sizeof(T) == 2;
  if (p.rope_at_use && !rot_in_prepass) assemble_t<T>(p, n, s);
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
    a.rope_tab = p.rope_tab;
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
