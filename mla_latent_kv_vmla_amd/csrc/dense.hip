// Launch sequences of the dense per-head baseline (VideoMLA paper, section 1 and
// appendix C.1: the layer whose cache holds every head's key and value).
//
//   prepare (once per ctx): the fp16 copy of W_O.
//   append: one GEMM x . [W_K; W_V]^T whose epilogue rotates each head's key by
//     3D-RoPE (all d_h channels, absolute frame index), writes it (fp16) to the
//     key row of its ring slot, and writes the value transposed (fp16) to the
//     value column of that slot; then the value columns past the valid keys up
//     to the next key-tile boundary are zeroed, so the attention kernel can
//     stage whole tiles.
//   attend: q = RoPE(W_Q x) scaled by log2(e)/sqrt(d_h) (fp16); the chunk's own
//     keys and values into staging with the same epilogue; dense flash
//     attention over ring + chunk on fp16 operands (attention.hip); out = W_O o.
// Keys, values, queries and the attention output are fp16: 16-bit like the
// pages' bf16 cache, with 11 significant bits.  Conversions saturate beyond
// fp16's range and raise the ctx's range flag.
#include "gemm.h"
#include "plan.h"

namespace vmla {

static Rope dense_rope(const DensePlan& p) {
  Rope r;
  r.set(p.pairs_t, p.pairs_h, p.grid_w, p.Tpf, p.freq, kMaxRopePairs, p.rope_tab, rope_tab_stride(p.Tpf, p.grid_w));
  return r;
}

// q[(b*nh + h)][t][j] = qscale * RoPE(W_Q^h x_t)[j]; token m is chunk token
// m % Nq of stream m / Nq, in frame frame0 + t / T.
struct EpiDenseQ {
  f16* q;
  int Nq, nh, dh;
  FastDiv nq, hd;  // Nq, dh
  float qscale;
  int64_t frame0;
  Rope rope;
  uint32_t* flag;
  __device__ void operator()(int, int m, int n, const float* v) const {
    const int b = (int)nq.div(m), t = m - b * Nq, h = (int)hd.div(n), j = n - h * dh;
    const int64_t frame = frame0 + (int)rope.tpf.div(t);
    const int s = (int)rope.tpf.mod(t);
    float a0 = v[0], a1 = v[1], a2 = v[2], a3 = v[3];
    rope.template rotate2<true>(j >> 1, frame, s, a0, a1);
    rope.template rotate2<true>((j >> 1) + 1, frame, s, a2, a3);
    store4(q + (((long)b * nh + h) * Nq + t) * dh + j, a0 * qscale, a1 * qscale, a2 * qscale, a3 * qscale, flag);
  }
};

// Features [0, nh*dh) are keys, [nh*dh, nh*(dh+dv)) values.  Key row / value
// column of token t: its ring slot row (frame % W)*T + s, or t for staging.
struct EpiDenseKV {
  f16* k;  // [B][nh][P][dh]
  f16* v;  // [B][nh][dv][P]
  long P;
  int Nq, nh, dh, dv, W;
  int ring;
  int wrel;  // frame0 mod W: chunk frame i sits in slot (wrel + i) mod W, wrel + i < 2W
  FastDiv nq, hd, vd;  // Nq, dh, dv
  int64_t frame0;
  Rope rope;
  uint32_t* flag;
  __device__ void operator()(int, int m, int n, const float* x) const {
    const int b = (int)nq.div(m), t = m - b * Nq;
    const int i = (int)rope.tpf.div(t), s = t - i * rope.tokens_per_frame;
    const int64_t frame = frame0 + i;
    const int slot = wrel + i >= W ? wrel + i - W : wrel + i;
    const long row = ring ? (long)slot * rope.tokens_per_frame + s : (long)t;
    if (n < nh * dh) {
      const int h = (int)hd.div(n), j = n - h * dh;
      float a0 = x[0], a1 = x[1], a2 = x[2], a3 = x[3];
      rope.template rotate2<true>(j >> 1, frame, s, a0, a1);
      rope.template rotate2<true>((j >> 1) + 1, frame, s, a2, a3);
      store4(k + (((long)b * nh + h) * P + row) * dh + j, a0, a1, a2, a3, flag);
    } else {
      const int n2 = n - nh * dh, h = (int)vd.div(n2), f = n2 - h * dv;
      f16* dst = v + (((long)b * nh + h) * dv + f) * P + (row & ~15L) + perm16((int)(row & 15));
      bool over = false;
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[i * P] = to_f16_sat(x[i], over);
      raise_range_flag(over, flag);
    }
  }
};

// Zero the value columns of keys [c0, c1) in `rows` transposed rows of stride P.
__global__ __launch_bounds__(256) void zero_value_columns(f16* v, long rows, long P, int c0, int c1) {
  const long w = c1 - c0;
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < rows * w; i += (long)gridDim.x * 256) {
    const long r = i / w;
    const int j = c0 + (int)(i % w);
    v[r * P + (j & ~15) + perm16(j & 15)] = (f16)0.f;
  }
}

void zero_value_columns_async(void* v, long rows, long P, int c0, int c1, hipStream_t s) {
  if (c1 <= c0) return;
  const long work = rows * (c1 - c0);
  const int grid = (int)((work + 255) / 256 < 1024 ? (work + 255) / 256 : 1024);
  zero_value_columns<<<grid, 256, 0, s>>>(static_cast<f16*>(v), rows, P, c0, c1);
}

template <typename T = bf16>
static GemmOps<T> dense_ops(const void* w, const void* w2, int n_split, const void* x, long ldx, int N, int M,
                            int K) {
  GemmOps<T> o;
  o.w = static_cast<const T*>(w);
  o.w2 = static_cast<const T*>(w2);
  o.ldw = K;
  o.wz = 0;
  o.x = static_cast<const T*>(x);
  o.ldx = ldx;
  o.xz = 0;
  o.N = N;
  o.M = M;
  o.K = K;
  o.n_split = n_split;
  return o;
}

// K/V of x's tokens (frames frame0..) into the ring or the staging buffers.
static void dense_kv(const DensePlan& p, const void* x, int64_t frame0, bool ring, hipStream_t s) {
  EpiDenseKV e;
  e.k = static_cast<f16*>(ring ? p.kring : p.kstage);
  e.v = static_cast<f16*>(ring ? p.vring : p.vstage);
  e.P = ring ? p.ring_stride : p.stage_stride;
  e.Nq = p.Nq;
  e.nh = p.nh;
  e.dh = p.dh;
  e.dv = p.dv;
  e.W = p.W;
  e.ring = ring ? 1 : 0;
  e.wrel = (int)(frame0 % p.W);
  e.nq = FastDiv((uint32_t)p.Nq);
  e.hd = FastDiv((uint32_t)p.dh);
  e.vd = FastDiv((uint32_t)p.dv);
  e.frame0 = frame0;
  e.rope = dense_rope(p);
  e.flag = p.flags;
  gemm<bf16, false>(dense_ops(p.w_k, p.w_v, p.nh * p.dh, x, p.d, p.nh * (p.dh + p.dv), p.B * p.Nq, p.d), 1, e, s);
}

static int round_tile(long keys) {
  return (int)((keys + kDenseKeyTile - 1) / kDenseKeyTile * kDenseKeyTile);
}

__global__ __launch_bounds__(256) void dense_convert_weight(f16* dst, const bf16* src, long n, uint32_t* flag) {
  bool over = false;
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long)gridDim.x * 256)
    dst[i] = to_f16_sat((float)src[i], over);
  raise_range_flag(over, flag);
}

hipError_t run_dense_prepare(const DensePlan& p, hipStream_t s) {
  hipError_t err = run_clear_flags(p.flags, s);
  if (err != hipSuccess) return err;
  err = run_rope_table(p.rope_tab, p.dh / 2, p.pairs_t, p.pairs_h, p.Tpf, p.grid_w, p.freq, s);
  if (err != hipSuccess) return err;
  const long n = (long)p.d * p.nh * p.dv;
  dense_convert_weight<<<(int)((n + 255) / 256 < 2048 ? (n + 255) / 256 : 2048), 256, 0, s>>>(
      static_cast<f16*>(p.wo), static_cast<const bf16*>(p.w_o), n, p.flags);
  return hipGetLastError();
}

hipError_t run_dense_append(const DensePlan& p, int64_t n, const void* x, hipStream_t s) {
  dense_kv(p, x, n, true, s);
  // valid ring keys after this append: min(n + C, W) frames
  const int64_t frames = n + p.C < p.W ? n + p.C : p.W;
  const long valid = (long)frames * p.Tpf;
  zero_value_columns_async(p.vring, (long)p.B * p.nh * p.dv, p.ring_stride, (int)valid, round_tile(valid), s);
  return hipGetLastError();
}

hipError_t run_dense_attend(const DensePlan& p, int64_t n, const void* x, void* out, hipStream_t s,
                            hipEvent_t ev0, hipEvent_t ev1) {
  const int M = p.B * p.Nq;
  {
    EpiDenseQ e;
    e.q = static_cast<f16*>(p.q);
    e.Nq = p.Nq;
    e.nh = p.nh;
    e.dh = p.dh;
    e.nq = FastDiv((uint32_t)p.Nq);
    e.hd = FastDiv((uint32_t)p.dh);
    e.qscale = p.qscale;
    e.frame0 = n;
    e.rope = dense_rope(p);
    e.flag = p.flags;
    gemm<bf16, false>(dense_ops(p.w_q, p.w_q, p.nh * p.dh, x, p.d, p.nh * p.dh, M, p.d), 1, e, s);
  }
  dense_kv(p, x, n, false, s);
  zero_value_columns_async(p.vstage, (long)p.B * p.nh * p.dv, p.stage_stride, p.Nq, p.stage_stride, s);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  {
    DenseAttnCall a;
    a.dh = p.dh;
    a.dv = p.dv;
    a.q = p.q;
    a.kring = p.kring;
    a.vring = p.vring;
    a.kstage = p.kstage;
    a.vstage = p.vstage;
    a.out = p.o;
    a.part_o = p.part_o;
    a.part_ml = p.part_ml;
    a.ev_start = ev0;
    a.ev_stop = ev1;
    a.B = p.B;
    a.H = p.nh;
    a.Nq = p.Nq;
    a.n_ring = (int)((n < p.W ? n : p.W) * p.Tpf);
    a.ring_stride = p.ring_stride;
    a.stage_stride = p.stage_stride;
    a.G = p.G;
    err = run_dense_attention(a, s);
    if (err != hipSuccess) return err;
  }
  {  // out = W_O o (fp16 operands, bf16 result)
    EpiStore<bf16> e{static_cast<bf16*>(out), p.d, 0};
    gemm<f16, false>(dense_ops<f16>(p.wo, p.wo, p.d, p.o, (long)p.nh * p.dv, p.d, M, p.nh * p.dv), 1, e, s);
  }
  return hipGetLastError();
}

}  // namespace vmla
