// The latent layer computed without absorption (VideoMLA paper, section 3.3:
// the cached latents are up-projected to per-head keys and values, which are
// then attended like a dense layer).  For the frozen-cache steps of a rollout
// (appendix D.5) the window is up-projected once per chunk and reused by every
// step:
//
//   expand: per stream and head, keys [W_UK^h c | k_r] of the valid ring rows
//     (one GEMM with the per-head lift [W_UK^h 0 ; 0 I], so k_r is copied
//     exactly, and turned at its local coordinate in the epilogue when the
//     cache holds it un-rotated) and values W_UV^h c, transposed (a GEMM with the operand
//     roles swapped, so each lane holds 4 consecutive keys of one value channel
//     and stores them together), then the value columns past the valid keys are
//     zeroed up to the key-tile boundary.
//   attend: the chunk's cache rows into staging and the per-head queries
//     [q_nope | RoPE(q_rope)] (not absorbed; the prepared qscale * W_UQ W_DQ),
//     one GEMM over x; the chunk's own keys and values by the same
//     up-projection, dense flash attention over the expanded window + chunk
//     (attention.hip), out = W_O o.
// Expanded keys and values, queries and the attention output are fp16, as in
// the dense layer; conversions saturate and raise the ctx's range flag.
#include "gemm.h"
#include "plan.h"

namespace vmla {

static Rope latent_rope(const Plan& p) {
  Rope r;
  r.set(p.pairs_t, p.pairs_h, p.grid_w, p.Tpf, p.freq, kMaxRopePairs, p.rope_tab, rope_tab_stride(p.Tpf, p.grid_w));
  return r;
}

// wext[h][r][c] (r < d_nope + d_r, c < d_c + d_r): W_UK^h[r][c] for r < d_nope and
// c < d_c; 1 where r - d_nope == c - d_c (copies k_r); 0 elsewhere.
__global__ __launch_bounds__(256) void build_key_lift(bf16* wext, const bf16* w_uk, int nh, int d_nope, int dc,
                                                      int dr) {
  const int D = dc + dr, dh = d_nope + dr;
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < (long)nh * dh * D; i += (long)gridDim.x * 256) {
    const int c = (int)(i % D);
    const long hr = i / D;
    const int r = (int)(hr % dh), h = (int)(hr / dh);
    float v;
    if (r < d_nope) v = c < dc ? (float)w_uk[((long)h * d_nope + r) * dc + c] : 0.f;
    else v = c == dc + (r - d_nope) ? 1.f : 0.f;
    wext[i] = (bf16)v;
  }
}

// Key rows: K[b][h][row m][n] (z = head).  With rot (ring rows of a
// rope_at_use layer, whose cache holds k^ un-rotated) the rotary features
// n >= d_nope are turned at the local coordinate of ring row m's frame.
struct EpiExpandKey {
  f16* k;
  long P;
  int nh, dh, b;
  uint32_t* flag;
  int rot, d_nope, S, W;
  int64_t n_frames;
  Rope rope;
  __device__ void operator()(int z, int m, int n, const float* v) const {
    float a0 = v[0], a1 = v[1], a2 = v[2], a3 = v[3];
    if (rot && n >= d_nope) {
      const int slot = (int)rope.tpf.div(m), s = m - slot * rope.tokens_per_frame;
      const int64_t tau = local_frame(slot, n_frames, S, W);
      const int pair = (n - d_nope) >> 1;
      rope.rotate2(pair, tau, s, a0, a1);
      rope.rotate2(pair + 1, tau, s, a2, a3);
    }
    store4(k + (((long)b * nh + z) * P + m) * dh + n, a0, a1, a2, a3, flag);
  }
};

// Transposed values from the swapped GEMM: "tokens" m are value channels,
// "features" n are key rows, so v holds keys n..n+3 of channel m.
struct EpiExpandValueT {
  f16* vt;
  long P;
  int nh, dv, b;
  uint32_t* flag;
  __device__ void operator()(int z, int m, int n, const float* v) const {
    store4(vt + (((long)b * nh + z) * dv + m) * P + (n & ~15) + perm16(n & 15), v[0], v[1], v[2], v[3], flag);
  }
};

template <typename T = bf16>
static GemmOps<T> gops(const void* w, long ldw, long wz, const void* x, long ldx, long xz, int N, int M, int K) {
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

static long round_up(long v, long m) { return (v + m - 1) / m * m; }

bool expanded_supported(const Plan& p) {
  return p.dtype == DType::BF16 && dense_attention_supported(DType::BF16, p.dh, p.dv);
}

// Up-project `rows` latent rows of every stream (row stride D, stream stride
// lat_bstride) into key rows / transposed value columns [0, rows) of stride P.
// rot_n >= 0: the rows are the ring of a rope_at_use layer after rot_n appends
// (k^ stored un-rotated; turned at use in the key epilogue).
static void up_project(const Plan& p, const DensePlan&, const bf16* wext, const void* lat, long lat_bstride,
                       int rows, f16* kdst, f16* vdst, long P, int64_t rot_n, hipStream_t s) {
  if (rows <= 0) return;
  for (int b = 0; b < p.B; ++b) {
    const bf16* lb = static_cast<const bf16*>(lat) + (long)b * lat_bstride;
    EpiExpandKey ek{kdst, P, p.nh, p.dh, b, p.flags, rot_n >= 0 ? 1 : 0, p.d_nope, p.S, p.W, rot_n,
                    latent_rope(p)};
    gemm<bf16, false>(gops(wext, p.D, (long)p.dh * p.D, lb, p.D, 0, p.dh, rows, p.D), p.nh, ek, s);
    EpiExpandValueT ev{vdst, P, p.nh, p.dv, b, p.flags};
    gemm<bf16, false>(gops(lb, p.D, 0, p.w_uv, p.dc, (long)p.dv * p.dc, rows, p.dv, p.dc), p.nh, ev, s);
  }
  zero_value_columns_async(vdst, (long)p.B * p.nh * p.dv, P, rows, (int)round_up(rows, kDenseKeyTile), s);
}

hipError_t run_expand(const Plan& p, const DensePlan& ex, void* wext_buf, int64_t n, hipStream_t s) {
  bf16* wext = static_cast<bf16*>(wext_buf);
  const long total = (long)p.nh * p.dh * p.D;
  build_key_lift<<<(int)((total + 255) / 256 < 1024 ? (total + 255) / 256 : 1024), 256, 0, s>>>(
      wext, static_cast<const bf16*>(p.w_uk), p.nh, p.d_nope, p.dc, p.dr);
  const int n_ring = (int)(cached_frames(p, n) * p.Tpf);
  // rope_at_use: the key epilogue turns k^ at each ring row's local coordinate
  up_project(p, ex, wext, p.cache, (long)(p.S + p.W) * p.Tpf * p.D, n_ring, static_cast<f16*>(ex.kring),
             static_cast<f16*>(ex.vring), ex.ring_stride, p.rope_at_use ? n : -1, s);
  return hipGetLastError();
}

hipError_t run_attend_expanded(const Plan& p, const DensePlan& ex, const void* wext, int64_t n, const void* x,
                               void* out, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
  const int M = p.B * p.Nq;
  const int64_t tq = p.rope_at_use ? cached_frames(p, n) : n;  // temporal coordinate of the chunk's first frame
  // the chunk's cache rows and its per-head queries, one GEMM over x
  hipError_t err = run_chunk_rows_and_queries(p, x, tq, QueryForm::PerHead, ex.q, s);
  if (err != hipSuccess) return err;
  up_project(p, ex, static_cast<const bf16*>(wext), p.stage, (long)p.Nq * p.D, p.Nq, static_cast<f16*>(ex.kstage),
             static_cast<f16*>(ex.vstage), ex.stage_stride, -1, s);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  {
    DenseAttnCall a;
    a.dh = p.dh;
    a.dv = p.dv;
    a.q = ex.q;
    a.kring = ex.kring;
    a.vring = ex.vring;
    a.kstage = ex.kstage;
    a.vstage = ex.vstage;
    a.out = ex.o;
    a.part_o = ex.part_o;
    a.part_ml = ex.part_ml;
    a.ev_start = ev0;
    a.ev_stop = ev1;
    a.B = p.B;
    a.H = p.nh;
    a.Nq = p.Nq;
    a.n_ring = (int)(cached_frames(p, n) * p.Tpf);
    a.ring_stride = ex.ring_stride;
    a.stage_stride = ex.stage_stride;
    a.G = ex.G;
    if ((err = run_dense_attention(a, s)) != hipSuccess) return err;
  }
  {  // out = W_O o (fp16 operands, bf16 result)
    EpiStore<bf16> e{static_cast<bf16*>(out), p.d, 0};
    gemm<f16, false>(gops<f16>(ex.wo, (long)p.nh * p.dv, 0, ex.o, (long)p.nh * p.dv, 0, p.d, M, p.nh * p.dv), 1, e,
                     s);
  }
  return hipGetLastError();
}

}  // namespace vmla
