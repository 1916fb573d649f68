// MFMA GEMM for the projections around latent attention:
//   Y[m][n] = sum_k X[m][k] * W[n][k]      (W in Linear layout [N][K])
//   Y[m][n] = sum_k X[m][k] * W[k][n]      (W_KN: W stored [K][N])
// batched over z with element strides.  Both operands have the type T (bf16,
// fp16 or fp32), accumulated in fp32.  The kernel computes tiles of Y^T
// (features n as MFMA rows, tokens m as MFMA columns), so each lane ends with
// four consecutive output features of one token -- the shape a rotary pair or
// a packed row store wants.  The epilogue functor receives (z, m, n, v[4]) for
// features n..n+3 of token m and owns every write.
#pragma once
#include "device_common.h"

namespace vmla {

template <typename T> struct GemmOps {
  const T* w;   // W base for rows [0, n_split)
  const T* w2;  // W base for rows [n_split, N) (row index rebased to 0); may equal w
  long ldw, wz; // W row stride and per-z stride (elements)
  const T* x;
  long ldx, xz; // X row stride and per-z stride (elements)
  int N, M, K, n_split;
};

#ifndef VMLA_GEMM_BK
#define VMLA_GEMM_BK 64
#endif
#ifndef VMLA_GEMM_BK_SMALL
#define VMLA_GEMM_BK_SMALL 128
#endif
constexpr int GEMM_BK = VMLA_GEMM_BK;  // k-values per pipeline stage (16-bit storage)

template <typename T, int BN, int BM, bool W_KN, class Epi>
__global__ __launch_bounds__(256) void gemm_kernel(GemmOps<T> op, Epi epi) {
  using MF = Mfma<T>;
  // k-values per stage: deeper stages halve the global-load round trips of
  // these latency-bound GEMMs; 64x64 tiles afford 128 (~70 KB of LDS), larger
  // tiles 64 (two workgroups per CU); fp32 tiles keep 32 (LDS)
  constexpr int BK = sizeof(T) != 2 ? 32 : (BN == 64 && BM == 64 ? VMLA_GEMM_BK_SMALL : GEMM_BK);
  constexpr int KPL = MF::KPL;
  constexpr int VEC = 16 / (int)sizeof(T);
  constexpr int STRIDE = BK + VEC;          // LDS row: BK k-values + 16 B pad
  constexpr int FN = BN / 64, FM = BM / 64;      // 32x32 tiles per wave (2x2 waves)
  constexpr int WV = BN * BK / VEC / 256;   // 16-B vectors per thread, W tile
  constexpr int XV = BM * BK / VEC / 256;
  static_assert(FN >= 1 && FM >= 1 && WV >= 1 && XV >= 1, "tile too small");

  __shared__ __attribute__((aligned(16))) T Ws[2][BN * STRIDE];
  __shared__ __attribute__((aligned(16))) T Xs[2][BM * STRIDE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, h32 = lane >> 5;
  const int wn = wave & 1, wm = wave >> 1;
  const int n0 = blockIdx.x * BN, m0 = blockIdx.y * BM, z = blockIdx.z;
  const T* wbase = op.w + (long)z * op.wz;
  const T* wbase2 = op.w2 + (long)z * op.wz;
  const T* xbase = op.x + (long)z * op.xz;

  u32x4 wr[WV], xr[XV];

  auto load_tiles = [&](int k0) {
#pragma unroll
    for (int i = 0; i < WV; ++i) {
      int v = tid + i * 256;
      u32x4 val = {0, 0, 0, 0};
      if constexpr (!W_KN) {
        int row = v / (BK / VEC), cv = v % (BK / VEC);
        int n = n0 + row, k = k0 + cv * VEC;
        if (n < op.N && k < op.K) {
          const T* src = n < op.n_split ? wbase + (long)n * op.ldw : wbase2 + (long)(n - op.n_split) * op.ldw;
          val = ld16(src + k);
        }
      } else {
        int krow = v / (BN / VEC), nv = v % (BN / VEC);
        int k = k0 + krow, n = n0 + nv * VEC;
        if (n < op.N && k < op.K) val = ld16(wbase + (long)k * op.ldw + n);
      }
      wr[i] = val;
    }
#pragma unroll
    for (int i = 0; i < XV; ++i) {
      int v = tid + i * 256;
      int row = v / (BK / VEC), cv = v % (BK / VEC);
      int m = m0 + row, k = k0 + cv * VEC;
      u32x4 val = {0, 0, 0, 0};
      if (m < op.M && k < op.K) val = ld16(xbase + (long)m * op.ldx + k);
      xr[i] = val;
    }
  };

  auto store_tiles = [&](int buf) {
#pragma unroll
    for (int i = 0; i < WV; ++i) {
      int v = tid + i * 256;
      if constexpr (!W_KN) {
        int row = v / (BK / VEC), cv = v % (BK / VEC);
        *reinterpret_cast<u32x4*>(&Ws[buf][row * STRIDE + cv * VEC]) = wr[i];
      } else {
        int krow = v / (BN / VEC), nv = v % (BN / VEC);
        const T* e = reinterpret_cast<const T*>(&wr[i]);
#pragma unroll
        for (int j = 0; j < VEC; ++j) Ws[buf][(nv * VEC + j) * STRIDE + krow] = e[j];
      }
    }
#pragma unroll
    for (int i = 0; i < XV; ++i) {
      int v = tid + i * 256;
      int row = v / (BK / VEC), cv = v % (BK / VEC);
      *reinterpret_cast<u32x4*>(&Xs[buf][row * STRIDE + cv * VEC]) = xr[i];
    }
  };

  f32x16 acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j) acc[i][j] = f32x16{};

  const int KT = (op.K + BK - 1) / BK;
  load_tiles(0);
  store_tiles(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < KT) load_tiles((kt + 1) * BK);
#pragma unroll
    for (int ks = 0; ks < BK / (2 * KPL); ++ks) {
      typename MF::Frag a[FN], b[FM];
      const int koff = ks * 2 * KPL + KPL * h32;
#pragma unroll
      for (int i = 0; i < FN; ++i)
        a[i] = MF::load(&Ws[buf][(wn * (BN / 2) + 32 * i + l32) * STRIDE + koff]);
#pragma unroll
      for (int j = 0; j < FM; ++j)
        b[j] = MF::load(&Xs[buf][(wm * (BM / 2) + 32 * j + l32) * STRIDE + koff]);
#pragma unroll
      for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j) acc[i][j] = MF::mma(a[i], b[j], acc[i][j]);
    }
    if (kt + 1 < KT) store_tiles(buf ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      const int m = m0 + wm * (BM / 2) + 32 * j + l32;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = n0 + wn * (BN / 2) + 32 * i + 8 * q + 4 * h32;
        if (m < op.M && n < op.N) {
          float v[4] = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
          epi(z, m, n, v);
        }
      }
    }
}

// Y[m][n] -> y[z*yz + m*ldy + n] in the output type O (fp16 outputs saturate
// and raise *flag, see store4)
template <typename O> struct EpiStore {
  O* y;
  long ldy, yz;
  uint32_t* flag = nullptr;
  __device__ void operator()(int z, int m, int n, const float* v) const {
    store4(y + (long)z * yz + (long)m * ldy + n, v[0], v[1], v[2], v[3], flag);
  }
};

// Tile shape: the largest of (features x tokens) = 128x128, 128x64, 64x128,
// 64x64 that wastes at most 15% of the padded tile area and still launches
// >= 256 workgroups (one per compute unit); otherwise the shape with the most
// workgroups.
template <typename T, bool W_KN, class Epi>
inline void gemm(const GemmOps<T>& op, int Z, const Epi& epi, hipStream_t s) {
  const int shapes[4][2] = {{128, 128}, {128, 64}, {64, 128}, {64, 64}};
  int pick = -1, best = 3;
  long best_wg = -1;
  for (int i = 0; i < 4; ++i) {
    const long bn = shapes[i][0], bm = shapes[i][1];
    const long tn = (op.N + bn - 1) / bn, tm = (op.M + bm - 1) / bm;
    const long wg = tn * tm * Z;
    const double waste = (double)(tn * bn) * (tm * bm) / ((double)op.N * op.M);
    if (pick < 0 && waste <= 1.15 && wg >= 256) pick = i;
    if (wg > best_wg) best_wg = wg, best = i;
  }
  if (pick < 0) pick = best;
  const int BN = shapes[pick][0], BM = shapes[pick][1];
  dim3 grid((op.N + BN - 1) / BN, (op.M + BM - 1) / BM, Z);
  if (BN == 128 && BM == 128) gemm_kernel<T, 128, 128, W_KN, Epi><<<grid, 256, 0, s>>>(op, epi);
  else if (BN == 128) gemm_kernel<T, 128, 64, W_KN, Epi><<<grid, 256, 0, s>>>(op, epi);
  else if (BM == 128) gemm_kernel<T, 64, 128, W_KN, Epi><<<grid, 256, 0, s>>>(op, epi);
  else gemm_kernel<T, 64, 64, W_KN, Epi><<<grid, 256, 0, s>>>(op, epi);
}

}  // namespace vmla
