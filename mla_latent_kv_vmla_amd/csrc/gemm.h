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
#include <type_traits>

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

constexpr int GEMM_BK = 64;         // k-values per pipeline stage (16-bit storage)
constexpr int GEMM_BK_SMALL = 128;  // the same for 64 x 64 tiles

template <typename T, int BN, int BM, bool W_KN, class Epi>
__global__ __launch_bounds__(256) void gemm_kernel(GemmOps<T> op, Epi epi) {
  using MF = Mfma<T>;
  // k-values per stage: deeper stages halve the global-load round trips of
  // these latency-bound GEMMs; 64x64 tiles afford 128 (~70 KB of LDS), larger
  // tiles 64 (two workgroups per CU); fp32 tiles keep 32 (LDS)
  constexpr int BK = sizeof(T) != 2 ? 32 : (BN == 64 && BM == 64 ? GEMM_BK_SMALL : GEMM_BK);
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

// ------------------------------------------------------------------------
// GEMM with LDS-DMA staging for 16-bit operands (W in Linear layout with one
// weight base, K a multiple of 64).  Same tile orientation and epilogue
// contract as gemm_kernel: features n are MFMA rows, tokens m MFMA columns.
//
// Staging: each 64-wide k stage of the W and X tiles is copied global -> LDS
// by buffer_load_dwordx4 ... lds (no registers, no VALU), NST stages in
// flight; a stage's loads are spread over the k sub-steps of the step before
// it, between its MFMAs.  The loads are issued from inline asm, so the compiler sees no LDS
// write it cannot order and does not wait for them before every LDS read; the
// kernel waits itself (vmcnt) before the barrier that publishes a stage.  Each
// tile's buffer resources start at its first row and end after its last valid
// row, so rows past N or M read as zero.
//
// LDS layout of one operand tile [rows][64] (128 B per row): rows are taken in
// pairs, pair R (rows 2R, 2R+1) fills 256 B, and 16-B chunk c (0..7) of row
// 2R + h sits at position (8h + c) ^ (R % 16) of the pair.  One wave-wide DMA
// load fills four pairs (1 KB), lanes 16j..16j+15 reading both rows of pair j
// as whole 128-B lines (half-line reads measured at half the rate).  A
// fragment read (16 lanes: 16 consecutive rows, one chunk) touches each 16-B
// bank group once.
// ------------------------------------------------------------------------
// Row epilogues.  An epilogue whose outputs are 16-bit values in rows that are
// contiguous along n may also provide
//   static constexpr bool kRows = true;
//   u32x2 pack(z, m, n, v[4], bool& over)  features n..n+3 of token m as four
//       16-bit values (its transforms and rounding; `over` set on saturation)
//   void* row(z, m, n)                     address of feature n of token m
//                                          (16-B aligned for n % 8 == 0)
//   void raise(bool over)                  record a saturation
//   bool rows_aligned() (host)             strides and base allow 16-B rows
// The DMA GEMM then stages its output tile through LDS and writes each token's
// features as whole 16-B chunks (16 lanes per 256 B of a row) instead of 8-B
// pieces of 32 different rows per store.
template <class E, class = void> struct HasRows : std::false_type {};
template <class E> struct HasRows<E, std::void_t<decltype(E::kRows)>> : std::integral_constant<bool, E::kRows> {};

// four values as 16-bit bit patterns: bf16 round to nearest even; fp16 round to
// nearest even, saturating finite values beyond its range (sets `over`)
template <typename O> __device__ inline u32x2 pack4(float a, float b, float c, float d, bool& over) {
  static_assert(sizeof(O) == 2, "16-bit output");
  if constexpr (std::is_same<O, f16>::value) {
    // one range test for the four values; the saturating path only when it fails
    const float mx = __builtin_fmaxf(__builtin_fmaxf(__builtin_fabsf(a), __builtin_fabsf(b)),
                                     __builtin_fmaxf(__builtin_fabsf(c), __builtin_fabsf(d)));
    if (!(mx > kF16Max))
      return u32x2{__builtin_bit_cast(uint32_t, f16x2{(f16)a, (f16)b}), __builtin_bit_cast(uint32_t, f16x2{(f16)c, (f16)d})};
    return u32x2{__builtin_bit_cast(uint32_t, f16x2{to_f16_sat(a, over), to_f16_sat(b, over)}),
                 __builtin_bit_cast(uint32_t, f16x2{to_f16_sat(c, over), to_f16_sat(d, over)})};
  } else {
    bf16x4 v;
    v[0] = (bf16)a; v[1] = (bf16)b; v[2] = (bf16)c; v[3] = (bf16)d;
    return __builtin_bit_cast(u32x2, v);
  }
}

template <typename T> struct GemmDmaOps {
  const T* w;    // [z][N][ldw], rows [0, N) in one buffer
  long ldw, wz;
  const T* x;    // [z][M][ldx]
  long ldx, xz;
  int N, M, K;
  int tn, tm, Z;  // tiles along N, along M, batch
};

template <typename T, int BN, int BM, int NWN, int NWM, int NST, class Epi>
__global__ __launch_bounds__(NWN * NWM * 64) void gemm_dma_kernel(GemmDmaOps<T> op, Epi epi) {
  static_assert(sizeof(T) == 2, "16-bit operands");
  using MF = Mfma<T>;
  constexpr int BK = 64;
  constexpr int NW = NWN * NWM;
  constexpr int WTN = BN / NWN, WTM = BM / NWM;  // wave tile
  constexpr int FN = WTN / 32, FM = WTM / 32;
  constexpr int BW = BN / 8, BX = BM / 8;        // 1-KB loads per stage of each operand
  constexpr int NLD = (BW + BX) / NW;            // DMA loads per wave per stage
  constexpr int STAGE = (BN + BM) * BK * 2;      // bytes
  static_assert(FN >= 1 && FM >= 1 && WTN % 32 == 0 && WTM % 32 == 0, "wave tile");
  static_assert(BW % NW == 0 && BX % NW == 0, "DMA split");
  static_assert(NST >= 2 && (NST - 2) * NLD < 64, "stages");
  // the 16-bit output tile [BM][BN] goes through LDS in rows of BN * 2 + 16 B
  constexpr int RS = BN * 2 + 16, CPR = BN / 8;
  constexpr int LDS_BYTES = HasRows<Epi>::value && BM * RS > NST * STAGE ? BM * RS : NST * STAGE;

  __shared__ __attribute__((aligned(1024))) char lds[LDS_BYTES];

  // XCD-aware tile order: launch index b runs on XCD b % 8; the tiles of one
  // XCD are consecutive in (z, m-tile, n-tile) order, so they share X rows.
  const int T_all = op.tn * op.tm * op.Z;
  const int per = (int)gridDim.x / 8;
  const int v = (int)(blockIdx.x % 8) * per + (int)(blockIdx.x / 8);
  if (v >= T_all) return;
  const int z = v / (op.tn * op.tm), rem = v % (op.tn * op.tm);
  const int n0 = (rem % op.tn) * BN, m0 = (rem / op.tn) * BM;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, h32 = lane >> 5;
  const int wn = wave % NWN, wm = wave / NWN;

  const T* wt = op.w + (long)z * op.wz + (long)n0 * op.ldw;
  const T* xt = op.x + (long)z * op.xz + (long)m0 * op.ldx;
  const int nrows_w = min(BN, op.N - n0), nrows_x = min(BM, op.M - m0);
  const auto rw = raw_rsrc(wt, (uint32_t)(((long)(nrows_w - 1) * op.ldw + op.K) * 2));
  const auto rx = raw_rsrc(xt, (uint32_t)(((long)(nrows_x - 1) * op.ldx + op.K) * 2));
  const auto rnone = raw_rsrc(op.w, 0u);

  // Load i of this wave fills 1-KB block j = wave + NW i of the stage (W tile
  // first, then X): row pairs 4jj..4jj+3 of its operand; lane L reads chunk
  // q & 7 of row 2R + q / 8, R = 4jj + L / 16, q = (L % 16) ^ (R % 16).
  uint32_t voff[NLD];
#pragma unroll
  for (int i = 0; i < NLD; ++i) {
    const bool isw = i < BW / NW;
    const int jj = isw ? wave + NW * i : wave + NW * i - BW;
    const int R = 4 * jj + (lane >> 4), q = (lane & 15) ^ (R & 15);
    const long ld = isw ? op.ldw : op.ldx;
    voff[i] = (uint32_t)(((long)(2 * R + (q >> 3)) * ld + 8 * (q & 7)) * 2);
  }
  const uint32_t lds0 = (uint32_t)(size_t)(__attribute__((address_space(3))) char*)lds;
  // loads i0 <= i < i1 of this wave for stage kt into LDS stage st
  auto issue = [&](int st, int kt, bool live, int i0, int i1) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      if (i < i0 || i >= i1) continue;
      const bool isw = i < BW / NW;
      const auto r = live ? (isw ? rw : rx) : rnone;
      dma16_lds(r, voff[i] + (uint32_t)(kt * BK * 2), lds0 + (uint32_t)(st * STAGE + (wave + NW * i) * 1024));
    }
  };

  f32x16 acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j) acc[i][j] = f32x16{};

  const int KT = op.K / BK;
#pragma unroll
  for (int s = 0; s < NST - 1; ++s) issue(s, s, s < KT, 0, NLD);
  int st = 0;
  for (int kt = 0; kt < KT; ++kt) {
    // this wave's loads of stage kt have landed; the barrier publishes every
    // wave's and frees the stage read in the previous step for the next loads
    wait_vmcnt<(NST - 2) * NLD>();
    __syncthreads();
    const int nst = st == 0 ? NST - 1 : st - 1, nkt = kt + NST - 1;
    const bool nlive = nkt < KT;
    const char* Wst = lds + st * STAGE;
    const char* Xst = Wst + BN * BK * 2;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      // the next stage's loads spread over the k sub-steps, between the MFMAs
      // (issued all at once after the barrier they delayed the first MFMAs)
      issue(nst, nkt, nlive, ks * NLD / (BK / 16), (ks + 1) * NLD / (BK / 16));
      // row r = 32 f + l32 of a fragment: pair r / 2, chunk 2 ks + h32
      const int lp = 256 * (l32 >> 1) + 16 * ((8 * (l32 & 1) + 2 * ks + h32) ^ (l32 >> 1));
      typename MF::Frag a[FN], b[FM];
#pragma unroll
      for (int i = 0; i < FN; ++i)
        a[i] = *reinterpret_cast<const typename MF::Frag*>(Wst + lp + (wn * WTN + 32 * i) * 128);
#pragma unroll
      for (int j = 0; j < FM; ++j)
        b[j] = *reinterpret_cast<const typename MF::Frag*>(Xst + lp + (wm * WTM + 32 * j) * 128);
#pragma unroll
      for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j) acc[i][j] = MF::mma(a[i], b[j], acc[i][j]);
    }
    st = st == NST - 1 ? 0 : st + 1;
  }
  // no DMA may still be writing this workgroup's LDS when it ends
  wait_vmcnt<0>();

  if constexpr (HasRows<Epi>::value) {
    // output tile [BM][BN] of 16-bit values through LDS, then whole 16-B
    // chunks of each token's row to the epilogue's destination
    __syncthreads();  // every wave is done reading the stages
    bool over = false;
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
      for (int j = 0; j < FM; ++j) {
        const int ml = wm * WTM + 32 * j + l32;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int nl = wn * WTN + 32 * i + 8 * q + 4 * h32;
          u32x2 bits = {0u, 0u};
          if (m0 + ml < op.M && n0 + nl < op.N) {
            float vv[4] = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
            bits = epi.pack(z, m0 + ml, n0 + nl, vv, over);
          }
          *reinterpret_cast<u32x2*>(lds + ml * RS + nl * 2) = bits;
        }
      }
    __syncthreads();
    for (int idx = tid; idx < BM * CPR; idx += NW * 64) {
      const int r = idx / CPR, c = idx % CPR;
      const int m = m0 + r, n = n0 + 8 * c;
      if (m < op.M && n < op.N)
        *reinterpret_cast<u32x4*>(epi.row(z, m, n)) = *reinterpret_cast<const u32x4*>(lds + r * RS + 16 * c);
    }
    epi.raise(over);
  } else {
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
      for (int j = 0; j < FM; ++j) {
        const int m = m0 + wm * WTM + 32 * j + l32;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = n0 + wn * WTN + 32 * i + 8 * q + 4 * h32;
          if (m < op.M && n < op.N) {
            float vv[4] = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
            epi(z, m, n, vv);
          }
        }
      }
  }
}

// Tile shapes of the DMA GEMM, two stages each:
// - 128 x 128, 4 waves (64 x 64 each): 64 KB of LDS, two workgroups per
//   compute unit;
// - 256 x 256, 8 waves (64 x 128 each): 128 KB of LDS (135 KB with the output
//   tile of a row epilogue), one workgroup per compute unit.
// On MI355X one round of 256 x 256 tiles (one per compute unit) took ~1.7x a
// round of 128 x 128 tiles (two per compute unit) on the Wan-1.3B projection
// shapes, the other 64..256-row shapes with 4 or 8 waves and 2..4 stages
// slower still; the larger tile is taken when it needs fewer rounds by that
// ratio (7/4), for epilogues that stage the output tile through LDS (the
// per-element epilogues keep the 128 x 128 tile: their 32 unrolled calls per
// lane at 256 x 256 do not stay in registers).
template <typename T, class Epi>
inline void launch_gemm_dma(GemmDmaOps<T> op, const Epi& epi, hipStream_t s) {
  const long t128 = (long)((op.N + 127) / 128) * ((op.M + 127) / 128) * op.Z;
  const long t256 = (long)((op.N + 255) / 256) * ((op.M + 255) / 256) * op.Z;
  const bool big = HasRows<Epi>::value && 7 * ((t256 + 255) / 256) < 4 * ((t128 + 511) / 512);
  const int BN = big ? 256 : 128, BM = BN;
  op.tn = (op.N + BN - 1) / BN;
  op.tm = (op.M + BM - 1) / BM;
  const int T_all = op.tn * op.tm * op.Z;
  const int grid = (T_all + 7) / 8 * 8;
  if constexpr (HasRows<Epi>::value) {
    if (big) {
      gemm_dma_kernel<T, 256, 256, 4, 2, 2, Epi><<<grid, 512, 0, s>>>(op, epi);
      return;
    }
  }
  gemm_dma_kernel<T, 128, 128, 2, 2, 2, Epi><<<grid, 256, 0, s>>>(op, epi);
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
  static constexpr bool kRows = sizeof(O) == 2;
  __device__ u32x2 pack(int, int, int, const float* v, bool& over) const {
    if constexpr (sizeof(O) == 2) return pack4<O>(v[0], v[1], v[2], v[3], over);
    else return u32x2{0u, 0u};
  }
  __device__ void* row(int z, int m, int n) const { return y + (long)z * yz + (long)m * ldy + n; }
  __device__ void raise(bool over) const { raise_range_flag(over, flag); }
  bool rows_aligned() const { return (uintptr_t)y % 16 == 0 && ldy % 8 == 0 && yz % 8 == 0; }
};

// Tile shape: the largest of (features x tokens) = 128x128, 128x64, 64x128,
// 64x64 that wastes at most 15% of the padded tile area and still launches
// >= 256 workgroups (one per compute unit); otherwise the shape with the most
// workgroups.
template <typename T, bool W_KN, class Epi>
inline void gemm(const GemmOps<T>& op, int Z, const Epi& epi, hipStream_t s) {
  if constexpr (sizeof(T) == 2 && !W_KN) {
    // the DMA kernel: 16-byte aligned rows, K in 64-wide stages, one weight base
    const bool one_base = op.n_split >= op.N || op.w2 == op.w + (long)op.n_split * op.ldw;
    const bool aligned = ((uintptr_t)op.w | (uintptr_t)op.x) % 16 == 0 && op.ldw % 8 == 0 && op.ldx % 8 == 0 &&
                         op.wz % 8 == 0 && op.xz % 8 == 0;
    // at least half the compute units busy with 128 x 128 tiles (smaller problems
    // keep the register-staged kernel's smaller tiles)
    const long tiles = (long)((op.N + 127) / 128) * ((op.M + 127) / 128) * Z;
    bool rows_ok = true;
    if constexpr (HasRows<Epi>::value) rows_ok = op.N % 8 == 0 && epi.rows_aligned();
    if (op.K % 64 == 0 && op.ldw >= op.K && op.ldx >= op.K && one_base && aligned && rows_ok && tiles >= 128) {
      GemmDmaOps<T> d;
      d.w = op.w;
      d.ldw = op.ldw;
      d.wz = op.wz;
      d.x = op.x;
      d.ldx = op.ldx;
      d.xz = op.xz;
      d.N = op.N;
      d.M = op.M;
      d.K = op.K;
      d.Z = Z;
      launch_gemm_dma<T>(d, epi, s);
      return;
    }
  }
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
