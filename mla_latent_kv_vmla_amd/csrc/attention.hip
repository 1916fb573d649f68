// Flash-style absorbed latent attention for gfx950.
//
// Every query row (token, head) of a chunk attends to the same keys: the cache
// rows [c | k_r] of the visible frames followed by the chunk's own rows
// (VideoMLA paper, appendix D.4: chunk-causal, the whole chunk and the whole
// window are visible).  With the per-head key and value lifts absorbed
// (score = q~ . [c | k_r], output = sum p * c, lifted by W_UV afterwards), all
// heads share one [c | k_r] key tile and one c value tile, so each tile is
// staged in LDS once per workgroup and reused by all of its query rows.
//
// Work layout (one workgroup = NW waves, 32*NB query rows per wave):
//   S^T[key][row]  = K_tile[key][:] . Qt[row][:]      (32x32x16 MFMA, keys as MFMA rows)
//   O^T[f][row]   += C^T[f][key] * P^T[key][row]     (the S^T accumulator is already
//                                                      the B operand of this product)
// so softmax statistics live per lane (one query row per lane pair) and P never
// leaves registers.
//
// Staging.  A key tile lives in LDS twice: row-major [key][D] (storage type) for
// the score product, and transposed [channel][key] for the value product.  The
// row-major copy is loaded straight from the cache / chunk rows with LDS-DMA
// loads (global_load_lds_dwordx4: lane L's 16 bytes land at M0 + 16 L), and the
// transposed copy is an image that a pre-pass kernel builds once per call in the
// workspace, already in LDS layout, so staging needs no registers and no VALU.
// LDS layouts (per stage; two stages in two distinct arrays):
//   Ks  [KTILE][D + 16 B]: 16-B chunk q of row r lives at chunk q ^ ((r >> 4) & 3)
//   C^T [DCP][KTILE + 16 B]: within every 16-key group the key index has bits 2
//       and 3 swapped, so the 8 keys a lane feeds to one value MFMA are one
//       contiguous 16-B read.  Both layouts read without bank conflicts.
//
// Numerics.  With bf16 storage the value product runs on fp16 operands: the
// transposed image holds the latents converted bf16 -> fp16 (exact for
// magnitudes in fp16's normal range, below 65504) and P is rounded to fp16.  When
// the softmax is nearly flat every probability sits just below 1, where bf16's
// spacing (2^-8) exceeds the spread of the probabilities themselves; fp16's
// spacing there is 2^-11, at the same MFMA rate.
//
// Scheduling is stream-K over (stream, row block, key tile): workgroup w owns
// iterations [w*I/G, (w+1)*I/G).  A row block finished by one workgroup is
// written directly; a row block split across workgroups leaves unnormalised
// partial states (at most two per workgroup) that the combine kernel merges
// with the usual log-sum-exp rule.  Scores are in log2 units (log2(e) is
// folded into the query), and the running maximum is only moved when a block
// exceeds it by more than 2^8, which keeps rescaling of the accumulator rare.
#include <type_traits>

#include "device_common.h"
#include "plan.h"

namespace vmla {

template <typename T> struct AttnArgs {
  const T* qt;     // [B][R][D]
  const T* cache;  // [B][.][D]
  const T* stage;  // [B][n_stage][D]
  T* out;          // [B][R][DC]
  float* part_o;   // [2G][kAttnMaxRows][DC]
  float* part_ml;  // [2G][kAttnMaxRows][2]
  void* vtiles;    // [B][KT] value-tile images
  long cbs, sbs;
  int R, n_ring, n_keys, RB, KT, B, G;
};

constexpr float kRescaleSlack = 8.0f;  // log2 units

__device__ inline float xor32(float v) { return __shfl_xor(v, 32); }

// Compile-time geometry of one instantiation.
template <typename T, int DC, int DR, int KTILE> struct TileGeo {
  using VT = typename std::conditional<sizeof(T) == 2, f16, float>::type;  // value-product operand
  static_assert(sizeof(VT) == sizeof(T), "tile sizing assumes equal widths");
  static constexpr int D = DC + DR;
  static constexpr int DCP = (DC + 31) / 32 * 32;
  static constexpr int VEC = 16 / (int)sizeof(T);  // elements per 16-B chunk
  static constexpr int KS = D + VEC;               // row-major tile row (+16 B)
  static constexpr int CS = KTILE + VEC;           // transposed tile row (+16 B)
  static constexpr int KCH = KS / VEC;             // 16-B chunks per row-major row
  static constexpr int CCH = CS / VEC;             // 16-B chunks per transposed row
  static constexpr int KPOS = KTILE * KCH;         // chunks of the row-major tile
  static constexpr int CPOS = DCP * CCH;           // chunks of the transposed tile
  static constexpr int KS_EL = KTILE * KS;
  static constexpr int BUF_EL = KS_EL + DCP * CS;
  static constexpr int KI = (KPOS + 63) / 64;      // wave-wide 1-KB loads per stage
  static constexpr int CI = (CPOS + 63) / 64;
  static constexpr size_t IMG_BYTES = (size_t)CPOS * 16;
  static_assert(DC % VEC == 0 && DR % VEC == 0, "unsupported widths");
  static_assert((D / VEC) % 4 == 0, "chunk swizzle works within groups of 4 chunks");
  static_assert(KTILE % 32 == 0, "bad tile");
  __device__ static int perm_group(int kg) { return (kg & ~3) | ((kg & 1) << 1) | ((kg >> 1) & 1); }
};

// Key row `key` of stream b, clamped to the last valid key (rows past n_keys
// are masked out of the scores, so their contents never matter): ring rows
// first, then the chunk's staged rows.
template <typename T, int D>
__device__ inline const T* key_row(const AttnArgs<T>& p, int b, int key) {
  key = key < p.n_keys ? key : p.n_keys - 1;
  return key < p.n_ring ? p.cache + (long)b * p.cbs + (long)key * D
                        : p.stage + (long)b * p.sbs + (long)(key - p.n_ring) * D;
}

// Pre-pass: transposed value-tile images.  Image (b, t) holds, for the keys of
// tile t, rows = latent channels (zero rows pad DC up to a multiple of 32) in the
// value-operand type, keys permuted within 16-key groups.
template <typename T, int DC, int DR, int KTILE>
__global__ __launch_bounds__(256) void latent_value_tiles(AttnArgs<T> p) {
  using G = TileGeo<T, DC, DR, KTILE>;
  using VT = typename G::VT;
  constexpr int KG = KTILE / 4, CV = DC / G::VEC;
  const int t = blockIdx.x, b = blockIdx.y;
  VT* img = reinterpret_cast<VT*>(static_cast<char*>(p.vtiles) + ((size_t)b * p.KT + t) * G::IMG_BYTES);
  for (int v = threadIdx.x; v < KG * CV; v += 256) {
    const int kg = v % KG, c = v / KG;
    u32x4 k[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) k[j] = ld16(key_row<T, G::D>(p, b, t * KTILE + 4 * kg + j) + c * G::VEC);
    const int pcol = 4 * G::perm_group(kg);
#pragma unroll
    for (int e = 0; e < G::VEC; ++e) {
      VT* dst = img + (c * G::VEC + e) * G::CS + pcol;
      if constexpr (sizeof(T) == 2) {
        const int dw = e >> 1;
        auto widen = [&](uint32_t word) {
          return (e & 1) ? __uint_as_float(word & 0xFFFF0000u) : __uint_as_float(word << 16);
        };
        f16x4 h;
#pragma unroll
        for (int j = 0; j < 4; ++j) h[j] = (f16)widen(k[j][dw]);
        *reinterpret_cast<f16x4*>(dst) = h;
      } else {
        *reinterpret_cast<u32x4*>(dst) = u32x4{k[0][e], k[1][e], k[2][e], k[3][e]};
      }
    }
  }
  for (int i = threadIdx.x; i < (G::DCP - DC) * G::CS; i += 256) img[DC * G::CS + i] = VT(0.f);
}

template <typename T, int DC, int DR, int KTILE, int NW, int NB>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(8 / NW, 8 / NW)))
void latent_attn_kernel(AttnArgs<T> p) {
  using G = TileGeo<T, DC, DR, KTILE>;
  using VT = typename G::VT;
  using MF = Mfma<T>;
  constexpr bool HALF = sizeof(T) == 2;
  constexpr int KPL = MF::KPL;
  constexpr int D = G::D, DCP = G::DCP, VEC = G::VEC, KS = G::KS, CS = G::CS;
  constexpr int RW = 32 * NB;               // query rows per wave
  constexpr int NKS = D / (2 * KPL);
  constexpr int NKB = KTILE / 32;
  constexpr int NFB = DCP / 32;
  constexpr int NI = G::KI + G::CI;         // 1-KB loads per stage, spread over the waves
  constexpr int NI_W = (NI + NW - 1) / NW;
  static_assert(NW * RW <= kAttnMaxRows, "row block too large");

  __shared__ __attribute__((aligned(16))) T lds0[G::BUF_EL];
  __shared__ __attribute__((aligned(16))) T lds1[G::BUF_EL];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, h32 = lane >> 5;
  const float NEG_INF = -__builtin_huge_valf();

  // Row-major staging: for each of this wave's loads, the (row, chunk) whose
  // swizzled LDS position is this lane's slot, packed as row << 12 | element offset.
  int kslot[NI_W];
#pragma unroll
  for (int k = 0; k < NI_W; ++k) {
    const int pos = (wave + k * NW) * 64 + lane;
    const int r = pos / G::KCH, phys = pos % G::KCH;
    const int q = phys < G::KCH - 1 ? (phys ^ ((r >> 4) & 3)) : 0;  // pad slot: any valid chunk
    kslot[k] = (r << 12) | (q * VEC);
  }

  // Issue the LDS-DMA loads of tile kt (both layouts) into stage `buf`.
  auto issue_tile = [&](int b, int kt, T* buf) {
    const int kbase = kt * KTILE;
    const T* base = nullptr;
    if (kbase + KTILE <= p.n_ring) base = p.cache + (long)b * p.cbs + (long)kbase * D;
    else if (kbase >= p.n_ring && kbase + KTILE <= p.n_keys)
      base = p.stage + (long)b * p.sbs + (long)(kbase - p.n_ring) * D;
    const char* img = static_cast<const char*>(p.vtiles) + ((size_t)b * p.KT + kt) * G::IMG_BYTES;
#pragma unroll
    for (int k = 0; k < NI_W; ++k) {
      const int idx = wave + k * NW;  // wave-uniform
      if (idx < G::KI) {
        const int pos = idx * 64 + lane;
        if (G::KPOS % 64 == 0 || pos < G::KPOS) {
          const int r = kslot[k] >> 12, off = kslot[k] & 0xFFF;
          const T* src = base ? base + r * D + off : key_row<T, D>(p, b, kbase + r) + off;
          lds_dma16(src, buf + idx * 64 * VEC);
        }
      } else if (idx < NI) {
        const int ci = idx - G::KI, pos = ci * 64 + lane;
        if (G::CPOS % 64 == 0 || pos < G::CPOS)
          lds_dma16(img + (size_t)pos * 16, buf + G::KS_EL + ci * 64 * VEC);
      }
    }
  };

  const long I = (long)p.B * p.RB * p.KT;
  const long it0 = (long)blockIdx.x * I / p.G, it1 = (long)(blockIdx.x + 1) * I / p.G;

  for (long it = it0; it < it1;) {
    const long unit = it / p.KT;
    const int kt0 = (int)(it % p.KT);
    const int kt1 = (int)((long)kt0 + (it1 - it) < p.KT ? (long)kt0 + (it1 - it) : p.KT);
    const int b = (int)(unit / p.RB), rb = (int)(unit % p.RB);
    const bool first_piece = (it == it0);
    const int row0 = rb * (NW * RW) + wave * RW;

    typename MF::Frag qf[NB][NKS];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int qrow = row0 + 32 * nb + l32;
      const T* qsrc = p.qt + ((long)b * p.R + qrow) * D + KPL * h32;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) qf[nb][ks] = qrow < p.R ? MF::load(qsrc + ks * 2 * KPL) : MF::zero();
    }
    f32x16 o[NB][NFB];
    float m_run[NB], l_run[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      m_run[nb] = NEG_INF;
      l_run[nb] = 0.f;
#pragma unroll
      for (int fb = 0; fb < NFB; ++fb) o[nb][fb] = f32x16{};
    }

    // all query-row blocks of one tile held in `cur`
    auto compute = [&](int kt, const T* cur) {
      const T* Ks = cur;
      const VT* Ct = reinterpret_cast<const VT*>(cur + G::KS_EL) + l32 * CS;
      const int kbase = kt * KTILE;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        // S^T for 32 keys x RW query rows; each K fragment feeds NB MFMAs
        f32x16 s[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) s[nb] = f32x16{};
        const int r = 32 * kb + l32;
        if constexpr (HALF) {  // chunk 2ks+h, swizzled: two per-lane bases, immediate offsets
          const int sw = (r >> 4) & 3;
          const T* b0 = Ks + r * KS + ((h32 ^ sw) * VEC);
          const T* b1 = Ks + r * KS + (((2 + h32) ^ sw) * VEC);
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks) {
            const auto a = MF::load((ks & 1 ? b1 : b0) + 4 * VEC * (ks >> 1));
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) s[nb] = MF::mma(a, qf[nb][ks], s[nb]);
          }
        } else {
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks) {
            const int e = ks * 2 * KPL + KPL * h32;
            const auto a = MF::load(&Ks[r * KS + (((e / VEC) ^ ((r >> 4) & 3)) * VEC) + e % VEC]);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) s[nb] = MF::mma(a, qf[nb][ks], s[nb]);
          }
        }
        if (kbase + 32 * kb + 32 > p.n_keys) {
#pragma unroll
          for (int rr = 0; rr < 16; ++rr)
            if (kbase + 32 * kb + 8 * (rr >> 2) + 4 * h32 + (rr & 3) >= p.n_keys)
#pragma unroll
              for (int nb = 0; nb < NB; ++nb) s[nb][rr] = NEG_INF;
        }
        // online softmax per query row (lane pair); every piece's first block
        // holds a valid key, so m_run is finite before any all-masked block
        bool need[NB], any_need = false;
        float mx[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          float m = s[nb][0];
#pragma unroll
          for (int rr = 1; rr < 16; ++rr) m = fmaxf(m, s[nb][rr]);
          mx[nb] = fmaxf(m, xor32(m));
          need[nb] = mx[nb] > m_run[nb] + kRescaleSlack;
          any_need |= need[nb];
        }
        if (__any(any_need)) {
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            const float mnew = need[nb] ? mx[nb] : m_run[nb];
            const float alpha = __builtin_amdgcn_exp2f(m_run[nb] - mnew);
            m_run[nb] = mnew;
            l_run[nb] *= alpha;
#pragma unroll
            for (int fb = 0; fb < NFB; ++fb) o[nb][fb] *= alpha;
          }
        }
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          float lsum = 0.f;
#pragma unroll
          for (int rr = 0; rr < 16; ++rr) {
            const float e = __builtin_amdgcn_exp2f(s[nb][rr] - m_run[nb]);
            s[nb][rr] = e;
            lsum += e;
          }
          l_run[nb] += lsum;
        }
        // O^T += C^T[f][keys] * P^T[keys][rows]; each C^T fragment feeds NB MFMAs
        if constexpr (HALF) {
          f16x8 pf[NB][2];
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
              for (int j = 0; j < 8; ++j) pf[nb][u][j] = (f16)s[nb][8 * u + j];
#pragma unroll
          for (int fb = 0; fb < NFB; ++fb)
#pragma unroll
            for (int u = 0; u < 2; ++u) {
              const f16x8 a = *reinterpret_cast<const f16x8*>(Ct + 32 * fb * CS + 32 * kb + 16 * u + 8 * h32);
#pragma unroll
              for (int nb = 0; nb < NB; ++nb)
                o[nb][fb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, pf[nb][u], o[nb][fb], 0, 0, 0);
            }
        } else {
#pragma unroll
          for (int fb = 0; fb < NFB; ++fb)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const f32x4 run = *reinterpret_cast<const f32x4*>(Ct + 32 * fb * CS + 32 * kb + 16 * (g >> 1) +
                                                                8 * h32 + 4 * (g & 1));
#pragma unroll
              for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) o[nb][fb] = Mfma<float>::mma(run[i], s[nb][4 * g + i], o[nb][fb]);
            }
        }
      }
    };

    // One tile: prefetch the next tile into the other stage, compute this one,
    // then wait for this thread's loads and meet at the barrier (which also
    // retires every read of `cur` before it is refilled).
    auto step = [&](int kt, const T* cur, T* nxt) {
      if (kt + 1 < kt1) issue_tile(b, kt + 1, nxt);
      compute(kt, cur);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    };

    issue_tile(b, kt0, lds0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int kt = kt0; kt < kt1; kt += 2) {
      step(kt, lds0, lds1);
      if (kt + 1 < kt1) step(kt + 1, lds1, lds0);
    }

    const bool full = (kt0 == 0 && kt1 == p.KT);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const float l_tot = l_run[nb] + xor32(l_run[nb]);
      const int qrow = row0 + 32 * nb + l32;
      if (full) {
        if (qrow < p.R) {
          T* dst = p.out + ((long)b * p.R + qrow) * DC;
          const float inv = 1.f / l_tot;
#pragma unroll
          for (int fb = 0; fb < NFB; ++fb)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int f = 32 * fb + 8 * q + 4 * h32;
              if (f < DC)
                store4(dst + f, o[nb][fb][4 * q] * inv, o[nb][fb][4 * q + 1] * inv, o[nb][fb][4 * q + 2] * inv,
                       o[nb][fb][4 * q + 3] * inv);
            }
        }
      } else if (row0 < p.R) {
        const long slot_row =
            (long)(2 * blockIdx.x + (first_piece ? 0 : 1)) * kAttnMaxRows + wave * RW + 32 * nb + l32;
        float* po = p.part_o + slot_row * DC;
#pragma unroll
        for (int fb = 0; fb < NFB; ++fb)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int f = 32 * fb + 8 * q + 4 * h32;
            if (f < DC)
              *reinterpret_cast<f32x4*>(po + f) =
                  f32x4{o[nb][fb][4 * q], o[nb][fb][4 * q + 1], o[nb][fb][4 * q + 2], o[nb][fb][4 * q + 3]};
          }
        if (h32 == 0) {
          p.part_ml[slot_row * 2] = m_run[nb];
          p.part_ml[slot_row * 2 + 1] = l_tot;
        }
      }
    }
    it += kt1 - kt0;
  }
}

// Merge the partial states of every row block that was split across workgroups.
// Workgroups w0..w1 hold the pieces of row block `unit`; every piece is its
// workgroup's first (slot 2w) except possibly w0's, which is its second
// (slot 2w0+1) when w0 started inside an earlier row block.
template <typename T, int DC, int ROWS>
__global__ __launch_bounds__(256) void latent_attn_combine(AttnArgs<T> p) {
  constexpr int SLICE = 16;  // rows per workgroup: many small workgroups hide load latency
  const long unit = blockIdx.x / (ROWS / SLICE);
  const int r0 = (int)(blockIdx.x % (ROWS / SLICE)) * SLICE;
  const long I = (long)p.B * p.RB * p.KT;
  const long i0 = unit * p.KT, i1 = i0 + p.KT;
  auto start = [&](long w) { return w * I / p.G; };
  long w0 = i0 * p.G / I;
  while (w0 + 1 < p.G && start(w0 + 1) <= i0) ++w0;
  long w1 = (i1 - 1) * p.G / I;
  while (w1 + 1 < p.G && start(w1 + 1) <= i1 - 1) ++w1;
  if (w0 == w1) return;  // one workgroup finished this row block and wrote it
  const long slot0 = 2 * w0 + (start(w0) < i0 ? 1 : 0);
  const int npieces = (int)(w1 - w0 + 1);
  const int b = (int)(unit / p.RB), rb = (int)(unit % p.RB);
  constexpr int Q = DC / 4;  // float4 columns per row
  for (int task = threadIdx.x; task < SLICE * Q; task += 256) {
    const int r = r0 + task / Q, f = (task % Q) * 4;
    const int row = rb * ROWS + r;
    if (row >= p.R) continue;
    float M = -__builtin_huge_valf();
    for (int k = 0; k < npieces; ++k) {
      const long sr = (k == 0 ? slot0 : 2 * (w0 + k)) * kAttnMaxRows + r;
      M = fmaxf(M, p.part_ml[sr * 2]);
    }
    float L = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int k = 0; k < npieces; ++k) {
      const long sr = (k == 0 ? slot0 : 2 * (w0 + k)) * kAttnMaxRows + r;
      const float sc = __builtin_amdgcn_exp2f(p.part_ml[sr * 2] - M);
      L += p.part_ml[sr * 2 + 1] * sc;
      acc += sc * *reinterpret_cast<const f32x4*>(p.part_o + sr * DC + f);
    }
    const float inv = 1.f / L;
    store4(p.out + ((long)b * p.R + row) * DC + f, acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
  }
}

template <typename T, int DC, int DR, int KTILE, int NW, int NB>
static hipError_t launch_latent(const AttnCall& c, hipStream_t s) {
  constexpr int ROWS = NW * 32 * NB;
  AttnArgs<T> a;
  a.qt = static_cast<const T*>(c.qt);
  a.cache = static_cast<const T*>(c.cache);
  a.stage = static_cast<const T*>(c.stage);
  a.out = static_cast<T*>(c.out);
  a.part_o = c.part_o;
  a.part_ml = c.part_ml;
  a.vtiles = c.vtiles;
  a.cbs = c.cache_bstride;
  a.sbs = c.stage_bstride;
  a.R = c.R;
  a.n_ring = c.n_ring;
  a.n_keys = c.n_ring + c.n_stage;
  a.RB = (c.R + ROWS - 1) / ROWS;
  a.KT = (a.n_keys + KTILE - 1) / KTILE;
  a.B = c.B;
  const long I = (long)a.B * a.RB * a.KT;
  a.G = (int)(c.G < I ? c.G : I);
  latent_value_tiles<T, DC, DR, KTILE><<<dim3(a.KT, a.B), 256, 0, s>>>(a);
  hipError_t err;
  if (c.ev_start && (err = hipEventRecord(c.ev_start, s)) != hipSuccess) return err;
  latent_attn_kernel<T, DC, DR, KTILE, NW, NB><<<a.G, NW * 64, 0, s>>>(a);
  if (c.ev_stop && (err = hipEventRecord(c.ev_stop, s)) != hipSuccess) return err;
  if (I != (long)a.G * a.KT)
    latent_attn_combine<T, DC, ROWS><<<a.B * a.RB * (ROWS / 16), 256, 0, s>>>(a);
  return hipGetLastError();
}

// Kernel shape per built (dtype, d_c, d_rope): keys per tile, waves per
// workgroup, 32-row blocks per wave.
struct LatentShape {
  int ktile, nw, nb;
};

static bool latent_shape(DType dt, int dc, int dr, LatentShape& sh) {
  if (dt == DType::F32) {
    if (dc == 24 && dr == 8) return sh = {64, 4, 1}, true;
    return false;
  }
  if (dc == 24 && dr == 8) return sh = {64, 4, 1}, true;
  if (dr == 32 && dc == 96) return sh = {64, 8, 1}, true;
  if (dr == 32 && dc == 192) return sh = {64, 8, 1}, true;
  if (dr == 32 && dc == 448) return sh = {32, 4, 1}, true;
  return false;
}

bool latent_attention_supported(DType dt, int dc, int dr) {
  LatentShape sh;
  return latent_shape(dt, dc, dr, sh);
}

size_t latent_value_tiles_bytes(DType dt, int dc, int dr, int B, int max_keys) {
  LatentShape sh;
  if (!latent_shape(dt, dc, dr, sh)) return 0;
  const size_t es = dt == DType::F32 ? 4 : 2;
  const size_t dcp = (size_t)(dc + 31) / 32 * 32;
  const size_t tiles = (size_t)(max_keys + sh.ktile - 1) / sh.ktile;
  return (size_t)B * tiles * dcp * (sh.ktile + 16 / es) * es;
}

hipError_t run_latent_attention(const AttnCall& c, hipStream_t s) {
  if (c.dtype == DType::F32) {
    if (c.dc == 24 && c.dr == 8) return launch_latent<float, 24, 8, 64, 4, 1>(c, s);
    return hipErrorInvalidValue;
  }
  if (c.dc == 24 && c.dr == 8) return launch_latent<bf16, 24, 8, 64, 4, 1>(c, s);
  if (c.dr == 32) {
    if (c.dc == 96) return launch_latent<bf16, 96, 32, 64, 8, 1>(c, s);
    if (c.dc == 192) return launch_latent<bf16, 192, 32, 64, 8, 1>(c, s);
    if (c.dc == 448) return launch_latent<bf16, 448, 32, 32, 4, 1>(c, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace vmla
