// Flash-style absorbed latent attention for gfx950.
//
// Every query row (token, head) of a chunk attends to the same keys: the cache
// rows [c | k_r] of the visible frames followed by the chunk's own rows
// (VideoMLA paper, appendix D.4: chunk-causal, the whole chunk and the whole
// window are visible).  With the per-head key and value lifts absorbed
// (score = q~ . [c | k_r], output = sum p * c, lifted by W_UV afterwards), all
// 12 heads share one [c | k_r] key tile and one c value tile, so each tile is
// staged in LDS once per workgroup and reused by all of its query rows.
//
// Layout of the work (one workgroup = NW waves, 32 query rows per wave):
//   S^T[key][row]  = K_tile[key][:] . Qt[row][:]      (32x32x16 bf16 MFMA, keys as MFMA rows)
//   O^T[f][row]   += C^T[f][key] * P^T[key][row]     (the S^T accumulator is already
//                                                      the B operand of this product)
// so softmax statistics live per lane (one query row per lane pair) and P never
// leaves registers.  The key tile is kept twice in LDS: row-major [key][D] for
// the score product and transposed [f][key] (latent part only) for the value
// product; both are written from one set of global loads.
//
// With bf16 storage the value product runs on fp16 operands: the transposed
// latent tile is converted bf16 -> fp16 while it is staged (exact for
// magnitudes in fp16's normal range, below 65504) and P is rounded to fp16.
// When the softmax is nearly flat every probability sits just below 1, where
// bf16's spacing (2^-8) exceeds the spread of the probabilities themselves;
// fp16's spacing there is 2^-11, at the same MFMA rate.
//
// Scheduling is stream-K over (stream, row block, key tile): workgroup w owns
// iterations [w*I/G, (w+1)*I/G).  A row block finished by one workgroup is
// written directly; a row block split across workgroups leaves unnormalised
// partial states (at most two per workgroup) that the combine kernel merges
// with the usual log-sum-exp rule.  Scores are in log2 units (log2(e) is
// folded into the query), and the running maximum is only moved when a tile
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
  long cbs, sbs;
  int R, n_ring, n_keys, RB, KT, B, G;
};

constexpr float kRescaleSlack = 8.0f;  // log2 units

__device__ inline float xor32(float v) { return __shfl_xor(v, 32); }

template <typename T, int DC, int DR, int KTILE, int NW>
__global__ __launch_bounds__(NW * 64) void latent_attn_kernel(AttnArgs<T> p) {
  using MF = Mfma<T>;
  constexpr int KPL = MF::KPL;
  constexpr int D = DC + DR;
  constexpr int DCP = (DC + 31) / 32 * 32;
  constexpr int VEC = 16 / (int)sizeof(T);
  constexpr int NT = NW * 64;
  constexpr int KS = D + VEC;       // row-major key tile stride (+16 B)
  constexpr int CS = KTILE + 4;     // transposed latent tile stride
  using VT = typename std::conditional<sizeof(T) == 2, f16, float>::type;  // value-product operand
  constexpr int KS_EL = KTILE * KS;
  constexpr int BUF_EL = KS_EL + DCP * CS;
  constexpr int NKS = D / (2 * KPL);
  constexpr int NKB = KTILE / 32;
  constexpr int NFB = DCP / 32;
  constexpr int CV = DC / VEC, RV = DR / VEC;
  constexpr int NCB = (KTILE / 4) * CV;  // blocks of 4 keys x VEC latent channels
  constexpr int NRC = KTILE * RV;        // 16-B chunks of the rotary part
  constexpr int CB_PER = (NCB + NT - 1) / NT;
  constexpr int RC_PER = (NRC + NT - 1) / NT;
  static_assert(D % (2 * KPL) == 0 && DC % VEC == 0 && DR % VEC == 0, "unsupported widths");
  static_assert(KTILE % 32 == 0 && NW * 32 <= kAttnMaxRows, "bad tile");

  __shared__ __attribute__((aligned(16))) T lds[2 * BUF_EL];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, h32 = lane >> 5;
  const float NEG_INF = -__builtin_huge_valf();

  if constexpr (DCP > DC) {  // padded channels of the transposed tile stay finite
    for (int i = tid; i < 2 * (DCP - DC) * CS; i += NT) {
      const int buf = i / ((DCP - DC) * CS), r = i % ((DCP - DC) * CS);
      reinterpret_cast<VT*>(lds + buf * BUF_EL + KS_EL)[DC * CS + r] = VT(0.f);
    }
  }

  u32x4 creg[CB_PER][4];
  u32x4 rreg[RC_PER];

  auto row_ptr = [&](int b, int key) -> const T* {
    if (key < p.n_ring) return p.cache + b * p.cbs + (long)key * D;
    if (key < p.n_keys) return p.stage + b * p.sbs + (long)(key - p.n_ring) * D;
    return nullptr;
  };

  auto load_tile = [&](int b, int kt) {
    const int kbase = kt * KTILE;
#pragma unroll
    for (int i = 0; i < CB_PER; ++i) {
      const int v = tid + i * NT;
      if (NCB % NT == 0 || v < NCB) {
        const int c = v % CV, kg = v / CV;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const T* src = row_ptr(b, kbase + 4 * kg + j);
          creg[i][j] = src ? ld16(src + c * VEC) : u32x4{0, 0, 0, 0};
        }
      }
    }
#pragma unroll
    for (int i = 0; i < RC_PER; ++i) {
      const int v = tid + i * NT;
      if (NRC % NT == 0 || v < NRC) {
        const int c = v % RV, key = v / RV;
        const T* src = row_ptr(b, kbase + key);
        rreg[i] = src ? ld16(src + DC + c * VEC) : u32x4{0, 0, 0, 0};
      }
    }
  };

  auto store_tile = [&](int buf) {
    T* Ks = lds + buf * BUF_EL;
    VT* Ct = reinterpret_cast<VT*>(Ks + KS_EL);
#pragma unroll
    for (int i = 0; i < CB_PER; ++i) {
      const int v = tid + i * NT;
      if (NCB % NT == 0 || v < NCB) {
        const int c = v % CV, kg = v / CV;
#pragma unroll
        for (int j = 0; j < 4; ++j) *reinterpret_cast<u32x4*>(&Ks[(4 * kg + j) * KS + c * VEC]) = creg[i][j];
        // transpose the 4 keys x VEC channels block into C^T rows
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          VT* dst = &Ct[(c * VEC + e) * CS + 4 * kg];
          if constexpr (sizeof(T) == 2) {
            const int dw = e >> 1;
            auto widen = [&](uint32_t word) {
              return (e & 1) ? __uint_as_float(word & 0xFFFF0000u) : __uint_as_float(word << 16);
            };
            f16x4 h;
#pragma unroll
            for (int j = 0; j < 4; ++j) h[j] = (f16)widen(creg[i][j][dw]);
            *reinterpret_cast<f16x4*>(dst) = h;
          } else {
            *reinterpret_cast<u32x4*>(dst) = u32x4{creg[i][0][e], creg[i][1][e], creg[i][2][e], creg[i][3][e]};
          }
        }
      }
    }
#pragma unroll
    for (int i = 0; i < RC_PER; ++i) {
      const int v = tid + i * NT;
      if (NRC % NT == 0 || v < NRC) {
        const int c = v % RV, key = v / RV;
        *reinterpret_cast<u32x4*>(&Ks[key * KS + DC + c * VEC]) = rreg[i];
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
    const int row0 = rb * (NW * 32) + wave * 32;
    const bool wave_active = row0 < p.R;
    const int qrow = row0 + l32;

    typename MF::Frag qf[NKS];
    {
      const T* qsrc = p.qt + ((long)b * p.R + qrow) * D + KPL * h32;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) qf[ks] = qrow < p.R ? MF::load(qsrc + ks * 2 * KPL) : MF::zero();
    }
    f32x16 o[NFB];
#pragma unroll
    for (int fb = 0; fb < NFB; ++fb) o[fb] = f32x16{};
    float m_run = NEG_INF, l_run = 0.f;

    load_tile(b, kt0);
    store_tile(0);
    __syncthreads();

    for (int kt = kt0; kt < kt1; ++kt) {
      const int buf = (kt - kt0) & 1;
      if (kt + 1 < kt1) load_tile(b, kt + 1);
      if (wave_active) {
        const T* Ks = lds + buf * BUF_EL;
        const VT* Ct = reinterpret_cast<const VT*>(Ks + KS_EL);
        const int kbase = kt * KTILE;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          // S^T for 32 keys x 32 query rows
          f32x16 s = f32x16{};
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks) {
            const auto a = MF::load(&Ks[(32 * kb + l32) * KS + ks * 2 * KPL + KPL * h32]);
            s = MF::mma(a, qf[ks], s);
          }
          if (kbase + 32 * kb + 32 > p.n_keys) {
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (kbase + 32 * kb + 8 * (r >> 2) + 4 * h32 + (r & 3) >= p.n_keys) s[r] = NEG_INF;
          }
          // online softmax; every 32-key block holds at least one valid key
          // except blocks wholly past n_keys, whose probabilities are all zero
          float mx = NEG_INF;
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
          mx = fmaxf(mx, xor32(mx));
          const bool need = mx > m_run + kRescaleSlack;
          if (__any(need)) {
            const float mnew = need ? mx : m_run;
            const float alpha = __builtin_amdgcn_exp2f(m_run - mnew);
            m_run = mnew;
            l_run *= alpha;
#pragma unroll
            for (int fb = 0; fb < NFB; ++fb) o[fb] *= alpha;
          }
          float lsum = 0.f;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float e = __builtin_amdgcn_exp2f(s[r] - m_run);
            s[r] = e;
            lsum += e;
          }
          l_run += lsum;
          // O^T += C^T[f][keys] * P^T[keys][rows]
          if constexpr (sizeof(T) == 2) {
            f16x8 pf[2];
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
              for (int j = 0; j < 8; ++j) pf[u][j] = (f16)s[8 * u + j];
#pragma unroll
            for (int fb = 0; fb < NFB; ++fb) {
              const VT* crow = &Ct[(32 * fb + l32) * CS + 32 * kb + 4 * h32];
#pragma unroll
              for (int u = 0; u < 2; ++u) {
                const f16x4 lo = *reinterpret_cast<const f16x4*>(crow + 16 * u);
                const f16x4 hi = *reinterpret_cast<const f16x4*>(crow + 16 * u + 8);
                const f16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                o[fb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, pf[u], o[fb], 0, 0, 0);
              }
            }
          } else {
#pragma unroll
            for (int fb = 0; fb < NFB; ++fb) {
              const VT* crow = &Ct[(32 * fb + l32) * CS + 32 * kb + 4 * h32];
#pragma unroll
              for (int g = 0; g < 4; ++g) {
                const f32x4 run = *reinterpret_cast<const f32x4*>(crow + 8 * g);
#pragma unroll
                for (int i = 0; i < 4; ++i) o[fb] = Mfma<float>::mma(run[i], s[4 * g + i], o[fb]);
              }
            }
          }
        }
      }
      if (kt + 1 < kt1) store_tile(buf ^ 1);
      __syncthreads();
    }

    const float l_tot = l_run + xor32(l_run);
    if (wave_active) {
      if (kt0 == 0 && kt1 == p.KT) {
        if (qrow < p.R) {
          T* dst = p.out + ((long)b * p.R + qrow) * DC;
          const float inv = 1.f / l_tot;
#pragma unroll
          for (int fb = 0; fb < NFB; ++fb)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int f = 32 * fb + 8 * q + 4 * h32;
              if (f < DC)
                store4(dst + f, o[fb][4 * q] * inv, o[fb][4 * q + 1] * inv, o[fb][4 * q + 2] * inv,
                       o[fb][4 * q + 3] * inv);
            }
        }
      } else {
        const long slot_row = (long)(2 * blockIdx.x + (first_piece ? 0 : 1)) * kAttnMaxRows + wave * 32 + l32;
        float* po = p.part_o + slot_row * DC;
#pragma unroll
        for (int fb = 0; fb < NFB; ++fb)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int f = 32 * fb + 8 * q + 4 * h32;
            if (f < DC)
              *reinterpret_cast<f32x4*>(po + f) = f32x4{o[fb][4 * q], o[fb][4 * q + 1], o[fb][4 * q + 2], o[fb][4 * q + 3]};
          }
        if (h32 == 0) {
          p.part_ml[slot_row * 2] = m_run;
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
  const long unit = blockIdx.x;
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
  for (int task = threadIdx.x; task < ROWS * Q; task += 256) {
    const int r = task / Q, f = (task % Q) * 4;
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

template <typename T, int DC, int DR, int KTILE, int NW>
static hipError_t launch_latent(const AttnCall& c, hipStream_t s) {
  constexpr int ROWS = NW * 32;
  AttnArgs<T> a;
  a.qt = static_cast<const T*>(c.qt);
  a.cache = static_cast<const T*>(c.cache);
  a.stage = static_cast<const T*>(c.stage);
  a.out = static_cast<T*>(c.out);
  a.part_o = c.part_o;
  a.part_ml = c.part_ml;
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
  latent_attn_kernel<T, DC, DR, KTILE, NW><<<a.G, NW * 64, 0, s>>>(a);
  if (I != (long)a.G * a.KT)
    latent_attn_combine<T, DC, ROWS><<<a.B * a.RB, 256, 0, s>>>(a);
  return hipGetLastError();
}

bool latent_attention_supported(DType dt, int dc, int dr) {
  if (dt == DType::F32) return dc == 24 && dr == 8;
  return (dc == 24 && dr == 8) || (dr == 32 && (dc == 96 || dc == 192 || dc == 448));
}

hipError_t run_latent_attention(const AttnCall& c, hipStream_t s) {
  if (c.dtype == DType::F32) {
    if (c.dc == 24 && c.dr == 8) return launch_latent<float, 24, 8, 64, 4>(c, s);
    return hipErrorInvalidValue;
  }
  if (c.dc == 24 && c.dr == 8) return launch_latent<bf16, 24, 8, 64, 4>(c, s);
  if (c.dr == 32) {
    if (c.dc == 96) return launch_latent<bf16, 96, 32, 64, 8>(c, s);
    if (c.dc == 192) return launch_latent<bf16, 192, 32, 64, 8>(c, s);
    if (c.dc == 448) return launch_latent<bf16, 448, 32, 32, 4>(c, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace vmla
