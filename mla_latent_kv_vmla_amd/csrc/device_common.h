// Device-side building blocks shared by the GEMM and attention kernels:
// storage types, 32x32 MFMA fragments for gfx950 (bf16, fp16, fp32) and small
// vector helpers.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vmla {

typedef __bf16 bf16;
typedef _Float16 f16;
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// One 32x32 MFMA step of C[32x32] += A[32 x 2*KPL] * B[2*KPL x 32].
// Lane l supplies row (l % 32) of A and column (l % 32) of B, each as KPL
// consecutive k-values starting at k = KPL * (l / 32); accumulator element r of
// lane l is C[8*(r/4) + 4*(l/32) + r%4][l % 32].
template <typename T> struct Mfma;

template <> struct Mfma<bf16> {
  static constexpr int KPL = 8;
  using Frag = bf16x8;
  __device__ static inline f32x16 mma(Frag a, Frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static inline Frag load(const bf16* p) { return *reinterpret_cast<const Frag*>(p); }
  __device__ static inline Frag zero() { return Frag{}; }
};

template <> struct Mfma<f16> {
  static constexpr int KPL = 8;
  using Frag = f16x8;
  __device__ static inline f32x16 mma(Frag a, Frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  __device__ static inline Frag load(const f16* p) { return *reinterpret_cast<const Frag*>(p); }
  __device__ static inline Frag zero() { return Frag{}; }
};

template <> struct Mfma<float> {
  static constexpr int KPL = 1;
  using Frag = float;
  __device__ static inline f32x16 mma(Frag a, Frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
  __device__ static inline Frag load(const float* p) { return *p; }
  __device__ static inline Frag zero() { return 0.f; }
};

// Store four consecutive values as the storage type (bf16: round to nearest even).
__device__ inline void store4(bf16* p, float a, float b, float c, float d) {
  bf16x4 v;
  v[0] = (bf16)a; v[1] = (bf16)b; v[2] = (bf16)c; v[3] = (bf16)d;
  *reinterpret_cast<bf16x4*>(p) = v;
}
__device__ inline void store4(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<f32x4*>(p) = f32x4{a, b, c, d};
}
// fp16, round to nearest even.  Used where the values cannot leave fp16's
// range (convex combinations of fp16 values).
__device__ inline void store4(f16* p, float a, float b, float c, float d) {
  *reinterpret_cast<f16x4*>(p) = f16x4{(f16)a, (f16)b, (f16)c, (f16)d};
}

// Largest finite fp16 magnitude.  The fp16 operand copies (queries, latent key
// tiles, intermediate activations, converted weights) saturate a finite value
// beyond it to +-kF16Max instead of rounding it to infinity, and record that
// they did in bit 0 of a range-flag word the host can read back.  NaN and
// infinite values pass through unchanged.
constexpr float kF16Max = 65504.f;
__device__ inline f16 to_f16_sat(float v, bool& over) {
  const float a = __builtin_fabsf(v);
  if (a > kF16Max && a < __builtin_huge_valf()) {
    over = true;
    v = __builtin_copysignf(kF16Max, v);
  }
  return (f16)v;
}
__device__ inline void raise_range_flag(bool over, uint32_t* flag) {
  if (over && flag) atomicOr(flag, 1u);
}

// Store four values in an epilogue's output type; fp16 outputs saturate and
// flag as above, bf16 and fp32 outputs cover fp32's range.
__device__ inline void store4(f16* p, float a, float b, float c, float d, uint32_t* flag) {
  bool over = false;
  *reinterpret_cast<f16x4*>(p) =
      f16x4{to_f16_sat(a, over), to_f16_sat(b, over), to_f16_sat(c, over), to_f16_sat(d, over)};
  raise_range_flag(over, flag);
}
__device__ inline void store4(bf16* p, float a, float b, float c, float d, uint32_t*) { store4(p, a, b, c, d); }
__device__ inline void store4(float* p, float a, float b, float c, float d, uint32_t*) { store4(p, a, b, c, d); }

// Eight bf16 values (one 16-byte vector) to fp16 by the rule above: round to
// nearest even (exact in fp16's normal range), finite values beyond kF16Max
// saturate and set `over`, NaN and infinities pass through.  The common case,
// every magnitude within range, costs one test per vector.
__device__ inline u32x4 bf16x8_to_f16x8(u32x4 v, bool& over) {
  float f[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(v[i] << 16);
    f[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
  }
  float m = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) m = __builtin_fmaxf(m, __builtin_fabsf(f[j]));
  u32x4 r;
  if (m > kF16Max) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      r[i] = __builtin_bit_cast(uint32_t, f16x2{to_f16_sat(f[2 * i], over), to_f16_sat(f[2 * i + 1], over)});
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = __builtin_bit_cast(uint32_t, f16x2{(f16)f[2 * i], (f16)f[2 * i + 1]});
  }
  return r;
}

// 16-byte global load / zero of one vector of storage elements.
__device__ inline u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// Buffer resource over `bytes` bytes at `base` for raw byte-offset loads; the
// hardware range check returns zero for any load past the end.
__device__ inline __amdgpu_buffer_rsrc_t raw_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

// LDS-DMA load through a buffer resource: each active lane copies the 16 bytes
// at byte offset `voff` of the buffer to LDS; lane L's bytes land at
// lds_wave_base + 16*L (lds_wave_base must be wave-uniform).  Completion is
// tracked by the vector-memory counter only (the MUBUF form, unlike the FLAT
// one, leaves the LDS counter to ordinary LDS reads, so those can be waited
// for one at a time).
__device__ inline void lds_dma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, void* lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_wave_base, 16, voff, 0,
                                           0, 0);
}

// LDS-DMA load issued from inline asm: each active lane copies the 16 bytes at
// byte offset `voff` of the buffer to LDS byte address lds_byte_addr + 16 *
// lane (lds_byte_addr wave-uniform, in an SGPR).  The compiler does not know
// this instruction writes LDS, so it adds no wait for it before LDS reads: the
// caller waits (wait_vmcnt) before the barrier that publishes the data, and
// before the workgroup ends.
__device__ inline void dma16_lds(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t lds_byte_addr) {
  // one wait state between the M0 write and the LDS-DMA that reads it
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds_byte_addr), "v"(voff), "s"(r)
               : "memory");
}
template <int N> __device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  if constexpr (N == 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Column of key j in a transposed value row: bits 2 and 3 of j swapped, so the
// 8 keys one lane feeds to a value MFMA are contiguous (and every aligned group
// of 4 keys stays contiguous).
__device__ inline int perm16(int j) { return (j & ~12) | ((j & 4) << 1) | ((j & 8) >> 1); }

// Exact x / d and x % d for 0 <= x < 2^31 and a divisor d >= 1 fixed per
// launch: one high multiply, one add and one shift (the magic-number method
// for dividends one bit narrower than the word: mul = floor(2^32 (2^s - d) / d)
// + 1 with 2^s >= d), where a division by a run-time value expands to a long
// instruction sequence.
struct FastDiv {
  uint32_t d = 1, mul = 1, shift = 0;
  FastDiv() = default;
  explicit FastDiv(uint32_t divisor) : d(divisor) {
    while (shift < 31 && (1u << shift) < d) ++shift;
    mul = (uint32_t)(((uint64_t)1 << 32) * (((uint64_t)1 << shift) - d) / d + 1);
  }
  __device__ inline uint32_t div(uint32_t x) const { return (__umulhi(x, mul) + x) >> shift; }
  __device__ inline uint32_t mod(uint32_t x) const { return x - div(x) * d; }
};

// 3D-RoPE description: per complex pair p its axis (t, h, w by index ranges)
// and angular frequency.  Token (frame f, position s in the frame) has
// coordinates (f, s / grid_w, s % grid_w).  The row and column angles take only
// grid_h and grid_w values: `tab` (when set) holds their cosine and sine,
// tab[2 (p * tab_stride + pos) + {0, 1}] for pair p of the h or w axis,
// computed once per ctx by rope_table with the same sincosf of the same
// argument, so a lookup returns the values the direct evaluation would.
// sin and cos of a rotary angle: one out-of-line copy, so that epilogues with
// many rotation sites do not each inline the argument reduction of sincosf
__device__ __attribute__((noinline)) inline void rope_sincos(float ang, float& sn, float& cs) { sincosf(ang, &sn, &cs); }

struct Rope {
  int pairs_t, pairs_h;     // pairs [0, t) turn with f, [t, t+h) with row, rest with column
  int grid_w, tokens_per_frame;
  float freq[64];
  const float* tab = nullptr;
  int tab_stride = 0;
  FastDiv gw, tpf;          // divisions by grid_w and by tokens_per_frame
  // host: every field (n frequencies, the rest of freq zero)
  void set(int pt, int ph, int grid_w_, int tokens, const float* f, int n, const float* table, int stride) {
    pairs_t = pt;
    pairs_h = ph;
    grid_w = grid_w_;
    tokens_per_frame = tokens;
    for (int i = 0; i < 64; ++i) freq[i] = i < n ? f[i] : 0.f;
    tab = table;
    tab_stride = stride;
    gw = FastDiv((uint32_t)grid_w_);
    tpf = FastDiv((uint32_t)tokens);
  }
  // cos and sin of the angle of pair `pair` for token s of frame `frame`;
  // OUTLINE: sincosf through the one out-of-line copy (for code with many
  // rotation sites, such as unrolled GEMM epilogues)
  template <bool OUTLINE = false>
  __device__ inline void angle(int pair, int64_t frame, int s, float& cs, float& sn) const {
    if (pair >= pairs_t && tab) {
      const int pos = pair < pairs_t + pairs_h ? (int)gw.div(s) : (int)gw.mod(s);
      const float2 v = reinterpret_cast<const float2*>(tab)[pair * tab_stride + pos];
      cs = v.x;
      sn = v.y;
    } else {
      float pos = pair < pairs_t ? (float)frame
                : (pair < pairs_t + pairs_h ? (float)gw.div(s) : (float)gw.mod(s));
      if constexpr (OUTLINE) rope_sincos(pos * freq[pair], sn, cs);
      else sincosf(pos * freq[pair], &sn, &cs);
    }
  }
  // (a, b) turned by the angle with cosine cs and sine sn
  __device__ static inline void turn(float cs, float sn, float& a, float& b) {
    float x = a * cs - b * sn;
    float y = a * sn + b * cs;
    a = x;
    b = y;
  }
  template <bool OUTLINE = false>
  __device__ inline void rotate2(int pair, int64_t frame, int s, float& a, float& b) const {
    float sn, cs;
    angle<OUTLINE>(pair, frame, s, cs, sn);
    turn(cs, sn, a, b);
  }
};

// Local temporal coordinate of the frame held in ring slot `slot` after n
// appends, with S pinned sink slots ahead of a W-frame FIFO: the frame's index
// in the visible context [sink frames, window frames oldest first], numbered
// from 0 without gaps (sink slot i holds frame i; window slot S + j holds the
// window frame f with (f - S) % W == j).
__device__ inline int64_t local_frame(int slot, int64_t n, int S, int W) {
  if (slot < S) return slot;
  const int64_t n_sink = n < S ? n : S;
  const int64_t w0 = n - W > S ? n - W : S;  // first window frame
  const int64_t f = w0 + ((((int64_t)(slot - S) - (w0 - S)) % W) + W) % W;
  return n_sink + (f - w0);
}

}  // namespace vmla
