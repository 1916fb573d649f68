// Device-side building blocks shared by the GEMM and attention kernels:
// storage types, 32x32 MFMA fragments for gfx950 and small vector helpers.
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

// Column of key j in a transposed value row: bits 2 and 3 of j swapped, so the
// 8 keys one lane feeds to a value MFMA are contiguous (and every aligned group
// of 4 keys stays contiguous).
__device__ inline int perm16(int j) { return (j & ~12) | ((j & 4) << 1) | ((j & 8) >> 1); }

// 3D-RoPE description: per complex pair p its axis (t, h, w by index ranges)
// and angular frequency.  Token (frame f, position s in the frame) has
// coordinates (f, s / grid_w, s % grid_w).
struct Rope {
  int pairs_t, pairs_h;     // pairs [0, t) turn with f, [t, t+h) with row, rest with column
  int grid_w, tokens_per_frame;
  float freq[64];
  __device__ inline void rotate2(int pair, int64_t frame, int s, float& a, float& b) const {
    float pos = pair < pairs_t ? (float)frame
              : (pair < pairs_t + pairs_h ? (float)(s / grid_w) : (float)(s % grid_w));
    float sn, cs;
    sincosf(pos * freq[pair], &sn, &cs);
    float x = a * cs - b * sn;
    float y = a * sn + b * cs;
    a = x;
    b = y;
  }
};

}  // namespace vmla
