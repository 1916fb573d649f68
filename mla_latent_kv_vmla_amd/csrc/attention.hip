// Flash-style attention for gfx950 over a chunk's visible keys, used by both
// layer types the library runs:
//   latent (absorbed) attention: every query row (token, head) scores the
//     head-shared cache rows [c | k_r] and sums c (VideoMLA paper, section 3.3;
//     the per-head key and value lifts are absorbed into the query and applied
//     to the output), so all heads share one key tile and one value tile;
//   dense per-head attention: the baseline of the paper's section 1 and
//     appendix C.1, per-head key rows and per-head values.
// Every chunk query sees every key of the window and of its own chunk
// (appendix D.4: chunk-causal, no mask inside the chunk or the window).  The
// keys come in two segments: segment 0 holds the ring rows of the cached frames
// in slot order (softmax does not depend on key order), segment 1 the chunk's
// own rows.  Each segment is tiled on its own; keys past a segment's end are
// masked.
//
// Work layout (one workgroup = NW waves, 32*NB query rows per wave):
//   S^T[key][row]  = K_tile[key][:] . Q[row][:]       (32x32x16 MFMA, keys as MFMA rows)
//   O^T[f][row]   += V^T[f][key] * P^T[key][row]      (the S^T accumulator is already
//                                                      the B operand of this product)
// so softmax statistics live per lane (one query row per lane pair) and P never
// leaves registers.  Two kernels share this layout: flash_attn_kernel (8 waves
// x 32 rows, two waves per SIMD hiding each other's softmax, or 4 waves at the
// widest score width; the dense layer, d_c = 448, fp32 storage and the tiny
// layer) and flash_attn_pipe_kernel (4 waves x 64 rows, one wave per SIMD that
// pipelines its own softmax under its MFMAs; latent d_c = 96 and 192 with bf16
// storage).
//
// Staging.  Tiles are copied into LDS with LDS-DMA loads through a buffer
// resource (buffer_load_dwordx4 ... lds: lane L's 16 bytes land at M0 + 16 L),
// so staging needs no registers and no VALU, and the resource's range check
// reads rows past a segment's end as zero.
//   Latent attention, bf16 storage: one row-major key tile [KTILE][D] in fp16
//     per stage, copied from the tiles a pre-pass converts once per call into
//     the workspace.  The value is the key's first DV channels, so the value
//     product reads its V^T fragments from that same tile with gfx950's
//     transposing LDS read (ds_read_b64_tr_b16): one key tile serves both
//     products.
//   Dense attention: the row-major key tile (bf16) plus a transposed value tile
//     [f][key] copied straight from value rows that the dense cache stores
//     transposed.
//   Latent attention, fp32 storage: the row-major key tile plus a transposed
//     value tile from images a pre-pass builds once per call.
// LDS layouts (per stage; two stages in two distinct arrays):
//   Ks  [KTILE][D + 16 B]
//   V^T [DVP][KTILE + 16 B]: within every 16-key group the key index has bits 2
//       and 3 swapped, so the 8 keys a lane feeds to one value MFMA are one
//       contiguous 16-B read.
// A 128-bit LDS read is served 16 lanes at a time from 64 four-byte banks; with
// the 16-B row pad the 16 rows one such group reads start in 16 distinct
// 16-B bank groups, so both layouts read without bank conflicts.  A transposing
// read gathers 8 bytes from each of 4 rows per 16-lane group; the pad puts
// those rows in distinct banks too.
//
// Numerics.  With bf16 storage the value product runs on fp16 operands (values
// held as fp16, P rounded to fp16).  When the softmax is nearly flat every
// probability sits just below 1, where bf16's spacing (2^-8) exceeds the
// spread of the probabilities themselves; fp16's spacing there is 2^-11, at
// the same MFMA rate.  The dense cache stores V as fp16.  Latent attention
// also takes its scores from fp16 operands, since the key tile is the value
// tile: the bf16 -> fp16 conversion of keys and absorbed queries is exact in
// fp16's normal range, so the scores are those of the bf16 inputs as long as
// every key and query element stays below 65504 in magnitude.
//
// Scheduling.  G persistent workgroups.  With at least two (stream, row block)
// units per workgroup, whole units go round-robin first; the remaining units
// are split stream-K over their key tiles: workgroup w owns pieces
// [w*I/G, (w+1)*I/G).  A row block finished by one workgroup is written
// directly; a row block split across workgroups leaves unnormalised partial
// states (at most two per workgroup) that the combine kernel merges with the
// usual log-sum-exp rule.  Block-causal mode (a whole clip) runs one workgroup
// per row block and skips the key tiles above its diagonal.  Scores are in log2
// units (log2(e) is folded into the query), and the running maximum is only
// moved when a block exceeds it by more than 8 (a factor 2^8), which keeps
// rescaling of the accumulator rare.
#include <hip/hip_ext.h>

#include <type_traits>

#include "device_common.h"
#include "plan.h"

namespace vmla {

// One attention launch.  Stream s (0..S-1) is an independent attention problem:
// a batch stream for latent attention (rows = token*heads + head), a (batch
// stream, head) pair for dense attention (rows = tokens).
template <typename T> struct FlashArgs {
  const void* q;            // row r of stream s: q + s*q_ss + r*D (query type: fp16 for 16-bit storage)
  long q_ss;
  const T* key0;            // ring segment: key k of stream s at key0 + s*key_ss0 + k*D
  const T* key1;            // chunk segment
  long key_ss0, key_ss1;
  const void* val0;         // value rows [f][key] (fp16 for bf16 storage) of the ring segment,
  const void* val1;         //   of the chunk segment; or the per-call pre-pass tiles (val0)
  long val_ss0, val_ss1;    // elements per stream
  int val_rs0, val_rs1;     // elements per value row
  void* out;                // row r of stream s: out + (s/heads)*out_so + (s%heads)*out_sh + r*out_rs
  long out_so, out_sh, out_rs;  //   (output type = value-operand type: fp16 for 16-bit storage)
  uint32_t* range_flag;     // latent key-tile pre-pass: raised when a cached element saturates
  // Rotation at use (latent key-tile pre-pass): with rot_ring, the ring segment
  // holds k^ un-rotated in channels [rot_dc, D); ring row r (slot r / T, token
  // r % T) is turned at the local coordinate of its slot's frame (rot_n frames
  // appended, rot_S sink slots, rot_W window slots) before the fp16 conversion.
  int rot_ring, rot_dc, rot_S, rot_W;
  int64_t rot_n;
  Rope rope;
  int heads;
  float* part_o;            // [2G][kAttnMaxRows][DV] of PartT<T> (normalised partial outputs)
  float* part_ml;           // [2G][kAttnMaxRows][2]
  int len0, len1, tiles0;   // keys per segment, key tiles of segment 0
  int R, RB, KT, S, G;      // rows per stream, row blocks per stream, key tiles, streams, workgroups
  // Units (stream, row block) 0..dp_units-1 go whole to workgroups round-robin
  // (unit j*G + w to workgroup w); the rest are split into key-tile pieces
  // (stream-K).  dp_units is a multiple of G.
  long dp_units;
  // Block-causal mode (causal_tokens > 0; keys in segment 1 only): row r sees
  // keys [0, (t / causal_tokens + 1) * causal_tokens) with t = r / row_div its
  // token.  One workgroup per row block, longest rows first, no split.
  int causal_tokens, row_div;
};

constexpr float kRescaleSlack = 8.0f;  // log2 units
constexpr int kAhead = 4;  // LDS fragment reads in flight ahead of their MFMA

// Maximum of two scores in the IEEE 754-2019 sense (a NaN operand gives NaN).
// fmaxf must first quiet a signalling NaN, so for operands the compiler cannot
// prove canonical (copies out of the accumulators) it adds a v_max_f32 x, x
// per operand; this form needs none, and chains of it issue as
// v_maximum3_f32, two new operands per instruction.  A NaN score reaches the
// output through its exponential either way.
__device__ inline float smax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// Split-KV partial outputs are stored normalised, O / l: a convex combination
// of value rows.  With 16-bit storage the values are fp16 copies already and
// the result is rounded to bf16, so the partials are fp16 (half the traffic
// of the stores and of the combine's reads); fp32 storage keeps fp32.
template <typename T> using PartT = typename std::conditional<sizeof(T) == 2, f16, float>::type;
template <typename T> __device__ inline void store_part4(PartT<T>* dst, float a, float b, float c, float d) {
  if constexpr (sizeof(T) == 2) *reinterpret_cast<f16x4*>(dst) = f16x4{(f16)a, (f16)b, (f16)c, (f16)d};
  else *reinterpret_cast<f32x4*>(dst) = f32x4{a, b, c, d};
}
template <typename T> __device__ inline f32x4 load_part4(const PartT<T>* src) {
  if constexpr (sizeof(T) == 2) {
    const f16x4 h = *reinterpret_cast<const f16x4*>(src);
    return f32x4{(float)h[0], (float)h[1], (float)h[2], (float)h[3]};
  } else {
    return *reinterpret_cast<const f32x4*>(src);
  }
}

// Max and sum over the lane pair (l, l ^ 32) that shares one query row: one
// v_permlane32_swap exchanges the two half-waves, and combining both of its
// results gives the pair's value in either lane.
__device__ inline float pair_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return smax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float pair_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// 32x32x16 f16 MFMAs with VGPR accumulators, issued from asm (the compiler keeps
// every MFMA of a kernel that needs AGPRs in the AGPR form).  The compiler does
// not see these as MFMAs: a VALU read of their result must come at least one
// MFMA issue plus a few wait states later (callers place one).
__device__ inline f32x16 mfma_vgpr(f16x8 a, f16x8 b, const f32x16& c) {
  f32x16 d;
  asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %3" : "=&v"(d) : "v"(a), "v"(b), "v"(c));
  return d;
}
__device__ inline void mfma_vgpr_acc(f32x16& acc, f16x8 a, f16x8 b) {
  asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}

// acc *= alpha for an accumulator held in AGPRs.  Each element passes through
// one VGPR temporary inside the asm.  Written as plain C++ the product needs the
// tuple in VGPRs, and the compiler then keeps a VGPR copy of every accumulator
// live across the whole key loop (the copies are hoisted out of the rare
// rescale branch), which at one wave per SIMD pushes the query fragments out
// to scratch.
__device__ inline void scale_acc_agpr(f32x16& acc, float alpha) {
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    float x = acc[r], t;
    asm volatile("v_accvgpr_read_b32 %0, %1\n\tv_mul_f32_e32 %0, %2, %0\n\tv_accvgpr_write_b32 %1, %0"
                 : "=&v"(t), "+a"(x)
                 : "v"(alpha));
    acc[r] = x;
  }
}

// Compile-time geometry of one instantiation: score width D, value width DV.
template <typename T, int D_, int DV, int KTILE> struct TileGeo {
  using VT = typename std::conditional<sizeof(T) == 2, f16, float>::type;  // value-product operand
  static_assert(sizeof(VT) == sizeof(T), "tile sizing assumes equal widths");
  static constexpr int D = D_;
  static constexpr int DVP = (DV + 31) / 32 * 32;
  static constexpr int VEC = 16 / (int)sizeof(T);  // elements per 16-B chunk
  static constexpr int KS = D + VEC;               // row-major tile row (+16 B)
  static constexpr int CS = KTILE + VEC;           // transposed tile row (+16 B)
  static constexpr int KCH = KS / VEC;             // 16-B chunks per row-major row
  static constexpr int CCH = CS / VEC;             // 16-B chunks per transposed row
  static constexpr int KPOS = KTILE * KCH;         // chunks of the row-major tile
  static constexpr int CPOS = DVP * CCH;           // chunks of the transposed tile
  static constexpr int KS_EL = KTILE * KS;
  static constexpr int BUF_EL = KS_EL + DVP * CS;
  static constexpr int KI = (KPOS + 63) / 64;      // wave-wide 1-KB loads per stage
  static constexpr int CI = (CPOS + 63) / 64;
  static constexpr size_t IMG_BYTES = (size_t)CPOS * 16;
  static_assert(D % VEC == 0 && DV % VEC == 0 && DV <= D, "unsupported widths");
  static_assert(KTILE % 32 == 0 && KTILE / VEC < 256, "bad tile");
  __device__ static int perm_group(int kg) { return (kg & ~3) | ((kg & 1) << 1) | ((kg >> 1) & 1); }
};

// Segment of key tile t: (segment, first key, keys in the segment).
template <typename T, int KTILE>
__device__ inline void tile_segment(const FlashArgs<T>& p, int t, int& g, int& kbase, int& len) {
  g = t >= p.tiles0 ? 1 : 0;
  kbase = (t - (g ? p.tiles0 : 0)) * KTILE;
  len = g ? p.len1 : p.len0;
}

// Pre-pass (latent attention, fp32 storage): transposed value-tile images.  Image (s, t)
// holds, for the keys of tile t, rows = the first DV key channels (zero rows
// pad DV up to a multiple of 32) in the value-operand type, keys permuted
// within 16-key groups.  Keys past the segment's end repeat its last key
// (their probabilities are zero).
template <typename T, int D, int DV, int KTILE>
__global__ __launch_bounds__(256) void latent_value_tiles(FlashArgs<T> p) {
  using G = TileGeo<T, D, DV, KTILE>;
  using VT = typename G::VT;
  constexpr int KG = KTILE / 4, CV = DV / G::VEC;
  const int t = blockIdx.x, s = blockIdx.y;
  int g, kbase, len;
  tile_segment<T, KTILE>(p, t, g, kbase, len);
  const T* keys = g ? p.key1 + s * p.key_ss1 : p.key0 + s * p.key_ss0;
  VT* img = reinterpret_cast<VT*>(const_cast<void*>(p.val0)) + ((size_t)s * p.KT + t) * (G::IMG_BYTES / sizeof(VT));
  for (int v = threadIdx.x; v < KG * CV; v += 256) {
    const int kg = v % KG, c = v / KG;
    u32x4 k[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int key = min(kbase + 4 * kg + j, len - 1);
      k[j] = ld16(keys + (long)key * D + c * G::VEC);
    }
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
  for (int i = threadIdx.x; i < (G::DVP - DV) * G::CS; i += 256) img[DV * G::CS + i] = VT(0.f);
}

// Pre-pass (latent attention, bf16 storage): fp16 copies of the key tiles.
// Tile (s, t) is row-major [KTILE][D] without padding, or (IMAGE) the byte
// image of the pipelined kernel's LDS tile (16-row regions of 1-KB blocks,
// see flash_attn_pipe_kernel), so that each of that kernel's wave-wide DMA
// loads copies 1 KB of contiguous bytes; keys past the segment's
// end repeat its last key (their probabilities are zero).  bf16 values in
// fp16's normal range convert exactly; a finite value beyond +-65504 saturates
// and raises the range flag.  With rotation at use, the ring rows' k^ channels
// are turned in fp32 at their local coordinate first (one rounding, to fp16).
template <typename T, int D, int KTILE, bool IMAGE>
__global__ __launch_bounds__(256) void latent_key_tiles(FlashArgs<T> p) {
  static_assert(std::is_same<T, bf16>::value, "the key tiles widen bf16");
  constexpr int CV = D / 8;
  const int t = blockIdx.x, s = blockIdx.y;
  int g, kbase, len;
  tile_segment<T, KTILE>(p, t, g, kbase, len);
  const T* keys = g ? p.key1 + s * p.key_ss1 : p.key0 + s * p.key_ss0;
  f16* img = reinterpret_cast<f16*>(const_cast<void*>(p.val0)) + ((size_t)s * p.KT + t) * (KTILE * D);
  bool over = false;
  for (int v = threadIdx.x; v < KTILE * CV; v += 256) {
    const int r = v / CV, c = v % CV;
    const int key = min(kbase + r, len - 1);
    const u32x4 k = ld16(keys + (long)key * D + c * 8);
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t w = k[e >> 1];
      x[e] = (e & 1) ? __uint_as_float(w & 0xFFFF0000u) : __uint_as_float(w << 16);
    }
    if (p.rot_ring && g == 0 && c * 8 >= p.rot_dc) {
      const int tpf = p.rope.tokens_per_frame;
      const int64_t tau = local_frame(key / tpf, p.rot_n, p.rot_S, p.rot_W);
      const int pair0 = (c * 8 - p.rot_dc) >> 1;
#pragma unroll
      for (int j = 0; j < 4; ++j) p.rope.rotate2(pair0 + j, tau, key % tpf, x[2 * j], x[2 * j + 1]);
    }
    f16x8 h;
#pragma unroll
    for (int e = 0; e < 8; ++e) h[e] = to_f16_sat(x[e], over);
    int off = r * D + c * 8;
    if constexpr (IMAGE) {  // region r / 16, block c / 4, slot 16 (c % 4) + ((r % 16) ^ 4 (c % 4))
      const int cc = c & 3;
      off = (r >> 4) * 16 * D + (c >> 2) * 512 + 8 * (16 * cc + ((r & 15) ^ (4 * cc)));
    }
    *reinterpret_cast<f16x8*>(img + off) = h;
  }
  raise_range_flag(over, p.range_flag);
}

// VROWS = false (latent): bf16 storage stages the pre-pass key tiles (val0) and
// reads V^T from them transposed; fp32 storage stages the keys and the
// pre-pass value images (val0).  VROWS = true (dense): the keys and value rows
// val0/val1 ([f][key], keys permuted within 16-key groups, zero past the
// segment's end up to the tile boundary).
template <typename T, int D, int DV, int KTILE, int NW, int NB, bool VROWS>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4)))
void flash_attn_kernel(FlashArgs<T> p) {
  using G = TileGeo<T, D, DV, KTILE>;
  using VT = typename G::VT;
  using MF = Mfma<T>;
  constexpr bool HALF = sizeof(T) == 2;
  constexpr int KPL = MF::KPL;
  constexpr int DVP = G::DVP, VEC = G::VEC, KS = G::KS, CS = G::CS;
  constexpr int RW = 32 * NB;               // query rows per wave
  constexpr int NKS = D / (2 * KPL);
  constexpr int NKB = KTILE / 32;
  constexpr int NFB = DVP / 32;
  constexpr bool VT_FROM_K = !VROWS && HALF;  // one fp16 key tile; V^T read transposed from it
  constexpr int NI = VT_FROM_K ? G::KI : G::KI + G::CI;  // 1-KB loads per stage, spread over the waves
  constexpr int NI_W = (NI + NW - 1) / NW;
  static_assert(NW * RW <= kAttnMaxRows, "row block too large");
  // Score widths up to 128 (d_c 24 and 96, the dense layer) are VALU-bound: a
  // block's softmax outweighs its MFMAs.  There the running max is folded into
  // the score MFMAs and the row sums use v_dot2; wider kernels have no register
  // room for the folded accumulators and keep the plain form.
  constexpr bool FOLD = HALF && D <= 128;
  // Score widths above 256 (d_c 448) run one wave per SIMD with the value
  // accumulators in AGPRs; their rescale must not move them to VGPRs.
  constexpr bool ACC_AGPR = HALF && D > 256;
  static_assert(!VROWS || DV % 32 == 0, "value rows need whole 32-channel blocks");
  static_assert(!VT_FROM_K || DVP <= D, "V^T fragments are read from the key tile's channels");

  __shared__ __attribute__((aligned(16))) T lds0[VT_FROM_K ? G::KS_EL : G::BUF_EL];
  __shared__ __attribute__((aligned(16))) T lds1[VT_FROM_K ? G::KS_EL : G::BUF_EL];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, h32 = lane >> 5;
  const float NEG_INF = -__builtin_huge_valf();

  // This lane's source in each of this wave's LDS-DMA loads of a stage, as an
  // element offset from the tile's base: row-major key tile (row r, chunk)
  // packed as r << 12 | offset in the row; value rows (channel f, chunk) packed
  // as f << 8 | offset in the row; images: byte offset.  The pad chunk of a row
  // loads any valid chunk.
  uint32_t slot[NI_W];
#pragma unroll
  for (int k = 0; k < NI_W; ++k) {
    const int idx = wave + k * NW;
    if (idx < G::KI) {
      const int pos = idx * 64 + lane;
      const int r = pos / G::KCH, c = pos % G::KCH;
      slot[k] = ((uint32_t)r << 12) | (uint32_t)((c < G::KCH - 1 ? c : 0) * VEC);
    } else {
      const int pos = (idx - G::KI) * 64 + lane;
      if constexpr (VROWS) {
        const int f = pos / G::CCH, c = pos % G::CCH;
        slot[k] = ((uint32_t)f << 8) | (uint32_t)((c < G::CCH - 1 ? c : 0) * VEC);
      } else {
        slot[k] = (uint32_t)pos * 16u;
      }
    }
  }

  // Issue the LDS-DMA loads of tile t of stream s (both layouts) into stage `buf`.
  // Key rows past the segment's end read as zero (buffer range check) and are
  // masked out of the scores.
  auto issue_tile = [&](int s, int t, T* buf) {
    int g, kbase, len;
    tile_segment<T, KTILE>(p, t, g, kbase, len);
    const auto krs = VT_FROM_K ? raw_rsrc(static_cast<const char*>(p.val0) + ((size_t)s * p.KT + t) * (KTILE * D * 2),
                                    (uint32_t)(KTILE * D * 2))
                         : raw_rsrc(g ? p.key1 + s * p.key_ss1 : p.key0 + s * p.key_ss0,
                                    (uint32_t)len * (uint32_t)(D * sizeof(T)));
    __amdgpu_buffer_rsrc_t vrs;
    uint32_t vrow = 0, vbase = 0;
    if constexpr (VROWS) {
      const long ss = g ? p.val_ss1 : p.val_ss0;
      vrs = raw_rsrc(static_cast<const VT*>(g ? p.val1 : p.val0) + ss * s, (uint32_t)(ss * sizeof(VT)));
      vrow = (uint32_t)(g ? p.val_rs1 : p.val_rs0);
      vbase = (uint32_t)kbase;
    } else {
      vrs = raw_rsrc(static_cast<const char*>(p.val0) + ((size_t)s * p.KT + t) * G::IMG_BYTES,
                     (uint32_t)G::IMG_BYTES);
    }
#pragma unroll
    for (int k = 0; k < NI_W; ++k) {
      const int idx = wave + k * NW;  // wave-uniform
      if (idx < G::KI) {
        const int pos = idx * 64 + lane;
        if (G::KPOS % 64 == 0 || pos < G::KPOS) {
          const uint32_t row = (VT_FROM_K ? 0u : (uint32_t)kbase) + (slot[k] >> 12);
          lds_dma16(krs, (row * D + (slot[k] & 0xFFFu)) * (uint32_t)sizeof(T), buf + idx * 64 * VEC);
        }
      } else if (idx < NI) {
        const int ci = idx - G::KI, pos = ci * 64 + lane;
        if (G::CPOS % 64 == 0 || pos < G::CPOS) {
          uint32_t off;
          if constexpr (VROWS) off = ((slot[k] >> 8) * vrow + vbase + (slot[k] & 0xFFu)) * (uint32_t)sizeof(VT);
          else off = slot[k];
          lds_dma16(vrs, off, buf + G::KS_EL + ci * 64 * VEC);
        }
      }
    }
  };

  const bool causal = p.causal_tokens > 0;
  // token limit (exclusive) of the keys row r may see in block-causal mode
  auto row_limit = [&](int r) {
    const int lim = (r / p.row_div / p.causal_tokens + 1) * p.causal_tokens;
    return lim < p.len1 ? lim : p.len1;
  };
  // Workgroups are dispatched round-robin over the 8 XCDs (each with its own
  // L2); the virtual index gives the workgroups of one XCD consecutive numbers,
  // so that they work on neighbouring row blocks of the same streams and share
  // those streams' keys in L2.
  const int vw = p.G % 8 == 0 ? (int)(blockIdx.x % 8) * (p.G / 8) + (int)(blockIdx.x / 8) : (int)blockIdx.x;
  // Whole units first: unit j*G + vw in round j, so in every round the
  // workgroups of one XCD hold consecutive row blocks, mostly of one stream.
  const int n_whole = causal ? 0 : (int)(p.dp_units / p.G);
  // Then this workgroup's share [it0, it1) of the key-tile pieces of the
  // remaining units: pieces of consecutive row blocks, where the first may start
  // and the last may end inside a row block.  The last piece (which starts at
  // key tile 0) is processed first, so every workgroup sweeps the key tiles in
  // increasing order from near tile 0 and the workgroups sharing an L2 stay
  // within a few dozen tiles of one another.  Block-causal mode: one whole row
  // block per workgroup, the longest (last) row blocks first.
  const long I = ((long)p.S * p.RB - (causal ? 0 : p.dp_units)) * p.KT;
  const long it0 = (long)vw * I / p.G, it1 = (long)(vw + 1) * I / p.G;
  const long u_first = causal ? (long)p.S * p.RB - 1 - blockIdx.x : p.dp_units + it0 / p.KT;
  const int npieces = causal ? 1 : (int)((it1 - 1) / p.KT - it0 / p.KT + 1);
  for (int job = 0; job < n_whole + npieces; ++job) {
    const bool whole = job < n_whole;
    const int k = job - n_whole;
    const int piece = whole ? 0 : npieces > 1 ? (k == 0 ? npieces - 1 : k - 1) : 0;
    const long unit = whole ? (long)job * p.G + vw : u_first + piece;
    const int s = (int)(unit / p.RB), rb = (int)(unit % p.RB);
    int kt0, kt1;
    if (causal) {  // tiles up to the last row's limit; the tiles above the block diagonal are skipped
      const int last_row = min((rb + 1) * (NW * RW), p.R) - 1;
      kt0 = 0;
      kt1 = p.tiles0 + (row_limit(last_row) + KTILE - 1) / KTILE;
    } else if (whole) {
      kt0 = 0;
      kt1 = p.KT;
    } else {
      kt0 = piece == 0 ? (int)(it0 % p.KT) : 0;
      kt1 = piece == npieces - 1 ? (int)((it1 - 1) % p.KT) + 1 : p.KT;
    }
    const bool first_piece = piece == 0;
    const int row0 = rb * (NW * RW) + wave * RW;
    // keys from which this workgroup's rows (uniform) / this lane's rows need masking
    const int mask_from_wg = causal ? row_limit(rb * (NW * RW)) : 0x7fffffff;
    int mask_from[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) mask_from[nb] = causal ? row_limit(row0 + 32 * nb + l32) : 0x7fffffff;

    // queries arrive in the score operand type (fp16 for 16-bit storage)
    using QFrag = typename std::conditional<VT_FROM_K, f16x8, typename MF::Frag>::type;
    QFrag qf[NB][NKS];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int qrow = row0 + 32 * nb + l32;
      const VT* qsrc = static_cast<const VT*>(p.q) + s * p.q_ss + (long)qrow * D + KPL * h32;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
        qf[nb][ks] = qrow < p.R ? *reinterpret_cast<const QFrag*>(qsrc + ks * 2 * KPL) : QFrag{};
    }
    f32x16 o[NB][NFB];
    float m_run[NB], l_run[NB];
    // FOLD: each lane's 16 scores of a block belong to one query row, so the
    // row's running maximum can enter the score MFMAs as their starting
    // accumulator (the splat -m_fold): they produce s - m_fold directly.
    // m_fold follows m_run at every rescale; it is 0 only before the first
    // block, whose rescale is always taken.
    f32x16 negm[NB];
    float m_fold[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      m_run[nb] = NEG_INF;
      l_run[nb] = 0.f;
      negm[nb] = f32x16{};
      m_fold[nb] = 0.f;
#pragma unroll
      for (int fb = 0; fb < NFB; ++fb) o[nb][fb] = f32x16{};
    }

    // all query-row blocks of one tile held in `cur`
    auto compute = [&](int t, const T* cur) {
      int g, kbase, len;
      tile_segment<T, KTILE>(p, t, g, kbase, len);
      const T* Ks = cur;
      const VT* Ct = reinterpret_cast<const VT*>(cur + G::KS_EL) + l32 * CS;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        // S^T for 32 keys x RW query rows; each K fragment feeds NB MFMAs
        f32x16 sc[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) sc[nb] = FOLD ? negm[nb] : f32x16{};
        const int r = 32 * kb + l32;
        if constexpr (HALF) {  // chunk 2ks+h of row r: one per-lane base, immediate offsets
          const T* kb0 = Ks + r * KS + h32 * VEC;
          // fragments are read kAhead steps before their MFMA; the scheduling
          // barriers keep the compiler from sinking each read onto its use
          auto kfrag = [&](int ks) {
            if constexpr (VT_FROM_K) return *reinterpret_cast<const f16x8*>(kb0 + 2 * VEC * ks);
            else return MF::load(kb0 + 2 * VEC * ks);
          };
          QFrag kq[kAhead];
#pragma unroll
          for (int i = 0; i < kAhead && i < NKS; ++i) kq[i] = kfrag(i);
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks) {
            __builtin_amdgcn_sched_barrier(0);
            const auto a = kq[ks % kAhead];
            if (ks + kAhead < NKS) kq[ks % kAhead] = kfrag(ks + kAhead);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
              if constexpr (VT_FROM_K) sc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, qf[nb][ks], sc[nb], 0, 0, 0);
              else sc[nb] = MF::mma(a, qf[nb][ks], sc[nb]);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        } else {
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks) {
            const int e = ks * 2 * KPL + KPL * h32;
            const auto a = MF::load(&Ks[r * KS + e]);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) sc[nb] = MF::mma(a, qf[nb][ks], sc[nb]);
          }
        }
        // the tail mask and the rescale below are rare: the empty volatile asm
        // keeps each a real (uniform) branch instead of code run on every block.
        // Keys past the segment's end, or (block-causal) past a row's limit, are masked.
        if (kbase + 32 * kb + 32 > min(len, mask_from_wg)) {
          asm volatile("");
#pragma unroll
          for (int rr = 0; rr < 16; ++rr) {
            const int key = kbase + 32 * kb + 8 * (rr >> 2) + 4 * h32 + (rr & 3);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
              if (key >= len || key >= mask_from[nb]) sc[nb][rr] = NEG_INF;
          }
        }
        // online softmax per query row (lane pair); every piece's first block
        // holds a valid key, so m_run is finite before any all-masked block
        bool need[NB], any_need = false;
        float mx[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          float m = sc[nb][0];
#pragma unroll
          for (int rr = 1; rr < 16; ++rr) m = smax(m, sc[nb][rr]);
          mx[nb] = pair_max(m) + (FOLD ? m_fold[nb] : 0.f);  // the row max of s itself
          need[nb] = mx[nb] > m_run[nb] + kRescaleSlack;
          any_need |= need[nb];
        }
        if (__any(any_need)) {
          asm volatile("");
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            const float mnew = need[nb] ? mx[nb] : m_run[nb];
            const float alpha = __builtin_amdgcn_exp2f(m_run[nb] - mnew);
            m_run[nb] = mnew;
            l_run[nb] *= alpha;
#pragma unroll
            for (int fb = 0; fb < NFB; ++fb) {
              if constexpr (ACC_AGPR) scale_acc_agpr(o[nb][fb], alpha);
              else o[nb][fb] *= alpha;
            }
            if constexpr (FOLD) {  // re-base this block's scores and the next blocks' start
              const float d = mnew - m_fold[nb];
#pragma unroll
              for (int rr = 0; rr < 16; ++rr) sc[nb][rr] -= d;
              m_fold[nb] = mnew;
#pragma unroll
              for (int rr = 0; rr < 16; ++rr) negm[nb][rr] = -mnew;
            }
          }
        }
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          if constexpr (FOLD) {  // sc already holds s - m_run; row sums below, from the fp16 operand
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) sc[nb][rr] = __builtin_amdgcn_exp2f(sc[nb][rr]);
          } else {
            float lsum = 0.f;
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) {
              const float e = __builtin_amdgcn_exp2f(sc[nb][rr] - m_run[nb]);
              sc[nb][rr] = e;
              lsum += e;
            }
            l_run[nb] += lsum;
          }
        }
        // O^T += V^T[f][keys] * P^T[keys][rows]; each V^T fragment feeds NB MFMAs
        if constexpr (HALF) {
          f16x8 pf[NB][2];
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
              for (int j = 0; j < 8; ++j) pf[nb][u][j] = (f16)sc[nb][8 * u + j];
          if constexpr (FOLD) {  // row sums of the fp16 probabilities the value MFMAs use, two per v_dot2
            const f16x2 one2 = {(f16)1.f, (f16)1.f};
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
              float lsum = 0.f;
#pragma unroll
              for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                  lsum = __builtin_amdgcn_fdot2(f16x2{pf[nb][u][2 * j], pf[nb][u][2 * j + 1]}, one2, lsum, false);
              l_run[nb] += lsum;
            }
          }
          constexpr int NV = 2 * NFB;
          auto vfrag = [&](int i) -> f16x8 {
            if constexpr (VT_FROM_K) {
              // Fragment i = (fb, u): element j of lane l is channel 32fb + l%32 of
              // key 32kb + 16u + 4h32 + j%4 + 8(j/4), the key order in which the
              // score accumulator hands over P^T.  In each 16-lane group the
              // transposing read gives output lane m element m%4 of the 8-byte
              // slots that source lanes m/4, m/4 + 4, m/4 + 8, m/4 + 12 address,
              // so source lane sl addresses key 32kb + 16u + 4h32 + sl/4 at
              // channel 32fb + 16(group%2) + 4(sl%4) (elements 0-3); the second
              // read takes the keys 8 rows further (elements 4-7).
              const int sl = lane & 15, gg = lane >> 4;
              const int e = (32 * kb + 16 * (i & 1) + 4 * h32 + (sl >> 2)) * KS + 32 * (i >> 1) + 16 * (gg & 1) +
                            4 * (sl & 3);
              typedef short s16x4_t __attribute__((ext_vector_type(4)));
              const s16x4_t a0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                  (__attribute__((address_space(3))) s16x4_t*)(Ks + e));
              const s16x4_t a1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                  (__attribute__((address_space(3))) s16x4_t*)(Ks + e + 8 * KS));
              typedef short s16x8_t __attribute__((ext_vector_type(8)));
              const s16x8_t w = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
              return __builtin_bit_cast(f16x8, w);
            } else {
              return *reinterpret_cast<const f16x8*>(Ct + 32 * (i >> 1) * CS + 32 * kb + 16 * (i & 1) + 8 * h32);
            }
          };
          f16x8 vq[kAhead];
#pragma unroll
          for (int i = 0; i < kAhead && i < NV; ++i) vq[i] = vfrag(i);
#pragma unroll
          for (int i = 0; i < NV; ++i) {
            __builtin_amdgcn_sched_barrier(0);
            const f16x8 a = vq[i % kAhead];
            if (i + kAhead < NV) vq[i % kAhead] = vfrag(i + kAhead);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
              o[nb][i >> 1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, pf[nb][i & 1], o[nb][i >> 1], 0, 0, 0);
          }
          __builtin_amdgcn_sched_barrier(0);
        } else {
#pragma unroll
          for (int fb = 0; fb < NFB; ++fb)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
              const f32x4 run = *reinterpret_cast<const f32x4*>(Ct + 32 * fb * CS + 32 * kb + 16 * (q4 >> 1) +
                                                                8 * h32 + 4 * (q4 & 1));
#pragma unroll
              for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) o[nb][fb] = Mfma<float>::mma(run[i], sc[nb][4 * q4 + i], o[nb][fb]);
            }
        }
      }
    };

    // One tile: prefetch the next tile into the other stage, compute this one,
    // then wait for this thread's loads and meet at the barrier (which also
    // retires every read of `cur` before it is refilled).
    auto step = [&](int t, const T* cur, T* nxt) {
      if (t + 1 < kt1) issue_tile(s, t + 1, nxt);
      compute(t, cur);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    };

    issue_tile(s, kt0, lds0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int t = kt0; t < kt1; t += 2) {
      step(t, lds0, lds1);
      if (t + 1 < kt1) step(t + 1, lds1, lds0);
    }

    const bool full = causal || (kt0 == 0 && kt1 == p.KT);
    VT* out_s = static_cast<VT*>(p.out) + (s / p.heads) * p.out_so + (s % p.heads) * p.out_sh;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const float l_tot = pair_sum(l_run[nb]);
      const int qrow = row0 + 32 * nb + l32;
      if (full) {
        if (qrow < p.R) {
          VT* dst = out_s + (long)qrow * p.out_rs;
          const float inv = 1.f / l_tot;
#pragma unroll
          for (int fb = 0; fb < NFB; ++fb)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
              const int f = 32 * fb + 8 * q4 + 4 * h32;
              if (f < DV)
                store4(dst + f, o[nb][fb][4 * q4] * inv, o[nb][fb][4 * q4 + 1] * inv, o[nb][fb][4 * q4 + 2] * inv,
                       o[nb][fb][4 * q4 + 3] * inv);
            }
        }
      } else if (row0 < p.R) {
        const long slot_row =
            (long)(2 * vw + (first_piece ? 0 : 1)) * kAttnMaxRows + wave * RW + 32 * nb + l32;
        PartT<T>* po = reinterpret_cast<PartT<T>*>(p.part_o) + slot_row * DV;
        const float inv = 1.f / l_tot;  // >= 1: the piece's first block holds a valid key
#pragma unroll
        for (int fb = 0; fb < NFB; ++fb)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const int f = 32 * fb + 8 * q4 + 4 * h32;
            if (f < DV)
              store_part4<T>(po + f, o[nb][fb][4 * q4] * inv, o[nb][fb][4 * q4 + 1] * inv, o[nb][fb][4 * q4 + 2] * inv,
                             o[nb][fb][4 * q4 + 3] * inv);
          }
        if (h32 == 0) {
          p.part_ml[slot_row * 2] = m_run[nb];
          p.part_ml[slot_row * 2 + 1] = l_tot;
        }
      }
    }
  }
}

// Issue-slot plan of the pipelined kernel's softmax work (see step() in
// flash_attn_pipe_kernel).  With NB 32-row blocks per wave, a step has
// NS = NQ + NB NV slots, one MFMA each (NQ score MFMAs, then NB NV value
// MFMAs: half 0 of the block's keys, then half 1).  Work items, with their
// cost in plain-VALU units (a v_exp_f32 counts 2), for NB = 2 (NB = 1 keeps
// the items of row block 0 only):
//   [0, 16)   exponential k of half 0 (row block k/8, element 8u + k%8 with u = 0)
//   [16, 24)  fp16 pack (+ v_dot2 row sum) of half-0 pair q (elements 2q, 2q+1)
//   [24, 40)  exponentials of half 1;  [40, 48) packs of half 1
//   [48, 80)  copy of score element e of the next block out of its accumulator
//   [80, 84)  block max over 8 elements;  [84, 86) pair max and rescale test
// Each item goes to the first slot at or after its predecessor's that has
// room within BUDGET units and follows its inputs (a pack one slot after its
// second exponential, copies after the last score MFMA, a max after its
// copies, a test after its maxes).  Half-u packs must precede the first value
// MFMA that reads them.  The plan uses the smallest budget that meets every
// deadline: about four plain VALU instructions fit behind one MFMA on gfx950.
// Packs cost 2 units with their v_dot2 row sum, 1 without it; then (LAG) each
// pack issues after the next pair's two exponentials, so a slot takes two
// exponentials or one with a pack (or two), and packing in issue order does
// not leave a slot at 2 or 3 units behind every pack.
struct PipeSlotPlan {
  static constexpr int NITEM = 86, MAXS = 128, MAXPER = 8;
  int slot_of[NITEM];
  int lo[MAXS], hi[MAXS];  // slot s issues items pipe_item_order(lo[s] .. hi[s]-1)
  int budget;
  bool ok;
};
constexpr int pipe_item_cost(int i, int pack_cost) {
  return (i >= 16 && i < 24) || (i >= 40 && i < 48) ? pack_cost : i < 48 ? 2 : i < 80 ? 1 : 4;
}
// Items in issue order: exponentials of each half interleaved with the packs
// they complete, then (COPIES) the copies, then maxes and tests.  Without
// copies (scores accumulated in VGPRs, which the maxes read directly) the
// order has 54 entries and skips items 48..79.
// With NB = 1 the order keeps its shape over the items of row block 0
// (exponentials 8 per half, packs 4, copies 16, maxes 2, one test).
constexpr int pipe_nitems(bool copies, int nb) { return 27 * nb + (copies ? 16 * nb : 0); }
constexpr int pipe_item_order(int j, bool copies, bool lag, int nb) {
  const int H = 12 * nb, np = 4 * nb;  // entries and exponential pairs per half
  if (j < 2 * H) {
    const int h = j / H, r = j % H;
    if (!lag) {  // per pair q: E[2q], E[2q+1], P[q]
      const int grp = r / 3, pos = r % 3;
      return pos < 2 ? 24 * h + 2 * grp + pos : 24 * h + 16 + grp;
    }
    // E[0], E[1], then E[2q], E[2q+1], P[q-1] for q = 1..np-1, then P[np-1]
    if (r < 2) return 24 * h + r;
    if (r == H - 1) return 24 * h + 16 + np - 1;
    const int grp = (r - 2) / 3, pos = (r - 2) % 3;
    return pos < 2 ? 24 * h + 2 * (grp + 1) + pos : 24 * h + 16 + grp;
  }
  j -= 2 * H;
  if (copies) {
    if (j < 16 * nb) return 48 + j;
    j -= 16 * nb;
  }
  return j < 2 * nb ? 80 + j : 84 + (j - 2 * nb);
}
constexpr PipeSlotPlan pipe_slot_plan_b(int NQ, int NV, int budget, bool copies, int pack_cost, bool lag, int nb) {
  PipeSlotPlan p{};
  p.budget = budget;
  p.ok = true;
  const int NS = NQ + nb * NV;
  const int NI = pipe_nitems(copies, nb);
  int load[128] = {};
  int cur = 0;
  for (int i = 0; i < PipeSlotPlan::NITEM; ++i) p.slot_of[i] = -1;
  for (int j = 0; j < NI; ++j) {
    const int i = pipe_item_order(j, copies, lag, nb);
    int earliest = cur;
    if (i >= 16 && i < 24) earliest = p.slot_of[2 * (i - 16) + 1] + 1;
    if (i >= 40 && i < 48) earliest = p.slot_of[24 + 2 * (i - 40) + 1] + 1;
    if (i >= 48 && i < 80) earliest = NQ + 1;
    if (i >= 80 && i < 84)
      earliest = copies ? p.slot_of[48 + 16 * ((i - 80) >> 1) + 8 * ((i - 80) & 1) + 7] + 1 : NQ + 1;
    if (i >= 84) earliest = p.slot_of[80 + 2 * (i - 84) + 1] + 1;
    int s = earliest > cur ? earliest : cur;
    while (s < NS && load[s] > 0 && load[s] + pipe_item_cost(i, pack_cost) > budget) ++s;
    if (s >= NS) {
      p.ok = false;
      return p;
    }
    p.slot_of[i] = s;
    load[s] += pipe_item_cost(i, pack_cost);
    cur = s;
    // a half-u pack of row block r precedes value MFMA slot NQ + u nb NV / 2 + r
    int deadline = NS - 1;
    if (i >= 16 && i < 24) deadline = NQ - 1 + ((i - 16) >> 2);
    if (i >= 40 && i < 48) deadline = NQ + nb * NV / 2 - 1 + ((i - 40) >> 2);
    if (s > deadline) p.ok = false;
  }
  // items go to slots in issue order, so each slot holds a run of it
  for (int s = 0; s < PipeSlotPlan::MAXS; ++s) p.lo[s] = p.hi[s] = PipeSlotPlan::NITEM;
  for (int j = NI - 1; j >= 0; --j) p.lo[p.slot_of[pipe_item_order(j, copies, lag, nb)]] = j;
  for (int j = 0; j < NI; ++j) p.hi[p.slot_of[pipe_item_order(j, copies, lag, nb)]] = j + 1;
  for (int s = 0; s < NS; ++s) {
    if (p.lo[s] == PipeSlotPlan::NITEM) p.lo[s] = p.hi[s] = 0;
    if (p.hi[s] - p.lo[s] > PipeSlotPlan::MAXPER) p.ok = false;
  }
  return p;
}
constexpr PipeSlotPlan pipe_slot_plan(int NQ, int NV, bool copies, int pack_cost, bool lag, int nb) {
  for (int b = 3; b <= 12; ++b) {
    const PipeSlotPlan p = pipe_slot_plan_b(NQ, NV, b, copies, pack_cost, lag, nb);
    if (p.ok) return p;
  }
  return pipe_slot_plan_b(NQ, NV, 0, copies, pack_cost, lag, nb);
}
template <int NQ, int NV, bool COPIES, int PACKC, bool LAG, int NB>
inline constexpr PipeSlotPlan kPipeSlotPlan = pipe_slot_plan(NQ, NV, COPIES, PACKC, LAG, NB);

// Software-pipelined latent attention, bf16 storage.  One workgroup = 4 waves
// (one per SIMD) x 64 query rows (two 32-row blocks), so every K and V fragment
// read from LDS feeds two MFMAs: half the LDS reads per FLOP of the 32-row
// kernel.  With a single wave per SIMD no other wave hides the softmax, so each
// wave hides its own: while the score MFMAs of 32-key block j+1 accumulate
// (AGPRs), the softmax of block j runs on a VGPR copy of its scores, its
// instructions placed one by one between the MFMAs; then the value MFMAs of
// block j run.  The score MFMAs start from a splat of -m (the row's running
// max), so they yield s - m and the softmax has no subtraction.  Three LDS
// stages hold the tile of block j (value product), the tile of block j+1
// (score product) and the tile two ahead (DMA in flight); one barrier per
// tile.  Same staging (fp16 key tiles, V^T by transposing reads), scheduling
// and numerics as flash_attn_kernel, whose comments cover them.
// VSC (score widths up to 128, or one row block per wave): the score
// accumulators live in VGPRs, two sets whose roles alternate every step (the
// current block's, on which its softmax runs, and the next block's, which the
// score MFMAs -- issued from asm in the VGPR form -- accumulate), so the
// softmax needs no AGPR copies.
// NB = 1 (d_c 448: 14 value blocks of 32 channels fill the AGPRs) gives each
// wave 32 rows, so each fragment read feeds one MFMA.  NST = 2 (a 64-key tile
// of 480 channels is 60 KB, so three stages exceed the LDS): tile t+1 takes
// the stage of tile t-1 once every wave is past it, i.e. its loads are issued
// in the first slots of the step that finishes the scores of tile t and must
// land by the next; they are issued from asm so that the compiler adds no
// wait for them before the LDS reads of that step.
template <int D, int DV, int KTILE, bool VSC, int NB, int NST>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void flash_attn_pipe_kernel(FlashArgs<bf16> p) {
  using T = bf16;
  using VT = f16;  // query, value-operand and output type
  using G = TileGeo<T, D, DV, KTILE>;
  constexpr int NW = 4, RW = 32 * NB;
  static_assert(NB == 1 || NB == 2, "one or two 32-row blocks per wave");
  static_assert(NST == 2 || NST == 3, "two or three LDS stages");
  // LDS key tile (16-B chunk c of key row r): four regions of 16 rows (wave w
  // loads region w), each of CH/4 blocks of 1 KB holding chunks 4k..4k+3 of
  // its rows; within a block, chunk c sits at 256 (c % 4) + 16 ((r % 16) ^
  // 4 (c % 4)) bytes.  A K-fragment read (16 lanes: 16 rows of one chunk) and a
  // transposing V read (32 lanes: 4 rows, 4 chunks) both touch every 16-B bank
  // group of the 64 banks once, and each lane's DMA source is a constant of
  // the lane plus 64 bytes per block (no address arithmetic per load).
  constexpr int VEC = 8, CH = D / 8, KS_EL = KTILE * D;
  constexpr int REG_EL = 16 * D;       // elements per 16-row region
  constexpr int KI = KTILE * CH / 64;  // 1-KB loads per tile
  constexpr int NKS = D / 16;    // score k-steps of 16 channels
  constexpr int NFB = G::DVP / 32;
  // VSC with two row blocks: one more value block whose A operand is a
  // constant 1.0 fragment, so its accumulator holds the row sums of P,
  // rescaled with O (no v_dot2 sums; with one row block the AGPRs are full)
  constexpr bool ONES = VSC && NB == 2;
  constexpr int NFV = NFB + (ONES ? 1 : 0);  // value accumulator blocks
  constexpr int NV = 2 * NFV;    // value MFMAs per block and row block
  constexpr int KA = NB == 2 ? 2 : 4;  // fragment reads in flight ahead of their first MFMA
  constexpr int NI_W = KI / NW;
  constexpr int DS = NST == 3 ? 4 : (NI_W + 1) / 2;  // slots carrying a tile's loads, two per slot
  static_assert(CH % 4 == 0 && KI % NW == 0 && KTILE == 16 * NW, "tile layout: one 16-row region per wave");
  static_assert(KTILE == 64, "two 32-key blocks per tile");
  static_assert(NW * RW <= kAttnMaxRows && G::DVP <= D, "bad shape");
  static_assert(NKS * 16 == D && G::DVP == DV, "whole 16-channel k-steps and 32-channel value blocks");

  __shared__ __attribute__((aligned(16))) T lds[NST * KS_EL];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = NST == 2 ? __builtin_amdgcn_readfirstlane(tid >> 6) : tid >> 6;
  const int l32 = lane & 31, h32 = lane >> 5;
  const float NEG_INF = -__builtin_huge_valf();

  auto tile_rsrc = [&](int s, int t) __attribute__((always_inline)) {
    return raw_rsrc(static_cast<const char*>(p.val0) + ((size_t)s * p.KT + t) * (KTILE * D * 2),
                    (uint32_t)(KTILE * D * 2));
  };
  // LDS-DMA load k (0..NI_W-1) of this wave's share of a tile: block k of
  // region `wave`; lane L fills slot L: chunk 4k + L/16 of row
  // 16 wave + ((L % 16) ^ 4 (L / 16)).  The pre-pass stores the tile as this
  // LDS image, so the load copies the block's 1 KB of contiguous bytes.
  // `st`: element offset of the destination stage.
  const uint32_t dma_voff = (uint32_t)((wave * REG_EL + 8 * lane) * 2);
  const uint32_t lds_u32 = (uint32_t)(size_t)(__attribute__((address_space(3))) T*)lds;
  auto issue_part = [&](__amdgpu_buffer_rsrc_t krs, uint32_t st, int k) __attribute__((always_inline)) {
    if constexpr (NST == 2)
      dma16_lds(krs, dma_voff + (uint32_t)(1024 * k), lds_u32 + 2 * (st + (uint32_t)(wave * REG_EL + k * 512)));
    else
      lds_dma16(krs, dma_voff + (uint32_t)(1024 * k), lds + st + wave * REG_EL + k * 512);
  };
  auto issue_tile = [&](int s, int t, uint32_t st) __attribute__((always_inline)) {
    const auto krs = tile_rsrc(s, t);
#pragma unroll
    for (int k = 0; k < NI_W; ++k) issue_part(krs, st, k);
  };

  const bool causal = p.causal_tokens > 0;
  auto row_limit = [&](int r) __attribute__((always_inline)) {
    const int lim = (r / p.row_div / p.causal_tokens + 1) * p.causal_tokens;
    return lim < p.len1 ? lim : p.len1;
  };
  const int vw = p.G % 8 == 0 ? (int)(blockIdx.x % 8) * (p.G / 8) + (int)(blockIdx.x / 8) : (int)blockIdx.x;
  const int n_whole = causal ? 0 : (int)(p.dp_units / p.G);
  const long I = ((long)p.S * p.RB - (causal ? 0 : p.dp_units)) * p.KT;
  const long it0 = (long)vw * I / p.G, it1 = (long)(vw + 1) * I / p.G;
  const long u_first = causal ? (long)p.S * p.RB - 1 - blockIdx.x : p.dp_units + it0 / p.KT;
  const int npieces = causal ? 1 : (int)((it1 - 1) / p.KT - it0 / p.KT + 1);
  for (int job = 0; job < n_whole + npieces; ++job) {
    const bool whole = job < n_whole;
    const int k = job - n_whole;
    const int piece = whole ? 0 : npieces > 1 ? (k == 0 ? npieces - 1 : k - 1) : 0;
    const long unit = whole ? (long)job * p.G + vw : u_first + piece;
    const int s = (int)(unit / p.RB), rb = (int)(unit % p.RB);
    int kt0, kt1;
    if (causal) {
      const int last_row = min((rb + 1) * (NW * RW), p.R) - 1;
      kt0 = 0;
      kt1 = p.tiles0 + (row_limit(last_row) + KTILE - 1) / KTILE;
    } else if (whole) {
      kt0 = 0;
      kt1 = p.KT;
    } else {
      kt0 = piece == 0 ? (int)(it0 % p.KT) : 0;
      kt1 = piece == npieces - 1 ? (int)((it1 - 1) % p.KT) + 1 : p.KT;
    }
    const bool first_piece = piece == 0;
    const int row0 = rb * (NW * RW) + wave * RW;
    const int mask_from_wg = causal ? row_limit(rb * (NW * RW)) : 0x7fffffff;
    int mask_from[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) mask_from[nb] = causal ? row_limit(row0 + 32 * nb + l32) : 0x7fffffff;
    const int ntiles = kt1 - kt0;
    // element offsets of the stages of tiles i, i+1, i+2 (rotated per tile; no
    // modulo, so LDS addresses stay provably non-negative and fragment offsets
    // fold into the read instructions)
    uint32_t st_cur = 0, st_nxt = KS_EL, st_nn = NST == 3 ? 2 * KS_EL : 0;

    // every wave is done with the stages of the previous job
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    issue_tile(s, kt0, st_cur);
    if (ntiles > 1) issue_tile(s, kt0 + 1, st_nxt);

    f16x8 qf[NB][NKS];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int qrow = row0 + 32 * nb + l32;
      const f16* qsrc = static_cast<const f16*>(p.q) + s * p.q_ss + (long)qrow * D + 8 * h32;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
        qf[nb][ks] = qrow < p.R ? *reinterpret_cast<const f16x8*>(qsrc + 16 * ks) : f16x8{};
    }
    f32x16 o[NB][NFV];
    float m_run[NB], l_run[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      l_run[nb] = 0.f;
#pragma unroll
      for (int fb = 0; fb < NFV; ++fb) {
        o[nb][fb] = f32x16{};
        asm volatile("" : "+a"(o[nb][fb]));
      }
    }
    f32x16 sc[NB];    // score accumulators of the next block (AGPRs; VSC: one of the two VGPR sets)
    f32x16 negm[NB];  // -m_run splat: the score MFMAs start from it, so they produce s - m_run
    f32x16 d[NB];     // scores (minus m_run) of the current block, copied out of sc (VGPRs; VSC: the other set)
    f16x8 kq[KA];     // K fragments of the next score product, read ahead
    f16x8 pf[NB][2];

    // LDS fragment readers (element offsets; a region is REG_EL elements, a
    // block 512, a chunk-of-block column 128, a slot 8).  K: row 32kb + l32
    // (region 2kb + l32/16), chunk 2ks + h32 (block ks/2, column
    // cc = 2 (ks % 2) + h32): one lane offset for even and one for odd ks.
    const int k_off0 = REG_EL * (l32 >> 4) + 128 * h32 + 8 * ((l32 & 15) ^ (4 * h32));
    const int k_off1 = REG_EL * (l32 >> 4) + 128 * h32 + 8 * ((l32 & 15) ^ (8 + 4 * h32));
    auto kfrag = [&](const T* buf, int kb, int ks) __attribute__((always_inline)) {
      return *reinterpret_cast<const f16x8*>(buf + ((ks & 1) ? k_off1 : k_off0) + 2 * REG_EL * kb + 512 * (ks >> 1) +
                                             256 * (ks & 1));
    };
    // V^T (as flash_attn_kernel, by transposing reads): source lane sl of
    // 16-lane group gg reads 8 bytes (half sl % 2) of row 32kb + 16u + 4h32 +
    // sl/4 (+ 8 for the second read; region 2kb + u), chunk 4fb + i with
    // i = 2(gg%2) + (sl%4)/2 (block fb, column i).
    const int v_sl = lane & 15, v_i = 2 * ((lane >> 4) & 1) + ((v_sl & 3) >> 1);
    const int v_off1 = 128 * v_i + 8 * ((4 * h32 + (v_sl >> 2)) ^ (4 * v_i)) + 4 * (v_sl & 1);
    const int v_off2 = 128 * v_i + 8 * ((8 + 4 * h32 + (v_sl >> 2)) ^ (4 * v_i)) + 4 * (v_sl & 1);
    auto vfrag = [&](const T* buf, int kb, int i) __attribute__((always_inline)) -> f16x8 {
      const int e0 = REG_EL * (2 * kb + (i & 1)) + 512 * (i >> 1);  // region of the block half, block fb
      typedef short s16x4_t __attribute__((ext_vector_type(4)));
      const s16x4_t a0 =
          __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)(buf + e0 + v_off1));
      const s16x4_t a1 =
          __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)(buf + e0 + v_off2));
      return __builtin_bit_cast(f16x8, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    // Keys past the segment's end, or (block-causal) past a row's limit, -> -inf.
    auto mask = [&](f32x16 (&sc)[NB], int t, int kb) __attribute__((always_inline)) {
      int g, kbase, len;
      tile_segment<T, KTILE>(p, t, g, kbase, len);
      if (kbase + 32 * kb + 32 > min(len, mask_from_wg)) {
        asm volatile("");
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
          const int key = kbase + 32 * kb + 8 * (rr >> 2) + 4 * h32 + (rr & 3);
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
            if (key >= len || key >= mask_from[nb]) sc[nb][rr] = NEG_INF;
        }
      }
    };
    // Plain scores of block kb of `buf` into sc, no overlap (first block of a job).
    auto qk_only = [&](f32x16 (&sc)[NB], const T* buf, int kb) __attribute__((always_inline)) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) sc[nb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const f16x8 a = kfrag(buf, kb, ks);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          if constexpr (VSC) mfma_vgpr_acc(sc[nb], a, qf[nb][ks]);
          else sc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, qf[nb][ks], sc[nb], 0, 0, 0);
        }
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        if constexpr (VSC) asm volatile("s_nop 7\n\ts_nop 7" : "+v"(sc[nb]));  // results before VALU reads
        else asm volatile("" : "+a"(sc[nb]));
      }
    };
    // Softmax work items of one block (d: VGPR copy of its scores), in the
    // order they are issued between MFMAs.  Elements of the block are taken in
    // two halves u: keys 16u..16u+15 of the block, i.e. rr = 8u..8u+7 of each
    // row block; half u feeds the value MFMAs with B operand pf[.][u].
    float mloc[NB], mx[NB], lsum[NB];
    bool need[NB];
    // q = 0..3: row block q/2, elements 8(q%2)..+7
    auto max_item = [&](const f32x16 (&d)[NB], int q) __attribute__((always_inline)) {
      const int nb = q >> 1, r0 = 8 * (q & 1);
      float m = r0 ? mloc[nb] : d[nb][0];
#pragma unroll
      for (int rr = (r0 ? 0 : 1); rr < 8; ++rr) m = smax(m, d[nb][r0 + rr]);
      mloc[nb] = m;
    };
    auto cmp_item = [&](int nb) __attribute__((always_inline)) {
      mx[nb] = pair_max(mloc[nb]);  // max of s - m_run over the row's keys of the block
      need[nb] = mx[nb] > kRescaleSlack;
    };
    auto set_negm = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) negm[nb][rr] = -m_run[nb];
        if constexpr (VSC) asm volatile("s_nop 3" : "+v"(negm[nb]));  // VALU writes before an MFMA reads them
        else asm volatile("" : "+a"(negm[nb]));
      }
    };
    // Rows whose block max exceeds m_run by more than the slack move m_run
    // up; o and l follow.  Rare: a real (uniform) branch.
    auto rescale = [&](f32x16 (&d)[NB]) __attribute__((always_inline)) {
      bool any_need = need[0];
#pragma unroll
      for (int nb = 1; nb < NB; ++nb) any_need = any_need || need[nb];
      if (__any(any_need)) {
        asm volatile("");
        asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 15");  // value MFMAs still writing o
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const float dm = need[nb] ? mx[nb] : 0.f;
          const float alpha = __builtin_amdgcn_exp2f(-dm);
          m_run[nb] += dm;
          l_run[nb] *= alpha;
#pragma unroll
          for (int fb = 0; fb < NFV; ++fb) scale_acc_agpr(o[nb][fb], alpha);
#pragma unroll
          for (int rr = 0; rr < 16; ++rr) d[nb][rr] -= dm;  // re-base this block's scores
        }
        set_negm();
      }
    };
    // element k (0..15) of half u: row block k/8, rr = 8u + k%8
    auto exp_item = [&](f32x16 (&d)[NB], int u, int k) __attribute__((always_inline)) {
      const int nb = k >> 3, rr = 8 * u + (k & 7);
      d[nb][rr] = __builtin_amdgcn_exp2f(d[nb][rr]);
    };
    // pair q (0..7) of half u: elements 2q, 2q+1 -> fp16 probabilities and their row sum
    auto pack_item = [&](const f32x16 (&d)[NB], int u, int q) __attribute__((always_inline)) {
      const int nb = q >> 2, j = 2 * (q & 3);
      const f16x2 one2 = {(f16)1.f, (f16)1.f};
      pf[nb][u][j] = (f16)d[nb][8 * u + j];
      pf[nb][u][j + 1] = (f16)d[nb][8 * u + j + 1];
      if constexpr (!ONES)
        lsum[nb] = __builtin_amdgcn_fdot2(f16x2{pf[nb][u][j], pf[nb][u][j + 1]}, one2, lsum[nb], false);
    };
    // value fragment n in issue order: half n/NFV, 32-channel block n%NFV (the
    // ones block: a constant 1.0 fragment, no LDS read)
    auto vfrag_n = [&](const T* buf, int kb, int n) __attribute__((always_inline)) -> f16x8 {
      if (ONES && n % NFV == NFB) {
        f16x8 one;
#pragma unroll
        for (int e = 0; e < 8; ++e) one[e] = (f16)1.f;
        return one;
      }
      return vfrag(buf, kb, 2 * (n % NFV) + n / NFV);
    };

    auto copy_item = [&](int e) __attribute__((always_inline)) {  // element e (0..31) of sc -> d
      float x = sc[e >> 4][e & 15];
      asm volatile("" : "+v"(x));
      d[e >> 4][e & 15] = x;
    };
    auto needs_mask = [&](int t, int kb) __attribute__((always_inline)) {
      int g, kbase, len;
      tile_segment<T, KTILE>(p, t, g, kbase, len);
      return kbase + 32 * kb + 32 > min(len, mask_from_wg);
    };

    // One pipelined block.  On entry d holds the scores of block (t, kb) and
    // mx/need its rescale test (both computed by the previous step, or by the
    // prologue); masked keys are applied here (rare) and the test redone.
    // Then 2*NKS score MFMAs of block (qbuf, qkb) into sc and 2*NV value MFMAs
    // of block (t, kb) from pbuf run as issue slots.  A wave issues in order,
    // and an MFMA occupies the matrix core for ~32 cycles; measured on gfx950,
    // about four plain VALU instructions (or two with one v_exp_f32) fit
    // behind one MFMA before they delay the next, so each slot carries about
    // that much:
    // the softmax items placed by PipeSlotPlan (exponentials and packs of
    // half 0 and half 1, then the next block's copy, max and rescale test; the
    // value MFMAs of half 0 need the packs of half 0 only), and in the last
    // four slots the loads of the tile two ahead (dma), two per slot.
    // prefetch: read the next step's first K fragments (nqbuf, nqkb) in the
    // last slots.  has_next = false (last block of a job): no score product.
    auto step = [&](const T* qbuf, int qkb, int t, int kb, const T* pbuf, bool has_next, bool kq_ready,
                    const T* nqbuf, int nqkb, bool prefetch, bool dma, __amdgpu_buffer_rsrc_t krs,
                    uint32_t dbuf, f32x16 (&d)[NB], f32x16 (&sc)[NB]) __attribute__((always_inline)) {
      if (needs_mask(t, kb)) {
        asm volatile("");
        mask(d, t, kb);
#pragma unroll
        for (int q = 0; q < 2 * NB; ++q) max_item(d, q);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) cmp_item(nb);
      }
      rescale(d);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) lsum[nb] = 0.f;
      if (!has_next) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
#pragma unroll
          for (int k = 0; k < 8 * NB; ++k) exp_item(d, u, k);
#pragma unroll
          for (int q = 0; q < 4 * NB; ++q) pack_item(d, u, q);
        }
#pragma unroll
        for (int n = 0; n < NV; ++n) {
          const f16x8 a = vfrag_n(pbuf, kb, n);
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
            o[nb][n % NFV] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, pf[nb][n / NFV], o[nb][n % NFV], 0, 0, 0);
        }
      } else {
        if (!kq_ready) {
#pragma unroll
          for (int i = 0; i < KA; ++i) kq[i] = kfrag(qbuf, qkb, i);
        }
        f16x8 vq[KA];
        constexpr int NQ = NB * NKS, NS = NQ + NB * NV;
        constexpr PipeSlotPlan plan = kPipeSlotPlan<NQ, NV, !VSC, ONES ? 1 : 2, ONES, NB>;
        static_assert(plan.ok, "no issue-slot plan meets the deadlines");
        auto slot_work = [&](int slot) __attribute__((always_inline)) {
          __builtin_amdgcn_sched_barrier(0);
          const int nb = slot % NB;
          if (slot < NQ) {  // score MFMA (k-step slot/NB, row block nb); next K fragment after the last use
            const int ks = slot / NB;
            if constexpr (VSC) {
              if (ks == 0) sc[nb] = mfma_vgpr(kq[ks % KA], qf[nb][ks], negm[nb]);
              else mfma_vgpr_acc(sc[nb], kq[ks % KA], qf[nb][ks]);
            } else {
              sc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kq[ks % KA], qf[nb][ks], ks == 0 ? negm[nb] : sc[nb], 0,
                                                              0, 0);
            }
            if (nb == NB - 1 && ks + KA < NKS) kq[ks % KA] = kfrag(qbuf, qkb, ks + KA);
            if (slot >= NQ - NB * KA && nb == 0)
              vq[(slot - (NQ - NB * KA)) / NB] = vfrag_n(pbuf, kb, (slot - (NQ - NB * KA)) / NB);
          } else {  // value MFMA (fragment n, row block nb)
            const int n = (slot - NQ) / NB;
            o[nb][n % NFV] =
                __builtin_amdgcn_mfma_f32_32x32x16_f16(vq[n % KA], pf[nb][n / NFV], o[nb][n % NFV], 0, 0, 0);
            if (nb == NB - 1 && n + KA < NV) vq[n % KA] = vfrag_n(pbuf, kb, n + KA);
          }
          // VSC: the maxes read the accumulators of MFMAs the compiler does not
          // track; wait states ahead of the first
          if constexpr (VSC)
            if (slot == plan.slot_of[80]) asm volatile("s_nop 7\n\ts_nop 3" ::: "memory");
#pragma unroll
          for (int k = 0; k < PipeSlotPlan::MAXPER; ++k) {
            const int j = plan.lo[slot] + k;
            if (j >= plan.hi[slot]) continue;
            const int i = pipe_item_order(j, !VSC, ONES, NB);
            if (i < 16) exp_item(d, 0, i);
            else if (i < 24) pack_item(d, 0, i - 16);
            else if (i < 40) exp_item(d, 1, i - 24);
            else if (i < 48) pack_item(d, 1, i - 40);
            else if (i < 80) {
              if constexpr (!VSC) copy_item(i - 48);
            } else if (i < 84) {
              if constexpr (VSC) max_item(sc, i - 80);  // the next block's scores, in the accumulators
              else max_item(d, i - 80);
            } else cmp_item(i - 84);
          }
          // NST = 3: after the step's last transposing read: the compiler cannot
          // tell the DMA's stage from the stages being read and waits for the
          // DMA before any later transposing read (the next step's first, ~25
          // slots on).  NST = 2: in the first slots (asm loads, no such wait).
          if (dma) {
            const int ds = NST == 3 ? slot - (NS - DS) : slot;
            if (ds >= 0 && ds < DS) {
#pragma unroll
              for (int k = 2 * ds; k < 2 * ds + 2 && k < NI_W; ++k) issue_part(krs, dbuf, k);
            }
          }
          if (prefetch && slot >= NS - NB * KA && slot % NB == NB - 1)
            kq[(slot - (NS - NB * KA)) / NB] = kfrag(nqbuf, nqkb, (slot - (NS - NB * KA)) / NB);
        };
        // eight loops, so each stays within the compiler's full-unroll size limit
        constexpr int NS8 = (NS + 7) / 8;
#pragma unroll
        for (int slot = 0; slot < NS8; ++slot) slot_work(slot);
#pragma unroll
        for (int slot = NS8; slot < 2 * NS8; ++slot) slot_work(slot);
#pragma unroll
        for (int slot = 2 * NS8; slot < 3 * NS8; ++slot) slot_work(slot);
#pragma unroll
        for (int slot = 3 * NS8; slot < 4 * NS8; ++slot) slot_work(slot);
#pragma unroll
        for (int slot = 4 * NS8; slot < 5 * NS8; ++slot) slot_work(slot);
#pragma unroll
        for (int slot = 5 * NS8; slot < 6 * NS8; ++slot) slot_work(slot);
#pragma unroll
        for (int slot = 6 * NS8; slot < 7 * NS8; ++slot) slot_work(slot);
#pragma unroll
        for (int slot = 7 * NS8; slot < NS; ++slot) slot_work(slot);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          if constexpr (VSC) asm volatile("" : "+v"(sc[nb]));
          else asm volatile("" : "+a"(sc[nb]));
        }
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        if constexpr (!ONES) l_run[nb] += lsum[nb];
#pragma unroll
        for (int fb = 0; fb < NFV; ++fb) asm volatile("" : "+a"(o[nb][fb]));
      }
    };

    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    // Prologue: block 0's plain scores; their row max starts m_run (every
    // job's first block holds a valid key for every row, so it is finite).
    // K fragments of block 1 read ahead.
    qk_only(VSC ? d : sc, lds + st_cur, 0);
#pragma unroll
    for (int i = 0; i < KA; ++i) kq[i] = kfrag(lds + st_cur, 1, i);
    if constexpr (!VSC) {
#pragma unroll
      for (int e = 0; e < 32; ++e) copy_item(e);
    }
    mask(d, kt0, 0);
#pragma unroll
    for (int q = 0; q < 2 * NB; ++q) max_item(d, q);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      m_run[nb] = pair_max(mloc[nb]);
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) d[nb][rr] -= m_run[nb];
      need[nb] = false;
    }
    set_negm();
    if constexpr (NST == 3) {
      for (int i = 0; i + 1 < ntiles; ++i) {
        const int t = kt0 + i;
        const T* cur = lds + st_cur;
        // Tile t+1 has landed and every wave is past tile t-1 (its last reads
        // were the value product of the previous step), whose stage takes tile
        // t+2.
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        // block 0 of tile t under the scores of its block 1, with the loads of
        // tile t+2 issued in its last slots; reads ahead the K fragments of
        // block 0 of tile t+1
        // (no tile t+2: an empty resource, whose loads write zeros into the free
        // stage, keeps the slots free of branches)
        const auto krs = i + 2 < ntiles ? tile_rsrc(s, t + 2) : raw_rsrc(p.val0, 0u);
        step(cur, 1, t, 0, cur, true, true, lds + st_nxt, 0, true, true, krs, st_nn, d, sc);
        // block 1 of tile t under the scores of block 0 of tile t+1; reads ahead
        // the K fragments of block 1 of tile t+1
        if constexpr (VSC) step(lds + st_nxt, 0, t, 1, cur, true, true, lds + st_nxt, 1, true, false, krs, st_nn, sc, d);
        else step(lds + st_nxt, 0, t, 1, cur, true, true, lds + st_nxt, 1, true, false, krs, st_nn, d, sc);
        const uint32_t st_old = st_cur;
        st_cur = st_nxt;
        st_nxt = st_nn;
        st_nn = st_old;
      }
    } else {
      for (int i = 0; i + 1 < ntiles; ++i) {
        const int t = kt0 + i;
        const T* cur = lds + st_cur;
        // Tile t+1: loaded by the prologue for i = 0; otherwise into the stage
        // of tile t-1 once every wave is past it (its last reads were the value
        // product of the previous step), issued in the first slots of block 0
        // of tile t, waited for before block 1.
        const bool load = i > 0;
        if (load) __syncthreads();
        const auto krs = load ? tile_rsrc(s, t + 1) : raw_rsrc(p.val0, 0u);
        step(cur, 1, t, 0, cur, true, true, lds + st_nxt, 0, !load, load, krs, st_nxt, d, sc);
        if (load) {
          wait_vmcnt<0>();
          __syncthreads();
        }
        if constexpr (VSC) step(lds + st_nxt, 0, t, 1, cur, true, !load, lds + st_nxt, 1, true, false, krs, st_nxt, sc, d);
        else step(lds + st_nxt, 0, t, 1, cur, true, !load, lds + st_nxt, 1, true, false, krs, st_nxt, d, sc);
        const uint32_t st_old = st_cur;
        st_cur = st_nxt;
        st_nxt = st_old;
      }
    }
    {  // last tile (landed: waited for at the previous tile's barrier, or in the prologue)
      const int t = kt1 - 1;
      const T* cur = lds + st_cur;
      const auto krs = tile_rsrc(s, t);
      step(cur, 1, t, 0, cur, true, true, cur, 0, false, false, krs, st_nn, d, sc);
      if constexpr (VSC) step(cur, 0, t, 1, cur, false, true, cur, 0, false, false, krs, st_nn, sc, d);
      else step(cur, 0, t, 1, cur, false, true, cur, 0, false, false, krs, st_nn, d, sc);
    }

    const bool full = causal || (kt0 == 0 && kt1 == p.KT);
    VT* out_s = static_cast<VT*>(p.out) + (s / p.heads) * p.out_so + (s % p.heads) * p.out_sh;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const float l_tot = ONES ? o[nb][NFB][0] : pair_sum(l_run[nb]);
      const int qrow = row0 + 32 * nb + l32;
      if (full) {
        if (qrow < p.R) {
          VT* dst = out_s + (long)qrow * p.out_rs;
          const float inv = 1.f / l_tot;
#pragma unroll
          for (int fb = 0; fb < NFB; ++fb)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
              const int f = 32 * fb + 8 * q4 + 4 * h32;
              if (f < DV)
                store4(dst + f, o[nb][fb][4 * q4] * inv, o[nb][fb][4 * q4 + 1] * inv, o[nb][fb][4 * q4 + 2] * inv,
                       o[nb][fb][4 * q4 + 3] * inv);
            }
        }
      } else if (row0 < p.R) {
        const long slot_row = (long)(2 * vw + (first_piece ? 0 : 1)) * kAttnMaxRows + wave * RW + 32 * nb + l32;
        PartT<T>* po = reinterpret_cast<PartT<T>*>(p.part_o) + slot_row * DV;
        const float inv = 1.f / l_tot;  // >= 1: the piece's first block holds a valid key
#pragma unroll
        for (int fb = 0; fb < NFB; ++fb)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const int f = 32 * fb + 8 * q4 + 4 * h32;
            if (f < DV)
              store_part4<T>(po + f, o[nb][fb][4 * q4] * inv, o[nb][fb][4 * q4 + 1] * inv, o[nb][fb][4 * q4 + 2] * inv,
                             o[nb][fb][4 * q4 + 3] * inv);
          }
        if (h32 == 0) {
          p.part_ml[slot_row * 2] = m_run[nb];
          p.part_ml[slot_row * 2 + 1] = l_tot;
        }
      }
    }
  }
}

// Merge the partial states of every row block that was split across workgroups
// (units past dp_units).  Workgroups w0..w1 (virtual indices) hold the pieces of
// row block `unit`;
// every piece is its workgroup's first (slot 2w) except possibly w0's, which is
// its second (slot 2w0+1) when w0 started inside an earlier row block.
template <typename T, int DV, int ROWS>
__global__ __launch_bounds__(256) void flash_attn_combine(FlashArgs<T> p) {
  constexpr int SLICE = 16;  // rows per workgroup: many small workgroups hide load latency
  const long unit = p.dp_units + blockIdx.x / (ROWS / SLICE);
  const int r0 = (int)(blockIdx.x % (ROWS / SLICE)) * SLICE;
  const long I = ((long)p.S * p.RB - p.dp_units) * p.KT;
  const long i0 = (unit - p.dp_units) * p.KT, i1 = i0 + p.KT;
  auto start = [&](long w) { return w * I / p.G; };
  long w0 = i0 * p.G / I;
  while (w0 + 1 < p.G && start(w0 + 1) <= i0) ++w0;
  long w1 = (i1 - 1) * p.G / I;
  while (w1 + 1 < p.G && start(w1 + 1) <= i1 - 1) ++w1;
  if (w0 == w1) return;  // one workgroup finished this row block and wrote it
  const long slot0 = 2 * w0 + (start(w0) < i0 ? 1 : 0);
  const int npieces = (int)(w1 - w0 + 1);
  const int s = (int)(unit / p.RB), rb = (int)(unit % p.RB);
  PartT<T>* out_s = static_cast<PartT<T>*>(p.out) + (s / p.heads) * p.out_so + (s % p.heads) * p.out_sh;
  constexpr int CW = sizeof(PartT<T>) == 2 ? 8 : 4;  // columns per task: one 16-byte partial load per piece
  static_assert(DV % CW == 0, "whole column groups");
  constexpr int Q = DV / CW;  // column groups per row
  for (int task = threadIdx.x; task < SLICE * Q; task += 256) {
    const int r = r0 + task / Q, f = (task % Q) * CW;
    const int row = rb * ROWS + r;
    if (row >= p.R) continue;
    float M = -__builtin_huge_valf();
    for (int k = 0; k < npieces; ++k) {
      const long sr = (k == 0 ? slot0 : 2 * (w0 + k)) * kAttnMaxRows + r;
      M = fmaxf(M, p.part_ml[sr * 2]);
    }
    float L = 0.f;
    f32x4 acc[CW / 4] = {};
    for (int k = 0; k < npieces; ++k) {
      const long sr = (k == 0 ? slot0 : 2 * (w0 + k)) * kAttnMaxRows + r;
      const float w = p.part_ml[sr * 2 + 1] * __builtin_amdgcn_exp2f(p.part_ml[sr * 2] - M);  // piece weight l 2^(m-M)
      L += w;
      const PartT<T>* src = reinterpret_cast<const PartT<T>*>(p.part_o) + sr * DV + f;
#pragma unroll
      for (int c = 0; c < CW / 4; ++c) acc[c] += w * load_part4<T>(src + 4 * c);
    }
    const float inv = 1.f / L;
#pragma unroll
    for (int c = 0; c < CW / 4; ++c)
      store4(out_s + (long)row * p.out_rs + f + 4 * c, acc[c][0] * inv, acc[c][1] * inv, acc[c][2] * inv,
             acc[c][3] * inv);
  }
}

// Fill in the tiling fields, then launch: (pre-pass,) attention, (combine).
template <typename T, int D, int DV, int KTILE, int NW, int NB, bool VROWS, bool PIPE = false>
static hipError_t launch_flash(FlashArgs<T> a, int G, hipEvent_t ev0, hipEvent_t ev1, hipStream_t s) {
  constexpr int ROWS = NW * 32 * NB;
  a.RB = (a.R + ROWS - 1) / ROWS;
  a.tiles0 = (a.len0 + KTILE - 1) / KTILE;
  a.KT = a.tiles0 + (a.len1 + KTILE - 1) / KTILE;
  const long U = (long)a.S * a.RB;
  const bool causal = a.causal_tokens > 0;
  a.G = causal ? (int)U : (int)(G < U * a.KT ? G : U * a.KT);  // block-causal: one workgroup per row block
  // With at least two units per workgroup, all but the last one to two rounds
  // of units go whole (no partial states, no combine); stream-K balances the rest.
  a.dp_units = !causal && U >= 2L * a.G ? (U / a.G - 1) * a.G : 0;
  const long I = (U - a.dp_units) * a.KT;
  if (a.row_div <= 0) a.row_div = 1;
  if constexpr (!VROWS) {
    if constexpr (sizeof(T) == 2) latent_key_tiles<T, D, KTILE, PIPE><<<dim3(a.KT, a.S), 256, 0, s>>>(a);
    else latent_value_tiles<T, D, DV, KTILE><<<dim3(a.KT, a.S), 256, 0, s>>>(a);
  }
  // The timing events (both or neither) are attached to the attention kernel's
  // own dispatch: they take its start and end time stamps, with no marker
  // packets of their own on the stream (a separate event record before and
  // after the kernel leaves a gap of several microseconds on each side).
  void* kernel;
  if constexpr (PIPE) {
    static_assert(NW == 4 && !VROWS && sizeof(T) == 2, "pipelined kernel shape");
    // three LDS stages where they fit; VGPR score accumulators where the
    // registers allow (score widths up to 128, or one row block per wave)
    constexpr int NST = 3 * KTILE * D * 2 <= 160 * 1024 ? 3 : 2;
    kernel = reinterpret_cast<void*>(&flash_attn_pipe_kernel<D, DV, KTILE, (D <= 128 || NB == 1), NB, NST>);
  } else {
    kernel = reinterpret_cast<void*>(&flash_attn_kernel<T, D, DV, KTILE, NW, NB, VROWS>);
  }
  void* args[] = {&a};
  hipError_t err = hipExtLaunchKernel(kernel, dim3(a.G), dim3(NW * 64), args, 0, s, ev0, ev1, 0);
  if (err != hipSuccess) return err;
  if (!causal && I != (long)a.G * a.KT)
    flash_attn_combine<T, DV, ROWS><<<(U - a.dp_units) * (ROWS / 16), 256, 0, s>>>(a);
  return hipGetLastError();
}

// Kernel shape per built latent (dtype, d_c, d_rope): keys per tile, waves per
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
  if (dr == 32 && dc == 96) return sh = {64, 4, 2}, true;
  if (dr == 32 && dc == 192) return sh = {64, 4, 2}, true;
  if (dr == 32 && dc == 448) return sh = {64, 4, 1}, true;
  return false;
}

bool latent_attention_supported(DType dt, int dc, int dr) {
  LatentShape sh;
  return latent_shape(dt, dc, dr, sh);
}

size_t latent_prepass_bytes(DType dt, int dc, int dr, int B, int max_ring_keys, int stage_keys) {
  LatentShape sh;
  if (!latent_shape(dt, dc, dr, sh)) return 0;
  const size_t es = dt == DType::F32 ? 4 : 2;
  const size_t dcp = (size_t)(dc + 31) / 32 * 32;
  const size_t tiles = (size_t)(max_ring_keys + sh.ktile - 1) / sh.ktile + (stage_keys + sh.ktile - 1) / sh.ktile;
  if (es == 2) return (size_t)B * tiles * sh.ktile * (size_t)(dc + dr) * 2;
  return (size_t)B * tiles * dcp * (sh.ktile + 16 / es) * es;
}

template <typename T>
static hipError_t latent_t(const AttnCall& c, hipStream_t s) {
  FlashArgs<T> a = {};
  a.q = c.qt;
  a.q_ss = (long)c.R * (c.dc + c.dr);
  a.range_flag = c.range_flag;
  a.key0 = static_cast<const T*>(c.cache);
  a.key1 = static_cast<const T*>(c.stage);
  a.key_ss0 = c.cache_bstride;
  a.key_ss1 = c.stage_bstride;
  a.val0 = c.vtiles;
  a.out = c.out;
  a.out_so = (long)c.R * c.dc;
  a.out_sh = 0;
  a.out_rs = c.dc;
  a.heads = 1;
  a.part_o = c.part_o;
  a.part_ml = c.part_ml;
  a.len0 = c.n_ring;
  a.len1 = c.n_stage;
  a.R = c.R;
  a.S = c.B;
  a.causal_tokens = c.causal_tokens;
  a.row_div = c.R / c.n_stage;  // rows are (token, head) pairs
  a.rot_ring = c.rot_ring;
  a.rot_dc = c.dc;
  a.rot_S = c.rot_S;
  a.rot_W = c.rot_W;
  a.rot_n = c.rot_n;
  a.rope.set(c.pairs_t, c.pairs_h, c.grid_w, c.tokens_per_frame, c.freq, kMaxRopePairs, c.rope_tab,
             rope_tab_stride(c.tokens_per_frame, c.grid_w));
  if constexpr (std::is_same<T, float>::value) {
    if (c.dc == 24 && c.dr == 8) return launch_flash<T, 32, 24, 64, 4, 1, false>(a, c.G, c.ev_start, c.ev_stop, s);
    return hipErrorInvalidValue;
  } else {
    if (c.dc == 24 && c.dr == 8) return launch_flash<T, 32, 24, 64, 4, 1, false>(a, c.G, c.ev_start, c.ev_stop, s);
    if (c.dr == 32) {
      if (c.dc == 96) return launch_flash<T, 128, 96, 64, 4, 2, false, true>(a, c.G, c.ev_start, c.ev_stop, s);
      if (c.dc == 192) return launch_flash<T, 224, 192, 64, 4, 2, false, true>(a, c.G, c.ev_start, c.ev_stop, s);
      if (c.dc == 448) return launch_flash<T, 480, 448, 64, 4, 1, false, true>(a, c.G, c.ev_start, c.ev_stop, s);
    }
    return hipErrorInvalidValue;
  }
}

hipError_t run_latent_attention(const AttnCall& c, hipStream_t s) {
  if (c.dtype == DType::F32) return latent_t<float>(c, s);
  return latent_t<bf16>(c, s);
}

bool dense_attention_supported(DType dt, int dh, int dv) {
  return dt == DType::BF16 && dh == 128 && dv == 128;
}

hipError_t run_dense_attention(const DenseAttnCall& c, hipStream_t s) {
  if (!dense_attention_supported(DType::BF16, c.dh, c.dv)) return hipErrorInvalidValue;
  FlashArgs<f16> a = {};
  a.q = c.q;
  a.q_ss = (long)c.Nq * c.dh;
  a.key0 = static_cast<const f16*>(c.kring);
  a.key1 = static_cast<const f16*>(c.kstage);
  a.key_ss0 = (long)c.ring_stride * c.dh;
  a.key_ss1 = (long)c.stage_stride * c.dh;
  a.val0 = c.vring;
  a.val1 = c.vstage;
  a.val_ss0 = (long)c.dv * c.ring_stride;
  a.val_ss1 = (long)c.dv * c.stage_stride;
  a.val_rs0 = c.ring_stride;
  a.val_rs1 = c.stage_stride;
  a.out = c.out;
  a.out_so = (long)c.Nq * c.H * c.dv;
  a.out_sh = c.dv;
  a.out_rs = (long)c.H * c.dv;
  a.heads = c.H;
  a.part_o = c.part_o;
  a.part_ml = c.part_ml;
  a.len0 = c.n_ring;
  a.len1 = c.Nq;
  a.R = c.Nq;
  a.S = c.B * c.H;
  return launch_flash<f16, 128, 128, kDenseKeyTile, 8, 1, true>(a, c.G, c.ev_start, c.ev_stop, s);
}

}  // namespace vmla
