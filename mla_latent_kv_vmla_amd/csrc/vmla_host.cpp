// Host runtime of libvmla.so: config validation, ring-buffer metadata,
// workspace carve-up and the C ABI declared in include/vmla.h, for the latent
// layer (vmla_*) and the dense per-head baseline (vmla_dense_*).  Every check
// runs before anything is enqueued; only the run_* pipelines touch HIP.
#include "vmla.h"

#include <hip/hip_runtime.h>
#include <math.h>
#include <mutex>
#include <new>
#include <string.h>

#include "plan.h"

using vmla::DType;
using vmla::DensePlan;
using vmla::ExpandedLayout;
using vmla::Plan;

struct vmla_ctx {
  vmla_config cfg;
  vmla_weights w;
  void* cache;
  void* workspace;
  float freq[vmla::kMaxRopePairs];
  int64_t n;  // frames appended (lockstep over the batch)
  int prepared;  // vmla_prepare has been enqueued
  // expanded latent path: buffer and frame count of the last vmla_expand
  const void* expanded;
  int64_t expanded_n;
};

struct vmla_dense_ctx {
  vmla_config cfg;
  vmla_dense_weights w;
  void* cache;
  void* workspace;
  float freq[vmla::kMaxRopePairs];
  int64_t n;
  int prepared;
};

namespace {

constexpr int kDefaultWorkgroups = 256;  // MI355X compute units

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t elem_bytes(const vmla_config* c) { return c->dtype == VMLA_DTYPE_F32 ? 4 : 2; }

constexpr long long kMaxGridY = 65535;  // launch-grid limit along y

// Checks common to both layer types.
int check_common(const vmla_config* c) {
  if (c->batch <= 0 || c->hidden <= 0 || c->n_heads <= 0 || c->d_rope <= 0 || c->d_v <= 0 ||
      c->d_nope < 0 || c->d_c < 0 || c->d_q < 0 || c->grid_h <= 0 || c->grid_w <= 0 ||
      c->window_frames <= 0 || c->chunk_frames <= 0 || c->attn_workgroups < 0 || c->sink_frames < 0)
    return VMLA_ERR_CONFIG;
  if (c->chunk_frames > c->window_frames) return VMLA_ERR_CONFIG;
  if (c->rope_at_use != 0 && c->rope_at_use != 1) return VMLA_ERR_CONFIG;
  if (c->sink_frames > 0 && !c->rope_at_use) return VMLA_ERR_CONFIG;
  if (c->rope_pairs_t < 0 || c->rope_pairs_h < 0 || c->rope_pairs_w < 0 ||
      2 * (c->rope_pairs_t + c->rope_pairs_h + c->rope_pairs_w) != c->d_rope ||
      c->d_rope / 2 > vmla::kMaxRopePairs)
    return VMLA_ERR_CONFIG;
  if (!(c->rope_theta > 0.f) || !isfinite(c->rope_theta)) return VMLA_ERR_CONFIG;
  if (c->d_nope % 8 || c->d_rope % 8 || c->d_c % 8 || c->d_v % 8 || c->d_q % 8 || c->hidden % 8)
    return VMLA_ERR_CONFIG;
  if (c->dtype != VMLA_DTYPE_BF16 && c->dtype != VMLA_DTYPE_F32) return VMLA_ERR_CONFIG;
  // sizes must fit the 32-bit row counters the kernels use
  const long long T = (long long)c->grid_h * c->grid_w;
  const long long rows = T * ((long long)c->sink_frames + c->window_frames) + T * c->chunk_frames;
  if (rows * c->n_heads > (1LL << 30) || (long long)c->batch * T * c->chunk_frames > (1LL << 30))
    return VMLA_ERR_CONFIG;
  // launch grids: streams and 64-token GEMM tiles of one call along grid y (at most 65,535)
  if (c->batch > kMaxGridY || (long long)c->batch * T * c->chunk_frames > 64LL * kMaxGridY)
    return VMLA_ERR_CONFIG;
  return VMLA_OK;
}

int check_config(const vmla_config* c) {
  if (!c) return VMLA_ERR_NULL;
  int st = check_common(c);
  if (st != VMLA_OK) return st;
  if (c->d_nope <= 0 || c->d_c <= 0 || c->d_q <= 0) return VMLA_ERR_CONFIG;
  // one stream's ring rows are addressed with 32-bit byte offsets
  const long long T = (long long)c->grid_h * c->grid_w;
  if (T * ((long long)c->sink_frames + c->window_frames) * (c->d_c + c->d_rope) * (long long)elem_bytes(c) >=
      (1LL << 31))
    return VMLA_ERR_CONFIG;
  if (!vmla::latent_attention_supported(static_cast<DType>(c->dtype), c->d_c, c->d_rope))
    return VMLA_ERR_UNSUPPORTED;
  return VMLA_OK;
}

// Keys per (stream, head) row of the dense ring: W*T padded to the key tile.
long long dense_ring_stride(const vmla_config* c) {
  const long long keys = (long long)c->grid_h * c->grid_w * c->window_frames;
  return (keys + vmla::kDenseKeyTile - 1) / vmla::kDenseKeyTile * vmla::kDenseKeyTile;
}

// Dense baseline: per-head query/key width d_rope (every channel rotated),
// value width d_v; the latent-only widths must be 0.
int check_dense_config(const vmla_config* c) {
  if (!c) return VMLA_ERR_NULL;
  int st = check_common(c);
  if (st != VMLA_OK) return st;
  if (c->d_nope != 0 || c->d_c != 0 || c->d_q != 0) return VMLA_ERR_CONFIG;
  if (c->sink_frames != 0 || c->rope_at_use != 0) return VMLA_ERR_UNSUPPORTED;
  // one (stream, head)'s keys and values are addressed with 32-bit byte offsets
  const int wmax = c->d_rope > c->d_v ? c->d_rope : c->d_v;
  if (dense_ring_stride(c) * wmax * 2 >= (1LL << 31)) return VMLA_ERR_CONFIG;
  if (!vmla::dense_attention_supported(static_cast<DType>(c->dtype), c->d_rope, c->d_v))
    return VMLA_ERR_UNSUPPORTED;
  return VMLA_OK;
}

// Default rotary table: omega_i = theta^(-2i / (2 p_a)) for i = 0..p_a-1 on each
// axis (t, h, w).
void default_freqs(const vmla_config* cfg, float* freq) {
  const int pa[3] = {cfg->rope_pairs_t, cfg->rope_pairs_h, cfg->rope_pairs_w};
  int k = 0;
  for (int a = 0; a < 3; ++a)
    for (int i = 0; i < pa[a]; ++i) freq[k++] = (float)pow((double)cfg->rope_theta, -2.0 * i / (2.0 * pa[a]));
}

// Geometry-only part of a plan (no pointers).
Plan geometry(const vmla_config* c) {
  Plan p;
  memset(&p, 0, sizeof(p));
  p.dtype = static_cast<DType>(c->dtype);
  p.B = c->batch;
  p.d = c->hidden;
  p.nh = c->n_heads;
  p.d_nope = c->d_nope;
  p.dr = c->d_rope;
  p.dv = c->d_v;
  p.dc = c->d_c;
  p.dq = c->d_q;
  p.D = c->d_c + c->d_rope;
  p.dh = c->d_nope + c->d_rope;
  p.Tpf = c->grid_h * c->grid_w;
  p.grid_w = c->grid_w;
  p.W = c->window_frames;
  p.C = c->chunk_frames;
  p.Nq = c->chunk_frames * p.Tpf;
  p.S = c->sink_frames;
  p.rope_at_use = c->rope_at_use;
  p.pairs_t = c->rope_pairs_t;
  p.pairs_h = c->rope_pairs_h;
  p.pairs_w = c->rope_pairs_w;
  p.qscale = (float)(1.4426950408889634 / sqrt((double)p.dh));
  p.G = c->attn_workgroups > 0 ? c->attn_workgroups : kDefaultWorkgroups;
  return p;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

namespace vmla {
WorkspaceLayout workspace_layout(const Plan& p) {
  const size_t es = p.dtype == DType::F32 ? 4 : 2;
  const size_t as = act_bytes(p.dtype);
  const size_t M = (size_t)p.B * p.Nq;
  WorkspaceLayout L;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += align256(bytes);
    return o;
  };
  L.flags = take(sizeof(uint32_t));
  L.rope_tab = take(rope_tab_bytes(p.dr / 2, p.Tpf, p.grid_w));
  L.wlat = take((size_t)p.D * p.d * as);
  L.wqa = take((size_t)p.nh * p.D * p.d * as);
  L.wuq = take((size_t)p.nh * p.dh * p.d * as);
  L.wuv = take((size_t)p.nh * p.dv * p.dc * as);
  L.wo = take((size_t)p.d * p.nh * p.dv * as);
  L.persistent = off;
  off = 0;
  L.stage = take(M * p.D * es);
  L.xa = take(p.dtype == DType::F32 ? 0 : M * p.d * as);
  L.ctab = take(p.dtype == DType::F32 ? 0 : (size_t)p.Nq * (p.dr / 2) * 2 * sizeof(float));
  // the per-head outputs reuse the absorbed queries' bytes: the queries are dead
  // once the attention kernel has run, before W_UV writes them
  L.qt = take(M * p.nh * (size_t)(p.D > p.dv ? p.D : p.dv) * as);
  L.o = L.qt;
  L.olat = take(M * p.nh * (size_t)p.dc * as);
  L.part_o = take((size_t)2 * p.G * kAttnMaxRows * p.dc * as);
  L.part_ml = take((size_t)2 * p.G * kAttnMaxRows * 2 * sizeof(float));
  L.vtiles = take(latent_prepass_bytes(p.dtype, p.dc, p.dr, p.B, (p.S + p.W) * p.Tpf, p.Nq));
  L.assembled = take(p.rope_at_use && p.dtype == DType::F32 ? (size_t)p.B * (p.S + p.W) * p.Tpf * p.D * es : 0);
  L.prep = 0;
  L.per_call = off > align256(prep_bytes(p)) ? off : align256(prep_bytes(p));
  L.total = L.persistent + L.per_call;
  return L;
}

DenseLayout dense_layout(const DensePlan& p, bool with_persistent) {
  DenseLayout L;
  const size_t heads = (size_t)p.B * p.nh;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += align256(bytes);
    return o;
  };
  L.kring = take(heads * p.ring_stride * p.dh * 2);
  L.vring = take(heads * p.ring_stride * p.dv * 2);
  L.cache_total = off;
  off = 0;
  L.flags = with_persistent ? take(sizeof(uint32_t)) : 0;
  L.rope_tab = with_persistent ? take(rope_tab_bytes(p.dh / 2, p.Tpf, p.grid_w)) : 0;
  L.wo = with_persistent ? take((size_t)p.d * p.nh * p.dv * 2) : 0;
  L.q = take(heads * p.Nq * p.dh * 2);
  L.kstage = take(heads * p.stage_stride * p.dh * 2);
  L.vstage = take(heads * p.stage_stride * p.dv * 2);
  L.o = take((size_t)p.B * p.Nq * p.nh * p.dv * 2);
  L.part_o = take((size_t)2 * p.G * kAttnMaxRows * p.dv * 2);
  L.part_ml = take((size_t)2 * p.G * kAttnMaxRows * 2 * sizeof(float));
  L.ws_total = off;
  return L;
}

ExpandedLayout expanded_layout(const Plan& p, DensePlan& ex) {
  memset(&ex, 0, sizeof(ex));
  ex.B = p.B;
  ex.d = p.d;
  ex.nh = p.nh;
  ex.dh = p.dh;
  ex.dv = p.dv;
  ex.Tpf = p.Tpf;
  ex.grid_w = p.grid_w;
  ex.W = p.W;
  ex.C = p.C;
  ex.Nq = p.Nq;
  ex.pairs_t = p.pairs_t;
  ex.pairs_h = p.pairs_h;
  ex.pairs_w = p.pairs_w;
  for (int i = 0; i < kMaxRopePairs; ++i) ex.freq[i] = p.freq[i];
  ex.rope_tab = p.rope_tab;
  ex.qscale = p.qscale;
  ex.G = p.G;
  ex.ring_stride = (int)(((long)(p.S + p.W) * p.Tpf + kDenseKeyTile - 1) / kDenseKeyTile * kDenseKeyTile);
  ex.stage_stride = (p.Nq + kDenseKeyTile - 1) / kDenseKeyTile * kDenseKeyTile;
  ExpandedLayout L;
  L.dense = dense_layout(ex, false);
  L.wext = L.dense.cache_total + L.dense.ws_total;
  L.total = L.wext + align256((size_t)p.nh * p.dh * p.D * 2);
  return L;
}
}  // namespace vmla

namespace {
DensePlan dense_geometry(const vmla_config* c) {
  DensePlan p;
  memset(&p, 0, sizeof(p));
  p.B = c->batch;
  p.d = c->hidden;
  p.nh = c->n_heads;
  p.dh = c->d_rope;
  p.dv = c->d_v;
  p.Tpf = c->grid_h * c->grid_w;
  p.grid_w = c->grid_w;
  p.W = c->window_frames;
  p.C = c->chunk_frames;
  p.Nq = c->chunk_frames * p.Tpf;
  p.pairs_t = c->rope_pairs_t;
  p.pairs_h = c->rope_pairs_h;
  p.pairs_w = c->rope_pairs_w;
  p.qscale = (float)(1.4426950408889634 / sqrt((double)p.dh));
  p.G = c->attn_workgroups > 0 ? c->attn_workgroups : kDefaultWorkgroups;
  p.ring_stride = (int)dense_ring_stride(c);
  p.stage_stride = (p.Nq + vmla::kDenseKeyTile - 1) / vmla::kDenseKeyTile * vmla::kDenseKeyTile;
  return p;
}
}  // namespace

extern "C" {

VMLA_API size_t vmla_cache_bytes(const vmla_config* cfg) {
  if (check_config(cfg) != VMLA_OK) return 0;
  return (size_t)cfg->batch * (cfg->sink_frames + cfg->window_frames) * cfg->grid_h * cfg->grid_w *
         (size_t)(cfg->d_c + cfg->d_rope) * elem_bytes(cfg);
}

VMLA_API size_t vmla_workspace_bytes(const vmla_config* cfg) {
  if (check_config(cfg) != VMLA_OK) return 0;
  return vmla::workspace_layout(geometry(cfg)).total;
}

VMLA_API int vmla_create(const vmla_config* cfg, const vmla_weights* w, void* cache, void* workspace,
                         const float* rope_freqs, vmla_ctx** out) {
  if (!out) return VMLA_ERR_NULL;
  *out = nullptr;
  int st = check_config(cfg);
  if (st != VMLA_OK) return st;
  if (!w || !cache || !workspace) return VMLA_ERR_NULL;
  const void* ptrs[] = {w->w_dkv, w->w_kr, w->w_dq, w->w_uq, w->w_uk, w->w_uv, w->w_o};
  for (const void* q : ptrs)
    if (!q) return VMLA_ERR_NULL;
  for (const void* q : ptrs)
    if (!aligned16(q)) return VMLA_ERR_ALIGN;
  if (!aligned16(cache) || !aligned16(workspace)) return VMLA_ERR_ALIGN;
  const int npairs = cfg->d_rope / 2;
  if (rope_freqs)
    for (int i = 0; i < npairs; ++i)
      if (!isfinite(rope_freqs[i])) return VMLA_ERR_ARG;

  vmla_ctx* c = new (std::nothrow) vmla_ctx;
  if (!c) return VMLA_ERR_STATE;
  memset(c, 0, sizeof(*c));
  c->cfg = *cfg;
  c->w = *w;
  c->cache = cache;
  c->workspace = workspace;
  c->n = 0;
  c->expanded = nullptr;
  c->expanded_n = -1;
  if (rope_freqs) {
    for (int i = 0; i < npairs; ++i) c->freq[i] = rope_freqs[i];
  } else {
    default_freqs(cfg, c->freq);
  }
  *out = c;
  return VMLA_OK;
}

// Point a plan's per-call regions at `base` (laid out by L).
static void set_per_call(Plan& p, const vmla::WorkspaceLayout& L, void* base) {
  char* ws = static_cast<char*>(base);
  p.stage = ws + L.stage;
  p.xa = ws + L.xa;
  p.ctab = ws + L.ctab;
  p.qt = ws + L.qt;
  p.olat = ws + L.olat;
  p.o = ws + L.o;
  p.part_o = reinterpret_cast<float*>(ws + L.part_o);
  p.part_ml = reinterpret_cast<float*>(ws + L.part_ml);
  p.vtiles = ws + L.vtiles;
  p.assembled = ws + L.assembled;
  p.prep = ws + L.prep;
}

// Weights, cache and the persistent workspace of a ctx on top of plan p's
// geometry (a chunk call's, or a clip's).
static void set_ctx_pointers(Plan& p, const vmla_ctx* c) {
  for (int i = 0; i < vmla::kMaxRopePairs; ++i) p.freq[i] = c->freq[i];
  p.w_dkv = c->w.w_dkv;
  p.w_kr = c->w.w_kr;
  p.w_dq = c->w.w_dq;
  p.w_uq = c->w.w_uq;
  p.w_uk = c->w.w_uk;
  p.w_uv = c->w.w_uv;
  p.w_o = c->w.w_o;
  p.cache = c->cache;
  const vmla::WorkspaceLayout L = vmla::workspace_layout(geometry(&c->cfg));
  char* ws = static_cast<char*>(c->workspace);
  p.flags = reinterpret_cast<uint32_t*>(ws + L.flags);
  p.rope_tab = reinterpret_cast<float*>(ws + L.rope_tab);
  p.wlat = ws + L.wlat;
  p.wqa = ws + L.wqa;
  p.wuq = ws + L.wuq;
  p.wuv = ws + L.wuv;
  p.wo = ws + L.wo;
}

static Plan make_plan(const vmla_ctx* c) {
  Plan p = geometry(&c->cfg);
  set_ctx_pointers(p, c);
  const vmla::WorkspaceLayout L = vmla::workspace_layout(p);
  set_per_call(p, L, static_cast<char*>(c->workspace) + L.persistent);
  return p;
}

VMLA_API int vmla_prepare(vmla_ctx* ctx, hipStream_t stream) {
  if (!ctx) return VMLA_ERR_NULL;
  if (vmla::run_prepare(make_plan(ctx), stream) != hipSuccess) return VMLA_ERR_HIP;
  ctx->prepared = 1;
  return VMLA_OK;
}

VMLA_API int vmla_range_flags(vmla_ctx* ctx, uint32_t* flags, hipStream_t stream) {
  if (!ctx || !flags) return VMLA_ERR_NULL;
  if (!ctx->prepared) return VMLA_ERR_STATE;
  uint32_t* dev = make_plan(ctx).flags;
  uint32_t v = 0;
  if (hipMemcpyAsync(&v, dev, sizeof(v), hipMemcpyDeviceToHost, stream) != hipSuccess) return VMLA_ERR_HIP;
  if (hipStreamSynchronize(stream) != hipSuccess) return VMLA_ERR_HIP;
  if (vmla::run_clear_flags(dev, stream) != hipSuccess) return VMLA_ERR_HIP;
  *flags = v;
  return VMLA_OK;
}

VMLA_API int vmla_compress_append(vmla_ctx* ctx, const void* x, hipStream_t stream) {
  if (!ctx || !x) return VMLA_ERR_NULL;
  if (!aligned16(x)) return VMLA_ERR_ALIGN;
  if (ctx->n > INT64_MAX / 2) return VMLA_ERR_STATE;
  Plan p = make_plan(ctx);
  if (vmla::run_compress(p, x, ctx->n, ctx->cache, true, stream) != hipSuccess) return VMLA_ERR_HIP;
  ctx->n += ctx->cfg.chunk_frames;
  return VMLA_OK;
}

VMLA_API int vmla_attend(vmla_ctx* ctx, const void* x, void* out, hipStream_t stream) {
  if (!ctx || !x || !out) return VMLA_ERR_NULL;
  if (!aligned16(x) || !aligned16(out)) return VMLA_ERR_ALIGN;
  if (!ctx->prepared) return VMLA_ERR_STATE;
  Plan p = make_plan(ctx);
  if (vmla::run_attend(p, ctx->n, x, out, stream) != hipSuccess) return VMLA_ERR_HIP;
  return VMLA_OK;
}

VMLA_API int vmla_attend_profiled(vmla_ctx* ctx, const void* x, void* out, hipEvent_t attn_start,
                                  hipEvent_t attn_stop, hipStream_t stream) {
  if (!ctx || !x || !out || !attn_start || !attn_stop) return VMLA_ERR_NULL;
  if (!aligned16(x) || !aligned16(out)) return VMLA_ERR_ALIGN;
  if (!ctx->prepared) return VMLA_ERR_STATE;
  Plan p = make_plan(ctx);
  if (vmla::run_attend(p, ctx->n, x, out, stream, attn_start, attn_stop) != hipSuccess) return VMLA_ERR_HIP;
  return VMLA_OK;
}

/* ------------------------------------------------------- allocation-free attend */

// Per-call buffers of vmla_attend_noalloc: one array per GPU, in the library's
// device code, allocated when the code object is loaded on that GPU and held
// until the process ends.  Its name is only a host-side stand-in for the
// symbol: host code uses the address hipGetSymbolAddress reports per device.
static __device__ __align__(256) unsigned char scratch[VMLA_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device, set on first use

// Device address of the current device's scratch array (nullptr on failure).
void* device_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}
}  // namespace

VMLA_API int vmla_attend_noalloc(vmla_ctx* ctx, const void* x, void* out, hipStream_t stream) {
  if (!ctx || !x || !out) return VMLA_ERR_NULL;
  if (!aligned16(x) || !aligned16(out)) return VMLA_ERR_ALIGN;
  if (!ctx->prepared) return VMLA_ERR_STATE;
  Plan p = geometry(&ctx->cfg);
  set_ctx_pointers(p, ctx);
  const vmla::WorkspaceLayout L = vmla::workspace_layout(p);
  if (L.per_call > VMLA_SCRATCH_BYTES) return VMLA_ERR_SCRATCH;
  void* base = device_scratch();
  if (!base) return VMLA_ERR_HIP;
  set_per_call(p, L, base);
  if (vmla::run_attend(p, ctx->n, x, out, stream) != hipSuccess) return VMLA_ERR_HIP;
  return VMLA_OK;
}

VMLA_API int vmla_compress(vmla_ctx* ctx, const void* x, int64_t frame0, void* latents_out,
                           hipStream_t stream) {
  if (!ctx || !x || !latents_out) return VMLA_ERR_NULL;
  if (!aligned16(x) || !aligned16(latents_out)) return VMLA_ERR_ALIGN;
  if (frame0 < 0 || frame0 > INT64_MAX / 2) return VMLA_ERR_ARG;
  Plan p = make_plan(ctx);
  if (vmla::run_compress(p, x, frame0, latents_out, false, stream) != hipSuccess) return VMLA_ERR_HIP;
  return VMLA_OK;
}

VMLA_API int vmla_cache_state(const vmla_ctx* ctx, int64_t* frames_appended, int64_t* first_valid_frame,
                              int32_t* n_valid_frames) {
  if (!ctx) return VMLA_ERR_NULL;
  const int64_t W = ctx->cfg.window_frames, S = ctx->cfg.sink_frames, n = ctx->n;
  const int64_t first_window = n - W > S ? n - W : S;
  if (frames_appended) *frames_appended = n;
  if (first_valid_frame) *first_valid_frame = first_window < n ? first_window : n;
  if (n_valid_frames) *n_valid_frames = (int32_t)vmla::cached_frames(geometry(&ctx->cfg), n);
  return VMLA_OK;
}

VMLA_API int vmla_reset(vmla_ctx* ctx) {
  if (!ctx) return VMLA_ERR_NULL;
  ctx->n = 0;
  ctx->expanded = nullptr;
  ctx->expanded_n = -1;
  return VMLA_OK;
}

/* ------------------------------------------------------- block-causal clip */

// Plan of a whole clip of window_frames frames: W*T query tokens, no ring,
// block-causal in chunk_frames*T token blocks.
static Plan clip_geometry(const vmla_config* cfg) {
  Plan p = geometry(cfg);
  p.causal_tokens = p.C * p.Tpf;
  p.C = p.W;
  p.Nq = p.W * p.Tpf;
  return p;
}

// A clip call runs window_frames*T query tokens per stream: the same launch-grid
// limit as a chunk call, for that token count.
static bool clip_fits(const vmla_config* cfg) {
  return (long long)cfg->batch * cfg->window_frames * cfg->grid_h * cfg->grid_w <= 64LL * kMaxGridY;
}

VMLA_API size_t vmla_clip_workspace_bytes(const vmla_config* cfg) {
  if (check_config(cfg) != VMLA_OK || !clip_fits(cfg)) return 0;
  return vmla::workspace_layout(clip_geometry(cfg)).per_call;
}

static int attend_clip(vmla_ctx* ctx, const void* x, void* clip_workspace, void* out, hipEvent_t e0, hipEvent_t e1,
                       hipStream_t stream) {
  if (!clip_fits(&ctx->cfg)) return VMLA_ERR_CONFIG;
  if (!aligned16(x) || !aligned16(clip_workspace) || !aligned16(out)) return VMLA_ERR_ALIGN;
  if (!ctx->prepared) return VMLA_ERR_STATE;
  Plan p = clip_geometry(&ctx->cfg);
  set_ctx_pointers(p, ctx);
  set_per_call(p, vmla::workspace_layout(p), clip_workspace);
  // the clip's frames are 0..W-1 and nothing is cached: attend at n = 0
  if (vmla::run_attend(p, 0, x, out, stream, e0, e1) != hipSuccess) return VMLA_ERR_HIP;
  return VMLA_OK;
}

VMLA_API int vmla_attend_clip(vmla_ctx* ctx, const void* x, void* clip_workspace, void* out, hipStream_t stream) {
  if (!ctx || !x || !clip_workspace || !out) return VMLA_ERR_NULL;
  return attend_clip(ctx, x, clip_workspace, out, nullptr, nullptr, stream);
}

VMLA_API int vmla_attend_clip_profiled(vmla_ctx* ctx, const void* x, void* clip_workspace, void* out,
                                       hipEvent_t attn_start, hipEvent_t attn_stop, hipStream_t stream) {
  if (!ctx || !x || !clip_workspace || !out || !attn_start || !attn_stop) return VMLA_ERR_NULL;
  return attend_clip(ctx, x, clip_workspace, out, attn_start, attn_stop, stream);
}

/* ------------------------------------------------------- expanded latent path */

static bool expanded_ok(const vmla_config* cfg) {
  return check_config(cfg) == VMLA_OK && vmla::expanded_supported(geometry(cfg));
}

VMLA_API size_t vmla_expanded_bytes(const vmla_config* cfg) {
  if (!expanded_ok(cfg)) return 0;
  DensePlan ex;
  return vmla::expanded_layout(geometry(cfg), ex).total;
}

// Expanded-buffer view of a ctx: dense regions and the key lift.
static DensePlan make_expanded_plan(const Plan& p, void* buf, void** wext) {
  DensePlan ex;
  const vmla::ExpandedLayout L = vmla::expanded_layout(p, ex);
  char* b = static_cast<char*>(buf);
  char* ws = b + L.dense.cache_total;
  ex.kring = b + L.dense.kring;
  ex.vring = b + L.dense.vring;
  ex.q = ws + L.dense.q;
  ex.kstage = ws + L.dense.kstage;
  ex.vstage = ws + L.dense.vstage;
  ex.o = ws + L.dense.o;
  ex.part_o = reinterpret_cast<float*>(ws + L.dense.part_o);
  ex.part_ml = reinterpret_cast<float*>(ws + L.dense.part_ml);
  ex.flags = p.flags;  // the latent ctx's range flag and fp16 W_O
  ex.wo = p.wo;
  *wext = b + L.wext;
  return ex;
}

VMLA_API int vmla_expand(vmla_ctx* ctx, void* expanded, hipStream_t stream) {
  if (!ctx || !expanded) return VMLA_ERR_NULL;
  if (!aligned16(expanded)) return VMLA_ERR_ALIGN;
  if (!expanded_ok(&ctx->cfg)) return VMLA_ERR_UNSUPPORTED;
  if (!ctx->prepared) return VMLA_ERR_STATE;
  Plan p = make_plan(ctx);
  void* wext;
  DensePlan ex = make_expanded_plan(p, expanded, &wext);
  if (vmla::run_expand(p, ex, wext, ctx->n, stream) != hipSuccess) return VMLA_ERR_HIP;
  ctx->expanded = expanded;
  ctx->expanded_n = ctx->n;
  return VMLA_OK;
}

static int attend_expanded(vmla_ctx* ctx, const void* expanded, const void* x, void* out, hipEvent_t e0,
                           hipEvent_t e1, hipStream_t stream) {
  if (!aligned16(expanded) || !aligned16(x) || !aligned16(out)) return VMLA_ERR_ALIGN;
  if (!expanded_ok(&ctx->cfg)) return VMLA_ERR_UNSUPPORTED;
  if (!ctx->prepared) return VMLA_ERR_STATE;
  if (ctx->expanded != expanded || ctx->expanded_n != ctx->n) return VMLA_ERR_STATE;
  Plan p = make_plan(ctx);
  void* wext;
  DensePlan ex = make_expanded_plan(p, const_cast<void*>(expanded), &wext);
  if (vmla::run_attend_expanded(p, ex, wext, ctx->n, x, out, stream, e0, e1) != hipSuccess) return VMLA_ERR_HIP;
  return VMLA_OK;
}

VMLA_API int vmla_attend_expanded(vmla_ctx* ctx, const void* expanded, const void* x, void* out,
                                  hipStream_t stream) {
  if (!ctx || !expanded || !x || !out) return VMLA_ERR_NULL;
  return attend_expanded(ctx, expanded, x, out, nullptr, nullptr, stream);
}

VMLA_API int vmla_attend_expanded_profiled(vmla_ctx* ctx, const void* expanded, const void* x, void* out,
                                           hipEvent_t attn_start, hipEvent_t attn_stop, hipStream_t stream) {
  if (!ctx || !expanded || !x || !out || !attn_start || !attn_stop) return VMLA_ERR_NULL;
  return attend_expanded(ctx, expanded, x, out, attn_start, attn_stop, stream);
}

VMLA_API void vmla_destroy(vmla_ctx* ctx) { delete ctx; }

/* ------------------------------------------------------------ dense baseline */

VMLA_API size_t vmla_dense_cache_bytes(const vmla_config* cfg) {
  if (check_dense_config(cfg) != VMLA_OK) return 0;
  return vmla::dense_layout(dense_geometry(cfg)).cache_total;
}

VMLA_API size_t vmla_dense_workspace_bytes(const vmla_config* cfg) {
  if (check_dense_config(cfg) != VMLA_OK) return 0;
  return vmla::dense_layout(dense_geometry(cfg)).ws_total;
}

VMLA_API int vmla_dense_create(const vmla_config* cfg, const vmla_dense_weights* w, void* cache,
                               void* workspace, const float* rope_freqs, vmla_dense_ctx** out) {
  if (!out) return VMLA_ERR_NULL;
  *out = nullptr;
  int st = check_dense_config(cfg);
  if (st != VMLA_OK) return st;
  if (!w || !cache || !workspace) return VMLA_ERR_NULL;
  const void* ptrs[] = {w->w_q, w->w_k, w->w_v, w->w_o};
  for (const void* q : ptrs)
    if (!q) return VMLA_ERR_NULL;
  for (const void* q : ptrs)
    if (!aligned16(q)) return VMLA_ERR_ALIGN;
  if (!aligned16(cache) || !aligned16(workspace)) return VMLA_ERR_ALIGN;
  const int npairs = cfg->d_rope / 2;
  if (rope_freqs)
    for (int i = 0; i < npairs; ++i)
      if (!isfinite(rope_freqs[i])) return VMLA_ERR_ARG;
  vmla_dense_ctx* c = new (std::nothrow) vmla_dense_ctx;
  if (!c) return VMLA_ERR_STATE;
  memset(c, 0, sizeof(*c));
  c->cfg = *cfg;
  c->w = *w;
  c->cache = cache;
  c->workspace = workspace;
  c->n = 0;
  if (rope_freqs) {
    for (int i = 0; i < npairs; ++i) c->freq[i] = rope_freqs[i];
  } else {
    default_freqs(cfg, c->freq);
  }
  *out = c;
  return VMLA_OK;
}

static DensePlan make_dense_plan(const vmla_dense_ctx* c) {
  DensePlan p = dense_geometry(&c->cfg);
  for (int i = 0; i < vmla::kMaxRopePairs; ++i) p.freq[i] = c->freq[i];
  p.w_q = c->w.w_q;
  p.w_k = c->w.w_k;
  p.w_v = c->w.w_v;
  p.w_o = c->w.w_o;
  const vmla::DenseLayout L = vmla::dense_layout(p);
  char* cache = static_cast<char*>(c->cache);
  char* ws = static_cast<char*>(c->workspace);
  p.kring = cache + L.kring;
  p.vring = cache + L.vring;
  p.flags = reinterpret_cast<uint32_t*>(ws + L.flags);
  p.rope_tab = reinterpret_cast<float*>(ws + L.rope_tab);
  p.wo = ws + L.wo;
  p.q = ws + L.q;
  p.kstage = ws + L.kstage;
  p.vstage = ws + L.vstage;
  p.o = ws + L.o;
  p.part_o = reinterpret_cast<float*>(ws + L.part_o);
  p.part_ml = reinterpret_cast<float*>(ws + L.part_ml);
  return p;
}

VMLA_API int vmla_dense_prepare(vmla_dense_ctx* ctx, hipStream_t stream) {
  if (!ctx) return VMLA_ERR_NULL;
  if (vmla::run_dense_prepare(make_dense_plan(ctx), stream) != hipSuccess) return VMLA_ERR_HIP;
  ctx->prepared = 1;
  return VMLA_OK;
}

VMLA_API int vmla_dense_range_flags(vmla_dense_ctx* ctx, uint32_t* flags, hipStream_t stream) {
  if (!ctx || !flags) return VMLA_ERR_NULL;
  if (!ctx->prepared) return VMLA_ERR_STATE;
  uint32_t* dev = make_dense_plan(ctx).flags;
  uint32_t v = 0;
  if (hipMemcpyAsync(&v, dev, sizeof(v), hipMemcpyDeviceToHost, stream) != hipSuccess) return VMLA_ERR_HIP;
  if (hipStreamSynchronize(stream) != hipSuccess) return VMLA_ERR_HIP;
  if (vmla::run_clear_flags(dev, stream) != hipSuccess) return VMLA_ERR_HIP;
  *flags = v;
  return VMLA_OK;
}

VMLA_API int vmla_dense_append(vmla_dense_ctx* ctx, const void* x, hipStream_t stream) {
  if (!ctx || !x) return VMLA_ERR_NULL;
  if (!aligned16(x)) return VMLA_ERR_ALIGN;
  if (ctx->n > INT64_MAX / 2) return VMLA_ERR_STATE;
  if (!ctx->prepared) return VMLA_ERR_STATE;
  if (vmla::run_dense_append(make_dense_plan(ctx), ctx->n, x, stream) != hipSuccess) return VMLA_ERR_HIP;
  ctx->n += ctx->cfg.chunk_frames;
  return VMLA_OK;
}

VMLA_API int vmla_dense_attend(vmla_dense_ctx* ctx, const void* x, void* out, hipStream_t stream) {
  if (!ctx || !x || !out) return VMLA_ERR_NULL;
  if (!aligned16(x) || !aligned16(out)) return VMLA_ERR_ALIGN;
  if (!ctx->prepared) return VMLA_ERR_STATE;
  if (vmla::run_dense_attend(make_dense_plan(ctx), ctx->n, x, out, stream) != hipSuccess) return VMLA_ERR_HIP;
  return VMLA_OK;
}

VMLA_API int vmla_dense_attend_profiled(vmla_dense_ctx* ctx, const void* x, void* out, hipEvent_t attn_start,
                                        hipEvent_t attn_stop, hipStream_t stream) {
  if (!ctx || !x || !out || !attn_start || !attn_stop) return VMLA_ERR_NULL;
  if (!aligned16(x) || !aligned16(out)) return VMLA_ERR_ALIGN;
  if (!ctx->prepared) return VMLA_ERR_STATE;
  if (vmla::run_dense_attend(make_dense_plan(ctx), ctx->n, x, out, stream, attn_start, attn_stop) != hipSuccess)
    return VMLA_ERR_HIP;
  return VMLA_OK;
}

VMLA_API int vmla_dense_cache_state(const vmla_dense_ctx* ctx, int64_t* frames_appended,
                                    int64_t* first_valid_frame, int32_t* n_valid_frames) {
  if (!ctx) return VMLA_ERR_NULL;
  const int64_t W = ctx->cfg.window_frames;
  if (frames_appended) *frames_appended = ctx->n;
  if (first_valid_frame) *first_valid_frame = ctx->n > W ? ctx->n - W : 0;
  if (n_valid_frames) *n_valid_frames = (int32_t)(ctx->n < W ? ctx->n : W);
  return VMLA_OK;
}

VMLA_API int vmla_dense_reset(vmla_dense_ctx* ctx) {
  if (!ctx) return VMLA_ERR_NULL;
  ctx->n = 0;
  return VMLA_OK;
}

VMLA_API void vmla_dense_destroy(vmla_dense_ctx* ctx) { delete ctx; }

VMLA_API const char* vmla_status_string(int status) {
  switch (status) {
    case VMLA_OK: return "ok";
    case VMLA_ERR_NULL: return "required pointer is NULL";
    case VMLA_ERR_CONFIG: return "invalid configuration";
    case VMLA_ERR_UNSUPPORTED: return "no kernel built for this (dtype, widths)";
    case VMLA_ERR_ALIGN: return "device pointer not 16-byte aligned";
    case VMLA_ERR_STATE: return "call not valid in the current state";
    case VMLA_ERR_ARG: return "argument out of range";
    case VMLA_ERR_HIP: return "HIP runtime error on launch";
    case VMLA_ERR_SCRATCH: return "per-call buffers exceed the library's scratch array (VMLA_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

}  // extern "C"
