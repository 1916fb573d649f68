"""ctypes binding of libvmla.so (C ABI in include/vmla.h).

The functions below carry the C names and marshal arguments only: every step
of the computation runs in the HIP library.  Device memory comes from torch
(plumbing); the library borrows it.  If the library is missing this module
raises on first use -- there is no fallback path.

`LatentAttention` (and `DenseAttention` for the dense per-head baseline) is a
convenience owner of one layer's device tensors (weights, ring cache,
workspace) that calls the same entry points.
"""
from __future__ import annotations

import ctypes
import os
import re
from ctypes import POINTER, byref, c_char_p, c_float, c_int, c_int32, c_int64, c_size_t, c_uint32, c_void_p

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libvmla.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "vmla.h")

VMLA_DTYPE_BF16, VMLA_DTYPE_F32 = 0, 1


def _status_codes() -> dict:
    """Status names and values as declared in the header."""
    txt = open(HEADER_PATH).read()
    return {k: int(v) for k, v in re.findall(r"(VMLA_(?:OK|ERR_\w+))\s*=\s*(\d+)", txt)}


STATUS = _status_codes()


class vmla_config(ctypes.Structure):
    _fields_ = [("batch", c_int32), ("hidden", c_int32), ("n_heads", c_int32), ("d_nope", c_int32),
                ("d_rope", c_int32), ("d_v", c_int32), ("d_c", c_int32), ("d_q", c_int32),
                ("rope_pairs_t", c_int32), ("rope_pairs_h", c_int32), ("rope_pairs_w", c_int32),
                ("rope_theta", c_float), ("grid_h", c_int32), ("grid_w", c_int32),
                ("window_frames", c_int32), ("chunk_frames", c_int32), ("dtype", c_int32),
                ("attn_workgroups", c_int32), ("sink_frames", c_int32), ("rope_at_use", c_int32)]


class vmla_weights(ctypes.Structure):
    _fields_ = [(n, c_void_p) for n in ("w_dkv", "w_kr", "w_dq", "w_uq", "w_uk", "w_uv", "w_o")]


class vmla_dense_weights(ctypes.Structure):
    _fields_ = [(n, c_void_p) for n in ("w_q", "w_k", "w_v", "w_o")]


class VmlaError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: status {code} ({vmla_status_string(code)})")


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing; build it with `python -m mla_latent_kv_vmla_amd.build`")
        try:  # bind to the HIP runtime torch already carries (one runtime per process)
            import torch  # noqa: F401
        except ImportError:
            pass
        L = ctypes.CDLL(LIB_PATH)
        L.vmla_cache_bytes.argtypes = [POINTER(vmla_config)]
        L.vmla_cache_bytes.restype = c_size_t
        L.vmla_workspace_bytes.argtypes = [POINTER(vmla_config)]
        L.vmla_workspace_bytes.restype = c_size_t
        L.vmla_create.argtypes = [POINTER(vmla_config), POINTER(vmla_weights), c_void_p, c_void_p,
                                  POINTER(c_float), POINTER(c_void_p)]
        L.vmla_create.restype = c_int
        L.vmla_prepare.argtypes = [c_void_p, c_void_p]
        L.vmla_prepare.restype = c_int
        L.vmla_range_flags.argtypes = [c_void_p, POINTER(c_uint32), c_void_p]
        L.vmla_range_flags.restype = c_int
        L.vmla_compress_append.argtypes = [c_void_p, c_void_p, c_void_p]
        L.vmla_compress_append.restype = c_int
        L.vmla_attend.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p]
        L.vmla_attend.restype = c_int
        L.vmla_attend_noalloc.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p]
        L.vmla_attend_noalloc.restype = c_int
        L.vmla_attend_profiled.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]
        L.vmla_attend_profiled.restype = c_int
        L.vmla_compress.argtypes = [c_void_p, c_void_p, c_int64, c_void_p, c_void_p]
        L.vmla_compress.restype = c_int
        L.vmla_cache_state.argtypes = [c_void_p, POINTER(c_int64), POINTER(c_int64), POINTER(c_int32)]
        L.vmla_cache_state.restype = c_int
        L.vmla_reset.argtypes = [c_void_p]
        L.vmla_reset.restype = c_int
        L.vmla_destroy.argtypes = [c_void_p]
        L.vmla_destroy.restype = None
        L.vmla_clip_workspace_bytes.argtypes = [POINTER(vmla_config)]
        L.vmla_clip_workspace_bytes.restype = c_size_t
        L.vmla_attend_clip.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]
        L.vmla_attend_clip.restype = c_int
        L.vmla_attend_clip_profiled.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                                c_void_p]
        L.vmla_attend_clip_profiled.restype = c_int
        L.vmla_expanded_bytes.argtypes = [POINTER(vmla_config)]
        L.vmla_expanded_bytes.restype = c_size_t
        L.vmla_expand.argtypes = [c_void_p, c_void_p, c_void_p]
        L.vmla_expand.restype = c_int
        L.vmla_attend_expanded.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]
        L.vmla_attend_expanded.restype = c_int
        L.vmla_attend_expanded_profiled.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                                    c_void_p]
        L.vmla_attend_expanded_profiled.restype = c_int
        L.vmla_dense_cache_bytes.argtypes = [POINTER(vmla_config)]
        L.vmla_dense_cache_bytes.restype = c_size_t
        L.vmla_dense_workspace_bytes.argtypes = [POINTER(vmla_config)]
        L.vmla_dense_workspace_bytes.restype = c_size_t
        L.vmla_dense_create.argtypes = [POINTER(vmla_config), POINTER(vmla_dense_weights), c_void_p, c_void_p,
                                        POINTER(c_float), POINTER(c_void_p)]
        L.vmla_dense_create.restype = c_int
        L.vmla_dense_prepare.argtypes = [c_void_p, c_void_p]
        L.vmla_dense_prepare.restype = c_int
        L.vmla_dense_range_flags.argtypes = [c_void_p, POINTER(c_uint32), c_void_p]
        L.vmla_dense_range_flags.restype = c_int
        L.vmla_dense_append.argtypes = [c_void_p, c_void_p, c_void_p]
        L.vmla_dense_append.restype = c_int
        L.vmla_dense_attend.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p]
        L.vmla_dense_attend.restype = c_int
        L.vmla_dense_attend_profiled.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]
        L.vmla_dense_attend_profiled.restype = c_int
        L.vmla_dense_cache_state.argtypes = [c_void_p, POINTER(c_int64), POINTER(c_int64), POINTER(c_int32)]
        L.vmla_dense_cache_state.restype = c_int
        L.vmla_dense_reset.argtypes = [c_void_p]
        L.vmla_dense_reset.restype = c_int
        L.vmla_dense_destroy.argtypes = [c_void_p]
        L.vmla_dense_destroy.restype = None
        L.vmla_status_string.argtypes = [c_int]
        L.vmla_status_string.restype = c_char_p
        _lib = L
    return _lib


def _check(code: int, where: str):
    if code != 0:
        raise VmlaError(code, where)


def _ptr(t) -> int:
    """Device address of a tensor (or an int address passed through)."""
    if t is None:
        return 0
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(s) -> int:
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


# ----------------------------------------------------------------------------- C entry points
def vmla_cache_bytes(cfg: vmla_config) -> int:
    return lib().vmla_cache_bytes(byref(cfg))


def vmla_workspace_bytes(cfg: vmla_config) -> int:
    return lib().vmla_workspace_bytes(byref(cfg))


def vmla_create(cfg: vmla_config, weights: vmla_weights, cache, workspace, rope_freqs=None) -> c_void_p:
    ctx = c_void_p()
    _check(lib().vmla_create(byref(cfg), byref(weights), _ptr(cache), _ptr(workspace), _freq_array(rope_freqs),
                             byref(ctx)), "vmla_create")
    return ctx


def vmla_prepare(ctx, stream=None) -> None:
    _check(lib().vmla_prepare(ctx, _stream(stream)), "vmla_prepare")


def vmla_range_flags(ctx, stream=None) -> int:
    v = c_uint32()
    _check(lib().vmla_range_flags(ctx, byref(v), _stream(stream)), "vmla_range_flags")
    return v.value


def vmla_compress_append(ctx, x, stream=None) -> None:
    _check(lib().vmla_compress_append(ctx, _ptr(x), _stream(stream)), "vmla_compress_append")


def vmla_attend(ctx, x, out, stream=None) -> None:
    _check(lib().vmla_attend(ctx, _ptr(x), _ptr(out), _stream(stream)), "vmla_attend")


def vmla_attend_noalloc(ctx, x, out, stream=None) -> None:
    _check(lib().vmla_attend_noalloc(ctx, _ptr(x), _ptr(out), _stream(stream)), "vmla_attend_noalloc")


def vmla_attend_profiled(ctx, x, out, attn_start: int, attn_stop: int, stream=None) -> None:
    _check(lib().vmla_attend_profiled(ctx, _ptr(x), _ptr(out), attn_start, attn_stop, _stream(stream)),
           "vmla_attend_profiled")


def vmla_compress(ctx, x, frame0: int, latents_out, stream=None) -> None:
    _check(lib().vmla_compress(ctx, _ptr(x), int(frame0), _ptr(latents_out), _stream(stream)), "vmla_compress")


def vmla_cache_state(ctx):
    n, first, nv = c_int64(), c_int64(), c_int32()
    _check(lib().vmla_cache_state(ctx, byref(n), byref(first), byref(nv)), "vmla_cache_state")
    return n.value, first.value, nv.value


def vmla_reset(ctx) -> None:
    _check(lib().vmla_reset(ctx), "vmla_reset")


def vmla_destroy(ctx) -> None:
    lib().vmla_destroy(ctx)


def vmla_clip_workspace_bytes(cfg: vmla_config) -> int:
    return lib().vmla_clip_workspace_bytes(byref(cfg))


def vmla_attend_clip(ctx, x, clip_workspace, out, stream=None) -> None:
    _check(lib().vmla_attend_clip(ctx, _ptr(x), _ptr(clip_workspace), _ptr(out), _stream(stream)),
           "vmla_attend_clip")


def vmla_attend_clip_profiled(ctx, x, clip_workspace, out, attn_start: int, attn_stop: int, stream=None) -> None:
    _check(lib().vmla_attend_clip_profiled(ctx, _ptr(x), _ptr(clip_workspace), _ptr(out), attn_start, attn_stop,
                                           _stream(stream)), "vmla_attend_clip_profiled")


def vmla_expanded_bytes(cfg: vmla_config) -> int:
    return lib().vmla_expanded_bytes(byref(cfg))


def vmla_expand(ctx, expanded, stream=None) -> None:
    _check(lib().vmla_expand(ctx, _ptr(expanded), _stream(stream)), "vmla_expand")


def vmla_attend_expanded(ctx, expanded, x, out, stream=None) -> None:
    _check(lib().vmla_attend_expanded(ctx, _ptr(expanded), _ptr(x), _ptr(out), _stream(stream)),
           "vmla_attend_expanded")


def vmla_attend_expanded_profiled(ctx, expanded, x, out, attn_start: int, attn_stop: int, stream=None) -> None:
    _check(lib().vmla_attend_expanded_profiled(ctx, _ptr(expanded), _ptr(x), _ptr(out), attn_start, attn_stop,
                                               _stream(stream)), "vmla_attend_expanded_profiled")


def _freq_array(rope_freqs):
    if rope_freqs is None:
        return None
    arr = (c_float * len(rope_freqs))(*[float(v) for v in rope_freqs])
    return ctypes.cast(arr, POINTER(c_float))


def vmla_dense_cache_bytes(cfg: vmla_config) -> int:
    return lib().vmla_dense_cache_bytes(byref(cfg))


def vmla_dense_workspace_bytes(cfg: vmla_config) -> int:
    return lib().vmla_dense_workspace_bytes(byref(cfg))


def vmla_dense_create(cfg: vmla_config, weights: vmla_dense_weights, cache, workspace, rope_freqs=None) -> c_void_p:
    ctx = c_void_p()
    _check(lib().vmla_dense_create(byref(cfg), byref(weights), _ptr(cache), _ptr(workspace),
                                   _freq_array(rope_freqs), byref(ctx)), "vmla_dense_create")
    return ctx


def vmla_dense_prepare(ctx, stream=None) -> None:
    _check(lib().vmla_dense_prepare(ctx, _stream(stream)), "vmla_dense_prepare")


def vmla_dense_range_flags(ctx, stream=None) -> int:
    v = c_uint32()
    _check(lib().vmla_dense_range_flags(ctx, byref(v), _stream(stream)), "vmla_dense_range_flags")
    return v.value


def vmla_dense_append(ctx, x, stream=None) -> None:
    _check(lib().vmla_dense_append(ctx, _ptr(x), _stream(stream)), "vmla_dense_append")


def vmla_dense_attend(ctx, x, out, stream=None) -> None:
    _check(lib().vmla_dense_attend(ctx, _ptr(x), _ptr(out), _stream(stream)), "vmla_dense_attend")


def vmla_dense_attend_profiled(ctx, x, out, attn_start: int, attn_stop: int, stream=None) -> None:
    _check(lib().vmla_dense_attend_profiled(ctx, _ptr(x), _ptr(out), attn_start, attn_stop, _stream(stream)),
           "vmla_dense_attend_profiled")


def vmla_dense_cache_state(ctx):
    n, first, nv = c_int64(), c_int64(), c_int32()
    _check(lib().vmla_dense_cache_state(ctx, byref(n), byref(first), byref(nv)), "vmla_dense_cache_state")
    return n.value, first.value, nv.value


def vmla_dense_reset(ctx) -> None:
    _check(lib().vmla_dense_reset(ctx), "vmla_dense_reset")


def vmla_dense_destroy(ctx) -> None:
    lib().vmla_dense_destroy(ctx)


def vmla_status_string(code: int) -> str:
    return lib().vmla_status_string(int(code)).decode()


# ----------------------------------------------------------------------------- helpers
def config_from_geometry(g, attn_workgroups: int = 0) -> vmla_config:
    """vmla_config for a workloads.LayerGeometry (or anything with the same fields)."""
    pt, ph, pw = g.rope_pairs
    return vmla_config(batch=g.batch, hidden=g.hidden, n_heads=g.n_heads, d_nope=g.d_nope, d_rope=g.d_rope,
                       d_v=g.d_v, d_c=g.d_c, d_q=g.d_q, rope_pairs_t=pt, rope_pairs_h=ph, rope_pairs_w=pw,
                       rope_theta=g.rope_theta, grid_h=g.grid_h, grid_w=g.grid_w,
                       window_frames=g.window_frames, chunk_frames=g.chunk_frames,
                       dtype=VMLA_DTYPE_F32 if g.dtype == "f32" else VMLA_DTYPE_BF16,
                       attn_workgroups=attn_workgroups, sink_frames=getattr(g, "sink_frames", 0),
                       rope_at_use=1 if getattr(g, "sink_frames", 0) > 0 or getattr(g, "rope_at_use", False) else 0)


def torch_dtype(g):
    import torch
    return torch.float32 if g.dtype == "f32" else torch.bfloat16


def _check_tensor(t, shape, dtype, device, what):
    """A device tensor handed to the library: contiguous, of this shape and
    dtype, on the layer's device (a host or foreign-device pointer would reach
    the kernels otherwise)."""
    if (tuple(t.shape) != tuple(shape) or t.dtype != dtype or not t.is_contiguous() or not t.is_cuda
            or t.device != device):
        raise ValueError(f"{what} must be a contiguous {dtype} tensor of shape {tuple(shape)} on {device}; "
                         f"got {t.dtype} {tuple(t.shape)} on {t.device}"
                         f"{'' if t.is_contiguous() else ' (not contiguous)'}")


class LatentAttention:
    """One layer: device weights, ring cache and workspace (torch-allocated),
    driven through the C entry points above."""

    WEIGHT_NAMES = ("w_dkv", "w_kr", "w_dq", "w_uq", "w_uk", "w_uv", "w_o")

    def __init__(self, g, weights: dict, device="cuda", attn_workgroups: int = 0, rope_freqs=None,
                 cache_fill: float | None = None):
        import torch
        self.g = g
        self.dtype = torch_dtype(g)
        self.cfg = config_from_geometry(g, attn_workgroups)
        cb, wb = vmla_cache_bytes(self.cfg), vmla_workspace_bytes(self.cfg)
        if cb == 0 or wb == 0:
            raise ValueError(f"geometry {g.name} is not accepted by the library")
        self.w = {}
        for n in self.WEIGHT_NAMES:
            t = weights[n]
            t = torch.as_tensor(t) if not isinstance(t, torch.Tensor) else t
            self.w[n] = t.to(device=device, dtype=self.dtype).contiguous()
        es = 4 if g.dtype == "f32" else 2
        self.cache = torch.empty(cb // es, dtype=self.dtype, device=device).view(
            g.batch, (getattr(g, "sink_frames", 0) + g.window_frames) * g.tokens_per_frame, g.latent_width)
        if cache_fill is not None:
            self.cache.fill_(cache_fill)
        self.workspace = torch.empty(wb, dtype=torch.uint8, device=device)
        self.device = self.workspace.device
        wts = vmla_weights(**{n: self.w[n].data_ptr() for n in self.WEIGHT_NAMES})
        if rope_freqs is None:
            rope_freqs = getattr(g, "rope_freqs", None)
        self.ctx = vmla_create(self.cfg, wts, self.cache, self.workspace, rope_freqs)
        vmla_prepare(self.ctx)

    def _check_x(self, x, out=None, tokens=None):
        g = self.g
        shape = (g.batch, g.n_q if tokens is None else tokens, g.hidden)
        _check_tensor(x, shape, self.dtype, self.device, "x")
        if out is not None:
            _check_tensor(out, shape, self.dtype, self.device, "out")

    def append(self, x, stream=None):
        self._check_x(x)
        vmla_compress_append(self.ctx, x, stream)

    def attend(self, x, out=None, stream=None):
        import torch
        self._check_x(x, out)
        if out is None:
            out = torch.empty_like(x)
        vmla_attend(self.ctx, x, out, stream)
        return out

    def compress(self, x, frame0: int, out=None, stream=None):
        import torch
        self._check_x(x)
        shape = (self.g.batch, self.g.n_q, self.g.latent_width)
        if out is None:
            out = torch.empty(shape, dtype=self.dtype, device=x.device)
        _check_tensor(out, shape, self.dtype, self.device, "out")
        vmla_compress(self.ctx, x, frame0, out, stream)
        return out

    def state(self):
        return vmla_cache_state(self.ctx)

    def reset(self):
        vmla_reset(self.ctx)

    def range_flags(self, stream=None) -> int:
        """Read and clear the range flag (bit 0: an fp16 operand copy saturated)."""
        return vmla_range_flags(self.ctx, stream)

    def attend_clip(self, x, out=None, stream=None):
        """Block-causal attention over a whole clip x [batch, window_frames*T, hidden]."""
        import torch
        g = self.g
        self._check_x(x, out, tokens=g.window_frames * g.tokens_per_frame)
        if getattr(self, "clip_workspace", None) is None:
            self.clip_workspace = torch.empty(vmla_clip_workspace_bytes(self.cfg), dtype=torch.uint8,
                                              device=self.cache.device)
        if out is None:
            out = torch.empty_like(x)
        vmla_attend_clip(self.ctx, x, self.clip_workspace, out, stream)
        return out

    def expand(self, stream=None):
        """Up-project the window to per-head keys/values (expanded path) into an
        owned buffer, allocated on first use."""
        import torch
        if getattr(self, "expanded", None) is None:
            nbytes = vmla_expanded_bytes(self.cfg)
            if nbytes == 0:
                raise ValueError(f"geometry {self.g.name} has no expanded path")
            self.expanded = torch.empty(nbytes, dtype=torch.uint8, device=self.cache.device)
        vmla_expand(self.ctx, self.expanded, stream)

    def attend_expanded(self, x, out=None, stream=None):
        import torch
        self._check_x(x, out)
        if out is None:
            out = torch.empty_like(x)
        vmla_attend_expanded(self.ctx, getattr(self, "expanded", None), x, out, stream)
        return out

    def close(self):
        if self.ctx:
            vmla_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class DenseAttention:
    """Dense per-head baseline layer: device weights, per-head K/V ring cache and
    workspace (torch-allocated), driven through the vmla_dense_* entry points.
    The geometry has d_nope = d_c = d_q = 0 and d_rope = per-head width."""

    WEIGHT_NAMES = ("w_q", "w_k", "w_v", "w_o")

    def __init__(self, g, weights: dict, device="cuda", attn_workgroups: int = 0, rope_freqs=None,
                 cache_fill: float | None = None):
        import torch
        self.g = g
        self.dtype = torch_dtype(g)
        self.cfg = config_from_geometry(g, attn_workgroups)
        cb, wb = vmla_dense_cache_bytes(self.cfg), vmla_dense_workspace_bytes(self.cfg)
        if cb == 0 or wb == 0:
            raise ValueError(f"geometry {g.name} is not accepted by the dense library path")
        self.w = {}
        for n in self.WEIGHT_NAMES:
            t = weights[n]
            t = torch.as_tensor(t) if not isinstance(t, torch.Tensor) else t
            self.w[n] = t.to(device=device, dtype=self.dtype).contiguous()
        self.cache = torch.empty(cb, dtype=torch.uint8, device=device)
        if cache_fill is not None:
            self.cache.view(torch.float16).fill_(cache_fill)
        self.workspace = torch.empty(wb, dtype=torch.uint8, device=device)
        self.device = self.workspace.device
        wts = vmla_dense_weights(**{n: self.w[n].data_ptr() for n in self.WEIGHT_NAMES})
        if rope_freqs is None:
            rope_freqs = getattr(g, "rope_freqs", None)
        self.ctx = vmla_dense_create(self.cfg, wts, self.cache, self.workspace, rope_freqs)
        vmla_dense_prepare(self.ctx)

    def _check_x(self, x, out=None):
        g = self.g
        shape = (g.batch, g.n_q, g.hidden)
        _check_tensor(x, shape, self.dtype, self.device, "x")
        if out is not None:
            _check_tensor(out, shape, self.dtype, self.device, "out")

    def append(self, x, stream=None):
        self._check_x(x)
        vmla_dense_append(self.ctx, x, stream)

    def range_flags(self, stream=None) -> int:
        """Read and clear the range flag (bit 0: an fp16 operand copy saturated)."""
        return vmla_dense_range_flags(self.ctx, stream)

    def attend(self, x, out=None, stream=None):
        import torch
        self._check_x(x, out)
        if out is None:
            out = torch.empty_like(x)
        vmla_dense_attend(self.ctx, x, out, stream)
        return out

    def state(self):
        return vmla_dense_cache_state(self.ctx)

    def reset(self):
        vmla_dense_reset(self.ctx)

    def close(self):
        if self.ctx:
            vmla_dense_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
