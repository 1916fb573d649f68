"""Layer geometries and seeded synthetic inputs for latent-KV video attention.

This module holds shapes and random numbers only; none of the attention
arithmetic lives here.  Both the HIP path (through the Python binding) and the
CPU oracle consume what it produces, so it imports neither of them.

Geometry sources (VideoMLA: Low-Rank Latent KV Cache for Minute-Scale
Autoregressive Video Diffusion, paper text):
  * Wan2.1-T2V-1.3B backbone: hidden 1536, 12 heads x 128, d_c = 192,
    d_q = 768, NoPE/RoPE split 96 + 32 (section 4.1).
  * 1,560 tokens per latent frame on a 30 x 52 grid, 21-frame window,
    3-frame chunks (appendix D.1).
  * Latent cache entry = content latent (d_c) + head-shared 3D-RoPE key
    (d_h^rope) (sections 3.1, 3.2).

Input recipe: every weight is N(0,1)/sqrt(fan_in); hidden states are drawn
N(0,1)/sqrt(hidden) ("literal"), N(0,1) ("unit"), or N(0,1) with the query
down-projection scaled by 4 ("sharp", which sharpens the softmax so that online
rescaling is exercised).  Streams are a counter-based Philox keyed by
(seed, layer, chunk, step, tensor id), so any step of a rollout can be rebuilt
on its own.
"""
from __future__ import annotations

import dataclasses
import hashlib
from dataclasses import dataclass, field

import numpy as np

F32, BF16 = "f32", "bf16"


@dataclass(frozen=True)
class LayerGeometry:
    name: str
    batch: int
    hidden: int
    n_heads: int
    d_nope: int
    d_rope: int
    d_v: int
    d_c: int
    d_q: int
    rope_pairs: tuple  # (t, h, w) complex pairs of the decoupled key
    rope_theta: float
    grid_h: int
    grid_w: int
    window_frames: int
    chunk_frames: int
    dtype: str
    # rollout shape (streaming workloads); 1/1/1 for a single call
    layers: int = 1
    chunks: int = 1
    steps: int = 1
    prefill_chunks: int = 0  # seeded appends before the measured attend
    sink_frames: int = 0     # pinned sink frames ahead of the window (long-horizon cache)
    rope_at_use: bool = False  # GPU layout choice: store k_r un-rotated, rotate per call (implied by sinks)
    rope_freqs: tuple = None   # explicit omega per rotary pair (axis order t, h, w); None: the default table

    @property
    def head_dim(self) -> int:
        return self.d_nope + self.d_rope

    @property
    def tokens_per_frame(self) -> int:
        return self.grid_h * self.grid_w

    @property
    def n_q(self) -> int:
        return self.chunk_frames * self.tokens_per_frame

    @property
    def latent_width(self) -> int:
        return self.d_c + self.d_rope

    def cached_frames(self, frames_appended: int) -> int:
        n, S = frames_appended, self.sink_frames
        return min(n, S) + max(0, min(n - S, self.window_frames))

    def n_k(self, frames_appended: int) -> int:
        return self.cached_frames(frames_appended) * self.tokens_per_frame + self.n_q

    def replace(self, **kw) -> "LayerGeometry":
        return dataclasses.replace(self, **kw)


TINY = LayerGeometry(
    name="tiny-f32", batch=1, hidden=64, n_heads=2, d_nope=8, d_rope=8, d_v=16, d_c=24,
    d_q=32, rope_pairs=(1, 1, 2), rope_theta=10000.0, grid_h=4, grid_w=4,
    window_frames=2, chunk_frames=1, dtype=F32, chunks=6, prefill_chunks=2)

WAN_LAYER = LayerGeometry(
    name="wan1.3b-layer", batch=1, hidden=1536, n_heads=12, d_nope=96, d_rope=32, d_v=128,
    d_c=192, d_q=768, rope_pairs=(4, 6, 6), rope_theta=10000.0, grid_h=30, grid_w=52,
    window_frames=21, chunk_frames=3, dtype=BF16, prefill_chunks=7)

WAN_ROLLOUT = WAN_LAYER.replace(name="wan1.3b-rollout-30L", layers=30, chunks=20, steps=4,
                                prefill_chunks=0)

# Dense per-head baseline: 12 heads x 128 per-head K and V, full 3D-RoPE on the
# 128-d keys split near-equally over (t, h, w) with t taking the remainder.
WAN_DENSE = WAN_LAYER.replace(name="wan1.3b-dense", d_nope=0, d_rope=128, d_c=0, d_q=0,
                              rope_pairs=(22, 21, 21))

# The dense baseline at the Wan widths on the small grid (parity at sizes the
# oracle finishes in seconds), and a tiny dense layer for the brute force.
WAN_DENSE_SMALL_GRID = WAN_DENSE.replace(name="wan-dense-grid6x10", grid_h=6, grid_w=10, window_frames=5,
                                         prefill_chunks=2)
TINY_DENSE = TINY.replace(name="tiny-dense", d_nope=0, d_rope=16, d_c=0, d_q=0, rope_pairs=(2, 3, 3))

STRESS = {dc: WAN_LAYER.replace(name=f"stress-b4-w42-dc{dc}", batch=4, window_frames=42, d_c=dc,
                                prefill_chunks=14)
          for dc in (96, 192, 448)}

# A reduced geometry with the Wan layer widths but a small grid: the oracle
# finishes it in a second, yet it spans several attention row blocks, several
# key tiles and ragged tails of both.
WAN_SMALL_GRID = WAN_LAYER.replace(name="wan-widths-grid6x10", grid_h=6, grid_w=10,
                                   window_frames=5, prefill_chunks=2)

# The long-horizon cache of the pages' rollouts: one sink frame and a six-frame
# window (10,920 cached keys), with re-indexed temporal coordinates.
WAN_SINK = WAN_LAYER.replace(name="wan1.3b-sink1-w6", sink_frames=1, window_frames=6, prefill_chunks=7)

GEOMETRIES = {g.name: g for g in (TINY, TINY_DENSE, WAN_LAYER, WAN_ROLLOUT, WAN_DENSE, WAN_DENSE_SMALL_GRID, WAN_SINK,
                                  WAN_SMALL_GRID,
                                  *STRESS.values())}


# ----------------------------------------------------------------------------- RNG
_TENSOR_IDS = {"w_dkv": 1, "w_kr": 2, "w_dq": 3, "w_uq": 4, "w_uk": 5, "w_uv": 6, "w_o": 7,
               "x": 8, "w_k": 9, "w_v": 10, "w_q": 11}


def _stream(seed: int, layer: int, chunk: int, step: int, tensor: str) -> np.random.Generator:
    """Counter-based Philox stream keyed by the tuple (seed, layer, chunk, step, tensor)."""
    ident = f"{seed}/{layer}/{chunk}/{step}/{_TENSOR_IDS[tensor]}".encode()
    key = np.frombuffer(hashlib.sha256(ident).digest()[:16], dtype=np.uint64)
    return np.random.Generator(np.random.Philox(key=key))


def _normal(shape, seed, layer, chunk, step, tensor, scale) -> np.ndarray:
    g = _stream(seed, layer, chunk, step, tensor)
    return (g.standard_normal(size=shape, dtype=np.float32) * np.float32(scale)).astype(np.float32)


def quantize(a: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to the storage type (bf16 round-to-nearest-even) and
    return them widened back to float32, so that both consumers see identical
    values."""
    if dtype == F32:
        return np.ascontiguousarray(a, dtype=np.float32)
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


@dataclass
class LatentWeights:
    """One layer's weights in PyTorch Linear layout ([out, in], row-major)."""
    w_dkv: np.ndarray  # [d_c, hidden]
    w_kr: np.ndarray   # [d_rope, hidden]
    w_dq: np.ndarray   # [d_q, hidden]
    w_uq: np.ndarray   # [n_heads*(d_nope+d_rope), d_q]; per head [q_nope ; q_rope]
    w_uk: np.ndarray   # [n_heads, d_nope, d_c]
    w_uv: np.ndarray   # [n_heads, d_v, d_c]
    w_o: np.ndarray    # [hidden, n_heads*d_v]

    def as_dict(self):
        return dataclasses.asdict(self)


def latent_weights(g: LayerGeometry, layer: int = 0, seed: int = 0, mode: str = "literal") -> LatentWeights:
    d, nh = g.hidden, g.n_heads
    dq_gain = 4.0 if mode == "sharp" else 1.0

    def w(name, shape, fan_in, gain=1.0):
        return quantize(_normal(shape, seed, layer, 0, 0, name, gain / np.sqrt(fan_in)), g.dtype)

    return LatentWeights(
        w_dkv=w("w_dkv", (g.d_c, d), d),
        w_kr=w("w_kr", (g.d_rope, d), d),
        w_dq=w("w_dq", (g.d_q, d), d, dq_gain),
        w_uq=w("w_uq", (nh * g.head_dim, g.d_q), g.d_q),
        w_uk=w("w_uk", (nh, g.d_nope, g.d_c), g.d_c),
        w_uv=w("w_uv", (nh, g.d_v, g.d_c), g.d_c),
        w_o=w("w_o", (d, nh * g.d_v), nh * g.d_v),
    )


@dataclass
class DenseWeights:
    """Dense per-head baseline weights, Linear layout."""
    w_q: np.ndarray  # [n_heads*128, hidden]
    w_k: np.ndarray  # [n_heads*128, hidden]
    w_v: np.ndarray  # [n_heads*d_v, hidden]
    w_o: np.ndarray  # [hidden, n_heads*d_v]


def dense_weights(g: LayerGeometry, layer: int = 0, seed: int = 0, mode: str = "literal") -> DenseWeights:
    d, nh = g.hidden, g.n_heads
    q_gain = 4.0 if mode == "sharp" else 1.0

    def w(name, shape, fan_in, gain=1.0):
        return quantize(_normal(shape, seed, layer, 0, 0, name, gain / np.sqrt(fan_in)), g.dtype)

    return DenseWeights(
        w_q=w("w_q", (nh * g.head_dim, d), d, q_gain),
        w_k=w("w_k", (nh * g.head_dim, d), d),
        w_v=w("w_v", (nh * g.d_v, d), d),
        w_o=w("w_o", (d, nh * g.d_v), nh * g.d_v),
    )


def hidden_states(g: LayerGeometry, layer: int = 0, chunk: int = 0, step: int = 0, seed: int = 0,
                  mode: str = "literal") -> np.ndarray:
    """Hidden states of one chunk, [batch, chunk_frames*tokens_per_frame, hidden]."""
    scale = 1.0 / np.sqrt(g.hidden) if mode == "literal" else 1.0
    x = _normal((g.batch, g.n_q, g.hidden), seed, layer, chunk, step, "x", scale)
    return quantize(x, g.dtype)
