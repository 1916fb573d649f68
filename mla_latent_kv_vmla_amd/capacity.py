"""Serving capacity of one GPU: how many independent streams fit.

Per stream, a rollout keeps every layer's cache resident (latent rows
[c | k_r] per token, or per-head K and V for the dense baseline), while the
per-call buffers (workspace, hidden states in and out) exist for one layer at
a time and scale with the batch; the layers' weights are a fixed cost.  The
layouts are the library's: `vmla_cache_bytes` / `vmla_workspace_bytes` (latent)
and `vmla_dense_cache_bytes` / `vmla_dense_workspace_bytes` (dense); the
formulas below restate them so that latent widths without a built kernel can be
priced too, and a test checks them against the library for every built shape
(VideoMLA paper, section 4.3 "Batch Scaling Under Fixed Memory" runs the same
sweep on its own hardware).
"""
from __future__ import annotations

from dataclasses import dataclass

ALIGN = 256
ATTN_MAX_ROWS = 256
DEFAULT_WORKGROUPS = 256
DENSE_KEY_TILE = 128


def _al(x: int) -> int:
    return (x + ALIGN - 1) // ALIGN * ALIGN


def latent_cache_bytes(g, batch: int = 1, es: int = 2) -> int:
    return batch * (g.sink_frames + g.window_frames) * g.tokens_per_frame * (g.d_c + g.d_rope) * es


def rope_table_bytes(g, pairs: int) -> int:
    """The rotary table of the row and column axes: per pair, cos and sin (fp32)
    for max(grid_h, grid_w) positions."""
    return pairs * max(g.grid_h, g.grid_w) * 2 * 4


def latent_workspace_bytes(g, batch: int = 1, es: int = 2, key_tile: int = 64,
                           workgroups: int = DEFAULT_WORKGROUPS, part: str = "total") -> int:
    """Mirror of the library's latent workspace layout for `batch` streams:
    part = "persistent" (range flag, rotary table and the prepared weights, per
    layer: [W_DKV; W_KR], the absorbed query weight and W_UQ (each with W_DQ
    taken in), W_UV, W_O), "per_call" (the buffers of one attend, at least the fp32 scratch
    the preparation of the query weight uses) or "total".  The activation type
    has the storage type's width (fp16 for bf16, fp32 for fp32)."""
    M = batch * g.n_q
    D, nh, dh = g.d_c + g.d_rope, g.n_heads, g.d_nope + g.d_rope
    dcp = (g.d_c + 31) // 32 * 32
    tiles = (-(-(g.sink_frames + g.window_frames) * g.tokens_per_frame // key_tile)
             + -(-g.n_q // key_tile))
    persistent = [4, rope_table_bytes(g, g.d_rope // 2), D * g.hidden * es, nh * D * g.hidden * es, nh * dh * g.hidden * es, nh * g.d_v * g.d_c * es,
                  g.hidden * nh * g.d_v * es]
    per_call = [M * D * es, M * g.hidden * es if es == 2 else 0,  # chunk rows; fp16 copy of x (16-bit storage)
                g.n_q * (g.d_rope // 2) * 8 if es == 2 else 0,  # the chunk tokens' rotary cos/sin (16-bit storage)
                M * nh * max(D, g.d_v) * es,  # absorbed queries, then per-head outputs
                M * nh * g.d_c * es, 2 * workgroups * ATTN_MAX_ROWS * g.d_c * es, 2 * workgroups * ATTN_MAX_ROWS * 2 * 4,
                # pre-pass tiles: fp16 key tiles (16-bit storage), transposed value images (fp32)
                batch * tiles * key_tile * D * 2 if es == 2 else batch * tiles * dcp * (key_tile + 16 // es) * es,
                # rotated copy of the visible rows: rotation at use with fp32 storage only
                batch * (g.sink_frames + g.window_frames) * g.tokens_per_frame * D * es
                if (g.rope_at_use or g.sink_frames) and es == 4 else 0]
    a = sum(_al(x) for x in persistent)
    b = max(sum(_al(x) for x in per_call), _al(nh * D * g.d_q * 4))
    return {"persistent": a, "per_call": b, "total": a + b}[part]


def dense_cache_bytes(g, batch: int = 1) -> int:
    P = -(-g.window_frames * g.tokens_per_frame // DENSE_KEY_TILE) * DENSE_KEY_TILE
    heads = batch * g.n_heads
    return _al(heads * P * g.head_dim * 2) + _al(heads * P * g.d_v * 2)


def dense_workspace_bytes(g, batch: int = 1, workgroups: int = DEFAULT_WORKGROUPS, part: str = "total") -> int:
    """Mirror of the dense workspace: persistent (range flag, rotary table, fp16 W_O) and per call."""
    S = -(-g.n_q // DENSE_KEY_TILE) * DENSE_KEY_TILE
    heads = batch * g.n_heads
    persistent = [4, rope_table_bytes(g, g.head_dim // 2), g.hidden * g.n_heads * g.d_v * 2]
    per_call = [heads * g.n_q * g.head_dim * 2, heads * S * g.head_dim * 2, heads * S * g.d_v * 2,
                batch * g.n_q * g.n_heads * g.d_v * 2, 2 * workgroups * ATTN_MAX_ROWS * g.d_v * 2,
                2 * workgroups * ATTN_MAX_ROWS * 2 * 4]
    a, b = sum(_al(x) for x in persistent), sum(_al(x) for x in per_call)
    return {"persistent": a, "per_call": b, "total": a + b}[part]


def latent_weight_bytes(g, es: int = 2) -> int:
    d, nh = g.hidden, g.n_heads
    return es * (g.d_c * d + g.d_rope * d + g.d_q * d + nh * g.head_dim * g.d_q + nh * g.d_nope * g.d_c
                 + nh * g.d_v * g.d_c + d * nh * g.d_v)


def dense_weight_bytes(g, es: int = 2) -> int:
    d, nh = g.hidden, g.n_heads
    return es * (nh * g.head_dim * d * 2 + nh * g.d_v * d + d * nh * g.d_v)


@dataclass
class Capacity:
    per_stream_bytes: int   # all layers' caches + this stream's share of one call's buffers
    fixed_bytes: int        # all layers' weights
    max_batch: int


def capacity(g, layers: int, budget_bytes: int, dense: bool = False) -> Capacity:
    """Largest batch whose caches (all layers), one layer's per-call buffers and
    all weights (each layer's own and its prepared copies) fit in budget_bytes.
    Per-call buffers are linear in the batch except the stream-K partial states,
    which are charged once."""
    io = 2 * g.n_q * g.hidden * 2  # x and out of one call, per stream
    if dense:
        cache = dense_cache_bytes(g) * layers
        fixed = (dense_weight_bytes(g) + dense_workspace_bytes(g, 1, part="persistent")) * (layers - 1)
        fixed += dense_weight_bytes(g)
        ws1, ws2 = dense_workspace_bytes(g, 1), dense_workspace_bytes(g, 2)
    else:
        cache = latent_cache_bytes(g) * layers
        fixed = (latent_weight_bytes(g) + latent_workspace_bytes(g, 1, part="persistent")) * (layers - 1)
        fixed += latent_weight_bytes(g)
        ws1, ws2 = latent_workspace_bytes(g, 1), latent_workspace_bytes(g, 2)
    slope = ws2 - ws1
    fixed += ws1 - slope  # the batch-independent part of the workspace
    per = cache + slope + io
    return Capacity(per, fixed, max(0, (budget_bytes - fixed) // per))
