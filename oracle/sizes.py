"""Cache-size arithmetic of the per-token KV layouts.

TEST INFRASTRUCTURE ONLY (see the package docstring).

VideoMLA paper, section 3.1: a dense per-head cache stores 2 * n_h * d_h scalars
per token per layer (keys and values of every head); the latent cache stores
d_c + d_h^rope.  Section 1 and section 4.1 give the Wan-1.3B figures.
Appendix D.1 gives the token grid: a 480x832 clip goes through the Wan VAE to a
60x104 latent, and a (1,2,2) patch embedding makes a 30x52 grid per frame.
"""
from __future__ import annotations


def dense_scalars_per_token(n_heads: int, head_dim: int) -> int:
    """Keys plus values of every head (section 1, section 3.1)."""
    return 2 * n_heads * head_dim


def latent_scalars_per_token(d_c: int, d_rope: int) -> int:
    """Shared content latent plus the head-shared decoupled RoPE key (section 3.1)."""
    return d_c + d_rope


def reduction_fraction(n_heads: int, head_dim: int, d_c: int, d_rope: int) -> float:
    return 1.0 - latent_scalars_per_token(d_c, d_rope) / dense_scalars_per_token(n_heads, head_dim)


def reduction_factor(n_heads: int, head_dim: int, d_c: int, d_rope: int) -> float:
    return dense_scalars_per_token(n_heads, head_dim) / latent_scalars_per_token(d_c, d_rope)


def cache_scalars(layers: int, frames: int, tokens_per_frame: int, scalars_per_token: int) -> int:
    return layers * frames * tokens_per_frame * scalars_per_token


def cache_bytes(layers: int, frames: int, tokens_per_frame: int, scalars_per_token: int,
                bytes_per_scalar: int = 2) -> int:
    return cache_scalars(layers, frames, tokens_per_frame, scalars_per_token) * bytes_per_scalar


def token_grid(height: int, width: int, vae_spatial_stride: int, patch_hw: tuple) -> tuple:
    """Tokens per latent frame from pixel size, VAE stride and patch size (appendix D.1)."""
    lh, lw = height // vae_spatial_stride, width // vae_spatial_stride
    return lh // patch_hw[0], lw // patch_hw[1]


def layer_cut_fraction(cached_layers: int, layers: int) -> float:
    """Storage cut of a design that caches only some layers with dense KV (section 1)."""
    return 1.0 - cached_layers / layers


def ratio_vs_partial_dense(cached_layers: int, layers: int, n_heads: int, head_dim: int,
                           d_c: int, d_rope: int) -> float:
    """Dense cache of `cached_layers` layers over a latent cache of all `layers`."""
    return (cached_layers * dense_scalars_per_token(n_heads, head_dim)) / (
        layers * latent_scalars_per_token(d_c, d_rope))
