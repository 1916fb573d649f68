"""Shared helpers of the GPU tests: build a layer from seeded inputs, roll the
ring forward, and compare against the oracle with the parity metric.

Parity metric (every attention comparison): max_abs = max |g - r| and
mean_rel = sum |g - r| / sum |r| over all compared output elements, against the
float64 oracle fed with the same (storage-rounded) inputs.

Bar: max_abs <= 2e-2 and mean_rel <= 5e-3 -- the stated bar for the layer
geometries' input recipe (weights and hidden states N(0,1)/sqrt(fan_in)), whose
softmax is nearly flat (score spread sigma_s ~ 1e-3).  The steeper variants the
tests add (unit hidden states, sharpened query projection) raise sigma_s to ~1
and ~4.  With bf16 storage every score is a dot product of two rounded operands
(cached latent row, absorbed query), so it carries an absolute error of order
u*|s| (u = 2^-8, the bf16 rounding unit), and softmax turns a score error into
the same relative error of that key's weight.  The derived bound is therefore
mean_rel <= 5e-3 + u*sigma_s and max_abs <= 2e-2*max(1, max|r|); for the
layer recipe it is the stated bar.  fp32 storage keeps the stated bar in every
variant (its u is 2^-24).
"""
from __future__ import annotations

import numpy as np

from mla_latent_kv_vmla_amd import vmla, workloads as wl

MAX_ABS, MEAN_REL = 2e-2, 5e-3
U_BF16 = 2.0 ** -8


def to_dev(a, g):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda").to(vmla.torch_dtype(g))


def to_np(t):
    return t.float().cpu().numpy().astype(np.float64)


def parity(gpu: np.ndarray, ref: np.ndarray):
    err = np.abs(gpu - ref)
    return float(err.max()), float(err.sum() / np.abs(ref).sum())


def bounds(ref, sigma_s: float = 0.0, dtype: str = wl.BF16):
    """(max_abs, mean_rel) bound for a comparison, see the module docstring."""
    if dtype == wl.F32:
        return MAX_ABS, MEAN_REL
    return MAX_ABS * max(1.0, float(np.abs(ref).max())), MEAN_REL + U_BF16 * sigma_s


def assert_parity(gpu, ref, what="", sigma_s: float = 0.0, dtype: str = wl.BF16):
    ma, mr = parity(gpu, ref)
    ba, br = bounds(ref, sigma_s, dtype)
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite output"
    assert ma <= ba and mr <= br, \
        f"{what}: max_abs={ma:.3e} (bound {ba:.3e}) mean_rel={mr:.3e} (bound {br:.3e}, sigma_s={sigma_s:.3f})"
    return ma, mr


class Rollout:
    """One layer on the GPU plus the host-side history the oracle needs."""

    def __init__(self, g, mode="literal", seed=0, layer=0, attn_workgroups=0, cache_fill=None):
        self.g, self.mode, self.seed, self.layer = g, mode, seed, layer
        self.w = wl.latent_weights(g, layer=layer, seed=seed, mode=mode)
        self.dev = vmla.LatentAttention(g, {k: to_dev(v, g) for k, v in self.w.as_dict().items()},
                                        attn_workgroups=attn_workgroups, cache_fill=cache_fill)
        self.hist = [dict() for _ in range(g.batch)]  # per stream: frame -> [T, hidden]
        self.n = 0

    def x(self, chunk, step=0):
        return wl.hidden_states(self.g, layer=self.layer, chunk=chunk, step=step, seed=self.seed, mode=self.mode)

    def append(self, x_np):
        g = self.g
        self.dev.append(to_dev(x_np, g))
        for b in range(g.batch):
            fr = x_np[b].reshape(g.chunk_frames, g.tokens_per_frame, g.hidden)
            for i in range(g.chunk_frames):
                self.hist[b][self.n + i] = fr[i]
        self.n += g.chunk_frames

    def attend(self, x_np):
        return to_np(self.dev.attend(to_dev(x_np, self.g)))

    def oracle(self, x_np, b=0, query_tokens=None):
        from oracle import mla
        return mla.attend(self.g, self.w, self.hist[b], self.n, x_np[b], query_tokens=query_tokens)

    def score_spread(self, x_np, b=0, query_tokens=None) -> float:
        """Mean over (head, query) of the standard deviation of the natural-unit
        scores over the visible keys, from the oracle."""
        from oracle import mla
        s = mla.scores(self.g, self.w, self.hist[b], self.n, x_np[b], query_tokens=query_tokens)
        return float(s.std(axis=-1).mean())

    def check(self, got_b, x_np, b=0, query_tokens=None, what=""):
        ref = self.oracle(x_np, b, query_tokens)
        sig = self.score_spread(x_np, b, query_tokens)
        return assert_parity(got_b, ref, what, sig, self.g.dtype)
