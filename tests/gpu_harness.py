"""Shared helpers of the GPU tests: build a layer from seeded inputs, roll the
ring forward, and compare against the oracle with the parity metric.

Parity metric (every attention comparison): max_abs = max |g - r| and
mean_rel = sum |g - r| / sum |r| over all compared output elements; the bar is
max_abs <= 2e-2 and mean_rel <= 5e-3 against the float64 oracle fed with the
same (storage-rounded) inputs.
"""
from __future__ import annotations

import numpy as np

from mla_latent_kv_vmla_amd import vmla, workloads as wl

MAX_ABS, MEAN_REL = 2e-2, 5e-3


def to_dev(a, g):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda").to(vmla.torch_dtype(g))


def to_np(t):
    return t.float().cpu().numpy().astype(np.float64)


def parity(gpu: np.ndarray, ref: np.ndarray):
    err = np.abs(gpu - ref)
    return float(err.max()), float(err.sum() / np.abs(ref).sum())


def assert_parity(gpu, ref, what=""):
    ma, mr = parity(gpu, ref)
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite output"
    assert ma <= MAX_ABS and mr <= MEAN_REL, f"{what}: max_abs={ma:.3e} mean_rel={mr:.3e}"
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
