"""Pinned sink frames and window re-indexing (rope_at_use) on the GPU.

The long-horizon cache of the pages keeps one sink frame ahead of a six-frame
window and rotates every visible key, and the chunk's queries, at local
temporal coordinates (appendix D.4, D.5).  The oracle implements exactly that
(its pins include brute force and independence from absolute time).  Cases:
ring placement with the sink pinned (c bit-exact, k_r stored un-rotated),
attention at every window state (fp32 and bf16, three scalings; d_c = 192,
96 and 448), rotation at use without a sink, the expanded path with a sink, and the full-size
sink + 6-frame Wan layer.  Same bar and tolerance derivation as gpu_harness.
"""
import numpy as np
import pytest

from gpu_harness import Rollout, to_dev, to_np
from mla_latent_kv_vmla_amd import workloads as wl
from oracle import mla, ring

pytestmark = pytest.mark.gpu

TINY_SINK = wl.TINY.replace(name="tiny-sink", sink_frames=1)
TINY_SINK_BF16 = TINY_SINK.replace(name="tiny-sink-bf16", dtype=wl.BF16)
SMALL_SINK = wl.WAN_SMALL_GRID.replace(name="wan-widths-grid6x10-sink1-w3", sink_frames=1, window_frames=3)


def _case(*a):
    print("case:", *a, flush=True)


def test_sink_ring_placement():
    import torch
    g = SMALL_SINK
    _case("sink ring", g.name)
    r = Rollout(g, mode="unit", cache_fill=-5.0)
    canary = r.dev.cache.clone()
    model = ring.RingModel(g.window_frames, g.tokens_per_frame, sink_frames=g.sink_frames)
    T, dc = g.tokens_per_frame, g.d_c
    frames = {}
    for k in range(6):
        x = r.x(chunk=k)
        for i in range(g.chunk_frames):
            frames[model.n + i] = x[0].reshape(g.chunk_frames, T, g.hidden)[i]
        rows_c = to_np(r.dev.compress(to_dev(x, g), model.n))[0][:, :dc]  # c does not depend on rotation
        r.dev.append(to_dev(x, g))
        model.append(g.chunk_frames)
        torch.cuda.synchronize()
        cache = to_np(r.dev.cache)[0]
        for slot, f in model.slot_map().items():
            got = cache[slot * T:(slot + 1) * T]
            if f >= model.n - g.chunk_frames:  # written by this append: c byte-identical to the compress rows
                i = f - (model.n - g.chunk_frames)
                np.testing.assert_array_equal(got[:, :dc], rows_c[i * T:(i + 1) * T])
            # k_r is stored before rotation: compare with the oracle's un-rotated k^
            _, kr_hat = mla.latents(frames[f].astype(np.float64), r.w.w_dkv.astype(np.float64),
                                    r.w.w_kr.astype(np.float64))
            assert np.abs(got[:, dc:] - kr_hat).max() <= 2 ** -8 * np.abs(kr_hat).max() + 1e-6, (slot, f)
        for slot in range(g.sink_frames + g.window_frames):
            if slot not in model.slot_map():
                assert torch.equal(r.dev.cache[:, slot * T:(slot + 1) * T], canary[:, slot * T:(slot + 1) * T])
        assert model.slot_map().get(0) == 0  # the sink stays


def _rollout(g, modes, n_chunks, expanded=False):
    for mode in modes:
        r = Rollout(g, mode=mode, cache_fill=float("nan"))
        for k in range(n_chunks):
            x = r.x(chunk=300 + k)
            _case("sink attend", g.name, mode, "n=", r.n, "expanded=", expanded)
            if expanded:
                r.dev.expand()
                got = to_np(r.dev.attend_expanded(to_dev(x, g)))
            else:
                got = r.attend(x)
            for b in range(g.batch):
                ma, mr = r.check(got[b], x, b, what=f"{g.name} {mode} n={r.n} b={b}")
                print(f"  b={b}: max_abs={ma:.3e} mean_rel={mr:.3e}", flush=True)
            r.append(r.x(chunk=k))


@pytest.mark.parametrize("g", [TINY_SINK, TINY_SINK_BF16], ids=lambda g: g.name)
def test_sink_tiny_all_window_states(g):
    # S=1, W=2, C=1: empty, sink only, partial, full, then the window slides past the pinned sink
    _rollout(g, ["literal", "unit", "sharp"], n_chunks=7)


@pytest.mark.parametrize("mode", ["literal", "unit", "sharp"])
def test_sink_wan_widths_small_grid(mode):
    _rollout(SMALL_SINK, [mode], n_chunks=5)


@pytest.mark.parametrize("dc", [96, 448])
def test_sink_other_latent_widths(dc):
    # the assembly pass and rotation at use with the other built latent widths
    _rollout(SMALL_SINK.replace(name=f"wan-widths-grid6x10-sink1-w3-dc{dc}", d_c=dc), ["sharp"], n_chunks=5)


def test_rope_at_use_without_sink():
    _rollout(wl.WAN_SMALL_GRID.replace(name="wan-widths-grid6x10-rope-at-use", rope_at_use=True), ["sharp"],
             n_chunks=4)


def test_sink_expanded_path():
    _rollout(SMALL_SINK, ["sharp"], n_chunks=5, expanded=True)


def test_sink_wan_layer_full_size_sampled():
    g = wl.WAN_SINK
    _case("sink wan-full")
    r = Rollout(g, mode="literal", cache_fill=float("nan"))
    for k in range(g.prefill_chunks):
        r.append(r.x(chunk=k))
    assert r.dev.state() == (21, 15, 7)
    x = r.x(chunk=g.prefill_chunks)
    got = r.attend(x)
    q = np.unique(np.concatenate([np.arange(8), np.arange(g.n_q - 8, g.n_q),
                                  np.random.default_rng(0).choice(g.n_q, 32, replace=False)]))
    ma, mr = r.check(got[0][q], x, 0, q, "sink wan-full literal")
    print(f"sink wan-full: max_abs={ma:.3e} mean_rel={mr:.3e}", flush=True)
