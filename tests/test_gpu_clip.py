"""Block-causal attention over a whole clip (vmla_attend_clip) against the
oracle's attend_clip: chunk q of the clip attends to chunks 0..q (the
training-time form of the layer).  Cases: the tiny fp32 layer, the Wan widths
on a 6x10 grid with a 5-frame clip in 3-frame chunks (a shorter last block,
row blocks straddling block boundaries; d_c = 192, 96 and 448), and the full 21-frame Wan clip
(32,760 tokens, 7 blocks) on sampled queries of three blocks, in the layer
recipe and the sharpened one.  Same bar as the other GPU tests (gpu_harness)."""
import numpy as np
import pytest

import rounding as rd
from gpu_harness import Rollout, assert_parity, to_dev, to_np
from mla_latent_kv_vmla_amd import workloads as wl
from oracle import mla

pytestmark = pytest.mark.gpu


def _clip_x(g, mode, seed=0):
    return wl.hidden_states(g.replace(chunk_frames=g.window_frames), chunk=500, mode=mode, seed=seed)


@pytest.mark.parametrize("g,mode", [(wl.TINY, "sharp"), (wl.WAN_SMALL_GRID, "literal"), (wl.WAN_SMALL_GRID, "sharp"),
                                    (wl.WAN_SMALL_GRID.replace(name="wan-widths-grid6x10-dc96", d_c=96), "sharp"),
                                    (wl.WAN_SMALL_GRID.replace(name="wan-widths-grid6x10-dc448", d_c=448), "sharp")],
                         ids=["tiny-sharp", "grid6x10-literal", "grid6x10-sharp", "grid6x10-dc96-sharp",
                              "grid6x10-dc448-sharp"])
def test_clip_matches_oracle(g, mode):
    print("case: clip", g.name, mode, flush=True)
    r = Rollout(g, mode=mode, cache_fill=float("nan"))
    x = _clip_x(g, mode)
    got = to_np(r.dev.attend_clip(to_dev(x, g)))
    assert r.dev.state() == (0, 0, 0)  # the cache and counter are untouched
    ref = mla.attend_clip(g, r.w, x[0])
    fl = rd.floor_clip(g, r.w, x[0], ref=ref) if g.dtype == wl.BF16 else None
    ma, mr = assert_parity(got[0], ref, f"clip {g.name} {mode}", fl)
    print(f"  max_abs={ma:.3e} mean_rel={mr:.3e}", flush=True)


@pytest.mark.parametrize("mode", ["literal", "sharp"])
def test_clip_wan_full_size_sampled(mode):
    g = wl.WAN_LAYER
    print("case: clip wan-full", mode, flush=True)
    r = Rollout(g, mode=mode)
    x = _clip_x(g, mode)
    got = to_np(r.dev.attend_clip(to_dev(x, g)))[0]
    assert np.all(np.isfinite(got))
    T, C, F = g.tokens_per_frame, g.chunk_frames, g.window_frames
    frames = x[0].reshape(F, T, g.hidden)
    rng = np.random.default_rng(5)
    for q in (0, 3, 6):
        q0 = q * C
        sample = np.unique(np.concatenate([[0, C * T - 1], rng.choice(C * T, 30, replace=False)]))
        hist = {f: frames[f] for f in range(q0)}
        ref = mla.attend(g, r.w, hist, q0, x[0][q0 * T:(q0 + C) * T], query_tokens=sample)
        fl = rd.floor(g, r.w, hist, q0, x[0][q0 * T:(q0 + C) * T], sample, ref=ref)
        ma, mr = assert_parity(got[q0 * T + sample], ref, f"clip wan block {q} {mode}", fl)
        print(f"  block {q}: max_abs={ma:.3e} mean_rel={mr:.3e}", flush=True)
