"""Parity on seeded random geometries at the Wan widths (12 heads x 128, hidden
1536, d_rope 32 in (4, 6, 6) pairs), against the CPU oracle on every query
token of every stream.

Each case draws:
- a latent frame grid from 1x1 up to 7x11 (tokens per frame from 1 to 77, so
  key tiles and row blocks end at arbitrary offsets);
- a window of 1-6 frames, chunks of 1-3 frames (at most the window) and 0-2
  pinned sink frames (rotation at use);
- 1-3 streams, a built latent width d_c in {96, 192, 448}, and 0 (default),
  1, 5 or 64 attention workgroups (different stream-K cuts);
- 0-5 appends before the attend, so the window is empty, partial, full or
  wrapped.
The expanded path is checked on the same state.  The sharpened query
projection makes the softmax peaked, so online rescaling is exercised.  A
fixed degenerate case adds the smallest geometry: one token per frame with
one-frame windows and chunks, at every built d_c, with and without a sink.  Same
bar and tolerance derivation as the other GPU tests (gpu_harness).
"""
import numpy as np
import pytest

from gpu_harness import Rollout, to_dev, to_np
from mla_latent_kv_vmla_amd import workloads as wl

pytestmark = pytest.mark.gpu

N_CASES = 24


def _draw(i):
    rng = np.random.default_rng(1000 + i)
    W = int(rng.integers(1, 7))
    S = int(rng.integers(0, 3))
    g = wl.WAN_LAYER.replace(
        name=f"random-{i}", batch=int(rng.integers(1, 4)), grid_h=int(rng.integers(1, 8)),
        grid_w=int(rng.integers(1, 12)), window_frames=W, chunk_frames=int(rng.integers(1, min(3, W) + 1)),
        d_c=int(rng.choice([96, 192, 448])), sink_frames=S, rope_at_use=S > 0)
    return g, int(rng.choice([0, 1, 5, 64])), int(rng.integers(0, 6))


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_geometry(i):
    g, G, appends = _draw(i)
    print(f"case: random {i}: B={g.batch} grid={g.grid_h}x{g.grid_w} W={g.window_frames} C={g.chunk_frames} "
          f"S={g.sink_frames} d_c={g.d_c} G={G} appends={appends}", flush=True)
    r = Rollout(g, mode="sharp", seed=i, attn_workgroups=G, cache_fill=float("nan"))
    for k in range(appends):
        r.append(r.x(chunk=k))
    x = r.x(chunk=77)
    got = r.attend(x)
    r.dev.expand()
    got_exp = to_np(r.dev.attend_expanded(to_dev(x, g)))
    for b in range(g.batch):
        ma, mr = r.check(got[b], x, b, what=f"random {i} absorbed b={b}")
        mae, mre = r.check(got_exp[b], x, b, what=f"random {i} expanded b={b}")
        print(f"  b={b}: absorbed max_abs={ma:.3e} mean_rel={mr:.3e}; expanded max_abs={mae:.3e} "
              f"mean_rel={mre:.3e}", flush=True)
    r.dev.close()


@pytest.mark.parametrize("dc", [96, 192, 448])
@pytest.mark.parametrize("sink", [0, 1])
def test_degenerate_single_token_frames(dc, sink):
    """The smallest geometry: one token per frame, a one-frame window and a
    one-frame chunk (12 query rows against 2 keys; with a sink, 3), two streams,
    through empty, full and sliding windows."""
    g = wl.WAN_LAYER.replace(name=f"one-token-dc{dc}-s{sink}", batch=2, grid_h=1, grid_w=1, window_frames=1,
                             chunk_frames=1, d_c=dc, sink_frames=sink, rope_at_use=sink > 0)
    print(f"case: one-token frames d_c={dc} sink={sink}", flush=True)
    r = Rollout(g, mode="sharp", seed=dc + sink, cache_fill=float("nan"))
    for k in range(4):
        x = r.x(chunk=50 + k)
        got = r.attend(x)
        r.dev.expand()
        got_exp = to_np(r.dev.attend_expanded(to_dev(x, g)))
        for b in range(g.batch):
            r.check(got[b], x, b, what=f"one-token d_c={dc} sink={sink} n={r.n} b={b}")
            r.check(got_exp[b], x, b, what=f"one-token expanded d_c={dc} sink={sink} n={r.n} b={b}")
        r.append(r.x(chunk=k))
    r.dev.close()
