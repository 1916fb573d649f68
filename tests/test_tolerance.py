"""CPU pins of the parity bound (tests/rounding.py): the rounding emulation is the
oracle's arithmetic, the library's rounding sequence stays inside the bound on
every input recipe, and the bound rejects the earlier bf16-intermediate
sequence on the steep recipe it was loosened for."""
import numpy as np
import pytest

import rounding as rd
from mla_latent_kv_vmla_amd import workloads as wl
from oracle import mla

SMALL = wl.WAN_SMALL_GRID


def _case(g, mode, appends, seed=0):
    w = wl.latent_weights(g, seed=seed, mode=mode)
    hist, n = {}, 0
    for k in range(appends):
        x = wl.hidden_states(g, chunk=k, seed=seed, mode=mode)[0].reshape(g.chunk_frames, g.tokens_per_frame,
                                                                          g.hidden)
        for i in range(g.chunk_frames):
            hist[n + i] = x[i]
        n += g.chunk_frames
    return w, hist, n, wl.hidden_states(g, chunk=50, seed=seed, mode=mode)[0]


@pytest.mark.parametrize("g", [wl.TINY, SMALL, wl.WAN_SINK.replace(grid_h=3, grid_w=5)], ids=lambda g: g.name)
def test_emulation_without_rounding_is_the_oracle(g):
    w, hist, n, x = _case(g, "unit", 4)
    ref = mla.attend(g, w, hist, n, x)
    got = rd.emulate(g, w, hist, n, x, steps={})
    assert np.allclose(got, ref, rtol=1e-10, atol=1e-12 * np.abs(ref).max())


def test_output_rounding_alone_is_the_rounded_oracle():
    g = SMALL
    w, hist, n, x = _case(g, "sharp", 3)
    ref = mla.attend(g, w, hist, n, x)
    got = rd.emulate(g, w, hist, n, x, steps={"u": "bf16"})
    # identical up to the float64 rounding of the two computations, then one bf16 rounding
    assert np.array_equal(got, rd.round_to(ref, "bf16")) or \
        np.mean(got != rd.round_to(ref, "bf16")) < 1e-3


def test_round_to_nearest_even():
    # 1 + 2^-8 lies halfway between bf16 neighbours 1 and 1 + 2^-7: ties go to the even one (1)
    assert rd.round_to(1 + 2.0 ** -8, "bf16") == 1.0
    assert rd.round_to(1 + 3 * 2.0 ** -8, "bf16") == 1 + 2 * 2.0 ** -7
    assert rd.round_to(1 + 2.0 ** -11, "fp16") == 1.0
    assert rd.round_to(-3.0, "bf16") == -3.0


@pytest.mark.parametrize("mode", ["literal", "unit", "sharp"])
@pytest.mark.parametrize("appends", [0, 2, 4])
def test_library_rounding_sequence_within_bound(mode, appends):
    """The fp16-intermediate sequence stays within max(bar, 1.1 x floor)."""
    g = SMALL
    w, hist, n, x = _case(g, mode, appends)
    ref = mla.attend(g, w, hist, n, x)
    fl = rd.floor(g, w, hist, n, x, ref=ref)
    ma, mr = rd.parity(rd.emulate(g, w, hist, n, x, steps=rd.AS_BUILT), ref)
    ba, br = rd.bounds(fl)
    assert ma <= ba and mr <= br, (ma, mr, ba, br, fl)
    # and it spends little beyond the unavoidable roundings
    assert mr <= 1.06 * fl[1], (mr, fl)


def _steep_cases():
    """Small steep cases where the output sample is small and single errors
    matter: the tiny layer with and without a sink at every window state, and
    the 24 seeded random geometries of the GPU parity tests."""
    from test_gpu_random_geometries import _draw
    tiny = wl.TINY.replace(name="tiny-bf16", dtype=wl.BF16)
    tiny_sink = tiny.replace(name="tiny-sink-bf16", sink_frames=1, rope_at_use=True)
    out = [(g, 0, n) for n in range(7) for g in (tiny, tiny_sink)]
    for i in range(24):
        g, _, appends = _draw(i)
        out.append((g, i, appends))
    return out


def test_library_rounding_sequence_within_bound_on_small_steep_cases():
    ratios = []
    for g, seed, appends in _steep_cases():
        w = wl.latent_weights(g, seed=seed, mode="sharp")
        hist, n = [dict() for _ in range(g.batch)], 0
        for k in range(appends):
            x = wl.hidden_states(g, chunk=k, seed=seed, mode="sharp")
            for b in range(g.batch):
                fr = x[b].reshape(g.chunk_frames, g.tokens_per_frame, g.hidden)
                for i in range(g.chunk_frames):
                    hist[b][n + i] = fr[i]
            n += g.chunk_frames
        x = wl.hidden_states(g, chunk=77, seed=seed, mode="sharp")
        for b in range(g.batch):
            ref = mla.attend(g, w, hist[b], n, x[b])
            fl = rd.floor(g, w, hist[b], n, x[b], ref=ref)
            ma, mr = rd.parity(rd.emulate(g, w, hist[b], n, x[b], steps=rd.AS_BUILT), ref)
            ba, br = rd.bounds(fl)
            assert ma <= ba and mr <= br, (g.name, n, b, ma, mr, fl)
            ratios.append((ma / fl[0], mr / fl[1]))
    r = np.asarray(ratios)
    print(f"as-built / floor over {len(r)} comparisons: max_abs up to {r[:, 0].max():.3f}, "
          f"mean_rel up to {r[:, 1].max():.3f}")
    assert r[:, 1].max() < rd.SLACK_MEAN and r[:, 0].max() < rd.SLACK_MAX


def test_bound_rejects_bf16_intermediates_on_steep_scores():
    """The earlier rounding sequence (bf16 c^Q, q_nope, absorbed query, latent
    and per-head outputs) exceeds the bound on the sharpened recipe, so the
    bound is tight enough to tell the two builds apart."""
    g = SMALL
    w, hist, n, x = _case(g, "sharp", 4)
    ref = mla.attend(g, w, hist, n, x)
    ma, mr = rd.parity(rd.emulate(g, w, hist, n, x, steps=rd.BF16_INTERMEDIATES), ref)
    ba, br = rd.bounds(rd.floor(g, w, hist, n, x, ref=ref))
    assert mr > br, (mr, br)


def test_floor_below_bar_for_the_layer_recipe():
    """On the layer recipe itself (hidden states N(0,1)/sqrt(hidden)) the
    unavoidable roundings sit well inside the stated bar, so the stated bar is
    what those comparisons are held to."""
    g = SMALL
    w, hist, n, x = _case(g, "literal", 4)
    fl = rd.floor(g, w, hist, n, x)
    assert fl[1] < 0.6 * rd.MEAN_REL and rd.bounds(fl) == (rd.MAX_ABS, rd.MEAN_REL)
