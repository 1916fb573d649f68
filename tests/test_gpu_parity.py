"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Cases span several attention row blocks and key tiles with ragged tails, partial
and wrapped windows, fp32 and bf16 storage, three input scalings, batched
streams, every stream-K split shape, the paper's (6, 5, 5) rotary allocation
and explicit frequency tables, a cached element beyond fp16's range, and the
full Wan-1.3B layer (every query token, two input scalings) in the launch
configuration the benchmark times.
"""
import json
import os

import numpy as np
import pytest

import rounding as rd
from gpu_harness import Rollout, assert_parity, to_dev, to_np
from mla_latent_kv_vmla_amd import workloads as wl
from oracle import mla, ring

pytestmark = pytest.mark.gpu

TINY_BF16 = wl.TINY.replace(name="tiny-bf16", dtype=wl.BF16)
SMALL = wl.WAN_SMALL_GRID


def _print_case(*a):
    print("case:", *a, flush=True)


@pytest.mark.parametrize("g", [wl.TINY, TINY_BF16, SMALL, wl.WAN_LAYER], ids=lambda g: g.name)
def test_compress_rows_match_oracle(g):
    _print_case("compress", g.name)
    r = Rollout(g, mode="unit")
    x = r.x(chunk=5)
    frame0 = 13
    got = to_np(r.dev.compress(to_dev(x, g), frame0))
    for b in range(g.batch):
        ref = mla.chunk_latents(g, r.w, x[b], frame0)
        scale = np.abs(ref).max()
        if g.dtype == wl.F32:
            tol = 1e-5 * np.abs(ref) + 1e-6 * scale
        else:  # one bf16 rounding of an fp32-accumulated value
            tol = 2.0 ** -8 * np.abs(ref) + 1e-5 * scale
        bad = np.abs(got[b] - ref) > tol
        assert not bad.any(), f"{bad.sum()} latent entries off; worst {np.abs(got[b] - ref).max():.3e}"


@pytest.mark.parametrize("g", [wl.TINY, SMALL.replace(window_frames=5, chunk_frames=2),
                               SMALL.replace(window_frames=4, chunk_frames=4)],
                         ids=["tiny-W2C1", "W5C2", "W4C4"])
def test_ring_append_bit_exact(g):
    """Append writes each frame's rows into slot f % W, byte-identical to the rows
    the compress hook produces for that frame, and leaves every other slot alone."""
    import torch
    _print_case("ring", g.name, g.window_frames, g.chunk_frames)
    r = Rollout(g, mode="unit", cache_fill=-5.0)
    canary = r.dev.cache.clone()
    model = ring.RingModel(g.window_frames, g.tokens_per_frame)
    T = g.tokens_per_frame
    rows_of_frame = {}
    for k in range(9):
        x = r.x(chunk=k)
        xd = to_dev(x, g)
        expect = r.dev.compress(xd, model.n)  # [B, C*T, D]
        for i in range(g.chunk_frames):
            rows_of_frame[model.n + i] = expect[:, i * T:(i + 1) * T].clone()
        r.dev.append(xd)
        model.append(g.chunk_frames)
        torch.cuda.synchronize()
        n, first, nvalid = r.dev.state()
        assert (n, first, nvalid) == (model.n, max(0, model.n - model.W), len(model.valid_frames()))
        occupied = model.slot_map()
        for slot in range(g.window_frames):
            got = r.dev.cache[:, slot * T:(slot + 1) * T]
            want = rows_of_frame[occupied[slot]] if slot in occupied else canary[:, slot * T:(slot + 1) * T]
            assert torch.equal(got.view(torch.int16 if got.dtype == torch.bfloat16 else torch.int32),
                               want.view(torch.int16 if want.dtype == torch.bfloat16 else torch.int32)), \
                f"slot {slot} after append {k}"


def _rollout_parity(g, modes, n_chunks, attn_workgroups=0, query_tokens=None):
    for mode in modes:
        r = Rollout(g, mode=mode, attn_workgroups=attn_workgroups, cache_fill=float("nan"))
        for k in range(n_chunks):
            x = r.x(chunk=100 + k)
            _print_case("attend", g.name, mode, "n=", r.n, "G=", attn_workgroups)
            got = r.attend(x)
            for b in range(g.batch):
                gb = got[b] if query_tokens is None else got[b][query_tokens]
                ma, mr = r.check(gb, x, b, query_tokens, f"{g.name} {mode} n={r.n} b={b}")
                print(f"  b={b}: max_abs={ma:.3e} mean_rel={mr:.3e}", flush=True)
            r.append(r.x(chunk=k))


@pytest.mark.parametrize("g", [wl.TINY, TINY_BF16], ids=lambda g: g.name)
def test_attend_tiny_all_window_states(g):
    # W=2, C=1: empty window, partial window, full, then wrapped several times
    _rollout_parity(g, ["literal", "unit", "sharp"], n_chunks=6)


@pytest.mark.parametrize("mode", ["literal", "unit", "sharp"])
def test_attend_wan_widths_small_grid(mode):
    # 180 queries x 12 heads = 2160 rows (8.4 row blocks of 256); 180..480 keys (ragged tiles)
    _rollout_parity(SMALL, [mode], n_chunks=4)


@pytest.mark.parametrize("G", [1, 3, 7, 64, 100000])
def test_attend_stream_k_splits(G):
    """Every way of cutting (row block, key tile) work across workgroups gives the
    same answer: one workgroup for everything, uneven cuts, one tile each."""
    _rollout_parity(SMALL, ["sharp"], n_chunks=3, attn_workgroups=G)


@pytest.mark.parametrize("dc", [96, 192, 448])
def test_attend_batched_streams_latent_widths(dc):
    g = wl.STRESS[dc].replace(grid_h=6, grid_w=10, window_frames=7)
    _rollout_parity(g, ["sharp"], n_chunks=4)


def test_attend_wan_layer_full_size_every_token():
    """The benchmark's workload: 21 cached frames (32,760 keys) + 3-frame chunk
    (4,680 queries x 12 heads), default launch configuration; every query token
    is compared, in the layer recipe and the sharpened one."""
    g = wl.WAN_LAYER
    for mode in ["literal", "sharp"]:
        _print_case("wan-full", mode)
        r = Rollout(g, mode=mode, cache_fill=float("nan"))
        for k in range(g.prefill_chunks):
            r.append(r.x(chunk=k))
        assert r.n == 21
        x = r.x(chunk=g.prefill_chunks)
        got = r.attend(x)
        assert np.all(np.isfinite(got))
        _print_case("wan-full", mode, "oracle")
        ma, mr = r.check(got[0], x, 0, None, f"wan-full {mode}")
        print(f"wan-full {mode}: max_abs={ma:.3e} mean_rel={mr:.3e}", flush=True)
        assert r.dev.range_flags() == 0
        r.dev.close()


def _bands(pairs):
    gold = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "rope_bands.json")))
    return tuple(gold["tables"]["%d,%d,%d" % pairs])


# The paper's own allocation of the decoupled key's 16 rotary pairs, (6, 5, 5)
# over (t, h, w) (section 4.1), and explicit frequency tables passed through
# vmla_create: the highest-frequency bands of the backbone's per-axis spectrum
# (tests/golden/rope_bands.json), for both allocations.
ROPE_VARIANTS = {
    "rope655": dict(rope_pairs=(6, 5, 5)),
    "bands466": dict(rope_freqs=_bands((4, 6, 6))),
    "bands655": dict(rope_pairs=(6, 5, 5), rope_freqs=_bands((6, 5, 5))),
}


@pytest.mark.parametrize("variant", sorted(ROPE_VARIANTS))
def test_attend_rope_variants_small_grid(variant):
    g = SMALL.replace(name=f"{SMALL.name}-{variant}", **ROPE_VARIANTS[variant])
    _rollout_parity(g, ["unit", "sharp"], n_chunks=4)


@pytest.mark.parametrize("variant", sorted(ROPE_VARIANTS))
def test_attend_rope_variants_wan_layer_sampled(variant):
    """Full Wan layer with the variant's rotary allocation/table, sharpened
    recipe (scores sensitive to the rotary term), 96 sampled query tokens."""
    g = wl.WAN_LAYER.replace(name=f"wan1.3b-layer-{variant}", **ROPE_VARIANTS[variant])
    _print_case("wan-full", variant)
    r = Rollout(g, mode="sharp", cache_fill=float("nan"))
    for k in range(g.prefill_chunks):
        r.append(r.x(chunk=k))
    x = r.x(chunk=g.prefill_chunks)
    got = r.attend(x)
    q = np.unique(np.concatenate([np.arange(8), np.arange(g.n_q - 8, g.n_q),
                                  np.random.default_rng(3).choice(g.n_q, 80, replace=False)]))
    ma, mr = r.check(got[0][q], x, 0, q, f"wan-full {variant}")
    print(f"wan-full {variant}: max_abs={ma:.3e} mean_rel={mr:.3e}", flush=True)
    r.dev.close()


def test_fp16_range_saturation_is_flagged():
    """A cached latent element beyond fp16's range (bf16 holds it; the fp16 key
    tiles cannot): the library saturates it to 65504, raises the range flag, and
    the output is the attention over the saturated cache."""
    import torch
    g = SMALL
    _print_case("range", g.name)
    r = Rollout(g, mode="unit", cache_fill=float("nan"))
    r.append(r.x(chunk=0))
    x = r.x(chunk=9)
    base = r.attend(x)
    assert r.dev.range_flags() == 0
    # frame 2 (slot 2), token 17: with n = 3 < W the ring row is also the visible key index
    row, ch = 2 * g.tokens_per_frame + 17, 5
    r.dev.cache[0, row, ch] = 1.0e6
    torch.cuda.synchronize()
    got = r.attend(x)
    assert r.dev.range_flags() == 1
    assert r.dev.range_flags() == 0  # reading clears it

    def saturate(c, kr):
        c[row, ch] = 65504.0
        return c, kr

    ref = rd.emulate(g, r.w, r.hist[0], r.n, x[0], edit=saturate)
    fl = rd.floor(g, r.w, r.hist[0], r.n, x[0], ref=ref, edit=saturate)
    # The saturated element dominates the rows that favour it, whose outputs reach
    # ~5e3 (the layer recipe's are ~1e-2): the relative metric carries the bound,
    # and the largest error is held to 2e-2 of the largest output.
    ma, mr = rd.parity(got[0], ref)
    assert np.all(np.isfinite(got[0]))
    assert mr <= rd.bounds(fl)[1], (mr, fl)
    assert ma <= rd.MAX_ABS * np.abs(ref).max(), (ma, np.abs(ref).max())
    print(f"  saturated: max_abs={ma:.3e} (max |ref| {np.abs(ref).max():.3e}) mean_rel={mr:.3e}", flush=True)
    assert np.abs(got[0] - base[0]).max() > 1.0  # the element dominates the queries that favour it
    r.dev.close()


def test_fp16_range_saturation_of_hidden_states_is_flagged():
    """A hidden-state element beyond fp16's range (2^20; bf16 holds it): the
    chunk GEMM stages x as fp16, so the element saturates to 65504 there, the
    range flag goes up, and the output is the attention of the saturated chunk
    (in an attend, x only feeds the chunk's own rows and queries).  The layer
    recipe keeps the other elements small, so the saturated token dominates
    only the scores it takes part in; the comparison takes the usual
    floor-based bound of that case."""
    g = SMALL
    _print_case("range-x", g.name)
    r = Rollout(g, mode="literal", cache_fill=float("nan"))
    r.append(r.x(chunk=0))
    r.append(r.x(chunk=1))
    x = r.x(chunk=9)
    base = r.attend(x)
    assert r.dev.range_flags() == 0
    tok, ch = 41, 7
    x[0, tok, ch] = 2.0 ** 20
    got = r.attend(x)
    assert r.dev.range_flags() == 1
    assert r.dev.range_flags() == 0
    xs = x.copy()
    xs[0, tok, ch] = 65504.0
    ref = mla.attend(g, r.w, r.hist[0], r.n, xs[0])
    fl = rd.floor(g, r.w, r.hist[0], r.n, xs[0], ref=ref)
    ma, mr = assert_parity(got[0], ref, "saturated x", fl)
    print(f"  saturated x: max_abs={ma:.3e} (max |ref| {np.abs(ref).max():.3e}) mean_rel={mr:.3e}", flush=True)
    assert np.abs(got[0] - base[0]).max() > 1.0
    r.dev.close()
