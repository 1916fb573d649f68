"""Pins of the CPU oracle to what the VideoMLA pages and mathematics fix.

Each test checks the oracle against something other than itself: figures the
pages print (tests/golden/page_figures.json), a library routine on a special
case, closed forms, invariants, or an independent brute force.
"""
import collections
import json
import math
import os
from types import SimpleNamespace

import numpy as np
import pytest

from oracle import brute, mla, ring, sizes
from mla_latent_kv_vmla_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
GOLD = json.load(open(os.path.join(GOLDEN, "page_figures.json")))


def gv(k):
    return GOLD[k]["value"]


def rounded(x, k):
    return round(x, GOLD[k].get("digits", 0))


# ----------------------------------------------------------------------------- sizes
def test_per_token_sizes_match_pages():
    nh, dh, dc, dr = gv("wan_heads"), gv("wan_head_dim"), gv("d_c"), gv("d_rope")
    assert sizes.dense_scalars_per_token(nh, dh) == gv("dense_scalars_per_token")
    assert sizes.latent_scalars_per_token(dc, dr) == gv("latent_scalars_per_token")
    assert rounded(100 * sizes.reduction_fraction(nh, dh, dc, dr), "reduction_percent") == gv("reduction_percent")
    assert rounded(sizes.reduction_factor(nh, dh, dc, dr), "reduction_factor") == gv("reduction_factor")
    assert gv("d_nope") + gv("d_rope") == dh


def test_token_grid_and_clip_match_pages():
    gh, gw = sizes.token_grid(*gv("clip_resolution"), 8, gv("patch_size")[1:])
    assert (gh * 2, gw * 2) == tuple(gv("vae_latent_grid"))
    assert gh * gw == gv("tokens_per_frame")
    assert gv("latent_frames_per_clip") * gh * gw == gv("tokens_per_clip")
    g = wl.WAN_LAYER
    assert (g.grid_h, g.grid_w) == (gh, gw)
    assert g.window_frames == gv("latent_frames_per_clip") and g.chunk_frames == gv("chunk_frames")


def test_dense_cache_size_matches_pages():
    T = gv("tokens_per_frame")
    n = sizes.cache_scalars(gv("wan_layers"), gv("latent_frames_per_clip"), T, gv("dense_scalars_per_token"))
    assert n == 3_019_161_600
    assert rounded(n / 1e9, "dense_cache_scalars_billion") == gv("dense_cache_scalars_billion")
    b = sizes.cache_bytes(gv("wan_layers"), gv("latent_frames_per_clip"), T, gv("dense_scalars_per_token"), 2)
    assert rounded(b / 1e9, "dense_cache_gb_bf16") == gv("dense_cache_gb_bf16")


def test_layer_cut_comparison_matches_pages():
    L, Lc = gv("wan_layers"), gv("scd_cached_layers")
    assert rounded(100 * sizes.layer_cut_fraction(Lc, L), "scd_cut_percent") == gv("scd_cut_percent")
    r = sizes.ratio_vs_partial_dense(Lc, L, gv("wan_heads"), gv("wan_head_dim"), gv("d_c"), gv("d_rope"))
    assert rounded(r, "vs_scd_factor") == gv("vs_scd_factor")


def test_sink_window_geometry_matches_pages():
    T = gv("tokens_per_frame")
    assert 1 * T == gv("sink_slots")
    assert gv("local_window_frames") * T == gv("local_window_slots")
    assert sum(gv("rope_pairs_paper")) * 2 == gv("d_rope")
    assert sum(wl.WAN_LAYER.rope_pairs) * 2 == gv("d_rope")


# ----------------------------------------------------------------------------- RoPE
def test_rope_frequencies_closed_form():
    # theta^(-2i/(2p)) per axis, written out by hand for theta = 1e4
    f = mla.rope_frequencies((4, 6, 6), 1e4)
    h6 = [1.0, 10 ** (-4 / 6), 10 ** (-8 / 6), 1e-2, 10 ** (-16 / 6), 10 ** (-20 / 6)]
    np.testing.assert_allclose(f, [1.0, 0.1, 0.01, 0.001] + h6 + h6, rtol=1e-14)
    np.testing.assert_allclose(mla.rope_frequencies((1, 1, 2), 1e4), [1.0, 1.0, 1.0, 0.01], rtol=1e-14)
    assert list(mla.pair_axes((1, 1, 2))) == [0, 1, 2, 2]


def test_backbone_band_frequencies_closed_form():
    """Leading bands of a wider per-axis spectrum, written out by hand: axis
    dims (44, 42, 42) at theta = 1e4 give omega = 10^(-8i/44) on t and
    10^(-8i/42) on h and w."""
    f = mla.backbone_band_frequencies((6, 5, 5), (44, 42, 42), 1e4)
    t = [10 ** (-8 * i / 44) for i in range(6)]
    hw = [10 ** (-8 * i / 42) for i in range(5)]
    np.testing.assert_allclose(f, t + hw + hw, rtol=1e-14)
    np.testing.assert_allclose(f[:2], [1.0, 0.657933224657568], rtol=1e-14)
    # an axis spectrum exactly as wide as the key's pairs is the default table
    np.testing.assert_array_equal(mla.backbone_band_frequencies((4, 6, 6), (8, 12, 12), 1e4),
                                  mla.rope_frequencies((4, 6, 6), 1e4))
    # the golden tables the GPU tests pass to the library were written from this function
    gold = json.load(open(os.path.join(GOLDEN, "rope_bands.json")))
    for key, table in gold["tables"].items():
        pairs = tuple(int(v) for v in key.split(","))
        np.testing.assert_allclose(table, mla.backbone_band_frequencies(pairs, tuple(gold["axis_dims"]),
                                                                        gold["theta"]), rtol=1e-15)


def test_explicit_rope_table_is_used_everywhere():
    """A geometry's explicit table: equal to the default when it is the default
    table, and followed identically by the numpy oracle and the brute force
    (complex rotation per pair) when it is not."""
    g = wl.TINY
    for n in (0, 3):
        w, hist, chunk = _tiny_inputs(n)
        base = mla.attend(g, w, hist, n, chunk)
        same = mla.attend(g.replace(rope_freqs=tuple(mla.rope_frequencies(g.rope_pairs, g.rope_theta))), w, hist, n,
                          chunk)
        np.testing.assert_array_equal(same, base)
        gt = g.replace(rope_freqs=(0.9, 0.35, 0.6, 0.05))
        ref = mla.attend(gt, w, hist, n, chunk)
        bf = np.asarray(brute.attend(gt, w, hist, n, chunk))
        np.testing.assert_allclose(ref, bf, rtol=1e-11, atol=1e-13)
        if n:
            assert np.abs(ref - base).max() > 1e-6  # the table changes the result


def test_rope_norm_identity_and_relative_invariance():
    rng = np.random.default_rng(0)
    pairs = (4, 6, 6)
    fr = mla.rope_frequencies(pairs, 1e4)
    q, k = rng.standard_normal((50, 32)), rng.standard_normal((50, 32))
    cq, ck = rng.integers(0, 40, (50, 3)), rng.integers(0, 40, (50, 3))
    rq = mla.rope_rotate(q, cq, pairs, fr)
    np.testing.assert_allclose(np.linalg.norm(rq, axis=1), np.linalg.norm(q, axis=1), rtol=1e-13)
    np.testing.assert_array_equal(mla.rope_rotate(q, np.zeros((50, 3), int), pairs, fr), q)
    s0 = rq @ mla.rope_rotate(k, ck, pairs, fr).T
    for axis in range(3):
        d = np.zeros(3, int)
        d[axis] = 17
        s1 = mla.rope_rotate(q, cq + d, pairs, fr) @ mla.rope_rotate(k, ck + d, pairs, fr).T
        np.testing.assert_allclose(s1, s0, atol=1e-11)
        # negative control: moving only the keys changes the scores
        s2 = rq @ mla.rope_rotate(k, ck + d, pairs, fr).T
        assert np.abs(s2 - s0).max() > 1e-2


def _tiny_inputs(n, mode="unit", seed=0, g=wl.TINY):
    w = wl.latent_weights(g, seed=seed, mode=mode)
    hist = {f: wl.hidden_states(g, chunk=f, seed=seed, mode=mode)[0].reshape(g.chunk_frames, -1, g.hidden)[0]
            for f in range(n)} if g.chunk_frames == 1 else None
    chunk = wl.hidden_states(g, chunk=1000 + n, seed=seed, mode=mode)[0]
    return w, hist, chunk


def test_rope_scores_closed_form_complex():
    """With W_UK = 0 every score is the rotary term alone; compare it with the
    complex-number form Re(sum_p q_p conj(k_p) e^{i (pos_q - pos_k) omega_p})."""
    g, n = wl.TINY, 5
    w, hist, chunk = _tiny_inputs(n)
    w.w_uk = np.zeros_like(w.w_uk)
    s = mla.scores(g, w, hist, n, chunk)
    T, first = 16, n - g.window_frames
    frames = list(range(first, n)) + [n]
    xk = np.concatenate([hist[f] for f in range(first, n)] + [chunk]).astype(np.float64)
    kh = xk @ w.w_kr.T.astype(np.float64)
    qh = ((chunk.astype(np.float64) @ w.w_dq.T) @ w.w_uq.T).reshape(16, 2, 16)[:, :, 8:]
    pos_k = [(f - first, s_ // 4, s_ % 4) for f in frames for s_ in range(T)]
    pos_q = [(n - first, s_ // 4, s_ % 4) for s_ in range(T)]
    omega = [1.0, 1.0, 1.0, 0.01]
    axis = [0, 1, 2, 2]
    for h in range(2):
        for i in range(16):
            for j in range(len(pos_k)):
                z = 0j
                for p in range(4):
                    qz = complex(qh[i, h, 2 * p], qh[i, h, 2 * p + 1])
                    kz = complex(kh[j, 2 * p], kh[j, 2 * p + 1])
                    z += qz * kz.conjugate() * np.exp(1j * (pos_q[i][axis[p]] - pos_k[j][axis[p]]) * omega[p])
                assert abs(s[h, i, j] - z.real / 4.0) < 1e-12


def test_absolute_frame_rows_give_window_local_scores():
    """Cache rows rotated with the absolute frame index (as written at append)
    reproduce the window-local scores: relative-position invariance of 3D-RoPE."""
    g, n = wl.TINY, 7
    w, hist, chunk = _tiny_inputs(n, mode="sharp")
    ref = mla.scores(g, w, hist, n, chunk)
    first = n - g.window_frames
    rows = np.concatenate([mla.chunk_latents(g, w, hist[f], f) for f in range(first, n)]
                          + [mla.chunk_latents(g, w, chunk, n)])
    qn, qr = mla.query_heads(chunk.astype(np.float64), w.w_dq.astype(np.float64),
                             w.w_uq.astype(np.float64), 2, 8, 8)
    qc = mla.token_coordinates(np.array([n]), 4, 4)
    qr = mla.rope_rotate(qr, qc, g.rope_pairs, mla.rope_frequencies(g.rope_pairs, g.rope_theta))
    for h in range(2):
        s = (qn[:, h] @ w.w_uk[h].astype(np.float64) @ rows[:, :24].T + qr[:, h] @ rows[:, 24:].T) / 4.0
        np.testing.assert_allclose(s, ref[h], atol=1e-12)


# ----------------------------------------------------------------------------- attention
@pytest.mark.parametrize("n", [0, 1, 2, 3, 5])
@pytest.mark.parametrize("mode", ["literal", "unit", "sharp"])
def test_brute_force_matches_numpy(n, mode):
    g = wl.TINY
    w, hist, chunk = _tiny_inputs(n, mode)
    u = mla.attend(g, w, hist, n, chunk)
    ub = np.array(brute.attend(g, w, hist, n, chunk))
    np.testing.assert_allclose(u, ub, rtol=1e-12, atol=1e-14 * np.abs(ub).max())


@pytest.mark.parametrize("mode", ["literal", "unit", "sharp"])
def test_absorbed_equals_explicit_tiny(mode):
    g, n = wl.TINY, 4
    w, hist, chunk = _tiny_inputs(n, mode)
    a = mla.attend(g, w, hist, n, chunk)
    b = mla.attend_absorbed(g, w, hist, n, chunk)
    assert np.abs(a - b).max() <= 1e-10 * np.abs(a).max()


def test_absorbed_equals_explicit_wan_widths():
    g = wl.WAN_SMALL_GRID
    n = 7
    w = wl.latent_weights(g, mode="sharp")
    hist = {f: wl.hidden_states(g, chunk=f, mode="unit")[0][:g.tokens_per_frame] for f in range(n)}
    chunk = wl.hidden_states(g, chunk=99, mode="unit")[0]
    q = np.arange(0, g.n_q, 7)
    a = mla.attend(g, w, hist, n, chunk, query_tokens=q)
    b = mla.attend_absorbed(g, w, hist, n, chunk, query_tokens=q)
    assert np.abs(a - b).max() <= 1e-10 * np.abs(a).max()


def test_mha_special_case_matches_library_sdpa():
    """d_r = 0, d_c = 2 n_h d_h, W_DKV = [W_K; W_V] and selector up-projections:
    latent attention must equal textbook multi-head attention (torch SDPA on CPU)."""
    import torch
    nh, dh, d, dq = 2, 8, 32, 16
    g = SimpleNamespace(hidden=d, n_heads=nh, d_nope=dh, d_rope=0, d_v=dh, d_c=2 * nh * dh, d_q=dq,
                        rope_pairs=(0, 0, 0), rope_theta=1e4, grid_h=2, grid_w=3, window_frames=2,
                        chunk_frames=1)
    rng = np.random.default_rng(3)
    wk, wv = rng.standard_normal((nh * dh, d)), rng.standard_normal((nh * dh, d))
    sel = np.zeros((2, nh, dh, 2 * nh * dh))
    for h in range(nh):
        sel[0, h, :, h * dh:(h + 1) * dh] = np.eye(dh)
        sel[1, h, :, nh * dh + h * dh:nh * dh + (h + 1) * dh] = np.eye(dh)
    w = SimpleNamespace(w_dkv=np.vstack([wk, wv]), w_kr=np.zeros((0, d)),
                        w_dq=rng.standard_normal((dq, d)) / 4, w_uq=rng.standard_normal((nh * dh, dq)) / 4,
                        w_uk=sel[0], w_uv=sel[1], w_o=rng.standard_normal((d, nh * dh)))
    n = 3
    hist = {f: rng.standard_normal((6, d)) for f in range(n)}
    chunk = rng.standard_normal((6, d))
    u = mla.attend(g, w, hist, n, chunk)

    xk = np.concatenate([hist[1], hist[2], chunk])
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))
    Q = t(chunk @ (w.w_uq @ w.w_dq).T).reshape(6, nh, dh).transpose(0, 1)
    K = t(xk @ wk.T).reshape(-1, nh, dh).transpose(0, 1)
    V = t(xk @ wv.T).reshape(-1, nh, dh).transpose(0, 1)
    O = torch.nn.functional.scaled_dot_product_attention(Q[None], K[None], V[None])[0]
    ref = O.transpose(0, 1).reshape(6, nh * dh).numpy() @ w.w_o.T
    np.testing.assert_allclose(u, ref, rtol=1e-10, atol=1e-12)


def test_softmax_rows_sum_to_one():
    g, n = wl.TINY, 3
    w, hist, chunk = _tiny_inputs(n, "sharp")
    _, probs = mla.attend(g, w, hist, n, chunk, return_probs=True)
    for p in probs:
        np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=1e-14)
        assert p.max() > 0.05  # the sharp inputs really are peaked


def test_zero_query_gives_mean_value():
    g, n = wl.TINY, 5
    w, hist, chunk = _tiny_inputs(n)
    w.w_dq = np.zeros_like(w.w_dq)
    u = mla.attend(g, w, hist, n, chunk)
    xk = np.concatenate([hist[3], hist[4], chunk]).astype(np.float64)
    c = xk @ w.w_dkv.T
    o = np.concatenate([(c @ w.w_uv[h].T).mean(axis=0) for h in range(2)])
    np.testing.assert_allclose(u, np.tile(o @ w.w_o.T, (16, 1)), rtol=1e-12)


def test_single_key_returns_its_value():
    g = wl.TINY.replace(grid_h=1, grid_w=1)
    w = wl.latent_weights(g, mode="unit")
    x = wl.hidden_states(g, mode="unit")[0].astype(np.float64)
    u = mla.attend(g, w, {}, 0, x)
    c = x @ w.w_dkv.T
    o = np.concatenate([c @ w.w_uv[h].T for h in range(2)], axis=1)
    np.testing.assert_allclose(u, o @ w.w_o.T, rtol=1e-12)


def test_key_order_does_not_matter():
    """Softmax attention is invariant under a joint permutation of the keys (each
    key keeps its own position), which is why a ring cache may hold the window in
    slot order.  The brute force processed in ring-slot order and in a random order
    matches the oracle's context order.  Negative control: moving keys to other
    positions (the two cached frames' contents swapped) does change the output."""
    g, n = wl.TINY, 5                       # W = 2, C = 1: frames 3, 4 cached, 4 in slot 0 (wrapped)
    w, hist, chunk = _tiny_inputs(n, "sharp")
    u = mla.attend(g, w, hist, n, chunk)
    T = g.grid_h * g.grid_w
    cached = [3, 4]
    slot_of = {f: f % g.window_frames for f in cached}
    ring_order = [cached.index(f) * T + s for f in sorted(cached, key=lambda f: slot_of[f]) for s in range(T)]
    ring_order += [len(cached) * T + s for s in range(g.n_q)]
    assert ring_order[:T] == list(range(T, 2 * T))   # the newer frame comes first in slot order
    for order in (ring_order, list(np.random.default_rng(3).permutation(len(ring_order)))):
        ub = np.array(brute.attend(g, w, hist, n, chunk, key_order=[int(j) for j in order]))
        np.testing.assert_allclose(ub, u, rtol=1e-11, atol=1e-14)
    swapped = dict(hist)
    swapped[3], swapped[4] = hist[4], hist[3]
    assert np.abs(mla.attend(g, w, swapped, n, chunk) - u).max() > 1e-3 * np.abs(u).max()


def test_window_excludes_evicted_frames():
    g, n = wl.TINY, 5
    w, hist, chunk = _tiny_inputs(n, "sharp")
    u = mla.attend(g, w, hist, n, chunk)
    h2 = dict(hist)
    h2[n - g.window_frames - 1] = hist[0] * 3.0  # left the window
    np.testing.assert_array_equal(mla.attend(g, w, h2, n, chunk), u)
    h3 = dict(hist)
    h3[n - g.window_frames] = hist[0] * 3.0        # oldest visible frame
    assert np.abs(mla.attend(g, w, h3, n, chunk) - u).max() > 1e-6 * np.abs(u).max()


# ----------------------------------------------------------------------------- ring
@pytest.mark.parametrize("W,C", [(2, 1), (21, 3), (5, 3), (42, 3), (4, 4)])
def test_ring_model_is_fifo(W, C):
    r = ring.RingModel(W, 7)
    fifo = collections.deque(maxlen=W)
    occupant = {}
    for k in range(1, 40):
        for f, s in r.append(C):
            if len(fifo) == W:
                evicted = fifo[0]
                assert occupant[s] == evicted  # the slot written held the frame FIFO evicts
            fifo.append(f)
            occupant[s] = f
        assert list(r.valid_frames()) == list(fifo)
        # closed form after k appends of C frames
        assert list(r.valid_frames()) == list(range(max(0, k * C - W), k * C))
        assert r.slot_map() == {f % W: f for f in fifo}
        assert r.valid_rows() == min(k * C, W) * 7
        # the valid slots are always rows [0, valid_rows) of the ring
        assert sorted(r.slot_map()) == list(range(min(k * C, W)))


def test_ring_rejects_chunk_larger_than_window():
    with pytest.raises(ValueError):
        ring.RingModel(2, 4).append(3)


# ----------------------------------------------------------------------------- inputs
def test_seeded_inputs_are_deterministic_and_distinct():
    g = wl.TINY
    a = wl.hidden_states(g, chunk=3, seed=1)
    b = wl.hidden_states(g, chunk=3, seed=1)
    c = wl.hidden_states(g, chunk=4, seed=1)
    np.testing.assert_array_equal(a, b)
    assert not np.array_equal(a, c)
    w = wl.latent_weights(wl.WAN_SMALL_GRID)
    assert w.w_uk.shape == (12, 96, 192) and w.w_o.shape == (1536, 1536)
    # bf16 storage: values are exactly representable in bf16
    v = w.w_dq.view(np.uint32)
    assert np.all((v & 0xFFFF) == 0)
    assert abs(w.w_dq.std() * math.sqrt(1536) - 1.0) < 0.02


# ----------------------------------------------------------------------------- dense baseline
def _tiny_dense_inputs(n, mode="unit", seed=0):
    g = wl.TINY_DENSE
    w = wl.dense_weights(g, seed=seed, mode=mode)
    hist = {f: wl.hidden_states(g, chunk=f, seed=seed, mode=mode)[0] for f in range(n)}  # one frame per chunk
    chunk = wl.hidden_states(g, chunk=1000 + n, seed=seed, mode=mode)[0]
    return g, w, hist, chunk


@pytest.mark.parametrize("n", [0, 1, 3, 5])
@pytest.mark.parametrize("mode", ["unit", "sharp"])
def test_dense_brute_force_matches_numpy(n, mode):
    """The dense baseline against the scalar-loop formulation (complex rotary pairs)."""
    g, w, hist, chunk = _tiny_dense_inputs(n, mode)
    u = mla.attend_dense(g, w, hist, n, chunk)
    ub = np.array(brute.attend_dense(g, w, hist, n, chunk))
    np.testing.assert_allclose(u, ub, rtol=1e-12, atol=1e-14 * np.abs(ub).max())


def test_dense_zero_query_gives_mean_value():
    """W_Q = 0 makes every score 0: each head returns the mean of its visible values."""
    g, w, hist, chunk = _tiny_dense_inputs(5)
    w.w_q = np.zeros_like(w.w_q)
    u = mla.attend_dense(g, w, hist, 5, chunk)
    xk = np.concatenate([hist[3], hist[4], chunk]).astype(np.float64)
    o = (xk @ w.w_v.T.astype(np.float64)).mean(axis=0)
    np.testing.assert_allclose(u, np.tile(o @ w.w_o.T.astype(np.float64), (16, 1)), rtol=1e-12)


def test_dense_window_excludes_evicted_frames():
    g, w, hist, chunk = _tiny_dense_inputs(5, "sharp")
    u = mla.attend_dense(g, w, hist, 5, chunk)
    h2 = dict(hist)
    h2[2] = hist[0] * 3.0  # frame 2 left the 2-frame window at n = 5
    np.testing.assert_array_equal(mla.attend_dense(g, w, h2, 5, chunk), u)
    h3 = dict(hist)
    h3[3] = hist[0] * 3.0  # oldest visible frame
    assert np.abs(mla.attend_dense(g, w, h3, 5, chunk) - u).max() > 1e-6 * np.abs(u).max()



# ----------------------------------------------------------------------------- sink frame + re-indexing
TINY_SINK = wl.TINY.replace(name="tiny-sink", sink_frames=1)


@pytest.mark.parametrize("n", [0, 1, 2, 3, 4, 6])
def test_sink_brute_force_matches_numpy(n):
    """One pinned sink frame ahead of the 2-frame window: both formulations agree
    at every window state (empty, sink only, partial, full, evicted)."""
    g = TINY_SINK
    w, hist, chunk = _tiny_inputs(n, "sharp", g=g)
    u = mla.attend(g, w, hist, n, chunk)
    ub = np.array(brute.attend(g, w, hist, n, chunk))
    np.testing.assert_allclose(u, ub, rtol=1e-12, atol=1e-14 * np.abs(ub).max())


def test_sink_visible_frames_and_local_coordinates():
    # S = 1, W = 2, C = 1: the sink stays, the window slides, the gap collapses
    assert mla.visible_frames(0, 2, 1, 1) == ([], [0])
    assert mla.visible_frames(1, 2, 1, 1) == ([0], [1])
    assert mla.visible_frames(3, 2, 1, 1) == ([0, 1, 2], [3])
    assert mla.visible_frames(7, 2, 1, 1) == ([0, 5, 6], [7])
    assert mla.visible_frames(7, 2, 1, 0) == ([5, 6], [7])


def test_reindexing_makes_output_independent_of_absolute_time():
    """With the sink and the window re-indexed (appendix D.5), an attend depends
    only on the visible content: the same sink, window and chunk at frame 4 and at
    frame 9 give the same output, to the last bit."""
    g = TINY_SINK
    w = wl.latent_weights(g, mode="sharp")
    frame = lambda k: wl.hidden_states(g, chunk=k, mode="unit")[0]
    chunk = wl.hidden_states(g, chunk=77, mode="unit")[0]
    h1 = {0: frame(0), 2: frame(1), 3: frame(2)}     # n = 4: sink 0, window 2..3
    h2 = {0: frame(0), 7: frame(1), 8: frame(2)}     # n = 9: sink 0, window 7..8
    np.testing.assert_array_equal(mla.attend(g, w, h1, 4, chunk), mla.attend(g, w, h2, 9, chunk))
    # the sink context is the plain window that holds the same frames in the same order
    g0 = g.replace(sink_frames=0, window_frames=3)
    a = mla.attend(g0, w, {1: frame(0), 2: frame(1), 3: frame(2)}, 4, chunk)
    b = mla.attend(g, w, {0: frame(0), 2: frame(1), 3: frame(2)}, 4, chunk)
    np.testing.assert_array_equal(a, b)  # same local frame order -> same result


@pytest.mark.parametrize("S,W,C", [(1, 6, 3), (1, 2, 1), (2, 4, 2), (1, 5, 2)])
def test_ring_model_with_sink(S, W, C):
    r = ring.RingModel(W, 10, sink_frames=S)
    for k in range(12):
        r.append(C)
        occ = r.slot_map()
        assert len(occ) == len(r.valid_frames()) == min(r.n, S) + max(0, min(r.n - S, W))
        assert all(occ[f] == f for f in range(min(r.n, S)))            # sinks pinned in slots 0..S-1
        window = [f for f in r.valid_frames() if f >= S]
        assert window == list(range(max(S, r.n - W), r.n))              # FIFO window
        assert sorted(occ) == list(range(len(occ)))                      # occupied slots are a prefix



# ----------------------------------------------------------------------------- block-causal clip
def test_clip_matches_masked_full_attention():
    """attend_clip (chunk by chunk) against the masked formulation: one score
    matrix over the whole clip with key j hidden from query i when j's chunk is
    later than i's (-inf before the softmax)."""
    g = wl.TINY.replace(name="tiny-clip", window_frames=5, chunk_frames=2)   # chunks of 2, 2, 1 frames
    w = wl.latent_weights(g, mode="sharp")
    T, F = 16, 5
    x = wl.hidden_states(g.replace(chunk_frames=F), chunk=3, mode="unit")[0].astype(np.float64)
    u = mla.attend_clip(g, w, x)
    # independent assembly over the full clip
    c, kr_hat = mla.latents(x, w.w_dkv, w.w_kr)
    freqs = mla.rope_frequencies(g.rope_pairs, g.rope_theta)
    coords = mla.token_coordinates(np.arange(F), 4, 4)
    kr = mla.rope_rotate(kr_hat, coords, g.rope_pairs, freqs)
    q_nope, qr_hat = mla.query_heads(x, w.w_dq, w.w_uq, g.n_heads, g.d_nope, g.d_rope)
    qr = mla.rope_rotate(qr_hat, coords, g.rope_pairs, freqs)
    chunk = np.arange(F * T) // T // 2
    hidden = chunk[None, :] > chunk[:, None]
    o = []
    for h in range(g.n_heads):
        s_ = (q_nope[:, h] @ (c @ w.w_uk[h].T).T + qr[:, h] @ kr.T) / np.sqrt(g.d_nope + g.d_rope)
        s_[hidden] = -np.inf
        p_ = np.exp(s_ - s_.max(axis=1, keepdims=True))
        p_ /= p_.sum(axis=1, keepdims=True)
        o.append(p_ @ (c @ w.w_uv[h].T))
    ref = np.concatenate(o, axis=1) @ w.w_o.T
    np.testing.assert_allclose(u, ref, rtol=1e-10, atol=1e-13)
    # the first chunk sees only itself; the second does see the first
    np.testing.assert_allclose(u[:2 * T], mla.attend(g, w, {}, 0, x[:2 * T]), rtol=1e-12)
