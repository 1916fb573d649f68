"""Pure-Python brute force of one chunk of latent attention, for tiny inputs.

TEST INFRASTRUCTURE ONLY (see the package docstring).

A second, independent formulation of the same definition as oracle.mla: scalar
loops over Python floats, rotary pairs handled as Python complex numbers
(channel 2p is the real part, 2p+1 the imaginary part; a rotation by angle a is
multiplication by e^{i a}), and the softmax written out term by term.  It is
meant to be slow and obvious; use it on inputs of a few thousand scalars.
"""
from __future__ import annotations

import cmath
import math


def _mat_vec(w, x):
    return [sum(wr[k] * x[k] for k in range(len(x))) for wr in w]


def _freq(pairs, theta):
    out = []
    for p in pairs:
        out += [theta ** (-2.0 * i / (2.0 * p)) for i in range(p)]
    return out


def _table(g):
    """The geometry's explicit rotary table (rope_freqs) if it has one, else the
    default per-axis spectrum."""
    t = getattr(g, "rope_freqs", None)
    return [float(v) for v in t] if t is not None else _freq(g.rope_pairs, g.rope_theta)


def _rotate(vec, coord, pairs, freqs):
    """vec: list of 2P floats; coord: (t, h, w); freqs: omega per pair."""
    axis = [a for a, p in enumerate(pairs) for _ in range(p)]
    out = []
    for p, om in enumerate(freqs):
        z = complex(vec[2 * p], vec[2 * p + 1]) * cmath.exp(1j * coord[axis[p]] * om)
        out += [z.real, z.imag]
    return out


def attend(g, wts, history, n, chunk_x, key_order=None):
    """u for every query token of the chunk, as nested lists [C*T][hidden].

    key_order: optional permutation (indices into the visible keys in context
    order) in which the keys, each with its own position, are processed; softmax
    attention does not depend on it (e.g. a ring cache's slot order)."""
    T = g.grid_h * g.grid_w
    W, C = g.window_frames, g.chunk_frames
    tolist = lambda a: [[float(v) for v in row] for row in a]
    # visible frames in context order: pinned sink frames, the recent window, the
    # chunk; a frame's local temporal coordinate is its index in that list
    S = getattr(g, "sink_frames", 0)
    frames = [f for f in range(n) if f < S or f >= max(S, n - W)] + list(range(n, n + C))
    keys_x, keys_pos = [], []
    for tau, fr in enumerate(frames):
        rows = tolist(history[fr]) if fr < n else tolist(chunk_x)[(fr - n) * T:(fr - n + 1) * T]
        for s in range(T):
            keys_x.append(rows[s])
            keys_pos.append((tau, s // g.grid_w, s % g.grid_w))
    n_cached = len(frames) - C
    if key_order is not None:
        assert sorted(key_order) == list(range(len(keys_x))), "key_order must be a permutation"
        keys_x = [keys_x[j] for j in key_order]
        keys_pos = [keys_pos[j] for j in key_order]
    w_dkv, w_kr, w_dq, w_uq, w_o = (tolist(getattr(wts, k)) for k in ("w_dkv", "w_kr", "w_dq", "w_uq", "w_o"))
    w_uk = [tolist(m) for m in wts.w_uk]
    w_uv = [tolist(m) for m in wts.w_uv]
    dh = g.d_nope + g.d_rope

    # per-key per-head reconstructed K and V
    K, V = [], []
    for xj, pj in zip(keys_x, keys_pos):
        c = _mat_vec(w_dkv, xj)
        kr = _rotate(_mat_vec(w_kr, xj), pj, g.rope_pairs, _table(g))
        K.append([_mat_vec(w_uk[h], c) + kr for h in range(g.n_heads)])
        V.append([_mat_vec(w_uv[h], c) for h in range(g.n_heads)])

    out = []
    chunk_rows = tolist(chunk_x)
    for i, xi in enumerate(chunk_rows):
        pos = (n_cached + i // T, (i % T) // g.grid_w, (i % T) % g.grid_w)
        cq = _mat_vec(w_dq, xi)
        qall = _mat_vec(w_uq, cq)
        o = []
        for h in range(g.n_heads):
            qh = qall[h * dh:(h + 1) * dh]
            q = qh[:g.d_nope] + _rotate(qh[g.d_nope:], pos, g.rope_pairs, _table(g))
            s = [sum(q[d] * K[j][h][d] for d in range(dh)) / math.sqrt(dh) for j in range(len(K))]
            m = max(s)
            e = [math.exp(v - m) for v in s]
            z = sum(e)
            o += [sum(e[j] / z * V[j][h][d] for j in range(len(K))) for d in range(g.d_v)]
        out.append(_mat_vec(w_o, o))
    return out


def attend_dense(g, wts, history, n, chunk_x):
    """Dense per-head baseline, same loops: q_h = RoPE(W_Q^h x), k_h = RoPE(W_K^h x)
    on every head channel, v_h = W_V^h x, window-local temporal coordinate."""
    T = g.grid_h * g.grid_w
    W, C = g.window_frames, g.chunk_frames
    tolist = lambda a: [[float(v) for v in row] for row in a]
    # visible frames in context order: pinned sink frames, the recent window, the
    # chunk; a frame's local temporal coordinate is its index in that list
    S = getattr(g, "sink_frames", 0)
    frames = [f for f in range(n) if f < S or f >= max(S, n - W)] + list(range(n, n + C))
    keys_x, keys_pos = [], []
    for tau, fr in enumerate(frames):
        rows = tolist(history[fr]) if fr < n else tolist(chunk_x)[(fr - n) * T:(fr - n + 1) * T]
        for s in range(T):
            keys_x.append(rows[s])
            keys_pos.append((tau, s // g.grid_w, s % g.grid_w))
    n_cached = len(frames) - C
    w_q, w_k, w_v, w_o = (tolist(getattr(wts, k)) for k in ("w_q", "w_k", "w_v", "w_o"))
    dh = g.d_nope + g.d_rope
    K, V = [], []
    for xj, pj in zip(keys_x, keys_pos):
        kall, vall = _mat_vec(w_k, xj), _mat_vec(w_v, xj)
        K.append([_rotate(kall[h * dh:(h + 1) * dh], pj, g.rope_pairs, _table(g)) for h in range(g.n_heads)])
        V.append([vall[h * g.d_v:(h + 1) * g.d_v] for h in range(g.n_heads)])
    out = []
    for i, xi in enumerate(tolist(chunk_x)):
        pos = (n_cached + i // T, (i % T) // g.grid_w, (i % T) % g.grid_w)
        qall = _mat_vec(w_q, xi)
        o = []
        for h in range(g.n_heads):
            q = _rotate(qall[h * dh:(h + 1) * dh], pos, g.rope_pairs, _table(g))
            s = [sum(q[d] * K[j][h][d] for d in range(dh)) / math.sqrt(dh) for j in range(len(K))]
            m = max(s)
            e = [math.exp(v - m) for v in s]
            z = sum(e)
            o += [sum(e[j] / z * V[j][h][d] for j in range(len(K))) for d in range(g.d_v)]
        out.append(_mat_vec(w_o, o))
    return out
