"""Plain numpy oracle for one chunk of VideoMLA latent attention.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Float64 throughout
unless a caller asks otherwise; no blocking, fusion or reordering beyond the
definitions below.

What is computed, for one stream and one query chunk (VideoMLA paper,
sections 3, 3.1-3.3, appendices C.1, D.1, D.4, D.5):

 1. Latents of every visible token j (section 3.1): the position-free content
    latent c_j = W_DKV x_j (d_c) and the decoupled positional key
    k^_j = W_KR x_j (d_r), kept before rotation (section 3.3 and D.5 store the
    positional key un-rotated and rotate it when the window is assembled).
 2. Visible keys (D.4, chunk-causal): the cached frames -- the S pinned sink
    frames [0, min(n, S)) (S = 0 unless a geometry sets sink_frames) and the
    recent window [max(S, n-W), n) -- plus the chunk's own frames [n, n+C);
    every query of the chunk sees all of them.
 3. Positions (C.1, D.5): token s of a frame sits at row s // grid_w, column
    s % grid_w; the temporal coordinate is local: a frame's index in the
    visible context [sink frames, window frames, chunk frames], for keys and
    queries alike (D.5 re-indexing; without a sink this is f - first frame).
 4. 3D-RoPE (section 3.2, 4.1, C.1): the d_r channels are complex pairs
    (2p, 2p+1); the first p_t pairs turn with tau, the next p_h with the row,
    the last p_w with the column; pair p turns by angle pos * omega_p.
 5. Queries: c^Q = W_DQ x; per head [q^nope_h ; q^_h^R] = W_UQ^h c^Q;
    q^R_h = RoPE(q^_h^R).  q^R is per head, k^R is shared (section 3.2).
 6. Explicit per-head reconstruction (section 3.3): k^nope_{j,h} = W_UK^h c_j,
    v_{j,h} = W_UV^h c_j, k^R_j = RoPE(k^_j).
 7. score_{i,j,h} = (q^nope_{i,h} . k^nope_{j,h} + q^R_{i,h} . k^R_j) / sqrt(d_h)
    with d_h = d_nope + d_r (section 3.3: same score shape as a dense head of
    the same per-head dimension); softmax over j with the maximum subtracted;
    o_{i,h} = sum_j p v_{j,h}; u_i = W_O [o_{i,1}; ...; o_{i,n_h}].

Readings of points the text leaves open (each is a reading, not a page fact):
  * no biases and no normalisation on c, q or k (none is mentioned);
  * softmax scale 1/sqrt(d_nope + d_r);
  * rotary bands: axis a with p_a pairs uses omega_i = theta^(-2i / (2 p_a)),
    i = 0..p_a-1 (the standard per-axis RoPE spectrum; the high-frequency
    bands read as the leading bands of each axis), unless the geometry carries
    an explicit table (rope_freqs), e.g. backbone_band_frequencies: the leading
    bands of a dense backbone's wider per-axis spectrum;
  * "complex pairs" are adjacent channels (2p, 2p+1), rotated counter-clockwise
    (multiplication by e^{i angle}).
"""
from __future__ import annotations

import numpy as np


# ----------------------------------------------------------------------------- RoPE
def rope_frequencies(pairs: tuple, theta: float) -> np.ndarray:
    """omega for every complex pair, axis order (t, h, w)."""
    out = []
    for p in pairs:
        i = np.arange(p, dtype=np.float64)
        out.append(np.power(float(theta), -2.0 * i / (2.0 * p)) if p > 0 else np.zeros(0))
    return np.concatenate(out)


def backbone_band_frequencies(pairs: tuple, axis_dims: tuple, theta: float) -> np.ndarray:
    """omega per complex pair when the decoupled key takes the highest-frequency
    bands of a dense backbone's per-axis rotary spectrum (sections 3.2 and 4.1
    allocate the decoupled key's pairs across the t, h, w axes on the
    high-frequency bands of each axis, as the backbone does).  Axis a of the
    backbone rotates axis_dims[a] channels with omega_i = theta^(-2i/axis_dims[a]),
    i = 0, 1, ...; the key's p_a pairs on that axis are the first p_a of them.
    With axis_dims = 2 * pairs this is rope_frequencies(pairs, theta)."""
    out = []
    for p, d in zip(pairs, axis_dims):
        assert 0 <= p <= d // 2
        i = np.arange(p, dtype=np.float64)
        out.append(np.power(float(theta), -2.0 * i / float(d)))
    return np.concatenate(out)


def frequencies(g) -> np.ndarray:
    """The rotary table of a geometry: its explicit per-pair table `rope_freqs`
    when it carries one (axis order t, h, w), else rope_frequencies."""
    table = getattr(g, "rope_freqs", None)
    if table is not None:
        table = np.asarray(table, dtype=np.float64)
        assert table.shape == (sum(g.rope_pairs),)
        return table
    return rope_frequencies(g.rope_pairs, g.rope_theta)


def pair_axes(pairs: tuple) -> np.ndarray:
    """Axis index (0 = t, 1 = h, 2 = w) of every complex pair."""
    return np.concatenate([np.full(p, a, dtype=np.int64) for a, p in enumerate(pairs)])


def token_coordinates(frame_coords: np.ndarray, grid_h: int, grid_w: int) -> np.ndarray:
    """[len(frame_coords) * grid_h * grid_w, 3] integer (t, h, w) per token, frames in order,
    tokens of a frame row-major over the (h, w) grid."""
    s = np.arange(grid_h * grid_w)
    t = np.repeat(np.asarray(frame_coords, dtype=np.int64), grid_h * grid_w)
    hh = np.tile(s // grid_w, len(frame_coords))
    ww = np.tile(s % grid_w, len(frame_coords))
    return np.stack([t, hh, ww], axis=1)


def rope_rotate(v: np.ndarray, coords: np.ndarray, pairs: tuple, freqs: np.ndarray) -> np.ndarray:
    """Rotate the last axis of v ([N, ..., 2P]) pairwise; coords is [N, 3]."""
    P = len(freqs)
    assert v.shape[-1] == 2 * P
    if P == 0:
        return v.copy()
    pos = coords[:, pair_axes(pairs)].astype(np.float64)        # [N, P]
    ang = pos * freqs[None, :]
    cos, sin = np.cos(ang), np.sin(ang)
    extra = v.ndim - 2
    cos = cos.reshape(cos.shape[:1] + (1,) * extra + cos.shape[1:])
    sin = sin.reshape(sin.shape[:1] + (1,) * extra + sin.shape[1:])
    a, b = v[..., 0::2], v[..., 1::2]
    out = np.empty_like(v, dtype=np.result_type(v, np.float64))
    out[..., 0::2] = a * cos - b * sin
    out[..., 1::2] = a * sin + b * cos
    return out


# ----------------------------------------------------------------------------- projections
def latents(x: np.ndarray, w_dkv: np.ndarray, w_kr: np.ndarray):
    """c = W_DKV x (content latent) and k^ = W_KR x (un-rotated positional key)."""
    return x @ w_dkv.T, x @ w_kr.T


def query_heads(x: np.ndarray, w_dq: np.ndarray, w_uq: np.ndarray, n_heads: int, d_nope: int,
                d_rope: int):
    """c^Q = W_DQ x; per head [q^nope ; q^R (un-rotated)] = W_UQ^h c^Q."""
    cq = x @ w_dq.T
    q = (cq @ w_uq.T).reshape(x.shape[0], n_heads, d_nope + d_rope)
    return q[..., :d_nope], q[..., d_nope:]


# ----------------------------------------------------------------------------- window
def visible_frames(n: int, window_frames: int, chunk_frames: int, sink_frames: int = 0):
    """(cached frames, chunk frames) in context order: sink frames [0, min(n, S)),
    then the window [max(S, n-W), n); chunk [n, n+C).  A frame's local temporal
    coordinate is its index in cached + chunk (appendix D.4, D.5)."""
    sink = list(range(min(n, sink_frames)))
    window = list(range(max(sink_frames, n - window_frames), n))
    return sink + window, list(range(n, n + chunk_frames))


class _Assembled:
    pass


def _assemble(g, wts, history, n, chunk_x, query_tokens, dtype):
    """Everything attention needs, for one stream: rotated keys/queries, latents."""
    f = lambda a: np.asarray(a, dtype=dtype)
    T = g.grid_h * g.grid_w
    cached, chunk = visible_frames(n, g.window_frames, g.chunk_frames, getattr(g, "sink_frames", 0))
    xk = [f(history[fr]).reshape(T, g.hidden) for fr in cached]
    xk.append(f(chunk_x).reshape(g.chunk_frames * T, g.hidden))
    xk = np.concatenate(xk, axis=0)
    freqs = frequencies(g)
    local = np.arange(len(cached) + len(chunk))  # local temporal coordinate of each visible frame

    A = _Assembled()
    A.c, kr_hat = latents(xk, f(wts.w_dkv), f(wts.w_kr))
    kcoords = token_coordinates(local, g.grid_h, g.grid_w)
    A.kr = rope_rotate(kr_hat, kcoords, g.rope_pairs, freqs)

    qi = np.arange(g.chunk_frames * T) if query_tokens is None else np.asarray(query_tokens)
    xq = f(chunk_x).reshape(g.chunk_frames * T, g.hidden)[qi]
    A.q_nope, qr_hat = query_heads(xq, f(wts.w_dq), f(wts.w_uq), g.n_heads, g.d_nope, g.d_rope)
    qcoords = token_coordinates(local[len(cached):], g.grid_h, g.grid_w)[qi]
    A.qr = rope_rotate(qr_hat, qcoords, g.rope_pairs, freqs)
    A.scale = 1.0 / np.sqrt(g.d_nope + g.d_rope)
    return A


def _softmax_rows(s: np.ndarray) -> np.ndarray:
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=-1, keepdims=True)


def attend(g, wts, history, n: int, chunk_x, query_tokens=None, dtype=np.float64,
           return_probs: bool = False):
    """Chunk attention of one stream with explicit per-head K/V reconstruction.

    g        geometry (attributes: hidden, n_heads, d_nope, d_rope, d_v, d_c, rope_pairs,
             rope_theta, grid_h, grid_w, window_frames, chunk_frames)
    wts      weights (attributes w_dkv, w_kr, w_dq, w_uq, w_uk, w_uv, w_o; Linear layout)
    history  indexable by absolute frame -> hidden states [T, hidden] of that appended frame
    n        frames appended before this chunk
    chunk_x  [C*T, hidden] hidden states of the chunk
    Returns u [len(query_tokens), hidden] (and per-head probabilities when asked).
    """
    A = _assemble(g, wts, history, n, chunk_x, query_tokens, dtype)
    w_uk = np.asarray(wts.w_uk, dtype=dtype)
    w_uv = np.asarray(wts.w_uv, dtype=dtype)
    nq = A.q_nope.shape[0]
    o = np.empty((nq, g.n_heads, g.d_v), dtype=dtype)
    probs = []
    for h in range(g.n_heads):
        k_nope = A.c @ w_uk[h].T          # [Nk, d_nope]  (section 3.3 reconstruction)
        v = A.c @ w_uv[h].T               # [Nk, d_v]
        s = (A.q_nope[:, h] @ k_nope.T + A.qr[:, h] @ A.kr.T) * A.scale
        p = _softmax_rows(s)
        o[:, h] = p @ v
        if return_probs:
            probs.append(p)
    u = o.reshape(nq, g.n_heads * g.d_v) @ np.asarray(wts.w_o, dtype=dtype).T
    return (u, probs) if return_probs else u


def attend_clip(g, wts, clip_x, dtype=np.float64):
    """Block-causal attention over a whole clip of window_frames frames (the
    training-time form, appendix D.4): tokens of chunk q (frames [qC, (q+1)C),
    the last chunk possibly shorter) attend to every token of chunks 0..q, with
    the clip's frame indices as temporal coordinates.  Written as the definition
    composes: chunk q is an attend() whose cached frames are all earlier frames."""
    T = g.grid_h * g.grid_w
    F, C = g.window_frames, g.chunk_frames
    frames = np.asarray(clip_x).reshape(F, T, g.hidden)
    out = []
    for q0 in range(0, F, C):
        c = min(C, F - q0)
        gq = g.replace(chunk_frames=c, sink_frames=0) if hasattr(g, "replace") else g
        hist = {f: frames[f] for f in range(q0)}
        out.append(attend(gq, wts, hist, q0, frames[q0:q0 + c].reshape(c * T, g.hidden), dtype=dtype))
    return np.concatenate(out, axis=0)


def attend_absorbed(g, wts, history, n: int, chunk_x, query_tokens=None, dtype=np.float64):
    """Same attention with W_UK folded into the query and W_UV applied after the
    probability-weighted sum of latents (the MLA absorption identity).  Kept only
    to check that the rearrangement is exact; the reference result is attend()."""
    A = _assemble(g, wts, history, n, chunk_x, query_tokens, dtype)
    w_uk = np.asarray(wts.w_uk, dtype=dtype)
    w_uv = np.asarray(wts.w_uv, dtype=dtype)
    nq = A.q_nope.shape[0]
    o = np.empty((nq, g.n_heads, g.d_v), dtype=dtype)
    for h in range(g.n_heads):
        q_lat = A.q_nope[:, h] @ w_uk[h]                  # [Nq, d_c]
        s = (q_lat @ A.c.T + A.qr[:, h] @ A.kr.T) * A.scale
        p = _softmax_rows(s)
        o[:, h] = (p @ A.c) @ w_uv[h].T
    return o.reshape(nq, g.n_heads * g.d_v) @ np.asarray(wts.w_o, dtype=dtype).T


def scores(g, wts, history, n: int, chunk_x, query_tokens=None, dtype=np.float64):
    """Pre-softmax scores [n_heads, Nq, Nk] (key order: cached frames ascending, then chunk)."""
    A = _assemble(g, wts, history, n, chunk_x, query_tokens, dtype)
    w_uk = np.asarray(wts.w_uk, dtype=dtype)
    out = []
    for h in range(g.n_heads):
        k_nope = A.c @ w_uk[h].T
        out.append((A.q_nope[:, h] @ k_nope.T + A.qr[:, h] @ A.kr.T) * A.scale)
    return np.stack(out)


def chunk_latents(g, wts, x, frame0: int, dtype=np.float64):
    """Cache rows [c | RoPE(k^)] for hidden states x ([C*T, hidden]) of frames
    frame0.. with the absolute frame index as temporal coordinate.  This is
    the row layout a cache holds when the key is rotated as it is written."""
    T = g.grid_h * g.grid_w
    x = np.asarray(x, dtype=dtype).reshape(-1, g.hidden)
    nfr = x.shape[0] // T
    c, kr_hat = latents(x, np.asarray(wts.w_dkv, dtype=dtype), np.asarray(wts.w_kr, dtype=dtype))
    coords = token_coordinates(np.arange(frame0, frame0 + nfr), g.grid_h, g.grid_w)
    kr = rope_rotate(kr_hat, coords, g.rope_pairs, frequencies(g))
    return np.concatenate([c, kr], axis=1)


# ----------------------------------------------------------------------------- dense baseline
def attend_dense(g, wts, history, n: int, chunk_x, query_tokens=None, dtype=np.float64,
                 return_scores: bool = False):
    """Dense per-head attention over the same window: K_h = RoPE(W_K^h x) on all
    head_dim channels, V_h = W_V^h x, same chunk-causal visibility and window-local
    temporal coordinate (the baseline layout of section 1 / appendix C.1).
    With return_scores, also the pre-softmax scores [n_heads, Nq, Nk]."""
    f = lambda a: np.asarray(a, dtype=dtype)
    T = g.grid_h * g.grid_w
    cached, chunk = visible_frames(n, g.window_frames, g.chunk_frames, getattr(g, "sink_frames", 0))
    xk = np.concatenate([f(history[fr]).reshape(T, g.hidden) for fr in cached]
                        + [f(chunk_x).reshape(-1, g.hidden)], axis=0)
    dh = g.head_dim
    freqs = frequencies(g)
    local = np.arange(len(cached) + len(chunk))
    kc = token_coordinates(local, g.grid_h, g.grid_w)
    k = rope_rotate((xk @ f(wts.w_k).T).reshape(-1, g.n_heads, dh), kc, g.rope_pairs, freqs)
    v = (xk @ f(wts.w_v).T).reshape(-1, g.n_heads, g.d_v)
    qi = np.arange(g.chunk_frames * T) if query_tokens is None else np.asarray(query_tokens)
    xq = f(chunk_x).reshape(-1, g.hidden)[qi]
    qc = token_coordinates(local[len(cached):], g.grid_h, g.grid_w)[qi]
    q = rope_rotate((xq @ f(wts.w_q).T).reshape(-1, g.n_heads, dh), qc, g.rope_pairs, freqs)
    o = np.empty((len(qi), g.n_heads, g.d_v), dtype=dtype)
    sc = []
    for h in range(g.n_heads):
        s = (q[:, h] @ k[:, h].T) / np.sqrt(dh)
        o[:, h] = _softmax_rows(s) @ v[:, h]
        if return_scores:
            sc.append(s)
    u = o.reshape(len(qi), -1) @ f(wts.w_o).T
    return (u, np.stack(sc)) if return_scores else u
