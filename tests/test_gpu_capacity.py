"""Parity at the largest serving batch.

The batch is the one whose 30-layer caches fit in this GPU's memory (capacity
arithmetic over the library's layouts, against the device's total memory less
a 6 GB margin): about 500 streams for the latent layer at d_c = 192, about 45
for the dense baseline.  One layer is allocated at that batch, so its cache,
workspace and hidden-state buffers reach several GB and the kernels address
the far end of each.  Streams 0 and B-1 carry seeded host inputs that the
oracle also sees; every other stream gets seeded device-random hidden states
of the same distribution.  After a full window of appends (7 chunks, 21
frames) one attend is compared with the oracle on sampled query tokens of the
two streams.
"""
import numpy as np
import pytest

from gpu_harness import assert_parity, to_dev, to_np
from mla_latent_kv_vmla_amd import capacity as cap, vmla, workloads as wl
from oracle import mla

pytestmark = pytest.mark.gpu

LAYERS = 30
MARGIN = 6 << 30


def _case(*a):
    print("case:", *a, flush=True)


def _max_batch(g, dense):
    import torch
    total = torch.cuda.mem_get_info()[1]
    return int(cap.capacity(g, LAYERS, total - MARGIN, dense=dense).max_batch)


@pytest.mark.parametrize("dense", [False, True], ids=["latent", "dense"])
def test_attend_at_max_serving_batch(dense):
    import torch
    torch.cuda.empty_cache()
    g0 = wl.WAN_DENSE if dense else wl.WAN_LAYER
    B = _max_batch(g0, dense)
    assert B >= 2
    g, g1 = g0.replace(batch=B), g0.replace(batch=1)
    _case("max serving batch", g.name, "B=", B)
    w = (wl.dense_weights if dense else wl.latent_weights)(g1)
    layer = (vmla.DenseAttention if dense else vmla.LatentAttention)(g, {k: to_dev(v, g) for k, v in vars(w).items()})
    gen = torch.Generator(device="cuda").manual_seed(5)
    ends = (0, B - 1)
    hist = {b: {} for b in ends}

    def chunk(k):
        x = torch.randn(B, g.n_q, g.hidden, generator=gen, device="cuda", dtype=torch.bfloat16).mul_(g.hidden ** -0.5)
        xs = {}
        for i, b in enumerate(ends):
            xs[b] = wl.hidden_states(g1, chunk=k, seed=1 + i)[0]
            x[b] = to_dev(xs[b], g)
        return x, xs

    prefill = g.window_frames // g.chunk_frames
    for k in range(prefill):
        x, xs = chunk(k)
        layer.append(x)
        for b in ends:
            fr = xs[b].reshape(g.chunk_frames, g.tokens_per_frame, g.hidden)
            for i in range(g.chunk_frames):
                hist[b][k * g.chunk_frames + i] = fr[i]
    n = layer.state()[0]
    assert n == g.window_frames
    x, xs = chunk(prefill)
    out = layer.attend(x)
    torch.cuda.synchronize()
    q = np.unique(np.concatenate([np.arange(4), np.arange(g.n_q - 4, g.n_q),
                                  np.random.default_rng(B).choice(g.n_q, 12, replace=False)]))
    for b in ends:
        got = to_np(out[b][torch.from_numpy(q).cuda()])
        if dense:
            ref = mla.attend_dense(g1, w, hist[b], n, xs[b], query_tokens=q)
        else:
            ref = mla.attend(g1, w, hist[b], n, xs[b], query_tokens=q)
        ma, mr = assert_parity(got, ref, f"{g.name} B={B} stream {b}")
        print(f"  stream {b} of {B}: max_abs={ma:.3e} mean_rel={mr:.3e}", flush=True)
    assert bool(torch.isfinite(out).all().item())
    layer.close()
    del layer, out, x
    torch.cuda.empty_cache()
