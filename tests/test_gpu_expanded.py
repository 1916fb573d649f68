"""Parity of the expanded (non-absorbed) latent path with the CPU oracle.

The oracle's attend() reconstructs the per-head keys and values explicitly,
which is exactly what the expanded path computes on the GPU (up-projected
window, per-head queries, dense flash kernel); the absorbed path (vmla_attend)
is the same function up to rounding.  Same bar and tolerance derivation as the
other GPU tests (gpu_harness).  Cases: Wan widths on a 6x10 grid over empty,
partial, full and wrapped windows with NaN canaries in unused cache slots, three
input scalings, stream-K cuts, d_c = 96 and 448, batched streams, the
stale-expansion guard, and the full Wan-1.3B layer on sampled queries.
"""
import numpy as np
import pytest

from gpu_harness import Rollout, assert_parity, to_dev, to_np
from mla_latent_kv_vmla_amd import vmla, workloads as wl

pytestmark = pytest.mark.gpu

SMALL = wl.WAN_SMALL_GRID


def _case(*a):
    print("case:", *a, flush=True)


def _expanded_rollout(g, mode, n_chunks, attn_workgroups=0):
    r = Rollout(g, mode=mode, attn_workgroups=attn_workgroups, cache_fill=float("nan"))
    for k in range(n_chunks):
        x = r.x(chunk=200 + k)
        _case("expanded attend", g.name, mode, "n=", r.n, "G=", attn_workgroups)
        r.dev.expand()
        xd = to_dev(x, g)
        got = to_np(r.dev.attend_expanded(xd))
        absorbed = to_np(r.dev.attend(xd))
        for b in range(g.batch):
            ma, mr = r.check(got[b], x, b, what=f"expanded {g.name} {mode} n={r.n} b={b}")
            d = np.abs(got[b] - absorbed[b]).sum() / np.abs(absorbed[b]).sum()
            print(f"  b={b}: max_abs={ma:.3e} mean_rel={mr:.3e} (vs absorbed {d:.3e})", flush=True)
        r.append(r.x(chunk=k))


@pytest.mark.parametrize("mode", ["literal", "unit", "sharp"])
def test_expanded_small_grid_all_window_states(mode):
    _expanded_rollout(SMALL, mode, n_chunks=4)


@pytest.mark.parametrize("G", [1, 7, 100000])
def test_expanded_stream_k_splits(G):
    _expanded_rollout(SMALL, "sharp", n_chunks=3, attn_workgroups=G)


@pytest.mark.parametrize("dc", [96, 448])
def test_expanded_other_latent_widths(dc):
    # the up-projection (key lift with its identity block, value GEMM) at the other built widths
    _expanded_rollout(SMALL.replace(name=f"wan-widths-grid6x10-dc{dc}", d_c=dc), "sharp", n_chunks=3)


def test_expanded_batched_streams():
    _expanded_rollout(wl.STRESS[192].replace(grid_h=6, grid_w=10, window_frames=7), "sharp", n_chunks=3)


def test_expanded_requires_fresh_expand():
    g = SMALL
    r = Rollout(g, mode="unit")
    r.append(r.x(chunk=0))
    r.dev.expand()
    x = to_dev(r.x(chunk=9), g)
    r.dev.attend_expanded(x)            # fresh: fine
    r.append(r.x(chunk=1))
    with pytest.raises(vmla.VmlaError) as e:
        r.dev.attend_expanded(x)        # the window changed since the last expand
    assert e.value.code == vmla.STATUS["VMLA_ERR_STATE"]
    r.dev.expand()
    got = to_np(r.dev.attend_expanded(x))
    r.check(got[0], r.x(chunk=9), 0, what="after re-expand")


def test_expanded_wan_layer_full_size_sampled():
    g = wl.WAN_LAYER
    _case("expanded wan-full")
    r = Rollout(g, mode="literal", cache_fill=float("nan"))
    for k in range(g.prefill_chunks):
        r.append(r.x(chunk=k))
    r.dev.expand()
    x = r.x(chunk=g.prefill_chunks)
    got = to_np(r.dev.attend_expanded(to_dev(x, g)))
    assert np.all(np.isfinite(got))
    q = np.unique(np.concatenate([np.arange(8), np.arange(g.n_q - 8, g.n_q),
                                  np.random.default_rng(0).choice(g.n_q, 32, replace=False)]))
    ma, mr = r.check(got[0][q], x, 0, q, "expanded wan-full literal")
    print(f"expanded wan-full: max_abs={ma:.3e} mean_rel={mr:.3e}", flush=True)
