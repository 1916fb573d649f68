"""vmla_attend_noalloc, the attend entry point whose per-call buffers live in the
library's scratch array: through the C ABI, against vmla_attend on the same
ctx and inputs.  Two calls in a row, the second with a smaller input (the full
Wan-1.3B layer, then the Wan widths on a 6x10 grid); each output is
bit-identical to the workspace path's (same kernels, same inputs) and within
the parity bound of the oracle.  A ctx whose per-call buffers exceed the array
(four streams of a 42-frame window) is refused before anything runs."""
import numpy as np
import pytest

from gpu_harness import Rollout, to_dev, to_np
from mla_latent_kv_vmla_amd import vmla, workloads as wl

pytestmark = pytest.mark.gpu


def test_noalloc_matches_workspace_path_two_calls_second_smaller():
    import torch
    cases = [(wl.WAN_LAYER, "sharp", wl.WAN_LAYER.prefill_chunks), (wl.WAN_SMALL_GRID, "unit", 2)]
    for g, mode, appends in cases:
        print(f"case: noalloc {g.name} {mode} appends={appends}", flush=True)
        r = Rollout(g, mode=mode, cache_fill=float("nan"))
        for k in range(appends):
            r.append(r.x(chunk=k))
        x = r.x(chunk=40)
        xd = to_dev(x, g)
        want = r.dev.attend(xd)
        got = torch.full_like(xd, float("nan"))
        vmla.vmla_attend_noalloc(r.dev.ctx, xd, got)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), want.view(torch.int16)), f"{g.name}: differs from vmla_attend"
        q = np.unique(np.concatenate([np.arange(4), np.arange(g.n_q - 4, g.n_q),
                                      np.random.default_rng(4).choice(g.n_q, min(40, g.n_q), replace=False)]))
        ma, mr = r.check(to_np(got)[0][q], x, 0, q, f"noalloc {g.name}")
        print(f"  {g.name}: identical to vmla_attend; max_abs={ma:.3e} mean_rel={mr:.3e}", flush=True)
        r.dev.close()


def test_noalloc_refuses_per_call_buffers_beyond_the_array():
    import torch
    g = wl.STRESS[192]
    print(f"case: noalloc refuses {g.name}", flush=True)
    r = Rollout(g, mode="literal")
    assert vmla.vmla_workspace_bytes(r.dev.cfg) > (128 << 20)
    x = to_dev(r.x(chunk=0), g)
    with pytest.raises(vmla.VmlaError) as e:
        vmla.vmla_attend_noalloc(r.dev.ctx, x, torch.empty_like(x))
    assert e.value.code == vmla.STATUS["VMLA_ERR_SCRATCH"]
    r.dev.close()
