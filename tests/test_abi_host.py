"""Host-side checks of the C ABI: the library loads without a GPU, exports every
symbol include/vmla.h declares, and rejects bad arguments before any HIP call.
No test here launches a kernel."""
import ctypes
import os
import re

import pytest

from mla_latent_kv_vmla_amd import vmla, workloads as wl

HEADERS = [os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", f)
           for f in sorted(os.listdir(os.path.join(os.path.dirname(os.path.dirname(__file__)), "include")))
           if f.endswith(".h")]

FAKE = 0x7F0000000000  # 16-byte aligned address that is never dereferenced


def declared_symbols():
    out = []
    for h in HEADERS:
        out += re.findall(r"VMLA_API\s+[\w\s\*]*?\b(vmla_\w+)\s*\(", open(h).read())
    return out


def test_library_exports_every_declared_symbol():
    syms = declared_symbols()
    assert len(syms) >= 10
    L = ctypes.CDLL(vmla.LIB_PATH)
    for s in syms:
        assert hasattr(L, s), f"{s} declared but not exported"


def test_library_resolves_every_symbol_at_load():
    """Eager binding: a kernel whose host launch stub was not emitted shows up as
    an undefined symbol here instead of on first use."""
    ctypes.CDLL(vmla.LIB_PATH, mode=os.RTLD_NOW | os.RTLD_LOCAL)


def test_status_strings_and_codes():
    assert vmla.STATUS["VMLA_OK"] == 0
    assert len(set(vmla.STATUS.values())) == len(vmla.STATUS)
    for name, code in vmla.STATUS.items():
        assert vmla.vmla_status_string(code) not in ("", "unknown status")
    assert vmla.vmla_status_string(999) == "unknown status"


def _cfg(g=wl.WAN_LAYER, **kw):
    c = vmla.config_from_geometry(g)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def test_cache_and_workspace_bytes():
    g = wl.WAN_LAYER
    assert vmla.vmla_cache_bytes(_cfg(g)) == 1 * 21 * 1560 * 224 * 2  # 14.68 MB, bf16 rows of 224
    t = wl.TINY
    assert vmla.vmla_cache_bytes(_cfg(t)) == 2 * 16 * 32 * 4
    ws = vmla.vmla_workspace_bytes(_cfg(g))
    nq = 4680
    lower = nq * (224 + 768 + 12 * 96 + 12 * 224 + 12 * 192 + 1536) * 2
    assert ws >= lower
    b4 = wl.STRESS[192]
    assert vmla.vmla_cache_bytes(_cfg(b4)) == 4 * 42 * 1560 * 224 * 2


PARAMS_INVALID = [
    ("batch", 0, "VMLA_ERR_CONFIG"), ("hidden", 12, "VMLA_ERR_CONFIG"), ("d_nope", 0, "VMLA_ERR_CONFIG"),
    ("chunk_frames", 22, "VMLA_ERR_CONFIG"), ("rope_pairs_t", 5, "VMLA_ERR_CONFIG"),
    ("rope_theta", 0.0, "VMLA_ERR_CONFIG"), ("dtype", 7, "VMLA_ERR_CONFIG"), ("grid_w", 0, "VMLA_ERR_CONFIG"),
    ("attn_workgroups", -1, "VMLA_ERR_CONFIG"),
    ("d_c", 200, "VMLA_ERR_UNSUPPORTED"), ("dtype", vmla.VMLA_DTYPE_F32, "VMLA_ERR_UNSUPPORTED"),
]


def test_launch_grid_limits():
    """Streams and 64-token GEMM tiles of one call run along grid y (at most
    65,535): the Wan layer accepts 896 streams (4,193,280 query tokens) and
    rejects 897; a tiny frame caps the batch itself at 65,535."""
    assert vmla.vmla_cache_bytes(_cfg(batch=896)) > 0
    assert vmla.vmla_cache_bytes(_cfg(batch=897)) == 0
    assert vmla.vmla_dense_cache_bytes(vmla.config_from_geometry(wl.WAN_DENSE.replace(batch=897))) == 0
    # a whole-clip call runs window_frames * T = 32,760 tokens per Wan stream: at most 128 streams
    assert vmla.vmla_clip_workspace_bytes(_cfg(batch=128)) > 0
    assert vmla.vmla_clip_workspace_bytes(_cfg(batch=129)) == 0
    tiny = wl.TINY.replace(dtype=wl.BF16)
    assert vmla.vmla_cache_bytes(vmla.config_from_geometry(tiny.replace(batch=65535))) > 0
    assert vmla.vmla_cache_bytes(vmla.config_from_geometry(tiny.replace(batch=65536))) == 0


@pytest.mark.parametrize("field,value,code", PARAMS_INVALID)
def test_invalid_configs_rejected(field, value, code):
    c = _cfg(**{field: value})
    assert vmla.vmla_cache_bytes(c) == 0 and vmla.vmla_workspace_bytes(c) == 0
    with pytest.raises(vmla.VmlaError) as e:
        vmla.vmla_create(c, _fake_weights(), FAKE, FAKE)
    assert e.value.code == vmla.STATUS[code]


def _fake_weights(**override):
    d = {n: FAKE + 256 * i for i, n in enumerate(vmla.LatentAttention.WEIGHT_NAMES)}
    d.update(override)
    return vmla.vmla_weights(**d)


def test_create_rejects_null_and_misaligned():
    c = _cfg()
    for n in vmla.LatentAttention.WEIGHT_NAMES:
        with pytest.raises(vmla.VmlaError) as e:
            vmla.vmla_create(c, _fake_weights(**{n: 0}), FAKE, FAKE)
        assert e.value.code == vmla.STATUS["VMLA_ERR_NULL"]
        with pytest.raises(vmla.VmlaError) as e:
            vmla.vmla_create(c, _fake_weights(**{n: FAKE + 8}), FAKE, FAKE)
        assert e.value.code == vmla.STATUS["VMLA_ERR_ALIGN"]
    for cache, ws, code in [(0, FAKE, "VMLA_ERR_NULL"), (FAKE, 0, "VMLA_ERR_NULL"),
                            (FAKE + 4, FAKE, "VMLA_ERR_ALIGN"), (FAKE, FAKE + 2, "VMLA_ERR_ALIGN")]:
        with pytest.raises(vmla.VmlaError) as e:
            vmla.vmla_create(c, _fake_weights(), cache, ws)
        assert e.value.code == vmla.STATUS[code]
    with pytest.raises(vmla.VmlaError) as e:
        vmla.vmla_create(c, _fake_weights(), FAKE, FAKE, rope_freqs=[float("nan")] * 16)
    assert e.value.code == vmla.STATUS["VMLA_ERR_ARG"]


def test_calls_reject_bad_arguments_before_launch():
    ctx = vmla.vmla_create(_cfg(), _fake_weights(), FAKE, FAKE)
    try:
        bad = [
            (lambda: vmla.vmla_attend(ctx, 0, FAKE, 0), "VMLA_ERR_NULL"),
            (lambda: vmla.vmla_attend(ctx, FAKE, 0, 0), "VMLA_ERR_NULL"),
            (lambda: vmla.vmla_attend(ctx, FAKE + 2, FAKE, 0), "VMLA_ERR_ALIGN"),
            (lambda: vmla.vmla_compress_append(ctx, 0, 0), "VMLA_ERR_NULL"),
            (lambda: vmla.vmla_compress_append(ctx, FAKE + 8, 0), "VMLA_ERR_ALIGN"),
            (lambda: vmla.vmla_compress(ctx, FAKE, -1, FAKE, 0), "VMLA_ERR_ARG"),
            (lambda: vmla.vmla_compress(ctx, FAKE, 0, 0, 0), "VMLA_ERR_NULL"),
            # attend-type calls before vmla_prepare
            (lambda: vmla.vmla_attend(ctx, FAKE, FAKE, 0), "VMLA_ERR_STATE"),
            (lambda: vmla.vmla_attend_noalloc(ctx, FAKE, FAKE, 0), "VMLA_ERR_STATE"),
            (lambda: vmla.vmla_attend_noalloc(ctx, 0, FAKE, 0), "VMLA_ERR_NULL"),
            (lambda: vmla.vmla_attend_noalloc(ctx, FAKE, FAKE + 4, 0), "VMLA_ERR_ALIGN"),
            (lambda: vmla.vmla_attend_clip(ctx, FAKE, FAKE, FAKE, 0), "VMLA_ERR_STATE"),
            (lambda: vmla.vmla_range_flags(ctx, 0), "VMLA_ERR_STATE"),
        ]
        for f, code in bad:
            with pytest.raises(vmla.VmlaError) as e:
                f()
            assert e.value.code == vmla.STATUS[code]
        # a rejected append leaves the frame counter alone
        assert vmla.vmla_cache_state(ctx) == (0, 0, 0)
        vmla.vmla_reset(ctx)
        assert vmla.vmla_cache_state(ctx) == (0, 0, 0)
    finally:
        vmla.vmla_destroy(ctx)
    vmla.vmla_destroy(None)  # NULL is ignored


def test_null_ctx_rejected():
    L = vmla.lib()
    assert L.vmla_reset(None) == vmla.STATUS["VMLA_ERR_NULL"]
    assert L.vmla_cache_state(None, None, None, None) == vmla.STATUS["VMLA_ERR_NULL"]
    assert L.vmla_attend(None, FAKE, FAKE, None) == vmla.STATUS["VMLA_ERR_NULL"]
    L = vmla.lib()
    assert L.vmla_dense_reset(None) == vmla.STATUS["VMLA_ERR_NULL"]
    assert L.vmla_dense_cache_state(None, None, None, None) == vmla.STATUS["VMLA_ERR_NULL"]
    assert L.vmla_dense_attend(None, FAKE, FAKE, None) == vmla.STATUS["VMLA_ERR_NULL"]
    assert L.vmla_dense_append(None, FAKE, None) == vmla.STATUS["VMLA_ERR_NULL"]


# ----------------------------------------------------------------------------- dense baseline
def test_dense_cache_and_workspace_bytes():
    g = wl.WAN_DENSE
    P = (21 * 1560 + 127) // 128 * 128  # ring keys per (stream, head), padded to the 128-key tile
    assert P == 32768
    assert vmla.vmla_dense_cache_bytes(_cfg(g)) == 12 * P * (128 + 128) * 2  # 201.3 MB: keys + values, 16-bit
    ws = vmla.vmla_dense_workspace_bytes(_cfg(g))
    S = (4680 + 127) // 128 * 128
    assert ws >= 12 * (4680 * 128 + 2 * S * 128) * 2 + 4680 * 1536 * 2
    # the latent entry points refuse the dense geometry and vice versa
    assert vmla.vmla_cache_bytes(_cfg(g)) == 0
    assert vmla.vmla_dense_cache_bytes(_cfg(wl.WAN_LAYER)) == 0


@pytest.mark.parametrize("field,value,code", [
    ("d_c", 192, "VMLA_ERR_CONFIG"), ("d_q", 768, "VMLA_ERR_CONFIG"), ("d_nope", 8, "VMLA_ERR_CONFIG"),
    ("rope_pairs_w", 20, "VMLA_ERR_CONFIG"), ("batch", 0, "VMLA_ERR_CONFIG"),
    ("d_v", 64, "VMLA_ERR_UNSUPPORTED"), ("dtype", vmla.VMLA_DTYPE_F32, "VMLA_ERR_UNSUPPORTED"),
])
def test_dense_invalid_configs_rejected(field, value, code):
    c = _cfg(wl.WAN_DENSE, **{field: value})
    assert vmla.vmla_dense_cache_bytes(c) == 0 and vmla.vmla_dense_workspace_bytes(c) == 0
    w = vmla.vmla_dense_weights(w_q=FAKE, w_k=FAKE + 256, w_v=FAKE + 512, w_o=FAKE + 768)
    with pytest.raises(vmla.VmlaError) as e:
        vmla.vmla_dense_create(c, w, FAKE, FAKE)
    assert e.value.code == vmla.STATUS[code]


def test_dense_create_and_argument_checks():
    c = _cfg(wl.WAN_DENSE)
    names = vmla.DenseAttention.WEIGHT_NAMES
    good = {n: FAKE + 256 * i for i, n in enumerate(names)}
    for n in names:
        for v, code in [(0, "VMLA_ERR_NULL"), (FAKE + 8, "VMLA_ERR_ALIGN")]:
            with pytest.raises(vmla.VmlaError) as e:
                vmla.vmla_dense_create(c, vmla.vmla_dense_weights(**{**good, n: v}), FAKE, FAKE)
            assert e.value.code == vmla.STATUS[code]
    ctx = vmla.vmla_dense_create(c, vmla.vmla_dense_weights(**good), FAKE, FAKE)
    try:
        for f, code in [(lambda: vmla.vmla_dense_attend(ctx, 0, FAKE, 0), "VMLA_ERR_NULL"),
                        (lambda: vmla.vmla_dense_attend(ctx, FAKE, FAKE + 2, 0), "VMLA_ERR_ALIGN"),
                        (lambda: vmla.vmla_dense_append(ctx, FAKE + 4, 0), "VMLA_ERR_ALIGN"),
                        (lambda: vmla.vmla_dense_attend_profiled(ctx, FAKE, FAKE, 0, 0, 0), "VMLA_ERR_NULL")]:
            with pytest.raises(vmla.VmlaError) as e:
                f()
            assert e.value.code == vmla.STATUS[code]
        assert vmla.vmla_dense_cache_state(ctx) == (0, 0, 0)
    finally:
        vmla.vmla_dense_destroy(ctx)


# ----------------------------------------------------------------------------- expanded latent path
def test_expanded_bytes_and_state_checks():
    g = wl.WAN_LAYER
    nb = vmla.vmla_expanded_bytes(_cfg(g))
    P = (21 * 1560 + 127) // 128 * 128
    assert nb >= 12 * P * 256 * 2  # per-head keys and values of the window
    assert vmla.vmla_expanded_bytes(_cfg(wl.TINY)) == 0          # fp32 / 16-wide heads: no expanded kernel
    assert vmla.vmla_expanded_bytes(_cfg(g, d_v=64)) == 0        # value width != 128
    ctx = vmla.vmla_create(_cfg(g), _fake_weights(), FAKE, FAKE)
    try:
        # attend before any expand, or with another buffer: rejected before launch
        for f, code in [(lambda: vmla.vmla_attend_expanded(ctx, FAKE, FAKE, FAKE, 0), "VMLA_ERR_STATE"),
                        (lambda: vmla.vmla_attend_expanded(ctx, 0, FAKE, FAKE, 0), "VMLA_ERR_NULL"),
                        (lambda: vmla.vmla_attend_expanded(ctx, FAKE + 4, FAKE, FAKE, 0), "VMLA_ERR_ALIGN"),
                        (lambda: vmla.vmla_expand(ctx, 0, 0), "VMLA_ERR_NULL"),
                        (lambda: vmla.vmla_expand(ctx, FAKE + 2, 0), "VMLA_ERR_ALIGN"),
                        (lambda: vmla.vmla_attend_expanded_profiled(ctx, FAKE, FAKE, FAKE, 0, 0, 0),
                         "VMLA_ERR_NULL")]:
            with pytest.raises(vmla.VmlaError) as e:
                f()
            assert e.value.code == vmla.STATUS[code]
    finally:
        vmla.vmla_destroy(ctx)
    tiny = vmla.vmla_create(_cfg(wl.TINY), _fake_weights(), FAKE, FAKE)
    try:
        with pytest.raises(vmla.VmlaError) as e:
            vmla.vmla_expand(tiny, FAKE, 0)
        assert e.value.code == vmla.STATUS["VMLA_ERR_UNSUPPORTED"]
    finally:
        vmla.vmla_destroy(tiny)


# ----------------------------------------------------------------------------- sink frames / rope at use
def test_sink_config_rules():
    g = wl.WAN_SINK
    assert vmla.vmla_cache_bytes(_cfg(g)) == (1 + 6) * 1560 * 224 * 2  # one sink slot + six window slots
    assert vmla.vmla_cache_bytes(_cfg(g, rope_at_use=0)) == 0           # a sink needs rotation at use
    assert vmla.vmla_cache_bytes(_cfg(g, rope_at_use=2)) == 0
    assert vmla.vmla_cache_bytes(_cfg(g, sink_frames=-1)) == 0
    # rope at use without sinks is a valid layout choice
    assert vmla.vmla_cache_bytes(_cfg(wl.WAN_LAYER, rope_at_use=1)) == vmla.vmla_cache_bytes(_cfg(wl.WAN_LAYER))
    # the dense baseline has no sink / rotate-at-use kernel
    c = _cfg(wl.WAN_DENSE, sink_frames=1, rope_at_use=1)
    w = vmla.vmla_dense_weights(w_q=FAKE, w_k=FAKE + 256, w_v=FAKE + 512, w_o=FAKE + 768)
    with pytest.raises(vmla.VmlaError) as e:
        vmla.vmla_dense_create(c, w, FAKE, FAKE)
    assert e.value.code == vmla.STATUS["VMLA_ERR_UNSUPPORTED"]
    ctx = vmla.vmla_create(_cfg(g), _fake_weights(), FAKE, FAKE)
    try:
        assert vmla.vmla_cache_state(ctx) == (0, 0, 0)
    finally:
        vmla.vmla_destroy(ctx)


# ----------------------------------------------------------------------------- capacity arithmetic
def test_capacity_formulas_match_the_library():
    from mla_latent_kv_vmla_amd import capacity as cap
    cases = [(wl.WAN_LAYER, 64), (wl.WAN_SINK, 64), (wl.STRESS[96], 64), (wl.STRESS[192], 64), (wl.STRESS[448], 64),
             (wl.WAN_SMALL_GRID, 64)]
    for g, kt in cases:
        assert cap.latent_cache_bytes(g, g.batch) == vmla.vmla_cache_bytes(_cfg(g)), g.name
        assert cap.latent_workspace_bytes(g, g.batch, key_tile=kt) == vmla.vmla_workspace_bytes(_cfg(g)), g.name
    for g in (wl.WAN_DENSE, wl.WAN_DENSE_SMALL_GRID):
        assert cap.dense_cache_bytes(g, g.batch) == vmla.vmla_dense_cache_bytes(_cfg(g))
        assert cap.dense_workspace_bytes(g, g.batch) == vmla.vmla_dense_workspace_bytes(_cfg(g))


def test_capacity_sweep_orders_as_the_cache_sizes():
    from mla_latent_kv_vmla_amd import capacity as cap
    budget = 288 * 10**9
    dense = cap.capacity(wl.WAN_DENSE, 30, budget, dense=True)
    prev = None
    for dc in (64, 128, 192, 256, 512):
        c = cap.capacity(wl.WAN_LAYER.replace(d_c=dc), 30, budget)
        assert c.max_batch > dense.max_batch
        if prev is not None:
            assert c.max_batch <= prev
        prev = c.max_batch
        assert (c.max_batch + 1) * c.per_stream_bytes + c.fixed_bytes > budget >= c.max_batch * c.per_stream_bytes + c.fixed_bytes
    # the latent caches alone are 224 / 3,072 of the dense ones at d_c = 192
    assert cap.latent_cache_bytes(wl.WAN_LAYER) * 3072 == pytest.approx(
        cap.dense_cache_bytes(wl.WAN_DENSE) * 224, rel=1e-3)  # dense rows padded to 128 keys
