#!/usr/bin/env python3
"""Benchmark of the latent-KV attention hot path on one MI355X.

One step = one chunk of one layer in the streaming rollout at the Wan2.1-1.3B
geometry (VideoMLA paper, section 4.1 and appendix D.1): `steps_per_chunk`
frozen-cache vmla_attend calls (the 4-step student sampler, appendix D.5)
followed by one vmla_compress_append that writes the chunk into the
21-frame ring and evicts the oldest frames.  The window is full (32,760 cached
keys + 4,680 chunk keys) for every timed step.  Inputs are seeded synthetic
tensors already resident in HBM; weights are random N(0,1)/sqrt(fan_in).
With the 30-layer rollout workload a step is that chunk for every layer in turn
(each with its own weights, ring and inputs), so the layers' caches (440 MB)
cycle through the GPU's last-level cache as they do in a rollout.

Prints one JSON line.  `value` = query tokens attended per second.
`roofline` describes the dominant kernel (latent attention) timed live with
HIP events recorded by the library around it; `cpu_baseline` times the CPU
oracle on a bounded sample of the same workload on this host's cores.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 (for fp32 workloads)
PEAK_HBM_GBS = 8000.0
METRIC = "query tokens/s and MFMA TFLOP/s (% peak) per layer, Wan-1.3B latent attn"
ATTN_SOURCE = os.path.join(ROOT, "mla_latent_kv_vmla_amd", "csrc", "attention.hip")


def is_dense(g) -> bool:
    return g.d_c == 0


def attention_flops(g, n_frames: int, expanded: bool = False) -> float:
    """Algorithmic FLOPs of one attention launch: per (query row, key) 2*(d_c+d_r)
    for the score and 2*d_c for the value sum (latent, absorbed), or 2*d_h + 2*d_v
    (dense, and the latent layer with its window expanded to per-head K/V)."""
    rows = g.batch * g.n_q * g.n_heads
    per = 2.0 * g.head_dim + 2.0 * g.d_v if (is_dense(g) or expanded) else 2.0 * (g.d_c + g.d_rope) + 2.0 * g.d_c
    return rows * g.n_k(n_frames) * per


def clip_attention_flops(g) -> float:
    """Algorithmic FLOPs of one block-causal clip launch: block q's rows against
    the keys of blocks 0..q."""
    T, C, F = g.tokens_per_frame, g.chunk_frames, g.window_frames
    per = 2.0 * (g.d_c + g.d_rope) + 2.0 * g.d_c
    tot = 0.0
    for q0 in range(0, F, C):
        c = min(C, F - q0)
        tot += g.batch * c * T * g.n_heads * (q0 + c) * T * per
    return tot


def attend_call_flops(g, n_frames: int, expanded: bool = False) -> float:
    """All algorithmic FLOPs of one attend call (projections + attention); for the
    expanded path the chunk's own keys/values are up-projected in the call (the
    window's expansion, once per chunk, is not counted here)."""
    M = g.batch * g.n_q
    d, nh, D = g.hidden, g.n_heads, g.d_c + g.d_rope
    if is_dense(g):
        gemm = 2.0 * M * d * nh * (2 * g.head_dim + g.d_v) + 2.0 * M * nh * g.d_v * d
    elif expanded:
        gemm = 2.0 * M * (d * D + d * g.d_q + g.d_q * nh * g.head_dim + nh * (g.head_dim * D + g.d_v * g.d_c)
                          + nh * g.d_v * d)
    else:
        gemm = 2.0 * M * (d * D + d * g.d_q + g.d_q * nh * g.head_dim
                          + nh * g.d_nope * g.d_c + nh * g.d_c * g.d_v + nh * g.d_v * d)
    return gemm + attention_flops(g, n_frames, expanded)


class HipEvents:
    """hipEvent_t handles from the HIP runtime torch has loaded."""

    def __init__(self):
        import torch  # noqa: F401  (loads the runtime first)
        self.h = ctypes.CDLL("libamdhip64.so.7")
        self.h.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.h.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self):
        e = ctypes.c_void_p()
        assert self.h.hipEventCreate(ctypes.byref(e)) == 0
        return e.value

    def elapsed_ms(self, a, b) -> float:
        t = ctypes.c_float()
        assert self.h.hipEventElapsedTime(ctypes.byref(t), a, b) == 0
        return t.value

    def destroy(self, e):
        self.h.hipEventDestroy(e)


def pmc_summary_path(g) -> str:
    return os.path.join(ROOT, "profiles", f"flash_attn_{g.name}_pmc.json")


def counter_summary(g) -> dict:
    """The committed rocprofv3 counter summary of this workload's attention kernel,
    if it was taken on the current kernel source (else empty)."""
    try:
        s = json.load(open(pmc_summary_path(g)))
        sha = hashlib.sha256(open(ATTN_SOURCE, "rb").read()).hexdigest()
        if s.get("attention_source_sha256") == sha:
            return s
    except (OSError, ValueError):
        pass
    return {}


def traffic_from_counters(g):
    """HBM bytes per launch of the attention kernel (calibrated FETCH_SIZE + WRITE_SIZE)."""
    return counter_summary(g).get("hbm_bytes_per_launch")


def trace_summary(g, path_tag="") -> dict:
    """The committed rocprofv3 kernel-trace summary of this workload, if it was
    taken on the current kernel source (else empty): average duration per kernel
    of the attend call, and the live HIP-event average of the same run."""
    try:
        p = os.path.join(ROOT, "profiles", f"flash_attn_{g.name}{path_tag}_kernel_stats.json")
        s = json.load(open(p))
        sha = hashlib.sha256(open(ATTN_SOURCE, "rb").read()).hexdigest()
        if s.get("attention_source_sha256") == sha:
            return s
    except (OSError, ValueError):
        pass
    return {}


def cpu_baseline(g, w, hist, n, x, sample_tokens: int):
    """The oracle as it stands (float64 numpy) on a contiguous sample of query
    tokens of the same call; returns query tokens/s of the sample."""
    import numpy as np
    from oracle import mla
    attend = mla.attend_dense if is_dense(g) else mla.attend
    threads = None
    try:
        from threadpoolctl import threadpool_info
        threads = max((p.get("num_threads") or 0) for p in threadpool_info()) or None
    except Exception:
        pass
    q = np.arange(sample_tokens)
    t0 = time.perf_counter()
    attend(g, w, hist, n, x, query_tokens=q)
    dt = time.perf_counter() - t0
    cpu_model = None
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), None)
    except OSError:
        pass
    return {"value": sample_tokens / dt, "unit": "query tokens/s", "cores": threads or os.cpu_count(),
            "kind": "oracle", "blas_threads": threads, "host_cpus": os.cpu_count(), "cpu_model": cpu_model,
            "sample": (f"{sample_tokens} of {g.n_q} query tokens (all {g.n_heads} heads) of one attend call "
                       f"against the full {g.n_k(n)} keys, float64 numpy; {dt:.1f} s")}


def capacity_run(args):
    """Memory-headroom sweep: the largest batch of independent streams whose
    30-layer caches stay resident on this GPU, for the latent layer at several
    d_c and for the dense baseline (arithmetic from the library's layouts, priced
    against this GPU's free memory).  Then, for the latent layer at d_c = 192 and
    for the dense layer, allocate exactly that: 30 layers' caches and weights plus
    one layer's per-call buffers, fill the first layer's window (7 chunk appends)
    and time one more append and one attend at that batch.  Inputs are seeded and
    generated on the device; only the first layer's ring is read, the others
    stand for the resident caches of a 30-layer model."""
    import torch
    from mla_latent_kv_vmla_amd import capacity as cap, vmla, workloads as wl
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    free, total = torch.cuda.mem_get_info()
    budget = free - (6 << 30)  # runtime, code objects and allocator rounding
    layers = 30
    sweep = []
    for dc in (64, 128, 192, 256, 512):
        c = cap.capacity(wl.WAN_LAYER.replace(d_c=dc), layers, budget)
        sweep.append({"d_c": dc, "per_stream_gb": round(c.per_stream_bytes / 1e9, 4), "max_batch": int(c.max_batch)})
    d = cap.capacity(wl.WAN_DENSE, layers, budget, dense=True)
    dense = {"per_stream_gb": round(d.per_stream_bytes / 1e9, 4), "max_batch": int(d.max_batch)}
    runs = {}
    gen = torch.Generator(device=dev).manual_seed(11)
    for name, g0, B, is_dense in (("latent_dc192", wl.WAN_LAYER, sweep[2]["max_batch"], False),
                                  ("dense", wl.WAN_DENSE, dense["max_batch"], True)):
        g = g0.replace(batch=B)
        print(f"capacity: {name} batch {B}", file=sys.stderr, flush=True)
        w = (wl.dense_weights if is_dense else wl.latent_weights)(g).__dict__
        lay = (vmla.DenseAttention if is_dense else vmla.LatentAttention)(g, w, device=dev)
        wbytes = sum(t.numel() * t.element_size() for t in lay.w.values())
        # every other layer also keeps its prepared weights (persistent workspace part)
        wbytes += (cap.dense_workspace_bytes(g, 1, part="persistent") if is_dense
                   else cap.latent_workspace_bytes(g, 1, part="persistent"))
        others = [torch.empty(lay.cache.numel() * lay.cache.element_size() + wbytes, dtype=torch.uint8, device=dev)
                  for _ in range(layers - 1)]
        x = torch.randn(B, g.n_q, g.hidden, generator=gen, device=dev, dtype=torch.bfloat16).mul_(g.hidden ** -0.5)
        out = torch.empty_like(x)
        allocated = torch.cuda.memory_allocated(dev)
        for _ in range(g.window_frames // g.chunk_frames):
            lay.append(x)
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record()
        lay.attend(x, out=out)
        e[1].record()
        lay.append(x)
        e[2].record()
        torch.cuda.synchronize()
        attend_ms = e[0].elapsed_time(e[1])
        runs[name] = {"batch": B, "allocated_gb": round(allocated / 1e9, 2), "frames_cached": lay.state()[2],
                      "attend_ms": round(attend_ms, 2), "append_ms": round(e[1].elapsed_time(e[2]), 2),
                      "attend_tokens_per_s": round(B * g.n_q / (attend_ms / 1e3)),
                      "output_finite": all(bool(torch.isfinite(out[i:i + 8]).all().item()) for i in range(0, B, 8))}
        lay.close()
        del lay, others, x, out
        torch.cuda.empty_cache()
    res = {"metric": "streams with 30-layer caches resident on one GPU (memory-headroom sweep)",
           "budget_gb": round(budget / 1e9, 2), "device_total_gb": round(total / 1e9, 2), "layers": layers,
           "workload": f"{wl.WAN_LAYER.name} chunk, {wl.WAN_LAYER.window_frames}-frame window",
           "latent": sweep, "dense": dense,
           "headroom_x": {str(r["d_c"]): round(r["max_batch"] / max(1, dense["max_batch"]), 2) for r in sweep},
           "run": runs}
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="wan1.3b-layer")
    ap.add_argument("--steps-per-chunk", type=int, default=4)
    ap.add_argument("--path", choices=("absorbed", "expanded", "clip"), default="absorbed",
                    help="latent layer: absorbed queries (default), the window up-projected once per chunk, "
                         "or one block-causal attend over a whole window-length clip per step")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=0,
                    help="query tokens the CPU oracle baseline times (0 = the whole attend call)")
    ap.add_argument("--calibrate-copy-mb", type=int, default=0,
                    help="after timing, run plain device copies of this size (counter calibration)")
    ap.add_argument("--capacity", action="store_true",
                    help="instead of the throughput step: the memory-headroom batch sweep (see capacity_run)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the latent-attention path runs on a single MI355X (how it would "
              "shard is described in the design notes, not implemented); --gpus above 1 is not supported.",
              file=sys.stderr)
        sys.exit(2)

    if args.capacity:
        capacity_run(args)
        return

    import numpy as np
    import torch
    from mla_latent_kv_vmla_amd import vmla, workloads as wl

    g = wl.GEOMETRIES[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    dt = vmla.torch_dtype(g)
    if is_dense(g):
        w = wl.dense_weights(g, mode="literal")
        layer = vmla.DenseAttention(g, {k: torch.from_numpy(v) for k, v in vars(w).items()})
        attend_profiled, append = vmla.vmla_dense_attend_profiled, vmla.vmla_dense_append
        kernel = "flash_attn_kernel (dense, per-head K/V)"
    else:
        w = wl.latent_weights(g, mode="literal")
        layer = vmla.LatentAttention(g, {k: torch.from_numpy(v) for k, v in w.as_dict().items()})
        # a multi-layer geometry (the streaming rollout) runs every layer per step, each
        # with its own seeded weights, ring cache and inputs
        extra_layers = [vmla.LatentAttention(g, {k: torch.from_numpy(v) for k, v in
                                                 wl.latent_weights(g, layer=l, mode="literal").as_dict().items()})
                        for l in range(1, g.layers if args.path == "absorbed" else 1)]
        attend_profiled, append = vmla.vmla_attend_profiled, vmla.vmla_compress_append
        # bf16 at d_c = 96, 192 and 448 runs the software-pipelined kernel
        lat = "flash_attn_pipe_kernel" if (g.d_c in (96, 192, 448) and g.dtype == "bf16") else "flash_attn_kernel"
        kernel = f"{lat} (latent, absorbed)"
        if args.path == "clip":
            clip_ws = torch.empty(vmla.vmla_clip_workspace_bytes(layer.cfg), dtype=torch.uint8, device=dev)
            kernel = f"{lat} (latent, block-causal clip)"
        if args.path == "expanded":
            expanded = torch.empty(vmla.vmla_expanded_bytes(layer.cfg), dtype=torch.uint8, device=dev)
            attend_profiled = lambda ctx, x, o, a, b, st: vmla.vmla_attend_expanded_profiled(ctx, expanded, x, o, a,
                                                                                            b, st)
            kernel = "flash_attn_kernel (latent window expanded to per-head K/V)"
    if is_dense(g):
        extra_layers = []
    layers = [layer] + extra_layers
    hist = {}
    # the window is full for every timed step: geometries without a prefill get one window's worth
    prefill_chunks = g.prefill_chunks or -(-g.window_frames // g.chunk_frames)
    for k in range(prefill_chunks):
        xk = wl.hidden_states(g, chunk=k)
        xkd = torch.from_numpy(xk).to(dev, dt)
        for l, lay in enumerate(layers):  # layer l's hidden states: layer 0's rolled by 37 l tokens
            lay.append(torch.roll(xkd, shifts=37 * l, dims=1).contiguous() if l else xkd)
        for i in range(g.chunk_frames):
            hist[k * g.chunk_frames + i] = xk[0].reshape(g.chunk_frames, g.tokens_per_frame, g.hidden)[i]
    n_prefill = layer.state()[0]
    xs_np = [wl.hidden_states(g, chunk=prefill_chunks, step=s) for s in range(args.steps_per_chunk)]
    xs = [torch.from_numpy(a).to(dev, dt) for a in xs_np]
    xs_layers = [xs] + [[torch.roll(x, shifts=37 * l, dims=1).contiguous() for x in xs]
                        for l in range(1, len(layers))]
    out = torch.empty_like(xs[0])
    if args.path == "clip":  # one whole window-length clip per step, no cache
        if is_dense(g):
            raise SystemExit("--path clip runs the latent layer")
        args.steps_per_chunk = 1
        gc = g.replace(chunk_frames=g.window_frames)
        xs_np = [wl.hidden_states(gc, chunk=999)]
        xs = [torch.from_numpy(xs_np[0]).to(dev, dt)]
        out = torch.empty_like(xs[0])
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream

    ev = HipEvents()
    L = len(layers)
    n_att = (args.warmup + args.steps) * args.steps_per_chunk * L
    ev_pairs = [(ev.create(), ev.create()) for _ in range(n_att)]
    step_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.warmup + args.steps)]

    def step(i):
        if args.path == "clip":
            a, b = ev_pairs[i]
            vmla.vmla_attend_clip_profiled(layer.ctx, xs[0], clip_ws, out, a, b, sh)
            return
        if args.path == "expanded" and not is_dense(g):
            vmla.vmla_expand(layer.ctx, expanded, sh)  # once per chunk: the frozen window's per-head K/V
        for l, lay in enumerate(layers):
            xl = xs_layers[l]
            for s in range(args.steps_per_chunk):
                a, b = ev_pairs[(i * L + l) * args.steps_per_chunk + s]
                attend_profiled(lay.ctx, xl[s], out, a, b, sh)
            append(lay.ctx, xl[-1], sh)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    region0 = torch.cuda.Event(enable_timing=True)
    region1 = torch.cuda.Event(enable_timing=True)
    region0.record(stream)
    for i in range(args.warmup, args.warmup + args.steps):
        step_ev[i][0].record(stream)
        step(i)
        step_ev[i][1].record(stream)
    region1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_region = region0.elapsed_time(region1)
    ms_per_step = ms_region / args.steps

    attn_ms = [ev.elapsed_ms(a, b) for a, b in ev_pairs[args.warmup * args.steps_per_chunk * L:]]
    attn_avg = float(np.mean(attn_ms))
    n_frames = layer.state()[0]  # frames appended; n_k counts the visible ones (sinks + window)
    flops_attn = (clip_attention_flops(g) if args.path == "clip"
                  else attention_flops(g, n_frames, expanded=args.path == "expanded"))
    achieved = flops_attn / (attn_avg * 1e-3) / 1e12
    peak = PEAK_F32_TFLOPS if g.dtype == wl.F32 else PEAK_BF16_TFLOPS
    tokens_per_step = (g.batch * g.window_frames * g.tokens_per_frame if args.path == "clip"
                       else g.batch * g.n_q * args.steps_per_chunk * L)
    value = tokens_per_step / (ms_per_step * 1e-3)
    call_flops = attend_call_flops(g, n_frames, expanded=args.path == "expanded")
    if args.path == "clip":
        call_flops = flops_attn

    if args.calibrate_copy_mb > 0:
        nbytes = args.calibrate_copy_mb << 20
        src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    traffic = traffic_from_counters(g) if args.path == "absorbed" else None
    # The attention step as the committed trace of this workload times it: the
    # key-tile pre-pass, the kernel and the split combine (same kernel source only)
    ts = trace_summary(g, "" if args.path == "absorbed" else f"-{args.path}")
    step_us = ts.get("attention_step_us")
    res = {
        "metric": METRIC,
        "value": value,
        "unit": "query tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if g.dtype == wl.F32 else "bf16",
        # operands of the matrix-core products: bf16 storage runs its attention
        # and the projections after c^Q on fp16 copies (same MFMA rate)
        "mfma_operands": "f32" if g.dtype == wl.F32 else "fp16",
        "data": "synthetic (seeded N(0,1)/sqrt(fan_in) weights and hidden states)",
        "config": {"workload": g.name if args.path == "absorbed" else f"{g.name}-{args.path}", "batch": g.batch,
                   "query_tokens_per_call": g.window_frames * g.tokens_per_frame if args.path == "clip" else g.n_q,
                   "keys_per_call": (g.window_frames * g.tokens_per_frame if args.path == "clip"
                                     else g.n_k(n_frames)),
                   "heads": g.n_heads, "head_dim": g.head_dim,
                   "d_c": g.d_c, "d_rope": g.d_rope,
                   "window_frames": g.window_frames, "chunk_frames": g.chunk_frames,
                   "layers": L, "attends_per_step": args.steps_per_chunk * L, "appends_per_step": L,
                   "expands_per_step": 1 if args.path == "expanded" else 0, "sink_frames": g.sink_frames},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                     "frac": achieved / peak, "traffic": traffic,
                     # counter bytes over the live launch time, against the 8 TB/s HBM peak
                     "hbm_gb_per_s": traffic / (attn_avg * 1e-3) / 1e9 if traffic else None,
                     "hbm_frac": traffic / (attn_avg * 1e-3) / 1e9 / PEAK_HBM_GBS if traffic else None,
                     "kernel": kernel,
                     "flops_per_launch": flops_attn, "avg_launch_ms": attn_avg,
                     # MFMA work the counters saw (padding included) and the matrix cores' busy share
                     "mfma_counter_flops_per_launch": (counter_summary(g).get("mfma_flops_per_launch")
                                                       if args.path == "absorbed" else None),
                     "mfma_busy_frac": counter_summary(g).get("mfma_busy_frac") if args.path == "absorbed" else None,
                     # the committed trace of this workload: kernel average, and the whole
                     # attention step (pre-pass + kernel + combine) against the same peak
                     "trace_kernel_avg_ms": ts.get("attention_kernel_us", 0) / 1e3 or None,
                     "trace_step_avg_ms": step_us / 1e3 if step_us else None,
                     "trace_step_frac": flops_attn / (step_us * 1e-6) / 1e12 / peak if step_us else None},
        "attend_call_tflops": call_flops * args.steps_per_chunk * L / (ms_per_step * 1e-3) / 1e12,
        "wall_s_timed_region": wall,
    }
    if not args.no_cpu_baseline and args.path != "clip" and L == 1:
        res["cpu_baseline"] = cpu_baseline(g, w, hist, n_prefill, xs_np[0][0], args.cpu_sample_tokens or g.n_q)
    for a, b in ev_pairs:
        ev.destroy(a)
        ev.destroy(b)
    for lay in layers:
        lay.close()
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
