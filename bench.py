#!/usr/bin/env python3
"""Throughput of block-causal ReLU linear attention with RoPE on one MI355X.

One step = one whole forward pass (block states, block prefix, readout) over
the workload's synthetic bf16 inputs, already resident in HBM.  Prints one JSON
line: token-heads/s for the whole step, the roofline of the dominant kernel
(algorithmic bytes / its HIP-event duration against 8 TB/s), per-kernel times,
the streaming per-block latency, and the fp64 oracle timed on a bounded
sample on the host cores.
"""

import argparse
import ctypes
import hashlib
import json
import multiprocessing as mp
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from linear_attention_video_relu_amd import workloads as W  # noqa: E402

METRIC = "tokens·heads/s and achieved HBM GB/s (% peak), block-causal LA fwd"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure


def rec_bytes(d):
    """Bytes of one fp32 (S, z) record at head dim d."""
    return (d * d + d) * 4


KERNEL_SOURCES = ("la_kernels.hip", "la_internal.h", "la_api.cpp")


# ---------------------------------------------------- counter-measured traffic

def kernel_source_digest():
    """sha256 over the sources that decide what the kernels load and store."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "linear_attention_video_relu_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` from the committed FETCH_SIZE / WRITE_SIZE passes.

    The summary under profiles/ carries a JSON block with the digest of the kernel
    sources the counters were taken on; when the sources have changed since, the
    figure no longer describes the built kernels and None is returned."""
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.md")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        m = re.search(r"```json\n(.*?)\n```", f.read(), re.S)
    if m is None:
        return None
    rec = json.loads(m.group(1))
    if rec.get("kernel_sources_sha256") != kernel_source_digest():
        return None
    return rec.get("kernels", {}).get(kernel, {}).get("traffic_bytes")


# ------------------------------------------------------------- CPU baseline leg

_CPU_JOB = {}


def _oracle_task(h):
    cfg, arrs = _CPU_JOB["cfg"], _CPU_JOB["arrs"]
    try:
        from threadpoolctl import threadpool_limits
        ctx = threadpool_limits(1)
    except Exception:
        ctx = None
    import oracle
    t = time.perf_counter()
    q, k, v = (W.to_f64(cfg, arrs[x][0, :, h]) for x in W.TENSORS)
    oracle.forward_head(q, k, v, cfg["tokens_per_frame"], cfg["block_frames"], W.oracle_rope(cfg))
    if ctx is not None:
        ctx.unregister()
    return time.perf_counter() - t


def cpu_model():
    """The host CPU's model name from /proc/cpuinfo (None if unreadable)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


# Worker processes of the oracle leg.  A one-GPU machine grants this process a
# share of 16 host cores whatever the affinity mask shows, and more workers
# than that oversubscribe the share.
MAX_CPU_WORKERS = 16


def cpu_baseline(cfg, arrs, n_heads):
    """Time the fp64 oracle on heads 0 .. n_heads-1 of batch row 0, one process per head.

    Runs before anything touches the GPU, so the forked workers inherit the drawn
    inputs without copying them."""
    _CPU_JOB.update(cfg=cfg, arrs=arrs)
    host_cores = len(os.sched_getaffinity(0))
    workers = max(1, min(n_heads, host_cores, MAX_CPU_WORKERS))
    ctxm = mp.get_context("fork")
    t = time.perf_counter()
    with ctxm.Pool(workers) as pool:
        per = pool.map(_oracle_task, list(range(n_heads)))
    wall = time.perf_counter() - t
    _CPU_JOB.clear()
    N = W.n_tokens(cfg)
    return {"value": n_heads * N / wall, "unit": "tokens·heads/s", "cores": workers,
            "workers": workers, "host_cores": host_cores, "cpu_model": cpu_model(),
            "kind": "oracle",
            "sample": f"{n_heads} of {cfg['B'] * cfg['H']} (batch, head) streams of {cfg['name']}, "
                      f"full length {N} tokens, fp64 numpy oracle (inputs widened from bf16 inside "
                      f"the timed work), one process per stream, 1 BLAS thread each; "
                      f"{sum(per):.1f} s of CPU work in {wall:.1f} s wall",
            "cpu_seconds": round(sum(per), 2), "wall_seconds": round(wall, 2)}


# ------------------------------------------------------------------- GPU timing

# Timing events: la_block_causal_forward_timed binds them to the kernels' own
# dispatches (start and end of the block-state kernel and of the readout), so
# they put no command between the kernels.  They are created without the
# system-scope fence (hipEventDisableSystemFence): an event that completes
# with that fence writes back and invalidates the caches, which would perturb
# the next kernel.  The timed region still ends with a device synchronize.
HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000


class HipEvents:
    def __init__(self, n, flags=HIP_EVENT_DISABLE_SYSTEM_FENCE):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.ev = (ctypes.c_void_p * n)()
        for i in range(n):
            e = ctypes.c_void_p()
            rc = self.hip.hipEventCreateWithFlags(ctypes.byref(e), ctypes.c_uint(flags))
            if rc != 0:
                raise RuntimeError(f"hipEventCreate failed: {rc}")
            self.ev[i] = e.value

    def marks(self, *slots):
        """The four-entry event array of one timed forward call (block-state start
        and end, readout start and end): slot numbers, or None for a point that is
        not recorded."""
        return (ctypes.c_void_p * 4)(*(None if i is None else self.ev[i] for i in slots))

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(self.ev[a]),
                                          ctypes.c_void_p(self.ev[b]))
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {rc}")
        return ms.value


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="minute_bf16", choices=sorted(W.WORKLOADS))
    ap.add_argument("--cpu-heads", type=int, default=30, help="oracle sample size (0 = skip)")
    ap.add_argument("--stream-reps", type=int, default=3, help="timed 40-call streaming runs (0 = skip)")
    ap.add_argument("--backward-steps", type=int, default=10,
                    help="timed la_block_causal_backward calls on the same workload (0 = skip)")
    ap.add_argument("--prologue-steps", type=int, default=10,
                    help="timed fused q/k/v + q/k RMSNorm forward calls on the same workload (0 = skip)")
    ap.add_argument("--tconv-steps", type=int, default=20,
                    help="timed cached temporal convolution calls at the workload's token grid (0 = skip)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a 1 GiB fill and a 1 GiB device copy, the known-size kernels "
                         "that scale the HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the path is measured on a single MI355X "
              "(--gpus 1); runs on several GPUs are not measured by this benchmark.", file=sys.stderr)
        sys.exit(2)

    cfg = W.workload(args.workload)
    B, H, N, d = cfg["B"], cfg["H"], W.n_tokens(cfg), cfg["head_dim"]
    tpf, bf = cfg["tokens_per_frame"], cfg["block_frames"]
    t = time.perf_counter()
    arrs = {x: W.draw(cfg, x) for x in W.TENSORS}
    print(f"[bench] drew {cfg['name']} inputs in {time.perf_counter() - t:.1f}s", file=sys.stderr, flush=True)

    cpu = None
    if args.cpu_heads > 0:
        cpu = cpu_baseline(cfg, arrs, args.cpu_heads)
        print(f"[bench] cpu baseline {cpu['value']:.3e} token-heads/s on {cpu['cores']} cores",
              file=sys.stderr, flush=True)

    import torch
    import __graft_entry__
    __graft_entry__.ensure_built()
    from linear_attention_video_relu_amd import lavr

    dev = torch.device("cuda:0")
    q, k, v = (W.to_torch(cfg, arrs[x], dev) for x in W.TENSORS)
    del arrs
    dt = q.dtype
    rope = lavr.RopeTable(cfg["rope"]["split"], cfg["grid"], cfg["frames"], cfg["rope"]["base"], dev)
    out = torch.empty_like(q)
    need = lavr.workspace_bytes(B, H, cfg["frames"], tpf, bf, head_dim=d, rope=rope)
    ws = torch.zeros(need, dtype=torch.uint8, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    code = lavr._dtype_code(dt)
    ptrs = [ctypes.c_void_p(x.data_ptr()) for x in (q, k, v, out)]

    def fwd():
        rc = lavr.lib.la_block_causal_forward(*ptrs, code, code, B, H, d, cfg["frames"], tpf, bf, 0,
                                              ctypes.byref(rope.desc), 1e-8,
                                              ctypes.c_void_p(ws.data_ptr()), need, stream)
        if rc:
            raise RuntimeError(lavr.status_string(rc))

    K = args.steps
    # Timed step i binds two events, slots 2i and 2i+1, to its readout's start
    # and end.  Each bound event still costs ~1.5 us of the timeline (20-step
    # runs at the steady clock: 1.1765 ms with no events, 1.1794 with the
    # readout's two, 1.1848 with all four), so the split of the rest of the step
    # into block state and prefix comes from a pass with all four after the
    # timed steps.
    ev = HipEvents(2 * K)
    marks = [ev.marks(None, None, 2 * i, 2 * i + 1) for i in range(K)]
    n_split = min(K, 10)
    ev_split = HipEvents(4 * n_split)
    marks_split = [ev_split.marks(4 * i, 4 * i + 1, 4 * i + 2, 4 * i + 3) for i in range(n_split)]

    def fwd_timed(m):
        rc = lavr.lib.la_block_causal_forward_timed(*ptrs, code, code, B, H, d, cfg["frames"], tpf,
                                                    bf, 0, ctypes.byref(rope.desc), 1e-8,
                                                    ctypes.c_void_p(ws.data_ptr()), need, stream, m)
        if rc:
            raise RuntimeError(lavr.status_string(rc))

    if args.calib_copy:
        x = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        x.fill_(1.0)                    # writes 1 GiB
        y = torch.empty_like(x)
        y.copy_(x)                      # reads 1 GiB, writes 1 GiB
        torch.cuda.synchronize(dev)
        del x, y
    for _ in range(args.warmup):
        fwd()
    torch.cuda.synchronize(dev)
    print(f"[bench] warmup done ({args.warmup} steps)", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    for i in range(K):
        fwd_timed(marks[i])
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / K
    # readout: its own two points; the rest of the step (block state, prefix and
    # the launch boundaries): from one readout's end to the next one's start
    t_read = np.array([ev.elapsed_ms(2 * i, 2 * i + 1) for i in range(K)])
    t_rest = np.array([ev.elapsed_ms(2 * i - 1, 2 * i) for i in range(1, K)])
    ev_span = ev.elapsed_ms(0, 2 * K - 1)      # readout 0 start .. readout K-1 end
    for i in range(n_split):
        fwd_timed(marks_split[i])
    torch.cuda.synchronize(dev)
    split = np.array([[ev_split.elapsed_ms(4 * i + a, 4 * i + a + 1) for a in range(3)]
                      for i in range(n_split)])
    k_state, k_prefix, k_read_split = (float(x) for x in split.mean(axis=0))
    k_read = float(t_read.mean())
    print(f"[bench] timed {K} steps: {ms_step:.4f} ms/step", file=sys.stderr, flush=True)

    th = B * N * H
    esz = 2 if dt == torch.bfloat16 else 4
    nb = -(-cfg["frames"] // bf)
    state_io = B * H * nb * rec_bytes(d)
    bytes_state = 2 * th * d * esz + state_io           # K, V read; block states out
    bytes_read = 2 * th * d * esz + state_io            # Q read, O written; block prefixes in
    bytes_step = 4 * th * d * esz + 2 * state_io
    kernels = {
        # block state and prefix from the four-point pass after the timed steps
        "k_block_state": {"ms": k_state, "alg_bytes": bytes_state,
                          "gbs": bytes_state / (k_state * 1e6), "source": f"{n_split} steps after"},
        "k_prefix+boundaries": {"ms": k_prefix, "source": f"{n_split} steps after"},
        "k_readout": {"ms": k_read, "alg_bytes": bytes_read, "gbs": bytes_read / (k_read * 1e6),
                      "source": "timed steps"},
        "k_block_state+k_prefix+boundaries": {"ms": float(t_rest.mean()) if K > 1 else None,
                                              "source": "timed steps"},
    }
    dom = "k_block_state" if k_state >= k_read_split else "k_readout"
    ach = kernels[dom]["gbs"]

    result = {
        "metric": METRIC,
        "value": th / (ms_step / 1e3),
        "unit": "tokens·heads/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if dt == torch.bfloat16 else "f32",
        "data": "synthetic",
        "config": {"workload": cfg["name"], "B": B, "N": N, "H": H, "head_dim": d,
                   "frames": cfg["frames"], "tokens_per_frame": tpf, "block_frames": bf,
                   "grid": list(cfg["grid"]), "rope_split": list(cfg["rope"]["split"]),
                   "rope_base": cfg["rope"]["base"], "eps": 1e-8},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": ach, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": ach / HBM_PEAK_GBS,
                     "traffic": measured_traffic(cfg["name"], dom)},
        "step_hbm_gbs": bytes_step / (ms_step * 1e6),
        "step_frac_of_peak": bytes_step / (ms_step * 1e6) / HBM_PEAK_GBS,
        # first readout's start to last readout's end, per step (K - 1 whole steps
        # plus one readout)
        "event_ms_per_step": (ev_span + float(t_rest.mean() if K > 1 else 0.0)) / K,
        "kernels": kernels,
        # per timed step, HIP-event ms of each kernel: the shader clock dips when
        # the heavy load starts and recovers over ~40 ms, and the trend shows how
        # much of the timed region falls in that ramp
        "step_trend": {"k_readout": [round(float(x), 4) for x in t_read],
                       "k_block_state+k_prefix+boundaries": [round(float(x), 4) for x in t_rest]},
        "cpu_baseline": cpu,
    }

    if args.stream_reps > 0:
        result["streaming"] = bench_streaming(lavr, torch, dev, args.stream_reps)
    if args.tconv_steps > 0:
        result["tconv"] = bench_tconv(lavr, torch, dev, cfg, args.tconv_steps)
    if args.prologue_steps > 0:
        result["prologue"] = bench_prologue(lavr, torch, dev, cfg, q, k, v, rope, args.prologue_steps)
    if args.backward_steps > 0:
        del out
        result["backward"] = bench_backward(lavr, torch, dev, cfg, q, k, v, rope, args.backward_steps)

    print(json.dumps(result), flush=True)


def bench_tconv(lavr, torch, dev, cfg, steps):
    """Time la_temporal_conv (kernel 3, bias, bf16 in and out) over the workload's
    token grid with C = H * head_dim channels, blocks of block_frames frames."""
    B, N, C = cfg["B"], W.n_tokens(cfg), cfg["H"] * cfg["head_dim"]
    tpf, bf = cfg["tokens_per_frame"], cfg["block_frames"]
    gen = torch.Generator(device=dev)
    gen.manual_seed(11)
    x = torch.randn((B, N, C), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
    w = torch.randn((3, C), generator=gen, device=dev, dtype=torch.float32) / 3 ** 0.5
    bias = 0.1 * torch.randn((C,), generator=gen, device=dev, dtype=torch.float32)
    y = torch.empty_like(x)
    for _ in range(3):
        lavr.temporal_conv(x, w, tpf, bf, bias=bias, out=y)
    torch.cuda.synchronize(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        lavr.temporal_conv(x, w, tpf, bf, bias=bias, out=y)
    e1.record()
    torch.cuda.synchronize(dev)
    ms = e0.elapsed_time(e1) / steps
    alg = 2 * B * N * C * 2                               # x read once, y written once
    del x, y
    torch.cuda.empty_cache()
    return {"ms": ms, "channels": C, "kt": 3, "alg_bytes": alg, "gbs": alg / (ms * 1e6),
            "frac_of_peak": alg / (ms * 1e6) / HBM_PEAK_GBS, "steps": steps}


def bench_prologue(lavr, torch, dev, cfg, q, k, v, rope, steps):
    """Time la_block_causal_forward_qkv with both norms on the fused (B, N, 3, C)
    form of the workload, and the unfused sequence it replaces (torch RMSNorm of
    q and k, a copy of v, then la_block_causal_forward) for comparison."""
    B, H, N, d = cfg["B"], cfg["H"], W.n_tokens(cfg), cfg["head_dim"]
    C = H * d
    tpf, bf = cfg["tokens_per_frame"], cfg["block_frames"]
    norm_eps = 1e-6
    qkv = torch.stack([t.reshape(B, N, C) for t in (q, k, v)], dim=2).contiguous()
    gq, gk = (torch.from_numpy(W.draw_norm_weight(cfg, w)).to(dev) for w in W.NORM_WEIGHTS)
    out = torch.empty((B, N, H, d), dtype=q.dtype, device=dev)
    ws = torch.zeros(lavr.qkv_workspace_bytes(B, H, cfg["frames"], tpf, bf, d, rope=rope), dtype=torch.uint8, device=dev)

    def fused():
        lavr.block_causal_forward_qkv(qkv, H, bf, tpf, rope, q_gamma=gq, k_gamma=gk, norm_eps=norm_eps,
                                      out=out, workspace=ws)

    def unfused():
        qn = torch.nn.functional.rms_norm(qkv[:, :, 0], (C,), gq.to(q.dtype), norm_eps)
        kn = torch.nn.functional.rms_norm(qkv[:, :, 1], (C,), gk.to(q.dtype), norm_eps)
        vc = qkv[:, :, 2].contiguous()
        lavr.block_causal_forward(qn.view(B, N, H, d), kn.view(B, N, H, d), vc.view(B, N, H, d), bf, tpf,
                                  rope, out=out)

    def timed(fn, n):
        for _ in range(3):
            fn()
        torch.cuda.synchronize(dev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize(dev)
        return e0.elapsed_time(e1) / n

    ms = timed(fused, steps)
    ms_unfused = timed(unfused, max(2, steps // 2))
    th = B * N * H
    esz = q.element_size()
    nb = -(-cfg["frames"] // bf)
    # each input element read once and out written once, plus the block records;
    # the build reads q and k a second time for the token scales (moved bytes)
    alg = 4 * th * d * esz + 2 * B * H * nb * rec_bytes(d)
    moved = alg + 2 * th * d * esz + 2 * 2 * B * N * 4
    del qkv, out, ws
    torch.cuda.empty_cache()
    return {"ms": ms, "tokens_heads_per_s": th / (ms / 1e3), "alg_bytes": alg, "moved_bytes": moved,
            "gbs_alg": alg / (ms * 1e6), "gbs_moved": moved / (ms * 1e6),
            "unfused_ms": ms_unfused, "norm_eps": norm_eps, "steps": steps}


def bench_backward(lavr, torch, dev, cfg, q, k, v, rope, steps):
    """Time la_block_causal_backward (dq, dk, dv in the input dtype) on the forward's inputs."""
    B, H, N, d = cfg["B"], cfg["H"], W.n_tokens(cfg), cfg["head_dim"]
    tpf, bf = cfg["tokens_per_frame"], cfg["block_frames"]
    gen = torch.Generator(device=dev)
    gen.manual_seed(7)
    g = torch.randn(q.shape, generator=gen, device=dev, dtype=torch.float32).to(q.dtype)
    grads = [torch.empty_like(q) for _ in range(3)]
    need = lavr.backward_workspace_bytes(B, H, cfg["frames"], tpf, bf, head_dim=d, rope=rope)
    ws = torch.zeros(need, dtype=torch.uint8, device=dev)
    code = lavr._dtype_code(q.dtype)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    ptrs = [ctypes.c_void_p(x.data_ptr()) for x in (q, k, v, g, *grads)]

    def call():
        rc = lavr.lib.la_block_causal_backward(*ptrs, code, code, B, H, d, cfg["frames"], tpf, bf, 0,
                                               ctypes.byref(rope.desc), 1e-8,
                                               ctypes.c_void_p(ws.data_ptr()), need, stream)
        if rc:
            raise RuntimeError(lavr.status_string(rc))

    for _ in range(3):
        call()
    torch.cuda.synchronize(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        call()
    e1.record()
    torch.cuda.synchronize(dev)
    ms = e0.elapsed_time(e1) / steps

    # training path: the forward's block prefixes reused (la_block_causal_backward_from_forward)
    lavr.lib.la_block_causal_forward(ptrs[0], ptrs[1], ptrs[2], ptrs[4], code, code, B, H, d, cfg["frames"],
                                     tpf, bf, 0, ctypes.byref(rope.desc), 1e-8,
                                     ctypes.c_void_p(ws.data_ptr()), need, stream)

    def call_ff():
        rc = lavr.lib.la_block_causal_backward_from_forward(*ptrs, code, code, B, H, d, cfg["frames"], tpf, bf,
                                                            0, ctypes.byref(rope.desc), 1e-8,
                                                            ctypes.c_void_p(ws.data_ptr()), need, stream)
        if rc:
            raise RuntimeError(lavr.status_string(rc))

    for _ in range(3):
        call_ff()
    torch.cuda.synchronize(dev)
    e0.record()
    for _ in range(steps):
        call_ff()
    e1.record()
    torch.cuda.synchronize(dev)
    ms_ff = e0.elapsed_time(e1) / steps
    th = B * N * H
    esz = q.element_size()
    nb = -(-cfg["frames"] // bf)
    # q, k, v, dout read; k, v read again for the block states; dq, dk, dv written;
    # (S, z) records: prefixes and suffixes written and read once each
    alg = 9 * th * d * esz + 4 * B * H * nb * rec_bytes(d)
    # from the forward: the block-state pass over k and v and its records drop out
    alg_ff = 7 * th * d * esz + 2 * B * H * nb * rec_bytes(d)
    return {"ms": ms, "tokens_heads_per_s": th / (ms / 1e3), "alg_bytes": alg,
            "gbs": alg / (ms * 1e6), "frac_of_peak": alg / (ms * 1e6) / HBM_PEAK_GBS, "steps": steps,
            "from_forward": {"ms": ms_ff, "tokens_heads_per_s": th / (ms_ff / 1e3), "alg_bytes": alg_ff,
                             "gbs": alg_ff / (ms_ff * 1e6), "frac_of_peak": alg_ff / (ms_ff * 1e6) / HBM_PEAK_GBS}}


def bench_streaming(lavr, torch, dev, reps):
    """Per-block latency of 40 la_stream_block calls (B=2, 70 heads, 3 frames of 30x52)."""
    cfg = W.workload("stream_bf16")
    tpf, bf = cfg["tokens_per_frame"], cfg["block_frames"]
    L = bf * tpf
    arrs = {x: W.draw(cfg, x) for x in W.TENSORS}
    q, k, v = (W.to_torch(cfg, arrs[x], dev) for x in W.TENSORS)
    del arrs
    nblk = cfg["frames"] // bf
    # one contiguous buffer per block, as a streaming caller would hold them
    blocks = [tuple(x[:, j * L:(j + 1) * L].contiguous() for x in (q, k, v)) for j in range(nblk)]
    del q, k, v
    outs = [torch.empty_like(blocks[0][0]) for _ in range(nblk)]
    rope = lavr.RopeTable(cfg["rope"]["split"], cfg["grid"], cfg["frames"], cfg["rope"]["base"], dev)
    need = lavr.workspace_bytes(cfg["B"], cfg["H"], bf, tpf, bf, rope=rope)
    ws = torch.zeros(need, dtype=torch.uint8, device=dev)
    times = []
    for rep in range(reps + 1):
        st = lavr.StreamState(cfg["B"], cfg["H"], device=dev)
        torch.cuda.synchronize(dev)
        t0 = time.perf_counter()
        for j in range(nblk):
            st.step(*blocks[j], tpf, rope, out=outs[j], workspace=ws)
        torch.cuda.synchronize(dev)
        if rep > 0:
            times.append((time.perf_counter() - t0) / nblk)
    per_call = float(np.median(times))
    th = cfg["B"] * L * cfg["H"]
    d = cfg["head_dim"]
    call_bytes = 4 * th * d * 2 + 2 * cfg["B"] * cfg["H"] * rec_bytes(d)
    return {"workload": cfg["name"], "calls": nblk, "ms_per_block": per_call * 1e3,
            "tokens_heads_per_s": th / per_call, "hbm_gbs": call_bytes / (per_call * 1e9),
            "reps": reps}


if __name__ == "__main__":
    main()
