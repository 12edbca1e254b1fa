"""Benchmark of the fused QK-norm + RoPE pass on one MI355X.

One step = one call of the pass over the whole workload (every Q and K head
of every token), in place on a device-resident fused QKV buffer.  Default
workload: Wan-A14B-shaped 32760 tokens x 3*40*128 bf16, interleaved RoPE,
one shared fp32 cos/sin row per token.

Prints ONE JSON line.  ``dtype`` is the arithmetic type of the kernels (fp32:
16-bit data are widened exactly, computed in fp32 and rounded once);
``config.data_dtype`` is the storage type.  ``value`` is achieved algorithmic
HBM throughput over the K timed steps, launched back to back (GB/s, bytes the
pass must move / time); ``roofline.achieved`` uses the mean kernel duration
from HIP events recorded around each launch on the launch stream, in a second
pass of K launches; ``cpu_baseline`` times the fp64 CPU oracle on a bounded
sample of the same workload.

  python bench.py --op fuse_scale_shift [--workload adaln_wan|adaln_flux|adaln_wan_cfg2]
                  [--dtype bf16|fp16] [--mod-dtype fp32|bf16|fp16] [--inplace] [--flush]
  python bench.py --op group_norm_silu [--workload gn_vae_out|gn_vae_up|gn_vae_mid]
                  [--dtype bf16|fp16] [--mod-dtype fp32|bf16|fp16] [--inplace] [--flush]
  python bench.py --op eager_chain [--workload flux|headline|mid] [--dtype bf16|fp16]
  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload headline]
                  [--layout shared|per_head] [--style interleaved|rotate_half]
                  [--dtype bf16|fp16] [--flush [--flush-mode clean|dirty]] [--graph]
                  [--no-cpu-baseline] [--calib-copy]

  python bench.py --op floor [--workload headline]

Other workloads (tiny, mid, flux, large) are reported the same way; with
--flush the caches are evicted before every timed call (outside that call's
event bracket; by default by reading a 1 GiB buffer, which leaves clean
lines, or with --flush-mode dirty by writing one) so that inputs smaller than
the 256 MB Infinity Cache come from HBM, and ``value`` then uses the per-call
event times.  ``pct_of_peak`` uses the mean call time, ``pct_of_peak_median``
the median.  --op floor times the pass beside no-arithmetic probes of its
access pattern (bench_floor.hip).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "QK-norm+RoPE µs/call and achieved HBM GB/s (% of peak), Wan 40×128 shape"
PEAK_GBS = 8000.0            # MI355X HBM3E peak, GB/s
CSRC = os.path.join(ROOT, "diffusion_transformer_qk_amd", "csrc")
# per step: the sources its kernels are built from (hashed, in order) and the
# committed record of HBM bytes per launch measured with rocprofv3 counters
KERNEL_SRCS = {
    "qknorm_rope": [os.path.join(CSRC, n) for n in ("qknorm_rope.hip", "device_common.h")],
    "fuse_scale_shift": [os.path.join(CSRC, n) for n in ("fuse_scale_shift.hip",
                                                         "device_common.h")],
    "group_norm_silu": [os.path.join(CSRC, n) for n in ("group_norm_silu.hip",
                                                        "device_common.h")],
}
TRAFFIC_FILES = {
    "qknorm_rope": os.path.join(ROOT, "profiles", "traffic_headline.json"),
    "fuse_scale_shift": os.path.join(ROOT, "profiles", "traffic_adaln_wan.json"),
    "group_norm_silu": os.path.join(ROOT, "profiles", "traffic_gn_vae_out.json"),
}
TRAFFIC_FILE = TRAFFIC_FILES["qknorm_rope"]


def kernel_source_hash(op: str = "qknorm_rope") -> str:
    """SHA-256 (16 hex) over the sources of one step's kernels, in order."""
    h = hashlib.sha256()
    for path in KERNEL_SRCS[op]:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def recorded_traffic(path: str, op: str, key: str):
    """HBM bytes per launch for run `key` from a counter record, if the record
    was taken on the current kernel sources; else None."""
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256_16") != kernel_source_hash(op):
        return None
    entry = rec.get("runs", {}).get(key)
    return None if entry is None else entry.get("bytes_per_launch")


def measured_traffic(workload: str, layout: str, style: str, dtype: str):
    """HBM bytes per launch of the QK-norm + RoPE kernel, if still current."""
    return recorded_traffic(TRAFFIC_FILE, "qknorm_rope",
                            "%s/%s/%s/%s" % (workload, layout, style, dtype))


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--op", default="qknorm_rope",
                    choices=["qknorm_rope", "fuse_scale_shift", "group_norm_silu",
                             "eager_chain", "floor"])
    ap.add_argument("--workload", default=None)
    ap.add_argument("--mod-dtype", default="fp32", choices=["fp32", "bf16", "fp16"])
    ap.add_argument("--inplace", action="store_true", help="AdaLN, group norm: write y over x")
    ap.add_argument("--layout", default="shared", choices=["shared", "per_head"])
    ap.add_argument("--style", default=None, choices=[None, "interleaved", "rotate_half"])
    ap.add_argument("--dtype", default=None, choices=[None, "bf16", "fp16"])
    ap.add_argument("--cos-dtype", default="fp32", choices=["fp32", "bf16"])
    ap.add_argument("--flush", action="store_true",
                    help="evict the caches before each timed call (cache-cold inputs)")
    ap.add_argument("--flush-mode", default="clean", choices=["clean", "dirty"],
                    help="clean: read a 1 GiB buffer (leaves clean lines); dirty: write 1 GiB "
                         "(leaves dirty lines whose write-back may land in the timed call)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="budget for the CPU-oracle sample")
    ap.add_argument("--calib-copy", action="store_true",
                    help="run only a plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--graph", action="store_true",
                    help="QK pass: also time calls replayed from a HIP graph of 20 "
                         "back-to-back launches (no per-launch host cost)")
    return ap.parse_args()


def calib_copy(steps: int):
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    print(json.dumps({"calib_copy_bytes_read": n, "calib_copy_bytes_written": n,
                      "copy_GBps": round(2 * n / dt / 1e9, 1), "steps": steps}))


def graph_call_us(launch, stream, steps: int, per_graph: int = 20) -> float:
    """Mean µs per call when `per_graph` back-to-back calls are replayed from
    one captured HIP graph (at least `steps` calls in all)."""
    import torch
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=stream):
        for _ in range(per_graph):
            launch()
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        graph.replay()                      # warm
    reps = max(1, -(-steps // per_graph))
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    with torch.cuda.stream(stream):
        for _ in range(reps):
            graph.replay()
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) * 1e3 / (reps * per_graph)


def cpu_baseline(qkv_cpu, w, qg, kg, cos, sin, style, budget_s, dtype="bf16"):
    """Time the fp64 oracle on the same workload: whole passes over every
    token (Q and K), repeated until ``budget_s`` is spent; median pass time."""
    import numpy as np

    import oracle
    import workloads as wl
    bits = wl.u16(qkv_cpu)
    H, D, T = w.heads, w.head_dim, w.tokens
    chunk = 2048
    out = np.empty((chunk, H, D), dtype=np.float64)
    c_np, s_np = cos.numpy(), sin.numpy()
    def tokens(a0, a1):
        for a in range(a0, a1, chunk):
            b = min(a1, a + chunk)
            for col0, g in ((0, qg), (H * D, kg)):
                oracle.qknorm_rope(bits, dtype, row_stride=3 * H * D, col0=col0, heads=H,
                                   head_dim=D, gamma=g.numpy(), eps=wl.EPS, cos=c_np, sin=s_np,
                                   style=style, t_begin=a, t_end=b, out=out[:b - a])

    per_pass, n = _cpu_passes(lambda: tokens(0, T), budget_s)
    nbytes = wl.algorithmic_bytes(T, H, D)
    sub = min(T, chunk)
    one = _single_core(lambda: tokens(0, sub))
    return {"value": round(nbytes / per_pass / 1e9, 3), "unit": "GB/s",
            "cores": oracle.max_threads(), "kind": "oracle",
            "ms_per_pass": round(per_pass * 1e3, 1),
            "sample": "whole passes over all %d tokens x %d Q+K heads: %d (median pass), fp64 "
                      "C oracle with OpenMP, fp64 output in %d-token chunks"
                      % (T, 2 * H, n, chunk),
            "single_core": {"value": round(wl.algorithmic_bytes(sub, H, D) / one / 1e9, 3),
                            "unit": "GB/s", "sample": "first %d tokens, median of 3" % sub},
            **_host()}


def _host():
    """The host CPU as lscpu names it (model name, and vendor / family /
    model / stepping, which identify the part when the name is generic),
    and the cores this process may use."""
    import subprocess
    fields = {}
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=20).stdout
        for line in out.splitlines():
            key, _, val = line.partition(":")
            fields[key.strip()] = val.strip()
    except (OSError, subprocess.SubprocessError):
        pass
    model = fields.get("Model name")
    if not model:
        try:
            with open("/proc/cpuinfo") as f:
                for line in f:
                    if line.startswith("model name"):
                        model = line.split(":", 1)[1].strip()
                        break
        except OSError:
            pass
    ident = "/".join(fields.get(k, "?") for k in ("Vendor ID", "CPU family", "Model", "Stepping"))
    return {"cpu_model": model or "unknown", "cpu_id": ident,
            "nproc": len(os.sched_getaffinity(0))}


def _single_core(sample_pass, reps=3):
    """Median seconds of `sample_pass` with the oracle on one thread."""
    import numpy as np

    import oracle
    threads = oracle.max_threads()
    oracle.set_threads(1)
    try:
        times = []
        for _ in range(reps):
            t0 = time.perf_counter()
            sample_pass()
            times.append(time.perf_counter() - t0)
    finally:
        oracle.set_threads(threads)
    return float(np.median(times))


def _cpu_passes(one_pass, budget_s):
    """Run whole oracle passes until `budget_s` is spent (at least one, at
    most 100); return (median seconds per pass, passes run)."""
    import numpy as np
    passes, spent = [], 0.0
    while not passes or (spent < budget_s and len(passes) < 100):
        t0 = time.perf_counter()
        one_pass()
        dt = time.perf_counter() - t0
        passes.append(dt)
        spent += dt
    return float(np.median(passes)), len(passes)


def cpu_baseline_adaln(x_cpu, w, sc, sh, mod_dtype, dtype, nbytes, budget_s):
    """The fp64 oracle over every row of the AdaLN workload, in 2048-row chunks."""
    import numpy as np

    import oracle
    import workloads as wl
    bits = wl.u16(x_cpu)
    scn = sc.numpy() if mod_dtype == "fp32" else wl.u16(sc)
    shn = sh.numpy() if mod_dtype == "fp32" else wl.u16(sh)
    chunk = 2048
    out = np.empty((chunk, w.hidden), dtype=np.float64)

    def rows(a0, a1):
        for a in range(a0, a1, chunk):
            b = min(a1, a + chunk)
            oracle.adaln(bits, dtype, hidden=w.hidden, rows_per_batch=w.rows_per_batch,
                         scale=scn, shift=shn, mod_dtype=mod_dtype, eps=wl.EPS, row_begin=a,
                         row_end=b, out=out[:b - a])

    per_pass, n = _cpu_passes(lambda: rows(0, w.rows), budget_s)
    sub = min(w.rows, chunk)
    one = _single_core(lambda: rows(0, sub))
    return {"value": round(nbytes / per_pass / 1e9, 3), "unit": "GB/s",
            "cores": oracle.max_threads(), "kind": "oracle",
            "ms_per_pass": round(per_pass * 1e3, 1),
            "sample": "whole passes over all %d rows x %d: %d (median pass), fp64 C oracle "
                      "with OpenMP, fp64 output in %d-row chunks" % (w.rows, w.hidden, n, chunk),
            "single_core": {"value": round(nbytes * sub / w.rows / one / 1e9, 3), "unit": "GB/s",
                            "sample": "first %d rows, median of 3" % sub},
            **_host()}


def cpu_baseline_gn(x_cpu, w, g, b, param_dtype, dtype, nbytes, budget_s):
    """The fp64 oracle over every group of the group-norm workload, one group
    at a time."""
    import numpy as np

    import oracle
    import workloads as wl
    bits = wl.u16(x_cpu)
    gn = g.numpy() if param_dtype == "fp32" else wl.u16(g)
    bn = b.numpy() if param_dtype == "fp32" else wl.u16(b)
    gsize = w.channels // w.groups * w.spatial
    pairs = w.n * w.groups
    chunk = max(1, min(pairs, (1 << 28) // (8 * gsize)))      # <= 256 MB of fp64 output
    out = np.empty(chunk * gsize, dtype=np.float64)

    def groups(a0, a1):
        for a in range(a0, a1, chunk):
            b = min(a1, a + chunk)
            oracle.group_norm_silu(bits, dtype, channels=w.channels, spatial=w.spatial,
                                   groups=w.groups, gamma=gn, beta=bn, param_dtype=param_dtype,
                                   eps=wl.EPS, group_begin=a, group_end=b,
                                   out=out[:(b - a) * gsize])

    per_pass, n = _cpu_passes(lambda: groups(0, pairs), budget_s)
    one = _single_core(lambda: groups(0, 1))
    return {"value": round(nbytes / per_pass / 1e9, 3), "unit": "GB/s",
            "cores": oracle.max_threads(), "kind": "oracle",
            "ms_per_pass": round(per_pass * 1e3, 1),
            "sample": "whole passes over all %d groups of %d elements: %d (median pass), fp64 C "
                      "oracle with OpenMP over groups, fp64 output %d groups at a time"
                      % (pairs, gsize, n, chunk),
            "single_core": {"value": round(nbytes / pairs / one / 1e9, 3), "unit": "GB/s",
                            "sample": "first group, median of 3"},
            **_host()}


class CacheFlush:
    """Evicts the GPU caches (4 MB L2 per die, 256 MB Infinity Cache) between
    timed calls with 1 GiB of traffic on the timed stream, outside the call's
    event pair.  "clean" reads a 1 GiB buffer (a sum into one float): the
    lines it leaves are clean, and the previous call's dirty lines are written
    back while it runs.  "dirty" writes 1 GiB instead; its own dirty lines
    are then written back during the next timed call and charged to it."""

    def __init__(self, mode: str, device):
        import torch
        self.mode = mode
        self.buf = torch.empty(1 << 28, dtype=torch.float32, device=device)
        self.buf.fill_(1.0)
        self.acc = torch.empty((), dtype=torch.float32, device=device)

    def __call__(self, i: int):
        import torch
        if self.mode == "clean":
            torch.sum(self.buf, dim=0, out=self.acc)
        else:
            self.buf.fill_(float(i))


def time_launches(launch, stream, steps, warmup, flush=None):
    """Warm up, then time `steps` launches on `stream`.

    Without flushing, two passes of `steps` launches each:
    1. back to back, bracketed only by a barrier, a synchronisation and one
       HIP event pair on `stream` (whole-job time: region ms and wall s);
    2. with a HIP event pair around every launch (per-launch µs).
    The per-launch events add a little host and queue work per launch, so
    they stay out of the whole-job region.  With `flush` (a CacheFlush), one
    pass: the caches are flushed before every launch, outside its event pair.

    Returns (per-launch µs array, region ms, wall s)."""
    import numpy as np
    import torch
    torch.cuda.synchronize()
    for _ in range(warmup):
        launch()
    torch.cuda.synchronize()
    region0 = torch.cuda.Event(enable_timing=True)
    region1 = torch.cuda.Event(enable_timing=True)
    if flush is None:
        torch.cuda.synchronize()
        wall0 = time.perf_counter()
        region0.record(stream)
        for _ in range(steps):
            launch()
        region1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
        region_ms = region0.elapsed_time(region1)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    torch.cuda.synchronize()
    wall1 = time.perf_counter()
    region0.record(stream)
    for i in range(steps):
        if flush is not None:
            with torch.cuda.stream(stream):
                flush(i)
        starts[i].record(stream)
        launch()
        ends[i].record(stream)
    region1.record(stream)
    torch.cuda.synchronize()
    if flush is not None:
        wall = time.perf_counter() - wall1
        region_ms = region0.elapsed_time(region1)
    per = np.array([a.elapsed_time(b) for a, b in zip(starts, ends)]) * 1e3
    return per, region_ms, wall


def bench_fuse_scale_shift(args):
    """AdaLN modulation on one of the ADALN_WORKLOADS; prints one JSON line."""
    import numpy as np
    import torch

    import diffusion_transformer_qk_amd as qkr
    import workloads as wl
    w = wl.ADALN_WORKLOADS[args.workload or "adaln_wan"]
    dtype = args.dtype or w.dtypes[0]
    dev = torch.device("cuda:0")
    x_cpu, sc, sh = wl.adaln_inputs(w.seed, w.rows, w.hidden, w.batches, dtype, args.mod_dtype)
    x = x_cpu.to(dev)
    scd, shd = sc.to(dev), sh.to(dev)
    y = x if args.inplace else torch.empty_like(x)
    mod_bytes = 4 if args.mod_dtype == "fp32" else 2
    nbytes = wl.adaln_bytes(w.rows, w.hidden, w.batches, mod_bytes=mod_bytes)
    stream = torch.cuda.Stream(device=dev)
    handle = stream.cuda_stream
    flush_buf = CacheFlush(args.flush_mode, dev) if args.flush else None

    def launch():
        qkr.fuse_scale_shift(x, scd, shd, out=y, eps=wl.EPS, rows_per_batch=w.rows_per_batch,
                             stream=handle)

    per, region_ms, wall = time_launches(launch, stream, args.steps, args.warmup, flush_buf)
    K = args.steps
    mean_us = float(per.mean())
    achieved = nbytes / (mean_us * 1e-6) / 1e9
    value = achieved if args.flush else nbytes * K / (region_ms * 1e-3) / 1e9
    result = {
        "metric": "AdaLN fuse_scale_shift µs/call and achieved HBM GB/s (% of peak)",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(region_ms / K, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "%s: x %s [%d, %d], %d modulation row(s) %s%s%s"
                               % (w.key, dtype, w.rows, w.hidden, w.batches, args.mod_dtype,
                                  ", in place" if args.inplace else "",
                                  (", cache flushed (%s)" % args.flush_mode) if args.flush
                                  else ""),
                   "rows": w.rows, "hidden": w.hidden, "batches": w.batches, "data_dtype": dtype,
                   "parallelism": "single GPU"},
        "us_per_call": {"mean": round(mean_us, 2), "median": round(float(np.median(per)), 2),
                        "p10": round(float(np.percentile(per, 10)), 2),
                        "p90": round(float(np.percentile(per, 90)), 2)},
        "pct_of_peak": round(100 * achieved / PEAK_GBS, 2),
        "pct_of_peak_median": round(100 * nbytes / (float(np.median(per)) * 1e-6) / 1e9
                                    / PEAK_GBS, 2),
        "bytes_per_call": nbytes, "wall_s_timed": round(wall, 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_GBS, 4),
                     "traffic": recorded_traffic(
                         TRAFFIC_FILES["fuse_scale_shift"], "fuse_scale_shift",
                         "%s/%s/%s/%s" % (w.key, dtype, args.mod_dtype,
                                          "inplace" if args.inplace else "out"))},
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_adaln(x_cpu, w, sc, sh, args.mod_dtype, dtype,
                                                    nbytes, args.cpu_seconds)
    print(json.dumps(result))
    return 0


def bench_group_norm_silu(args):
    """Group norm + SiLU on one of the GN_WORKLOADS; prints one JSON line."""
    import numpy as np
    import torch

    import diffusion_transformer_qk_amd as qkr
    import workloads as wl
    w = wl.GN_WORKLOADS[args.workload or "gn_vae_out"]
    dtype = args.dtype or w.dtypes[0]
    dev = torch.device("cuda:0")
    x_cpu, g, b = wl.gn_inputs(w.seed, w.n, w.channels, w.spatial, dtype, args.mod_dtype)
    x = x_cpu.to(dev).view(w.n, w.channels, w.height, w.width)
    gd, bd = g.to(dev), b.to(dev)
    y = x if args.inplace else torch.empty_like(x)
    need = qkr.group_norm_silu_workspace_size(w.n, w.channels, w.spatial, w.groups)
    sched, chunk = qkr.group_norm_silu_schedule(w.n, w.channels, w.spatial, w.groups)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    pbytes = 4 if args.mod_dtype == "fp32" else 2
    nbytes = wl.gn_bytes(w.n, w.channels, w.spatial, param_bytes=pbytes)
    stream = torch.cuda.Stream(device=dev)
    handle = stream.cuda_stream
    flush_buf = CacheFlush(args.flush_mode, dev) if args.flush else None

    def launch():
        qkr.group_norm_silu(x, gd, bd, w.groups, out=y, eps=wl.EPS, workspace=ws, stream=handle)

    per, region_ms, wall = time_launches(launch, stream, args.steps, args.warmup, flush_buf)
    K = args.steps
    mean_us = float(per.mean())
    achieved = nbytes / (mean_us * 1e-6) / 1e9
    value = achieved if args.flush else nbytes * K / (region_ms * 1e-3) / 1e9
    result = {
        "metric": "group_norm_silu µs/call and achieved HBM GB/s (% of peak)",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(region_ms / K, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "%s: x %s [%d, %d, %d, %d], %d groups, %s affine%s%s"
                               % (w.key, dtype, w.n, w.channels, w.height, w.width, w.groups,
                                  args.mod_dtype, ", in place" if args.inplace else "",
                                  (", cache flushed (%s)" % args.flush_mode) if args.flush
                                  else ""),
                   "n": w.n, "channels": w.channels, "spatial": w.spatial, "groups": w.groups,
                   "schedule": sched, "chunk_elems": chunk, "workspace_bytes": need,
                   "data_dtype": dtype, "parallelism": "single GPU"},
        "us_per_call": {"mean": round(mean_us, 2), "median": round(float(np.median(per)), 2),
                        "p10": round(float(np.percentile(per, 10)), 2),
                        "p90": round(float(np.percentile(per, 90)), 2)},
        "pct_of_peak": round(100 * achieved / PEAK_GBS, 2),
        "pct_of_peak_median": round(100 * nbytes / (float(np.median(per)) * 1e-6) / 1e9
                                    / PEAK_GBS, 2),
        "bytes_per_call": nbytes, "wall_s_timed": round(wall, 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_GBS, 4),
                     "traffic": recorded_traffic(
                         TRAFFIC_FILES["group_norm_silu"], "group_norm_silu",
                         "%s/%s/%s/%s" % (w.key, dtype, args.mod_dtype,
                                          "inplace" if args.inplace else "out"))},
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_gn(x_cpu, w, g, b, args.mod_dtype, dtype, nbytes,
                                                 args.cpu_seconds)
    print(json.dumps(result))
    return 0


def eager_chain(x, gamma, cos, sin, eps, style):
    """The unfused form of the pass on one tensor in PyTorch eager mode, as a
    DiT block runs it without a fused kernel ([FLUX PR], intro: a chain of
    per-head RMSNorms and RoPEs; its microbench compares against PyTorch
    eager bf16).  A comparison leg for timing only, never the product path.

    x [T, H, D] (any strides) in bf16/fp16; gamma [D] in x's dtype, as a
    norm module's weight; cos, sin [T, D] fp32.  The norm's output is
    rounded to x's dtype, then RoPE runs on that rounded tensor in fp32 and
    rounds again.  Returns a new [T, H, D] tensor; x is not modified."""
    import torch
    import torch.nn.functional as F
    D = x.shape[-1]
    n = F.rms_norm(x, (D,), weight=gamma, eps=eps)
    if style == "interleaved":              # partner of 2i is 2i+1, with the sign of the sine
        pairs = n.unflatten(-1, (D // 2, 2))
        rot = torch.stack((-pairs[..., 1], pairs[..., 0]), dim=-1).flatten(-2)
    else:                                   # partner of i is i + D/2
        rot = torch.cat((-n[..., D // 2:], n[..., :D // 2]), dim=-1)
    c, s = cos.unsqueeze(1), sin.unsqueeze(1)
    return (n.float() * c + rot.float() * s).to(x.dtype)


def bench_eager_chain(args):
    """Fused pass vs the eager unfused chain on the same tensors and stream,
    the form of the [FLUX PR] kernel microbench.  On the FLUX workload the
    shapes are its text stream (512 tokens), image stream (4096) and the
    joint sequence (4608), 48 heads of 128; other workloads run whole.
    Prints one JSON line; `value` is the speedup on the last (largest) shape."""
    import numpy as np
    import torch

    import diffusion_transformer_qk_amd as qkr
    import workloads as wl
    w = wl.WORKLOADS[args.workload or "flux"]
    style = args.style or w.styles[0]
    dtype = args.dtype or "bf16"
    H, D, T = w.heads, w.head_dim, w.tokens
    dev = torch.device("cuda:0")
    qg, kg = wl.norm_weights(w.seed, D)
    cos, sin = wl.workload_tables(w, style)
    c, s = cos.to(dev), sin.to(dev)
    g1, g2 = qg.to(dev), kg.to(dev)
    # the norm module's weight lives in the data dtype; the fused call gets
    # the same values widened to fp32, so both compute the same function
    tdt = wl.DTYPES[dtype]
    g1e, g2e = g1.to(tdt), g2.to(tdt)
    g1f, g2f = g1e.float(), g2e.float()
    if w.layout == "fused":
        qkv = wl.fused_qkv(w.seed, T, H, D, dtype).to(dev)
        q_all = qkv[:, :H * D].view(T, H, D)
        k_all = qkv[:, H * D:2 * H * D].view(T, H, D)
    else:
        q_cpu, k_cpu = wl.separate_qk(w.seed, T, H, D, (dtype,))[dtype]
        q_all, k_all = q_cpu.to(dev), k_cpu.to(dev)
    if w.key == "flux":
        spans = [("text stream", 0, w.text_tokens), ("image stream", w.text_tokens, T),
                 ("joint sequence", 0, T)]
    else:
        spans = [(w.key, 0, T)]
    stream = torch.cuda.Stream(device=dev)
    handle = stream.cuda_stream
    shapes = []
    for name, a, b in spans:
        # contiguous copies of the token range, so that both sides read the
        # same dense [tokens, H, D] tensors (fused mode keeps its row stride)
        if w.layout == "fused":
            buf = qkv[a:b].clone()
            q, k = buf[:, :H * D].view(b - a, H, D), buf[:, H * D:2 * H * D].view(b - a, H, D)
            tensors = dict(qkv=buf)
        else:
            q, k = q_all[a:b].clone(), k_all[a:b].clone()
            tensors = dict(q=q, k=k)
        cs, ss = c[a:b].contiguous(), s[a:b].contiguous()
        q0, k0 = q.clone(), k.clone()

        def eager():
            with torch.cuda.stream(stream):
                eager_chain(q0, g1e, cs, ss, wl.EPS, style)
                eager_chain(k0, g2e, cs, ss, wl.EPS, style)

        def fused():
            qkr.qknorm_rope_fused(**tensors, q_gamma=g1f, k_gamma=g2f, cos=cs, sin=ss,
                                  eps=wl.EPS, style=style, stream=handle)

        per_e, _, _ = time_launches(eager, stream, args.steps, args.warmup)
        per_f, _, _ = time_launches(fused, stream, args.steps, args.warmup)
        nbytes = wl.algorithmic_bytes(b - a, H, D)
        fe, ff = float(per_e.mean()), float(per_f.mean())
        shapes.append({"shape": "%s [%d, %d, %d] x {q, k}" % (name, b - a, H, D),
                       "tokens": b - a, "eager_us": round(fe, 2), "fused_us": round(ff, 2),
                       "speedup": round(fe / ff, 2),
                       "fused_pct_of_peak": round(100 * nbytes / (ff * 1e-6) / 1e9 / PEAK_GBS, 2)})
    last = shapes[-1]
    result = {
        "metric": "fused QK-norm+RoPE speedup over the PyTorch eager unfused chain",
        "value": last["speedup"], "unit": "x", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "%s: %s %s, %d heads x %d, %s RoPE, shared fp32 cos/sin; eager: "
                               "F.rms_norm -> round -> RoPE -> round per tensor, warm caches"
                               % (w.key, "fused QKV" if w.layout == "fused" else "separate q, k",
                                  dtype, H, D, style),
                   "data_dtype": dtype, "parallelism": "single GPU"},
        "shapes": shapes,
        "context": "[FLUX PR] reports 15.8x-25.7x over PyTorch eager bf16 across FLUX.2 shapes "
                   "on another machine",
    }
    print(json.dumps(result))
    return 0


FLOOR_LIB = os.path.join(ROOT, "bench_floor.so")


def _floor_lib():
    """bench_floor.so with its one entry point typed."""
    import ctypes
    if not os.path.exists(FLOOR_LIB):
        raise RuntimeError("bench_floor.so is not built; run __graft_entry__.build()")
    lib = ctypes.CDLL(FLOOR_LIB)
    vp, i64, i32, u32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_uint32
    lib.qkr_floor.argtypes = [vp, vp, i64, i32, i64, vp, vp, vp, u32, i32, i32, vp, vp]
    lib.qkr_floor.restype = ctypes.c_int
    return lib


def _run_floor_legs(legs, stream, args, dev):
    """Two rounds of every (key, what, launch, bytes) leg, the second in
    reverse order; returns (rounds, best µs per leg)."""
    import numpy as np
    flush = CacheFlush(args.flush_mode, dev) if args.flush else None
    rounds = []
    for order in (legs, legs[::-1]):
        res = {}
        for key, _, launch, nbytes in order:
            per, region_ms, _ = time_launches(launch, stream, args.steps, args.warmup, flush)
            us = float(per.mean()) if flush else region_ms * 1e3 / args.steps
            res[key] = {"us": round(us, 2), "mean_us": round(float(per.mean()), 2),
                        "median_us": round(float(np.median(per)), 2),
                        "pct_of_peak": round(100 * nbytes / (us * 1e-6) / 1e9 / PEAK_GBS, 2)}
        rounds.append(res)
    best = {k: min(r[k]["us"] for r in rounds) for k, _, _, _ in legs}
    return rounds, best


def bench_floor_steps(args):
    """The AdaLN or group-norm step beside out-of-place probes of its bytes
    (bench_floor.so mode 6: the x bytes read and written to a second buffer
    by one wave per row of heads * 128 elements, no arithmetic), with and
    without the QK pass's residency rule, the x bytes read alone and written
    alone, and a plain device copy; two rounds, one stream.  Rows are the
    step's own rows for AdaLN (hidden = heads * 128) and 4096-element slices
    of x for group norm.  Prints one JSON line; `value` is the step's time
    over the faster out-of-place probe's."""
    import torch

    import diffusion_transformer_qk_amd as qkr
    import workloads as wl
    lib = _floor_lib()
    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream(device=dev)
    handle = stream.cuda_stream
    dtype = args.dtype
    if args.workload in wl.ADALN_WORKLOADS:
        w = wl.ADALN_WORKLOADS[args.workload]
        dtype = dtype or w.dtypes[0]
        x_cpu, sc, sh = wl.adaln_inputs(w.seed, w.rows, w.hidden, w.batches, dtype, args.mod_dtype)
        x = x_cpu.to(dev)
        scd, shd = sc.to(dev), sh.to(dev)
        y = torch.empty_like(x)
        nbytes = wl.adaln_bytes(w.rows, w.hidden, w.batches,
                                mod_bytes=4 if args.mod_dtype == "fp32" else 2)
        rows, width = w.rows, w.hidden
        desc = "%s: x %s [%d, %d], %d modulation row(s) %s" % (w.key, dtype, w.rows, w.hidden,
                                                             w.batches, args.mod_dtype)

        def the_pass():
            qkr.fuse_scale_shift(x, scd, shd, out=y, eps=wl.EPS, stream=handle)
    else:
        w = wl.GN_WORKLOADS[args.workload]
        dtype = dtype or w.dtypes[0]
        x_cpu, g, b = wl.gn_inputs(w.seed, w.n, w.channels, w.spatial, dtype, args.mod_dtype)
        x = x_cpu.to(dev).view(w.n, w.channels, w.height, w.width)
        gd, bd = g.to(dev), b.to(dev)
        y = torch.empty_like(x)
        need = qkr.group_norm_silu_workspace_size(w.n, w.channels, w.spatial, w.groups)
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
        nbytes = wl.gn_bytes(w.n, w.channels, w.spatial,
                             param_bytes=4 if args.mod_dtype == "fp32" else 2)
        width = 4096
        rows = x.numel() // width
        desc = "%s: x %s [%d, %d, %d, %d], %d groups, %s affine" % (
            w.key, dtype, w.n, w.channels, w.height, w.width, w.groups, args.mod_dtype)

        def the_pass():
            qkr.group_norm_silu(x, gd, bd, w.groups, out=y, eps=wl.EPS, workspace=ws,
                                stream=handle)
    heads = width // 128
    if width % 128 or heads > 48 or x.numel() != rows * width:
        raise ValueError("the out-of-place probes take rows of at most 48 x 128 elements")
    src = x.reshape(rows, width).clone()
    dst = torch.empty_like(src)
    scratch = src.clone()
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    x_bytes = rows * width * 2
    magic = 0x9E3779B9

    def probe(mode, buf, cap=1, out=None):
        def launch():
            rc = lib.qkr_floor(buf.data_ptr(), None, rows, heads, width, None, None,
                               sink.data_ptr(), magic, mode, cap,
                               out.data_ptr() if out is not None else None, handle)
            if rc != 0:
                raise RuntimeError("qkr_floor returned %d" % rc)
        return launch

    def copy():
        with torch.cuda.stream(stream):
            dst.copy_(src)

    legs = [
        ("pass", "the step (%s)" % ("fuse_scale_shift" if args.workload in wl.ADALN_WORKLOADS
                                    else "group_norm_silu"), the_pass, nbytes),
        ("floor_oop", "no arithmetic: x read, written to a second buffer, the pass's "
                      "residency rule", probe(6, src, 1, dst), 2 * x_bytes),
        ("floor_oop_uncapped", "floor_oop without the residency cap", probe(6, src, 0, dst),
         2 * x_bytes),
        ("read_only", "the x bytes read alone", probe(3, src), x_bytes),
        ("write_only", "the x bytes written alone (zeros, into a scratch copy)",
         probe(4, scratch), x_bytes),
        ("copy", "device copy of the x bytes (torch copy_)", copy, 2 * x_bytes),
    ]
    rounds, best = _run_floor_legs(legs, stream, args, dev)
    floor = min(best["floor_oop"], best["floor_oop_uncapped"])
    result = {
        "metric": "step time over an out-of-place stream of the same bytes",
        "value": round(best["pass"] / floor, 4), "unit": "x",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "higher_is_better": False,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": desc + ((", cache flushed (%s)" % args.flush_mode)
                                       if args.flush else ""),
                   "probe_rows": rows, "probe_row_elements": width,
                   "timing": "mean per call, caches flushed before each" if args.flush
                             else "back to back", "parallelism": "single GPU"},
        "legs": {k: {"what": what, "bytes": b} for k, what, _, b in legs},
        "rounds": rounds,
        "best_us": best,
        "read_then_write_us": round(best["read_only"] + best["write_only"], 2),
    }
    print(json.dumps(result))
    return 0


def bench_floor(args):
    """The pass beside data-movement probes of its access pattern
    (bench_floor.hip, a library of its own) on one workload, in one process
    on one stream, two rounds (the second in reverse order).  Legs: the pass;
    the probe that moves the same bytes the same way with no arithmetic
    (floor_table, with the cos/sin staging); the Q/K bytes in place with the
    same phases (every wave's loads complete, then a workgroup barrier, then
    the stores: floor_phase), with the wave's wait but no barrier
    (floor_wave, and floor_wave_uncapped without the pass's residency cap),
    and with each store issued as its load arrives (floor_qk); the Q/K bytes
    read only and written only; for a fused buffer the Q/K bytes with no V
    gaps; and a plain device copy of the Q/K bytes.  Every probe but
    floor_wave_uncapped applies the pass's residency rule.  Back-to-back time per call,
    or with --flush the mean per-call time with the caches evicted before
    each call.  Prints one JSON line; `value` is the pass's time over
    floor_table's.  An AdaLN or group-norm workload runs bench_floor_steps."""
    import torch

    import diffusion_transformer_qk_amd as qkr
    import workloads as wl
    if args.workload in wl.ADALN_WORKLOADS or args.workload in wl.GN_WORKLOADS:
        return bench_floor_steps(args)
    lib = _floor_lib()
    w = wl.WORKLOADS[args.workload or "headline"]
    style = args.style or w.styles[0]
    dtype = args.dtype or w.dtypes[0]
    T, H, D = w.tokens, w.heads, w.head_dim
    if D != 128 or H > 48:
        raise ValueError("the floor probes cover head_dim 128 with at most 48 heads")
    dev = torch.device("cuda:0")
    qg, kg = wl.norm_weights(w.seed, D)
    cos, sin = wl.workload_tables(w, style)
    g1, g2, c, s = qg.to(dev), kg.to(dev), cos.to(dev), sin.to(dev)
    fused = w.layout == "fused"
    if fused:
        qkv = wl.fused_qkv(w.seed, T, H, D, dtype).to(dev)
        probe_buf = qkv.clone()
        tensors = dict(qkv=qkv)
        x0, x1, stride = probe_buf.data_ptr(), probe_buf.data_ptr() + H * D * 2, 3 * H * D
        flat = torch.empty((T, 2 * H * D), dtype=qkv.dtype, device=dev)
        flat.copy_(qkv[:, :2 * H * D])
    else:
        q_cpu, k_cpu = wl.separate_qk(w.seed, T, H, D, (dtype,))[dtype]
        tensors = dict(q=q_cpu.to(dev), k=k_cpu.to(dev))
        pq, pk = tensors["q"].clone(), tensors["k"].clone()
        x0, x1, stride = pq.data_ptr(), pk.data_ptr(), H * D
        flat = torch.cat([tensors["q"].view(T, -1), tensors["k"].view(T, -1)], dim=1)
    src = flat.clone()
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    stream = torch.cuda.Stream(device=dev)
    handle = stream.cuda_stream
    qk_bytes = T * 2 * H * D * 2 * 2
    table_bytes = T * D * 4 * 2
    magic = 0x9E3779B9

    def probe(mode, a0=None, a1=None, row=None, cap=1):
        b0, b1, st = (x0, x1, stride) if a0 is None else (a0, a1, row)

        def launch():
            rc = lib.qkr_floor(b0, b1, T, H, st, c.data_ptr(), s.data_ptr(), sink.data_ptr(),
                               magic, mode, cap, None, handle)
            if rc != 0:
                raise RuntimeError("qkr_floor returned %d" % rc)
        return launch

    def copy():
        with torch.cuda.stream(stream):
            flat.copy_(src)

    def the_pass():
        qkr.qknorm_rope_fused(**tensors, q_gamma=g1, k_gamma=g2, cos=c, sin=s, eps=wl.EPS,
                              style=style, stream=handle)

    legs = [
        ("pass", "the pass (qknorm_rope_fused), shared fp32 cos/sin", the_pass,
         qk_bytes + table_bytes),
        ("floor_table", "no arithmetic: Q/K in place, cos/sin rows staged in LDS behind a barrier",
         probe(1), qk_bytes + table_bytes),
        ("floor_phase", "no arithmetic: Q/K in place, each wave waits for all its loads, then "
                        "a workgroup barrier, then the stores", probe(2), qk_bytes),
        ("floor_wave", "no arithmetic: Q/K in place, each wave waits for all its loads before "
                       "its first store", probe(5), qk_bytes),
        ("floor_wave_uncapped", "floor_wave without the residency cap (all the waves the "
                                "registers allow)", probe(5, cap=0), qk_bytes),
        ("floor_qk", "no arithmetic: Q/K in place, each store as soon as its load arrives",
         probe(0), qk_bytes),
        ("read_only", "the Q/K loads alone", probe(3), qk_bytes // 2),
        ("write_only", "the Q/K stores alone (zeros)", probe(4), qk_bytes // 2),
    ]
    if fused:
        legs.append(("floor_flat", "no arithmetic: the Q/K bytes with no V gaps, no barrier",
                     probe(0, flat.data_ptr(), flat.data_ptr() + H * D * 2, 2 * H * D),
                     qk_bytes))
    legs.append(("copy", "device copy of the Q/K bytes (torch copy_, %d B each way)"
                 % (qk_bytes // 2), copy, qk_bytes))
    rounds, best = _run_floor_legs(legs, stream, args, dev)
    result = {
        "metric": "pass time over the data-movement floor of its access pattern",
        "value": round(best["pass"] / best["floor_table"], 4), "unit": "x",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "higher_is_better": False,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "%s: %s %s [%d, %s%dx%d], %s RoPE, shared fp32 cos/sin%s"
                               % (w.key, "fused QKV" if fused else "separate q, k", dtype, T,
                                  "3x" if fused else "", H, D, style,
                                  (", cache flushed (%s)" % args.flush_mode) if args.flush
                                  else ""),
                   "timing": "mean per call, caches flushed before each" if args.flush
                             else "back to back", "parallelism": "single GPU"},
        "legs": {k: {"what": what, "bytes": nbytes} for k, what, _, nbytes in legs},
        "rounds": rounds,
        "best_us": best,
        "read_then_write_us": round(best["read_only"] + best["write_only"], 2),
    }
    print(json.dumps(result))
    return 0


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py: measures one GPU only (the pass needs no collective; "
              "run with --gpus 1)", file=sys.stderr)
        return 2
    import numpy as np
    import torch

    import diffusion_transformer_qk_amd as qkr
    import workloads as wl

    if args.calib_copy:
        calib_copy(max(1, args.steps))
        return 0

    qkr.load_library()
    if args.op == "fuse_scale_shift":
        return bench_fuse_scale_shift(args)
    if args.op == "group_norm_silu":
        return bench_group_norm_silu(args)
    if args.op == "eager_chain":
        return bench_eager_chain(args)
    if args.op == "floor":
        return bench_floor(args)
    args.workload = args.workload or "headline"
    w = wl.WORKLOADS[args.workload]
    style = args.style or w.styles[0]
    dtype = args.dtype or w.dtypes[0]
    H, D, T = w.heads, w.head_dim, w.tokens
    dev = torch.device("cuda:0")

    qg, kg = wl.norm_weights(w.seed, D)
    cos, sin = wl.workload_tables(w, style)
    g1, g2 = qg.to(dev), kg.to(dev)
    cos_bytes = 4
    if args.cos_dtype == "bf16":
        cos_t, sin_t = wl.workload_tables(w, style, dtype="bf16")
        c, s = cos_t.to(dev), sin_t.to(dev)
        cos_bytes = 2
    else:
        c, s = cos.to(dev), sin.to(dev)
    if args.layout == "per_head":
        c, s = wl.expand_per_head(c, H), wl.expand_per_head(s, H)
    qkv_cpu = None
    if w.layout == "fused":
        qkv_cpu = wl.fused_qkv(w.seed, T, H, D, dtype)
        x = qkv_cpu.to(dev)
        tensors = dict(qkv=x)
    else:
        q_cpu, k_cpu = wl.separate_qk(w.seed, T, H, D, (dtype,))[dtype]
        tensors = dict(q=q_cpu.to(dev), k=k_cpu.to(dev))
    nbytes = wl.algorithmic_bytes(T, H, D, cos_layout=args.layout, cos_bytes=cos_bytes)

    stream = torch.cuda.Stream(device=dev)
    handle = stream.cuda_stream
    flush_buf = CacheFlush(args.flush_mode, dev) if args.flush else None

    def launch():
        qkr.qknorm_rope_fused(**tensors, q_gamma=g1, k_gamma=g2, cos=c, sin=s, eps=wl.EPS,
                              style=style, cos_layout=args.layout, stream=handle)

    K = args.steps
    per, region_ms, wall = time_launches(launch, stream, K, args.warmup, flush_buf)
    graph_us = graph_call_us(launch, stream, K) if args.graph and not args.flush else None
    mean_us = float(per.mean())
    achieved = nbytes / (mean_us * 1e-6) / 1e9
    # with flushing, the region also holds the flush writes: use the call times
    value = achieved if args.flush else nbytes * K / (region_ms * 1e-3) / 1e9
    info = qkr.kernel_info(D, args.layout,
                           qkr.binding.QKR_BF16 if cos_bytes == 2 else qkr.binding.QKR_FP32, style,
                           qkr.binding.QKR_FP16 if dtype == "fp16" else qkr.binding.QKR_BF16,
                           heads=H, tokens=T, tensors="fused" if w.layout == "fused" else "pair")

    traffic = (measured_traffic(args.workload, args.layout, style, dtype)
               if args.cos_dtype == "fp32" else None)
    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(region_ms / K, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "%s: %s %s [%d, %s%dx%d], %s RoPE, %s %s cos/sin%s"
                               % (w.key, "fused QKV" if w.layout == "fused" else "separate q, k",
                                  dtype, T, "3x" if w.layout == "fused" else "", H, D, style,
                                  args.layout, args.cos_dtype,
                                  (", cache flushed (%s)" % args.flush_mode) if args.flush
                                  else ""),
                   "tokens": T, "heads": H, "head_dim": D, "layout": args.layout,
                   "style": style, "data_dtype": dtype, "parallelism": "single GPU"},
        "us_per_call": {"mean": round(mean_us, 2), "median": round(float(np.median(per)), 2),
                        "p10": round(float(np.percentile(per, 10)), 2),
                        "p90": round(float(np.percentile(per, 90)), 2)},
        "pct_of_peak": round(100 * achieved / PEAK_GBS, 2),
        "pct_of_peak_median": round(100 * nbytes / (float(np.median(per)) * 1e-6) / 1e9
                                    / PEAK_GBS, 2),
        "bytes_per_call": nbytes,
        "wall_s_timed": round(wall, 4),
        "kernel": info,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_GBS, 4),
                     "traffic": traffic},
    }
    if graph_us is not None:
        result["graph_us_per_call"] = round(graph_us, 2)
    if (not args.no_cpu_baseline and qkv_cpu is not None and args.layout == "shared"
            and args.cos_dtype == "fp32"):
        result["cpu_baseline"] = cpu_baseline(qkv_cpu, w, qg, kg, cos, sin, style,
                                              args.cpu_seconds, dtype)
    print(json.dumps(result))
    return 0


if __name__ == "__main__":
    sys.exit(main())
