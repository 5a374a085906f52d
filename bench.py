"""Throughput of Newton-Schulz orthogonalization on one MI355X.

Default workload: one Llama-8B MLP-shaped matrix, 4096 x 14336 bf16, with
N(0,1) entries times log-uniform column scales in [1e-3, 1], orthogonalized
by the Gram form (5 tuned steps, restart before step 4).  A step is one full
ns_orthogonalize call on a matrix already resident in HBM: norm, staging,
every product, and the final cast back into the caller's buffer.  The call
works in place, so each step orthogonalizes the previous step's output; the
products are dense, so the work does not depend on the values.

Other workloads (--workload): the transposed and square Llama shapes, the
MoE expert batch (128 x 2048 x 1408 and transposed), the NanoGPT-124M
weight set (two grouped calls per step -- the square attention weights, and
the wide and tall MLP weights together -- each on a stream of its own unless
--serial; --per-shape runs three batched calls), the ROOT split of a 2048 x 8192
Student-t gradient followed by orthogonalization of its robust part, and a
256 x 1024 fp32 matrix, and a whole Muon step (momentum, orthogonalization,
weight update) with the 4096 x 14336 matrix as the gradient.  `value`
counts matrices per second.

Prints one JSON line.  Besides the driver's fields it carries:
  tflops / mfma_frac     algorithmic (symmetric-aware) TFLOP/s of the whole
                         step and its fraction of the fp16/bf16 dense peak;
  standard_form          the same measurement for the standard form;
  roofline               the dominant kernel's achieved rate (HIP events
                         bound to each launch, in an instrumented run of the
                         same number of steps right after the timed region),
                         on algorithmic FLOPs; issued_tflops / issued_frac
                         count the MFMA work the launches actually issue
                         (whole diagonal tiles, padded edges) instead;
  kernels                per-kernel-kind average launch times (the
                         instrumented run);
  ms_per_step_instrumented, ms_p10_p50_p90
                         the instrumented run's time per call and its
                         per-call spread.
  cpu_baseline           the fp64 oracle on the host cores (bounded sample),
                         with the host CPU model;
  quality                (ROOT workload) the MSE of the result against the
                         exact polar factor of the split's robust part.
"""

from __future__ import annotations

import argparse
import ctypes
import glob
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = ("NS orthogonalizations/sec + TFLOP/s (MFMA % of peak) at "
          "4096x14336 bf16")
PEAK_TFLOPS = {"f16": 2500.0, "bf16": 2500.0, "f32": 157.3}
PEAK_HBM_GBS = 8000.0
# Sources whose change invalidates a committed HBM-traffic measurement.
KERNEL_SOURCES = ["newton_schulz_matrix_amd/csrc/products.hpp",
                  "newton_schulz_matrix_amd/csrc/stage.hpp",
                  "newton_schulz_matrix_amd/csrc/plan.hpp",
                  "newton_schulz_matrix_amd/csrc/api.hip"]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama8b-mlp",
                    choices=["llama8b-mlp", "llama8b-down", "llama8b-square",
                             "moe-experts", "moe-experts-t", "small-fp32",
                             "nanogpt-set", "root-split", "muon-step",
                             "copy-calibration"])
    ap.add_argument("--shape", type=int, nargs=2, default=None,
                    metavar=("ROWS", "COLS"),
                    help="one ROWS x COLS column-scaled bf16 matrix instead "
                         "of --workload")
    ap.add_argument("--mode", default="gram", choices=["gram", "standard"])
    ap.add_argument("--internal", default=None, choices=[None, "fp16"])
    ap.add_argument("--restart-mask", type=int, default=1 << 4)
    ap.add_argument("--tile", type=int, default=0, choices=[0, 128, 192, 256],
                    help="force the products' tile edge (0: automatic)")
    ap.add_argument("--serial", action="store_true",
                    help="run a multi-call step's calls one after another on "
                         "one stream (default: one stream per call)")
    ap.add_argument("--per-shape", action="store_true",
                    help="NanoGPT set: one batched call per stored shape "
                         "(three calls) instead of two grouped calls")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-standard", action="store_true",
                    help="skip the standard-form companion measurement")
    return ap.parse_args()


def workload_input(name, shape=None, grouped=True):
    """(list of host input tensors, I/O dtype name, step kind).

    The kind is "ns" (orthogonalize each input), "root" (ROOT split, then
    orthogonalize the robust part) or "muon" (a whole Muon step with the
    input as the gradient).  A 3-D tensor is one batched call, a list of 2-D
    tensors one grouped call; several inputs run as one call each per step.
    """
    import workloads
    if shape is not None:
        return [workloads.column_scaled(shape[0], shape[1], seed=3)], "bf16", "ns"
    if name == "llama8b-mlp":
        return [workloads.llama8b((4096, 14336))], "bf16", "ns"
    if name == "llama8b-down":
        return [workloads.llama8b((14336, 4096))], "bf16", "ns"
    if name == "llama8b-square":
        return [workloads.llama8b((4096, 4096))], "bf16", "ns"
    if name == "moe-experts":
        return [workloads.moe_experts(128, 2048, 1408)], "bf16", "ns"
    if name == "moe-experts-t":
        return [workloads.moe_experts(128, 1408, 2048)], "bf16", "ns"
    if name == "small-fp32":
        return [workloads.small_fp32()], "fp32", "ns"
    if name == "nanogpt-set":
        import torch
        groups = workloads.nanogpt_set()
        if grouped:
            # Two groups: the square attention weights and the MLP weights,
            # wide and tall together (one shape up to orientation).
            return ([torch.stack(groups["768x768"]),
                     list(groups["768x3072"]) + list(groups["3072x768"])],
                    "bf16", "ns")
        return [torch.stack(g) for g in groups.values()], "bf16", "ns"
    if name == "root-split":
        return [workloads.heavy_tailed()], "bf16", "root"
    if name == "muon-step":
        return [workloads.llama8b((4096, 14336))], "bf16", "muon"
    raise ValueError(name)


class Events:
    """Raw hipEvent_t handles from the HIP runtime torch loaded."""

    def __init__(self, count):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [
            ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.arr = (ctypes.c_void_p * count)()
        for i in range(count):
            h = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(h)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.arr[i] = h
        self.count = count

    def elapsed_ms(self, i, j):
        ms = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), self.arr[i],
                                        self.arr[j]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)

    def close(self):
        for i in range(self.count):
            self.hip.hipEventDestroy(self.arr[i])


def make_trace(events, capacity, kind_mask):
    from newton_schulz_matrix_amd._binding import Trace
    t = Trace()
    t.events = ctypes.cast(events.arr, ctypes.POINTER(ctypes.c_void_p))
    kinds = (ctypes.c_int32 * capacity)()
    flops = (ctypes.c_double * capacity)()
    nbytes = (ctypes.c_double * capacity)()
    t.kinds = kinds
    t.flops = flops
    t.bytes = nbytes
    t.capacity = capacity
    t.count = 0
    t.kind_mask = kind_mask
    t._keep = (kinds, flops, nbytes)
    return t


def trace_stats(events, t):
    from newton_schulz_matrix_amd._binding import KERNEL_KINDS
    stats = {}
    for i in range(t.count):
        kind = KERNEL_KINDS[t.kinds[i]]
        ms = events.elapsed_ms(2 * i, 2 * i + 1)
        s = stats.setdefault(kind, {"launches": 0, "ms": 0.0, "flops": 0.0,
                                    "bytes": 0.0})
        s["launches"] += 1
        s["ms"] += ms
        s["flops"] += t.flops[i]
        s["bytes"] += t.bytes[i]
    return stats


def make_step(inputs, mode, args, kind):
    """A closure running one step: every input once (after the split)."""
    import torch
    import newton_schulz_matrix_amd as nsa
    calls = []
    for x in inputs:
        if isinstance(x, list):
            n, m = min(x[0].shape), max(x[0].shape)
            ws = torch.empty(nsa.grouped_workspace_size(
                n, m, len(x), x[0].dtype, mode, args.restart_mask,
                args.internal, args.tile) + 256, dtype=torch.uint8,
                device=x[0].device)
            calls.append((nsa.orthogonalize_grouped, x,
                          dict(mode=mode, restart_mask=args.restart_mask,
                               internal=args.internal, workspace=ws,
                               tile=args.tile), None))
            continue
        batched = x.dim() == 3
        fn = nsa.orthogonalize_batched if batched else nsa.orthogonalize
        rows, cols = x.shape[-2], x.shape[-1]
        nb = x.shape[0] if batched else 1
        size = (nsa.muon_workspace_size if kind == "muon" else
                nsa.workspace_size)
        ws = torch.empty(size(rows, cols, nb, x.dtype, mode,
                              args.restart_mask, args.internal, args.tile)
                         + 256, dtype=torch.uint8, device=x.device)
        kw = dict(mode=mode, restart_mask=args.restart_mask,
                  internal=args.internal, workspace=ws, tile=args.tile)
        extra = None
        if kind == "root":
            # The ROOT split reads the original gradient and writes B into
            # the buffer the orthogonalization then works on in place.
            extra = x.clone()
        elif kind == "muon":
            # x is the gradient; a zero weight and momentum to update.
            extra = (torch.zeros_like(x),
                     torch.zeros(x.shape, dtype=torch.float32, device=x.device))
        calls.append((fn, x, kw, extra))

    # Calls on different inputs are independent: with several, each gets a
    # stream of its own (default priority), forked from and joined back into
    # the caller's stream, so one call's short launches overlap another's.
    dev0 = torch.device("cuda:0")
    streams = ([torch.cuda.Stream(device=dev0) for _ in calls]
               if len(calls) > 1 and not args.serial else None)

    def step(trace=None):
        if streams is None:
            run_calls(trace, [None] * len(calls))
            return
        main = torch.cuda.current_stream()
        for s in streams:
            s.wait_stream(main)
        run_calls(trace, streams)
        for s in streams:
            main.wait_stream(s)

    def run_calls(trace, call_streams):
        import contextlib
        for (fn, x, kw, extra), s in zip(calls, call_streams):
            ctx = torch.cuda.stream(s) if s is not None else contextlib.nullcontext()
            with ctx:
                one_call(fn, x, kw, extra, trace)

    def one_call(fn, x, kw, extra, trace):
        tkw = dict(kw) if trace is None else dict(kw, trace=trace)
        if kind == "muon":
            w, m = extra
            nsa.muon_step(w, x, m, 0.02, 0.95, True, **tkw)
            return
        if kind == "root":
            nsa.soft_threshold_split(extra, out_b=x)
        fn(x, **tkw)
    return step


def run_form(inputs, mode, steps, warmup, args, kind="ns"):
    """Warm up, time `steps` plain steps, then `steps` instrumented ones.

    The timed region (`ms_per_step`) runs the calls exactly as a user would,
    with one event at each end.  Timing single launches needs HIP events on
    the stream, which leave the GPU idle for several microseconds around
    each traced launch, so the per-launch times (the roofline and the
    per-kernel figures) and the per-call spread come from a second run of
    `steps` calls with every launch traced, right after the timed region.
    """
    import torch
    step = make_step(inputs, mode, args, kind)
    # Untraced warm-up; the first launch of each kernel also loads its code
    # object.
    for _ in range(max(warmup, 1)):
        step()
    torch.cuda.synchronize()

    # Timed region: `steps` plain calls.
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for _ in range(steps):
        step()
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = start.elapsed_time(stop)

    # Instrumented run: events bound to every launch and at every call
    # boundary.
    per_call = 64 * len(inputs)
    ev = Events(2 * per_call * steps)
    tr = make_trace(ev, per_call * steps, 0xFFFFFFFF)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    marks[0].record()
    for i in range(steps):
        step(tr)
        marks[i + 1].record()
    torch.cuda.synchronize()
    inst_ms = marks[0].elapsed_time(marks[-1])
    per_call = sorted(marks[i].elapsed_time(marks[i + 1]) for i in range(steps))

    def pct(q):
        return per_call[min(len(per_call) - 1, int(q * (len(per_call) - 1) + 0.5))]

    timed = trace_stats(ev, tr)
    ev.close()
    dominant = max(timed, key=lambda k: timed[k]["ms"])
    return {"ms_per_step": total_ms / steps, "wall_s": wall,
            "ms_per_step_instrumented": inst_ms / steps,
            "ms_p10": pct(0.1), "ms_p50": pct(0.5), "ms_p90": pct(0.9),
            "dominant": dominant, "timed_kernels": timed}


def _code_only(text):
    """C++ source without comments and whitespace (string literals kept)."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if text.startswith("//", i):
            i = text.find("\n", i)
            i = n if i < 0 else i
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
        elif c == '"' or c == "'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        else:
            if not c.isspace():
                out.append(c)
            i += 1
    return "".join(out)


def sources_digest():
    """Digest of the kernel sources' code: comments and layout do not count."""
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def committed_traffic(kind, workload, mode, tile):
    """HBM bytes per launch of `kind` from the rocprofv3 counter summaries.

    A summary in profiles/ carries lines
      traffic: kind=K workload=W mode=M tile=T fetch_bytes=F write_bytes=B sources=H
    (FETCH_SIZE and WRITE_SIZE per dispatch, scaled by a plain copy's
    readings).  They count only while H matches the current kernel sources.
    """
    digest = sources_digest()
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        with open(path) as f:
            for line in f:
                if not line.startswith("traffic:"):
                    continue
                kv = dict(re.findall(r"(\w+)=(\S+)", line))
                if (kv.get("kind") == kind and kv.get("workload") == workload
                        and kv.get("mode") == mode
                        and kv.get("tile") == str(tile)
                        and kv.get("sources") == digest):
                    return (float(kv["fetch_bytes"]) + float(kv["write_bytes"]),
                            os.path.relpath(path, ROOT))
    return None, None


def issued_flops(kind, batch, rows, cols, tile, internal):
    """MFMA work one launch of a symmetric product actually issues: whole
    upper-triangle tiles of `tile` (diagonal tiles in full, ragged edges
    padded) over the contraction rounded up to the k-tile.  kind "sym" is an
    n x n product (contraction n), "gram" X X^T (contraction m); None for
    other kinds."""
    if kind not in ("sym", "gram"):
        return None
    n, m = min(rows, cols), max(rows, cols)
    kt = 32 if internal == "fp32" else 64          # elements per 128-byte k-tile row
    k = n if kind == "sym" else m
    k_pad = -(-k // kt) * kt
    t = -(-n // tile)
    return batch * (t * (t + 1) // 2) * tile * tile * k_pad * 2.0


def cpu_baseline(m_cpu, mode, restart_mask):
    import numpy as np
    import oracle
    from threadpoolctl import threadpool_info
    m64 = m_cpu.double().numpy()
    restarts = tuple(k for k in range(1, 33) if (restart_mask >> k) & 1)

    def once():
        t0 = time.perf_counter()
        if mode == "gram":
            oracle.ns_gram(m64, 5, oracle.TUNED_ABC, restarts)
        else:
            oracle.ns_standard(m64, 5, oracle.TUNED_ABC)
        return time.perf_counter() - t0

    once()                                    # warm-up (BLAS threads, caches)
    times = sorted(once() for _ in range(3))
    dt = times[1]
    threads = [d.get("num_threads") for d in threadpool_info()
               if d.get("user_api") == "blas"]
    cores = int(max(threads)) if threads else len(os.sched_getaffinity(0))
    return {"value": 1.0 / dt, "unit": "orth/s", "cores": cores,
            "kind": "oracle", "cpu_model": cpu_model(),
            "host_cpus": os.cpu_count(),
            "cpus_allowed": len(os.sched_getaffinity(0)),
            "sample": f"full {m64.shape[0]}x{m64.shape[1]} {mode}-form "
                      f"orthogonalizations in fp64 (numpy/OpenBLAS): median "
                      f"of 3 after 1 warm-up, {dt:.1f} s each"}


def cpu_model():
    """The host CPU's model name from /proc/cpuinfo, with its family, model
    and stepping numbers (a virtualized host may report a generic name)."""
    fields = {}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if not line.strip():
                    break                      # the first processor only
                key, _, val = line.partition(":")
                fields[key.strip()] = val.strip()
    except OSError:
        pass
    name = fields.get("model name", "unknown")
    ids = [f"{k} {fields[k]}" for k in ("cpu family", "model", "stepping") if k in fields]
    return f"{name} ({', '.join(ids)})" if ids else name


def root_quality(host_input, mode, args):
    """The ROOT workload's reported quantity: the orthogonalization MSE of
    NS(B) against B's exact polar factor, ||NS(B) - polar(B)||_F^2 / n
    (B the robust part of the split, n its smaller side), with the polar
    factor from LAPACK's symmetric eigensolver on the host."""
    import numpy as np
    import torch
    import newton_schulz_matrix_amd as nsa
    m = host_input.to("cuda:0")
    b, _ = nsa.soft_threshold_split(m)
    x = b.clone()
    nsa.orthogonalize(x, mode=mode, restart_mask=args.restart_mask)
    # The same B with ROOT's per-shape coefficients (not the timed step).
    x_root = b.clone()
    nsa.orthogonalize(x_root, mode=mode, restart_mask=args.restart_mask,
                      abc=nsa.root_coefficients(*b.shape))
    torch.cuda.synchronize()
    b64 = b.double().cpu().numpy()
    wide = b64.shape[0] <= b64.shape[1]
    bw = b64 if wide else b64.T
    w, v = np.linalg.eigh(bw @ bw.T)
    polar = (v / np.sqrt(w)) @ v.T @ bw
    if not wide:
        polar = polar.T

    def mse(y):
        return float(np.sum((y.double().cpu().numpy() - polar) ** 2) / min(b64.shape))
    return {"mse_vs_polar": mse(x), "form": mode,
            "mse_vs_polar_root_coefficients": mse(x_root),
            "definition": "||NS(B) - polar(B)||_F^2 / min(rows, cols); "
                          "polar from numpy.linalg.eigh of B B^T; the timed "
                          "step uses the tuned triple"}


def copy_calibration(args):
    """A plain 1 GiB device-to-device copy, for scaling HBM byte counters.

    rocprofv3's FETCH_SIZE and WRITE_SIZE counters of this copy read against
    its known 1 GiB read and 1 GiB write give the factor by which the
    counters of the product kernels are scaled.
    """
    import torch
    n = 1 << 29                                   # bf16 elements = 1 GiB
    src = torch.ones(n, dtype=torch.bfloat16, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(args.warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(args.steps):
        dst.copy_(src)
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / args.steps
    print(json.dumps({"workload": "copy-calibration", "bytes_read": 2 * n,
                      "bytes_written": 2 * n, "ms_per_copy": ms,
                      "gbs": 4 * n / (ms * 1e-3) / 1e9}), flush=True)


def main():
    args = parse()
    if args.workload == "copy-calibration":
        copy_calibration(args)
        return
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only; --gpus {args.gpus} "
              "is not supported (multi-GPU sharding is described in the design "
              "notes, not built)", file=sys.stderr)
        sys.exit(2)
    import torch
    import newton_schulz_matrix_amd as nsa
    from newton_schulz_matrix_amd.flops import ns_flops

    dev = torch.device("cuda:0")
    if args.shape is not None:
        args.workload = f"column-scaled-{args.shape[0]}x{args.shape[1]}"
    host_inputs, io, kind = workload_input(args.workload, args.shape,
                                           grouped=not args.per_shape)
    inputs = [[x.to(dev) for x in m] if isinstance(m, list) else m.to(dev)
              for m in host_inputs]
    shapes = []
    for m in host_inputs:
        if isinstance(m, list):
            shapes += [(1, x.shape[0], x.shape[1]) for x in m]
        else:
            shapes.append((m.shape[0] if m.dim() == 3 else 1, m.shape[-2],
                           m.shape[-1]))
    matrices = sum(b for b, _, _ in shapes)
    internal = args.internal or ("fp16" if io != "fp32" else "fp32")
    dtype = {"fp16": "f16", "bf16": "bf16", "fp32": "f32"}[internal]

    def total_flops(mode):
        return sum(b * ns_flops(r, c, 5, mode, args.restart_mask)
                   for b, r, c in shapes)

    res = run_form(inputs, args.mode, args.steps, args.warmup, args, kind)
    ms = res["ms_per_step"]
    flops = total_flops(args.mode)
    value = matrices * 1000.0 / ms
    tflops = flops / (ms * 1e-3) / 1e12

    dom = res["dominant"]
    ks = res["timed_kernels"][dom]
    avg_ms = ks["ms"] / ks["launches"]
    if dom in ("norm", "stage", "threshold"):
        achieved = ks["bytes"] / ks["launches"] / (avg_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS,
                "unit": "GB/s"}
    else:
        achieved = ks["flops"] / ks["launches"] / (avg_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved,
                "peak": PEAK_TFLOPS[dtype], "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    traffic, traffic_src = committed_traffic(dom, args.workload, args.mode,
                                             args.tile or "auto")
    roof["traffic"] = traffic
    if traffic_src:
        roof["traffic_source"] = traffic_src
    roof["kernel"] = dom
    roof["avg_launch_ms"] = avg_ms
    roof["launches_timed"] = ks["launches"]
    # Supplementary: the same launches counted by the MFMA work they issue
    # (whole diagonal tiles, padded edges), which separates the kernel's own
    # rate from the tile geometry's overhead.  Single-call steps only.
    if len(shapes) == 1 and not any(isinstance(m, list) for m in host_inputs):
        b, r, c = shapes[0]
        plan = nsa.plan_kernels(r, c, b, {"bf16": torch.bfloat16, "fp16": torch.float16,
                                          "fp32": torch.float32}[io], args.mode,
                                5, args.restart_mask, args.internal, args.tile)
        edge = [int(k.split(",")[1]) for k in plan if k.startswith("nn<")]
        issued = issued_flops(dom, b, r, c, edge[0], internal) if edge else None
        if issued:
            roof["issued_tflops"] = issued / (avg_ms * 1e-3) / 1e12
            roof["issued_frac"] = roof["issued_tflops"] / roof["peak"]

    kernels = {}
    for k, s in res["timed_kernels"].items():
        avg = s["ms"] / s["launches"]
        entry = {"launches_per_step": s["launches"] / args.steps,
                 "avg_ms": avg}
        if s["flops"] > 0:
            entry["tflops"] = s["flops"] / s["launches"] / (avg * 1e-3) / 1e12
        else:
            entry["gbs"] = s["bytes"] / s["launches"] / (avg * 1e-3) / 1e9
        kernels[k] = entry

    out = {
        "metric": METRIC,
        "value": value,
        "unit": "orth/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "ms_per_step_instrumented": res["ms_per_step_instrumented"],
        "ms_p10_p50_p90": [res["ms_p10"], res["ms_p50"], res["ms_p90"]],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": args.workload,
                   "shapes": [f"{b}x{r}x{c}" for b, r, c in shapes],
                   "rows": shapes[0][1], "cols": shapes[0][2],
                   "batch": matrices, "io_dtype": io, "mode": args.mode,
                   "step": kind,
                   "ns_steps": 5, "abc": list(nsa.TUNED_ABC),
                   "restart_mask": args.restart_mask,
                   "tile": args.tile or "auto",
                   "streams": len(inputs) if len(inputs) > 1 and not args.serial else 1,
                   "calls": len(inputs),
                   "grouped": any(isinstance(m, list) for m in host_inputs),
                   "parallelism": "single-gpu"},
        "tflops": tflops,
        "mfma_frac": tflops / PEAK_TFLOPS[dtype],
        "roofline": roof,
        "kernels": kernels,
    }
    if not args.no_standard and args.mode == "gram":
        std = run_form(inputs, "standard", max(args.steps // 2, 3), 2, args,
                       kind)
        out["standard_form"] = {
            "ms_per_step": std["ms_per_step"],
            "orth_per_s": matrices * 1000.0 / std["ms_per_step"],
            "tflops": total_flops("standard") / (std["ms_per_step"] * 1e-3)
            / 1e12,
            "gram_speedup": std["ms_per_step"] / ms}
    if kind == "root":
        out["quality"] = root_quality(host_inputs[0], args.mode, args)
    if not args.no_cpu_baseline:
        first = host_inputs[0]
        first = first[0] if isinstance(first, list) else first
        sample = first if first.dim() == 2 else first[0]
        cb = cpu_baseline(sample, args.mode, args.restart_mask)
        if first.dim() == 3 or len(host_inputs) > 1:
            cb["sample"] += " (one matrix of the set; orth/s per matrix)"
        out["cpu_baseline"] = cb
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
