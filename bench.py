"""Benchmark: fused lm_head projection + cross-entropy, forward + backward, on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload llama3] [--cpu-rows R | --no-cpu-baseline]
    python bench.py --path ce [--workload ce_llama3] ...

One step = flce_forward + flce_backward over one batch of synthetic input already
resident in HBM (loss, lse, dH, dW all produced).  Prints one JSON line.

--path single measures flce_forward_backward with the single-pass workspace (the logits
computed once, 6·N·V·D flops; scratch about 25% of the 16-bit N x V logit bytes, above
the 5% the default path keeps): same workload and credit (8·N·V·D) as the default line.

--path norm measures the RMSNorm that produces H (include/flce_norm.h): one step =
flce_rmsnorm_forward + flce_rmsnorm_backward at 16384 x 4096 bf16; its roofline is the
backward call (rms_bwd and its two small dgamma passes) against the HBM peak.

--path ce measures the cross-entropy over materialised logits instead (include/flce_ce.h):
one step = flce_ce_forward + flce_ce_backward over bf16 logits [16384, 128256] in HBM
(loss, lse, dZ into a separate buffer); its roofline is the backward kernel (ce_rows_bwd)
against the HBM peak (8 TB/s), 2 V es + 12 bytes per row (ce_row_bytes).

value        tokens per second (N / mean step time over the timed steps), the whole job
             on one GPU; per-step median/min/max from events around each step
kernels      per GEMM kernel kind (forward tiles, dz recompute, dH, dW): launches per step, mean
             launch duration and achieved TFLOP/s, from a second timed region of the same K
             steps in which every launch carries its own start/stop events
             (flce_timing_begin: hipExtLaunchKernel stamps them from the dispatch itself, on
             the launch stream); the region's own step time is reported beside it
roofline     the kernel kind with the largest share of the step: its algorithmic flops per
             launch (2 x rows x vocabulary rows x D of the launch's chunk) over its mean launch
             duration, against the bf16 dense MFMA peak (2.5 PFLOP/s); traffic from the
             committed rocprofv3 counter record of that kernel when it matches the current
             kernel source, else null
cpu_baseline the fp64 oracle timed on this host's cores on the first R rows of the same
             workload (full vocabulary and hidden size), scaled to tokens/s

Modes that only read rocprofv3 output and need no GPU: --summarize-trace (per-kernel
durations), --summarize-counters (HBM traffic records), --summarize-occupancy (clock,
MFMA busy, LDS), --summarize-memstall (L2 hits, L1-to-L2 read latency, L1 pending stalls),
--summarize-mops (executed MFMA flops against the credited ones).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused linear-CE fwd+bwd tokens/s at N=16384,D=4096,V=128256; % bf16 MFMA peak"
METRIC_CE = "cross-entropy over materialised logits fwd+bwd tokens/s at N=16384,V=128256; % HBM peak"
METRIC_NORM = "RMSNorm fwd+fused bwd tokens/s at N=16384,D=4096; % HBM peak"
METRIC_SINGLE = "fused linear-CE fwd+bwd in one call, single pass, tokens/s at N=16384,D=4096,V=128256; % bf16 MFMA peak"


def workload_metric(metric: str, cfg) -> str:
    """The metric's text with the sizes of the workload actually run (the headline string
    for the Llama-3-shaped bf16 head it is quoted on; fp16 runs say so)."""
    import re
    sizes = ",".join(f"{k}={getattr(cfg, k)}" for k in ("N", "D", "V") if f"{k}=" in metric and hasattr(cfg, k))
    out = re.sub(r"at [NDV]=\d+(,[NDV]=\d+)*", f"at {sizes}", metric) if sizes else metric
    if getattr(cfg, "dtype", "bf16") == "f16":
        out = out.replace("% bf16 MFMA peak", "% fp16 MFMA peak")
    return out
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0
CSRC = os.path.join(ROOT, "linear_cross_entropy_lm_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")
# path -> (default workload, kernel source)
PATHS = {
    "fused": ("llama3", os.path.join(CSRC, "flce.hip")),
    "single": ("llama3", os.path.join(CSRC, "flce.hip")),
    "ce": ("ce_llama3", os.path.join(CSRC, "ce_logits.hip")),
    "norm": ("norm_llama3", os.path.join(CSRC, "rmsnorm.hip")),
}
# kernel kind -> (substring of its rocprofv3 kernel names, flce_kernel_id values of its launches)
KINDS = {
    "fwd_tiles16": (r"fwd_tiles16<[^<>]*, false>", (0,)),
    "fwd_tiles": (r"fwd_tiles<[^<>]*, false>", (0,)),
    "fwd_tiles16_keep": (r"fwd_tiles16<[^<>]*, true>", (1,)),
    "fwd_tiles_keep": (r"fwd_tiles<[^<>]*, true>", (1,)),
    "bwd_dz16": ("bwd_dz16<", (5,)),
    "bwd_dz": ("bwd_dz<", (5,)),
    "bwd_dhdw": ("bwd_dhdw<", (6,)),
    "keep_to_dz": ("keep_to_dz<", (8,)),
    "ce_rows_bwd": ("ce_rows_bwd", ()),
    "rms_bwd": ("rms_bwd", ()),
}
# kernel kind -> its committed HBM traffic record (profiles/<record>_<workload>_traffic.json)
TRAFFIC_RECORD = {"fwd_tiles16": "fwd_tiles", "fwd_tiles16_keep": "fwd_tiles_keep"}


def traffic_path(kind: str, workload: str, path: str = "fused") -> str:
    """The counter record of kernel `kind` on `workload` under schedule `path`.  A kind that
    both schedules launch (the dH + dW launch) runs other chunk shapes in the single pass,
    so that path's record carries its own name."""
    base = TRAFFIC_RECORD.get(kind, kind)
    if path == "single" and kind in GEMM_KINDS["fused"]["f16"]:
        base += "_single"
    return os.path.join(PROFILES, f"{base}_{workload}_traffic.json")


def code_digest(text: str) -> str:
    """Digest of a C++/HIP source's code: comments removed and whitespace collapsed, so an
    edit to comments alone does not make a counter record stale."""
    import re
    code = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    code = re.sub(r"//[^\n]*", " ", code)
    code = " ".join(code.split())
    return hashlib.sha256(code.encode()).hexdigest()[:16]


def source_digest(path: str = "fused") -> str:
    with open(PATHS[path][1], encoding="utf-8") as f:
        return code_digest(f.read())


def load_traffic(kind: str, workload: str, path: str = "fused"):
    """HBM bytes per launch of kernel `kind` on `workload` from its committed counter record,
    or None when absent, taken on a different kernel source, on another workload or under
    another schedule."""
    try:
        with open(traffic_path(kind, workload, path)) as f:
            t = json.load(f)
    except OSError:
        return None
    if (t.get("source_digest") != source_digest(path) or t.get("workload") != workload
            or t.get("path", path) != path):
        return None
    return t.get("hbm_bytes_per_launch")


def ce_row_bytes(V: int, es: int) -> tuple[int, int]:
    """Algorithmic HBM bytes per row of the cross-entropy over logits: forward reads the
    row (V es) and its label (8) and writes lse (4), the row's loss term (8) and flag (4);
    backward reads the row, label and lse and writes the row of dZ (V es)."""
    return V * es + 24, 2 * V * es + 12


def norm_bytes(N: int, D: int, es: int, grid: int) -> tuple[int, int]:
    """Algorithmic HBM bytes of the RMSNorm calls: forward reads X and gamma and writes H and
    rstd; the backward call reads X, dH, rstd and gamma, writes dX, and writes then reads
    the fp32 dgamma partials (one row of D per backward workgroup, then one per 32 of those)
    and writes dgamma."""
    groups = -(-grid // 32)
    fwd = 2 * N * D * es + 4 * N + D * es
    bwd = 3 * N * D * es + 4 * N + D * es + 2 * grid * D * 4 + 2 * groups * D * 4 + D * 4
    return fwd, bwd


def _counter_per_dispatch(csv_dir: str, counter: str, kernel_pattern: str):
    """Mean value of `counter` over the dispatches of kernels whose name matches the regular
    expression kernel_pattern, from a rocprofv3 --pmc --output-format csv directory."""
    import csv
    import glob
    import re
    vals = {}
    for path in glob.glob(os.path.join(csv_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] == counter and re.search(kernel_pattern, r["Kernel_Name"]):
                    vals[r["Dispatch_Id"]] = vals.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    if not vals:
        raise SystemExit(f"no {counter} samples for {kernel_pattern!r} under {csv_dir}")
    return sum(vals.values()) / len(vals), len(vals)


def summarize_counters(root: str, copy_bytes: int, path: str, kinds: list[str], workload: str) -> list[dict]:
    """Write each kernel kind's HBM traffic record from four rocprofv3 --pmc runs under
    root: F (FETCH_SIZE) and W (WRITE_SIZE) of `bench.py [--path ...] --steps 1 --warmup 0
    --no-cpu-baseline`, FC and WC of `bench.py --calibrate-copy copy_bytes`.  Each counter
    is scaled by what it reads for the copy (copy_bytes read and copy_bytes written); a
    kind's figure is the mean over its dispatches."""
    cf, _ = _counter_per_dispatch(os.path.join(root, "FC"), "FETCH_SIZE", "copyBuffer")
    cw, _ = _counter_per_dispatch(os.path.join(root, "WC"), "WRITE_SIZE", "copyBuffer")
    f_factor = copy_bytes / (cf * 1024.0)
    w_factor = copy_bytes / (cw * 1024.0)
    out = []
    for kind in kinds:
        pattern = KINDS[kind][0]
        fetch, n_f = _counter_per_dispatch(os.path.join(root, "F"), "FETCH_SIZE", pattern)
        write, n_w = _counter_per_dispatch(os.path.join(root, "W"), "WRITE_SIZE", pattern)
        rec = {"kernel": kind, "kernel_name_pattern": pattern, "workload": workload, "path": path,
               "source_digest": source_digest(path),
               "fetch_kib_per_launch": fetch, "write_kib_per_launch": write, "launches": [n_f, n_w],
               "copy_bytes": copy_bytes, "copy_fetch_kib": cf, "copy_write_kib": cw,
               "fetch_factor": f_factor, "write_factor": w_factor,
               "hbm_bytes_per_launch": fetch * 1024.0 * f_factor + write * 1024.0 * w_factor}
        with open(traffic_path(kind, workload, path), "w") as f:
            json.dump(rec, f, indent=1)
            f.write("\n")
        out.append(rec)
    return out


def host_cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def device_info() -> dict:
    import torch
    p = torch.cuda.get_device_properties(0)
    return {"name": p.name, "arch": getattr(p, "gcnArchName", ""), "compute_units": p.multi_processor_count,
            "memory_gb": round(p.total_memory / 1e9, 1)}


def cpu_baseline(inp, rows: int) -> dict:
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    H = inp.h64()[:rows]
    y = inp.y64()[:rows]
    W = inp.w64()
    t0 = time.perf_counter()
    oracle.forward_backward(H, W, y)
    dt = time.perf_counter() - t0
    del W
    return {"value": rows / dt, "unit": "tokens/s", "cores": int(cores), "cpu_model": host_cpu_model(), "kind": "oracle",
            "sample": f"first {rows} of {inp.cfg.N} token rows, full V={inp.cfg.V}, D={inp.cfg.D}: "
                      f"fp64 loss, lse, dH and dW in {dt:.1f} s",
            "seconds": dt, "fp64_gflops": 6.0 * rows * inp.cfg.V * inp.cfg.D / dt / 1e9}


def cpu_baseline_ce(inp, rows: int) -> dict:
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    Z = inp.z64(np.arange(rows))
    y = inp.y64()[:rows]
    t0 = time.perf_counter()
    oracle.ce_from_logits(Z, y)
    dt = time.perf_counter() - t0
    return {"value": rows / dt, "unit": "tokens/s", "cores": int(cores), "cpu_model": host_cpu_model(), "kind": "oracle",
            "sample": f"first {rows} of {inp.cfg.N} logit rows, full V={inp.cfg.V}: fp64 loss, lse and dZ "
                      f"in {dt:.1f} s", "seconds": dt}


def _common(args, metric, value, ms, dtype, data, config):
    return {"metric": metric, "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": dtype, "data": data, "config": config, "device": device_info()}


class HipEvents:
    """n raw hipEvent_t handles, timing enabled, from the HIP runtime torch and the library
    share (libamdhip64.so.7 is already loaded by torch: dlopen returns that copy)."""

    def __init__(self, n: int):
        import ctypes
        self.ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.arr = (ctypes.c_void_p * n)()
        for i in range(n):
            e = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.arr[i] = e.value

    def elapsed_ms(self, i: int, j: int) -> float:
        ms = self.ct.c_float()
        if self.hip.hipEventElapsedTime(self.ct.byref(ms), self.arr[i], self.arr[j]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def close(self):
        for e in self.arr:
            self.hip.hipEventDestroy(e)


def chunk_spans(total: int, chunk: int) -> list[tuple[int, int]]:
    """(first row, rows) of each chunk: chunk i of n covers 256-row tiles [i T / n, (i + 1) T / n)
    (the library's chunking, include/flce.h)."""
    n, tiles = -(-total // chunk), -(-total // 256)
    out = []
    for i in range(n):
        a, b = i * tiles // n * 256, (i + 1) * tiles // n * 256
        out.append((a, min(b, total) - a))
    return out


def gemm_launch_flops(path: str, N: int, D: int, V: int, tc: int, vc: int) -> list[tuple[int, float]]:
    """(flce_kernel_id, algorithmic flops) of each GEMM launch of one step, in launch order:
    2 x tokens x vocabulary rows x D of each contraction the launch runs.  The recomputing
    path: the forward over all of N x V, then per chunk (token chunk, vocabulary chunk) a dz
    launch and one launch with both dH and dW.  The single pass: per token chunk of tc rows,
    the keep forward and one launch with dH (K = V) and dW."""
    out = []
    if path == "fused":
        out.append((0, 2.0 * N * V * D))
        for _, tr in chunk_spans(N, tc):
            for _, vr in chunk_spans(V, vc):
                f = 2.0 * tr * vr * D
                out += [(5, f), (6, 2.0 * f)]
    else:  # single pass, token chunks of tc over the whole vocabulary
        for ci in range(-(-N // tc)):
            f = 2.0 * min(tc, N - ci * tc) * V * D
            out += [(1, f), (6, 2.0 * f)]
    return out


GEMM_KINDS = {"fused": {"f16": ["fwd_tiles16", "bwd_dz16", "bwd_dhdw"], "f32": ["fwd_tiles", "bwd_dz", "bwd_dhdw"]},
              "single": {"f16": ["fwd_tiles16_keep", "bwd_dhdw"], "f32": ["fwd_tiles_keep", "bwd_dhdw"]}}


def time_launches(args, B, step, stream, path: str, cfg, tc: int, vc: int) -> dict:
    """A second timed region of args.steps steps in which every launch carries its own
    start/stop events (flce_timing_begin).  Returns per GEMM kernel kind: launches per step,
    mean launch duration, algorithmic flops per launch and achieved TFLOP/s, plus the
    region's step time; checks that the launches ran in the order the chunking implies."""
    import ctypes
    import torch
    expect = gemm_launch_flops(path, cfg.N, cfg.D, cfg.V, tc, vc)
    cap = args.steps * (3 * len(expect) + 64)  # every launch takes a pair, the small kernels too
    ev = HipEvents(2 * cap)
    ids = (ctypes.c_int32 * cap)()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    if B.lib.flce_timing_begin(ev.arr, ids, cap) != 0:
        raise RuntimeError("flce_timing_begin failed")
    try:
        start.record(stream)
        for _ in range(args.steps):
            step()
        end.record(stream)
    finally:
        n = B.lib.flce_timing_end()
    torch.cuda.synchronize()
    gemm = {k for k, _ in expect}
    got = [(ids[i], ev.elapsed_ms(2 * i, 2 * i + 1)) for i in range(n) if ids[i] in gemm]
    ev.close()
    if [k for k, _ in got] != [k for k, _ in expect] * args.steps:
        raise RuntimeError("GEMM launches did not follow the expected chunk order")
    family = "f32" if cfg.dtype == "f32" else "f16"
    kinds = {}
    for kind in GEMM_KINDS[path][family]:
        kid = set(KINDS[kind][1])
        durs = [d for (k, d) in got if k in kid]
        if not durs:
            continue
        flops = [f for (k, f) in expect if k in kid] * args.steps
        mean_ms = sum(durs) / len(durs)
        mean_flop = sum(flops) / len(flops)
        kinds[kind] = {"launches_per_step": len(durs) // args.steps, "mean_us": mean_ms * 1e3,
                       "ms_per_step": sum(durs) / args.steps, "flop_per_launch": mean_flop,
                       "tflops": mean_flop / (mean_ms * 1e-3) / 1e12,
                       "frac": mean_flop / (mean_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}
        for k in sorted(kid):
            dk = [d for (kk, d) in got if kk == k]
            if dk:
                kinds[kind].setdefault("variants", {})[B.KERNEL_NAMES[k]] = {
                    "launches_per_step": len(dk) // args.steps, "mean_us": sum(dk) / len(dk) * 1e3}
    return {"kernels": kinds, "step_ms": start.elapsed_time(end) / args.steps}


def gemm_roofline(timing: dict, workload: str, path: str) -> dict:
    """The roofline object of the GEMM kind with the largest time per step."""
    kind, k = max(timing["kernels"].items(), key=lambda kv: kv[1]["ms_per_step"])
    return {"kernel": kind, "bound": "mfma", "achieved": k["tflops"], "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": k["frac"], "traffic": load_traffic(kind, workload, path),
            "flop_per_launch": k["flop_per_launch"], "mean_us": k["mean_us"],
            "launches_per_step": k["launches_per_step"],
            "share_of_step": k["ms_per_step"] / timing["step_ms"]}


def run_fused(args) -> dict:
    import torch
    from linear_cross_entropy_lm_amd import binding as B
    from linear_cross_entropy_lm_amd import inputs as I
    from linear_cross_entropy_lm_amd.scratch import scratch_fraction

    cfg = I.CONFIGS[args.workload or "llama3"]
    inp = I.generate(cfg)
    dev = "cuda:0"
    H, W, y = inp.device_tensors(dev)
    N, D, V = cfg.N, cfg.D, cfg.V
    ws_bytes = B.flce_workspace_bytes(N, D, V, H.dtype)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    loss = torch.empty(1, dtype=torch.float32, device=dev)
    lse = torch.empty(N, dtype=torch.float32, device=dev)
    nv = torch.empty(1, dtype=torch.int32, device=dev)
    st = torch.empty(1, dtype=torch.int32, device=dev)
    dH = torch.empty_like(H)
    dW = torch.empty(V, D, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        B.flce_forward(H, W, y, loss, lse, nv, st, ws, stream=stream)
        if ev is not None:
            ev[1].record(stream)
        B.flce_backward(H, W, y, lse, nv, None, dH, dW, ws, stream=stream)
        if ev is not None:
            ev[2].record(stream)

    ms, fwd_ms, step_ms, peak_delta, sclk = _time_steps(args, step, stream)
    if int(st.item()) != 0:
        raise RuntimeError("dev_status reports invalid labels")
    tc, vc = B.flce_backward_chunks(N, D, V, H.dtype, ws_bytes)
    timing = None if args.no_kernel_timing else time_launches(args, B, step, stream, "fused", cfg, tc, vc)

    flop_step = 8.0 * N * V * D
    out = _common(args, workload_metric(METRIC, cfg), N / (ms * 1e-3), ms, cfg.dtype,
                  "synthetic: seeded Gaussian H with unit-RMS rows, W ~ N(0, 0.02^2), uniform labels, "
                  f"{cfg.n_ignored} ignore_index rows",
                  {"workload": f"{cfg.name}-shaped lm_head + cross-entropy, fwd+bwd", "N": N, "D": D,
                   "V": V, "batch": cfg.batch, "seq_len": cfg.seq, "parallelism": "single GPU"})
    out.update({
        "mfma_peak_frac": flop_step / (ms * 1e-3) / (PEAK_BF16_TFLOPS * 1e12),
        "useful_flop_frac": 0.75 * flop_step / (ms * 1e-3) / (PEAK_BF16_TFLOPS * 1e12),
        "fwd_ms": fwd_ms,
        "bwd_ms": ms - fwd_ms,
        "step_ms_median": step_ms[len(step_ms) // 2],
        "step_ms_min": step_ms[0],
        "step_ms_max": step_ms[-1],
        "sclk_mhz": sclk,
        "scratch_bytes": ws_bytes,
        "torch_peak_alloc_delta_bytes": int(peak_delta),
        "scratch_frac_of_unfused_logits": scratch_fraction(ws_bytes, N, V),
        "loss": float(loss.item()),
        "chunks": {"token": tc, "vocab": vc},
        "kernels": timing and timing["kernels"],
        "kernel_timing_step_ms": timing and timing["step_ms"],
        "roofline": timing and gemm_roofline(timing, cfg.name, "fused"),
        "cpu_baseline": None,
    })
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inp, args.cpu_rows or 1024)
    return out


def run_single(args) -> dict:
    import torch
    from linear_cross_entropy_lm_amd import binding as B
    from linear_cross_entropy_lm_amd import inputs as I
    from linear_cross_entropy_lm_amd.scratch import scratch_fraction

    cfg = I.CONFIGS[args.workload or "llama3"]
    inp = I.generate(cfg)
    dev = "cuda:0"
    H, W, y = inp.device_tensors(dev)
    N, D, V = cfg.N, cfg.D, cfg.V
    ws_bytes = int(B.flce_forward_backward_workspace_bytes(N, D, V, H.dtype) * args.sp_workspace)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    loss = torch.empty(1, dtype=torch.float32, device=dev)
    lse = torch.empty(N, dtype=torch.float32, device=dev)
    nv = torch.empty(1, dtype=torch.int32, device=dev)
    st = torch.empty(1, dtype=torch.int32, device=dev)
    dH = torch.empty_like(H)
    dW = torch.empty(V, D, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
            ev[1].record(stream)
        B.flce_forward_backward(H, W, y, None, loss, lse, nv, st, dH, dW, ws, stream=stream)
        if ev is not None:
            ev[2].record(stream)

    ms, _, step_ms, peak_delta, sclk = _time_steps(args, step, stream)
    if int(st.item()) != 0:
        raise RuntimeError("dev_status reports invalid labels")
    tc = B.flce_forward_backward_chunk(N, D, V, H.dtype, ws_bytes)
    if tc == 0:
        raise RuntimeError("the workspace does not buy the single-pass schedule")
    timing = None if args.no_kernel_timing else time_launches(args, B, step, stream, "single", cfg, tc, 0)
    flop_credit = 8.0 * N * V * D
    out = _common(args, workload_metric(METRIC_SINGLE, cfg), N / (ms * 1e-3), ms, cfg.dtype,
                  "synthetic: seeded Gaussian H with unit-RMS rows, W ~ N(0, 0.02^2), uniform labels, "
                  f"{cfg.n_ignored} ignore_index rows",
                  {"workload": f"{cfg.name}-shaped lm_head + cross-entropy, fwd+bwd in one call (single pass)",
                   "N": N, "D": D, "V": V, "batch": cfg.batch, "seq_len": cfg.seq, "parallelism": "single GPU"})
    out.update({
        "mfma_peak_frac": 0.75 * flop_credit / (ms * 1e-3) / (PEAK_BF16_TFLOPS * 1e12),
        "credited_flop_frac": flop_credit / (ms * 1e-3) / (PEAK_BF16_TFLOPS * 1e12),
        "step_ms_median": step_ms[len(step_ms) // 2],
        "step_ms_min": step_ms[0],
        "step_ms_max": step_ms[-1],
        "sclk_mhz": sclk,
        "scratch_bytes": ws_bytes,
        "torch_peak_alloc_delta_bytes": int(peak_delta),
        "scratch_frac_of_unfused_logits": scratch_fraction(ws_bytes, N, V),
        "loss": float(loss.item()),
        "token_chunk": tc,
        "kernels": timing and timing["kernels"],
        "kernel_timing_step_ms": timing and timing["step_ms"],
        "roofline": timing and gemm_roofline(timing, cfg.name, "single"),
        "cpu_baseline": None,
    })
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inp, args.cpu_rows or 1024)
    return out


def run_ce(args) -> dict:
    import torch
    from linear_cross_entropy_lm_amd import binding as B
    from linear_cross_entropy_lm_amd import inputs as I

    cfg = I.LOGIT_CONFIGS[args.workload or "ce_llama3"]
    inp = I.generate_logits(cfg)
    dev = "cuda:0"
    Z, y = inp.device_tensors(dev)
    N, V = cfg.N, cfg.V
    es = Z.element_size()
    ws = torch.empty(B.flce_ce_workspace_bytes(N), dtype=torch.uint8, device=dev)
    loss = torch.empty(1, dtype=torch.float32, device=dev)
    lse = torch.empty(N, dtype=torch.float32, device=dev)
    nv = torch.empty(1, dtype=torch.int32, device=dev)
    st = torch.empty(1, dtype=torch.int32, device=dev)
    dZ = torch.empty_like(Z)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        B.flce_ce_forward(Z, y, loss, lse, nv, st, ws, stream=stream)
        if ev is not None:
            ev[1].record(stream)
        B.flce_ce_backward(Z, y, lse, nv, None, dZ, stream=stream)
        if ev is not None:
            ev[2].record(stream)

    ms, fwd_ms, step_ms, peak_delta, sclk = _time_steps(args, step, stream)
    if int(st.item()) != 0:
        raise RuntimeError("dev_status reports invalid labels")
    bwd_ms = ms - fwd_ms
    fwd_row, bwd_row = ce_row_bytes(V, es)
    achieved = bwd_row * N / (bwd_ms * 1e-3) / 1e9
    step_bytes = (fwd_row + bwd_row) * N
    out = _common(args, workload_metric(METRIC_CE, cfg), N / (ms * 1e-3), ms, cfg.dtype,
                  f"synthetic: seeded logits N(0, {cfg.z_std}^2), uniform labels, {cfg.n_ignored} ignore_index rows",
                  {"workload": f"{cfg.name}: cross-entropy over materialised logits, fwd+bwd", "N": N, "V": V,
                   "row_pitch": cfg.pitch, "parallelism": "single GPU"})
    out.update({
        "hbm_peak_frac": step_bytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "fwd_ms": fwd_ms,
        "bwd_ms": bwd_ms,
        "fwd_gbs": fwd_row * N / (fwd_ms * 1e-3) / 1e9,
        "step_ms_median": step_ms[len(step_ms) // 2],
        "step_ms_min": step_ms[0],
        "step_ms_max": step_ms[-1],
        "sclk_mhz": sclk,
        "torch_peak_alloc_delta_bytes": int(peak_delta),
        "loss": float(loss.item()),
        "roofline": {"kernel": "ce_rows_bwd", "bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS, "traffic": load_traffic("ce_rows_bwd", cfg.name, "ce")},
        "cpu_baseline": None,
    })
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_ce(inp, args.cpu_rows or 8192)
    return out


def cpu_baseline_norm(inp) -> dict:
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    X, g, dH = inp.x64(), inp.gamma64(), inp.dh64()
    t0 = time.perf_counter()
    oracle.rmsnorm_forward(X, g, inp.cfg.eps)
    oracle.rmsnorm_backward(X, g, dH, inp.cfg.eps)
    dt = time.perf_counter() - t0
    return {"value": inp.cfg.N / dt, "unit": "tokens/s", "cores": int(cores), "cpu_model": host_cpu_model(), "kind": "oracle",
            "sample": f"all {inp.cfg.N} rows, D={inp.cfg.D}: fp64 H, rstd, dX and dgamma in {dt:.1f} s",
            "seconds": dt}


def run_norm(args) -> dict:
    import torch
    from linear_cross_entropy_lm_amd import binding as B
    from linear_cross_entropy_lm_amd import inputs as I

    cfg = I.NORM_CONFIGS[args.workload or "norm_llama3"]
    inp = I.generate_norm(cfg)
    dev = "cuda:0"
    X, g, dH = inp.device_tensors(dev)
    N, D = cfg.N, cfg.D
    es = X.element_size()
    H = torch.empty_like(X)
    rstd = torch.empty(N, dtype=torch.float32, device=dev)
    dX = torch.empty_like(X)
    dg = torch.empty(D, dtype=torch.float32, device=dev)
    ws = torch.empty(B.flce_rmsnorm_workspace_bytes(N, D), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        B.flce_rmsnorm_forward(X, g, H, rstd, cfg.eps, stream=stream)
        if ev is not None:
            ev[1].record(stream)
        B.flce_rmsnorm_backward(X, g, rstd, dH, dX, dg, ws, stream=stream)
        if ev is not None:
            ev[2].record(stream)

    ms, fwd_ms, step_ms, peak_delta, sclk = _time_steps(args, step, stream)
    bwd_ms = ms - fwd_ms
    fwd_b, bwd_b = norm_bytes(N, D, es, min(N, 512))
    achieved = bwd_b / (bwd_ms * 1e-3) / 1e9
    out = _common(args, workload_metric(METRIC_NORM, cfg), N / (ms * 1e-3), ms, cfg.dtype,
                  f"synthetic: seeded X ~ N(0, {cfg.x_std}^2), gamma ~ 1 + N(0, {cfg.gamma_std}^2), "
                  f"dH ~ N(0, {cfg.dh_std}^2), eps {cfg.eps:g}",
                  {"workload": f"{cfg.name}: RMSNorm of the hidden states before the lm_head, fwd + fused bwd",
                   "N": N, "D": D, "parallelism": "single GPU"})
    out.update({
        "hbm_peak_frac": (fwd_b + bwd_b) / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "fwd_ms": fwd_ms,
        "bwd_ms": bwd_ms,
        "fwd_gbs": fwd_b / (fwd_ms * 1e-3) / 1e9,
        "step_ms_median": step_ms[len(step_ms) // 2],
        "step_ms_min": step_ms[0],
        "step_ms_max": step_ms[-1],
        "sclk_mhz": sclk,
        "torch_peak_alloc_delta_bytes": int(peak_delta),
        "roofline": {"kernel": "rms_bwd (+ 2 dgamma passes)", "bound": "hbm", "achieved": achieved,
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS,
                     "traffic": load_traffic("rms_bwd", cfg.name, "norm")},
        "cpu_baseline": None,
    })
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_norm(inp)
    return out


def run_unfused_memory(args) -> dict:
    """The pages' memory experiment, as context: peak device memory (torch's
    max_memory_allocated, above what is held before) of the unfused head -- logits H W^T
    materialised in the input type, F.cross_entropy, autograd's backward into H and W --
    beside the fused library's whole workspace, on the Llama-2- and Llama-3-shaped
    workloads.  Plain 2-D products only.  One line per workload; no timing."""
    import torch
    import torch.nn.functional as F
    from linear_cross_entropy_lm_amd import binding as B
    from linear_cross_entropy_lm_amd import inputs as I
    out = []
    for name in (args.workload or "llama2,llama3").split(","):
        cfg = I.CONFIGS[name]
        inp = I.generate(cfg)
        H, W, y = inp.device_tensors("cuda:0")
        H.requires_grad_(True)
        W.requires_grad_(True)
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        held = torch.cuda.memory_allocated()
        torch.cuda.reset_peak_memory_stats()
        loss = F.cross_entropy(torch.mm(H, W.t()), y, ignore_index=-100)
        loss.backward()
        torch.cuda.synchronize()
        peak = torch.cuda.max_memory_allocated() - held
        grads = H.grad.numel() * H.grad.element_size() + W.grad.numel() * W.grad.element_size()
        ws = B.flce_workspace_bytes(cfg.N, cfg.D, cfg.V, H.dtype)
        logit_bytes = cfg.N * cfg.V * H.element_size()
        out.append({"workload": name, "N": cfg.N, "D": cfg.D, "V": cfg.V, "dtype": cfg.dtype,
                    "unfused_peak_bytes": int(peak), "unfused_peak_minus_grads": int(peak - grads),
                    "logit_bytes": int(logit_bytes), "fused_workspace_bytes": int(ws),
                    "fused_workspace_frac_of_logits": ws / logit_bytes, "loss": float(loss.item())})
        del H, W, y, loss
        torch.cuda.empty_cache()
    return {"memory": out}


def _parse_sclk_mhz(text: str):
    """The current level of an amdgpu pp_dpm_sclk listing ("1: 1650Mhz *") in MHz, or None."""
    import re
    for line in text.splitlines():
        if line.rstrip().endswith("*"):
            m = re.search(r"(\d+)\s*mhz", line, re.I)
            if m:
                return float(m.group(1))
    return None


def sclk_path():
    """The pp_dpm_sclk file of cuda:0: the DRM card whose PCI address matches the device's,
    or the only card that has one; None when it cannot be told (or is not readable)."""
    import glob
    import torch
    cards = [p for p in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")) if os.access(p, os.R_OK)]
    p = torch.cuda.get_device_properties(0)
    want = None
    if all(hasattr(p, a) for a in ("pci_domain_id", "pci_bus_id", "pci_device_id")):
        want = f"{p.pci_domain_id:04x}:{p.pci_bus_id:02x}:{p.pci_device_id:02x}"
    for c in cards:
        if want and os.path.basename(os.path.realpath(os.path.dirname(c))).lower().startswith(want):
            return c
    return cards[0] if len(cards) == 1 and want is None else None


class SclkSampler:
    """Reads the shader clock every `period` seconds on a background thread while active
    (a read of a sysfs text file: no GPU call); summary() gives the median, min and max MHz."""

    def __init__(self, path, period: float = 0.05):
        import threading
        self.path, self.period, self.samples = path, period, []
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True) if path else None

    def _run(self):
        while not self._stop.is_set():
            try:
                with open(self.path) as f:
                    v = _parse_sclk_mhz(f.read())
            except OSError:
                v = None
            if v is not None:
                self.samples.append(v)
            self._stop.wait(self.period)

    def __enter__(self):
        if self._thread:
            self._thread.start()
        return self

    def __exit__(self, *exc):
        if self._thread:
            self._stop.set()
            self._thread.join()

    def summary(self):
        if not self.samples:
            return None
        v = sorted(self.samples)
        return {"median": v[len(v) // 2], "min": v[0], "max": v[-1], "samples": len(v),
                "source": "pp_dpm_sclk current level, sampled every 50 ms over the timed steps"}


def _time_steps(args, step, stream):
    """W warmup steps, one step under torch's allocator peak tracking (the library
    allocates nothing, so the peak stays at what is already held), then K timed steps
    with events around each step and around the whole run.  Returns the mean step ms, the
    mean ms of the first half of each step (the forward), the sorted per-step ms, the
    allocator peak delta and the shader clock sampled over the timed steps (or None)."""
    import torch
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    held = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    step()
    torch.cuda.synchronize()
    peak_delta = torch.cuda.max_memory_allocated() - held
    evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    with SclkSampler(sclk_path()) as clk:
        start.record(stream)
        for k in range(args.steps):
            step(evs[k])
        end.record(stream)
        torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    fwd_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    step_ms = sorted(e[0].elapsed_time(e[2]) for e in evs)
    return ms, fwd_ms, step_ms, peak_delta, clk.summary()


def summarize_trace(path: str) -> list[dict]:
    """Per kernel (full name), from a rocprofv3 --kernel-trace output: dispatches, mean, min
    and max duration in us and the share of all kernel time.  `path` is the output directory
    (its *kernel_trace.csv, or else its *results.db) or a results database itself."""
    import csv
    import glob
    import sqlite3
    durs = {}
    csvs = glob.glob(os.path.join(path, "**", "*kernel_trace.csv"), recursive=True) if os.path.isdir(path) else []
    if csvs:
        for f in csvs:
            with open(f) as fh:
                for r in csv.DictReader(fh):
                    durs.setdefault(r["Kernel_Name"], []).append(
                        (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3)
    else:
        dbs = glob.glob(os.path.join(path, "**", "*results.db"), recursive=True) if os.path.isdir(path) else [path]
        for db in dbs:
            con = sqlite3.connect(db)
            for name, start, end in con.execute("select name, start, end from kernels"):
                durs.setdefault(name, []).append((end - start) * 1e-3)
            con.close()
    total = sum(sum(v) for v in durs.values())
    out = [{"kernel": k, "dispatches": len(v), "mean_us": sum(v) / len(v), "min_us": min(v), "max_us": max(v),
            "share": sum(v) / total} for k, v in durs.items()]
    return sorted(out, key=lambda r: -r["share"])


def _counter_dispatches(csv_dir: str) -> list[dict]:
    """Every dispatch in the rocprofv3 --pmc csv output under csv_dir: the kernel's short
    name, its grid and workgroup sizes and its duration in seconds ("s") where the rows
    carry them, and each counter summed over the rows (instances) that report it."""
    import csv
    import glob
    import re
    disp = {}
    for path in glob.glob(os.path.join(csv_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for r in csv.DictReader(f):
                d = disp.get((path, r["Dispatch_Id"]))
                if d is None:
                    d = {"name": re.sub(r"\(anonymous namespace\)::|void ", "", r["Kernel_Name"]).split("(")[0].strip()}
                    if r.get("Grid_Size"):
                        d["grid"], d["wg"] = int(r["Grid_Size"]), int(r["Workgroup_Size"])
                    if r.get("Start_Timestamp"):
                        d["s"] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
                    disp[(path, r["Dispatch_Id"])] = d
                d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return list(disp.values())


OCCUPANCY_COUNTERS = ("GRBM_GUI_ACTIVE", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_LDS_IDX_ACTIVE", "SQ_LDS_BANK_CONFLICT",
                      "SQ_LDS_ADDR_CONFLICT", "SQ_BUSY_CU_CYCLES", "SQ_WAIT_INST_LDS", "SQ_LDS_DATA_FIFO_FULL")
MI355X_XCDS, MI355X_CUS, MI355X_SIMDS = 8, 256, 1024


def summarize_occupancy(csv_dir: str, min_us: float = 100.0) -> list[dict]:
    """Per kernel (name and launch shape), from one rocprofv3 --pmc run of OCCUPANCY_COUNTERS
    (--output-format csv, whose rows carry each dispatch's start and end): the mean duration,
    the shader clock (GRBM_GUI_ACTIVE is summed over the 8 XCDs, so one XCD's busy cycles
    over the duration), the fraction of those cycles the MFMA pipes are busy (per SIMD), the
    product clock x MFMA busy (GHz of fully busy MFMA issue), and the LDS-active, LDS
    bank-conflict and LDS-issue-wait fractions (per CU, per CU, per SIMD; the wait counter is
    in units of 4 cycles).  Kernels whose mean duration is under min_us are left out."""
    agg = {}
    for d in _counter_dispatches(csv_dir):
        if not all(c in d for c in OCCUPANCY_COUNTERS):
            continue
        a = agg.setdefault((d["name"], d["grid"] // d["wg"], d["wg"]), {c: 0.0 for c in OCCUPANCY_COUNTERS + ("s", "n")})
        a["n"] += 1
        for c in OCCUPANCY_COUNTERS + ("s",):
            a[c] += d[c]
    out = []
    for (name, grid, wg), a in agg.items():
        if a["s"] / a["n"] * 1e6 < min_us:
            continue
        cyc = a["GRBM_GUI_ACTIVE"] / MI355X_XCDS
        clk = cyc / a["s"] / 1e9
        mfma = a["SQ_VALU_MFMA_BUSY_CYCLES"] / (cyc * MI355X_SIMDS)
        out.append({"kernel": name, "grid": grid, "workgroup": wg, "dispatches": int(a["n"]),
                    "mean_us": a["s"] / a["n"] * 1e6, "clock_ghz": clk, "mfma_busy": mfma,
                    "mfma_busy_ghz": clk * mfma, "lds_active": a["SQ_LDS_IDX_ACTIVE"] / (cyc * MI355X_CUS),
                    "lds_bank_conflict": a["SQ_LDS_BANK_CONFLICT"] / (cyc * MI355X_CUS),
                    "lds_issue_wait": 4 * a["SQ_WAIT_INST_LDS"] / (cyc * MI355X_SIMDS)})
    return out


MEMSTALL_COUNTERS = ("GRBM_GUI_ACTIVE", "SQ_VALU_MFMA_BUSY_CYCLES", "TCC_HIT_sum", "TCC_MISS_sum",
                     "TCP_TCC_READ_REQ_LATENCY_sum", "TCP_TCC_READ_REQ_sum", "TCP_PENDING_STALL_CYCLES_sum")


def summarize_memstall(csv_dir: str, min_us: float = 100.0) -> list[dict]:
    """Per kernel, from one rocprofv3 --pmc run of MEMSTALL_COUNTERS (csv, with each
    dispatch's start and end): clock and MFMA busy as in summarize_occupancy, the L2 hit
    rate, the mean latency of the L1's read requests to the L2 in cycles and in ns, and the
    fraction of each CU's cycles in which its L1 held requests back because too many were
    pending.  Kernels whose mean duration is under min_us are left out."""
    agg = {}
    for d in _counter_dispatches(csv_dir):
        if not all(c in d for c in MEMSTALL_COUNTERS):
            continue
        a = agg.setdefault(d["name"], {c: 0.0 for c in MEMSTALL_COUNTERS + ("s", "n")})
        a["n"] += 1
        for c in MEMSTALL_COUNTERS + ("s",):
            a[c] += d[c]
    out = []
    for name, a in agg.items():
        if a["s"] / a["n"] * 1e6 < min_us:
            continue
        cyc = a["GRBM_GUI_ACTIVE"] / MI355X_XCDS
        clk = cyc / a["s"] / 1e9
        lat = a["TCP_TCC_READ_REQ_LATENCY_sum"] / max(a["TCP_TCC_READ_REQ_sum"], 1.0)
        out.append({"kernel": name, "dispatches": int(a["n"]), "mean_us": a["s"] / a["n"] * 1e6, "clock_ghz": clk,
                    "mfma_busy": a["SQ_VALU_MFMA_BUSY_CYCLES"] / (cyc * MI355X_SIMDS),
                    "l2_hit": a["TCC_HIT_sum"] / max(a["TCC_HIT_sum"] + a["TCC_MISS_sum"], 1.0),
                    "l1_l2_read_latency_cycles": lat, "l1_l2_read_latency_ns": lat / clk,
                    "l1_pending_stall": a["TCP_PENDING_STALL_CYCLES_sum"] / (cyc * MI355X_CUS)})
    return out


MOPS_COUNTERS = ("SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_VALU_MFMA_MOPS_F16", "SQ_INSTS_VALU_MFMA_MOPS_F32")


def summarize_mops(csv_dir: str, workload: str, path: str = "fused") -> list[dict]:
    """Executed matrix-core flops, from one rocprofv3 --pmc run of MOPS_COUNTERS under
    csv_dir (each counter counts multiplies and adds over 512, summed over the chip): one
    record per kernel (dispatches, flops per dispatch), then one for the whole run per call
    of the path (the calls are counted by fwd_finalize, launched once per forward or
    one-call pass), set against the flops the path is credited with: 8 N V D for the
    recomputing schedule (forward, dz recompute, dH, dW), 6 N V D for the single pass."""
    from linear_cross_entropy_lm_amd import inputs as I
    per = {}
    for d in _counter_dispatches(csv_dir):
        a = per.setdefault(d["name"], {"dispatches": 0, "flop": 0.0})
        a["dispatches"] += 1
        a["flop"] += 512.0 * sum(d.get(c, 0.0) for c in MOPS_COUNTERS)
    calls = sum(a["dispatches"] for n, a in per.items() if n.startswith("fwd_finalize"))
    out = [{"kernel": n, "dispatches": a["dispatches"], "tflop_per_dispatch": a["flop"] / a["dispatches"] / 1e12}
           for n, a in sorted(per.items(), key=lambda kv: -kv[1]["flop"]) if a["flop"] > 0]
    cfg = I.CONFIGS[workload]
    credited = (6 if path == "single" else 8) * cfg.N * cfg.V * cfg.D
    total = sum(a["flop"] for a in per.values())
    out.append({"workload": workload, "path": path, "calls": calls,
                "executed_tflop_per_call": total / max(calls, 1) / 1e12, "credited_tflop_per_call": credited / 1e12,
                "executed_over_credited": total / max(calls, 1) / credited})
    return out


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=int(os.environ.get("WORLD_SIZE", "1")))
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--path", choices=sorted(PATHS) + ["unfused-memory"], default="fused",
                    help="fused: lm_head projection + cross-entropy (default); single: the same in one "
                         "call without logit recompute (25%% scratch); ce: cross-entropy over materialised "
                         "logits; norm: the RMSNorm that produces H")
    ap.add_argument("--workload", default=None, help="default llama3 (fused), ce_llama3 (ce), norm_llama3 (norm)")
    ap.add_argument("--sp-workspace", type=float, default=1.0, metavar="F",
                    help="--path single: workspace = F x the least single-pass workspace (2.0: token "
                         "chunks of 8192 at the Llama-3 shape)")
    ap.add_argument("--cpu-rows", type=int, default=None,
                    help="rows of the oracle sample (default 1024 fused, 8192 ce: 10-20 s of CPU work)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-kernel-timing", action="store_true",
                    help="skip the second timed region with per-launch events (no per-kernel list, no roofline)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run one device-to-device copy of BYTES bytes (counter calibration)")
    ap.add_argument("--summarize-counters", metavar="DIR",
                    help="only write the path's traffic record from rocprofv3 counter runs under DIR "
                         "(subdirectories F, W, FC, WC); no GPU needed")
    ap.add_argument("--summarize-trace", metavar="PATH",
                    help="only print per-kernel dispatch counts and durations from a rocprofv3 --kernel-trace "
                         "output directory or results database; no GPU needed")
    ap.add_argument("--summarize-occupancy", metavar="DIR",
                    help="only print, per kernel, clock, MFMA-busy and LDS figures from one rocprofv3 --pmc "
                         "run of bench.OCCUPANCY_COUNTERS under DIR; no GPU needed")
    ap.add_argument("--summarize-memstall", metavar="DIR",
                    help="only print, per kernel, L2 hit rate, L1-to-L2 read latency and L1 pending stalls "
                         "from one rocprofv3 --pmc run of bench.MEMSTALL_COUNTERS under DIR; no GPU needed")
    ap.add_argument("--summarize-mops", metavar="DIR",
                    help="only print executed MFMA flops per kernel and per call, from one rocprofv3 --pmc run "
                         "of bench.MOPS_COUNTERS under DIR (--path, --workload name the run); no GPU needed")
    ap.add_argument("--copy-bytes", type=int, default=1 << 30)
    ap.add_argument("--kinds", default=None,
                    help="--summarize-counters: comma-separated kernel kinds (default: the path's GEMMs)")
    args = ap.parse_args()
    if args.summarize_trace:
        for rec in summarize_trace(args.summarize_trace):
            print(json.dumps(rec), flush=True)
        return 0
    if args.summarize_occupancy:
        for rec in summarize_occupancy(args.summarize_occupancy):
            print(json.dumps(rec), flush=True)
        return 0
    if args.summarize_memstall:
        for rec in summarize_memstall(args.summarize_memstall):
            print(json.dumps(rec), flush=True)
        return 0
    if args.summarize_mops:
        for rec in summarize_mops(args.summarize_mops, args.workload or "llama3", args.path):
            print(json.dumps(rec), flush=True)
        return 0
    if args.summarize_counters:
        kinds = args.kinds.split(",") if args.kinds else {
            "fused": ["fwd_tiles16", "bwd_dz16", "bwd_dhdw"], "single": ["fwd_tiles16_keep", "bwd_dhdw"],
            "ce": ["ce_rows_bwd"], "norm": ["rms_bwd"]}[args.path]
        for rec in summarize_counters(args.summarize_counters, args.copy_bytes, args.path, kinds,
                                      args.workload or PATHS[args.path][0]):
            print(json.dumps(rec), flush=True)
        return 0
    if args.calibrate_copy:
        import torch
        src = torch.ones(args.calibrate_copy // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copied_bytes": args.calibrate_copy}), flush=True)
        return 0
    if args.gpus != 1:
        print(f"bench.py: this build runs on exactly one GPU (asked for {args.gpus}); the multi-GPU "
              "sharding of the path is described, not built.", file=sys.stderr)
        return 2
    out = {"ce": run_ce, "norm": run_norm, "single": run_single, "fused": run_fused,
           "unfused-memory": run_unfused_memory}[args.path](args)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
