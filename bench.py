"""Throughput of the 3-Newton ParaGRU / ParaLSTM solve on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

A step is one whole solve over one batch of seeded synthetic inputs already
resident in HBM: workspace reset, all K Newton iterations in one fused launch
(the iterate stays on chip between iterations), flag finalisation; for the
adjoint workload also the reverse-scan launch. Prints one JSON line with the
throughput in solved state elements (B*L*D) per second; the roofline of the
fused launch (vector-ALU issue slots per element over its duration, timed with
HIP events on the stream the kernels run on); the same solve with one launch
per iteration and its HBM roofline; and the fp64 CPU oracle timed on a bounded
sample of the same workload. Scan workloads (--workload scan_*) time the
linear scan alone.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
PEAK_HBM_GBS = 8000.0  # MI355X HBM3E peak
# vector ALU issue peak without packed fp32: 256 CUs x 64 lanes x 2.4 GHz
# lane-operations per second (the fp32 vector 157.3 TFLOP/s counts a packed
# FMA, 4 flops, per lane-operation)
# fp32 vector issue slots: 256 CUs x 128 lane-slots per clock x 2.4 GHz, the
# chip's published fp32 vector peak (157.3 TFLOP/s) counted one FMA per slot.
# Measured on the card: a stream of non-packed v_mul_f32 / v_fma_f32 issues
# about 108 lane-ops per clock per CU once two or more waves share a SIMD (one
# wave alone: about 51), and v_exp_f32 / v_rcp_f32 about 31, i.e. four slots.
PEAK_VALU_TSLOTS = 256 * 128 * 2.4e9 / 1e12
PEAK_F32_MATRIX_TFLOPS = 157.3  # MI355X dense fp32 matrix-core peak


# VALU issue slots per state element per Newton iteration (cell, Jacobian,
# scan), transcendentals at four slots each: GRU about 40 VALU + 6
# transcendental, LSTM about 70 + 10
def alu_slots(cell: str) -> int:
    return 63 if cell == "gru" else 110

# algorithmic HBM bytes per state element for one Newton-iteration launch:
# read the gate inputs (G per element) and, after the first iteration, the
# previous iterate; write the new iterate (NS fp32 state components).
def iter_bytes(cell: str, u_bytes: int, k: int) -> int:
    G, NS = (3, 1) if cell == "gru" else (4, 2)
    return G * u_bytes + NS * 4 * (1 if k == 1 else 2)


# adjoint: read u, the trajectory and dh, write du (fp32)
def adjoint_bytes(cell: str, u_bytes: int) -> int:
    G, NS = (3, 1) if cell == "gru" else (4, 2)
    return G * u_bytes + NS * 4 + 4 + G * 4


def source_digest() -> str:
    """Digest of the kernel sources with comments and blank lines removed, so
    that counters stay tied to the code they were taken on, not its comments."""
    h = hashlib.sha256()
    for p in sorted((ROOT / "nonlinear_rnn_solve_newton_amd" / "csrc").glob("*")):
        text = re.sub(r"/\*.*?\*/", "", p.read_text(), flags=re.S)
        lines = (re.sub(r"//.*$", "", ln).rstrip() for ln in text.splitlines())
        h.update(p.name.encode())
        h.update("\n".join(ln for ln in lines if ln).encode())
    return h.hexdigest()[:16]


class HipEvents:
    """hipEvent_t handles through the HIP runtime's C API."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        evs = []
        for _ in range(n):
            e = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            evs.append(e.value)
        return evs

    def ms(self, a, b):
        out = ctypes.c_float()
        if self.hip.hipEventSynchronize(ctypes.c_void_p(b)) != 0:
            raise RuntimeError("hipEventSynchronize failed")
        if self.hip.hipEventElapsedTime(ctypes.byref(out), ctypes.c_void_p(a), ctypes.c_void_p(b)) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(out.value)

    def destroy(self, evs):
        for e in evs:
            self.hip.hipEventDestroy(ctypes.c_void_p(e))


def traffic_path(workload: str, kernel: str = "newton_iter") -> Path:
    return ROOT / "profiles" / f"{kernel}_{workload}_traffic.json"


def load_traffic(workload: str, digest: str, kernel: str = "newton_iter"):
    """Counter-measured HBM bytes per launch for the current kernel sources, if profiled."""
    f = traffic_path(workload, kernel)
    if not f.exists():
        return None
    try:
        d = json.loads(f.read_text())
    except ValueError:
        return None
    if d.get("source_digest") != digest:
        return None
    return d.get("bytes_per_launch")


def traffic_from_counters(workload: str, fetch_csv: str, write_csv: str, iters: int,
                          kernel: str = "newton_iter") -> dict:
    """Per-launch HBM bytes of the Newton-iteration (or scan) kernel from two rocprofv3
    --pmc runs (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch) of
    `bench.py --copy-calibration`. Each counter is scaled by bytes / counter of
    the 1 GiB device copy in the same run."""
    import csv

    def read(path, counter):
        rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]
        rows.sort(key=lambda r: int(r["Dispatch_Id"]))
        copy = [float(r["Counter_Value"]) * 1024 for r in rows
                if "copyBuffer" in r["Kernel_Name"] and float(r["Counter_Value"]) > 1e5]
        if kernel == "dense":  # one scan = the launches from one transfer launch to the next
            its = []
            for r in rows:
                if "pararnn::dense_" not in r["Kernel_Name"]:
                    continue
                if "dense_chunk_kernel" in r["Kernel_Name"]:
                    its.append(0.0)
                if its:
                    its[-1] += float(r["Counter_Value"]) * 1024
            return copy, its
        its = [float(r["Counter_Value"]) * 1024 for r in rows if f"{kernel}_kernel" in r["Kernel_Name"]]
        return copy, its

    calib = float(1 << 30)
    fc, fi = read(fetch_csv, "FETCH_SIZE")
    wc, wi = read(write_csv, "WRITE_SIZE")
    fscale = calib / (sum(fc) / len(fc))
    wscale = calib / (sum(wc) / len(wc))
    # dispatches come in solves of `iters` launches; average each launch index
    per_k = []
    for k in range(iters):
        f = [v * fscale for j, v in enumerate(fi) if j % iters == k]
        w = [v * wscale for j, v in enumerate(wi) if j % iters == k]
        per_k.append({"fetch": sum(f) / len(f), "write": sum(w) / len(w)})
    mean = sum(x["fetch"] + x["write"] for x in per_k) / iters
    return {"workload": workload, "source_digest": source_digest(), "bytes_per_launch": mean,
            "per_launch": per_k, "fetch_scale": fscale, "write_scale": wscale,
            "calibration": "1 GiB hipMemcpy device copy (__amd_rocclr_copyBuffer) in the same run"}


def write_stats_summary(workload: str, stats_csv: str) -> str:
    """profiles/<workload>_kernel_stats.md from rocprofv3 --kernel-trace --stats output."""
    import csv

    rows = list(csv.DictReader(open(stats_csv)))
    lines = [f"# rocprofv3 kernel statistics: {workload}", "",
             "Command (on the MI355X box, from /tmp with TMPDIR=/tmp):", "",
             f"    rocprofv3 --kernel-trace --stats --output-format csv -d <out> -o run -- "
             f"python3 <repo>/bench.py --workload {workload} --steps 5 --warmup 2 --no-cpu-baseline", "",
             f"Kernel sources digest: {source_digest()} (bench.py source_digest()).", "",
             "| kernel | calls | average ns | min ns | max ns | % time |", "|---|---|---|---|---|---|"]
    for r in rows:
        lines.append(f"| `{r['Name'][:100]}` | {r['Calls']} | {float(r['AverageNs']):.0f} | {r['MinNs']} | "
                     f"{r['MaxNs']} | {float(r['Percentage']):.2f} |")
    text = "\n".join(lines) + "\n"
    (ROOT / "profiles" / f"{workload}_kernel_stats.md").write_text(text)
    return text


def cpu_baseline(w, x, iters, target_s=12.0):
    """fp64 oracle Newton solve on a channel sample of the same workload."""
    from nonlinear_rnn_solve_newton_amd.workloads import gather_channels, sample_channels
    from oracle import oracle as O

    nthreads = O.default_threads()
    BD = w.B * w.D

    def run(n):
        ch = sample_channels(w.B, w.D, n, seed=99)
        u = gather_channels(x.u, ch, w.D)
        a = x.a[:, ch % w.D].contiguous()
        t0 = time.perf_counter()
        O.newton(w.cell, u, a, K=iters, nthreads=nthreads)
        t1 = time.perf_counter()
        O.seq(w.cell, u, a, nthreads=nthreads)
        t2 = time.perf_counter()
        return len(ch), t1 - t0, t2 - t1

    n0 = min(BD, max(nthreads, 16))
    n, t_newton, _ = run(n0)
    per_chan = t_newton / n
    n = int(min(BD, max(n0, target_s / max(per_chan, 1e-9))))
    n = max(nthreads, n - n % max(nthreads, 1)) if n < BD else n
    n, t_newton, t_seq = run(n)
    elems = n * w.L
    return {
        "value": elems / t_newton,
        "unit": "elems/s",
        "cores": nthreads,
        "kind": "oracle",
        "sample": f"{n} of {BD} channels (b, d) over the full L={w.L}, {iters} fp64 Newton iterations; "
                  f"{t_newton:.2f} s",
        "sequential_value": elems / t_seq,
    }


# linear scan alone: read NS*NS coefficient planes and NS input planes, write
# NS state planes, fp32
def scan_bytes(ns: int) -> int:
    return 4 * (ns * ns + 2 * ns)


def cpu_baseline_scan(w, x, target_s=12.0):
    """fp64 oracle scan on a sample of batch rows of the same workload (all D)."""
    from oracle import oracle as O

    nthreads = O.default_threads()

    def run(nb):
        A = x.A[:nb] if w.ns == 1 else x.A[:, :, :nb]
        b = x.b[:nb] if w.ns == 1 else x.b[:, :nb]
        s0 = x.s0[None, :nb] if w.ns == 1 else x.s0[:, :nb]
        t0 = time.perf_counter()
        O.scan(A, b, s0, nthreads=nthreads)
        return time.perf_counter() - t0

    t1 = run(1)
    nb = int(min(w.B, max(1, target_s / max(t1, 1e-9))))
    t = run(nb) if nb > 1 else t1
    elems = nb * w.L * w.D
    return {"value": elems / t, "unit": "elems/s", "cores": nthreads, "kind": "oracle",
            "sample": f"{nb} of {w.B} batch rows (all D={w.D}, full L={w.L}), fp64 loop; {t:.2f} s"}


def bench_scan_dense(w, args):
    """The dense recurrence (pararnn_scan_dense): chunk transfers on the matrix
    cores, carries, then the recurrence per chunk."""
    import torch
    from nonlinear_rnn_solve_newton_amd import binding
    from nonlinear_rnn_solve_newton_amd.workloads import dense_workload_inputs

    dev = torch.device("cuda:0")
    x = dense_workload_inputs(w)
    A, b, s0 = x.A.to(dev), x.b.to(dev), x.s0.to(dev)
    hip = HipEvents()
    ev = hip.create(3)
    first = binding.scan_dense(A, b, s0)
    ws, out = first["ws"], first["s"]
    for _ in range(args.warmup):
        binding.scan_dense(A, b, s0, out=out, ws=ws)
    torch.cuda.synchronize()
    kms = []
    for _ in range(args.steps):
        binding.scan_dense(A, b, s0, out=out, ws=ws, events=ev)
        kms.append(hip.ms(ev[1], ev[2]))
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(args.steps):
        binding.scan_dense(A, b, s0, out=out, ws=ws)
    stop.record()
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(stop) / args.steps
    t = sum(kms) / len(kms)
    steps = w.B * w.L
    nbytes = steps * (w.n * w.n + 2 * w.n) * 4  # read A and b once, write s once
    flops = steps * 2 * 32 ** 3  # one 32x32x32 transfer product per step (fp32 matrix cores)
    achieved = nbytes / (t * 1e-3) / 1e9
    result = {
        "metric": "scanned state elems/s (B*L*n) of the dense recurrence s_l = A_l s_{l-1} + b_l",
        "value": w.N / (ms_step * 1e-3), "unit": "elems/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (seeded; A = 0.95 x random orthogonal, b, s0 ~ N(0,1))",
        "config": {"workload": w.name, "B": w.B, "L": w.L, "n": w.n},
        "roofline": {"bound": "hbm", "kernel": "dense_chunk_kernel + dense_carry_kernel + dense_apply_kernel",
                     "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS,
                     "traffic": load_traffic(w.name, source_digest(), "dense"),
                     "algorithmic_bytes_per_launch": [nbytes], "launch_ms": [t]},
        "matrix_cores": {"achieved": flops / (t * 1e-3) / 1e12, "peak": PEAK_F32_MATRIX_TFLOPS,
                         "unit": "TFLOP/s", "frac": flops / (t * 1e-3) / 1e12 / PEAK_F32_MATRIX_TFLOPS},
        "timing": {"scan_ms": t, "source_digest": source_digest()},
    }
    if args.copy_calibration:
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        result["copy_calibration_bytes"] = src.numel() * 4
    if not args.no_cpu_baseline:
        from oracle import oracle as O
        nthreads = O.default_threads()
        t0 = time.perf_counter()
        O.scan_dense(x.A, x.b, x.s0, nthreads=nthreads)
        dt = time.perf_counter() - t0
        result["cpu_baseline"] = {"value": w.N / dt, "unit": "elems/s", "cores": min(nthreads, w.B),
                                  "kind": "oracle",
                                  "sample": f"the whole workload ({w.B} rows), fp64 loop; {dt:.2f} s"}
    hip.destroy(ev)
    print(json.dumps(result), flush=True)
    return 0


def bench_scan(w, args):
    """The linear scan alone (pararnn_scan_diag / pararnn_scan_block2)."""
    import torch
    from nonlinear_rnn_solve_newton_amd import binding
    from nonlinear_rnn_solve_newton_amd.workloads import scan_workload_inputs

    dev = torch.device("cuda:0")
    x = scan_workload_inputs(w)
    A, b, s0 = x.A.to(dev), x.b.to(dev), x.s0.to(dev)
    hip = HipEvents()
    ev = hip.create(3)
    first = binding.scan(A, b, s0)
    ws, out = first["ws"], first["s"]
    for _ in range(args.warmup):
        binding.scan(A, b, s0, out=out, ws=ws)
    torch.cuda.synchronize()
    scan_ms, clear_ms = [], []
    for _ in range(args.steps):
        binding.scan(A, b, s0, out=out, ws=ws, events=ev)
        clear_ms.append(hip.ms(ev[0], ev[1]))
        scan_ms.append(hip.ms(ev[1], ev[2]))
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(args.steps):
        binding.scan(A, b, s0, out=out, ws=ws)
    stop.record()
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(stop) / args.steps
    mean = lambda v: sum(v) / len(v)  # noqa: E731
    kms = mean(scan_ms)
    nbytes = scan_bytes(w.ns) * w.N
    achieved = nbytes / (kms * 1e-3) / 1e9
    digest = source_digest()
    result = {
        "metric": "scanned state elems/s (B*L*D) of the linear scan s_l = A_l s_{l-1} + b_l",
        "value": w.N / (ms_step * 1e-3),
        "unit": "elems/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded; A ~ U(-0.95, 0.95) per block row sum, b, s0 ~ N(0,1))",
        "config": {"workload": w.name, "block": "diag" if w.ns == 1 else "2x2", "B": w.B, "L": w.L, "D": w.D},
        "roofline": {"bound": "hbm", "kernel": "scan_kernel", "achieved": achieved, "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS,
                     "traffic": load_traffic(w.name, digest, "scan"),
                     "algorithmic_bytes_per_launch": [nbytes], "launch_ms": [kms]},
        # reset: from the marker before the workspace reset to the scan's start
        "timing": {"reset_to_launch_ms": mean(clear_ms), "scan_ms": kms, "source_digest": digest},
    }
    if args.copy_calibration:
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        result["copy_calibration_bytes"] = src.numel() * 4
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_scan(w, x)
    hip.destroy(ev)
    print(json.dumps(result), flush=True)
    return 0


def bench_generic(w, args):
    """The workload's cell written as a user cell in torch, solved by the
    generic tier; reported next to the fused kernels, not instead of them."""
    import torch
    from nonlinear_rnn_solve_newton_amd import generic
    from nonlinear_rnn_solve_newton_amd.workloads import workload_inputs

    dev = torch.device("cuda:0")
    x = workload_inputs(w)
    u, a = x.u.to(dev), x.a.to(dev)
    if w.cell == "gru":
        run = lambda: generic.newton_solve(lambda h, uu: generic.gru_step(h, uu, a), u,  # noqa: E731
                                           B=w.B, L=w.L, D=w.D, iters=w.iters)
    else:
        run = lambda: generic.newton_solve(lambda s, uu: generic.lstm_step(s, uu, a), u,  # noqa: E731
                                           B=w.B, L=w.L, D=w.D, iters=w.iters, block=2)
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(args.steps):
        run()
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / args.steps
    print(json.dumps({
        "metric": "solved state elems/s (B*L*D) per 3-Newton solve, generic-cell tier",
        "value": w.N / (ms * 1e-3), "unit": "elems/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic (same inputs as the fused workload)",
        "config": {"workload": w.name, "tier": "generic: torch cell, torch.func.jvp Jacobian, "
                   "pararnn_scan_diag / pararnn_scan_block2 per iteration"},
    }), flush=True)
    return 0


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--generic", action="store_true",
                    help="run the workload's cell through the generic-cell tier (torch cell + forward-mode "
                         "AD Jacobian + the library's scan) instead of the fused kernels")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration for profiling)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/newton_iter_<workload>_traffic.json from rocprofv3 counter CSVs")
    ap.add_argument("--stats-summary", metavar="KERNEL_STATS_CSV",
                    help="write profiles/<workload>_kernel_stats.md from a rocprofv3 --stats CSV")
    args = ap.parse_args(argv)
    sys.path.insert(0, str(ROOT))
    from nonlinear_rnn_solve_newton_amd.workloads import DENSE_WORKLOADS, HEADLINE, SCAN_WORKLOADS, WORKLOADS
    name = args.workload or HEADLINE
    if name not in WORKLOADS and name not in SCAN_WORKLOADS and name not in DENSE_WORKLOADS:
        print(json.dumps({"error": f"unknown workload {name}",
                          "workloads": sorted(WORKLOADS) + sorted(SCAN_WORKLOADS) + sorted(DENSE_WORKLOADS)}))
        return 2
    if args.stats_summary:
        print(write_stats_summary(name, args.stats_summary))
        return 0
    if args.traffic_from:
        if name in SCAN_WORKLOADS:
            d = traffic_from_counters(name, *args.traffic_from, iters=1, kernel="scan")
            traffic_path(name, "scan").write_text(json.dumps(d, indent=1) + "\n")
        elif name in DENSE_WORKLOADS:
            d = traffic_from_counters(name, *args.traffic_from, iters=1, kernel="dense")
            traffic_path(name, "dense").write_text(json.dumps(d, indent=1) + "\n")
        else:
            d = traffic_from_counters(name, *args.traffic_from, iters=WORKLOADS[name].iters)
            traffic_path(name).write_text(json.dumps(d, indent=1) + "\n")
            print(json.dumps(d))
            d = traffic_from_counters(name, *args.traffic_from, iters=1, kernel="newton_fused")
            traffic_path(name, "newton_fused").write_text(json.dumps(d, indent=1) + "\n")
        print(json.dumps(d))
        return 0
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "the library runs on one GPU; sharding across GPUs is described in the "
                                   "design notes, not implemented", "n_gpus": args.gpus}))
        return 2

    if name in SCAN_WORKLOADS:
        return bench_scan(SCAN_WORKLOADS[name], args)
    if name in DENSE_WORKLOADS:
        return bench_scan_dense(DENSE_WORKLOADS[name], args)
    if args.generic:
        return bench_generic(WORKLOADS[name], args)

    import torch

    from nonlinear_rnn_solve_newton_amd import binding
    from nonlinear_rnn_solve_newton_amd.workloads import workload_inputs

    w = WORKLOADS[name]
    K = w.iters
    dev = torch.device("cuda:0")
    x = workload_inputs(w)
    u, a = x.u.to(dev), x.a.to(dev)
    dh = x.dh.to(dev) if w.adjoint else None
    u_bytes = 2 if w.u_dtype == "bf16" else 4
    torch.cuda.synchronize()

    hip = HipEvents()
    ev = hip.create(K + 2)
    ev_adj = hip.create(3) if w.adjoint else None
    mean = lambda v: sum(v) / len(v)  # noqa: E731

    def time_schedule(schedule):
        """One schedule of the solve (plus the adjoint for the adjoint workload):
        per-step time without events, and per-kernel times from events."""
        first = binding.solve(w.cell, u, a, iters=K, schedule=schedule)
        ws, out = first["ws"], {k: first[k] for k in ("h", "c") if k in first}
        gadj = binding.adjoint(w.cell, u, a, out["h"], dh, c=out.get("c")) if w.adjoint else None

        def step(events=None, events_adj=None):
            binding.solve(w.cell, u, a, iters=K, ws=ws, out=out, events=events, schedule=schedule)
            if w.adjoint:
                binding.adjoint(w.cell, u, a, out["h"], dh, c=out.get("c"), ws=gadj["ws"], du=gadj["du"],
                                events=events_adj)

        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        launch_ms = [[] for _ in range(K)]
        clear_ms, adj_ms = [], []
        for _ in range(args.steps):
            step(ev, ev_adj)
            # per-kernel times: read back after the step (events are reused).
            # The library stamps the launches' own starts and ends into the
            # events (event 1: the first launch's start; k + 1: the end of
            # iteration k's launch, for the fused schedule its one launch and
            # then markers right after it)
            clear_ms.append(hip.ms(ev[0], ev[1]))
            for k in range(K):
                launch_ms[k].append(hip.ms(ev[k + 1], ev[k + 2]))
            if w.adjoint:
                adj_ms.append(hip.ms(ev_adj[1], ev_adj[2]))
        # the event read-backs synchronise once per step; the step time comes
        # from a loop without them
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record()
        for _ in range(args.steps):
            step()
        stop.record()
        torch.cuda.synchronize()
        return {"ms_step": start.elapsed_time(stop) / args.steps, "clear_ms": mean(clear_ms),
                "launch_ms": [mean(v) for v in launch_ms], "adj_ms": mean(adj_ms) if adj_ms else None,
                "out": out, "gadj": gadj}

    N = w.N
    bytes_k = [iter_bytes(w.cell, u_bytes, k + 1) * N for k in range(K)]
    digest = source_digest()
    fused = time_schedule("fused")
    per_it = time_schedule("per_iteration")
    out, gadj = fused["out"], fused["gadj"]
    # events 1 and 2: the start and end of the one fused launch, stamped by
    # its dispatch (the later events are markers recorded after it)
    t_fused = fused["launch_ms"][0]
    slots = alu_slots(w.cell) * K * N
    alu = slots / (t_fused * 1e-3) / 1e12
    hbm_it = sum(bytes_k) / K / (mean(per_it["launch_ms"]) * 1e-3) / 1e9
    result = {
        "metric": "solved state elems/s (B*L*D) per 3-Newton solve; HBM GB/s as % of peak",
        "value": N / (fused["ms_step"] * 1e-3),
        "unit": "elems/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": fused["ms_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded; u ~ N(0,1) stored " + w.u_dtype + ", a ~ U(-amax, amax))",
        "config": {"workload": w.name, "cell": w.cell, "B": w.B, "L": w.L, "D": w.D,
                   "newton_iters": K, "u_dtype": w.u_dtype, "adjoint": w.adjoint, "schedule": "fused"},
        # the fused launch keeps the iterate on chip: it moves the gate inputs
        # once and the final iterate once, and is bound by vector ALU issue
        "roofline": {
            "bound": "alu",
            "kernel": "newton_fused_kernel",
            "achieved": alu,
            "peak": PEAK_VALU_TSLOTS,
            "unit": "T issue-slots/s (fp32 VALU lane-ops, transcendentals at 4 slots)",
            "frac": alu / PEAK_VALU_TSLOTS,
            "traffic": load_traffic(w.name, digest, "newton_fused"),
            "algorithmic_slots_per_launch": slots,
            "launch_ms": t_fused,
        },
        # the same solve in the method's per-iteration form: its algorithmic
        # bytes (inputs + previous iterate read, new iterate written, per iteration)
        "hbm_equivalent": {
            "achieved": sum(bytes_k) / (fused["ms_step"] * 1e-3) / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": sum(bytes_k) / (fused["ms_step"] * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "note": "algorithmic bytes of the per-iteration method per solve / fused solve time"},
        "per_iteration_schedule": {
            "ms_per_step": per_it["ms_step"],
            "roofline": {"bound": "hbm", "kernel": "newton_iter_kernel", "achieved": hbm_it,
                         "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": hbm_it / PEAK_HBM_GBS,
                         "traffic": load_traffic(w.name, digest), "algorithmic_bytes_per_launch": bytes_k,
                         "launch_ms": per_it["launch_ms"]},
        },
        "timing": {
            # from the marker before the workspace reset to the fused launch's
            # start: the reset kernel and both dispatches
            "reset_to_launch_ms": fused["clear_ms"],
            "fused_launch_ms": t_fused,
            "source_digest": digest,
        },
    }
    adj_ms = [fused["adj_ms"]] if w.adjoint else []
    if w.adjoint:
        # the same adjoint with the parameter and initial-state gradients
        # (da, ds0) requested: their partials ride in the reverse scan, plus a
        # fixed-order reduction launch
        gfull = binding.adjoint(w.cell, u, a, out["h"], dh, c=out.get("c"), du=gadj["du"],
                                want_ds0=True, want_da=True)  # a workspace with room for the da partials
        grad_ms = []
        for _ in range(args.steps):
            binding.adjoint(w.cell, u, a, out["h"], dh, c=out.get("c"), ws=gfull["ws"], du=gfull["du"],
                            want_ds0=True, want_da=True, events=ev_adj)
            grad_ms.append(hip.ms(ev_adj[1], ev_adj[2]))
        torch.cuda.synchronize()
        amean = adj_ms[0]
        result["timing"]["adjoint_ms"] = amean
        result["timing"]["adjoint_with_da_ds0_ms"] = mean(grad_ms)
        result["adjoint_roofline"] = {
            "bound": "hbm", "kernel": "adjoint_kernel",
            "achieved": adjoint_bytes(w.cell, u_bytes) * N / (amean * 1e-3) / 1e9,
            "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": adjoint_bytes(w.cell, u_bytes) * N / (amean * 1e-3) / 1e9 / PEAK_HBM_GBS,
        }
    if args.copy_calibration:
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        result["copy_calibration_bytes"] = src.numel() * 4
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, x, K)
    hip.destroy(ev + (ev_adj or []))
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
