"""Throughput of the 3-Newton ParaLSTM / ParaGRU solve on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

A step is one whole pass of the hot path over one batch of seeded synthetic
inputs already resident in HBM. For the default workload (ParaLSTM, B=16,
L=2048, D=4096, forward solve plus adjoint) that is: workspace reset, all K
Newton iterations in one fused launch (the iterate stays on chip between
iterations), flag finalisation, then the reverse-scan adjoint launch giving
dL/du. The other workloads (--workload NAME) are the forward solve alone, or
the linear scan alone for the scan_* workloads.

Prints one JSON line: solved state elements (B*L*D) per second over exactly K
timed steps; the mean, median and minimum step time; per kernel the duration
stamped by its own dispatch and its roofline (the fused Newton launch against
the vector-ALU issue peak with its instructions counted by rocprofv3, and
against HBM with the bytes it moves; the adjoint against HBM), the dominant
kernel's under "roofline"; the same solve with one launch per iteration;
same-run device ceilings (a device copy, the measured VALU issue rates); and
the fp64 CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import re
import statistics
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
PROFILES = ROOT / "profiles"
PEAK_HBM_GBS = 8000.0  # MI355X HBM3E peak
# Vector-ALU issue peak for the code this library runs: 256 CUs x 4 SIMDs x
# 16 lanes x 2.4 GHz = 39.3 T lane operations per second, one issue slot per
# fp32 lane operation. The published fp32 vector peak (157.3 TFLOP/s) is this
# rate x 2 flops per FMA x 2 lanes per packed (v_pk_*_f32) instruction; the
# library is built without packed fp32, so one instruction serves one lane.
PEAK_VALU_TSLOTS = 256 * 4 * 16 * 2.4e9 / 1e12
# A transcendental (v_exp_f32, v_rcp_f32) takes two issue slots: the
# issue-rate kernels measure it at half the FMA rate on this chip.
TRANS_SLOTS = 2
PEAK_F32_MATRIX_TFLOPS = 157.3  # MI355X dense fp32 matrix-core peak


# algorithmic HBM bytes per state element for one Newton-iteration launch of
# the per-iteration schedule: read the gate inputs (G per element) and, after
# the first iteration, the previous iterate; write the new iterate (NS fp32
# state components).
def iter_bytes(cell: str, u_bytes: int, k: int) -> int:
    G, NS = (3, 1) if cell == "gru" else (4, 2)
    return G * u_bytes + NS * 4 * (1 if k == 1 else 2)


# the fused launch (all K iterations, iterate on chip): read the gate inputs
# once, write the final iterate once
def fused_bytes(cell: str, u_bytes: int) -> int:
    G, NS = (3, 1) if cell == "gru" else (4, 2)
    return G * u_bytes + NS * 4


# adjoint: read u, the trajectory and dh, write du (fp32)
def adjoint_bytes(cell: str, u_bytes: int) -> int:
    G, NS = (3, 1) if cell == "gru" else (4, 2)
    return G * u_bytes + NS * 4 + 4 + G * 4


def source_digest() -> str:
    """Digest of the solver's kernel sources with comments and blank lines
    removed, so that counters stay tied to the code they were taken on, not
    its comments. The measurement kernels (ceilings.hip) are not included."""
    h = hashlib.sha256()
    csrc = ROOT / "nonlinear_rnn_solve_newton_amd" / "csrc"
    for p in sorted(list(csrc.glob("*.h")) + [csrc / "pararnn.hip"]):
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


def stats(v):
    """mean, median and minimum of a list of times (ms)"""
    return {"mean": sum(v) / len(v), "median": statistics.median(v), "min": min(v), "max": max(v), "n": len(v)}


# ---------------------------------------------------------------------------
# Counter files under profiles/: per-launch HBM bytes (FETCH_SIZE + WRITE_SIZE)
# and VALU instruction counts, each tagged with the source digest it was taken
# on; a file for other sources is ignored.

def traffic_path(workload: str, kernel: str = "newton_iter") -> Path:
    return PROFILES / f"{kernel}_{workload}_traffic.json"


def valu_path(workload: str, kernel: str = "newton_fused") -> Path:
    return PROFILES / f"{kernel}_{workload}_valu.json"


def load_profile(path: Path, digest: str):
    if not path.exists():
        return None
    try:
        d = json.loads(path.read_text())
    except ValueError:
        return None
    return d if d.get("source_digest") == digest else None


def load_traffic(workload: str, digest: str, kernel: str = "newton_iter"):
    """Counter-measured HBM bytes per launch for the current kernel sources, if profiled."""
    d = load_profile(traffic_path(workload, kernel), digest)
    return None if d is None else d.get("bytes_per_launch")


def _counter_rows(path, counter):
    import csv

    rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    return rows


PMC_PREFIX = "rocprofv3 --pmc {counters} --output-format csv -d <out> -o run -- python3 <repo>/bench.py --workload {w} "


def pmc_commands(workload: str, scan: bool) -> dict:
    """The rocprofv3 counter runs whose CSVs the summaries below convert, as
    run on the GPU machine (from /tmp with TMPDIR=/tmp), one run per counter set."""
    extra = "" if scan else " --no-ceilings"
    return {
        "FETCH_SIZE": PMC_PREFIX.format(counters="FETCH_SIZE", w=workload)
        + f"--steps 3 --warmup 1 --no-cpu-baseline{extra} --copy-calibration",
        "WRITE_SIZE": PMC_PREFIX.format(counters="WRITE_SIZE", w=workload)
        + f"--steps 3 --warmup 1 --no-cpu-baseline{extra} --copy-calibration",
        "SQ": PMC_PREFIX.format(counters=" ".join(SQ_PASS), w=workload)
        + "--steps 3 --warmup 1 --no-cpu-baseline --no-ceilings --no-per-iteration",
    }


def traffic_from_counters(workload: str, fetch_csv: str, write_csv: str, iters: int,
                          kernel: str = "newton_iter") -> dict:
    """Per-launch HBM bytes of one kernel from two rocprofv3 --pmc runs
    (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch) of `bench.py
    --copy-calibration`. Each counter is scaled by bytes / counter of the
    1 GiB device copy in the same run."""

    def read(path, counter):
        rows = _counter_rows(path, counter)
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
    return {"workload": workload, "kernel": f"{kernel}_kernel", "source_digest": source_digest(),
            "bytes_per_launch": mean, "per_launch": per_k, "fetch_scale": fscale, "write_scale": wscale,
            "calibration": "1 GiB hipMemcpy device copy (__amd_rocclr_copyBuffer) in the same run",
            "commands": [c for n, c in pmc_commands(workload, kernel in ("scan", "dense")).items() if n != "SQ"]}


# SQ counters of one --pmc pass: instruction counts are per wave (64 lanes).
VALU_COUNTERS = ("SQ_INSTS_VALU", "SQ_INSTS_VALU_TRANS_F32")
SQ_PASS = VALU_COUNTERS + ("SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY",
                           "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_ANY")


def valu_from_counters(workload: str, csv_path: str, elements: int, iters: int, trans_in_valu: bool,
                       kernel: str = "newton_fused") -> dict:
    """VALU issue slots per launch of one kernel from a rocprofv3 --pmc run with
    SQ_INSTS_VALU and SQ_INSTS_VALU_TRANS_F32 (wave instructions per
    dispatch): lane slots = 64 x (regular + TRANS_SLOTS x transcendental). The
    per-launch means of every other SQ counter of the pass are kept too.
    trans_in_valu says whether SQ_INSTS_VALU already counts the
    transcendentals (measured with the issue-rate probe's exp-only kernel)."""
    import csv

    names = sorted({r["Counter_Name"] for r in csv.DictReader(open(csv_path))})
    per = {}
    for c in names:
        vals = [float(r["Counter_Value"]) for r in _counter_rows(csv_path, c) if f"{kernel}_kernel" in r["Kernel_Name"]]
        if vals:
            per[c] = sum(vals) / len(vals)
    for c in VALU_COUNTERS:
        if c not in per:
            raise ValueError(f"no {c} rows for {kernel}_kernel in {csv_path}")
    trans = per["SQ_INSTS_VALU_TRANS_F32"]
    regular = per["SQ_INSTS_VALU"] - (trans if trans_in_valu else 0.0)
    slots = 64.0 * (regular + TRANS_SLOTS * trans)
    return {"workload": workload, "kernel": f"{kernel}_kernel", "source_digest": source_digest(),
            "per_launch": per, "trans_in_valu": trans_in_valu, "elements": elements, "iterations": iters,
            "regular_per_element_iteration": 64.0 * regular / (elements * iters),
            "trans_per_element_iteration": 64.0 * trans / (elements * iters),
            "slots_per_launch": slots, "slots_per_element_iteration": slots / (elements * iters),
            "slot_rule": f"64 lanes x (regular VALU + {TRANS_SLOTS} x transcendental) wave instructions",
            "command": pmc_commands(workload, False)["SQ"]}


def write_stats_summary(workload: str, stats_csv: str, command: str) -> str:
    """profiles/<workload>_kernel_stats.md from rocprofv3 --kernel-trace --stats output."""
    import csv

    rows = list(csv.DictReader(open(stats_csv)))
    lines = [f"# rocprofv3 kernel statistics: {workload}", "",
             "Command (on the MI355X box, from /tmp with TMPDIR=/tmp):", "", f"    {command}", "",
             f"Kernel sources digest: {source_digest()} (bench.py source_digest()).", "",
             "| kernel | calls | average ns | min ns | max ns | % time |", "|---|---|---|---|---|---|"]
    for r in rows:
        lines.append(f"| `{r['Name'][:110]}` | {r['Calls']} | {float(r['AverageNs']):.0f} | {r['MinNs']} | "
                     f"{r['MaxNs']} | {float(r['Percentage']):.2f} |")
    text = "\n".join(lines) + "\n"
    (PROFILES / f"{workload}_kernel_stats.md").write_text(text)
    return text


# ---------------------------------------------------------------------------
# Same-run device ceilings: a device-to-device copy through torch, the
# streaming bandwidth and the VALU issue rates of the measurement kernels
# (ceilings.hip).

def _ceil_lib():
    from nonlinear_rnn_solve_newton_amd import build

    if not build.CEIL_LIB.exists():
        return None
    L = ctypes.CDLL(str(build.CEIL_LIB))
    L.ceil_issue_launch.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float, ctypes.c_float,
                                    ctypes.c_void_p, ctypes.c_void_p]
    L.ceil_stream_launch.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_longlong, ctypes.POINTER(ctypes.c_void_p),
                                     ctypes.POINTER(ctypes.c_void_p), ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    return L


def device_ceilings(dev, hip):
    import torch

    out = {}
    src = torch.empty(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s.record()
    for _ in range(5):
        dst.copy_(src)
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / 5
    gbs = 2 * src.numel() * 4 / (ms * 1e-3) / 1e9
    out["device_copy"] = {"gbs": gbs, "frac": gbs / PEAK_HBM_GBS, "bytes": 2 * src.numel() * 4,
                          "what": "torch copy_ of 1 GiB, read + write bytes"}
    del src, dst
    L = _ceil_lib()
    if L is not None:
        out["streams"] = stream_rates(dev, hip, L)
        out["valu_issue"] = issue_rates(dev, hip, L)
    return out


def stream_rates(dev, hip, L, n16=1 << 24):
    """HBM bytes per second of the streaming kernels: 16-byte loads and
    stores over arrays of 256 MiB, read-only, write-only, copy and the
    adjoint's mix (5 arrays read, 4 written: 20 bytes read per 16 written),
    with nontemporal and with default-policy accesses, best of five launches."""
    import torch

    arrays = [torch.ones(n16 * 4, dtype=torch.float32, device=dev) for _ in range(9)]
    sink = torch.zeros(4, dtype=torch.float32, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    ev = hip.create(2)
    rec = hip.hip.hipEventRecord
    rec.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    res = {}
    for name, r, w, nt in [(f"{n}{'_nt' if nt else ''}", r, w, nt) for n, r, w in
                           (("read", 1, 0), ("write", 0, 1), ("copy", 1, 1), ("read5_write4", 5, 4))
                           for nt in (1, 0)]:
        pin = (ctypes.c_void_p * 5)(*[t.data_ptr() for t in arrays[:r]])
        pout = (ctypes.c_void_p * 4)(*[t.data_ptr() for t in arrays[5:5 + w]])
        best = None
        for _ in range(5):
            rec(ctypes.c_void_p(ev[0]), stream)
            if L.ceil_stream_launch(r, w, nt, n16, pin, pout, ctypes.c_void_p(sink.data_ptr()), 256 * 32, stream):
                raise RuntimeError("ceil_stream_launch failed")
            rec(ctypes.c_void_p(ev[1]), stream)
            t = hip.ms(ev[0], ev[1])
            best = t if best is None else min(best, t)
        gbs = n16 * 16 * (r + w) / (best * 1e-3) / 1e9
        res[name] = {"gbs": gbs, "frac": gbs / PEAK_HBM_GBS}
    hip.destroy(ev)
    del arrays
    return res


def issue_probe() -> int:
    """The issue-rate kernels once each, for a counter pass: 768 workgroups
    of 256 lanes (3 waves per SIMD on every SIMD), plain FMA chains (kind 0),
    v_exp_f32 chains (kind 1) and the sigmoid-shaped mix (kind 2)."""
    import torch

    L = _ceil_lib()
    if L is None:
        print(json.dumps({"error": "libceilings.so is not built"}))
        return 2
    dev = torch.device("cuda:0")
    blocks = 256 * 3
    buf = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    for kind, iters in ((0, 200), (1, 100), (2, 100)):
        if L.ceil_issue_launch(kind, blocks, iters, 0.999, 1e-3, ctypes.c_void_p(buf.data_ptr()), stream):
            raise RuntimeError("ceil_issue_launch failed")
        torch.cuda.synchronize()
        print(json.dumps({"kind": kind, "lanes": blocks * 256, "steps_per_lane": iters * L.ceil_issue_steps_per_trip()}),
              flush=True)
    return 0


def issue_rates(dev, hip, L, waves_per_simd=(1, 2, 3, 8)):
    """Lane operations per second of the issue-rate kernels, per waves per
    SIMD (all 256 CUs x 4 SIMDs filled): plain fp32 FMA, v_exp_f32, and the
    sigmoid-shaped mix, the last also in issue slots (transcendentals at
    TRANS_SLOTS) against the issue peak."""
    import torch

    steps = L.ceil_issue_steps_per_trip()
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    ev = hip.create(2)
    rec = hip.hip.hipEventRecord
    rec.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    res = {}
    for wps in waves_per_simd:
        blocks = 256 * wps  # 4 waves per block: one per SIMD
        buf = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
        row = {}
        for kind, name, iters, per_step in ((0, "fma", 2000, 1), (1, "exp", 500, 1), (2, "sigmoid_mix", 400, 4)):
            L.ceil_issue_launch(kind, blocks, 10, 0.999, 1e-3, ctypes.c_void_p(buf.data_ptr()), stream)
            rec(ctypes.c_void_p(ev[0]), stream)
            if L.ceil_issue_launch(kind, blocks, iters, 0.999, 1e-3, ctypes.c_void_p(buf.data_ptr()), stream):
                raise RuntimeError("ceil_issue_launch failed")
            rec(ctypes.c_void_p(ev[1]), stream)
            t = hip.ms(ev[0], ev[1]) * 1e-3
            lane_steps = blocks * 256.0 * iters * steps
            row[name] = {"lane_ops_per_s": lane_steps * per_step / t,
                         "per_clock_per_cu_at_2p4GHz": lane_steps * per_step / t / (256 * 2.4e9)}
            if kind == 2:  # 2 regular + 2 transcendental instructions per step
                row[name]["slots_per_s"] = lane_steps * (2 + 2 * TRANS_SLOTS) / t
                row[name]["slot_frac_of_peak"] = row[name]["slots_per_s"] / (PEAK_VALU_TSLOTS * 1e12)
        res[f"{wps}_waves_per_simd"] = row
    hip.destroy(ev)
    return res


# ---------------------------------------------------------------------------
# CPU baseline: the fp64 oracle as it stands, on a channel sample.

def cpu_baseline(w, x, iters, target_s=15.0, single_s=3.0):
    """The fp64 oracle on a sample of channels (b, d) of the same workload, full
    L: its Newton solve (K iterations) and, for the adjoint workload, its BPTT
    along that solve; plus the sequential recurrence, and a one-thread run."""
    from nonlinear_rnn_solve_newton_amd.workloads import gather_channels, sample_channels
    from oracle import oracle as O

    nthreads = O.default_threads()
    BD = w.B * w.D

    def run(n, threads):
        ch = sample_channels(w.B, w.D, n, seed=99)
        u = gather_channels(x.u, ch, w.D)
        a = x.a[:, ch % w.D].contiguous()
        t0 = time.perf_counter()
        S, _ = O.newton(w.cell, u, a, K=iters, nthreads=threads)
        t1 = time.perf_counter()
        if w.adjoint:
            O.adjoint(w.cell, u, a, S, gather_channels(x.dh, ch, w.D), nthreads=threads)
        t2 = time.perf_counter()
        O.seq(w.cell, u, a, nthreads=threads)
        t3 = time.perf_counter()
        return len(ch), t1 - t0, t2 - t1, t3 - t2

    def scaled(threads, target):
        # grow the sample until it takes at least half the target time (or is
        # the whole workload): a small first sample overstates the per-channel
        # cost (thread start-up), so one extrapolation falls short
        n = min(BD, max(threads, 16))
        while True:
            res = run(n, threads)
            t = res[1] + res[2]
            if n >= BD or t >= 0.5 * target:
                return res
            m = int(min(BD, max(2 * n, n * target / max(t, 1e-9))))
            n = max(threads, m - m % max(threads, 1)) if m < BD else m

    n, tn, ta, ts = scaled(nthreads, target_s)
    elems = n * w.L
    what = f"{iters} fp64 Newton iterations" + (" + BPTT along them" if w.adjoint else "")
    res = {"value": elems / (tn + ta), "unit": "elems/s", "cores": nthreads, "kind": "oracle",
           "sample": f"{n} of {BD} channels (b, d) over the full L={w.L}, {what}; {tn + ta:.2f} s",
           "newton_value": elems / tn, "sequential_value": elems / ts}
    if w.adjoint:
        res["adjoint_value"] = elems / ta
    n1, tn1, ta1, ts1 = scaled(1, single_s)
    res["single_thread"] = {"value": n1 * w.L / (tn1 + ta1), "cores": 1,
                            "sample": f"{n1} channels over the full L={w.L}, {what}; {tn1 + ta1:.2f} s",
                            "sequential_value": n1 * w.L / ts1}
    return res


# ---------------------------------------------------------------------------
# The linear scan alone and the dense recurrence (the scan tier).

def scan_bytes(ns: int) -> int:
    """read NS*NS coefficient planes and NS input planes, write NS state planes, fp32"""
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


def timed_steps(step, steps, warmup):
    """warm-up, then exactly `steps` steps between two synchronisations (ms per
    step from events on the stream the launches go to), then the same number
    of steps each bracketed by events, for the median and minimum"""
    import torch

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        step()
    stop.record()
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(stop) / steps
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    evs[0].record()
    for i in range(steps):
        step()
        evs[i + 1].record()
    torch.cuda.synchronize()
    return ms_step, stats([evs[i].elapsed_time(evs[i + 1]) for i in range(steps)])


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
    step = lambda: binding.scan_dense(A, b, s0, out=out, ws=ws)  # noqa: E731
    ms_step, step_stats = timed_steps(step, args.steps, args.warmup)
    kms = []
    for _ in range(args.steps):
        binding.scan_dense(A, b, s0, out=out, ws=ws, events=ev)
        kms.append(hip.ms(ev[1], ev[2]))
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
                     "algorithmic_bytes_per_launch": nbytes, "launch_ms": stats(kms)},
        "matrix_cores": {"achieved": flops / (t * 1e-3) / 1e12, "peak": PEAK_F32_MATRIX_TFLOPS,
                         "unit": "TFLOP/s", "frac": flops / (t * 1e-3) / 1e12 / PEAK_F32_MATRIX_TFLOPS},
        "timing": {"step_ms": step_stats, "scan_ms": stats(kms), "source_digest": source_digest()},
    }
    if args.copy_calibration:
        copy_calibration(dev)
        result["copy_calibration_bytes"] = 1 << 30
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


def copy_calibration(dev):
    """A plain 1 GiB device copy (hipMemcpy's copy kernel), whose counters scale
    the FETCH_SIZE / WRITE_SIZE readings of the same run."""
    import torch

    src = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()


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
    step = lambda: binding.scan(A, b, s0, out=out, ws=ws)  # noqa: E731
    ms_step, step_stats = timed_steps(step, args.steps, args.warmup)
    scan_ms, clear_ms = [], []
    for _ in range(args.steps):
        binding.scan(A, b, s0, out=out, ws=ws, events=ev)
        clear_ms.append(hip.ms(ev[0], ev[1]))
        scan_ms.append(hip.ms(ev[1], ev[2]))
    kms = sum(scan_ms) / len(scan_ms)
    nbytes = scan_bytes(w.ns) * w.N
    achieved = nbytes / (kms * 1e-3) / 1e9
    digest = source_digest()
    result = {
        "metric": "scanned state elems/s (B*L*D) of the linear scan s_l = A_l s_{l-1} + b_l",
        "value": w.N / (ms_step * 1e-3), "unit": "elems/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (seeded; A ~ U(-0.95, 0.95) per block row sum, b, s0 ~ N(0,1))",
        "config": {"workload": w.name, "block": "diag" if w.ns == 1 else "2x2", "B": w.B, "L": w.L, "D": w.D},
        "roofline": {"bound": "hbm", "kernel": "scan_kernel", "achieved": achieved, "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS,
                     "traffic": load_traffic(w.name, digest, "scan"),
                     "algorithmic_bytes_per_launch": nbytes, "launch_ms": stats(scan_ms)},
        # reset: from the marker before the workspace reset to the scan's start
        "timing": {"step_ms": step_stats, "reset_to_launch_ms": stats(clear_ms), "source_digest": digest},
    }
    if args.copy_calibration:
        copy_calibration(dev)
        result["copy_calibration_bytes"] = 1 << 30
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
    ms, st = timed_steps(run, args.steps, args.warmup)
    print(json.dumps({
        "metric": "solved state elems/s (B*L*D) per 3-Newton solve, generic-cell tier",
        "value": w.N / (ms * 1e-3), "unit": "elems/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic (same inputs as the fused workload)",
        "config": {"workload": w.name, "tier": "generic: torch cell, torch.func.jvp Jacobian, "
                   "pararnn_scan_diag / pararnn_scan_block2 per iteration"},
        "timing": {"step_ms": st},
    }), flush=True)
    return 0


# ---------------------------------------------------------------------------
# The Newton solve (and adjoint) workloads.

def kernel_record(name, bound, ms, work, unit, peak, traffic=None, **extra):
    """One kernel's roofline: `work` algorithmic units (bytes or issue slots)
    per launch over its mean launch duration."""
    if work is None:
        achieved = None
    elif unit == "GB/s":
        achieved = work / (ms["mean"] * 1e-3) / 1e9
    else:
        achieved = work / (ms["mean"] * 1e-3) / 1e12
    rec = {"bound": bound, "kernel": name, "achieved": achieved, "peak": peak, "unit": unit,
           "frac": None if achieved is None else achieved / peak, "traffic": traffic, "launch_ms": ms}
    rec.update(extra)
    return rec


def bench_solve(w, args):
    import torch

    from nonlinear_rnn_solve_newton_amd import binding
    from nonlinear_rnn_solve_newton_amd.workloads import workload_inputs

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

    def time_schedule(schedule):
        """One schedule of the solve (plus the adjoint for the adjoint
        workload): step times without events, then per-kernel durations
        stamped by the launches' own dispatches."""
        first = binding.solve(w.cell, u, a, iters=K, schedule=schedule)
        ws, out = first["ws"], {k: first[k] for k in ("h", "c") if k in first}
        gadj = binding.adjoint(w.cell, u, a, out["h"], dh, c=out.get("c")) if w.adjoint else None

        def step(events=None, events_adj=None):
            binding.solve(w.cell, u, a, iters=K, ws=ws, out=out, events=events, schedule=schedule)
            if w.adjoint:
                binding.adjoint(w.cell, u, a, out["h"], dh, c=out.get("c"), ws=gadj["ws"], du=gadj["du"],
                                events=events_adj)

        def kernel_times():
            launch_ms = [[] for _ in range(K)]
            clear_ms, adj_ms = [], []
            for _ in range(args.steps):
                step(ev, ev_adj)
                # event 1: the first launch's start; k + 1: the end of
                # iteration k's launch (for the fused schedule its one launch,
                # then markers right after it)
                clear_ms.append(hip.ms(ev[0], ev[1]))
                for k in range(K):
                    launch_ms[k].append(hip.ms(ev[k + 1], ev[k + 2]))
                if w.adjoint:
                    adj_ms.append(hip.ms(ev_adj[1], ev_adj[2]))
            return launch_ms, clear_ms, adj_ms

        # the per-kernel timing runs once before the timed steps, which lets
        # the clocks settle under this load (its figures are not used), and
        # once after them for the reported kernel durations
        kernel_times()
        ms_step, step_stats = timed_steps(step, args.steps, args.warmup)
        launch_ms, clear_ms, adj_ms = kernel_times()
        return {"ms_step": ms_step, "step": step_stats, "clear_ms": stats(clear_ms),
                "launch_ms": [stats(v) for v in launch_ms], "adj_ms": stats(adj_ms) if adj_ms else None,
                "out": out, "gadj": gadj}

    N = w.N
    digest = source_digest()
    fused = time_schedule("fused")
    per_it = time_schedule("per_iteration") if not args.no_per_iteration else None
    out = fused["out"]

    # the fused launch: bound by vector-ALU issue; its work is the VALU issue
    # slots rocprofv3 counted for these sources, and its own HBM bytes (gate
    # inputs once, final iterate once)
    t_fused = fused["launch_ms"][0]
    valu = load_profile(valu_path(w.name), digest)
    fb = fused_bytes(w.cell, u_bytes) * N
    fused_rec = kernel_record(
        "newton_fused_kernel", "alu", t_fused, None if valu is None else valu["slots_per_launch"],
        "T VALU issue slots/s", PEAK_VALU_TSLOTS, load_traffic(w.name, digest, "newton_fused"),
        valu_counters=None if valu is None else str(valu_path(w.name).relative_to(ROOT)),
        slots_per_element_iteration=None if valu is None else valu["slots_per_element_iteration"],
        hbm_own={"bytes_per_launch": fb, "achieved": fb / (t_fused["mean"] * 1e-3) / 1e9, "peak": PEAK_HBM_GBS,
                 "unit": "GB/s", "frac": fb / (t_fused["mean"] * 1e-3) / 1e9 / PEAK_HBM_GBS})
    kernels = [fused_rec]
    if w.adjoint:
        ab = adjoint_bytes(w.cell, u_bytes) * N
        kernels.append(kernel_record("adjoint_kernel", "hbm", fused["adj_ms"], ab, "GB/s", PEAK_HBM_GBS,
                                     load_traffic(w.name, digest, "adjoint"), algorithmic_bytes_per_launch=ab))
    dominant = max(kernels, key=lambda r: r["launch_ms"]["mean"])
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
        "data": "synthetic (seeded; u ~ N(0,1) stored " + w.u_dtype + ", a ~ U(-amax, amax)"
                + (", dL/dh ~ N(0,1)" if w.adjoint else "") + ")",
        "config": {"workload": w.name, "cell": w.cell, "B": w.B, "L": w.L, "D": w.D, "newton_iters": K,
                   "u_dtype": w.u_dtype, "adjoint": w.adjoint, "schedule": "fused"},
        "roofline": dominant,
        "kernels": kernels,
        "timing": {
            "step_ms": fused["step"],
            # from the marker before the workspace reset to the fused launch's
            # start: the reset kernel and both dispatches
            "reset_to_launch_ms": fused["clear_ms"],
            "source_digest": digest,
        },
    }
    if per_it is not None:
        bytes_k = [iter_bytes(w.cell, u_bytes, k + 1) * N for k in range(K)]
        t_it = [s["mean"] for s in per_it["launch_ms"]]
        hbm_it = sum(bytes_k) / (sum(t_it) * 1e-3) / 1e9
        result["per_iteration_schedule"] = {
            "ms_per_step": per_it["ms_step"], "step_ms": per_it["step"],
            "roofline": {"bound": "hbm", "kernel": "newton_iter_kernel", "achieved": hbm_it, "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": hbm_it / PEAK_HBM_GBS, "traffic": load_traffic(w.name, digest),
                         "algorithmic_bytes_per_launch": bytes_k, "launch_ms": per_it["launch_ms"]},
        }
    if w.adjoint:
        # the same adjoint with the parameter and initial-state gradients
        # (da, ds0) requested: their partials ride in the reverse scan, plus a
        # fixed-order reduction launch
        gfull = binding.adjoint(w.cell, u, a, out["h"], dh, c=out.get("c"), want_ds0=True, want_da=True)
        grad_ms = []
        for _ in range(args.steps):
            binding.adjoint(w.cell, u, a, out["h"], dh, c=out.get("c"), ws=gfull["ws"], du=gfull["du"],
                            want_ds0=True, want_da=True, events=ev_adj)
            grad_ms.append(hip.ms(ev_adj[1], ev_adj[2]))
        torch.cuda.synchronize()
        result["timing"]["adjoint_with_da_ds0_ms"] = stats(grad_ms)
        del gfull
    if not args.no_ceilings:
        result["device_ceilings"] = device_ceilings(dev, hip)
    if args.copy_calibration:
        copy_calibration(dev)
        result["copy_calibration_bytes"] = 1 << 30
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, x, K)
    hip.destroy(ev + (ev_adj or []))
    print(json.dumps(result), flush=True)
    return 0


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-per-iteration", action="store_true", help="skip the per-iteration schedule")
    ap.add_argument("--no-ceilings", action="store_true", help="skip the same-run device ceilings")
    ap.add_argument("--generic", action="store_true",
                    help="run the workload's cell through the generic-cell tier (torch cell + forward-mode "
                         "AD Jacobian + the library's scan) instead of the fused kernels")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration for profiling)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/<kernel>_<workload>_traffic.json from rocprofv3 counter CSVs")
    ap.add_argument("--valu-from", metavar="SQ_CSV",
                    help="write profiles/newton_fused_<workload>_valu.json from a rocprofv3 --pmc CSV with "
                         "SQ_INSTS_VALU and SQ_INSTS_VALU_TRANS_F32")
    ap.add_argument("--trans-in-valu", choices=("yes", "no"), default="yes",
                    help="whether SQ_INSTS_VALU counts the transcendentals too (with --valu-from)")
    ap.add_argument("--stats-summary", metavar="KERNEL_STATS_CSV",
                    help="write profiles/<workload>_kernel_stats.md from a rocprofv3 --stats CSV")
    ap.add_argument("--stats-command", default=None, help="the rocprofv3 command, for --stats-summary")
    ap.add_argument("--issue-probe", action="store_true",
                    help="launch the VALU issue-rate kernels once each (for a counter pass) and exit")
    args = ap.parse_args(argv)
    if args.issue_probe:
        return issue_probe()
    sys.path.insert(0, str(ROOT))
    from nonlinear_rnn_solve_newton_amd.workloads import DENSE_WORKLOADS, HEADLINE, SCAN_WORKLOADS, WORKLOADS
    name = args.workload or HEADLINE
    if name not in WORKLOADS and name not in SCAN_WORKLOADS and name not in DENSE_WORKLOADS:
        print(json.dumps({"error": f"unknown workload {name}",
                          "workloads": sorted(WORKLOADS) + sorted(SCAN_WORKLOADS) + sorted(DENSE_WORKLOADS)}))
        return 2
    if args.stats_summary:
        cmd = args.stats_command or (
            "rocprofv3 --kernel-trace --stats --output-format csv -d <out> -o run -- "
            f"python3 <repo>/bench.py --workload {name} --steps 5 --warmup 2 --no-cpu-baseline --no-ceilings")
        print(write_stats_summary(name, args.stats_summary, cmd))
        return 0
    if args.valu_from:
        w = WORKLOADS[name]
        kernels = [("newton_fused", w.iters)] + ([("adjoint", 1)] if w.adjoint else [])
        for kern, iters in kernels:
            d = valu_from_counters(name, args.valu_from, w.N, iters, args.trans_in_valu == "yes", kernel=kern)
            valu_path(name, kern).write_text(json.dumps(d, indent=1) + "\n")
            print(json.dumps(d))
        return 0
    if args.traffic_from:
        if name in SCAN_WORKLOADS:
            d = traffic_from_counters(name, *args.traffic_from, iters=1, kernel="scan")
            traffic_path(name, "scan").write_text(json.dumps(d, indent=1) + "\n")
        elif name in DENSE_WORKLOADS:
            d = traffic_from_counters(name, *args.traffic_from, iters=1, kernel="dense")
            traffic_path(name, "dense").write_text(json.dumps(d, indent=1) + "\n")
        else:
            kernels = [("newton_iter", WORKLOADS[name].iters), ("newton_fused", 1)]
            if WORKLOADS[name].adjoint:
                kernels.append(("adjoint", 1))
            for kern, iters in kernels:
                d = traffic_from_counters(name, *args.traffic_from, iters=iters, kernel=kern)
                traffic_path(name, kern).write_text(json.dumps(d, indent=1) + "\n")
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
    return bench_solve(WORKLOADS[name], args)


if __name__ == "__main__":
    sys.exit(main())
