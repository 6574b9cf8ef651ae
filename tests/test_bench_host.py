"""Host logic of bench.py on the CPU: the per-launch HBM bytes built from
rocprofv3 counter CSVs (scaled by the calibration copy, grouped into calls),
and the refusal of more than one GPU."""
import csv
import json
import subprocess
import sys
from pathlib import Path

import bench

ROOT = Path(__file__).resolve().parents[1]
GIB = float(1 << 30)


def write_csv(path, counter, dispatches):
    """dispatches: (kernel name, counter value in KiB) in dispatch order"""
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, (name, kib) in enumerate(dispatches):
            w.writerow({"Dispatch_Id": i + 1, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": kib})


def calibration(counter_kib):
    return [("__amd_rocclr_copyBuffer", 0.0), ("__amd_rocclr_copyBuffer", counter_kib)]


def test_dense_traffic_sums_each_scan(tmp_path):
    """A scan is every dense launch from one transfer launch to the next,
    whatever their number; other kernels in between are not counted."""
    scan_f = [("void pararnn::dense_chunk_kernel<true>(pararnn::DenseArgs)", 10.0),
              ("pararnn::dense_carry_kernel(pararnn::DenseArgs)", 1.0),
              ("pararnn::ws_clear_kernel(...)", 99.0),
              ("void pararnn::dense_apply_kernel<true>(pararnn::DenseArgs)", 20.0)]
    scan_w = [(n, v) for n, v in zip([d[0] for d in scan_f], [5.0, 0.0, 77.0, 2.0])]
    # FETCH_SIZE reads half of the copy's bytes, WRITE_SIZE all of them
    write_csv(tmp_path / "f.csv", "FETCH_SIZE", calibration(GIB / 2 / 1024) + scan_f * 2)
    write_csv(tmp_path / "w.csv", "WRITE_SIZE", calibration(GIB / 1024) + scan_w * 2)
    d = bench.traffic_from_counters("dense_case", str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), 1,
                                    kernel="dense")
    assert d["fetch_scale"] == 2.0 and d["write_scale"] == 1.0
    assert d["per_launch"] == [{"fetch": 31 * 1024 * 2.0, "write": 7 * 1024 * 1.0}]
    assert d["bytes_per_launch"] == 31 * 2048 + 7 * 1024


def test_iteration_traffic_averages_each_launch_index(tmp_path):
    """Per-iteration launches come in solves of K; launch k is averaged over
    the solves, and bytes_per_launch is the mean over k."""
    name = "void pararnn::newton_iter_kernel<...>(pararnn::IterArgs)"
    f = [(name, v) for v in (1.0, 2.0, 3.0, 3.0, 4.0, 5.0)]
    w = [(name, v) for v in (6.0, 6.0, 6.0, 8.0, 8.0, 8.0)]
    write_csv(tmp_path / "f.csv", "FETCH_SIZE", calibration(GIB / 1024) + f)
    write_csv(tmp_path / "w.csv", "WRITE_SIZE", calibration(GIB / 1024) + w)
    d = bench.traffic_from_counters("iter_case", str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), 3)
    assert [x["fetch"] for x in d["per_launch"]] == [2048.0, 3072.0, 4096.0]
    assert [x["write"] for x in d["per_launch"]] == [7168.0] * 3
    assert d["bytes_per_launch"] == 3072.0 + 7168.0


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       cwd=ROOT, timeout=300)
    assert r.returncode != 0
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert msg["n_gpus"] == 2 and "one GPU" in msg["error"]


def test_adjoint_traffic_uses_its_own_launches(tmp_path):
    """The adjoint's bytes come from its own dispatches, not the solve's."""
    adj = "void pararnn::adjoint_kernel<...>(pararnn::AdjArgs)"
    fused = "void pararnn::newton_fused_kernel<...>(pararnn::FusedArgs)"
    f = [(fused, 100.0), (adj, 10.0), (fused, 100.0), (adj, 14.0)]
    w = [(fused, 50.0), (adj, 4.0), (fused, 50.0), (adj, 6.0)]
    write_csv(tmp_path / "f.csv", "FETCH_SIZE", calibration(GIB / 2 / 1024) + f)
    write_csv(tmp_path / "w.csv", "WRITE_SIZE", calibration(GIB / 1024) + w)
    d = bench.traffic_from_counters("adj_case", str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), 1,
                                    kernel="adjoint")
    assert d["per_launch"] == [{"fetch": 12 * 1024 * 2.0, "write": 5 * 1024 * 1.0}]
    assert d["kernel"] == "adjoint_kernel"


def test_valu_slots_from_counters(tmp_path):
    """Issue slots = 64 lanes x (regular + TRANS_SLOTS x transcendental) wave
    instructions, with the transcendentals taken out of SQ_INSTS_VALU when
    that counter includes them."""
    name = "void pararnn::newton_fused_kernel<...>(pararnn::FusedArgs)"
    with open(tmp_path / "v.csv", "w", newline="") as fh:
        wr = csv.DictWriter(fh, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        wr.writeheader()
        for i, (c, v) in enumerate([("SQ_INSTS_VALU", 1000.0), ("SQ_INSTS_VALU_TRANS_F32", 100.0),
                                    ("SQ_INSTS_VALU", 1200.0), ("SQ_INSTS_VALU_TRANS_F32", 100.0)]):
            wr.writerow({"Dispatch_Id": i // 2 + 1, "Kernel_Name": name, "Counter_Name": c, "Counter_Value": v})
    d = bench.valu_from_counters("v_case", str(tmp_path / "v.csv"), elements=64, iters=2, trans_in_valu=True)
    assert d["per_launch"] == {"SQ_INSTS_VALU": 1100.0, "SQ_INSTS_VALU_TRANS_F32": 100.0}
    T = bench.TRANS_SLOTS
    assert d["slots_per_launch"] == 64.0 * (1000.0 + T * 100.0)
    assert d["slots_per_element_iteration"] == 64.0 * (1000.0 + T * 100.0) / 128
    d2 = bench.valu_from_counters("v_case", str(tmp_path / "v.csv"), elements=64, iters=2, trans_in_valu=False)
    assert d2["slots_per_launch"] == 64.0 * (1100.0 + T * 100.0)


def test_kernel_record_fraction():
    ms = bench.stats([2.0, 1.0, 3.0])
    assert ms["mean"] == 2.0 and ms["median"] == 2.0 and ms["min"] == 1.0
    r = bench.kernel_record("k", "hbm", ms, 8e9, "GB/s", 8000.0)
    assert abs(r["achieved"] - 4000.0) < 1e-9 and abs(r["frac"] - 0.5) < 1e-12
    r = bench.kernel_record("k", "alu", ms, None, "T VALU issue slots/s", 78.65)
    assert r["achieved"] is None and r["frac"] is None
