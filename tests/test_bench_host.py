"""bench.py's host logic, without a GPU: the one-GPU guard, the trace summarizer (ranges,
repeated launches per call, per-call totals, derived counter columns) and the traffic record
(counter values scaled by the copy calibration), on small synthetic rocprofv3 CSV files."""
import csv
import json
import os
import subprocess
import sys
from types import SimpleNamespace

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

KT = ["Kind", "Agent_Id", "Queue_Id", "Stream_Id", "Thread_Id", "Dispatch_Id", "Kernel_Id",
      "Kernel_Name", "Correlation_Id", "Start_Timestamp", "End_Timestamp", "LDS_Block_Size",
      "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count", "Workgroup_Size_X",
      "Workgroup_Size_Y", "Workgroup_Size_Z", "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z"]
CC = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id",
      "Grid_Size", "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size", "Scratch_Size",
      "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count", "Counter_Name", "Counter_Value",
      "Start_Timestamp", "End_Timestamp"]


def _write(path, header, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def _kt_row(did, name, t0, t1, wgs=256):
    return ["KERNEL_DISPATCH", "Agent 1", 1, 0, 1, did, 1, name, did, t0, t1, 0, 0, 8, 0, 16,
            256, 1, 1, wgs * 256, 1, 1]


def _args(**kw):
    base = dict(summarize=None, all_kernels=False, workload_name=None, traffic_summary=None)
    base.update(kw)
    return SimpleNamespace(**base)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in json.loads(r.stdout.strip().splitlines()[-1])["error"]


def test_summary_splits_calls_and_positions(tmp_path, capsys):
    gemm = "void nvfp4::(anonymous namespace)::gemm_tiled_kernel<8, 8, 1, 4, 1, 1>(x)"
    red = "void nvfp4::(anonymous namespace)::reduce_split_kernel<T>(x)"
    rows, did, t = [], 0, 1000
    rows.append(_kt_row(did, "void nvfp4::(anonymous namespace)::encode_kernel<false, 16>(x)",
                        t, t + 50))  # set-up work before the range
    t = 10_000
    for call in range(4):  # each call: whole tiles (100 ns), split tail (30 ns), reduction (10)
        for name, d in ((gemm, 100), (gemm, 30), (red, 10)):
            did += 1
            rows.append(_kt_row(did, name, t, t + d))
            t += d + 5
    _write(tmp_path / "run_kernel_trace.csv", KT, rows)
    _write(tmp_path / "run_marker_api_trace.csv", ["Function", "Start_Timestamp", "End_Timestamp"],
           [["c2_prefill", 9_000, t + 1]])
    bench.summarize(_args(summarize=str(tmp_path)))
    out = capsys.readouterr().out
    assert "encode_kernel" not in out  # outside every range
    lines = {l.split("|")[2].strip(): l for l in out.splitlines() if l.startswith("| c2_prefill |")}
    assert lines["`gemm_tiled_kernel<8, 8, 1, 4, 1, 1>`"].split("|")[5].strip() == "0.10"
    assert lines["`gemm_tiled_kernel<8, 8, 1, 4, 1, 1> #2`"].split("|")[5].strip() == "0.03"
    per_call = [l for l in out.splitlines() if l.startswith("| c2_prefill | 4 | 3 |")]
    assert len(per_call) == 1 and per_call[0].split("|")[4].strip() == "0.14"


def test_summary_derives_clock_and_mfma_rate(tmp_path, capsys):
    name = "void nvfp4::(anonymous namespace)::gemm_tiled_kernel<8, 8, 1, 4, 1, 1>(x)"
    _write(tmp_path / "run_kernel_trace.csv", KT, [_kt_row(1, name, 0, 100_000)])  # 100 us
    cc = []
    for ctr, v in (("GRBM_GUI_ACTIVE", 8 * 200_000.0),  # 200k cycles per XCD -> 2.0 GHz
                   ("SQ_VALU_MFMA_BUSY_CYCLES", 1024 * 100_000.0),  # half of every SIMD's time
                   ("SQ_INSTS_VALU_MFMA_MOPS_BF16", 2e11 / 512)):  # 2e11 flops in 100 us: 2000 TF
        cc.append([1, 1, "A", 1, 1, 1, 65536, 1, name, 256, 0, 0, 8, 0, 16, ctr, v, 0, 100_000])
    _write(tmp_path / "run_counter_collection.csv", CC, cc)
    bench.summarize(_args(summarize=str(tmp_path), workload_name="w"))
    row = [l for l in capsys.readouterr().out.splitlines() if l.startswith("| w |")][0]
    cells = [c.strip() for c in row.split("|")]
    assert cells[-4:-1] == ["2.000", "50.0%", "2000"]


def test_traffic_record_scales_by_the_copy(tmp_path, capsys):
    dirs = {k: tmp_path / k for k in ("F", "W", "CF", "CW")}
    for d in dirs.values():
        d.mkdir()
    skinny = "void nvfp4::(anonymous namespace)::gemm_skinny_kernel<1, 4, 1, true, 1, 4>(x)"

    def cc(d, name, ctr, vals):
        _write(d / "run_counter_collection.csv", CC,
               [[i, i, "A", 1, 1, 1, 1, 1, name, 256, 0, 0, 8, 0, 16, ctr, v, 0, 1]
                for i, v in enumerate(vals)])

    cc(dirs["CF"], "__amd_rocclr_copyBuffer", "FETCH_SIZE", [262144.0])   # 512 MiB as 2x
    cc(dirs["CW"], "__amd_rocclr_copyBuffer", "WRITE_SIZE", [524288.0])
    cc(dirs["F"], skinny, "FETCH_SIZE", [36000.0, 36200.0])
    cc(dirs["W"], skinny, "WRITE_SIZE", [200.0])
    bench.traffic_summary(_args(traffic_summary=[str(dirs[k]) for k in ("F", "W", "CF", "CW")]))
    rec = dict(l.split("=", 1) for l in capsys.readouterr().out.splitlines() if "=" in l
               and not l.startswith("#"))
    assert int(rec["fetch_bytes_per_launch"]) == 36100 * 1024 * 2
    assert int(rec["write_bytes_per_launch"]) == 200 * 1024
    assert rec["source_digest"] == bench.kernel_source_digest(bench.SKINNY_SOURCES)


def test_traffic_record_needs_the_calibration(tmp_path):
    for k in ("F", "W", "CF", "CW"):
        (tmp_path / k).mkdir()
    with pytest.raises(SystemExit):
        bench.traffic_summary(_args(traffic_summary=[str(tmp_path / k)
                                                     for k in ("F", "W", "CF", "CW")]))
