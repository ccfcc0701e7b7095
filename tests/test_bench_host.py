"""Host logic of bench.py (no GPU): the rocprofv3 trace and counter summaries
that the profiles are made from, and the algorithmic work of the workloads."""
import csv

import pytest

import bench
from workloads import WORKLOADS


def _write(path, fields, rows):
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=fields)
        w.writeheader()
        w.writerows(rows)


def test_trace_summary_takes_the_flushed_and_back_to_back_dispatches(tmp_path, capsys):
    # two workloads separated by a 2 s gap; the first runs 5 untimed launches
    # of 100 us, then 3 flushed ones of 50 us (each after a flush fill kernel),
    # then 3 back-to-back ones of 40 us
    rows, t = [], 0
    for dur in [100] * 5:
        rows.append({"Kernel_Name": "attn_fwd_kernelA", "Start_Timestamp": t,
                     "End_Timestamp": t + dur * 1000})
        t += 200_000
    for dur in [50, 52, 48]:
        rows.append({"Kernel_Name": "void at::native::fill", "Start_Timestamp": t,
                     "End_Timestamp": t + 90_000})
        t += 100_000
        rows.append({"Kernel_Name": "attn_fwd_kernelA", "Start_Timestamp": t,
                     "End_Timestamp": t + dur * 1000})
        t += 200_000
    for dur in [40] * 3:
        rows.append({"Kernel_Name": "attn_fwd_kernelA", "Start_Timestamp": t,
                     "End_Timestamp": t + dur * 1000})
        t += 200_000
    t += 2_000_000_000
    for dur in [7, 7, 9, 9, 9, 9, 9]:
        for k in ("attnB", "combine"):
            rows.append({"Kernel_Name": k, "Start_Timestamp": t, "End_Timestamp": t + dur * 1000})
            t += 50_000
    p = tmp_path / "trace.csv"
    _write(p, ["Kernel_Name", "Start_Timestamp", "End_Timestamp"], rows)
    bench.trace_summary(str(p), 3, ["first", "second"])
    out = capsys.readouterr().out.splitlines()
    body = [ln for ln in out if ln.startswith("| first") or ln.startswith("| second")]
    assert len(body) == 6  # the flush fill kernel is left out
    assert "`attn_fwd_kernelA` | flushed | 3 | 50.00 | 50.00 | 48.00 | 52.00" in body[0]
    assert "`attn_fwd_kernelA` | back-to-back | 3 | 40.00 | 40.00 | 40.00 | 40.00" in body[1]
    assert "`attnB` | flushed | 3 | 8.33 |" in body[2] and "`attnB` | back-to-back | 3 | 9.00 |" in body[3]
    assert "`combine` | back-to-back | 3 | 9.00 |" in body[5]
    machine = [ln for ln in out if ln.startswith("trace_kernel_us_back_to_back")]
    assert len(machine) == 1 and machine[0].split()[1:3] == ["first", "40.000"]


def test_traffic_summary_scales_by_the_copy_calibration(tmp_path, capsys):
    fields = ["Kernel_Name", "Counter_Value"]
    # a 1 MiB copy read as 512 KiB by FETCH_SIZE and 1024 KiB by WRITE_SIZE
    _write(tmp_path / "cf.csv", fields, [{"Kernel_Name": "__amd_copy", "Counter_Value": 512}])
    _write(tmp_path / "cw.csv", fields, [{"Kernel_Name": "__amd_copy", "Counter_Value": 1024}])
    _write(tmp_path / "f.csv", fields, [
        {"Kernel_Name": "void fmha::attn_fwd_kernel<64>(p)", "Counter_Value": 1000},
        {"Kernel_Name": "void fmha::attn_fwd_kernel<64>(p)", "Counter_Value": 3000},
        {"Kernel_Name": "void at::native::fill(x)", "Counter_Value": 5}])
    _write(tmp_path / "w.csv", fields, [
        {"Kernel_Name": "void fmha::attn_fwd_kernel<64>(p)", "Counter_Value": 10}])
    w = WORKLOADS["decode_gqa_d64"]
    bench.traffic_summary(w, str(tmp_path / "f.csv"), str(tmp_path / "w.csv"),
                          str(tmp_path / "cf.csv"), str(tmp_path / "cw.csv"), calib_mib=1)
    out = capsys.readouterr().out
    # mean FETCH 2000 KiB x 2 (scale) + WRITE 10 KiB x 1
    line = [ln for ln in out.splitlines() if ln.startswith("traffic_bytes_per_launch")][0]
    assert line.split()[1] == w.name and int(line.split()[2]) == 2000 * 1024 * 2 + 10 * 1024
    assert "at::native" not in out


@pytest.mark.parametrize("name,flops,nbytes", [
    # 4 * B * Hq * D * visible pairs; Q, K, V read once, O and LSE written once
    ("single_tile_d16", 4 * 16 * 128 * 128, 2 * (3 * 128 * 16 + 128 * 16) + 4 * 128),
    ("decode_gqa_d64", 4 * 64 * 32 * 64 * 8192,
     2 * (64 * 32 * 64 + 2 * 64 * 8 * 8192 * 64 + 64 * 32 * 64) + 4 * 64 * 32),
    ("decode_mqa_d576_dv512_v_in_k", 2 * (576 + 512) * 32 * 64 * 16384,
     2 * (32 * 64 * 576 + 32 * 16384 * 576 + 32 * 64 * 512) + 4 * 32 * 64),
])
def test_workload_algorithmic_counts(name, flops, nbytes):
    w = WORKLOADS[name]
    assert w.flops() == flops and w.bytes() == nbytes


def test_counter_summary_derived_metrics(tmp_path, capsys):
    _write(tmp_path / "agent.csv", ["Agent_Type", "Num_Xcc", "Cu_Count", "Simd_Count"], [
        {"Agent_Type": "CPU", "Num_Xcc": 1, "Cu_Count": 16, "Simd_Count": 0},
        {"Agent_Type": "GPU", "Num_Xcc": 8, "Cu_Count": 256, "Simd_Count": 1024}])
    k = "void fmha::attn_fwd_kernel<64>(p)"
    rows = [{"Kernel_Name": k, "Counter_Name": c, "Counter_Value": v} for c, v in [
        ("GRBM_GUI_ACTIVE", 8 * 1000),            # 1000 cycles per XCD
        ("SQ_VALU_MFMA_BUSY_CYCLES", 1024 * 250),  # 25 % of SIMD cycles
        ("SQ_INSTS_MFMA", 1024 * 250 // 32),
        ("SQ_ACTIVE_INST_VALU", 256 * 500),       # 50 %
        ("SQ_WAVE_CYCLES", 256 * 1000 * 3 / 4),   # 3 waves per CU
        ("SQ_WAIT_INST_ANY", 256 * 1000 * 3 / 8)]] + [
        {"Kernel_Name": "void at::native::fill(x)", "Counter_Name": "GRBM_GUI_ACTIVE",
         "Counter_Value": 5}]
    _write(tmp_path / "c.csv", ["Kernel_Name", "Counter_Name", "Counter_Value"], rows)
    bench.counter_summary(str(tmp_path / "agent.csv"), [str(tmp_path / "c.csv")])
    out = capsys.readouterr().out
    assert "kernel cycles (GRBM_GUI_ACTIVE / XCDs): 1000.00" in out
    assert "MFMA busy, % of SIMD cycles: 25.00" in out
    assert "MFMA busy cycles per MFMA instruction: 32.00" in out
    assert "VALU busy, %: 50.00" in out
    assert "resident waves per CU (mean): 3.00" in out
    assert "wave time waiting to issue, %: 50.00" in out
    assert "at::native" not in out
