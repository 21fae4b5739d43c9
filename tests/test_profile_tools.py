"""Host-side checks of the profile tooling: the traffic table bench.py writes from
rocprofv3 counter CSVs, and the trace / counter summaries of profiling.py.  The
CSVs here are small synthetic files in rocprofv3's column layout; no GPU runs."""

import csv
import json
import os

import pytest

import bench
from grouped_query_attention_prefill_amd import profiling

COUNTER_COLS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id", "Grid_Size",
                "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size", "Scratch_Size", "VGPR_Count",
                "Accum_VGPR_Count", "SGPR_Count", "Counter_Name", "Counter_Value", "Start_Timestamp",
                "End_Timestamp"]
TRACE_COLS = ["Kind", "Agent_Id", "Queue_Id", "Stream_Id", "Thread_Id", "Dispatch_Id", "Kernel_Id", "Kernel_Name",
              "Correlation_Id", "Start_Timestamp", "End_Timestamp", "LDS_Block_Size", "Scratch_Size", "VGPR_Count",
              "Accum_VGPR_Count", "SGPR_Count", "Workgroup_Size_X", "Workgroup_Size_Y", "Workgroup_Size_Z",
              "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z"]


def _write(path, cols, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=cols)
        w.writeheader()
        for r in rows:
            w.writerow({c: r.get(c, 0) for c in cols})


def _counter_rows(counter, dispatches):
    """dispatches: list of (kernel name, grid, value)."""
    return [{"Dispatch_Id": i, "Kernel_Name": name, "Grid_Size": grid, "Counter_Name": counter,
             "Counter_Value": value} for i, (name, grid, value) in enumerate(dispatches)]


PREFILL = "void gqa::(anonymous namespace)::prefill_bf16_kernel<128, false, false>(gqa::PrefillParams)"
DECODE = "void gqa::(anonymous namespace)::decode16_bf16_kernel<128, false, false>(gqa::DecodeParams)"
COMBINE = "void gqa::(anonymous namespace)::decode_combine_kernel<128, false>(gqa::DecodeParams)"
ROPE = "void gqa::(anonymous namespace)::rope_heads_kernel<unsigned short, 8>(gqa::(anonymous namespace)::RopeSeg)"
BWD = ["gqa::(anonymous namespace)::bwd_dkdv16_kernel(gqa::BwdParams)",
       "void gqa::(anonymous namespace)::bwd_dq_kernel<128>(gqa::BwdParams)"]
COPY = "__amd_rocclr_copyBuffer"


def _fake_runs(out, fetch_scale=2.0):
    """Counter CSVs for every run bench.py lists, with known per-dispatch values (KiB)."""
    want = {}
    for counter, row, d, _ in bench.traffic_commands(out):
        scale = fetch_scale if counter == "FETCH_SIZE" else 1.0
        if row == "copy":
            disp = [(COPY, 512, (1 << 30) / 1024 / scale)] * 2
        elif row.endswith("_backward"):
            disp = [(BWD[0], 10, 2000.0), (BWD[1], 10, 3000.0)] * 2
            want[(counter, row)] = (2000.0 + 3000.0) * 1024 * scale
        elif row.endswith("_qk_rope"):
            # the fused Q+K launch has the largest grid; the Q-only launch must not count
            disp = [(ROPE, 1310720, 40.0), (ROPE, 1048576, 32.0), (PREFILL, 262144, 999.0)]
            want[(counter, row)] = 40.0 * 1024 * scale
        elif row.startswith("prefill"):
            disp = [(PREFILL, 262144, 10.0), (PREFILL, 262144, 14.0)]
            want[(counter, row)] = 12.0 * 1024 * scale
        else:
            disp = [(DECODE, 1024, 500.0), (COMBINE, 64, 7.0), (DECODE, 1024, 700.0)]
            want[(counter, row)] = 600.0 * 1024 * scale
        _write(os.path.join(d, "p_counter_collection.csv"), COUNTER_COLS, _counter_rows(counter, disp))
    return want


def test_traffic_commands_cover_every_row(tmp_path):
    cmds = bench.traffic_commands(str(tmp_path))
    rows = {row for _, row, _, _ in cmds}
    assert rows == {"copy", *bench.TRAFFIC_ROWS}
    for counter, _, d, c in cmds:
        assert c[:3] == ["rocprofv3", "--pmc", counter]
        assert "--" in c and c[c.index("--") + 2].endswith("bench.py")
        assert d.startswith(str(tmp_path))


def test_write_traffic_scales_and_selects(tmp_path, monkeypatch):
    out = str(tmp_path / "runs")
    want = _fake_runs(out)
    prof = tmp_path / "repo" / "profiles"
    prof.mkdir(parents=True)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path / "repo"))
    monkeypatch.setattr(bench, "source_hash", lambda files: "h" + str(len(files)))
    bench.write_traffic(out)
    t = json.loads((prof / "traffic.json").read_text())
    assert t["_calibration"]["fetch_scale"] == pytest.approx(2.0)
    assert t["_calibration"]["write_scale"] == pytest.approx(1.0)
    for row in bench.TRAFFIC_ROWS:
        e = t["rows"][row]
        # KiB x 1024, times the copy's calibration (2 for FETCH_SIZE, 1 for WRITE_SIZE)
        assert e["read"] == round(want[("FETCH_SIZE", row)])
        assert e["written"] == round(want[("WRITE_SIZE", row)])
        assert e["hbm_bytes_per_launch"] == e["read"] + e["written"]
    assert len(t["rows"]["prefill_causal_bf16_T4096_backward"]["kernels"]) == 2
    md = (prof / "hbm_traffic_counters.md").read_text()
    assert "gqa::bwd_dkdv16_kernel" in md and "copyBuffer" not in md.split("| bench row")[1]


def test_measured_traffic_requires_matching_source(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "traffic.json").write_text(json.dumps(
        {"rows": {"prefill_causal_bf16_T4096": {"hbm_bytes_per_launch": 123, "source_hash": "abc"}}}))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "source_hash", lambda files: "abc")
    assert bench.measured_traffic("prefill_causal_bf16_T4096") == 123
    monkeypatch.setattr(bench, "source_hash", lambda files: "changed")
    assert bench.measured_traffic("prefill_causal_bf16_T4096") is None
    assert bench.measured_traffic("decode_bf16_B64_T8192") is None


def test_trace_summary_groups_and_skips_torch(tmp_path):
    rows = []
    t = 1000
    for i in range(30):
        for name, grid, us in ((PREFILL, 262144, 100 + (i >= 10) * 20),
                               ("void at::native::reduce_kernel<512>(float)", 4096, 50),
                               (COMBINE, 8192, 5)):
            rows.append({"Kind": "KERNEL_DISPATCH", "Kernel_Name": name, "Start_Timestamp": t,
                         "End_Timestamp": t + us * 1000, "Grid_Size_X": grid, "Grid_Size_Y": 1, "Grid_Size_Z": 1,
                         "Workgroup_Size_X": 256, "VGPR_Count": 64})
            t += us * 1000 + 10
    _write(str(tmp_path / "trace" / "b_kernel_trace.csv"), TRACE_COLS, rows)
    md = profiling.trace_summary(str(tmp_path / "trace"), last=20)
    lines = [ln for ln in md.splitlines() if ln.startswith("| `")]
    assert len(lines) == 2 and "reduce_kernel" not in md
    cells = [c.strip() for c in lines[0].split("|")]
    assert cells[1] == "`gqa::prefill_bf16_kernel<128, false, false>`"
    assert cells[7] == "30"                    # launches
    assert float(cells[8]) == pytest.approx((10 * 100 + 20 * 120) / 30, abs=0.01)
    assert float(cells[9]) == pytest.approx(120.0)   # the last 20


def test_counter_summary_means(tmp_path):
    rows = _counter_rows("SQ_INSTS_MFMA", [(PREFILL, 1, 10.0), (PREFILL, 1, 30.0), (COMBINE, 1, 5.0)])
    rows += _counter_rows("GRBM_GUI_ACTIVE", [(PREFILL, 1, 4.0), (PREFILL, 1, 6.0)])
    _write(str(tmp_path / "c" / "p_counter_collection.csv"), COUNTER_COLS, rows)
    md = profiling.counter_summary(str(tmp_path / "c"), ["prefill_bf16_kernel"])
    assert "| SQ_INSTS_MFMA | 20 |" in md and "| GRBM_GUI_ACTIVE | 5 |" in md
    assert "combine" not in md
