"""Host logic of the rocprofv3 summaries: counter calibration and source-hash gating."""

import csv
import json
import subprocess
import sys

from block_masked_causal_amd import profile_summary as ps

HEAD = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id",
        "Grid_Size", "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size",
        "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count", "Counter_Name",
        "Counter_Value", "Start_Timestamp", "End_Timestamp"]


def _csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(HEAD)
        for disp, name, vals in rows:
            for v in vals:  # one row per counter dimension; summed per dispatch
                w.writerow([disp, disp, "Agent 1", 1, 1, 1, 64, 1, name, 64, 0, 0, 8, 0, 8,
                            counter, v, 0, 1])


MARK = "void at::native::vectorized_elementwise_kernel<4, at::native::FillFunctor<long>, x>"


def test_traffic_scales_by_copy_and_splits_calls_at_markers(tmp_path):
    copy_bytes = 1 << 20
    plan = tmp_path / "plan.json"
    json.dump({"copy_bytes": copy_bytes, "calls": ["block_decode_attention",
                                                   "loop_decode_attention"]}, open(plan, "w"))
    # FETCH_SIZE reads half of the copy, WRITE_SIZE all of it; the same kernels serve
    # two calls, told apart only by the marker dispatch before each
    _csv(tmp_path / "f.csv", "FETCH_SIZE", [
        (0, "__amd_rocclr_copyBuffer", [900.0]),              # a setup copy before the pass
        (1, MARK, [0.0]),                                     # the marker tensor is created
        (2, "__amd_rocclr_copyBuffer", [256.0, 256.0]),       # the calibration copy
        (3, MARK, [0.0]),
        (4, "void decode_split_kernel<128, 16>(DecodeArgs)", [100.0]),
        (5, "void decode_merge_kernel<128>(DecodeArgs)", [10.0]),
        (6, MARK, [0.0]),
        (7, "void decode_split_kernel<128, 16>(DecodeArgs)", [300.0]),
    ])
    _csv(tmp_path / "w.csv", "WRITE_SIZE", [
        (0, "__amd_rocclr_copyBuffer", [1800.0]),
        (1, MARK, [0.0]),
        (2, "__amd_rocclr_copyBuffer", [1024.0]),
        (3, MARK, [0.0]),
        (4, "void decode_split_kernel<128, 16>(DecodeArgs)", [40.0]),
        (5, "void decode_merge_kernel<128>(DecodeArgs)", [4.0]),
        (6, MARK, [0.0]),
        (7, "void decode_split_kernel<128, 16>(DecodeArgs)", [8.0]),
    ])
    out = tmp_path / "t.json"
    subprocess.run([sys.executable, "-m", "block_masked_causal_amd.profile_summary", "traffic",
                    "--fetch", str(tmp_path / "f.csv"), "--write", str(tmp_path / "w.csv"),
                    "--plan", str(plan), "--cmd-fetch", "F", "--cmd-write", "W",
                    "--out", str(out)], check=True)
    data = json.load(open(out))
    assert data["calibration"]["fetch_factor"] == 2.0
    assert data["calibration"]["write_factor"] == 1.0
    dec = data["calls"]["block_decode_attention"]
    assert dec["bytes"] == (110 * 2 + 44) * 1024 and dec["dispatches"] == 2
    assert data["calls"]["loop_decode_attention"]["bytes"] == (300 * 2 + 8) * 1024
    assert (tmp_path / "t.md").exists()
    # unchanged sources: the figure is reported; a stale hash: it is dropped
    assert ps.load_traffic(str(out))["block_decode_attention"] == dec["bytes"]
    dec["sha256"] = "0" * 64
    json.dump(data, open(out, "w"))
    assert "block_decode_attention" not in ps.load_traffic(str(out))


def test_segments_reject_a_plan_that_does_not_match_the_markers(tmp_path):
    import pytest
    rows = [(0, MARK, {}), (1, "__amd_rocclr_copyBuffer", {}), (2, MARK, {}),
            (3, "k", {"X": 1.0})]
    with pytest.raises(SystemExit):
        ps.segments(rows, ["a", "b"])
    with pytest.raises(SystemExit):
        ps.segments(rows + [(4, MARK, {}), (5, MARK, {})], ["a", "b"])
    with pytest.raises(SystemExit):
        ps.segments(rows[2:], ["a"])          # no calibration copy after a marker
    assert list(ps.segments(rows, ["a"])) == ["a"]


def test_counter_table_derives_mfma_busy(tmp_path):
    plan = tmp_path / "plan.json"
    json.dump({"copy_bytes": 1, "calls": ["two_stream_attention"]}, open(plan, "w"))
    path = tmp_path / "c.csv"
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(HEAD)
        rows = [(0, MARK, "GRBM_GUI_ACTIVE", 5.0),
                (1, "__amd_rocclr_copyBuffer", "GRBM_GUI_ACTIVE", 50.0),
                (2, MARK, "GRBM_GUI_ACTIVE", 5.0),
                (3, "K", "GRBM_GUI_ACTIVE", 8000.0),
                (3, "K", "SQ_VALU_MFMA_BUSY_CYCLES", 256000.0),
                (3, "K", "SQ_INSTS_MFMA", 10.0),
                (3, "K", "SQ_INSTS_VALU", 135.0)]
        for disp, name, ctr, val in rows:
            w.writerow([disp, disp, "Agent 1", 1, 1, 1, 64, 1, name, 64, 0, 0, 8, 0, 8,
                        ctr, val, 0, 1])
    out = tmp_path / "c.md"
    subprocess.run([sys.executable, "-m", "block_masked_causal_amd.profile_summary", "counters",
                    str(path), "--plan", str(plan), "--title", "T", "--cmd", "C",
                    "--out", str(out)], check=True)
    text = open(out).read()
    assert "| two_stream_attention | `K` | 1000 | 25.0 |" in text
    assert "| 13.50 |" in text


def test_missing_traffic_file_reports_nothing(tmp_path):
    assert ps.load_traffic(str(tmp_path / "absent.json")) == {}
