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


def test_traffic_scales_by_copy_and_sums_call_kernels(tmp_path):
    copy_bytes = 1 << 20
    # FETCH_SIZE reads half of the copy, WRITE_SIZE all of it
    _csv(tmp_path / "f.csv", "FETCH_SIZE", [
        (1, "__amd_rocclr_copyBuffer", [256.0, 256.0]),
        (2, "__amd_rocclr_copyBuffer", [1.0]),                # small incidental copy
        (3, "void decode_split_kernel<128, 16>(DecodeArgs)", [100.0]),
        (4, "void decode_merge_kernel<128>(DecodeArgs)", [10.0]),
    ])
    _csv(tmp_path / "w.csv", "WRITE_SIZE", [
        (1, "__amd_rocclr_copyBuffer", [1024.0]),
        (2, "__amd_rocclr_copyBuffer", [2.0]),
        (3, "void decode_split_kernel<128, 16>(DecodeArgs)", [40.0]),
        (4, "void decode_merge_kernel<128>(DecodeArgs)", [4.0]),
    ])
    out = tmp_path / "t.json"
    subprocess.run([sys.executable, "-m", "block_masked_causal_amd.profile_summary", "traffic",
                    "--fetch", str(tmp_path / "f.csv"), "--write", str(tmp_path / "w.csv"),
                    "--copy-bytes", str(copy_bytes), "--cmd-fetch", "F", "--cmd-write", "W",
                    "--out", str(out)], check=True)
    data = json.load(open(out))
    assert data["calibration"]["fetch_factor"] == 2.0
    assert data["calibration"]["write_factor"] == 1.0
    dec = data["calls"]["block_decode_attention"]
    assert dec["bytes"] == (110 * 2 + 44) * 1024
    assert (tmp_path / "t.md").exists()
    # unchanged sources: the figure is reported; a stale hash: it is dropped
    assert ps.load_traffic(str(out))["block_decode_attention"] == dec["bytes"]
    dec["sha256"] = "0" * 64
    json.dump(data, open(out, "w"))
    assert "block_decode_attention" not in ps.load_traffic(str(out))


def test_missing_traffic_file_reports_nothing(tmp_path):
    assert ps.load_traffic(str(tmp_path / "absent.json")) == {}
